"""Each planted mistake in the oracle (tests/planted.py) must fail at least one CPU pin. The pins run in a pytest
session of their own with the mutation applied (ORACLE_PLANT), so the mistaken oracle never leaks into other tests.
"""
import os
import subprocess
import sys

import pytest

import planted

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("name", sorted(planted.MUTATIONS))
def test_mutation_applies_once(name):
    assert planted.mutated_source(name) != planted.source_of(planted.MUTATIONS[name][0])


def _run_pins(name):
    files, kexpr = planted.MUTATIONS[name][3]
    cmd = [sys.executable, "-m", "pytest", files, "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu"]
    if kexpr:
        cmd += ["-k", kexpr]
    env = dict(os.environ)
    if name:
        env["ORACLE_PLANT"] = name
    else:
        env.pop("ORACLE_PLANT", None)
    return subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


@pytest.mark.parametrize("name", sorted(planted.MUTATIONS))
def test_planted_mistake_fails_a_pin(name):
    r = _run_pins(name)
    tail = (r.stdout + r.stderr)[-600:]
    assert r.returncode == 1 and " failed" in r.stdout, f"{name} ({planted.MUTATIONS[name][4]}) was not caught:\n{tail}"


@pytest.mark.parametrize("pins", sorted({m[3] for m in planted.MUTATIONS.values()}, key=str))
def test_same_pins_pass_without_a_mutation(pins):
    files, kexpr = pins
    cmd = [sys.executable, "-m", "pytest", files, "-q", "-p", "no:cacheprovider", "-m", "not gpu"]
    if kexpr:
        cmd += ["-k", kexpr]
    env = {k: v for k, v in os.environ.items() if k != "ORACLE_PLANT"}
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout + r.stderr)[-600:]

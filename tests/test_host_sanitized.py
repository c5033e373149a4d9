"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/native/check_host.cpp unit-tests the checks applied to words read back from a workspace (job_valid on random and
garbage jobs, clamp_count, the layout signatures, the tree launch's item map and workspace regions) and drives every
entry point through its host-side argument checks (no call reaches a HIP call, so no GPU is needed). The library's
sources are compiled with both sanitizers on the host pass (the device code is built as usual and never runs) and
linked into one executable with the checks.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "lossless_draft_verification_spec_amd", "csrc")
SOURCES = ["sv_api.cpp", "sv_dense.hip", "sv_sparse.hip", "sv_support.hip", "sv_greedy.hip", "sv_tree.hip"]
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm compilers missing")


def test_host_code_is_clean_under_sanitizers(tmp_path):
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC, *SAN]
    procs, objs = [], []
    paths = [os.path.join(CSRC, s) for s in SOURCES] + [os.path.join(ROOT, "tests", "native", "check_host.cpp")]
    for path in paths:
        obj = str(tmp_path / (os.path.basename(path) + ".o"))
        # every file is compiled as HIP: the headers declare device functions beside host code (the device pass is
        # built as usual, the sanitizers instrument only the host pass)
        procs.append(subprocess.Popen([HIPCC, *flags, "-x", "hip", "-c", path, "-o", obj], stdout=subprocess.PIPE,
                                      stderr=subprocess.STDOUT, text=True))
        objs.append(obj)
    for p in procs:
        out = p.communicate()[0]
        assert p.returncode == 0, out[-2000:]
    exe = str(tmp_path / "check_host")
    link = subprocess.run([CLANG, "-fsanitize=address,undefined", *objs, "-L/opt/rocm/lib", "-lamdhip64",
                           "-Wl,-rpath,/opt/rocm/lib", "-o", exe], capture_output=True, text=True)
    assert link.returncode == 0, link.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "ALL HOST CHECKS PASSED" in r.stdout, (r.stdout + r.stderr)[-3000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-3000:]

"""Batched speculative-sampling verifier for AMD Instinct MI355X (gfx950).

The verifier itself is the HIP library ``libsv.so`` (C ABI in ``include/sv.h``); ``sv`` is its ctypes binding and
``workloads`` draws seeded synthetic inputs. The binding is imported on first use of one of its names, so that the
input generators work without the built library; using a verifier entry point without the library raises.
"""
_BINDING = ("sv_verify_dense", "sv_verify_onehot_draft", "sv_verify_sparse", "sv_workspace_bytes",
            "sv_status_string", "SVError", "workspace", "sv_build_support", "sv_support_workspace_bytes",
            "sv_build_support_pair", "support_workspace", "sv_verify_greedy",
            "sv_confidence_commit")


def __getattr__(name):
    if name in _BINDING:
        from . import sv
        return getattr(sv, name)
    raise AttributeError(name)


__all__ = list(_BINDING)

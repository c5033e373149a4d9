"""Python binding of the verifier's C ABI (``include/sv.h``), over ctypes.

Argument marshalling only: tensors are checked for device, dtype and layout, outputs and the workspace are allocated
with torch on the input's device, and the C entry point of the same name is called on the current torch stream.
Every step of the verification runs in the HIP library; there is no fallback. Importing this module raises if the
library has not been built.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsv.so")

SV_OK = 0
SV_F32, SV_BF16 = 0, 1
SV_KIND_DENSE, SV_KIND_ONEHOT, SV_KIND_SPARSE, SV_KIND_GREEDY, SV_KIND_TREE = 0, 1, 2, 3, 4
SV_FLAG_NONFINITE, SV_FLAG_ID_RANGE, SV_FLAG_EMPTY_RESIDUAL, SV_FLAG_Q_ZERO, SV_FLAG_INTERNAL = 1, 2, 4, 8, 16
SV_MAX_GAMMA, SV_MAX_K = 1024, 256
SV_NOALLOC_SCRATCH_BYTES = 16 << 20
SV_MAX_TREE_NODES = 1024
SV_ERR_SCRATCH = -9

EXPORTS = ("sv_workspace_bytes", "sv_status_string", "sv_verify_dense", "sv_verify_dense_noalloc",
           "sv_verify_onehot_draft", "sv_verify_sparse", "sv_support_workspace_bytes", "sv_build_support",
           "sv_build_support_pair", "sv_verify_greedy", "sv_confidence_commit", "sv_verify_tree")


def _load() -> ctypes.CDLL:
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with `python -m lossless_draft_verification_spec_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I64, I32, SZ, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    lib.sv_workspace_bytes.argtypes = [ctypes.c_int, I64, I32, I64]
    lib.sv_workspace_bytes.restype = SZ
    lib.sv_status_string.argtypes = [ctypes.c_int]
    lib.sv_status_string.restype = ctypes.c_char_p
    lib.sv_verify_dense.argtypes = [P, I64, I64, P, I64, I64, ctypes.c_int, I64, I32, I64, P, P, P, F, I32, P, P,
                                    P, P, P, P, P, P, P, SZ, P]
    lib.sv_verify_dense.restype = ctypes.c_int
    lib.sv_verify_dense_noalloc.argtypes = [P, I64, I64, P, I64, I64, ctypes.c_int, I64, I32, I64, P, P, P, F, I32,
                                            P, P, P, P, P, P, P, P, P]
    lib.sv_verify_dense_noalloc.restype = ctypes.c_int
    lib.sv_verify_onehot_draft.argtypes = [P, I64, I64, ctypes.c_int, I64, I32, I64, P, P, P, F, I32, P, P,
                                           P, P, P, P, P, P, SZ, P]
    lib.sv_verify_onehot_draft.restype = ctypes.c_int
    lib.sv_verify_sparse.argtypes = [P, P, P, P, I64, I32, I32, I32, I64, P, P, P, I32, P, P, P, P, P, P, P, P, SZ, P]
    lib.sv_verify_sparse.restype = ctypes.c_int
    lib.sv_support_workspace_bytes.argtypes = [I64, I64, I32]
    lib.sv_support_workspace_bytes.restype = SZ
    lib.sv_build_support.argtypes = [P, I64, ctypes.c_int, I64, I64, F, I32, F, I32, P, P, P, P, P, SZ, P]
    lib.sv_build_support.restype = ctypes.c_int
    lib.sv_build_support_pair.argtypes = [P, I64, I64, P, I64, I64, ctypes.c_int, I64, F, I32, F, I32,
                                          P, P, P, P, P, P, P, P, P, SZ, P]
    lib.sv_build_support_pair.restype = ctypes.c_int
    lib.sv_verify_greedy.argtypes = [P, I64, I64, ctypes.c_int, I64, I32, I64, P, I32, P, P, P, P, P, P, P, SZ, P]
    lib.sv_verify_greedy.restype = ctypes.c_int
    lib.sv_confidence_commit.argtypes = [P, I64, I64, ctypes.c_int, I64, I32, I64, P, F, P, P, P, P, P, P, SZ, P]
    lib.sv_confidence_commit.restype = ctypes.c_int
    lib.sv_verify_tree.argtypes = [P, I64, I64, ctypes.c_int, I64, I32, I64, P, P, P, P, F, P, P, P, P, P, P, P, SZ, P]
    lib.sv_verify_tree.restype = ctypes.c_int
    return lib


LIB = _load()


class SVError(RuntimeError):
    def __init__(self, status: int):
        super().__init__(f"sv status {status}: {sv_status_string(status)}")
        self.status = status


def sv_workspace_bytes(kind: int, B: int, gamma: int, V_or_k: int) -> int:
    return int(LIB.sv_workspace_bytes(kind, B, gamma, V_or_k))


def sv_support_workspace_bytes(rows: int, V: int, k: int) -> int:
    return int(LIB.sv_support_workspace_bytes(rows, V, k))


def sv_status_string(status: int) -> str:
    return LIB.sv_status_string(status).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, name, dtype, shape, device):
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _logits_layout(t, name, rows, B, device):
    if t.device != device or t.dim() != 3 or t.shape[0] != B or t.shape[1] < rows:
        raise ValueError(f"{name}: expected a [B={B}, >={rows}, V] tensor on {device}")
    if t.stride(2) != 1 and t.shape[2] > 1:
        raise ValueError(f"{name}: the vocabulary axis must be contiguous")
    # a size-1 axis may carry any stride (numpy's newaxis gives 0); it is never stepped, so pass 1
    seq = t.stride(0) if t.shape[0] > 1 else 1
    row = t.stride(1) if t.shape[1] > 1 else 1
    return seq, row


def _zeroed_workspace(n: int, device) -> torch.Tensor | None:
    if n == (1 << 64) - 1:
        raise SVError(-2)
    if n == 0:
        return None
    # any initial contents are valid (the first workgroup of a call clears the control words when the workspace
    # header does not name the call's layout); a zero-filled buffer keeps fresh allocations reproducible
    ws = torch.zeros(n + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    return ws[off:off + n]


def workspace(kind: int, B: int, gamma: int, V_or_k: int, device) -> torch.Tensor | None:
    return _zeroed_workspace(sv_workspace_bytes(kind, B, gamma, V_or_k), device)


def support_workspace(rows: int, V: int, k: int, device) -> torch.Tensor | None:
    return _zeroed_workspace(sv_support_workspace_bytes(rows, V, k), device)


def _dtype_code(t):
    if t.dtype == torch.float32:
        return SV_F32
    if t.dtype == torch.bfloat16:
        return SV_BF16
    raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")


def _outputs(B, G, device, out, names):
    out = {} if out is None else out
    spec = {"accept": ((B, G), torch.uint8), "n_accepted": ((B,), torch.int32), "out_token": ((B,), torch.int32),
            "p_draft": ((B, G), torch.float32), "q_draft": ((B, G), torch.float32), "flags": ((B,), torch.int32)}
    for n in names:
        if n not in out:
            shape, dt = spec[n]
            out[n] = torch.empty(shape, dtype=dt, device=device)
    return out


def sv_verify_dense(target, draft, draft_ids, u_accept, u_sample, temperature, bonus=1, start=None, order=None, *,
                    out=None, ws=None, stream=None, outputs=("accept", "n_accepted", "out_token", "p_draft",
                                                            "q_draft", "flags")):
    """Dense verification (see ``sv_verify_dense`` in include/sv.h). target [B, gamma+bonus, V], draft [B, gamma, V]
    (float32 or bfloat16, vocabulary axis contiguous); draft_ids int32 [B, gamma]; u_accept float32 [B, gamma];
    u_sample float32 [B, gamma + 1]; start int32 [B] (updated in place) or None; order int32 [B, gamma] or None.
    Returns a dict of output tensors (flags as int32 holding the uint32 bits)."""
    B, G = draft_ids.shape
    dev = target.device
    V = target.shape[-1]
    t_seq, t_row = _logits_layout(target, "target", G + bonus, B, dev)
    d_seq, d_row = _logits_layout(draft, "draft", G, B, dev)
    if draft.dtype != target.dtype or draft.shape[-1] != V:
        raise ValueError("draft must match target in dtype and vocabulary size")
    _need(draft_ids, "draft_ids", torch.int32, (B, G), dev)
    _need(u_accept, "u_accept", torch.float32, (B, G), dev)
    _need(u_sample, "u_sample", torch.float32, (B, G + 1), dev)
    if start is not None:
        _need(start, "start", torch.int32, (B,), dev)
    if order is not None:
        _need(order, "order", torch.int32, (B, G), dev)
    o = _outputs(B, G, dev, out, outputs)
    if ws is None:
        ws = workspace(SV_KIND_DENSE, B, G, V, dev)
    st = LIB.sv_verify_dense(_ptr(target), t_seq, t_row, _ptr(draft), d_seq, d_row, _dtype_code(target), B, G, V,
                             _ptr(draft_ids), _ptr(u_accept), _ptr(u_sample), float(temperature), int(bonus),
                             _ptr(start), _ptr(order), _ptr(o.get("accept")), _ptr(o["n_accepted"]),
                             _ptr(o["out_token"]), _ptr(o.get("p_draft")), _ptr(o.get("q_draft")), _ptr(o.get("flags")),
                             _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream))
    if st != SV_OK:
        raise SVError(st)
    return o


def sv_verify_dense_noalloc(target, draft, draft_ids, u_accept, u_sample, temperature, bonus=1, start=None,
                            order=None, *, out=None, stream=None,
                            outputs=("accept", "n_accepted", "out_token", "p_draft", "q_draft", "flags")):
    """sv_verify_dense on the library's static per-GPU scratch (see ``sv_verify_dense_noalloc`` in include/sv.h):
    no workspace argument. Outputs are allocated here unless `out` holds them already."""
    B, G = draft_ids.shape
    dev = target.device
    V = target.shape[-1]
    t_seq, t_row = _logits_layout(target, "target", G + bonus, B, dev)
    d_seq, d_row = _logits_layout(draft, "draft", G, B, dev)
    if draft.dtype != target.dtype or draft.shape[-1] != V:
        raise ValueError("draft must match target in dtype and vocabulary size")
    _need(draft_ids, "draft_ids", torch.int32, (B, G), dev)
    _need(u_accept, "u_accept", torch.float32, (B, G), dev)
    _need(u_sample, "u_sample", torch.float32, (B, G + 1), dev)
    if start is not None:
        _need(start, "start", torch.int32, (B,), dev)
    if order is not None:
        _need(order, "order", torch.int32, (B, G), dev)
    o = _outputs(B, G, dev, out, outputs)
    st = LIB.sv_verify_dense_noalloc(_ptr(target), t_seq, t_row, _ptr(draft), d_seq, d_row, _dtype_code(target), B, G,
                                     V, _ptr(draft_ids), _ptr(u_accept), _ptr(u_sample), float(temperature), int(bonus),
                                     _ptr(start), _ptr(order), _ptr(o.get("accept")), _ptr(o["n_accepted"]),
                                     _ptr(o["out_token"]), _ptr(o.get("p_draft")), _ptr(o.get("q_draft")),
                                     _ptr(o.get("flags")), _stream(stream))
    if st != SV_OK:
        raise SVError(st)
    return o


def sv_verify_onehot_draft(target, draft_ids, u_accept, u_sample, temperature, bonus=1, start=None, order=None, *,
                           out=None, ws=None, stream=None,
                           outputs=("accept", "n_accepted", "out_token", "p_draft", "flags")):
    """Greedy-draft verification (see ``sv_verify_onehot_draft`` in include/sv.h): q is one-hot at each draft id."""
    B, G = draft_ids.shape
    dev = target.device
    V = target.shape[-1]
    t_seq, t_row = _logits_layout(target, "target", G + bonus, B, dev)
    _need(draft_ids, "draft_ids", torch.int32, (B, G), dev)
    _need(u_accept, "u_accept", torch.float32, (B, G), dev)
    _need(u_sample, "u_sample", torch.float32, (B, G + 1), dev)
    if start is not None:
        _need(start, "start", torch.int32, (B,), dev)
    if order is not None:
        _need(order, "order", torch.int32, (B, G), dev)
    o = _outputs(B, G, dev, out, outputs)
    if ws is None:
        ws = workspace(SV_KIND_ONEHOT, B, G, V, dev)
    st = LIB.sv_verify_onehot_draft(_ptr(target), t_seq, t_row, _dtype_code(target), B, G, V, _ptr(draft_ids),
                                    _ptr(u_accept), _ptr(u_sample), float(temperature), int(bonus), _ptr(start),
                                    _ptr(order), _ptr(o.get("accept")), _ptr(o["n_accepted"]), _ptr(o["out_token"]),
                                    _ptr(o.get("p_draft")), _ptr(o.get("flags")), _ptr(ws),
                                    0 if ws is None else ws.numel(), _stream(stream))
    if st != SV_OK:
        raise SVError(st)
    return o


def sv_verify_greedy(target, draft_ids, bonus=1, start=None, order=None, *, out=None, ws=None, stream=None,
                     outputs=("accept", "n_accepted", "out_token", "flags")):
    """Greedy verification at temperature 0 (see ``sv_verify_greedy`` in include/sv.h): a draft is kept when it is
    the argmax of its target row. target [B, gamma+bonus, V] float32 or bfloat16 (vocabulary axis contiguous);
    draft_ids int32 [B, gamma]; start int32 [B] (updated in place) or None; order int32 [B, gamma] or None."""
    B, G = draft_ids.shape
    dev = target.device
    V = target.shape[-1]
    t_seq, t_row = _logits_layout(target, "target", G + bonus, B, dev)
    _need(draft_ids, "draft_ids", torch.int32, (B, G), dev)
    if start is not None:
        _need(start, "start", torch.int32, (B,), dev)
    if order is not None:
        _need(order, "order", torch.int32, (B, G), dev)
    o = _outputs(B, G, dev, out, outputs)
    if ws is None:
        ws = workspace(SV_KIND_GREEDY, B, G, V, dev)
    st = LIB.sv_verify_greedy(_ptr(target), t_seq, t_row, _dtype_code(target), B, G, V, _ptr(draft_ids), int(bonus),
                              _ptr(start), _ptr(order), _ptr(o.get("accept")), _ptr(o["n_accepted"]),
                              _ptr(o["out_token"]), _ptr(o.get("flags")), _ptr(ws), 0 if ws is None else ws.numel(),
                              _stream(stream))
    if st != SV_OK:
        raise SVError(st)
    return o


def sv_confidence_commit(logits, tau, masked=None, *, out=None, ws=None, stream=None):
    """Confidence-threshold commit (see ``sv_confidence_commit`` in include/sv.h). logits [B, W, V] float32 or
    bfloat16 (vocabulary axis contiguous); masked uint8 [B, W] or None. Returns commit, token, confidence, n_commit,
    flags."""
    B, W, V = logits.shape
    dev = logits.device
    l_seq, l_row = _logits_layout(logits, "logits", W, B, dev)
    if masked is not None:
        _need(masked, "masked", torch.uint8, (B, W), dev)
    o = {} if out is None else out
    for name, shape, dt in (("commit", (B, W), torch.uint8), ("token", (B, W), torch.int32),
                            ("confidence", (B, W), torch.float32), ("n_commit", (B,), torch.int32),
                            ("flags", (B,), torch.int32)):
        if name not in o:
            o[name] = torch.empty(shape, dtype=dt, device=dev)
    if ws is None:
        ws = workspace(SV_KIND_GREEDY, B, W, V, dev)
    st = LIB.sv_confidence_commit(_ptr(logits), l_seq, l_row, _dtype_code(logits), B, W, V, _ptr(masked), float(tau),
                                  _ptr(o["commit"]), _ptr(o["token"]), _ptr(o["confidence"]), _ptr(o["n_commit"]),
                                  _ptr(o["flags"]), _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream))
    if st != SV_OK:
        raise SVError(st)
    return o


def sv_verify_sparse(p_ids, p_probs, q_ids, q_probs, spec_ids, u_accept, u_sample, bonus=1, vocab_size=0, *,
                     out=None, stream=None,
                     outputs=("accept", "n_accepted", "out_token", "correction_probs", "p_spec", "q_spec", "flags")):
    """Sparse top-k verification (see ``sv_verify_sparse`` in include/sv.h). p_ids/p_probs [B, gamma+bonus, kp],
    q_ids/q_probs [B, gamma, kq] (int32 / float32, contiguous); spec_ids int32 [B, gamma]."""
    B, G = spec_ids.shape
    dev = spec_ids.device
    kp, kq = p_ids.shape[-1], q_ids.shape[-1]
    _need(p_ids, "p_ids", torch.int32, (B, G + bonus, kp), dev)
    _need(p_probs, "p_probs", torch.float32, (B, G + bonus, kp), dev)
    _need(q_ids, "q_ids", torch.int32, (B, G, kq), dev)
    _need(q_probs, "q_probs", torch.float32, (B, G, kq), dev)
    _need(spec_ids, "spec_ids", torch.int32, (B, G), dev)
    _need(u_accept, "u_accept", torch.float32, (B, G), dev)
    _need(u_sample, "u_sample", torch.float32, (B, G + 1), dev)
    o = {} if out is None else out
    spec = {"accept": ((B, G), torch.uint8), "n_accepted": ((B,), torch.int32), "out_token": ((B,), torch.int32),
            "correction_probs": ((B, G, kp), torch.float32), "p_spec": ((B, G), torch.float32),
            "q_spec": ((B, G), torch.float32), "flags": ((B,), torch.int32)}
    for n in outputs:
        if n not in o:
            o[n] = torch.empty(spec[n][0], dtype=spec[n][1], device=dev)
    st = LIB.sv_verify_sparse(_ptr(p_ids), _ptr(p_probs), _ptr(q_ids), _ptr(q_probs), B, G, kp, kq, int(vocab_size),
                              _ptr(spec_ids), _ptr(u_accept), _ptr(u_sample), int(bonus), _ptr(o.get("accept")),
                              _ptr(o["n_accepted"]), _ptr(o["out_token"]), _ptr(o.get("correction_probs")),
                              _ptr(o.get("p_spec")), _ptr(o.get("q_spec")), _ptr(o.get("flags")), None, 0,
                              _stream(stream))
    if st != SV_OK:
        raise SVError(st)
    return o


def _support_rows(logits, name):
    """(rows, ld, leading shape) of a logits tensor for the support builder."""
    V = logits.shape[-1]
    lead = tuple(logits.shape[:-1])
    if logits.dim() == 2 and logits.stride(-1) == 1:
        rows = logits.shape[0]
        ld = logits.stride(0) if rows > 1 else V
    elif logits.is_contiguous():
        rows = 1
        for d in lead:
            rows *= d
        ld = V
    else:
        raise ValueError(f"{name} must be contiguous, or 2-D with a contiguous vocabulary axis")
    return rows, ld, lead


def _support_out(out, lead, k, dev):
    o = {} if out is None else out
    spec = {"ids": (lead + (k,), torch.int32), "probs": (lead + (k,), torch.float32), "count": (lead, torch.int32),
            "flags": (lead, torch.int32)}
    for n, (shape, dt) in spec.items():
        if n not in o:
            o[n] = torch.empty(shape, dtype=dt, device=dev)
        else:
            _need(o[n], n, dt, shape, dev)
    return o


def sv_build_support(logits, k, top_p, temperature=1.0, renorm=True, *, out=None, ws=None, stream=None):
    """Top-k / top-p supports of logit rows (see ``sv_build_support`` in include/sv.h). logits [..., V] float32 or
    bfloat16: a contiguous tensor, or a 2-D tensor whose rows may be strided. Returns a dict: ids [..., k] int32,
    probs [..., k] float32, count [...] int32, flags [...] int32 (the uint32 bits)."""
    dev = logits.device
    V = logits.shape[-1]
    rows, ld, lead = _support_rows(logits, "logits")
    o = _support_out(out, lead, k, dev)
    if ws is None:
        ws = support_workspace(rows, V, k, dev)
    st = LIB.sv_build_support(_ptr(logits), ld, _dtype_code(logits), rows, V, float(temperature), int(k),
                              float(top_p), 1 if renorm else 0, _ptr(o["ids"]), _ptr(o["probs"]), _ptr(o["count"]),
                              _ptr(o["flags"]), _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream))
    if st != SV_OK:
        raise SVError(st)
    return o


def sv_build_support_pair(logits_a, logits_b, k, top_p, temperature=1.0, renorm=True, *, out_a=None, out_b=None,
                          ws=None, stream=None):
    """Supports of two sets of logit rows in one launch (see ``sv_build_support_pair`` in include/sv.h): each set as
    the logits of ``sv_build_support``, of one dtype and vocabulary size. Returns the two output dicts."""
    dev = logits_a.device
    V = logits_a.shape[-1]
    if logits_b.shape[-1] != V or logits_b.dtype != logits_a.dtype or logits_b.device != dev:
        raise ValueError("logits_a and logits_b must share the vocabulary size, dtype and device")
    rows_a, ld_a, lead_a = _support_rows(logits_a, "logits_a")
    rows_b, ld_b, lead_b = _support_rows(logits_b, "logits_b")
    oa = _support_out(out_a, lead_a, k, dev)
    ob = _support_out(out_b, lead_b, k, dev)
    if ws is None:
        ws = support_workspace(rows_a + rows_b, V, k, dev)
    st = LIB.sv_build_support_pair(_ptr(logits_a), ld_a, rows_a, _ptr(logits_b), ld_b, rows_b,
                                   _dtype_code(logits_a), V, float(temperature), int(k), float(top_p),
                                   1 if renorm else 0,
                                   _ptr(oa["ids"]), _ptr(oa["probs"]), _ptr(oa["count"]), _ptr(oa["flags"]),
                                   _ptr(ob["ids"]), _ptr(ob["probs"]), _ptr(ob["count"]), _ptr(ob["flags"]),
                                   _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream))
    if st != SV_OK:
        raise SVError(st)
    return oa, ob


def sv_verify_tree(target, parent, token, u_accept, u_sample, temperature, *, out=None, ws=None, stream=None):
    """Tree verification (see ``sv_verify_tree`` in include/sv.h). target [B, N, V] float32 or bfloat16 (vocabulary
    axis contiguous): row i is the target's distribution after the path to node i; parent, token int32 [B, N];
    u_accept, u_sample float32 [B, N]. Returns accept, n_accepted, path, out_token, p_test, flags."""
    B, N = parent.shape
    dev = target.device
    V = target.shape[-1]
    t_seq, t_row = _logits_layout(target, "target", N, B, dev)
    _need(parent, "parent", torch.int32, (B, N), dev)
    _need(token, "token", torch.int32, (B, N), dev)
    _need(u_accept, "u_accept", torch.float32, (B, N), dev)
    _need(u_sample, "u_sample", torch.float32, (B, N), dev)
    o = {} if out is None else out
    for name, shape, dt in (("accept", (B, N), torch.uint8), ("n_accepted", (B,), torch.int32),
                            ("path", (B, N), torch.int32), ("out_token", (B,), torch.int32),
                            ("p_test", (B, N), torch.float32), ("flags", (B,), torch.int32)):
        if name not in o:
            o[name] = torch.empty(shape, dtype=dt, device=dev)
    if ws is None:
        ws = workspace(SV_KIND_TREE, B, N, V, dev)
    st = LIB.sv_verify_tree(_ptr(target), t_seq, t_row, _dtype_code(target), B, N, V, _ptr(parent), _ptr(token),
                            _ptr(u_accept), _ptr(u_sample), float(temperature), _ptr(o["accept"]), _ptr(o["n_accepted"]),
                            _ptr(o["path"]), _ptr(o["out_token"]), _ptr(o["p_test"]), _ptr(o["flags"]), _ptr(ws),
                            0 if ws is None else ws.numel(), _stream(stream))
    if st != SV_OK:
        raise SVError(st)
    return o

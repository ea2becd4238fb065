"""Python binding of liblizard_attn.so, the Lizard hybrid attention library.

Argument marshalling only: torch tensors provide device memory and the
current HIP stream; every step of the layer runs in the library's HIP
kernels.  There is no fallback: without the built library every call
raises.  The names mirror the C ABI in include/lizard_attn.h.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Dict, Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblizard_attn.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "lizard_attn.h")

LIZARD_F32, LIZARD_BF16 = 0, 1
STATUS = {
    0: "LIZARD_OK", -1: "LIZARD_E_NULL", -2: "LIZARD_E_SHAPE", -3: "LIZARD_E_DTYPE",
    -4: "LIZARD_E_ALIGN", -5: "LIZARD_E_WORKSPACE", -6: "LIZARD_E_UNSUPPORTED", -7: "LIZARD_E_LAUNCH",
}
STATUS_CODE = {v: k for k, v in STATUS.items()}


class LizardParams(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("L", ctypes.c_int32),
        ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("chunk", ctypes.c_int32),
        ("window", ctypes.c_int32), ("n_meta", ctypes.c_int32),
        ("alpha", ctypes.c_float), ("softmax_scale", ctypes.c_float),
        ("dtype", ctypes.c_int),
    ]


class LizardError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} returned {STATUS.get(status, status)}")


_lib: Optional[ctypes.CDLL] = None
_vp = ctypes.c_void_p


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m subquadratic_attention_amd.build`")
    # torch first: its HIP runtime is then the one the library binds to (a
    # library loaded before torch would bind another copy of the runtime,
    # whose launches fail on torch's device memory)
    _torch()
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(LizardParams)
    lib.lizard_attn_fwd.argtypes = [P] + [_vp] * 10
    lib.lizard_attn_fwd.restype = ctypes.c_int
    lib.lizard_attn_bwd_workspace_size.argtypes = [P]
    lib.lizard_attn_bwd_workspace_size.restype = ctypes.c_size_t
    lib.lizard_attn_bwd.argtypes = [P] + [_vp] * 13 + [ctypes.c_size_t, _vp]
    lib.lizard_attn_bwd.restype = ctypes.c_int
    lib.lizard_decode_step.argtypes = [P, ctypes.c_int64] + [_vp] * 10
    lib.lizard_decode_step.restype = ctypes.c_int
    lib.lizard_attn_fwd_logit.argtypes = [P] + [_vp] * 10
    lib.lizard_attn_fwd_logit.restype = ctypes.c_int
    lib.lizard_attn_bwd_logit.argtypes = [P] + [_vp] * 13 + [ctypes.c_size_t, _vp]
    lib.lizard_attn_bwd_logit.restype = ctypes.c_int
    lib.lizard_decode_step_logit.argtypes = [P, ctypes.c_int64] + [_vp] * 10
    lib.lizard_decode_step_logit.restype = ctypes.c_int
    lib.lizard_attn_fwd_continue.argtypes = [P] + [_vp] * 9 + [ctypes.c_int32] + [_vp] * 5
    lib.lizard_attn_fwd_continue.restype = ctypes.c_int
    lib.lizard_attn_fwd_split_workspace_size.argtypes = [P]
    lib.lizard_attn_fwd_split_workspace_size.restype = ctypes.c_size_t
    lib.lizard_attn_fwd_split.argtypes = [P] + [_vp] * 9 + [ctypes.c_int32] + [_vp] * 5 + [ctypes.c_size_t, _vp]
    lib.lizard_attn_fwd_split.restype = ctypes.c_int
    lib.lizard_attn_fwd_split_noalloc.argtypes = [P] + [_vp] * 9 + [ctypes.c_int32] + [_vp] * 5
    lib.lizard_attn_fwd_split_noalloc.restype = ctypes.c_int
    lib.lizard_attn_chunk_states_size.argtypes = [P]
    lib.lizard_attn_chunk_states_size.restype = ctypes.c_size_t
    lib.lizard_attn_fwd_train.argtypes = [P] + [_vp] * 12
    lib.lizard_attn_fwd_train.restype = ctypes.c_int
    lib.lizard_attn_bwd_train.argtypes = [P] + [_vp] * 15 + [ctypes.c_size_t, _vp]
    lib.lizard_attn_bwd_train.restype = ctypes.c_int
    lib.lizard_softmax_attn_fwd.argtypes = [P] + [_vp] * 6
    lib.lizard_softmax_attn_fwd.restype = ctypes.c_int
    lib.lizard_transfer_loss.argtypes = [P] + [_vp] * 5
    lib.lizard_transfer_loss.restype = ctypes.c_int
    for fn in ("lizard_decode_tokens", "lizard_decode_tokens_logit"):
        getattr(lib, fn).argtypes = [P, _vp, ctypes.c_int32] + [_vp] * 10
        getattr(lib, fn).restype = ctypes.c_int
    lib.lizard_status_string.argtypes = [ctypes.c_int]
    lib.lizard_status_string.restype = ctypes.c_char_p
    lib.lizard_abi_version.argtypes = []
    lib.lizard_abi_version.restype = ctypes.c_int
    _lib = lib
    return lib


def make_params(B, H, L, d, *, window, n_meta, alpha, dtype, chunk=64, softmax_scale=0.0) -> LizardParams:
    return LizardParams(B, H, L, d, d, chunk, window, n_meta, float(alpha), float(softmax_scale), int(dtype))


# ---------------------------------------------------------------------------
# torch-level wrappers
# ---------------------------------------------------------------------------

def _torch():
    import torch

    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return LIZARD_BF16
    if t.dtype == torch.float32:
        return LIZARD_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _expect(name: str, t, shape, dtype, device) -> None:
    """Shape, dtype and device of one tensor argument, checked before any
    pointer reaches the library (a wrong size or dtype would make a kernel
    read or write past the allocation).  None passes (optional arguments)."""
    if t is None:
        return
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(int(x) for x in shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")


def _expect_seq_inputs(q, k, v, meta_k, log_g=None, gate_logit=None):
    """q, k, v [B, H, L, d] in one dtype; log_g float32 and gate_logit q's
    dtype, both [B, H, L, d]; meta_k [H, m, d] in q's dtype."""
    torch = _torch()
    _dtype_code(q)
    if q.dim() != 4:
        raise ValueError(f"q: expected [B, H, L, d], got shape {tuple(q.shape)}")
    B, H, L, d = q.shape
    for name, t in (("k", k), ("v", v)):
        if t is None:
            raise ValueError(f"{name} is required")
        _expect(name, t, q.shape, q.dtype, q.device)
    _expect("log_g", log_g, q.shape, torch.float32, q.device)
    _expect("gate_logit", gate_logit, q.shape, q.dtype, q.device)
    if meta_k is not None:
        if meta_k.dim() != 3:
            raise ValueError(f"meta_k: expected [H, m, d], got shape {tuple(meta_k.shape)}")
        _expect("meta_k", meta_k, (H, meta_k.shape[1], d), q.dtype, q.device)


def _expect_fwd_out(o, q):
    torch = _torch()
    B, H, L, d = q.shape
    _expect("y", o.get("y"), q.shape, q.dtype, q.device)
    _expect("lse", o.get("lse"), (B, H, L), torch.float32, q.device)
    _expect("y_anchor", o.get("y_anchor"), q.shape, q.dtype, q.device)
    _expect("state", o.get("state"), (B, H, d, d), torch.float32, q.device)


def _expect_bwd(q, meta_k, lse, dy, o, gkey, gate, workspace, ws_bytes):
    torch = _torch()
    B, H, L, d = q.shape
    _expect("lse", lse, (B, H, L), torch.float32, q.device)
    _expect("dy", dy, q.shape, q.dtype, q.device)
    for key in ("dq", "dk", "dv"):
        _expect(key, o.get(key), q.shape, q.dtype, q.device)
    _expect(gkey, o.get(gkey), q.shape, gate.dtype, q.device)
    if meta_k is not None:
        _expect("dmeta", o.get("dmeta"), meta_k.shape, torch.float32, q.device)
    if workspace is not None:
        if workspace.dtype != torch.uint8 or workspace.device != q.device or workspace.numel() < ws_bytes:
            raise ValueError(f"workspace: a uint8 tensor of at least {ws_bytes} bytes on {q.device} is required")


def _stream(device) -> int:
    return _torch().cuda.current_stream(device).cuda_stream


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise LizardError(fn, status)


def lizard_attn_fwd(q, k, v, log_g, meta_k, *, window: int, alpha: float, softmax_scale: float = 0.0,
                    chunk: int = 64, need_lse: bool = False, need_y_anchor: bool = False,
                    need_state: bool = False, out: Optional[Dict] = None) -> Dict:
    """Forward pass.  q, k, v: [B, H, L, d]; log_g: [B, H, L, d] float32;
    meta_k: [H, m, d].  Returns {"y", and optionally "lse", "y_anchor",
    "state"}; pass ``out`` (same keys) to reuse preallocated outputs."""
    return _fwd("lizard_attn_fwd", q, k, v, log_g, meta_k, window, alpha, softmax_scale, chunk, need_lse,
                need_y_anchor, need_state, out)


def lizard_attn_fwd_logit(q, k, v, gate_logit, meta_k, *, window: int, alpha: float, softmax_scale: float = 0.0,
                          chunk: int = 64, need_lse: bool = False, need_y_anchor: bool = False,
                          need_state: bool = False, out: Optional[Dict] = None) -> Dict:
    """Forward pass with the gates given by their logits: gate_logit
    [B, H, L, d] in q's dtype (log_g = log sigmoid(gate_logit) in-kernel)."""
    return _fwd("lizard_attn_fwd_logit", q, k, v, gate_logit, meta_k, window, alpha, softmax_scale, chunk, need_lse,
                need_y_anchor, need_state, out)


def _fwd(fn, q, k, v, gate, meta_k, window, alpha, softmax_scale, chunk, need_lse, need_y_anchor, need_state, out):
    torch = _torch()
    lib = load_library()
    logit = fn.endswith("_logit")
    _expect_seq_inputs(q, k, v, meta_k, log_g=None if logit else gate, gate_logit=gate if logit else None)
    if gate is None:
        raise ValueError("the gates are required")
    B, H, L, d = q.shape
    m = meta_k.shape[1] if meta_k is not None else 0
    dt = _dtype_code(q)
    p = make_params(B, H, L, d, window=window, n_meta=m, alpha=alpha, dtype=dt, chunk=chunk,
                    softmax_scale=softmax_scale)
    o = dict(out) if out is not None else {}
    if "y" not in o:
        o["y"] = torch.empty_like(q)
    if need_lse and "lse" not in o:
        o["lse"] = torch.empty((B, H, L), device=q.device, dtype=torch.float32)
    if need_y_anchor and "y_anchor" not in o:
        o["y_anchor"] = torch.empty_like(q)
    if need_state and "state" not in o:
        o["state"] = torch.empty((B, H, d, d), device=q.device, dtype=torch.float32)
    _expect_fwd_out(o, q)
    st = getattr(lib, fn)(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(meta_k),
                          _ptr(o["y"]), _ptr(o.get("lse")), _ptr(o.get("y_anchor")), _ptr(o.get("state")),
                          _stream(q.device))
    _check(fn, st)
    return o


def lizard_attn_bwd_workspace_size(B, H, L, d, *, window: int, n_meta: int, dtype: int, chunk: int = 64) -> int:
    lib = load_library()
    p = make_params(B, H, L, d, window=window, n_meta=n_meta, alpha=0.0, dtype=dtype, chunk=chunk)
    return int(lib.lizard_attn_bwd_workspace_size(ctypes.byref(p)))


def lizard_attn_bwd(q, k, v, log_g, meta_k, lse, dy, *, window: int, alpha: float, softmax_scale: float = 0.0,
                    chunk: int = 64, workspace=None, out: Optional[Dict] = None) -> Dict:
    """Backward pass of sum(dy * Y).  Returns {"dq", "dk", "dv", "dlog_g",
    "dmeta"} (dmeta summed over the batch)."""
    return _bwd("lizard_attn_bwd", "dlog_g", q, k, v, log_g, meta_k, lse, dy, window, alpha, softmax_scale, chunk,
                workspace, out)


def lizard_attn_bwd_logit(q, k, v, gate_logit, meta_k, lse, dy, *, window: int, alpha: float,
                          softmax_scale: float = 0.0, chunk: int = 64, workspace=None, out: Optional[Dict] = None) -> Dict:
    """Backward pass with the gates given by their logits.  Returns {"dq",
    "dk", "dv", "dgate_logit" (q's dtype), "dmeta"}."""
    return _bwd("lizard_attn_bwd_logit", "dgate_logit", q, k, v, gate_logit, meta_k, lse, dy, window, alpha,
                softmax_scale, chunk, workspace, out)


def _bwd(fn, gkey, q, k, v, gate, meta_k, lse, dy, window, alpha, softmax_scale, chunk, workspace, out):
    torch = _torch()
    lib = load_library()
    logit = gkey == "dgate_logit"
    _expect_seq_inputs(q, k, v, meta_k, log_g=None if logit else gate, gate_logit=gate if logit else None)
    if gate is None or lse is None or dy is None:
        raise ValueError("the gates, lse and dy are required")
    B, H, L, d = q.shape
    m = meta_k.shape[1] if meta_k is not None else 0
    dt = _dtype_code(q)
    p = make_params(B, H, L, d, window=window, n_meta=m, alpha=alpha, dtype=dt, chunk=chunk,
                    softmax_scale=softmax_scale)
    ws_bytes = int(lib.lizard_attn_bwd_workspace_size(ctypes.byref(p)))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), device=q.device, dtype=torch.uint8)
    o = dict(out) if out is not None else {}
    for key, like in (("dq", q), ("dk", k), ("dv", v)):
        if key not in o:
            o[key] = torch.empty_like(like)
    if gkey not in o:
        o[gkey] = torch.empty_like(gate)
    if "dmeta" not in o:
        o["dmeta"] = torch.empty((H, m, d), device=q.device, dtype=torch.float32) if m > 0 else None
    _expect_bwd(q, meta_k, lse, dy, o, gkey, gate, workspace, ws_bytes)
    st = getattr(lib, fn)(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(meta_k), _ptr(lse),
                          _ptr(dy), _ptr(o["dq"]), _ptr(o["dk"]), _ptr(o["dv"]), _ptr(o[gkey]),
                          _ptr(o["dmeta"]), _ptr(workspace), workspace.numel(), _stream(q.device))
    _check(fn, st)
    return o


def lizard_attn_fwd_train(q, k, v, meta_k, *, log_g=None, gate_logit=None, window: int, alpha: float,
                          softmax_scale: float = 0.0, chunk: int = 64, need_y_anchor: bool = False,
                          need_state: bool = False, out: Optional[Dict] = None) -> Dict:
    """The forward pass of a training step: lizard_attn_fwd (log_g) or
    lizard_attn_fwd_logit (gate_logit) that also keeps the chunk-start states
    for lizard_attn_bwd_train.  Returns {"y", "lse", "chunk_states" [B, H,
    ceil(L/64), d, d] in q's dtype, and optionally "y_anchor", "state"}."""
    torch = _torch()
    lib = load_library()
    if (log_g is None) == (gate_logit is None):
        raise ValueError("exactly one of log_g and gate_logit is required")
    _expect_seq_inputs(q, k, v, meta_k, log_g=log_g, gate_logit=gate_logit)
    B, H, L, d = q.shape
    m = meta_k.shape[1] if meta_k is not None else 0
    p = make_params(B, H, L, d, window=window, n_meta=m, alpha=alpha, dtype=_dtype_code(q), chunk=chunk,
                    softmax_scale=softmax_scale)
    o = dict(out) if out is not None else {}
    if "y" not in o:
        o["y"] = torch.empty_like(q)
    if "lse" not in o:
        o["lse"] = torch.empty((B, H, L), device=q.device, dtype=torch.float32)
    if "chunk_states" not in o:
        o["chunk_states"] = torch.empty((B, H, (L + 63) // 64, d, d), device=q.device, dtype=q.dtype)
    if need_y_anchor and "y_anchor" not in o:
        o["y_anchor"] = torch.empty_like(q)
    if need_state and "state" not in o:
        o["state"] = torch.empty((B, H, d, d), device=q.device, dtype=torch.float32)
    _expect_fwd_out(o, q)
    _expect("chunk_states", o["chunk_states"], (B, H, (L + 63) // 64, d, d), q.dtype, q.device)
    st = lib.lizard_attn_fwd_train(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(log_g), _ptr(gate_logit),
                                   _ptr(meta_k), _ptr(o["y"]), _ptr(o["lse"]), _ptr(o.get("y_anchor")),
                                   _ptr(o.get("state")), _ptr(o["chunk_states"]), _stream(q.device))
    _check("lizard_attn_fwd_train", st)
    return o


def lizard_attn_bwd_train(q, k, v, meta_k, lse, chunk_states, dy, *, log_g=None, gate_logit=None, window: int,
                          alpha: float, softmax_scale: float = 0.0, chunk: int = 64, workspace=None,
                          out: Optional[Dict] = None) -> Dict:
    """lizard_attn_bwd (log_g) or lizard_attn_bwd_logit (gate_logit) reading
    the chunk-start states lizard_attn_fwd_train kept.  Returns {"dq", "dk",
    "dv", "dlog_g" or "dgate_logit", "dmeta"}."""
    torch = _torch()
    lib = load_library()
    if (log_g is None) == (gate_logit is None):
        raise ValueError("exactly one of log_g and gate_logit is required")
    _expect_seq_inputs(q, k, v, meta_k, log_g=log_g, gate_logit=gate_logit)
    if lse is None or dy is None or chunk_states is None:
        raise ValueError("lse, chunk_states and dy are required")
    B, H, L, d = q.shape
    _expect("chunk_states", chunk_states, (B, H, (L + 63) // 64, d, d), q.dtype, q.device)
    m = meta_k.shape[1] if meta_k is not None else 0
    p = make_params(B, H, L, d, window=window, n_meta=m, alpha=alpha, dtype=_dtype_code(q), chunk=chunk,
                    softmax_scale=softmax_scale)
    ws_bytes = int(lib.lizard_attn_bwd_workspace_size(ctypes.byref(p)))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), device=q.device, dtype=torch.uint8)
    gate = gate_logit if gate_logit is not None else log_g
    gkey = "dgate_logit" if gate_logit is not None else "dlog_g"
    o = dict(out) if out is not None else {}
    for key, like in (("dq", q), ("dk", k), ("dv", v)):
        if key not in o:
            o[key] = torch.empty_like(like)
    if gkey not in o:
        o[gkey] = torch.empty_like(gate)
    if "dmeta" not in o:
        o["dmeta"] = torch.empty((H, m, d), device=q.device, dtype=torch.float32) if m > 0 else None
    _expect_bwd(q, meta_k, lse, dy, o, gkey, gate, workspace, ws_bytes)
    st = lib.lizard_attn_bwd_train(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(log_g), _ptr(gate_logit),
                                   _ptr(meta_k), _ptr(lse), _ptr(chunk_states), _ptr(dy), _ptr(o["dq"]),
                                   _ptr(o["dk"]), _ptr(o["dv"]), _ptr(o[gkey]), _ptr(o["dmeta"]), _ptr(workspace),
                                   workspace.numel(), _stream(q.device))
    _check("lizard_attn_bwd_train", st)
    return o


def lizard_decode_step(pos: int, q_t, k_t, v_t, log_g_t, meta_k, state, k_ring, v_ring, *, alpha: float,
                       softmax_scale: float = 0.0, y_t=None):
    """One decode step at absolute position ``pos`` (same for every row).
    q_t, k_t, v_t: [B, H, d]; log_g_t: [B, H, d] float32; state:
    [B, H, d, d] float32 (in-out); rings: [B, H, w, d] (in-out).  Returns y_t."""
    return _decode("lizard_decode_step", pos, q_t, k_t, v_t, log_g_t, meta_k, state, k_ring, v_ring, alpha,
                   softmax_scale, y_t)


def lizard_decode_step_logit(pos: int, q_t, k_t, v_t, gate_logit_t, meta_k, state, k_ring, v_ring, *,
                             alpha: float, softmax_scale: float = 0.0, y_t=None):
    """lizard_decode_step with the token's gates given by their logits
    (gate_logit_t: [B, H, d] in q's dtype)."""
    return _decode("lizard_decode_step_logit", pos, q_t, k_t, v_t, gate_logit_t, meta_k, state, k_ring, v_ring,
                   alpha, softmax_scale, y_t)


def _decode(fn, pos, q_t, k_t, v_t, gate, meta_k, state, k_ring, v_ring, alpha, softmax_scale, y_t):
    torch = _torch()
    lib = load_library()
    _dtype_code(q_t)
    if q_t.dim() != 3:
        raise ValueError(f"q_t: expected [B, H, d], got shape {tuple(q_t.shape)}")
    B, H, d = q_t.shape
    _expect_decode(fn, q_t, k_t, v_t, gate, meta_k, state, k_ring, v_ring, y_t)
    w = k_ring.shape[2]
    m = meta_k.shape[1] if meta_k is not None else 0
    p = make_params(B, H, 0, d, window=w, n_meta=m, alpha=alpha, dtype=_dtype_code(q_t),
                    softmax_scale=softmax_scale)
    if y_t is None:
        y_t = torch.empty_like(q_t)
    st = getattr(lib, fn)(ctypes.byref(p), int(pos), _ptr(q_t), _ptr(k_t), _ptr(v_t), _ptr(gate),
                          _ptr(meta_k), _ptr(state), _ptr(k_ring), _ptr(v_ring), _ptr(y_t),
                          _stream(q_t.device))
    _check(fn, st)
    return y_t


def _expect_decode(fn, q, k, v, gate, meta_k, state, k_ring, v_ring, y):
    """Decode arguments: k, v, y like q ([B, H, d] or [B, H, T, d]); the
    gates float32 (log-gates) or q's dtype (logits) in q's shape; state
    float32 [B, H, d, d]; rings [B, H, w, d] in q's dtype; meta_k [H, m, d]."""
    torch = _torch()
    B, H, d = q.shape[0], q.shape[1], q.shape[-1]
    for name, t in (("k", k), ("v", v), ("gates", gate), ("state", state), ("k_ring", k_ring), ("v_ring", v_ring)):
        if t is None:
            raise ValueError(f"{name} is required")
    _expect("k", k, q.shape, q.dtype, q.device)
    _expect("v", v, q.shape, q.dtype, q.device)
    _expect("gates", gate, q.shape, q.dtype if fn.endswith("_logit") else torch.float32, q.device)
    _expect("state", state, (B, H, d, d), torch.float32, q.device)
    if k_ring.dim() != 4:
        raise ValueError(f"k_ring: expected [B, H, w, d], got shape {tuple(k_ring.shape)}")
    _expect("k_ring", k_ring, (B, H, k_ring.shape[2], d), q.dtype, q.device)
    _expect("v_ring", v_ring, k_ring.shape, q.dtype, q.device)
    _expect("y", y, q.shape, q.dtype, q.device)
    if meta_k is not None:
        if meta_k.dim() != 3:
            raise ValueError(f"meta_k: expected [H, m, d], got shape {tuple(meta_k.shape)}")
        _expect("meta_k", meta_k, (H, meta_k.shape[1], d), q.dtype, q.device)


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def lizard_decode_tokens(pos, q, k, v, log_g, meta_k, state, k_ring, v_ring, *, alpha: float,
                         softmax_scale: float = 0.0, y=None):
    """Serving decode: T new tokens per row, each row at its own position.
    pos: [B] int64 on the GPU (negative = row inactive); q, k, v: [B, H, T, d];
    log_g: [B, H, T, d] float32; state / rings as lizard_decode_step.
    Returns y [B, H, T, d]."""
    return _decode_tokens("lizard_decode_tokens", pos, q, k, v, log_g, meta_k, state, k_ring, v_ring, alpha,
                          softmax_scale, y)


def lizard_decode_tokens_logit(pos, q, k, v, gate_logit, meta_k, state, k_ring, v_ring, *, alpha: float,
                               softmax_scale: float = 0.0, y=None):
    """lizard_decode_tokens with the gates given by their logits (q's dtype)."""
    return _decode_tokens("lizard_decode_tokens_logit", pos, q, k, v, gate_logit, meta_k, state, k_ring, v_ring,
                          alpha, softmax_scale, y)


def _decode_tokens(fn, pos, q, k, v, gate, meta_k, state, k_ring, v_ring, alpha, softmax_scale, y):
    torch = _torch()
    lib = load_library()
    _dtype_code(q)
    if q.dim() != 4:
        raise ValueError(f"q: expected [B, H, T, d], got shape {tuple(q.shape)}")
    B, H, T, d = q.shape
    _expect_decode(fn, q, k, v, gate, meta_k, state, k_ring, v_ring, y)
    w = k_ring.shape[2]
    m = meta_k.shape[1] if meta_k is not None else 0
    if pos.dtype != torch.int64 or tuple(pos.shape) != (B,) or pos.device != q.device:
        raise ValueError(f"pos must be an int64 tensor of shape [B] on {q.device}")
    p = make_params(B, H, 0, d, window=w, n_meta=m, alpha=alpha, dtype=_dtype_code(q), softmax_scale=softmax_scale)
    if y is None:
        y = torch.empty_like(q)
    st = getattr(lib, fn)(ctypes.byref(p), _ptr(pos), int(T), _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(meta_k),
                          _ptr(state), _ptr(k_ring), _ptr(v_ring), _ptr(y), _stream(q.device))
    _check(fn, st)
    return y


def _expect_continue(q, k, v, meta_k, log_g, gate_logit, state_in, k_halo, v_halo):
    """A continued segment: one of log_g / gate_logit, state_in float32
    [B, H, d, d], k_halo and v_halo [B, H, h, d] in q's dtype (both or none)."""
    torch = _torch()
    if (log_g is None) == (gate_logit is None):
        raise ValueError("exactly one of log_g and gate_logit is required")
    _expect_seq_inputs(q, k, v, meta_k, log_g=log_g, gate_logit=gate_logit)
    B, H, L, d = q.shape
    _expect("state_in", state_in, (B, H, d, d), torch.float32, q.device)
    if (k_halo is None) != (v_halo is None):
        raise ValueError("k_halo and v_halo go together")
    if k_halo is not None:
        if k_halo.dim() != 4:
            raise ValueError(f"k_halo: expected [B, H, h, d], got shape {tuple(k_halo.shape)}")
        _expect("k_halo", k_halo, (B, H, k_halo.shape[2], d), q.dtype, q.device)
        _expect("v_halo", v_halo, k_halo.shape, q.dtype, q.device)


def lizard_attn_fwd_continue(q, k, v, meta_k, *, log_g=None, gate_logit=None, state_in=None, k_halo=None,
                             v_halo=None, window: int, alpha: float, softmax_scale: float = 0.0, chunk: int = 64,
                             need_lse: bool = False, need_y_anchor: bool = False, need_state: bool = False,
                             out: Optional[Dict] = None) -> Dict:
    """Forward pass of a segment that continues a sequence: state_in [B, H, d, d]
    float32 (the previous segment's state), k_halo / v_halo [B, H, h, d] (the
    previous h <= window - 1 tokens).  Gates as log_g (float32) or gate_logit."""
    torch = _torch()
    lib = load_library()
    _expect_continue(q, k, v, meta_k, log_g, gate_logit, state_in, k_halo, v_halo)
    B, H, L, d = q.shape
    m = meta_k.shape[1] if meta_k is not None else 0
    hl = 0 if k_halo is None else int(k_halo.shape[2])
    p = make_params(B, H, L, d, window=window, n_meta=m, alpha=alpha, dtype=_dtype_code(q), chunk=chunk,
                    softmax_scale=softmax_scale)
    o = dict(out) if out is not None else {}
    if "y" not in o:
        o["y"] = torch.empty_like(q)
    if need_lse and "lse" not in o:
        o["lse"] = torch.empty((B, H, L), device=q.device, dtype=torch.float32)
    if need_y_anchor and "y_anchor" not in o:
        o["y_anchor"] = torch.empty_like(q)
    if need_state and "state" not in o:
        o["state"] = torch.empty((B, H, d, d), device=q.device, dtype=torch.float32)
    _expect_fwd_out(o, q)
    st = lib.lizard_attn_fwd_continue(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(log_g), _ptr(gate_logit),
                                      _ptr(meta_k), _ptr(state_in), _ptr(k_halo), _ptr(v_halo), hl, _ptr(o["y"]),
                                      _ptr(o.get("lse")), _ptr(o.get("y_anchor")), _ptr(o.get("state")),
                                      _stream(q.device))
    _check("lizard_attn_fwd_continue", st)
    return o


def lizard_attn_fwd_split(q, k, v, meta_k, *, log_g=None, gate_logit=None, state_in=None, k_halo=None,
                          v_halo=None, window: int, alpha: float, softmax_scale: float = 0.0, chunk: int = 64,
                          need_lse: bool = False, need_y_anchor: bool = False, need_state: bool = False,
                          workspace=None, out: Optional[Dict] = None) -> Dict:
    """lizard_attn_fwd_continue with long sequences cut into segments that run
    side by side (few heads, long L).  workspace: a uint8 device tensor of at
    least lizard_attn_fwd_split_workspace_size bytes (allocated when None)."""
    torch = _torch()
    lib = load_library()
    _expect_continue(q, k, v, meta_k, log_g, gate_logit, state_in, k_halo, v_halo)
    B, H, L, d = q.shape
    m = meta_k.shape[1] if meta_k is not None else 0
    hl = 0 if k_halo is None else int(k_halo.shape[2])
    p = make_params(B, H, L, d, window=window, n_meta=m, alpha=alpha, dtype=_dtype_code(q), chunk=chunk,
                    softmax_scale=softmax_scale)
    need = lib.lizard_attn_fwd_split_workspace_size(ctypes.byref(p))
    if workspace is None and need > 0:
        workspace = torch.empty(need, device=q.device, dtype=torch.uint8)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    o = dict(out) if out is not None else {}
    if "y" not in o:
        o["y"] = torch.empty_like(q)
    if need_lse and "lse" not in o:
        o["lse"] = torch.empty((B, H, L), device=q.device, dtype=torch.float32)
    if need_y_anchor and "y_anchor" not in o:
        o["y_anchor"] = torch.empty_like(q)
    if need_state and "state" not in o:
        o["state"] = torch.empty((B, H, d, d), device=q.device, dtype=torch.float32)
    _expect_fwd_out(o, q)
    if workspace is not None and (workspace.dtype != torch.uint8 or workspace.device != q.device):
        raise ValueError(f"workspace: a uint8 tensor on {q.device} is required")
    st = lib.lizard_attn_fwd_split(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(log_g), _ptr(gate_logit),
                                   _ptr(meta_k), _ptr(state_in), _ptr(k_halo), _ptr(v_halo), hl, _ptr(o["y"]),
                                   _ptr(o.get("lse")), _ptr(o.get("y_anchor")), _ptr(o.get("state")), _ptr(workspace),
                                   ws_bytes, _stream(q.device))
    _check("lizard_attn_fwd_split", st)
    return o


def lizard_attn_fwd_split_noalloc(q, k, v, meta_k, *, log_g=None, gate_logit=None, state_in=None, k_halo=None,
                                  v_halo=None, window: int, alpha: float, softmax_scale: float = 0.0, chunk: int = 64,
                                  need_lse: bool = False, need_y_anchor: bool = False, need_state: bool = False,
                                  out: Optional[Dict] = None) -> Dict:
    """lizard_attn_fwd_split with its workspace in the library's fixed scratch
    (NOALLOC_SCRATCH_BYTES per GPU): no workspace argument and no allocation by
    the library.  Pass every output in ``out`` for a call that allocates
    nothing at all (missing outputs are allocated here, as in the other
    calls).  Calls that may overlap on one GPU share the scratch and must be
    ordered by the caller."""
    torch = _torch()
    lib = load_library()
    _expect_continue(q, k, v, meta_k, log_g, gate_logit, state_in, k_halo, v_halo)
    B, H, L, d = q.shape
    m = meta_k.shape[1] if meta_k is not None else 0
    hl = 0 if k_halo is None else int(k_halo.shape[2])
    p = make_params(B, H, L, d, window=window, n_meta=m, alpha=alpha, dtype=_dtype_code(q), chunk=chunk,
                    softmax_scale=softmax_scale)
    o = dict(out) if out is not None else {}
    if "y" not in o:
        o["y"] = torch.empty_like(q)
    if need_lse and "lse" not in o:
        o["lse"] = torch.empty((B, H, L), device=q.device, dtype=torch.float32)
    if need_y_anchor and "y_anchor" not in o:
        o["y_anchor"] = torch.empty_like(q)
    if need_state and "state" not in o:
        o["state"] = torch.empty((B, H, d, d), device=q.device, dtype=torch.float32)
    _expect_fwd_out(o, q)
    st = lib.lizard_attn_fwd_split_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(log_g), _ptr(gate_logit),
                                           _ptr(meta_k), _ptr(state_in), _ptr(k_halo), _ptr(v_halo), hl, _ptr(o["y"]),
                                           _ptr(o.get("lse")), _ptr(o.get("y_anchor")), _ptr(o.get("state")),
                                           _stream(q.device))
    _check("lizard_attn_fwd_split_noalloc", st)
    return o


NOALLOC_SCRATCH_BYTES = 64 << 20   # LIZARD_NOALLOC_SCRATCH_BYTES of include/lizard_attn.h


def lizard_attn_fwd_split_workspace_size(B: int, H: int, L: int, d: int, *, dtype_code: int = 1,
                                         window: int = 64, n_meta: int = 0) -> int:
    """Workspace bytes lizard_attn_fwd_split needs (0: it runs as one pass)."""
    lib = load_library()
    p = make_params(B, H, L, d, window=window, n_meta=n_meta, alpha=0.0, dtype=dtype_code)
    return int(lib.lizard_attn_fwd_split_workspace_size(ctypes.byref(p)))


def lizard_softmax_attn_fwd(q, k, v, *, softmax_scale: float = 0.0, need_lse: bool = False,
                            out: Optional[Dict] = None) -> Dict:
    """Causal softmax attention over all earlier tokens (the stage-1 teacher).
    Returns {"y", and optionally "lse"}."""
    torch = _torch()
    lib = load_library()
    _expect_seq_inputs(q, k, v, None)
    B, H, L, d = q.shape
    p = make_params(B, H, L, d, window=1, n_meta=0, alpha=0.0, dtype=_dtype_code(q), softmax_scale=softmax_scale)
    o = dict(out) if out is not None else {}
    if "y" not in o:
        o["y"] = torch.empty_like(q)
    if need_lse and "lse" not in o:
        o["lse"] = torch.empty((B, H, L), device=q.device, dtype=torch.float32)
    _expect_fwd_out(o, q)
    st = lib.lizard_softmax_attn_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o["y"]), _ptr(o.get("lse")),
                                     _stream(q.device))
    _check("lizard_softmax_attn_fwd", st)
    return o


def lizard_transfer_loss(y, y_teacher, *, dy=None, loss_bh=None):
    """mean((y - y_teacher)^2): returns (dy = 2 (y - y_teacher) / N, loss_bh [B, H]
    float32 whose sum is the loss)."""
    torch = _torch()
    lib = load_library()
    _dtype_code(y)
    if y.dim() != 4:
        raise ValueError(f"y: expected [B, H, L, d], got shape {tuple(y.shape)}")
    B, H, L, d = y.shape
    _expect("y_teacher", y_teacher, y.shape, y.dtype, y.device)
    _expect("dy", dy, y.shape, y.dtype, y.device)
    _expect("loss_bh", loss_bh, (B, H), torch.float32, y.device)
    p = make_params(B, H, L, d, window=1, n_meta=0, alpha=0.0, dtype=_dtype_code(y))
    if dy is None:
        dy = torch.empty_like(y)
    if loss_bh is None:
        loss_bh = torch.empty((B, H), device=y.device, dtype=torch.float32)
    st = lib.lizard_transfer_loss(ctypes.byref(p), _ptr(y), _ptr(y_teacher), _ptr(dy), _ptr(loss_bh),
                                  _stream(y.device))
    _check("lizard_transfer_loss", st)
    return dy, loss_bh

"""Helpers for the GPU parity tests: upload seeded float64 inputs in their
storage precision, download results as float64, and the tolerance rule
max|err| <= tau * max|ref| (tau = 1e-4 for float32, 2e-2 for bfloat16)."""
from __future__ import annotations

import sys

import numpy as np

import seeded_inputs as si

TAU = {"f32": 1e-4, "bf16": 2e-2}


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def up(x: np.ndarray, dtype: str):
    """float64 numpy -> torch tensor on cuda:0 in the storage dtype."""
    import torch

    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    if dtype == "bf16":
        bits = si.round_bf16_bits(x)
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    raise ValueError(dtype)


def up_f32(x: np.ndarray):
    import torch

    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def down(t) -> np.ndarray:
    import torch

    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    return float(np.abs(got - ref).max() / max(1e-30, np.abs(ref).max()))


def assert_close(got, ref, dtype: str, what: str, tau=None):
    tau = TAU[dtype] if tau is None else tau
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    e = rel_err(got, ref)
    assert e <= tau, f"{what}: max|err|/max|ref| = {e:.3e} > {tau:.0e}"
    return e


def flat(a: np.ndarray) -> np.ndarray:
    """[B, H, ...] -> [B*H, ...]"""
    return a.reshape(a.shape[0] * a.shape[1], *a.shape[2:])


def meta_per_slice(meta: np.ndarray, B: int) -> np.ndarray:
    """[H, m, d] -> [B*H, m, d] (the same sink keys for every batch row)."""
    return np.broadcast_to(meta[None], (B,) + meta.shape).reshape(B * meta.shape[0], *meta.shape[1:])


def up_storage(a: np.ndarray):
    """Storage-form numpy array (uint16 bfloat16 bits or float32) -> cuda tensor."""
    import torch

    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def upload_workload(w, L=None, with_dy=False, with_logit=False):
    """All inputs of a workload on the GPU (generated per slice, in parallel)."""
    st = si.storage_inputs(w, L=L, with_dy=with_dy, with_logit=with_logit)
    return {k: up_storage(v) for k, v in st.items()}


# ---------------------------------------------------------------------------
# Poisoned, canary-guarded outputs
# ---------------------------------------------------------------------------

CANARY = 4096          # elements after every output buffer
_INT_VIEW = {"torch.bfloat16": "int16", "torch.float16": "int16", "torch.float32": "int32", "torch.int64": "int64",
             "torch.uint8": "uint8"}


class PoisonedLib:
    """The Python binding with every output buffer the binding would
    allocate allocated here instead: filled with NaN (so an element a kernel
    never writes fails the finiteness check of every comparison and every
    bitwise repeat) and followed by CANARY elements of a finite sentinel (so
    a write past the end of an output changes them).  Workspaces are filled
    with 0xff bytes (NaN in both float types), since the library must not
    depend on their contents.  Outputs a test passes itself are left as
    given.  check_canaries() synchronises and compares every tail bit for
    bit; the conftest runs it after each test."""

    def __init__(self, sqa):
        self._sqa = sqa
        self._guards = []

    def __getattr__(self, name):
        return getattr(self._sqa, name)

    # -- allocation --
    def _buf(self, shape, dtype, fill=float("nan")):
        import torch

        n = 1
        for s in shape:
            n *= int(s)
        base = torch.full((n + CANARY,), fill, device="cuda", dtype=dtype)
        base[n:] = -77.0 if dtype.is_floating_point else 77
        self._guards.append((base, n, base[n:].clone()))
        return base[:n].view(*shape)

    def _ws(self, nbytes):
        import torch

        base = torch.full((max(int(nbytes), 16) + CANARY,), 255, device="cuda", dtype=torch.uint8)
        self._guards.append((base, max(int(nbytes), 16), base[max(int(nbytes), 16):].clone()))
        return base[:max(int(nbytes), 16)]

    def check_canaries(self):
        import torch

        if not self._guards:
            return
        torch.cuda.synchronize()
        bad = []
        for base, n, ref in self._guards:
            iv = getattr(torch, _INT_VIEW[str(base.dtype)])
            if not torch.equal(base[n:].view(iv), ref.view(iv)):
                bad.append((tuple(base.shape), str(base.dtype), n))
        self._guards.clear()
        assert not bad, f"writes past the end of an output buffer: {bad}"

    # -- forward family --
    def _fwd_out(self, q, out, lse=False, y_anchor=False, state=False, chunk_states=False):
        import torch

        B, H, L, d = q.shape
        o = dict(out) if out is not None else {}
        if "y" not in o:
            o["y"] = self._buf((B, H, L, d), q.dtype)
        if lse and "lse" not in o:
            o["lse"] = self._buf((B, H, L), torch.float32)
        if y_anchor and "y_anchor" not in o:
            o["y_anchor"] = self._buf((B, H, L, d), q.dtype)
        if state and "state" not in o:
            o["state"] = self._buf((B, H, d, d), torch.float32)
        if chunk_states and "chunk_states" not in o:
            o["chunk_states"] = self._buf((B, H, (L + 63) // 64, d, d), q.dtype)
        return o

    def _call_fwd(self, name, q, args, kw, chunk_states=False):
        kw = dict(kw)
        kw["out"] = self._fwd_out(q, kw.get("out"), kw.get("need_lse", False) or chunk_states,
                                  kw.get("need_y_anchor", False), kw.get("need_state", False), chunk_states)
        return getattr(self._sqa, name)(q, *args, **kw)

    def lizard_attn_fwd(self, q, *args, **kw):
        return self._call_fwd("lizard_attn_fwd", q, args, kw)

    def lizard_attn_fwd_logit(self, q, *args, **kw):
        return self._call_fwd("lizard_attn_fwd_logit", q, args, kw)

    def lizard_attn_fwd_continue(self, q, *args, **kw):
        return self._call_fwd("lizard_attn_fwd_continue", q, args, kw)

    def lizard_attn_fwd_split(self, q, k, v, meta_k, **kw):
        if kw.get("workspace") is None:
            B, H, L, d = q.shape
            m = 0 if meta_k is None else int(meta_k.shape[1])
            need = self._sqa.lizard_attn_fwd_split_workspace_size(
                B, H, L, d, dtype_code=self._sqa._dtype_code(q), window=kw["window"], n_meta=m)
            if need > 0:
                kw["workspace"] = self._ws(need)
        return self._call_fwd("lizard_attn_fwd_split", q, (k, v, meta_k), kw)

    def lizard_attn_fwd_train(self, q, *args, **kw):
        return self._call_fwd("lizard_attn_fwd_train", q, args, kw, chunk_states=True)

    def lizard_softmax_attn_fwd(self, q, *args, **kw):
        return self._call_fwd("lizard_softmax_attn_fwd", q, args, kw)

    # -- backward family --
    def _bwd_out(self, q, k, v, gate, gkey, meta_k, out):
        import torch

        o = dict(out) if out is not None else {}
        for key, like in (("dq", q), ("dk", k), ("dv", v), (gkey, gate)):
            if key not in o:
                o[key] = self._buf(tuple(like.shape), like.dtype)
        if "dmeta" not in o and meta_k is not None and meta_k.shape[1] > 0:
            o["dmeta"] = self._buf(tuple(meta_k.shape), torch.float32)
        return o

    def _bwd_ws(self, q, meta_k, window, kw):
        if kw.get("workspace") is None:
            B, H, L, d = q.shape
            m = 0 if meta_k is None else int(meta_k.shape[1])
            kw["workspace"] = self._ws(self._sqa.lizard_attn_bwd_workspace_size(
                B, H, L, d, window=window, n_meta=m, dtype=self._sqa._dtype_code(q)))

    def lizard_attn_bwd(self, q, k, v, log_g, meta_k, lse, dy, **kw):
        kw["out"] = self._bwd_out(q, k, v, log_g, "dlog_g", meta_k, kw.get("out"))
        self._bwd_ws(q, meta_k, kw["window"], kw)
        return self._sqa.lizard_attn_bwd(q, k, v, log_g, meta_k, lse, dy, **kw)

    def lizard_attn_bwd_logit(self, q, k, v, gate_logit, meta_k, lse, dy, **kw):
        kw["out"] = self._bwd_out(q, k, v, gate_logit, "dgate_logit", meta_k, kw.get("out"))
        self._bwd_ws(q, meta_k, kw["window"], kw)
        return self._sqa.lizard_attn_bwd_logit(q, k, v, gate_logit, meta_k, lse, dy, **kw)

    def lizard_attn_bwd_train(self, q, k, v, meta_k, lse, chunk_states, dy, **kw):
        logit = kw.get("gate_logit") is not None
        gate = kw["gate_logit"] if logit else kw["log_g"]
        kw["out"] = self._bwd_out(q, k, v, gate, "dgate_logit" if logit else "dlog_g", meta_k, kw.get("out"))
        self._bwd_ws(q, meta_k, kw["window"], kw)
        return self._sqa.lizard_attn_bwd_train(q, k, v, meta_k, lse, chunk_states, dy, **kw)

    # -- decode family --
    def lizard_decode_step(self, pos, q_t, *args, **kw):
        if kw.get("y_t") is None:
            kw["y_t"] = self._buf(tuple(q_t.shape), q_t.dtype)
        return self._sqa.lizard_decode_step(pos, q_t, *args, **kw)

    def lizard_decode_step_logit(self, pos, q_t, *args, **kw):
        if kw.get("y_t") is None:
            kw["y_t"] = self._buf(tuple(q_t.shape), q_t.dtype)
        return self._sqa.lizard_decode_step_logit(pos, q_t, *args, **kw)

    def lizard_decode_tokens(self, pos, q, *args, **kw):
        if kw.get("y") is None:
            kw["y"] = self._buf(tuple(q.shape), q.dtype)
        return self._sqa.lizard_decode_tokens(pos, q, *args, **kw)

    def lizard_decode_tokens_logit(self, pos, q, *args, **kw):
        if kw.get("y") is None:
            kw["y"] = self._buf(tuple(q.shape), q.dtype)
        return self._sqa.lizard_decode_tokens_logit(pos, q, *args, **kw)

    # -- stage 1 --
    def lizard_transfer_loss(self, y, y_teacher, *, dy=None, loss_bh=None):
        import torch

        if dy is None:
            dy = self._buf(tuple(y.shape), y.dtype)
        if loss_bh is None:
            loss_bh = self._buf(tuple(y.shape[:2]), torch.float32)
        return self._sqa.lizard_transfer_loss(y, y_teacher, dy=dy, loss_bh=loss_bh)

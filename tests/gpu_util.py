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

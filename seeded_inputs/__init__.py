"""Seeded synthetic inputs for the Lizard hybrid attention layer.

This module is shared by the tests, the benchmark and the oracle's callers.
It draws random numbers and rounds them to the storage precision; it holds
none of the layer's arithmetic.  Every (config, tensor, batch, head) slice
has its own counter-keyed stream
``PCG64(SeedSequence(ROOT_SEED, spawn_key=(cfg, tensor, b, h)))`` so any
slice can be regenerated alone, which is how the oracle checks sampled heads
of the large workloads.

Distributions (the workloads of the Lizard layer on LLaMA-3-8B-shaped
attention, H=32 and d=128; "Lizard: An Efficient Linearization Framework for
Large Language Models", gist.science, section 4 "Ergebnisse"):

* q, k, v ~ N(0, 1) / 8
* gate logits ~ N(mu_g, sd_g) per token per key dim, and the log-gate handed
  to the layer is log(sigmoid(logit)), computed in float64 and rounded once
  to float32 (the gate is a sigmoid of a learned projection; same page,
  section 2, "Kernkomponenten", item 1).  The entry points that take the
  logits themselves get the same draws rounded to the storage dtype
  ("gate_logit").
* meta-memory sink keys ~ N(0, 1) / 8, one set per head
* upstream gradient dY ~ N(0, 1)

Tensors in bfloat16 are rounded from float64 to the nearest bfloat16 with
ties to even, once; the float64 widening of those bits is what the oracle
consumes.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Sequence

import numpy as np

ROOT_SEED = 250709025

# tensor ids in the spawn key
T_Q, T_K, T_V, T_GATE, T_META, T_DY = 0, 1, 2, 3, 4, 5


@dataclasses.dataclass(frozen=True)
class Workload:
    """Sizes and input distributions of one workload."""

    name: str
    cfg_id: int
    dtype: str  # "f32" or "bf16"
    B: int
    H: int
    L: int
    d: int
    chunk: int = 64
    window: int = 64
    n_meta: int = 4
    alpha: float = 0.5
    gate_mu: float = 3.0
    gate_sd: float = 1.0
    qkv_sd: float = 0.125
    meta_sd: float = 0.125
    steps: int = 0  # decode steps after an L-token prefill


# Workload table.  The first is the small case the oracle finishes in
# seconds; the second is the Llama-3-8B-shaped prefill layer the benchmark
# times; then long-context prefill, decode and the training backward.
WORKLOADS: Dict[str, Workload] = {
    "tiny_fwd_f32": Workload("tiny_fwd_f32", 0, "f32", B=1, H=2, L=256, d=64),
    "llama3_8b_prefill_bf16": Workload("llama3_8b_prefill_bf16", 1, "bf16", B=4, H=32, L=4096, d=128),
    "long_ctx_32k_bf16": Workload("long_ctx_32k_bf16", 2, "bf16", B=1, H=32, L=32768, d=128,
                                  gate_mu=2.0, gate_sd=2.0),
    "decode_b64_bf16": Workload("decode_b64_bf16", 3, "bf16", B=64, H=32, L=2048, d=128, steps=1024),
    "train_bwd_bf16": Workload("train_bwd_bf16", 4, "bf16", B=8, H=32, L=2048, d=128),
    # the prefill at d=64 in both operand types (the fp32 build of the forward
    # kernel exists at d=64 only): the bf16-vs-fp32 ablation
    "prefill_d64_bf16": Workload("prefill_d64_bf16", 5, "bf16", B=4, H=32, L=4096, d=64),
    "prefill_d64_f32": Workload("prefill_d64_f32", 6, "f32", B=4, H=32, L=4096, d=64),
    # the training step (forward keeping lse and the chunk states, then the
    # backward) on the backward's shapes at d=64 in both operand types: the
    # ablation of the pages' training-throughput claim
    "train_d64_bf16": Workload("train_d64_bf16", 7, "bf16", B=8, H=32, L=2048, d=64),
    "train_d64_f32": Workload("train_d64_f32", 8, "f32", B=8, H=32, L=2048, d=64),
}


def _rng(cfg: int, tensor: int, b: int, h: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(ROOT_SEED, spawn_key=(cfg, tensor, b, h))))


def round_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64/float32 values to bfloat16 (nearest, ties to even).

    Returns the 16-bit patterns as uint16.  Values are first rounded to
    float32 (exact for the distributions used here up to one float32 ulp,
    far below bfloat16 resolution), then the low 16 bits are rounded away.
    """
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to the storage dtype and widen back to float64."""
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(round_bf16_bits(x))
    raise ValueError(dtype)


def _log_sigmoid(x: np.ndarray) -> np.ndarray:
    # log(1/(1+e^{-x})) without overflow for large |x|
    return -np.logaddexp(0.0, -x)


def slice_inputs(w: Workload, b: int, h: int, L: Optional[int] = None, with_dy: bool = False) -> Dict[str, np.ndarray]:
    """Float64 values (already rounded to storage precision) of one (b, h) slice.

    Returns q, k, v [L, d], log_g [L, d] (float32 values), gate_logit
    [L, d] (the same draws in the storage dtype), and dy [L, d] if
    requested.  ``L`` defaults to the workload's length (for decode
    workloads: prefill length + steps).
    """
    if L is None:
        L = w.L + w.steps
    d = w.d
    out = {}
    for name, tid in (("q", T_Q), ("k", T_K), ("v", T_V)):
        out[name] = round_to(_rng(w.cfg_id, tid, b, h).standard_normal((L, d)) * w.qkv_sd, w.dtype)
    logits = _rng(w.cfg_id, T_GATE, b, h).normal(w.gate_mu, w.gate_sd, size=(L, d))
    out["log_g"] = _log_sigmoid(logits).astype(np.float32).astype(np.float64)
    out["gate_logit"] = round_to(logits, w.dtype)
    if with_dy:
        out["dy"] = round_to(_rng(w.cfg_id, T_DY, b, h).standard_normal((L, d)), w.dtype)
    return out


def meta_keys(w: Workload, h: int) -> np.ndarray:
    """Meta-memory sink keys of head h: [m, d] float64 (rounded)."""
    return round_to(_rng(w.cfg_id, T_META, 0, h).standard_normal((w.n_meta, w.d)) * w.meta_sd, w.dtype)


def full_inputs(w: Workload, L: Optional[int] = None, with_dy: bool = False,
                heads: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """Whole [B, H, L, d] inputs (float64 values) plus meta keys [H, m, d]."""
    if L is None:
        L = w.L + w.steps
    Hs = list(range(w.H)) if heads is None else list(heads)
    names = ["q", "k", "v", "log_g", "gate_logit"] + (["dy"] if with_dy else [])
    arrs = {n: np.empty((w.B, len(Hs), L, w.d), dtype=np.float64) for n in names}
    for b in range(w.B):
        for j, h in enumerate(Hs):
            s = slice_inputs(w, b, h, L=L, with_dy=with_dy)
            for n in names:
                arrs[n][b, j] = s[n]
    arrs["meta_k"] = np.stack([meta_keys(w, h) for h in Hs]) if w.n_meta > 0 else np.zeros((len(Hs), 0, w.d))
    return arrs


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array for upload: float32 array, or uint16 bfloat16 bit patterns."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return round_bf16_bits(x)
    raise ValueError(dtype)


def custom_inputs(seed: int, B: int, H: int, L: int, d: int, n_meta: int, dtype: str, *,
                  qk_sd: float = 0.125, v_sd: float = 0.125, meta_sd: float = 0.125,
                  gate_mu: float = 3.0, gate_sd: float = 1.0, hard_reset_frac: float = 0.0,
                  with_dy: bool = False) -> Dict[str, np.ndarray]:
    """Inputs for parity variants outside the fixed workloads (sharp logits,
    slow or hard-reset gates, ragged lengths).  Hard resets set the gate
    logit, and so log_g, to -1000 on a random fraction of tokens (all key
    dims of that token)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(ROOT_SEED, spawn_key=(1000 + seed,))))
    out = {
        "q": round_to(rng.standard_normal((B, H, L, d)) * qk_sd, dtype),
        "k": round_to(rng.standard_normal((B, H, L, d)) * qk_sd, dtype),
        "v": round_to(rng.standard_normal((B, H, L, d)) * v_sd, dtype),
    }
    logits = rng.normal(gate_mu, gate_sd, size=(B, H, L, d))
    if hard_reset_frac > 0:
        hit = rng.random((B, H, L)) < hard_reset_frac
        logits[hit] = -1000.0   # log sigmoid(-1000) = -1000 to double precision
    out["log_g"] = _log_sigmoid(logits).astype(np.float32).astype(np.float64)
    out["gate_logit"] = round_to(logits, dtype)
    out["meta_k"] = round_to(rng.standard_normal((H, n_meta, d)) * meta_sd, dtype)
    if with_dy:
        out["dy"] = round_to(rng.standard_normal((B, H, L, d)), dtype)
    return out


def _storage_row(args):
    w, b, L, with_dy = args
    rows = {}
    for h in range(w.H):
        s = slice_inputs(w, b, h, L=L, with_dy=with_dy)
        for n, a in s.items():
            st = np.ascontiguousarray(a, dtype=np.float32) if n == "log_g" else to_storage(a, w.dtype)
            rows.setdefault(n, []).append(st)
    return b, {n: np.stack(v) for n, v in rows.items()}


def storage_inputs(w: Workload, L: Optional[int] = None, with_dy: bool = False,
                   workers: Optional[int] = None, with_logit: bool = False) -> Dict[str, np.ndarray]:
    """Whole [B, H, L, d] inputs in storage form (uint16 bfloat16 bits or
    float32; log_g always float32), identical to the slices that
    ``slice_inputs`` returns, generated in parallel over batch rows."""
    import concurrent.futures
    import multiprocessing as mp
    import os

    if L is None:
        L = w.L + w.steps
    names = ["q", "k", "v", "log_g"] + (["dy"] if with_dy else []) + (["gate_logit"] if with_logit else [])
    sdt = np.uint16 if w.dtype == "bf16" else np.float32
    out = {n: np.empty((w.B, w.H, L, w.d), dtype=np.float32 if n == "log_g" else sdt) for n in names}
    if workers is None:
        workers = min(16, os.cpu_count() or 1, w.B)
    jobs = [(w, b, L, with_dy) for b in range(w.B)]
    if workers <= 1:
        results = map(_storage_row, jobs)
        for b, rows in results:
            for n in names:
                out[n][b] = rows[n]
    else:
        with concurrent.futures.ProcessPoolExecutor(workers, mp_context=mp.get_context("fork")) as ex:
            for b, rows in ex.map(_storage_row, jobs):
                for n in names:
                    out[n][b] = rows[n]
    meta = np.stack([meta_keys(w, h) for h in range(w.H)]) if w.n_meta > 0 else np.zeros((w.H, 0, w.d))
    out["meta_k"] = to_storage(meta, w.dtype)
    return out

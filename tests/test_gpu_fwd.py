"""GPU parity of lizard_attn_fwd against the float64 oracle."""
import math

import numpy as np
import pytest

import oracle
import seeded_inputs as si
from tests.gpu_util import assert_close, down, flat, log, meta_per_slice, up, up_f32, upload_workload

pytestmark = pytest.mark.gpu


def gpu_fwd(sqa, x, dtype, window, alpha, scale=0.0):
    m = x["meta_k"].shape[1]
    meta = up(x["meta_k"], dtype) if m > 0 else None
    out = sqa.lizard_attn_fwd(up(x["q"], dtype), up(x["k"], dtype), up(x["v"], dtype), up_f32(x["log_g"]), meta,
                              window=window, alpha=alpha, softmax_scale=scale, need_lse=True,
                              need_y_anchor=True, need_state=True)
    import torch

    torch.cuda.synchronize()
    return {k: down(v) for k, v in out.items()}


def ref_fwd(x, window, alpha, scale=None):
    B = x["q"].shape[0]
    o = oracle.lizard_fwd(flat(x["q"]), flat(x["k"]), flat(x["v"]), flat(x["log_g"]),
                          meta_per_slice(x["meta_k"], B), window, alpha, scale)
    shp = x["q"].shape
    return {"y": o["y"].reshape(shp), "y_anchor": o["y_anchor"].reshape(shp), "lse": o["lse"].reshape(shp[:3]),
            "state": o["state"].reshape(shp[0], shp[1], shp[3], shp[3])}


def compare(got, ref, dtype, tag):
    errs = {}
    for key in ("y", "y_anchor", "lse", "state"):
        errs[key] = assert_close(got[key], ref[key], dtype, f"{tag} {key}")
    log(f"{tag}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))


def test_tiny_workload_f32(gpu_lib):
    w = si.WORKLOADS["tiny_fwd_f32"]
    x = si.full_inputs(w)
    log("tiny_fwd_f32 B=1 H=2 L=256 d=64")
    compare(gpu_fwd(gpu_lib, x, "f32", w.window, w.alpha), ref_fwd(x, w.window, w.alpha), "f32", "tiny")


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 64), ("bf16", 128)])
@pytest.mark.parametrize("L", [1, 17, 64, 100, 200, 300])
def test_ragged_lengths(gpu_lib, dtype, d, L):
    x = si.custom_inputs(1, 2, 3, L, d, 4, dtype)
    log(f"ragged dtype={dtype} d={d} L={L}")
    compare(gpu_fwd(gpu_lib, x, dtype, 64, 0.5), ref_fwd(x, 64, 0.5), dtype, f"L={L}")


@pytest.mark.parametrize("window", [1, 2, 7, 33, 63, 64])
@pytest.mark.parametrize("n_meta", [0, 1, 16])
def test_window_and_sinks(gpu_lib, window, n_meta):
    # sharp logits so the anchor branch and its sinks carry weight
    x = si.custom_inputs(2, 1, 2, 160, 64, n_meta, "f32", qk_sd=1.0, meta_sd=1.0)
    log(f"window={window} n_meta={n_meta}")
    compare(gpu_fwd(gpu_lib, x, "f32", window, 0.5), ref_fwd(x, window, 0.5), "f32", f"w={window} m={n_meta}")


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128)])
@pytest.mark.parametrize("variant", ["sharp", "slow_gate", "fast_gate", "hard_reset", "outliers", "wide_chunk",
                                     "wide_blocks", "wide_mixed"])
def test_variants(gpu_lib, dtype, d, variant):
    # wide_chunk: chunk decay spans between one and two times the
    # factorisable limit (about 2^-121 over 64 tokens: the shifted reference
    # point); wide_blocks: spans beyond twice the limit (about 2^-280) while
    # every 16-token block's stays within it (blockwise factorisation);
    # wide_mixed: all kinds of chunk and block
    kw = {
        "sharp": dict(qk_sd=1.0, meta_sd=1.0),
        "slow_gate": dict(gate_mu=8.0, gate_sd=1.0),
        "fast_gate": dict(gate_mu=-2.0, gate_sd=4.0),
        "hard_reset": dict(hard_reset_frac=0.01, gate_mu=2.0, gate_sd=2.0),
        "wide_chunk": dict(gate_mu=-1.0, gate_sd=0.5),
        "wide_blocks": dict(gate_mu=-3.0, gate_sd=0.3),
        "wide_mixed": dict(gate_mu=0.0, gate_sd=3.0),
        "outliers": dict(),
    }[variant]
    x = si.custom_inputs(3, 2, 2, 256, d, 4, dtype, **kw)
    if variant == "outliers":
        # a few massive activations in q and k
        rng = np.random.default_rng(5)
        for key in ("q", "k"):
            idx = rng.integers(0, x[key].size, 40)
            x[key].flat[idx] *= 50.0
            x[key] = si.round_to(x[key], dtype)
    log(f"variant={variant} dtype={dtype} d={d}")
    compare(gpu_fwd(gpu_lib, x, dtype, 64, 0.5), ref_fwd(x, 64, 0.5), dtype, variant)


def test_hard_reset_everywhere(gpu_lib):
    """log g = -1000 on every token: every block takes the pairwise path and
    the gated branch reduces to (q_t . k_t) v_t."""
    x = si.custom_inputs(4, 1, 2, 130, 64, 2, "f32")
    x["log_g"][:] = -1000.0
    got = gpu_fwd(gpu_lib, x, "f32", 16, 0.0)
    ref = (x["q"] * x["k"]).sum(-1, keepdims=True) * x["v"]
    assert_close(got["y"], ref, "f32", "hard reset y")


def test_alpha_linearity(gpu_lib):
    x = si.custom_inputs(5, 1, 2, 192, 128, 4, "bf16", qk_sd=1.0, meta_sd=1.0)
    a0 = gpu_fwd(gpu_lib, x, "bf16", 64, 0.0)
    ref = ref_fwd(x, 64, 0.0)
    assert_close(a0["y"], ref["y"], "bf16", "alpha=0 y (gated branch alone)")
    assert_close(a0["y_anchor"], ref["y_anchor"], "bf16", "alpha=0 y_anchor")


def test_scale_parameter(gpu_lib):
    x = si.custom_inputs(6, 1, 2, 100, 64, 3, "f32", qk_sd=0.5, meta_sd=0.5)
    compare(gpu_fwd(gpu_lib, x, "f32", 20, 0.5, scale=0.3), ref_fwd(x, 20, 0.5, scale=0.3), "f32", "scale=0.3")


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128)])
def test_mask_probes_exact(gpu_lib, dtype, d):
    """Row b probes key position p = b: q = 1/sqrt(d), gate 1, mu = 0,
    k = v = 0 except k_p = 1/sqrt(d), v_p = e_0.  The zero / non-zero pattern of
    y_anchor must be exactly the window, that of y at alpha = 0 exactly t >= p."""
    L, w, m = 150, 37, 2
    B = L
    q = np.full((B, 1, L, d), 1 / math.sqrt(d))
    k = np.zeros((B, 1, L, d))
    v = np.zeros((B, 1, L, d))
    for b in range(B):
        k[b, 0, b] = 1 / math.sqrt(d)
        v[b, 0, b, 0] = 1.0
    x = {"q": si.round_to(q, dtype), "k": si.round_to(k, dtype), "v": v, "log_g": np.zeros((B, 1, L, d)),
         "meta_k": np.zeros((1, m, d))}
    got = gpu_fwd(gpu_lib, x, dtype, w, 0.0)
    t = np.arange(L)[None, :]
    p = np.arange(B)[:, None]
    want_a = (p <= t) & (p >= t - w + 1)
    want_g = t >= p
    assert np.array_equal(got["y_anchor"][:, 0, :, 0] != 0, want_a)
    assert np.array_equal(got["y"][:, 0, :, 0] != 0, want_g)
    # and every other column stays exactly zero
    assert not got["y_anchor"][:, 0, :, 1:].any()


def test_deterministic(gpu_lib):
    x = si.custom_inputs(7, 2, 4, 320, 128, 4, "bf16")
    a = gpu_fwd(gpu_lib, x, "bf16", 64, 0.5)
    b = gpu_fwd(gpu_lib, x, "bf16", 64, 0.5)
    for key in a:
        assert np.array_equal(a[key], b[key]), key


def test_empty_inputs(gpu_lib):
    import torch

    for B, H, L in ((0, 2, 64), (1, 0, 64), (1, 2, 0)):
        z = torch.zeros((B, H, L, 64), device="cuda", dtype=torch.bfloat16)
        lg = torch.zeros((B, H, L, 64), device="cuda", dtype=torch.float32)
        meta = torch.zeros((H, 2, 64), device="cuda", dtype=torch.bfloat16)
        out = gpu_lib.lizard_attn_fwd(z, z, z, lg, meta, window=8, alpha=0.5, need_state=True)
        torch.cuda.synchronize()
        if B * H > 0:
            assert not out["state"].any()  # L = 0: the initial state, zero


def _sampled_slices(B, H):
    rng = np.random.default_rng(11)
    picks = {(0, 0), (B - 1, H - 1)}
    while len(picks) < 4:
        picks.add((int(rng.integers(0, B)), int(rng.integers(0, H))))
    return sorted(picks)


@pytest.mark.parametrize("name", ["llama3_8b_prefill_bf16", "long_ctx_32k_bf16", "prefill_d64_bf16", "prefill_d64_f32"])
def test_full_size_workload_sampled(gpu_lib, name):
    """The benchmark's launch configuration at full size; sampled (b, h)
    slices over the full length are compared with the oracle."""
    import torch

    w = si.WORKLOADS[name]
    log(f"{name}: generating B={w.B} H={w.H} L={w.L} d={w.d}")
    x = upload_workload(w)
    out = gpu_lib.lizard_attn_fwd(x["q"], x["k"], x["v"], x["log_g"], x["meta_k"], window=w.window,
                                  alpha=w.alpha, need_lse=True, need_y_anchor=True, need_state=True)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out["y"]).all())
    for b, h in _sampled_slices(w.B, w.H):
        s = si.slice_inputs(w, b, h)
        o = oracle.lizard_fwd(s["q"][None], s["k"][None], s["v"][None], s["log_g"][None],
                              si.meta_keys(w, h)[None], w.window, w.alpha)
        errs = [assert_close(down(out[key][b, h]), o[key][0], w.dtype, f"{name} {key}[{b},{h}]")
                for key in ("y", "y_anchor", "lse", "state")]
        log(f"{name} slice ({b},{h}): " + " ".join(f"{e:.2e}" for e in errs))

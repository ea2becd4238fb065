"""GPU parity of lizard_attn_bwd against the float64 oracle's analytic
gradients (which are themselves pinned by finite differences and torch
autograd in the CPU tests)."""
import numpy as np
import pytest

import oracle
import seeded_inputs as si
from tests.gpu_util import assert_close, down, flat, log, meta_per_slice, up, up_f32, upload_workload

pytestmark = pytest.mark.gpu

KEYS = ("dq", "dk", "dv", "dlog_g")


def gpu_bwd(sqa, x, dtype, window, alpha, scale=0.0):
    import torch

    m = x["meta_k"].shape[1]
    q, k, v, dy = (up(x[n], dtype) for n in ("q", "k", "v", "dy"))
    lg = up_f32(x["log_g"])
    meta = up(x["meta_k"], dtype) if m > 0 else None
    fw = sqa.lizard_attn_fwd(q, k, v, lg, meta, window=window, alpha=alpha, softmax_scale=scale, need_lse=True)
    g = sqa.lizard_attn_bwd(q, k, v, lg, meta, fw["lse"], dy, window=window, alpha=alpha, softmax_scale=scale)
    torch.cuda.synchronize()
    return {kk: (down(vv) if vv is not None else None) for kk, vv in g.items()}


def ref_bwd(x, window, alpha, scale=None):
    B, H = x["q"].shape[:2]
    r = oracle.lizard_bwd(flat(x["q"]), flat(x["k"]), flat(x["v"]), flat(x["log_g"]),
                          meta_per_slice(x["meta_k"], B), window, alpha, flat(x["dy"]), scale)
    shp = x["q"].shape
    out = {kk: r[kk].reshape(shp) for kk in KEYS}
    out["dmeta"] = r["dmeta"].reshape(B, H, *r["dmeta"].shape[1:]).sum(0)
    # dlog_g sums the terms q*dq - k*dk of the gated branch, which cancel
    # (exactly so at L = 1): its error is measured against their magnitude
    out["dlog_g_scale"] = float(np.abs(flat(x["q"]) * r["dq_gate"]).max())
    return out


def compare(got, ref, dtype, tag):
    from tests.gpu_util import TAU

    errs = {}
    for kk in KEYS:
        if kk == "dlog_g":
            scale = max(float(np.abs(ref[kk]).max()), ref["dlog_g_scale"])
            e = float(np.abs(got[kk] - ref[kk]).max()) / scale
            assert np.isfinite(got[kk]).all() and e <= TAU[dtype], f"{tag} dlog_g: {e:.3e} (scale {scale:.3e})"
            errs[kk] = e
            continue
        errs[kk] = assert_close(got[kk], ref[kk], dtype, f"{tag} {kk}")
    if ref["dmeta"].size:
        errs["dmeta"] = assert_close(got["dmeta"], ref["dmeta"], dtype, f"{tag} dmeta")
    log(f"{tag}: " + " ".join(f"{kk}={v:.2e}" for kk, v in errs.items()))


def test_tiny_workload_f32(gpu_lib):
    w = si.WORKLOADS["tiny_fwd_f32"]
    x = si.full_inputs(w, with_dy=True)
    log("bwd tiny f32 B=1 H=2 L=256 d=64")
    compare(gpu_bwd(gpu_lib, x, "f32", w.window, w.alpha), ref_bwd(x, w.window, w.alpha), "f32", "tiny")


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 64), ("bf16", 128)])
@pytest.mark.parametrize("L", [1, 40, 64, 150, 256])
def test_ragged_lengths(gpu_lib, dtype, d, L):
    x = si.custom_inputs(30, 2, 2, L, d, 4, dtype, with_dy=True, qk_sd=0.5, meta_sd=0.5)
    log(f"bwd ragged dtype={dtype} d={d} L={L}")
    compare(gpu_bwd(gpu_lib, x, dtype, 64, 0.5), ref_bwd(x, 64, 0.5), dtype, f"L={L}")


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128)])
@pytest.mark.parametrize("window,n_meta", [(1, 0), (7, 1), (33, 16), (64, 4)])
def test_window_and_sinks(gpu_lib, dtype, d, window, n_meta):
    # (bf16 at d = 128 runs the anchor walk: every window mask and sink count)
    x = si.custom_inputs(31, 1, 3, 200, d, n_meta, dtype, with_dy=True, qk_sd=1.0, meta_sd=1.0)
    log(f"bwd {dtype} d={d} window={window} n_meta={n_meta}")
    compare(gpu_bwd(gpu_lib, x, dtype, window, 0.7), ref_bwd(x, window, 0.7), dtype, f"w={window} m={n_meta}")


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128)])
@pytest.mark.parametrize("variant", ["sharp", "fast_gate", "hard_reset", "slow_gate", "wide_chunk", "wide_blocks",
                                     "wide_mixed"])
def test_variants(gpu_lib, dtype, d, variant):
    # wide_chunk: chunk decay spans between one and two times the
    # factorisable limit (the shifted reference point); wide_blocks: beyond
    # twice the limit (the pairwise path); wide_mixed: chunks of all kinds
    kw = {
        "sharp": dict(qk_sd=1.0, meta_sd=1.0),
        "fast_gate": dict(gate_mu=-2.0, gate_sd=4.0),
        "hard_reset": dict(hard_reset_frac=0.02, gate_mu=2.0, gate_sd=2.0),
        "slow_gate": dict(gate_mu=8.0, gate_sd=1.0),
        "wide_chunk": dict(gate_mu=-1.0, gate_sd=0.5),
        "wide_blocks": dict(gate_mu=-3.0, gate_sd=0.3),
        "wide_mixed": dict(gate_mu=0.0, gate_sd=3.0),
    }[variant]
    x = si.custom_inputs(32, 2, 2, 192, d, 4, dtype, with_dy=True, **kw)
    log(f"bwd variant={variant} dtype={dtype} d={d}")
    compare(gpu_bwd(gpu_lib, x, dtype, 64, 0.5), ref_bwd(x, 64, 0.5), dtype, variant)


def test_scale_parameter(gpu_lib):
    x = si.custom_inputs(33, 1, 2, 100, 64, 3, "f32", with_dy=True, qk_sd=0.5, meta_sd=0.5)
    compare(gpu_bwd(gpu_lib, x, "f32", 20, 0.5, scale=0.3), ref_bwd(x, 20, 0.5, scale=0.3), "f32", "scale=0.3")


def test_deterministic(gpu_lib):
    x = si.custom_inputs(34, 2, 4, 320, 128, 4, "bf16", with_dy=True)
    a = gpu_bwd(gpu_lib, x, "bf16", 64, 0.5)
    b = gpu_bwd(gpu_lib, x, "bf16", 64, 0.5)
    for kk in a:
        assert np.array_equal(a[kk], b[kk]), kk


def test_empty_batch_zero_sink_gradient(gpu_lib):
    import torch

    z = torch.zeros((0, 2, 64, 64), device="cuda", dtype=torch.bfloat16)
    lg = torch.zeros((0, 2, 64, 64), device="cuda", dtype=torch.float32)
    meta = torch.zeros((2, 3, 64), device="cuda", dtype=torch.bfloat16)
    lse = torch.zeros((0, 2, 64), device="cuda", dtype=torch.float32)
    out = {"dmeta": torch.full((2, 3, 64), 7.0, device="cuda", dtype=torch.float32)}
    g = gpu_lib.lizard_attn_bwd(z, z, z, lg, meta, lse, z, window=8, alpha=0.5, out=out)
    torch.cuda.synchronize()
    assert not g["dmeta"].any()


def test_full_size_workload_sampled(gpu_lib):
    """B=8, H=32, L=2048, d=128, the launch configuration the benchmark times;
    sampled (b, h) slices of dq, dk, dv, dlog_g, and the sink-key gradient of
    the sampled heads (summed over all batch rows) against the oracle."""
    import torch

    w = si.WORKLOADS["train_bwd_bf16"]
    log(f"bwd workload B={w.B} H={w.H} L={w.L}: generating")
    x = upload_workload(w, with_dy=True)
    fw = gpu_lib.lizard_attn_fwd(x["q"], x["k"], x["v"], x["log_g"], x["meta_k"], window=w.window, alpha=w.alpha,
                                 need_lse=True)
    g = gpu_lib.lizard_attn_bwd(x["q"], x["k"], x["v"], x["log_g"], x["meta_k"], fw["lse"], x["dy"],
                                window=w.window, alpha=w.alpha)
    torch.cuda.synchronize()
    for kk in ("dq", "dk", "dv", "dlog_g", "dmeta"):
        assert bool(torch.isfinite(g[kk]).all()), kk
    picks = [(0, 0), (w.B - 1, w.H - 1), (3, 17), (6, 4)]
    for b, h in picks:
        s = si.slice_inputs(w, b, h, with_dy=True)
        r = oracle.lizard_bwd(s["q"][None], s["k"][None], s["v"][None], s["log_g"][None], si.meta_keys(w, h)[None],
                              w.window, w.alpha, s["dy"][None])
        errs = [assert_close(down(g[kk][b, h]), r[kk][0], "bf16", f"bwd {kk}[{b},{h}]") for kk in KEYS]
        log(f"bwd slice ({b},{h}): " + " ".join(f"{e:.2e}" for e in errs))
    for h in (0, w.H - 1):
        xs = [si.slice_inputs(w, b, h, with_dy=True) for b in range(w.B)]
        st = lambda n: np.stack([x_[n] for x_ in xs])  # noqa: E731
        mk = np.broadcast_to(si.meta_keys(w, h)[None], (w.B, w.n_meta, w.d))
        _, _, _, dmu = oracle.anchor_bwd(st("q"), st("k"), st("v"), mk, w.window, w.alpha * st("dy"))
        e = assert_close(down(g["dmeta"][h]), dmu.sum(0), "bf16", f"bwd dmeta[{h}]")
        log(f"bwd dmeta head {h}: {e:.2e}")


def test_flagged_chunks_over_several_scan_blocks(gpu_lib):
    """bf16 at d = 128 with every chunk's decay span beyond twice the
    factorisable limit (each chunk left by the reverse walk to the last
    launch) and more flags than one scan workgroup reads (1 x 16 heads x 33
    chunks = 528 > 512): the last launch's flag-scan workgroups and its
    sink-sum workgroups side by side.  Sampled heads, with their sink-key
    gradients, against the oracle."""
    B, H, L, d = 1, 16, 2112, 128
    x = si.custom_inputs(35, B, H, L, d, 4, "bf16", with_dy=True, gate_mu=-3.0, gate_sd=0.3)
    log(f"bwd all chunks flagged B={B} H={H} L={L}")
    g = gpu_bwd(gpu_lib, x, "bf16", 64, 0.5)
    for h in (0, H - 1):
        xs = {n: x[n][:, h:h + 1] for n in ("q", "k", "v", "log_g", "dy")}
        xs["meta_k"] = x["meta_k"][h:h + 1]
        got = {kk: g[kk][:, h:h + 1] for kk in KEYS}
        got["dmeta"] = g["dmeta"][h:h + 1]
        compare(got, ref_bwd(xs, 64, 0.5), "bf16", f"flagged head {h}")


@pytest.mark.parametrize("n_meta", [0, 16])
def test_flagged_chunks_and_sink_counts(gpu_lib, n_meta):
    """Every chunk flagged (bf16, d = 128) with no sink keys (the last launch
    then has flag-scan workgroups only) and with the most sink keys."""
    x = si.custom_inputs(36, 2, 2, 192, 128, n_meta, "bf16", with_dy=True, gate_mu=-3.0, gate_sd=0.3,
                         qk_sd=0.5, meta_sd=0.5)
    log(f"bwd all chunks flagged n_meta={n_meta}")
    compare(gpu_bwd(gpu_lib, x, "bf16", 64, 0.5), ref_bwd(x, 64, 0.5), "bf16", f"flagged m={n_meta}")

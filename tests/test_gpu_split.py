"""GPU parity of lizard_attn_fwd_split (long sequences over few heads, cut
into segments that run side by side) against the float64 oracle: the split
must give the one-pass results, with gates that decay fast (most carried
terms vanish), slowly (every chunk of every segment is corrected) or with
hard resets, ragged lengths, both gate forms and a continued sequence."""
import numpy as np
import pytest

import oracle
import seeded_inputs as si
from tests.gpu_util import assert_close, down, flat, log, meta_per_slice, up, up_f32, upload_workload

pytestmark = pytest.mark.gpu

GATES = {"fast": dict(gate_mu=2.0, gate_sd=2.0), "slow": dict(gate_mu=6.0, gate_sd=1.0),
         "reset": dict(gate_mu=4.0, gate_sd=1.0, hard_reset_frac=0.01),
         "wide": dict(gate_mu=0.0, gate_sd=3.0)}   # chunks of every decay-span tier


def _segments(sqa, B, H, L, d, dtype):
    return sqa.lizard_attn_fwd_split_workspace_size(B, H, L, d, dtype_code=sqa.LIZARD_BF16 if dtype == "bf16"
                                                     else sqa.LIZARD_F32)


def _ref(x, w, alpha, logit, state_in=None, k_halo=None, v_halo=None):
    B = x["q"].shape[0]
    lg = oracle.log_sigmoid(flat(x["gate_logit"])) if logit else flat(x["log_g"])
    o = oracle.lizard_fwd_continue(flat(x["q"]), flat(x["k"]), flat(x["v"]), lg, meta_per_slice(x["meta_k"], B), w,
                                   alpha, state_in=state_in, k_halo=k_halo, v_halo=v_halo)
    shp = x["q"].shape
    return {"y": o["y"].reshape(shp), "y_anchor": o["y_anchor"].reshape(shp), "lse": o["lse"].reshape(shp[:3]),
            "state": o["state"].reshape(shp[0], shp[1], shp[3], shp[3])}


def _run_split(sqa, x, dtype, w, alpha, logit, workspace=None, **cont):
    import torch

    gate = dict(gate_logit=up(x["gate_logit"], dtype)) if logit else dict(log_g=up_f32(x["log_g"]))
    out = sqa.lizard_attn_fwd_split(up(x["q"], dtype), up(x["k"], dtype), up(x["v"], dtype), up(x["meta_k"], dtype),
                                    window=w, alpha=alpha, need_lse=True, need_y_anchor=True, need_state=True,
                                    workspace=workspace, **gate, **cont)
    torch.cuda.synchronize()
    return {k: down(v) for k, v in out.items()}


def _compare(got, ref, dtype, tag):
    errs = {key: assert_close(got[key], ref[key], dtype, f"{tag} {key}") for key in ("y", "y_anchor", "lse", "state")}
    log(f"{tag}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))


# (dtype, d, B, H, L): every case is split (workspace size > 0); L ragged or not
SHAPES = [("bf16", 128, 1, 2, 2011), ("bf16", 128, 1, 1, 4096), ("bf16", 64, 1, 3, 3000), ("f32", 64, 1, 1, 1100)]


@pytest.mark.parametrize("gates", sorted(GATES))
@pytest.mark.parametrize("dtype,d,B,H,L", SHAPES)
def test_split_matches_oracle(gpu_lib, dtype, d, B, H, L, gates):
    assert _segments(gpu_lib, B, H, L, d, dtype) > 0, "this shape must be split"
    x = si.custom_inputs(40, B, H, L, d, 4, dtype, **GATES[gates])
    tag = f"split {dtype} d={d} B={B} H={H} L={L} gates={gates}"
    log(tag)
    _compare(_run_split(gpu_lib, x, dtype, 64, 0.5, False), _ref(x, 64, 0.5, False), dtype, tag)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_split_logit_gates(gpu_lib, dtype, d):
    L = 1500
    x = si.custom_inputs(41, 1, 1, L, d, 2, dtype, gate_mu=3.0, gate_sd=1.5)
    tag = f"split logit {dtype} d={d} L={L}"
    log(tag)
    _compare(_run_split(gpu_lib, x, dtype, 33, 0.7, True), _ref(x, 33, 0.7, True), dtype, tag)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_split_continued_sequence(gpu_lib, dtype, d):
    """state_in and the halo enter the first segment only; the oracle's
    continuation of the same sequence decides."""
    P, L, w = 300, 1250, 48
    x = si.custom_inputs(42, 1, 2, P + L, d, 3, dtype, gate_mu=4.0, gate_sd=1.0)
    seg = {k: x[k][:, :, P:] for k in ("q", "k", "v", "log_g", "gate_logit")}
    seg["meta_k"] = x["meta_k"]
    pre = oracle.lizard_fwd(flat(x["q"][:, :, :P]), flat(x["k"][:, :, :P]), flat(x["v"][:, :, :P]),
                            flat(x["log_g"][:, :, :P]), meta_per_slice(x["meta_k"], 1), w, 0.5)
    h = w - 1
    kh, vh = x["k"][:, :, P - h:P], x["v"][:, :, P - h:P]
    tag = f"split continue {dtype} d={d} P={P} L={L}"
    log(tag)
    # the state is passed in float32, the precision the library keeps it in
    state_in = pre["state"].astype(np.float32).astype(np.float64)
    got = _run_split(gpu_lib, seg, dtype, w, 0.5, False, state_in=up_f32(state_in.reshape(1, 2, d, d)),
                     k_halo=up(kh, dtype), v_halo=up(vh, dtype))
    ref = _ref(seg, w, 0.5, False, state_in=state_in, k_halo=flat(kh), v_halo=flat(vh))
    _compare(got, ref, dtype, tag)


def test_split_equals_one_pass_on_short_sequences(gpu_lib):
    """Where no split pays (many heads or short L) the call runs as one pass
    and needs no workspace: its results are the one-pass call's, bit for bit."""
    import torch

    assert _segments(gpu_lib, 4, 32, 512, 128, "bf16") == 0
    x = si.custom_inputs(43, 2, 2, 700, 128, 4, "bf16")
    assert _segments(gpu_lib, 2, 2, 700, 128, "bf16") == 0
    a = _run_split(gpu_lib, x, "bf16", 64, 0.5, False)
    q, k, v, lg, meta = up(x["q"], "bf16"), up(x["k"], "bf16"), up(x["v"], "bf16"), up_f32(x["log_g"]), \
        up(x["meta_k"], "bf16")
    b = gpu_lib.lizard_attn_fwd(q, k, v, lg, meta, window=64, alpha=0.5, need_lse=True, need_y_anchor=True,
                                need_state=True)
    torch.cuda.synchronize()
    for key in ("y", "y_anchor", "lse", "state"):
        assert np.array_equal(a[key], down(b[key])), key


def test_split_workspace_reuse(gpu_lib):
    """One workspace for two calls of different sizes (its contents on entry
    are ignored); both match the oracle."""
    import torch

    need = _segments(gpu_lib, 1, 2, 3000, 128, "bf16")
    ws = torch.full((need,), 0x7f, device="cuda", dtype=torch.uint8)   # NaN-like garbage in the float parts
    for L, seed in ((3000, 44), (1800, 45)):
        x = si.custom_inputs(seed, 1, 2, L, 128, 4, "bf16", gate_mu=5.0, gate_sd=1.0)
        assert 0 < _segments(gpu_lib, 1, 2, L, 128, "bf16") <= need
        tag = f"split workspace reuse L={L}"
        log(tag)
        _compare(_run_split(gpu_lib, x, "bf16", 64, 0.5, False, workspace=ws), _ref(x, 64, 0.5, False), "bf16", tag)


def test_split_full_size_long_context_sampled(gpu_lib):
    """The long-context workload (B=1, H=32, L=32768, gates N(2,2)) through the
    split call in the benchmark's launch configuration; sampled heads over the
    full length are compared with the oracle."""
    import torch

    w = si.WORKLOADS["long_ctx_32k_bf16"]
    assert _segments(gpu_lib, w.B, w.H, w.L, w.d, w.dtype) > 0
    log(f"split full size: generating B={w.B} H={w.H} L={w.L} d={w.d}")
    x = upload_workload(w)
    out = gpu_lib.lizard_attn_fwd_split(x["q"], x["k"], x["v"], x["meta_k"], log_g=x["log_g"], window=w.window,
                                        alpha=w.alpha, need_lse=True, need_y_anchor=True, need_state=True)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out["y"]).all())
    rng = np.random.default_rng(12)
    heads = sorted({0, w.H - 1, *[int(h) for h in rng.integers(0, w.H, 2)]})
    for h in heads:
        s = si.slice_inputs(w, 0, h)
        o = oracle.lizard_fwd(s["q"][None], s["k"][None], s["v"][None], s["log_g"][None],
                              si.meta_keys(w, h)[None], w.window, w.alpha)
        errs = [assert_close(down(out[key][0, h]), o[key][0], w.dtype, f"split 32k {key}[0,{h}]")
                for key in ("y", "y_anchor", "lse", "state")]
        log(f"split 32k head {h}: " + " ".join(f"{e:.2e}" for e in errs))


@pytest.mark.parametrize("entry", ["fwd", "fwd_logit", "fwd_continue"])
def test_named_calls_take_the_split_schedule(gpu_lib, entry):
    """Where a split pays, lizard_attn_fwd (and its logit and continued forms)
    runs the split schedule itself, with a workspace of its own: its results
    are lizard_attn_fwd_split's, bit for bit (the same kernels on the same
    segments), and so the oracle's to the split's tolerance."""
    import torch

    dtype, d, B, H, L, w = "bf16", 128, 1, 2, 2011, 64
    assert _segments(gpu_lib, B, H, L, d, dtype) > 0, "this shape must be split"
    x = si.custom_inputs(44, B, H, L, d, 4, dtype, **GATES["slow"])
    logit = entry == "fwd_logit"
    tag = f"named call {entry} {dtype} d={d} L={L}"
    log(tag)
    a = _run_split(gpu_lib, x, dtype, w, 0.5, logit)
    q, k, v, meta = up(x["q"], dtype), up(x["k"], dtype), up(x["v"], dtype), up(x["meta_k"], dtype)
    kw = dict(window=w, alpha=0.5, need_lse=True, need_y_anchor=True, need_state=True)
    if entry == "fwd":
        b = gpu_lib.lizard_attn_fwd(q, k, v, up_f32(x["log_g"]), meta, **kw)
    elif entry == "fwd_logit":
        b = gpu_lib.lizard_attn_fwd_logit(q, k, v, up(x["gate_logit"], dtype), meta, **kw)
    else:
        b = gpu_lib.lizard_attn_fwd_continue(q, k, v, meta, log_g=up_f32(x["log_g"]), **kw)
    torch.cuda.synchronize()
    for key in ("y", "y_anchor", "lse", "state"):
        assert np.array_equal(a[key], down(b[key])), key
    _compare({kk: down(vv) for kk, vv in b.items()}, _ref(x, w, 0.5, logit), dtype, tag)

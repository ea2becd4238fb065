"""GPU parity of the training pair lizard_attn_fwd_train / lizard_attn_bwd_train:
the forward's outputs are those of lizard_attn_fwd bit for bit, the chunk-start
states it keeps are the oracle's recurrent states at every chunk start, and the
backward that reads them gives lizard_attn_bwd's results (which recomputes
them: bit for bit at bf16, to float rounding at fp32) and the oracle's
gradients."""
import numpy as np
import pytest

import oracle
import seeded_inputs as si
from tests.gpu_util import TAU, assert_close, down, flat, log, meta_per_slice, up, up_f32, upload_workload

pytestmark = pytest.mark.gpu

GKEY = {False: "dlog_g", True: "dgate_logit"}


def _upload(x, dtype, logit):
    q, k, v, dy = (up(x[n], dtype) for n in ("q", "k", "v", "dy"))
    meta = up(x["meta_k"], dtype) if x["meta_k"].shape[1] > 0 else None
    gate = dict(gate_logit=up(x["gate_logit"], dtype)) if logit else dict(log_g=up_f32(x["log_g"]))
    return q, k, v, dy, meta, gate


@pytest.mark.parametrize("gates", ["N(2,2)", "N(0,3)"])
@pytest.mark.parametrize("logit", [False, True])
@pytest.mark.parametrize("dtype,d,L", [("f32", 64, 150), ("bf16", 128, 200), ("bf16", 64, 64), ("bf16", 128, 1)])
def test_train_pair_matches_the_plain_calls(gpu_lib, dtype, d, L, logit, gates):
    """N(0,3) gate logits put chunks in every decay-span tier (the pairwise
    path included) on both sides."""
    import torch

    mu, sd = {"N(2,2)": (2.0, 2.0), "N(0,3)": (0.0, 3.0)}[gates]
    x = si.custom_inputs(70, 2, 2, L, d, 4, dtype, with_dy=True, gate_mu=mu, gate_sd=sd)
    log(f"train pair dtype={dtype} d={d} L={L} logit={logit} gates={gates}")
    q, k, v, dy, meta, gate = _upload(x, dtype, logit)
    kw = dict(window=48, alpha=0.5)
    tr = gpu_lib.lizard_attn_fwd_train(q, k, v, meta, need_y_anchor=True, need_state=True, **gate, **kw)
    if logit:
        fw = gpu_lib.lizard_attn_fwd_logit(q, k, v, gate["gate_logit"], meta, need_lse=True, need_y_anchor=True,
                                           need_state=True, **kw)
    else:
        fw = gpu_lib.lizard_attn_fwd(q, k, v, gate["log_g"], meta, need_lse=True, need_y_anchor=True,
                                     need_state=True, **kw)
    torch.cuda.synchronize()
    for key in ("y", "lse", "y_anchor", "state"):
        assert torch.equal(tr[key], fw[key]), key
    gb = gpu_lib.lizard_attn_bwd_train(q, k, v, meta, tr["lse"], tr["chunk_states"], dy, **gate, **kw)
    if logit:
        gr = gpu_lib.lizard_attn_bwd_logit(q, k, v, gate["gate_logit"], meta, fw["lse"], dy, **kw)
    else:
        gr = gpu_lib.lizard_attn_bwd(q, k, v, gate["log_g"], meta, fw["lse"], dy, **kw)
    torch.cuda.synchronize()
    for key in ("dq", "dk", "dv", GKEY[logit], "dmeta"):
        if dtype == "bf16":
            assert torch.equal(gb[key], gr[key]), key
        else:
            # fp32: the two forward instances that write the chunk states may
            # round the carried state differently in the last bits
            assert_close(down(gb[key]), down(gr[key]), "f32", f"saved vs recomputed {key}", tau=1e-5)


@pytest.mark.parametrize("dtype,d,L", [("f32", 64, 200), ("bf16", 128, 300)])
def test_chunk_states_are_the_recurrent_states(gpu_lib, dtype, d, L):
    """chunk_states[c] is S after the first 64c tokens (the oracle's
    recurrence run over that prefix; zero for c = 0), to the state's storage
    precision."""
    import torch

    x = si.custom_inputs(71, 1, 3, L, d, 2, dtype, with_dy=True, gate_mu=3.0, gate_sd=1.5)
    q, k, v, _, meta, gate = _upload(x, dtype, False)
    tr = gpu_lib.lizard_attn_fwd_train(q, k, v, meta, window=64, alpha=0.5, **gate)
    torch.cuda.synchronize()
    cs = down(tr["chunk_states"])[0]              # [H, nc, d, d]
    nc = (L + 63) // 64
    assert cs.shape == (3, nc, d, d)
    assert not cs[:, 0].any()
    for c in range(1, nc):
        t = 64 * c
        _, S = oracle.gla_recurrent(flat(x["q"][:, :, :t]), flat(x["k"][:, :, :t]), flat(x["v"][:, :, :t]),
                                    flat(x["log_g"][:, :, :t]))
        e = assert_close(cs[:, c], S, dtype, f"chunk state {c}")
        log(f"chunk state {c}: {e:.2e}")


@pytest.mark.parametrize("logit", [False, True])
def test_train_pair_against_the_oracle(gpu_lib, logit):
    import torch

    dtype, d, L = "bf16", 128, 230
    x = si.custom_inputs(72, 2, 2, L, d, 4, dtype, with_dy=True)
    q, k, v, dy, meta, gate = _upload(x, dtype, logit)
    kw = dict(window=64, alpha=0.5)
    tr = gpu_lib.lizard_attn_fwd_train(q, k, v, meta, **gate, **kw)
    g = gpu_lib.lizard_attn_bwd_train(q, k, v, meta, tr["lse"], tr["chunk_states"], dy, **gate, **kw)
    torch.cuda.synchronize()
    B = 2
    if logit:
        r = oracle.lizard_bwd_logit(flat(x["q"]), flat(x["k"]), flat(x["v"]), flat(x["gate_logit"]),
                                    meta_per_slice(x["meta_k"], B), 64, 0.5, flat(x["dy"]))
    else:
        r = oracle.lizard_bwd(flat(x["q"]), flat(x["k"]), flat(x["v"]), flat(x["log_g"]),
                              meta_per_slice(x["meta_k"], B), 64, 0.5, flat(x["dy"]))
    shp = x["q"].shape
    for key in ("dq", "dk", "dv"):
        e = assert_close(down(g[key]), r[key].reshape(shp), dtype, f"train {key}")
        log(f"train {key}: {e:.2e}")
    gk = GKEY[logit]
    ref = r[gk].reshape(shp)
    scale = max(float(np.abs(ref).max()), float(np.abs(flat(x["q"]) * r["dq_gate"]).max()))
    e = float(np.abs(down(g[gk]) - ref).max()) / scale
    assert e <= TAU[dtype], f"train {gk}: {e:.3e}"


@pytest.mark.parametrize("name", ["train_bwd_bf16", "train_d64_bf16", "train_d64_f32"])
def test_train_pair_full_size_sampled(gpu_lib, name):
    """The training workloads through the training pair, in the launch
    configuration the benchmark times (the stage-1 step at B=8, H=32,
    L=2048, d=128; the bf16-vs-fp32 training-step ablation at d=64 in both
    operand types): y and lse, then dq, dk, dv and dlog_g of four sampled
    (b, h) slices against the oracle, and the sink-key gradient of two heads
    summed over every batch row."""
    import torch

    w = si.WORKLOADS[name]
    log(f"train pair {name} B={w.B} H={w.H} L={w.L} d={w.d}: generating")
    x = upload_workload(w, with_dy=True)
    tr = gpu_lib.lizard_attn_fwd_train(x["q"], x["k"], x["v"], x["meta_k"], log_g=x["log_g"], window=w.window,
                                       alpha=w.alpha)
    g = gpu_lib.lizard_attn_bwd_train(x["q"], x["k"], x["v"], x["meta_k"], tr["lse"], tr["chunk_states"], x["dy"],
                                      log_g=x["log_g"], window=w.window, alpha=w.alpha)
    torch.cuda.synchronize()
    for kk in ("dq", "dk", "dv", "dlog_g", "dmeta"):
        assert bool(torch.isfinite(g[kk]).all()), kk
    for b, h in [(0, 0), (w.B - 1, w.H - 1), (5, 9), (2, 26)]:
        s = si.slice_inputs(w, b, h, with_dy=True)
        mk = si.meta_keys(w, h)[None]
        o = oracle.lizard_fwd(s["q"][None], s["k"][None], s["v"][None], s["log_g"][None], mk, w.window, w.alpha)
        r = oracle.lizard_bwd(s["q"][None], s["k"][None], s["v"][None], s["log_g"][None], mk, w.window, w.alpha,
                              s["dy"][None])
        errs = [assert_close(down(tr["y"][b, h]), o["y"][0], w.dtype, f"train y[{b},{h}]"),
                assert_close(down(tr["lse"][b, h]), o["lse"][0], w.dtype, f"train lse[{b},{h}]")]
        errs += [assert_close(down(g[kk][b, h]), r[kk][0], w.dtype, f"train {kk}[{b},{h}]")
                 for kk in ("dq", "dk", "dv")]
        scale = max(float(np.abs(r["dlog_g"]).max()), float(np.abs(s["q"] * r["dq_gate"][0]).max()))
        e = float(np.abs(down(g["dlog_g"][b, h]) - r["dlog_g"][0]).max()) / scale
        assert e <= TAU[w.dtype], f"train dlog_g[{b},{h}]: {e:.3e}"
        log(f"train slice ({b},{h}): " + " ".join(f"{e_:.2e}" for e_ in errs) + f" dlog_g {e:.2e}")
    for h in (0, w.H - 1):
        xs = [si.slice_inputs(w, b, h, with_dy=True) for b in range(w.B)]
        st = lambda n: np.stack([x_[n] for x_ in xs])  # noqa: E731
        mk = np.broadcast_to(si.meta_keys(w, h)[None], (w.B, w.n_meta, w.d))
        _, _, _, dmu = oracle.anchor_bwd(st("q"), st("k"), st("v"), mk, w.window, w.alpha * st("dy"))
        e = assert_close(down(g["dmeta"][h]), dmu.sum(0), w.dtype, f"train dmeta[{h}]")
        log(f"train dmeta head {h}: {e:.2e}")

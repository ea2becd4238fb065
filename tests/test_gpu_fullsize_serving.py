"""Full-size parity, at the launch configurations the benchmark times, of
the legs beyond the three base calls: the 4K prefill and the training
backward with gate logits, the batch-64 serving decode at T = 4 tokens per
call, and the stage-1 teacher.  Sampled (b, h) slices are compared with the
float64 oracle over their full length."""
import numpy as np
import pytest

import oracle
import seeded_inputs as si
from tests.gpu_util import TAU, assert_close, down, log, upload_workload

pytestmark = pytest.mark.gpu


def test_fwd_logit_full_size(gpu_lib):
    import torch

    w = si.WORKLOADS["llama3_8b_prefill_bf16"]
    log(f"fwd_logit full size B={w.B} H={w.H} L={w.L}: generating")
    x = upload_workload(w, with_logit=True)
    out = gpu_lib.lizard_attn_fwd_logit(x["q"], x["k"], x["v"], x["gate_logit"], x["meta_k"], window=w.window,
                                        alpha=w.alpha, need_lse=True)
    torch.cuda.synchronize()
    for b, h in [(0, 0), (w.B - 1, w.H - 1), (2, 13)]:
        s = si.slice_inputs(w, b, h)
        o = oracle.lizard_fwd_logit(s["q"][None], s["k"][None], s["v"][None], s["gate_logit"][None],
                                    si.meta_keys(w, h)[None], w.window, w.alpha)
        e1 = assert_close(down(out["y"][b, h]), o["y"][0], "bf16", f"fwd_logit y[{b},{h}]")
        e2 = assert_close(down(out["lse"][b, h]), o["lse"][0], "bf16", f"fwd_logit lse[{b},{h}]")
        log(f"fwd_logit slice ({b},{h}): {e1:.2e} {e2:.2e}")


def test_bwd_logit_full_size(gpu_lib):
    import torch

    w = si.WORKLOADS["train_bwd_bf16"]
    log(f"bwd_logit full size B={w.B} H={w.H} L={w.L}: generating")
    x = upload_workload(w, with_dy=True, with_logit=True)
    fw = gpu_lib.lizard_attn_fwd_logit(x["q"], x["k"], x["v"], x["gate_logit"], x["meta_k"], window=w.window,
                                       alpha=w.alpha, need_lse=True)
    g = gpu_lib.lizard_attn_bwd_logit(x["q"], x["k"], x["v"], x["gate_logit"], x["meta_k"], fw["lse"], x["dy"],
                                      window=w.window, alpha=w.alpha)
    torch.cuda.synchronize()
    for b, h in [(0, 0), (w.B - 1, w.H - 1), (5, 11), (2, 30)]:
        s = si.slice_inputs(w, b, h, with_dy=True)
        r = oracle.lizard_bwd_logit(s["q"][None], s["k"][None], s["v"][None], s["gate_logit"][None],
                                    si.meta_keys(w, h)[None], w.window, w.alpha, s["dy"][None])
        errs = [assert_close(down(g[kk][b, h]), r[kk][0], "bf16", f"bwd_logit {kk}[{b},{h}]")
                for kk in ("dq", "dk", "dv", "dgate_logit")]
        log(f"bwd_logit slice ({b},{h}): " + " ".join(f"{e:.2e}" for e in errs))
    # the sink-key gradient of two heads, summed over every batch row
    for h in (0, w.H - 1):
        xs = [si.slice_inputs(w, b, h, with_dy=True) for b in range(w.B)]
        st = lambda n: np.stack([x_[n] for x_ in xs])  # noqa: E731
        mk = np.broadcast_to(si.meta_keys(w, h)[None], (w.B, w.n_meta, w.d))
        _, _, _, dmu = oracle.anchor_bwd(st("q"), st("k"), st("v"), mk, w.window, w.alpha * st("dy"))
        e = assert_close(down(g["dmeta"][h]), dmu.sum(0), "bf16", f"bwd_logit dmeta[{h}]")
        log(f"bwd_logit dmeta head {h}: {e:.2e}")


def test_decode_tokens_full_size(gpu_lib):
    """Batch 64, H=32: after the 2048-token prefill, 64 tokens as 16 calls of
    T = 4 (the benchmark's serving leg) against the oracle's forward."""
    import torch

    w = si.WORKLOADS["decode_b64_bf16"]
    L0, T, calls = w.L, 4, 16
    log(f"decode_tokens full size B={w.B} H={w.H}: generating")
    x = upload_workload(w, L=L0 + T * calls)
    pre = gpu_lib.lizard_attn_fwd(x["q"][:, :, :L0].contiguous(), x["k"][:, :, :L0].contiguous(),
                                  x["v"][:, :, :L0].contiguous(), x["log_g"][:, :, :L0].contiguous(), x["meta_k"],
                                  window=w.window, alpha=w.alpha, need_state=True)
    state = pre["state"]
    kr = x["k"][:, :, L0 - w.window:L0].contiguous()   # (L0 - w) is a multiple of w: slot p mod w is row p - (L0 - w)
    vr = x["v"][:, :, L0 - w.window:L0].contiguous()
    ys = []
    for i in range(calls):
        sl = slice(L0 + T * i, L0 + T * (i + 1))
        pos = torch.full((w.B,), L0 + T * i, device="cuda", dtype=torch.int64)
        ys.append(gpu_lib.lizard_decode_tokens(pos, x["q"][:, :, sl].contiguous(), x["k"][:, :, sl].contiguous(),
                                               x["v"][:, :, sl].contiguous(), x["log_g"][:, :, sl].contiguous(),
                                               x["meta_k"], state, kr, vr, alpha=w.alpha))
    y = torch.cat(ys, dim=2)
    torch.cuda.synchronize()
    for b, h in [(0, 0), (w.B - 1, w.H - 1), (33, 9)]:
        s = si.slice_inputs(w, b, h, L=L0 + T * calls)
        o = oracle.lizard_fwd(s["q"][None], s["k"][None], s["v"][None], s["log_g"][None], si.meta_keys(w, h)[None],
                              w.window, w.alpha)
        e = assert_close(down(y[b, h]), o["y"][0, L0:], "bf16", f"decode_tokens y[{b},{h}]")
        log(f"decode_tokens slice ({b},{h}): {e:.2e}")


def test_stage1_full_size(gpu_lib):
    """The stage-1 step at B=8, H=32, L=2048 (the benchmark's leg): the
    teacher's outputs and the layer's gate and value gradients of sampled
    slices; the per-head losses of those slices."""
    import torch

    w = si.WORKLOADS["train_bwd_bf16"]
    log(f"stage1 full size B={w.B} H={w.H} L={w.L}: generating")
    x = upload_workload(w)
    yt = gpu_lib.lizard_softmax_attn_fwd(x["q"], x["k"], x["v"])["y"]
    fw = gpu_lib.lizard_attn_fwd(x["q"], x["k"], x["v"], x["log_g"], x["meta_k"], window=w.window, alpha=w.alpha,
                                 need_lse=True)
    dy, loss_bh = gpu_lib.lizard_transfer_loss(fw["y"], yt)
    g = gpu_lib.lizard_attn_bwd(x["q"], x["k"], x["v"], x["log_g"], x["meta_k"], fw["lse"], dy, window=w.window,
                                alpha=w.alpha)
    torch.cuda.synchronize()
    n_all = w.B * w.H * w.L * w.d
    for b, h in [(0, 0), (w.B - 1, w.H - 1)]:
        s = si.slice_inputs(w, b, h)
        y_t, _ = oracle.softmax_attention_causal(s["q"][None], s["k"][None], s["v"][None])
        e_t = assert_close(down(yt[b, h]), y_t[0], "bf16", f"teacher y[{b},{h}]")
        y = oracle.lizard_fwd(s["q"][None], s["k"][None], s["v"][None], s["log_g"][None], si.meta_keys(w, h)[None],
                              w.window, w.alpha)["y"]
        err = y - y_t
        # the loss kernel on the y and y_T it was given (this head's share of
        # the mean over all B*H*L*d elements), float32 sums in a fixed order
        e_own = down(fw["y"][b, h]) - down(yt[b, h])
        own_bh = float((e_own * e_own).sum() / n_all)
        assert abs(float(loss_bh[b, h]) - own_bh) <= 1e-5 * own_bh, (float(loss_bh[b, h]), own_bh)
        assert_close(down(fw["y"][b, h]), y[0], "bf16", f"stage1 y[{b},{h}]")
        r = oracle.lizard_bwd(s["q"][None], s["k"][None], s["v"][None], s["log_g"][None], si.meta_keys(w, h)[None],
                              w.window, w.alpha, 2.0 * err / n_all)
        errs = [assert_close(down(g[kk][b, h]), r[kk][0], "bf16", f"stage1 {kk}[{b},{h}]") for kk in ("dq", "dk", "dv")]
        scale = max(float(np.abs(r["dlog_g"]).max()), float(np.abs(s["q"] * r["dq_gate"][0]).max()))
        e_lg = float(np.abs(down(g["dlog_g"][b, h]) - r["dlog_g"][0]).max()) / scale
        assert e_lg <= TAU["bf16"], f"stage1 dlog_g[{b},{h}] {e_lg:.3e}"
        log(f"stage1 slice ({b},{h}): teacher {e_t:.2e} " + " ".join(f"{e:.2e}" for e in errs) + f" dlog_g {e_lg:.2e}")

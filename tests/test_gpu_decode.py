"""GPU parity of lizard_decode_step: a prefill followed by decode steps must
equal the forward pass over the concatenated sequence (oracle), the ring
must hold the inputs bit for bit, and a snapshot must resume bit-identically."""
import numpy as np
import pytest

import oracle
import seeded_inputs as si
from tests.gpu_util import assert_close, down, flat, log, meta_per_slice, up, up_f32, upload_workload

pytestmark = pytest.mark.gpu


def _nan_like(t):
    import torch

    return torch.full_like(t, float("nan"))


def run_decode(sqa, q, k, v, lg, meta, w, alpha, L0, steps, y_sink=None):
    """q, k, v, lg: [B, H, L, d] cuda tensors.  Prefill L0 tokens on the GPU,
    then decode the next ``steps``.  Returns (ys [steps, B, H, d], state, rings)."""
    import torch

    B, H, L, d = q.shape
    if L0 > 0:
        pre = sqa.lizard_attn_fwd(q[:, :, :L0].contiguous(), k[:, :, :L0].contiguous(), v[:, :, :L0].contiguous(),
                                  lg[:, :, :L0].contiguous(), meta, window=w, alpha=alpha, need_state=True)
        state = pre["state"]
    else:
        state = torch.zeros((B, H, d, d), device="cuda", dtype=torch.float32)
    kr = _nan_like(torch.empty((B, H, w, d), device="cuda", dtype=q.dtype))  # unwritten slots are never read
    vr = _nan_like(kr)
    for p in range(max(0, L0 - w), L0):
        kr[:, :, p % w] = k[:, :, p]
        vr[:, :, p % w] = v[:, :, p]
    ys = torch.full((steps, B, H, d), float("nan"), device="cuda", dtype=q.dtype) if y_sink is None else y_sink
    for i in range(steps):
        pos = L0 + i
        sqa.lizard_decode_step(pos, q[:, :, pos].contiguous(), k[:, :, pos].contiguous(), v[:, :, pos].contiguous(),
                               lg[:, :, pos].contiguous(), meta, state, kr, vr, alpha=alpha, y_t=ys[i])
    torch.cuda.synchronize()
    return ys, state, kr, vr


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 64), ("bf16", 128)])
@pytest.mark.parametrize("L0,steps,w", [(0, 40, 16), (100, 70, 64), (64, 5, 64), (37, 30, 1), (130, 20, 7)])
def test_decode_continues_prefill(gpu_lib, dtype, d, L0, steps, w):
    L = L0 + steps
    x = si.custom_inputs(20, 2, 3, L, d, 4, dtype, qk_sd=1.0, meta_sd=1.0)
    log(f"decode dtype={dtype} d={d} L0={L0} steps={steps} w={w}")
    ys, state, _, _ = run_decode(gpu_lib, up(x["q"], dtype), up(x["k"], dtype), up(x["v"], dtype), up_f32(x["log_g"]),
                                 up(x["meta_k"], dtype), w, 0.5, L0, steps)
    ref = oracle.lizard_fwd(flat(x["q"]), flat(x["k"]), flat(x["v"]), flat(x["log_g"]),
                            meta_per_slice(x["meta_k"], 2), w, 0.5)
    got = down(ys).transpose(1, 2, 0, 3).reshape(6, steps, d)
    assert_close(got, ref["y"][:, L0:], dtype, "decode y")
    assert_close(down(state).reshape(6, d, d), ref["state"], dtype, "decode state")


def test_ring_contents_bitwise(gpu_lib):
    import torch

    d, w, L0, steps = 64, 16, 50, 23
    x = si.custom_inputs(21, 1, 2, L0 + steps, d, 2, "bf16")
    k = up(x["k"], "bf16")
    v = up(x["v"], "bf16")
    _, _, kr, vr = run_decode(gpu_lib, up(x["q"], "bf16"), k, v, up_f32(x["log_g"]), up(x["meta_k"], "bf16"),
                              w, 0.5, L0, steps)
    for p in range(L0 + steps - w, L0 + steps):
        assert torch.equal(kr[:, :, p % w].view(torch.int16), k[:, :, p].view(torch.int16))
        assert torch.equal(vr[:, :, p % w].view(torch.int16), v[:, :, p].view(torch.int16))


def test_snapshot_restore_bit_identical(gpu_lib):
    import torch

    d, w = 128, 64
    x = si.custom_inputs(22, 2, 2, 200, d, 4, "bf16")
    q, k, v, lg, meta = (up(x["q"], "bf16"), up(x["k"], "bf16"), up(x["v"], "bf16"), up_f32(x["log_g"]),
                         up(x["meta_k"], "bf16"))
    _, state, kr, vr = run_decode(gpu_lib, q, k, v, lg, meta, w, 0.5, 120, 30)
    snap = (state.clone(), kr.clone(), vr.clone())
    outs = []
    for _ in range(2):
        st, a, b = snap[0].clone(), snap[1].clone(), snap[2].clone()
        ys = []
        for pos in range(150, 200):
            ys.append(gpu_lib.lizard_decode_step(pos, q[:, :, pos].contiguous(), k[:, :, pos].contiguous(),
                                                 v[:, :, pos].contiguous(), lg[:, :, pos].contiguous(), meta, st, a, b,
                                                 alpha=0.5))
        torch.cuda.synchronize()
        outs.append((torch.stack(ys), st))
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1], outs[1][1])


def test_full_size_decode_sampled(gpu_lib):
    """Batch 64, H=32, d=128: a 2048-token prefill then 1024 steps, the
    launch configuration the benchmark times; sampled (b, h) slices of every
    step are compared with the oracle's forward over all 3072 tokens."""
    import torch

    w = si.WORKLOADS["decode_b64_bf16"]
    L0, steps = w.L, w.steps
    log(f"decode workload B={w.B} H={w.H} prefill={L0} steps={steps}: generating")
    x = upload_workload(w)
    picks = [(0, 0), (w.B - 1, w.H - 1), (17, 5), (40, 22)]
    ys, state, kr, _ = run_decode(gpu_lib, x["q"], x["k"], x["v"], x["log_g"], x["meta_k"], w.window, w.alpha,
                                  L0, steps)
    assert bool(torch.isfinite(ys).all())
    for b, h in picks:
        s = si.slice_inputs(w, b, h)
        o = oracle.lizard_fwd(s["q"][None], s["k"][None], s["v"][None], s["log_g"][None], si.meta_keys(w, h)[None],
                              w.window, w.alpha)
        e1 = assert_close(down(ys[:, b, h]), o["y"][0, L0:], "bf16", f"decode y[{b},{h}]")
        e2 = assert_close(down(state[b, h]), o["state"][0], "bf16", f"decode state[{b},{h}]")
        log(f"decode slice ({b},{h}): y {e1:.2e} state {e2:.2e}")
    for p in range(L0 + steps - w.window, L0 + steps):
        assert torch.equal(kr[:, :, p % w.window].view(torch.int16), x["k"][:, :, p].view(torch.int16))

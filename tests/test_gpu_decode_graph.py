"""Decode steps recorded once into a HIP graph (through torch.cuda.graph) and
replayed: every replay must give what the same steps launched one by one give,
bit for bit (outputs, fp32 state, key and value rings), with eager work and a
synchronisation between the replays.  The decode calls launch one kernel each
and allocate nothing, so they can be captured; the parity of the steps
themselves with the oracle is tested in test_gpu_decode and test_gpu_serving.

Two forms: lizard_decode_step with the positions as call arguments (recorded
into the graph: a replay repeats the captured positions), and
lizard_decode_tokens with the positions in device memory, advanced inside the
graph by an in-place add, the form of a serving loop that replays one graph
per token."""
import pytest

import seeded_inputs as si
from tests.gpu_util import log
from tests.test_gpu_serving import _prefill_rows

pytestmark = pytest.mark.gpu

B, H, L0, S, W = 2, 3, 90, 6, 16


def _setup(gpu_lib, dtype, d, seed):
    x = si.custom_inputs(seed, B, H, L0 + S, d, 4, dtype)
    return _prefill_rows(gpu_lib, x, dtype, [L0] * B, W, 0.5)


def _check_replays(g, restore, outs, ref, what):
    import torch

    for rep in range(3):
        outs[0].fill_(float("nan"))   # the outputs; the state and rings are restored
        restore()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("y", "state", "k_ring", "v_ring"), outs, ref):
            assert bool(torch.isfinite(a).all()), f"{what} replay {rep}: {name} not finite"
            assert torch.equal(a, b), f"{what} replay {rep}: {name} differs from the eager steps"
        log(f"{what}: replay {rep} equals the eager steps bit for bit")


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_graph_of_decode_steps(gpu_lib, dtype, d):
    import torch

    log(f"decode graph, positions as arguments, dtype={dtype} d={d} S={S}")
    q, k, v, lg, meta, state, kr, vr = _setup(gpu_lib, dtype, d, 61)
    st0, kr0, vr0 = state.clone(), kr.clone(), vr.clone()
    steps = [tuple(t[:, :, L0 + i].contiguous() for t in (q, k, v, lg)) for i in range(S)]
    y_e = torch.empty((S, B, H, d), device="cuda", dtype=q.dtype)
    for i, (qi, ki, vi, gi) in enumerate(steps):
        gpu_lib.lizard_decode_step(L0 + i, qi, ki, vi, gi, meta, state, kr, vr, alpha=0.5, y_t=y_e[i])
    torch.cuda.synchronize()
    ref = (y_e.clone(), state.clone(), kr.clone(), vr.clone())

    def restore():
        state.copy_(st0)
        kr.copy_(kr0)
        vr.copy_(vr0)

    y_g = torch.empty_like(y_e)
    restore()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i, (qi, ki, vi, gi) in enumerate(steps):
            gpu_lib.lizard_decode_step(L0 + i, qi, ki, vi, gi, meta, state, kr, vr, alpha=0.5, y_t=y_g[i])
    _check_replays(g, restore, (y_g, state, kr, vr), ref, "decode_step graph")


@pytest.mark.parametrize("dtype,d", [("bf16", 128)])
def test_graph_of_serving_tokens(gpu_lib, dtype, d):
    import torch

    log(f"decode graph, device positions advanced in the graph, dtype={dtype} d={d} S={S}")
    q, k, v, lg, meta, state, kr, vr = _setup(gpu_lib, dtype, d, 62)
    st0, kr0, vr0 = state.clone(), kr.clone(), vr.clone()
    steps = [tuple(t[:, :, L0 + i:L0 + i + 1].contiguous() for t in (q, k, v, lg)) for i in range(S)]
    pos = torch.full((B,), L0, device="cuda", dtype=torch.int64)
    y_e = torch.empty((S, B, H, 1, d), device="cuda", dtype=q.dtype)
    for i, (qi, ki, vi, gi) in enumerate(steps):
        gpu_lib.lizard_decode_tokens(pos, qi, ki, vi, gi, meta, state, kr, vr, alpha=0.5, y=y_e[i])
        pos.add_(1)
    torch.cuda.synchronize()
    assert pos.tolist() == [L0 + S] * B
    ref = (y_e.clone(), state.clone(), kr.clone(), vr.clone())

    def restore():
        state.copy_(st0)
        kr.copy_(kr0)
        vr.copy_(vr0)
        pos.fill_(L0)

    y_g = torch.empty_like(y_e)
    restore()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i, (qi, ki, vi, gi) in enumerate(steps):
            gpu_lib.lizard_decode_tokens(pos, qi, ki, vi, gi, meta, state, kr, vr, alpha=0.5, y=y_g[i])
            pos.add_(1)
    _check_replays(g, restore, (y_g, state, kr, vr), ref, "decode_tokens graph")
    assert pos.tolist() == [L0 + S] * B

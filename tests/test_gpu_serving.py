"""GPU parity of the serving decode (lizard_decode_tokens): T tokens per
call and a position per batch row.  T tokens in one call must equal T
single decode steps bit for bit (same arithmetic, the state kept in
registers between them), rows at different positions must each match the
oracle's forward pass over their own sequence, and inactive rows (negative
position) must be left untouched."""
import numpy as np
import pytest

import oracle
import seeded_inputs as si
from tests.gpu_util import assert_close, down, flat, log, meta_per_slice, up, up_f32

pytestmark = pytest.mark.gpu


def _prefill_rows(sqa, x, dtype, L0s, w, alpha):
    """Per batch row b, a GPU prefill of its first L0s[b] tokens (B = 1 calls):
    returns the stacked state [B, H, d, d] and rings [B, H, w, d]."""
    import torch

    B, H, L, d = x["q"].shape
    q, k, v, lg, meta = up(x["q"], dtype), up(x["k"], dtype), up(x["v"], dtype), up_f32(x["log_g"]), up(x["meta_k"], dtype)
    state = torch.zeros((B, H, d, d), device="cuda", dtype=torch.float32)
    kr = torch.full((B, H, w, d), float("nan"), device="cuda", dtype=q.dtype)
    vr = torch.full_like(kr, float("nan"))
    for b, L0 in enumerate(L0s):
        if L0 > 0:
            pre = sqa.lizard_attn_fwd(q[b:b + 1, :, :L0].contiguous(), k[b:b + 1, :, :L0].contiguous(),
                                      v[b:b + 1, :, :L0].contiguous(), lg[b:b + 1, :, :L0].contiguous(), meta,
                                      window=w, alpha=alpha, need_state=True)
            state[b] = pre["state"][0]
        for p in range(max(0, L0 - w), L0):
            kr[b, :, p % w] = k[b, :, p]
            vr[b, :, p % w] = v[b, :, p]
    return q, k, v, lg, meta, state, kr, vr


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128)])
@pytest.mark.parametrize("T,w", [(1, 64), (4, 64), (7, 16), (70, 64), (3, 1)])
def test_tokens_equal_single_steps_bitwise(gpu_lib, dtype, d, T, w):
    import torch

    B, H, L0 = 2, 3, 90
    x = si.custom_inputs(50, B, H, L0 + T, d, 4, dtype)
    log(f"decode_tokens vs steps dtype={dtype} d={d} T={T} w={w}")
    q, k, v, lg, meta, state, kr, vr = _prefill_rows(gpu_lib, x, dtype, [L0] * B, w, 0.5)
    st1, kr1, vr1 = state.clone(), kr.clone(), vr.clone()
    ys1 = torch.full((T, B, H, d), float("nan"), device="cuda", dtype=q.dtype)
    for i in range(T):
        pos = L0 + i
        gpu_lib.lizard_decode_step(pos, q[:, :, pos].contiguous(), k[:, :, pos].contiguous(), v[:, :, pos].contiguous(),
                                   lg[:, :, pos].contiguous(), meta, st1, kr1, vr1, alpha=0.5, y_t=ys1[i])
    ys1 = ys1.permute(1, 2, 0, 3).contiguous()
    pos = torch.full((B,), L0, device="cuda", dtype=torch.int64)
    sl = slice(L0, L0 + T)
    y2 = gpu_lib.lizard_decode_tokens(pos, q[:, :, sl].contiguous(), k[:, :, sl].contiguous(),
                                      v[:, :, sl].contiguous(), lg[:, :, sl].contiguous(), meta, state, kr, vr,
                                      alpha=0.5)
    torch.cuda.synchronize()
    assert torch.equal(y2.view(torch.int16 if dtype == "bf16" else torch.int32),
                       ys1.view(torch.int16 if dtype == "bf16" else torch.int32))
    assert torch.equal(state.view(torch.int32), st1.view(torch.int32))
    kv = torch.int16 if dtype == "bf16" else torch.int32
    assert torch.equal(kr.view(kv), kr1.view(kv)) or torch.equal(torch.nan_to_num(kr), torch.nan_to_num(kr1))
    assert torch.equal(torch.nan_to_num(vr), torch.nan_to_num(vr1))
    # and the oracle
    ref = oracle.lizard_fwd(flat(x["q"]), flat(x["k"]), flat(x["v"]), flat(x["log_g"]),
                            meta_per_slice(x["meta_k"], B), w, 0.5)
    assert_close(down(y2).reshape(B * H, T, d), ref["y"][:, L0:], dtype, "decode_tokens y")
    assert_close(down(state).reshape(B * H, d, d), ref["state"], dtype, "decode_tokens state")


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 64), ("bf16", 128)])
def test_rows_at_their_own_positions(gpu_lib, dtype, d):
    """Four rows at positions 0, 37, 64 and 200 (and one inactive row) take
    T = 5 tokens each in one call."""
    import torch

    L0s = [0, 37, 64, 200, 11]
    B, H, T, w = len(L0s), 2, 5, 64
    Lmax = max(L0s) + T
    x = si.custom_inputs(51, B, H, Lmax, d, 3, dtype)
    log(f"decode_tokens per-row positions dtype={dtype} d={d}")
    q, k, v, lg, meta, state, kr, vr = _prefill_rows(gpu_lib, x, dtype, L0s, w, 0.5)
    # the last row is inactive: a negative position
    pos_host = list(L0s[:-1]) + [-1]
    pos = torch.tensor(pos_host, device="cuda", dtype=torch.int64)
    idx = torch.tensor([[max(p0, 0) + j for j in range(T)] for p0 in L0s], device="cuda")
    gat = lambda t: torch.stack([t[b, :, idx[b]] for b in range(B)]).contiguous()
    yq, yk, yv, ylg = gat(q), gat(k), gat(v), gat(lg)
    y = torch.full_like(yq, 7.0)
    st_inactive, kr_inactive, vr_inactive = state[-1].clone(), kr[-1].clone(), vr[-1].clone()
    gpu_lib.lizard_decode_tokens(pos, yq, yk, yv, ylg, meta, state, kr, vr, alpha=0.5, y=y)
    torch.cuda.synchronize()
    for b, L0 in enumerate(L0s[:-1]):
        L = L0 + T
        ref = oracle.lizard_fwd(flat(x["q"][b:b + 1, :, :L]), flat(x["k"][b:b + 1, :, :L]), flat(x["v"][b:b + 1, :, :L]),
                                flat(x["log_g"][b:b + 1, :, :L]), x["meta_k"], w, 0.5)
        assert_close(down(y[b]), ref["y"][:, L0:], dtype, f"row {b} y")
        assert_close(down(state[b]), ref["state"], dtype, f"row {b} state")
    # untouched inactive row
    assert torch.equal(state[-1].view(torch.int32), st_inactive.view(torch.int32))
    assert torch.equal(torch.nan_to_num(kr[-1]), torch.nan_to_num(kr_inactive))
    assert torch.equal(torch.nan_to_num(vr[-1]), torch.nan_to_num(vr_inactive))
    assert bool((y[-1] == 7.0).all())


def test_tokens_logit(gpu_lib):
    """lizard_decode_tokens_logit against the oracle fed with the logits."""
    import torch

    dtype, d, B, H, L0, T, w = "bf16", 128, 2, 2, 80, 6, 64
    x = si.custom_inputs(52, B, H, L0 + T, d, 4, dtype)
    q, k, v, xg, meta = (up(x[n], dtype) for n in ("q", "k", "v", "gate_logit", "meta_k"))
    pre = gpu_lib.lizard_attn_fwd_logit(q[:, :, :L0].contiguous(), k[:, :, :L0].contiguous(),
                                        v[:, :, :L0].contiguous(), xg[:, :, :L0].contiguous(), meta, window=w,
                                        alpha=0.5, need_state=True)
    state = pre["state"]
    kr = torch.full((B, H, w, d), float("nan"), device="cuda", dtype=q.dtype)
    vr = torch.full_like(kr, float("nan"))
    for p in range(max(0, L0 - w), L0):
        kr[:, :, p % w] = k[:, :, p]
        vr[:, :, p % w] = v[:, :, p]
    pos = torch.full((B,), L0, device="cuda", dtype=torch.int64)
    sl = slice(L0, L0 + T)
    y = gpu_lib.lizard_decode_tokens_logit(pos, q[:, :, sl].contiguous(), k[:, :, sl].contiguous(),
                                           v[:, :, sl].contiguous(), xg[:, :, sl].contiguous(), meta, state, kr, vr,
                                           alpha=0.5)
    torch.cuda.synchronize()
    ref = oracle.lizard_fwd_logit(flat(x["q"]), flat(x["k"]), flat(x["v"]), flat(x["gate_logit"]),
                                  meta_per_slice(x["meta_k"], B), w, 0.5)
    assert_close(down(y).reshape(B * H, T, d), ref["y"][:, L0:], dtype, "decode_tokens_logit y")


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 64), ("bf16", 128)])
@pytest.mark.parametrize("cuts,w", [((100,), 64), ((10, 70), 64), ((64, 128), 16), ((33,), 1), ((5, 6, 200), 64)])
def test_prefill_in_segments(gpu_lib, dtype, d, cuts, w):
    """A sequence prefilled as segments (lizard_attn_fwd_continue with the
    previous segment's state and last min(w-1, P) keys / values) equals the
    oracle's one pass over the whole sequence, outputs, lse and final state."""
    import torch

    B, H, L = 2, 2, 260
    x = si.custom_inputs(53, B, H, L, d, 4, dtype)
    log(f"continue dtype={dtype} d={d} cuts={cuts} w={w}")
    q, k, v, lg, meta = up(x["q"], dtype), up(x["k"], dtype), up(x["v"], dtype), up_f32(x["log_g"]), up(x["meta_k"], dtype)
    ref = oracle.lizard_fwd(flat(x["q"]), flat(x["k"]), flat(x["v"]), flat(x["log_g"]), meta_per_slice(x["meta_k"], B),
                            w, 0.5)
    bounds = (0,) + cuts + (L,)
    state = None
    for a, b in zip(bounds[:-1], bounds[1:]):
        h = min(w - 1, a)
        kh = k[:, :, a - h:a].contiguous() if h else None
        vh = v[:, :, a - h:a].contiguous() if h else None
        seg = gpu_lib.lizard_attn_fwd_continue(q[:, :, a:b].contiguous(), k[:, :, a:b].contiguous(),
                                               v[:, :, a:b].contiguous(), meta, log_g=lg[:, :, a:b].contiguous(),
                                               state_in=state, k_halo=kh, v_halo=vh, window=w, alpha=0.5,
                                               need_lse=True, need_state=True)
        torch.cuda.synchronize()
        assert_close(down(seg["y"]).reshape(B * H, b - a, d), ref["y"][:, a:b], dtype, f"segment {a}:{b} y")
        assert_close(down(seg["lse"]).reshape(B * H, b - a), ref["lse"][:, a:b], "f32", f"segment {a}:{b} lse",
                     tau=2e-2 if dtype == "bf16" else 1e-4)
        state = seg["state"]
    assert_close(down(state).reshape(B * H, d, d), ref["state"], dtype, "final state")


def test_prefill_in_segments_logit(gpu_lib):
    """The same with the gates given by their logits."""
    import torch

    dtype, d, B, H, L, w, cut = "bf16", 128, 1, 3, 200, 64, 90
    x = si.custom_inputs(54, B, H, L, d, 4, dtype)
    q, k, v, xg, meta = (up(x[n], dtype) for n in ("q", "k", "v", "gate_logit", "meta_k"))
    first = gpu_lib.lizard_attn_fwd_logit(q[:, :, :cut].contiguous(), k[:, :, :cut].contiguous(),
                                          v[:, :, :cut].contiguous(), xg[:, :, :cut].contiguous(), meta, window=w,
                                          alpha=0.5, need_state=True)
    seg = gpu_lib.lizard_attn_fwd_continue(q[:, :, cut:].contiguous(), k[:, :, cut:].contiguous(),
                                           v[:, :, cut:].contiguous(), meta, gate_logit=xg[:, :, cut:].contiguous(),
                                           state_in=first["state"], k_halo=k[:, :, cut - w + 1:cut].contiguous(),
                                           v_halo=v[:, :, cut - w + 1:cut].contiguous(), window=w, alpha=0.5)
    torch.cuda.synchronize()
    ref = oracle.lizard_fwd_logit(flat(x["q"]), flat(x["k"]), flat(x["v"]), flat(x["gate_logit"]),
                                  meta_per_slice(x["meta_k"], B), w, 0.5)
    assert_close(down(seg["y"]).reshape(B * H, L - cut, d), ref["y"][:, cut:], dtype, "continued y (logits)")

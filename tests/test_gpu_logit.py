"""GPU parity of the entry points that take the gate logits
(lizard_attn_fwd_logit, lizard_attn_bwd_logit, lizard_decode_step_logit)
against the float64 oracle fed with the same logits (oracle.lizard_*_logit,
pinned against torch's logsigmoid and autograd in the CPU tests)."""
import numpy as np
import pytest

import oracle
import seeded_inputs as si
from tests.gpu_util import TAU, assert_close, down, flat, log, meta_per_slice, up

pytestmark = pytest.mark.gpu


def _inputs(seed, B, H, L, d, m, dtype, **kw):
    return si.custom_inputs(seed, B, H, L, d, m, dtype, with_dy=True, **kw)


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 64), ("bf16", 128)])
@pytest.mark.parametrize("L", [1, 150, 256])
def test_fwd_logit(gpu_lib, dtype, d, L):
    x = _inputs(40, 2, 3, L, d, 4, dtype)
    log(f"fwd_logit dtype={dtype} d={d} L={L}")
    q, k, v, xg, meta = (up(x[n], dtype) for n in ("q", "k", "v", "gate_logit", "meta_k"))
    out = gpu_lib.lizard_attn_fwd_logit(q, k, v, xg, meta, window=64, alpha=0.5, need_lse=True, need_state=True)
    ref = oracle.lizard_fwd_logit(flat(x["q"]), flat(x["k"]), flat(x["v"]), flat(x["gate_logit"]),
                                  meta_per_slice(x["meta_k"], 2), 64, 0.5)
    assert_close(down(out["y"]).reshape(6, L, d), ref["y"], dtype, "y")
    assert_close(down(out["state"]).reshape(6, d, d), ref["state"], dtype, "state")
    assert_close(down(out["lse"]).reshape(6, L), ref["lse"], "f32", "lse", tau=TAU[dtype])


@pytest.mark.parametrize("variant", ["plain", "hard_reset", "wide_logits"])
def test_fwd_logit_gate_variants(gpu_lib, variant):
    """Hard resets (logit -1000, gate 0) and logits spread over +-20 (gates
    from ~1e-9 to ~1, the wide-span path included)."""
    kw = {"plain": {}, "hard_reset": {"hard_reset_frac": 0.05}, "wide_logits": {"gate_mu": 0.0, "gate_sd": 8.0}}
    dtype, d, L = "bf16", 128, 200
    x = _inputs(41, 1, 4, L, d, 4, dtype, **kw[variant])
    log(f"fwd_logit variant={variant}")
    q, k, v, xg, meta = (up(x[n], dtype) for n in ("q", "k", "v", "gate_logit", "meta_k"))
    out = gpu_lib.lizard_attn_fwd_logit(q, k, v, xg, meta, window=64, alpha=0.5)
    ref = oracle.lizard_fwd_logit(flat(x["q"]), flat(x["k"]), flat(x["v"]), flat(x["gate_logit"]),
                                  meta_per_slice(x["meta_k"], 1), 64, 0.5)
    assert_close(down(out["y"]).reshape(4, L, d), ref["y"], dtype, "y")


def _bwd_compare(got, x, dtype, B, tag, window=64, alpha=0.5):
    r = oracle.lizard_bwd_logit(flat(x["q"]), flat(x["k"]), flat(x["v"]), flat(x["gate_logit"]),
                                meta_per_slice(x["meta_k"], B), window, alpha, flat(x["dy"]))
    shp = x["q"].shape
    errs = {}
    for kk in ("dq", "dk", "dv"):
        errs[kk] = assert_close(got[kk], r[kk].reshape(shp), dtype, f"{tag} {kk}")
    # dgate_logit = dlog_g * sigmoid(-x); dlog_g is a sum of cancelling terms
    # q*dq - k*dk, so its error is measured against their magnitude times the
    # largest sigmoid(-x) factor (the rule of the log-gate backward test)
    sig = np.exp(oracle.log_sigmoid(-flat(x["gate_logit"])))
    scale = max(float(np.abs(r["dgate_logit"]).max()),
                float(np.abs(flat(x["q"]) * r["dq_gate"]).max()) * float(sig.max()))
    ref_dg = r["dgate_logit"].reshape(shp)
    e = float(np.abs(got["dgate_logit"] - ref_dg).max()) / scale
    assert np.isfinite(got["dgate_logit"]).all() and e <= TAU[dtype], f"{tag} dgate_logit: {e:.3e}"
    errs["dgate_logit"] = e
    H = shp[1]
    dmeta = r["dmeta"].reshape(B, H, *r["dmeta"].shape[1:]).sum(0)
    if dmeta.size:
        errs["dmeta"] = assert_close(got["dmeta"], dmeta, dtype, f"{tag} dmeta")
    log(f"{tag}: " + " ".join(f"{kk}={v:.2e}" for kk, v in errs.items()))


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 64), ("bf16", 128)])
@pytest.mark.parametrize("L", [1, 40, 150, 256])
def test_bwd_logit(gpu_lib, dtype, d, L):
    import torch

    B = 2
    x = _inputs(42, B, 2, L, d, 4, dtype)
    log(f"bwd_logit dtype={dtype} d={d} L={L}")
    q, k, v, xg, meta, dy = (up(x[n], dtype) for n in ("q", "k", "v", "gate_logit", "meta_k", "dy"))
    fw = gpu_lib.lizard_attn_fwd_logit(q, k, v, xg, meta, window=64, alpha=0.5, need_lse=True)
    g = gpu_lib.lizard_attn_bwd_logit(q, k, v, xg, meta, fw["lse"], dy, window=64, alpha=0.5)
    torch.cuda.synchronize()
    got = {kk: down(vv) for kk, vv in g.items() if vv is not None}
    _bwd_compare(got, x, dtype, B, f"bwd_logit {dtype} d={d} L={L}")


@pytest.mark.parametrize("variant", ["hard_reset", "wide_logits"])
def test_bwd_logit_gate_variants(gpu_lib, variant):
    import torch

    kw = {"hard_reset": {"hard_reset_frac": 0.05}, "wide_logits": {"gate_mu": 0.0, "gate_sd": 8.0}}
    dtype, d, L, B = "bf16", 128, 200, 1
    x = _inputs(43, B, 3, L, d, 4, dtype, **kw[variant])
    log(f"bwd_logit variant={variant}")
    q, k, v, xg, meta, dy = (up(x[n], dtype) for n in ("q", "k", "v", "gate_logit", "meta_k", "dy"))
    fw = gpu_lib.lizard_attn_fwd_logit(q, k, v, xg, meta, window=64, alpha=0.5, need_lse=True)
    g = gpu_lib.lizard_attn_bwd_logit(q, k, v, xg, meta, fw["lse"], dy, window=64, alpha=0.5)
    torch.cuda.synchronize()
    got = {kk: down(vv) for kk, vv in g.items() if vv is not None}
    _bwd_compare(got, x, dtype, B, f"bwd_logit {variant}")


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128)])
def test_decode_logit_continues_prefill(gpu_lib, dtype, d):
    """A logit-fed prefill of L0 tokens, then logit-fed decode steps, equals
    the oracle's logit-fed forward pass over the whole sequence."""
    import torch

    B, H, L0, steps, w = 2, 3, 100, 30, 64
    L = L0 + steps
    x = _inputs(44, B, H, L, d, 4, dtype)
    log(f"decode_logit dtype={dtype} d={d}")
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
    ys = torch.full((steps, B, H, d), float("nan"), device="cuda", dtype=q.dtype)
    for i in range(steps):
        pos = L0 + i
        gpu_lib.lizard_decode_step_logit(pos, q[:, :, pos].contiguous(), k[:, :, pos].contiguous(),
                                         v[:, :, pos].contiguous(), xg[:, :, pos].contiguous(), meta, state, kr, vr,
                                         alpha=0.5, y_t=ys[i])
    torch.cuda.synchronize()
    ref = oracle.lizard_fwd_logit(flat(x["q"]), flat(x["k"]), flat(x["v"]), flat(x["gate_logit"]),
                                  meta_per_slice(x["meta_k"], B), w, 0.5)
    got = down(ys).transpose(1, 2, 0, 3).reshape(B * H, steps, d)
    assert_close(got, ref["y"][:, L0:], dtype, "decode_logit y")
    assert_close(down(state).reshape(B * H, d, d), ref["state"], dtype, "decode_logit state")


def test_logit_and_log_gate_paths_agree(gpu_lib):
    """Feeding the kernels log sigmoid(x) in float32 or x itself gives the
    same outputs up to float32 evaluation of the log-sigmoid (the two paths
    share every kernel but the gate prologue / epilogue)."""
    import torch

    dtype, d, L, B = "bf16", 128, 192, 2
    x = _inputs(45, B, 2, L, d, 4, dtype)
    q, k, v, xg, meta, dy = (up(x[n], dtype) for n in ("q", "k", "v", "gate_logit", "meta_k", "dy"))
    lg = torch.nn.functional.logsigmoid(xg.float()).contiguous()
    a = gpu_lib.lizard_attn_fwd_logit(q, k, v, xg, meta, window=64, alpha=0.5, need_lse=True)
    b = gpu_lib.lizard_attn_fwd(q, k, v, lg, meta, window=64, alpha=0.5, need_lse=True)
    ga = gpu_lib.lizard_attn_bwd_logit(q, k, v, xg, meta, a["lse"], dy, window=64, alpha=0.5)
    gb = gpu_lib.lizard_attn_bwd(q, k, v, lg, meta, b["lse"], dy, window=64, alpha=0.5)
    torch.cuda.synchronize()
    assert_close(down(a["y"]), down(b["y"]), dtype, "y (logit vs log-gate)", tau=1e-2)
    for kk in ("dq", "dk", "dv"):
        assert_close(down(ga[kk]), down(gb[kk]), dtype, f"{kk} (logit vs log-gate)", tau=1e-2)
    dg_from_lg = down(gb["dlog_g"]) * torch.sigmoid(-xg.float()).cpu().numpy().astype(np.float64)
    assert_close(down(ga["dgate_logit"]), dg_from_lg, dtype, "dgate_logit (logit vs log-gate)", tau=1e-2)

"""The seeded input generator: reproducible per slice, bfloat16 rounding
matches torch's float32 -> bfloat16 conversion (round to nearest even)."""
import numpy as np
import torch

import seeded_inputs as si


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000) * 10.0 ** rng.integers(-30, 30, 100000),
                        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, 1e-40, 65504.0])]).astype(np.float32)
    # ties: low half exactly 0x8000
    ties = (np.arange(1000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties])
    ours = si.round_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_slices_reproducible_and_distinct():
    w = si.WORKLOADS["tiny_fwd_f32"]
    a = si.slice_inputs(w, 0, 1)
    b = si.slice_inputs(w, 0, 1)
    c = si.slice_inputs(w, 0, 0)
    for n in ("q", "k", "v", "log_g"):
        assert np.array_equal(a[n], b[n])
        assert not np.array_equal(a[n], c[n])
    assert (a["log_g"] <= 0).all()
    assert abs(a["q"].std() - 0.125) < 0.01


def test_full_inputs_match_slices():
    w = si.WORKLOADS["tiny_fwd_f32"]
    full = si.full_inputs(w, L=64)
    s = si.slice_inputs(w, 0, 1, L=64)
    assert np.array_equal(full["k"][0, 1], s["k"])
    assert full["meta_k"].shape == (2, 4, 64)


def test_bf16_values_are_representable():
    w = si.WORKLOADS["llama3_8b_prefill_bf16"]
    s = si.slice_inputs(w, 1, 3, L=128)
    bits = si.round_bf16_bits(s["q"])
    assert np.array_equal(si.bf16_bits_to_f64(bits), s["q"])


def test_oracle_regression_snapshot():
    import os

    import oracle

    w = si.WORKLOADS["tiny_fwd_f32"]
    x = si.full_inputs(w)
    N = w.B * w.H
    r = lambda a: a.reshape(N, *a.shape[2:])  # noqa: E731
    meta = np.broadcast_to(x["meta_k"][None], (w.B,) + x["meta_k"].shape).reshape(N, w.n_meta, w.d)
    out = oracle.lizard_fwd(r(x["q"]), r(x["k"]), r(x["v"]), r(x["log_g"]), meta, w.window, w.alpha)
    snap = np.load(os.path.join(os.path.dirname(__file__), "golden", "oracle_tiny_regression.npz"))
    assert np.allclose(out["y"][:, ::7], snap["y"], rtol=0, atol=1e-13)
    assert np.allclose(out["lse"], snap["lse"], rtol=0, atol=1e-13)
    assert np.allclose(out["state"], snap["state"], rtol=0, atol=1e-13)

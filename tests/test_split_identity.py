"""The algebra the split forward (lizard_attn_fwd_split) relies on, checked on
the oracle's recurrence alone (no GPU): the gated recurrence is linear in its
state (de section 2 "Kernkomponenten" item 1: S_t = diag(g_t) S_{t-1} +
k_t v_t^T), so a sequence cut into segments run from a zero state gives the
one-pass result once

  S_in(s+1) = diag(exp(A_s)) S_in(s) + dS_s          (A_s: the segment's log-gate total)
  o_t      += (q_t * exp(R_t))^T S_in(s)              (R_t: log-gates from the segment start to t)

and the chunk-start states the training forward keeps are the recurrence's
states at multiples of 64 tokens.  These are statements about the method,
pinned here against the oracle's step-by-step recurrence on small inputs."""
import numpy as np
import pytest

import oracle


def _inputs(seed, N=2, L=300, d=8, mu=1.5, sd=1.5):
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((N, L, d)) * 0.5 for _ in range(3))
    log_g = oracle.log_sigmoid(rng.normal(mu, sd, size=(N, L, d)))
    return q, k, v, log_g


@pytest.mark.parametrize("bounds", [(0, 64, 192, 300), (0, 128, 300), (0, 1, 2, 299, 300)])
def test_segments_chained_by_the_state_scan_give_the_one_pass_result(bounds):
    q, k, v, log_g = _inputs(1)
    o_full, S_full = oracle.gla_recurrent(q, k, v, log_g)
    S_in = np.zeros_like(S_full)
    o = np.empty_like(o_full)
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        sl = slice(lo, hi)
        o_seg, dS = oracle.gla_recurrent(q[:, sl], k[:, sl], v[:, sl], log_g[:, sl])   # from a zero state
        R = np.cumsum(log_g[:, sl], axis=1)                                           # inclusive, from lo
        o[:, sl] = o_seg + np.einsum("nti,nij->ntj", q[:, sl] * np.exp(R), S_in)
        S_in = np.exp(R[:, -1])[:, :, None] * S_in + dS                               # the scan
    assert np.allclose(o, o_full, rtol=1e-12, atol=1e-12)
    assert np.allclose(S_in, S_full, rtol=1e-12, atol=1e-12)


def test_a_segment_from_its_incoming_state_needs_no_correction():
    """Segment 0 of the split runs from state_in itself (a continued sequence):
    its outputs and final state are then complete."""
    q, k, v, log_g = _inputs(2)
    S0 = np.random.default_rng(3).standard_normal((2, 8, 8))
    o_full, S_full = oracle.gla_recurrent(q, k, v, log_g, S0)
    o_a, S_a = oracle.gla_recurrent(q[:, :100], k[:, :100], v[:, :100], log_g[:, :100], S0)
    o_b, S_b = oracle.gla_recurrent(q[:, 100:], k[:, 100:], v[:, 100:], log_g[:, 100:], S_a)
    assert np.allclose(np.concatenate([o_a, o_b], 1), o_full, rtol=1e-12, atol=1e-12)
    assert np.allclose(S_b, S_full, rtol=1e-12, atol=1e-12)


def test_the_correction_vanishes_below_the_cut():
    """Past a decay of 2^-128 from the segment start the incoming state's term
    is below 2^-128 of |q| |S_in| d: the chunks the correction leaves alone."""
    q, k, v, log_g = _inputs(4, mu=-1.0, sd=0.5)     # about 2^-1.9 per token
    R2 = np.cumsum(log_g, axis=1) / np.log(2)          # log2 decay from the start
    S_in = np.random.default_rng(5).standard_normal((2, 8, 8))
    term = np.abs(np.einsum("nti,nij->ntj", q * np.exp(R2 * np.log(2)), S_in))
    bound = np.abs(q).max() * np.abs(S_in).max() * 8 * 2.0 ** -128
    cut = R2.max(axis=2) < -128                        # every dimension below the cut
    assert cut.any()
    assert (term[cut] <= bound).all()


def test_chunk_start_states_are_prefix_states():
    """What the training forward keeps: S after 64c tokens is the state the
    recurrence carries into chunk c (so chunk c's outputs follow from it)."""
    q, k, v, log_g = _inputs(6, L=200)
    o_full, _ = oracle.gla_recurrent(q, k, v, log_g)
    for c in (1, 2, 3):
        t = 64 * c
        _, S_c = oracle.gla_recurrent(q[:, :t], k[:, :t], v[:, :t], log_g[:, :t])
        o_rest, _ = oracle.gla_recurrent(q[:, t:], k[:, t:], v[:, t:], log_g[:, t:], S_c)
        assert np.allclose(o_rest, o_full[:, t:], rtol=1e-12, atol=1e-12)

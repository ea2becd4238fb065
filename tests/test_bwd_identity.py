"""The algebra the backward gate kernel uses for the boundary term of dlog_g,
checked on the oracle's step-by-step recurrence and its reverse mode (no GPU).

For chunk c ending before token e, the terms q_u.dq_u - k_u.dk_u of all
tokens u >= e sum, per key dimension i, to x_i = sum_j S_{c+1}[i][j] G[i][j],
with S_{c+1} the state after token e-1 and G = sum_{u>=e} diag(prod_{e<=v<=u}
g_v) q_u dO_u^T the state gradient carried into the chunk.  Because the
recurrence gives S_{c+1} = diag(e^{B}) S_c + sum_s diag(e^{B - beta_s}) k_s v_s^T
over the chunk's tokens s (B its log-gate total, beta_s the inclusive prefix;
de section 2 "Kernkomponenten" item 1 for the recurrence), x_i is also

  e^{B_i} sum_j S_c[i][j] G[i][j] + sum_s k_si e^{B_i - beta_si} (G v_s)_i,

which needs only the chunk's own state and operands."""
import numpy as np

import oracle


def _inputs(seed, N=2, L=200, d=8, mu=1.5, sd=1.5):
    rng = np.random.default_rng(seed)
    q, k, v, do = (rng.standard_normal((N, L, d)) * 0.5 for _ in range(4))
    log_g = oracle.log_sigmoid(rng.normal(mu, sd, size=(N, L, d)))
    return q, k, v, log_g, do


def _carried_gradient(q, log_g, do, e):
    """G for the boundary before token e, from its defining sum."""
    N, L, d = q.shape
    G = np.zeros((N, d, do.shape[-1]))
    for u in range(e, L):
        decay = np.exp(log_g[:, e:u + 1].sum(axis=1))          # prod_{e<=v<=u} g_v
        G += (decay * q[:, u])[:, :, None] * do[:, u, None, :]
    return G


def test_later_tokens_sum_to_the_boundary_product():
    q, k, v, log_g, do = _inputs(1)
    dq, dk, _, dlg = oracle.gla_bwd_recurrent(q, k, v, log_g, do)
    for e in (64, 128, 150):
        lhs = (q[:, e:] * dq[:, e:] - k[:, e:] * dk[:, e:]).sum(axis=1)
        _, S = oracle.gla_recurrent(q[:, :e], k[:, :e], v[:, :e], log_g[:, :e])   # state after token e-1
        rhs = (S * _carried_gradient(q, log_g, do, e)).sum(axis=2)
        assert np.allclose(lhs, rhs, rtol=1e-10, atol=1e-12), e
        # and the suffix form of dlog_g it completes (token e-1 sees exactly
        # its own term plus the boundary product)
        own = q[:, e - 1] * dq[:, e - 1] - k[:, e - 1] * dk[:, e - 1]
        assert np.allclose(dlg[:, e - 1], own + rhs, rtol=1e-10, atol=1e-12), e


def test_boundary_product_from_the_chunk_start_state():
    q, k, v, log_g, _ = _inputs(2, L=64)
    rng = np.random.default_rng(3)
    S_c = rng.standard_normal((2, 8, 8))
    G = rng.standard_normal((2, 8, 8))
    _, S_next = oracle.gla_recurrent(q, k, v, log_g, S_c)
    direct = (S_next * G).sum(axis=2)
    beta = np.cumsum(log_g, axis=1)                            # inclusive prefix
    B = beta[:, -1]
    Gv = np.einsum("nij,nsj->nsi", G, v)                       # (G v_s)_i
    split = np.exp(B) * (S_c * G).sum(axis=2) + (k * np.exp(B[:, None] - beta) * Gv).sum(axis=1)
    assert np.allclose(direct, split, rtol=1e-12, atol=1e-12)
    # a wrong reading (the decay taken from the chunk start) fails
    wrong = np.exp(B) * (S_c * G).sum(axis=2) + (k * np.exp(beta) * Gv).sum(axis=1)
    assert not np.allclose(direct, wrong, rtol=1e-6)

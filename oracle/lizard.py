"""Float64 definitions of the Lizard hybrid attention layer (the oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Every function takes float64 numpy arrays with a leading "slice" axis N
(one slice = one (batch, head) pair): q, k [N, L, dk], v [N, L, dv],
log_g [N, L, dk] (log of the sigmoid gate, <= 0), meta_k [N, m, dk].

What the pages fix and what is read into them
---------------------------------------------
Citations name the page ("Lizard" explainer on gist.science in German (de),
Italian (it) or Portuguese (pt)) and its section.

* Gate.  Gamma_i = sigmoid(W_gamma x_i): de §2 "Kernkomponenten" item 1;
  it §2 "Architettura Ibrida".  Reading: one gate value per token and per key
  dimension; the layer receives log(Gamma) in float32, so log_g <= 0.
* Gated linear attention.  The pages describe a data-adaptive recurrent
  structure whose hidden state is updated incrementally with O(1) memory and
  whose decay of past information the gate controls (de §2 item 1; pt §2A).
  Reading: S_t = diag(g_t) S_{t-1} + k_t v_t^T, o_t = S_t^T q_t, S_{-1} = 0
  (the token's own pair is not decayed and o_t includes token t).  No
  feature map and no normaliser are applied (the pages define none).
* Anchor window.  A local sliding window of width w plus m learnable
  meta-memory tokens acting as attention sinks that steady the distribution
  without contributing to the output (de §2 item 2; it §2 "Anchor Window
  Attention"; pt §2A).  Reading: token keys s in [max(0, t-w+1), t]
  (w keys including t, so a ring of exactly w slots holds them); the sink
  logits enter the softmax maximum and denominator with zero values; logits
  are scaled by 1/sqrt(dk) by default; no positional encoding in either
  branch (the gate replaces RoPE, de §2 item 1).
* Hybrid output.  Y = Y_gate + alpha * Y_anchor (de §2 item 3; pt §2A).
* Training.  The layer is trained end to end (de §2 "Trainingsprozess"),
  so gradients of L = sum(dY * Y) are defined for q, k, v, log_g and the
  meta keys; alpha and the softmax scale are constants.
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import numpy as np

# ---------------------------------------------------------------------------
# Gated linear attention branch
# ---------------------------------------------------------------------------


def gla_recurrent(q, k, v, log_g, state0: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Step-by-step recurrence S_t = diag(g_t) S_{t-1} + k_t v_t^T, o_t = S_t^T q_t.

    The primary definition of the gated branch (de §2 "Kernkomponenten"
    item 1: recurrent structure, incremental hidden-state updates).
    Returns (o [N, L, dv], S_final [N, dk, dv]).
    """
    N, L, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((N, dk, dv)) if state0 is None else np.array(state0, dtype=np.float64, copy=True)
    o = np.empty((N, L, dv))
    for t in range(L):
        S = np.exp(log_g[:, t, :])[:, :, None] * S + k[:, t, :, None] * v[:, t, None, :]
        o[:, t, :] = np.einsum("ni,nij->nj", q[:, t, :], S)
    return o, S


def gla_quadratic(q, k, v, log_g) -> np.ndarray:
    """Masked-decay (parallel) form of the same recurrence, S_{-1} = 0.

    With b_t = sum_{u<=t} log_g_u, unrolling the recurrence gives
    o_t = sum_{s<=t} (sum_i q_ti k_si exp(b_ti - b_si)) v_s.  Every exponent
    is <= 0, so nothing overflows.
    """
    N, L, dk = q.shape
    b = np.cumsum(log_g, axis=1)
    o = np.empty((N, L, v.shape[-1]))
    for t in range(L):
        decay = np.exp(b[:, t:t + 1, :] - b[:, :t + 1, :])  # [N, t+1, dk]
        a = np.einsum("ni,nsi->ns", q[:, t, :], k[:, :t + 1, :] * decay)
        o[:, t, :] = np.einsum("ns,nsj->nj", a, v[:, :t + 1, :])
    return o


def gla_chunked(q, k, v, log_g, chunk: int, state0: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Chunk form of the recurrence (log-space prefix sums inside each chunk).

    The log-space reparametrisation folds cumulative gate terms into the
    query and key sides so the chunk work becomes matrix products (de §2
    "Hardware-bewusster Algorithmus"; it §2 "Algoritmo Consapevole
    dell'Hardware").  For chunk c starting at t0 with beta_t = sum of log_g
    over [t0, t] and B_c = beta at the chunk's last row:
      o_t = (q_t * e^{beta_t})^T S_c + sum_{t0<=s<=t} (sum_i q_ti k_si e^{beta_ti - beta_si}) v_s
      S_{c+1} = diag(e^{B_c}) S_c + sum_s (k_s * e^{B_c - beta_s}) v_s^T
    All exponents are <= 0.  Returns (o, S_final).
    """
    N, L, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((N, dk, dv)) if state0 is None else np.array(state0, dtype=np.float64, copy=True)
    o = np.empty((N, L, dv))
    for t0 in range(0, L, chunk):
        t1 = min(L, t0 + chunk)
        qc, kc, vc = q[:, t0:t1], k[:, t0:t1], v[:, t0:t1]
        beta = np.cumsum(log_g[:, t0:t1], axis=1)  # [N, C, dk]
        Bc = beta[:, -1, :]  # [N, dk]
        inter = np.einsum("nti,nij->ntj", qc * np.exp(beta), S)
        C = t1 - t0
        A = np.zeros((N, C, C))
        for t in range(C):
            dec = np.exp(beta[:, t:t + 1, :] - beta[:, :t + 1, :])
            A[:, t, :t + 1] = np.einsum("ni,nsi->ns", qc[:, t], kc[:, :t + 1] * dec)
        o[:, t0:t1] = inter + np.einsum("nts,nsj->ntj", A, vc)
        S = np.exp(Bc)[:, :, None] * S + np.einsum("nsi,nsj->nij", kc * np.exp(Bc[:, None, :] - beta), vc)
    return o, S


# ---------------------------------------------------------------------------
# Anchor branch: sliding window plus meta-memory sinks
# ---------------------------------------------------------------------------


def _window_start(t: int, w: int) -> int:
    return max(0, t - w + 1)


def anchor_window(q, k, v, meta_k, w: int, scale: Optional[float] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax over the w most recent keys (incl. t) plus m sink keys.

    de §2 "Kernkomponenten" item 2; it §2 "Anchor Window Attention": the sink
    logits scale * q_t . mu_i enter the softmax's maximum and denominator; their
    values are zero, so they only absorb weight.  Returns
    (Y_anchor [N, L, dv], lse [N, L]) with lse = log of the full denominator
    (window + sinks) including the running maximum.
    """
    N, L, dk = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(dk)
    y = np.empty((N, L, v.shape[-1]))
    lse = np.empty((N, L))
    for t in range(L):
        s0 = _window_start(t, w)
        z = scale * np.einsum("ni,nsi->ns", q[:, t], k[:, s0:t + 1])  # [N, n_t]
        zeta = scale * np.einsum("ni,nmi->nm", q[:, t], meta_k)  # [N, m]
        M = np.maximum(z.max(axis=1), zeta.max(axis=1) if zeta.shape[1] else -np.inf)
        ez = np.exp(z - M[:, None])
        den = ez.sum(axis=1) + np.exp(zeta - M[:, None]).sum(axis=1)
        y[:, t] = np.einsum("ns,nsj->nj", ez, v[:, s0:t + 1]) / den[:, None]
        lse[:, t] = M + np.log(den)
    return y, lse


def anchor_bruteforce(q, k, v, meta_k, w: int, scale: Optional[float] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Same result by brute force: the full L x (L + m) logit matrix, token
    columns outside the window set to -inf, sink columns always open, a row
    softmax, then a product with [V; 0]."""
    N, L, dk = q.shape
    m = meta_k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(dk)
    Z = scale * np.einsum("nti,nsi->nts", q, k)
    t_idx = np.arange(L)[:, None]
    s_idx = np.arange(L)[None, :]
    inside = (s_idx <= t_idx) & (s_idx >= t_idx - w + 1)
    Z = np.where(inside[None], Z, -np.inf)
    Zs = scale * np.einsum("nti,nmi->ntm", q, meta_k)
    full = np.concatenate([Z, Zs], axis=2)
    M = full.max(axis=2, keepdims=True)
    E = np.exp(full - M)
    den = E.sum(axis=2, keepdims=True)
    P = E / den
    vals = np.concatenate([v, np.zeros((N, m, v.shape[-1]))], axis=1)
    return np.einsum("ntu,nuj->ntj", P, vals), (M + np.log(den))[..., 0]


# ---------------------------------------------------------------------------
# The hybrid layer
# ---------------------------------------------------------------------------


def lizard_fwd(q, k, v, log_g, meta_k, w: int, alpha: float, scale: Optional[float] = None):
    """Y = Y_gate + alpha * Y_anchor (de §2 "Kernkomponenten" item 3).

    Returns a dict with y, y_gate, y_anchor, lse and state (S_{L-1}).
    """
    o, S = gla_recurrent(q, k, v, log_g)
    ya, lse = anchor_window(q, k, v, meta_k, w, scale)
    return {"y": o + alpha * ya, "y_gate": o, "y_anchor": ya, "lse": lse, "state": S}


def lizard_decode_step(state, k_ring, v_ring, pos: int, q_t, k_t, v_t, log_g_t, meta_k, w: int, alpha: float,
                       scale: Optional[float] = None):
    """One constant-memory inference step at absolute position ``pos``.

    Constant memory by incremental hidden-state updates (de §2 item 1; de §4
    "Effizienz").  The state [N, dk, dv] and the rings [N, w, d] are updated
    and returned as new arrays (inputs untouched).  Token p lives in ring
    slot p mod w; the incoming token is written first, then the window
    max(0, pos-w+1)..pos is read.  Returns (y [N, dv], state, k_ring, v_ring).
    """
    N, dk = q_t.shape
    if scale is None:
        scale = 1.0 / math.sqrt(dk)
    S = np.exp(log_g_t)[:, :, None] * state + k_t[:, :, None] * v_t[:, None, :]
    o = np.einsum("ni,nij->nj", q_t, S)
    kr = np.array(k_ring, copy=True)
    vr = np.array(v_ring, copy=True)
    kr[:, pos % w] = k_t
    vr[:, pos % w] = v_t
    slots = [p % w for p in range(_window_start(pos, w), pos + 1)]
    z = scale * np.einsum("ni,nsi->ns", q_t, kr[:, slots])
    zeta = scale * np.einsum("ni,nmi->nm", q_t, meta_k)
    M = np.maximum(z.max(axis=1), zeta.max(axis=1) if zeta.shape[1] else -np.inf)
    ez = np.exp(z - M[:, None])
    den = ez.sum(axis=1) + np.exp(zeta - M[:, None]).sum(axis=1)
    ya = np.einsum("ns,nsj->nj", ez, vr[:, slots]) / den[:, None]
    return o + alpha * ya, S, kr, vr


# ---------------------------------------------------------------------------
# Gradients (loss L = sum(dY * Y))
# ---------------------------------------------------------------------------


def gla_bwd_recurrent(q, k, v, log_g, do):
    """Reverse-mode differentiation of the recurrence, step by step.

    Forward stores every S_t; backward runs t = L-1 .. 0 with the adjoint
    dS_t = diag(g_{t+1}) dS_{t+1} + q_t do_t^T and
      dq_t = S_t do_t,  dk_t = dS_t v_t,  dv_t = dS_t^T k_t,
      dlog_g_t = g_t * rowsum(dS_t * S_{t-1}).
    Returns (dq, dk, dv, dlog_g).
    """
    N, L, dk = q.shape
    dv_ = v.shape[-1]
    g = np.exp(log_g)
    S_all = np.empty((L + 1, N, dk, dv_))  # S_all[t+1] = S_t, S_all[0] = S_{-1} = 0
    S_all[0] = 0.0
    for t in range(L):
        S_all[t + 1] = g[:, t, :, None] * S_all[t] + k[:, t, :, None] * v[:, t, None, :]
    dq = np.empty_like(q)
    dkk = np.empty_like(k)
    dvv = np.empty_like(v)
    dlg = np.empty_like(log_g)
    dS = np.zeros((N, dk, dv_))
    for t in range(L - 1, -1, -1):
        dS = dS + q[:, t, :, None] * do[:, t, None, :]
        St = S_all[t + 1]
        dq[:, t] = np.einsum("nij,nj->ni", St, do[:, t])
        dkk[:, t] = np.einsum("nij,nj->ni", dS, v[:, t])
        dvv[:, t] = np.einsum("nij,ni->nj", dS, k[:, t])
        dlg[:, t] = g[:, t] * np.einsum("nij,nij->ni", dS, S_all[t])
        dS = g[:, t, :, None] * dS
    return dq, dkk, dvv, dlg


def anchor_bwd(q, k, v, meta_k, w: int, dya, scale: Optional[float] = None):
    """Gradient of sum(dya * Y_anchor) by the explicit softmax derivative.

    For query t with probabilities P over window keys and sinks:
    dP_j = dya_t . v_j (window; zero for sinks, whose values are zero),
    D_t = sum_j P_j dP_j, dZ_j = P_j (dP_j - D_t);
    dq_t = scale (sum_j dZ_j k_j + sum_i dZ_i mu_i), dk_j += scale dZ_j q_t,
    dv_j += P_j dya_t, dmu_i += scale dZ_i q_t.
    Returns (dq, dk, dv, dmeta [N, m, dk]).
    """
    N, L, dk = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(dk)
    dq = np.zeros_like(q)
    dkk = np.zeros_like(k)
    dvv = np.zeros_like(v)
    dmu = np.zeros_like(meta_k)
    for t in range(L):
        s0 = _window_start(t, w)
        z = scale * np.einsum("ni,nsi->ns", q[:, t], k[:, s0:t + 1])
        zeta = scale * np.einsum("ni,nmi->nm", q[:, t], meta_k)
        full = np.concatenate([z, zeta], axis=1)
        M = full.max(axis=1, keepdims=True)
        E = np.exp(full - M)
        P = E / E.sum(axis=1, keepdims=True)
        n = t + 1 - s0
        Pw, Ps = P[:, :n], P[:, n:]
        dP = np.einsum("nj,nsj->ns", dya[:, t], v[:, s0:t + 1])
        D = (Pw * dP).sum(axis=1, keepdims=True)
        dZw = Pw * (dP - D)
        dZs = -Ps * D
        dq[:, t] = scale * (np.einsum("ns,nsi->ni", dZw, k[:, s0:t + 1]) + np.einsum("nm,nmi->ni", dZs, meta_k))
        dkk[:, s0:t + 1] += scale * dZw[:, :, None] * q[:, t, None, :]
        dvv[:, s0:t + 1] += Pw[:, :, None] * dya[:, t, None, :]
        dmu += scale * dZs[:, :, None] * q[:, t, None, :]
    return dq, dkk, dvv, dmu


def lizard_bwd(q, k, v, log_g, meta_k, w: int, alpha: float, dy, scale: Optional[float] = None):
    """Gradients of sum(dy * Y) for Y = Y_gate + alpha * Y_anchor.

    Returns a dict: dq, dk, dv, dlog_g [N, L, dk] and dmeta [N, m, dk] (per
    slice; the layer's meta-key gradient sums these over the batch).
    """
    gq, gk, gv, glg = gla_bwd_recurrent(q, k, v, log_g, dy)
    aq, ak, av, amu = anchor_bwd(q, k, v, meta_k, w, alpha * dy, scale)
    return {"dq": gq + aq, "dk": gk + ak, "dv": gv + av, "dlog_g": glg, "dmeta": amu,
            "dq_gate": gq, "dk_gate": gk}


def lizard_fwd_continue(q, k, v, log_g, meta_k, w: int, alpha: float, state_in=None, k_halo=None, v_halo=None,
                        scale: Optional[float] = None):
    """A segment that continues a sequence (chunked prefill; de §2 item 1 and
    §4 "Effizienz": the recurrent state carries the whole past).  The gated
    branch starts from state_in (S before the segment's first token); the
    window of the segment's first tokens reaches back into k_halo / v_halo
    [N, h, d], the h tokens just before the segment.  Returns y, y_anchor,
    lse of the segment's tokens and its final state."""
    o, S = gla_recurrent(q, k, v, log_g, state_in)
    h = 0 if k_halo is None else k_halo.shape[1]
    if h:
        qq = np.concatenate([np.zeros((q.shape[0], h, q.shape[2])), q], axis=1)   # halo queries: unused rows
        ya, lse = anchor_window(qq, np.concatenate([k_halo, k], axis=1), np.concatenate([v_halo, v], axis=1),
                                meta_k, w, scale)
        ya, lse = ya[:, h:], lse[:, h:]
    else:
        ya, lse = anchor_window(q, k, v, meta_k, w, scale)
    return {"y": o + alpha * ya, "y_anchor": ya, "lse": lse, "state": S}


# ---------------------------------------------------------------------------
# Gate from its logits
# ---------------------------------------------------------------------------


def log_sigmoid(x):
    """log Gamma for the gate Gamma = sigmoid(x), x = W_gamma x_i the gate
    projection's output (de §2 "Kernkomponenten" item 1; it §2 "Architettura
    Ibrida").  Written as min(x, 0) - log(1 + e^{-|x|}): no overflow for
    either sign, and the small tail -e^{-x} for large x is kept by log1p."""
    x = np.asarray(x, dtype=np.float64)
    return np.minimum(x, 0.0) - np.log1p(np.exp(-np.abs(x)))


def lizard_fwd_logit(q, k, v, gate_logit, meta_k, w: int, alpha: float, scale: Optional[float] = None):
    """The layer fed with gate logits: log_g = log_sigmoid(gate_logit)."""
    return lizard_fwd(q, k, v, log_sigmoid(gate_logit), meta_k, w, alpha, scale)


def lizard_bwd_logit(q, k, v, gate_logit, meta_k, w: int, alpha: float, dy, scale: Optional[float] = None):
    """Gradients of sum(dy * Y) with the gate given by its logits.  Chain
    rule through the log-sigmoid: d/dx log sigmoid(x) = 1 - sigmoid(x) =
    sigmoid(-x) = exp(log_sigmoid(-x)).  Adds "dgate_logit" to lizard_bwd's
    dict."""
    r = lizard_bwd(q, k, v, log_sigmoid(gate_logit), meta_k, w, alpha, dy, scale)
    r["dgate_logit"] = r["dlog_g"] * np.exp(log_sigmoid(-np.asarray(gate_logit, dtype=np.float64)))
    return r


def lizard_decode_step_logit(state, k_ring, v_ring, pos: int, q_t, k_t, v_t, gate_logit_t, meta_k, w: int,
                             alpha: float, scale: Optional[float] = None):
    """lizard_decode_step with the token's gate given by its logits."""
    return lizard_decode_step(state, k_ring, v_ring, pos, q_t, k_t, v_t, log_sigmoid(gate_logit_t), meta_k, w, alpha,
                              scale)


# ---------------------------------------------------------------------------
# Stage-1 attention transfer
# ---------------------------------------------------------------------------


def softmax_attention_causal(q, k, v, scale: Optional[float] = None):
    """The teacher of stage 1: softmax attention over every earlier token
    (stage 1 fits the layer to the outputs of the attention it replaces; de §2
    "Trainingsprozess", it §2 "Fase di Addestramento").  Returns (y, lse)."""
    N, L, dk = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(dk)
    Z = scale * np.einsum("nti,nsi->nts", q, k)
    Z = np.where(np.tril(np.ones((L, L), dtype=bool))[None], Z, -np.inf)
    M = Z.max(axis=2, keepdims=True)
    E = np.exp(Z - M)
    den = E.sum(axis=2, keepdims=True)
    return np.einsum("nts,nsj->ntj", E, v) / den, (M + np.log(den))[:, :, 0]


def transfer_loss(y, y_teacher):
    """mean((y - y_teacher)^2) over all elements, and its gradient
    2 (y - y_teacher) / N with respect to y."""
    e = np.asarray(y, dtype=np.float64) - np.asarray(y_teacher, dtype=np.float64)
    return float((e * e).sum() / e.size), 2.0 * e / e.size


def stage1_step(q, k, v, log_g, meta_k, w: int, alpha: float, scale: Optional[float] = None):
    """One synthetic stage-1 step on the same q, k, v: the teacher's outputs
    are the fixed target, the layer's outputs are fitted to them.  Returns the
    loss and the layer's gradients (dq, dk, dv, dlog_g, dmeta; in stage 1 the
    gates and the sink keys are what trains)."""
    yt, _ = softmax_attention_causal(q, k, v, scale)
    y = lizard_fwd(q, k, v, log_g, meta_k, w, alpha, scale)["y"]
    loss, dy = transfer_loss(y, yt)
    g = lizard_bwd(q, k, v, log_g, meta_k, w, alpha, dy, scale)
    g["loss"] = loss
    g["y_teacher"] = yt
    g["y"] = y
    return g

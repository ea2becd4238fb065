"""Pins of the float64 oracle against facts the mathematics fixes.

Each pin takes an oracle module ``O`` (normally ``oracle.lizard``) and
returns the largest violation it measured; the tests assert that it is
below a tolerance, and the mutation test checks that deliberately broken
copies of the oracle fail at least one pin.  None of these re-types the
oracle's own formula: each compares against a closed form, a hand-worked
case, a library routine (torch on CPU in float64), brute force or finite
differences.
"""
from __future__ import annotations

import math

import numpy as np

TOL = 1e-10


def _rand(seed, N=2, L=37, d=8, m=3, gate_scale=0.4):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((N, L, d)) * 0.6
    k = rng.standard_normal((N, L, d)) * 0.6
    v = rng.standard_normal((N, L, d))
    lg = -np.abs(rng.standard_normal((N, L, d))) * gate_scale
    mu = rng.standard_normal((N, m, d)) * 0.6
    return q, k, v, lg, mu


def _rel(a, b):
    return float(np.abs(a - b).max() / max(1e-300, np.abs(b).max()))


# --- gated branch ---------------------------------------------------------

def p1_recurrent_equals_quadratic(O):
    q, k, v, lg, _ = _rand(1)
    o_r, _ = O.gla_recurrent(q, k, v, lg)
    o_q = O.gla_quadratic(q, k, v, lg)
    return _rel(o_r, o_q)


def p2_unit_gate_is_causal_linear_attention(O):
    """g == 1: o = tril(Q K^T) V and the final state is sum_t k_t v_t^T."""
    q, k, v, _, _ = _rand(2)
    lg = np.zeros_like(q)
    o, S = O.gla_recurrent(q, k, v, lg)
    ref = np.tril(q @ k.transpose(0, 2, 1)) @ v
    Sref = k.transpose(0, 2, 1) @ v
    oq = O.gla_quadratic(q, k, v, lg)
    return max(_rel(o, ref), _rel(S, Sref), _rel(oq, ref))


def p3_hard_reset_gate(O):
    """log g = -1000 (g == 0 in float64): o_t = (q_t . k_t) v_t."""
    q, k, v, _, _ = _rand(3)
    lg = np.full_like(q, -1000.0)
    ref = (q * k).sum(-1, keepdims=True) * v
    o, _ = O.gla_recurrent(q, k, v, lg)
    oq = O.gla_quadratic(q, k, v, lg)
    oc, _ = O.gla_chunked(q, k, v, lg, 8)
    return max(_rel(o, ref), _rel(oq, ref), _rel(oc, ref))


def p4_scalar_gate_is_decayed_attention(O):
    """A constant scalar gate gamma: o = (Q K^T * Gamma) V, Gamma_ts = gamma^(t-s), s <= t."""
    q, k, v, _, _ = _rand(4)
    gamma = 0.83
    lg = np.full_like(q, math.log(gamma))
    L = q.shape[1]
    t = np.arange(L)[:, None]
    s = np.arange(L)[None, :]
    Gam = np.where(s <= t, gamma ** np.maximum(t - s, 0), 0.0)
    ref = ((q @ k.transpose(0, 2, 1)) * Gam) @ v
    o, _ = O.gla_recurrent(q, k, v, lg)
    return _rel(o, ref)


def p5_single_token(O):
    q, k, v, lg, _ = _rand(5, L=1)
    ref = (q * k).sum(-1, keepdims=True) * v
    o, S = O.gla_recurrent(q, k, v, lg)
    return max(_rel(o, ref), _rel(S, k[:, 0, :, None] * v[:, 0, None, :]))


def p6_two_tokens_by_hand(O):
    """L = 2, dk = dv = 2 worked by hand.

    q0 = (1, 2), k0 = (3, -1), v0 = (1, 0); q1 = (0, 1), k1 = (1, 1), v1 = (2, 3);
    g1 = (1/2, 1/4) (g0 is irrelevant: it multiplies the zero initial state).
    S0 = k0 v0^T = [[3, 0], [-1, 0]];  o0 = S0^T q0 = (3*1 + -1*2, 0) = (1, 0).
    S1 = diag(g1) S0 + k1 v1^T = [[1.5 + 2, 3], [-0.25 + 2, 3]] = [[3.5, 3], [1.75, 3]];
    o1 = S1^T q1 = (1.75, 3).
    """
    q = np.array([[[1.0, 2.0], [0.0, 1.0]]])
    k = np.array([[[3.0, -1.0], [1.0, 1.0]]])
    v = np.array([[[1.0, 0.0], [2.0, 3.0]]])
    lg = np.log(np.array([[[0.9, 0.7], [0.5, 0.25]]]))
    o, S = O.gla_recurrent(q, k, v, lg)
    ref_o = np.array([[[1.0, 0.0], [1.75, 3.0]]])
    ref_S = np.array([[[3.5, 3.0], [1.75, 3.0]]])
    oq = O.gla_quadratic(q, k, v, lg)
    return max(float(np.abs(o - ref_o).max()), float(np.abs(S - ref_S).max()), float(np.abs(oq - ref_o).max()))


def p7_chunk_form_any_chunk(O):
    q, k, v, lg, _ = _rand(7, L=45)
    o, S = O.gla_recurrent(q, k, v, lg)
    err = 0.0
    for C in (1, 8, 16, 64, 45):
        oc, Sc = O.gla_chunked(q, k, v, lg, C)
        err = max(err, _rel(oc, o), _rel(Sc, S))
    # with an initial state as well
    S0 = np.random.default_rng(70).standard_normal(S.shape)
    o2, S2 = O.gla_recurrent(q, k, v, lg, S0)
    oc2, Sc2 = O.gla_chunked(q, k, v, lg, 16, S0)
    return max(err, _rel(oc2, o2), _rel(Sc2, S2))


# --- anchor branch --------------------------------------------------------

def p8_window_equals_bruteforce(O):
    err = 0.0
    for w in (1, 3, 8, 64):
        q, k, v, _, mu = _rand(8 + w, L=29)
        y, lse = O.anchor_window(q, k, v, mu, w)
        yb, lb = O.anchor_bruteforce(q, k, v, mu, w)
        err = max(err, _rel(y, yb), _rel(lse, lb))
    return err


def p9_full_window_no_sinks_is_causal_sdpa(O):
    import torch

    q, k, v, _, _ = _rand(9, L=33)
    mu = np.zeros((q.shape[0], 0, q.shape[2]))
    y, _ = O.anchor_window(q, k, v, mu, w=40)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=True).numpy()
    return _rel(y, ref)


def p10_window_one_no_sinks_copies_value(O):
    q, k, v, _, _ = _rand(10)
    mu = np.zeros((q.shape[0], 0, q.shape[2]))
    y, lse = O.anchor_window(q, k, v, mu, w=1)
    d = q.shape[2]
    return max(_rel(y, v), _rel(lse, (q * k).sum(-1) / math.sqrt(d)))


def p11_uniform_weights(O):
    """k = 0 and mu = 0: every logit is 0, weights are 1/(n_t + m)."""
    q, _, v, _, mu = _rand(11, L=20)
    k = np.zeros_like(q)
    mu = np.zeros_like(mu)
    w, m = 6, mu.shape[1]
    y, lse = O.anchor_window(q, k, v, mu, w)
    ref = np.empty_like(y)
    ref_l = np.empty(y.shape[:2])
    for t in range(q.shape[1]):
        s0 = max(0, t - w + 1)
        n = t + 1 - s0
        ref[:, t] = v[:, s0:t + 1].sum(1) / (n + m)
        ref_l[:, t] = math.log(n + m)
    return max(_rel(y, ref), _rel(lse, ref_l))


def p11b_one_key_one_sink_by_hand(O):
    """t = 0 sees key 0 and one sink: y_0 = e^z / (e^z + e^zeta) v_0 with
    z = q0.k0/sqrt(d), zeta = q0.mu/sqrt(d).  q0 = (2, 0), k0 = (1, 0),
    mu = (-1, 0), d = 2: z = sqrt(2), zeta = -sqrt(2)."""
    q = np.array([[[2.0, 0.0]]])
    k = np.array([[[1.0, 0.0]]])
    v = np.array([[[3.0, -1.0]]])
    mu = np.array([[[-1.0, 0.0]]])
    y, lse = O.anchor_window(q, k, v, mu, w=4)
    r = math.sqrt(2.0)
    wgt = math.exp(r) / (math.exp(r) + math.exp(-r))
    return max(float(np.abs(y[0, 0] - wgt * v[0, 0]).max()),
               abs(float(lse[0, 0]) - math.log(math.exp(r) + math.exp(-r))))


def p12_mask_probes(O):
    """Position probes: q_t = 1/sqrt(d), gate 1, mu = 0, k = v = 0 except
    k_p = 1/sqrt(d), v_p = 1.  y_anchor_t != 0 iff p in window(t);
    y_gate_t != 0 iff t >= p.  Returns the number of mismatching positions."""
    L, d, w, m = 24, 4, 5, 2
    bad = 0
    for p in range(L):
        q = np.full((1, L, d), 1 / math.sqrt(d))
        k = np.zeros((1, L, d))
        v = np.zeros((1, L, d))
        k[0, p] = 1 / math.sqrt(d)
        v[0, p] = 1.0
        lg = np.zeros((1, L, d))
        mu = np.zeros((1, m, d))
        out = O.lizard_fwd(q, k, v, lg, mu, w, 0.5)
        t = np.arange(L)
        want_a = (p <= t) & (p >= t - w + 1)
        want_g = t >= p
        bad += int(((out["y_anchor"][0, :, 0] != 0) != want_a).sum())
        bad += int(((out["y_gate"][0, :, 0] != 0) != want_g).sum())
    return float(bad)


def p13_linear_in_alpha(O):
    q, k, v, lg, mu = _rand(13)
    y0 = O.lizard_fwd(q, k, v, lg, mu, 7, 0.0)
    y1 = O.lizard_fwd(q, k, v, lg, mu, 7, 0.7)
    o, _ = O.gla_recurrent(q, k, v, lg)
    ya, _ = O.anchor_bruteforce(q, k, v, mu, 7)
    return max(_rel(y0["y"], o), _rel(y1["y"], o + 0.7 * ya))


# --- decode ----------------------------------------------------------------

def _decode_run(O, q, k, v, lg, mu, w, alpha, L0):
    N, L, d = q.shape
    if L0 > 0:
        pre = O.lizard_fwd(q[:, :L0], k[:, :L0], v[:, :L0], lg[:, :L0], mu, w, alpha)
        S = pre["state"]
    else:
        S = np.zeros((N, d, v.shape[2]))
    kr = np.full((N, w, d), np.nan)  # slots not yet written must never be read
    vr = np.full((N, w, v.shape[2]), np.nan)
    for p in range(max(0, L0 - w), L0):
        kr[:, p % w] = k[:, p]
        vr[:, p % w] = v[:, p]
    ys = []
    for pos in range(L0, L):
        y, S, kr, vr = O.lizard_decode_step(S, kr, vr, pos, q[:, pos], k[:, pos], v[:, pos], lg[:, pos], mu, w, alpha)
        ys.append(y)
    return np.stack(ys, axis=1), S


def p14_decode_continues_prefill(O):
    q, k, v, lg, mu = _rand(14, L=30)
    full = O.lizard_fwd(q, k, v, lg, mu, 6, 0.5)
    yd, S = _decode_run(O, q, k, v, lg, mu, 6, 0.5, L0=17)
    return max(_rel(yd, full["y"][:, 17:]), _rel(S, full["state"]))


def p16_decode_from_empty(O):
    q, k, v, lg, mu = _rand(16, L=12)
    full = O.lizard_fwd(q, k, v, lg, mu, 5, 0.5)
    yd, _ = _decode_run(O, q, k, v, lg, mu, 5, 0.5, L0=0)
    return _rel(yd, full["y"])


# --- gradients --------------------------------------------------------------

def _loss(O, q, k, v, lg, mu, w, alpha, dy):
    return float((O.lizard_fwd(q, k, v, lg, mu, w, alpha)["y"] * dy).sum())


def p17_finite_differences(O, n_coords=12):
    """Central differences (h = 1e-6) on random coordinates of every input."""
    q, k, v, lg, mu = _rand(17, N=1, L=14, d=4, m=2)
    w, alpha = 4, 0.5
    dy = np.random.default_rng(170).standard_normal(v.shape)
    g = O.lizard_bwd(q, k, v, lg, mu, w, alpha, dy)
    args = {"q": q, "k": k, "v": v, "lg": lg, "mu": mu}
    grads = {"q": g["dq"], "k": g["dk"], "v": g["dv"], "lg": g["dlog_g"], "mu": g["dmeta"]}
    rng = np.random.default_rng(171)
    h = 1e-6
    worst = 0.0
    for name, arr in args.items():
        for _ in range(n_coords):
            idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
            plus = dict(args)
            minus = dict(args)
            plus[name] = arr.copy()
            plus[name][idx] += h
            minus[name] = arr.copy()
            minus[name][idx] -= h
            fd = (_loss(O, plus["q"], plus["k"], plus["v"], plus["lg"], plus["mu"], w, alpha, dy)
                  - _loss(O, minus["q"], minus["k"], minus["v"], minus["lg"], minus["mu"], w, alpha, dy)) / (2 * h)
            worst = max(worst, abs(fd - grads[name][idx]) / (1.0 + abs(fd)))
    return worst


def _torch_layer(q, k, v, lg, mu, w, alpha):
    """The layer in torch float64 on CPU: masked-decay form plus brute-force
    masked softmax with sink columns, so torch.autograd can differentiate it."""
    import torch

    N, L, d = q.shape
    b = torch.cumsum(lg, dim=1)
    diff = b[:, :, None, :] - b[:, None, :, :]  # [N, t, s, i]
    tri = torch.tril(torch.ones(L, L, dtype=torch.bool))
    E = torch.where(tri[None, :, :, None], torch.exp(torch.where(tri[None, :, :, None], diff, torch.zeros_like(diff))),
                    torch.zeros_like(diff))
    A = torch.einsum("nti,nsi,ntsi->nts", q, k, E)
    yg = A @ v
    sc = 1.0 / math.sqrt(d)
    Z = sc * (q @ k.transpose(1, 2))
    t = torch.arange(L)[:, None]
    s = torch.arange(L)[None, :]
    inside = (s <= t) & (s >= t - w + 1)
    Z = torch.where(inside[None], Z, torch.full_like(Z, -math.inf))
    Zs = sc * (q @ mu.transpose(1, 2))
    P = torch.softmax(torch.cat([Z, Zs], dim=2), dim=2)
    ya = P[:, :, :L] @ v
    return yg + alpha * ya


def p18_torch_autograd(O):
    import torch

    q, k, v, lg, mu = _rand(18, N=2, L=19, d=5, m=3)
    w, alpha = 6, 0.5
    dy = np.random.default_rng(180).standard_normal(v.shape)
    g = O.lizard_bwd(q, k, v, lg, mu, w, alpha, dy)
    ts = [torch.tensor(a, requires_grad=True) for a in (q, k, v, lg, mu)]
    y = _torch_layer(*ts, w, alpha)
    y.backward(torch.from_numpy(dy))
    fwd = O.lizard_fwd(q, k, v, lg, mu, w, alpha)["y"]
    errs = [_rel(fwd, y.detach().numpy())]
    for t_, key in zip(ts, ("dq", "dk", "dv", "dlog_g", "dmeta")):
        errs.append(_rel(g[key], t_.grad.numpy()))
    return max(errs)


def p19_log_gate_gradient_identity(O):
    """dlog_g_t = sum_{u>=t} (q_u * dq_u - k_u * dk_u) over the gated branch's
    dq, dk, and dlog_g_0 = 0 (the first gate multiplies the zero initial
    state)."""
    q, k, v, lg, _ = _rand(19, L=26)
    do = np.random.default_rng(190).standard_normal(v.shape)
    dq, dk, _, dlg = O.gla_bwd_recurrent(q, k, v, lg, do)
    db = q * dq - k * dk
    ref = np.flip(np.cumsum(np.flip(db, 1), 1), 1)
    return max(_rel(dlg, ref), float(np.abs(dlg[:, 0]).max()) / float(np.abs(dlg).max()))


def p20_sdpa_gradients(O):
    """m = 0, w >= L and a zero gated branch (q . k terms still feed the gate,
    so compare the anchor gradients alone) against autograd of torch's SDPA."""
    import torch

    q, k, v, _, _ = _rand(20, L=15)
    dya = np.random.default_rng(200).standard_normal(v.shape)
    mu = np.zeros((q.shape[0], 0, q.shape[2]))
    dq, dk, dv, _ = O.anchor_bwd(q, k, v, mu, 20, dya)
    ts = [torch.tensor(a, requires_grad=True) for a in (q, k, v)]
    y = torch.nn.functional.scaled_dot_product_attention(*ts, is_causal=True)
    y.backward(torch.from_numpy(dya))
    return max(_rel(dq, ts[0].grad.numpy()), _rel(dk, ts[1].grad.numpy()), _rel(dv, ts[2].grad.numpy()))



# --- gate given by its logits -------------------------------------------------

def p21_log_sigmoid(O):
    """log sigmoid against torch's float64 logsigmoid (a different
    implementation) over [-60, 60], the closed form log sigmoid(0) = -log 2,
    and the identity log sigmoid(x) - log sigmoid(-x) = x."""
    import torch

    x = np.concatenate([np.linspace(-60.0, 60.0, 4801), [0.0, 1e-12, -1e-12, 35.0, -35.0]])
    ref = torch.nn.functional.logsigmoid(torch.from_numpy(x)).numpy()
    got = O.log_sigmoid(x)
    err_lib = float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), 1e-300)))
    err_zero = abs(float(O.log_sigmoid(np.array(0.0))) + math.log(2.0))
    err_sym = float(np.abs(O.log_sigmoid(x) - O.log_sigmoid(-x) - x).max() / 60.0)
    return max(err_lib, err_zero, err_sym)


def p22_logit_gradients(O):
    """The layer fed with gate logits against torch autograd through
    torch's logsigmoid (forward output and every gradient, the logits'
    included)."""
    import torch

    q, k, v, _, mu = _rand(22, N=2, L=17, d=5, m=2)
    x = np.random.default_rng(220).normal(1.5, 2.0, size=q.shape)
    w, alpha = 5, 0.5
    dy = np.random.default_rng(221).standard_normal(v.shape)
    g = O.lizard_bwd_logit(q, k, v, x, mu, w, alpha, dy)
    fwd = O.lizard_fwd_logit(q, k, v, x, mu, w, alpha)["y"]
    ts = [torch.tensor(a, requires_grad=True) for a in (q, k, v, x, mu)]
    y = _torch_layer(ts[0], ts[1], ts[2], torch.nn.functional.logsigmoid(ts[3]), ts[4], w, alpha)
    y.backward(torch.from_numpy(dy))
    errs = [_rel(fwd, y.detach().numpy())]
    for t_, key in zip(ts, ("dq", "dk", "dv", "dgate_logit", "dmeta")):
        errs.append(_rel(g[key], t_.grad.numpy()))
    return max(errs)


def p23_logit_decode_continues_prefill(O):
    """Decoding token L-1 after a logit-fed prefill of L-1 tokens gives the
    logit-fed prefill's output at L-1 (and its final state)."""
    q, k, v, _, mu = _rand(23, N=2, L=21, d=6, m=2)
    x = np.random.default_rng(230).normal(2.0, 1.5, size=q.shape)
    w, alpha, L = 6, 0.5, q.shape[1]
    full = O.lizard_fwd_logit(q, k, v, x, mu, w, alpha)
    pre = O.lizard_fwd_logit(q[:, :L - 1], k[:, :L - 1], v[:, :L - 1], x[:, :L - 1], mu, w, alpha)
    kr = np.zeros((q.shape[0], w, q.shape[2]))
    vr = np.zeros_like(kr)
    for p in range(max(0, L - 1 - w), L - 1):
        kr[:, p % w] = k[:, p]
        vr[:, p % w] = v[:, p]
    y, S, _, _ = O.lizard_decode_step_logit(pre["state"], kr, vr, L - 1, q[:, L - 1], k[:, L - 1], v[:, L - 1],
                                            x[:, L - 1], mu, w, alpha)
    return max(_rel(y, full["y"][:, L - 1]), _rel(S, full["state"]))


def p24_segments_equal_one_pass(O):
    """A sequence processed as segments (each continuing from the previous
    one's state and its last min(w - 1, P) keys / values) equals one pass
    over the whole sequence, for split points inside and outside the first
    window and a window of one."""
    q, k, v, lg, mu = _rand(24, N=2, L=40, d=5, m=2)
    worst = 0.0
    for w, cuts in ((6, (3, 17, 18, 33)), (1, (1, 20)), (40, (7,))):
        whole = O.lizard_fwd(q, k, v, lg, mu, w, 0.5)
        bounds = (0,) + cuts + (q.shape[1],)
        S = None
        for a, b in zip(bounds[:-1], bounds[1:]):
            h = min(w - 1, a)
            kh = k[:, a - h:a] if h else None
            vh = v[:, a - h:a] if h else None
            seg = O.lizard_fwd_continue(q[:, a:b], k[:, a:b], v[:, a:b], lg[:, a:b], mu, w, 0.5, S, kh, vh)
            S = seg["state"]
            for key in ("y", "lse"):
                worst = max(worst, _rel(seg[key], whole[key][:, a:b]))
        worst = max(worst, _rel(S, whole["state"]))
    return worst


# --- stage-1 attention transfer -------------------------------------------------

def p25_teacher_is_sdpa(O):
    """The causal softmax teacher against torch's scaled_dot_product_attention
    (is_causal, float64), default and explicit scale, and its lse against a
    direct logsumexp."""
    import torch

    q, k, v, _, _ = _rand(25, L=23, d=7)
    errs = []
    for sc in (None, 0.3):
        y, lse = O.softmax_attention_causal(q, k, v, sc)
        ref = torch.nn.functional.scaled_dot_product_attention(
            *(torch.from_numpy(a) for a in (q, k, v)), is_causal=True, scale=sc).numpy()
        errs.append(_rel(y, ref))
        s = (1.0 / math.sqrt(q.shape[2])) if sc is None else sc
        Z = s * np.einsum("nti,nsi->nts", q, k)
        lref = np.array([[np.log(np.exp(Z[n, t, :t + 1]).sum()) for t in range(q.shape[1])] for n in range(q.shape[0])])
        errs.append(_rel(lse, lref))
    return max(errs)


def p26_stage1_finite_differences(O, n_coords=10):
    """The stage-1 gradients (teacher output held fixed) against central
    differences of mean((Y - Y_teacher)^2) on log-gates and sink keys."""
    q, k, v, lg, mu = _rand(26, N=1, L=12, d=4, m=2)
    w, alpha = 4, 0.5
    g = O.stage1_step(q, k, v, lg, mu, w, alpha)
    yt = g["y_teacher"]
    rng = np.random.default_rng(260)
    h = 1e-6
    worst = 0.0
    for name, arr, grad in (("lg", lg, g["dlog_g"]), ("mu", mu, g["dmeta"])):
        for _ in range(n_coords):
            idx = tuple(int(rng.integers(0, s_)) for s_ in arr.shape)
            vals = []
            for sign in (1.0, -1.0):
                a2 = arr.copy()
                a2[idx] += sign * h
                lg2, mu2 = (a2, mu) if name == "lg" else (lg, a2)
                y = O.lizard_fwd(q, k, v, lg2, mu2, w, alpha)["y"]
                vals.append(float(((y - yt) ** 2).mean()))
            fd = (vals[0] - vals[1]) / (2 * h)
            worst = max(worst, abs(fd - grad[idx]) / (1e-3 + abs(fd)))
    return worst


def p27_transfer_loss_by_hand(O):
    """The output-matching loss worked by hand.  y = (1, 2, -1, 0) against a
    zero teacher: the mean of the squares is (1 + 4 + 1 + 0) / 4 = 1.5 and the
    gradient 2 (y - y_T) / N is (0.5, 1, -0.5, 0).  y = (3, 1) against
    y_T = (1, 1): (4 + 0) / 2 = 2, gradient (2, 0).  A mean over every element
    of a [1, 2, 2, 1] tensor (4 elements): errors (1, -1, 2, 0) give 6 / 4 =
    1.5."""
    worst = 0.0
    cases = (
        (np.array([1.0, 2.0, -1.0, 0.0]), np.zeros(4), 1.5, np.array([0.5, 1.0, -0.5, 0.0])),
        (np.array([3.0, 1.0]), np.array([1.0, 1.0]), 2.0, np.array([2.0, 0.0])),
        (np.array([1.0, -1.0, 2.0, 0.0]).reshape(1, 2, 2, 1), np.zeros((1, 2, 2, 1)), 1.5,
         np.array([0.5, -0.5, 1.0, 0.0]).reshape(1, 2, 2, 1)),
    )
    for y, yt, loss_ref, g_ref in cases:
        loss, g = O.transfer_loss(y, yt)
        worst = max(worst, abs(loss - loss_ref) / loss_ref, float(np.abs(g - g_ref).max()))
    return worst

ALL_PINS = {
    "P1": p1_recurrent_equals_quadratic,
    "P2": p2_unit_gate_is_causal_linear_attention,
    "P3": p3_hard_reset_gate,
    "P4": p4_scalar_gate_is_decayed_attention,
    "P5": p5_single_token,
    "P6": p6_two_tokens_by_hand,
    "P7": p7_chunk_form_any_chunk,
    "P8": p8_window_equals_bruteforce,
    "P9": p9_full_window_no_sinks_is_causal_sdpa,
    "P10": p10_window_one_no_sinks_copies_value,
    "P11": p11_uniform_weights,
    "P11b": p11b_one_key_one_sink_by_hand,
    "P12": p12_mask_probes,
    "P13": p13_linear_in_alpha,
    "P14": p14_decode_continues_prefill,
    "P16": p16_decode_from_empty,
    "P17": p17_finite_differences,
    "P18": p18_torch_autograd,
    "P19": p19_log_gate_gradient_identity,
    "P20": p20_sdpa_gradients,
    "P21": p21_log_sigmoid,
    "P22": p22_logit_gradients,
    "P23": p23_logit_decode_continues_prefill,
    "P24": p24_segments_equal_one_pass,
    "P25": p25_teacher_is_sdpa,
    "P26": p26_stage1_finite_differences,
    "P27": p27_transfer_loss_by_hand,
}

# finite differences carry O(h^2) truncation and O(eps/h) rounding error
PIN_TOL = {k: TOL for k in ALL_PINS}
PIN_TOL["P17"] = 1e-6
PIN_TOL["P26"] = 1e-5
PIN_TOL["P12"] = 0.5  # an exact count of mismatches: must be 0

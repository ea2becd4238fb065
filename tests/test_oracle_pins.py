"""The oracle against facts outside itself (closed forms, hand-worked cases,
brute force, torch CPU routines, finite differences), and a check that
plausible mistakes planted in a copy of the oracle fail at least one pin."""
import os
import types

import numpy as np
import pytest

import oracle.lizard as O
from tests import oracle_pins as pins

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "lizard.py")


@pytest.fixture(autouse=True)
def _strict_fp():
    with np.errstate(over="raise", invalid="raise", divide="raise"):
        yield


@pytest.mark.parametrize("name", sorted(pins.ALL_PINS))
def test_pin(name):
    err = pins.ALL_PINS[name](O)
    assert err <= pins.PIN_TOL[name], f"{name}: {err}"


# Each mutation is a plausible slip: an off-by-one window, a dropped sink,
# decaying the token's own pair, a sign, a dropped alpha, a transposed
# operand, a missing scale, a wrong softmax factor, a reversed exponent,
# a wrong carry exponent, a wrong ring slot, a wrong state reset.
MUTATIONS = [
    ("window off by one", "return max(0, t - w + 1)", "return max(0, t - w)"),
    ("sink left out of the denominator",
     "den = ez.sum(axis=1) + np.exp(zeta - M[:, None]).sum(axis=1)\n        y[:, t]",
     "den = ez.sum(axis=1)\n        y[:, t]"),
    ("own pair decayed",
     "S = np.exp(log_g[:, t, :])[:, :, None] * S + k[:, t, :, None] * v[:, t, None, :]",
     "S = np.exp(log_g[:, t, :])[:, :, None] * (S + k[:, t, :, None] * v[:, t, None, :])"),
    ("log-gate gradient sign", "dlg[:, t] = g[:, t] *", "dlg[:, t] = -g[:, t] *"),
    ("alpha dropped in backward", "anchor_bwd(q, k, v, meta_k, w, alpha * dy, scale)",
     "anchor_bwd(q, k, v, meta_k, w, dy, scale)"),
    ("readout transposed", 'o[:, t, :] = np.einsum("ni,nij->nj", q[:, t, :], S)',
     'o[:, t, :] = np.einsum("nj,nij->ni", q[:, t, :], S)'),
    ("softmax scale missing", "    if scale is None:\n        scale = 1.0 / math.sqrt(dk)\n    y = np.empty",
     "    if scale is None:\n        scale = 1.0\n    y = np.empty"),
    ("value gradient uses dZ", "dvv[:, s0:t + 1] += Pw[:, :, None]", "dvv[:, s0:t + 1] += dZw[:, :, None]"),
    ("decay exponent reversed", "decay = np.exp(b[:, t:t + 1, :] - b[:, :t + 1, :])",
     "decay = np.exp(b[:, :t + 1, :] - b[:, t:t + 1, :])"),
    ("chunk carry exponent", "kc * np.exp(Bc[:, None, :] - beta)", "kc * np.exp(-beta)"),
    ("ring slot", "kr[:, pos % w] = k_t", "kr[:, (pos + 1) % w] = k_t"),
    ("key gradient misses the decay adjoint", "dS = g[:, t, :, None] * dS", "dS = dS"),
    ("sink gradient sign", "dZs = -Ps * D", "dZs = Ps * D"),
    ("logit gradient factor sigmoid(x)", "np.exp(log_sigmoid(-np.asarray(gate_logit, dtype=np.float64)))",
     "np.exp(log_sigmoid(np.asarray(gate_logit, dtype=np.float64)))"),
    ("log-sigmoid tail sign", "np.minimum(x, 0.0) - np.log1p(np.exp(-np.abs(x)))",
     "np.minimum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))"),
    ("decode logits not through the log-sigmoid", "log_sigmoid(gate_logit_t), meta_k, w, alpha,",
     "gate_logit_t, meta_k, w, alpha,"),
    ("continuation drops the incoming state", "o, S = gla_recurrent(q, k, v, log_g, state_in)",
     "o, S = gla_recurrent(q, k, v, log_g)"),
    ("teacher sees one future key", "Z = np.where(np.tril(np.ones((L, L), dtype=bool))[None], Z, -np.inf)",
     "Z = np.where(np.tril(np.ones((L, L), dtype=bool), 1)[None], Z, -np.inf)"),
    ("loss gradient without the factor 2", "return float((e * e).sum() / e.size), 2.0 * e / e.size",
     "return float((e * e).sum() / e.size), e / e.size"),
    ("loss summed instead of averaged", "return float((e * e).sum() / e.size), 2.0 * e / e.size",
     "return float((e * e).sum()), 2.0 * e / e.size"),
    ("continuation ignores the halo", "        ya, lse = ya[:, h:], lse[:, h:]\n",
     "        ya, lse = anchor_window(q, k, v, meta_k, w, scale)\n"),
]


def _mutant(old, new):
    src = open(ORACLE_SRC).read()
    assert src.count(old) == 1, f"mutation anchor not found once: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("label,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_fails_a_pin(label, old, new):
    M = _mutant(old, new)
    for name, fn in pins.ALL_PINS.items():
        try:
            with np.errstate(all="ignore"):
                err = fn(M)
        except Exception:
            return  # the mutant broke loudly: caught
        if not (err <= pins.PIN_TOL[name]):
            return
    pytest.fail(f"mutation '{label}' passed every pin")

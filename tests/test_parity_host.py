"""Host logic of the parity gates (no GPU): the scale-aware argmax gate accepts exact picks
and near ties within tau_t, and rejects a pick beyond tau_t, a pick outside the recorded
largest logits, and too many excused tokens."""
import math

import numpy as np
import pytest

from _parity import LogitRecord, argmax_gate, argmax_gate_rows, rms_row_norm


def _rows(n=200, V=50, d=16, seed=0):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((n, d))
    E = rng.standard_normal((V, d))
    return h, E, h @ E.T


def _tau(h, E, prec="bf16"):
    u = 2.0 ** -8 if prec == "bf16" else 2.0 ** -20
    return 8 * u * np.linalg.norm(h, axis=1) * rms_row_norm(E) / math.sqrt(h.shape[1])


def test_exact_picks_pass():
    h, E, z = _rows()
    n_mis, _, worst = argmax_gate_rows(np.argmax(z, axis=1), z, h, E, "bf16", "exact")
    assert n_mis == 0 and worst == 0.0


def test_a_near_tie_within_tau_is_excused():
    h, E, z = _rows()
    tau = _tau(h, E)
    z = z.copy()
    top = np.argsort(-z[0])
    z[0, top[1]] = z[0, top[0]] - 0.5 * tau[0]     # runner-up within tau of the maximum
    am = np.argmax(z, axis=1)
    am[0] = top[1]
    n_mis, near, worst = argmax_gate_rows(am, z, h, E, "bf16", "near tie")
    assert n_mis == 1 and near >= 1 and worst == pytest.approx(0.5)


def test_a_pick_beyond_tau_fails():
    h, E, z = _rows()
    tau = _tau(h, E)
    z = z.copy()
    top = np.argsort(-z[0])
    z[0, top[1]] = z[0, top[0]] - 2.0 * tau[0]
    am = np.argmax(z, axis=1)
    am[0] = top[1]
    with pytest.raises(AssertionError):
        argmax_gate_rows(am, z, h, E, "bf16", "planted")


def test_a_pick_outside_the_recorded_top_fails():
    h, E, z = _rows(V=100)
    am = np.argmax(z, axis=1)
    am[3] = int(np.argmin(z[3]))
    with pytest.raises(AssertionError):
        argmax_gate_rows(am, z, h, E, "fp32", "planted")


def test_too_many_excused_ties_fail():
    h, E, z = _rows(n=100)
    z = z.copy()
    am = np.argmax(z, axis=1)
    for t in range(10):                              # 10% exact ties, GPU picks the other one
        top = np.argsort(-z[t])
        z[t, top[1]] = z[t, top[0]]
        am[t] = max(top[0], top[1])
    rec = LogitRecord()
    rec.add(z, h)
    vals, ids, hn = rec.arrays()
    with pytest.raises(AssertionError, match="too many"):
        argmax_gate(am, np.argmax(z, axis=1), vals, ids, hn, rms_row_norm(E), h.shape[1], "bf16", "planted")


def test_record_orders_ties_by_lowest_id():
    rec = LogitRecord()
    rec.add(np.array([[1.0, 5.0, 5.0, 2.0]]), np.ones((1, 2)))
    vals, ids, _ = rec.arrays()
    assert ids[0, :2].tolist() == [1, 2] and vals[0, 0] == 5.0

"""Evaluation, snapshots and the Settlement rule ([SGF], Settlement) through the C ABI vs the
fp64 oracle.

  * ttt_evaluate scores a passage at the current weights (losses within the per-token loss
    gate) and changes nothing (token count, records and weights bitwise the same);
  * ttt_snapshot / ttt_restore return the fast state bitwise;
  * ttt_settle_chunk: A = L(q, W) - L(q, W + delta) within the A gate of the oracle's, the
    same keep / restore decision, and the weights after the decision within the weight gates
    (exactly W0 after a rejection); both branches are exercised.
Gates: those of tests/_parity.py, plus |A - A_oracle| <= A_TOL + 1e-3 |A_oracle| (below).
"""
import numpy as np
import pytest

from _parity import TOL, device_weights, inputs, log, oracle_run, rel_l2

import oracle as O

pytestmark = pytest.mark.gpu

# A is the difference of two passage means. Each mean's error is at most the largest per-token
# loss error, which the parity runs measure at <= 1e-4 (bf16, after the loss compensation; the
# 760M shape is the worst) and <= 2e-6 (fp32); so |A - A_oracle| <= 2 x those, plus a relative
# 1e-3 for the large losses of an overshooting step.
A_TOL = {"bf16": 2e-4, "fp32": 4e-6}


def _ctx(w, dev, max_tokens, precision=None, **kw):
    import test_long_context_chunk_amd as ttt
    return ttt.TTT.from_workload(w, dev, max_tokens=max_tokens, precision=precision or w.precision, **kw)


def _tok(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def _state(ctx, w, kind="delta"):
    return {f"{n}.{l}": ctx.fast_weight(l, n, kind).cpu().numpy().astype(np.float64)
            for l in range(w.n_blocks) for n in w.fast_names()}


@pytest.mark.parametrize("precision", ["bf16", "fp32"])
def test_evaluate_scores_without_changing_anything(ttt_lib, precision):
    w, x, P = inputs("single")
    b = w.chunk
    ctx = _ctx(w, device_weights(P, precision), 4 * b, precision)
    ctx.prefill(_tok(x[:b + 1]))
    before = (ctx.consumed(), ctx.token_losses().cpu().numpy(), _state(ctx, w))
    q = x[2 * b:4 * b + 1]  # two chunks later in the stream, never trained on
    losses, mean = ctx.evaluate(_tok(q))
    losses = losses.cpu().numpy().astype(np.float64)
    mean = float(mean.cpu().numpy()[0])
    after = (ctx.consumed(), ctx.token_losses().cpu().numpy(), _state(ctx, w))
    assert ctx.sync() == 0
    ctx.close()
    assert before[0] == after[0] and np.array_equal(before[1], after[1])
    for k in before[2]:
        assert np.array_equal(before[2][k], after[2][k])
    model = O.Model.from_workload(w)
    orc = oracle_run(w, P, x, 1, key="single")
    Pw = {**O.as_f64(P), **orc.weights}
    ref, _, _ = O.token_losses(model, Pw, q[:-1], q[1:])
    dl = np.abs(losses - ref).max()
    log(f"[evaluate single {precision}] loss {dl:.3g} mean {abs(mean - ref.mean()):.3g}")
    assert dl <= TOL[precision]["loss"]
    assert abs(mean - losses.mean()) <= 1e-5 * max(1.0, abs(mean))


def test_snapshot_restore_is_bitwise(ttt_lib):
    w, x, P = inputs("single")
    b = w.chunk
    dev = device_weights(P, "bf16")
    a = _ctx(w, dev, 4 * b)
    a.prefill(_tok(x[:2 * b + 1]))
    c = _ctx(w, dev, 4 * b)
    c.prefill(_tok(x[:b + 1]))
    s1 = _state(c, w)
    c.snapshot()
    c.prefill(_tok(x[b:2 * b + 1]))
    c.restore()
    for k, v in _state(c, w).items():
        assert np.array_equal(v, s1[k]), k
    c.prefill(_tok(x[2 * b:3 * b + 1]))  # after the restore: the step of chunk 3 from W_1
    import test_long_context_chunk_amd as ttt
    c2 = _ctx(w, dev, 4 * b)
    c2.prefill(_tok(x[:b + 1]))
    c2.prefill(_tok(x[2 * b:3 * b + 1]))
    for k, v in _state(c, w).items():
        assert np.array_equal(v, _state(c2, w)[k]), k
    with pytest.raises(ttt.TTTError):
        a.restore()  # no snapshot taken
    for z in (a, c, c2):
        assert z.sync() == 0
        z.close()


# The rule on the candidate chunk at W0 with the passage q = the candidate's own text, so that
# the sign of A is known in advance: a small step descends (A ~ eta ||G||^2 > 0, kept) and a far
# too large one overshoots (A < 0, restored). At these random-init weights almost any moderate
# step lowers any passage's loss, so a held-out passage cannot force a rejection; the step size
# can. (At the workloads' own rates the single-block shape moves A by ~1e-6, below the gate,
# so it runs at a larger rate.)
CASES = [("single", "bf16", 100.0, 1), ("single", "fp32", 100.0, 1), ("s760m", "bf16", 0.005, 1),
         ("s760m", "bf16", 5.0, 0), ("s760m", "fp32", 5.0, 0)]


@pytest.mark.parametrize("name,precision,lr,expect", CASES)
def test_settlement_matches_oracle(ttt_lib, name, precision, lr, expect):
    w, x, P = inputs(name)
    b = w.chunk
    model = O.Model.from_workload(w, lr=lr)
    cand = x[:b + 1]
    A_o, keep_o, W_o, g_o, s_o = O.settle_step(model, P, cand, cand)
    assert int(keep_o) == expect
    ctx = _ctx(w, device_weights(P, precision), 2 * b, precision, lr=lr)
    A, kept = ctx.settle(_tok(cand), _tok(cand))
    A, kept = float(A.cpu().numpy()[0]), int(kept.cpu().numpy()[0])
    D = _state(ctx, w)
    Wg = _state(ctx, w, "W")
    stats = ctx.chunk_stats().cpu().numpy()
    assert ctx.consumed() == b and ctx.sync() == 0
    ctx.close()
    tol = A_TOL[precision] + 1e-3 * abs(A_o)
    log(f"[settle {name} {precision} lr={lr}] A {A:.6g} vs {A_o:.6g} kept {kept} vs {int(keep_o)} g {stats[0, 0]:.5g} vs {g_o:.5g}")
    assert abs(A - A_o) <= tol
    assert abs(A_o) > tol
    assert kept == int(keep_o)
    assert abs(stats[0, 0] - g_o) <= TOL[precision]["g"] * g_o
    if kept:
        for k in W_o:
            assert rel_l2(Wg[k], W_o[k]) <= TOL[precision]["w"], k
            assert rel_l2(D[k], W_o[k] - O.as_f64(P)[k]) <= TOL[precision]["dw"], k
    else:
        for k, v in D.items():
            assert not v.any(), k  # restored to W0 exactly

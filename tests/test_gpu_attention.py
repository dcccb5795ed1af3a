"""Blocks with frozen sliding-window attention ("End-to-End Test-Time Training for Long
Context", section 3: a window of k >= b positions before the MLPs) through the C ABI, vs the
fp64 oracle.

The attention runs in bf16 with heads of 128. Each position's key and value are computed at
its own chunk's weights and kept in a ring; later chunks read them as constants, and the
inner loop backpropagates through the current chunk's queries, keys and values into the fast
blocks below. Checks: windows shorter than, equal to and longer than the chunk and than the
whole stream, one and two heads, with and without the static MLP, several prefill calls,
batched streams, the fuller-block 760M shape (sampled), decoding (each decoded row's key and
value join the ring at once; a filled chunk's step reads the window in front of it),
passage scoring and Settlement (the passage is a sequence of its own, scored over rings of
its own; the stream's rings are left as they are), and the calls an attention context
refuses. Gates are those of tests/_parity.py (bf16).
"""
import numpy as np
import pytest

from _parity import TOL, argmax_gate_rows, compare, device_weights, gpu_run, log, oracle_run, rel_l2

import oracle as O
import ttt_workloads as W

pytestmark = pytest.mark.gpu

BASE = dict(vocab=2000, d_model=128, d_hidden=256, n_blocks=3, n_tokens=256, chunk=64, lr=0.05, swa_heads=1)


@pytest.mark.parametrize("window,static,d,calls,chunk", [
    (96, 192, 128, 2, 64),   # window between the chunk and the stream, static MLP, two calls
    (64, 0, 256, 1, 64),     # window = chunk, two heads, no static MLP
    (40, 0, 128, 4, 64),     # window shorter than the chunk, one call per chunk
    (1000, 128, 128, 1, 64), # window longer than the stream (full causal attention)
    (1, 0, 128, 2, 64),      # window 1: each position attends to itself only
    (80, 128, 128, 1, 48),   # chunk of 48: a ragged query block and key blocks across chunks
    (300, 0, 128, 2, 512),   # chunk of 512: the dK, dV pass split over query-block shares
    (800, 0, 128, 2, 1024),  # window below a 1024-token chunk: four dK, dV shares, capped by the window
])
def test_attention_blocks_match_the_oracle(ttt_lib, window, static, d, calls, chunk):
    w = W.preset("e2e760m", **dict(BASE, d_model=d, swa_heads=d // 128, swa_window=window, static_hidden=static,
                                   chunk=chunk, n_tokens=4 * chunk))
    P = W.init_weights(w, 12)
    x = W.token_stream(w, 13)
    log(f"attention window={window} static={static} d={d} calls={calls}")
    g = gpu_run(w, P, x, calls=calls)
    assert g["status"] == 0
    orc = oracle_run(w, P, x, w.n_chunks, gpu_argmax=g["argmax"])
    compare(g, orc, w, "bf16", w.n_chunks, label=f"attn-w{window}")


def test_attention_batched_streams(ttt_lib):
    """Three streams of one batched context (each its own ring), against the oracle."""
    from test_gpu_batch import gpu_run_batch
    w = W.preset("e2e760m", **dict(BASE, swa_window=100, static_hidden=128))
    P = W.init_weights(w, 14)
    xs = [W.token_stream(w, 15), W.token_stream(w, 16), W.token_stream(w, 15)]
    gs = gpu_run_batch(w, P, xs, w.n_tokens, calls=2)
    for z, (g, x) in enumerate(zip(gs, xs)):
        assert g["status"] == 0
        compare(g, oracle_run(w, P, x, w.n_chunks), w, "bf16", w.n_chunks, label=f"attn-batch stream {z}")
    assert np.array_equal(gs[0]["losses"], gs[2]["losses"])


def test_e2e760m_attention_past_the_window(ttt_lib):
    """The fuller 760M block (12 heads, window 8K, static MLP) in the benchmark's launch
    configuration, 11 chunks in one prefill call: chunks 9-11 see a full 8192-key window and
    the key/value ring (window + chunk = 9216 slots) wraps at chunk 10; every token, step
    and update against the oracle."""
    n_chunks = 11
    w = W.preset("e2e760m", n_tokens=n_chunks * 1024)
    P = W.init_weights(w, 0)
    x = W.token_stream(w, 0)
    log(f"attention e2e760m: {n_chunks} chunks")
    g = gpu_run(w, P, x)
    assert g["status"] == 0
    log(f"oracle e2e760m: {n_chunks} chunks")
    compare(g, oracle_run(w, P, x, n_chunks), w, "bf16", n_chunks, label="e2e760m-attn")


def test_batched_attention_context_refuses_single_stream_calls(ttt_lib):
    import ctypes
    import torch
    import test_long_context_chunk_amd as ttt
    w = W.preset("e2e760m", **dict(BASE, swa_window=64, static_hidden=0, n_blocks=1))
    P = W.init_weights(w, 0)
    ctx = ttt.TTT.from_workload(w, device_weights(P, "bf16"), max_tokens=128, streams=2)
    lib, c = ctx._lib, ctx._ctx
    tok = torch.zeros(130, dtype=torch.int32, device="cuda")
    p = ctypes.c_void_p(tok.data_ptr())
    assert lib.ttt_decode(c, p, 1, None, None) == -1
    assert lib.ttt_evaluate(c, p, 64, None, None) == -1
    assert lib.ttt_snapshot(c) == -1
    assert lib.ttt_settle_chunk(c, p, p, 64, None, None) == -1
    assert ctx.consumed() == 0 and ctx.sync() == 0
    ctx.close()


def _tok(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


@pytest.mark.parametrize("window,d", [(40, 128), (96, 256), (1000, 128), (1, 128)])
def test_attention_decode_matches_oracle_decode(ttt_lib, window, d):
    """One prefilled chunk, then 1.5 chunks decoded in two calls (one step in between):
    every decoded row's logits and the fast weights after the step, against the oracle's
    token-by-token decode."""
    import test_long_context_chunk_amd as ttt
    w = W.preset("e2e760m", **dict(BASE, d_model=d, swa_heads=d // 128, swa_window=window, static_hidden=128))
    P = W.init_weights(w, 17)
    x = W.token_stream(w, 18)
    b = w.chunk
    n = b + b // 2
    log(f"attention decode window={window} d={d}")
    ctx = ttt.TTT.from_workload(w, device_weights(P, "bf16"), max_tokens=w.n_tokens)
    ctx.prefill(_tok(x[:b + 1]))
    am1, z1 = ctx.decode(_tok(x[b:b + 40 + 1]), want_logits=True)
    am2, z2 = ctx.decode(_tok(x[b + 40:b + n + 1]), want_logits=True)
    zg = np.concatenate([z1.cpu().numpy(), z2.cpu().numpy()]).astype(np.float64)
    am = np.concatenate([am1.cpu().numpy(), am2.cpu().numpy()]).astype(np.int64)
    assert ctx.decode_pending() == n - b
    Dg = {f"{k}.{l}": ctx.fast_weight(l, k, "delta").cpu().numpy().astype(np.float64)
          for l in range(w.n_blocks) for k in w.fast_names()}
    assert ctx.sync() == 0
    ctx.close()
    rows = []
    orc = O.decode_ttt(O.Model.from_workload(w), P, x[:b + n + 1],
                       logit_probe=lambda t, z, h: rows.append((t, z.copy(), h.copy())))
    Z = np.stack([z for t, z, h in rows if t >= b])
    H = np.stack([h for t, z, h in rows if t >= b])
    tol = TOL["bf16"]
    dz = float(np.max(np.abs(zg - Z)))
    dd = max(rel_l2(Dg[k], orc.delta[k]) for k in orc.delta)
    log(f"[attention decode w{window}] logits {dz:.3g} D {dd:.3g}")
    assert dz <= tol["logit"]
    assert dd <= tol["dw"]
    argmax_gate_rows(am, Z, H, P["E_out"], "bf16", f"attention decode w{window}")


def test_attention_decoded_chunk_is_bitwise_the_prefilled_step(ttt_lib):
    """Prefill of chunks 0-1 vs prefill of chunk 0 and chunk 1 decoded (three uneven calls),
    then chunk 2 prefilled on both: chunk 1's step re-files its keys from its own forward, so
    every loss, step and update of the two contexts is bitwise equal."""
    import test_long_context_chunk_amd as ttt
    w = W.preset("e2e760m", **dict(BASE, swa_window=100, static_hidden=128))
    P = W.init_weights(w, 19)
    x = W.token_stream(w, 20)
    b = w.chunk
    dev = device_weights(P, "bf16")
    a = ttt.TTT.from_workload(w, dev, max_tokens=w.n_tokens)
    a.prefill(_tok(x[:2 * b + 1]))
    c = ttt.TTT.from_workload(w, dev, max_tokens=w.n_tokens)
    c.prefill(_tok(x[:b + 1]))
    for s0, e in [(b, b + 5), (b + 5, b + 50), (b + 50, 2 * b)]:
        c.decode(_tok(x[s0:e + 1]))
    assert c.decode_pending() == 0 and c.consumed() == 2 * b
    for ctx in (a, c):
        ctx.prefill(_tok(x[2 * b:3 * b + 1]))
    assert np.array_equal(a.token_losses().cpu().numpy(), c.token_losses().cpu().numpy())
    assert np.array_equal(a.chunk_stats().cpu().numpy(), c.chunk_stats().cpu().numpy())
    for l in range(w.n_blocks):
        for k in w.fast_names():
            assert np.array_equal(a.fast_weight(l, k, "delta").cpu().numpy(),
                                  c.fast_weight(l, k, "delta").cpu().numpy()), (k, l)
    assert a.sync() == 0 and c.sync() == 0
    a.close()
    c.close()


def test_e2e760m_attention_decode_sampled(ttt_lib):
    """The fuller 760M block: two prefilled chunks, then 16 decoded rows scored at the
    stepped weights against the oracle's logits (the rows read the prefilled keys)."""
    import test_long_context_chunk_amd as ttt
    w = W.preset("e2e760m", n_tokens=3072)
    P = W.init_weights(w, 0)
    x = W.token_stream(w, 0)
    b, n = w.chunk, 16
    T0 = 2 * b
    log("attention decode e2e760m")
    ctx = ttt.TTT.from_workload(w, device_weights(P, "bf16"), max_tokens=T0 + b)
    ctx.prefill(_tok(x[:T0 + 1]))
    am, z = ctx.decode(_tok(x[T0:T0 + n + 1]), want_logits=True)
    z = z.cpu().numpy().astype(np.float64)
    am = am.cpu().numpy().astype(np.int64)
    assert ctx.sync() == 0
    ctx.close()
    model = O.Model.from_workload(w)
    orc = oracle_run(w, P, x, 2)
    Pw = dict(O.as_f64(P))
    Pw.update(orc.weights)
    zo, ho, _ = O.logits(model, Pw, x[T0:T0 + n], orc.kv)
    dz = float(np.max(np.abs(z - zo)))
    log(f"[attention decode e2e760m] logits {dz:.3g}")
    assert dz <= TOL["bf16"]["logit"]
    argmax_gate_rows(am, zo, ho, P["E_out"], "bf16", "attention decode e2e760m")


SETTLE = dict(BASE, swa_window=96, static_hidden=128)


def test_attention_evaluate_scores_the_passage_alone(ttt_lib):
    """A three-chunk passage (its rings wrap) scored after one prefilled chunk: per-token
    losses and their mean against the oracle's passage scoring at the stepped weights; then the
    stream goes on exactly as if nothing had been scored (losses and updates bitwise)."""
    import test_long_context_chunk_amd as ttt
    w = W.preset("e2e760m", **SETTLE)
    P = W.init_weights(w, 21)
    x = W.token_stream(w, 22)
    q = W.token_stream(w, 23)[:3 * w.chunk + 1]
    b = w.chunk
    dev = device_weights(P, "bf16")
    a = ttt.TTT.from_workload(w, dev, max_tokens=w.n_tokens)
    a.prefill(_tok(x[:b + 1]))
    losses, mean = a.evaluate(_tok(q))
    losses = losses.cpu().numpy().astype(np.float64)
    mean = float(mean.cpu().numpy()[0])
    a.prefill(_tok(x[b:2 * b + 1]))
    c = ttt.TTT.from_workload(w, dev, max_tokens=w.n_tokens)
    c.prefill(_tok(x[:2 * b + 1]))
    assert np.array_equal(a.token_losses().cpu().numpy(), c.token_losses().cpu().numpy())
    for l in range(w.n_blocks):
        for k in w.fast_names():
            assert np.array_equal(a.fast_weight(l, k, "delta").cpu().numpy(),
                                  c.fast_weight(l, k, "delta").cpu().numpy()), (k, l)
    assert a.sync() == 0 and c.sync() == 0
    a.close()
    c.close()
    model = O.Model.from_workload(w)
    one = O.run_ttt(model, P, x[:b + 1])
    W1 = {**O.as_f64(P), **one.weights}
    lo, _, _ = O.token_losses(model, W1, q[:-1], q[1:])
    dl = float(np.max(np.abs(losses - lo)))
    dm = abs(mean - O.passage_loss(model, W1, q))
    log(f"[attention evaluate] losses {dl:.3g} mean {dm:.3g}")
    assert dl <= TOL["bf16"]["loss"] and dm <= TOL["bf16"]["loss"]


@pytest.mark.parametrize("lr,expect", [(1.0, 1), (20.0, 0)])
def test_attention_settlement_matches_oracle(ttt_lib, lr, expect):
    """One prefilled chunk, then a candidate chunk under the Settlement rule with the passage
    = its own text (kept at a moderate rate, rejected at an overshooting one), then one more
    prefilled chunk. A twin context prefills the candidate instead, which gives the GPU's own
    W and W + delta (the candidate's step is the prefill step, bit for bit), and scores the
    passage at each. Checks: the oracle's settle_step from the stream's cache takes the same
    decision; A is the difference of the GPU's own passage means at W and W + delta; those
    passage losses match the oracle's at the GPU's two weight sets, token by token, within the
    bf16 loss gate (the step's own error is left to the update gate: at an overshooting rate
    A magnifies it); the state after the decision is the twin's W + delta or W bit for bit;
    and the next chunk's losses (which read the candidate's keys either way) match the
    oracle's."""
    import test_long_context_chunk_amd as ttt
    w = W.preset("e2e760m", **dict(SETTLE, lr=lr))
    P = W.init_weights(w, 21)
    x = W.token_stream(w, 22)
    b = w.chunk
    dev = device_weights(P, "bf16")
    cand = x[b:2 * b + 1]

    def state(ctx, kind):
        return {f"{k}.{l}": ctx.fast_weight(l, k, kind).cpu().numpy().astype(np.float64)
                for l in range(w.n_blocks) for k in w.fast_names()}
    twin = ttt.TTT.from_workload(w, dev, max_tokens=w.n_tokens, lr=lr)
    twin.prefill(_tok(x[:b + 1]))
    W1g, D1g = state(twin, "W"), state(twin, "delta")
    E1 = twin.evaluate(_tok(cand))[0].cpu().numpy().astype(np.float64)
    twin.prefill(_tok(cand))
    W2g, D2g = state(twin, "W"), state(twin, "delta")
    E2 = twin.evaluate(_tok(cand))[0].cpu().numpy().astype(np.float64)
    assert twin.sync() == 0
    twin.close()
    ctx = ttt.TTT.from_workload(w, dev, max_tokens=w.n_tokens, lr=lr)
    ctx.prefill(_tok(x[:b + 1]))
    A, kept = ctx.settle(_tok(cand), _tok(cand))
    A, kept = float(A.cpu().numpy()[0]), int(kept.cpu().numpy()[0])
    Dg = state(ctx, "delta")
    ctx.prefill(_tok(x[2 * b:3 * b + 1]))
    nxt = ctx.token_losses(2 * b, b).cpu().numpy().astype(np.float64)
    assert ctx.consumed() == 3 * b and ctx.sync() == 0
    ctx.close()
    model = O.Model.from_workload(w, lr=lr)
    Pf = O.as_f64(P)
    one = O.run_ttt(model, P, x[:b + 1])
    W1 = {**Pf, **one.weights}
    A_o, keep_o, Wn, _, _ = O.settle_step(model, W1, cand, cand, kv=one.kv)
    assert int(keep_o) == expect
    t1, _, _ = O.token_losses(model, {**Pf, **W1g}, cand[:-1], cand[1:])
    t2, _, _ = O.token_losses(model, {**Pf, **W2g}, cand[:-1], cand[1:])
    A_g = float(np.mean(t1) - np.mean(t2))
    A_e = float(np.mean(E1) - np.mean(E2))
    kv = O.chunk_loss_and_grads(model, W1, cand[:-1], cand[1:], kv=one.kv)[1]["kv"]
    lo, _, _ = O.token_losses(model, {**W1, **Wn}, x[2 * b:3 * b], x[2 * b + 1:3 * b + 1], kv=kv)
    dl = float(np.max(np.abs(nxt - lo)))
    d1, d2 = float(np.max(np.abs(E1 - t1))), float(np.max(np.abs(E2 - t2)))
    log(f"[attention settle lr={lr}] A {A:.6g} vs {A_e:.6g} from the GPU's passage scores, {A_g:.6g} oracle's at "
        f"the GPU's weights ({A_o:.6g} oracle's own); passage losses at W {d1:.3g}, at W + delta {d2:.3g}; "
        f"kept {kept} next-chunk losses {dl:.3g}")
    assert abs(A - A_e) <= 1e-6 * (1.0 + abs(A_e))
    assert d1 <= TOL["bf16"]["loss"] and d2 <= TOL["bf16"]["loss"]
    assert (A_g >= 0) == bool(expect) and (A >= 0) == bool(expect)
    assert kept == expect
    after = D2g if kept else D1g
    for k in Dg:
        assert np.array_equal(Dg[k], after[k]), k
    assert dl <= TOL["bf16"]["loss"]


def test_attention_scoring_between_decoded_tokens_leaves_the_stream_alone(ttt_lib):
    """Prefill, decode part of a chunk, score a passage, decode the rest of the chunk and
    prefill one more: every loss, step and update equals the same calls without the passage
    (the passage rings are apart from the stream's, and a pending chunk keeps its ids)."""
    import test_long_context_chunk_amd as ttt
    w = W.preset("e2e760m", **dict(BASE, swa_window=100, static_hidden=128))
    P = W.init_weights(w, 24)
    x = W.token_stream(w, 25)
    q = W.token_stream(w, 26)[:2 * w.chunk + 1]
    b = w.chunk
    dev = device_weights(P, "bf16")
    runs = []
    for score in (False, True):
        ctx = ttt.TTT.from_workload(w, dev, max_tokens=w.n_tokens)
        ctx.prefill(_tok(x[:b + 1]))
        ctx.decode(_tok(x[b:b + 30 + 1]))
        if score:
            ctx.evaluate(_tok(q))
        ctx.decode(_tok(x[b + 30:2 * b + 1]))
        ctx.prefill(_tok(x[2 * b:3 * b + 1]))
        out = dict(losses=ctx.token_losses().cpu().numpy(), stats=ctx.chunk_stats().cpu().numpy(),
                   D={f"{k}.{l}": ctx.fast_weight(l, k, "delta").cpu().numpy()
                      for l in range(w.n_blocks) for k in w.fast_names()})
        assert ctx.sync() == 0 and ctx.consumed() == 3 * b
        ctx.close()
        runs.append(out)
    a, c = runs
    assert np.array_equal(a["losses"], c["losses"])
    assert np.array_equal(a["stats"], c["stats"])
    for k in a["D"]:
        assert np.array_equal(a["D"][k], c["D"][k]), k

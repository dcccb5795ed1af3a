"""Decoding through the C ABI ([E2E] Method: decoding; section 3.2) vs the fp64 oracle.

ttt_decode predicts each token from the one before at the current fast weights and takes
the chunk's step whenever b decoded pairs fill a mini-batch. Checks:
  * toy (b = 1, fp32): the whole stream decoded in three calls against the oracle's
    token-by-token decode (losses, argmax, logits, final weights);
  * single (bf16 and fp32): one prefilled chunk, then a decoded chunk plus a partial one,
    against the chunked oracle (losses from the returned logits, logits on sampled rows,
    argmax validity, weights after the decoded chunk);
  * a decoded chunk is bitwise the same step as a prefilled one (same weights, same
    recorded losses);
  * the 760M and In-Place shapes: a partial decoded chunk after prefill;
  * argument and state errors.
Gates are those of tests/_parity.py.
"""
import numpy as np
import pytest

from _parity import TOL, LogitRecord, argmax_gate, argmax_gate_rows, device_weights, inputs, log, oracle_run, rel_l2, \
    rms_row_norm

import oracle as O

pytestmark = pytest.mark.gpu


def _lse_loss(z, tgt):
    z = z.astype(np.float64)
    m = z.max(axis=1)
    lse = m + np.log(np.exp(z - m[:, None]).sum(axis=1))
    return lse - z[np.arange(z.shape[0]), tgt]


def _ctx(w, dev, max_tokens, precision=None, **kw):
    import test_long_context_chunk_amd as ttt
    return ttt.TTT.from_workload(w, dev, max_tokens=max_tokens, precision=precision or w.precision, **kw)


def _tok(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def _weights(ctx, w, kind):
    out = {}
    for l in range(w.n_blocks):
        for n in w.fast_names():
            out[f"{n}.{l}"] = ctx.fast_weight(l, n, kind).cpu().numpy().astype(np.float64)
    return out


def test_decode_toy_fp32_matches_oracle_decode(ttt_lib):
    """b = 1: every decoded token is its own mini-batch; three calls over the whole stream."""
    w, x, P = inputs("toy")
    model = O.Model.from_workload(w)
    rows, hs = [], []
    orc = O.decode_ttt(model, P, x, logit_probe=lambda t, z, h: (rows.append(z.copy()), hs.append(h.copy())))
    Z, H = np.stack(rows), np.stack(hs)
    ctx = _ctx(w, device_weights(P, "fp32"), w.n_tokens, "fp32")
    am, zs = [], []
    for a, b in [(0, 40), (40, 90), (90, w.n_tokens)]:
        a_, z_ = ctx.decode(_tok(x[a:b + 1]), want_logits=True)
        am.append(a_.cpu().numpy())
        zs.append(z_.cpu().numpy())
    am, zg = np.concatenate(am), np.concatenate(zs)
    assert ctx.consumed() == w.n_tokens and ctx.decode_pending() == 0
    rec = ctx.token_losses().cpu().numpy().astype(np.float64)
    tol = TOL["fp32"]
    dl = np.abs(_lse_loss(zg, x[1:]) - orc.losses).max()
    dr = np.abs(rec - orc.losses).max()
    dz = np.abs(zg - Z).max()
    Wg, Dg = _weights(ctx, w, "W"), _weights(ctx, w, "delta")
    wr = max(rel_l2(Wg[k], orc.weights[k]) for k in orc.weights)
    dr2 = max(rel_l2(Dg[k], orc.delta[k]) for k in orc.delta)
    log(f"[decode toy fp32] loss(from logits) {dl:.3g} loss(recorded) {dr:.3g} logits {dz:.3g} W {wr:.3g} D {dr2:.3g}")
    assert ctx.sync() == 0
    ctx.close()
    assert dl <= tol["loss"] and dr <= tol["loss"] and dz <= tol["logit"]
    assert wr <= tol["w"] and dr2 <= tol["dw"]
    argmax_gate_rows(am, Z, H, P["E_out"], "fp32", "decode toy")


def test_decoded_chunk_is_bitwise_the_prefilled_step(ttt_lib):
    """Prefill of two chunks vs prefill of one and a decoded one (three uneven calls): the
    step, the weights and the recorded losses of the second chunk are bitwise equal."""
    w, x, P = inputs("single", n_tokens=4096)
    dev = device_weights(P, "bf16")
    b = w.chunk
    a = _ctx(w, dev, 4 * b)
    a.prefill(_tok(x[:2 * b + 1]))
    c = _ctx(w, dev, 4 * b)
    c.prefill(_tok(x[:b + 1]))
    for s, e in [(b, b + 300), (b + 300, b + 800), (b + 800, 2 * b)]:
        c.decode(_tok(x[s:e + 1]))
    assert c.decode_pending() == 0 and c.consumed() == 2 * b
    assert np.array_equal(a.token_losses().cpu().numpy(), c.token_losses().cpu().numpy())
    assert np.array_equal(a.token_argmax().cpu().numpy(), c.token_argmax().cpu().numpy())
    assert np.array_equal(a.chunk_stats().cpu().numpy(), c.chunk_stats().cpu().numpy())
    Da, Dc = _weights(a, w, "delta"), _weights(c, w, "delta")
    for k in Da:
        assert np.array_equal(Da[k], Dc[k]), k
    assert a.sync() == 0 and c.sync() == 0
    a.close()
    c.close()


@pytest.mark.parametrize("precision", ["bf16", "fp32"])
def test_decode_single_matches_oracle(ttt_lib, precision):
    """One prefilled chunk, then one decoded chunk and 64 more decoded tokens in one call."""
    w, x, P = inputs("single", n_tokens=4096)
    model = O.Model.from_workload(w)
    b = w.chunk
    ctx = _ctx(w, device_weights(P, precision), 4 * b, precision)
    ctx.prefill(_tok(x[:b + 1]))
    n = b + 64
    am, z = ctx.decode(_tok(x[b:b + n + 1]), want_logits=True)
    am, z = am.cpu().numpy().astype(np.int64), z.cpu().numpy()
    rec = ctx.token_losses(b, n).cpu().numpy().astype(np.float64)
    Wg, Dg = _weights(ctx, w, "W"), _weights(ctx, w, "delta")
    assert ctx.decode_pending() == 64
    assert ctx.sync() == 0
    ctx.close()
    # oracle: chunk 2 scored at W_1 (its logits seen through the probe), then the tail at W_2
    sample = np.arange(0, b, 97)
    rec2, zs = LogitRecord(), {}

    def probe(i, zz, h):
        if i == 1:
            rec2.add(zz, h)
            for r in sample:
                zs[r] = zz[r].copy()

    orc = O.run_ttt(model, P, x[:2 * b + 1], logit_probe=probe)
    Pw = dict(O.as_f64(P))
    Pw.update(orc.weights)
    zt, ht, _ = O.logits(model, Pw, x[2 * b:2 * b + 64])
    l_tail, _, _, _ = O.ce_stats(zt, x[2 * b + 1:2 * b + 65])
    ref = np.concatenate([orc.losses[b:2 * b], l_tail])
    tol = TOL[precision]
    dl = np.abs(_lse_loss(z, x[b + 1:b + n + 1]) - ref).max()
    dtail = np.abs(rec[b:] - l_tail).max()
    dz = max(np.abs(z[r] - zs[r]).max() for r in sample)
    dzt = np.abs(z[b:] - zt).max()
    wr = max(rel_l2(Wg[k], orc.weights[k]) for k in orc.weights)
    dr = max(rel_l2(Dg[k], orc.delta[k]) for k in orc.delta)
    log(f"[decode single {precision}] loss {dl:.3g} tail(recorded) {dtail:.3g} logits {dz:.3g}/{dzt:.3g} "
        f"W {wr:.3g} D {dr:.3g}")
    assert dl <= tol["loss"] and dtail <= tol["loss"]
    assert dz <= tol["logit"] and dzt <= tol["logit"]
    assert wr <= tol["w"] and dr <= tol["dw"]
    rec2.add(zt, ht)
    vals, ids, hn = rec2.arrays()
    am_o = np.concatenate([orc.argmax[b:2 * b], np.argmax(zt, axis=1)])
    argmax_gate(am, am_o, vals, ids, hn, rms_row_norm(P["E_out"]), w.d_model, precision, f"decode single")


@pytest.mark.parametrize("name,pre_chunks,n", [("s760m", 2, 48), ("inplace", 1, 16)])
def test_decode_partial_chunk_large_shapes(ttt_lib, name, pre_chunks, n):
    """After prefill, a partial decoded chunk is scored at the prefilled weights."""
    w, x, P = inputs(name)
    model = O.Model.from_workload(w)
    b = w.chunk
    T0 = pre_chunks * b
    ctx = _ctx(w, device_weights(P, "bf16"), T0 + b)
    ctx.prefill(_tok(x[:T0 + 1]))
    am, z = ctx.decode(_tok(x[T0:T0 + n + 1]), want_logits=True)
    am, z = am.cpu().numpy().astype(np.int64), z.cpu().numpy()
    rec = ctx.token_losses(T0, n).cpu().numpy().astype(np.float64)
    assert ctx.decode_pending() == n and ctx.sync() == 0
    ctx.close()
    orc = oracle_run(w, P, x, pre_chunks, key=name)
    Pw = dict(O.as_f64(P))
    Pw.update(orc.weights)
    zo, ho, _ = O.logits(model, Pw, x[T0:T0 + n])
    lo, _, _, _ = O.ce_stats(zo, x[T0 + 1:T0 + n + 1])
    tol = TOL["bf16"]
    dl = np.abs(rec - lo).max()
    dz = np.abs(z - zo).max()
    log(f"[decode {name}] loss {dl:.3g} logits {dz:.3g}")
    assert dl <= tol["loss"] and dz <= tol["logit"]
    argmax_gate_rows(am, zo, ho, P["E_out"], "bf16", f"decode {name}")


def test_decode_state_and_argument_errors(ttt_lib):
    import test_long_context_chunk_amd as ttt
    w, x, P = inputs("single", n_tokens=4096)
    b = w.chunk
    ctx = _ctx(w, device_weights(P, "bf16"), 2 * b)
    ctx.decode(_tok(x[:1]))  # n = 0: nothing happens
    assert ctx.consumed() == 0
    ctx.decode(_tok(x[:11]))
    assert ctx.decode_pending() == 10 and ctx.consumed() == 10
    with pytest.raises(ttt.TTTError) as e:  # a partial decoded chunk is pending
        ctx.prefill(_tok(x[10:10 + b + 1]))
    assert e.value.status == -1
    with pytest.raises(ttt.TTTError) as e:  # beyond max_tokens
        ctx.decode(_tok(x[10:10 + 2 * b + 1]))
    assert e.value.status == -1
    bad = x[10:20].astype(np.int32).copy()
    bad[3] = w.vocab + 7
    ctx.decode(_tok(bad))
    assert ctx.sync() == -4  # TTT_ERANGE
    with pytest.raises(ttt.TTTError) as e:
        ctx.decode(_tok(x[19:22]))
    assert e.value.status == -6  # TTT_ESTATE
    ctx.reset()
    assert ctx.sync() == 0 and ctx.decode_pending() == 0 and ctx.consumed() == 0
    ctx.close()

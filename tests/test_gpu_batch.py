"""Batched independent streams (one context, several token streams advanced together) vs the
fp64 oracle run on each stream alone, through the C ABI.

Each stream of a batched context is its own inner loop from the shared initial weights
("Self-Generated Feedback Destabilizes Test-Time Training", How it works: several sequences
adapted side by side, each with its own clipped step per chunk), so stream z must pass the
same gates (tests/_parity.py) against the oracle fed stream z's tokens alone. Two streams
fed the same tokens must agree bit for bit (no stream reads another's rows, weights or
clip), and the calls a batched context does not support must refuse without enqueuing.
"""
import numpy as np
import pytest

from _parity import TOL, compare, device_weights, log, oracle_run

import ttt_workloads as W

pytestmark = pytest.mark.gpu


def gpu_run_batch(w, P, xs, n_tokens, precision=None, calls=1, dev=None):
    """Run the streams xs (one token array each) through one batched context; per-stream
    records as gpu_run returns them."""
    import torch
    import test_long_context_chunk_amd as ttt
    prec = precision or w.precision
    dev = dev if dev is not None else device_weights(P, prec)
    nb = len(xs)
    ctx = ttt.TTT.from_workload(w, dev, max_tokens=n_tokens, precision=prec, streams=nb)
    assert ctx._lib.ttt_streams(ctx._ctx) == nb
    # row z: stream z's ids, padded on the right so the row stride differs from the count
    ld = n_tokens + 1 + 7
    tok = np.zeros((nb, ld), dtype=np.int32)
    for z, x in enumerate(xs):
        tok[z, :n_tokens + 1] = x[:n_tokens + 1]
    tok = torch.from_numpy(tok).cuda()
    per = n_tokens // calls
    assert per % w.chunk == 0
    for c in range(calls):
        ctx.prefill_batch(tok[:, c * per: (c + 1) * per + 1])
    outs = []
    for z in range(nb):
        o = dict(losses=ctx.token_losses(s=z).cpu().numpy().astype(np.float64),
                 argmax=ctx.token_argmax(s=z).cpu().numpy().astype(np.int64),
                 stats=ctx.chunk_stats(s=z).cpu().numpy().astype(np.float64))
        Wf, Df = {}, {}
        for l in range(w.n_blocks):
            for n in w.fast_names():
                Wf[f"{n}.{l}"] = ctx.fast_weight(l, n, "W", s=z).cpu().numpy().astype(np.float64)
                Df[f"{n}.{l}"] = ctx.fast_weight(l, n, "delta", s=z).cpu().numpy().astype(np.float64)
        o["W"], o["D"] = Wf, Df
        outs.append(o)
    status = ctx.sync()
    ctx.close()
    for o in outs:
        o["status"] = status
    return outs


def _same(a, b):
    assert np.array_equal(a["losses"], b["losses"])
    assert np.array_equal(a["argmax"], b["argmax"])
    assert np.array_equal(a["stats"], b["stats"])
    for k in a["D"]:
        assert np.array_equal(a["D"][k], b["D"][k]), k


SMALL = {
    # 3 pre-RMSNorm GELU blocks: every grouped product and both weight gradients per block
    "gelu": dict(vocab=2000, d_model=128, d_hidden=384, n_blocks=3, n_tokens=256, chunk=64),
    # one SwiGLU block, W2 fast, frozen gate/up over all streams' rows
    "swiglu": dict(vocab=3000, d_model=128, d_hidden=320, n_blocks=1, n_tokens=256, chunk=64),
}
BASE = {"gelu": "s125m", "swiglu": "inplace"}


@pytest.mark.parametrize("precision", ["bf16", "fp32"])
@pytest.mark.parametrize("kind", ["gelu", "swiglu"])
def test_batched_streams_match_the_oracle(ttt_lib, kind, precision):
    """Three streams, two prefill calls of two chunks; streams 0 and 2 carry the same tokens."""
    over = SMALL[kind]
    w = W.preset(BASE[kind], precision=precision, lr=0.05, **over)
    P = W.init_weights(w, 0)
    xs = [W.token_stream(w, 11), W.token_stream(w, 12), W.token_stream(w, 11)]
    n_chunks = w.n_tokens // w.chunk
    log(f"batch {kind} {precision} streams=3 chunks={n_chunks}")
    gs = gpu_run_batch(w, P, xs, w.n_tokens, calls=2)
    for z, (g, x) in enumerate(zip(gs, xs)):
        assert g["status"] == 0
        orc = oracle_run(w, P, x, n_chunks, gpu_argmax=g["argmax"])
        compare(g, orc, w, precision, n_chunks, label=f"batch-{kind} stream {z}")
    _same(gs[0], gs[2])
    # the two distinct streams did adapt differently
    assert not np.array_equal(gs[0]["D"]["W2.0"], gs[1]["D"]["W2.0"])


def test_batched_chunk_smaller_than_a_tile(ttt_lib):
    """chunk 64 with 256-row tiles: each stream's rows are a quarter of an M tile, and the
    products with frozen weights cover several streams per tile; 5 streams (a ragged tail)."""
    w = W.preset("s125m", precision="bf16", vocab=1000, d_model=64, d_hidden=192, n_blocks=2, n_tokens=128,
                 chunk=64, lr=0.05)
    P = W.init_weights(w, 1)
    xs = [W.token_stream(w, 30 + z) for z in range(5)]
    gs = gpu_run_batch(w, P, xs, w.n_tokens)
    for z, (g, x) in enumerate(zip(gs, xs)):
        assert g["status"] == 0
        compare(g, oracle_run(w, P, x, 2), w, "bf16", 2, label=f"batch-5 stream {z}")


@pytest.mark.parametrize("streams", [8])
def test_s760m_batched_sampled(ttt_lib, streams):
    """The 760M shape in the batched benchmark's launch configuration (8 streams, chunk
    1024), 4 chunks: streams 0 and 7 (sampled) against the oracle, every stream finite."""
    w = W.preset("s760m", n_tokens=4096)
    P = W.init_weights(w, 0)
    xs = [W.token_stream(w, z) for z in range(streams)]
    log(f"batch s760m streams={streams}")
    gs = gpu_run_batch(w, P, xs, w.n_tokens)
    for g in gs:
        assert g["status"] == 0
        assert np.all(np.isfinite(g["losses"]))
    for z in (0, streams - 1):
        compare(gs[z], oracle_run(w, P, xs[z], w.n_chunks), w, "bf16", w.n_chunks, label=f"batch-s760m stream {z}")


def test_batched_context_refuses_single_stream_calls(ttt_lib):
    import ctypes
    import torch
    import test_long_context_chunk_amd as ttt
    w = W.preset("s125m", precision="bf16", vocab=1000, d_model=64, d_hidden=192, n_blocks=1, n_tokens=128,
                 chunk=64)
    P = W.init_weights(w, 0)
    ctx = ttt.TTT.from_workload(w, device_weights(P, "bf16"), max_tokens=128, streams=2)
    lib, c = ctx._lib, ctx._ctx
    tok = torch.zeros(130, dtype=torch.int32, device="cuda")
    p = ctypes.c_void_p(tok.data_ptr())
    assert lib.ttt_prefill_chunks(c, p, 64) == -1
    assert lib.ttt_decode(c, p, 1, None, None) == -1
    assert lib.ttt_evaluate(c, p, 64, None, None) == -1
    assert lib.ttt_snapshot(c) == -1
    assert lib.ttt_restore(c) == -1
    assert lib.ttt_settle_chunk(c, p, p, 64, None, None) == -1
    assert lib.ttt_prefill_batch(c, p, 64, 64) == -1        # row stride below n + 1
    assert lib.ttt_prefill_batch(c, p, 65, 32) == -1        # not whole chunks
    assert lib.ttt_stream_token_losses(c, 2, p, 0, 0) == -1  # stream out of range
    assert lib.ttt_stream_fast_weights(c, -1, 0, 2, 0, p) == -1
    assert ctx.consumed() == 0
    ctx.close()

"""Blocks with frozen sliding-window attention ("End-to-End Test-Time Training for Long
Context", section 3: a window of k >= b positions before the MLPs) through the C ABI, vs the
fp64 oracle.

The attention runs in bf16 with heads of 128. Each position's key and value are computed at
its own chunk's weights and kept in a ring; later chunks read them as constants, and the
inner loop backpropagates through the current chunk's queries, keys and values into the fast
blocks below. Checks: windows shorter than, equal to and longer than the chunk and than the
whole stream, one and two heads, with and without the static MLP, several prefill calls,
batched streams, the fuller-block 760M shape (sampled), and the calls an attention context
refuses. Gates are those of tests/_parity.py (bf16).
"""
import numpy as np
import pytest

from _parity import compare, device_weights, gpu_run, log, oracle_run

import ttt_workloads as W

pytestmark = pytest.mark.gpu

BASE = dict(vocab=2000, d_model=128, d_hidden=256, n_blocks=3, n_tokens=256, chunk=64, lr=0.05, swa_heads=1)


@pytest.mark.parametrize("window,static,d,calls", [
    (96, 192, 128, 2),   # window between the chunk and the stream, static MLP, two calls
    (64, 0, 256, 1),     # window = chunk, two heads, no static MLP
    (40, 0, 128, 4),     # window shorter than the chunk, one call per chunk
    (1000, 128, 128, 1), # window longer than the stream (full causal attention)
])
def test_attention_blocks_match_the_oracle(ttt_lib, window, static, d, calls):
    w = W.preset("e2e760m", **dict(BASE, d_model=d, swa_heads=d // 128, swa_window=window, static_hidden=static))
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


def test_e2e760m_attention_sampled(ttt_lib):
    """The fuller 760M block (12 heads, window 8K, static MLP) in the benchmark's launch
    configuration: the first two chunks against the oracle."""
    w = W.preset("e2e760m", n_tokens=2048)
    P = W.init_weights(w, 0)
    x = W.token_stream(w, 0)
    log("attention e2e760m")
    g = gpu_run(w, P, x)
    assert g["status"] == 0
    compare(g, oracle_run(w, P, x, 2), w, "bf16", 2, label="e2e760m-attn")


def test_attention_context_refuses_single_row_calls(ttt_lib):
    import ctypes
    import torch
    import test_long_context_chunk_amd as ttt
    w = W.preset("e2e760m", **dict(BASE, swa_window=64, static_hidden=0, n_blocks=1))
    P = W.init_weights(w, 0)
    ctx = ttt.TTT.from_workload(w, device_weights(P, "bf16"), max_tokens=128)
    lib, c = ctx._lib, ctx._ctx
    tok = torch.zeros(130, dtype=torch.int32, device="cuda")
    p = ctypes.c_void_p(tok.data_ptr())
    assert lib.ttt_decode(c, p, 1, None, None) == -1
    assert lib.ttt_evaluate(c, p, 64, None, None) == -1
    assert lib.ttt_snapshot(c) == -1
    assert lib.ttt_settle_chunk(c, p, p, 64, None, None) == -1
    ctx.prefill(tok[:65])
    assert ctx.sync() == 0 and ctx.consumed() == 64
    ctx.close()

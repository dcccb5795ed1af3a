"""ttt_settle_chunk_noalloc: the Settlement step with its snapshot in the library's static
scratch (for callers that cannot allocate), against ttt_settle_chunk on a twin context.

Two calls in a row on one GPU, the second on a smaller context (a smaller snapshot in the
same array): each leaves A, the decision, the recorded losses, the chunk statistics and the
fast state bit for bit as ttt_settle_chunk does (same kernels, same order), and the stream
then goes on identically. The call allocates no device memory (free memory is unchanged
across it), and a context whose snapshot exceeds the array is refused with nothing enqueued.
"""
import numpy as np
import pytest

from _parity import device_weights, inputs, log

pytestmark = pytest.mark.gpu


def _tok(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def _state(ctx, w):
    return {f"{n}.{l}": ctx.fast_weight(l, n, "delta").cpu().numpy() for l in range(w.n_blocks)
            for n in w.fast_names()}


def _twin_settle(name, precision, lr, expect, **over):
    import torch
    import test_long_context_chunk_amd as ttt
    w, x, P = inputs(name, 0, **over)
    b = w.chunk
    dev = device_weights(P, precision)
    a = ttt.TTT.from_workload(w, dev, max_tokens=3 * b, precision=precision, lr=lr)
    c = ttt.TTT.from_workload(w, dev, max_tokens=3 * b, precision=precision, lr=lr)
    for z in (a, c):
        z.prefill(_tok(x[:b + 1]))
    cand, q = _tok(x[b:2 * b + 1]), _tok(x[b:2 * b + 1])  # the candidate's own text: A's sign is known
    A1, k1 = a.settle(cand, q)
    A2 = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
    k2 = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    c.settle_noalloc(cand, q, A2, k2)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    A1, k1 = float(A1.cpu()[0]), int(k1.cpu()[0])
    A2, k2 = float(A2.cpu()[0]), int(k2.cpu()[0])
    log(f"[no-alloc settle {name} {precision} lr={lr}] A {A1:.6g} / {A2:.6g} kept {k1} / {k2} "
        f"free memory change {free1 - free0}")
    assert k1 == expect and k2 == k1
    assert np.float32(A1).tobytes() == np.float32(A2).tobytes()
    assert free1 == free0
    assert a.consumed() == c.consumed() == 2 * b
    assert np.array_equal(a.token_losses().cpu().numpy(), c.token_losses().cpu().numpy())
    assert np.array_equal(a.chunk_stats().cpu().numpy(), c.chunk_stats().cpu().numpy())
    sa, sc = _state(a, w), _state(c, w)
    for k in sa:
        assert np.array_equal(sa[k], sc[k]), k
    for z in (a, c):
        z.prefill(_tok(x[2 * b:3 * b + 1]))
    assert np.array_equal(a.token_losses().cpu().numpy(), c.token_losses().cpu().numpy())
    sa, sc = _state(a, w), _state(c, w)
    for k in sa:
        assert np.array_equal(sa[k], sc[k]), k
    assert a.sync() == 0 and c.sync() == 0
    a.close()
    c.close()


def test_noalloc_settlement_two_calls_in_a_row(ttt_lib):
    # first: the single-block shape (4.7M fast parameters, a 37.7 MB snapshot), kept
    _twin_settle("single", "bf16", 100.0, 1, n_tokens=3072)
    # second, smaller: d = 256, m = 1024 (0.5M fast parameters), fp32, an overshooting step
    # that the rule rejects
    _twin_settle("single", "fp32", 5000.0, 0, vocab=4096, d_model=256, d_hidden=1024, chunk=256, n_tokens=768)


def test_noalloc_settlement_refuses_a_snapshot_beyond_the_array(ttt_lib):
    import test_long_context_chunk_amd as ttt
    w, x, P = inputs("s125m", 0, n_tokens=2048)  # 14.2M fast parameters: 113 MB > 64 MiB
    ctx = ttt.TTT.from_workload(w, device_weights(P, "bf16"), max_tokens=2048)
    import torch
    A = torch.zeros(1, dtype=torch.float32, device="cuda")
    k = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(ttt.TTTError) as e:
        ctx.settle_noalloc(_tok(x[:1025]), _tok(x[:1025]), A, k)
    assert e.value.status == -1  # TTT_EINVAL
    assert ctx.consumed() == 0 and ctx.sync() == 0
    ctx.close()

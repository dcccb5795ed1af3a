"""Blocks with a frozen static MLP before the fast one ("End-to-End Test-Time Training for
Long Context", section 3.1, two MLP layers per block) through the C ABI, vs the fp64 oracle.

The static MLP is never updated, but the inner loop backpropagates through it for every
fast block below it, and in bf16 its rounded operands join the loss compensation. Checks:
prefill parity at a small shape (both norms, both precisions, two calls), a batched
context, decode across a chunk boundary, the fuller-block 760M shape in the benchmark's
launch configuration (sampled), and that Ws2 = 0 reproduces the plain model's GPU run.
Gates are those of tests/_parity.py.
"""
import numpy as np
import pytest

from _parity import TOL, argmax_gate_rows, compare, device_weights, gpu_run, log, oracle_run, rel_l2

import oracle as O
import ttt_workloads as W

pytestmark = pytest.mark.gpu

SMALL = dict(vocab=2000, d_model=128, d_hidden=256, n_blocks=3, n_tokens=256, chunk=64, static_hidden=192,
             lr=0.05, swa_window=0, swa_heads=0)


def _tok(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


@pytest.mark.parametrize("precision,norm", [("bf16", "rms"), ("fp32", "rms"), ("bf16", "none"), ("fp32", "none")])
def test_static_mlp_blocks_match_the_oracle(ttt_lib, precision, norm):
    w = W.preset("e2e760m", precision=precision, norm=norm, **SMALL)
    P = W.init_weights(w, 3)
    x = W.token_stream(w, 4)
    log(f"static {precision} {norm}")
    g = gpu_run(w, P, x, calls=2)
    assert g["status"] == 0
    orc = oracle_run(w, P, x, w.n_chunks, gpu_argmax=g["argmax"])
    compare(g, orc, w, precision, w.n_chunks, label=f"static-{norm}")


def test_static_mlp_batched_streams(ttt_lib):
    """Two streams of one batched context, each against the oracle on its own tokens."""
    from test_gpu_batch import gpu_run_batch
    w = W.preset("e2e760m", **SMALL)
    P = W.init_weights(w, 5)
    xs = [W.token_stream(w, 6), W.token_stream(w, 7)]
    gs = gpu_run_batch(w, P, xs, w.n_tokens)
    for z, (g, x) in enumerate(zip(gs, xs)):
        assert g["status"] == 0
        compare(g, oracle_run(w, P, x, w.n_chunks), w, "bf16", w.n_chunks, label=f"static-batch stream {z}")


@pytest.mark.parametrize("precision", ["bf16", "fp32"])
def test_static_mlp_decode_matches_oracle_decode(ttt_lib, precision):
    """One prefilled chunk, then 1.5 chunks decoded in two calls (one step in between)."""
    import test_long_context_chunk_amd as ttt
    w = W.preset("e2e760m", precision=precision, **SMALL)
    P = W.init_weights(w, 8)
    x = W.token_stream(w, 9)
    b = w.chunk
    n = b + b // 2
    ctx = ttt.TTT.from_workload(w, device_weights(P, precision), max_tokens=w.n_tokens)
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
    model = O.Model.from_workload(w)
    rows = []
    # the oracle's decode: one prefilled chunk's step, then token by token with a step at the
    # chunk boundary (the first b tokens decoded, then prefill-equivalent)
    orc = O.decode_ttt(model, P, x[:b + n + 1], logit_probe=lambda t, z, h: rows.append((t, z.copy(), h.copy())))
    Z = np.stack([z for t, z, h in rows if t >= b])
    H = np.stack([h for t, z, h in rows if t >= b])
    tol = TOL[precision]
    dz = float(np.max(np.abs(zg - Z)))
    dd = max(rel_l2(Dg[k], orc.delta[k]) for k in orc.delta)
    log(f"[static decode {precision}] logits {dz:.3g} D {dd:.3g}")
    assert dz <= tol["logit"]
    assert dd <= tol["dw"]
    argmax_gate_rows(am, Z, H, P["E_out"], precision, f"static decode")


def test_e2e760m_two_chunks_sampled(ttt_lib):
    """The fuller-block 760M shape (d=1536, fast and static hidden 3072, 3 blocks) in the
    benchmark's launch configuration: the first two chunks against the oracle."""
    w = W.preset("e2e760m", n_tokens=2048, swa_window=0, swa_heads=0)
    P = W.init_weights(w, 0)
    x = W.token_stream(w, 0)
    log("static e2e760m")
    g = gpu_run(w, P, x)
    assert g["status"] == 0
    compare(g, oracle_run(w, P, x, 2), w, "bf16", 2, label="e2e760m")


def test_zero_static_projection_reproduces_the_plain_gpu_run(ttt_lib):
    """Ws2 = 0 on the GPU (fp32): every static MLP adds exact zeros and passes the gradient
    through unchanged, so losses, steps and updates equal a plain context's bit for bit."""
    w = W.preset("e2e760m", precision="fp32", **SMALL)
    P = W.init_weights(w, 10)
    for l in range(w.n_blocks):
        P[f"Ws2.{l}"] = np.zeros_like(P[f"Ws2.{l}"])
    x = W.token_stream(w, 11)
    a = gpu_run(w, P, x)
    plain = w.replace(static_hidden=0)
    b = gpu_run(plain, {k: v for k, v in P.items() if not k.startswith("Ws")}, x)
    assert np.array_equal(a["losses"], b["losses"])
    assert np.array_equal(a["stats"], b["stats"])
    for k in a["D"]:
        assert np.array_equal(a["D"][k], b["D"][k]), k

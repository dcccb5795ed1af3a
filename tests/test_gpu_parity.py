"""HIP path (through the C ABI) vs the fp64 oracle on the same seeded inputs.

Every test here needs an MI355X and the built library; it fails loudly if the library
cannot be loaded. Gates are described in tests/_parity.py.
"""
import math

import numpy as np
import pytest

from _parity import TOL, compare, device_weights, gpu_run, inputs, log, oracle_run, rel_l2

import oracle as O
import ttt_workloads as W

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------------- GEMM tile engine
GEMM_SHAPES = [(1, 64, 64), (1, 256, 256), (16, 8, 8), (37, 100, 136), (128, 128, 64), (1024, 16384, 64), (520, 33000, 128),
               (130, 129, 520), (257, 300, 72), (64, 64, 6144), (1024, 768, 200), (300, 700, 2048), (1024, 6144, 3072)]


@pytest.mark.parametrize("precision", ["bf16", "fp32"])
@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_gemm_tile_engine_ragged(ttt_lib, precision, M, N, K):
    import torch
    rng = np.random.default_rng(M * 7919 + N * 31 + K)
    X = rng.standard_normal((M, K)).astype(np.float32)
    Y = rng.standard_normal((N, K)).astype(np.float32)
    if precision == "bf16":
        X, Y = W.round_to_bf16(X), W.round_to_bf16(Y)
    log(f"gemm {precision} M={M} N={N} K={K}")
    C = ttt_lib.gemm_test_hook(ttt_lib.to_device(X, precision), ttt_lib.to_device(Y, precision), precision)
    torch.cuda.synchronize()
    C = C.cpu().numpy().astype(np.float64)
    ref = X.astype(np.float64) @ Y.astype(np.float64).T
    bound = (K + 2) * 2.0 ** -24 * (np.abs(X).astype(np.float64) @ np.abs(Y).astype(np.float64).T) + 1e-30
    assert np.all(np.abs(C - ref) <= bound), float(np.max(np.abs(C - ref) / bound))


# ---------------------------------------------------------------------- gather (bit-exact ids)
@pytest.mark.parametrize("precision", ["bf16", "fp32"])
def test_gather_rows_are_exact(ttt_lib, precision):
    """L = 0 and E_out = I: the logits are the gathered embedding row itself, so the argmax
    names which row was gathered (integer result, compared exactly) and the loss is the CE
    of that exact row."""
    V = d = 64
    rng = np.random.default_rng(5)
    E_in = rng.uniform(-1, 0, (V, d)).astype(np.float32)
    peak = (np.arange(V) * 7) % d
    E_in[np.arange(V), peak] = 1.0
    P = {"E_in": E_in, "E_out": np.eye(V, d, dtype=np.float32)}
    w = W.Workload(name="gather", vocab=V, d_model=d, d_hidden=64, n_blocks=0, mlp="gelu", norm="none",
                   precision=precision, n_tokens=96, chunk=32, lr=0.0, clip=0.0, stream="markov")
    if precision == "bf16":
        P = {k: W.round_to_bf16(v) for k, v in P.items()}
    x = rng.integers(0, V, 97).astype(np.int32)
    g = gpu_run(w, P, x)
    assert g["status"] == 0
    assert np.array_equal(g["argmax"], peak[x[:-1]])
    static = O.static_losses(O.Model.from_workload(w), P, x)
    assert np.max(np.abs(g["losses"] - static)) <= TOL[precision]["loss"] * 0.1


@pytest.mark.parametrize("precision", ["bf16", "fp32"])
def test_lm_head_only_matches_naive_loss(ttt_lib, precision):
    """n_blocks = 0: every loss is the static l_t(W0) of the oracle (vocab tiles ragged)."""
    w = W.preset("single", vocab=1000, d_model=64, d_hidden=64, n_blocks=0, n_tokens=256, chunk=64,
                 precision=precision)
    _, x, P = inputs("single", 0, vocab=1000, d_model=64, d_hidden=64, n_blocks=0, n_tokens=256, chunk=64)
    g = gpu_run(w, P, x)
    orc = oracle_run(w, P, x, 4, gpu_argmax=g["argmax"])
    compare(g, orc, w, precision, 4, check_weights=False, label="lm-head")


# ---------------------------------------------------------------------- the five workloads
def test_toy_fp32_per_token_full(ttt_lib):
    """MLP-only bigram toy: chunk 1 (per-token rule), fp32, all 128 steps."""
    w, x, P = inputs("toy")
    g = gpu_run(w, P, x)
    orc = oracle_run(w, P, x, w.n_chunks, gpu_argmax=g["argmax"])
    compare(g, orc, w, "fp32", w.n_chunks, label="toy")


@pytest.fixture(scope="module")
def single_oracle():
    w, x, P = inputs("single")
    return oracle_run(w, P, x, w.n_chunks, key="single")


@pytest.mark.parametrize("precision", ["bf16", "fp32"])
def test_single_block_full_stream(ttt_lib, single_oracle, precision):
    """One GELU block, d=768, m=3072, V=32000, b=1024, 8 chunks, clip 1.0."""
    w, x, P = inputs("single")
    g = gpu_run(w, P, x, precision=precision)
    assert g["status"] == 0
    orc = single_oracle
    # the argmax validity gate needs the oracle logits at the GPU's picks
    orc_p = oracle_run(w, P, x, 2, gpu_argmax=g["argmax"])
    compare(g, orc_p, w, precision, 2, check_weights=False, label="single-argmax")
    compare(g, orc, w, precision, w.n_chunks, label="single")


@pytest.fixture(scope="module")
def s760m_oracle():
    w, x, P = inputs("s760m")
    return oracle_run(w, P, x, 2, key="s760m")


@pytest.mark.parametrize("precision", ["bf16", "fp32"])
def test_s760m_two_chunk_prefix(ttt_lib, s760m_oracle, precision):
    """760M shape (3 pre-RMSNorm GELU blocks, d=1536, m=6144): first two chunks."""
    w, x, P = inputs("s760m")
    g = gpu_run(w, P, x, n_tokens=2 * w.chunk, precision=precision)
    assert g["status"] == 0
    compare(g, s760m_oracle, w, precision, 2, label="s760m")


def test_s760m_full_stream_properties(ttt_lib, s760m_oracle):
    """Full 32K-token stream in the benchmark's launch configuration (one prefill call):
    its first two chunks match the oracle's prefix; the first chunks obey the clip identity
    ||W_i - W_{i-1}||_F = lr * min(g_i, c); the same stream fed as per-chunk calls gives
    bitwise identical losses and updates."""
    import torch
    import test_long_context_chunk_amd as ttt
    w, x, P = inputs("s760m")
    dev = device_weights(P, "bf16")
    full = gpu_run(w, P, x, dev=dev)
    assert full["status"] == 0
    assert np.all(np.isfinite(full["losses"]))
    orc = s760m_oracle
    n = 2 * w.chunk
    assert np.max(np.abs(full["losses"][:n] - orc.losses[:n])) <= TOL["bf16"]["loss"]
    assert np.max(np.abs(full["stats"][:2, 0] - orc.grad_norm[:2]) / orc.grad_norm[:2]) <= TOL["bf16"]["g"]

    ctx = ttt.TTT.from_workload(w, dev, max_tokens=w.n_tokens)
    tok = torch.from_numpy(x.astype(np.int32)).cuda()
    keys = list(full["D"])

    def delta():
        return {k: ctx.fast_weight(int(k.split(".")[1]), k.split(".")[0], "delta").cpu().numpy().astype(np.float64)
                for k in keys}

    prev = {k: np.zeros_like(full["D"][k]) for k in keys}
    worst = 0.0
    for i in range(w.n_chunks):
        ctx.prefill(tok[i * w.chunk:(i + 1) * w.chunk + 1])
        if i < 4:
            D = delta()
            g_i, s_i = ctx.chunk_stats(i, 1).cpu().numpy()[0]
            step = math.sqrt(sum(float(np.sum((D[k] - prev[k]) ** 2)) for k in keys))
            expect = w.lr * min(g_i, w.clip)
            worst = max(worst, abs(step - expect) / expect)
            prev = D
    losses = ctx.token_losses().cpu().numpy()
    D = delta()
    ctx.close()
    log(f"[s760m full] clip identity worst rel err {worst:.3g}")
    assert worst <= 1e-3
    assert np.array_equal(losses, full["losses"].astype(np.float32))
    for k in keys:
        assert np.array_equal(D[k], full["D"][k])


def test_s760m_zero_lr_full_stream_is_static(ttt_lib):
    """eta = 0 over the whole 32K stream: every loss is the static l_t(W0), checked by the
    oracle on sampled tokens one by one; the fast weights do not move."""
    w, x, P = inputs("s760m")
    g = gpu_run(w, P, x, lr=0.0)
    rng = np.random.default_rng(0)
    idx = np.sort(rng.choice(w.n_tokens, 96, replace=False))
    model = O.Model.from_workload(w)
    ref, _, _ = O.token_losses(model, O.as_f64(P), x[idx], x[idx + 1])
    assert np.max(np.abs(g["losses"][idx] - ref)) <= TOL["bf16"]["loss"]
    for k, D in g["D"].items():
        assert not D.any()


@pytest.mark.parametrize("precision", ["bf16", "fp32"])
def test_s125m_two_chunk_prefix(ttt_lib, precision):
    """125M-style stack (3 pre-RMSNorm blocks, d=768): first two chunks of the 128K stream."""
    w, x, P = inputs("s125m")
    orc = oracle_run(w, P, x, 2, key="s125m")
    g = gpu_run(w, P, x, n_tokens=2 * w.chunk, precision=precision)
    assert g["status"] == 0
    compare(g, orc, w, precision, 2, label="s125m")


def test_inplace_swiglu_first_chunk(ttt_lib):
    """In-Place shape: SwiGLU (gate/up frozen), only W2 fast, V=151936, b=512."""
    w, x, P = inputs("inplace")
    orc = oracle_run(w, P, x, 1, key="inplace")
    g = gpu_run(w, P, x, n_tokens=w.chunk)
    assert g["status"] == 0
    compare(g, orc, w, "bf16", 1, label="inplace")


# ---------------------------------------------------------------------- determinism, errors
def test_runs_are_bitwise_deterministic(ttt_lib):
    w, x, P = inputs("single")
    dev = device_weights(P, "bf16")
    a = gpu_run(w, P, x, n_tokens=3 * w.chunk, dev=dev)
    b = gpu_run(w, P, x, n_tokens=3 * w.chunk, dev=dev)
    assert np.array_equal(a["losses"], b["losses"])
    assert np.array_equal(a["stats"], b["stats"])
    for k in a["D"]:
        assert np.array_equal(a["D"][k], b["D"][k])


def test_reset_restores_initial_weights(ttt_lib):
    import torch
    import test_long_context_chunk_amd as ttt
    w, x, P = inputs("single", n_tokens=2048)
    dev = device_weights(P, "bf16")
    ctx = ttt.TTT.from_workload(w, dev, max_tokens=2048)
    tok = torch.from_numpy(x[:2049].astype(np.int32)).cuda()
    ctx.prefill(tok)
    l1 = ctx.token_losses().cpu().numpy()
    ctx.reset()
    assert ctx.consumed() == 0
    assert not ctx.fast_weight(0, "W2", "delta").any().item()
    ctx.prefill(tok)
    assert np.array_equal(l1, ctx.token_losses().cpu().numpy())
    ctx.close()


def test_out_of_range_token_is_a_sticky_error(ttt_lib):
    import torch
    import test_long_context_chunk_amd as ttt
    w, x, P = inputs("single", n_tokens=2048)
    ctx = ttt.TTT.from_workload(w, device_weights(P, "bf16"), max_tokens=2048)
    bad = x[:1025].astype(np.int32).copy()
    bad[100] = w.vocab + 5
    ctx.prefill(torch.from_numpy(bad).cuda())
    assert ctx.sync() == -4  # TTT_ERANGE
    with pytest.raises(ttt.TTTError) as e:
        ctx.prefill(torch.from_numpy(x[1024:2049].astype(np.int32)).cuda())
    assert e.value.status == -6  # TTT_ESTATE
    ctx.reset()
    assert ctx.sync() == 0
    ctx.close()


def test_nonfinite_gradient_skips_the_step(ttt_lib):
    """A NaN in an embedding row read by chunk 1 makes g non-finite: that chunk takes no
    step (stats s = 0), the error is reported, and the weights stay exactly W0."""
    import test_long_context_chunk_amd as ttt
    w, x, P = inputs("single", n_tokens=2048)
    P = dict(P)
    E = P["E_in"].copy()
    E[x[3]] = np.nan
    P["E_in"] = E
    g = gpu_run(w, P, x, n_tokens=1024)
    assert g["status"] == -5  # TTT_ENONFINITE
    assert g["stats"][0, 1] == 0.0
    for D in g["D"].values():
        assert not D.any()


def test_prefill_argument_errors(ttt_lib):
    import torch
    import test_long_context_chunk_amd as ttt
    w, x, P = inputs("single", n_tokens=2048)
    ctx = ttt.TTT.from_workload(w, device_weights(P, "bf16"), max_tokens=1024)
    tok = torch.from_numpy(x[:2049].astype(np.int32)).cuda()
    with pytest.raises(ttt.TTTError):
        ctx.prefill(tok[:1000])  # not a multiple of the chunk
    with pytest.raises(ttt.TTTError):
        ctx.prefill(tok)  # beyond max_tokens
    ctx.close()

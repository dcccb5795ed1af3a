"""HIP path (through the C ABI) vs the fp64 oracle on the same seeded inputs.

Every test here needs an MI355X and the built library; it fails loudly if the library
cannot be loaded. Gates are described in tests/_parity.py.
"""
import math

import numpy as np
import pytest

from _parity import TOL, argmax_gate_rows, compare, device_weights, gpu_run, inputs, log, oracle_run, rel_l2

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


# (M, N, K, splits): the 760M up product (one slab) and down product (5 slabs), the In-Place
# down product (M = 512), ragged rows and columns with an uneven last slab and an empty one;
# on 256 x 64 tiles the 125M-style up product and a ragged one; a short-K product (its tile
# plan walks the two segments one after the other).
PAIR_SHAPES = [(1024, 6144, 1536, 1), (1024, 1536, 6144, 5), (512, 2560, 9728, 4), (300, 200, 576, 3),
               (257, 130, 1024, 7), (1024, 3072, 768, 1), (300, 200, 576, 1), (1, 8, 64, 1)]


@pytest.mark.parametrize("form", [0, 1, 2])
@pytest.mark.parametrize("M,N,K,splits", PAIR_SHAPES)
def test_gemm_two_weights_shared_rows(ttt_lib, M, N, K, splits, form):
    """The bf16 forward product X (W0 + rn(D))^T as two K-segments over the same rows of X,
    split over K into slabs, in each form of the tile engine (the inner loop's choice, the
    segments one after the other, shared X slices): the slab sum within the fp32
    accumulation bound of the fp64 product, on ragged shapes."""
    import torch
    rng = np.random.default_rng(M * 7 + N * 13 + K + splits)
    X = W.round_to_bf16(rng.standard_normal((M, K)).astype(np.float32))
    Y = W.round_to_bf16(0.02 * rng.standard_normal((N, K)).astype(np.float32))
    Y2 = W.round_to_bf16(1e-4 * rng.standard_normal((N, K)).astype(np.float32))
    log(f"gemm pair M={M} N={N} K={K} splits={splits} form={form}")
    C = ttt_lib.gemm_pair_test_hook(ttt_lib.to_device(X, "bf16"), ttt_lib.to_device(Y, "bf16"),
                                    ttt_lib.to_device(Y2, "bf16"), splits, form)
    torch.cuda.synchronize()
    C = C.cpu().numpy().astype(np.float64).sum(axis=0)
    X64, Y64, Y264 = (a.astype(np.float64) for a in (X, Y, Y2))
    ref = X64 @ Y64.T + X64 @ Y264.T
    bound = (2 * K + splits + 2) * 2.0 ** -24 * (np.abs(X64) @ (np.abs(Y64) + np.abs(Y264)).T) + 1e-30
    assert np.all(np.abs(C - ref) <= bound), float(np.max(np.abs(C - ref) / bound))
    # the update's own contribution is resolved (a path that dropped Y2 fails here)
    assert np.all(np.abs(C - X64 @ Y64.T - X64 @ Y264.T) <= 0.5 * np.abs(X64 @ Y264.T) + bound)


# ---------------------------------------------------------------------- weight-gradient GEMM
# (M, N, K): the 760M W2 and W1 gradients (192 x 192 tiles), the fuller block's (128 x 128),
# ragged 128-row tiles over three and one 64-token slices, one 8 x 8 tile.
GRAD_SHAPES = [(6144, 1536, 1024), (1536, 6144, 1024), (3072, 1536, 1024), (1096, 1000, 192), (1000, 1096, 64),
               (8, 8, 64)]


@pytest.mark.parametrize("M,N,K", GRAD_SHAPES)
def test_grad_token_major_matches_transposed(ttt_lib, M, N, K):
    """A chunk gradient G = X^T Y over K tokens ([E2E] eq. 5) from the token-major operands
    (as the chunk's products write them) and from their transposed copies: both within the
    fp32-accumulation bound of the fp64 product plus one bf16 rounding, and their per-tile
    sums of squares (the grad-norm partials) within 1e-4 of the fp64 sum. On 192 x 192 tiles
    both kernels feed the MFMAs the same k order, so G and the partials are bitwise equal."""
    import torch
    rng = np.random.default_rng(M * 7919 + N * 31 + K)
    X = W.round_to_bf16(rng.standard_normal((K, M)).astype(np.float32))
    Y = W.round_to_bf16(rng.standard_normal((K, N)).astype(np.float32))
    Xd = torch.from_numpy(X).to(torch.bfloat16).cuda()
    Yd = torch.from_numpy(Y).to(torch.bfloat16).cuda()
    log(f"grad M={M} N={N} K={K}")
    Gk, sk = ttt_lib.grad_test_hook(Xd, Yd, True)
    Gt, st = ttt_lib.grad_test_hook(Xd.t().contiguous(), Yd.t().contiguous(), False)
    torch.cuda.synchronize()
    ref = X.astype(np.float64).T @ Y.astype(np.float64)
    bound = (K + 2) * 2.0 ** -24 * (np.abs(X).astype(np.float64).T @ np.abs(Y).astype(np.float64))
    bound += 2.0 ** -8 * np.abs(ref) + 1e-30
    for G in (Gk, Gt):
        g = G.float().cpu().numpy().astype(np.float64)
        assert np.all(np.abs(g - ref) <= bound), float(np.max(np.abs(g - ref) / bound))
    ss = float(np.sum(ref * ref))
    for sl in (sk, st):
        assert abs(float(sl.double().sum().item()) - ss) <= 1e-4 * ss
    # the planner's choice for short K: 192 x 192 tiles when they leave fewer outputs per CU
    # over their rounds (256 workgroups a round) than 128 x 128 tiles (512 a round)
    t192 = ((M + 191) // 192) * ((N + 191) // 192)
    t128 = ((M + 127) // 128) * ((N + 127) // 128)
    if (t192 + 255) // 256 * 192 * 192 < (t128 + 511) // 512 * 2 * 128 * 128:
        assert torch.equal(Gk, Gt)
        assert torch.equal(sk, st)


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


def test_lm_head_square_tiles_ragged(ttt_lib):
    """The LM head on 256 x 256 tiles (it fills at least one round of them) with ragged rows
    and columns: n_blocks = 0, chunk 1000, V = 32008 (a last column tile of 8), d = 1536;
    every loss is the static l_t(W0) of the oracle, every argmax gated."""
    kw = dict(vocab=32008, d_model=1536, d_hidden=64, n_blocks=0, n_tokens=1000, chunk=1000)
    w = W.preset("single", **kw)
    _, x, P = inputs("single", 0, **kw)
    log("lm head on 256 x 256 tiles: V=32008 d=1536 b=1000")
    g = gpu_run(w, P, x)
    assert g["status"] == 0
    compare(g, oracle_run(w, P, x, 1), w, "bf16", 1, check_weights=False, label="lm-head-square")


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
    compare(g, single_oracle, w, precision, w.n_chunks, label="single")


def _ttt_change_gate(g, g_static, orc, orc_static, n, label):
    """fp32 mode: the loss change that test-time training causes, l_t - l_t(W0), matches the
    oracle's within 5% of the oracle's largest change plus 2e-6 (the loss gates alone cannot
    see it where it is smaller than they are)."""
    ch_g = g["losses"][:n] - g_static[:n]
    ch_o = orc.losses[:n] - orc_static[:n]
    bound = 0.05 * float(np.max(np.abs(ch_o))) + 2e-6
    err = float(np.max(np.abs(ch_g - ch_o)))
    log(f"[ttt-change {label}] oracle max |change| {float(np.max(np.abs(ch_o))):.3g} mean {float(np.mean(ch_o)):.3g}; "
        f"GPU error {err:.3g} (bound {bound:.3g})")
    assert float(np.max(np.abs(ch_o))) > 0.0
    assert err <= bound


def test_single_block_fp32_ttt_loss_change(ttt_lib, single_oracle):
    """fp32, all 8 chunks of the single-block stream: the TTT-induced loss change."""
    w, x, P = inputs("single")
    dev = device_weights(P, "fp32")
    g = gpu_run(w, P, x, precision="fp32", dev=dev)
    g0 = gpu_run(w, P, x, precision="fp32", dev=dev, lr=0.0)
    orc_static = O.static_losses(O.Model.from_workload(w), P, x)
    _ttt_change_gate(g, g0["losses"], single_oracle, orc_static, w.n_tokens, "single fp32")


@pytest.fixture(scope="module")
def s760m_oracle():
    """The whole 32-chunk 760M-shape stream (about 40 s of fp64 on 16 host cores)."""
    w, x, P = inputs("s760m")
    log("oracle s760m: 32 chunks")
    return oracle_run(w, P, x, w.n_chunks, key="s760m")


@pytest.mark.parametrize("precision", ["bf16", "fp32"])
def test_s760m_full_stream(ttt_lib, s760m_oracle, precision):
    """760M shape (3 pre-RMSNorm GELU blocks, d=1536, m=6144), the whole 32K stream in the
    benchmark's launch configuration (one prefill call), every token and every chunk."""
    w, x, P = inputs("s760m")
    g = gpu_run(w, P, x, precision=precision)
    assert g["status"] == 0
    compare(g, s760m_oracle, w, precision, w.n_chunks, label="s760m")


def test_s760m_fp32_ttt_loss_change(ttt_lib, s760m_oracle):
    """fp32, first 4 chunks of the 760M shape: the TTT-induced loss change."""
    w, x, P = inputs("s760m")
    n = 4 * w.chunk
    dev = device_weights(P, "fp32")
    g = gpu_run(w, P, x, n_tokens=n, precision="fp32", dev=dev)
    g0 = gpu_run(w, P, x, n_tokens=n, precision="fp32", dev=dev, lr=0.0)
    orc_static = O.static_losses(O.Model.from_workload(w), P, x, n_tokens=n)
    _ttt_change_gate(g, g0["losses"], s760m_oracle, orc_static, n, "s760m fp32")


def test_s760m_full_stream_properties(ttt_lib):
    """Full 32K-token stream: the first chunks obey the clip identity
    ||W_i - W_{i-1}||_F = lr * min(g_i, c); the same stream fed as per-chunk calls gives
    bitwise identical losses and updates to one call."""
    import torch
    import test_long_context_chunk_amd as ttt
    w, x, P = inputs("s760m")
    dev = device_weights(P, "bf16")
    full = gpu_run(w, P, x, dev=dev)
    assert full["status"] == 0
    assert np.all(np.isfinite(full["losses"]))

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


@pytest.fixture(scope="module")
def s125m_oracle():
    w, x, P = inputs("s125m")
    log("oracle s125m: 16 chunks")
    return oracle_run(w, P, x, 16, key="s125m")


@pytest.mark.parametrize("precision", ["bf16", "fp32"])
def test_s125m_sixteen_chunk_prefix(ttt_lib, s125m_oracle, precision):
    """125M-style stack (3 pre-RMSNorm blocks, d=768): the first 16 chunks of the 128K stream."""
    w, x, P = inputs("s125m")
    g = gpu_run(w, P, x, n_tokens=16 * w.chunk, precision=precision)
    assert g["status"] == 0
    compare(g, s125m_oracle, w, precision, 16, label="s125m")


def test_inplace_swiglu_four_chunks(ttt_lib):
    """In-Place shape: SwiGLU (gate/up frozen), only W2 fast, V=151936, b=512; 4 chunks."""
    w, x, P = inputs("inplace")
    log("oracle inplace: 4 chunks")
    orc = oracle_run(w, P, x, 4, key="inplace")
    g = gpu_run(w, P, x, n_tokens=4 * w.chunk)
    assert g["status"] == 0
    compare(g, orc, w, "bf16", 4, label="inplace")


@pytest.mark.parametrize("name", ["s125m", "inplace"])
def test_full_stream_zero_lr_is_static(ttt_lib, name):
    """eta = 0 over the whole stream in the benchmark's launch configuration (the 125M-style
    stack's 128K tokens, the In-Place shape's 64K): sampled tokens one by one against the
    oracle's static l_t(W0) ([E2E] eq. 4), losses and the argmax gate; the fast weights do not
    move."""
    w, x, P = inputs(name)
    log(f"{name}: full stream at lr 0 ({w.n_tokens} tokens)")
    g = gpu_run(w, P, x, lr=0.0)
    assert g["status"] == 0
    rng = np.random.default_rng(11)
    idx = np.sort(rng.choice(w.n_tokens, 64, replace=False))
    model = O.Model.from_workload(w)
    z, h, _ = O.logits(model, O.as_f64(P), x[idx])
    ref, _, _, _ = O.ce_stats(z, x[idx + 1])
    err = float(np.max(np.abs(g["losses"][idx] - ref)))
    log(f"[{name} lr 0, 64 sampled tokens] loss max |d| {err:.3g}")
    assert err <= TOL["bf16"]["loss"]
    argmax_gate_rows(g["argmax"][idx], z, h, P["E_out"], "bf16", label=f"{name}-lr0")
    for k, D in g["D"].items():
        assert not D.any(), k


@pytest.mark.parametrize("name", ["s125m", "inplace", "e2e760m"])
def test_full_stream_properties(ttt_lib, name):
    """The whole stream (128K tokens of the 125M-style stack, 64K of the In-Place shape, 32K of
    the fuller block with window-8192 attention, its rings wrapping three times over): one
    prefill call leaves every loss finite and every argmax a valid id; every chunk's clip
    scale is min(1, c / g_i) of its own grad norm ([SGF] "how it works"); the first chunks'
    steps obey ||W_i - W_{i-1}||_F = lr min(g_i, c); and the same stream as per-chunk calls
    gives bitwise the same losses and updates."""
    import torch
    import test_long_context_chunk_amd as ttt
    w, x, P = inputs(name)
    dev = device_weights(P, "bf16")
    log(f"{name}: full stream ({w.n_tokens} tokens), one call")
    full = gpu_run(w, P, x, dev=dev)
    assert full["status"] == 0
    assert np.all(np.isfinite(full["losses"]))
    assert full["argmax"].min() >= 0 and full["argmax"].max() < w.vocab
    g_i, s_i = full["stats"][:, 0], full["stats"][:, 1]
    assert np.all(np.isfinite(g_i)) and np.all(g_i > 0)
    assert np.max(np.abs(s_i - np.minimum(1.0, w.clip / g_i))) <= 1e-6
    log(f"{name}: per-chunk calls ({w.n_chunks})")
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
        if i < 3:
            D = delta()
            gi, si = ctx.chunk_stats(i, 1).cpu().numpy()[0]
            step = math.sqrt(sum(float(np.sum((D[k] - prev[k]) ** 2)) for k in keys))
            expect = w.lr * min(gi, w.clip)
            worst = max(worst, abs(step - expect) / expect)
            prev = D
    losses = ctx.token_losses().cpu().numpy()
    D = delta()
    ctx.close()
    log(f"[{name} full] clip identity worst rel err {worst:.3g}")
    assert worst <= 1e-3
    assert np.array_equal(losses, full["losses"].astype(np.float32))
    for k in keys:
        assert np.array_equal(D[k], full["D"][k]), k


def test_narrow_tile_products_ragged(ttt_lib):
    """Long-K products whose 256 x 128 tiles would leave most CUs idle run on 256 x 64 tiles:
    here d = 1152 (K above 1024), m = 1000 and V = 3000 (ragged against 64 columns) and chunk
    200 (ragged against 256 rows), so the up product (GELU epilogue), dA (its partial dots
    through LDS) and the LM head (32-column CE records) all take that plan; three chunks,
    every gate."""
    w = W.preset("s125m", vocab=3000, d_model=1152, d_hidden=1000, n_blocks=2, n_tokens=600, chunk=200, lr=0.05)
    P = W.init_weights(w, 5)
    x = W.token_stream(w, 6)
    log("narrow tiles: d=1152 m=1000 V=3000 b=200")
    g = gpu_run(w, P, x)
    assert g["status"] == 0
    compare(g, oracle_run(w, P, x, 3), w, "bf16", 3, label="narrow-tiles")


def test_token_major_gradients_ragged(ttt_lib):
    """bf16 weight gradients read the activations token-major when the chunk is a whole
    number of 64-token slices: here chunk 192 (three slices, an odd count against the
    two-stage loop) with d = 1000 and m = 1096, neither a multiple of the 128-row tiles, so
    the edge tiles clamp their columns and mask their outputs; three chunks, every gate."""
    w = W.preset("s125m", vocab=3000, d_model=1000, d_hidden=1096, n_blocks=2, n_tokens=576, chunk=192, lr=0.05)
    P = W.init_weights(w, 7)
    x = W.token_stream(w, 8)
    log("token-major gradients: d=1000 m=1096 b=192")
    g = gpu_run(w, P, x)
    assert g["status"] == 0
    compare(g, oracle_run(w, P, x, 3), w, "bf16", 3, label="token-major")


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


def test_absurd_capacity_is_out_of_memory(ttt_lib):
    """A context whose per-token records cannot fit (max_tokens = 2^42: 16 TiB of losses)
    fails with TTT_ENOMEM, frees what it had allocated, and leaves the device usable: a
    normal context created next runs and matches a fresh run bit for bit."""
    import torch
    import test_long_context_chunk_amd as ttt
    w, x, P = inputs("single", n_tokens=1024)
    dev = device_weights(P, "bf16")
    with pytest.raises(ttt.TTTError) as e:
        ttt.TTT.from_workload(w, dev, max_tokens=1 << 42)
    assert e.value.status == -2  # TTT_ENOMEM
    torch.cuda.synchronize()
    a = gpu_run(w, P, x, dev=dev)
    b = gpu_run(w, P, x, dev=dev)
    assert a["status"] == 0 and np.array_equal(a["losses"], b["losses"])


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

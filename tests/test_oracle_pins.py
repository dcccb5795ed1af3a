"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Pages cited (by title and section/equation):
  [E2E] "End-to-End Test-Time Training for Long Context" review (kimjy99.github.io)
  [SGF] "Self-Generated Feedback Destabilizes Test-Time Training" summary (onedev.kr)
The pages print no worked numeric example of the inner loop, so each pin is a
closed form, an identity the equations imply, a library special case, finite
differences, or an independently written second implementation (torch fp64
autograd on the CPU). None of these tests calls the HIP library.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import oracle.ttt_oracle as O
import ttt_workloads as W


def tiny_model(mlp="gelu", norm="none", L=2, b=3, lr=0.3, clip=0.0, V=11, d=6, m=10, ms=0, win=0, heads=0):
    return O.Model(vocab=V, d_model=d, d_hidden=m, n_blocks=L, mlp=mlp, norm=norm,
                   eps=1e-6, chunk=b, lr=lr, clip=clip, static_hidden=ms, swa_window=win, swa_heads=heads)


def tiny_params(model, seed=0, std=0.5):
    rng = np.random.default_rng(seed)
    P = {"E_in": rng.normal(0, std, (model.vocab, model.d_model)),
         "E_out": rng.normal(0, std, (model.vocab, model.d_model))}
    for l in range(model.n_blocks):
        if model.mlp == "gelu":
            P[f"W1.{l}"] = rng.normal(0, std, (model.d_model, model.d_hidden))
        else:
            P[f"Wg.{l}"] = rng.normal(0, std, (model.d_model, model.d_hidden))
            P[f"Wu.{l}"] = rng.normal(0, std, (model.d_model, model.d_hidden))
        P[f"W2.{l}"] = rng.normal(0, std, (model.d_hidden, model.d_model))
    for l in range(model.n_blocks if model.static_hidden > 0 else 0):
        P[f"Ws1.{l}"] = rng.normal(0, std, (model.d_model, model.static_hidden))
        P[f"Ws2.{l}"] = rng.normal(0, std, (model.static_hidden, model.d_model))
    for l in range(model.n_blocks if model.swa_window > 0 else 0):
        for n in ("Wq", "Wk", "Wv", "Wo"):
            P[f"{n}.{l}"] = rng.normal(0, std, (model.d_model, model.d_model))
    return P


def tiny_tokens(model, n, seed=1):
    rng = np.random.default_rng(seed)
    x = rng.integers(0, model.vocab, n + 1)
    x[0] = 0
    return x


COMBOS = [("gelu", "none"), ("gelu", "rms"), ("swiglu_w2", "none"), ("swiglu_w2", "rms")]


# ------------------------------------------------------------------ P1 finite differences
def fd_check(model, P, x_prev, x_tgt, h=1e-5):
    _, _, G = O.chunk_loss_and_grads(model, P, x_prev, x_tgt)
    worst = 0.0
    for k in model.fast_keys():
        fd = np.zeros_like(P[k])
        for idx in np.ndindex(P[k].shape):
            Pp = dict(P); Pp[k] = P[k].copy(); Pp[k][idx] += h
            Pm = dict(P); Pm[k] = P[k].copy(); Pm[k][idx] -= h
            lp, _, _ = O.chunk_loss_and_grads(model, Pp, x_prev, x_tgt)
            lm, _, _ = O.chunk_loss_and_grads(model, Pm, x_prev, x_tgt)
            fd[idx] = (lp - lm) / (2 * h)
        rel = np.linalg.norm(fd - G[k]) / max(np.linalg.norm(G[k]), 1e-30)
        worst = max(worst, rel)
    return worst


@pytest.mark.parametrize("mlp,norm", COMBOS)
def test_p1_finite_differences(mlp, norm):
    """Backprop of eq. (1) through every block type matches central differences."""
    model = tiny_model(mlp, norm, L=2, b=3)
    P = tiny_params(model, seed=3)
    x = tiny_tokens(model, 3, seed=4)
    assert fd_check(model, P, x[:-1], x[1:]) < 1e-6


# ------------------------------------------------------------------ P2 b = 1 is eq. (2)
@pytest.mark.parametrize("mlp,norm", COMBOS)
def test_p2_chunk_one_is_per_token_rule(mlp, norm):
    """[E2E] eq. (5) with b = 1 is the online rule of eq. (2): W_t = W_{t-1} - eta grad l_t(W_{t-1})."""
    model = tiny_model(mlp, norm, L=2, b=1, lr=0.2)
    P = tiny_params(model, seed=5)
    x = tiny_tokens(model, 9, seed=6)
    res = O.run_ttt(model, P, x)
    # independent loop: explicit sequence of single-token steps
    Wc = {k: P[k].copy() for k in model.fast_keys()}
    losses = []
    for t in range(1, len(x)):
        Pt = dict(P); Pt.update(Wc)
        lt, _, G = O.chunk_loss_and_grads(model, Pt, x[t - 1:t], x[t:t + 1])
        losses.append(lt)
        for k in Wc:
            Wc[k] = Wc[k] - model.lr * G[k]
    np.testing.assert_allclose(res.losses, losses, rtol=1e-12, atol=0)
    for k in Wc:
        np.testing.assert_allclose(res.weights[k], Wc[k], rtol=1e-12, atol=1e-15)


# ------------------------------------------------------------------ P3 eta = 0 is L_naive
@pytest.mark.parametrize("mlp,norm", COMBOS)
def test_p3_zero_lr_is_naive_loss(mlp, norm):
    """[E2E] eq. (6) at eta = 0 equals eq. (4): every l_t is scored at W_0, and W never moves."""
    model = tiny_model(mlp, norm, L=2, b=4, lr=0.0)
    P = tiny_params(model, seed=7)
    x = tiny_tokens(model, 12, seed=8)
    res = O.run_ttt(model, P, x)
    naive = O.static_losses(model, P, x)
    assert abs(res.mean_loss - naive.mean()) <= 1e-15 * abs(naive.mean()) + 1e-15
    for k in model.fast_keys():
        assert np.array_equal(res.weights[k], P[k])
        assert not res.delta[k].any()


# ------------------------------------------------------------------ P4 chunk gradient is a mean
@pytest.mark.parametrize("mlp,norm", COMBOS)
def test_p4_chunk_gradient_is_mean_of_token_gradients(mlp, norm):
    """[E2E] eq. (5): the chunk step uses (1/b) sum_t grad l_t at the same W."""
    b = 5
    model = tiny_model(mlp, norm, L=2, b=b)
    one = tiny_model(mlp, norm, L=2, b=1)
    P = tiny_params(model, seed=9)
    x = tiny_tokens(model, b, seed=10)
    _, _, G = O.chunk_loss_and_grads(model, P, x[:-1], x[1:])
    for k in model.fast_keys():
        acc = np.zeros_like(P[k])
        for t in range(b):
            _, _, Gt = O.chunk_loss_and_grads(one, P, x[t:t + 1], x[t + 1:t + 2])
            acc += Gt[k]
        np.testing.assert_allclose(G[k], acc / b, rtol=1e-12, atol=1e-17)


# ------------------------------------------------------------------ P5 TTT helps on Markov data
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_p5_markov_ttt_beats_static(seed):
    """[E2E] section 2 (toy figure): on bigram-structured data TTT lowers the test loss
    below the static-weight loss L_naive. Checked on the toy workload in fp64."""
    w = W.preset("toy")
    x = W.token_stream(w, seed)
    P = W.init_weights(w, seed)
    model = O.Model.from_workload(w)
    res = O.run_ttt(model, P, x)
    naive = O.static_losses(model, P, x)
    assert res.mean_loss < naive.mean()


# ------------------------------------------------------------------ P6 closed form E_out = 0
@pytest.mark.parametrize("mlp,norm", COMBOS)
def test_p6_zero_head_gives_log_vocab(mlp, norm):
    """With E_out = 0 every logit is 0: l_t = ln V exactly, the gradient is 0, W stays put."""
    model = tiny_model(mlp, norm, L=2, b=2, lr=0.5)
    P = tiny_params(model, seed=11)
    P["E_out"] = np.zeros_like(P["E_out"])
    x = tiny_tokens(model, 6, seed=12)
    res = O.run_ttt(model, P, x)
    assert np.all(res.losses == math.log(model.vocab))
    assert np.all(res.grad_norm == 0.0)
    for k in model.fast_keys():
        assert np.array_equal(res.weights[k], P[k])


# ------------------------------------------------------------------ P7 W2 = 0 wiring
def test_p7_zero_down_projection_kills_w1_gradient():
    """One GELU block with W2 = 0: dA = dH W2^T = 0, so G_W1 = 0 exactly, while G_W2 != 0."""
    model = tiny_model("gelu", "rms", L=1, b=4)
    P = tiny_params(model, seed=13)
    P["W2.0"] = np.zeros_like(P["W2.0"])
    x = tiny_tokens(model, 4, seed=14)
    _, _, G = O.chunk_loss_and_grads(model, P, x[:-1], x[1:])
    assert not G["W1.0"].any()
    assert np.abs(G["W2.0"]).max() > 1e-3


# ------------------------------------------------------------------ P8 clip identity
@pytest.mark.parametrize("clip", [0.0, 0.05, 1e3])
def test_p8_clipped_step_length(clip):
    """[SGF] clipped step: ||W_i - W_{i-1}||_F over all fast tensors = eta * min(g_i, c)."""
    model = tiny_model("gelu", "rms", L=2, b=2, lr=0.3, clip=clip)
    P = tiny_params(model, seed=15)
    x = tiny_tokens(model, 8, seed=16)
    prev = {k: P[k].copy() for k in model.fast_keys()}
    for i in range(4):
        res = O.run_ttt(model, P, x, n_chunks=i + 1)
        step = math.sqrt(sum(np.sum((res.weights[k] - prev[k]) ** 2) for k in prev))
        g = res.grad_norm[i]
        expect = model.lr * (g if clip <= 0 else min(g, clip))
        assert abs(step - expect) <= 1e-12 * expect
        if 0 < clip < g:
            assert res.scale[i] < 1.0
        prev = {k: res.weights[k].copy() for k in prev}


# ------------------------------------------------------------------ P9 logsumexp special case
def test_p9_logsumexp_matches_library():
    rng = np.random.default_rng(17)
    for z in [rng.normal(0, 3, (7, 50)), rng.normal(0, 1, (3, 1000)) * 1e4,
              np.array([[1e4, -1e4, 0.0], [-1e4, -1e4, -1e4]])]:
        np.testing.assert_allclose(O.logsumexp_rows(z), scipy.special.logsumexp(z, axis=1),
                                   rtol=1e-14, atol=0)


# ------------------------------------------------------------------ P10 second implementation
def torch_ttt(model, P0, tokens):
    """Independent implementation of eq. (5)/(6) + clipped step with torch fp64 autograd."""
    t = lambda a: torch.tensor(a, dtype=torch.float64)
    E_in, E_out = t(P0["E_in"]), t(P0["E_out"])
    frozen = {k: t(v) for k, v in P0.items() if k.startswith(("Wg", "Wu", "Ws", "Wq", "Wk", "Wv", "Wo"))}
    fast = {k: t(P0[k]) for k in model.fast_keys()}
    x = torch.tensor(np.asarray(tokens), dtype=torch.long)
    b = model.chunk
    losses, gnorms = [], []
    # attention: the detached keys/values of every earlier position (the whole history; the
    # window is applied by the position mask alone)
    past = [None] * model.n_blocks
    for i in range((len(tokens) - 1) // b):
        params = {k: v.clone().requires_grad_(True) for k, v in fast.items()}
        ctx, tgt = x[i * b:(i + 1) * b], x[i * b + 1:(i + 1) * b + 1]
        h = E_in[ctx]

        def norm(v):
            if model.norm == "rms":
                return v * torch.rsqrt(v.pow(2).mean(-1, keepdim=True) + model.eps)
            return v

        for l in range(model.n_blocks):
            if model.swa_window > 0:
                na = norm(h)
                q, k, v = na @ frozen[f"Wq.{l}"], na @ frozen[f"Wk.{l}"], na @ frozen[f"Wv.{l}"]
                K = k if past[l] is None else torch.cat([past[l][0], k])
                Vv = v if past[l] is None else torch.cat([past[l][1], v])
                start = i * b - (K.shape[0] - b)  # absolute position of the first key
                pq = torch.arange(i * b, i * b + b)[:, None]
                pk = torch.arange(start, start + K.shape[0])[None, :]
                allowed = (pk <= pq) & (pk > pq - model.swa_window)
                H = model.swa_heads
                split = lambda a: a.reshape(a.shape[0], H, -1).transpose(0, 1)
                o = torch.nn.functional.scaled_dot_product_attention(split(q), split(K), split(Vv),
                                                                     attn_mask=allowed)
                h = h + o.transpose(0, 1).reshape(b, -1) @ frozen[f"Wo.{l}"]
                past[l] = (K.detach(), Vv.detach())
            if model.static_hidden > 0:
                hs = torch.nn.functional.gelu(norm(h) @ frozen[f"Ws1.{l}"], approximate="none")
                h = h + hs @ frozen[f"Ws2.{l}"]
            n = norm(h)
            if model.mlp == "gelu":
                a = torch.nn.functional.gelu(n @ params[f"W1.{l}"], approximate="none")
            else:
                a = torch.nn.functional.silu(n @ frozen[f"Wg.{l}"]) * (n @ frozen[f"Wu.{l}"])
            h = h + a @ params[f"W2.{l}"]
        z = h @ E_out.T
        per_tok = torch.nn.functional.cross_entropy(z, tgt, reduction="none")
        grads = torch.autograd.grad(per_tok.mean(), list(params.values()))
        g = math.sqrt(sum(float((gr * gr).sum()) for gr in grads))
        s = 1.0 if (model.clip <= 0 or g <= model.clip) else model.clip / g
        for (k, _), gr in zip(params.items(), grads):
            fast[k] = fast[k] - model.lr * s * gr
        losses.append(per_tok.detach().numpy())
        gnorms.append(g)
    return np.concatenate(losses), np.array(gnorms), {k: v.numpy() for k, v in fast.items()}


def test_p9b_ce_stats_worked_rows():
    """ce_stats on hand-made rows whose results are known exactly: the argmax is the first
    maximum (ties to the lowest index), the margin is the gap between the two largest values
    (0 at a tie), the loss is lse minus the target's logit, and a one-column row has loss 0
    and an infinite margin."""
    z = np.array([[1.0, 3.0, 2.0, 3.0],
                  [0.5, -1.0, 2.25, 0.0],
                  [-4.0, -4.0, -4.0, -4.0]])
    loss, lse, am, margin = O.ce_stats(z, np.array([2, 2, 3]))
    assert am.tolist() == [1, 2, 0]
    assert margin.tolist() == [0.0, 1.75, 0.0]
    assert lse[0] == pytest.approx(math.log(math.exp(1) + 2 * math.exp(3) + math.exp(2)), rel=1e-15)
    assert lse[1] == pytest.approx(math.log(math.exp(0.5) + math.exp(-1) + math.exp(2.25) + 1.0), rel=1e-15)
    assert lse[2] == pytest.approx(-4.0 + math.log(4.0), rel=1e-15)
    assert loss.tolist() == pytest.approx([lse[0] - 2.0, lse[1] - 2.25, math.log(4.0)], rel=1e-15)
    l1, _, a1, m1 = O.ce_stats(np.array([[7.0], [-2.0]]), np.array([0, 0]))
    assert l1.tolist() == [0.0, 0.0] and a1.tolist() == [0, 0] and np.all(np.isinf(m1))


@pytest.mark.parametrize("mlp,norm", COMBOS)
@pytest.mark.parametrize("clip", [0.0, 0.1])
def test_p10_torch_autograd_second_opinion(mlp, norm, clip):
    model = tiny_model(mlp, norm, L=3, b=3, lr=0.4, clip=clip)
    P = tiny_params(model, seed=18)
    x = tiny_tokens(model, 12, seed=19)
    res = O.run_ttt(model, P, x)
    tl, tg, tw = torch_ttt(model, P, x)
    np.testing.assert_allclose(res.losses, tl, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(res.grad_norm, tg, rtol=1e-12)
    for k in model.fast_keys():
        np.testing.assert_allclose(res.weights[k], tw[k], rtol=1e-12, atol=1e-14)
        # the update itself (the part the stated weight gate cannot see)
        np.testing.assert_allclose(res.delta[k], tw[k] - P[k], rtol=1e-9, atol=1e-15)


@pytest.mark.parametrize("norm", ["none", "rms"])
def test_p10_static_mlp_second_opinion(norm):
    """With a frozen static MLP before each fast one ([E2E] section 3.1): losses, norms and
    updates against torch autograd, which differentiates through the static MLPs itself."""
    model = tiny_model("gelu", norm, L=3, b=3, lr=0.4, clip=0.2, ms=7)
    P = tiny_params(model, seed=21)
    x = tiny_tokens(model, 12, seed=22)
    res = O.run_ttt(model, P, x)
    tl, tg, tw = torch_ttt(model, P, x)
    np.testing.assert_allclose(res.losses, tl, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(res.grad_norm, tg, rtol=1e-12)
    for k in model.fast_keys():
        np.testing.assert_allclose(res.delta[k], tw[k] - P[k], rtol=1e-9, atol=1e-15)


@pytest.mark.parametrize("norm", ["none", "rms"])
def test_p1_finite_differences_through_static_mlps(norm):
    """The lower blocks' gradients pass through the static MLPs of the blocks above."""
    model = tiny_model("gelu", norm, L=2, b=3, ms=5)
    P = tiny_params(model, seed=23)
    x = tiny_tokens(model, 3, seed=24)
    assert fd_check(model, P, x[:-1], x[1:]) < 1e-6


@pytest.mark.parametrize("norm,win,b,ms", [("rms", 5, 3, 0), ("none", 4, 4, 6), ("rms", 20, 3, 5), ("rms", 1, 3, 0),
                                           ("rms", 7, 4, 0), ("none", 11, 3, 4)])
def test_p16_attention_second_opinion(norm, win, b, ms):
    """Sliding-window attention ([E2E] section 3) with its key/value cache across chunks:
    losses, norms and updates against torch autograd over torch's own masked attention
    (window shorter and longer than the stream, equal to the chunk, and 1)."""
    model = tiny_model("gelu", norm, L=3, b=b, lr=0.4, clip=0.3, ms=ms, win=win, heads=2)
    P = tiny_params(model, seed=31)
    x = tiny_tokens(model, 4 * b, seed=32)
    res = O.run_ttt(model, P, x)
    tl, tg, tw = torch_ttt(model, P, x)
    np.testing.assert_allclose(res.losses, tl, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(res.grad_norm, tg, rtol=1e-11)
    for k in model.fast_keys():
        np.testing.assert_allclose(res.delta[k], tw[k] - P[k], rtol=1e-9, atol=1e-15)


@pytest.mark.parametrize("norm", ["none", "rms"])
def test_p1_finite_differences_through_attention(norm):
    """The lower blocks' gradients pass through the attention of the blocks above (within a
    chunk: the chunk's queries, keys and values all depend on the fast weights below)."""
    model = tiny_model("gelu", norm, L=2, b=4, win=3, heads=2)
    P = tiny_params(model, seed=33)
    x = tiny_tokens(model, 4, seed=34)
    assert fd_check(model, P, x[:-1], x[1:]) < 1e-6


def test_p17_zero_output_projection_is_the_plain_model():
    """Wo = 0: the attention adds exact zeros and passes the gradient through unchanged."""
    model = tiny_model("gelu", "rms", L=2, b=3, lr=0.3, clip=0.5, ms=4, win=4, heads=2)
    P = tiny_params(model, seed=35)
    for l in range(model.n_blocks):
        P[f"Wo.{l}"] = np.zeros_like(P[f"Wo.{l}"])
    x = tiny_tokens(model, 9, seed=36)
    a = O.run_ttt(model, P, x)
    plain = tiny_model("gelu", "rms", L=2, b=3, lr=0.3, clip=0.5, ms=4)
    b = O.run_ttt(plain, {k: v for k, v in P.items() if k[:2] not in ("Wq", "Wk", "Wv", "Wo")}, x)
    assert np.array_equal(a.losses, b.losses)
    for k in model.fast_keys():
        assert np.array_equal(a.weights[k], b.weights[k])


def test_p18_window_one_is_a_linear_residual_map():
    """Window 1: each query sees only its own key, so the attention output is n Wv Wo; the
    losses equal those of a model whose block adds norm(h) Wv Wo, computed here directly."""
    model = tiny_model("gelu", "rms", L=1, b=3, lr=0.0, win=1, heads=2)
    P = tiny_params(model, seed=37)
    x = tiny_tokens(model, 6, seed=38)
    res = O.run_ttt(model, P, x)
    h = P["E_in"][x[:-1]]
    n = h / np.sqrt(np.mean(h * h, axis=1) + model.eps)[:, None]
    h = h + n @ P["Wv.0"] @ P["Wo.0"]
    n = h / np.sqrt(np.mean(h * h, axis=1) + model.eps)[:, None]
    h = h + O.gelu(n @ P["W1.0"]) @ P["W2.0"]
    z = h @ P["E_out"].T
    ref = scipy.special.logsumexp(z, axis=1) - z[np.arange(len(z)), x[1:]]
    np.testing.assert_allclose(res.losses, ref, rtol=1e-12)


@pytest.mark.parametrize("win,b,ms", [(5, 3, 0), (2, 4, 3), (40, 3, 0)])
def test_p19_decoding_with_attention_equals_prefill(win, b, ms):
    """[E2E] section 3.2 with the attention of section 3: decoding whole mini-batches token by
    token (each token's key and value joining the cache at once) takes the same steps and
    scores the same losses as prefilling them, to rounding."""
    model = tiny_model("gelu", "rms", L=2, b=b, lr=0.4, clip=0.3, ms=ms, win=win, heads=2)
    P = tiny_params(model, seed=43)
    x = tiny_tokens(model, 4 * b, seed=44)
    pre = O.run_ttt(model, P, x)
    dec = O.decode_ttt(model, P, x)
    np.testing.assert_allclose(dec.losses, pre.losses, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dec.grad_norm, pre.grad_norm, rtol=1e-12)
    for k in model.fast_keys():
        np.testing.assert_allclose(dec.weights[k], pre.weights[k], rtol=1e-12, atol=1e-15)


def test_p20_passage_with_attention_is_a_stream_of_its_own():
    """[SGF] Settlement scores a passage with the attention left as it is; read as a sequence
    of its own, L(q, W) equals the mean loss of prefilling q from an empty cache at eta = 0
    (chunk by chunk, each chunk reading the cache of the ones before)."""
    model = tiny_model("gelu", "rms", L=2, b=3, lr=0.0, win=4, heads=2, ms=3)
    P = tiny_params(model, seed=47)
    q = tiny_tokens(model, 12, seed=48)
    whole = O.passage_loss(model, P, q)
    chunked = O.run_ttt(model, P, q)
    assert abs(whole - float(chunked.losses.mean())) <= 1e-12 * abs(whole)


def test_p21_kept_candidate_with_attention_is_the_stream_step():
    """A kept Settlement candidate, stepped from the stream's cache in front of it, lands on
    the weights the plain chunk loop reaches after the same chunk ([SGF] Settlement with the
    step of [E2E] eq. (5)); the candidate here is scored on its own text, so it is kept."""
    model = tiny_model("gelu", "rms", L=2, b=3, lr=0.2, clip=0.5, win=5, heads=2)
    P = tiny_params(model, seed=49)
    x = tiny_tokens(model, 6, seed=50)
    one = O.run_ttt(model, P, x[:4])
    two = O.run_ttt(model, P, x)
    W1 = {**O.as_f64(P), **one.weights}
    cand = x[3:]
    A, keep, Wn, g, s = O.settle_step(model, W1, cand, cand, kv=one.kv)
    assert keep and A > 0
    for k in model.fast_keys():
        np.testing.assert_allclose(Wn[k], two.weights[k], rtol=1e-12, atol=1e-15)
    # without the stream's cache the candidate's step is another one
    _, _, Wc, _, _ = O.settle_step(model, W1, cand, cand)
    assert max(np.max(np.abs(Wc[k] - two.weights[k])) for k in model.fast_keys()) > 1e-6


def test_pins_catch_a_decode_cache_one_token_behind(monkeypatch):
    """A decoded token that does not see the token just before it (the cache extended one
    token late) breaks the decode = prefill identity."""
    model = tiny_model("gelu", "rms", L=2, b=3, lr=0.4, win=5, heads=2)
    P = tiny_params(model, seed=45)
    x = tiny_tokens(model, 9, seed=46)
    pre = O.run_ttt(model, P, x)
    real_swa = O.swa_forward

    def lagging(model, P, l, n, kv):
        if n.shape[0] == 1 and kv is not None and kv["k"].shape[0] > 0:
            kv = dict(k=kv["k"][:-1], v=kv["v"][:-1])
        return real_swa(model, P, l, n, kv)
    monkeypatch.setattr(O, "swa_forward", lagging)
    dec = O.decode_ttt(model, P, x)
    assert np.max(np.abs(dec.losses - pre.losses)) > 1e-6


def test_pins_catch_a_cache_cut_short_by_index_wrap(monkeypatch):
    """A cache that keeps only the last (window - 1) - n rows while fewer than window - 1
    positions exist (a negative slice start wrapping around) is caught by the torch second
    opinion, which keeps the whole history and masks by position."""
    def wrong(model, kv, c):
        keep = model.swa_window - 1
        return [dict(k=c[l]["att"]["K"][c[l]["att"]["K"].shape[0] - keep:],
                     v=c[l]["att"]["V"][c[l]["att"]["V"].shape[0] - keep:]) for l in range(model.n_blocks)]
    monkeypatch.setattr(O, "next_kv", wrong)
    model = tiny_model("gelu", "rms", L=2, b=4, lr=0.4, win=7, heads=2)
    P = tiny_params(model, seed=41)
    x = tiny_tokens(model, 12, seed=42)
    res = O.run_ttt(model, P, x)
    tl, _, _ = torch_ttt(model, P, x)
    assert np.max(np.abs(res.losses - tl)) > 1e-6


def test_pins_catch_a_window_one_key_too_wide(monkeypatch):
    """A window mask that lets each query see window + 1 keys (an off-by-one) is caught by
    the torch second opinion once the stream is longer than the window."""
    def wrong(nc, b, window):
        pq = nc + np.arange(b)[:, None]
        pk = np.arange(nc + b)[None, :]
        return (pk <= pq) & (pk >= pq - window)
    monkeypatch.setattr(O, "window_mask", wrong)
    model = tiny_model("gelu", "rms", L=2, b=3, lr=0.4, win=4, heads=2)
    P = tiny_params(model, seed=39)
    x = tiny_tokens(model, 12, seed=40)
    res = O.run_ttt(model, P, x)
    tl, _, _ = torch_ttt(model, P, x)
    assert np.max(np.abs(res.losses - tl)) > 1e-6


def test_p15_zero_static_projection_is_the_plain_model():
    """Ws2 = 0: every static MLP adds exactly zero and passes the gradient through
    unchanged, so the run equals the model without static MLPs, bit for bit."""
    model = tiny_model("gelu", "rms", L=3, b=2, lr=0.3, clip=0.5, ms=4)
    P = tiny_params(model, seed=25)
    for l in range(model.n_blocks):
        P[f"Ws2.{l}"] = np.zeros_like(P[f"Ws2.{l}"])
    x = tiny_tokens(model, 8, seed=26)
    a = O.run_ttt(model, P, x)
    plain = tiny_model("gelu", "rms", L=3, b=2, lr=0.3, clip=0.5)
    b = O.run_ttt(plain, {k: v for k, v in P.items() if not k.startswith("Ws")}, x)
    assert np.array_equal(a.losses, b.losses)
    assert np.array_equal(a.grad_norm, b.grad_norm)
    for k in model.fast_keys():
        assert np.array_equal(a.weights[k], b.weights[k])


def test_p10_realistic_shape_one_chunk():
    """Same second opinion at a real width (single-block shape, narrowed vocab, 1 chunk)."""
    w = W.preset("single", vocab=512, chunk=64, n_tokens=64)
    model = O.Model.from_workload(w)
    P = W.init_weights(w, 0)
    x = W.token_stream(w, 0)
    res = O.run_ttt(model, P, x)
    tl, tg, tw = torch_ttt(model, P, x)
    np.testing.assert_allclose(res.losses, tl, rtol=1e-12)
    for k in model.fast_keys():
        np.testing.assert_allclose(res.delta[k], tw[k] - P[k], rtol=1e-9, atol=1e-16)


# ------------------------------------------------------------------ closed-form bigram example
def test_closed_form_two_token_bigram():
    """Hand-derived example: V=2, d=m=1, one GELU block, b=1, no norm.

    E_in = [[1], [1]], E_out = [[1], [-1]], W1 = [[0]], W2 = [[w]], x = (0, 0, 1).
    t=1: h = 1 + gelu(0) w = 1, z = (1, -1), target 0:
         l_1 = ln(1 + e^-2); p_1 = 1/(1+e^2); dh = -2 p_1;
         G_W1 = n * (dh * w * gelu'(0)) = -w p_1 (gelu'(0) = 1/2), G_W2 = gelu(0) dh = 0.
         W1 <- eta * w * p_1.
    t=2: u = eta w p_1, h = 1 + gelu(u) w, z = (h, -h), target 1: l_2 = ln(1 + e^{2h}).
    """
    w2, eta = 0.5, 0.7
    model = O.Model(vocab=2, d_model=1, d_hidden=1, n_blocks=1, mlp="gelu", norm="none",
                    chunk=1, lr=eta, clip=0.0)
    P = {"E_in": np.array([[1.0], [1.0]]), "E_out": np.array([[1.0], [-1.0]]),
         "W1.0": np.array([[0.0]]), "W2.0": np.array([[w2]])}
    res = O.run_ttt(model, P, np.array([0, 0, 1]))
    p1 = 1.0 / (1.0 + math.e ** 2)
    l1 = math.log1p(math.exp(-2.0))
    u = eta * w2 * p1
    gelu_u = 0.5 * u * (1.0 + math.erf(u / math.sqrt(2.0)))
    h = 1.0 + gelu_u * w2
    l2 = math.log1p(math.exp(2.0 * h))
    assert res.losses[0] == pytest.approx(l1, rel=1e-15)
    assert res.losses[1] == pytest.approx(l2, rel=1e-14)
    assert res.grad_norm[0] == pytest.approx(w2 * p1, rel=1e-15)
    g2 = res.grad_norm[1]
    assert g2 > 0
    # W2 got no gradient in step 1 (a = gelu(0) = 0)
    _, _, G = O.chunk_loss_and_grads(model, P, np.array([0]), np.array([0]))
    assert G["W2.0"][0, 0] == 0.0
    assert G["W1.0"][0, 0] == pytest.approx(-w2 * p1, rel=1e-15)


# ------------------------------------------------------------------ the pins catch planted mistakes
def test_pins_catch_wrong_gelu_derivative(monkeypatch):
    """Planting a dropped term in the oracle's GELU' (on the CPU) must fail the FD pin."""
    monkeypatch.setattr(O, "gelu_prime", lambda u: 0.5 * (1.0 + scipy.special.erf(u / O.SQRT2)))
    model = tiny_model("gelu", "none", L=1, b=3)
    P = tiny_params(model, seed=3)
    x = tiny_tokens(model, 3, seed=4)
    assert fd_check(model, P, x[:-1], x[1:]) > 1e-3


def test_pins_catch_wrong_silu_derivative(monkeypatch):
    monkeypatch.setattr(O, "silu_prime", lambda g: O.sigmoid(g))
    model = tiny_model("swiglu_w2", "rms", L=2, b=3)
    P = tiny_params(model, seed=3)
    x = tiny_tokens(model, 3, seed=4)
    assert fd_check(model, P, x[:-1], x[1:]) > 1e-3


def test_pins_catch_static_mlp_backward_without_norm_jacobian(monkeypatch):
    """Planting a dropped pre-norm Jacobian in the static MLP's backward fails the FD pin."""
    def wrong(model, P, l, c, dh):
        da = dh @ P[f"Ws2.{l}"].T
        return dh + (da * O.gelu_prime(c["us"])) @ P[f"Ws1.{l}"].T
    monkeypatch.setattr(O, "static_mlp_backward", wrong)
    model = tiny_model("gelu", "rms", L=2, b=3, ms=5)
    P = tiny_params(model, seed=23)
    x = tiny_tokens(model, 3, seed=24)
    assert fd_check(model, P, x[:-1], x[1:]) > 1e-3


def test_pins_catch_unclipped_step(monkeypatch):
    monkeypatch.setattr(O, "clip_scale", lambda g, c: 1.0)
    model = tiny_model("gelu", "rms", L=2, b=2, lr=0.3, clip=0.05)
    P = tiny_params(model, seed=15)
    x = tiny_tokens(model, 4, seed=16)
    res = O.run_ttt(model, P, x, n_chunks=1)
    step = math.sqrt(sum(np.sum(res.delta[k] ** 2) for k in model.fast_keys()))
    assert abs(step - model.lr * min(res.grad_norm[0], model.clip)) > 1e-3


def test_pins_catch_off_by_one_target():
    """Scoring x_{t-1} instead of x_t (an index slip) breaks the closed form."""
    model = O.Model(vocab=2, d_model=1, d_hidden=1, n_blocks=1, chunk=1, lr=0.0)
    P = {"E_in": np.array([[1.0], [1.0]]), "E_out": np.array([[1.0], [-1.0]]),
         "W1.0": np.array([[0.0]]), "W2.0": np.array([[0.5]])}
    good, _, _ = O.token_losses(model, P, np.array([0]), np.array([1]))
    slip, _, _ = O.token_losses(model, P, np.array([0]), np.array([0]))
    assert good[0] == pytest.approx(math.log1p(math.exp(2.0)), rel=1e-15)
    assert abs(slip[0] - good[0]) > 1.0


# ------------------------------------------------------------------ P11/P12 decoding
@pytest.mark.parametrize("mlp,norm", COMBOS)
@pytest.mark.parametrize("clip", [0.0, 0.05])
def test_p11_decoding_full_chunks_equals_prefill(mlp, norm, clip):
    """[E2E] section 3.2: prefilled tokens are consumed in T/b mini-batches, and decoded tokens
    take a step each time they fill one, so decoding a stream of whole chunks token by token
    scores every token at the same weights and ends at the same weights as the chunked loop."""
    model = tiny_model(mlp, norm, L=2, b=3, lr=0.3, clip=clip)
    P = tiny_params(model, seed=21)
    x = tiny_tokens(model, 12, seed=22)
    pre = O.run_ttt(model, P, x)
    dec = O.decode_ttt(model, P, x)
    np.testing.assert_allclose(dec.losses, pre.losses, rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(dec.argmax, pre.argmax)
    np.testing.assert_allclose(dec.grad_norm, pre.grad_norm, rtol=1e-12)
    np.testing.assert_allclose(dec.scale, pre.scale, rtol=1e-12)
    for k in model.fast_keys():
        np.testing.assert_allclose(dec.weights[k], pre.weights[k], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("mlp,norm", [("gelu", "rms"), ("swiglu_w2", "none")])
def test_p12_partial_chunk_takes_no_step(mlp, norm):
    """Decoded tokens that do not fill a mini-batch are scored at the last chunk's weights and
    leave the weights alone (section 3.2: the step waits for a full mini-batch)."""
    model = tiny_model(mlp, norm, L=2, b=4, lr=0.3, clip=0.0)
    P = tiny_params(model, seed=23)
    x = tiny_tokens(model, 11, seed=24)  # two full chunks, then 3 decoded tokens
    dec = O.decode_ttt(model, P, x)
    pre = O.run_ttt(model, P, x[:9])
    assert len(dec.grad_norm) == 2
    for k in model.fast_keys():
        np.testing.assert_allclose(dec.weights[k], pre.weights[k], rtol=1e-12, atol=1e-14)
    Pw = dict(O.as_f64(P))
    Pw.update(pre.weights)
    tail, tail_am, _ = O.token_losses(model, Pw, x[8:11], x[9:12])
    np.testing.assert_allclose(dec.losses[8:], tail, rtol=1e-12)
    np.testing.assert_array_equal(dec.argmax[8:], tail_am)


def test_pins_catch_decode_stepping_one_token_late():
    """A decode that scores the first token after a full mini-batch before stepping (the step one
    token late) differs from the chunked loop, so P11 would catch it."""
    model = tiny_model("gelu", "rms", L=2, b=3, lr=0.3, clip=0.0)
    P = O.as_f64(tiny_params(model, seed=25))
    x = tiny_tokens(model, 6, seed=26)
    pre = O.run_ttt(model, P, x)
    keys = model.fast_keys()
    D = {k: np.zeros_like(P[k]) for k in keys}
    late = []
    for t in range(1, 7):
        Pt = dict(P)
        for k in keys:
            Pt[k] = P[k] + D[k]
        l, _, _ = O.token_losses(model, Pt, x[t - 1:t], x[t:t + 1])
        late.append(l[0])
        if t == 4:  # should have stepped after t == 3
            _, _, G = O.chunk_loss_and_grads(model, Pt, x[0:3], x[1:4])
            for k in keys:
                D[k] = D[k] - model.lr * G[k]
    assert abs(late[3] - pre.losses[3]) > 1e-6


# ------------------------------------------------------------------ P13/P14 Settlement
@pytest.mark.parametrize("mlp,norm", COMBOS)
def test_p13_settlement_gain_is_first_order_descent(mlp, norm):
    """With the candidate's own text as the passage and no clipping, W + delta = W - eta G with
    G = grad L(q, W), so A(delta; W, q) = L(q, W) - L(q, W - eta G) = eta ||G||^2 + O(eta^2):
    A / eta tends to ||G||^2 (calculus, [SGF] Settlement's A), and the step is kept."""
    model = tiny_model(mlp, norm, L=2, b=4, lr=1.0, clip=0.0)
    P = O.as_f64(tiny_params(model, seed=31))
    cand = tiny_tokens(model, 4, seed=32)
    _, _, G = O.chunk_loss_and_grads(model, P, cand[:-1], cand[1:])
    g2 = sum(float(np.sum(G[k] ** 2)) for k in model.fast_keys())
    errs = []
    for eta in (1e-3, 5e-4):
        m = O.Model(**{**model.__dict__, "lr": eta})
        A, keep, _, _, _ = O.settle_step(m, P, cand, cand)
        assert keep
        errs.append(abs(A / eta - g2) / g2)
    assert errs[1] < errs[0] and errs[1] < 5e-3  # the O(eta) remainder halves with eta


def test_p14_settlement_keeps_or_restores_exactly():
    """A >= 0 keeps exactly the prefill step; A < 0 leaves W untouched (the rule's two branches)."""
    model = tiny_model("gelu", "rms", L=2, b=4, lr=0.5, clip=0.0)
    P = O.as_f64(tiny_params(model, seed=33))
    cand = tiny_tokens(model, 4, seed=34)
    kept, rejected = 0, 0
    for seed in range(35, 47):
        q = tiny_tokens(model, 8, seed=seed)
        A, keep, Wn, g, s = O.settle_step(model, P, cand, q)
        direct = O.passage_loss(model, P, q) - O.passage_loss(model, {**P, **Wn}, q)
        if keep:
            kept += 1
            step = O.run_ttt(model, P, cand)
            for k in model.fast_keys():
                np.testing.assert_allclose(Wn[k], step.weights[k], rtol=1e-12, atol=1e-14)
            assert direct == pytest.approx(A, abs=1e-12)
        else:
            rejected += 1
            for k in model.fast_keys():
                assert np.array_equal(Wn[k], P[k])
            assert A < 0 and direct == 0.0
    assert kept > 0 and rejected > 0


def test_pins_catch_settlement_sign_slip():
    """A written as L(q, W + delta) - L(q, W) fails P13 (the own-text step would be rejected)."""
    model = tiny_model("gelu", "none", L=1, b=4, lr=1e-3, clip=0.0)
    P = O.as_f64(tiny_params(model, seed=48))
    cand = tiny_tokens(model, 4, seed=49)
    A, keep, _, _, _ = O.settle_step(model, P, cand, cand)
    assert keep and A > 0 and not (-A >= 0.0)


# ------------------------------------------------------------------ non-finite chunk is skipped
def test_nonfinite_gradient_skips_update():
    model = tiny_model("gelu", "none", L=1, b=2, lr=0.3)
    P = tiny_params(model, seed=20)
    P["E_in"] = P["E_in"].copy()
    P["E_in"][3, 0] = np.nan
    x = np.array([0, 3, 1, 2, 4])  # chunk 1 reads E_in[3] (NaN), chunk 2 does not
    res = O.run_ttt(model, P, x)
    assert res.skipped.tolist() == [True, False]
    assert np.isfinite(res.delta["W1.0"]).all()
    assert res.delta["W1.0"].any()


# ------------------------------------------------------------------ input generator sanity
def test_workload_streams_are_seeded_and_in_range():
    w = W.preset("single", n_tokens=4096)
    a, b = W.token_stream(w, 3), W.token_stream(w, 3)
    assert np.array_equal(a, b) and a[0] == W.BOS
    assert a.min() >= 0 and a.max() < w.vocab
    c = W.token_stream(w, 4)
    assert not np.array_equal(a, c)
    P = W.init_weights(w.replace(vocab=512), 0)
    for k, v in P.items():
        assert np.array_equal(W.round_to_bf16(v), v)  # bf16-exact
        assert 0.018 < v.std() < 0.022

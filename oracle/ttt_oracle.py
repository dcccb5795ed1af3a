"""fp64 CPU oracle of the chunk-wise test-time-training (TTT) inner loop.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or link
this module: only the tests, the smoke check and the CPU-baseline leg of the
benchmark use it, to check the HIP library against plain definitions.

It is a plain, slow, readable restatement of the method in float64 numpy, with
hand-derived backpropagation, written from these pages:

  [E2E] "[논문리뷰] End-to-End Test-Time Training for Long Context"
        (review on kimjy99.github.io)
        - Method: prefill conditions on x_0..x_T, x_0 is BOS.
        - section 1, eq. (1): l_t(W) = CE(f(x_{t-1}; W), x_t).
        - section 1, eq. (2): per-token update W_t = W_{t-1} - eta * grad l_t(W_{t-1}).
        - section 2, eq. (3)/(4): test loss L(W_0; X) and the static L_naive(W_0; X).
        - section 3, eq. (5): mini-batch update
              W_i = W_{i-1} - eta * (1/b) * sum_{t in chunk i} grad l_t(W_{i-1}).
        - section 3, eq. (6): L(W_0; X) = (1/T) sum_i sum_{t in chunk i} l_t(W_{i-1}).
        - section 3: sliding-window attention of a fixed window k, with k >= b so that
          the tokens of a mini-batch see each other before the step.
        - section 3.1: only the MLP layers are updated; embedding, normalisation and
          attention layers stay frozen; "two MLP layers per block": a static MLP is added
          to each TTT'd block to hold pre-trained knowledge, and only the other is updated.
  [IPT] "[논문리뷰] In-Place Test-Time Training" (blog.secrett2633.cloud)
        - section 1 (Key Terms): the MLP block's final projection is the fast
          weight; the sequence is split into chunks updated one after another.
  [SGF] "Self-Generated Feedback Destabilizes Test-Time Training" (summary on
        onedev.kr), "how it works": one *clipped* gradient step per 1024-token
        chunk on the last three layers' feed-forward modules.

Readings where the pages leave a step open (each is also listed in the design
notes of the repository):
  * f = embedding -> L residual MLP blocks -> LM head; no biases, no final norm,
    untied input embedding E_in and output head E_out (both frozen).
  * "rms" blocks are pre-norm: n = h * (mean_j h_j^2 + eps)^(-1/2), no gain.
  * the static MLP (when present) is a frozen GELU MLP with its own pre-norm and residual,
    placed before the fast MLP of the same block: h <- h + GELU(norm(h) Ws1) Ws2, then
    h <- h + MLP_fast(norm(h)).
  * sliding-window attention (when present) comes first in each block, with its own
    pre-norm and residual: H heads of size d/H, q = n Wq, k = n Wk, v = n Wv, softmax of
    q.k / sqrt(d/H) over the keys of the last `window` positions up to and including the
    query's own, o = sum p v, output o Wo; no positional encoding (the causal window is the
    only order the pages give). Row t of the stream (conditioning token x_t) is position t.
    Each position's key and value are computed once, when its chunk is processed, at that
    chunk's weights W_{i-1}; later chunks read them as constants (no gradient flows into an
    earlier chunk's keys or values).
  * GELU is the exact erf form; its derivative is Phi(u) + u * phi(u).
  * SwiGLU block (In-Place shape): a = SiLU(n Wg) * (n Wu); Wg, Wu frozen, W2 fast.
  * clipping: global L2 norm g over all fast tensors of the chunk-mean gradient,
    scale s = min(1, c/g); c <= 0 disables it; g = 0 gives s = 1.
  * a chunk whose g is not finite takes no step (the update is skipped).
  * argmax ties resolve to the lowest index.

Arrays: E_in, E_out [V, d]; W1, Wg, Wu [d, m]; W2 [m, d]; Ws1 [d, m_s]; Ws2 [m_s, d];
Wq, Wk, Wv, Wo [d, d]; all row-major, rows of activations are tokens.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Tuple

import numpy as np
from scipy.special import erf

SQRT2 = math.sqrt(2.0)
INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


@dataclasses.dataclass(frozen=True)
class Model:
    vocab: int
    d_model: int
    d_hidden: int
    n_blocks: int
    mlp: str = "gelu"        # "gelu" | "swiglu_w2"
    norm: str = "none"       # "none" | "rms"
    eps: float = 1e-6
    chunk: int = 1           # b
    lr: float = 0.0          # eta
    clip: float = 0.0        # c; <= 0 disables clipping
    static_hidden: int = 0   # m_s of the frozen static MLP in every block (0: none)
    swa_window: int = 0      # keys per query of the frozen sliding-window attention (0: none)
    swa_heads: int = 0       # its heads (head size d / heads)

    @classmethod
    def from_workload(cls, w, **kw) -> "Model":
        base = dict(vocab=w.vocab, d_model=w.d_model, d_hidden=w.d_hidden,
                    n_blocks=w.n_blocks, mlp=w.mlp, norm=w.norm, eps=w.eps,
                    chunk=w.chunk, lr=w.lr, clip=w.clip,
                    static_hidden=getattr(w, "static_hidden", 0),
                    swa_window=getattr(w, "swa_window", 0), swa_heads=getattr(w, "swa_heads", 0))
        base.update(kw)
        return cls(**base)

    def fast_names(self) -> List[str]:
        # [E2E] section 3.1 updates the whole MLP; [IPT] section 1 only its final projection.
        return ["W1", "W2"] if self.mlp == "gelu" else ["W2"]

    def fast_keys(self) -> List[str]:
        return [f"{n}.{l}" for l in range(self.n_blocks) for n in self.fast_names()]


def as_f64(weights: Dict[str, np.ndarray]) -> Dict[str, np.ndarray]:
    return {k: np.asarray(v, dtype=np.float64) for k, v in weights.items()}


# ------------------------------------------------------------- elementwise maps
def gelu(u):
    """Exact GELU: u * Phi(u), Phi the standard normal CDF."""
    return 0.5 * u * (1.0 + erf(u / SQRT2))


def gelu_prime(u):
    """d/du [u Phi(u)] = Phi(u) + u phi(u)."""
    return 0.5 * (1.0 + erf(u / SQRT2)) + u * INV_SQRT_2PI * np.exp(-0.5 * u * u)


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def silu(x):
    return x * sigmoid(x)


def silu_prime(x):
    s = sigmoid(x)
    return s * (1.0 + x * (1.0 - s))


def logsumexp_rows(z: np.ndarray) -> np.ndarray:
    """log sum_v exp(z[t, v]) per row, shifted by the row max for stability."""
    m = z.max(axis=1)
    return m + np.log(np.exp(z - m[:, None]).sum(axis=1))


# ------------------------------------------------------------- model f(x; W)
def pre_norm(model: Model, h: np.ndarray):
    """The block's pre-norm: (n, r) with n = h r, r = (mean_j h_j^2 + eps)^(-1/2) for "rms";
    (h, None) for "none"."""
    if model.norm == "rms":
        r = 1.0 / np.sqrt(np.mean(h * h, axis=1) + model.eps)
        return h * r[:, None], r
    return h, None


def pre_norm_backward(model: Model, n: np.ndarray, r, dn: np.ndarray) -> np.ndarray:
    """Gradient at h from the gradient dn at n = norm(h):
    rms: r (dn - n mean_j(dn_j n_j)); none: dn."""
    if model.norm == "rms":
        return r[:, None] * (dn - n * np.mean(dn * n, axis=1)[:, None])
    return dn


def static_mlp_backward(model: Model, P, l: int, c, dh: np.ndarray) -> np.ndarray:
    """Gradient at the static MLP's input h from the gradient dh at its output
    h + GELU(n Ws1) Ws2 (frozen weights: no weight gradient)."""
    da = dh @ P[f"Ws2.{l}"].T
    du = da * gelu_prime(c["us"])
    dn = du @ P[f"Ws1.{l}"].T
    return dh + pre_norm_backward(model, c["ns"], c["rs"], dn)


def window_mask(nc: int, b: int, window: int) -> np.ndarray:
    """[b, nc + b] boolean: query i (position nc + i) sees key j (position j) when
    pos_i - window < j <= pos_i, i.e. the last `window` positions up to its own."""
    pq = nc + np.arange(b)[:, None]
    pk = np.arange(nc + b)[None, :]
    return (pk <= pq) & (pk > pq - window)


def swa_forward(model: Model, P, l: int, n: np.ndarray, kv):
    """Sliding-window attention of block l over the chunk's rows (normed input n [b, d]).

    kv: the keys and values of the positions before the chunk (dict k, v [n_c, d], n_c <
    window; None for none). Query i sits at position n_c + i, key j of [cached; chunk] at j;
    query i sees keys j with pos_i - window < j <= pos_i. Returns the output [b, d] and what
    the backward needs (including the chunk's own keys and values, for the next chunk)."""
    b, d = n.shape
    H = model.swa_heads
    dh = d // H
    q = n @ P[f"Wq.{l}"]
    k = n @ P[f"Wk.{l}"]
    v = n @ P[f"Wv.{l}"]
    kc = kv["k"] if kv is not None else np.zeros((0, d))
    vc = kv["v"] if kv is not None else np.zeros((0, d))
    K = np.vstack([kc, k])
    V = np.vstack([vc, v])
    nc = kc.shape[0]
    mask = window_mask(nc, b, model.swa_window)
    o = np.zeros((b, d))
    probs = []
    for hd in range(H):
        cs = slice(hd * dh, (hd + 1) * dh)
        sc = (q[:, cs] @ K[:, cs].T) / math.sqrt(dh)
        sc = np.where(mask, sc, -np.inf)
        mx = sc.max(axis=1, keepdims=True)
        e = np.exp(sc - mx)
        p = e / e.sum(axis=1, keepdims=True)
        o[:, cs] = p @ V[:, cs]
        probs.append(p)
    return o @ P[f"Wo.{l}"], dict(q=q, k=k, v=v, K=K, V=V, probs=probs, o=o, nc=nc)


def swa_backward(model: Model, P, l: int, c, dh: np.ndarray) -> np.ndarray:
    """Gradient at the attention's normed input from the gradient dh at its output (frozen
    weights; the cached keys and values of earlier chunks are constants)."""
    a = c["att"]
    b, d = dh.shape
    H = model.swa_heads
    dhd = d // H
    do = dh @ P[f"Wo.{l}"].T
    dq = np.zeros((b, d))
    dK = np.zeros_like(a["K"])
    dV = np.zeros_like(a["V"])
    for hd in range(H):
        cs = slice(hd * dhd, (hd + 1) * dhd)
        p = a["probs"][hd]
        dV[:, cs] = p.T @ do[:, cs]
        dp = do[:, cs] @ a["V"][:, cs].T
        ds = p * (dp - np.sum(dp * p, axis=1, keepdims=True))
        dq[:, cs] = ds @ a["K"][:, cs] / math.sqrt(dhd)
        dK[:, cs] = ds.T @ a["q"][:, cs] / math.sqrt(dhd)
    nc = a["nc"]
    dk, dv = dK[nc:], dV[nc:]
    return dq @ P[f"Wq.{l}"].T + dk @ P[f"Wk.{l}"].T + dv @ P[f"Wv.{l}"].T


def next_kv(model: Model, kv, c):
    """The cache after a chunk: the last window - 1 positions of [cached; chunk]."""
    keep = model.swa_window - 1
    out = []
    for l in range(model.n_blocks):
        a = c[l]["att"]
        start = max(0, a["K"].shape[0] - keep)  # fewer rows than that so far: all of them
        out.append(dict(k=a["K"][start:], v=a["V"][start:]))
    return out


def forward(model: Model, P: Dict[str, np.ndarray], x_prev: np.ndarray, kv=None):
    """Hidden state h^L for each conditioning token x_{t-1}, plus a cache for backprop.

    [E2E] section 1: f reads only x_{t-1} in the MLP-only model. The stack is
    h^0 = E_in[x_{t-1}]; h^l = h^{l-1} + MLP_l(norm(h^{l-1})), with the frozen static MLP
    of the block first when the model has one ([E2E] section 3.1), and the frozen
    sliding-window attention before both when the model has one ([E2E] section 3; kv holds
    each block's keys and values of the positions before these rows).
    """
    h = P["E_in"][x_prev]
    cache = []
    for l in range(model.n_blocks):
        c = {}
        if model.swa_window > 0:
            na, ra = pre_norm(model, h)
            out, att = swa_forward(model, P, l, na, kv[l] if kv is not None else None)
            h = h + out
            c.update(na=na, ra=ra, att=att)
        if model.static_hidden > 0:
            ns, rs = pre_norm(model, h)
            us = ns @ P[f"Ws1.{l}"]
            h = h + gelu(us) @ P[f"Ws2.{l}"]
            c.update(ns=ns, rs=rs, us=us)
        h_in = h
        n, r = pre_norm(model, h_in)
        if model.mlp == "gelu":
            u = n @ P[f"W1.{l}"]
            a = gelu(u)
            c.update(n=n, r=r, u=u, a=a)
        else:
            g = n @ P[f"Wg.{l}"]
            v = n @ P[f"Wu.{l}"]
            a = silu(g) * v
            c.update(n=n, r=r, g=g, v=v, a=a)
        h = h_in + a @ P[f"W2.{l}"]
        cache.append(c)
    return h, cache


def logits(model: Model, P, x_prev, kv=None):
    h, cache = forward(model, P, x_prev, kv)
    return h @ P["E_out"].T, h, cache


def ce_stats(z: np.ndarray, x_tgt: np.ndarray):
    """Per row: loss = logsumexp(z_t) - z_t[x_t], lse, argmax (first maximum), top-2 gap."""
    lse = logsumexp_rows(z)
    rows = np.arange(z.shape[0])
    loss = lse - z[rows, x_tgt]
    am = np.argmax(z, axis=1)  # numpy returns the first maximum
    if z.shape[1] > 1:
        part = np.partition(z, -2, axis=1)
        margin = part[:, -1] - part[:, -2]
    else:
        margin = np.full(z.shape[0], np.inf)
    return loss, lse, am.astype(np.int64), margin


def token_losses(model: Model, P, x_prev, x_tgt, kv=None):
    """[E2E] eq. (1): l_t = CE(f(x_{t-1}; W), x_t) = logsumexp(z_t) - z_t[x_t].

    Also returns argmax_t (lowest index on ties) and the top-2 logit margin.
    """
    z, _, _ = logits(model, P, x_prev, kv)
    loss, _, am, margin = ce_stats(z, x_tgt)
    return loss, am, margin


def chunk_loss_and_grads(model: Model, P, x_prev, x_tgt, logit_probe=None, kv=None):
    """Mean chunk loss (1/b) sum_t l_t(W) and its gradient w.r.t. every fast tensor.

    This is the quantity differentiated in [E2E] eq. (5). Backprop by hand:
      dz = (softmax(z) - onehot(x_t)) / b,  dh = dz E_out
      per block, top to bottom:
        G_W2 = a^T dh ;  da = dh W2^T
        gelu:   du = da * gelu'(u) ; G_W1 = n^T du ; dn = du W1^T
        swiglu: dg = da * v * silu'(g) ; dv = da * silu(g) ; dn = dg Wg^T + dv Wu^T
        rms:    dh <- dh + r * (dn - n * mean_j(dn_j n_j))
        none:   dh <- dh + dn
        static MLP below the fast one: dh <- its input gradient (static_mlp_backward)
        attention below both: dh <- dh + norm'(swa_backward(dh))
      (the embedding is frozen, so the lowest block stops after its weight grads)
    With attention, kv holds the earlier positions' keys and values, and the returned info
    carries the cache after this chunk ("kv").
    """
    b = x_prev.shape[0]
    z, h, cache = logits(model, P, x_prev, kv)
    if logit_probe is not None:
        logit_probe(z, h)
    losses, lse, am, margin = ce_stats(z, x_tgt)
    rows = np.arange(b)
    p = np.exp(z - lse[:, None])
    dz = p
    dz[rows, x_tgt] -= 1.0
    dz /= b
    dh = dz @ P["E_out"]
    grads = {}
    for l in reversed(range(model.n_blocks)):
        c = cache[l]
        W2 = P[f"W2.{l}"]
        grads[f"W2.{l}"] = c["a"].T @ dh
        if model.mlp == "gelu":
            da = dh @ W2.T
            du = da * gelu_prime(c["u"])
            grads[f"W1.{l}"] = c["n"].T @ du
            if l == 0:
                break
            dn = du @ P[f"W1.{l}"].T
        else:
            if l == 0:
                break
            da = dh @ W2.T
            dg = da * c["v"] * silu_prime(c["g"])
            dv = da * silu(c["g"])
            dn = dg @ P[f"Wg.{l}"].T + dv @ P[f"Wu.{l}"].T
        dh = dh + pre_norm_backward(model, c["n"], c["r"], dn)
        if model.static_hidden > 0:
            dh = static_mlp_backward(model, P, l, c, dh)
        if model.swa_window > 0:
            dh = dh + pre_norm_backward(model, c["na"], c["ra"], swa_backward(model, P, l, c, dh))
    info = dict(losses=losses, argmax=am, margin=margin)
    if model.swa_window > 0:
        info["kv"] = next_kv(model, kv, cache)
    return float(losses.mean()), info, grads


def clip_scale(g: float, c: float) -> float:
    """[SGF] "one clipped gradient step": s = min(1, c/g); c <= 0 means no clipping."""
    if c <= 0.0 or g <= c:
        return 1.0
    return c / g


# ------------------------------------------------------------- the inner loop
@dataclasses.dataclass
class TTTResult:
    losses: np.ndarray          # l_t(W_{i-1}) for t = 1..T  ([E2E] eq. 6 summands)
    argmax: np.ndarray          # argmax of the logits that scored l_t
    margin: np.ndarray          # top-2 logit gap of those logits
    grad_norm: np.ndarray       # g_i per chunk
    scale: np.ndarray           # s_i per chunk
    skipped: np.ndarray         # chunk took no step (non-finite g)
    delta: Dict[str, np.ndarray]   # D = W_{T/b} - W_0 per fast tensor
    weights: Dict[str, np.ndarray]  # W_{T/b} = W_0 + D
    kv: Optional[list] = None   # attention: the keys and values the run leaves in the cache

    @property
    def mean_loss(self) -> float:
        return float(self.losses.mean())


def run_ttt(model: Model, P0: Dict[str, np.ndarray], tokens: np.ndarray,
            n_chunks: Optional[int] = None, logit_probe=None) -> TTTResult:
    """Sequential chunk loop of [E2E] eq. (5)/(6) with the clipped step of [SGF].

    tokens = x_0..x_T with T a multiple of b. Chunk i scores and differentiates
    tokens t = (i-1)b+1 .. ib at W_{i-1} (the weights before its own step), then
    steps W_i = W_{i-1} - eta * s_i * G_i. The fast state is kept as W_0 + D so
    that the accumulated update D is exact. logit_probe(i, z, h), when given, sees chunk
    i's logits z and the hidden rows h that produced them (for checks that need values the
    result does not keep).
    """
    P0 = as_f64(P0)
    tokens = np.asarray(tokens, dtype=np.int64)
    b = model.chunk
    T = tokens.shape[0] - 1
    if T % b != 0:
        raise ValueError("T must be a multiple of the chunk size")
    nc = T // b if n_chunks is None else n_chunks
    keys = model.fast_keys()
    D = {k: np.zeros_like(P0[k]) for k in keys}
    losses, argm, marg = [], [], []
    gn, sc, sk = [], [], []
    kv = None  # attention: keys and values of the positions before the chunk
    for i in range(nc):
        P = dict(P0)
        for k in keys:
            P[k] = P0[k] + D[k]
        x_prev = tokens[i * b: i * b + b]
        x_tgt = tokens[i * b + 1: i * b + b + 1]
        _, st, G = chunk_loss_and_grads(model, P, x_prev, x_tgt, logit_probe=(
            None if logit_probe is None else (lambda z, h, i=i: logit_probe(i, z, h))), kv=kv)
        kv = st.get("kv")
        losses.append(st["losses"])
        argm.append(st["argmax"])
        marg.append(st["margin"])
        g = math.sqrt(sum(float(np.sum(G[k] * G[k])) for k in keys))
        if not math.isfinite(g):
            gn.append(g)
            sc.append(0.0)
            sk.append(True)
            continue
        s = clip_scale(g, model.clip)
        for k in keys:
            D[k] = D[k] - model.lr * s * G[k]
        gn.append(g)
        sc.append(s)
        sk.append(False)
    Wf = {k: P0[k] + D[k] for k in keys}
    return TTTResult(np.concatenate(losses) if losses else np.zeros(0),
                     np.concatenate(argm) if argm else np.zeros(0, np.int64),
                     np.concatenate(marg) if marg else np.zeros(0),
                     np.asarray(gn), np.asarray(sc), np.asarray(sk, dtype=bool),
                     D, Wf, kv)


def decode_ttt(model: Model, P0: Dict[str, np.ndarray], tokens: np.ndarray, logit_probe=None) -> TTTResult:
    """Token-by-token decoding with test-time training, [E2E] Method and section 3.2.

    tokens = x_0..x_T (any T >= 0). Decoding predicts the next token's distribution from
    the last token at the current weights (Method: p^_{t+1} = f(x_t; W)), and takes a
    gradient step only when the decoded tokens fill a mini-batch of b; decoding then goes on
    with the updated weights (section 3.2). So token t is scored at the weights left by the
    last completed chunk before it, and a trailing partial chunk takes no step. The step is
    the clipped mini-batch step of [E2E] eq. (5) / [SGF]. logit_probe(t - 1, z, h), when
    given, sees the logits row that scored token t and the hidden row that produced it.

    With attention, each decoded token's key and value are computed at the weights current
    when it is decoded and join the cache at once; a filled mini-batch's step starts from the
    cache as it stood before the mini-batch (its own keys come from its own rows, computed at
    the same weights).
    """
    P0 = as_f64(P0)
    tokens = np.asarray(tokens, dtype=np.int64)
    b = model.chunk
    T = tokens.shape[0] - 1
    keys = model.fast_keys()
    D = {k: np.zeros_like(P0[k]) for k in keys}
    losses, argm, marg = [], [], []
    gn, sc, sk = [], [], []
    start = 0  # the pending mini-batch starts with the pair (x_start, x_start+1)
    att = model.swa_window > 0
    kv = None        # attention: keys and values of the positions decoded so far
    kv_start = None  # and as they stood before the pending mini-batch
    for t in range(1, T + 1):
        P = dict(P0)
        for k in keys:
            P[k] = P0[k] + D[k]
        z, hL, cache = logits(model, P, tokens[t - 1:t], kv)
        if att:
            kv = next_kv(model, kv, cache)
        if logit_probe is not None:
            logit_probe(t - 1, z[0], hL[0])
        l, _, am, mg = ce_stats(z, tokens[t:t + 1])
        losses.append(l[0])
        argm.append(am[0])
        marg.append(mg[0])
        if t - start == b:
            # the decoded tokens fill a mini-batch: one clipped step on it, at the weights
            # that scored it
            _, _, G = chunk_loss_and_grads(model, P, tokens[start:t], tokens[start + 1:t + 1], kv=kv_start)
            g = math.sqrt(sum(float(np.sum(G[k] * G[k])) for k in keys))
            if math.isfinite(g):
                s = clip_scale(g, model.clip)
                for k in keys:
                    D[k] = D[k] - model.lr * s * G[k]
                gn.append(g)
                sc.append(s)
                sk.append(False)
            else:
                gn.append(g)
                sc.append(0.0)
                sk.append(True)
            start = t
            kv_start = kv
    Wf = {k: P0[k] + D[k] for k in keys}
    return TTTResult(np.asarray(losses, dtype=np.float64), np.asarray(argm, dtype=np.int64),
                     np.asarray(marg, dtype=np.float64), np.asarray(gn), np.asarray(sc),
                     np.asarray(sk, dtype=bool), D, Wf, kv)


def passage_loss(model: Model, P: Dict[str, np.ndarray], q: np.ndarray) -> float:
    """L(q, W): the mean next-token loss of a passage q_0..q_n at fixed weights (no step).

    With attention the passage is a sequence of its own: its positions attend only within it
    (an empty cache at q_0), and the stream's cache is neither read nor changed. [SGF],
    Settlement, compares the two candidate states with the attention left as it is, so only
    the fast weights differ between the two scores; scoring the passage apart from the stream
    is the plainest reading of that.
    """
    q = np.asarray(q, dtype=np.int64)
    l, _, _ = token_losses(model, as_f64(P), q[:-1], q[1:])
    return float(l.mean())


def settle_step(model: Model, P: Dict[str, np.ndarray], cand: np.ndarray, q: np.ndarray, kv=None):
    """The Settlement rule of [SGF] for one candidate chunk.

    From the current weights W (P), the candidate's update delta is the clipped mini-batch
    step of [E2E] eq. (5) on the candidate chunk cand_0..cand_b. On the held-out passage q,
    A(delta; W, q) = L(q, W) - L(q, W + delta), and delta is committed only if A >= 0.
    Returns (A, committed, the weights after the decision, g, s).

    With attention, kv is the stream's cache in front of the candidate chunk. The chunk is
    part of the stream whatever the decision: its keys and values (computed at W) join the
    cache, as chunk_loss_and_grads(..., kv=kv)[1]["kv"] gives them.
    """
    P = as_f64(P)
    cand = np.asarray(cand, dtype=np.int64)
    keys = model.fast_keys()
    _, _, G = chunk_loss_and_grads(model, P, cand[:-1], cand[1:], kv=kv)
    g = math.sqrt(sum(float(np.sum(G[k] * G[k])) for k in keys))
    s = clip_scale(g, model.clip) if math.isfinite(g) else 0.0
    Pd = dict(P)
    for k in keys:
        Pd[k] = P[k] - model.lr * s * G[k]
    A = passage_loss(model, P, q) - passage_loss(model, Pd, q)
    keep = bool(A >= 0.0)
    return A, keep, ({k: Pd[k] for k in keys} if keep else {k: P[k] for k in keys}), g, s


def static_losses(model: Model, P0, tokens, n_tokens: Optional[int] = None) -> np.ndarray:
    """l_t(W_0) for every t: the summands of L_naive, [E2E] eq. (4)."""
    P0 = as_f64(P0)
    tokens = np.asarray(tokens, dtype=np.int64)
    T = tokens.shape[0] - 1 if n_tokens is None else n_tokens
    out = []
    step = 4096 if model.swa_window == 0 else max(model.chunk, 1)
    kv = None
    for s in range(0, T, step):
        e = min(T, s + step)
        z, _, cache = logits(model, P0, tokens[s:e], kv)
        l, _, _, _ = ce_stats(z, tokens[s + 1:e + 1])
        if model.swa_window > 0:
            kv = next_kv(model, kv, cache)
        out.append(l)
    return np.concatenate(out)

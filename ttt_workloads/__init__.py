"""Seeded synthetic workloads for the chunk-wise test-time-training (TTT) inner loop.

This module only *generates inputs*: the workload presets (shapes and
hyper-parameters), token streams and initial weights. It holds none of the
method's arithmetic (no forward pass, loss, gradient or update), so that both
the fp64 oracle and the HIP path can take their inputs from it without sharing
any computation.

Where the inputs come from (page: "End-to-End Test-Time Training for Long
Context", review on kimjy99.github.io):
  * the stream is x_0 .. x_T with x_0 the BOS token (Method section);
  * the toy model is effectively a bigram model, so the toy stream is a sparse
    bigram Markov chain (section 1, "TTT via Next-Token Prediction").
The pages' own workloads are book text and long-context suites that are not
available here; the Zipf + sparse-Markov streams below stand in for them with
the same vocabulary sizes, stream lengths and chunking.

Recipe (every draw comes from numpy's PCG64, seeded by one master seed per
workload and split with SeedSequence.spawn):
  * sparse Markov chain: every id v gets 8 distinct successors drawn uniformly
    from [0, V) and transition probabilities ~ Dirichlet(0.5 * 1_8);
  * Zipf(s=1.1) on a finite support: P(id = k-1) proportional to k^-1.1 for
    k = 1..V, sampled by inverse CDF;
  * stream: x_0 = 0; for t >= 1 the "markov" stream draws x_t from the chain
    row of x_{t-1}; the "zipf_markov" stream draws Zipf with probability 1/2,
    otherwise the chain row of x_{t-1};
  * weights: every tensor i.i.d. N(0, 0.02^2) (0.02 is the standard deviation),
    rounded to bfloat16 (round-to-nearest-even) for bf16 workloads so that both
    sides start from exactly the same values.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

BOS = 0

# The five benchmark workloads, and the fuller-block variant of the 760M shape. "fp32"
# workloads keep weights in float32; "bf16" ones
# round every initial tensor to bfloat16.
PRESETS: Dict[str, dict] = {
    # MLP-only bigram toy: per-token update (chunk 1), no clipping.
    "toy": dict(vocab=256, d_model=64, d_hidden=256, n_blocks=1, mlp="gelu",
                norm="none", precision="fp32", n_tokens=128, chunk=1,
                lr=0.1, clip=0.0, stream="markov"),
    # One residual GELU block, both W1 and W2 fast.
    "single": dict(vocab=32000, d_model=768, d_hidden=3072, n_blocks=1,
                   mlp="gelu", norm="none", precision="bf16", n_tokens=8192,
                   chunk=1024, lr=0.01, clip=1.0, stream="zipf_markov"),
    # Last three residual blocks of a 125M-style model, pre-RMSNorm, 128K stream.
    "s125m": dict(vocab=32000, d_model=768, d_hidden=3072, n_blocks=3,
                  mlp="gelu", norm="rms", precision="bf16", n_tokens=131072,
                  chunk=1024, lr=0.01, clip=1.0, stream="zipf_markov"),
    # 760M-shaped three-block stack.
    "s760m": dict(vocab=32000, d_model=1536, d_hidden=6144, n_blocks=3,
                  mlp="gelu", norm="rms", precision="bf16", n_tokens=32768,
                  chunk=1024, lr=0.005, clip=1.0, stream="zipf_markov"),
    # Fuller TTT-E2E block at the 760M shape: frozen sliding-window attention (window 8K
    # over 1K chunks, 12 heads of 128) and a frozen static MLP before the fast one in each
    # block, the MLP hidden size split between the two so the parameters stay equal.
    "e2e760m": dict(vocab=32000, d_model=1536, d_hidden=3072, n_blocks=3,
                    mlp="gelu", norm="rms", precision="bf16", n_tokens=32768,
                    chunk=1024, lr=0.005, clip=1.0, stream="zipf_markov", static_hidden=3072,
                    swa_window=8192, swa_heads=12),
    # In-Place-TTT shape: SwiGLU with frozen gate/up, only the down-projection fast.
    "inplace": dict(vocab=151936, d_model=2560, d_hidden=9728, n_blocks=1,
                    mlp="swiglu_w2", norm="rms", precision="bf16",
                    n_tokens=65536, chunk=512, lr=0.005, clip=1.0,
                    stream="zipf_markov"),
}

RMS_EPS = 1e-6
INIT_STD = 0.02


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    vocab: int
    d_model: int
    d_hidden: int
    n_blocks: int
    mlp: str          # "gelu" (W1, W2 fast) | "swiglu_w2" (gate/up frozen, W2 fast)
    norm: str         # "none" | "rms"
    precision: str    # "fp32" | "bf16"
    n_tokens: int     # T
    chunk: int        # b
    lr: float         # eta
    clip: float       # <= 0 disables clipping
    stream: str       # "markov" | "zipf_markov"
    eps: float = RMS_EPS
    static_hidden: int = 0  # hidden size of a frozen static MLP before the fast one (0: none)
    swa_window: int = 0     # keys per query of a frozen sliding-window attention first (0: none)
    swa_heads: int = 0      # its heads

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def n_chunks(self) -> int:
        return self.n_tokens // self.chunk

    def fast_names(self) -> List[str]:
        return ["W1", "W2"] if self.mlp == "gelu" else ["W2"]


def preset(name: str, **overrides) -> Workload:
    kw = dict(PRESETS[name])
    kw.update(overrides)
    return Workload(name=name, **kw)


# ---------------------------------------------------------------- bf16 rounding
def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); return float32.

    NaN stays NaN. This only prepares inputs: both sides receive these exact values.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = (bits + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    out = rounded.view(np.float32).copy()
    nan = np.isnan(a)
    if nan.any():
        out[nan] = np.nan
    return out


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array holding exact bf16 values -> uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ---------------------------------------------------------------- token streams
def _seeds(seed: int, n: int) -> List[np.random.SeedSequence]:
    return np.random.SeedSequence(seed).spawn(n)


def markov_chain(vocab: int, rng: np.random.Generator, k: int = 8,
                 alpha: float = 0.5):
    """Sparse bigram chain: k distinct successors per id, Dirichlet(alpha) probabilities.

    Returns (succ [V, k] int64, cum [V, k] float64 cumulative probabilities).
    """
    k = min(k, vocab)
    succ = rng.integers(0, vocab, size=(vocab, k))
    while True:  # redraw rows holding a repeated successor
        s = np.sort(succ, axis=1)
        bad = np.nonzero((s[:, 1:] == s[:, :-1]).any(axis=1))[0]
        if bad.size == 0:
            break
        succ[bad] = rng.integers(0, vocab, size=(bad.size, k))
    probs = rng.dirichlet(np.full(k, alpha), size=vocab)
    cum = np.cumsum(probs, axis=1)
    cum[:, -1] = 1.0
    return succ, cum


def zipf_cdf(vocab: int, s: float = 1.1) -> np.ndarray:
    w = np.arange(1, vocab + 1, dtype=np.float64) ** (-s)
    cdf = np.cumsum(w)
    return cdf / cdf[-1]


def token_stream(w: Workload, seed: int = 0, n_tokens: Optional[int] = None) -> np.ndarray:
    """Ids x_0..x_T (int32, length T+1) with x_0 = BOS = 0."""
    T = w.n_tokens if n_tokens is None else n_tokens
    s_chain, s_stream = _seeds(seed, 2)
    succ, cum = markov_chain(w.vocab, np.random.default_rng(s_chain))
    rng = np.random.default_rng(s_stream)
    u_chain = rng.random(T)
    coin = rng.random(T) < 0.5
    zipf = np.searchsorted(zipf_cdf(w.vocab), rng.random(T), side="right")
    zipf = np.minimum(zipf, w.vocab - 1)
    use_zipf = coin if w.stream == "zipf_markov" else np.zeros(T, dtype=bool)
    x = np.empty(T + 1, dtype=np.int64)
    x[0] = BOS
    k = succ.shape[1]
    for t in range(1, T + 1):
        if use_zipf[t - 1]:
            x[t] = zipf[t - 1]
        else:
            prev = x[t - 1]
            j = int(np.searchsorted(cum[prev], u_chain[t - 1], side="right"))
            x[t] = succ[prev, min(j, k - 1)]
    return x.astype(np.int32)


# ---------------------------------------------------------------- weights
def weight_shapes(w: Workload) -> Dict[str, tuple]:
    """Row-major shapes. W1/Wg/Wu map d -> m ([d, m]); W2 maps m -> d ([m, d])."""
    shapes = {"E_in": (w.vocab, w.d_model), "E_out": (w.vocab, w.d_model)}
    for l in range(w.n_blocks):
        if w.mlp == "gelu":
            shapes[f"W1.{l}"] = (w.d_model, w.d_hidden)
        else:
            shapes[f"Wg.{l}"] = (w.d_model, w.d_hidden)
            shapes[f"Wu.{l}"] = (w.d_model, w.d_hidden)
        shapes[f"W2.{l}"] = (w.d_hidden, w.d_model)
        if w.static_hidden > 0:
            shapes[f"Ws1.{l}"] = (w.d_model, w.static_hidden)
            shapes[f"Ws2.{l}"] = (w.static_hidden, w.d_model)
        if w.swa_window > 0:
            for n in ("Wk", "Wo", "Wq", "Wv"):
                shapes[f"{n}.{l}"] = (w.d_model, w.d_model)
    return shapes


def init_weights(w: Workload, seed: int = 0, std: float = INIT_STD) -> Dict[str, np.ndarray]:
    """All tensors i.i.d. N(0, std^2) as float32; bf16-exact for bf16 workloads.

    Each tensor has its own child seed, so a tensor's values do not depend on
    which other tensors are drawn.
    """
    shapes = weight_shapes(w)
    names = sorted(shapes)
    kids = _seeds(seed + 1_000_003, len(names))
    out = {}
    for name, ss in zip(names, kids):
        rng = np.random.default_rng(ss)
        a = rng.standard_normal(shapes[name], dtype=np.float32)
        a *= np.float32(std)
        if w.precision == "bf16":
            a = round_to_bf16(a)
        out[name] = a
    return out

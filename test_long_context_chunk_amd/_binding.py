"""ctypes binding of the HIP library declared in include/ttt.h.

Argument marshalling only: torch tensors are used for device memory and streams, their
pointers are handed to the library, and every step of the inner loop runs in the
library's HIP kernels. There is no fallback: if the library is missing or fails to load,
constructing a context raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

from .build import lib_path

c_int32, c_int64, c_float, c_void_p = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p

ABI_VERSION = 1
STATUS = {0: "TTT_OK", -1: "TTT_EINVAL", -2: "TTT_ENOMEM", -3: "TTT_EDEVICE",
          -4: "TTT_ERANGE", -5: "TTT_ENONFINITE", -6: "TTT_ESTATE"}
MLP = {"gelu": 0, "swiglu_w2": 1}
NORM = {"none": 0, "rms": 1}
PRECISION = {"fp32": 0, "bf16": 1}
# ttt_kernel_kind order of include/ttt.h
KERNEL_KINDS = ["gather", "norm", "transpose", "up", "down", "residual", "ce_fwd", "ce_merge", "ce_prob",
                "ce_dy", "dy_sum", "du", "dw", "dhn", "norm_bwd", "gradnorm", "update", "dec_gemv", "attn", "attn_bwd"]

# Functions declared in include/ttt.h, with their ctypes signatures.
SIGNATURES = {
    "ttt_create": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p]),
    "ttt_create_batch": (c_int32, [c_void_p, c_void_p, c_int32, c_void_p, c_void_p]),
    "ttt_create_ext": (c_int32, [c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_void_p]),
    "ttt_streams": (c_int32, [c_void_p]),
    "ttt_prefill_chunks": (c_int32, [c_void_p, c_void_p, c_int64]),
    "ttt_prefill_batch": (c_int32, [c_void_p, c_void_p, c_int64, c_int64]),
    "ttt_stream_token_losses": (c_int32, [c_void_p, c_int32, c_void_p, c_int64, c_int64]),
    "ttt_stream_token_argmax": (c_int32, [c_void_p, c_int32, c_void_p, c_int64, c_int64]),
    "ttt_stream_chunk_stats": (c_int32, [c_void_p, c_int32, c_void_p, c_int64, c_int64]),
    "ttt_stream_fast_weights": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_int32, c_void_p]),
    "ttt_token_losses": (c_int32, [c_void_p, c_void_p, c_int64, c_int64]),
    "ttt_token_argmax": (c_int32, [c_void_p, c_void_p, c_int64, c_int64]),
    "ttt_chunk_stats": (c_int32, [c_void_p, c_void_p, c_int64, c_int64]),
    "ttt_fast_weights": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_void_p]),
    "ttt_reset": (c_int32, [c_void_p]),
    "ttt_sync": (c_int32, [c_void_p]),
    "ttt_tokens_consumed": (c_int64, [c_void_p]),
    "ttt_destroy": (c_int32, [c_void_p]),
    "ttt_status_string": (ctypes.c_char_p, [c_int32]),
    "ttt_decode": (c_int32, [c_void_p, c_void_p, c_int64, c_void_p, c_void_p]),
    "ttt_decode_pending": (c_int64, [c_void_p]),
    "ttt_evaluate": (c_int32, [c_void_p, c_void_p, c_int64, c_void_p, c_void_p]),
    "ttt_snapshot": (c_int32, [c_void_p]),
    "ttt_restore": (c_int32, [c_void_p]),
    "ttt_settle_chunk": (c_int32, [c_void_p, c_void_p, c_void_p, c_int64, c_void_p, c_void_p]),
    "ttt_settle_chunk_noalloc": (c_int32, [c_void_p, c_void_p, c_void_p, c_int64, c_void_p, c_void_p]),
    "ttt_profile_enable": (c_int32, [c_void_p, ctypes.c_uint32]),
    "ttt_profile_period": (c_int32, [c_void_p, c_int32]),
    "ttt_profile_read": (c_int32, [c_void_p, c_void_p, c_void_p]),
    "ttt_test_gemm": (c_int32, [c_int32, c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_int64,
                                c_int32, c_int32, c_int32, c_void_p]),
    "ttt_test_gemm_pair": (c_int32, [c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_int64,
                                     c_int32, c_int32, c_int32, c_int32, c_int32, c_void_p]),
    "ttt_test_grad": (c_int32, [c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_int32,
                                c_int32, c_int32, c_int32, c_void_p]),
}


class Config(ctypes.Structure):
    _fields_ = [("abi_version", c_int32), ("vocab", c_int32), ("d_model", c_int32),
                ("d_hidden", c_int32), ("n_blocks", c_int32), ("mlp", c_int32), ("norm", c_int32),
                ("precision", c_int32), ("chunk", c_int32), ("reserved", c_int32),
                ("max_tokens", c_int64), ("lr", c_float), ("clip", c_float),
                ("rms_eps", c_float), ("reserved_f", c_float)]


class Weights(ctypes.Structure):
    _fields_ = [("embed", c_void_p), ("lm_head", c_void_p), ("w1", ctypes.POINTER(c_void_p)),
                ("w_up", ctypes.POINTER(c_void_p)), ("w2", ctypes.POINTER(c_void_p))]


class BlockExt(ctypes.Structure):
    _fields_ = [("static_hidden", c_int32), ("swa_window", c_int32), ("swa_heads", c_int32),
                ("reserved", c_int32)] + [(n, ctypes.POINTER(c_void_p)) for n in ("ws1", "ws2", "wq", "wk", "wv", "wo")]


class TTTError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({_status_string(status)})")


_LIB: Optional[ctypes.CDLL] = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the HIP library (after torch, so that both share one HIP runtime)."""
    global _LIB
    if _LIB is not None and path is None:
        return _LIB
    p = path or lib_path()
    if not os.path.exists(p):
        raise RuntimeError(f"HIP library {p} is not built: run `python -m test_long_context_chunk_amd.build`")
    import torch  # noqa: F401  (loads torch's libamdhip64 first; ours binds to the same soname)
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _LIB = lib
    return lib


def _status_string(s: int) -> str:
    try:
        return load_library().ttt_status_string(s).decode()
    except Exception:
        return "?"


def _check(status: int, what: str):
    if status != 0:
        raise TTTError(status, what)


# Sticky conditions found on the device (id out of range, non-finite gradient norm): the
# record copies still complete, so getters return their data and sync() reports the status.
_STICKY = (-4, -5)


def _check_copy(status: int, what: str):
    if status != 0 and status not in _STICKY:
        raise TTTError(status, what)


def _ptr(t) -> int:
    return t.data_ptr()


def _stream_handle(stream) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def to_device(a, precision: str, device="cuda"):
    """numpy float32 array -> contiguous device tensor in the GEMM precision (bf16 bits or fp32)."""
    import numpy as np
    import torch
    a = np.ascontiguousarray(a, dtype=np.float32)
    t = torch.from_numpy(a)
    if precision == "bf16":
        # values are bf16-exact already; the cast keeps them bit for bit
        t = t.to(torch.bfloat16)
    return t.to(device).contiguous()


class TTT:
    """One context of the library: private fast weights, bound to one HIP stream. With
    streams > 1, that many independent token streams advanced together (prefill_batch and
    the readers' `s` argument)."""

    def __init__(self, *, vocab: int, d_model: int, d_hidden: int, n_blocks: int, mlp: str,
                 norm: str, precision: str, chunk: int, max_tokens: int, lr: float, clip: float,
                 rms_eps: float = 1e-6, weights: Dict[str, "object"], stream=None, streams: int = 1,
                 static_hidden: int = 0, swa_window: int = 0, swa_heads: int = 0):
        import torch
        self._lib = load_library()
        self.vocab, self.d_model, self.d_hidden, self.n_blocks = vocab, d_model, d_hidden, n_blocks
        self.mlp, self.norm, self.precision, self.chunk = mlp, norm, precision, chunk
        self.max_tokens = max_tokens
        self.streams = streams
        self.static_hidden = static_hidden
        self.swa_window, self.swa_heads = swa_window, swa_heads
        self._stream = stream if stream is not None else torch.cuda.current_stream()
        dt = torch.bfloat16 if precision == "bf16" else torch.float32
        for k, t in weights.items():
            if t.dtype != dt or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"weight {k} must be a contiguous {dt} device tensor")
        cfg = Config(ABI_VERSION, vocab, d_model, d_hidden, n_blocks, MLP[mlp], NORM[norm],
                     PRECISION[precision], chunk, 0, max_tokens, lr, clip, rms_eps, 0.0)
        L = n_blocks
        first = "W1" if mlp == "gelu" else "Wg"
        w1 = (c_void_p * max(L, 1))(*[_ptr(weights[f"{first}.{l}"]) for l in range(L)])
        w2 = (c_void_p * max(L, 1))(*[_ptr(weights[f"W2.{l}"]) for l in range(L)])
        wup = (c_void_p * max(L, 1))(*[_ptr(weights[f"Wu.{l}"]) for l in range(L)]) if mlp == "swiglu_w2" else None
        w = Weights(_ptr(weights["E_in"]), _ptr(weights["E_out"]),
                    ctypes.cast(w1, ctypes.POINTER(c_void_p)),
                    ctypes.cast(wup, ctypes.POINTER(c_void_p)) if wup is not None else None,
                    ctypes.cast(w2, ctypes.POINTER(c_void_p)))
        ext = None
        if static_hidden > 0 or swa_window > 0:
            def arr(name, on):
                if not on:
                    return None
                a = (c_void_p * max(L, 1))(*[_ptr(weights[f"{name}.{l}"]) for l in range(L)])
                self._keep.append(a)
                return ctypes.cast(a, ctypes.POINTER(c_void_p))
            self._keep = []
            s_on, a_on = static_hidden > 0, swa_window > 0
            ext = BlockExt(static_hidden, swa_window, swa_heads, 0, arr("Ws1", s_on), arr("Ws2", s_on),
                           arr("Wq", a_on), arr("Wk", a_on), arr("Wv", a_on), arr("Wo", a_on))
        ctx = c_void_p()
        _check(self._lib.ttt_create_ext(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(ext) if ext else None,
                                        streams, c_void_p(_stream_handle(self._stream)), ctypes.byref(ctx)),
               "ttt_create_ext")
        self._ctx = ctx

    @classmethod
    def from_workload(cls, w, weights: Dict[str, "object"], max_tokens: Optional[int] = None, stream=None, **kw):
        """Create from a workload description (any object with the preset fields)."""
        args = dict(vocab=w.vocab, d_model=w.d_model, d_hidden=w.d_hidden, n_blocks=w.n_blocks,
                    mlp=w.mlp, norm=w.norm, precision=w.precision, chunk=w.chunk,
                    max_tokens=max_tokens or w.n_tokens, lr=w.lr, clip=w.clip, rms_eps=w.eps,
                    static_hidden=getattr(w, "static_hidden", 0), swa_window=getattr(w, "swa_window", 0),
                    swa_heads=getattr(w, "swa_heads", 0))
        args.update(kw)
        return cls(weights=weights, stream=stream, **args)

    # ------------------------------------------------------------------ calls
    def prefill(self, tokens) -> None:
        """tokens: device int32 [n + 1]; runs n / chunk TTT steps (enqueued)."""
        import torch
        if tokens.dtype != torch.int32 or not tokens.is_cuda or not tokens.is_contiguous():
            raise ValueError("tokens must be a contiguous int32 device tensor")
        n = tokens.numel() - 1
        _check(self._lib.ttt_prefill_chunks(self._ctx, c_void_p(_ptr(tokens)), n), "ttt_prefill_chunks")

    def prefill_batch(self, tokens) -> None:
        """tokens: device int32 [streams x ld] (row z: stream z's n + 1 ids, n = ld - 1); runs
        n / chunk steps of every stream (enqueued)."""
        import torch
        if tokens.dtype != torch.int32 or not tokens.is_cuda or tokens.dim() != 2 or tokens.stride(1) != 1:
            raise ValueError("tokens must be an int32 device tensor [streams x ld] with unit column stride")
        if tokens.shape[0] != self.streams:
            raise ValueError(f"tokens has {tokens.shape[0]} rows for {self.streams} streams")
        n = tokens.shape[1] - 1
        _check(self._lib.ttt_prefill_batch(self._ctx, c_void_p(_ptr(tokens)), tokens.stride(0), n),
               "ttt_prefill_batch")

    def decode(self, tokens, want_logits: bool = False):
        """tokens: device int32 [n + 1] (tokens[0] = the stream's last token). Predicts each of
        tokens[1..n] from the one before at the current weights, stepping whenever a chunk fills.
        Returns (argmax int32 [n], logits fp32 [n x vocab] or None)."""
        import torch
        if tokens.dtype != torch.int32 or not tokens.is_cuda or not tokens.is_contiguous():
            raise ValueError("tokens must be a contiguous int32 device tensor")
        n = tokens.numel() - 1
        am = torch.empty(max(n, 0), dtype=torch.int32, device="cuda")
        z = torch.empty((max(n, 0), self.vocab), dtype=torch.float32, device="cuda") if want_logits else None
        _check(self._lib.ttt_decode(self._ctx, c_void_p(_ptr(tokens)), n, c_void_p(_ptr(am) if n > 0 else None),
                                    c_void_p(_ptr(z)) if (z is not None and n > 0) else None), "ttt_decode")
        return am, z

    def evaluate(self, q):
        """q: device int32 [nq + 1]. Returns (per-token losses fp32 [nq], mean fp32 [1]) at the
        current weights; nothing changes."""
        import torch
        if q.dtype != torch.int32 or not q.is_cuda or not q.is_contiguous():
            raise ValueError("q must be a contiguous int32 device tensor")
        nq = q.numel() - 1
        losses = torch.empty(max(nq, 1), dtype=torch.float32, device="cuda")
        mean = torch.empty(1, dtype=torch.float32, device="cuda")
        _check(self._lib.ttt_evaluate(self._ctx, c_void_p(_ptr(q)), nq, c_void_p(_ptr(losses)), c_void_p(_ptr(mean))),
               "ttt_evaluate")
        return losses[:nq], mean

    def snapshot(self) -> None:
        _check(self._lib.ttt_snapshot(self._ctx), "ttt_snapshot")

    def restore(self) -> None:
        _check(self._lib.ttt_restore(self._ctx), "ttt_restore")

    def settle(self, tokens, q):
        """One candidate chunk (tokens: device int32 [chunk + 1]) under the Settlement rule
        against the passage q (device int32 [nq + 1]). Returns (A fp32 [1], committed int32 [1])."""
        import torch
        for t in (tokens, q):
            if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
                raise ValueError("tokens and q must be contiguous int32 device tensors")
        A = torch.empty(1, dtype=torch.float32, device="cuda")
        kept = torch.empty(1, dtype=torch.int32, device="cuda")
        _check(self._lib.ttt_settle_chunk(self._ctx, c_void_p(_ptr(tokens)), c_void_p(_ptr(q)), q.numel() - 1,
                                          c_void_p(_ptr(A)), c_void_p(_ptr(kept))), "ttt_settle_chunk")
        return A, kept

    def settle_noalloc(self, tokens, q, A, kept) -> None:
        """settle() through ttt_settle_chunk_noalloc, into caller-provided outputs (A: device
        fp32 [1], kept: device int32 [1]); the library allocates nothing for it."""
        import torch
        for t in (tokens, q):
            if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
                raise ValueError("tokens and q must be contiguous int32 device tensors")
        _check(self._lib.ttt_settle_chunk_noalloc(self._ctx, c_void_p(_ptr(tokens)), c_void_p(_ptr(q)),
                                                  q.numel() - 1, c_void_p(_ptr(A)), c_void_p(_ptr(kept))),
               "ttt_settle_chunk_noalloc")

    def decode_pending(self) -> int:
        return int(self._lib.ttt_decode_pending(self._ctx))

    def token_losses(self, offset: int = 0, n: Optional[int] = None, s: int = 0):
        import torch
        n = self.consumed() - offset if n is None else n
        out = torch.empty(n, dtype=torch.float32, device="cuda")
        _check_copy(self._lib.ttt_stream_token_losses(self._ctx, s, c_void_p(_ptr(out)), offset, n),
                    "ttt_stream_token_losses")
        return out

    def token_argmax(self, offset: int = 0, n: Optional[int] = None, s: int = 0):
        import torch
        n = self.consumed() - offset if n is None else n
        out = torch.empty(n, dtype=torch.int32, device="cuda")
        _check_copy(self._lib.ttt_stream_token_argmax(self._ctx, s, c_void_p(_ptr(out)), offset, n),
                    "ttt_stream_token_argmax")
        return out

    def chunk_stats(self, offset: int = 0, n: Optional[int] = None, s: int = 0):
        import torch
        n = self.consumed() // self.chunk - offset if n is None else n
        out = torch.empty((n, 2), dtype=torch.float32, device="cuda")
        _check_copy(self._lib.ttt_stream_chunk_stats(self._ctx, s, c_void_p(_ptr(out)), offset, n),
                    "ttt_stream_chunk_stats")
        return out

    def fast_weight(self, block: int, which: str, kind: str = "W", s: int = 0):
        """which: "W1" | "W2"; kind: "W" (current) | "delta" (W - W0); s: stream. fp32 device tensor."""
        import torch
        shape = (self.d_model, self.d_hidden) if which == "W1" else (self.d_hidden, self.d_model)
        out = torch.empty(shape, dtype=torch.float32, device="cuda")
        _check_copy(self._lib.ttt_stream_fast_weights(self._ctx, s, block, 1 if which == "W1" else 2,
                                                      0 if kind == "W" else 1, c_void_p(_ptr(out))),
                    "ttt_stream_fast_weights")
        return out

    def profile(self, kinds, period: int = 1) -> None:
        """Bracket launches of the given kernel kinds (names of KERNEL_KINDS) with HIP events,
        in every period-th chunk."""
        mask = 0
        for k in kinds:
            mask |= 1 << KERNEL_KINDS.index(k)
        _check(self._lib.ttt_profile_period(self._ctx, int(period)), "ttt_profile_period")
        _check(self._lib.ttt_profile_enable(self._ctx, mask), "ttt_profile_enable")

    def profile_read(self) -> Dict[str, tuple]:
        """{kind: (total_ms, launches)} for the bracketed launches since the last read."""
        tot = (ctypes.c_double * len(KERNEL_KINDS))()
        cnt = (c_int64 * len(KERNEL_KINDS))()
        _check(self._lib.ttt_profile_read(self._ctx, ctypes.cast(tot, c_void_p), ctypes.cast(cnt, c_void_p)),
               "ttt_profile_read")
        return {k: (tot[i], cnt[i]) for i, k in enumerate(KERNEL_KINDS) if cnt[i] > 0}

    def reset(self) -> None:
        _check(self._lib.ttt_reset(self._ctx), "ttt_reset")

    def sync(self) -> int:
        return self._lib.ttt_sync(self._ctx)

    def consumed(self) -> int:
        return int(self._lib.ttt_tokens_consumed(self._ctx))

    def close(self) -> None:
        if getattr(self, "_ctx", None):
            self._lib.ttt_destroy(self._ctx)
            self._ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def grad_test_hook(X, Y, token_major: bool, stream=None):
    """The weight-gradient GEMM (bf16 G and per-tile sums of squares) through the library's
    kernels (test hook). token_major: X [K x M], Y [K x N]; else X [M x K], Y [N x K]."""
    import torch
    lib = load_library()
    if token_major:
        K, M = X.shape
        N = Y.shape[1]
    else:
        M, K = X.shape
        N = Y.shape[0]
    G = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    slots = torch.zeros(((M + 127) // 128) * ((N + 127) // 128), dtype=torch.float32, device="cuda")
    _check(lib.ttt_test_grad(c_void_p(_ptr(X)), X.stride(0), c_void_p(_ptr(Y)), Y.stride(0), c_void_p(_ptr(G)), N,
                             c_void_p(_ptr(slots)), M, N, K, 1 if token_major else 0,
                             c_void_p(_stream_handle(stream))), "ttt_test_grad")
    return G, slots


def gemm_pair_test_hook(X, Y, Y2, splits: int = 1, form: int = 0, stream=None):
    """C = X (Y + Y2)^T (bf16 operands, two K-segments over the same X rows) through the
    library's GEMM tile engine (test hook); returns the fp32 slabs [splits x M x N]. form: 0 the
    inner loop's choice, 1 the segments one after the other, 2 shared X slices."""
    import torch
    lib = load_library()
    M, K = X.shape
    N = Y.shape[0]
    C = torch.empty((splits, M, N), dtype=torch.float32, device="cuda")
    _check(lib.ttt_test_gemm_pair(c_void_p(_ptr(X)), X.stride(0), c_void_p(_ptr(Y)), Y.stride(0), c_void_p(_ptr(Y2)),
                                  Y2.stride(0), c_void_p(_ptr(C)), N, M, N, K, splits, form,
                                  c_void_p(_stream_handle(stream))), "ttt_test_gemm_pair")
    return C


def gemm_test_hook(X, Y, precision: str, stream=None):
    """C = X Y^T through the library's GEMM tile engine (test hook)."""
    import torch
    lib = load_library()
    M, K = X.shape
    N = Y.shape[0]
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    _check(lib.ttt_test_gemm(PRECISION[precision], c_void_p(_ptr(X)), X.stride(0), c_void_p(_ptr(Y)),
                             Y.stride(0), c_void_p(_ptr(C)), N, M, N, K,
                             c_void_p(_stream_handle(stream))), "ttt_test_gemm")
    return C

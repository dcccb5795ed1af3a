"""Shared helpers of the GPU parity tests: seeded inputs, one GPU run, one oracle run, gates.

Gates (element by element on the same seeded inputs):
  bf16 mode: per-token loss |delta| <= 1e-2; final fast weights relative L2 <= 2e-2; the
             accumulated update D = W - W0 relative L2 <= 2e-2; per-chunk grad norm
             relative error <= 1e-2.
  fp32 mode: the same at 1e-4 (grad norm 1e-5).
  argmax:    exact, except tokens whose oracle logit at the GPU's pick is within the loss
             tolerance of the oracle's maximum (a near tie that either precision may break
             either way); those are counted, and every pick must be such a valid one.
"""
from __future__ import annotations

import math
import sys
from typing import Dict, Optional

import numpy as np

import oracle as O
import ttt_workloads as W

TOL = {
    "bf16": dict(loss=1e-2, w=2e-2, dw=2e-2, g=1e-2, logit=1e-2),
    "fp32": dict(loss=1e-4, w=1e-4, dw=1e-4, g=1e-5, logit=1e-4),
}

_INPUTS: Dict[tuple, tuple] = {}
_ORACLE: Dict[tuple, object] = {}


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def inputs(name: str, seed: int = 0, **over):
    key = (name, seed, tuple(sorted(over.items())))
    if key not in _INPUTS:
        w = W.preset(name, **over)
        _INPUTS[key] = (w, W.token_stream(w, seed), W.init_weights(w, seed))
    return _INPUTS[key]


def device_weights(P, precision):
    import test_long_context_chunk_amd as ttt
    return {k: ttt.to_device(v, precision) for k, v in P.items()}


def gpu_run(w, P, x, n_tokens: Optional[int] = None, precision: Optional[str] = None, calls: int = 1,
            dev=None, keep_ctx=False, **cfg_over):
    import torch
    import test_long_context_chunk_amd as ttt
    prec = precision or w.precision
    T = n_tokens if n_tokens is not None else len(x) - 1
    dev = dev if dev is not None else device_weights(P, prec)
    ctx = ttt.TTT.from_workload(w, dev, max_tokens=T, precision=prec, **cfg_over)
    tok = torch.from_numpy(np.ascontiguousarray(x[:T + 1], dtype=np.int32)).cuda()
    per = T // calls
    assert per % w.chunk == 0
    for c in range(calls):
        ctx.prefill(tok[c * per: (c + 1) * per + 1])
    out = dict(losses=ctx.token_losses().cpu().numpy().astype(np.float64),
               argmax=ctx.token_argmax().cpu().numpy().astype(np.int64),
               stats=ctx.chunk_stats().cpu().numpy().astype(np.float64))
    Wf, Df = {}, {}
    for l in range(w.n_blocks):
        for n in w.fast_names():
            Wf[f"{n}.{l}"] = ctx.fast_weight(l, n, "W").cpu().numpy().astype(np.float64)
            Df[f"{n}.{l}"] = ctx.fast_weight(l, n, "delta").cpu().numpy().astype(np.float64)
    out["W"], out["D"] = Wf, Df
    out["status"] = ctx.sync()
    if keep_ctx:
        out["ctx"] = ctx
    else:
        ctx.close()
    return out


def oracle_run(w, P, x, n_chunks: int, gpu_argmax: Optional[np.ndarray] = None, key=None):
    """fp64 oracle over the first n_chunks chunks; with gpu_argmax, also the oracle's logit
    at the GPU's pick and its own maximum (for the argmax validity gate)."""
    model = O.Model.from_workload(w)
    b = w.chunk
    at_pick, top = [], []

    def probe(i, z):
        if gpu_argmax is not None:
            rows = np.arange(z.shape[0])
            at_pick.append(z[rows, gpu_argmax[i * b:(i + 1) * b]])
            top.append(z.max(axis=1))

    ck = None if key is None else (key, n_chunks)
    if ck is not None and ck in _ORACLE and gpu_argmax is None:
        return _ORACLE[ck]
    res = O.run_ttt(model, P, x[:n_chunks * b + 1], n_chunks=n_chunks, logit_probe=probe)
    if gpu_argmax is not None:
        res.pick_gap = np.concatenate(top) - np.concatenate(at_pick)
    if ck is not None:
        _ORACLE[ck] = res
    return res


def rel_l2(a, b):
    nb = float(np.linalg.norm(b))
    return float(np.linalg.norm(a - b)) / nb if nb > 0 else float(np.linalg.norm(a - b))


def compare(gpu, orc, w, precision: str, n_chunks: int, check_weights: bool = True, label: str = ""):
    """Assert every gate on the first n_chunks chunks; return the measured errors."""
    tol = TOL[precision]
    b = w.chunk
    n = n_chunks * b
    rep = {}
    dl = np.abs(gpu["losses"][:n] - orc.losses[:n])
    rep["loss_max_abs"] = float(dl.max())
    am_g, am_o = gpu["argmax"][:n], orc.argmax[:n]
    mism = am_g != am_o
    rep["argmax_mismatch"] = int(mism.sum())
    if hasattr(orc, "pick_gap"):
        rep["argmax_worst_pick_gap"] = float(orc.pick_gap[:n].max())
    g_g = gpu["stats"][:n_chunks, 0]
    rep["gnorm_max_rel"] = float(np.max(np.abs(g_g - orc.grad_norm[:n_chunks]) /
                                        np.maximum(orc.grad_norm[:n_chunks], 1e-30)))
    rep["scale_max_abs"] = float(np.max(np.abs(gpu["stats"][:n_chunks, 1] - orc.scale[:n_chunks])))
    if check_weights:
        rep["W_rel_l2"] = max(rel_l2(gpu["W"][k], orc.weights[k]) for k in orc.weights)
        rep["D_rel_l2"] = max(rel_l2(gpu["D"][k], orc.delta[k]) for k in orc.delta)
    log(f"[parity {label} {precision} {n_chunks} chunks] " + " ".join(f"{k}={v:.3g}" for k, v in rep.items()))
    assert rep["loss_max_abs"] <= tol["loss"], rep
    if hasattr(orc, "pick_gap"):
        # every pick is the maximum or within the logit tolerance of it
        assert rep["argmax_worst_pick_gap"] <= tol["logit"], rep
    assert rep["gnorm_max_rel"] <= tol["g"], rep
    assert rep["scale_max_abs"] <= tol["g"], rep
    if check_weights:
        assert rep["W_rel_l2"] <= tol["w"], rep
        assert rep["D_rel_l2"] <= tol["dw"], rep
    return rep

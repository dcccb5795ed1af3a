"""Shared helpers of the GPU parity tests: seeded inputs, one GPU run, one oracle run, gates.

Gates (element by element on the same seeded inputs):
  bf16 mode: per-token loss |delta| <= 1e-2; final fast weights relative L2 <= 2e-2; the
             accumulated update D = W - W0 relative L2 <= 2e-2; per-chunk grad norm
             relative error <= 1e-2.
  fp32 mode: the same at 1e-4 (grad norm 1e-5).
  argmax:    exact, except at a near tie: a token whose GPU pick differs from the oracle's
             is excused only if the oracle's own logit at the GPU's pick is within tau_t of
             the oracle's maximum, with the scale-aware bound
                 tau_t = 8 u ||y_t||_2 rho / sqrt(d),
             y_t the hidden row that feeds the LM head, rho the RMS row norm of E_out and
             u = 2^-8 (bf16 operands) or 2^-20 (fp32): an estimate of the logit error that
             rounding y_t alone causes, with room. Excused tokens are counted and logged,
             and their number is bounded (at most 5% of the compared tokens).
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
# unit roundoff of the operands the LM head reads, for the near-tie bound tau_t
ARGMAX_U = {"bf16": 2.0 ** -8, "fp32": 2.0 ** -20}
ARGMAX_EXCUSED_FRAC = 0.05
TOPK = 16

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


class LogitRecord:
    """Per scored token: the oracle's TOPK largest logits (values, ids; descending, lowest id
    first among equal values) and the L2 norm of the hidden row that fed the LM head."""

    def __init__(self):
        self.vals, self.ids, self.hnorm = [], [], []

    def add(self, z: np.ndarray, h: np.ndarray):
        z = np.atleast_2d(z)
        h = np.atleast_2d(h)
        k = min(TOPK, z.shape[1])
        part = np.argpartition(-z, k - 1, axis=1)[:, :k]
        v = np.take_along_axis(z, part, axis=1)
        order = np.lexsort((part, -v), axis=1)
        self.ids.append(np.take_along_axis(part, order, axis=1))
        self.vals.append(np.take_along_axis(v, order, axis=1))
        self.hnorm.append(np.linalg.norm(h, axis=1))

    def arrays(self):
        return np.concatenate(self.vals), np.concatenate(self.ids), np.concatenate(self.hnorm)


def argmax_gate(am_gpu: np.ndarray, am_orc: np.ndarray, top_vals: np.ndarray, top_ids: np.ndarray,
                hnorm: np.ndarray, rho: float, d: int, precision: str, label: str = ""):
    """Assert the argmax gate (see the module docstring); return (mismatches, near ties, worst
    gap / tau). A GPU pick outside the oracle's TOPK largest logits is never excused."""
    n = len(am_gpu)
    tau = 8.0 * ARGMAX_U[precision] * hnorm[:n] * rho / math.sqrt(d)
    mism = np.flatnonzero(am_gpu[:n] != am_orc[:n])
    gaps = np.full(len(mism), np.inf)
    for j, t in enumerate(mism):
        hit = np.flatnonzero(top_ids[t] == am_gpu[t])
        if len(hit):
            gaps[j] = top_vals[t, 0] - top_vals[t, hit[0]]
    near = int(np.sum(top_vals[:n, 0] - top_vals[:n, 1] <= tau)) if top_vals.shape[1] > 1 else 0
    worst = float(np.max(gaps / tau[mism])) if len(mism) else 0.0
    log(f"[argmax {label} {precision}] tokens={n} excused={len(mism)} oracle near-ties(<=tau)={near} "
        f"worst gap/tau={worst:.3g} tau median={float(np.median(tau)) if n else 0.0:.3g}")
    assert worst <= 1.0, (label, "a GPU pick differs from the oracle's by more than tau_t", worst)
    assert len(mism) <= max(2, ARGMAX_EXCUSED_FRAC * n), (label, "too many excused near ties", len(mism), n)
    return len(mism), near, worst


def argmax_gate_rows(am_gpu: np.ndarray, z: np.ndarray, h: np.ndarray, E_out: np.ndarray, precision: str,
                     label: str = ""):
    """The argmax gate against whole oracle logit rows z (with the hidden rows h that fed the
    head); the oracle's pick is the first maximum of each row."""
    rec = LogitRecord()
    rec.add(z, h)
    vals, ids, hn = rec.arrays()
    return argmax_gate(np.asarray(am_gpu), np.argmax(np.atleast_2d(z), axis=1), vals, ids, hn,
                       rms_row_norm(E_out), np.atleast_2d(h).shape[1], precision, label)


def rms_row_norm(E: np.ndarray) -> float:
    E = np.asarray(E, dtype=np.float64)
    return float(np.sqrt(np.mean(np.sum(E * E, axis=1))))


def oracle_run(w, P, x, n_chunks: int, gpu_argmax=None, key=None):
    """fp64 oracle over the first n_chunks chunks. The result also carries, per scored token,
    the oracle's largest logits and the norm of the row that fed the head (for the argmax
    gate), and rho, the RMS row norm of E_out. gpu_argmax is accepted for old callers and
    ignored: every run records what the gate needs."""
    ck = None if key is None else (key, n_chunks)
    if ck is not None and ck in _ORACLE:
        return _ORACLE[ck]
    model = O.Model.from_workload(w)
    b = w.chunk
    rec = LogitRecord()
    res = O.run_ttt(model, P, x[:n_chunks * b + 1], n_chunks=n_chunks,
                    logit_probe=lambda i, z, h: rec.add(z, h))
    res.top_vals, res.top_ids, res.hnorm = rec.arrays()
    res.rho = rms_row_norm(P["E_out"])
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
    g_g = gpu["stats"][:n_chunks, 0]
    rep["gnorm_max_rel"] = float(np.max(np.abs(g_g - orc.grad_norm[:n_chunks]) /
                                        np.maximum(orc.grad_norm[:n_chunks], 1e-30)))
    rep["scale_max_abs"] = float(np.max(np.abs(gpu["stats"][:n_chunks, 1] - orc.scale[:n_chunks])))
    if check_weights:
        rep["W_rel_l2"] = max(rel_l2(gpu["W"][k], orc.weights[k]) for k in orc.weights)
        rep["D_rel_l2"] = max(rel_l2(gpu["D"][k], orc.delta[k]) for k in orc.delta)
    log(f"[parity {label} {precision} {n_chunks} chunks] " + " ".join(f"{k}={v:.3g}" for k, v in rep.items()))
    assert rep["loss_max_abs"] <= tol["loss"], rep
    rep["argmax_excused"], rep["argmax_near_ties"], rep["argmax_worst_gap_over_tau"] = argmax_gate(
        gpu["argmax"][:n], orc.argmax[:n], orc.top_vals, orc.top_ids, orc.hnorm, orc.rho, w.d_model,
        precision, label)
    assert rep["gnorm_max_rel"] <= tol["g"], rep
    assert rep["scale_max_abs"] <= tol["g"], rep
    if check_weights:
        assert rep["W_rel_l2"] <= tol["w"], rep
        assert rep["D_rel_l2"] <= tol["dw"], rep
    return rep

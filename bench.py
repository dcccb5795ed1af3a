#!/usr/bin/env python3
"""Throughput of the chunk-wise TTT inner loop on one MI355X.

One step = one full prefill of the workload's token stream through the HIP library: for
each chunk of b tokens, forward through the fast blocks, next-token CE through the frozen
LM head, backward to the fast weights, global-norm clip and SGD step; chunks in sequence.
Steps continue the same context (the fast state keeps learning), so no reset sits inside
the timed region.

Prints one JSON line on stdout; diagnostics go to stderr.
  python bench.py [--steps K] [--warmup W] [--workload s760m] [--no-cpu-baseline]
                  [--calibrate-copy]   (a 256 MiB device copy first: the reference kernel of
                                        known size for scaling the FETCH_SIZE / WRITE_SIZE
                                        counters in a rocprofv3 --pmc run of this script)

roofline.traffic comes from the committed counter summary profiles/traffic_<workload>.md
and is null unless that summary was taken on the current GEMM sources (sha256 match).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 2.5e15     # MI355X dense bf16 MFMA, flop/s
PEAK_FP32 = 157.3e12   # MI355X fp32 matrix, flop/s
PEAK_HBM = 8.0e12      # MI355X HBM3E, byte/s
METRIC = "TTT inner-loop tokens/s (fwd+bwd+update) at 1 GPU; % of bf16 MFMA peak"


PROFILE_PERIOD = 8
DECODE_PERIOD = 16
PEAK_HBM_GBS = 8000.0


def eprint(*a):
    print(*a, file=sys.stderr, flush=True)


def device_peak() -> dict:
    """The bf16 dense MFMA peak derived from the device itself: compute units x peak engine
    clock x 4096 flop per clock and CU (gfx950: a 32x32x16 bf16 MFMA per SIMD every 8 x 4 clocks,
    four SIMDs), beside the published 2.5 PFLOP/s."""
    import ctypes
    import torch
    cus = int(torch.cuda.get_device_properties(0).multi_processor_count)
    khz = None
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        v = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(v), 5, 0) == 0 and 500_000 <= v.value <= 5_000_000:
            khz = v.value  # hipDeviceAttributeClockRate: peak clock in kHz
    except OSError:
        pass
    out = {"cus": cus, "flop_per_clk_per_cu": 4096, "published_tflops": PEAK_BF16 / 1e12}
    if khz is not None:
        out["max_engine_clock_mhz"] = khz / 1e3
        out["device_tflops"] = cus * khz * 1e3 * 4096 / 1e12
    return out


def alg_flops_per_token(w) -> float:
    """Algorithmic flops per token: what the method must compute, no recompute.

    GELU blocks: forward 4dm per block; backward 8dm per block above the lowest (dA, G2,
    G1, dHn) and 6dm for the lowest (no dHn). SwiGLU with only W2 fast: forward 6dm,
    backward 2dm (G2). LM head: 2Vd logits + 2Vd for dY.
    """
    d, m, L, V = w.d_model, w.d_hidden, w.n_blocks, w.vocab
    if w.mlp == "gelu":
        blocks = 4 * d * m * L + (8 * d * m * (L - 1) + 6 * d * m if L > 0 else 0)
    else:
        blocks = 8 * d * m * L
    return float(blocks + 4 * V * d)


def kind_flops_per_chunk(w, kind: str) -> float:
    """Flops one chunk's launches of a GEMM kind perform (each counted once, no padding)."""
    b, d, m, V, L = w.chunk, w.d_model, w.d_hidden, w.vocab, w.n_blocks
    g = w.mlp == "gelu"
    table = {
        "ce_fwd": 2.0 * b * V * d,
        "ce_dy": 2.0 * b * V * d,
        "up": (2.0 if g else 4.0) * b * d * m * L,
        "down": 2.0 * b * d * m * L,
        "du": 2.0 * b * d * m * L if g else 0.0,
        "dw": (4.0 if g else 2.0) * b * d * m * L,
        "dhn": 2.0 * b * d * m * max(L - 1, 0) if g else 0.0,
    }
    return table.get(kind, 0.0)


# GEMM kinds whose launches use a kernel no other kind uses (so a per-kernel counter
# average is that kind's average); the epilogue type names the kernel.
KIND_KERNEL = {"up": "EpiGelu", "du": "EpiDU", "dw": "EpiGrad", "ce_fwd": "EpiCEPartial"}
GEMM_SOURCES = ["test_long_context_chunk_amd/csrc/gemm.h", "test_long_context_chunk_amd/csrc/gemm_inst.hip",
                "test_long_context_chunk_amd/csrc/common.h"]
ATTENTION_SOURCES = ["test_long_context_chunk_amd/csrc/attention.hip", "test_long_context_chunk_amd/csrc/common.h"]


def split_k(M: int, N: int, K: int, K2: int) -> int:
    """Split-K slabs the library gives a bf16 product on 256 x 128 tiles (256 workgroup slots,
    at least 4 K-slices of 64 per slab, at most 8 slabs): host-side accounting only."""
    tiles = -(-M // 256) * -(-N // 128)
    return max(1, min(256 // tiles, (K + K2) // 64 // 4, 8))


def hbm_kernel_bytes(w, kind: str) -> float:
    """Bytes one launch of an HBM-bound kernel kind moves (reads + writes), from the shapes; the
    split-K slabs the row kernels sum are counted. bf16 workloads (2-byte operands)."""
    b, d, m, V, L = w.chunk, w.d_model, w.d_hidden, w.vocab, w.n_blocks
    es = 2 if w.precision == "bf16" else 4
    comp = w.precision == "bf16"  # the bf16 loss compensation keeps rounding residuals
    nrec = -(-V // 64)
    if kind == "update":  # per fast tensor: G, D read and written, W0, Wop, WtT
        params = d * m
        return float(params * (es + 8 + es + es + es))
    if kind == "ce_prob":  # numerators read, dlogits written in place, one record per 64 columns
        return float(2 * b * V * es + b * nrec * 4 + 2 * b * 4)
    if kind == "gather":  # embedding rows in; residual, normed rows, their residual, scale out
        return float(b * 4 + b * d * es + b * d * 4 + b * d * es + (b * d * es if comp else 0) + b * 4)
    if kind == "residual":  # slabs and residual in; residual, next pre-norm (and residual) out
        S = split_k(b, d, m, m if es == 2 else 0)
        return float(S * b * d * 4 + b * d * 4 + b * d * 4 + b * d * es + (b * d * es if comp else 0) + b * 4)
    if kind == "norm_bwd":  # slabs, normed rows, scale, residual gradient in; gradient out (fp32, bf16)
        S = split_k(b, d, m, 0)
        return float(S * b * d * 4 + b * d * es + b * 4 + b * d * 4 + (b * d * es if comp else 0) + b * d * 4 +
                     b * d * es)
    if kind == "dy_sum":  # slabs in; dY (fp32, bf16) out; H and its bf16 copy for the compensation
        S = split_k(b, d, V, 0)
        return float(S * b * d * 4 + b * d * 4 + b * d * es + ((b * d * 4 + b * d * es) if comp else 0))
    return 0.0


HBM_KINDS = ["update", "ce_prob", "gather", "residual", "norm_bwd", "dy_sum"]


def sources_sha256(sources) -> str:
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def gemm_sources_sha256() -> str:
    return sources_sha256(GEMM_SOURCES)


def measured_traffic(workload: str, kind: str):
    """HBM bytes per launch of `kind` from the committed counter summary, or None.

    The summary holds lines `traffic <kind> <kernel> fetch_kib=<F> write_kib=<W> bytes=<B>`
    (counters per dispatch, already scaled by the copy-kernel factors) and the sha256 of
    the GEMM sources the counters were taken on; a different sha means the kernels changed
    since, and the figure no longer applies.
    """
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    # the attention kernels live in their own sources, recorded on a line of their own
    label, sha = ("attention", sources_sha256(ATTENTION_SOURCES)) if kind == "attn" else ("gemm", gemm_sources_sha256())
    m = re.search(rf"^{label}_sources_sha256:\s*([0-9a-f]{{64}})", text, re.M)
    if not m or m.group(1) != sha:
        return None
    m = re.search(rf"^traffic {re.escape(kind)} \S+ fetch_kib=\S+ write_kib=\S+ bytes=(\S+)", text, re.M)
    return float(m.group(1)) if m else None


def calibrate_copy():
    """A plain device-to-device copy of 256 MiB, three times (for counter scaling)."""
    import torch
    n = 64 << 20
    src = torch.ones(n, device="cuda", dtype=torch.float32)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    eprint("[bench] calibration copy: 3 x 268435456 bytes read + written")
    del src, dst


def cpu_cores() -> int:
    """Threads the oracle's numpy BLAS runs with (the host cores it uses)."""
    try:
        from threadpoolctl import threadpool_info
        return int(max((i.get("num_threads", 1) for i in threadpool_info()), default=1))
    except Exception:
        return os.cpu_count() or 1


def cpu_baseline(w, P, x, n_chunks: int):
    """The fp64 oracle, as it stands, on the first n_chunks chunks of the same stream."""
    import numpy as np
    import oracle as O
    threads = cpu_cores()
    model = O.Model.from_workload(w)
    t0 = time.perf_counter()
    O.run_ttt(model, P, x[:n_chunks * w.chunk + 1], n_chunks=n_chunks)
    dt = time.perf_counter() - t0
    return {"value": n_chunks * w.chunk / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {n_chunks} chunks ({n_chunks * w.chunk} tokens) of the same stream, fp64 numpy, "
                      f"{dt:.1f} s"}


def decode_bytes_per_token(w) -> float:
    """Algorithmic HBM bytes of one decoded token: one copy, in the workload's precision, of
    every weight the forward reads (the fast tensors as W = W0 + D), plus the LM head; with the
    fuller block also the static MLP, q|k|v and Wo, and one copy of the keys and values of a full
    window."""
    es = 2 if w.precision == "bf16" else 4
    dm = w.d_model * w.d_hidden * es
    per_block = (2 * dm if w.mlp == "gelu" else 3 * dm)
    ms = getattr(w, "static_hidden", 0)
    per_block += 2 * w.d_model * ms * es
    if getattr(w, "swa_window", 0) > 0:
        per_block += 4 * w.d_model * w.d_model * es + 2 * w.swa_window * w.d_model * es
    return float(w.n_blocks * per_block + w.vocab * w.d_model * es)


def decode_impl_bytes_per_token(w) -> float:
    """What this implementation reads per decoded token: the bf16 fast tensors as two segments
    (W0 and rn(D)); with attention, the keys and values in one half-precision copy, as the
    method's own bytes count them."""
    es = 2 if w.precision == "bf16" else 4
    segs = 2 if w.precision == "bf16" else 1
    dm = w.d_model * w.d_hidden * es
    per_block = (segs * dm if w.mlp == "gelu" else 2 * dm) + segs * dm
    ms = getattr(w, "static_hidden", 0)
    per_block += 2 * w.d_model * ms * es
    if getattr(w, "swa_window", 0) > 0:
        per_block += 4 * w.d_model * w.d_model * es + 2 * w.swa_window * w.d_model * 2
    return float(w.n_blocks * per_block + w.vocab * w.d_model * es)


def decode_bench(ctx, w, x, P, cpu: bool) -> dict:
    """Decode one chunk's worth of tokens (b predictions and the chunk's step) after the timed
    prefill steps, one token per call of the product path; the one-row products are traced
    with events in every DECODE_PERIOD-th token."""
    import numpy as np
    import torch
    b = w.chunk
    T = w.n_tokens
    ids = np.concatenate([[x[T]], x[1:b + 1]]).astype(np.int32)
    tok = torch.from_numpy(ids).cuda()
    ctx.decode(tok)  # warm-up: one full decoded chunk
    torch.cuda.synchronize()
    ctx.profile(["dec_gemv"], period=DECODE_PERIOD)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ctx.decode(tok)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    prof = ctx.profile_read()
    ctx.profile([])
    gemv_ms, gemv_n = prof.get("dec_gemv", (0.0, 0))
    # per block: up and down, the static MLP's two, q|k|v and Wo; then the LM head
    per_block = 2 + (2 if getattr(w, "static_hidden", 0) > 0 else 0) + (2 if getattr(w, "swa_window", 0) > 0 else 0)
    per_tok = per_block * w.n_blocks + 1
    traced_tokens = max(gemv_n // per_tok, 1)
    bpt = decode_bytes_per_token(w)
    impl_bpt = decode_impl_bytes_per_token(w)
    gemv_s_per_tok = gemv_ms * 1e-3 / traced_tokens
    # the products are ~10 us launches, so an event bracket around each adds a large share of
    # dispatch time: the roofline uses the whole token's time instead (a lower bound on the
    # kernels' bandwidth), and the bracketed figure is reported beside it
    achieved = bpt / (dt / b) / 1e9
    att = getattr(w, "swa_window", 0) > 0
    out = {
        "metric": "decode tokens/s (one prediction per token, the TTT step every chunk)",
        "value": b / dt, "unit": "tokens/s", "us_per_token": dt / b * 1e6, "tokens": b,
        "roofline": {"bound": "hbm", "kernel": "decode token (one-row products + CE merge" +
                     (" + attention over a full window)" if att else ")"),
                     "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                     "traffic": None, "bytes_per_token": bpt,
                     "impl_bytes_per_token": impl_bpt,
                     "impl_achieved": impl_bpt / (dt / b) / 1e9,
                     "gemv_event_us_per_token": gemv_s_per_tok * 1e6, "gemv_launches_traced": gemv_n,
                     "kernel_name": "k_gemv"},
    }
    if cpu:
        import oracle as O
        n = 32
        model = O.Model.from_workload(w)
        t0 = time.perf_counter()
        O.decode_ttt(model, P, ids[:n + 1])
        cdt = time.perf_counter() - t0
        threads = cpu_cores()
        out["cpu_baseline"] = {"value": n / cdt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
                               "sample": f"{n} decoded tokens of the same shape, fp64 numpy, {cdt:.1f} s"}
    return out


def fwd_flops_per_token(w) -> float:
    """Algorithmic flops of one token's forward pass (the blocks and the LM head)."""
    d, m, L, V = w.d_model, w.d_hidden, w.n_blocks, w.vocab
    blocks = (4 if w.mlp == "gelu" else 6) * d * m * L
    return float(blocks + 2 * V * d)


def settle_bench(ctx, w, x, P, cpu: bool, n: int = 3) -> dict:
    """The Settlement rule on one candidate chunk with a one-chunk held-out passage, timed over
    n settlements after a warm-up one: two passage evaluations and one training chunk each."""
    import numpy as np
    import torch
    b = w.chunk
    cand = torch.from_numpy(x[:b + 1].astype(np.int32)).cuda()
    q = torch.from_numpy(x[b:2 * b + 1].astype(np.int32)).cuda()
    ctx.settle(cand, q)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n):
        ctx.settle(cand, q)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / n
    flops = 2 * b * fwd_flops_per_token(w) + b * alg_flops_per_token(w)
    achieved = flops / dt / 1e12
    peak = (PEAK_BF16 if w.precision == "bf16" else PEAK_FP32) / 1e12
    out = {
        "metric": "Settlement candidates/s (one candidate chunk, one-chunk held-out passage)",
        "value": 1.0 / dt, "unit": "candidates/s", "ms_per_candidate": dt * 1e3, "candidates": n,
        "roofline": {"bound": "mfma", "kernel": "whole rule (2 passage evaluations + 1 training chunk)",
                     "achieved": achieved, "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak,
                     "traffic": None, "alg_flops_per_candidate": flops},
    }
    if cpu:
        import oracle as O
        model = O.Model.from_workload(w)
        t0 = time.perf_counter()
        O.settle_step(model, P, x[:b + 1], x[b:2 * b + 1])
        cdt = time.perf_counter() - t0
        threads = cpu_cores()
        out["cpu_baseline"] = {"value": 1.0 / cdt, "unit": "candidates/s", "cores": int(threads), "kind": "oracle",
                               "sample": f"one candidate at the same shape, fp64 numpy, {cdt:.1f} s"}
    return out


def batch_bench(w, P, seed: int, streams: int, steps: int, warmup: int) -> dict:
    """Several independent streams advanced by one batched context: every step runs the full
    stream of each of `streams` token streams (seeds seed .. seed + streams - 1) in lockstep,
    chunk i of all streams in one chunk step. Reports whole-job tokens/s over all streams and
    the roofline of the dominant GEMM kind (grouped over the streams)."""
    import numpy as np
    import torch
    import ttt_workloads as W
    import test_long_context_chunk_amd as ttt
    T = w.n_tokens
    dev = {k: ttt.to_device(v, w.precision) for k, v in P.items()}
    ctx = ttt.TTT.from_workload(w, dev, max_tokens=T * (warmup + steps + 1), streams=streams)
    del dev
    tok = np.stack([W.token_stream(w, seed + z).astype(np.int32) for z in range(streams)])
    tok = torch.from_numpy(tok).cuda()
    torch.cuda.synchronize()
    ctx.profile(ttt._binding.KERNEL_KINDS)
    ctx.prefill_batch(tok)
    prof = ctx.profile_read()
    ctx.profile([])
    gemm_kinds = {k: v for k, v in prof.items() if kind_flops_per_chunk(w, k) > 0}
    dom = max(gemm_kinds, key=lambda k: gemm_kinds[k][0])
    for _ in range(warmup):
        ctx.prefill_batch(tok)
    torch.cuda.synchronize()
    ctx.profile([dom], period=PROFILE_PERIOD)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        ctx.prefill_batch(tok)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    dprof = ctx.profile_read()
    ctx.profile([])
    status = ctx.sync()
    last = [ctx.token_losses(T * warmup + T, 8, s=z).cpu().numpy() for z in (0, streams - 1)]
    ctx.close()
    if status != 0 or not all(np.all(np.isfinite(v)) for v in last):
        eprint(f"[bench] batched streams: status {status} or non-finite losses")
        sys.exit(1)
    value = steps * T * streams / elapsed
    dom_ms, dom_n = dprof.get(dom, (0.0, 0))
    launches_per_chunk = max(1, round(prof[dom][1] / w.n_chunks))
    per_launch = streams * kind_flops_per_chunk(w, dom) / launches_per_chunk
    avg_s = dom_ms * 1e-3 / max(dom_n, 1)
    achieved = per_launch / avg_s / 1e12 if avg_s > 0 else 0.0
    peak = (PEAK_BF16 if w.precision == "bf16" else PEAK_FP32) / 1e12
    eprint(f"[bench] {streams} batched streams: {value:.0f} tokens/s, {elapsed / steps * 1e3:.1f} ms per step; "
           f"{dom} {avg_s * 1e6:.1f} us per launch, {achieved:.1f} TFLOP/s")
    return {
        "metric": "TTT inner-loop tokens/s over independent streams advanced together (all streams)",
        "value": value, "unit": "tokens/s", "streams": streams, "tokens_per_step": T * streams,
        "ms_per_step": elapsed / steps * 1e3, "steps": steps, "warmup": warmup,
        "frac_of_bf16_peak": value * alg_flops_per_token(w) / PEAK_BF16,
        "roofline": {
            "bound": "mfma", "kernel": dom, "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
            "frac": achieved / peak, "traffic": None, "alg_flops_per_launch": per_launch,
            "avg_launch_us": avg_s * 1e6, "launches": dom_n,
            "kernel_name": KIND_KERNEL.get(dom, "EpiStoreF32"),
        },
    }


def visible_keys(w, pos: int, n: int) -> int:
    """Keys the attention reads for the n rows from position pos: sum of min(window, p + 1)."""
    k = w.swa_window
    total = 0
    for p in range(pos, pos + n):
        total += min(k, p + 1)
    return total


def e2e_flops_per_step(w, pos: int = 0) -> dict:
    """Algorithmic flops of one step over T tokens of the fuller block from stream position
    pos (attention, static MLP, fast MLP per block), no recompute: per token and block, the
    attention projections 8d^2 forward and (blocks above the lowest) 8d^2 backward, the
    attention core 4d per visible key forward and 4d per visible key plus 4d per visible key
    of the chunk backward; the static MLP 4 d m_s forward and 4 d m_s backward above the
    lowest; the fast MLP and LM head as in the plain step. The timed steps continue the stream
    past its first window, where every query sees the whole window."""
    d, ms, L, T, b = w.d_model, w.static_hidden, w.n_blocks, w.n_tokens, w.chunk
    keys = visible_keys(w, pos, T)
    chunk_keys = 0  # visible keys that lie in the query's own chunk
    for i in range(T // b):
        for q in range(b):
            chunk_keys += min(w.swa_window, q + 1)
    proj = 8.0 * d * d * T * (L + (L - 1))
    core_fwd = 4.0 * d * keys * L
    core_bwd = (4.0 * d * keys + 4.0 * d * chunk_keys) * (L - 1)
    static = 4.0 * d * ms * T * (L + (L - 1))
    return dict(total=alg_flops_per_token(w) * T + proj + core_fwd + core_bwd + static, attn_fwd=core_fwd)


def e2e_bench(steps: int, warmup: int, seed: int, cpu: bool, cpu_chunks: int = 2, decode: bool = True) -> dict:
    """The fuller TTT-E2E block at the 760M shape: frozen sliding-window attention (window 8K,
    12 heads) and a frozen static MLP before each of the 3 fast MLPs; one stream, whole-stream
    steps. Roofline: the attention forward kernel, traced on every chunk."""
    import numpy as np
    import torch
    import ttt_workloads as W
    import test_long_context_chunk_amd as ttt
    w = W.preset("e2e760m")
    T = w.n_tokens
    P = W.init_weights(w, seed)
    x = W.token_stream(w, seed)
    dev = {k: ttt.to_device(v, w.precision) for k, v in P.items()}
    ctx = ttt.TTT.from_workload(w, dev, max_tokens=T * (warmup + steps + 1) + 2 * w.chunk)
    del dev
    tok = torch.from_numpy(x.astype(np.int32)).cuda()
    torch.cuda.synchronize()
    ctx.profile(ttt._binding.KERNEL_KINDS)
    ctx.prefill(tok)
    prof = ctx.profile_read()
    ctx.profile([])
    tot = sum(v[0] for v in prof.values())
    eprint(f"[bench] e2e760m per-kind time of one traced step ({tot:.1f} ms with events):")
    for k, (ms, n) in sorted(prof.items(), key=lambda kv: -kv[1][0])[:8]:
        eprint(f"  {k:10s} {ms:9.3f} ms {100 * ms / tot:5.1f}%  {n:5d} launches")
    for _ in range(warmup):
        ctx.prefill(tok)
    torch.cuda.synchronize()
    ctx.profile(["attn"], period=1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        ctx.prefill(tok)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    aprof = ctx.profile_read()
    ctx.profile([])
    dec = decode_bench(ctx, w, x, P, cpu=cpu) if decode else None
    status = ctx.sync()
    last = ctx.token_losses(T * (warmup + 1), 8).cpu().numpy()
    ctx.close()
    if status != 0 or not np.all(np.isfinite(last)):
        eprint(f"[bench] e2e760m: status {status} or non-finite losses")
        sys.exit(1)
    fl = e2e_flops_per_step(w, T * (warmup + 1))  # the timed steps' positions
    value = steps * T / elapsed
    a_ms, a_n = aprof.get("attn", (0.0, 0))
    per_launch = fl["attn_fwd"] / max(1, w.n_chunks * w.n_blocks)
    avg_s = a_ms * 1e-3 / max(a_n, 1)
    achieved = per_launch / avg_s / 1e12 if avg_s > 0 else 0.0
    eprint(f"[bench] e2e760m: {value:.0f} tokens/s, {elapsed / steps * 1e3:.1f} ms per step; attention forward "
           f"{avg_s * 1e6:.1f} us per launch, {achieved:.1f} TFLOP/s (algorithmic)")
    out = {
        "metric": "TTT inner-loop tokens/s with the fuller block (sliding-window attention + static MLP + fast MLP)",
        "value": value, "unit": "tokens/s", "ms_per_step": elapsed / steps * 1e3, "steps": steps, "warmup": warmup,
        "config": {"workload": f"e2e760m: 3 x [SWA window {w.swa_window}, {w.swa_heads} heads; static MLP "
                               f"m_s={w.static_hidden}; fast GELU MLP m={w.d_hidden}], d={w.d_model}, V={w.vocab}",
                   "tokens_per_step": T, "chunk": w.chunk},
        "frac_of_bf16_peak": value * fl["total"] / T / PEAK_BF16,
        "alg_flops_per_token": fl["total"] / T,
        "roofline": {
            "bound": "mfma", "kernel": "attn", "achieved": achieved, "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s",
            "frac": achieved * 1e12 / PEAK_BF16, "traffic": measured_traffic(w.name, "attn"),
            "alg_flops_per_launch": per_launch, "avg_launch_us": avg_s * 1e6, "launches": a_n, "kernel_name": "k_swa_fwd",
            "note": "half-precision q, k, v and p, one MFMA per product step: executed flops equal the "
                    "algorithmic ones (no recompute)",
        },
    }
    if dec is not None:
        out["decode"] = dec
    if cpu:
        import oracle as O
        eprint(f"[bench] timing the fp64 oracle on {cpu_chunks} full-window chunks of e2e760m ...")
        model = O.Model.from_workload(w)
        Pf = O.as_f64(P)
        rng = np.random.default_rng(seed)
        # a cache of window - 1 positions per block, as every chunk of the timed steps sees: its
        # keys and values are synthetic (their values do not change the oracle's work)
        kv = [dict(k=rng.standard_normal((w.swa_window - 1, w.d_model)),
                   v=rng.standard_normal((w.swa_window - 1, w.d_model))) for _ in range(w.n_blocks)]
        b = w.chunk
        t0 = time.perf_counter()
        for i in range(cpu_chunks):
            _, st, _ = O.chunk_loss_and_grads(model, Pf, x[i * b:i * b + b], x[i * b + 1:i * b + b + 1], kv=kv)
            kv = st["kv"]
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": cpu_chunks * b / dt, "unit": "tokens/s", "cores": cpu_cores(),
                               "kind": "oracle",
                               "sample": f"{cpu_chunks} chunks ({cpu_chunks * b} tokens) at a full window: the oracle's "
                                         f"chunk step (forward, loss, gradients) with a cache of {w.swa_window - 1} "
                                         f"earlier positions per block, fp64 numpy, {dt:.1f} s"}
    return out


def workload_bench(w, P, x, steps: int, warmup: int, keep_ctx: bool = False, seed: int = 0):
    """Whole-stream prefill steps of workload w: tokens/s, the fraction of the bf16 peak in
    algorithmic flops, the dominant GEMM kind's roofline (HIP events on the library stream, every
    PROFILE_PERIOD-th chunk of the timed steps), and the bandwidth of the HBM-bound kernel kinds
    (events around every launch of one untimed traced step)."""
    import numpy as np
    import torch
    import test_long_context_chunk_amd as ttt
    T = w.n_tokens
    eprint(f"[bench] workload {w.name}: V={w.vocab} d={w.d_model} m={w.d_hidden} L={w.n_blocks} "
           f"mlp={w.mlp} norm={w.norm} T={T} b={w.chunk} {w.precision}")
    dev = {k: ttt.to_device(v, w.precision) for k, v in P.items()}
    total_steps = warmup + steps + 2
    ctx = ttt.TTT.from_workload(w, dev, max_tokens=T * total_steps)
    del dev
    tok = torch.from_numpy(x.astype(np.int32)).cuda()
    torch.cuda.synchronize()

    # untimed: one step with every kernel kind traced -> breakdown and the dominant kind
    ctx.profile(ttt._binding.KERNEL_KINDS)
    ctx.prefill(tok)
    prof = ctx.profile_read()
    ctx.profile([])
    tot = sum(v[0] for k, v in prof.items() if k != "update")
    eprint(f"[bench] {w.name}: per-kind time of one traced step (events around every launch; the SGD steps run "
           f"beside the main stream and are listed apart):")
    for k, (ms, n) in sorted(prof.items(), key=lambda kv: -kv[1][0]):
        f = kind_flops_per_chunk(w, k) * w.n_chunks
        rate = f / (ms * 1e-3) / 1e12 if f > 0 and ms > 0 else 0.0
        by = hbm_kernel_bytes(w, k) * n
        bw = by / (ms * 1e-3) / 1e9 if by > 0 and ms > 0 else 0.0
        eprint(f"  {k:10s} {ms:9.3f} ms {100 * ms / tot if k != 'update' else 0.0:5.1f}%  {n:5d} launches  "
               f"{rate:8.1f} TFLOP/s {bw:8.1f} GB/s")
    hbm = {}
    for k in HBM_KINDS:
        ms, n = prof.get(k, (0.0, 0))
        by = hbm_kernel_bytes(w, k)
        if n > 0 and ms > 0 and by > 0:
            gbs = by * n / (ms * 1e-3) / 1e9
            hbm[k] = {"bytes_per_launch": by, "avg_launch_us": ms * 1e3 / n, "achieved": gbs, "peak": PEAK_HBM_GBS,
                      "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS, "launches": n}
    gemm_kinds = {k: v for k, v in prof.items() if kind_flops_per_chunk(w, k) > 0}
    dom = max(gemm_kinds, key=lambda k: gemm_kinds[k][0])

    for _ in range(warmup):
        ctx.prefill(tok)
    torch.cuda.synchronize()

    # timed: exactly `steps` steps; only the dominant kind is bracketed by events, in every
    # PROFILE_PERIOD-th chunk (each event costs a few microseconds of stream time)
    ctx.profile([dom], period=PROFILE_PERIOD)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        ctx.prefill(tok)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    dprof = ctx.profile_read()
    ctx.profile([])
    status = ctx.sync()
    if status != 0:
        eprint(f"[bench] library reported status {status}")
        sys.exit(1)
    losses = ctx.token_losses(T * (total_steps - steps - 2 + 1), 8).cpu().numpy()
    if not np.all(np.isfinite(losses)):
        eprint("[bench] non-finite losses")
        sys.exit(1)

    tokens_per_s = steps * T / elapsed
    fpt = alg_flops_per_token(w)
    dom_ms, dom_n = dprof.get(dom, (0.0, 0))
    # launches of that kind per chunk, from the untimed step where every chunk was traced
    launches_per_chunk = max(1, round(prof[dom][1] / w.n_chunks))
    per_launch = kind_flops_per_chunk(w, dom) / launches_per_chunk
    avg_s = dom_ms * 1e-3 / max(dom_n, 1)
    achieved = per_launch / avg_s / 1e12 if avg_s > 0 else 0.0
    peak = (PEAK_BF16 if w.precision == "bf16" else PEAK_FP32) / 1e12
    eprint(f"[bench] {w.name}: {tokens_per_s:.0f} tokens/s, {elapsed / steps * 1e3:.2f} ms per step; {dom} "
           f"{avg_s * 1e6:.1f} us per launch, {achieved:.1f} TFLOP/s")
    out = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": elapsed / steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.precision,
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: {w.n_blocks} x {'pre-RMSNorm ' if w.norm == 'rms' else ''}"
                        f"{'GELU' if w.mlp == 'gelu' else 'SwiGLU(W2 fast)'} block, d={w.d_model}, "
                        f"m={w.d_hidden}, V={w.vocab}",
            "tokens_per_step": T, "chunk": w.chunk, "lr": w.lr, "clip": w.clip,
            "stream": f"Zipf(1.1) + sparse Markov, seed {seed}",
        },
        "frac_of_bf16_peak": tokens_per_s * fpt / PEAK_BF16,
        "alg_flops_per_token": fpt,
        "roofline": {
            "bound": "mfma", "kernel": dom, "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
            "frac": achieved / peak, "traffic": measured_traffic(w.name, dom),
            "alg_flops_per_launch": per_launch, "avg_launch_us": avg_s * 1e6, "launches": dom_n,
            "kernel_name": KIND_KERNEL.get(dom, "EpiStoreF32"),
        },
        "hbm_kernels": hbm,
    }
    if keep_ctx:
        return out, ctx
    ctx.close()
    return out


# The other preset workloads (one block at d 768, three blocks at d 768, the In-Place shape),
# measured beside the headline: name, oracle chunks timed for their CPU baseline (about 2 - 10 s
# each on 16 host cores).
OTHER_WORKLOADS = [("single", 8), ("s125m", 16), ("inplace", 4)]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="s760m")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-chunks", type=int, default=10)
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-settle", action="store_true")
    ap.add_argument("--streams", type=int, default=8,
                    help="independent streams of the batched measurement (0: skip it)")
    ap.add_argument("--no-e2e", action="store_true", help="skip the fuller-block (attention) measurement")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads (single block, 125M-style stack, In-Place shape)")
    ap.add_argument("--only", choices=["batch", "e2e"], default=None,
                    help="run only that measurement and print its object as the line (for kernel traces)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        eprint("bench.py measures one GPU only: the library runs each token stream's inner loop on a "
               "single MI355X and has no multi-GPU path; run with --gpus 1.")
        sys.exit(2)

    import numpy as np
    import torch
    import ttt_workloads as W
    import test_long_context_chunk_amd as ttt

    if args.calibrate_copy:
        calibrate_copy()
    if args.only == "e2e":
        print(json.dumps(e2e_bench(args.steps, args.warmup, args.seed, cpu=not args.no_cpu_baseline,
                                   decode=not args.no_decode)), flush=True)
        return
    if args.only == "batch":
        wb = W.preset(args.workload)
        print(json.dumps(batch_bench(wb, W.init_weights(wb, args.seed), args.seed, args.streams, args.steps,
                                     args.warmup)), flush=True)
        return
    w = W.preset(args.workload)
    x = W.token_stream(w, args.seed)
    P = W.init_weights(w, args.seed)
    out, ctx = workload_bench(w, P, x, args.steps, args.warmup, keep_ctx=True, seed=args.seed)
    out["device_peak"] = device_peak()
    if not args.no_decode:
        out["decode"] = decode_bench(ctx, w, x, P, cpu=not args.no_cpu_baseline)
    if not args.no_settle:
        out["settle"] = settle_bench(ctx, w, x, P, cpu=not args.no_cpu_baseline)
    ctx.close()
    if args.streams > 0:
        out["batch"] = batch_bench(w, P, args.seed, args.streams, args.steps, args.warmup)
    if not args.no_e2e:
        out["e2e"] = e2e_bench(args.steps, args.warmup, args.seed, cpu=not args.no_cpu_baseline)
    if not args.no_configs:
        out["configs"] = {}
        for name, cchunks in OTHER_WORKLOADS:
            wo = W.preset(name)
            xo, Po = W.token_stream(wo, args.seed), W.init_weights(wo, args.seed)
            o = workload_bench(wo, Po, xo, args.steps, args.warmup, seed=args.seed)
            for key in ("metric", "n_gpus", "higher_is_better", "scaling", "vs_baseline", "data"):
                o.pop(key, None)
            if not args.no_cpu_baseline:
                eprint(f"[bench] timing the fp64 oracle on {cchunks} chunks of {name} ...")
                o["cpu_baseline"] = cpu_baseline(wo, Po, xo, cchunks)
            out["configs"][name] = o
    if not args.no_cpu_baseline:
        eprint(f"[bench] timing the fp64 oracle on {args.cpu_chunks} chunks ...")
        out["cpu_baseline"] = cpu_baseline(w, P, x, args.cpu_chunks)
        if "batch" in out:
            # the oracle runs streams one after another: its per-token rate is the same
            out["batch"]["cpu_baseline"] = out["cpu_baseline"]
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

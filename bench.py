#!/usr/bin/env python3
"""Benchmark of the multi-head attention path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole hot path over one batch of synthetic input.  The
default workload is the long-context causal self-attention where the n^2 term
dominates (B=2, n=8192, h=16, d=64, bf16, via mha_forward) -- the largest of the
five configurations that fit one GPU.  The same run also times the other four
(tiny fp32 encoder, base encoder with projections, base decoder with causal
mask, big cross-attention with projections) on the GPU only and reports them
under "configs".  Inputs are seeded N(0,1) / Xavier draws, resident in HBM
before timing; each step reads the next of several rotating input sets so that
caches cannot hold the batch between steps.  The K timed steps are issued twice,
replayed from HIP graphs and launched straight onto the stream; the step time
is that of the faster way (config.issue), and both are reported.

The training workloads (``--workload *_bwd``) time the backward pass instead:
dq, dk, dv from resident q, k, v, the forward output, its row statistic and an
N(0,1) output gradient, via mha_backward (mha_backward_gqa when the key/value
heads are shared).

Prints one JSON line: whole-job throughput (algorithmic TFLOP/s), tokens/s, the
roofline of the dominant kernel (its time measured with HIP events around it on
the launch stream) and the fp64 oracle timed on the host as a CPU baseline
(headline workload only).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import pathlib
import sys
import time

import numpy as np

ROOT = pathlib.Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "MHA fwd TFLOP/s + % bf16 MFMA peak (and HBM GB/s); tokens/s, 1 GPU"
PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}  # dense MFMA bf16/f16; fp32 vector
PEAK_HBM_GBPS = 8000.0
ES = {"bf16": 2, "f16": 2, "f32": 4}
TRAFFIC_FILE = ROOT / "profiles" / "traffic.json"
# The five configurations of the benchmark; the headline is the largest that fits one GPU.
CONFIGS = ("tiny_encoder_f32", "base_encoder_proj", "base_decoder_causal", "big_cross_proj", "long_causal")
HEADLINE = "long_causal"
CSRC = ROOT / "transformer_head_scaled_softmax_amd" / "csrc"
KERNEL_SOURCES = {"qkv_projection": ["gemm_mfma.hip", "mfma_util.h"],
                  "attention": ["attn_mfma.hip", "mfma_util.h"],
                  "qkv_attention": ["proj_attn.hip", "mfma_util.h"],
                  "out_projection": ["gemm_mfma.hip", "mfma_util.h"], "attention_f32": ["attn_f32.hip"],
                  "decode": ["decode_mfma.hip", "mfma_util.h"], "decode_combine": ["decode_mfma.hip", "mfma_util.h"],
                  "out_projection_ln": ["gemm_mfma.hip", "mfma_util.h"], "ln_rows": ["gemm_mfma.hip", "mfma_util.h"],
                  "bwd_dq": ["bwd_mfma.hip", "mfma_util.h"], "bwd_dkdv": ["bwd_mfma.hip", "mfma_util.h"],
                  "bwd_fused": ["bwd_mfma.hip", "mfma_util.h"]}
KERNEL_SYMBOLS = {"qkv_projection": "gemm_mfma_kernel", "attention": ("attn_mfma_kernel", "attn_short_kernel"),
                  "qkv_attention": "proj_attn_kernel", "out_projection": "gemm_mfma_kernel",
                  "attention_f32": "attn_f32_kernel", "decode": "decode_mfma_kernel",
                  "decode_combine": "decode_combine_kernel", "out_projection_ln": "gemm_mfma_kernel",
                  "ln_rows": "ln_rows_kernel", "bwd_dq": "bwd_dq_kernel", "bwd_dkdv": "bwd_dkdv_kernel",
                  "bwd_fused": "bwd_short_kernel"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# Algorithmic work (visible scores only; padded or masked work is not counted).

def visible_counts(w, lens):
    """Number of visible (query, key) pairs per (b, h)."""
    Ls = np.full(w.B, w.Nk) if lens is None else np.clip(lens, 0, w.Nk)
    i = np.arange(w.Nq)
    tot = 0
    for L in Ls:
        tot += int(np.minimum(L, i + 1).sum()) if w.mask == 1 else int(L) * w.Nq
    return tot * w.H


def attention_flops(w, lens):
    return 4.0 * w.d * visible_counts(w, lens)  # 2d for q.k, 2d for p*v per visible pair


def attention_bytes(w, lens):
    es = ES[w.dtype]
    Ls = np.full(w.B, w.Nk) if lens is None else np.clip(lens, 0, w.Nk)
    qo = 2 * w.B * w.H * w.Nq * w.d * es
    kv = 2 * int(Ls.sum()) * w.H * w.d * es
    return qo + kv + (0 if lens is None else 4 * w.B)


def decode_visible(w, lens):
    """Visible (query, cache slot) pairs of one decoding step, over all query heads:
    query i of Nq sees slots j <= L - Nq + i under the causal mask, all L otherwise."""
    Ls = np.full(w.B, w.Nk) if lens is None else np.clip(lens, 0, w.Nk)
    i = np.arange(w.Nq)
    tot = 0
    for L in Ls:
        tot += int(np.clip(L - w.Nq + i + 1, 0, None).sum()) if w.mask == 1 else int(L) * w.Nq
    return tot * w.H


def decode_work(w, lens, nsplit):
    """(flops, bytes) per launch of the decoding kernel and of the combining
    kernel.  Bytes: the new queries, the filled cache slots of every cache head
    (read once whatever the head grouping), the fill lengths, and the output rows
    (written by the combining kernel when the caches are cut into chunks)."""
    es = ES[w.dtype]
    Ls = np.full(w.B, w.Nk) if lens is None else np.clip(lens, 0, w.Nk)
    qo = w.B * w.H * w.Nq * w.d * es
    kv = 2 * int(Ls.sum()) * w.kv_heads * w.d * es
    lb = 0 if lens is None else 4 * w.B
    f = 4.0 * w.d * decode_visible(w, lens)
    if nsplit > 1:
        return {"decode": (f, qo + kv + lb), "decode_combine": (0.0, qo + lb)}
    return {"decode": (f, 2 * qo + kv + lb)}


def backward_work(w, lens):
    """(flops, bytes) per launch of the two backward kernels, and the step's
    algorithmic FLOPs.  Per visible (query, key) pair the gradients need five
    products of 2d FLOPs: S (recomputed; the weights are not stored), dP, dV,
    dQ and dK -- the step's count.  The dQ kernel forms S, dP and dQ (6d), the
    dK/dV kernel S, dP, dV and dK (8d).  Bytes: the dQ kernel reads q, dout,
    out, lse and the visible rows of k and v and writes dq and D; the dK/dV
    kernel reads k, v (visible rows), q, dout, lse and D and writes dk, dv.
    Shared key/value heads count once.  The single-launch kernel of short
    problems does both parts' products (14d) and keeps D on chip."""
    es = ES[w.dtype]
    pairs = visible_counts(w, lens)
    Ls = np.full(w.B, w.Nk) if lens is None else np.clip(lens, 0, w.Nk)
    qrow = w.B * w.H * w.Nq * w.d * es
    krow = w.B * w.kv_heads * w.Nk * w.d * es
    kvis = 2 * int(Ls.sum()) * w.kv_heads * w.d * es
    stat = w.B * w.H * w.Nq * 4
    lb = 0 if lens is None else 4 * w.B
    dq = (6.0 * w.d * pairs, 3 * qrow + stat + kvis + qrow + stat + lb)
    dkdv = (8.0 * w.d * pairs, kvis + 2 * qrow + 2 * stat + 2 * krow + lb)
    # one launch for both parts (sentence-length problems): D stays on chip
    fused = (14.0 * w.d * pairs, 3 * qrow + stat + kvis + qrow + 2 * krow + lb)
    return {"bwd_dq": dq, "bwd_dkdv": dkdv, "bwd_fused": fused}, 10.0 * w.d * pairs


def projection_flops(w):
    D, HD, HKV = w.D, w.H * w.d, w.kv_heads * w.d  # HKV: width of the (shared) K and V projections
    qkv = 2.0 * w.B * (w.Nq * D * HD + 2 * w.Nk * D * HKV)
    out = 2.0 * w.B * w.Nq * HD * D
    return qkv, out


def proj_path_bytes(w, lens):
    """Inputs + weights + output of the whole projection path (the norm's scale
    and shift with it; x_q, its residual, is read once)."""
    es = ES[w.dtype]
    D, HD, HKV = w.D, w.H * w.d, w.kv_heads * w.d
    x = w.B * w.Nq * D + (w.B * w.Nk * D if w.cross else 0)
    weights = (HD + 2 * HKV) * D + D * HD + (2 * D if w.ln else 0)
    return (x + weights + w.B * w.Nq * D) * es + (0 if lens is None else 4 * w.B)


def stage_work(w, lens):
    """(flops, bytes) per launch of each kernel of the projection path: the
    unfused plan's three kernels and the fused plan's projection+attention
    kernel (whose bytes are x, the three input weights, the head outputs it
    writes and the key lengths)."""
    es = ES[w.dtype]
    D, HD, HKV = w.D, w.H * w.d, w.kv_heads * w.d
    qkv_f, out_f = projection_flops(w)
    x_bytes = (w.B * w.Nq * D + (w.B * w.Nk * D if w.cross else 0)) * es
    qkv_b = x_bytes + (HD + 2 * HKV) * D * es + (w.B * w.Nq * HD + 2 * w.B * w.Nk * HKV) * es
    out_b = (w.B * w.Nq * HD + D * HD + w.B * w.Nq * D) * es
    fused_b = x_bytes + (HD + 2 * HKV) * D * es + w.B * w.Nq * HD * es + (0 if lens is None else 4 * w.B)
    rows = w.B * w.Nq * D * es
    return {"qkv_projection": (qkv_f, qkv_b),
            "attention": (attention_flops(w, lens), attention_bytes(w, lens)),
            "qkv_attention": (qkv_f + attention_flops(w, lens), fused_b),
            "out_projection": (out_f, out_b),
            # with the norm, the projection's epilogue also reads the residual rows and
            # stores per-row tile statistics; the second pass reads the rows and the
            # statistics and writes the rows
            "out_projection_ln": (out_f, out_b + rows + w.B * w.Nq * ((D + 63) // 64) * 8),
            "ln_rows": (0.0, 2 * rows + w.B * w.Nq * ((D + 63) // 64) * 8 + 2 * D * es)}


# ---------------------------------------------------------------------------
# HIP events through the runtime's C API (torch's events only see torch's stream
# objects; these are recorded by the library on the launch stream).

class Hip:
    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        st = self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b)
        assert st == 0, f"hipEventElapsedTime failed ({st})"
        return ms.value

    def destroy(self, e):
        self.lib.hipEventDestroy(e)


# ---------------------------------------------------------------------------

def traffic_for(kernel_key: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None if
    absent or taken on a different version of the kernel's source."""
    if not TRAFFIC_FILE.exists():
        return None
    data = json.loads(TRAFFIC_FILE.read_text())
    ent = data.get(f"{workload}:{kernel_key}")
    if not ent:
        return None
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(kernel_key, []):
        h.update((CSRC / f).read_bytes())
    if ent.get("source_sha256") != h.hexdigest():
        return None
    return ent["fetch_bytes"] + ent["write_bytes"]


def roofline(kind_flops, kind_bytes, seconds, dtype, kernel_key, workload):
    ai = kind_flops / kind_bytes
    ridge = PEAK_TFLOPS[dtype] * 1e12 / (PEAK_HBM_GBPS * 1e9)
    if ai >= ridge:
        ach = kind_flops / seconds / 1e12
        peak = PEAK_TFLOPS[dtype]
        bound, unit = ("mfma" if dtype != "f32" else "alu"), "TFLOP/s"
    else:
        ach = kind_bytes / seconds / 1e9
        peak, bound, unit = PEAK_HBM_GBPS, "hbm", "GB/s"
    return {"bound": bound, "achieved": round(ach, 3), "peak": peak, "unit": unit,
            "frac": round(ach / peak, 4), "traffic": traffic_for(kernel_key, workload),
            "kernel": kernel_key, "algorithmic_flops": kind_flops, "algorithmic_bytes": kind_bytes}


def host_cpu() -> dict:
    """The host's logical CPU count, the CPUs this process may run on, and the
    CPU model name."""
    import os
    model = None
    try:
        for line in pathlib.Path("/proc/cpuinfo").read_text().splitlines():
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        affinity = os.cpu_count()
    return {"host_logical_cpus": os.cpu_count(), "affinity_cpus": affinity, "cpu_model": model}


def cpu_baseline(w, inp_sets, seconds_target):
    """Time the fp64 oracle on whole batches of the same workload (long sequences:
    sampled rows) until about ``seconds_target`` seconds of CPU work.  ``cores``
    is the number of threads the oracle ran on: every CPU this process may use,
    at most 16 (the CPU share of one GPU on the test machines)."""
    import oracle
    threads = oracle.default_threads()
    done_flops, t0, n = 0.0, time.perf_counter(), 0
    while True:
        inp = inp_sets[n % len(inp_sets)]
        if w.proj:
            if w.ln:
                oracle.mha_proj_ln(inp["x_q"], inp["x_kv"], inp["W_Q"], inp["W_K"], inp["W_V"], inp["W_O"],
                                   H=w.H, gamma=inp["ln_gamma"], beta=inp["ln_beta"], eps=1e-5,
                                   mask_kind=w.mask, key_lens=inp["key_lens"], nthreads=threads)
            elif w.Hkv is not None:
                oracle.mha_proj_gqa(inp["x_q"], inp["x_kv"], inp["W_Q"], inp["W_K"], inp["W_V"], inp["W_O"],
                                    H=w.H, H_kv=w.Hkv, mask_kind=w.mask, key_lens=inp["key_lens"], nthreads=threads)
            else:
                oracle.mha_proj(inp["x_q"], inp["x_kv"], inp["W_Q"], inp["W_K"], inp["W_V"], inp["W_O"],
                                H=w.H, mask_kind=w.mask, key_lens=inp["key_lens"], nthreads=threads)
            qkv_f, out_f = projection_flops(w)
            done_flops += qkv_f + out_f + attention_flops(w, inp["key_lens"])
            sample = "whole batches"
        elif w.decode:
            oracle.decode(inp["q"], inp["k_cache"], inp["v_cache"], mask_kind=w.mask,
                          cache_lens=inp["cache_lens"], nthreads=threads)
            done_flops += 4.0 * w.d * decode_visible(w, inp["cache_lens"])
            sample = "whole batches"
        elif w.backward and w.Nq * w.Nk > 1 << 22:
            # one (b, h) slice per thread, stacked as heads of one sequence
            g = np.random.Generator(np.random.PCG64(100 + n))
            picks = [(int(g.integers(w.B)), int(g.integers(w.H))) for _ in range(threads)]
            G = w.H // w.kv_heads  # query head h reads key/value head h // G
            st = {k_: np.stack([inp[k_][b, h // G if k_ in ("k", "v") else h] for b, h in picks])[None]
                  for k_ in ("q", "k", "v", "dout")}
            oracle.attention_backward(st["q"], st["k"], st["v"], st["dout"], mask_kind=w.mask, nthreads=threads)
            pairs = (w.Nq * (w.Nq + 1) // 2) if w.mask == 1 else w.Nq * w.Nk
            done_flops += 10.0 * w.d * pairs * len(picks)
            sample = f"passes over {len(picks)} (b, h) slices"
        elif w.backward:
            oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["dout"], mask_kind=w.mask,
                                      key_lens=inp["key_lens"], nthreads=threads)
            done_flops += 10.0 * w.d * visible_counts(w, inp["key_lens"])
            sample = "whole batches"
        elif w.Nq * w.Nk > 1 << 22:
            from transformer_head_scaled_softmax_amd import synth
            rows = synth.sample_rows(w.B, w.H, w.Nq, seed=100 + n, n_random=4)
            oracle.attention_rows(inp["q"], inp["k"], inp["v"], rows, mask_kind=w.mask,
                                  key_lens=inp["key_lens"], nthreads=threads)
            i = rows[:, 2]
            vis = np.minimum(i + 1, w.Nk) if w.mask == 1 else np.full(len(i), w.Nk)
            done_flops += 4.0 * w.d * float(vis.sum())
            sample = f"sampled rows ({len(rows)} per pass)"
        else:
            oracle.attention(inp["q"], inp["k"], inp["v"], mask_kind=w.mask,
                             key_lens=inp["key_lens"], nthreads=threads)
            done_flops += attention_flops(w, inp["key_lens"])
            sample = "whole batches"
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds_target:
            break
    rate = done_flops / el
    res = {"value": round(rate / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
           "kind": "oracle", "sample": f"{n} {sample} of {w.name}, fp64, {el:.1f} s",
           "tokens_per_s": round(n * w.B * w.Nq / el, 1) if sample == "whole batches" else None,
           **host_cpu()}
    if sample != "whole batches":
        # the whole step at the sampled rate, labelled as an extrapolation
        full = (backward_work(w, None)[1] if w.backward else attention_flops(w, None))
        res["extrapolated_full_step_s"] = round(full / rate, 1)
        res["tokens_per_s_extrapolated"] = round(w.B * w.Nq / (full / rate), 3)
    return res


def measure(w, steps: int, warmup: int, sets: int = 0, plan: str = "auto"):
    """Run ``warmup`` untimed steps of workload ``w``, then time ``steps`` steps
    (graph replay, then plain stream launches) and the same steps through the
    timed entry points (per-kernel dispatch times).  ``plan`` forces the kernel
    plan of a projection workload (auto, unfused, fused; the grouped-query entry
    points take none).  Returns the result line (without the CPU baseline) and
    the host copies of the first input sets."""
    import torch
    import transformer_head_scaled_softmax_amd as mha
    from transformer_head_scaled_softmax_amd import synth

    dev = torch.device("cuda:0")
    lib = mha.load()
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[w.dtype]
    es = ES[w.dtype]

    def to_dev(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev, tdt)

    # Input sets: a batch's own inputs and output.  Weights are the model's and are
    # shared by every batch.
    if w.proj:
        per_set = (w.B * w.Nq * w.D * 2 + (w.B * w.Nk * w.D if w.cross else 0)) * es
    elif w.decode:
        per_set = (2 * w.B * w.H * w.Nq * w.d + 2 * w.B * w.kv_heads * w.Nk * w.d) * es
    elif w.backward:  # q, out, dout, dq and k, v, dk, dv (+ lse)
        per_set = (4 * w.B * w.H * w.Nq * w.d + 4 * w.B * w.kv_heads * w.Nk * w.d) * es + 4 * w.B * w.H * w.Nq
    else:
        per_set = (2 * w.B * w.H * w.Nq * w.d + 2 * w.B * w.H * w.Nk * w.d) * es
    nsets = sets or int(min(64, max(2, math.ceil((1 << 30) / per_set))))
    log(f"[bench] workload {w.name}: {w.description}; {nsets} rotating input sets "
        f"({per_set * nsets / 2**20:.0f} MiB)")
    host_sets, dev_sets = [], []
    for s in range(nsets):
        inp = synth.workload_inputs(w, seed=w.seed * 1000 + s)
        if w.decode:
            inp["key_lens"] = inp["cache_lens"]
        lens_t = None if inp["key_lens"] is None else torch.from_numpy(inp["key_lens"]).to(dev)
        if w.proj:
            d = {"x_q": to_dev(inp["x_q"]), "x_kv": to_dev(inp["x_kv"]), "key_lens": lens_t,
                 "out": torch.empty((w.B, w.Nq, w.D), dtype=tdt, device=dev)}
        elif w.decode:
            d = {n_: to_dev(inp[n_]) for n_ in ("q", "k_cache", "v_cache")}
            d["key_lens"] = lens_t
            d["out"] = torch.empty((w.B, w.H, w.Nq, w.d), dtype=tdt, device=dev)
        elif w.backward:
            # The forward pass (with its row statistic) runs once here, untimed:
            # a step is the backward pass over resident q, k, v, out, dout, lse.
            d = {n_: to_dev(inp[n_]) for n_ in ("q", "k", "v", "dout")}
            d["key_lens"] = lens_t
            d["out"], d["lse"] = mha.forward_lse(d["q"], d["k"], d["v"], mask_kind=w.mask, key_lens=lens_t)
            for n_ in ("q", "k", "v"):
                d["d" + n_] = torch.empty_like(d[n_])
        else:
            d = {n_: to_dev(inp[n_]) for n_ in ("q", "k", "v")}
            d["key_lens"] = lens_t
            d["out"] = torch.empty((w.B, w.H, w.Nq, w.d), dtype=tdt, device=dev)
        dev_sets.append(d)
        host_sets.append(inp if s < 2 else {"key_lens": inp["key_lens"]})
    lens_list = [h["key_lens"] for h in host_sets]

    hip = Hip()
    hip.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    code = {"f32": 0, "bf16": 1, "f16": 2}[w.dtype]
    scale = ctypes.c_float(1.0 / math.sqrt(w.d))

    if w.proj:
        wts = synth.workload_inputs(w)  # seed of the workload: the model weights
        W = {n_: to_dev(wts[n_]) for n_ in ("W_Q", "W_K", "W_V", "W_O") + (("ln_gamma", "ln_beta") if w.ln else ())}
        gqa = w.Hkv is not None and w.Hkv != w.H  # shared key/value projections
        plan_code = {"auto": 0, "unfused": 1, "fused": 2}[plan]
        if plan_code and gqa:
            raise SystemExit("--plan: the grouped-query projection entry points choose their own plan")
        if gqa:
            need = lib.mha_proj_gqa_workspace_bytes(w.B, w.Nq, w.Nk, w.D, w.H, w.Hkv, w.d, w.d, code)
        else:
            need = (lib.mha_proj_ln_workspace_bytes if w.ln else lib.mha_proj_workspace_bytes)(
                w.B, w.Nq, w.Nk, w.D, w.H, w.d, w.d, code)
        ws = torch.empty(need, dtype=torch.uint8, device=dev)

        def step(i, sp, events=None):
            d = dev_sets[i % nsets]
            lp = None if d["key_lens"] is None else d["key_lens"].data_ptr()
            xkv = None if d["x_kv"] is None else d["x_kv"].data_ptr()
            head = (d["x_q"].data_ptr(), xkv, W["W_Q"].data_ptr(), W["W_K"].data_ptr(),
                    W["W_V"].data_ptr(), W["W_O"].data_ptr(), None, None, None, None)
            tail = (w.B, w.Nq, w.Nk, w.D, w.H, w.d, w.d, w.mask, lp, scale, code, ws.data_ptr(), need, sp)
            if w.ln:
                argsv = (*head, W["ln_gamma"].data_ptr(), W["ln_beta"].data_ptr(), ctypes.c_float(1e-5),
                         d["out"].data_ptr(), *tail)
                st = (lib.mha_proj_ln_forward(*argsv) if events is None and not plan_code
                      else lib.mha_proj_ln_forward_timed(*argsv, events, plan_code))
            elif gqa:
                argsv = (*head, d["out"].data_ptr(), *tail[:5], w.Hkv, *tail[5:])
                st = (lib.mha_proj_forward_gqa(*argsv) if events is None
                      else lib.mha_proj_forward_gqa_timed(*argsv, events))
            else:
                argsv = (*head, d["out"].data_ptr(), *tail)
                st = (lib.mha_proj_forward(*argsv) if events is None and not plan_code
                      else lib.mha_proj_forward_timed(*argsv, events, plan_code))
            if st != 0:
                raise RuntimeError(lib.mha_last_error_message().decode())
        # Kernel -> (start, end) event indices of mha_proj_forward_timed.
        # --plan fused on sizes the fused kernel does not take fails in the
        # library with MHA_ERR_UNSUPPORTED.
        fused = plan == "fused" or (plan == "auto" and lib.mha_proj_fused(w.B, w.Nq, w.Nk, w.D, w.d, w.d,
                                                                          0 if w.cross else 1))
        if fused:
            stage_events = {"qkv_attention": (0, 1), "out_projection": (4, 5)}
        else:
            stage_events = {"qkv_projection": (0, 1), "attention": (2, 3), "out_projection": (4, 5)}
        n_events = 6
        if w.ln:
            stage_events["out_projection_ln"] = stage_events.pop("out_projection")
            stage_events["ln_rows"] = (6, 7)
            n_events = 8
    elif w.decode:
        Hkv = w.kv_heads
        need = lib.mha_decode_workspace_bytes(w.B, w.H, Hkv, w.Nq, w.Nk, w.d, w.d, code)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        nsplit = lib.mha_decode_split(w.B, w.H, Hkv, w.Nq, w.Nk, w.d, w.d, code)
        assert nsplit >= 1, "the decoding workloads run on the split decoding kernel"

        def step(i, sp, events=None):
            d = dev_sets[i % nsets]
            lp = None if d["key_lens"] is None else d["key_lens"].data_ptr()
            argsv = (d["q"].data_ptr(), d["k_cache"].data_ptr(), d["v_cache"].data_ptr(), d["out"].data_ptr(),
                     w.B, w.H, Hkv, w.Nq, w.Nk, w.d, w.d, w.mask, lp, scale, code, ws.data_ptr(), need, sp)
            st = (lib.mha_decode_forward(*argsv) if events is None
                  else lib.mha_decode_forward_timed(*argsv, events))
            if st != 0:
                raise RuntimeError(lib.mha_last_error_message().decode())
        stage_events = {"decode": (0, 1)}
        if nsplit > 1:
            stage_events["decode_combine"] = (2, 3)
        n_events = 4
    elif w.backward:
        need = lib.mha_backward_gqa_workspace_bytes(w.B, w.H, w.kv_heads, w.Nq, w.Nk, w.d, w.d, code)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

        def step(i, sp, events=None):
            d = dev_sets[i % nsets]
            lp = None if d["key_lens"] is None else d["key_lens"].data_ptr()
            ptrs = tuple(d[n_].data_ptr() for n_ in ("q", "k", "v", "out", "dout", "lse", "dq", "dk", "dv"))
            tail = (w.Nq, w.Nk, w.d, w.d, w.mask, lp, scale, code, ws.data_ptr(), need, sp)
            if w.Hkv is not None:  # shared key/value heads
                argsv = ptrs + (w.B, w.H, w.Hkv) + tail
                st = lib.mha_backward_gqa(*argsv) if events is None else lib.mha_backward_gqa_timed(*argsv, events)
            else:
                argsv = ptrs + (w.B, w.H) + tail
                st = lib.mha_backward(*argsv) if events is None else lib.mha_backward_timed(*argsv, events)
            if st != 0:
                raise RuntimeError(lib.mha_last_error_message().decode())
        if lib.mha_backward_single_launch(w.B, w.H, w.kv_heads, w.Nq, w.Nk, w.d, w.d, code):
            stage_events = {"bwd_fused": (0, 1)}
        else:
            stage_events = {"bwd_dq": (0, 1), "bwd_dkdv": (2, 3)}
        n_events = 4
    else:
        def step(i, sp, events=None):
            d = dev_sets[i % nsets]
            lp = None if d["key_lens"] is None else d["key_lens"].data_ptr()
            argsv = (d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(), d["out"].data_ptr(),
                     w.B, w.H, w.Nq, w.Nk, w.d, w.d, w.mask, lp, scale, code, sp)
            st = lib.mha_forward(*argsv) if events is None else lib.mha_forward_timed(*argsv, events)
            if st != 0:
                raise RuntimeError(lib.mha_last_error_message().decode())
        stage_events = {("attention_f32" if w.dtype == "f32" else "attention"): (0, 1)}
        n_events = 2

    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    t0 = time.perf_counter()
    for i in range(warmup):
        step(i, sp)
    torch.cuda.synchronize()
    host_us_per_step = (time.perf_counter() - t0) / max(1, warmup) * 1e6

    # Timed region 1 (the reported throughput): the K steps replayed from HIP
    # graphs, as a serving loop would issue them, so host launch overhead does
    # not stall the GPU.  One graph holds one step per input set.
    K = steps
    G = min(nsets, K)
    cap = torch.cuda.Stream()

    def capture(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            step(0, ctypes.c_void_p(cap.cuda_stream))  # warm the capture stream
        cap.synchronize()
        with torch.cuda.graph(g, stream=cap):
            csp = ctypes.c_void_p(cap.cuda_stream)
            for i in range(n):
                step(warmup + i, csp)
        return g

    g_full = capture(G)
    g_rest = capture(K % G) if K % G else None
    reps = K // G
    for _ in range(2):
        g_full.replay()
    torch.cuda.synchronize()
    start, end = hip.event(), hip.event()
    cur = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    hip.lib.hipEventRecord(start, cur)
    for _ in range(reps):
        g_full.replay()
    if g_rest is not None:
        g_rest.replay()
    hip.lib.hipEventRecord(end, cur)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_step_graph = hip.elapsed_ms(start, end) / K

    # Timed region 1b: the same K steps issued straight onto the stream, with
    # events only around the whole run.  A long kernel per step gains nothing
    # from a graph (ROCm dispatches each kernel node of a graph with more
    # latency than a plain stream launch); the step time reported is that of
    # the faster of the two ways of issuing, named in config.issue.
    torch.cuda.synchronize()
    t_wall_s = time.perf_counter()
    hip.lib.hipEventRecord(start, cur)
    for i in range(K):
        step(warmup + i, cur)
    hip.lib.hipEventRecord(end, cur)
    torch.cuda.synchronize()
    t_wall_s = time.perf_counter() - t_wall_s
    ms_step_stream = hip.elapsed_ms(start, end) / K
    issue = "HIP graph replay" if ms_step_graph <= ms_step_stream else "stream launches"
    ms_step = min(ms_step_graph, ms_step_stream)
    t_wall = t_wall if ms_step_graph <= ms_step_stream else t_wall_s

    # Timed region 2 (per-kernel times): the same K steps issued directly on the
    # stream through the timed entry points, whose events take each kernel's own
    # start and end timestamps from its dispatch (hipExtLaunchKernel).
    ev_arrays = [(ctypes.c_void_p * n_events)(*[hip.event() for _ in range(n_events)])
                 for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        step(warmup + i, sp, ev_arrays[i])
    torch.cuda.synchronize()
    per = {n_: [] for n_ in stage_events}
    for evs in ev_arrays:
        for n_, (a_, b_) in stage_events.items():
            per[n_].append(hip.elapsed_ms(evs[a_], evs[b_]))
    avg = {n_: float(np.mean(v)) for n_, v in per.items()}
    last_end = max(b_ for _, b_ in stage_events.values())  # some events may stay unrecorded
    eager_ms_step = hip.elapsed_ms(ev_arrays[0][0], ev_arrays[-1][last_end]) / K

    used = [lens_list[(warmup + i) % nsets] for i in range(K)]
    att_f = float(np.mean([attention_flops(w, L) for L in used]))
    if w.proj:
        qkv_f, out_f = projection_flops(w)
        flops = qkv_f + out_f + att_f
        bytes_ = float(np.mean([proj_path_bytes(w, L) for L in used]))
    elif w.decode:
        works = [decode_work(w, L, nsplit) for L in used]
        flops = float(np.mean([sum(f for f, _ in wk.values()) for wk in works]))
        bytes_ = float(np.mean([decode_work(w, L, 1)["decode"][1] for L in used]))  # whole step
    elif w.backward:
        works = [backward_work(w, L) for L in used]
        flops = float(np.mean([f for _, f in works]))
        # whole step: q, k, v (visible rows), out, dout, lse in; dq, dk, dv out
        Lm = [np.full(w.B, w.Nk) if L is None else np.clip(L, 0, w.Nk) for L in used]
        bytes_ = float(np.mean([(4 * w.B * w.H * w.Nq * w.d + 2 * int(L.sum()) * w.H * w.d
                                 + 2 * w.B * w.H * w.Nk * w.d) * es + 4 * w.B * w.H * w.Nq for L in Lm]))
    else:
        flops = att_f
        bytes_ = float(np.mean([attention_bytes(w, L) for L in used]))
    sec = ms_step / 1e3
    result = {
        "metric": METRIC, "value": round(flops / sec / 1e12, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": K, "warmup": warmup, "ms_per_step": round(ms_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) activations, Xavier-uniform weights, uniform key lengths)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "d_k": w.d,
                   "d_v": w.d, "D": w.D if w.proj else None, "projections": w.proj,
                   "mask": "causal" if w.mask == 1 else "none",
                   "key_lens": None if w.lens is None else f"U{{{w.lens[0]}..{w.lens[1]}}}",
                   "input_sets": nsets, "issue": issue,
                   **({"plan": plan} if w.proj and plan != "auto" else {}),
                   **({"residual_layer_norm": True} if w.ln else {}),
                   **({"decode": True, "H_kv": w.kv_heads, "cache_slots": w.Nk, "waves": nsplit}
                      if w.decode else {}),
                   **({"pass": "backward (dq, dk, dv from q, k, v, out, dout, lse)",
                       "flops_per_visible_pair": 10 * w.d} if w.backward else {}),
                   **({"H_kv": w.kv_heads} if (w.backward or w.proj) and w.Hkv is not None else {})},
        "tokens_per_s": round(w.B * w.Nq / sec, 1),
        "frac_bf16_peak": round(flops / sec / 1e12 / PEAK_TFLOPS["bf16"], 5),
        "hbm_gbps_algorithmic": round(bytes_ / sec / 1e9, 1),
        "ms_per_step_graph": round(ms_step_graph, 6),
        "ms_per_step_stream": round(ms_step_stream, 6),
        "ms_per_step_eager": round(eager_ms_step, 6),
        "host_us_per_step": round(host_us_per_step, 2),
        "wall_s_timed": round(t_wall, 4),
        "kernel_ms": {n_: round(v, 6) for n_, v in avg.items()},
    }

    # Roofline of the dominant kernel.
    dom = max(avg, key=avg.get)
    if w.proj:
        f_, b_ = stage_work(w, None)[dom]
        if dom in ("attention", "qkv_attention"):  # these depend on the drawn key lengths
            f_ = float(np.mean([stage_work(w, L)[dom][0] for L in used]))
            b_ = float(np.mean([stage_work(w, L)[dom][1] for L in used]))
    elif w.decode:
        f_ = float(np.mean([wk[dom][0] for wk in works]))
        b_ = float(np.mean([wk[dom][1] for wk in works]))
    elif w.backward:
        f_ = float(np.mean([wk[dom][0] for wk, _ in works]))
        b_ = float(np.mean([wk[dom][1] for wk, _ in works]))
    else:
        f_, b_ = flops, bytes_
    result["roofline"] = roofline(f_, b_, avg[dom] / 1e3, w.dtype, dom,
                                  w.name + ("" if plan == "auto" else "_" + plan))

    return result, host_sets


def main():
    from transformer_head_scaled_softmax_amd import synth

    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(synth.WORKLOADS))
    ap.add_argument("--sets", type=int, default=0, help="rotating input sets (0: enough for >= 1 GiB)")
    ap.add_argument("--plan", default="auto", choices=("auto", "unfused", "fused"),
                    help="kernel plan of a projection workload (default: the library's choice)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="time only --workload (by default a run of one of the five configurations also "
                         "times the other four, GPU only)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (for HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import transformer_head_scaled_softmax_amd as mha

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = 256 << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 5}))
        return

    w = synth.WORKLOADS[args.workload]
    result, host_sets = measure(w, args.steps, args.warmup, args.sets, args.plan)
    if not args.no_cpu_baseline:
        log(f"[bench] GPU done: {result['ms_per_step'] * 1e3:.2f} us/step; timing the fp64 oracle "
            f"for ~{args.cpu_seconds:.0f} s")
        result["cpu_baseline"] = cpu_baseline(w, [h for h in host_sets if "x_q" in h or "q" in h],
                                              args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    del host_sets
    if not args.no_other_configs and w.name in CONFIGS:
        # The other configurations, GPU only, same step definition and timing.
        others = {}
        for name in CONFIGS:
            if name == w.name:
                continue
            torch.cuda.empty_cache()
            r, _ = measure(synth.WORKLOADS[name], args.steps, min(args.warmup, 20), 0)
            others[name] = {k: r[k] for k in ("ms_per_step", "value", "unit", "tokens_per_s",
                                              "hbm_gbps_algorithmic", "dtype", "kernel_ms")}
            others[name]["issue"] = r["config"]["issue"]
            others[name]["roofline"] = {k: r["roofline"][k] for k in ("kernel", "bound", "achieved", "peak",
                                                                       "unit", "frac")}
        result["configs"] = others
    print(json.dumps(result), flush=True)

if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of IO-aware exact attention on one AMD Instinct MI355X.

A step is one pass of the attention hot path over one batch: the forward
(fa_fwd: O and LSE) followed by the recomputation-based backward (fa_bwd: dQ,
dK, dV) at B=2, H=16, Sq=Sk=8192, d=128, bf16, non-causal, iid N(0,1) inputs
(seed 2000), all resident in HBM before timing starts.  Throughput counts the
method's algorithmic flops: 4*B*H*Sq*Sk*d for the forward and 2.5 times that
for the backward (five GEMM-shaped products: the recomputed scores, dP, dV,
dK, dQ), so fwd+bwd = 14*B*H*Sq*Sk*d.  Any extra recomputation the kernels do
is not counted.

Printed: one JSON line with the whole-step TFLOP/s; each kernel of the step
timed on its own (HIP events on the stream it is launched on); the roofline
of the dominant kernel (the dK/dV backward kernel: four of the five backward
products) against the dense bf16 MFMA peak (256 CU x 2.4 GHz x 4096
flop/clk/CU = 2516.6 TFLOP/s); secondary workloads (causal, decode, varlen,
FP8, the forward sweep); and the fp64 CPU oracle timed on a bounded sample of
the step.
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import torch  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6
PEAK_HBM_GBPS = 8000.0
PEAK_FP8_TFLOPS = 5033.2
WORKLOAD = dict(B=2, S=8192, H=16, d=128, causal=False, seed=2000)


def fwd_flops(B, Sq, Sk, H, d, causal):
    return 4.0 * B * H * Sq * Sk * d / (2 if causal else 1)


def kernel_source_hash(files):
    """Hash of the kernel sources a counter record was taken on, with
    comments and whitespace removed (an edit of a comment leaves the kernel,
    and so the record, unchanged)."""
    import re
    h = hashlib.sha256()
    for name in files:
        with open(os.path.join(ROOT, "io_aware_exact_amd", "csrc", name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


BWD_SOURCES = ("bwd.hip", "device_common.h", "fa_internal.h")
FWD_SOURCES = ("fwd_pp.hip", "device_common.h", "fa_internal.h")


def traffic_from_profile(name, files):
    """HBM bytes per launch of a kernel from the committed counter summary
    profiles/<name>_traffic.json, or None if it is missing or was taken on a
    different kernel source."""
    path = os.path.join(ROOT, "profiles", name + "_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash(files):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline_leg(q, k, v, do, o, lse, causal, fp8_rows):
    """Everything that runs the fp64 oracle (it never enters a timed GPU
    region):
      * the baseline: the oracle's forward+backward on one full (batch 0,
        head 0) slice of the step, converted to a TFLOP/s rate with the same
        algorithmic flop count;
      * a sampled check of the step's O and LSE (rows {0, 1, S-1} plus 13
        seeded rows of (b, h) = (0, 0) and (B-1, H-1));
      * the FP8 workload's RMS error against the oracle on the original fp32
        inputs, for per-block FP8, per-tensor FP8 and bf16 inputs (rows
        sampled by leg_fp8), and the per-tensor / per-block ratio."""
    import numpy as np
    import oracle
    from io_aware_exact_amd import inputs
    B, S, H, d = q.shape
    t0 = time.perf_counter()
    oracle.attention_bwd(q[:1, :, :1], k[:1, :, :1], v[:1, :, :1], do[:1, :, :1], causal, None)
    dt = time.perf_counter() - t0
    flops = 3.5 * fwd_flops(1, S, S, 1, d, causal)
    out = {"cpu_baseline": {
        "value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"fp64 forward+backward of one full (b,h) slice of the step (S={S}, d={d}) "
                  f"took {dt:.1f} s; rate uses the step's algorithmic flops"}}
    rows = inputs.sample_indices(S, 13, 77, always=(0, 1, S - 1))
    bi, hi, ii = [], [], []
    for b, h in ((0, 0), (B - 1, H - 1)):
        for i in rows:
            bi.append(b), hi.append(h), ii.append(i)
    o_ref, lse_ref = oracle.attention_fwd_rows(q, k, v, bi, hi, ii, causal)
    o_got = o[bi, ii, hi].float().cpu().numpy()
    l_got = lse[bi, hi, ii].cpu().numpy()
    out["check"] = {"o_max_abs": float(np.abs(o_got - o_ref).max()),
                    "lse_max_abs": float(np.abs(l_got - lse_ref).max())}
    if fp8_rows is not None:
        X, (fbi, fhi, fii), got = fp8_rows
        ref, _ = oracle.attention_fwd_rows(*X, fbi, fhi, fii, False)
        rms = {name: float(np.sqrt(np.mean((g - ref) ** 2))) for name, g in got.items()}
        out["fp8_rms"] = {
            "workload": "fp8 workload, 64 seeded rows x 16 heads, vs fp64 oracle on the "
                        "original fp32 inputs",
            "per_block_fp8": rms["fp8_block"], "per_tensor_fp8": rms["fp8_tensor"],
            "bf16": rms["bf16"], "mx_fp8": rms["mx"],
            "per_tensor_over_per_block": rms["fp8_tensor"] / rms["fp8_block"]}
    return out


def time_calls(fn, reps, warmup=2, warm_ms=100.0, min_ms=200.0):
    """Times fn() launched back to back on the current stream, after at
    least `warmup` calls and about `warm_ms` of untimed work (the first
    launches on fresh buffers run slower): max(reps, 20) calls, more if
    needed to cover `min_ms`.  Each call is bracketed by HIP events on the
    stream.  Returns {"mean", "median", "min"} in ms and the call count."""
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(warmup):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    per_call = max(e0.elapsed_time(e1) / max(warmup, 1), 1e-3)
    for _ in range(min(int(warm_ms / per_call), 200)):
        fn()
    torch.cuda.synchronize()
    n = max(reps, 20, min(int(min_ms / per_call) + 1, 2000))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    ev[0].record(stream)
    for i in range(n):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    each = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(n))
    return {"mean": ev[0].elapsed_time(ev[n]) / n, "median": each[n // 2], "min": each[0], "n": n}


def timing(t):
    return {"mean_ms": round(t["mean"], 4), "median_ms": round(t["median"], 4),
            "min_ms": round(t["min"], 4), "calls": t["n"]}


def leg_causal(reps):
    """fwd and fwd+bwd at B=2, H=16, S=8192, d=128, causal (flops halved)."""
    from io_aware_exact_amd import fa, inputs
    B, S, H, d = 2, 8192, 16, 128
    q, k, v, do = inputs.qkv(B, S, S, H, H, d, 2000, device="cuda", with_dout=True)
    o = torch.empty((B, S, H, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
    grads = tuple(torch.empty_like(x) for x in (q, k, v))
    a = fa.bwd_args(q, k, v, o, do, lse, *grads, True, None)
    ws = torch.empty(int(fa.lib().fa_bwd_workspace_size(ctypes.byref(a))), dtype=torch.uint8,
                     device="cuda")
    tf_ = time_calls(lambda: fa.fwd(q, k, v, True, out=o, lse=lse), reps)
    tb = time_calls(lambda: fa.bwd(q, k, v, o, do, lse, True, out=grads, workspace=ws), reps)
    ms_f, ms_b = tf_["mean"], tb["mean"]
    ff = fwd_flops(B, S, S, H, d, True)
    return {"workload": "B=2 H=16 Sq=Sk=8192 d=128 causal",
            "fwd_tflops": round(ff / ms_f / 1e9, 2), "fwd_ms": round(ms_f, 4),
            "fwd_bwd_tflops": round(3.5 * ff / (ms_f + ms_b) / 1e9, 2),
            "bwd_ms": round(ms_b, 4), "fwd_timing": timing(tf_), "bwd_timing": timing(tb)}


def leg_decode(reps):
    """Split-KV decode: B=64, Sq=1, Sk=32768, Hq=32, Hkv=8, d=128, causal.
    HBM-bound: reports K+V bytes / time against 8 TB/s."""
    from io_aware_exact_amd import fa, inputs
    B, Sq, Sk, Hq, Hkv, d = 64, 1, 32768, 32, 8, 128
    q, k, v = inputs.qkv(B, Sq, Sk, Hq, Hkv, d, 3100, device="cuda")
    o = torch.empty((B, Sq, Hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device="cuda")
    ws = torch.empty(fa.fwd_workspace_bytes(q, k, v, True), dtype=torch.uint8, device="cuda")
    t = time_calls(lambda: fa.fwd(q, k, v, True, out=o, lse=lse, workspace=ws), reps)
    ms = t["mean"]
    kv_bytes = 2 * B * Sk * Hkv * d * 2
    io_bytes = kv_bytes + 2 * (B * Sq * Hq * d * 2) + B * Hq * Sq * 4
    return {"workload": "decode B=64 Sq=1 Sk=32768 Hq=32 Hkv=8 d=128",
            "ms": round(ms, 4), "gbps": round(io_bytes / ms / 1e6, 1),
            "frac_of_hbm": round(io_bytes / ms / 1e6 / PEAK_HBM_GBPS, 4),
            "tflops": round(4.0 * B * Hq * Sq * Sk * d / ms / 1e9, 2), "timing": timing(t)}


def leg_varlen(reps):
    """Packed varlen + GQA forward and backward: 16 sequences, lengths uniform
    on [128, 32768] (seed 3000), Hq=32, Hkv=8, d=128, causal; dO ~ N(0,1)
    (seed 3002).  Gradient and workspace buffers are allocated before timing."""
    from io_aware_exact_amd import fa, inputs
    lens = inputs.varlen_lengths(16, 128, 32768, 3000)
    Hq, Hkv, d = 32, 8, 128
    q, k, v = inputs.packed_qkv(lens, lens, Hq, Hkv, d, 3001, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(3002)
    do = torch.randn(q.shape, generator=g, device="cuda").to(torch.bfloat16)
    cu = inputs.cu_seqlens(lens, device="cuda")
    T, mx = sum(lens), max(lens)
    o = torch.empty((T, Hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((Hq, T), dtype=torch.float32, device="cuda")
    tv = time_calls(lambda: fa.fwd_varlen(q, k, v, cu, cu, mx, mx, True, out=o, lse=lse), reps)
    ms = tv["mean"]
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    a = fa.bwd_varlen_args(q, k, v, o, do, lse, *grads, cu, cu, mx, mx, True, None)
    ws = torch.empty(max(int(fa.lib().fa_bwd_varlen_workspace_size(ctypes.byref(a))), 1),
                     dtype=torch.uint8, device="cuda")
    tvb = time_calls(lambda: fa.bwd_varlen(q, k, v, o, do, lse, cu, cu, mx, mx, True,
                                           out=grads, workspace=ws), reps)
    ms_b = tvb["mean"]
    pairs = sum(L * (L + 1) // 2 for L in lens)
    flops_half = sum(2.0 * Hq * d * L * L for L in lens)
    return {"workload": "varlen 16 seqs U[128,32768] Hq=32 Hkv=8 d=128 causal",
            "total_tokens": T, "ms": round(ms, 3),
            "tflops": round(flops_half / ms / 1e9, 2),
            "tflops_exact_pairs": round(4.0 * Hq * d * pairs / ms / 1e9, 2),
            "bwd_ms": round(ms_b, 3),
            "fwd_bwd_tflops": round(3.5 * flops_half / (ms + ms_b) / 1e9, 2),
            "fwd_bwd_tflops_exact_pairs": round(14.0 * Hq * d * pairs / (ms + ms_b) / 1e9, 2),
            "fwd_timing": timing(tv), "bwd_timing": timing(tvb)}


def leg_kvcache(reps):
    """KV-cache attention (fa_fwd_kvcache) on a paged cache of 256-token pages
    handed out in a shuffled order (seed 3201):
    decode -- B=64, Hq=32, Hkv=8, d=128, 32767 cached tokens plus one
    appended per sequence (the dense decode's workload, read through the
    block table; the append is inside the timed call);
    prefill -- B=4 sequences with 15360 cached tokens and a 1024-token chunk
    appended and attended causally (Sq = Snew = 1024)."""
    from io_aware_exact_amd import fa
    out = {}
    Hq, Hkv, d, ps = 32, 8, 128, 256
    for name, B, L, sq in (("decode", 64, 32767, 1), ("prefill", 4, 15360, 1024)):
        per = (L + sq + ps - 1) // ps
        g = torch.Generator(device="cuda")
        g.manual_seed(3200)
        kc = torch.randn((B * per, ps, Hkv, d), generator=g, device="cuda").to(torch.bfloat16)
        vc = torch.randn((B * per, ps, Hkv, d), generator=g, device="cuda").to(torch.bfloat16)
        q = torch.randn((B, sq, Hq, d), generator=g, device="cuda").to(torch.bfloat16)
        kn = torch.randn((B, sq, Hkv, d), generator=g, device="cuda").to(torch.bfloat16)
        vn = torch.randn((B, sq, Hkv, d), generator=g, device="cuda").to(torch.bfloat16)
        gc = torch.Generator(device="cpu")
        gc.manual_seed(3201)
        bt = torch.randperm(B * per, generator=gc).to(torch.int32).view(B, per).cuda()
        lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
        o = torch.empty_like(q)
        lse = torch.empty((B, Hq, sq), dtype=torch.float32, device="cuda")
        a = fa.kvcache_args(q, kc, vc, lens, bt, kn, vn, o, lse, True, None)
        n = int(fa.lib().fa_fwd_kvcache_workspace_size(ctypes.byref(a)))
        ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
        t = time_calls(lambda: fa.fwd_kvcache(q, kc, vc, lens, bt, kn, vn, True, out=o, lse=lse,
                                              workspace=ws), reps)
        ms = t["mean"]
        Lk = L + sq
        kv_bytes = 2 * B * Lk * Hkv * d * 2
        io_bytes = kv_bytes + 2 * B * sq * Hq * d * 2 + B * Hq * sq * 4 + 2 * B * sq * Hkv * d * 2
        pairs = B * sum(min(Lk, i + 1 + Lk - sq) for i in range(sq))
        out[name] = {"workload": f"paged KV cache B={B} cached={L} new={sq} Hq={Hq} Hkv={Hkv} "
                                 f"d={d} page={ps} causal",
                     "ms": round(ms, 4), "gbps": round(io_bytes / ms / 1e6, 1),
                     "frac_of_hbm": round(io_bytes / ms / 1e6 / PEAK_HBM_GBPS, 4),
                     "tflops": round(4.0 * Hq * d * pairs / ms / 1e9, 2), "timing": timing(t)}
        del kc, vc
        torch.cuda.empty_cache()
    return out


def leg_fp8(reps, keep_rows=None):
    """FP8 (E4M3, per-block scales) forward: B=1, H=16, S=16384, d=128,
    non-causal, inputs N(0,1) + Bernoulli(0.001) N(0,100) (seed 4000), and
    the MX variant on the same inputs.  Quantisation is input preparation and
    is not timed.  With keep_rows (a dict), 64 seeded rows of every head of
    the per-block, per-tensor, MX and bf16 outputs are left there, with the
    inputs, for the RMS comparison against the oracle."""
    from io_aware_exact_amd import fa, inputs
    B, S, H, d = 1, 16384, 16, 128
    X = [inputs.outlier_normal((B, S, H, d), 4000 + i, device="cuda") for i in range(3)]
    qkv = [fa.quantize_fp8(x) for x in X]
    codes = [c for c, _ in qkv]
    scales = [s for _, s in qkv]
    o = torch.empty((B, S, H, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
    t = time_calls(lambda: fa.fwd_fp8(*codes, *scales, False, out=o, lse=lse), reps)
    ms = t["mean"]
    ff = fwd_flops(B, S, S, H, d, False)
    # FP8 backward on the same inputs: dO ~ N(0,1) (seed 4003), the forward's
    # O and LSE; gradients and workspace allocated before timing
    g = torch.Generator(device="cuda")
    g.manual_seed(4003)
    dout = torch.randn((B, S, H, d), generator=g, device="cuda").to(torch.bfloat16)
    fa.fwd_fp8(*codes, *scales, False, out=o, lse=lse)
    grads = tuple(torch.empty((B, S, H, d), dtype=torch.bfloat16, device="cuda") for _ in range(3))
    a = fa.bwd_fp8_args(*codes, scales, o, dout, lse, *grads, False, None)
    ws = torch.empty(int(fa.lib().fa_bwd_workspace_size(ctypes.byref(a))), dtype=torch.uint8, device="cuda")

    def bwd(stages=0):
        return lambda: fa.bwd_fp8(*codes, scales, o, dout, lse, False, out=grads, workspace=ws, stages=stages)
    tb = time_calls(bwd(), reps)
    tb_k = {name: time_calls(bwd(st), reps) for name, st in
            (("bwd_fp8_preprocess_kernel", fa.FA_BWD_PREPROCESS), ("bwd_dkdv_fp8_kernel", fa.FA_BWD_DKDV),
             ("bwd_dq_fp8_kernel", fa.FA_BWD_DQ))}
    del ws, grads, dout
    mx = [fa.quantize_mxfp8(X[0], 0), fa.quantize_mxfp8(X[1], 0), fa.quantize_mxfp8(X[2], 1)]
    o_mx = torch.empty_like(o)
    tm = time_calls(lambda: fa.fwd_mxfp8(*[c for c, _ in mx], *[s for _, s in mx], False,
                                         out=o_mx, lse=lse), reps)
    ms_mx = tm["mean"]
    if keep_rows is not None:
        rows = inputs.sample_indices(S, 61, 4001, always=(0, 1, S - 1))
        bi = [0] * (len(rows) * H)
        hi = [h for h in range(H) for _ in rows]
        ii = [i for _ in range(H) for i in rows]
        ten = [fa.quantize_fp8(x, per_tensor=True) for x in X]
        o_ten, _ = fa.fwd_fp8(*[c for c, _ in ten], *[s for _, s in ten], False)
        o_bf, _ = fa.fwd(*[x.to(torch.bfloat16) for x in X], False)
        fa.fwd_fp8(*codes, *scales, False, out=o, lse=lse)
        torch.cuda.synchronize()
        keep_rows["rows"] = ([x.cpu() for x in X], (bi, hi, ii),
                             {name: y[bi, ii, hi].float().cpu().numpy()
                              for name, y in (("fp8_block", o), ("fp8_tensor", o_ten),
                                              ("bf16", o_bf), ("mx", o_mx))})
    return {"workload": "fp8 e4m3 fwd B=1 H=16 S=16384 d=128 non-causal, per-block scales",
            "ms": round(ms, 4), "tflops": round(ff / ms / 1e9, 2),
            "frac_of_fp8_peak": round(ff / ms / 1e9 / PEAK_FP8_TFLOPS, 4), "timing": timing(t),
            "bwd": {"workload": "FP8 backward (all five products on FP8 MFMA), same shape and inputs, "
                                "dO ~ N(0,1)",
                    "ms": round(tb["mean"], 4), "bwd_tflops": round(2.5 * ff / tb["mean"] / 1e9, 2),
                    "fwd_bwd_tflops": round(3.5 * ff / (ms + tb["mean"]) / 1e9, 2),
                    "fwd_bwd_frac_of_fp8_peak": round(3.5 * ff / (ms + tb["mean"]) / 1e9 / PEAK_FP8_TFLOPS, 4),
                    "timing": timing(tb),
                    "kernels": {k: timing(v) for k, v in tb_k.items()}},
            "mx": {"workload": "MX fp8 (E8M0 scale per 32 elements) fwd, same shape and inputs",
                   "ms": round(ms_mx, 4), "tflops": round(ff / ms_mx / 1e9, 2),
                   "frac_of_fp8_peak": round(ff / ms_mx / 1e9 / PEAK_FP8_TFLOPS, 4),
                   "timing": timing(tm)}}


def leg_sweep(reps):
    """bf16 forward sweep at B*S = 16384 tokens, H = 16: TFLOP/s per
    (d, causal) and S (flops halved when causal)."""
    from io_aware_exact_amd import fa, inputs
    out = {}
    for d in (64, 128):
        for causal in (False, True):
            row = {}
            for S in (512, 1024, 2048, 4096, 8192, 16384):
                B, H = 16384 // S, 16
                q, k, v = inputs.qkv(B, S, S, H, H, d, 1000, device="cuda")
                o = torch.empty_like(q)
                lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
                ms = time_calls(lambda: fa.fwd(q, k, v, causal, out=o, lse=lse), reps)["mean"]
                row[str(S)] = round(fwd_flops(B, S, S, H, d, causal) / ms / 1e9, 1)
            out[f"d{d}_{'causal' if causal else 'noncausal'}"] = row
    return out


def leg_gemm(reps):
    """The box's sustained dense bf16 MFMA rate, measured on a plain library
    GEMM (torch.matmul -> hipBLASLt, M = N = K = 8192, bf16 in, fp32
    accumulate, bf16 out): the practical ceiling the attention kernels'
    MFMA rate is compared with (not part of the attention path)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    n = 8192
    a = torch.randn((n, n), generator=g, device="cuda").to(torch.bfloat16)
    b = torch.randn((n, n), generator=g, device="cuda").to(torch.bfloat16)
    c = torch.empty((n, n), dtype=torch.bfloat16, device="cuda")
    t = time_calls(lambda: torch.matmul(a, b, out=c), reps)
    flops = 2.0 * n ** 3
    out = {"workload": "bf16 GEMM 8192x8192x8192 (torch.matmul, hipBLASLt)", "ms": round(t["mean"], 4),
           "tflops": round(flops / t["mean"] / 1e9, 2),
           "frac_of_peak": round(flops / t["mean"] / 1e9 / PEAK_BF16_TFLOPS, 4), "timing": timing(t)}
    # the same product in E4M3 (torch._scaled_mm, per-tensor scales, bf16
    # out): the sustained fp8 MFMA rate the FP8 kernels are compared with
    del c
    try:
        a8 = a.to(torch.float8_e4m3fn)
        b8 = b.to(torch.float8_e4m3fn).t().contiguous().t()     # column-major B
        one = torch.ones((), dtype=torch.float32, device="cuda")
        c8 = torch._scaled_mm(a8, b8, scale_a=one, scale_b=one, out_dtype=torch.bfloat16)
        t8 = time_calls(lambda: torch._scaled_mm(a8, b8, scale_a=one, scale_b=one, out_dtype=torch.bfloat16), reps)
        ref = torch.matmul(a8[:64].float(), b8.float())
        err = float((c8[:64].float() - ref).abs().max() / ref.abs().max())
        out["fp8"] = {"workload": "E4M3 GEMM 8192x8192x8192 (torch._scaled_mm, hipBLASLt, bf16 out)",
                      "ms": round(t8["mean"], 4), "tflops": round(flops / t8["mean"] / 1e9, 2),
                      "frac_of_peak": round(flops / t8["mean"] / 1e9 / PEAK_FP8_TFLOPS, 4),
                      "max_rel_err_first_rows": round(err, 5), "timing": timing(t8)}
    except (RuntimeError, TypeError, AttributeError) as e:
        out["fp8"] = {"error": str(e).splitlines()[0][:200]}
    return out


def leg_dqaccum(reps):
    """Cost of the dQ accumulation a fused backward would add (measurement
    probe `libfa_probe.so`, not part of the path): the dK/dV kernel's grid at
    B=2, H=16, S=8192, d=128 (2048 workgroups of 128 keys, one per CU at a
    time) adding a 64 x 128 fp32 partial for each of its 128 query tiles into
    a 128 MB accumulator -- by device-scope atomics (mode 0), by racy plain
    read-modify-write (mode 1, a floor for any ordered scheme) and by plain
    stores (mode 2)."""
    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "io_aware_exact_amd")
    L = ctypes.CDLL(os.path.join(here, "libfa_probe.so"))
    L.fa_probe_dq_accum.restype = ctypes.c_int
    L.fa_probe_dq_accum.argtypes = [ctypes.c_void_p] + [ctypes.c_int] * 5 + [ctypes.c_void_p]
    B, H, S, d = 2, 16, 8192, 128
    acc = torch.zeros((B * H, S, d), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def run(mode):
        rc = L.fa_probe_dq_accum(acc.data_ptr(), B, H, S, d, mode, ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"fa_probe_dq_accum returned {rc}")
    run(0)
    torch.cuda.synchronize()
    ok = bool((acc == S // 128).all().item())
    partial_bytes = B * H * (S // 128) * (S // 64) * 64 * d * 4     # bytes of partials added
    out = {"workload": "dQ partial adds of a fused backward, B=2 H=16 S=8192 d=128 (2048 workgroups x 128 tiles x 32 KB)",
           "partial_bytes": partial_bytes, "atomic_result_exact": ok}
    for mode, name in ((0, "atomic_add"), (1, "plain_rmw"), (2, "plain_store")):
        t = time_calls(lambda: run(mode), reps)
        out[name] = {"ms": round(t["mean"], 4), "partial_gbps": round(partial_bytes / t["mean"] / 1e6, 1),
                     "timing": timing(t)}
    return out


def leg_hbmread(reps):
    """The box's sustained HBM read rate, measured with a plain streaming
    kernel (measurement probe `libfa_probe.so`, not part of the path): 8 GiB
    of random bytes read once per launch in 16-byte loads, ordinary and
    non-temporal, 4 to 16 loads in flight per thread, over several grid
    sizes.  The practical ceiling the
    HBM-bound decode kernel is compared with."""
    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "io_aware_exact_amd")
    L = ctypes.CDLL(os.path.join(here, "libfa_probe.so"))
    L.fa_probe_hbm_read.restype = ctypes.c_int
    L.fa_probe_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_uint64,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    nbytes = 8 << 30
    g = torch.Generator(device="cuda")
    g.manual_seed(6)
    buf = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)
    grids = (2048, 4096, 8192, 16384, 32768)
    out = torch.empty(max(grids) * 256, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def run(grid, mode):
        rc = L.fa_probe_hbm_read(buf.data_ptr(), nbytes, out.data_ptr(), out.numel(), grid, mode,
                                 ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"fa_probe_hbm_read returned {rc}")
    res = {"workload": "HBM read of 8 GiB, 16-byte loads (plain streaming kernel)", "bytes": nbytes, "runs": {}}
    best = None
    for mode, name in ((0, "plain_u4"), (1, "nontemporal_u4"), (2, "nontemporal_u8"), (3, "nontemporal_u16")):
        for grid in grids:
            t = time_calls(lambda: run(grid, mode), reps)
            gbps = nbytes / t["median"] / 1e6
            res["runs"][f"{name}_grid{grid}"] = {"median_ms": round(t["median"], 4), "gbps": round(gbps, 1)}
            if best is None or gbps > best[0]:
                best = (gbps, f"{name}_grid{grid}")
    res["best_gbps"] = round(best[0], 1)
    res["best_run"] = best[1]
    res["best_frac_of_hbm"] = round(best[0] / PEAK_HBM_GBPS, 4)
    del buf
    return res


def leg_fixedcost(reps):
    """Fixed cost per launch of the three main kernels: each timed at B=2,
    H=16, d=128, non-causal with the other length 8192 and the swept one at
    1024..8192 (forward and dQ: key length; dK/dV: query length), and a
    least-squares line through the medians.  The intercept is the part of a
    launch that does not scale with the sweep (workgroup start-up, operand
    loads before the loop, pipeline fill and drain, stores), paid once per
    round of workgroups."""
    from io_aware_exact_amd import fa, inputs
    B, H, d, S = 2, 16, 128, 8192
    out = {"workload": "B=2 H=16 d=128 non-causal, one length 8192, the other 1024..8192"}
    for name in ("fwd", "dkdv", "dq"):
        xs, ys = [], []
        for L in (1024, 2048, 4096, 8192):
            Sq, Sk = (S, L) if name in ("fwd", "dq") else (L, S)
            q, k, v, do = inputs.qkv(B, Sq, Sk, H, H, d, 1234, device="cuda", with_dout=True)
            o = torch.empty_like(q)
            lse = torch.empty((B, H, Sq), dtype=torch.float32, device="cuda")
            fa.fwd(q, k, v, False, out=o, lse=lse)
            grads = tuple(torch.empty_like(x) for x in (q, k, v))
            a = fa.bwd_args(q, k, v, o, do, lse, *grads, False, None)
            ws = torch.empty(int(fa.lib().fa_bwd_workspace_size(ctypes.byref(a))), dtype=torch.uint8,
                             device="cuda")
            fa.bwd(q, k, v, o, do, lse, False, out=grads, workspace=ws)
            if name == "fwd":
                fn = lambda: fa.fwd(q, k, v, False, out=o, lse=lse)
            else:
                st = fa.FA_BWD_DKDV if name == "dkdv" else fa.FA_BWD_DQ
                fn = lambda: fa.bwd(q, k, v, o, do, lse, False, out=grads, workspace=ws, stages=st)
            t = time_calls(fn, reps)["median"]
            xs.append(L)
            ys.append(t)
        n = len(xs)
        mx, my = sum(xs) / n, sum(ys) / n
        slope = sum((x - mx) * (y - my) for x, y in zip(xs, ys)) / sum((x - mx) ** 2 for x in xs)
        out[name] = {"lengths": xs, "median_ms": [round(y, 4) for y in ys],
                     "intercept_us": round((my - slope * mx) * 1e3, 1), "us_per_1024": round(slope * 1024 * 1e3, 1)}
        del q, k, v, do, o, grads, ws
        torch.cuda.empty_cache()
    return out


def leg_main(reps, with_bwd):
    """The main workload alone (B=2, H=16, S=8192, d=128, non-causal): fwd, or
    fwd then bwd, reps times -- for profiling."""
    from io_aware_exact_amd import fa, inputs
    W = WORKLOAD
    B, S, H, d, causal = W["B"], W["S"], W["H"], W["d"], W["causal"]
    q, k, v, do = inputs.qkv(B, S, S, H, H, d, W["seed"], device="cuda", with_dout=True)
    o = torch.empty((B, S, H, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
    grads = tuple(torch.empty_like(x) for x in (q, k, v))
    a = fa.bwd_args(q, k, v, o, do, lse, *grads, causal, None)
    ws = torch.empty(int(fa.lib().fa_bwd_workspace_size(ctypes.byref(a))), dtype=torch.uint8,
                     device="cuda")

    def step():
        fa.fwd(q, k, v, causal, out=o, lse=lse)
        if with_bwd:
            fa.bwd(q, k, v, o, do, lse, causal, out=grads, workspace=ws)
    t = time_calls(step, reps)
    ms = t["mean"]
    ff = fwd_flops(B, S, S, H, d, causal) * (3.5 if with_bwd else 1.0)
    return {"ms": round(ms, 4), "tflops": round(ff / ms / 1e9, 2), "timing": timing(t)}


def extra_legs(args, keep_rows=None):
    out = {}
    if args.only in ("fwd", "fwdbwd"):
        return {args.only: leg_main(args.steps, args.only == "fwdbwd")}
    for name, fn, reps in (("gemm", leg_gemm, 20), ("hbmread", leg_hbmread, 20), ("dqaccum", leg_dqaccum, 20),
                           ("fixedcost", leg_fixedcost, 20),
                           ("causal", leg_causal, 20),
                           ("decode", leg_decode, 20),
                           ("varlen", leg_varlen, 20), ("kvcache", leg_kvcache, 20),
                           ("fp8", leg_fp8, 20),
                           ("sweep", leg_sweep, 20)):
        if args.only and args.only != name:
            continue
        out[name] = fn(reps, keep_rows) if name == "fp8" else fn(reps)
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the secondary workloads (causal, decode, varlen)")
    ap.add_argument("--only", choices=["decode", "varlen", "kvcache", "causal", "fp8", "sweep", "fwd",
                                       "fwdbwd", "gemm", "dqaccum", "hbmread", "fixedcost"],
                    help="run one secondary workload alone (for profiling)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (3 launches), the reference "
                         "for scaling HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(batch and heads shard with no exchange, so N GPUs run N copies of this step)",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        x = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": x.numel() * 4,
                          "copy_calibration_bytes_written": y.numel() * 4, "launches": 3}))
        return
    from io_aware_exact_amd import fa, inputs
    fa.lib()
    if args.only:
        print(json.dumps(extra_legs(args)), flush=True)
        return

    W = WORKLOAD
    B, S, H, d, causal = W["B"], W["S"], W["H"], W["d"], W["causal"]
    q, k, v, do = inputs.qkv(B, S, S, H, H, d, W["seed"], device="cuda", with_dout=True)
    o = torch.empty((B, S, H, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
    grads = tuple(torch.empty((B, S, H, d), dtype=torch.bfloat16, device="cuda") for _ in range(3))
    a = fa.bwd_args(q, k, v, o, do, lse, *grads, causal, None)
    ws = torch.empty(max(1, int(fa.lib().fa_bwd_workspace_size(ctypes.byref(a)))),
                     dtype=torch.uint8, device="cuda")

    def step():
        fa.fwd(q, k, v, causal, out=o, lse=lse)
        fa.bwd(q, k, v, o, do, lse, causal, out=grads, workspace=ws)

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # exactly args.steps steps between two synchronisations; an event after
    # each step also gives the per-step median and minimum
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev[0].elapsed_time(ev[args.steps]) / args.steps
    per_step = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))

    # each kernel of the step alone, launched back to back on the same stream
    # (one launch per call: fa_fwd, and fa_bwd restricted to one stage; the
    # workspace already holds D from the step above)
    reps = max(args.steps, 20)
    t_fwd = time_calls(lambda: fa.fwd(q, k, v, causal, out=o, lse=lse), reps)
    t_pre = time_calls(lambda: fa.bwd(q, k, v, o, do, lse, causal, out=grads, workspace=ws,
                                      stages=fa.FA_BWD_PREPROCESS), reps)
    t_dkdv = time_calls(lambda: fa.bwd(q, k, v, o, do, lse, causal, out=grads, workspace=ws,
                                       stages=fa.FA_BWD_DKDV), reps)
    t_dq = time_calls(lambda: fa.bwd(q, k, v, o, do, lse, causal, out=grads, workspace=ws,
                                     stages=fa.FA_BWD_DQ), reps)
    ms_fwd, ms_pre, ms_dkdv, ms_dq = t_fwd["mean"], t_pre["mean"], t_dkdv["mean"], t_dq["mean"]

    ff = fwd_flops(B, S, S, H, d, causal)
    gemm = ff / 2                       # one GEMM-shaped product: 2*B*H*Sq*Sk*d
    step_flops = 3.5 * ff
    value = step_flops / (ms_step * 1e-3) / 1e12

    def tf(flops, ms):
        return round(flops / ms / 1e9, 2)

    kernels = {
        "fwd_bf16_pp_kernel": {"ms": round(ms_fwd, 4), "algorithmic_tflops": tf(2 * gemm, ms_fwd),
                               "timing": timing(t_fwd)},
        "bwd_preprocess_kernel": {"ms": round(ms_pre, 4), "timing": timing(t_pre)},
        "bwd_dkdv_kernel": {"ms": round(ms_dkdv, 4), "algorithmic_tflops": tf(4 * gemm, ms_dkdv),
                            "timing": timing(t_dkdv)},
        "bwd_dq_kernel": {"ms": round(ms_dq, 4), "algorithmic_tflops": tf(gemm, ms_dq),
                          "executed_tflops": tf(3 * gemm, ms_dq), "timing": timing(t_dq)},
    }
    dk_tf = 4 * gemm / ms_dkdv / 1e9

    line = {
        "metric": "attention fwd+bwd TFLOP/s (bf16, d=128)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "step_median_ms": round(per_step[len(per_step) // 2], 4),
        "step_min_ms": round(per_step[0], 4),
        "wall_s": round(wall, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic iid N(0,1), seed 2000",
        "config": {"workload": f"exact attention fwd+bwd, B={B} H={H} Sq=Sk={S} d={d} non-causal",
                   "B": B, "H": H, "Sq": S, "Sk": S, "d": d, "causal": causal},
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "fwd": {"tflops": tf(ff, ms_fwd), "ms": round(ms_fwd, 4),
                "frac_of_peak": round(ff / ms_fwd / 1e9 / PEAK_BF16_TFLOPS, 4)},
        "kernels": kernels,
        "roofline": {"kernel": "bwd_dkdv_kernel<128,false,false>", "bound": "mfma",
                     "achieved": round(dk_tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(dk_tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_from_profile("bwd_dkdv_b2_h16_s8192_d128", BWD_SOURCES)},
        "roofline_fwd": {"kernel": "fwd_bf16_pp_kernel<128,false,false,0>", "bound": "mfma",
                         "achieved": tf(ff, ms_fwd), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(ff / ms_fwd / 1e9 / PEAK_BF16_TFLOPS, 4),
                         "traffic": traffic_from_profile("fwd_bf16_b2_h16_s8192_d128", FWD_SOURCES)},
    }
    keep = {} if not args.no_cpu_baseline else None
    if not args.no_extra:
        line["extra"] = extra_legs(args, keep)
    if not args.no_cpu_baseline:
        line.update(cpu_baseline_leg(q, k, v, do, o, lse, causal, keep.get("rows")))
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

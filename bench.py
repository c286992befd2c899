#!/usr/bin/env python3
"""Benchmark of the LLM.int8() decomposition matmul on one MI355X.

A step is one llmint8_matmul call (outlier detection, row quantization, the
int8 MFMA GEMM with the fused dequantize + fp16 outlier epilogue) on the
6.7B-style FFN fc1 shape: X [4096,4096] fp16 with 6 outlier feature dims
holding +-U(20,60) in 75 % of rows, W [4096,16384] as int8 CB + SCB (quantized
once before timing, as the method does when the weight is loaded),
threshold 6.0.  Inputs are seeded and synthetic and resident in HBM before the
timed region.

Before its warmup steps, each timed loop runs untimed calls of its step for
settle_ms (40 ms) of wall time, so that the power-managed clock has settled
(a sustained MFMA load first drives it through a ~15 ms dip).

The JSON line also carries:
  roofline      the GEMM kernel's own duration (HIP events recorded around its
                launch on the stream it runs on, in a second pass of the same
                steps right after the timed ones) against the dense int8 MFMA
                peak, and beside it the measured MFMA ceiling on the
                workload's own operands (the clock is power-managed under a
                sustained MFMA load);
  cpu_baseline  the plain CPU oracle timed on a bounded sample of the same work;
  decode        the weight-streaming kernel at T in {1,4,16}, K=12288, N=49152
                (604 MB of CB, two copies rotated), against HBM bandwidth;
  configs       the other workloads: the 1.3B-style up-projection, fc2 of the
                FFN pair on fc1's real ReLU'd output and the pair as one step,
                and the attention-projection sweep (--no-configs skips them).
"""
import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

INT8_PEAK_TOPS = 5000.0      # MI355X dense int8 MFMA, TOP/s
FP16_PEAK_TFLOPS = 2500.0    # MI355X dense fp16 MFMA, TFLOP/s
FP8_PEAK_TFLOPS = 5000.0     # MI355X dense fp8 MFMA, TFLOP/s
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def profiled_traffic(summary, key="traffic_bytes_per_launch"):
    """HBM bytes per launch from a committed rocprofv3 counter summary in profiles/.

    The summary records a hash of the kernel's sources; when the sources have
    changed since the counters were taken the figure no longer describes the
    kernel and None is returned."""
    import hashlib
    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    try:
        want, files = fields["kernel_sources_sha256_16"].split(None, 1)
        h = hashlib.sha256()
        for f in files.strip("()").split():
            h.update(open(os.path.join(ROOT, f), "rb").read())
        if h.hexdigest()[:16] != want:
            return None
        return int(fields[key].split()[0])   # a figure may carry a note after it
    except (KeyError, ValueError, IndexError, OSError):
        return None


class HipEvents:
    """hipEvent_t handles through the HIP runtime torch has already loaded.

    Created with hipEventDisableSystemFence: they only time the kernel they
    bracket, and a default event record performs a system-scope cache
    writeback and invalidation that holds up the next kernel by several
    microseconds (which would land in the timed steps)."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.made = []

    def create(self):
        e = ctypes.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError("hipEventCreateWithFlags failed: %d" % rc)
        self.made.append(e.value)
        return e.value

    def record(self, e, stream):
        rc = self.hip.hipEventRecord(ctypes.c_void_p(e), ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError("hipEventRecord failed: %d" % rc)

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed: %d" % rc)
        return float(ms.value)

    def close(self):
        for e in self.made:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))
        self.made = []


# Wall time of untimed calls of a step before its warmup steps (--settle-ms).
# The GPU's power manager answers a sudden sustained MFMA load with a dip:
# fc1 GEMMs run at ~245 us for about ten calls, slow to 300-325 us, and
# settle near 255 us after about sixty (measured: 280.5 us per step timed
# right after 10 warmup steps, 258.1 after 60, 255.9 after 200, and 258.2
# over 500 steps timed from the start).  Settling first makes the timed steps
# and the kernel-event pass after them see the same, sustained clock.
SETTLE_MS = 40.0


def settle(torch, fn):
    """Untimed calls of fn (batches of 8, each synchronized) for SETTLE_MS of
    wall time; returns the number of calls."""
    n = 0
    if SETTLE_MS <= 0:
        return n
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < SETTLE_MS:
        for _ in range(8):
            fn()
        n += 8
        torch.cuda.synchronize()
    return n


def timed_steps(torch, L, X, CBs, SCB, thr, out, ws, steps, warmup, ev, extra=None):
    """`warmup` untimed steps, `steps` timed ones (plain llmint8_matmul calls), then
    `steps` more with HIP events recorded around the main kernel on its stream.
    An event record between two kernels holds the second back by a few
    microseconds, so the events stay out of the timed steps.  Returns
    (ms per step, mean main-kernel ms, per-launch main-kernel ms).  With a
    dict `extra`, the second pass also records an event before each call:
    extra["step_ms"] and extra["pre_ms"] get each call's time from it to the
    end of the main kernel and to its start (the quantization kernels plus
    the one event record's gap), in the same pass as the kernel times."""
    settle(torch, lambda: L.llmint8_matmul(X, CBs[0], SCB, thr, out=out, ws=ws))
    for i in range(warmup):
        L.llmint8_matmul(X, CBs[i % len(CBs)], SCB, thr, out=out, ws=ws)
    pairs = [(ev.create(), ev.create()) for _ in range(steps)]
    pre = [ev.create() for _ in range(steps)] if extra is not None else None
    stream = torch.cuda.current_stream(X.device).cuda_stream
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        L.llmint8_matmul(X, CBs[i % len(CBs)], SCB, thr, out=out, ws=ws)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(steps):
        if pre is not None:
            ev.record(pre[i], stream)
        L.llmint8_matmul_path(X, CBs[i % len(CBs)], SCB, thr, out=out, ws=ws, path=L.PATH_AUTO,
                              main_start=pairs[i][0], main_stop=pairs[i][1])
    torch.cuda.synchronize()
    kern = [ev.elapsed_ms(a, b) for a, b in pairs]
    if pre is not None:
        extra["step_ms"] = [ev.elapsed_ms(p, b) for p, (a, b) in zip(pre, pairs)]
        extra["pre_ms"] = [ev.elapsed_ms(p, a) for p, (a, b) in zip(pre, pairs)]
    return (t1 - t0) * 1e3 / steps, float(np.mean(kern)), kern


def spread_us(kern_ms):
    """Median and p10/p90 of per-launch kernel times, in microseconds."""
    q = np.percentile(np.asarray(kern_ms) * 1e3, [50, 10, 90])
    return {"kernel_us_median": round(float(q[0]), 2), "kernel_us_p10": round(float(q[1]), 2),
            "kernel_us_p90": round(float(q[2]), 2)}


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(X, W_t, thr, rows):
    import oracle
    CBh, SCBh = oracle.quantize_weight(W_t)
    sel = np.arange(rows)
    t0 = time.perf_counter()
    oracle.matmul(X, CBh, SCBh, thr, rows=sel)
    dt = time.perf_counter() - t0
    T, K = X.shape
    N = W_t.shape[0]
    return {"value": 2.0 * rows * K * N / dt / 1e12, "unit": "TOP/s", "cores": oracle.num_threads(),
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": "rows 0..%d of X (%d of %d) against all %d output columns; the outlier set is "
                      "found from all rows; %.1f s wall" % (rows - 1, rows, T, N, dt)}


def decode_bench(torch, L, workloads, steps, warmup, ev, dev):
    log("decode: generating W [12288,49152] ...")
    d1 = workloads.decode_175b(1, with_weight=True)
    W = torch.from_numpy(d1.pop("W_t")).to(dev)
    CB, SCB = L.llmint8_quantize_weight(W)
    del W
    CB2 = CB.clone()                 # rotate two copies: 2 x 604 MB, beyond the 256 MB MALL
    torch.cuda.synchronize()
    K, N = CB.shape[1], CB.shape[0]
    res = {}
    for T in (1, 4, 16):
        d = d1 if T == 1 else workloads.decode_175b(T, with_weight=False)
        X = torch.from_numpy(d["X"]).to(dev)
        out = torch.empty((T, N), dtype=torch.float16, device=dev)
        ws = torch.empty((L.llmint8_workspace_bytes(T, K, N),), dtype=torch.uint8, device=dev)
        ms, kms, kern = timed_steps(torch, L, X, [CB, CB2], SCB, 6.0, out, ws, steps, warmup, ev)
        alg = K * N + 4 * N + T * K + 4 * T + 2 * T * N
        res["T%d" % T] = {"kernel_us": round(kms * 1e3, 2), "step_us": round(ms * 1e3, 2),
                          "kernel_GBs": round(alg / (kms * 1e-3) / 1e9, 1),
                          "step_GBs": round(alg / (ms * 1e-3) / 1e9, 1),
                          "frac_hbm": round(alg / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                          "alg_bytes": alg,
                          "traffic": profiled_traffic("k_decode_175b_fc1.txt",
                                                      "traffic_bytes_per_launch_T%d" % T)}
        res["T%d" % T].update(spread_us(kern))
        log("decode T=%d: kernel %.1f us (%.0f GB/s), step %.1f us" % (T, kms * 1e3, alg / kms / 1e6, ms * 1e3))
    return res


def ffn_pair(torch, L, d, steps, warmup, ev, dev, entry):
    """The 6.7B-style FFN: fc1 (X [4096,4096] -> [4096,16384]) with the ReLU
    fused into its output, then fc2 ([4096,16384] -> [4096,4096]) on that
    output, both through the decomposition at threshold 6.  Returns the fc2
    call on its own (on the ReLU'd fc1 output: most of its columns hold a
    value above 6, so the fp16 outlier product dominates; with the fp16 MFMA
    ceiling on fc2's own operands, X = that output and W2 in fp16) and the
    pair as one step (2*T*K*N ops per layer), also with the ReLU as a
    separate torch pass between the layers, for the cost of the unfused
    chain."""
    X = torch.from_numpy(d["X"]).to(dev)
    CB1, SCB1 = L.llmint8_quantize_weight(torch.from_numpy(d["W_t"]).to(dev))
    W2 = torch.from_numpy(d["W2_t"]).to(dev)
    CB2, SCB2 = L.llmint8_quantize_weight(W2)
    T, D = X.shape
    F = CB1.shape[0]
    h = torch.empty((T, F), dtype=torch.float16, device=dev)
    y = torch.empty((T, D), dtype=torch.float16, device=dev)
    ws = torch.empty((max(L.llmint8_workspace_bytes(T, D, F), L.llmint8_workspace_bytes(T, F, D)),),
                     dtype=torch.uint8, device=dev)
    L.llmint8_matmul_act(X, CB1, SCB1, 6.0, L.ACT_RELU, out=h, ws=ws)
    n2 = int(L.llmint8_quantize_act(h, 6.0)[3].cpu()[0])
    ms, kms, _ = timed_steps(torch, L, h, [CB2], SCB2, 6.0, y, ws, steps, warmup, ev)
    fc2 = entry(T, F, D, 6.0, n2, ms, kms)
    fc2["input"] = "the fc1 output of this workload with the ReLU fused (llmint8_matmul_act)"
    fc2["step_frac_fp16_peak"] = round(2.0 * T * F * D / (ms * 1e-3) / 1e12 / FP16_PEAK_TFLOPS, 4)
    ceil16 = mfma_ceiling(torch, L, h, W2, ev)
    fc2["fp16_mfma_ceiling_TFLOPS"] = round(ceil16, 1)
    log("config ffn_6p7b_fc2 (on the ReLU'd fc1 output): n=%d step %.1f us (%.0f TOP/s); "
        "fp16 MFMA ceiling on its operands %.0f TFLOP/s" % (n2, ms * 1e3, 2.0 * T * F * D / ms / 1e9,
                                                             ceil16))
    del W2

    def fused():
        L.llmint8_matmul_act(X, CB1, SCB1, 6.0, L.ACT_RELU, out=h, ws=ws)
        L.llmint8_matmul(h, CB2, SCB2, 6.0, out=y, ws=ws)

    def unfused():
        L.llmint8_matmul(X, CB1, SCB1, 6.0, out=h, ws=ws)
        torch.relu_(h)
        L.llmint8_matmul(h, CB2, SCB2, 6.0, out=y, ws=ws)

    def per_step(fn):
        settle(torch, fn)
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps

    s_f = per_step(fused)
    s_u = per_step(unfused)
    ops = 2.0 * T * D * F * 2
    pair = {"T": T, "D": D, "F": F, "threshold": 6.0, "fc2_n_outliers": n2,
            "step_us": round(s_f * 1e6, 2), "step_TOPS": round(ops / s_f / 1e12, 1),
            "step_frac_int8_peak": round(ops / s_f / 1e12 / INT8_PEAK_TOPS, 4),
            "unfused_step_us": round(s_u * 1e6, 2)}
    log("config ffn_6p7b_pair: fc1+ReLU+fc2 %.1f us (%.0f TOP/s), ReLU as a separate pass %.1f us"
        % (s_f * 1e6, ops / s_f / 1e12, s_u * 1e6))
    del X, CB1, SCB1, CB2, SCB2, h, y, ws
    torch.cuda.empty_cache()
    return {"ffn_6p7b_fc2": fc2, "ffn_6p7b_pair": pair}


def fp16_weight_step(torch, L, d, steps, warmup, dev):
    """fc1 with the weight kept in fp16 (has_fp16_weights=True): every step
    quantizes W [16384,4096] (llmint8_quantize_weight) before the matmul."""
    X = torch.from_numpy(d["X"]).to(dev)
    W = torch.from_numpy(d["W_t"]).to(dev)
    N, K = W.shape
    T = X.shape[0]
    CB = torch.empty((N, K), dtype=torch.int8, device=dev)
    SCB = torch.empty((N,), dtype=torch.float32, device=dev)
    out = torch.empty((T, N), dtype=torch.float16, device=dev)
    ws = torch.empty((L.llmint8_workspace_bytes(T, K, N),), dtype=torch.uint8, device=dev)

    def step():
        L.llmint8_quantize_weight(W, CB=CB, SCB=SCB)
        L.llmint8_matmul(X, CB, SCB, 6.0, out=out, ws=ws)

    settle(torch, step)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    s = (time.perf_counter() - t0) / steps
    ops = 2.0 * T * K * N
    wbytes = 3.0 * N * K + 4 * N    # quantization reads 2 B and writes 1 B per weight
    log("config ffn_6p7b_fc1_fp16_weights: quantize W + matmul %.1f us (%.0f TOP/s)"
        % (s * 1e6, ops / s / 1e12))
    del X, W, CB, SCB, out, ws
    torch.cuda.empty_cache()
    return {"T": T, "K": K, "N": N, "threshold": 6.0, "step_us": round(s * 1e6, 2),
            "step_TOPS": round(ops / s / 1e12, 1), "weight_quant_bytes": wbytes}


def timed_calls(torch, plain, evented, steps, warmup, ev):
    """timed_steps for any entry point: plain(i) is one call, evented(i, e0,
    e1) the same call with events around its main kernel."""
    settle(torch, lambda: plain(0))
    for i in range(warmup):
        plain(i)
    pairs = [(ev.create(), ev.create()) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        plain(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(steps):
        evented(i, pairs[i][0], pairs[i][1])
    torch.cuda.synchronize()
    kern = [ev.elapsed_ms(a, b) for a, b in pairs]
    return (t1 - t0) * 1e3 / steps, float(np.mean(kern)), kern


def zeropoint_bench(torch, L, workloads, steps, warmup, ev, dev):
    """The zero-point (asymmetric) variant on the same workloads: fc1 (the
    GEMM path; k_gemm with the shifted-product epilogue) and the 175B decode
    shape at T in {1, 4, 16} (the weight-streaming kernel; two weight copies
    rotated).  Same ops and algorithmic bytes as the absmax lines, plus the
    per-column zp and code sums (8 B per column)."""
    res = {}
    d = workloads.ffn_6p7b(with_fc2=False)
    X = torch.from_numpy(d["X"]).to(dev)
    CB, ND, ZP, RS = L.llmint8_quantize_weight_zp(torch.from_numpy(d["W_t"]).to(dev))
    T, K = X.shape
    N = CB.shape[0]
    out = torch.empty((T, N), dtype=torch.float16, device=dev)
    ws = torch.empty((L.llmint8_workspace_bytes(T, K, N),), dtype=torch.uint8, device=dev)
    ms, kms, kern = timed_calls(
        torch, lambda i: L.llmint8_matmul_zp(X, CB, ND, ZP, RS, 6.0, out=out, ws=ws),
        lambda i, a, b: L.llmint8_matmul_zp_path(X, CB, ND, ZP, RS, 6.0, out=out, ws=ws,
                                                 main_start=a, main_stop=b),
        steps, warmup, ev)
    ops = 2.0 * T * K * N
    res["fc1"] = {"T": T, "K": K, "N": N, "threshold": 6.0, "step_us": round(ms * 1e3, 2),
                  "step_TOPS": round(ops / (ms * 1e-3) / 1e12, 1),
                  "gemm_kernel_us": round(kms * 1e3, 2),
                  "gemm_frac_int8_peak": round(ops / (kms * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4)}
    res["fc1"].update(spread_us(kern))
    log("zero-point fc1: %.1f us/step (%.0f TOP/s), GEMM kernel %.1f us (%.1f%% of int8 peak)"
        % (ms * 1e3, ops / ms / 1e9, kms * 1e3, 100 * ops / (kms * 1e-3) / 1e12 / INT8_PEAK_TOPS))
    del X, CB, ND, ZP, RS, out, ws, d
    torch.cuda.empty_cache()

    d1 = workloads.decode_175b(1, with_weight=True)
    CB, ND, ZP, RS = L.llmint8_quantize_weight_zp(torch.from_numpy(d1.pop("W_t")).to(dev))
    CBs = [CB, CB.clone()]
    K, N = CB.shape[1], CB.shape[0]
    for T in (1, 4, 16):
        dd = d1 if T == 1 else workloads.decode_175b(T, with_weight=False)
        X = torch.from_numpy(dd["X"]).to(dev)
        out = torch.empty((T, N), dtype=torch.float16, device=dev)
        ws = torch.empty((L.llmint8_workspace_bytes(T, K, N),), dtype=torch.uint8, device=dev)
        ms, kms, kern = timed_calls(
            torch, lambda i: L.llmint8_matmul_zp(X, CBs[i % 2], ND, ZP, RS, 6.0, out=out, ws=ws),
            lambda i, a, b: L.llmint8_matmul_zp_path(X, CBs[i % 2], ND, ZP, RS, 6.0, out=out,
                                                     ws=ws, main_start=a, main_stop=b),
            steps, warmup, ev)
        alg = K * N + 12 * N + T * K + 12 * T + 2 * T * N
        res["decode_T%d" % T] = {"kernel_us": round(kms * 1e3, 2), "step_us": round(ms * 1e3, 2),
                                 "kernel_GBs": round(alg / (kms * 1e-3) / 1e9, 1),
                                 "frac_hbm": round(alg / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                 "alg_bytes": alg}
        res["decode_T%d" % T].update(spread_us(kern))
        log("zero-point decode T=%d: kernel %.1f us (%.0f GB/s), step %.1f us"
            % (T, kms * 1e3, alg / kms / 1e6, ms * 1e3))
    del CBs, CB, ND, ZP, RS
    torch.cuda.empty_cache()
    return res


def fp8_bench(torch, L, workloads, steps, warmup, ev, dev, fmt="f8"):
    """The FP8 variant (fmt "f8": E5M2, "e4m3": E4M3) on the same workloads:
    fc1 (the GEMM path, v_mfma_f32_32x32x64_f8f6f4; roofline: the dense fp8
    peak, 5.0 PFLOP/s) and the 175B decode shape at T in {1, 4, 16} (two
    weight copies rotated; the same algorithmic bytes as the int8 weight
    stream)."""
    qw = getattr(L, "llmint8_quantize_weight_" + fmt)
    mm = getattr(L, "llmint8_matmul_" + fmt)
    mmp = getattr(L, "llmint8_matmul_%s_path" % fmt)
    tag = "fp8" if fmt == "f8" else fmt
    res = {}
    d = workloads.ffn_6p7b(with_fc2=False)
    X = torch.from_numpy(d["X"]).to(dev)
    CB8, SC8 = qw(torch.from_numpy(d["W_t"]).to(dev))
    T, K = X.shape
    N = CB8.shape[0]
    out = torch.empty((T, N), dtype=torch.float16, device=dev)
    ws = torch.empty((L.llmint8_workspace_bytes(T, K, N),), dtype=torch.uint8, device=dev)
    ms, kms, kern = timed_calls(
        torch, lambda i: mm(X, CB8, SC8, 6.0, out=out, ws=ws),
        lambda i, a, b: mmp(X, CB8, SC8, 6.0, out=out, ws=ws, main_start=a, main_stop=b),
        steps, warmup, ev)
    ops = 2.0 * T * K * N
    res["fc1"] = {"T": T, "K": K, "N": N, "threshold": 6.0, "step_us": round(ms * 1e3, 2),
                  "step_TFLOPS": round(ops / (ms * 1e-3) / 1e12, 1),
                  "gemm_kernel_us": round(kms * 1e3, 2),
                  "gemm_frac_fp8_peak": round(ops / (kms * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 4)}
    res["fc1"].update(spread_us(kern))
    log("%s fc1: %.1f us/step (%.0f TFLOP/s), GEMM kernel %.1f us (%.1f%% of the fp8 peak)"
        % (tag, ms * 1e3, ops / ms / 1e9, kms * 1e3, 100 * ops / (kms * 1e-3) / 1e12 / FP8_PEAK_TFLOPS))
    del X, CB8, SC8, out, ws, d
    torch.cuda.empty_cache()

    d1 = workloads.decode_175b(1, with_weight=True)
    CB8, SC8 = qw(torch.from_numpy(d1.pop("W_t")).to(dev))
    CBs = [CB8, CB8.clone()]
    K, N = CB8.shape[1], CB8.shape[0]
    for T in (1, 4, 16):
        dd = d1 if T == 1 else workloads.decode_175b(T, with_weight=False)
        X = torch.from_numpy(dd["X"]).to(dev)
        out = torch.empty((T, N), dtype=torch.float16, device=dev)
        ws = torch.empty((L.llmint8_workspace_bytes(T, K, N),), dtype=torch.uint8, device=dev)
        ms, kms, kern = timed_calls(
            torch, lambda i: mm(X, CBs[i % 2], SC8, 6.0, out=out, ws=ws),
            lambda i, a, b: mmp(X, CBs[i % 2], SC8, 6.0, out=out, ws=ws, main_start=a,
                                main_stop=b),
            steps, warmup, ev)
        alg = K * N + 4 * N + T * K + 4 * T + 2 * T * N
        res["decode_T%d" % T] = {"kernel_us": round(kms * 1e3, 2), "step_us": round(ms * 1e3, 2),
                                 "kernel_GBs": round(alg / (kms * 1e-3) / 1e9, 1),
                                 "frac_hbm": round(alg / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                 "alg_bytes": alg}
        res["decode_T%d" % T].update(spread_us(kern))
        log("%s decode T=%d: kernel %.1f us (%.0f GB/s), step %.1f us"
            % (tag, T, kms * 1e3, alg / kms / 1e6, ms * 1e3))
    del CBs, CB8, SC8
    torch.cuda.empty_cache()
    return res


def mfma_ceiling(torch, L, A, B, ev, blocks=1024, iters=128, reps=10):
    """The MFMA rate on A's and B's own bits (see llmint8_mfma_ceiling): 3 warm-up
    launches, then `reps` timed back to back, each bracketed by HIP events on
    its stream; returns ops (or flops) per second of the mean launch, in 1e12."""
    settle(torch, lambda: L.llmint8_mfma_ceiling(A, B, blocks, iters))
    for _ in range(3):
        L.llmint8_mfma_ceiling(A, B, blocks, iters)
    pairs = [(ev.create(), ev.create()) for _ in range(reps)]
    ops = 0.0
    for a, b in pairs:
        _, ops = L.llmint8_mfma_ceiling(A, B, blocks, iters, start=a, stop=b)
    torch.cuda.synchronize()
    ms = float(np.mean([ev.elapsed_ms(a, b) for a, b in pairs]))
    return ops / (ms * 1e-3) / 1e12


def configs_bench(torch, L, workloads, steps, warmup, ev, dev):
    """The other workloads, each timed like the main one (step = one
    llmint8_matmul call; 2*T*K*N ops): the 1.3B-style up-projection, the
    6.7B-style FFN pair (fc1 with the ReLU fused into its output, then fc2 on
    that very output, so fc2 sees the outlier set a real ReLU'd fc1 output
    has), fc1 with its weight quantized in every step (fp16 weights kept) and
    the attention-projection sweep (outlier dims n in {0,6,32,128}, threshold
    0 and inf, T = 4095).  The GEMM kernel's own time (HIP events) is given
    where k_gemm does the work (up to 32 outlier columns); past that the
    work is in the many-outlier kernel and the step time is the figure."""
    res = {}

    def entry(T, K, N, thr, n, ms, kms):
        ops = 2.0 * T * K * N
        r = {"T": T, "K": K, "N": N, "threshold": thr if np.isfinite(thr) else "inf",
             "n_outliers": n,
             "step_us": round(ms * 1e3, 2), "step_TOPS": round(ops / (ms * 1e-3) / 1e12, 1),
             "step_frac_int8_peak": round(ops / (ms * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4)}
        if n <= 32:
            r["gemm_kernel_us"] = round(kms * 1e3, 2)
            r["gemm_frac_int8_peak"] = round(ops / (kms * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4)
        if n == K:
            r["step_frac_fp16_peak"] = round(ops / (ms * 1e-3) / 1e12 / FP16_PEAK_TFLOPS, 4)
        return r

    def run(name, X_h, W_h, thr):
        X = torch.from_numpy(X_h).to(dev)
        W = torch.from_numpy(W_h).to(dev)
        CB, SCB = L.llmint8_quantize_weight(W)
        del W
        T, K = X.shape
        N = CB.shape[0]
        out = torch.empty((T, N), dtype=torch.float16, device=dev)
        ws = torch.empty((L.llmint8_workspace_bytes(T, K, N),), dtype=torch.uint8, device=dev)
        n = int(L.llmint8_quantize_act(X, thr)[3].cpu()[0])
        ms, kms, _ = timed_steps(torch, L, X, [CB], SCB, thr, out, ws, steps, warmup, ev)
        res[name] = entry(T, K, N, thr, n, ms, kms)
        log("config %s: n=%d step %.1f us (%.0f TOP/s)" % (name, n, ms * 1e3, 2.0 * T * K * N / ms / 1e9))
        del CB, SCB, X, out, ws
        torch.cuda.empty_cache()

    d = workloads.up_proj_1p3b()
    run("up_proj_1p3b", d["X"], d["W_t"], 6.0)
    d = workloads.ffn_6p7b(with_fc2=True)
    res.update(ffn_pair(torch, L, d, steps, warmup, ev, dev, entry))
    res["ffn_6p7b_fc1_fp16_weights"] = fp16_weight_step(torch, L, d, steps, warmup, dev)
    del d
    W5 = workloads.attn_proj_sweep(0)["W_t"]
    for nd in (0, 6, 32, 128):
        run("attn_proj_n%d" % nd, workloads.attn_proj_sweep(nd, with_weight=False)["X"], W5, 6.0)
    X6 = workloads.attn_proj_sweep(6, with_weight=False)["X"]
    run("attn_proj_thr0", X6, W5, 0.0)
    run("attn_proj_thrinf", X6, W5, float("inf"))
    run("attn_proj_T4095", workloads.attn_proj_sweep(6, T=4095, with_weight=False)["X"], W5, 6.0)
    return res


def main():
    global SETTLE_MS
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-rows", type=int, default=4096, help="rows of the CPU-oracle sample (4096 = the whole workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads (1.3B up-proj, the FFN pair's fc2, the attention sweep)")
    ap.add_argument("--config-steps", type=int, default=20,
                    help="timed steps per other workload (at most --steps)")
    ap.add_argument("--fp8", action="store_true",
                    help="also time the FP8 variant, E5M2 and E4M3 (fc1 and the decode shape)")
    ap.add_argument("--zeropoint", action="store_true",
                    help="also time the zero-point variant (fc1 and the decode shape)")
    ap.add_argument("--settle-ms", type=float, default=SETTLE_MS,
                    help="wall time of untimed calls of each timed step before its warmup steps "
                         "(lets the power-managed clock settle; 0: none)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="run one 256 MiB device-to-device copy first (a kernel of known traffic, "
                         "for scaling hardware byte counters)")
    args = ap.parse_args()
    SETTLE_MS = args.settle_ms
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d, WORLD_SIZE %d requested)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import torch
    from int8_quantized_matmul_02_amd import llmint8 as L
    from int8_quantized_matmul_02_amd import workloads

    dev = torch.device("cuda", 0)
    ev = HipEvents()
    if args.copy_calib:
        src = torch.ones((256 << 20,), dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    log("fc1 workload: generating inputs ...")
    d = workloads.ffn_6p7b(with_fc2=False)
    X_h, W_h, thr = d["X"], d["W_t"], d["threshold"]
    X = torch.from_numpy(X_h).to(dev)
    W = torch.from_numpy(W_h).to(dev)
    CB, SCB = L.llmint8_quantize_weight(W)
    del W
    T, K = X.shape
    N = CB.shape[0]
    out = torch.empty((T, N), dtype=torch.float16, device=dev)
    ws = torch.empty((L.llmint8_workspace_bytes(T, K, N),), dtype=torch.uint8, device=dev)
    _, _, _, n_out = L.llmint8_quantize_act(X, thr)
    n_outliers = int(n_out.cpu()[0])

    same_pass = {}
    ms, gemm_ms, gemm_kern = timed_steps(torch, L, X, [CB], SCB, thr, out, ws, args.steps,
                                         args.warmup, ev, extra=same_pass)
    ops = 2.0 * T * K * N
    value = ops / (ms * 1e-3) / 1e12
    achieved = ops / (gemm_ms * 1e-3) / 1e12
    log("fc1: %.1f us/step (%.0f TOP/s), GEMM kernel %.1f us (%.0f TOP/s, %.1f%% of int8 peak)"
        % (ms * 1e3, value, gemm_ms * 1e3, achieved, 100 * achieved / INT8_PEAK_TOPS))

    result = {
        "metric": "int8-decomp matmul TOPS (% int8 MFMA peak) prefill; GB/s (% HBM) decode",
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": SETTLE_MS,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic (seeded fp16 activations with planted outlier dims; random N(0,0.02) weights)",
        "config": {"workload": "6.7B-style FFN fc1: X[4096,4096] fp16, 6 outlier dims +-U(20,60) in 75% "
                               "of rows, W[4096,16384] int8 CB+SCB, threshold 6.0",
                   "T": T, "K": K, "N": N, "threshold": thr, "n_outliers": n_outliers},
        "roofline": {"bound": "mfma", "kernel": "k_gemm_both (int8 MFMA GEMM + fused epilogue; "
                                                 "its many-outlier path is idle at 6 outlier columns)",
                     "achieved": round(achieved, 2), "peak": INT8_PEAK_TOPS, "unit": "TOP/s",
                     "frac": round(achieved / INT8_PEAK_TOPS, 4),
                     "traffic": profiled_traffic("k_gemm_ffn_6p7b_fc1.txt"),
                     "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-calibrated)",
                     "kernel_us": round(gemm_ms * 1e3, 2), "ops_per_launch": ops,
                     "kernel_timing": "HIP events around the kernel on its stream, in a second pass of "
                                      "the same steps (event records add a few us per step, so they "
                                      "stay out of ms_per_step); before the warmup steps, untimed "
                                      "calls for settle_ms of wall time let the power-managed "
                                      "clock settle, so both passes see the sustained clock"},
    }
    result["roofline"].update(spread_us(gemm_kern))
    med = lambda v: round(float(np.median(np.asarray(v) * 1e3)), 2)
    result["roofline"]["same_pass"] = {
        "step_us_median": med(same_pass["step_ms"]),
        "before_kernel_us_median": med(same_pass["pre_ms"]),
        "note": "event before each call to the end / start of k_gemm_both, in the pass that "
                "times the kernel: the quantization kernels and one event record's gap come "
                "before the kernel; the plain steps of ms_per_step ran just before it"}
    Xq = L.llmint8_quantize_act(X, thr)[0]
    ceil8 = mfma_ceiling(torch, L, Xq, CB, ev)
    del Xq
    result["roofline"]["ceiling"] = {
        "kernel": "k_mfma_ceiling: v_mfma_i32_32x32x32_i8 on 16 accumulators from registers, "
                  "nothing else in the loop, operands = 16-byte fragments of this workload's Xq and CB",
        "achieved": round(ceil8, 1), "unit": "TOP/s", "frac_of_peak": round(ceil8 / INT8_PEAK_TOPS, 4),
        "kernel_frac_of_ceiling": round(achieved / ceil8, 4)}
    log("int8 MFMA ceiling on fc1's operands: %.0f TOP/s (%.1f%% of the spec peak); k_gemm at %.1f%% of it"
        % (ceil8, 100 * ceil8 / INT8_PEAK_TOPS, 100 * achieved / ceil8))
    if not args.no_decode:
        result["decode"] = decode_bench(torch, L, workloads, args.steps, args.warmup, ev, dev)
    if not args.no_configs:
        result["configs"] = configs_bench(torch, L, workloads, min(args.steps, args.config_steps),
                                          min(args.warmup, 3), ev, dev)
    if args.zeropoint:
        result["zeropoint"] = zeropoint_bench(torch, L, workloads, args.steps, args.warmup, ev, dev)
    if args.fp8:
        result["fp8"] = fp8_bench(torch, L, workloads, args.steps, args.warmup, ev, dev)
        result["fp8_e4m3"] = fp8_bench(torch, L, workloads, args.steps, args.warmup, ev, dev,
                                       fmt="e4m3")
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on %d rows ..." % args.cpu_rows)
        result["cpu_baseline"] = cpu_baseline(X_h, W_h, thr, args.cpu_rows)
    ev.close()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

"""Benchmark of the gfx950 dense GEMM library on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--configs all|none|c1,c4,...]
                    [--no-cpu] [--copy-calib] [--no-calib]

One step is one pass of the thin-GEMM workload the pages single out: the BF16
x.W1 up-projection of an MoE FFN, [1,4096] x [4096,14336], and the query x
128-key cache product [1,4096] x [4096,128] (B = K_cache^T).  Both run
through the C ABI (view parse, plan, skinny streaming kernel, epilogue), with
every input already resident in HBM: W1 and the cache are rotated over enough
distinct copies (>= 1 GiB in all) that neither the 256 MB Infinity Cache nor
the L2 can serve a repeat.  The two products are independent, so each runs on
its own HIP stream (both at the default priority): the cache product's 128
one-wave workgroups run beside the x.W1 grid (256 workgroups of 8 waves, one
per CU, which leaves room for more waves on every CU).
`value` is the step's algorithmic bytes (each operand read once, C written
once) per second over K steps; `one_stream` repeats the measurement with both
products on one stream, one after the other.

The JSON line also carries:
  roofline      the x.W1 kernel's achieved HBM rate (its algorithmic bytes over
                its average launch duration: K back-to-back launches between HIP
                events on the launch stream, a second timed region) against the
                8 TB/s HBM3E peak, and the
                HBM traffic read from rocprofv3 counters (profiles/), or null when
                the kernel source changed since they were taken;
  cpu_baseline  the FP64 CPU oracle on the same step, on the host's cores, with
                the CPU model and, under `configs`, the oracle timed on every
                workload (median of 3 for M <= 64, one run otherwise, and the
                64x512x512 problem on one core as well);
  measured_peaks  what this device sustains under ideal code, measured in the
                same run (register-only MFMA loops, a 2 GiB streaming read, the
                launch floor); roofline.frac_of_measured and each config's
                frac_measured_* divide by these instead of the data-sheet peaks;
  configs       every other workload shape timed the same way (TFLOPS and the
                fraction of the dense MFMA peak for M >= 64, GB/s and the
                fraction of HBM peak for the thin and HBM-bound shapes; c5_tail is
                an FP8 shape whose last wave of tiles is short), the
                FP8 quantizer producing the FP8 GEMM's operands (q_a: A per
                token, q_b: B per 128x128 block; GB/s against HBM peak), and
                the fused bias + GELU epilogue on three of the GEMMs (*_gelu:
                vs_plain_us is its cost over the plain GEMM, unfused_floor_us
                the least a separate bias + GELU pass over C would take),
                each GEMM config's `tuned` record (dg_gemm_tune's choice among
                its candidate plans, timed again over the rotated buffers,
                with the tuning time and the calls that pay it back), and
                moe8: the 8 MoE expert GEMMs [1,512] x [512,4096] in one
                dg_gemm_grouped call, against the same GEMMs as 8 dg_gemm calls;
                moe8_prefill: the same with 64 tokens per expert ([64,512] x
                [512,4096] each, the grouped matrix-core launch).
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

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_PEAK = {"bf16": 2516.6, "f16": 2516.6, "fp8": 5033.2}   # dense TFLOP/s
CACHE_DEFEAT_BYTES = 1 << 30   # rotate buffer sets until this many bytes are distinct
DOMINANT_KERNEL = "skinny_bn"  # the kernel that moves the x.W1 bytes
KERNEL_SOURCES = ["dense_gemm_19_amd/csrc/skinny.hip"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "skinny_bn_c2a_traffic.txt")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- workload bytes and flops

def algorithmic(case):
    """(bytes, flops) of one GEMM: each operand read once, C written once (and
    read once more when beta != 0), plus the FP8 scale tensors."""
    import math
    M, N, K = case.mnk
    es = lambda t: t.element_size()
    b = M * K * es(case.A) + K * N * es(case.B) + M * N * es(case.C) * (2 if case.beta != 0 else 1)
    if case.bias is not None:
        b += N * es(case.bias)
    if case.fp8:
        b += 4 * (M * math.ceil(K / 128) + math.ceil(K / 128) * math.ceil(N / 128))
    return b, 2.0 * M * N * K


def storage_bytes(case):
    tot = 0
    for t in (case.A, case.B, case.C, case.A_scale, case.B_scale, case.bias):
        if t is not None:
            tot += t.untyped_storage().nbytes()
    return tot


# ---------------------------------------------------------------- device buffer sets

def clone_view(t):
    """A copy of t's whole storage at a new address, viewed with t's geometry."""
    import torch
    if t is None:
        return None
    raw = torch.empty(0, dtype=torch.uint8, device=t.device).set_(t.untyped_storage())
    dup = raw.clone()
    return torch.empty(0, dtype=t.dtype, device=t.device).set_(
        dup.untyped_storage(), t.storage_offset(), t.shape, t.stride())


def rotated_sets(case, device, min_bytes=CACHE_DEFEAT_BYTES, max_sets=4096):
    import synth
    d0 = case.to(device)
    per = storage_bytes(d0)
    P = max(2, min(max_sets, -(-min_bytes // max(per, 1))))
    sets = [d0]
    for _ in range(P - 1):
        sets.append(synth.Case(d0.name, clone_view(d0.A), clone_view(d0.B), clone_view(d0.C),
                               d0.alpha, d0.beta, clone_view(d0.A_scale), clone_view(d0.B_scale),
                               d0.rtol, {}, clone_view(d0.bias), d0.act))
    return sets


class Call:
    """One prepared C-ABI call: the dg_view structs are built once, so the timed
    loop pays only for the ctypes call itself (the library still validates,
    plans and launches on every call)."""

    def __init__(self, dg, c, stream):
        import ctypes
        self.views = [dg.view_of(t) for t in ((c.A, c.A_scale, c.B, c.B_scale, c.C) if c.fp8
                                              else (c.A, c.B, c.C))]
        self.args = [ctypes.byref(v) for v in self.views]
        self.name = "dg_gemm_fp8" if c.fp8 else "dg_gemm"
        if c.fused:   # the fused-epilogue entry point: + bias view and activation code
            self.bias = dg.view_of(c.bias) if c.bias is not None else None
            act = {"none": dg.DG_ACT_NONE, "relu": dg.DG_ACT_RELU, "gelu_tanh": dg.DG_ACT_GELU_TANH}[c.act]
            self.args += [ctypes.byref(self.bias) if self.bias is not None else None, act]
            self.name += "_epilogue"
        self.args += [c.alpha, c.beta, stream]
        self.fn = getattr(dg.lib(), self.name)

    def __call__(self):
        return self.fn(*self.args)


def prepared(dg, sets, stream=None):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    return [Call(dg, c, stream) for c in sets]


class QuantCall:
    """One prepared dg_quant_fp8 call (views built once)."""

    def __init__(self, dg, x, q, sc, mode, stream):
        import ctypes
        self.views = [dg.view_of(t) for t in (x, q, sc)]
        self.args = [ctypes.byref(v) for v in self.views] + [mode, stream]
        self.fn = dg.lib().dg_quant_fp8
        self.name = "dg_quant_fp8"

    def __call__(self):
        return self.fn(*self.args)


# The FP8 workload's producers: its A operand quantized per token, its B
# operand per 128x128 block, from BF16 N(0,1) sources (the same draws as the
# quantizer's parity tests at these sizes).
QUANT_CONFIGS = {"q_a": (4096, 4096, 0, 106), "q_b": (4096, 7168, 1, 107)}


def time_quant(dg, name, trials=5):
    """Per-launch time of dg_quant_fp8 on one workload over rotated buffer sets."""
    import torch
    import synth
    M, K, mode, seed = QUANT_CONFIGS[name]
    x0 = synth.to_dtype(synth.draw(synth.rng(seed), (M, K), "normal", 1.0), torch.bfloat16).to("cuda:0")
    srows = M if mode == 0 else (M + 127) // 128
    nsc = srows * ((K + 127) // 128)
    per = M * K * 3 + nsc * 4
    P = max(2, -(-CACHE_DEFEAT_BYTES // per))
    stream = torch.cuda.current_stream().cuda_stream
    sets = []
    for _ in range(P):
        x = x0.clone()
        q = torch.empty(M, K, dtype=torch.float8_e4m3fn, device="cuda:0")
        sc = torch.empty(srows, (K + 127) // 128, dtype=torch.float32, device="cuda:0")
        sets.append((x, q, sc))
    calls = [QuantCall(dg, x, q, sc, mode, stream) for x, q, sc in sets]
    nbytes = M * K * 2 + M * K + nsc * 4
    reps = max(20, min(2000, int(2e-3 / max(nbytes / 6e12, 2e-6))))
    warm(calls)
    times = []
    for _ in range(trials):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        run_checked(calls, range(reps))
        e1.record()
        e1.synchronize()
        times.append(e0.elapsed_time(e1) * 1e-3 / reps)
    times.sort()
    t = times[len(times) // 2]
    gbs = nbytes / t / 1e9
    del sets, calls
    torch.cuda.empty_cache()
    return {"us": round(t * 1e6, 3), "us_min": round(times[0] * 1e6, 3), "reps": reps, "buffer_sets": P,
            "gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "dtype": "bf16->e4m3",
            "shape": [M, K], "mode": "token 1x128" if mode == 0 else "block 128x128",
            "path": "quant", "algorithmic_bytes": nbytes}


def time_grouped(dg, name="moe8", trials=5):
    """MoE experts through dg_gemm_grouped, one call per step, against the same
    8 GEMMs as 8 dg_gemm calls, both over rotated buffer sets.  moe8: decode,
    8 x [1,512] x [512,4096] with one token row shared (the grouped streaming
    kernel); moe8_prefill: 64 tokens per expert, 8 x [64,512] x [512,4096],
    each expert its own token block (the grouped matrix-core launch)."""
    import torch
    import synth
    shared = name == "moe8"
    experts = synth.moe_experts() if shared else synth.moe_experts(M=64, seed=109, shared_x=False)
    E = len(experts)
    d0 = [c.to("cuda:0") for c in experts]
    x = d0[0].A
    per = sum(storage_bytes(c) for c in d0) - ((E - 1) * x.untyped_storage().nbytes() if shared else 0)
    P = max(2, -(-CACHE_DEFEAT_BYTES // per))
    sets = [d0] + [[synth.Case(c.name, x if shared else clone_view(c.A), clone_view(c.B), clone_view(c.C))
                    for c in d0] for _ in range(P - 1)]
    stream = torch.cuda.current_stream().cuda_stream
    L = dg.lib()

    class Grouped:
        name = "dg_gemm_grouped"

        def __init__(self, cs):
            self.a = dg._view_array([c.A for c in cs])
            self.b = dg._view_array([c.B for c in cs])
            self.c = dg._view_array([c.C for c in cs])

        def __call__(self):
            return L.dg_gemm_grouped(E, self.a, self.b, self.c, 1.0, 0.0, stream)

    grouped = [Grouped(cs) for cs in sets]
    separate = [Call(dg, c, stream) for cs in sets for c in cs]
    nbytes = sum(algorithmic(c)[0] for c in experts) - ((E - 1) * algorithmic_a_bytes(experts[0]) if shared else 0)
    flops = sum(2.0 * c.mnk[0] * c.mnk[1] * c.mnk[2] for c in experts)

    def timed(calls, per_step):
        reps = 200
        warm(calls)
        ts = []
        for _ in range(trials):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            run_checked(calls, range(reps * per_step))
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3 / reps)
        ts.sort()
        return ts[len(ts) // 2], ts[0]

    tg, tg_min = timed(grouped, 1)
    ts_, ts_min = timed(separate, E)
    plan = dg.grouped_plan([c.A for c in d0], [c.B for c in d0], [c.C for c in d0])
    del sets, grouped, separate, d0
    torch.cuda.empty_cache()
    M = experts[0].mnk[0]
    return {"us": round(tg * 1e6, 3), "us_min": round(tg_min * 1e6, 3), "buffer_sets": P,
            "tflops": round(flops / tg / 1e12, 2),
            "gbs": round(nbytes / tg / 1e9, 1), "frac_hbm_peak": round(nbytes / tg / 1e9 / HBM_PEAK_GBS, 4),
            "separate_us": round(ts_ * 1e6, 3), "separate_gbs": round(nbytes / ts_ / 1e9, 1),
            "speedup_vs_separate": round(ts_ / tg, 3), "dtype": "bf16", "mnk": [M, 4096, 512],
            "experts": E, "path": "skinny grouped" if M <= 8 else "matrix-core grouped", "plan": plan,
            "algorithmic_bytes": nbytes}


def algorithmic_a_bytes(case):
    """Bytes of the A operand (read once however many groups share it)."""
    M, N, K = case.mnk
    return M * K * case.A.element_size()


def run_checked(calls, idx):
    """Launch calls[i % len] for i in idx; raise on the first non-zero status."""
    n = len(calls)
    bad = 0
    for i in idx:
        bad |= calls[i % n]()
    if bad:
        raise RuntimeError(f"{calls[0].name} returned an error status in the timed loop")


# ---------------------------------------------------------------- timing

WARM_MS = 150.0   # sustained work before any timed region (the clocks ramp up over ~30 ms)


def warm(calls, ms=WARM_MS):
    """Run the calls back to back for about `ms` milliseconds: under sustained
    load the same kernel runs up to ~12 % faster than in its first
    milliseconds (BF16 4096^3: 141 us per launch in the first 20 launches,
    110 us after ~30 ms), and every timed region should see the steady state."""
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    run_checked(calls, range(10))
    e1.record()
    e1.synchronize()
    per = max(e0.elapsed_time(e1) / 10, 1e-3)
    run_checked(calls, range(int(ms / per) + 1))
    torch.cuda.synchronize()


def time_calls(calls, reps, trials):
    """Median and minimum per-launch time of `reps` launches between two events."""
    import torch
    warm(calls)
    per = []
    for _ in range(trials):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        run_checked(calls, range(reps))
        e1.record()
        e1.synchronize()
        per.append(e0.elapsed_time(e1) * 1e-3 / reps)
    per.sort()
    return per[len(per) // 2], per[0]


def time_config(dg, name, reps=None, trials=5, tune=False):
    """Per-launch time of one workload over rotated buffer sets (median of
    trials); with tune, the problem is then tuned (dg_gemm_tune on the first
    buffer set) and timed again the same way with the tuned plan."""
    import torch
    import synth
    case = synth.config(name)
    sets = rotated_sets(case, "cuda:0")
    calls = prepared(dg, sets)
    nbytes, flops = algorithmic(case)
    if reps is None:   # aim for a few ms per trial
        reps = max(20, min(2000, int(2e-3 / max(flops / 2e15, nbytes / 6e12, 2e-6))))
    t, t_min = time_calls(calls, reps, trials)
    per = [t_min]
    M = case.mnk[0]
    plan = dg.plan(sets[0].A, sets[0].B, sets[0].C, case.alpha, case.beta, sets[0].A_scale,
                   sets[0].B_scale)
    dt = "fp8" if case.fp8 else ("bf16" if case.A.dtype == torch.bfloat16 else "f16")
    tflops = flops / t / 1e12
    gbs = nbytes / t / 1e9
    rec = {"us": round(t * 1e6, 3), "us_min": round(per[0] * 1e6, 3), "reps": reps,
           "buffer_sets": len(sets), "tflops": round(tflops, 2),
           "frac_mfma_peak": round(tflops / MFMA_PEAK[dt], 4), "gbs": round(gbs, 1),
           "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "dtype": dt, "mnk": list(case.mnk),
           "c_elem_bytes": case.C.element_size(), "path": re.search(r"path=(\S+)", plan).group(1)}
    m = re.search(r"tile=(\S+)", plan)
    if m:
        rec["tile"] = m.group(1)
    m = re.search(r"splits=(\d+)", plan)
    if m:
        rec["splits"] = int(m.group(1))
    if case.fused:
        rec["epilogue"] = f"+bias({str(case.bias.dtype).split('.')[-1]}) {case.act}" if case.bias is not None \
            else case.act
    if tune:
        s0 = sets[0]
        r = dg.tune(s0.A, s0.B, s0.C, s0.A_scale, s0.B_scale, reps=3)
        tt, tt_min = time_calls(calls, reps, trials)
        rec["tuned"] = {"us": round(tt * 1e6, 3), "us_min": round(tt_min * 1e6, 3),
                        "speedup": round(t / tt, 4), "tune_ms": round(r["tune_ms"], 2),
                        "candidates": r["candidates"], "chosen": r["chosen"],
                        "tuner_default_us": round(r["default_us"], 3), "tuner_best_us": round(r["best_us"], 3),
                        "plan": r["plan"].split(" | ")[0].split(" path=")[1], "sets": r["sets"],
                        "calls_to_amortize": (round(r["tune_ms"] * 1e-3 / (t - tt)) if tt < t else None)}
        dg.tune_clear()
    del sets
    torch.cuda.empty_cache()
    return rec


def source_hash():
    """Hash of the dominant kernel's sources with comments and blank space
    removed, so that a change of comments alone keeps the measured traffic."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES + ["dense_gemm_19_amd/csrc/device_common.hpp",
                               "dense_gemm_19_amd/csrc/kernels.hpp"]:
        with open(os.path.join(ROOT, p)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def traffic_from_profiles(launch_bytes):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, or None if it is missing or the kernel changed since."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m_hash = re.search(r"^source_hash:\s*(\S+)", text, re.M)
    m_t = re.search(r"^hbm_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not m_hash or not m_t or m_hash.group(1) != source_hash():
        return None
    return float(m_t.group(1))


def cpu_baseline(cases, budget_s=12.0):
    """The FP64 oracle on whole steps, repeated until about budget_s of CPU work."""
    import oracle
    nbytes = sum(algorithmic(c)[0] for c in cases)
    views = [(oracle.host_view(c.A), oracle.host_view(c.B)) for c in cases]
    reps, t_total = 0, 0.0
    while t_total < budget_s and reps < 400:
        t0 = time.perf_counter()
        for c, (a, b) in zip(cases, views):
            oracle.ref_gemm(a, b, None, c.alpha, 0.0)
        t_total += time.perf_counter() - t0
        reps += 1
    return {"value": round(nbytes * reps / t_total / 1e9, 4), "unit": "GB/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{reps} whole steps (x.W1 1x4096x14336 + q.K_cache^T 1x4096x128, BF16 in, "
                      f"FP64 arithmetic) in {t_total:.1f} s",
            "cpu_model": cpu_model()}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_oracle_configs(names=("c1", "c2a", "c2b", "c3", "c4", "c5_128", "c5_4096")):
    """The oracle timed on every workload, on all host threads: the small
    shapes (M <= 64) as the median of 3 runs, the others one run each, and the
    FP16 64x512x512 problem once more on one core.  Seconds and FP64 GFLOP/s
    (2MNK per run; the sum of |a*b| the bound needs is formed in the same pass)."""
    import statistics
    import oracle
    import synth
    out = {}
    for name in names:
        c = synth.config(name)
        hv = [None if t is None else oracle.host_view(t) for t in (c.A, c.B, c.A_scale, c.B_scale)]
        cin = oracle.host_view(c.C) if c.beta != 0 else None
        M, N, K = c.mnk
        runs = 3 if M <= 64 else 1
        ts = []
        for _ in range(runs):
            t0 = time.perf_counter()
            oracle.ref_gemm(hv[0], hv[1], cin, c.alpha, c.beta, A_scale=hv[2], B_scale=hv[3])
            ts.append(time.perf_counter() - t0)
        t = statistics.median(ts)
        out[name] = {"s": round(t, 4), "gflops_fp64": round(2.0 * M * N * K / t / 1e9, 2), "runs": runs,
                     "threads": oracle.num_threads()}
        if name == "c1":
            t0 = time.perf_counter()
            oracle.ref_gemm(hv[0], hv[1], cin, c.alpha, c.beta, nthreads=1)
            t1 = time.perf_counter() - t0
            out["c1_one_core"] = {"s": round(t1, 4), "gflops_fp64": round(2.0 * M * N * K / t1 / 1e9, 2),
                                  "runs": 1, "threads": 1}
    return out


def measured_peaks(dg, nbytes=2 << 30):
    """The denominators the hardware sustains under ideal code, measured now on
    this device through the library's calibration entry points: register-only
    matrix-instruction loops, a streaming read of 2 GiB (far above the 256 MB
    last-level cache), and the back-to-back launch floor."""
    import torch
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
    torch.cuda.synchronize()
    r = {"hbm_read_gbs": round(dg.calib_read(buf), 1),
         "mfma_bf16_tflops": round(dg.calib_mfma(dg.DG_BF16), 1),
         "mfma_fp8_tflops": round(dg.calib_mfma(dg.DG_F8E4M3), 1),
         "launch_floor_us": round(dg.calib_launch(), 3),
         "how": "register-only 16x16x32 BF16 / 16x16x128 FP8 MFMA loops on every CU; "
                "16-byte nontemporal streaming read of 2 GiB; 2000 back-to-back empty launches"}
    del buf
    torch.cuda.empty_cache()
    return r


def copy_calibration(nbytes=1 << 30):
    """A plain device copy of known size, for scaling rocprofv3 byte counters."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    log(f"copy calibration: {nbytes} bytes read, {nbytes} bytes written")


# ---------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    # (5000 steps of ~26 us: the clocks reach their sustained state before timing)
    ap.add_argument("--warmup", type=int, default=5000)
    ap.add_argument("--configs", default="all",
                    help="other workloads to time: all, none, or a comma list of "
                         "c1,c3,c4,c5_128,c5_4096,c5_tail (GEMMs), <config>_gelu (the same GEMM with a "
                         "fused bias + GELU epilogue), q_a,q_b (the FP8 quantizer) and moe8 (8 MoE "
                         "expert GEMMs in one grouped call; moe8_prefill: the same with 64 tokens per expert)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a 1 GiB device copy (for counter calibration)")
    ap.add_argument("--no-tune", action="store_true",
                    help="skip tuning the GEMM configs (dg_gemm_tune, then a second timing with the tuned plan)")
    ap.add_argument("--no-calib", action="store_true",
                    help="skip the measured peaks (register-only MFMA loops, 2 GiB read, launch floor)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library runs on a single MI355X and has no "
              "multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import dense_gemm_19_amd as dg
    dg.lib()   # raises if the HIP library is missing: there is no fallback
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = "cuda:0"

    # ---- the step: x.W1 and q.K_cache^T (each on its own stream), rotated over >= 1 GiB of distinct buffers
    c2a, c2b = synth.config("c2a"), synth.config("c2b")
    sa_sets = rotated_sets(c2a, dev)
    sb_sets = rotated_sets(c2b, dev)
    P = max(len(sa_sets), len(sb_sets))
    bytes_a, _ = algorithmic(c2a)
    bytes_b, _ = algorithmic(c2b)
    step_bytes = bytes_a + bytes_b
    log(f"step: x.W1 {c2a.mnk} + q.Kc {c2b.mnk}; {step_bytes} algorithmic bytes; "
        f"{len(sa_sets)} / {len(sb_sets)} rotated buffer sets")
    log("plan x.W1:", dg.plan(sa_sets[0].A, sa_sets[0].B, sa_sets[0].C))
    log("plan q.Kc:", dg.plan(sb_sets[0].A, sb_sets[0].B, sb_sets[0].C))

    main_stream = torch.cuda.current_stream()
    side_stream = torch.cuda.Stream()   # default priority, like every stream here
    calls_a = prepared(dg, sa_sets)
    calls_b = prepared(dg, sb_sets, side_stream.cuda_stream)
    calls_b1 = prepared(dg, sb_sets)     # the same calls on the main stream
    na, nb = len(calls_a), len(calls_b)

    def steps(lo, hi, cb):
        bad = 0
        for i in range(lo, hi):
            bad |= calls_a[i % na]()
            bad |= cb[i % nb]()
        if bad:
            raise RuntimeError("dg_gemm returned an error status in the timed loop")

    def timed_steps(cb, two_streams):
        # K whole steps between an event pair on the main stream; with two
        # streams the side stream starts after the first event and the main
        # stream waits for all of its work before the second
        t_start = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        t_start.record(main_stream)
        if two_streams:
            side_stream.wait_event(t_start)
        steps(args.warmup, args.warmup + args.steps, cb)
        if two_streams:
            joined = torch.cuda.Event()
            joined.record(side_stream)
            main_stream.wait_event(joined)
        t_end.record(main_stream)
        torch.cuda.synchronize()
        return t_start.elapsed_time(t_end)

    steps(0, args.warmup, calls_b)
    torch.cuda.synchronize()
    # timed region 1: K whole steps, the two products on two streams
    ms_total = timed_steps(calls_b, True)
    ms_step = ms_total / args.steps
    value = step_bytes / (ms_step * 1e-3) / 1e9
    # the same steps with both products on the main stream, one after the other
    steps(0, args.warmup // 5, calls_b1)
    torch.cuda.synchronize()
    ms_total1 = timed_steps(calls_b1, False)
    ms_step1 = ms_total1 / args.steps
    value1 = step_bytes / (ms_step1 * 1e-3) / 1e9
    # timed region 2: the x.W1 launch alone, K launches back to back between a
    # HIP event pair on the stream the library launches on: the dominant
    # kernel's average launch duration
    k0 = torch.cuda.Event(enable_timing=True)
    k1 = torch.cuda.Event(enable_timing=True)
    k0.record()
    bad = 0
    for i in range(args.steps):
        bad |= calls_a[i % na]()
    k1.record()
    torch.cuda.synchronize()
    if bad:
        raise RuntimeError("dg_gemm returned an error status")
    k_avg = k0.elapsed_time(k1) / args.steps
    achieved = bytes_a / (k_avg * 1e-3) / 1e9
    log(f"{args.steps} steps in {ms_total:.3f} ms: {ms_step * 1e3:.2f} us/step, {value:.1f} GB/s "
        f"(one stream: {ms_step1 * 1e3:.2f} us/step, {value1:.1f} GB/s); "
        f"x.W1 launch avg {k_avg * 1e3:.2f} us -> {achieved:.1f} GB/s")
    traffic = traffic_from_profiles(bytes_a)
    del sa_sets, sb_sets
    torch.cuda.empty_cache()

    # ---- the other workloads
    others = {}
    names = [] if args.configs == "none" else (
        ["c1", "c3", "c4", "c5_128", "c5_4096", "c5_tail", "q_a", "q_b", "c2a_gelu", "c4_gelu", "c5_4096_gelu",
         "moe8", "moe8_prefill"]
        if args.configs == "all" else args.configs.split(","))
    for n in names:
        others[n] = (time_quant(dg, n) if n in QUANT_CONFIGS else time_grouped(dg, n) if n.startswith("moe8")
                     else time_config(dg, n, tune=not args.no_tune and not n.endswith("_gelu")))
        log(n, json.dumps(others[n]))
    # fused epilogue: its cost over the plain GEMM of the same operands, and the
    # least a separate bias + GELU pass would add (read C and write it again
    # once, at the HBM peak)
    # (the plain x.W1 time is the step's second timed region)
    plain_us = {n: r["us"] for n, r in others.items()}
    plain_us["c2a"] = round(k_avg * 1e3, 3)
    for n, r in others.items():
        base = n[:-5] if n.endswith("_gelu") else None
        if base in plain_us:
            M, N = r["mnk"][0], r["mnk"][1]
            r["vs_plain_us"] = round(r["us"] - plain_us[base], 3)
            r["unfused_floor_us"] = round(plain_us[base] + 2 * M * N * r["c_elem_bytes"] / (HBM_PEAK_GBS * 1e3), 3)

    if args.copy_calib:
        copy_calibration()

    measured = None
    if not args.no_calib:
        measured = measured_peaks(dg)
        log("measured peaks:", json.dumps(measured))

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline([c2a, c2b])
        cpu["configs"] = cpu_oracle_configs()
        log("cpu baseline:", json.dumps(cpu))

    out = {
        "metric": "GB/s & % HBM peak (M=1 thin GEMM); TFLOPS & % MFMA peak (M>=64) in configs",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "thin BF16 GEMM: x[1,4096] . W1[4096,14336] (row-major W1) + "
                               "q[1,4096] . K_cache[128,4096]^T, FP32 accumulate, BF16 C",
                   "M": 1, "K": 4096, "N": [14336, 128], "buffer_sets": P,
                   "inputs": "N(0,1) seeded, resident in HBM, rotated over >= 1 GiB",
                   "parallelism": "single GPU; the two independent products on two HIP streams"},
        "one_stream": {"value": round(value1, 1), "ms_per_step": round(ms_step1, 6)},
        "roofline": {"bound": "hbm", "kernel": DOMINANT_KERNEL, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes": bytes_a,
                     "avg_launch_us": round(k_avg * 1e3, 3)},
        "cpu_baseline": cpu,
        "measured_peaks": measured,
        "configs": others,
    }
    if measured:
        out["roofline"]["frac_of_measured"] = round(achieved / measured["hbm_read_gbs"], 4)
        for n, r in others.items():
            if "gbs" not in r:
                continue
            if "tflops" in r:
                peak = measured["mfma_fp8_tflops"] if r["dtype"] == "fp8" else measured["mfma_bf16_tflops"]
                r["frac_measured_mfma"] = round(r["tflops"] / peak, 4)
            r["frac_measured_hbm"] = round(r["gbs"] / measured["hbm_read_gbs"], 4)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

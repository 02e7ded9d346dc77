#!/usr/bin/env python3
"""Throughput of the batch-invariant bf16 GEMM on one MI355X.

One step = the whole hot path over one batch of synthetic input: the
Llama-3.1-8B FFN down-projection layer (W bf16 [4096, 14336], the layer whose
GEMM throughput LLM-42's reading notes compare in §2.3 Fig. 4a) called at
every M of the sweep 1, 2, 4, ..., 8192 with x = bf16(SiLU(a) * b).  Each call
dispatches on M between the weight-streaming and the tiled MFMA kernels, all
realising one pinned reduction tree.

value = sum over the sweep of 2*M*N*K / total time (TFLOP/s), inputs resident
in HBM before the timed region.  To keep the 256 MB Infinity Cache from
serving the weights to the decode-size calls, the calls rotate over copies of
W totalling at least 1 GiB (identical values, separate memory).

Also reported: the dominant kernel's roofline (achieved vs MI355X peak, from
HIP events around its runs of consecutive launches in the timed region, the
only events there),
per-M times (events around every launch, in as many instrumented steps run
before the timed region; the events around single launches are created
without the system-scope fence that a default event's record performs, an L2
write-back and invalidate that would slow the launch after it), HBM traffic from rocprof
counters when a current measurement is committed under profiles/, and the CPU
oracle's throughput on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
KERNEL_SRC = os.path.join(ROOT, "invariant_bi_gemm_amd", "csrc", "bigemm_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_llama8b_down_sweep.txt")

WORKLOADS = {
    "llama8b_down": dict(n=4096, k=14336, std=0.02, x="silu_mul", ms=[2 ** i for i in range(14)],
                         desc="Llama-3.1-8B FFN down-proj, W bf16 [4096,14336], x=bf16(SiLU(a)*b), "
                              "M sweep 1,2,4,...,8192"),
    "llama8b_gate_up": dict(n=28672, k=4096, std=0.02, x="rms", ms=[32, 544, 2080, 8224],
                            desc="Llama-3.1-8B fused gate+up, W bf16 [28672,4096], RMS-normalised rows, "
                                 "M in {32,544,2080,8224}"),
    "llama70b_down_tp8": dict(n=8192, k=3584, std=0.015, x="normal", ms=[1, 8, 64, 512, 4096, 16384],
                              desc="Llama-3.1-70B down-proj TP-8 shard, W bf16 [8192,3584], "
                                   "M in {1,8,64,512,4096,16384}"),
}

# Qwen3-30B-A3B-style MoE expert GEMMs: 128 experts, top-8 routing.
MOE = dict(experts=128, topk=8, up=(1536, 2048), down=(2048, 768), tokens=[1, 16, 256, 4096], std=0.02,
           desc="MoE expert GEMMs (Qwen3-30B-A3B-style): 128 experts, top-8 of softmax(N(0,1) logits), "
                "up W bf16 [128,1536,2048] and down W bf16 [128,2048,768], T in {1,16,256,4096} tokens")


def kernel_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


CLOCK_FILE = os.path.join(ROOT, "profiles", "clock_llama8b_down_sweep.txt")


def read_profile_kv(path: str, kernel: str):
    """key = value lines of a committed profile summary, or None when absent,
    for another kernel, or taken on another version of the kernels."""
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            key, val = line.split("=", 1)
            kv[key.strip()] = val.strip()
    if kv.get("kernel_source_sha256_16") != kernel_hash() or kv.get("kernel") != kernel:
        return None
    return kv


def read_clock(kernel: str):
    """The engine clock the kernel sustains (GHz) from committed rocprof
    counters: busy cycles (GRBM_GUI_ACTIVE) over the dispatch's duration."""
    kv = read_profile_kv(CLOCK_FILE, kernel)
    try:
        return float(kv["sustained_clock_ghz"]) if kv else None
    except (KeyError, ValueError):
        return None


def read_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from committed rocprof counters, or
    None when absent or taken on another version of the kernels."""
    kv = read_profile_kv(TRAFFIC_FILE, kernel)
    try:
        return float(kv["hbm_bytes_per_launch"]) if kv else None
    except (KeyError, ValueError):
        return None


def make_inputs(wl, seed=42):
    import numpy as np

    import synth

    n, k = wl["n"], wl["k"]
    w = synth.normal_bf16(seed, (n, k), wl["std"])
    mmax = max(wl["ms"])
    if wl["x"] == "silu_mul":
        x = synth.silu_mul_bf16(seed + 1, (mmax, k))
    elif wl["x"] == "rms":
        x = synth.rms_rows_bf16(seed + 1, (mmax, k))
    else:
        x = synth.normal_bf16(seed + 1, (mmax, k))
    return np.ascontiguousarray(w), np.ascontiguousarray(x)


def to_dev(bits):
    import numpy as np
    import torch

    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to("cuda:0")


def host_cpu() -> str:
    """The host CPU's model name (Linux /proc/cpuinfo), for the CPU baseline."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w_bits, x_bits, n, k, target_s=15.0):
    """The oracle, as it stands, on the host cores: rows of the same layer.

    Times a small probe first, then enough rows for about `target_s` seconds.
    """
    import numpy as np

    import oracle

    threads = oracle.max_threads()
    oracle.gemm_f64(x_bits[:2], w_bits)  # load and warm the library
    t0 = time.perf_counter()
    oracle.gemm_f64(x_bits[:4], w_bits)
    probe = max(time.perf_counter() - t0, 1e-3) / 4
    rows = int(max(4, min(x_bits.shape[0], target_s / probe)))
    idx = np.arange(rows)
    t0 = time.perf_counter()
    oracle.gemm_f64(x_bits, w_bits, rows=idx)
    dt = time.perf_counter() - t0
    tflops = 2.0 * rows * n * k / dt / 1e12
    return {"value": tflops, "unit": "TFLOPS", "cores": threads, "cpu": host_cpu(), "kind": "oracle",
            "sample": "fp64 oracle on %d rows (all %d columns) of the same layer, %.1f s" % (rows, n, dt)}


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence (hip_runtime_api.h)
_hip_rt = None


def _hip():
    """The HIP runtime torch has loaded (soname libamdhip64.so.7; dlopen
    returns the loaded copy, so events and streams are shared with torch)."""
    global _hip_rt
    if _hip_rt is None:
        import ctypes

        import torch  # noqa: F401  (loads the runtime first)

        lib = ctypes.CDLL("libamdhip64.so.7")
        vp = ctypes.c_void_p
        lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), ctypes.c_uint]
        lib.hipEventRecord.argtypes = [vp, vp]
        lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
        lib.hipEventDestroy.argtypes = [vp]
        _hip_rt = lib
    return _hip_rt


class LaunchEvent:
    """A HIP timing event for the events around single launches: created with
    hipEventDisableSystemFence, so recording it does not write back and
    invalidate the caches as a default event does (measured: about 5 us of GPU
    time per record, and a cold L2 for the launch after it).  Used like
    torch.cuda.Event(enable_timing=True): record() on torch's current stream
    (or `stream`, a raw hipStream_t), elapsed_time(end) in ms once both have
    completed.  The timed region itself is bracketed by default events and a
    device synchronisation."""

    def __init__(self):
        import ctypes

        self._lib = _hip()
        self._e = ctypes.c_void_p()
        st = self._lib.hipEventCreateWithFlags(ctypes.byref(self._e), HIP_EVENT_DISABLE_SYSTEM_FENCE)
        if st != 0:
            raise RuntimeError("hipEventCreateWithFlags failed: %d" % st)

    def record(self, stream=None):
        import ctypes

        import torch

        s = torch.cuda.current_stream().cuda_stream if stream is None else stream
        st = self._lib.hipEventRecord(self._e, ctypes.c_void_p(s))
        if st != 0:
            raise RuntimeError("hipEventRecord failed: %d" % st)

    def elapsed_time(self, end) -> float:
        import ctypes

        ms = ctypes.c_float()
        st = self._lib.hipEventElapsedTime(ctypes.byref(ms), self._e, end._e)
        if st != 0:
            raise RuntimeError("hipEventElapsedTime failed: %d" % st)
        return ms.value

    def __del__(self):
        if getattr(self, "_e", None) and self._e.value:
            self._lib.hipEventDestroy(self._e)
            self._e = None


def _time_calls(fn, reps):
    import torch

    for _ in range(2):
        fn(0)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


SPLITK_CHOICES = (1, 2, 4, 8)

# A second pin of the down-projection, tuned for a chunked-prefill serving
# profile (most calls 64..1024 rows) instead of the sweep's one call per M.
PREFILL_PINS = os.path.join(ROOT, "invariant_bi_gemm_amd", "pins", "gfx950_chunked_prefill.txt")
PREFILL_PROFILE = "1:4,16:4,64:8,128:16,256:16,512:16,1024:8,2048:2,4096:1,8192:1"


def alternative_pin(bg, ws, xd, ms, n, k, steps, warmup, table_ms):
    """The sweep under the chunked-prefill pin (its own tree and tiling),
    timed like the headline's per-M figures (events around each launch,
    median over the steps), and both pins' costs over that profile (Detent eq. 3: sum of
    count x time) -- the pin follows the workload profile."""
    import ctypes

    import numpy as np
    import torch

    import invariant_bi_gemm_amd.tuner as tuner

    if not os.path.exists(PREFILL_PINS):
        return None
    _, _, _, rows = tuner.read_table(PREFILL_PINS)
    if ("gfx950", n, k) not in rows:
        return None
    s_, smax, tiling = rows[("gfx950", n, k)]
    pin = {"splits": s_, "stream_max_m": smax, "tiling": tiling}
    hs = [bg.Gemm(w, pin=pin) for w in ws]
    copies = len(hs)
    lib = bg.load()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    xp = ctypes.c_void_p(xd.data_ptr())
    ys = {m: torch.empty((m, n), dtype=torch.float32, device="cuda:0") for m in ms}
    yps = {m: ctypes.c_void_p(ys[m].data_ptr()) for m in ms}
    call = [0]

    def step(events=None):
        for j, m in enumerate(ms):
            h = hs[call[0] % copies]._h
            call[0] += 1
            if events is not None:
                events[j][0].record()
            st = lib.bi_gemm_run(h, xp, m, yps[m], stream)
            if st != 0:
                bg.check(st)
            if events is not None:
                events[j][1].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [[[LaunchEvent(), LaunchEvent()] for _ in ms]
          for _ in range(steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        step(ev[i])
    t1.record()
    torch.cuda.synchronize()
    per = {m: float(np.median([ev[i][j][0].elapsed_time(ev[i][j][1]) for i in range(steps)])) for j, m in enumerate(ms)}
    prof = tuner.parse_profile(PREFILL_PROFILE)
    cost_alt = sum(c * per[m] for m, c in prof if m in per)
    cost_tab = sum(c * table_ms[m] for m, c in prof if m in table_ms)
    out = {"what": "the same sweep under the pin tuned for a chunked-prefill profile (%s): tree of %d splits, "
                   "tiling %s; events around each launch, median over the steps" % (PREFILL_PROFILE, s_,
                                                                                  tuner.format_tiling(tiling)),
           "pins_file": os.path.relpath(PREFILL_PINS, ROOT),
           "sweep_ms_per_step": round(t0.elapsed_time(t1) / steps, 4),
           "profile_cost_us": {"sweep_pin": round(cost_tab * 1e3, 1), "chunked_prefill_pin": round(cost_alt * 1e3, 1)},
           "per_m": [{"M": m, "us": round(per[m] * 1e3, 2), "kernel": hs[0].kernel_name(m),
                      "sweep_pin_us": round(table_ms[m] * 1e3, 2)} for m in ms]}
    for h in hs:
        h.close()
    return out


def invariance_cost(bg, ws, xd, ms, n, k, reps=10):
    """Cost of invariance: the pinned call at each M against the fastest
    NON-invariant GEMM this library can run for that M -- any of its kernel
    kinds with 1, 2, 4 or 8 concurrent K splits (bi_gemm_run_splitk), the
    fastest chosen per M as a batch-dependent selector would (LLM-42 notes,
    §2.3 Fig. 4a: the vendor GEMM adapts tile and split-K to the shape).  Both
    timed back to back with weights rotating over the same copies.  hipBLASLt
    (torch.matmul, bf16 output: half the output bytes) is context, with
    whether its rows keep their bits across M."""
    import torch

    copies = len(ws)
    ys = {m: torch.empty((m, n), dtype=torch.float32, device="cuda:0") for m in ms}
    pinned_hs = [bg.Gemm(w) for w in ws]
    pinned = {m: _time_calls(lambda i: pinned_hs[i % copies](xd[:m], out=ys[m]), reps) for m in ms}
    splits = [p for p in SPLITK_CHOICES if k % (64 * p) == 0]
    best = {}
    for m in ms:
        wsp = torch.empty(max(splits) * m * n, dtype=torch.float32, device="cuda:0")
        for kind in bg.KERNEL_KINDS:
            if kind.startswith("stream") and m > 256:
                continue
            for p_ in splits:
                t = _time_calls(lambda i: pinned_hs[i % copies].run_splitk(xd[:m], kind, p_, out=ys[m],
                                                                            workspace=wsp), reps)
                if m not in best or t < best[m][0]:
                    best[m] = (t, kind, p_)
        del wsp
    rows = []
    tot_pin = tot_best = tot_blas = 0.0
    wts = [w.t() for w in ws]
    probe = xd[:1]
    ref_row = torch.matmul(probe, wts[0]).view(torch.int16)
    for m in ms:
        tb = _time_calls(lambda i: torch.matmul(xd[:m], wts[i % copies]), reps)
        same = bool(torch.equal(torch.matmul(xd[:m], wts[0])[:1].view(torch.int16), ref_row))
        tot_pin += pinned[m]
        tot_best += best[m][0]
        tot_blas += tb
        rows.append({"M": m, "pinned_us": round(pinned[m] * 1e3, 2),
                     "noninvariant_us": round(best[m][0] * 1e3, 2),
                     "noninvariant_choice": {"kernel": best[m][1], "concurrent_splits": best[m][2]},
                     "invariant_over_noninvariant": round(pinned[m] / best[m][0], 3),
                     "hipblaslt_bf16out_us": round(tb * 1e3, 2),
                     "hipblaslt_row0_same_bits_as_M1": same})
    return {"what": "pinned (batch-invariant) call vs the fastest non-invariant GEMM of this library at each M "
                    "(any kernel kind, 1/2/4/8 concurrent K splits, chosen per M), both timed back to back "
                    "with rotated weights, fp32 output; hipBLASLt (torch.matmul, bf16 output) as context",
            "ratio_invariant_over_noninvariant_sweep": round(tot_pin / tot_best, 4),
            "pinned_sweep_ms": round(tot_pin, 4),
            "noninvariant_sweep_ms": round(tot_best, 4),
            "hipblaslt_bf16out_sweep_ms": round(tot_blas, 4),
            "per_m": rows}


# MI355X's peak engine clock: the nominal bf16 peak is quoted at it
PEAK_CLOCK_GHZ = 2.4


def run_moe(args, bg):
    """One step = the up and the down expert GEMM at every token count T of
    the sweep (rows = 8T, grouped by expert).  Weights rotate over copies so
    the Infinity Cache does not hold the touched experts between calls."""
    import numpy as np
    import torch

    import synth

    E, topk = MOE["experts"], MOE["topk"]
    shapes = {"up": MOE["up"], "down": MOE["down"]}
    copies = 2
    handles, wbits = {}, {}
    for i, (name, (n, k)) in enumerate(shapes.items()):
        wbits[name] = synth.normal_bf16(42 + i, (E, n, k), MOE["std"])
        w0 = to_dev(wbits[name])
        handles[name] = [bg.GroupedGemm(w0)] + [bg.GroupedGemm(w0.clone()) for _ in range(copies - 1)]
    calls = []  # (T, name, x, offsets, y, flops, bytes)
    for t in MOE["tokens"]:
        tok, off, _ = synth.moe_routing(42 + t, t, E, topk)
        touched = int(np.count_nonzero(np.diff(off)))
        r = len(tok)
        for name, (n, k) in shapes.items():
            x_tok = synth.normal_bf16(43 + t + k, (t, k))
            x = to_dev(np.ascontiguousarray(x_tok[tok]))
            y = torch.empty((r, n), dtype=torch.float32, device="cuda:0")
            calls.append((t, name, x, torch.as_tensor(off, device="cuda:0"), y, 2.0 * r * n * k,
                          2.0 * touched * n * k + 2.0 * r * k + 4.0 * r * n, touched))
    # straight to the C ABI with precomputed arguments, as in the dense sweep
    import ctypes

    lib = bg.load()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    cargs = [(tuple(h._h for h in handles[name]), ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(off.data_ptr()),
              int(x.shape[0]), ctypes.c_void_p(y.data_ptr())) for (_, name, x, off, y, _, _, _) in calls]
    run = lib.bi_grouped_gemm_run
    call_no = [0]

    def step(events=None):
        for j, (hs, xp, offp, r, yp) in enumerate(cargs):
            h = hs[call_no[0] % copies]
            call_no[0] += 1
            if events is not None:
                events[j][0].record()
            st = run(h, xp, offp, r, yp, stream)
            if st != 0:
                bg.check(st)
            if events is not None:
                events[j][1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [[[LaunchEvent(), LaunchEvent()] for _ in calls]
          for _ in range(args.steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for s_ in range(args.steps):
        step(ev[s_])
    t1.record()
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps
    per = [float(np.mean([ev[s_][j][0].elapsed_time(ev[s_][j][1]) for s_ in range(args.steps)]))
           for j in range(len(calls))]
    step_flops = sum(c[5] for c in calls)
    rows = []
    for (t, name, _, _, _, fl, by, touched), ms in zip(calls, per):
        rows.append({"T": t, "gemm": name, "rows": 8 * t, "experts_touched": touched, "us": round(ms * 1e3, 2),
                     "tflops": round(fl / (ms * 1e-3) / 1e12, 1), "hbm_gbs": round(by / (ms * 1e-3) / 1e9, 0)})
    dom = max(range(len(calls)), key=lambda j: per[j])
    t, name, _, _, _, fl, by, _ = calls[dom]
    # the binding roofline: the larger of the MFMA time and the HBM time of
    # the call's algorithmic work
    if fl / (PEAK_BF16_TFLOPS * 1e12) >= by / (PEAK_HBM_GBS * 1e9):
        ach = fl / (per[dom] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    else:
        ach = by / (per[dom] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof.update({"frac": roof["achieved"] / roof["peak"], "traffic": None,
                 "kernel": "grouped %s GEMM at T=%d (all its grouped kernels)" % (name, t),
                 "launches_per_step": 1, "avg_launch_us": per[dom] * 1e3})
    cpu = None
    if not args.no_cpu_baseline:
        cpu = moe_cpu_baseline(wbits, calls)
    out = {
        "metric": "batch-invariant bf16 GEMM TFLOPS (M sweep) + % MFMA/HBM roofline, 1 GPU",
        "value": round(step_flops / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; W ~ N(0,%g), x ~ N(0,1), routing from N(0,1) logits)" % MOE["std"],
        "config": {"workload": MOE["desc"], "tokens": MOE["tokens"], "weight_copies_rotated": copies,
                   "kernel_source_sha256_16": kernel_hash()},
        "roofline": roof,
        "cpu_baseline": cpu,
        "per_call": rows,
    }
    print(json.dumps(out), flush=True)
    return 0


def moe_cpu_baseline(wbits, calls, target_s=15.0):
    """The oracle's grouped GEMM on the host cores, on a bounded sample: the
    T=4096 up-projection rows, as many as fit in about `target_s` seconds."""
    import numpy as np
    import torch

    import oracle

    t, name, x, off, _, _, _, _ = next(c for c in calls if c[0] == 4096 and c[1] == "up")
    xb = x.view(torch.int16).cpu().numpy().view(np.uint16)
    offs = off.cpu().numpy()
    w = wbits[name]
    n, k = w.shape[1], w.shape[2]
    t0 = time.perf_counter()
    oracle.grouped_f64(xb, w, offs, rows=np.arange(4))
    probe = max(time.perf_counter() - t0, 1e-3) / 4
    nrows = int(max(4, min(xb.shape[0], target_s / probe)))
    t0 = time.perf_counter()
    oracle.grouped_f64(xb, w, offs, rows=np.arange(nrows))
    dt = time.perf_counter() - t0
    return {"value": 2.0 * nrows * n * k / dt / 1e12, "unit": "TFLOPS", "cores": oracle.max_threads(),
            "cpu": host_cpu(), "kind": "oracle",
            "sample": "fp64 oracle, grouped up-projection (N=%d, K=%d), first %d of the %d rows at T=%d, %.1f s"
                      % (n, k, nrows, xb.shape[0], t, dt)}


def _moe_layer_weights(seed=42):
    import synth

    E, H, I = MOE["experts"], MOE["up"][1], MOE["down"][1]
    return (synth.normal_bf16(seed + 10, (E, H), MOE["std"]),
            synth.normal_bf16(seed + 11, (E, 2 * I, H), MOE["std"]),
            synth.normal_bf16(seed + 12, (E, H, I), MOE["std"]))


def moe_layer_work(t, touched_up, touched_down):
    """Algorithmic flops and HBM bytes of each step of the layer at T tokens
    (R = kT rows); a GEMM's weight bytes count only the touched experts."""
    E, k, H, I = MOE["experts"], MOE["topk"], MOE["up"][1], MOE["down"][1]
    r = k * t
    return [
        ("router GEMM", 2.0 * t * E * H, 2.0 * E * H + 2.0 * t * H + 4.0 * t * E),
        ("top-k", 0.0, 4.0 * t * E + 8.0 * t * k),
        ("grouping", 0.0, 4.0 * t * k + 4.0 * (E + 1) + 8.0 * r),
        ("up GEMM (rows read from x by index)", 2.0 * r * 2 * I * H,
         2.0 * touched_up * 2 * I * H + 2.0 * t * H + 4.0 * r + 4.0 * r * 2 * I),
        ("SwiGLU", 0.0, 4.0 * r * 2 * I + 2.0 * r * I),
        ("down GEMM", 2.0 * r * H * I, 2.0 * touched_down * H * I + 2.0 * r * I + 4.0 * r * H),
        ("combine", 0.0, 4.0 * r * H + 12.0 * t * k + 4.0 * t * H),
    ]


def _roof(flops, nbytes, us):
    """The binding roofline of one kernel's algorithmic work and its achieved rate."""
    if flops / (PEAK_BF16_TFLOPS * 1e12) >= nbytes / (PEAK_HBM_GBS * 1e9):
        a = flops / (us * 1e-6) / 1e12
        return {"bound": "mfma", "achieved": a, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": a / PEAK_BF16_TFLOPS}
    a = nbytes / (us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": a, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": a / PEAK_HBM_GBS}


def run_moe_layer(args, bg):
    """One step = the whole expert layer (router, top-k, grouping, up
    projection reading token rows by index, SwiGLU, down projection, combine;
    one bi_moe_run call) at
    every token count T of the sweep.  Two layer handles over two copies of
    the weights alternate, so the Infinity Cache does not keep a call's
    experts for the next call of the same T.  A second pass runs the steps
    one by one through their own entry points (the same bits) with events
    around each, for the per-kernel breakdown and roofline.  Where the layer
    applies SwiGLU in the up projection's epilogue (T = 256 and 4096 here), that pass
    times the up projection and SwiGLU as the two separate calls."""
    import ctypes

    import numpy as np
    import torch

    import synth

    E, k, H, I = MOE["experts"], MOE["topk"], MOE["up"][1], MOE["down"][1]
    tokens = MOE["tokens"]
    tmax = max(tokens)
    wr, wu, wd = _moe_layer_weights()
    dev = [tuple(to_dev(w) for w in (wr, wu, wd))]
    dev.append(tuple(w.clone() for w in dev[0]))
    layers = [bg.MoeLayer(*d, k=k, max_tokens=tmax) for d in dev]
    xs = {t: to_dev(synth.normal_bf16(500 + t, (t, H))) for t in tokens}
    ys = {t: torch.empty((t, H), dtype=torch.float32, device="cuda:0") for t in tokens}
    lib = bg.load()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    cargs = [(t, ctypes.c_void_p(xs[t].data_ptr()), ctypes.c_void_p(ys[t].data_ptr())) for t in tokens]
    hs = [l._h for l in layers]
    call_no = [0]

    def step(events=None):
        for j, (t, xp, yp) in enumerate(cargs):
            h = hs[call_no[0] % 2]
            call_no[0] += 1
            if events is not None:
                events[j][0].record()
            st = lib.bi_moe_run(h, xp, t, yp, stream)
            if st != 0:
                bg.check(st)
            if events is not None:
                events[j][1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [[[LaunchEvent(), LaunchEvent()] for _ in tokens]
          for _ in range(args.steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for s_ in range(args.steps):
        step(ev[s_])
    t1.record()
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps
    per_t = {t: float(np.mean([ev[s_][j][0].elapsed_time(ev[s_][j][1]) for s_ in range(args.steps)]))
             for j, t in enumerate(tokens)}

    # per-step breakdown: the steps called one by one on the same inputs
    breakdown, layer_flops = [], {}
    for t in tokens:
        steps_t, touched = _moe_steps_timed(bg, lib, dev, xs[t], t, args.steps)
        work = moe_layer_work(t, touched, touched)
        layer_flops[t] = sum(w[1] for w in work)
        for (name, fl, by), us in zip(work, steps_t):
            r = _roof(fl, by, us)
            breakdown.append({"T": t, "step": name, "us": round(us, 2), "bound": r["bound"],
                              "achieved": round(r["achieved"], 1), "unit": r["unit"], "frac": round(r["frac"], 3),
                              "_work": (fl, by), "_us": us})
    step_flops = sum(layer_flops.values())
    dom = max(breakdown, key=lambda b: b["_us"])
    roof = _roof(dom["_work"][0], dom["_work"][1], dom["_us"])
    t = dom["T"]
    for b in breakdown:
        del b["_work"], b["_us"]
    roof.update({"traffic": None, "kernel": "%s at T=%d" % (dom["step"], t), "launches_per_step": 1,
                 "avg_launch_us": dom["us"]})
    cpu = None
    if not args.no_cpu_baseline:
        cpu = moe_layer_cpu_baseline(wr, wu, wd)
    per = [{"T": t, "us": round(per_t[t] * 1e3, 2), "tflops": round(layer_flops[t] / (per_t[t] * 1e-3) / 1e12, 1),
            "tokens_per_s": round(t / (per_t[t] * 1e-3), 0)} for t in tokens]
    out = {
        "metric": "batch-invariant bf16 GEMM TFLOPS (M sweep) + % MFMA/HBM roofline, 1 GPU",
        "value": round(step_flops / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; W ~ N(0,%g), x ~ N(0,1); routing computed by the layer)" % MOE["std"],
        "config": {"workload": "MoE expert layer (Qwen3-30B-A3B-style): router [128,2048], top-8, "
                               "up [128,1536,2048], SwiGLU, down [128,2048,768], combine; T in {1,16,256,4096}",
                   "tokens": tokens, "weight_copies_rotated": 2, "kernel_source_sha256_16": kernel_hash()},
        "roofline": roof,
        "cpu_baseline": cpu,
        "per_T": per,
        "steps_breakdown": breakdown,
        "breakdown_note": "steps through their own entry points, each run queued behind a short spin kernel so "
                          "that the events time the GPU rather than the host's launches; the layer itself runs the "
                          "up projection and SwiGLU as one kernel when the rows average 16 or more per expert "
                          "(T = 256 and 4096 here)",
    }
    print(json.dumps(out), flush=True)
    return 0


SPIN_CYCLES = 2_000_000  # the spin kernel's clock cycles: about 1 ms, longer than queueing a run's calls


def _moe_steps_timed(bg, lib, dev, x, t, reps):
    """The layer's steps through their own entry points, events around each;
    mean microseconds per step over `reps` runs alternating the two weight
    copies, and the number of experts the routing touches."""
    import ctypes

    import numpy as np
    import torch

    E, k, H, I = MOE["experts"], MOE["topk"], MOE["up"][1], MOE["down"][1]
    r = t * k
    d = "cuda:0"
    logits = torch.empty((t, E), dtype=torch.float32, device=d)
    ids = torch.empty((t, k), dtype=torch.int32, device=d)
    w = torch.empty((t, k), dtype=torch.float32, device=d)
    off = torch.empty(E + 1, dtype=torch.int32, device=d)
    tok = torch.empty(r, dtype=torch.int32, device=d)
    row_of = torch.empty((t, k), dtype=torch.int32, device=d)
    h = torch.empty((r, 2 * I), dtype=torch.float32, device=d)
    a = torch.empty((r, I), dtype=torch.bfloat16, device=d)
    o = torch.empty((r, H), dtype=torch.float32, device=d)
    y = torch.empty((t, H), dtype=torch.float32, device=d)
    P = lambda v: ctypes.c_void_p(v.data_ptr())  # noqa: E731
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    handles = [(bg.Gemm(wr), bg.GroupedGemm(wu), bg.GroupedGemm(wd)) for wr, wu, wd in dev]
    calls = [
        lambda g: g[0].run_ptr(x.data_ptr(), t, logits.data_ptr()),
        lambda g: lib.bi_moe_topk(P(logits), t, E, k, P(ids), P(w), st),
        lambda g: lib.bi_moe_permute(P(ids), t, E, k, P(off), P(tok), P(row_of), st),
        lambda g: lib.bi_grouped_gemm_run_indexed(g[1]._h, P(x), t, P(tok), P(off), r, P(h), st),
        lambda g: lib.bi_swiglu(P(h), r, I, P(a), st),
        lambda g: lib.bi_grouped_gemm_run(g[2]._h, P(a), P(off), r, P(o), st),
        lambda g: lib.bi_moe_combine(P(o), r, P(ids), P(w), P(row_of), t, k, H, P(y), st),
    ]
    for c in calls:
        bg.check(c(handles[0]) or 0)
    torch.cuda.synchronize()
    touched = int(np.count_nonzero(np.diff(off.cpu().numpy())))
    ev = [[(LaunchEvent(), LaunchEvent()) for _ in calls]
          for _ in range(reps)]
    for i in range(reps):
        g = handles[i % len(handles)]
        # a short spin kernel ahead of each run, so that the host has queued
        # the run's calls before the GPU reaches them: the events then time
        # the GPU's work, not the host's launches (which at T = 1 take longer)
        torch.cuda._sleep(SPIN_CYCLES)
        for j, c in enumerate(calls):
            ev[i][j][0].record()
            bg.check(c(g) or 0)
            ev[i][j][1].record()
    torch.cuda.synchronize()
    us = [float(np.mean([ev[i][j][0].elapsed_time(ev[i][j][1]) for i in range(reps)])) * 1e3
          for j in range(len(calls))]
    return us, touched


def moe_layer_cpu_baseline(wr, wu, wd, target_s=15.0):
    """The oracle's steps of the layer chained on the host cores, on a bounded
    sample: as many tokens of the T=4096 input as fit in about `target_s`."""
    import numpy as np

    import oracle
    import synth

    E, k, H, I = MOE["experts"], MOE["topk"], MOE["up"][1], MOE["down"][1]
    x = synth.normal_bf16(500 + 4096, (4096, H))

    def chain(xb):
        lg, _ = oracle.gemm_f64(xb, wr)
        ids, w = oracle.moe_topk(lg.astype(np.float32), k)
        off, tok, row_of = oracle.moe_permute(ids, E)
        h, _ = oracle.grouped_f64(xb[tok], wu, off)
        a = synth.f32_to_bf16_bits(oracle.swiglu_f64(h.astype(np.float32)).astype(np.float32))
        o, _ = oracle.grouped_f64(a, wd, off)
        return oracle.moe_combine_f64(o.astype(np.float32), w.astype(np.float32), row_of)[0]

    chain(x[:1])
    t0 = time.perf_counter()
    chain(x[:4])
    probe = max(time.perf_counter() - t0, 1e-3) / 4
    n = int(max(4, min(4096, target_s / probe)))
    t0 = time.perf_counter()
    chain(x[:n])
    dt = time.perf_counter() - t0
    fl = n * (2.0 * E * H + 2.0 * k * 2 * I * H + 2.0 * k * H * I)
    return {"value": fl / dt / 1e12, "unit": "TFLOPS", "cores": oracle.max_threads(), "cpu": host_cpu(),
            "kind": "oracle",
            "sample": "fp64 oracle steps of the layer chained on the first %d of the 4096 tokens, %.1f s" % (n, dt)}


def run_norm_gate_up(args, bg):
    """One step = at every M of the gate+up sweep, RMSNorm of the raw hidden
    rows (bf16 [M, 4096], rows at scales 2^-4 .. 2^4, gain near 1) followed
    by the gate+up projection of the normalised rows (W bf16 [28672, 4096]),
    weights rotating over copies as in the dense sweep.  Reports the GEMM
    throughput of the pair (TFLOPS), and the norm's own time and HBM rate."""
    import ctypes

    import numpy as np
    import torch

    import synth

    wl = WORKLOADS["llama8b_gate_up"]
    n, k, ms = wl["n"], wl["k"], list(wl["ms"])
    if args.m:
        ms = [int(v) for v in args.m.split(",")]
    mmax = max(ms)
    w0 = to_dev(synth.normal_bf16(42, (n, k), wl["std"]))
    copies = max(1, int(np.ceil(args.rotate_gib * 2 ** 30 / (2 * n * k))))
    ws = [w0] + [w0.clone() for _ in range(copies - 1)]
    handles = [bg.Gemm(w) for w in ws]
    raw = synth.normal_bf16(43, (mmax, k))
    scale = np.exp2(synth.rng(44).integers(-4, 5, size=(mmax, 1))).astype(np.float32)
    xraw = to_dev(synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(raw) * scale))
    gain_f = 1.0 + synth.bf16_bits_to_f32(synth.normal_bf16(45, (k,), 0.1))
    gain = to_dev(synth.f32_to_bf16_bits(gain_f.astype(np.float32)))
    xn = torch.empty((mmax, k), dtype=torch.bfloat16, device="cuda:0")
    ys = {m: torch.empty((m, n), dtype=torch.float32, device="cuda:0") for m in ms}
    lib = bg.load()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    hps = [h._h for h in handles]
    call_no = [0]

    def step(events=None):
        for j, m in enumerate(ms):
            h = hps[call_no[0] % copies]
            call_no[0] += 1
            if events is not None:
                events[j][0].record()
            st = lib.bi_rmsnorm(P(xraw), P(gain), m, k, ctypes.c_float(1e-5), P(xn), stream)
            if st != 0:
                bg.check(st)
            if events is not None:
                events[j][1].record()
            st = lib.bi_gemm_run(h, P(xn), m, P(ys[m]), stream)
            if st != 0:
                bg.check(st)
            if events is not None:
                events[j][2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [[[LaunchEvent() for _ in range(3)] for _ in ms] for _ in range(args.steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for s_ in range(args.steps):
        step(ev[s_])
    t1.record()
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps
    norm_us = {m: 1e3 * float(np.median([ev[s_][j][0].elapsed_time(ev[s_][j][1]) for s_ in range(args.steps)]))
               for j, m in enumerate(ms)}
    gemm_us = {m: 1e3 * float(np.median([ev[s_][j][1].elapsed_time(ev[s_][j][2]) for s_ in range(args.steps)]))
               for j, m in enumerate(ms)}
    flops = {m: 2.0 * m * n * k for m in ms}
    norm_bytes = {m: 4.0 * m * k + 2.0 * k for m in ms}
    names = {m: handles[0].kernel_name(m) for m in ms}
    # dominant kernel: the GEMM kernel with the most time per step
    by_kernel = {}
    for m in ms:
        d = by_kernel.setdefault(names[m], [0.0, 0.0, 0.0, 0])
        d[0] += gemm_us[m]
        d[1] += flops[m]
        d[2] += 2.0 * n * k + 2.0 * m * k + 4.0 * m * n
        d[3] += 1
    dom = max(by_kernel, key=lambda kn: by_kernel[kn][0])
    us, fl, by, launches = by_kernel[dom]
    roof = _roof(fl, by, us)
    roof.update({"traffic": None, "kernel": dom, "launches_per_step": launches, "avg_launch_us": us / launches})
    norm_total_us = sum(norm_us.values())
    norm_roof = _roof(0.0, sum(norm_bytes.values()), norm_total_us)

    # A/B: the norm fused into the GEMM's prologue (bi_rmsnorm_gemm_run: an
    # r-per-row pass, then the GEMM normalising its x tiles in LDS), same
    # inputs and weight rotation, events around each call
    rstd = torch.empty(mmax, dtype=torch.float32, device="cuda:0")

    def fused_step(events=None):
        for j, m in enumerate(ms):
            h = hps[call_no[0] % copies]
            call_no[0] += 1
            if events is not None:
                events[j][0].record()
            st = lib.bi_rmsnorm_gemm_run(h, P(xraw), P(gain), ctypes.c_float(1e-5), m, P(rstd), P(ys[m]), stream)
            if st != 0:
                bg.check(st)
            if events is not None:
                events[j][1].record()

    for _ in range(args.warmup):
        fused_step()
    torch.cuda.synchronize()
    fev = [[[LaunchEvent() for _ in range(2)] for _ in ms] for _ in range(args.steps)]
    f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    f0.record()
    for s_ in range(args.steps):
        fused_step(fev[s_])
    f1.record()
    torch.cuda.synchronize()
    fused_ms_per_step = f0.elapsed_time(f1) / args.steps
    fused_us = {m: 1e3 * float(np.median([fev[s_][j][0].elapsed_time(fev[s_][j][1]) for s_ in range(args.steps)]))
                for j, m in enumerate(ms)}
    fused_ab = {"what": "norm fused into the GEMM prologue (r-per-row pass, then the GEMM normalising its x tiles "
                        "in LDS) against bi_rmsnorm then bi_gemm_run; bit-identical outputs",
                "separate_ms_per_step": round(ms_per_step, 4), "fused_ms_per_step": round(fused_ms_per_step, 4),
                "per_m": [{"M": m, "separate_us": round(norm_us[m] + gemm_us[m], 2), "fused_us": round(fused_us[m], 2),
                           "fused_gemm_kernel": handles[0].rmsnorm_kernel_name(m), "separate_gemm_kernel": names[m]}
                          for m in ms]}
    per = [{"M": m, "norm_us": round(norm_us[m], 2), "norm_gbs": round(norm_bytes[m] / (norm_us[m] * 1e-6) / 1e9, 0),
            "gemm_us": round(gemm_us[m], 2), "gemm_kernel": names[m],
            "gemm_tflops": round(flops[m] / (gemm_us[m] * 1e-6) / 1e12, 1)} for m in ms]
    out = {
        "metric": "batch-invariant bf16 GEMM TFLOPS (M sweep) + % MFMA/HBM roofline, 1 GPU",
        "value": round(sum(flops.values()) / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; W ~ N(0,%g), raw rows N(0,1) at scales 2^-4..2^4, gain ~ 1+N(0,0.1))" % wl["std"],
        "config": {"workload": "Llama-3.1-8B RMSNorm (H=4096, eps 1e-5) then fused gate+up GEMM, "
                               "W bf16 [28672,4096], M in {32,544,2080,8224}",
                   "m_sweep": ms, "weight_copies_rotated": copies, "kernel_source_sha256_16": kernel_hash()},
        "roofline": roof,
        "norm_roofline": dict(norm_roof, kernel="rmsnorm_rows",
                              share_of_step=round(norm_total_us / (ms_per_step * 1e3), 4)),
        "fused_norm_ab": fused_ab,
        "cpu_baseline": None,
        "per_m": per,
    }
    print(json.dumps(out), flush=True)
    return 0


ATTN = dict(batch=256, hq=32, hkv=8, d=128, split=512, splits_tried=[256, 512, 1024, 2048], median=1024.0,
            sigma=0.8, lo=16, hi=8192, pool=32768)


def run_decode_attn(args, bg):
    """One step = one decode-attention call over a Llama-3.1-8B decode batch:
    256 sequences (a decode batch of CoRun's size) with ragged KV lengths
    (lognormal, median 1024, clipped to 16 .. 8192), 32 query heads, 8 kv
    heads, head dim 128, split size 512.  The KV cache is bf16, token-major;
    its values come from a seeded pool of 32768 token rows repeated to the
    batch's length (values do not change the work).  Roofline: HBM, with the
    keys, values, queries and outputs as the algorithmic bytes."""
    import ctypes

    import numpy as np
    import torch

    import synth

    a = ATTN
    lengths = synth.decode_lengths(800, a["batch"], a["median"], a["sigma"], a["lo"], a["hi"])
    st = np.zeros(a["batch"] + 1, np.int32)
    st[1:] = np.cumsum(lengths)
    ntok = int(st[-1])
    row = a["hkv"] * a["d"]
    pool_k = to_dev(synth.normal_bf16(801, (a["pool"], row)))
    pool_v = to_dev(synth.normal_bf16(802, (a["pool"], row)))
    reps = (ntok + a["pool"] - 1) // a["pool"]
    k = pool_k.repeat(reps, 1)[:ntok].reshape(ntok, a["hkv"], a["d"]).contiguous()
    v = pool_v.repeat(reps, 1)[:ntok].reshape(ntok, a["hkv"], a["d"]).contiguous()
    del pool_k, pool_v
    q = to_dev(synth.normal_bf16(803, (a["batch"], a["hq"], a["d"])))
    std = torch.as_tensor(st, device="cuda:0")
    out = torch.empty((a["batch"], a["hq"], a["d"]), dtype=torch.float32, device="cuda:0")
    scale = 1.0 / np.sqrt(a["d"])
    kv_bytes = 2.0 * 2 * ntok * row
    alg_bytes = kv_bytes + 2.0 * q.numel() + 4.0 * out.numel()
    flops = 4.0 * float(lengths.sum()) * a["hq"] * a["d"]
    lib = bg.load()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731

    def timed(split, steps, warmup):
        att = bg.DecodeAttention(a["hq"], a["hkv"], split, a["batch"], a["hi"])
        args_ = (att._h, P(q), P(k), P(v), P(std), a["batch"], ntok, ctypes.c_float(scale), P(out), stream)
        for _ in range(warmup):
            bg.check(lib.bi_attn_decode(*args_))
        torch.cuda.synchronize()
        ev = [(LaunchEvent(), LaunchEvent()) for _ in range(steps)]
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for e0, e1 in ev:
            e0.record()
            st_ = lib.bi_attn_decode(*args_)
            if st_ != 0:
                bg.check(st_)
            e1.record()
        t1.record()
        torch.cuda.synchronize()
        att.close()
        return t0.elapsed_time(t1) / steps, float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))

    sweep = {}
    for split in a["splits_tried"]:
        if split != a["split"]:
            sweep[split] = round(timed(split, 5, 2)[1] * 1e3, 2)
    ms_per_step, per_call = timed(a["split"], args.steps, args.warmup)
    sweep[a["split"]] = round(per_call * 1e3, 2)
    roof = _roof(0.0, alg_bytes, per_call * 1e3)
    roof.update({"traffic": None, "kernel": "attn_split + attn_combine (one call)", "launches_per_step": 1,
                 "avg_launch_us": per_call * 1e3})
    cpu = None
    if not args.no_cpu_baseline:
        cpu = attn_cpu_baseline(q, k, v, st, scale)
    out_j = {
        "metric": "batch-invariant bf16 GEMM TFLOPS (M sweep) + % MFMA/HBM roofline, 1 GPU",
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 3),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; q, K, V ~ N(0,1); lengths lognormal median 1024, 16..8192)",
        "config": {"workload": "Llama-3.1-8B decode attention: 256 sequences, 32 q heads, 8 kv heads, head dim 128, "
                               "ragged KV lengths, split size 512",
                   "total_keys": ntok, "kv_bytes": kv_bytes, "split": a["split"]},
        "roofline": roof,
        "cpu_baseline": cpu,
        "split_sweep_us": sweep,
        "kv_gbs": round(kv_bytes / (per_call * 1e-3) / 1e9, 0),
    }
    print(json.dumps(out_j), flush=True)
    return 0


def attn_cpu_baseline(q, k, v, st, scale, target_s=10.0):
    """The oracle on the host cores, on a bounded sample: the first sequences
    of the batch, as many as fit in about `target_s` seconds."""
    import numpy as np
    import torch

    import oracle

    qb = q.view(torch.int16).cpu().numpy().view(np.uint16)
    b = 0
    t_total = 0.0
    keys = 0
    while b < len(st) - 1 and t_total < target_s:
        lo, hi = int(st[b]), int(st[b + 1])
        kb = k[lo:hi].view(torch.int16).cpu().numpy().view(np.uint16)
        vb = v[lo:hi].view(torch.int16).cpu().numpy().view(np.uint16)
        t0 = time.perf_counter()
        oracle.decode_attn_f64(qb[b:b + 1], kb, vb, np.array([0, hi - lo], np.int32), scale)
        t_total += time.perf_counter() - t0
        keys += hi - lo
        b += 1
    flops = 4.0 * keys * q.shape[1] * q.shape[2]
    return {"value": flops / t_total / 1e12, "unit": "TFLOPS", "cores": oracle.max_threads(), "cpu": host_cpu(),
            "kind": "oracle",
            "sample": "fp64 oracle on the first %d sequences (%d keys) of the batch, %.1f s" % (b, keys, t_total)}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama8b_down",
                    choices=sorted(WORKLOADS) + ["moe", "moe_layer", "norm_gate_up", "decode_attn"])
    ap.add_argument("--rotate-gib", type=float, default=1.0,
                    help="weight copies to rotate over, in GiB (defeats the Infinity Cache)")
    ap.add_argument("--m", type=str, default=None,
                    help="comma-separated M values replacing the workload's sweep (profiling)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--no-compare", action="store_true",
                    help="skip the cost-of-invariance and hipBLASLt context measurements")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path "
              "(rows are independent, so data parallelism needs no exchange); "
              "run with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import invariant_bi_gemm_amd as bg

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    bg.load()
    if args.workload == "moe":
        return run_moe(args, bg)
    if args.workload == "moe_layer":
        return run_moe_layer(args, bg)
    if args.workload == "norm_gate_up":
        return run_norm_gate_up(args, bg)
    if args.workload == "decode_attn":
        return run_decode_attn(args, bg)
    wl = dict(WORKLOADS[args.workload])
    if args.m:
        wl["ms"] = [int(v) for v in args.m.split(",")]
    n, k, ms = wl["n"], wl["k"], wl["ms"]
    w_bits, x_bits = make_inputs(wl)
    w0 = to_dev(w_bits)
    copies = max(1, int(np.ceil(args.rotate_gib * 2 ** 30 / (2 * n * k))))
    ws = [w0] + [w0.clone() for _ in range(copies - 1)]
    handles = [bg.Gemm(w) for w in ws]
    xd = to_dev(x_bits)
    ys = {m: torch.empty((m, n), dtype=torch.float32, device="cuda:0") for m in ms}
    names = {m: handles[0].kernel_name(m) for m in ms}
    flops = {m: 2.0 * m * n * k for m in ms}
    hbm_bytes = {m: 2.0 * n * k + 2.0 * m * k + 4.0 * m * n for m in ms}

    if args.copy_calibration:
        a = torch.empty(2 ** 29, dtype=torch.int16, device="cuda:0")  # 1 GiB
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    # the timed calls go straight to the C ABI with precomputed arguments, so
    # the host keeps ahead of the GPU even for the decode-size calls
    import ctypes

    lib = bg.load()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    xp = ctypes.c_void_p(xd.data_ptr())
    yps = {m: ctypes.c_void_p(ys[m].data_ptr()) for m in ms}
    hps = [h._h for h in handles]
    run = lib.bi_gemm_run
    call_no = [0]

    def step(events=None, spans=None):
        # events[i]: the event pair around the launches of span i, spans the
        # (first, last) launch indices of each span (None: every launch its
        # own span)
        first = {a: i for i, (a, _) in enumerate(spans)} if spans is not None else None
        last = {b: i for i, (_, b) in enumerate(spans)} if spans is not None else None
        for j, m in enumerate(ms):
            h = hps[call_no[0] % copies]
            call_no[0] += 1
            if events is not None and (first is None or j in first):
                events[j if first is None else first[j]][0].record()
            st = run(h, xp, m, yps[m], stream)
            if st != 0:
                bg.check(st)
            if events is not None and (last is None or j in last):
                events[j if last is None else last[j]][1].record()

    def new_events():
        return [[[LaunchEvent(), LaunchEvent()] for _ in ms]
                for _ in range(args.steps)]

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # per call: K instrumented steps, outside the timed region, with an event
    # pair around every launch (the median over the steps of each launch's
    # pair); the pairs leave gaps of about 8 us between launches (6% of a
    # step in the kernel trace), so the timed steps carry only the dominant
    # kernel's
    ev = new_events()
    for s in range(args.steps):
        step(ev[s])
    torch.cuda.synchronize()
    per_call_ms = {m: float(np.median([ev[s][j][0].elapsed_time(ev[s][j][1]) for s in range(args.steps)]))
                   for j, m in enumerate(ms)}

    # dominant kernel: the one with the most time per step
    by_kernel = {}
    for m in ms:
        d = by_kernel.setdefault(names[m], {"ms": 0.0, "flops": 0.0, "bytes": 0.0, "launches": 0})
        d["flops"] += flops[m]
        d["bytes"] += hbm_bytes[m]
        d["launches"] += 1
        d["ms_probe"] = d.get("ms_probe", 0.0) + per_call_ms[m]
    dom = max(by_kernel, key=lambda kname: by_kernel[kname]["ms_probe"])
    dom_calls = [j for j, m in enumerate(ms) if names[m] == dom]
    # its launches as runs of consecutive calls, one event pair around each
    # run (every pair leaves a gap of a few us before the next launch)
    dom_spans = []
    for j in dom_calls:
        if dom_spans and dom_spans[-1][1] == j - 1:
            dom_spans[-1] = (dom_spans[-1][0], j)
        else:
            dom_spans.append((j, j))

    # timed region: K steps, events around the dominant kernel's runs of
    # launches (on the launch stream) for its roofline
    ev = new_events()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for s in range(args.steps):
        step(ev[s], dom_spans)
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    # per step: the dominant kernel's time, the sum of its spans; the median
    # over the timed steps
    dom_ms = float(np.median([sum(ev[s][i][0].elapsed_time(ev[s][i][1]) for i in range(len(dom_spans)))
                              for s in range(args.steps)]))

    step_flops = sum(flops.values())
    ms_per_step = total_ms / args.steps
    value = step_flops / (ms_per_step * 1e-3) / 1e12

    d = by_kernel[dom]
    d["ms"] = dom_ms
    if "stream" in dom:
        achieved = d["bytes"] / (d["ms"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        achieved = d["flops"] / (d["ms"] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    # the committed counter profiles were taken on the default workload's
    # sweep (llama8b_down, every M): another workload gets null, not that
    # sweep's figures for a kernel of the same name
    profiled = args.workload == "llama8b_down" and not args.m
    roof["traffic"] = read_traffic(dom) if profiled else None
    roof["kernel"] = dom
    roof["launches_per_step"] = d["launches"]
    roof["avg_launch_us"] = d["ms"] * 1e3 / d["launches"]
    roof["launch_us_statistic"] = ("the kernel's time per step (an event pair around each run of its consecutive "
                                   "launches, the only events in the timed region), median over the timed steps, "
                                   "divided by its launches per step")
    roof["event_spans_per_step"] = len(dom_spans)
    # the MFMA peak scales with the engine clock: the same fraction against
    # the peak at the clock the kernel sustains (committed rocprof counters of
    # the current kernels; null otherwise)
    clock = read_clock(dom) if profiled else None
    roof["sustained_clock_ghz"] = clock
    roof["clock_source"] = ("rocprof GRBM_GUI_ACTIVE / dispatch duration, %s" % os.path.relpath(CLOCK_FILE, ROOT)
                            if clock else "no current counter profile of this workload")
    if clock and roof["bound"] == "mfma":
        peak_at_clock = PEAK_BF16_TFLOPS * clock / PEAK_CLOCK_GHZ
        roof["peak_at_sustained_clock"] = round(peak_at_clock, 1)
        roof["frac_at_sustained_clock"] = roof["achieved"] / peak_at_clock

    per_m = []  # from the instrumented steps before the timed region
    for m in ms:
        t = per_call_ms[m] * 1e-3
        per_m.append({"M": m, "us": round(per_call_ms[m] * 1e3, 2), "kernel": names[m],
                      "tflops": round(flops[m] / t / 1e12, 1),
                      "hbm_gbs": round(hbm_bytes[m] / t / 1e9, 0)})

    compare = None
    alt = None
    if not args.no_compare:
        compare = invariance_cost(bg, ws, xd, ms, n, k)
        if args.workload == "llama8b_down" and not args.m:
            alt = alternative_pin(bg, ws, xd, ms, n, k, args.steps, args.warmup, per_call_ms)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w_bits, x_bits, n, k)

    out = {
        "metric": "batch-invariant bf16 GEMM TFLOPS (M sweep) + % MFMA/HBM roofline, 1 GPU",
        "value": round(value, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; W ~ N(0,%g), %s)" % (wl["std"], wl["x"]),
        "config": {"workload": wl["desc"], "N": n, "K": k, "m_sweep": ms,
                   "weight_copies_rotated": copies, "kernel_source_sha256_16": kernel_hash()},
        "roofline": roof,
        "cpu_baseline": cpu,
        "per_m": per_m,
        "invariance_cost": compare,
        "alternative_pin": alt,
        "peak_tflops_in_sweep": max(p["tflops"] for p in per_m),
        "context": "pages' numbers (H100, other hardware): vendor GEMM 527 TFLOPS vs Triton "
                   "batch-invariant 194 TFLOPS peak on this layer",
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

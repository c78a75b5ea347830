#!/usr/bin/env python3
"""MoE-layer benchmark on one MI355X.

One step = one moe_forward call: router GEMM + softmax top-k, dispatch, routed and shared SwiGLU
experts, weighted combine -- the whole forward pass of the block over one batch of synthetic input
that is already resident in HBM. Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload prefill|decode|mid|skew|tiny]

The default workload is the prefill-shaped large layer (T=16384, d=8192, E=512, k=10,
I=I_shared=2048, bf16, fp32 router), bound by the bf16 matrix cores; the line's "decode" key holds
the decode-shaped run (T=32, the first 32 rows of the same input) on the same weights in the same
process, bound by HBM. Step times are per-step HIP events on the library's stream; `value` is
tokens / median step time. The dominant kernel (grouped gate/up GEMM) is timed with HIP events
recorded around its launch inside every timed step; its algorithmic FLOPs (prefill) or bytes
(decode) over its median launch time give the roofline fraction. The CPU oracle is timed on a
bounded token sample of the headline workload as a reported baseline.
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

METRIC = "MoE-layer tokens/s; % HBM BW peak (decode) / % bf16 MFMA peak (prefill)"
KERNEL_FFN_GATE_UP = 3
# sources the dominant kernel (grouped gate/up GEMM) is compiled from
KERNEL_SOURCES = [os.path.join(ROOT, "sparse_mixture_experts_softmax_amd", "csrc", f)
                  for f in ("grouped_ffn.hip", "stream_gemm.h", "moe_internal.h")]


def kernel_source_hash():
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        h.update(open(path, "rb").read())
    return h.hexdigest()


class HipEvents:
    """Raw HIP events through libamdhip64 (torch's events only see torch's current stream object)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    # hipEventDisableSystemFence: a timing-only event, recorded without the system-scope fence
    # (cache write-back and invalidation) that a default event performs. Around the dominant
    # kernel in every timed step, default events cost ~6 us of idle GPU before the kernel and
    # after it.
    DISABLE_SYSTEM_FENCE = 0x20000000

    def create(self, timing_only=False):
        ev = ctypes.c_void_p()
        if timing_only:
            rc = self.hip.hipEventCreateWithFlags(ctypes.byref(ev), self.DISABLE_SYSTEM_FENCE)
        else:
            rc = self.hip.hipEventCreate(ctypes.byref(ev))
        if rc != 0:
            raise RuntimeError("hipEventCreate failed: %d" % rc)
        return ev

    def record(self, ev, stream):
        rc = self.hip.hipEventRecord(ev, ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError("hipEventRecord failed: %d" % rc)

    def ms(self, a, b):
        self.hip.hipEventSynchronize(b)
        out = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(out), a, b)
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed: %d" % rc)
        return float(out.value)

    def destroy(self, ev):
        self.hip.hipEventDestroy(ev)


def traffic_for(workload):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3 counter summary,
    or None if there is none or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "ffn_gate_up_%s_traffic.json" % workload)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(cfg, sample_tokens):
    """The CPU oracle, as it stands, on a seeded sample of the workload's tokens."""
    import numpy as np

    import oracle
    import synthetic as syn

    rng = np.random.default_rng(99)
    tokens = np.sort(rng.choice(cfg.T, size=min(sample_tokens, cfg.T), replace=False))
    x = syn.host_x(cfg, rows=tokens)
    wr = syn.host_router(cfg)
    bias = syn.router_bias(cfg)
    idx, _, _, _ = oracle.router(x, wr, cfg.k, renorm=bool(cfg.renorm), bias=bias)
    need = sorted(set(idx.ravel().tolist()))
    wg, wu, wd = [None] * cfg.E, [None] * cfg.E, [None] * cfg.E
    for e in need:
        wg[e], wu[e], wd[e] = syn.host_expert(cfg, e)
    wgs, wus, wds = syn.host_shared(cfg)
    # whole passes over the sample until at least CPU_MIN_S of oracle time
    passes, dt = 0, 0.0
    while dt < CPU_MIN_S and passes < 1000:
        t0 = time.perf_counter()
        oracle.forward(x, wr, wg, wu, wd, wgs, wus, wds, cfg.k, renorm=bool(cfg.renorm), bias=bias)
        dt += time.perf_counter() - t0
        passes += 1
    return {"value": passes * len(tokens) / dt, "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": "%d of the %d tokens (seeded), the whole block per token, %d pass(es), %.1f s, on %s"
                      % (len(tokens), cfg.T, passes, dt, cpu_model())}


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), for the baseline's record."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


CPU_SAMPLE = {"tiny": 64, "mid": 4096, "decode": 32, "prefill": 16, "skew": 16}
CPU_MIN_S = 10.0


def calibrate():
    """Reference points on this GPU, outside the MoE path: the vendor bf16 GEMM (torch.matmul,
    hipBLASLt) on dense shapes, including one expert's gate/up shape, and device copy bandwidth."""
    import torch

    def t_ms(fn, n=20):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    out = {"matmul_bf16": [], "copy": []}
    for (M, K, N) in [(8192, 8192, 8192), (4096, 8192, 4096), (16384, 2048, 8192), (320, 8192, 4096)]:
        A = torch.randn(M, K, device="cuda", dtype=torch.bfloat16)
        B = torch.randn(K, N, device="cuda", dtype=torch.bfloat16)
        ms = t_ms(lambda: A @ B)
        out["matmul_bf16"].append({"M": M, "K": K, "N": N, "ms": ms, "tflops": 2 * M * K * N / ms / 1e9})
        del A, B
    for nbytes in [1 << 30, 4 << 30]:
        src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        ms = t_ms(lambda: dst.copy_(src), 10)
        out["copy"].append({"bytes": nbytes, "ms": ms, "read_plus_write_tbps": 2 * nbytes / ms / 1e9})
        del src, dst
    print(json.dumps(out), flush=True)


SWEEP_T = [1, 2, 4, 8, 16, 32, 64, 128, 256, 512]


def sweep(steps, warmup):
    """Token-count sweep at the large layer shape (d=8192, E=512, k=10, I=I_shared=2048, bf16):
    one JSON line per T with the layer's tokens/s and its fraction of HBM peak over the bytes the
    routing of that input requires (touched experts, shared expert, router weight, x and out)."""
    import torch

    import sparse_mixture_experts_softmax_amd as moe
    import synthetic as syn
    from sparse_mixture_experts_softmax_amd import workload as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    moe.load_library()
    big = syn.CONFIGS["decode"].with_(name="sweep", T=max(SWEEP_T))
    print("bench: sweep %s at T in %s" % (big, SWEEP_T), file=sys.stderr, flush=True)
    inp = syn.device_inputs(big, device=dev)  # token t's row does not depend on T
    stream = torch.cuda.current_stream(dev).cuda_stream
    hip = HipEvents()
    for T in SWEEP_T:
        cfg = big.with_(T=T)
        x = inp["x"][:T]
        dims = moe.dims_for(x, inp["w_router"], inp["wg"], inp["wg_s"], cfg.k, bool(cfg.renorm))
        ws = moe.workspace(dims, dev)
        out = torch.empty_like(x)

        def step():
            moe.moe_forward(x, inp["w_router"], inp["wg"], inp["wu"], inp["wd"], inp["wg_s"], inp["wu_s"],
                            inp["wd_s"], cfg.k, renormalize=bool(cfg.renorm), router_bias=None, ws=ws, out=out,
                            dims=dims)

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        a, b = hip.create(), hip.create()
        hip.record(a, stream)
        for _ in range(steps):
            step()
        hip.record(b, stream)
        ms = hip.ms(a, b) / steps
        hip.destroy(a)
        hip.destroy(b)
        _, idx, _, _ = moe.moe_forward(x, inp["w_router"], inp["wg"], inp["wu"], inp["wd"], inp["wg_s"], inp["wu_s"],
                                       inp["wd_s"], cfg.k, renormalize=True, return_routing=True, ws=ws, dims=dims)
        torch.cuda.synchronize()
        touched = wl.touched_experts(idx.cpu().numpy(), cfg.E)
        nbytes = wl.algorithmic_bytes(T, cfg.d, cfg.E, cfg.I, cfg.Is, cfg.dtype, touched)
        print(json.dumps({"T": T, "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3), "touched_experts": touched,
                          "algorithmic_bytes": nbytes, "hbm_frac": nbytes / (ms * 1e-3) / wl.HBM_PEAK_BPS,
                          "config": {"workload": "sweep", "d": cfg.d, "E": cfg.E, "k": cfg.k, "I": cfg.I,
                                     "I_shared": cfg.Is, "dtype": "bf16"}}), flush=True)


def median(v):
    v = sorted(v)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


class Run:
    """One forward variant over fixed inputs: bf16/fp32 experts, FP8 experts, or the block with
    its norm and residual."""

    def __init__(self, moe, cfg, x, inp, ws, out, dims, fp8=None, gamma=None):
        self.moe, self.cfg, self.x, self.inp, self.ws, self.out, self.dims = moe, cfg, x, inp, ws, out, dims
        self.fp8, self.gamma = fp8, gamma

    def __call__(self, return_routing=False):
        moe, cfg, inp = self.moe, self.cfg, self.inp
        kw = dict(renormalize=bool(cfg.renorm), router_bias=inp["bias"], ws=self.ws, dims=self.dims,
                  return_routing=return_routing)
        if not return_routing:
            kw["out"] = self.out
        if self.fp8 is not None:
            return moe.moe_forward_fp8(self.x, inp["w_router"], self.fp8, cfg.k, **kw)
        if self.gamma is not None:
            return moe.moe_forward_block(self.x, self.gamma, inp["w_router"], inp["wg"], inp["wu"], inp["wd"],
                                         inp["wg_s"], inp["wu_s"], inp["wd_s"], cfg.k, **kw)
        return moe.moe_forward(self.x, inp["w_router"], inp["wg"], inp["wu"], inp["wd"], inp["wg_s"], inp["wu_s"],
                               inp["wd_s"], cfg.k, **kw)


def measure(run, lib, hip, stream, steps, warmup):
    """Times `steps` forward calls after `warmup` untimed ones: per-step HIP events on the
    library's stream (the steps run back to back; event k ends step k and starts step k+1), and
    the dominant kernel's own pair of timing-only events inside every step. Returns (step times,
    kernel times, wall seconds of the timed region, routing of the input)."""
    import torch
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    marks = [hip.create(timing_only=True) for _ in range(steps + 1)]
    pairs = [(hip.create(timing_only=True), hip.create(timing_only=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    hip.record(marks[0], stream)
    for i, (a, b) in enumerate(pairs):
        rc = lib.moe_profile_next_forward(KERNEL_FFN_GATE_UP, a, b)
        if rc != 0:
            raise RuntimeError(lib.moe_last_error().decode())
        run()
        hip.record(marks[i + 1], stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = [hip.ms(marks[i], marks[i + 1]) for i in range(steps)]
    kern_ms = [hip.ms(a, b) for a, b in pairs]
    for ev in marks:
        hip.destroy(ev)
    for a, b in pairs:
        hip.destroy(a)
        hip.destroy(b)
    _, idx, _, _ = run(return_routing=True)
    torch.cuda.synchronize()
    return step_ms, kern_ms, wall, idx.cpu().numpy()


def kernel_label(cfg, fp8):
    """The gate/up kernel the library launches for this workload, as a trace names it."""
    import sparse_mixture_experts_softmax_amd as moe
    dims = moe.MoeDims(T=cfg.T, d=cfg.d, E=cfg.E, k=cfg.k, I=cfg.I, I_shared=cfg.Is, dtype=cfg.dtype,
                       renormalize=cfg.renorm)
    name = moe.moe_kernel_name(dims, moe.KERNEL_FFN_GATE_UP, fp8)
    return name + (" (gate/up, e4m3 weights)" if fp8 else " (gate/up)")


def roofline(wl, syn, cfg, kb, kf, kern_med_ms, fp8):
    """The dominant kernel against its bound: HBM when its algorithmic bytes take longer at 8 TB/s
    than its FLOPs at the matrix cores' peak, the matrix cores otherwise."""
    peak_flops = wl.BF16_MFMA_PEAK_FLOPS if cfg.dtype == syn.BF16 else wl.FP32_VECTOR_PEAK_FLOPS
    t_s = kern_med_ms * 1e-3
    if kb / wl.HBM_PEAK_BPS >= kf / peak_flops:
        roof = {"bound": "hbm", "achieved": kb / t_s / 1e9, "peak": wl.HBM_PEAK_BPS / 1e9, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma" if cfg.dtype == syn.BF16 else "alu", "achieved": kf / t_s / 1e12,
                "peak": peak_flops / 1e12, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["kernel"] = kernel_label(cfg, fp8)
    roof["kernel_ms"] = kern_med_ms
    roof["algorithmic_bytes"] = kb
    roof["algorithmic_flops"] = kf
    return roof


def summarize(wl, syn, cfg, step_ms, kern_ms, idx, fp8):
    """Tokens/s, the layer's fractions of both peaks, and the dominant kernel's roofline."""
    touched = wl.touched_experts(idx, cfg.E)
    ms = median(step_ms)
    if fp8:
        kb = wl.ffn1_algorithmic_bytes_fp8(cfg.T, cfg.d, cfg.I, cfg.Is, touched)
        lb = wl.algorithmic_bytes_fp8(cfg.T, cfg.d, cfg.E, cfg.I, cfg.Is, touched)
    else:
        kb = wl.ffn1_algorithmic_bytes(cfg.T, cfg.d, cfg.I, cfg.Is, cfg.dtype, touched)
        lb = wl.algorithmic_bytes(cfg.T, cfg.d, cfg.E, cfg.I, cfg.Is, cfg.dtype, touched)
    kf = wl.ffn1_flops(cfg.T, cfg.d, cfg.k, cfg.I, cfg.Is)
    lf = wl.expert_flops(cfg.T, cfg.d, cfg.k, cfg.I, cfg.Is)
    peak_flops = wl.BF16_MFMA_PEAK_FLOPS if cfg.dtype == syn.BF16 else wl.FP32_VECTOR_PEAK_FLOPS
    roof = roofline(wl, syn, cfg, kb, kf, median(kern_ms), fp8)
    layer = {"touched_experts": touched, "algorithmic_bytes": lb, "expert_flops": lf,
             "router_flops": wl.router_flops(cfg.T, cfg.d, cfg.E),
             "hbm_frac": lb / (ms * 1e-3) / wl.HBM_PEAK_BPS, "mfma_frac": lf / (ms * 1e-3) / peak_flops,
             "ms_per_step_mean": sum(step_ms) / len(step_ms), "ms_per_step_min": min(step_ms),
             "ms_per_step_max": max(step_ms)}
    return ms, cfg.T / (ms * 1e-3), roof, layer


def workload_name(cfg, block=False, fp8=False):
    return "%s MoE layer: T=%d, d=%d, E=%d, k=%d, I=%d, shared I=%d, %s, fp32 router%s%s" % (
        cfg.name, cfg.T, cfg.d, cfg.E, cfg.k, cfg.I, cfg.Is, cfg.dtype_name,
        ", Zipf(%.1f) router bias" % cfg.zipf_alpha if cfg.zipf_alpha else "",
        ", RMSNorm in front and residual add" if block else ", FP8 e4m3 expert weights" if fp8 else "")


def _csv_rows(directory, suffix):
    """Rows of every rocprofv3 CSV under `directory` whose file name ends in `suffix`."""
    import csv
    rows = []
    for base, _, files in os.walk(directory):
        for f in sorted(files):
            if f.endswith(suffix):
                with open(os.path.join(base, f), newline="") as fh:
                    rows.extend(csv.DictReader(fh))
    if not rows:
        raise SystemExit("no *%s under %s" % (suffix, directory))
    return rows


def _short_kernel_name(name):
    """A kernel's demangled name without return type, argument list and clone suffix."""
    name = name.replace(" [clone .kd]", "").replace("(anonymous namespace)::", "").replace("moe::", "").strip()
    if name.startswith("void "):
        name = name[5:]
    depth, cut = 0, len(name)
    for i, ch in enumerate(name):  # the argument list is the first '(' outside template brackets
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            cut = i
            break
    return name[:cut]


def _per_dispatch(rows, counter):
    """{dispatch id: (kernel, grid size, value)} of one counter in a counter-collection CSV."""
    out = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        key = r["Dispatch_Id"]
        prev = out.get(key, (None, 0, 0.0))[2]
        out[key] = (_short_kernel_name(r["Kernel_Name"]), int(r["Grid_Size"]), prev + float(r["Counter_Value"]))
    return out


def summarize_traffic(workload, fetch_dir, write_dir, commands):
    """HBM bytes per launch of the gate/up GEMM from two rocprofv3 --pmc runs of bench.py
    --copy-calibration (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled by what the
    same counter reads for the 1 GiB device copy in the same process. Prints the JSON record that
    bench.py reads back as `roofline.traffic`."""
    import synthetic as syn

    cfg = syn.CONFIGS[workload]
    kname = kernel_label(cfg, False).split(" (")[0]
    res = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        disp = _per_dispatch(_csv_rows(d, "counter_collection.csv"), counter)
        kv = [v for (n, _, v) in disp.values() if n == kname]
        copies = [(g, v) for (n, g, v) in disp.values() if "copyBuffer" in n]
        if not kv or not copies:
            raise SystemExit("%s: no dispatch of %s or of the copy kernel" % (counter, kname))
        gmax = max(g for g, _ in copies)
        cv = [v for g, v in copies if g == gmax]
        res[counter] = (sum(kv) / len(kv), len(kv), sum(cv) / len(cv), len(cv))
    nbytes = 1 << 30
    fscale = nbytes / 1024.0 / res["FETCH_SIZE"][2]
    wscale = nbytes / 1024.0 / res["WRITE_SIZE"][2]
    fetch_b = res["FETCH_SIZE"][0] * 1024.0 * fscale
    write_b = res["WRITE_SIZE"][0] * 1024.0 * wscale
    # the algorithmic bytes depend on the routing (experts touched): taken from the bench line
    # that the profiled run printed, saved as bench.json beside the FETCH_SIZE results
    algo = None
    line = os.path.join(fetch_dir, "bench.json")
    if os.path.exists(line):
        algo = json.load(open(line))["roofline"]["algorithmic_bytes"]
    rec = {"workload": workload_name(cfg), "commands": commands, "kernel": kname + " (grouped gate/up GEMM)",
           "dispatches": res["FETCH_SIZE"][1], "copy_dispatches": res["FETCH_SIZE"][3],
           "fetch_kib_per_dispatch": res["FETCH_SIZE"][0], "write_kib_per_dispatch": res["WRITE_SIZE"][0],
           "copy_calibration": {"bytes_copied": nbytes, "fetch_kib": res["FETCH_SIZE"][2],
                                "write_kib": res["WRITE_SIZE"][2], "fetch_scale": fscale, "write_scale": wscale},
           "bytes_per_launch": fetch_b + write_b, "fetch_bytes_per_launch": fetch_b,
           "write_bytes_per_launch": write_b,
           "algorithmic_bytes_per_launch": algo,
           "kernel_source_sha256": kernel_source_hash()}
    print(json.dumps(rec, indent=1))


def summarize_trace(title, trace_dir, command):
    """Per-kernel table of a rocprofv3 --kernel-trace --stats run (its kernel_stats CSV)."""
    rows = _csv_rows(trace_dir, "kernel_stats.csv")
    agg = {}
    for r in rows:
        n = _short_kernel_name(r["Name"])
        c, t = agg.get(n, (0, 0.0))
        agg[n] = (c + int(r["Calls"]), t + float(r["TotalDurationNs"]))
    total = sum(t for _, t in agg.values())
    print("# rocprofv3 kernel trace, %s" % title)
    print("# command (repo root): %s" % command)
    print("%-52s %8s %12s %12s %8s" % ("kernel", "calls", "avg_us", "total_ms", "pct"))
    for n, (c, t) in sorted(agg.items(), key=lambda kv: -kv[1][1]):
        print("%-52s %8d %12.1f %12.3f %8.3g" % (n[:52], c, t / c / 1e3, t / 1e6, 100.0 * t / total))


DECODE_STEPS = 50  # the decode leg's timed steps (its median is over 50 runs)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill", choices=["tiny", "mid", "decode", "prefill", "skew"])
    ap.add_argument("--tokens", type=int, default=None, help="override the workload's token count T")
    ap.add_argument("--fp8", action="store_true",
                    help="expert weights in FP8 (e4m3, power-of-two column scales), quantised before timing")
    ap.add_argument("--block", action="store_true",
                    help="time the block between its neighbours: zero-centred RMSNorm in front, residual add after")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode leg of the prefill workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB device copy, the reference kernel for HBM byte counters")
    ap.add_argument("--calibrate", action="store_true",
                    help="only measure reference points (vendor bf16 GEMM, device copy) and exit")
    ap.add_argument("--sweep", action="store_true",
                    help="only run the token-count sweep T = 1 .. 512 at the large layer shape, one line per T")
    ap.add_argument("--summarize-traffic", nargs=3, metavar=("WORKLOAD", "FETCH_DIR", "WRITE_DIR"),
                    help="print the gate/up HBM-traffic record from two rocprofv3 --pmc runs (no GPU use)")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TITLE", "TRACE_DIR"),
                    help="print the per-kernel table of a rocprofv3 --kernel-trace --stats run (no GPU use)")
    ap.add_argument("--command", action="append", default=[],
                    help="with --summarize-*: the profiler command(s) that made the run, for the record")
    args = ap.parse_args()

    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic, commands=args.command)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace, command="; ".join(args.command))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus %d, WORLD_SIZE %d)"
              % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    if args.calibrate:
        calibrate()
        return
    if args.sweep:
        sweep(args.steps, args.warmup)
        return
    if args.fp8 and args.block:
        print("bench.py: --fp8 and --block are separate entry points; pick one", file=sys.stderr)
        sys.exit(2)

    import torch

    import sparse_mixture_experts_softmax_amd as moe
    import synthetic as syn
    from sparse_mixture_experts_softmax_amd import workload as wl

    cfg = syn.CONFIGS[args.workload]
    if args.tokens is not None:
        cfg = cfg.with_(T=args.tokens)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = moe.load_library()
    print("bench: %s, generating inputs on the device" % (cfg,), file=sys.stderr, flush=True)
    inp = syn.device_inputs(cfg, device=dev)
    x = inp["x"]
    dims = moe.dims_for(x, inp["w_router"], inp["wg"], inp["wg_s"], cfg.k, bool(cfg.renorm))
    ws = moe.workspace(dims, dev)
    out = torch.empty_like(x)
    gamma = syn.device_gamma(cfg, device=dev) if args.block else None
    fp8 = None
    if args.fp8:
        fp8 = moe.Fp8Experts(inp["wg"], inp["wu"], inp["wd"], inp["wg_s"], inp["wu_s"], inp["wd_s"])
        for key in ("wg", "wu", "wd", "wg_s", "wu_s", "wd_s"):  # the bf16 copies are not needed any more
            inp[key] = None
        torch.cuda.empty_cache()

    stream = torch.cuda.current_stream(dev).cuda_stream
    hip = HipEvents()
    run = Run(moe, cfg, x, inp, ws, out, dims, fp8=fp8, gamma=gamma)
    print("bench: timing %d steps after %d warm-up steps" % (args.steps, args.warmup), file=sys.stderr, flush=True)
    step_ms, kern_ms, wall, idx = measure(run, lib, hip, stream, args.steps, args.warmup)
    ms, tps, roof, layer = summarize(wl, syn, cfg, step_ms, kern_ms, idx, fp8 is not None)
    plain = fp8 is None and not args.block and args.tokens is None
    roof["traffic"] = traffic_for(cfg.name) if plain else None

    # the decode leg: the first 32 rows of the same input on the same weights (the decode
    # workload's x is exactly those rows), its own median over DECODE_STEPS steps
    decode = None
    if args.workload == "prefill" and args.tokens is None and not args.no_decode:
        dcfg = syn.CONFIGS["decode"]
        if fp8 is not None:
            dcfg = dcfg.with_(name="decode")
        xd = x[:dcfg.T]
        ddims = moe.MoeDims(dcfg.T, dims.d, dims.E, dims.k, dims.I, dims.I_shared, dims.dtype, dims.renormalize)
        dws = moe.workspace(ddims, dev)
        drun = Run(moe, dcfg, xd, inp, dws, torch.empty_like(xd), ddims, fp8=fp8,
                   gamma=gamma)
        print("bench: decode leg, %d steps" % DECODE_STEPS, file=sys.stderr, flush=True)
        dstep, dkern, dwall, didx = measure(drun, lib, hip, stream, DECODE_STEPS, args.warmup)
        dms, dtps, droof, dlayer = summarize(wl, syn, dcfg, dstep, dkern, didx, fp8 is not None)
        droof["traffic"] = traffic_for("decode") if (fp8 is None and not args.block) else None
        decode = {"workload": workload_name(dcfg, args.block, fp8 is not None), "T": dcfg.T, "steps": DECODE_STEPS,
                  "ms_per_step": dms, "tokens_per_s": dtps, "layer_hbm_frac": dlayer["hbm_frac"],
                  "roofline": droof, "layer": dlayer}

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle on a token sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(cfg, CPU_SAMPLE[cfg.name])

    res = {
        "metric": METRIC, "value": tps, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if cfg.dtype == syn.BF16 else "f32", "data": "synthetic",
        "config": {"workload": workload_name(cfg, args.block, fp8 is not None),
                   "T": cfg.T, "d": cfg.d, "E": cfg.E, "k": cfg.k, "I": cfg.I, "I_shared": cfg.Is,
                   "renormalize": cfg.renorm, "seed": cfg.seed},
        "roofline": roof, "layer": layer, "decode": decode, "cpu_baseline": cpu, "wall_s_timed": wall,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

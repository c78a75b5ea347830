#!/usr/bin/env python3
"""MoE-layer benchmark on one MI355X.

One step = one moe_forward call: router GEMM + softmax top-k, dispatch, routed and shared SwiGLU
experts, weighted combine -- the whole forward pass of the block over one batch of synthetic input
that is already resident in HBM. Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload mid|decode|prefill|skew|tiny]

The default workload is the mid-size bf16 layer (T=4096, d=2048, E=256, k=8, I=512, one shared
expert with I=512). The dominant kernel (grouped gate/up GEMM) is timed with HIP events recorded
around its launch inside every timed step; its algorithmic bytes / FLOPs give the roofline fraction.
The CPU oracle is timed on a bounded token sample of the same workload as a reported baseline.
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


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mid", choices=["tiny", "mid", "decode", "prefill", "skew"])
    ap.add_argument("--tokens", type=int, default=None, help="override the workload's token count T")
    ap.add_argument("--fp8", action="store_true",
                    help="expert weights in FP8 (e4m3, power-of-two column scales), quantised before timing")
    ap.add_argument("--block", action="store_true",
                    help="time the block between its neighbours: zero-centred RMSNorm in front, residual add after")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB device copy, the reference kernel for HBM byte counters")
    ap.add_argument("--calibrate", action="store_true",
                    help="only measure reference points (vendor bf16 GEMM, device copy) and exit")
    ap.add_argument("--sweep", action="store_true",
                    help="only run the token-count sweep T = 1 .. 512 at the large layer shape, one line per T")
    args = ap.parse_args()

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
    if args.fp8 and args.block:
        print("bench.py: --fp8 and --block are separate entry points; pick one", file=sys.stderr)
        sys.exit(2)
    fp8 = None
    if args.fp8:
        fp8 = moe.Fp8Experts(inp["wg"], inp["wu"], inp["wd"], inp["wg_s"], inp["wu_s"], inp["wd_s"])
        for key in ("wg", "wu", "wd", "wg_s", "wu_s", "wd_s"):  # the bf16 copies are not needed any more
            inp[key] = None
        torch.cuda.empty_cache()

    def step():
        if fp8 is not None:
            moe.moe_forward_fp8(x, inp["w_router"], fp8, cfg.k, renormalize=bool(cfg.renorm), router_bias=inp["bias"],
                                ws=ws, out=out, dims=dims)
        elif args.block:
            moe.moe_forward_block(x, gamma, inp["w_router"], inp["wg"], inp["wu"], inp["wd"], inp["wg_s"],
                                  inp["wu_s"], inp["wd_s"], cfg.k, renormalize=bool(cfg.renorm),
                                  router_bias=inp["bias"], ws=ws, out=out, dims=dims)
        else:
            moe.moe_forward(x, inp["w_router"], inp["wg"], inp["wu"], inp["wd"], inp["wg_s"], inp["wu_s"],
                            inp["wd_s"], cfg.k, renormalize=bool(cfg.renorm), router_bias=inp["bias"], ws=ws, out=out,
                            dims=dims)

    stream = torch.cuda.current_stream(dev).cuda_stream
    hip = HipEvents()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    pairs = [(hip.create(timing_only=True), hip.create(timing_only=True)) for _ in range(K)]
    t_beg, t_end = hip.create(), hip.create()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    hip.record(t_beg, stream)
    for a, b in pairs:
        rc = lib.moe_profile_next_forward(KERNEL_FFN_GATE_UP, a, b)
        if rc != 0:
            raise RuntimeError(lib.moe_last_error().decode())
        step()
    hip.record(t_end, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = hip.ms(t_beg, t_end)
    kern_ms = [hip.ms(a, b) for a, b in pairs]
    kern_avg_ms = sum(kern_ms) / len(kern_ms)
    for a, b in pairs:
        hip.destroy(a)
        hip.destroy(b)

    # routing of this input, for the algorithmic work actually required
    if fp8 is not None:
        _, idx, _, _ = moe.moe_forward_fp8(x, inp["w_router"], fp8, cfg.k, renormalize=bool(cfg.renorm),
                                           router_bias=inp["bias"], return_routing=True, ws=ws, dims=dims)
    elif args.block:
        _, idx, _, _ = moe.moe_forward_block(x, gamma, inp["w_router"], inp["wg"], inp["wu"], inp["wd"], inp["wg_s"],
                                             inp["wu_s"], inp["wd_s"], cfg.k, renormalize=bool(cfg.renorm),
                                             router_bias=inp["bias"], return_routing=True, ws=ws, dims=dims)
    else:
        _, idx, _, _ = moe.moe_forward(x, inp["w_router"], inp["wg"], inp["wu"], inp["wd"], inp["wg_s"],
                                       inp["wu_s"], inp["wd_s"], cfg.k, renormalize=bool(cfg.renorm),
                                       router_bias=inp["bias"], return_routing=True, ws=ws, dims=dims)
    torch.cuda.synchronize()
    touched = wl.touched_experts(idx.cpu().numpy(), cfg.E)

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    ms_per_step = total_ms / K
    tokens_per_s = cfg.T / (ms_per_step * 1e-3)
    if fp8 is not None:
        kb = wl.ffn1_algorithmic_bytes_fp8(cfg.T, cfg.d, cfg.I, cfg.Is, touched, cfg.k)
    else:
        kb = wl.ffn1_algorithmic_bytes(cfg.T, cfg.d, cfg.I, cfg.Is, cfg.dtype, touched, cfg.k)
    kf = wl.ffn1_flops(cfg.T, cfg.d, cfg.k, cfg.I, cfg.Is)
    peak_flops = wl.BF16_MFMA_PEAK_FLOPS if cfg.dtype == syn.BF16 else wl.FP32_VECTOR_PEAK_FLOPS
    t_s = kern_avg_ms * 1e-3
    if kb / wl.HBM_PEAK_BPS >= kf / peak_flops:
        roof = {"bound": "hbm", "achieved": kb / t_s / 1e9, "peak": wl.HBM_PEAK_BPS / 1e9, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma" if cfg.dtype == syn.BF16 else "alu", "achieved": kf / t_s / 1e12,
                "peak": peak_flops / 1e12, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = None if (fp8 is not None or args.block or args.tokens is not None) else traffic_for(cfg.name)
    roof["kernel"] = ("ffn_fp8_stream_kernel<true, 4> (gate/up, e4m3 weights)" if fp8 is not None else
                      "ffn_mfma_stream_kernel<true, ...> (gate/up)" if cfg.dtype == syn.BF16 else "ffn_f32_kernel<true>")
    roof["kernel_ms"] = kern_avg_ms
    roof["algorithmic_bytes"] = kb
    roof["algorithmic_flops"] = kf

    if fp8 is not None:
        lb = wl.algorithmic_bytes_fp8(cfg.T, cfg.d, cfg.E, cfg.I, cfg.Is, touched)
    else:
        lb = wl.algorithmic_bytes(cfg.T, cfg.d, cfg.E, cfg.I, cfg.Is, cfg.dtype, touched)
    lf = wl.expert_flops(cfg.T, cfg.d, cfg.k, cfg.I, cfg.Is)
    layer = {"touched_experts": touched, "algorithmic_bytes": lb, "expert_flops": lf,
             "router_flops": wl.router_flops(cfg.T, cfg.d, cfg.E),
             "hbm_frac": lb / (ms_per_step * 1e-3) / wl.HBM_PEAK_BPS,
             "mfma_frac": lf / (ms_per_step * 1e-3) / peak_flops}

    cpu = None
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle on a token sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(cfg, CPU_SAMPLE[cfg.name])

    res = {
        "metric": METRIC, "value": tokens_per_s, "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if cfg.dtype == syn.BF16 else "f32", "data": "synthetic",
        "config": {"workload": "%s MoE layer: T=%d, d=%d, E=%d, k=%d, I=%d, shared I=%d, %s, fp32 router%s%s"
                   % (cfg.name, cfg.T, cfg.d, cfg.E, cfg.k, cfg.I, cfg.Is, cfg.dtype_name,
                      ", Zipf(%.1f) router bias" % cfg.zipf_alpha if cfg.zipf_alpha else "",
                      ", RMSNorm in front and residual add" if args.block else
                      ", FP8 e4m3 expert weights" if fp8 is not None else ""),
                   "T": cfg.T, "d": cfg.d, "E": cfg.E, "k": cfg.k, "I": cfg.I, "I_shared": cfg.Is,
                   "renormalize": cfg.renorm, "seed": cfg.seed},
        "roofline": roof, "layer": layer, "cpu_baseline": cpu, "wall_s_timed": wall,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

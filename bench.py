"""Benchmark of the 2D relative-position attention forward on one MI355X.

A step is one forward pass of the headline workload (DeiT-S with iRPE
contextual Product keys: batch 64, 14 x 14 grid + class token, 6 heads,
d = 64, bf16, an 81 x 64 key table shared by the heads) over one batch of
synthetic input already in HBM.  The timed steps cycle through enough input
copies that the working set is larger than the 256 MB Infinity Cache, so
every step reads its inputs from HBM; the same launch on one resident buffer
set (inputs held by the Infinity Cache) is also reported, as "warm".  The
other bf16 workloads (Swin-T stage-1 windows, DeiT-S with query/key/value
terms, the 56 x 56 high-resolution grid and the mode / mapping variants) are
timed the same way and reported under "secondary".

Per-launch kernel time comes from HIP events on the stream the kernel is
launched on, recorded at the ends of up to 10 consecutive batches of the timed
launches: the mean over all of them is the headline, and the median, p10 and
p90 of the batch means are reported beside it.  Algorithmic counts: FLOP = 4 T^2 d per unit (QK^T and PV) +
2 n K d per contextual term (n positioned tokens, K table rows); bytes = q,
k, v read once + o written once.

The CPU baseline is the fp64 oracle, run in a process pool over (batch,
head) images of the same workload before the GPU is touched.

HBM traffic per launch comes from rocprofv3 FETCH_SIZE / WRITE_SIZE passes
over this script with ``--calib-probe`` (a read-only sum and a write-only fill
of known size calibrate the two counters separately); the figure is read from
profiles/ and reported only while the forward kernel's sources still hash to
the value it was measured with.
"""

import argparse
import json
import math
import multiprocessing as mp
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from vision_transformer_attention_amd.workloads import WORKLOADS, make_inputs  # noqa: E402

METRIC = "2D-RPE attention fwd TFLOP/s and % bf16 MFMA peak (DeiT-S iRPE-K, Swin-T W7)"
HEADLINE = "deit_s_irpe_k"
SECONDARY = ("swin_t_w7", "deit_s_irpe_qkv", "highres_irpe_k", "deit_s_irpe_bias", "deit_s_irpe_k_cross",
             "detr_irpe_k", "deit_s_irpe_bias_euclid", "detr_wide_irpe_k", "swin_t_w7_irpe_qkv")
PEAK_MFMA_BF16 = 2500.0      # TFLOP/s, dense, MI355X
PEAK_HBM = 8000.0            # GB/s, MI355X HBM3E
MALL_BYTES = 256 << 20
PROFILES = os.path.join(ROOT, "profiles")
COLD_SET_BYTES = 512 << 20   # cycle through at least this much input per step sequence
CPU_SHARE = 16               # host threads per GPU on the measurement host


def flops_bytes(w):
    """Algorithmic FLOP and HBM bytes of one forward of workload w."""
    r, c = (w.window, w.window) if w.window else (w.grid_h, w.grid_w)
    n = r * c
    t = w.prefix + n
    units = w.batch * w.heads * ((w.grid_h // w.window) * (w.grid_w // w.window) if w.window else 1)
    terms = len(w.terms) if w.mode == "contextual" else 0
    flop = units * (4.0 * t * t * w.head_dim + terms * 2.0 * n * w.table_rows * w.head_dim)
    elem = 2 if w.dtype == "bf16" else 4
    nbytes = 4.0 * w.batch * w.heads * w.tokens * w.head_dim * elem
    return flop, nbytes


# ------------------------------------------------------------------------------ CPU baseline

_CPU = {}


def _oracle_worker(args):
    name, pairs = args
    from oracle import Spec, attention
    import numpy as np
    w = WORKLOADS[name]
    x = _CPU["x"]
    spec = Spec(w.grid_h, w.grid_w, window=w.window, prefix=w.prefix, mode=w.mode, terms=w.terms, map=w.map,
                alpha=w.alpha, beta=w.beta, gamma=w.gamma, reading=w.reading,
                tables_per_head=w.tables_per_head, method=w.method)
    for b, h in pairs:
        attention(spec, x["q"], x["k"], x["v"], bias=x.get("bias"), rq=x.get("rq"), rk=x.get("rk"),
                  rv=x.get("rv"), batch_sel=[b], heads_sel=[h])
    return len(pairs)


def cpu_baseline(name, budget_s=20.0):
    """Time the oracle over a bounded sample of (batch, head) images of `name`."""
    os.environ.setdefault("OMP_NUM_THREADS", "1")
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=1)
    except Exception:
        limiter = None
    w = WORKLOADS[name]
    x = make_inputs(w)
    _CPU["x"] = x
    # estimate the per-image cost (after one warm-up image)
    _oracle_worker((name, [(0, 0)]))
    t0 = time.perf_counter()
    _oracle_worker((name, [(0, 1 % w.heads)]))
    per_img = max(time.perf_counter() - t0, 1e-3)
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    # the host shares its CPUs among its GPUs: one GPU's share is 16 threads, whatever
    # the affinity mask shows, so the pool never takes more than that
    cores = max(1, min(cores, CPU_SHARE))
    n_img = w.batch * w.heads
    # about budget_s seconds of single-core oracle work, cycling over the workload's images
    n_sample = max(cores, int(budget_s / per_img))
    pairs = [((i % n_img) // w.heads, (i % n_img) % w.heads) for i in range(n_sample)]
    chunks = [pairs[i::cores] for i in range(cores)]
    ctx = mp.get_context("fork")
    with ctx.Pool(cores) as pool:
        t0 = time.perf_counter()
        done = sum(pool.map(_oracle_worker, [(name, c) for c in chunks if c]))
        wall = time.perf_counter() - t0
    if limiter is not None:
        limiter.unregister() if hasattr(limiter, "unregister") else None
    flop, _ = flops_bytes(w)
    flop_sample = flop * done / n_img
    _CPU.clear()
    return {"value": flop_sample / wall / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} (batch, head) images of {name} (the workload has {n_img}; images repeat "
                      f"when the sample is larger), fp64 NumPy oracle, {wall:.2f} s wall on {cores} "
                      f"processes (1 BLAS thread each; at most {CPU_SHARE}, one GPU's share of the host)",
            "cpu_model": cpu_model(), "seconds": wall}


def cpu_model():
    """The host CPU's model string (from /proc/cpuinfo), or the platform's name."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


def measured_traffic(name):
    """(bytes per launch, note) from profiles/traffic_<name>.txt if the kernel is unchanged."""
    from vision_transformer_attention_amd.profile_summary import kernel_source_hash
    path = os.path.join(PROFILES, f"traffic_{name}.txt")
    if not os.path.exists(path):
        return None, "no counter summary for this workload"
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith(" "):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    try:
        fetch = float(kv["fetch_bytes_per_launch"])
        write = float(kv["write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None, "counter summary incomplete"
    if kv.get("kernel_source_hash") != kernel_source_hash():
        return None, "kernel changed since the counters were taken"
    return {"fetch": fetch, "write": write, "total": fetch + write}, path


# ------------------------------------------------------------------------------ GPU timing

def _device_inputs(w, copies, dev):
    import torch
    x = make_inputs(w)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    base = {n: torch.from_numpy(a).to(torch.float32 if n == "bias" else tdt).to(dev).contiguous()
            for n, a in x.items()}
    sets = [base]
    for _ in range(copies - 1):
        sets.append({n: (t.clone() if n in ("q", "k", "v") else t) for n, t in base.items()})
    outs = [torch.empty_like(base["q"]) for _ in range(copies)]
    return sets, outs


def _prepared(w, d, o):
    import vision_transformer_attention_amd as pkg
    return pkg.prepare_fwd(d["q"], d["k"], d["v"], out=o, grid=(w.grid_h, w.grid_w), window=w.window,
                           prefix_tokens=w.prefix, mode=w.mode, terms="".join(sorted(w.terms)), map=w.map,
                           alpha=w.alpha, beta=w.beta, gamma=w.gamma, rounding=w.reading,
                           bias=d.get("bias"), rq=d.get("rq"), rk=d.get("rk"), rv=d.get("rv"),
                           method=w.method)


def _batched_events(launch, steps, stream, batches=10):
    """Launch `steps` times in up to `batches` consecutive batches with a HIP event
    on `stream` at each batch boundary.  Returns (mean ms per launch over all
    steps, [ms per launch of each batch])."""
    import torch
    nb = max(1, min(batches, steps))
    bounds = [round(steps * j / nb) for j in range(nb + 1)]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(nb + 1)]
    evs[0].record(stream)
    for j in range(nb):
        for i in range(bounds[j], bounds[j + 1]):
            launch(i)
        evs[j + 1].record(stream)
    torch.cuda.synchronize()
    per = [evs[j].elapsed_time(evs[j + 1]) / (bounds[j + 1] - bounds[j]) for j in range(nb)]
    return evs[0].elapsed_time(evs[nb]) / steps, per


def _quantiles(per):
    """Median, p10 and p90 (linear interpolation) of per-batch launch times, in us."""
    import numpy as np
    a = np.asarray(per, dtype=np.float64) * 1e3
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)), "p90": float(np.percentile(a, 90)),
            "batches": len(per)}


def time_workload(name, steps, warmup, dev, cold=True):
    """Per-launch time (ms) over `steps` launches, HIP events on the launch stream.

    Cold: the launches cycle through enough HBM-resident input copies that the
    256 MB Infinity Cache cannot hold them, and the timed launches continue the
    rotation where the warm-up stopped, so no timed launch reuses a copy the
    warm-up has just read (with fewer steps than copies none repeats at all).
    Warm: one resident buffer set.  Returns (mean ms, batch quantiles, wall s,
    copies, outputs finite)."""
    import torch
    w = WORKLOADS[name]
    _, nbytes = flops_bytes(w)
    copies = max(1, math.ceil(COLD_SET_BYTES / nbytes)) if cold else 1
    sets, outs = _device_inputs(w, copies, dev)
    calls = [_prepared(w, sets[i], outs[i]) for i in range(copies)]
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    for i in range(warmup):
        calls[i % copies](sp)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms, per = _batched_events(lambda i: calls[(warmup + i) % copies](sp), steps, stream)
    wall = time.perf_counter() - t0
    ok = bool(torch.isfinite(outs[0]).all().item())
    del sets, outs, calls
    torch.cuda.empty_cache()
    return ms, _quantiles(per), wall, copies, ok


def time_backward(name, steps, warmup, dev):
    """Average time (ms) of one rpe_attn_bwd call on `name` (one resident buffer set),
    HIP events on the launch stream; the log-sum-exp comes from the forward."""
    import numpy as np
    import torch
    import vision_transformer_attention_amd as pkg
    w = WORKLOADS[name]
    sets, outs = _device_inputs(w, 1, dev)
    d = sets[0]
    dout = torch.from_numpy(np.random.default_rng(77).standard_normal(w.qkv_shape)).to(d["q"].dtype).to(dev)
    kw = dict(grid=(w.grid_h, w.grid_w), window=w.window, prefix_tokens=w.prefix, mode=w.mode,
              terms="".join(sorted(w.terms)), map=w.map, alpha=w.alpha, beta=w.beta, gamma=w.gamma,
              rounding=w.reading, bias=d.get("bias"), rq=d.get("rq"), rk=d.get("rk"), rv=d.get("rv"),
              method=w.method)
    _, lse = pkg.rpe_attn_fwd(d["q"], d["k"], d["v"], return_lse=True, **kw)
    g, call = pkg.prepare_bwd(d["q"], d["k"], d["v"], dout, lse, **kw)
    stream = torch.cuda.current_stream(dev)
    for _ in range(warmup):
        call(stream.cuda_stream)
    torch.cuda.synchronize()
    ms, _ = _batched_events(lambda i: call(stream.cuda_stream), steps, stream, batches=1)
    ok = all(bool(torch.isfinite(t).all().item()) for t in g.values())
    del sets, outs, g, call
    torch.cuda.empty_cache()
    return ms, ok


def measure_roofs(dev):
    """Ceilings measured on this GPU by librpe_roofs.so (include/rpe_roofs.h), each
    timed with HIP events on the launch stream after an untimed launch: HBM copy
    and read of 1 GiB buffers, 20 passes per launch over 38 MB and 77 MB buffers
    that the Infinity Cache holds, bf16 MFMA, scalar fp32 FMA and exp2 rates."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "vision_transformer_attention_amd", "librpe_roofs.so"))
    vp, i32, i64, dp = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.POINTER(ctypes.c_double)
    lib.rpe_roof_copy.argtypes = [vp, vp, i64, vp, dp]
    lib.rpe_roof_read.argtypes = [vp, i64, i32, vp, vp, dp]
    for f in (lib.rpe_roof_mfma_bf16, lib.rpe_roof_fma_f32, lib.rpe_roof_exp2_f32):
        f.argtypes = [i32, vp, vp, dp]
    for f in (lib.rpe_roof_copy, lib.rpe_roof_read, lib.rpe_roof_mfma_bf16, lib.rpe_roof_fma_f32,
              lib.rpe_roof_exp2_f32):
        f.restype = i32
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    sink = torch.zeros(64, dtype=torch.float32, device=dev)
    work = ctypes.c_double(0.0)

    def rate(call, launches):
        def go(_):
            st = call()
            if st != 0:
                raise RuntimeError(f"roof probe failed with status {st}")
        go(0)
        torch.cuda.synchronize()
        ms, _ = _batched_events(go, launches, stream, batches=1)
        return work.value / (ms * 1e-3)

    out = {}
    gib = 1 << 30
    src = torch.ones(gib // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    out["hbm_copy_GBs"] = rate(lambda: lib.rpe_roof_copy(src.data_ptr(), dst.data_ptr(), gib, sp,
                                                         ctypes.byref(work)), 10) / 1e9
    out["hbm_read_GBs"] = rate(lambda: lib.rpe_roof_read(src.data_ptr(), gib, 1, sink.data_ptr(), sp,
                                                         ctypes.byref(work)), 10) / 1e9
    del src, dst
    for mb in (38, 77):
        buf = torch.ones(mb * 1000 * 1000 // 16 * 4, dtype=torch.float32, device=dev)
        nb = buf.numel() * 4
        out[f"cache_read_GBs_{mb}MB"] = rate(lambda: lib.rpe_roof_read(buf.data_ptr(), nb, 20, sink.data_ptr(), sp,
                                                                       ctypes.byref(work)), 10) / 1e9
        del buf
    out["mfma_bf16_TFLOPs"] = rate(lambda: lib.rpe_roof_mfma_bf16(2000, sink.data_ptr(), sp,
                                                                  ctypes.byref(work)), 3) / 1e12
    out["fma_f32_TFLOPs"] = rate(lambda: lib.rpe_roof_fma_f32(20000, sink.data_ptr(), sp,
                                                              ctypes.byref(work)), 5) / 1e12
    out["exp2_f32_Gps"] = rate(lambda: lib.rpe_roof_exp2_f32(20000, sink.data_ptr(), sp,
                                                             ctypes.byref(work)), 5) / 1e9
    torch.cuda.synchronize()
    out["note"] = ("measured on this GPU (librpe_roofs.so, include/rpe_roofs.h); the roofline fractions use "
                   "the published peaks, measured_frac the measured HBM copy or bf16 MFMA rate; fma_f32 counts "
                   "scalar (non-packed) FMAs")
    return out


def summarize(name, ms):
    w = WORKLOADS[name]
    flop, nbytes = flops_bytes(w)
    tflops = flop / (ms * 1e-3) / 1e12
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"ms": ms, "tflops": tflops, "mfma_frac": tflops / PEAK_MFMA_BF16, "gbs": gbs,
            "hbm_frac": gbs / PEAK_HBM, "flop": flop, "bytes": nbytes}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE, choices=list(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--warm-only", action="store_true", help="time one resident buffer set only")
    ap.add_argument("--no-warm", action="store_true",
                    help="skip the headline's warm timing (one resident buffer set)")
    ap.add_argument("--no-roofs", action="store_true", help="skip the measured machine roofs")
    ap.add_argument("--calib-probe", type=int, default=0, metavar="MIB",
                    help="after timing, run 3 read-only passes (a sum) and 3 write-only passes (a fill) "
                         "over MIB MiB: the known bytes that calibrate the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the forward shards by batch/head with no communication; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.workload)       # before any GPU call (forks a pool)
        print(f"cpu baseline: {cpu['sample']}", file=sys.stderr, flush=True)

    import torch
    dev = torch.device("cuda:0")
    import vision_transformer_attention_amd as pkg
    pkg.load()

    torch.cuda.synchronize()
    ms_cold, q_cold, wall, copies, ok = time_workload(args.workload, args.steps, args.warmup, dev,
                                                      cold=not args.warm_only)
    print(f"{args.workload}: {ms_cold * 1e3:.2f} us/launch over {copies} buffer sets (median {q_cold['median']:.2f}, "
          f"p10 {q_cold['p10']:.2f}, p90 {q_cold['p90']:.2f}), finite={ok}", file=sys.stderr, flush=True)
    ms_warm = q_warm = None
    if not args.no_warm and not args.warm_only:
        ms_warm, q_warm, _, _, _ = time_workload(args.workload, args.steps, args.warmup, dev, cold=False)
        print(f"{args.workload} warm: {ms_warm * 1e3:.2f} us/launch", file=sys.stderr, flush=True)
    head = summarize(args.workload, ms_cold)
    w = WORKLOADS[args.workload]
    secondary = {}
    if not args.no_secondary:
        for name in SECONDARY:
            if name == args.workload:
                continue
            mc, qc, _, _, okc = time_workload(name, args.steps, args.warmup, dev, cold=True)
            mw, _, _, _, _ = time_workload(name, args.steps, args.warmup, dev, cold=False)
            s = summarize(name, mc)
            sw = summarize(name, mw)
            secondary[name] = {"description": WORKLOADS[name].description, "us_per_launch": mc * 1e3,
                               "us_median": qc["median"], "us_p10": qc["p10"], "us_p90": qc["p90"],
                               "tflops": s["tflops"], "mfma_frac": s["mfma_frac"], "gbs": s["gbs"],
                               "hbm_frac": s["hbm_frac"], "warm_us_per_launch": mw * 1e3,
                               "warm_tflops": sw["tflops"], "warm_mfma_frac": sw["mfma_frac"],
                               "finite": okc}
            print(f"{name}: {mc * 1e3:.2f} us cold, {mw * 1e3:.2f} us warm", file=sys.stderr, flush=True)
    backward = None
    if not args.no_secondary:
        mb, okb = time_backward(args.workload, 10, 2, dev)
        fb, _ = flops_bytes(w)
        backward = {"workload": w.description, "us_per_call": mb * 1e3,
                    "tflops": 2.5 * fb / (mb * 1e-3) / 1e12, "finite": okb,
                    "note": "kernel sequence over a workspace (matrix-core products for bf16); TFLOP/s counts 2.5x the forward's FLOP"}
        print(f"backward {args.workload}: {mb * 1e3:.1f} us per call", file=sys.stderr, flush=True)
    roofs = None
    if not args.no_roofs:
        roofs = measure_roofs(dev)
        print("measured roofs: " + ", ".join(f"{k} {v:.1f}" for k, v in roofs.items() if k != "note"),
              file=sys.stderr, flush=True)
    if args.calib_probe > 0:
        # known bytes: a sum reads the whole tensor (and writes a few partials), a fill
        # writes it (and reads nothing)
        n = args.calib_probe << 20
        buf = torch.empty(n // 4, dtype=torch.float32, device=dev)
        buf.fill_(1.0)
        torch.cuda.synchronize()
        for _ in range(3):
            buf.sum()
        torch.cuda.synchronize()
        for _ in range(3):
            buf.fill_(2.0)
        torch.cuda.synchronize()
        del buf
    flop, nbytes = flops_bytes(w)
    intensity = flop / nbytes
    ridge = PEAK_MFMA_BF16 * 1e12 / (PEAK_HBM * 1e9)
    if intensity < ridge:
        roof = {"bound": "hbm", "achieved": head["gbs"], "peak": PEAK_HBM, "unit": "GB/s",
                "frac": head["gbs"] / PEAK_HBM, "traffic": None}
    else:
        roof = {"bound": "mfma", "achieved": head["tflops"], "peak": PEAK_MFMA_BF16, "unit": "TFLOP/s",
                "frac": head["tflops"] / PEAK_MFMA_BF16, "traffic": None}
    traffic, tnote = measured_traffic(args.workload)
    if traffic is not None:
        roof["traffic"] = traffic["total"]
        roof["traffic_fetch"] = traffic["fetch"]
        roof["traffic_write"] = traffic["write"]
    roof["traffic_source"] = tnote if traffic is None else os.path.relpath(tnote, ROOT)
    if roofs is not None:
        roof["measured_peak"] = roofs["hbm_copy_GBs"] if roof["bound"] == "hbm" else roofs["mfma_bf16_TFLOPs"]
        roof["measured_frac"] = roof["achieved"] / roof["measured_peak"]
    roof["kernel"] = "rpe_fwd_kernel"
    roof["algorithmic_bytes_per_launch"] = nbytes
    roof["algorithmic_flop_per_launch"] = flop
    line = {
        "metric": METRIC,
        "value": head["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_cold,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02^2) tables; inputs cycled through "
                f"{copies} HBM-resident copies so each step reads from HBM)",
        "config": {"workload": w.description, "global_batch": w.batch, "seq_len": w.tokens,
                   "parallelism": "none (1 GPU)"},
        "mfma_frac": head["mfma_frac"],
        "roofline": roof,
        "us_per_launch": ms_cold * 1e3,
        "us_per_launch_quantiles": dict(q_cold, note=f"per-launch means of {q_cold['batches']} consecutive "
                                                     "batches of the timed launches (HIP events at batch ends)"),
        "cpu_baseline": None if cpu is None else {k: v for k, v in cpu.items() if k != "seconds"},
        "secondary": secondary,
        "backward": backward,
        "measured_roofs": roofs,
    }
    if ms_warm is not None:
        warm = summarize(args.workload, ms_warm)
        line["warm"] = {"us_per_launch": ms_warm * 1e3, "us_median": q_warm["median"], "us_p10": q_warm["p10"],
                        "us_p90": q_warm["p90"], "tflops": warm["tflops"], "mfma_frac": warm["mfma_frac"],
                        "gbs": warm["gbs"], "hbm_frac": warm["hbm_frac"],
                        "note": "one resident buffer set (inputs stay in the 256 MB Infinity Cache); "
                                "value above is the cold rate"}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

"""Benchmark of the Range-Doppler focusing path on one MI355X.

One JSON line on stdout.  `value` is the headline: range-compression throughput in GB/s on the
4096 lines x 4096 samples complex64 workload (TBP-1000 chirp, Hamming, 5 targets + unit
clutter), counting one read and one write of every sample (2 * Na * Nr * 8 bytes per call).
A step is one rd_range_compress call over one 4096 x 4096 batch, which for this workload is
the whole hot path.  The line also reports the full focusing chain (rd_focus) on the
4096 x 4096 airborne scene in Mpixel/s, with its fraction of the HBM roofline for the
five-sweep and the compulsory byte models, and the CPU oracle timed on this host.

Also reported (not the headline): range compression of the 8192 x 6000 (mixed-radix) and
16384 x 16384 workloads, focusing of the 16384 x 16384 scene, per-stage times of the 4096 x 4096
chain, and the vendor FFT library (torch.fft on rocFFT: forward FFT, filter multiply, inverse
FFT as three launches) on the 4096 x 4096 range compression as a comparison.

Inputs are HBM-resident before timing starts; buffers rotate over 4 input/output pairs (1 GiB
per workload) so successive steps do not replay from the 256 MB Infinity Cache (the larger
workloads exceed it on their own).  Timing uses HIP events recorded on the stream the kernels
are launched on.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
ROTATE = 4


def kernel_source_hash() -> str:
    h = hashlib.sha1()
    for f in ("fft_core.hpp", "rd_kernels.hip", "rd_kernels.hpp"):
        with open(os.path.join(ROOT, "range_doppler_focusing_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:12]


def read_traffic(path: str, src_hash: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it was taken on the
    current kernel source; else None."""
    try:
        kv = {}
        for line in open(path):
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
        if kv.get("kernel_source_sha1") != src_hash:
            return None
        return float(kv["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def read_chain_traffic(path: str, src_hash: str):
    """Calibrated HBM KiB per launch of each kernel of the focusing chains, from the committed
    counter summary (a markdown table), if it was taken on the current kernel source; else None."""
    try:
        text = open(path).read()
        if f"kernel_source_sha1: {src_hash}." not in text:
            return None
        head = next(l for l in text.splitlines() if l.startswith("| counter |"))
        row = next(l for l in text.splitlines() if l.startswith("| HBM KiB (calibrated) |"))
        names = [c.strip() for c in head.strip("|").split("|")][1:]
        vals = [float(c) for c in row.strip("|").split("|")[1:]]
        return {n: v for n, v in zip(names, vals)}
    except (OSError, StopIteration, ValueError):
        return None


SETTLE_S = 0.3


def note(msg: str) -> None:
    """A progress line on stderr (the JSON result is the only stdout line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def time_steps(torch, fn, steps: int, warmup: int, stream):
    """ms per step over exactly `steps` calls, after `warmup` untimed calls.  Before those, the
    step runs for SETTLE_S seconds (untimed, in long batches): the GPU's clocks ramp up over the
    first few milliseconds of sustained load, and a timed region that starts from an idle GPU
    measures the ramp rather than the kernels."""
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < SETTLE_S:
        for _ in range(64):
            fn(i)
            i += 1
        torch.cuda.synchronize()
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        fn(i)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps  # ms per step


def cpu_oracle_rc(cfg, echo, budget_s: float = 10.0):
    """The CPU oracle's range compression of the whole workload (float64; its FFTs on the
    oracle's worker threads), repeated until about `budget_s` seconds have run, at least 3 times
    after a warm-up; returns (median s, runs)."""
    from oracle import rd_oracle as O
    p = cfg.plan_params()
    O.range_compress(echo, p)          # warm-up (FFT plans, page faults)
    ts = []
    t_start = time.perf_counter()
    while len(ts) < 3 or (time.perf_counter() - t_start < budget_s and len(ts) < 200):
        t0 = time.perf_counter()
        O.range_compress(echo, p)
        ts.append(time.perf_counter() - t0)
    return statistics.median(ts), len(ts)


def cpu_oracle_focus(cfg, echo, runs: int = 3):
    """The CPU oracle's whole chain (float64; its FFTs on the oracle's worker threads, the RCMC
    and filter arithmetic in NumPy on one thread) on the whole scene: one warm-up run, then the
    median of `runs`; returns (median s, runs)."""
    from oracle import rd_oracle as O
    O.focus_stages(echo, cfg.plan_params())
    ts = []
    for _ in range(runs):
        t0 = time.perf_counter()
        O.focus_stages(echo, cfg.plan_params())
        ts.append(time.perf_counter() - t0)
    return statistics.median(ts), runs


def gpu_noise(torch, shape, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randn(shape, dtype=torch.complex64, device="cuda", generator=g)


def vendor_fft_comparison(torch, rdf, cfg, stream, steps, warmup):
    """Range compression with the vendor FFT library through torch.fft (rocFFT): forward FFT,
    multiply by the matched filter, inverse FFT -- three launches and three HBM round trips.
    A reported comparison only; its result is checked against rd_range_compress."""
    import math
    p = cfg.plan_params()
    fs, tp, bw = p["fs_hz"], p["pulse_s"], p["bandwidth_hz"]
    L = math.ceil(tp * fs - 1e-6)
    n = torch.arange(L, dtype=torch.float64)
    t = n / fs - tp / 2
    w = (0.54 - 0.46 * torch.cos(2 * math.pi * n / (L - 1))) if p["range_window"] == 1 else 1.0
    h = torch.zeros(cfg.Nr, dtype=torch.complex128)
    h[:L] = w * torch.exp(1j * math.pi * (bw / tp) * t * t)
    H = torch.fft.fft(h).conj().to(torch.complex64).to("cuda")
    xs = [gpu_noise(torch, (cfg.Na, cfg.Nr), cfg.seed + i) for i in range(ROTATE)]
    ys = [torch.empty_like(xs[0]) for _ in range(ROTATE)]

    def step(i):
        X = torch.fft.fft(xs[i % ROTATE], dim=1)
        X.mul_(H)
        torch.fft.ifft(X, dim=1, out=ys[i % ROTATE])

    ms = time_steps(torch, step, steps, warmup, stream)
    plan = rdf.Plan(**p)
    ref = plan.range_compress(xs[0])
    plan.close()
    step(0)
    torch.cuda.synchronize()
    err = float(torch.linalg.vector_norm(ys[0] - ref) / torch.linalg.vector_norm(ref))
    del xs, ys
    torch.cuda.empty_cache()
    gbs = 2 * cfg.Na * cfg.Nr * 8 / (ms * 1e-3) / 1e9
    return {"workload": "range compression 4096 x 4096 complex64 via torch.fft (rocFFT), 3 launches",
            "ms_per_step": round(ms, 5), "value": round(gbs, 1), "unit": "GB/s",
            "rel_l2_vs_rd_range_compress": err}


def main():
    global SETTLE_S
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle", type=float, default=SETTLE_S,
                    help="seconds of untimed running before each warm-up (0 for counter runs)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-focus", action="store_true", help="skip the full-chain measurement")
    ap.add_argument("--only", choices=["rc", "focus", "large", "vendor", "turn", "bp", "pad", "wk", "f16",
                                       "rc6000", "rc16384", "focus16384"], default=None,
                    help="run one workload only (for profiling); rc6000 / rc16384 / focus16384: one of the "
                         "large workloads on its own")
    ap.add_argument("--no-large", action="store_true",
                    help="skip the 8192 x 6000 and 16384 x 16384 workloads")
    args = ap.parse_args()
    SETTLE_S = args.settle
    if args.gpus != 1:
        print(f"bench.py: the focusing path runs on one GPU; --gpus {args.gpus} is not supported "
              "(sharding across GPUs is a design note, not implemented)", file=sys.stderr)
        sys.exit(2)

    import torch

    import range_doppler_focusing_amd as rdf
    from rdscene import C2, C3, C4, C5, cached_scene

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    src_hash = kernel_source_hash()
    out = {}

    # ---------------------------------------------------------------- range compression (value)
    cfg = C2
    rc_ms = None
    if args.only in (None, "rc"):
        sc = cached_scene(cfg)
        echo0 = torch.from_numpy(sc.echo).to("cuda")
        ins = [echo0] + [echo0.clone() for _ in range(ROTATE - 1)]
        outs = [torch.empty_like(echo0) for _ in range(ROTATE)]
        plan = rdf.Plan(**cfg.plan_params())
        rc_ms = time_steps(torch, lambda i: rdf.rd_range_compress(plan.handle, ins[i % ROTATE],
                                                                  outs[i % ROTATE], stream),
                           args.steps, args.warmup, stream)
        plan.close()
        del ins, outs, echo0
        torch.cuda.empty_cache()
    rc_bytes = 2 * cfg.Na * cfg.Nr * 8
    rc_gbs = rc_bytes / (rc_ms * 1e-3) / 1e9 if rc_ms else None
    if rc_ms:
        note(f"range compression 4096 x 4096: {rc_ms * 1e3:.1f} us")

    # ---------------------------------------------------------------- full chain
    fcfg = C3
    focus_ms = None
    stage_ms = None
    if args.only in (None, "focus") and not args.no_focus:
        fsc = cached_scene(fcfg)
        e0 = torch.from_numpy(fsc.echo).to("cuda")
        fins = [e0] + [e0.clone() for _ in range(ROTATE - 1)]
        fouts = [torch.empty_like(e0) for _ in range(ROTATE)]
        fplan = rdf.Plan(**fcfg.plan_params())
        focus_ms = time_steps(torch, lambda i: rdf.rd_focus(fplan.handle, fins[i % ROTATE],
                                                            fouts[i % ROTATE], stream),
                              max(10, args.steps // 2), args.warmup, stream)
        # the chain's two halves on their own (the range half is the same kernel as the headline)
        az_ms = time_steps(torch, lambda i: rdf.rd_azimuth_focus(fplan.handle, fins[i % ROTATE],
                                                                 fouts[i % ROTATE], stream),
                           max(10, args.steps // 2), args.warmup, stream)
        rc_alone_ms = time_steps(torch, lambda i: rdf.rd_range_compress(fplan.handle, fins[i % ROTATE],
                                                                        fouts[i % ROTATE], stream),
                                 max(10, args.steps // 2), args.warmup, stream)
        img_bytes = fcfg.Na * fcfg.Nr * 8
        stage_ms = {"rd_range_compress_ms": round(rc_alone_ms, 4),
                    "rd_range_compress_GBps": round(2 * img_bytes / (rc_alone_ms * 1e-3) / 1e9, 1),
                    "rd_azimuth_focus_ms": round(az_ms, 4),
                    # four azimuth transform steps and the RCMC pass: five sweeps of 16 B a pixel
                    "rd_azimuth_focus_GBps_80B_per_px": round(10 * img_bytes / (az_ms * 1e-3) / 1e9, 1),
                    "note": "each half timed on its own from an HBM-resident input; inside rd_focus "
                            "the range-compressed image stays in the Infinity Cache for the azimuth "
                            "passes, so the chain takes less than the sum"}
        fplan.close()
        del fins, fouts, e0
        torch.cuda.empty_cache()
    px = fcfg.Na * fcfg.Nr
    mpx = px / (focus_ms * 1e-3) / 1e6 if focus_ms else None
    if focus_ms:
        note(f"rd_focus 4096 x 4096: {focus_ms * 1e3:.1f} us")

    # ---------------------------------------------------------------- omega-k
    wk = None
    if args.only in (None, "wk") and not args.no_focus:
        wk = []
        for wcfg, steps in ((fcfg, max(10, args.steps // 2)), (C5, 5)):
            ref = int(round((wcfg.r_ref_m - wcfg.range_bin0_m) / wcfg.dr))
            big = wcfg.Na * wcfg.Nr > 4096 * 4096
            nrot = 1 if big else ROTATE
            if big:
                xs = [gpu_noise(torch, (wcfg.Na, wcfg.Nr), wcfg.seed)]
            else:
                x0 = torch.from_numpy(cached_scene(wcfg).echo).to("cuda")
                xs = [x0] + [x0.clone() for _ in range(nrot - 1)]
            ys = [torch.empty_like(xs[0]) for _ in range(nrot)]
            wplan = rdf.Plan(**wcfg.plan_params())
            ms = time_steps(torch, lambda i: rdf.rd_omega_k(wplan.handle, xs[i % nrot], ys[i % nrot], ref, stream),
                            steps, 2, stream)
            wplan.close()
            del xs, ys
            torch.cuda.empty_cache()
            m = wcfg.Na * wcfg.Nr / (ms * 1e-3) / 1e6
            rec = {"workload": f"omega-k focusing (rd_omega_k), {wcfg.Na} x {wcfg.Nr} complex64, reference bin {ref}",
                   "ms_per_step": round(ms, 4), "steps": steps, "value": round(m, 1), "unit": "Mpixel/s",
                   "roofline_frac_80B_per_px": round(m * 1e6 * 80 / (HBM_PEAK_GBS * 1e9), 4),
                   "data": "seeded complex Gaussian noise on the device" if big else
                           "synthetic scene (seeded point targets + clutter)"}
            if not big and not args.no_cpu and args.only is None:
                # the oracle on the first 1024 pulses of the same geometry (a quarter of the scene)
                from oracle import rd_oracle as O
                sub = wcfg.with_(Na=1024)
                t0 = time.perf_counter()
                O.omega_k(cached_scene(wcfg).echo[:1024], sub.plan_params(), ref)
                tw = time.perf_counter() - t0
                rec["cpu_baseline"] = {"value": round(1024 * wcfg.Nr / tw / 1e6, 4), "unit": "Mpixel/s",
                                       "cores": O.workers(), "kind": "oracle",
                                       "sample": f"1024 pulses x {wcfg.Nr} of the same geometry, one run ({tw:.1f} s)"}
            wk.append(rec)
            note(f"omega-k {wcfg.Na} x {wcfg.Nr}: {ms * 1e3:.1f} us")

    # ---------------------------------------------------------------- CPU oracle
    cpu = None
    cpu_focus = None
    if not args.no_cpu and args.only is None:
        from oracle import rd_oracle as O
        cores = O.workers()  # the oracle's FFT threads: this process's CPUs, capped by OMP_NUM_THREADS
        note(f"oracle on {cores} worker threads (host reports {os.cpu_count()} CPUs, "
             f"{len(os.sched_getaffinity(0))} in this process's affinity set)")
        t, runs = cpu_oracle_rc(cfg, cached_scene(cfg).echo)
        note(f"oracle range compression: {t:.2f} s per run")
        cpu = {"value": rc_bytes / t / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
               "sample": f"whole 4096x4096 range compression (float64, scipy.fft on {cores} threads), "
                         f"warm-up then median of {runs} runs ({t:.3f} s each)"}
        if focus_ms:
            tf, fr = cpu_oracle_focus(fcfg, cached_scene(fcfg).echo)
            note(f"oracle rd focus: {tf:.2f} s per run")
            cpu_focus = {"value": px / tf / 1e6, "unit": "Mpixel/s", "cores": cores, "kind": "oracle",
                         "sample": f"whole 4096x4096 rd focus (float64; FFTs on {cores} threads, RCMC and "
                                   f"filter on one), warm-up then median of {fr} runs ({tf:.2f} s each)"}

    # ---------------------------------------------------------------- larger workloads
    large = None
    single = {"rc6000": (C4, "rc"), "rc16384": (C5, "rc"), "focus16384": (C5, "focus")}
    if (args.only in (None, "large") or args.only in single) and not args.no_large:
        large = []
        for wcfg, kind, steps in ((C4, "rc", 20), (C5, "rc", 10), (C5, "focus", 5)):
            if args.only in single and single[args.only] != (wcfg, kind):
                continue
            x = gpu_noise(torch, (wcfg.Na, wcfg.Nr), wcfg.seed)
            y = torch.empty_like(x)
            plan = rdf.Plan(**wcfg.plan_params())
            call = rdf.rd_range_compress if kind == "rc" else rdf.rd_focus
            ms = time_steps(torch, lambda i: call(plan.handle, x, y, stream), steps, 2, stream)
            plan.close()
            del x, y
            torch.cuda.empty_cache()
            px = wcfg.Na * wcfg.Nr
            rec = {"workload": f"{'range compression' if kind == 'rc' else 'full RD focusing'}, "
                               f"{wcfg.Na} x {wcfg.Nr} complex64",
                   "ms_per_step": round(ms, 4), "steps": steps,
                   "data": "seeded complex Gaussian noise on the device (timing is data-independent)"}
            if kind == "rc":
                gbs = 2 * px * 8 / (ms * 1e-3) / 1e9
                rec.update({"value": round(gbs, 1), "unit": "GB/s",
                            "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                            "lines_per_s": round(wcfg.Na / (ms * 1e-3), 1)})
            else:
                m = px / (ms * 1e-3) / 1e6
                rec.update({"value": round(m, 1), "unit": "Mpixel/s",
                            "roofline_frac_80B_per_px": round(m * 1e6 * 80 / (HBM_PEAK_GBS * 1e9), 4)})
            large.append(rec)
            note(f"{rec['workload']}: {ms * 1e3:.1f} us")

    # ---------------------------------------------------------------- binary16 storage
    if (args.only in (None, "large", "f16")) and not args.no_large:
        large = large or []
        sc = cached_scene(cfg)
        e16 = torch.from_numpy(sc.echo).to("cuda").view(torch.float32).to(torch.float16).view(cfg.Na, cfg.Nr, 2)
        ins = [e16] + [e16.clone() for _ in range(ROTATE - 1)]
        outs = [torch.empty_like(e16) for _ in range(ROTATE)]
        plan = rdf.Plan(**cfg.plan_params())
        ms = time_steps(torch, lambda i: rdf.rd_range_compress_f16(plan.handle, ins[i % ROTATE], outs[i % ROTATE], stream),
                        args.steps, args.warmup, stream)
        plan.close()
        del ins, outs, e16
        torch.cuda.empty_cache()
        b16 = 2 * cfg.Na * cfg.Nr * 4
        gbs = b16 / (ms * 1e-3) / 1e9
        large.append({"workload": "range compression with binary16 storage (rd_range_compress_f16), "
                                  f"{cfg.Na} x {cfg.Nr}, float32 arithmetic, same chirp as the headline",
                      "ms_per_step": round(ms, 4), "steps": args.steps, "value": round(gbs, 1), "unit": "GB/s",
                      "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                      "samples_per_s": round(cfg.Na * cfg.Nr / (ms * 1e-3), 1),
                      "data": "the headline scene rounded to binary16"})
        note(f"binary16 range compression: {ms * 1e3:.1f} us")
        # the whole range-Doppler chain with binary16 storage: 4096 x 4096 airborne scene and
        # the 16384 x 16384 scene (five sweeps of 8 B a pixel in the pages' model: 40 B/px)
        for zcfg, steps in ((fcfg, max(10, args.steps // 2)), (C5, max(5, args.steps // 20))):
            zs = cached_scene(zcfg)
            z16 = torch.from_numpy(zs.echo).to("cuda").view(torch.float32).to(torch.float16).view(zcfg.Na, zcfg.Nr, 2)
            rot = ROTATE if zcfg is fcfg else 2
            ins = [z16] + [z16.clone() for _ in range(rot - 1)]
            outs = [torch.empty_like(z16) for _ in range(rot)]
            plan = rdf.Plan(**zcfg.plan_params())
            ms = time_steps(torch, lambda i: rdf.rd_focus_f16(plan.handle, ins[i % rot], outs[i % rot], stream),
                            steps, args.warmup, stream)
            plan.close()
            del ins, outs, z16
            torch.cuda.empty_cache()
            mp = zcfg.Na * zcfg.Nr / (ms * 1e-3) / 1e6
            large.append({"workload": f"full RD focusing with binary16 storage (rd_focus_f16), {zcfg.Na} x {zcfg.Nr}, "
                                      "float32 arithmetic, image / Na",
                          "ms_per_step": round(ms, 4), "steps": steps, "value": round(mp, 1), "unit": "Mpixel/s",
                          "roofline_frac_40B_per_px": round(mp * 1e6 * 40 / (HBM_PEAK_GBS * 1e9), 4),
                          "data": "the focusing scene rounded to binary16"})
            note(f"rd_focus_f16 {zcfg.Na} x {zcfg.Nr}: {ms * 1e3:.1f} us")
        # omega-k with binary16 storage on the 4096 x 4096 airborne scene
        ref = int(round((fcfg.r_ref_m - fcfg.range_bin0_m) / fcfg.dr))
        z16 = torch.from_numpy(cached_scene(fcfg).echo).to("cuda").view(torch.float32).to(torch.float16).view(
            fcfg.Na, fcfg.Nr, 2)
        ins = [z16] + [z16.clone() for _ in range(ROTATE - 1)]
        outs = [torch.empty_like(z16) for _ in range(ROTATE)]
        plan = rdf.Plan(**fcfg.plan_params())
        steps = max(10, args.steps // 2)
        ms = time_steps(torch, lambda i: rdf.rd_omega_k_f16(plan.handle, ins[i % ROTATE], outs[i % ROTATE], ref, stream),
                        steps, args.warmup, stream)
        plan.close()
        del ins, outs, z16
        torch.cuda.empty_cache()
        mp = fcfg.Na * fcfg.Nr / (ms * 1e-3) / 1e6
        large.append({"workload": f"omega-k focusing with binary16 storage (rd_omega_k_f16), {fcfg.Na} x {fcfg.Nr}, "
                                  f"float32 arithmetic, image / Na, reference bin {ref}",
                      "ms_per_step": round(ms, 4), "steps": steps, "value": round(mp, 1), "unit": "Mpixel/s",
                      "roofline_frac_40B_per_px": round(mp * 1e6 * 40 / (HBM_PEAK_GBS * 1e9), 4),
                      "data": "the focusing scene rounded to binary16"})
        note(f"rd_omega_k_f16 {fcfg.Na} x {fcfg.Nr}: {ms * 1e3:.1f} us")

    # ---------------------------------------------------------------- a line length with no built transform
    if (args.only in (None, "large", "pad")) and not args.no_large:
        large = large or []
        na, nr, fs = 16384, 1200, 120e6
        pp = dict(Na=na, Nr=nr, pulse_s=400 / fs, bandwidth_hz=100e6, fs_hz=fs, range_window=1)
        x = gpu_noise(torch, (na, nr), 31)
        y = torch.empty_like(x)
        plan = rdf.Plan(**pp)
        ms = time_steps(torch, lambda i: rdf.rd_range_compress(plan.handle, x, y, stream), 50, 3, stream)
        plan.close()
        gbs = 2 * na * nr * 8 / (ms * 1e-3) / 1e9
        m = 256
        while m < nr + 400 - 1:          # padded length: power of two >= Nr + L - 1
            m *= 2
        rec = {"workload": f"range compression of {nr}-sample lines (no built transform: exact "
                           f"zero-padded {m}-point convolution), {na} x {nr} complex64, "
                           "3.33 us / 100 MHz chirp at 120 MHz (400 samples), Hamming",
               "ms_per_step": round(ms, 4), "steps": 50, "value": round(gbs, 1), "unit": "GB/s",
               "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "lines_per_s": round(na / (ms * 1e-3), 1),
               "data": "seeded complex Gaussian noise on the device (timing is data-independent)"}
        if not args.no_cpu:
            from oracle import rd_oracle as O
            xh = x.cpu().numpy()
            t0 = time.perf_counter()
            O.range_compress(xh, pp)
            tc = time.perf_counter() - t0
            rec["cpu_baseline"] = {"value": round(2 * na * nr * 8 / tc / 1e9, 3), "unit": "GB/s",
                                   "cores": O.workers(), "kind": "oracle",
                                   "sample": f"all {na} lines, one run ({tc:.2f} s)"}
        large.append(rec)
        note(f"padded range compression 16384 x 1200: {ms * 1e3:.1f} us")
        del x, y
        torch.cuda.empty_cache()
        # range-Doppler focusing at that line length (the 4096-pulse airborne geometry with a
        # 1 us pulse): padded range compression, azimuth steps, RCMC on 1200-sample rows
        acfg = fcfg.with_(Nr=1200, pulse_s=1e-6)
        x = gpu_noise(torch, (acfg.Na, acfg.Nr), 32)
        y = torch.empty_like(x)
        plan = rdf.Plan(**acfg.plan_params())
        ms = time_steps(torch, lambda i: rdf.rd_focus(plan.handle, x, y, stream), 50, 3, stream)
        plan.close()
        m = acfg.Na * acfg.Nr / (ms * 1e-3) / 1e6
        large.append({"workload": f"full RD focusing at a line length with no built transform, {acfg.Na} x {acfg.Nr} "
                                  "complex64 (9.6 GHz, 1 us / 300 MHz at 360 MHz, PRF 1.5 kHz, 150 m/s, 10 km)",
                      "ms_per_step": round(ms, 4), "steps": 50, "value": round(m, 1), "unit": "Mpixel/s",
                      "roofline_frac_80B_per_px": round(m * 1e6 * 80 / (HBM_PEAK_GBS * 1e9), 4),
                      "data": "seeded complex Gaussian noise on the device (timing is data-independent)"})
        note(f"rd_focus {acfg.Na} x {acfg.Nr}: {ms * 1e3:.1f} us")
        del x, y
        torch.cuda.empty_cache()
        # the image size of the pages' airborne test (1200 range samples x 800 pulses): neither
        # length is a power of two (800 = 32 x 25 azimuth steps, 1200 padded range compression)
        ocfg = fcfg.with_(Na=800, Nr=1200, pulse_s=1e-6)
        x = gpu_noise(torch, (ocfg.Na, ocfg.Nr), 33)
        y = torch.empty_like(x)
        plan = rdf.Plan(**ocfg.plan_params())
        ms = time_steps(torch, lambda i: rdf.rd_focus(plan.handle, x, y, stream), 100, 3, stream)
        plan.close()
        large.append({"workload": f"full RD focusing of a {ocfg.Nr} x {ocfg.Na} image (range x azimuth; no power-of-two "
                                  "length), 9.6 GHz, 1 us / 300 MHz at 360 MHz, PRF 1.5 kHz, 150 m/s, 10 km",
                      "ms_per_step": round(ms, 4), "steps": 100, "value": round(1e3 / ms, 1), "unit": "images/s",
                      "mpixel_per_s": round(ocfg.Na * ocfg.Nr / (ms * 1e-3) / 1e6, 1),
                      "data": "seeded complex Gaussian noise on the device (timing is data-independent)"})
        note(f"rd_focus {ocfg.Na} x {ocfg.Nr}: {ms * 1e3:.1f} us")
        del x, y
        torch.cuda.empty_cache()
        # a prime azimuth length: the Bluestein form of the azimuth transform (M = 2048)
        pcfg = fcfg.with_(Na=997, Nr=1024, pulse_s=1e-6)
        x = gpu_noise(torch, (pcfg.Na, pcfg.Nr), 34)
        y = torch.empty_like(x)
        plan = rdf.Plan(**pcfg.plan_params())
        ms = time_steps(torch, lambda i: rdf.rd_focus(plan.handle, x, y, stream), 100, 3, stream)
        plan.close()
        large.append({"workload": f"full RD focusing with a prime azimuth length (Bluestein form), {pcfg.Na} x {pcfg.Nr} "
                                  "complex64, 9.6 GHz, 1 us / 300 MHz at 360 MHz, PRF 1.5 kHz, 150 m/s, 10 km",
                      "ms_per_step": round(ms, 4), "steps": 100,
                      "value": round(pcfg.Na * pcfg.Nr / (ms * 1e-3) / 1e6, 1), "unit": "Mpixel/s",
                      "data": "seeded complex Gaussian noise on the device (timing is data-independent)"})
        note(f"rd_focus {pcfg.Na} x {pcfg.Nr}: {ms * 1e3:.1f} us")
        del x, y
        torch.cuda.empty_cache()

    # ---------------------------------------------------------------- corner turn
    if (args.only in (None, "large", "turn")) and not args.no_large:
        large = large or []
        for rows, cols in ((4096, 4096), (16384, 16384)):
            nrot = ROTATE if rows * cols <= 4096 * 4096 else 1
            xs = [gpu_noise(torch, (rows, cols), 11 + i) for i in range(nrot)]
            ys = [torch.empty((cols, rows), dtype=torch.complex64, device="cuda") for _ in range(nrot)]
            ms = time_steps(torch, lambda i: rdf.rd_corner_turn(xs[i % nrot], ys[i % nrot], rows, cols, stream),
                            50 if nrot > 1 else 10, 2, stream)
            gbs = 2 * rows * cols * 8 / (ms * 1e-3) / 1e9
            large.append({"workload": f"corner turn (rd_corner_turn), {rows} x {cols} complex64",
                          "ms_per_step": round(ms, 4), "value": round(gbs, 1), "unit": "GB/s",
                          "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                          "data": "seeded complex Gaussian noise on the device"})
            note(f"corner turn {rows} x {cols}: {ms * 1e3:.1f} us")
            del xs, ys
            torch.cuda.empty_cache()

    # ---------------------------------------------------------------- back-projection
    if (args.only in (None, "large", "bp")) and not args.no_large:
        large = large or []
        bcfg = C3
        bp = bcfg.plan_params()
        dr = 299_792_458.0 / (2.0 * bp["fs_hz"])
        nx = ny = 1024
        grid = dict(nx=nx, ny=ny, x0_m=bcfg.velocity_mps * (bcfg.Na // 2 - nx // 2) / bcfg.prf_hz,
                    dx_m=bcfg.velocity_mps / bcfg.prf_hz,
                    r0_m=bp["range_bin0_m"] + (bcfg.Nr // 2 - ny // 2) * dr, dr_m=dr)
        rc = gpu_noise(torch, (bcfg.Na, bcfg.Nr), 21)
        img = torch.empty((nx, ny), dtype=torch.complex64, device="cuda")
        bplan = rdf.Plan(**bp)
        ms = time_steps(torch, lambda i: rdf.rd_backproject(bplan.handle, rc, img, grid, stream), 5, 1, stream)
        bplan.close()
        pp = bcfg.Na * nx * ny
        rec = {"workload": f"back-projection (rd_backproject), {bcfg.Na} pulses x {bcfg.Nr} samples "
                           f"onto {nx} x {ny} pixels (4096 x 4096 airborne geometry)",
               "ms_per_step": round(ms, 4), "value": round(pp / (ms * 1e-3) / 1e9, 2),
               "unit": "Gpixel-pulses/s",
               "data": "seeded complex Gaussian noise on the device (timing is data-independent)"}
        if not args.no_cpu:
            # the oracle on a 32 x 32 corner of the same grid, all 4096 pulses
            from oracle import rd_oracle as O
            rc_h = rc.cpu().numpy()
            sub = dict(grid, nx=32, ny=32)
            t0 = time.perf_counter()
            O.backproject(rc_h, bp, sub)
            tb = time.perf_counter() - t0
            rec["cpu_baseline"] = {"value": round(bcfg.Na * 32 * 32 / tb / 1e9, 5), "unit": "Gpixel-pulses/s",
                                   "cores": 1, "kind": "oracle",
                                   "sample": f"32 x 32 pixels x {bcfg.Na} pulses, one run ({tb:.1f} s)"}
        large.append(rec)
        note(f"back-projection: {ms:.2f} ms")
        del rc, img
        torch.cuda.empty_cache()

    # ---------------------------------------------------------------- vendor FFT comparison
    vendor = None
    if args.only in (None, "vendor"):
        vendor = vendor_fft_comparison(torch, rdf, C2, stream, args.steps, args.warmup)

    traffic = read_traffic(os.path.join(ROOT, "profiles", "range_compress_4096x4096_traffic.txt"), src_hash)
    line = {
        "metric": "range-compressed GB/s (% HBM peak) and RD-focused Mpixel/s, 4096x4096 c64",
        "value": round(rc_gbs, 2) if rc_gbs else None,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(rc_ms, 5) if rc_ms else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "c64 (fp32 complex)",
        "data": "synthetic (seeded point targets + Gaussian clutter)",
        "config": {"workload": "range compression, 4096 lines x 4096 samples complex64, "
                               "10 us / 100 MHz chirp at 120 MHz, Hamming",
                   "Na": cfg.Na, "Nr": cfg.Nr, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(rc_gbs, 2) if rc_gbs else None,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(rc_gbs / HBM_PEAK_GBS, 4) if rc_gbs else None,
                     "traffic": traffic,
                     "kernel": "k_range_compress_4096",
                     "algorithmic_bytes_per_launch": rc_bytes},
        "cpu_baseline": cpu,
        "rd_focus": None if not focus_ms else {
            "workload": "full RD focusing, 4096 x 4096 complex64 airborne scene "
                        "(9.6 GHz, 300 MHz, PRF 1.5 kHz, 150 m/s, 10 km, 16 targets)",
            "ms_per_step": round(focus_ms, 4), "value": round(mpx, 1), "unit": "Mpixel/s",
            "roofline_frac_80B_per_px": round(mpx * 1e6 * 80 / (HBM_PEAK_GBS * 1e9), 4),
            "roofline_frac_32B_per_px": round(mpx * 1e6 * 32 / (HBM_PEAK_GBS * 1e9), 4),
            "stages": stage_ms,
            "hbm_kib_per_kernel_launch": read_chain_traffic(
                os.path.join(ROOT, "profiles", "rd_chain_4096x4096_counters.md"), src_hash),
            "cpu_baseline": cpu_focus},
        "omega_k": wk,
        "other_workloads": large,
        "vendor_fft_comparison": vendor,
        "kernel_source_sha1": src_hash,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()

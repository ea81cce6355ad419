"""Bench: exact tiled attention on one MI355X.

One step = one pass of the whole hot path over one batch: fa_fwd (writes O
and LSE) followed by fa_bwd (recomputes P from LSE, writes dQ, dK, dV), on
the causal bf16 workload [B=2, H=16, N=4096, d=128] with seeded synthetic
inputs already resident in device memory. The JSON line also carries the
forward-only figure of the causal [2, 16, 8192, 128] workload, the roofline
of the dominant kernel, and the CPU oracle timed on a bounded sample.

Every timed section is preceded by 0.3 s of the same work back to back (the
shader clock ramps up over the first tens of milliseconds after an idle
spell), then the W warm-up steps, then exactly K timed steps between two
device synchronisations.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
       python bench.py --summarize-pmc DIR --copy-mib M [--workload NAME]
                                      (HBM traffic summary of that workload, no GPU)
       python bench.py --sweep        (N = 2k..16k sweep, markdown table on stdout)
       python bench.py --gemm-ref     (vendor bf16 GEMM rate, for context)
       python bench.py --std-sweep [--std-n N] [--no-settle]
                                      (fused fa_fwd vs standard fa_fwd_standard, N = 1k..16k)
       python bench.py --summarize-std DIR   (their HBM bytes from per-N counter passes, no GPU)
       python bench.py --oracle-all   (the CPU oracle on every workload of the statement, no GPU)
       python bench.py --km-sweep [--km-n N] [--km-bc BC] [--no-settle]
                                      (key-major fa_fwd_keymajor over its key-block sizes)
       python bench.py --summarize-km DIR    (its HBM bytes vs block size, no GPU)
"""
import argparse
import csv
import glob
import hashlib
import json
import math
import os
import re
import statistics
import sys
import time
import types

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 4096 FLOP/clk x 2.4 GHz (published 2.5 PFLOP/s dense)
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def attn_pairs(N, mask, window):
    """Number of allowed (query, key) pairs per head."""
    if mask == "causal":
        return N * (N + 1) // 2
    if mask == "local":
        w = min(window, N - 1)
        return N * (2 * w + 1) - w * (w + 1)
    return N * N


def fwd_flops(w):
    """Algorithmic forward FLOPs: 4*B*H*N^2*d, halved under a causal mask;
    band masks count the allowed pairs (4*B*H*pairs*d)."""
    B, H, N, d = w.shape
    if w.mask == "causal":
        return 4.0 * B * H * N * N * d / 2
    if w.mask == "local":
        return 4.0 * B * H * attn_pairs(N, "local", w.window) * d
    return 4.0 * B * H * N * N * d


def bwd_flops(w):
    """Algorithmic backward FLOPs: five N^2 d contractions (QK^T recompute,
    dO V^T, P^T dO, dS^T Q, dS K) = 10*B*H*N^2*d, halved under causal."""
    return 2.5 * fwd_flops(w)


def fwd_bytes(w):
    B, H, N, d = w.shape
    es = 2 if w.dtype == "bf16" else 4
    return 4 * B * H * N * d * es + B * H * N * 4  # Q, K, V read, O written + LSE


def bwd_bytes(w):
    B, H, N, d = w.shape
    es = 2 if w.dtype == "bf16" else 4
    # read Q, K, V, O, dO, LSE; write dQ, dK, dV
    return 8 * B * H * N * d * es + B * H * N * 4


def kernel_source_sha():
    """Hash of the HIP sources: HBM traffic counters taken on other sources
    are not reported."""
    h = hashlib.sha256()
    for path in sorted(glob.glob(os.path.join(ROOT, "exact_tiled_attention_fwd_amd", "csrc", "*"))):
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# Entry point each kernel belongs to (one bf16 fa_bwd call = two launches, dQ then
# dK/dV; the float32 path adds a launch for D).
UNIT_OF_KERNEL = (("fwd_bf16", "fa_fwd"), ("fwd_f32", "fa_fwd"), ("bwd_pre", "fa_bwd"),
                  ("bwd_dkdv", "fa_bwd"), ("bwd_dq", "fa_bwd"))
TRAFFIC_TAG = "traffic-json:"


def _pmc_per_dispatch(path, counter):
    """Mean over dispatches of one counter, per kernel name (KiB)."""
    per = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            key = (r["Kernel_Name"], r["Dispatch_Id"])
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (name, _), v in per.items():
        out.setdefault(name, []).append(v)
    return {n: sum(v) / len(v) for n, v in out.items()}


def summarize_pmc(d, copy_mib, workload):
    """Markdown summary of the FETCH_SIZE / WRITE_SIZE passes in directory d
    (bytes between L2 and the memory fabric; the MALL may serve part of them):
    bench run on `workload` (fetch_*, write_*) and the copy calibration
    (copy_fetch_*, copy_write_*). Counter readings are scaled so that the
    plain copy of copy_mib MiB reads and writes exactly that many bytes."""
    one = lambda pat: sorted(glob.glob(os.path.join(d, pat)))[0]
    cf = _pmc_per_dispatch(one("copy_fetch*_counter_collection.csv"), "FETCH_SIZE")
    cw = _pmc_per_dispatch(one("copy_write*_counter_collection.csv"), "WRITE_SIZE")
    ck = [n for n in cf if "copyBuffer" in n or "copy" in n.lower()][0]
    nbytes = copy_mib * (1 << 20)
    f_fetch = nbytes / (cf[ck] * 1024.0)
    f_write = nbytes / (cw[ck] * 1024.0)
    fe = _pmc_per_dispatch(one("fetch*_counter_collection.csv"), "FETCH_SIZE")
    wr = _pmc_per_dispatch(one("write*_counter_collection.csv"), "WRITE_SIZE")
    units, rows = {}, []
    for name in sorted(fe):
        unit = next((u for key, u in UNIT_OF_KERNEL if key in name), None)
        if unit is None:
            continue
        rb = fe[name] * 1024.0 * f_fetch
        wb = wr.get(name, 0.0) * 1024.0 * f_write
        rows.append((name, fe[name], wr.get(name, 0.0), rb, wb))
        u = units.setdefault(unit, {"read_bytes": 0.0, "write_bytes": 0.0})
        u["read_bytes"] += rb
        u["write_bytes"] += wb
    lines = ["| Kernel | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch | read bytes | written bytes |",
             "|---|---|---|---|---|"]
    for name, f_, w_, rb, wb in rows:
        short = re.sub(r"\(.*", "", name)
        lines.append(f"| `{short}` | {f_:.0f} | {w_:.0f} | {rb / 1e6:.1f} MB | {wb / 1e6:.1f} MB |")
    meta = {"source_sha": kernel_source_sha(), "workload": workload,
            "fetch_factor": round(f_fetch, 4),
            "write_factor": round(f_write, 4),
            "units": {u: {k: round(v) for k, v in x.items()} for u, x in units.items()}}
    lines += ["", f"Calibration: the {copy_mib} MiB copy (`{ck}`) reads {cf[ck]:.0f} KiB and writes "
              f"{cw[ck]:.0f} KiB by the counters, so FETCH_SIZE is scaled by {f_fetch:.3f} and "
              f"WRITE_SIZE by {f_write:.3f}.", ""]
    for u, x in units.items():
        lines.append(f"- `{u}` per call: {x['read_bytes'] / 1e6:.1f} MB read + "
                     f"{x['write_bytes'] / 1e6:.1f} MB written between L2 and the memory fabric "
                     f"(HBM or the MALL)")
    lines += ["", f"<!-- {TRAFFIC_TAG} {json.dumps(meta)} -->"]
    return "\n".join(lines)


def load_traffic(unit, workload, profiles_dir=None):
    """HBM bytes per call of `unit` on `workload` from a committed counter
    summary, or None when none was taken on this workload with the current
    kernel sources."""
    sha = kernel_source_sha()
    pdir = profiles_dir or os.path.join(ROOT, "profiles")
    for path in sorted(glob.glob(os.path.join(pdir, "*.md"))):
        with open(path) as f:
            text = f.read()
        m = re.search(re.escape(TRAFFIC_TAG) + r"\s*(\{.*\})\s*-->", text)
        if not m:
            continue
        meta = json.loads(m.group(1))
        if (meta.get("source_sha") == sha and meta.get("workload") == workload
                and unit in meta.get("units", {})):
            x = meta["units"][unit]
            return int(x["read_bytes"] + x["write_bytes"]), os.path.relpath(path, ROOT)
    return None, None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-headline", action="store_true")
    ap.add_argument("--fwd-only", action="store_true",
                    help="time fa_fwd alone on the workload (profiling aid)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="instead of attention, time a plain device copy of this many MiB "
                         "(calibrates the HBM byte counters)")
    ap.add_argument("--summarize-pmc", default=None,
                    help="print the HBM traffic summary of the rocprofv3 counter CSVs in DIR")
    ap.add_argument("--copy-mib", type=int, default=1024,
                    help="size of the calibration copy used with --summarize-pmc")
    ap.add_argument("--gemm-ref", action="store_true",
                    help="time torch.matmul (hipBLASLt) on bf16 8192^3 and 4096^3 for context")
    ap.add_argument("--std-sweep", action="store_true",
                    help="fused fa_fwd vs the standard unfused fa_fwd_standard, bf16 [1,16,N,64], "
                         "no mask, N = 1024..16384; prints a markdown table")
    ap.add_argument("--std-n", type=int, default=0, help="only this N in --std-sweep")
    ap.add_argument("--no-settle", action="store_true",
                    help="--std-sweep: skip the clock settle and the warm launches "
                         "(counter passes: only the flushed launches run)")
    ap.add_argument("--std-bwd", action="store_true",
                    help="--std-sweep: the backward pair instead (fused fa_bwd vs fa_bwd_standard, "
                         "which reads the P stored by fa_fwd_standard)")
    ap.add_argument("--summarize-std-bwd", default=None,
                    help="HBM bytes of the fused vs standard backward from per-N counter CSVs in DIR")
    ap.add_argument("--summarize-std", default=None,
                    help="HBM bytes of fused vs standard from the per-N counter CSVs in DIR")
    ap.add_argument("--km-sweep", action="store_true",
                    help="key-major fa_fwd_keymajor vs the query-major fa_fwd, bf16 [1,16,N,64], "
                         "no mask, N in {2048, 4096}, key blocks 32..256")
    ap.add_argument("--km-n", type=int, default=0, help="only this N in --km-sweep")
    ap.add_argument("--km-bc", type=int, default=0, help="only this key-block size in --km-sweep")
    ap.add_argument("--summarize-km", default=None,
                    help="HBM bytes of the key-major forward per block size from counter CSVs in DIR")
    ap.add_argument("--summarize-util", default=None,
                    help="summarize unit-utilization counter passes (MfmaUtil, VALUBusy, LdsUtil, "
                         "...) in DIR per kernel (no GPU)")
    ap.add_argument("--tile-sweep", action="store_true",
                    help="every forward kernel shape (fa_fwd_tuned cfg 0..8) on the causal "
                         "[2,16,8192,128] and unmasked [4,16,2048,64] workloads; markdown table")
    ap.add_argument("--oracle-all", action="store_true",
                    help="time the CPU oracle (dense and tiled forward; dense backward where the "
                         "workload has one) on every workload of the statement; no GPU")
    ap.add_argument("--sweep", action="store_true",
                    help="time fa_fwd and fa_bwd over N = 2048..16384 (B = 32768/N, H = 16), "
                         "d in {64, 128}, mask in {none, causal}; prints a markdown table")
    args = ap.parse_args()
    if args.summarize_pmc:
        print(summarize_pmc(args.summarize_pmc, args.copy_mib,
                            args.workload or "bf16_causal_bwd_b2h16_n4096_d128"))
        return
    if args.summarize_std:
        print(summarize_std(args.summarize_std, args.copy_mib))
        return
    if args.summarize_std_bwd:
        print(summarize_std_bwd(args.summarize_std_bwd, args.copy_mib))
        return
    if args.summarize_km:
        print(summarize_km(args.summarize_km, args.copy_mib))
        return
    if args.summarize_util:
        print(summarize_util(args.summarize_util))
        return
    if args.oracle_all:
        print(oracle_all())
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: runs on one GPU only (heads shard across GPUs without "
              "communication, but no multi-GPU path is built); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import exact_tiled_attention_fwd_amd as fa
    from exact_tiled_attention_fwd_amd.synth import WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    fa._native.ensure_built()  # compiles only when no library is there
    fa.load()  # fail loudly if the HIP library is still missing
    dev = torch.device("cuda", 0)

    if args.copy_probe_mib:
        copy_probe(torch, dev, args)
        return
    if args.sweep:
        sweep(torch, fa, dev, args)
        return
    if args.tile_sweep:
        tile_sweep(torch, fa, dev, args)
        return
    if args.gemm_ref:
        gemm_ref(torch, dev)
        return
    if args.std_sweep and args.std_bwd:
        std_bwd_sweep(torch, fa, dev, args)
        return
    if args.std_sweep:
        std_sweep(torch, fa, dev, args)
        return
    if args.km_sweep:
        km_sweep(torch, fa, dev, args)
        return

    have_bwd = not args.fwd_only
    name = args.workload or "bf16_causal_bwd_b2h16_n4096_d128"
    w = WORKLOADS[name]
    inp = make_inputs(w, with_dout=True)
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "dout"))
    B, H, N, d = w.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, d, q.dtype), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def fwd():
        fa.fa_fwd(q, k, v, o, lse, w.scale, w.mask, w.window, stream)

    def bwd():
        fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, w.scale, w.mask, w.window, stream)

    def step():
        fwd()
        if have_bwd:
            bwd()

    CLOCK_SETTLE_S = 0.3

    def settle(fn):
        """Run fn back to back for CLOCK_SETTLE_S seconds: the shader clock
        ramps up over the first tens of milliseconds of load after an idle
        spell (e.g. host-side input generation), and the W warm-up steps
        alone are too short for that."""
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < CLOCK_SETTLE_S:
            for _ in range(8):
                fn()
            torch.cuda.synchronize()

    def timed(fn, reps):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s.record(stream)
        for _ in range(reps):
            fn()
        e.record(stream)
        torch.cuda.synchronize()
        return s.elapsed_time(e) / reps  # ms

    if not args.no_headline:  # headline inputs first: no idle gap between timed sections
        hw = WORKLOADS["bf16_causal_b2h16_n8192_d128"]
        hin = make_inputs(hw)
        hq, hk, hv = (hin[n].to(dev) for n in ("q", "k", "v"))
        ho = torch.empty_like(hq)
        hl = torch.empty(hq.shape[:-1], dtype=torch.float32, device=dev)
        del hin

    peaks = measured_peaks(torch, fa, dev, stream)
    settle(step)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms_step = timed(step, args.steps)
    wall = time.perf_counter() - t0
    flops_step = fwd_flops(w) + (bwd_flops(w) if have_bwd else 0.0)
    value = flops_step / (ms_step * 1e-3) / 1e12

    # per-kernel-unit launch durations over the same number of launches
    ms_fwd = timed(fwd, args.steps)
    kernels = {"fa_fwd": (ms_fwd, fwd_flops(w), fwd_bytes(w))}
    if have_bwd:
        ms_bwd = timed(bwd, args.steps)
        kernels["fa_bwd"] = (ms_bwd, bwd_flops(w), bwd_bytes(w))
    dom = max(kernels, key=lambda n: kernels[n][0])
    ms_dom, fl_dom, by_dom = kernels[dom]
    achieved = fl_dom / (ms_dom * 1e-3) / 1e12
    traffic, traffic_src = load_traffic(dom, w.name)
    # which roof binds: arithmetic intensity against the ridge of the published peaks
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    if fl_dom / by_dom >= ridge:
        bound, unit, peak, pk_meas = "mfma", "TFLOP/s", PEAK_BF16_TFLOPS, peaks["mfma_bf16_tflops"]
    else:
        achieved = by_dom / (ms_dom * 1e-3) / 1e9
        bound, unit, peak, pk_meas = "hbm", "GB/s", PEAK_HBM_GBS, peaks["hbm_copy_gbs"]
    roofline = {"bound": bound, "achieved": round(achieved, 1), "peak": peak,
                "unit": unit, "frac": round(achieved / peak, 4),
                "traffic": traffic, "traffic_unit": "bytes per call", "traffic_source": traffic_src,
                "traffic_counts": "bytes between L2 and the memory fabric (FETCH_SIZE + WRITE_SIZE, "
                                  "scaled by a device copy of known size); the 256 MB MALL behind "
                                  "the fabric may serve part of them, so they bound HBM bytes "
                                  "from above",
                "algorithmic_bytes_per_launch": by_dom, "kernel": dom,
                "arithmetic_intensity": round(fl_dom / by_dom, 1),
                "peak_measured": round(pk_meas, 1),
                "frac_of_measured": round(achieved / pk_meas, 4),
                "algorithmic_flop_per_launch": fl_dom,
                "avg_launch_us": round(ms_dom * 1e3, 2)}

    out = {
        "metric": "attention fwd/bwd TFLOP/s (bf16) + % of MI355X MFMA peak, N=2k-16k",
        "value": round(value, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded torch.randn, bf16-rounded)",
        "config": {"workload": name, "batch": B, "heads": H, "seq_len": N, "head_dim": d,
                   "mask": w.mask, "window": w.window if w.mask == "local" else None,
                   "step": "fa_fwd + fa_bwd" if have_bwd else "fa_fwd",
                   "pct_of_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
                   "fwd_tflops": round(fwd_flops(w) / (ms_fwd * 1e-3) / 1e12, 1),
                   "bwd_tflops": round(bwd_flops(w) / (kernels["fa_bwd"][0] * 1e-3) / 1e12, 1)
                   if have_bwd else None,
                   "wall_s_timed": round(wall, 3),
                   "clock_settle_s": CLOCK_SETTLE_S},
        "roofline": roofline,
        "probes": {k_: round(v_, 1) for k_, v_ in peaks.items()},
    }

    # The same step with cold caches: each of K launches follows a 512 MiB
    # device write that evicts L2 and the 256 MB MALL; median of the K.
    flush_buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    ms_step_fl = flushed_median(torch, step, stream, flush_buf, args.steps)
    out["flushed"] = {"ms_per_step_median": round(ms_step_fl, 4),
                      "tflops": round(flops_step / (ms_step_fl * 1e-3) / 1e12, 1),
                      "reps": args.steps, "flush_bytes": FLUSH_BYTES}

    if not args.no_headline:
        def hfwd():
            fa.fa_fwd(hq, hk, hv, ho, hl, hw.scale, hw.mask, hw.window, stream)
        settle(hfwd)
        for _ in range(args.warmup):
            hfwd()
        hms = timed(hfwd, args.steps)
        ht = fwd_flops(hw) / (hms * 1e-3) / 1e12
        hms_fl = flushed_median(torch, hfwd, stream, flush_buf, args.steps)
        ht_fl = fwd_flops(hw) / (hms_fl * 1e-3) / 1e12
        out["headline_forward"] = {
            "workload": hw.name, "tflops": round(ht, 1),
            "frac_of_peak": round(ht / PEAK_BF16_TFLOPS, 4), "avg_launch_us": round(hms * 1e3, 2),
            "hbm_gbs": round(fwd_bytes(hw) / (hms * 1e-3) / 1e9, 1),
            "flushed_median_us": round(hms_fl * 1e3, 2), "flushed_tflops": round(ht_fl, 1),
            "flushed_frac_of_peak": round(ht_fl / PEAK_BF16_TFLOPS, 4)}
        del hq, hk, hv, ho, hl
    del flush_buf

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, inp, have_bwd)

    print(json.dumps(out), flush=True)


FLUSH_BYTES = 512 << 20  # larger than L2 plus the 256 MB MALL


def flushed_median(torch, fn, stream, flush_buf, reps):
    """Median milliseconds of `reps` launches of fn, each preceded by a write
    of flush_buf (outside the timed span) so that fn starts with cold caches;
    events on the launch stream around fn only."""
    times = []
    for i in range(reps):
        flush_buf.fill_(i & 255)
        s_, e_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s_.record(stream)
        fn()
        e_.record(stream)
        e_.synchronize()
        times.append(s_.elapsed_time(e_))
    return statistics.median(times)


def measured_peaks(torch, fa, dev, stream):
    """The library's roofline probes, best of three runs each: sustained
    bf16 MFMA TFLOP/s of register-operand MFMAs on every compute unit, and
    HBM GB/s of a 1 GiB device copy (read + write)."""
    mf = max(fa.fa_probe_mfma_bf16(100000, stream) for _ in range(3))
    src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    cp = max(fa.fa_probe_copy(src, dst, 10, stream) for _ in range(3))
    del src, dst
    return {"mfma_bf16_tflops": mf, "hbm_copy_gbs": cp}


def sweep(torch, fa, dev, args):
    """fa_fwd and fa_bwd over N = 2048..16384 with B = 32768/N and H = 16,
    d in {64, 128}, mask in {none, causal}. Inputs are N(0,1) bf16 drawn on
    the device (seeded; timing only, no parity). Each entry point first runs
    back to back for 0.1 s (clock settle); 'warm' is the mean of K launches
    back to back, 'flushed' the median of K launches each preceded by a
    512 MiB device write that evicts L2 and the 256 MB MALL."""
    stream = torch.cuda.current_stream(dev)
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    reps = max(args.steps, 5)
    peaks = measured_peaks(torch, fa, dev, stream)
    print(f"Measured ceilings: bf16 MFMA {peaks['mfma_bf16_tflops']:.0f} TFLOP/s, "
          f"HBM copy {peaks['hbm_copy_gbs']:.0f} GB/s.\n")
    print("| d | mask | N | B | unit | flushed µs | warm µs | TFLOP/s (flushed) | % of 2516.6 | "
          "% of measured | HBM GB/s (algorithmic bytes, flushed) |")
    print("|---|---|---|---|---|---|---|---|---|---|---|")

    def one(fn):
        s_, e_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s_.record(stream)
        fn()
        e_.record(stream)
        e_.synchronize()
        return s_.elapsed_time(e_)

    for d in (64, 128):
        for mask in ("none", "causal"):
            for N in (2048, 4096, 8192, 16384):
                B, H = 32768 // N, 16
                g = torch.Generator(device=dev).manual_seed(7919 * N + d)
                q, k, v, do = (torch.randn(B, H, N, d, generator=g, device=dev).to(torch.bfloat16)
                               for _ in range(4))
                o = torch.empty_like(q)
                lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
                dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
                ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, d, q.dtype), dtype=torch.uint8,
                                 device=dev)
                scale = d ** -0.5
                w = types.SimpleNamespace(shape=(B, H, N, d), mask=mask, window=0, dtype="bf16")
                units = (("fa_fwd", lambda: fa.fa_fwd(q, k, v, o, lse, scale, mask, 0, stream),
                          fwd_flops(w), fwd_bytes(w)),
                         ("fa_bwd", lambda: fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, scale,
                                                      mask, 0, stream),
                          bwd_flops(w), bwd_bytes(w)))
                units[0][1]()  # O and LSE for the backward
                for name, fn, flops, nbytes in units:
                    torch.cuda.synchronize()
                    t0 = time.perf_counter()
                    while time.perf_counter() - t0 < 0.1:
                        fn()
                        torch.cuda.synchronize()
                    s_, e_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    s_.record(stream)
                    for _ in range(reps):
                        fn()
                    e_.record(stream)
                    e_.synchronize()
                    warm = s_.elapsed_time(e_) / reps
                    fl = []
                    for i in range(reps):
                        scratch.fill_(i & 255)
                        fl.append(one(fn))
                    ms = statistics.median(fl)
                    tf = flops / (ms * 1e-3) / 1e12
                    print(f"| {d} | {mask} | {N} | {B} | {name} | {ms * 1e3:.1f} | {warm * 1e3:.1f} | "
                          f"{tf:.1f} | {100 * tf / PEAK_BF16_TFLOPS:.1f} | "
                          f"{100 * tf / peaks['mfma_bf16_tflops']:.1f} | "
                          f"{nbytes / (ms * 1e-3) / 1e9:.0f} |", flush=True)
                del q, k, v, do, o, lse, dq, dk, dv, ws


# Forward kernel shapes of fa_fwd_tuned (include/fa_tuning.h), per head dim:
# (cfg, query rows per wave x waves, keys per tile, kernel). cfg 5 and 6 at
# d = 128 are the default again and are not repeated.
TILE_CFGS = {
    128: [(0, "32 x 8", 128, "tile (default)"), (1, "32 x 8", 64, "tile"),
          (2, "32 x 8", 128, "block-pipelined"), (3, "32 x 8", 64, "block-pipelined"),
          (4, "32 x 4", 64, "tile"), (7, "32 x 4", 160, "tile, derived B_c and B_r"),
          (8, "32 x 8", 160, "block-pipelined, derived B_c")],
    64: [(0, "64 x 8", 64, "tile, two blocks per wave (default)"), (1, "32 x 8", 64, "tile"),
         (2, "32 x 8", 128, "block-pipelined"), (3, "32 x 8", 128, "tile"),
         (4, "32 x 4", 64, "tile"), (5, "32 x 8", 64, "block-pipelined"),
         (6, "64 x 4", 64, "tile, two blocks per wave"),
         (7, "32 x 2", 320, "tile, derived B_c and B_r"),
         (8, "32 x 8", 320, "block-pipelined, derived B_c")],
}


def tile_sweep(torch, fa, dev, args):
    """Every forward kernel shape on the causal [2,16,8192,128] workload and
    the unmasked [4,16,2048,64] one (seeded inputs of those workloads): each
    shape runs back to back for 0.2 s (clock settle), then K launches timed
    with events on the launch stream. Under rocprofv3 --kernel-trace each
    shape is a kernel of its own name, so the trace gives the same table."""
    from exact_tiled_attention_fwd_amd.synth import WORKLOADS, make_inputs
    stream = torch.cuda.current_stream(dev)
    reps = max(args.steps, 5)
    print("| workload | cfg | rows per wave x waves | keys per tile | kernel | µs | TFLOP/s | "
          "% of 2516.6 |")
    print("|---|---|---|---|---|---|---|---|")
    for name in ("bf16_causal_b2h16_n8192_d128", "bf16_b4h16_n2048_d64"):
        w = WORKLOADS[name]
        inp = make_inputs(w)
        q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev)
        for cfg, rows, bc, kern in TILE_CFGS[w.d]:
            fn = lambda: fa.fa_fwd_tuned(q, k, v, o, lse, w.scale, w.mask, w.window, cfg, stream)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            while time.perf_counter() - t0 < 0.2:
                fn()
                torch.cuda.synchronize()
            s_, e_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s_.record(stream)
            for _ in range(reps):
                fn()
            e_.record(stream)
            e_.synchronize()
            ms = s_.elapsed_time(e_) / reps
            tf = fwd_flops(w) / (ms * 1e-3) / 1e12
            print(f"| {name} | {cfg} | {rows} | {bc} | {kern} | {ms * 1e3:.1f} | {tf:.1f} | "
                  f"{100 * tf / PEAK_BF16_TFLOPS:.1f} |", flush=True)
        del q, k, v, o, lse


def time_unit(torch, fn, stream, scratch, reps, settle=True):
    """(flushed, warm) milliseconds of fn: 'flushed' is the median of `reps`
    launches each preceded by a write of `scratch` (evicting L2 and the
    MALL), event-timed around the launch only; 'warm' the mean of `reps`
    launches back to back after 0.1 s of them (clock settle), NaN when
    settle is False (counter passes run only the flushed launches)."""
    warm = float("nan")
    if settle:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.1:
            fn()
            torch.cuda.synchronize()
        s_, e_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s_.record(stream)
        for _ in range(reps):
            fn()
        e_.record(stream)
        e_.synchronize()
        warm = s_.elapsed_time(e_) / reps
    fl = []
    for i in range(reps):
        scratch.fill_(i & 255)
        s_, e_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s_.record(stream)
        fn()
        e_.record(stream)
        e_.synchronize()
        fl.append(s_.elapsed_time(e_))
    return statistics.median(fl), warm


STD_NS = (1024, 2048, 4096, 8192, 16384)


def std_bytes(N, B=1, H=16, d=64):
    """Algorithmic HBM bytes of the two forwards at bf16 [B,H,N,d]: the fused
    one reads Q, K, V and writes O, LSE; the standard one also writes S
    (float32) and reads it back, writes P (bf16) and reads it back."""
    fused = 4 * B * H * N * d * 2 + B * H * N * 4
    return fused, fused + B * H * N * N * (4 + 4 + 2 + 2)


def std_sweep(torch, fa, dev, args):
    """Time the fused forward and the standard (unfused) one on the notes'
    setting (d = 64, no mask), B = 1, H = 16, N = 1024..16384 (or --std-n).
    'flushed': median of launches each preceded by a 512 MiB device write
    (evicts L2 and the 256 MB MALL); 'warm': mean of launches back to back
    after a 0.1 s clock settle."""
    stream = torch.cuda.current_stream(dev)
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    reps = max(args.steps, 3)
    print("| N | fused flushed µs | fused warm µs | standard flushed µs | standard warm µs | "
          "standard / fused (flushed) | fused bytes (MB) | standard bytes (MB) | "
          "standard workspace (GB) |")
    print("|---|---|---|---|---|---|---|---|---|")
    B, H, d = 1, 16, 64
    for N in ([args.std_n] if args.std_n else STD_NS):
        g = torch.Generator(device=dev).manual_seed(104729 + N)
        q, k, v = (torch.randn(B, H, N, d, generator=g, device=dev).to(torch.bfloat16)
                   for _ in range(3))
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        wsb = fa.fa_fwd_standard_workspace_bytes(B, H, N, d, q.dtype)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
        units = (lambda: fa.fa_fwd(q, k, v, o, lse, 0.125, "none", 0, stream),
                 lambda: fa.fa_fwd_standard(q, k, v, o, lse, ws, 0.125, "none", 0, stream))
        res = [time_unit(torch, fn, stream, scratch, reps, not args.no_settle) for fn in units]
        fb, sb = std_bytes(N, B, H, d)
        (ff, fw), (sf, sw) = res
        print(f"| {N} | {ff * 1e3:.1f} | {fw * 1e3:.1f} | {sf * 1e3:.1f} | {sw * 1e3:.1f} | "
              f"{sf / ff:.2f} | {fb / 1e6:.1f} | {sb / 1e6:.1f} | {wsb / 1e9:.2f} |", flush=True)
        del q, k, v, o, lse, ws


def std_bwd_bytes(N, B=1, H=16, d=64):
    """Algorithmic HBM bytes of the two backwards at bf16 [B,H,N,d]. The
    fused one reads Q, K, V, O, dO and the LSE and writes dQ, dK, dV
    (bwd_bytes). The standard one reads Q, K, V, dO, writes dQ, dK, dV, and
    moves per (query, key) pair: P read twice (dV and dS steps, 2 x 2 B), dP
    written and read (2 x 4 B), dS written (2 B) and read twice (dQ and dK
    steps, 2 x 2 B): 18 B."""
    fused = 8 * B * H * N * d * 2 + B * H * N * 4
    std = 7 * B * H * N * d * 2 + B * H * N * N * 18
    return fused, std


def std_bwd_sweep(torch, fa, dev, args):
    """Time the fused backward (fa_bwd, recomputing P) and the standard one
    (fa_bwd_standard, reading the P that fa_fwd_standard stored) on the
    notes' setting (d = 64, no mask), B = 1, H = 16, N = 1024..16384 (or
    --std-n); flushed and warm as in std_sweep."""
    stream = torch.cuda.current_stream(dev)
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    reps = max(args.steps, 3)
    print("| N | fused bwd flushed µs | fused bwd warm µs | standard bwd flushed µs | "
          "standard bwd warm µs | standard / fused (flushed) | fused bytes (MB) | "
          "standard bytes (MB) |")
    print("|---|---|---|---|---|---|---|---|")
    B, H, d = 1, 16, 64
    for N in ([args.std_n] if args.std_n else STD_NS):
        g = torch.Generator(device=dev).manual_seed(104729 + N)
        q, k, v, do = (torch.randn(B, H, N, d, generator=g, device=dev).to(torch.bfloat16)
                       for _ in range(4))
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        wsf = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, d, q.dtype), dtype=torch.uint8,
                          device=dev)
        fws = torch.empty(fa.fa_fwd_standard_workspace_bytes(B, H, N, d, q.dtype),
                          dtype=torch.uint8, device=dev)
        bws = torch.empty(fa.fa_bwd_standard_workspace_bytes(B, H, N, d, q.dtype),
                          dtype=torch.uint8, device=dev)
        fa.fa_fwd_standard(q, k, v, o, lse, fws, 0.125, "none", 0, stream)  # P for the standard bwd
        fa.fa_fwd(q, k, v, o, lse, 0.125, "none", 0, stream)                # O, LSE for the fused
        units = (lambda: fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, wsf, 0.125, "none", 0, stream),
                 lambda: fa.fa_bwd_standard(q, k, v, do, fws, dq, dk, dv, bws, 0.125, stream))
        res = [time_unit(torch, fn, stream, scratch, reps, not args.no_settle) for fn in units]
        fb, sb = std_bwd_bytes(N, B, H, d)
        (ff, fw), (sf, sw) = res
        print(f"| {N} | {ff * 1e3:.1f} | {fw * 1e3:.1f} | {sf * 1e3:.1f} | {sw * 1e3:.1f} | "
              f"{sf / ff:.2f} | {fb / 1e6:.1f} | {sb / 1e6:.1f} |", flush=True)
        del q, k, v, do, o, lse, dq, dk, dv, wsf, fws, bws


def _pmc_median_per_dispatch(path, counter):
    """Median over dispatches of one counter, per kernel name (KiB), with the
    number of dispatches."""
    per = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            key = (r["Kernel_Name"], r["Dispatch_Id"])
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (name, _), v in per.items():
        out.setdefault(name, []).append(v)
    return {n: (statistics.median(v), len(v)) for n, v in out.items()}


def summarize_std_bwd(d, copy_mib):
    """Measured HBM bytes per call of the fused and the standard backward for
    each N whose counter CSVs are in d (bfetch_N<n>_*, bwrite_N<n>_*, plus the
    copy calibration), against std_bwd_bytes(). Each kernel counts with the
    median over its dispatches (the one-off forwards that set up P, O and LSE
    are dispatched once, the backwards several times), times its dispatches
    per call (two for the transposed product: dV and dK)."""
    one = lambda pat: sorted(glob.glob(os.path.join(d, pat)))[0]
    cf = _pmc_per_dispatch(one("copy_fetch*_counter_collection.csv"), "FETCH_SIZE")
    cw = _pmc_per_dispatch(one("copy_write*_counter_collection.csv"), "WRITE_SIZE")
    ck = [n for n in cf if "copy" in n.lower()][0]
    nbytes = copy_mib * (1 << 20)
    f_fetch, f_write = nbytes / (cf[ck] * 1024.0), nbytes / (cw[ck] * 1024.0)
    per_call = {"bwd_dq": 1, "bwd_dkdv": 1, "std_scores": 1, "std_xty": 2, "std_ds": 1,
                "std_pv_kernel<64, false>": 1, "std_pv_kernel<128, false>": 1}
    lines = ["| N | kernel | read MB per dispatch | written MB per dispatch | dispatches per call |",
             "|---|---|---|---|---|"]
    totals = []
    for N in STD_NS:
        fp = glob.glob(os.path.join(d, f"bfetch_N{N}_counter_collection.csv"))
        wp = glob.glob(os.path.join(d, f"bwrite_N{N}_counter_collection.csv"))
        if not fp or not wp:
            continue
        fe = _pmc_median_per_dispatch(fp[0], "FETCH_SIZE")
        wr = _pmc_median_per_dispatch(wp[0], "WRITE_SIZE")
        sums = {"fused": 0.0, "standard": 0.0}
        for name in sorted(fe):
            short = re.sub(r"\(.*", "", name).replace("void ", "")
            key = next((k_ for k_ in per_call if k_ in short), None)
            if key is None:
                continue
            unit = "fused" if key.startswith("bwd_") else "standard"
            rb = fe[name][0] * 1024.0 * f_fetch
            wb = wr.get(name, (0.0, 0))[0] * 1024.0 * f_write
            sums[unit] += (rb + wb) * per_call[key]
            lines.append(f"| {N} | `{short}` | {rb / 1e6:.1f} | {wb / 1e6:.1f} | {per_call[key]} |")
        totals.append((N, sums))
    lines += ["", "| N | fused bwd MB (algorithmic) | standard bwd MB (algorithmic) | "
              "standard / fused bytes |", "|---|---|---|---|"]
    for N, sums in totals:
        fb, sb = std_bwd_bytes(N)
        lines.append(f"| {N} | {sums['fused'] / 1e6:.1f} ({fb / 1e6:.1f}) | "
                     f"{sums['standard'] / 1e6:.1f} ({sb / 1e6:.1f}) | "
                     f"{sums['standard'] / max(sums['fused'], 1.0):.1f} |")
    lines += ["", f"Calibration: FETCH_SIZE x {f_fetch:.3f}, WRITE_SIZE x {f_write:.3f} "
              f"(a {copy_mib} MiB copy through `{ck}`)."]
    return "\n".join(lines)


def summarize_std(d, copy_mib):
    """Measured HBM bytes per call of the fused and the standard forward for
    each N whose counter CSVs are in d (fetch_N<n>_*, write_N<n>_*, plus the
    copy calibration copy_fetch*, copy_write*), against the algorithmic
    bytes of std_bytes()."""
    one = lambda pat: sorted(glob.glob(os.path.join(d, pat)))[0]
    cf = _pmc_per_dispatch(one("copy_fetch*_counter_collection.csv"), "FETCH_SIZE")
    cw = _pmc_per_dispatch(one("copy_write*_counter_collection.csv"), "WRITE_SIZE")
    ck = [n for n in cf if "copy" in n.lower()][0]
    nbytes = copy_mib * (1 << 20)
    f_fetch, f_write = nbytes / (cf[ck] * 1024.0), nbytes / (cw[ck] * 1024.0)
    lines = ["| N | kernel | read MB | written MB |", "|---|---|---|---|"]
    totals = []
    for N in STD_NS:
        fp = glob.glob(os.path.join(d, f"fetch_N{N}_counter_collection.csv"))
        wp = glob.glob(os.path.join(d, f"write_N{N}_counter_collection.csv"))
        if not fp or not wp:
            continue
        fe, wr = _pmc_per_dispatch(fp[0], "FETCH_SIZE"), _pmc_per_dispatch(wp[0], "WRITE_SIZE")
        sums = {"fused": [0.0, 0.0], "standard": [0.0, 0.0]}
        for name in sorted(fe):
            unit = "standard" if "std_" in name else "fused" if "fwd_bf16" in name else None
            if unit is None:
                continue
            rb, wb = fe[name] * 1024.0 * f_fetch, wr.get(name, 0.0) * 1024.0 * f_write
            sums[unit][0] += rb
            sums[unit][1] += wb
            lines.append(f"| {N} | `{re.sub(r'[(<].*', '', name)}` | {rb / 1e6:.1f} | {wb / 1e6:.1f} |")
        totals.append((N, sums))
    lines += ["", "| N | fused read+write MB (algorithmic) | standard read+write MB (algorithmic) | "
              "standard / fused bytes |", "|---|---|---|---|"]
    for N, sums in totals:
        fb, sb = std_bytes(N)
        fm, sm = sum(sums["fused"]), sum(sums["standard"])
        lines.append(f"| {N} | {fm / 1e6:.1f} ({fb / 1e6:.1f}) | {sm / 1e6:.1f} ({sb / 1e6:.1f}) | "
                     f"{sm / fm:.1f} |")
    lines += ["", f"Calibration: FETCH_SIZE x {f_fetch:.3f}, WRITE_SIZE x {f_write:.3f} "
              f"(a {copy_mib} MiB copy through `{ck}`)."]
    return "\n".join(lines)


KM_NS = (2048, 4096)
KM_BCS = (32, 64, 128, 256)


def km_bytes(N, bc, B=1, H=16, d=64):
    """Model of the key-major forward's device-memory bytes at bf16 [B,H,N,d]:
    each of the T_c = ceil(N/bc) launches reads all of Q and reads and writes
    the running state of every row (two lanes x (d/2 + 3) floats); K and V
    are read once per head and launch (L2 serves the other workgroups); the
    finalize pass reads the state once more and writes O and LSE."""
    tc = -(-N // bc)
    rows = B * H * (-(-N // 256)) * 256
    state = rows * 2 * (d // 2 + 3) * 4
    per_launch = B * H * N * d * 2 + 2 * state + B * H * bc * d * 2 * 2
    return state + tc * per_launch + state + B * H * N * (d * 2 + 4)


def km_sweep(torch, fa, dev, args):
    """The key-major forward (outer loop over key blocks, state through
    device memory) against the query-major fa_fwd on bf16 [1, 16, N, 64]
    without a mask: time and modelled bytes per key-block size."""
    stream = torch.cuda.current_stream(dev)
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    reps = max(args.steps, 3)
    print("| N | order | key block B_c | launches | flushed µs | warm µs | modelled bytes (MB) |")
    print("|---|---|---|---|---|---|---|")
    B, H, d = 1, 16, 64
    for N in ([args.km_n] if args.km_n else KM_NS):
        g = torch.Generator(device=dev).manual_seed(130363 + N)
        q, k, v = (torch.randn(B, H, N, d, generator=g, device=dev).to(torch.bfloat16)
                   for _ in range(3))
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        ws = torch.empty(fa.fa_fwd_keymajor_workspace_bytes(B, H, N, d, q.dtype), dtype=torch.uint8,
                         device=dev)
        if not args.km_bc:
            f, w = time_unit(torch, lambda: fa.fa_fwd(q, k, v, o, lse, 0.125, "none", 0, stream),
                             stream, scratch, reps, not args.no_settle)
            fb, _ = std_bytes(N, B, H, d)
            print(f"| {N} | query-major (fa_fwd) | — | 1 | {f * 1e3:.1f} | {w * 1e3:.1f} | "
                  f"{fb / 1e6:.1f} |", flush=True)
        for bc in ([args.km_bc] if args.km_bc else KM_BCS):
            f, w = time_unit(torch, lambda: fa.fa_fwd_keymajor(q, k, v, o, lse, ws, 0.125, "none",
                                                               0, bc, stream),
                             stream, scratch, reps, not args.no_settle)
            print(f"| {N} | key-major | {bc} | {-(-N // bc) + 2} | {f * 1e3:.1f} | {w * 1e3:.1f} | "
                  f"{km_bytes(N, bc, B, H, d) / 1e6:.1f} |", flush=True)
        del q, k, v, o, lse, ws


def summarize_km(d, copy_mib):
    """Measured device-memory bytes of one key-major forward per (N, B_c)
    from counter CSVs fetch_N<n>_bc<b>_*, write_N<n>_bc<b>_* (summed over
    the init, step and finalize launches of one call), against km_bytes()."""
    one = lambda pat: sorted(glob.glob(os.path.join(d, pat)))[0]
    cf = _pmc_per_dispatch(one("copy_fetch*_counter_collection.csv"), "FETCH_SIZE")
    cw = _pmc_per_dispatch(one("copy_write*_counter_collection.csv"), "WRITE_SIZE")
    ck = [n for n in cf if "copy" in n.lower()][0]
    nbytes = copy_mib * (1 << 20)
    f_fetch, f_write = nbytes / (cf[ck] * 1024.0), nbytes / (cw[ck] * 1024.0)

    def per_call(path, counter):
        """Per call: sum over one call's dispatches of the km_* kernels
        (calls are identical, so total / number of finalize launches)."""
        tot, calls = 0.0, 0
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter or "km_" not in r["Kernel_Name"]:
                    continue
                tot += float(r["Counter_Value"])
                calls += "finalize" in r["Kernel_Name"]
        return tot / max(calls, 1)

    lines = ["| N | B_c | measured read MB | measured written MB | measured total MB | modelled MB |",
             "|---|---|---|---|---|---|"]
    pts = []
    for N in KM_NS:
        for bc in KM_BCS:
            fp = glob.glob(os.path.join(d, f"fetch_N{N}_bc{bc}_counter_collection.csv"))
            wp = glob.glob(os.path.join(d, f"write_N{N}_bc{bc}_counter_collection.csv"))
            if not fp or not wp:
                continue
            rb = per_call(fp[0], "FETCH_SIZE") * 1024.0 * f_fetch
            wb = per_call(wp[0], "WRITE_SIZE") * 1024.0 * f_write
            pts.append((N, bc, rb + wb))
            lines.append(f"| {N} | {bc} | {rb / 1e6:.1f} | {wb / 1e6:.1f} | {(rb + wb) / 1e6:.1f} | "
                         f"{km_bytes(N, bc) / 1e6:.1f} |")
    # bytes ~ a + b * N^2 / B_c at fixed d: least squares over the points
    if len(pts) >= 3:
        xs = [N * N / bc for N, bc, _ in pts]
        ys = [y for _, _, y in pts]
        n = len(xs)
        mx, my = sum(xs) / n, sum(ys) / n
        b = sum((x - mx) * (y - my) for x, y in zip(xs, ys)) / sum((x - mx) ** 2 for x in xs)
        a = my - b * mx
        ss = sum((y - my) ** 2 for y in ys)
        r2 = 1 - sum((y - (a + b * x)) ** 2 for x, y in zip(xs, ys)) / ss if ss > 0 else 1.0
        lines += ["", f"Least-squares fit bytes = a + b * N^2 / B_c: a = {a / 1e6:.1f} MB, "
                  f"b = {b:.1f} bytes, R^2 = {r2:.4f}."]
    lines += ["", f"Calibration: FETCH_SIZE x {f_fetch:.3f}, WRITE_SIZE x {f_write:.3f} "
              f"(a {copy_mib} MiB copy through `{ck}`)."]
    return "\n".join(lines)


def summarize_util(d):
    """Per attention kernel, the mean over its dispatches of every counter
    or derived metric found in the counter CSVs of directory d (one column
    per counter, passes merged)."""
    vals = {}
    for path in sorted(glob.glob(os.path.join(d, "*_counter_collection.csv"))):
        per = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                name = re.sub(r"\(.*", "", r["Kernel_Name"]).replace("void ", "")
                if "fa::" not in name or "probe" in name:
                    continue
                key = (name, r["Counter_Name"], r["Dispatch_Id"])
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
        for (name, ctr, _), v in per.items():
            vals.setdefault(name, {}).setdefault(ctr, []).append(v)
    ctrs = sorted({c for x in vals.values() for c in x})
    lines = ["| Kernel | dispatches | " + " | ".join(ctrs) + " |",
             "|---|---|" + "---|" * len(ctrs)]
    for name in sorted(vals):
        x = vals[name]
        n = max(len(v) for v in x.values())
        cells = []
        for c in ctrs:
            v = x.get(c)
            cells.append("—" if not v else (f"{sum(v) / len(v):.4g}"))
        lines.append(f"| `{name}` | {n} | " + " | ".join(cells) + " |")
    return "\n".join(lines)


def gemm_ref(torch, dev):
    """The vendor library's dense bf16 GEMM (torch.matmul -> hipBLASLt) on
    square shapes: context for what a plain contraction sustains on this card."""
    out = {}
    for n in (4096, 8192):
        a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
        b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.3:  # clock settle
            a @ b
            torch.cuda.synchronize()
        reps = 20
        s_, e_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s_.record()
        for _ in range(reps):
            a @ b
        e_.record()
        e_.synchronize()
        ms = s_.elapsed_time(e_) / reps
        out[f"bf16_gemm_{n}^3_tflops"] = round(2.0 * n ** 3 / (ms * 1e-3) / 1e12, 1)
    print(json.dumps(out), flush=True)


def copy_probe(torch, dev, args):
    """A plain device-to-device copy of known size: its FETCH_SIZE and
    WRITE_SIZE counters give the factor that turns counter readings into
    bytes."""
    n = args.copy_probe_mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(args.steps):
        dst.copy_(src)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / args.steps
    print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n,
                      "launches": args.steps + args.warmup, "avg_ms": round(ms, 4),
                      "gbs": round(2 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)


def cpu_model():
    """The host CPU's model name (first 'model name' of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def omp_threads():
    """Threads the OpenMP oracle runs with: OMP_NUM_THREADS when set, else
    the CPUs this process may run on."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        return int(env)
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_baseline(w, inp, have_bwd, target_s=12.0):
    """The CPU oracle (plain double C, OpenMP), as the tests use it, on
    consecutive (batch, head) slices of the same workload until about
    target_s seconds of CPU work: per slice the dense forward, the tiled
    online forward (128 x 128 tiles) and, when the step has a backward, the
    dense backward. `value` is the dense forward + dense backward rate, the
    oracle's counterpart of the GPU step."""
    import oracle
    B, H, N, d = w.shape
    flat = {n: inp[n].reshape(B * H, N, d) for n in ("q", "k", "v", "dout")}
    one = type(w)(**{**w.__dict__, "B": 1, "H": 1})
    t_dense = t_tiled = t_bwd = 0.0
    t0 = time.perf_counter()
    n = 0
    while n < B * H and (n == 0 or (time.perf_counter() - t0) < target_s):
        sl = {k_: t[n:n + 1] for k_, t in flat.items()}
        a = time.perf_counter()
        oracle.fwd_dense(sl["q"], sl["k"], sl["v"], w.scale, w.mask, w.window)
        b = time.perf_counter()
        oracle.fwd_tiled(sl["q"], sl["k"], sl["v"], w.scale, 128, 128, w.mask, w.window)
        c = time.perf_counter()
        if have_bwd:
            oracle.bwd_dense(sl["q"], sl["k"], sl["v"], sl["dout"], w.scale, w.mask, w.window)
        t_dense += b - a
        t_tiled += c - b
        t_bwd += time.perf_counter() - c
        n += 1
    ff, fb = fwd_flops(one) * n, (bwd_flops(one) * n if have_bwd else 0.0)
    return {"value": round((ff + fb) / (t_dense + t_bwd) / 1e12, 6), "unit": "TFLOP/s",
            "cores": omp_threads(), "kind": "oracle", "cpu_model": cpu_model(),
            "seconds": round(t_dense + t_tiled + t_bwd, 2),
            "dense_fwd_s": round(t_dense, 6), "dense_fwd_tflops": round(ff / t_dense / 1e12, 6),
            "tiled_fwd_s": round(t_tiled, 6), "tiled_fwd_tflops": round(ff / t_tiled / 1e12, 6),
            "dense_bwd_s": round(t_bwd, 6) if have_bwd else None,
            "dense_bwd_tflops": round(fb / t_bwd / 1e12, 6) if have_bwd else None,
            "sample": f"{n} of {B * H} (b,h) slices [1,1,{N},{d}] of {w.name}: dense forward"
                      + (" + dense backward" if have_bwd else "")
                      + " (value); tiled forward 128x128 timed beside; float64, OpenMP"}


# The five workloads of the statement, in its order (c1 .. c5).
STATEMENT_WORKLOADS = ("toy_fp32_n6_d4", "bf16_b4h16_n2048_d64", "bf16_causal_b2h16_n8192_d128",
                       "bf16_local128_x8_b1h32_n16384_d128", "bf16_causal_bwd_b2h16_n4096_d128")


def oracle_all(target_s=6.0):
    """The CPU oracle as it stands on every workload of the statement: per
    workload, consecutive (batch, head) slices until about target_s seconds,
    each through the dense forward, the tiled online forward (128 x 128 tiles;
    2 x 2 on the 6-row toy) and, where the workload has a backward, the dense
    backward. Rates use the bench's FLOP formulas; the whole-workload time is
    the per-slice mean times the slice count. Markdown on stdout."""
    import oracle
    from exact_tiled_attention_fwd_amd.synth import WORKLOADS, make_inputs
    out = [f"Host: {cpu_model()}; {os.cpu_count()} CPUs visible; the oracle ran with "
           f"{omp_threads()} OpenMP threads.", "",
           "| Config | Workload | Slices timed | Dense fwd s/slice | Dense fwd GFLOP/s "
           "| Tiled fwd s/slice | Tiled fwd GFLOP/s | Dense bwd s/slice | Dense bwd GFLOP/s "
           "| Whole workload (dense), s |",
           "|---|---|---|---|---|---|---|---|---|---|"]
    toy = make_inputs(WORKLOADS["toy_fp32_n6_d4"])  # first call loads the library: untimed
    oracle.fwd_dense(toy["q"], toy["k"], toy["v"], 0.5, "none", 0)
    for ci, name in enumerate(STATEMENT_WORKLOADS, 1):
        w = WORKLOADS[name]
        has_bwd = name == "bf16_causal_bwd_b2h16_n4096_d128"
        inp = make_inputs(w, with_dout=has_bwd)
        B, H, N, d = w.shape
        keys = ("q", "k", "v", "dout") if has_bwd else ("q", "k", "v")
        flat = {k_: inp[k_].reshape(B * H, N, d) for k_ in keys}
        one = type(w)(**{**w.__dict__, "B": 1, "H": 1})
        tile = 128 if N >= 128 else 2
        td = tt = tb = 0.0
        n = 0
        t0 = time.perf_counter()
        while n < B * H and (n == 0 or time.perf_counter() - t0 < target_s):
            sl = {k_: t[n:n + 1] for k_, t in flat.items()}
            a = time.perf_counter()
            oracle.fwd_dense(sl["q"], sl["k"], sl["v"], w.scale, w.mask, w.window)
            b = time.perf_counter()
            oracle.fwd_tiled(sl["q"], sl["k"], sl["v"], w.scale, tile, tile, w.mask, w.window)
            c = time.perf_counter()
            if has_bwd:
                oracle.bwd_dense(sl["q"], sl["k"], sl["v"], sl["dout"], w.scale, w.mask, w.window)
            td += b - a
            tt += c - b
            tb += time.perf_counter() - c
            n += 1
        ff, fb = fwd_flops(one), bwd_flops(one)
        g = lambda flop, t: f"{flop * n / t / 1e9:.2f}" if t > 0 else "—"
        bwd_cols = (f"{tb / n:.4g} | {g(fb, tb)}" if has_bwd else "— | —")
        whole = (td + tb) / n * B * H
        out.append(f"| c{ci} | `{name}` | {n} of {B * H} | {td / n:.4g} | {g(ff, td)} | "
                   f"{tt / n:.4g} ({tile}×{tile}) | {g(ff, tt)} | {bwd_cols} | {whole:.4g} |")
    return "\n".join(out)


if __name__ == "__main__":
    main()

"""Benchmark of the W8A8 linear hot path on one MI355X.

A step is one pass of the int W8A8 linear forward on the headline shape
(X bf16 [4096, 3072], W [12288, 3072] int8 tensor-wise, bias [12288]):
row-wise act-quant of X, then the int8 GEMM with the fused dequant epilogue
writing bf16 Y.  Weight quantization is done once per weight before timing
(frozen weights).  Inputs live in HBM before the timed region; R buffer sets
(X, Xq, sx, Wq, Y) are rotated so that every step reads cold HBM rather than
the 256 MB Infinity Cache.

Printed: one JSON line with the step throughput (TOPS over the whole step),
the GEMM kernel's roofline (int8 MFMA dense peak 5.0 POPS), the act-quant
kernel's HBM rate, per-row figures of the other paths (fp8 train step, DiT
shapes, SVDQuant, Q8_0) and the CPU oracle timed on a bounded sample.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0     # MI355X dense int8 MFMA, 5.0 POPS
PEAK_FP8_TFLOPS = 5000.0    # dense fp8 MFMA
PEAK_HBM_GBS = 8000.0       # HBM3E 8 TB/s
PEAK_VALU_LANE_TOPS = 39.32  # non-packed f32 VALU lane operations: 256 CU x 4 SIMD x 16 lanes x 2.4 GHz
M, K, N = 4096, 3072, 12288
ROTATE = 4       # buffer sets of the step (4 x 150 MB, past the 256 MB Infinity Cache)
AQ_ROTATE = 16   # buffer sets of the act-quant timing (16 x 38 MB: every launch reads cold HBM)
AQ_ITERS = 200


def _args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    # Under this load the GPU settles at a power-limited clock after ~30 ms of
    # work; shorter warm-ups time the ramp (launch times swing by +-20% there).
    p.add_argument("--steps", type=int, default=400)
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-rows", action="store_true", help="skip the per-row figures of the other paths")
    p.add_argument("--cpu-rows", type=int, default=512,
                   help="rows of the one-thread oracle sample (about 7 s of one CPU core)")
    p.add_argument("--cpu-rows-all", type=int, default=M,
                   help="rows of the all-thread oracle sample")
    p.add_argument("--settle-ms", type=float, default=100.0,
                   help="untimed steps for at least this long before the warm-up steps (the GPU's clock ramps "
                        "under a sustained load for ~30 ms)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also run one plain 512 MiB device copy (reference for HBM byte counters)")
    return p.parse_args()


def _bf16(t_bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(t_bits).view(np.int16)).view(torch.bfloat16).cuda()


def _time_launches(fn, iters, warmup, prefill=False):
    """Average duration (ms) of fn(i) over iters launches, HIP events on the
    current stream (the stream the library launches on).

    prefill: for kernels about as short as the Python call that launches them
    (~8 us), the launches are queued behind a short GPU spin first, so that the
    GPU runs them back to back instead of waiting for the host."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if prefill:
        torch.cuda._sleep(1_000_000 + 50_000 * iters)   # ~25 us of spin per queued launch
    e0.record()
    for i in range(iters):
        fn(i)
    e1.record()
    e1.synchronize()
    return e0.elapsed_time(e1) / iters


def _code_only(text):
    """C++ source without comments and with whitespace collapsed: a comment
    edit leaves the hash of the kernel's code unchanged (string literals with
    comment markers do not occur in these files)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def _kernel_hash():
    """Hash of the GEMM's code (gemm.hip and the headers it includes from the
    library), stored with the counter summaries in profiles/."""
    h = hashlib.sha256()
    for f in ("gemm.hip", "common.hpp", "internal.hpp"):
        with open(os.path.join(ROOT, "w8a8_quantized_linear_quant_amd", "csrc", f)) as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def _traffic_from_profile(kernel_hash):
    """L2-to-fabric bytes per GEMM launch (FETCH_SIZE + WRITE_SIZE, calibrated)
    from the committed rocprofv3 counter summary,
    if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "gemm_int8_M4096_N12288_K3072_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_hash") != kernel_hash:
        return None
    try:
        return float(vals["l2_fabric_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def measured_peaks(w8, torch, a_codes, b_codes):
    """Ceilings measured on this GPU: the sustained int8 MFMA rate on fragments
    of the given codes (TOPS) and the bandwidth of a plain device copy (GB/s)."""
    pairs = 16384                       # ~10 ms per probe launch
    cus = w8.library().w8a8_probe_sink_count() // 256
    ops = pairs * 32 * 2 * 32 ** 3 * 4 * cus
    sink = w8.probe_mfma_i8(a_codes, b_codes, pairs)
    w8.probe_mfma_i8(a_codes, b_codes, pairs, sink=sink)
    ms = _time_launches(lambda i: w8.probe_mfma_i8(a_codes, b_codes, pairs, sink=sink), 3, 1)
    mfma_tops = ops / (ms * 1e-3) / 1e12
    src = torch.empty(1 << 29, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    ms_copy = _time_launches(lambda i: dst.copy_(src), 5, 2)
    copy_gbs = 2.0 * src.numel() / (ms_copy * 1e-3) / 1e9
    del src, dst
    return round(mfma_tops, 1), round(copy_gbs, 1)


def copy_same_bytes(torch, nbytes):
    """Time (ms) of a plain device-to-device copy moving `nbytes` in all (half
    read, half written), over enough buffer pairs that every launch misses
    the 256 MB Infinity Cache, timed like the rows: the streaming rate a kernel
    moving that many bytes can expect (short transfers do not reach the rate
    of a long copy)."""
    half = max(16, int(nbytes // 2) // 16 * 16)
    sets = max(2, int(np.ceil(600e6 / (2.0 * half))))
    bufs = [(torch.empty(half, dtype=torch.uint8, device="cuda").fill_(1),
             torch.empty(half, dtype=torch.uint8, device="cuda")) for _ in range(sets)]
    ms = _time_row(lambda i: bufs[i % sets][1].copy_(bufs[i % sets][0]))
    del bufs
    return ms


def cpu_baseline(x_bits, w_bits, b_bits, rows, rows_all):
    """The oracle (plain C) on the same workload, scaled to TOPS of the linear:
    act-quant + int8 linear of the first `rows` rows on one thread, then of
    the first `rows_all` rows split into row slices over all host threads
    (a thread pool calling the oracle's C functions, which release the GIL;
    the oracle's arithmetic is untouched).  The weight quantization is timed
    apart (once per frozen weight)."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    t0 = time.perf_counter()
    wq, _, sw = oracle.quant_weight_tensorwise(oracle.INT8, w_bits)
    t1 = time.perf_counter()

    def run(lo, hi):
        xq, sx = oracle.quant_act_rowwise(oracle.INT8, x_bits[lo:hi])
        oracle.linear(oracle.INT8, xq, sx, wq, sw, b_bits)

    run(0, rows)
    t2 = time.perf_counter()
    threads = _host_threads()
    step = -(-rows_all // threads)
    with ThreadPoolExecutor(max_workers=threads) as ex:
        t3 = time.perf_counter()
        list(ex.map(lambda i: run(i, min(i + step, rows_all)), range(0, rows_all, step)))
        t4 = time.perf_counter()
    one = 2.0 * rows * N * K / (t2 - t1) / 1e12
    allc = 2.0 * rows_all * N * K / (t4 - t3) / 1e12
    return {"value": round(allc, 6), "unit": "TOPS", "cores": threads, "kind": "oracle",
            "sample": f"act-quant + int8 linear of the first {rows_all} of {M} rows ({rows_all}x{N}x{K}) in "
                      f"{threads} row slices on {threads} threads; weight quant ({N}x{K}, one thread) timed "
                      f"apart: {t1 - t0:.2f} s",
            "seconds": round(t4 - t3, 2),
            "single_thread": {"value": round(one, 6), "unit": "TOPS", "cores": 1, "seconds": round(t2 - t1, 2),
                              "sample": f"first {rows} rows ({rows}x{N}x{K})"},
            "host_cpu": _host_cpu(), "host_threads": os.cpu_count()}


def _host_threads():
    """Threads the CPU baseline may use: the process's CPU affinity, else
    os.cpu_count(), capped by OMP_NUM_THREADS where that is set (the host
    share the process was given)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def _host_cpu():
    """The host CPU's model name (Linux /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    args = _args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path is single-GPU "
              "and multi-GPU sharding is a design note, not a measured configuration.", file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads
    import w8a8_quantized_linear_quant_amd as w8

    torch.cuda.init()
    d = workloads.svdq()
    x_bits, r_bits, b_bits = d["x"], d["r"], d["bias"]
    print(f"[bench] inputs ready: X {x_bits.shape}, W {r_bits.shape}", file=sys.stderr, flush=True)

    # R rotating buffer sets; the weight is quantized once per set (amortized).
    sets = []
    x0, w0, bias = _bf16(x_bits), _bf16(r_bits), _bf16(b_bits)
    for i in range(ROTATE):
        xi = x0 if i == 0 else x0.clone()
        wq, _, sw = w8.w8a8_quant_weight_tensorwise(w0 if i == 0 else w0.clone())
        sets.append({
            "x": xi, "wq": wq, "sw": sw, "bias": bias.clone(),
            "xq": torch.empty((M, K), dtype=torch.int8, device="cuda"),
            "sx": torch.empty(M, dtype=torch.float32, device="cuda"),
            "y": torch.empty((M, N), dtype=torch.bfloat16, device="cuda"),
        })
    torch.cuda.synchronize()

    def act_quant(i):
        s = sets[i % ROTATE]
        w8.w8a8_quant_act_rowwise(s["x"], out=s["xq"], scale=s["sx"])

    def gemm(i):
        s = sets[i % ROTATE]
        w8.w8a8_linear(s["xq"], s["sx"], s["wq"], s["sw"], s["bias"], out=s["y"])

    def step(i):
        act_quant(i)
        gemm(i)

    # ---- the timed steps.  The GPU's clock ramps for ~30 ms under a sustained
    # load and again after an idle pause: steps run untimed until settle_ms
    # of them have passed, then the W warm-up steps, then the K timed ones.
    settle_steps = 0
    if args.settle_ms > 0:
        es0, es1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        es0.record()
        while True:
            for _ in range(10):
                step(settle_steps)
                settle_steps += 1
            es1.record()
            es1.synchronize()
            if es0.elapsed_time(es1) >= args.settle_ms:
                break
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    ms_step = e0.elapsed_time(e1) / args.steps
    ops = 2.0 * M * N * K
    tops = ops / (ms_step * 1e-3) / 1e12
    print(f"[bench] step {ms_step * 1e3:.1f} us ({t_wall:.2f} s wall for {args.steps} steps)", file=sys.stderr,
          flush=True)

    # ---- per-kernel averages (same launches, timed apart); the act-quant
    # kernel on its own input sets, enough of them that each launch reads cold HBM
    iters = max(args.steps, 20)
    ms_gemm = _time_launches(gemm, iters, 100)
    each = np.array(_time_each(gemm, iters)) * 1e3
    spread = {"us_p10": round(float(np.percentile(each, 10)), 2), "us_median": round(float(np.median(each)), 2),
              "us_p90": round(float(np.percentile(each, 90)), 2)}
    aq_sets = [(sets[0]["x"].clone(), torch.empty((M, K), dtype=torch.int8, device="cuda"),
                torch.empty(M, dtype=torch.float32, device="cuda")) for _ in range(AQ_ROTATE)]

    def act_quant_cold(i):
        xa, qa, sa = aq_sets[i % AQ_ROTATE]
        w8.w8a8_quant_act_rowwise(xa, out=qa, scale=sa)

    ms_aq = _time_launches(act_quant_cold, AQ_ITERS, 2 * AQ_ROTATE, prefill=True)
    del aq_sets
    gemm_tops = ops / (ms_gemm * 1e-3) / 1e12
    aq_bytes = 2.0 * M * K + M * K + 4.0 * M
    aq_gbs = aq_bytes / (ms_aq * 1e-3) / 1e9
    khash = _kernel_hash()
    roofline = {"bound": "mfma", "achieved": round(gemm_tops, 1), "peak": PEAK_INT8_TOPS, "unit": "TOPS",
                "frac": round(gemm_tops / PEAK_INT8_TOPS, 4), "traffic": _traffic_from_profile(khash),
                "traffic_counts": "L2-to-fabric bytes per launch (FETCH_SIZE + WRITE_SIZE): L2 misses, "
                                  "including those the Infinity Cache serves, not HBM bytes alone",
                "kernel": "gemm_kernel<int8, bf16 epilogue>", "us_per_launch": round(ms_gemm * 1e3, 2),
                "algorithmic_ops_per_launch": ops, "kernel_source_hash": khash, **spread}
    act = {"bound": "hbm", "achieved": round(aq_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
           "frac": round(aq_gbs / PEAK_HBM_GBS, 4), "us_per_launch": round(ms_aq * 1e3, 2),
           "algorithmic_bytes_per_launch": aq_bytes, "kernel": "act_quant_rowwise_kernel<int8>",
           "launches": AQ_ITERS, "buffer_sets": AQ_ROTATE}
    # the same rates against ceilings measured here, in the same power state
    mfma_tops, copy_gbs = measured_peaks(w8, torch, sets[0]["xq"], sets[0]["wq"])
    roofline.update(measured_peak=mfma_tops, frac_of_measured_peak=round(gemm_tops / mfma_tops, 4),
                    measured_peak_how="int8 MFMA loop (v_mfma_i32_16x16x64_i8, the GEMM's instruction, one wave per SIMD, all CUs) "
                                      "on fragments of this step's activation and weight codes")
    act.update(measured_peak=copy_gbs, frac_of_measured_peak=round(aq_gbs / copy_gbs, 4),
               measured_peak_how="device-to-device copy of 512 MiB, read + write bytes")
    ms_copy = copy_same_bytes(torch, aq_bytes)
    act.update(copy_same_bytes_us=round(ms_copy * 1e3, 2), copy_same_bytes_GBs=round(aq_bytes / ms_copy / 1e6, 1),
               frac_of_same_size_copy=round(ms_copy / ms_aq, 4))

    if args.calibrate_copy:
        src = torch.empty(1 << 29, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    rows = {} if args.no_rows else other_rows(w8, torch, workloads, args)
    svdq_row = rows.get("svdq_linear_M4096_K3072_N12288_r32")
    if svdq_row:
        # the SVDQuant linear against the plain step timed above (act-quant +
        # product of the same shape): the low-rank branch's share of the time
        svdq_row["plain_step_us"] = round(ms_step * 1e3, 1)
        svdq_row["over_plain_step"] = round(svdq_row["us"] / (ms_step * 1e3) - 1.0, 4)
    for s in sets:
        s.clear()
    torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        cpu = cpu_baseline(x_bits, r_bits, b_bits, args.cpu_rows, args.cpu_rows_all)

    out = {
        "metric": "W8A8 linear TOPS (M4096 K3072 N12288) + act-quant GB/s, % of roofline",
        "value": round(tops, 1), "unit": "TOPS", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int8", "data": "synthetic (seeded numpy PCG64, transformer-shaped; no dataset)",
        "config": {"workload": "int W8A8 linear forward: row-wise act-quant X[4096,3072] bf16 + int8 GEMM "
                               "vs W[12288,3072] (tensor-wise) + dequant/bias epilogue -> bf16 Y",
                   "M": M, "K": K, "N": N, "bias": True, "rotating_buffer_sets": ROTATE,
                   "settle_steps": settle_steps, "settle_ms": args.settle_ms},
        "roofline": roofline,
        "act_quant": act,
        "cpu_baseline": cpu,
        "rows": rows,
    }
    print(json.dumps(out), flush=True)


def _time_each(fn, iters):
    """Per-launch durations (ms) of fn(i), an event pair around every launch."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for i, (a, b) in enumerate(ev):
        a.record()
        fn(i)
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def _time_row(fn, settle_ms=30.0, span_ms=30.0):
    """_time_launches sized by time: ~settle_ms of untimed launches (the clock
    settles under load), then launches covering ~span_ms; short kernels are
    queued behind a spin (prefill)."""
    est = _time_launches(fn, 2, 1)
    warm = max(3, int(settle_ms / est))
    iters = min(2000, max(10, int(span_ms / est)))
    return _time_launches(fn, iters, warm, prefill=est < 0.04)


def other_rows(w8, torch, workloads, args):
    """Per-kernel figures of the other hot-path rows (not part of `value`)."""
    res = {}
    # tensor-wise weight quantization of W [12288, 3072] (one-time per frozen
    # weight): the max pass and the code pass read W twice and write the codes;
    # 4 weight copies (302 MB) rotate past the 256 MB Infinity Cache
    d = workloads.svdq()
    w0 = _bf16(d["r"])
    wsets = [(w0 if j == 0 else w0.clone(), torch.empty((N, K), dtype=torch.int8, device="cuda"),
              torch.empty(4, dtype=torch.float32, device="cuda"),
              torch.empty(w8.w8a8_weight_workspace_bytes(N, K), dtype=torch.uint8, device="cuda")) for j in range(4)]
    ms = _time_row(lambda i: w8.w8a8_quant_weight_tensorwise(wsets[i % 4][0], out=wsets[i % 4][1],
                                                               scale=wsets[i % 4][2], workspace=wsets[i % 4][3]))
    res["weight_quant_int8_N12288_K3072"] = {"us": round(ms * 1e3, 1),
                                             "GB/s": round((2 * 2.0 * N * K + N * K) / ms / 1e6, 1)}
    del w0, wsets
    # SVDQuant at the headline shape, r = 32
    x, l1, l2, rr, b = (_bf16(d[k]) for k in ("x", "l1", "l2", "r", "bias"))
    rq, _, sr = w8.w8a8_quant_weight_tensorwise(rr)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
    sx = torch.empty(M, dtype=torch.float32, device="cuda")
    ws = torch.empty(w8.svdq_workspace_bytes(M, 32), dtype=torch.uint8, device="cuda")
    ms = _time_row(lambda i: w8.svdq_linear(x, rq, sr, l1, l2, b, out=y, xq_out=xq, x_scale_out=sx,
                                                 workspace=ws))
    ops = 2.0 * M * N * K + 2.0 * M * K * 32 + 2.0 * M * 32 * N
    res["svdq_linear_M4096_K3072_N12288_r32"] = {"us": round(ms * 1e3, 1), "TOPS": round(ops / ms / 1e9, 1)}
    del x, l1, l2, rr, b, rq, y, xq, ws
    # DiT shapes
    d = workloads.dit()
    x = _bf16(d["x"])
    xq, sx = w8.w8a8_quant_act_rowwise(x)
    for name, wk, bk in (("dit_M4608_K3072_N3072", "w1", "b1"), ("dit_M4608_K3072_N12288", "w2", "b2")):
        wq, _, sw = w8.w8a8_quant_weight_tensorwise(_bf16(d[wk]))
        bb = _bf16(d[bk])
        nn = wq.shape[0]
        y = torch.empty((4608, nn), dtype=torch.bfloat16, device="cuda")
        ms = _time_row(lambda i: w8.w8a8_linear(xq, sx, wq, sw, bb, out=y))
        res[name] = {"us": round(ms * 1e3, 1), "TOPS": round(2.0 * 4608 * nn * 3072 / ms / 1e9, 1)}
    # act-quant of the DiT X [4608, 3072] (int8), 16 cold buffer sets
    aq = [(x if j == 0 else x.clone(), torch.empty((4608, K), dtype=torch.int8, device="cuda"),
           torch.empty(4608, dtype=torch.float32, device="cuda")) for j in range(AQ_ROTATE)]
    ms = _time_row(lambda i: w8.w8a8_quant_act_rowwise(aq[i % AQ_ROTATE][0], out=aq[i % AQ_ROTATE][1],
                                                       scale=aq[i % AQ_ROTATE][2]))
    res["act_quant_int8_X4608x3072"] = {"us": round(ms * 1e3, 1), "GB/s": round((3.0 * 4608 * K + 4 * 4608) / ms / 1e6, 1)}
    del x, xq, y, aq
    # fp8 train step shapes
    d = workloads.fp8_step()
    wq, wqt, sw = w8.w8a8_quant_weight_tensorwise(_bf16(d["w"]), qtype=w8.FP8_E4M3, transposed=True)
    x = _bf16(d["x"])
    # act-quant of the forward X [8192, 3072] (e4m3), 8 cold buffer sets of 75.5 MB
    aq = [(x if j == 0 else x.clone(), torch.empty((8192, K), dtype=torch.float8_e4m3fn, device="cuda"),
           torch.empty(8192, dtype=torch.float32, device="cuda")) for j in range(8)]
    ms = _time_row(lambda i: w8.w8a8_quant_act_rowwise(aq[i % 8][0], qtype=w8.FP8_E4M3, out=aq[i % 8][1],
                                                       scale=aq[i % 8][2]))
    res["act_quant_fp8_X8192x3072"] = {"us": round(ms * 1e3, 1), "GB/s": round((3.0 * 8192 * K + 4 * 8192) / ms / 1e6, 1)}
    del aq
    xq, sx = w8.w8a8_quant_act_rowwise(x, qtype=w8.FP8_E4M3)
    y = torch.empty((8192, N), dtype=torch.bfloat16, device="cuda")
    ms = _time_row(lambda i: w8.w8a8_linear(xq, sx, wq, sw, out=y))
    res["fp8_fwd_M8192_K3072_N12288"] = {"us": round(ms * 1e3, 1),
                                         "TFLOPS": round(2.0 * 8192 * N * K / ms / 1e9, 1)}
    dy = _bf16(d["dy"])
    dyq = torch.empty((8192, N), dtype=torch.float8_e4m3fn, device="cuda")
    sdy = torch.empty(8192, dtype=torch.float32, device="cuda")
    ms = _time_row(lambda i: w8.w8a8_quant_act_rowwise(dy, qtype=w8.FP8_E4M3, out=dyq, scale=sdy))
    bytes_ = 3.0 * 8192 * N + 4 * 8192
    res["act_quant_fp8_dY_8192x12288"] = {"us": round(ms * 1e3, 1), "GB/s": round(bytes_ / ms / 1e6, 1)}
    dx = torch.empty((8192, K), dtype=torch.bfloat16, device="cuda")
    ms = _time_row(lambda i: w8.w8a8_linear_backward_dx(dyq, sdy, wqt, sw, out=dx))
    res["fp8_bwd_dx_M8192_N12288_K3072"] = {"us": round(ms * 1e3, 1),
                                            "TFLOPS": round(2.0 * 8192 * N * K / ms / 1e9, 1)}
    # the int8 analogue of the train step's dX
    wq8, wqt8, sw8 = w8.w8a8_quant_weight_tensorwise(_bf16(d["w"]), qtype=w8.INT8, transposed=True)
    dyq8, sdy8 = w8.w8a8_quant_act_rowwise(dy, qtype=w8.INT8)
    ms = _time_row(lambda i: w8.w8a8_linear_backward_dx(dyq8, sdy8, wqt8, sw8, out=dx))
    res["int8_bwd_dx_M8192_N12288_K3072"] = {"us": round(ms * 1e3, 1),
                                             "TOPS": round(2.0 * 8192 * N * K / ms / 1e9, 1)}
    del wq, wqt, x, xq, y, dy, dyq, dx, wq8, wqt8, dyq8
    # Q8_0 (8 buffer sets of 85 MB, 680 MB in all: every launch reads cold HBM,
    # not the 256 MB Infinity Cache)
    v0 = torch.from_numpy(workloads.q8_0_vector()).cuda()
    n = v0.numel()
    qs = [(v0 if j == 0 else v0.clone(), torch.empty(w8.q8_0_nbytes(n), dtype=torch.uint8, device="cuda"),
           torch.empty(n, dtype=torch.float32, device="cuda")) for j in range(8)]
    ms = _time_row(lambda i: w8.q8_0_quantize(qs[i % 8][0], out=qs[i % 8][1]))
    qbytes = 4.0 * n + w8.q8_0_nbytes(n)
    res["q8_0_quantize_n16777221"] = {"us": round(ms * 1e3, 1), "GB/s": round(qbytes / ms / 1e6, 1)}
    ms = _time_row(lambda i: w8.q8_0_dequantize(qs[i % 8][1], n, out=qs[i % 8][2]))
    res["q8_0_dequantize_n16777221"] = {
        "us": round(ms * 1e3, 1), "GB/s": round(qbytes / ms / 1e6, 1),
        "note": "reads are cold; its 67 MB of f32 output per launch is written back from the Infinity Cache "
                "(write-back) partly after the launch, so the rate is not a cold-HBM write rate"}
    del v0, qs
    # GGUF A8: Q8_0 weight [12288, 3072] -> per-channel int8 / e4m3, then the linear at the headline shape
    d = workloads.gguf()
    gb = torch.from_numpy(d["w_blocks"]).cuda()
    x = _bf16(d["x"])
    bb = _bf16(d["bias"])
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    gbs = [gb] + [gb.clone() for _ in range(3)]    # 4 x 78 MB moved per launch: cold HBM
    for qt, tag in ((w8.INT8, "int8"), (w8.FP8_E4M3, "fp8")):
        wqs = [torch.empty((N, K), dtype=torch.int8 if qt == w8.INT8 else torch.float8_e4m3fn, device="cuda")
               for _ in range(4)]
        sws = [torch.empty(N, dtype=torch.float32, device="cuda") for _ in range(4)]
        ms = _time_row(lambda i: w8.gguf_a8_requant_q8_0(gbs[i % 4], N, K, qtype=qt, out=wqs[i % 4], scale=sws[i % 4]))
        wq, sw = wqs[0], sws[0]
        rbytes = 1.0 * gb.numel() + N * K + 4.0 * N  # blocks read once, codes and scales written
        res[f"gguf_a8_requant_{tag}_N12288_K3072"] = {"us": round(ms * 1e3, 1), "GB/s": round(rbytes / ms / 1e6, 1)}
        xq, sx = w8.w8a8_quant_act_rowwise(x, qtype=qt)
        ms = _time_row(lambda i: w8.gguf_a8_linear(xq, sx, wq, sw, bb, out=y))
        res[f"gguf_a8_linear_{tag}_M4096_K3072_N12288"] = {"us": round(ms * 1e3, 1),
                                                           "TOPS": round(2.0 * M * N * K / ms / 1e9, 1)}
    # act-quant of the headline X with the Hadamard rotation fused (K = 3072: three 1024-blocks)
    d = workloads.svdq()
    xh0 = _bf16(d["x"])
    hs = [(xh0.clone(), torch.empty((M, K), dtype=torch.int8, device="cuda"),
           torch.empty(M, dtype=torch.float32, device="cuda")) for _ in range(AQ_ROTATE)]
    ms = _time_row(lambda i: w8.w8a8_quant_act_rowwise_hadamard(hs[i % AQ_ROTATE][0], out=hs[i % AQ_ROTATE][1],
                                                                scale=hs[i % AQ_ROTATE][2]))
    res["act_quant_hadamard_int8_X4096x3072"] = {"us": round(ms * 1e3, 1),
                                                 "GB/s": round((3.0 * M * K + 4 * M) / ms / 1e6, 1)}
    # its VALU side: M K (log2 b + 2) lane operations (the transform's sums and
    # differences, one absmax and one division per element) against plain f32
    # issue, 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz = 39.3 T lane-ops/s
    lane_ops = float(M * K * (10 + 2))
    res["act_quant_hadamard_int8_X4096x3072"]["alu"] = {
        "lane_ops_per_launch": lane_ops, "achieved_T_per_s": round(lane_ops / ms / 1e9, 2),
        "peak_T_per_s": PEAK_VALU_LANE_TOPS, "frac": round(lane_ops / ms / 1e9 / PEAK_VALU_LANE_TOPS, 4)}
    del xh0, hs
    # SVDQuant weight preparation of the SVDQuant workload's weight, r = 32, 2 power iterations
    d = workloads.svdq()
    l2p, l1p, rp = (torch.from_numpy(workloads.bf16_bits_to_f32(d[k])).double() for k in ("l2", "l1", "r"))
    wsv = (l2p @ l1p + rp).float().to(torch.bfloat16).cuda()
    del l2p, l1p, rp
    s = w8.svdq_prepare_subspace(32)
    om = _bf16(workloads.normal_bf16(np.random.default_rng(11), (s, K), 1.0))
    l1o = torch.empty((32, K), dtype=torch.bfloat16, device="cuda")
    l2o = torch.empty((N, 32), dtype=torch.bfloat16, device="cuda")
    ro = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
    so = torch.empty(32, dtype=torch.float32, device="cuda")
    ws = torch.empty(w8.svdq_prepare_workspace_bytes(N, K, 32), dtype=torch.uint8, device="cuda")
    ms = _time_launches(lambda i: w8.svdq_prepare(wsv, 32, om, iters=2, l1=l1o, l2=l2o, residual=ro, sigma=so,
                                                  workspace=ws), 5, 1)
    res["svdq_prepare_N12288_K3072_r32_iters2"] = {"us": round(ms * 1e3, 1)}
    torch.cuda.synchronize()
    # each row against its own roofline: dense 8-bit MFMA (int8 5.0 POPS, fp8
    # 5.0 PFLOP/s; the SVDQuant row's few bf16 flops are counted at that rate
    # too) or HBM (8 TB/s)
    for v in res.values():
        for unit, bound, peak in (("TOPS", "mfma", PEAK_INT8_TOPS), ("TFLOPS", "mfma", PEAK_FP8_TFLOPS),
                                  ("GB/s", "hbm", PEAK_HBM_GBS)):
            if unit in v:
                v.update(bound=bound, peak=peak, frac=round(v[unit] / peak, 4))
    # each HBM row beside a plain copy of its own algorithmic bytes
    for v in res.values():
        if "GB/s" in v:
            nbytes = v["GB/s"] * v["us"] * 1e3
            ms_copy = copy_same_bytes(torch, nbytes)
            v.update(copy_same_bytes_us=round(ms_copy * 1e3, 1), frac_of_same_size_copy=round(ms_copy * 1e3 / v["us"], 4))
    return res


if __name__ == "__main__":
    main()

"""Benchmark of the weight-only quantized GEMM on one MI355X.

A step is one pass of the decode workload the headline metric is quoted on: W4A16 with
fp16 activations, int4 weights in groups of 128 along K with fp16 scales, and the four
GEMMs M in {1, 16} x (N, K) in {(4096, 4096), (11008, 4096)}.  Every launch reads a
different copy of the packed weights (rotating copies, >= 512 MB per shape, more than the
256 MB last-level cache), so the weight stream comes from HBM.  The K timed steps are one
HIP-graph replay; `value` is the effective weight bandwidth (packed weight + scale bytes /
time) over them.

Also reported: a `roofline` object for the decode kernel; `secondary`, every other
workload shape timed the same way (rotating >= 512 MB of weight copies): the INT4 prefill
M = 4096 over the group-size sweep, the FP8 shapes (M = 1, 16, 8192 x 10240 x 5120,
32768 x 3200 x 5120, 16384 x 12800 x 5120), the FP4 shapes (M = 1, 128, 8192 x 8192 x 8192),
FP8 with fp16 activations and a bias (M = 1, 16, 8192 x 10240 x 5120) and the INT2 and NF4
shapes (M = 1, 16, 4096 x 4096 x 4096), each with TFLOP/s and weight GB/s as fractions of the MFMA and HBM peaks; the CPU oracle
timed on the host as `cpu_baseline`; `hbm_context`, a hand-written streaming-read kernel
(non-temporal 16-byte loads, no arithmetic) over the decode weight and scale byte counts
and over 2 GiB, the time a kernel needs just to read those bytes; `host_overhead`, host
time per qgemm_run call (validation, plan, launch); and `comparators`: on the decode
shapes, the vendor 16-bit GEMM (hipBLASLt through torch) on a resident 16-bit weight and
the cast-copy path (whole weight dequantized into HBM by torch ops, then that GEMM) --
context, not target.  `--all` adds comparators for the FP8 / FP4 shapes and the INT4 prefill.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--all] [--no-cpu]
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2516.6  # dense fp16/bf16 MFMA, published (no sparsity)
METRIC = "effective weight GB/s at M=1/16 and TFLOP/s at M=4096, % of MI355X roofline"

DECODE_SHAPES = [(1, 4096, 4096), (16, 4096, 4096), (1, 11008, 4096), (16, 11008, 4096)]
PREFILL_G = [32, 64, 128, 256]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def weight_bytes(fmt, N, K, G):
    if fmt == "int4":
        return N * K // 2 + (K // G) * N * 2
    if fmt == "int2":
        return N * K // 4 + (K // G) * N * 2
    if fmt == "nf4":                     # + the 256-byte code-book header of the scales
        return N * K // 2 + (K // G) * N * 2 + 256
    if fmt in ("fp8", "fp8h"):
        return N * K
    return N * K // 2 + N * K // 16


class Gemm:
    """One GEMM with rotating device copies of its packed weights."""

    def __init__(self, q, torch, fmt, M, N, K, G, key, min_rotate_bytes, with_bias=False):
        import synthetic
        self.fmt, self.M, self.N, self.K, self.G = fmt, M, N, K, G
        self.p = q.problem(M, N, K, fmt, group_size=G if fmt in q.GROUP_SCALED else None)
        pq = q.problem(1, N, K, fmt, group_size=G if fmt in q.GROUP_SCALED else None)
        w = synthetic.weights(N, K, 0.05 if fmt in ("fp8", "fp8h") else 0.02, key)
        codes, scales, alpha = q.quantize(pq, w)            # the library's own quantizer
        wpk, spk = q.pack(pq, codes, scales)
        self.wbytes = weight_bytes(fmt, N, K, G)
        assert self.wbytes == wpk.size + (0 if spk is None else spk.size)
        ncopies = max(2, -(-min_rotate_bytes // self.wbytes))
        w0 = torch.from_numpy(wpk).cuda()
        s0 = None if spk is None else torch.from_numpy(spk).cuda()
        self.w = [w0] + [w0.clone() for _ in range(ncopies - 1)]
        self.s = [s0] + [None if s0 is None else s0.clone() for _ in range(ncopies - 1)]
        self.alpha = torch.tensor([alpha], dtype=torch.float32, device="cuda")
        kind = "f16" if fmt in ("int4", "int2", "nf4", "fp8h") else "bf16"
        self.A = synthetic.activations(M, K, kind, key).cuda()
        odt = torch.float16 if kind == "f16" else torch.bfloat16
        self.out = torch.empty((M, N), dtype=odt, device="cuda")
        self.bias = synthetic.bias(N, kind, key).cuda() if with_bias else None
        self.ws = q.alloc_workspace(self.p)
        self.i = 0
        self.q = q
        self.label = (f"{fmt} M={M} N={N} K={K}" + (f" G={G}" if fmt in q.GROUP_SCALED else "")
                      + (" +bias" if with_bias else ""))

    def launch(self):
        c = self.i % len(self.w)
        self.i += 1
        self.q.run(self.p, self.A, self.w[c], self.s[c], None if self.fmt in self.q.GROUP_SCALED else self.alpha,
                   self.out, self.ws, bias=self.bias)

    @property
    def flops(self):
        return 2.0 * self.M * self.N * self.K


def measure(torch, g, n):
    """Graph of n launches of one GEMM (each on the next weight copy), timed over 3 replays
    after a warm one: time per launch, TFLOP/s and weight GB/s with their fractions of the
    MFMA and HBM peaks, and which of the two bounds the shape (the larger ideal time)."""
    gg = graph_of(torch, g.launch, n)
    us = time_graph(torch, gg, 3) * 1e3 / n
    del gg
    tf = g.flops / (us * 1e-6) / 1e12
    gbs = g.wbytes / (us * 1e-6) / 1e9
    t_mfma = g.flops / (MFMA_F16_PEAK_TFLOPS * 1e12)
    t_hbm = g.wbytes / (HBM_PEAK_GBS * 1e9)
    return {"gemm": g.label, "us_per_launch": round(us, 3), "TFLOPs": round(tf, 1),
            "frac_mfma": round(tf / MFMA_F16_PEAK_TFLOPS, 4), "weight_GBps": round(gbs, 1),
            "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "bound": "mfma" if t_mfma > t_hbm else "hbm",
            "frac_bound": round(max(t_mfma, t_hbm) / (us * 1e-6), 4), "weight_copies": len(g.w)}


def graph_of(torch, fn, n):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                          # one eager call on the side stream before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for _ in range(n):
            fn()
    torch.cuda.synchronize()
    return g


def time_graph(torch, g, reps=1):
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g.replay()                        # untimed: the first replay uploads the graph and first-touches buffers
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps        # ms


def _probe_lib():
    """The measurement helpers built next to libqgemm.so (streaming read, host time per call)."""
    import ctypes
    import weight_only_quantized_qgemm_amd as q
    lib = ctypes.CDLL(os.path.join(os.path.dirname(q.LIB_PATH), "libqgemm_probe.so"))
    vp, ll = ctypes.c_void_p, ctypes.c_longlong
    lib.qgemm_probe_stream.argtypes = [vp, ll, vp, ll, vp, ctypes.c_int, vp]
    lib.qgemm_probe_stream.restype = ctypes.c_int
    lib.qgemm_probe_stream_groups.argtypes = [ll, ctypes.c_int]
    lib.qgemm_probe_stream_groups.restype = ll
    lib.qgemm_probe_host_ns.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp, ctypes.c_int,
                                        ctypes.POINTER(ctypes.c_double)]
    lib.qgemm_probe_host_ns.restype = ctypes.c_int
    return lib


def hbm_context(torch, cases, rot_bytes):
    """Achievable-HBM context for the decode figures: a hand-written streaming-read kernel
    (non-temporal 16-byte loads, all of a thread's loads in flight before any is consumed,
    one XOR per workgroup stored) over rotating buffers of the given byte counts, graph-timed
    like the GEMMs.  cases: (label, weight bytes, scale bytes); with scale bytes > 0 the
    kernel reads a second buffer of that size in the same launch, like the decode kernel's
    scale stream.  Loads per thread U in {2, 4, 8} are each timed and the fastest is
    reported.  GB/s counts the bytes read."""
    lib = _probe_lib()
    stream = torch.cuda.current_stream().cuda_stream
    res = []
    for label, wbytes, sbytes in cases:
        nbytes = wbytes + sbytes
        ncopies = max(2, -(-rot_bytes // nbytes))
        src = [torch.ones(wbytes // 8, dtype=torch.int64, device="cuda") for _ in range(ncopies)]
        sc = [torch.ones(max(sbytes, 16) // 8, dtype=torch.int64, device="cuda") for _ in range(ncopies)]
        sink = torch.empty(int(lib.qgemm_probe_stream_groups(wbytes // 16, 1)) + 64, dtype=torch.int32,
                           device="cuda")
        best = None
        for U in (2, 4, 8):
            i = [0]

            def fn():
                c = i[0] % ncopies
                i[0] += 1
                st = lib.qgemm_probe_stream(src[c].data_ptr(), wbytes, sc[c].data_ptr() if sbytes else None,
                                            sbytes, sink.data_ptr(), U, torch.cuda.current_stream().cuda_stream)
                assert st == 0, f"streaming probe failed: {st}"
            n = 8 if nbytes > (256 << 20) else 64
            gg = graph_of(torch, fn, n)
            us = time_graph(torch, gg, 3) * 1e3 / n
            del gg
            if best is None or us < best[0]:
                best = (us, U)
        res.append({"case": label, "bytes": nbytes, "weight_bytes": wbytes, "scale_bytes": sbytes,
                    "stream_us": round(best[0], 3), "loads_per_thread": best[1],
                    "read_GBps": round(nbytes / (best[0] * 1e-6) / 1e9, 1)})
        del src, sc, sink
        torch.cuda.empty_cache()
    del stream
    return res


def host_overhead(q, torch, gemms, iters=2000):
    """Host microseconds per call, measured in C (no Python overhead): qgemm_workspace_bytes
    (validation + launch plan) and qgemm_run (validation, plan and the kernel launch)."""
    import ctypes
    lib = _probe_lib()
    rows = []
    for g in gemms:
        ns = (ctypes.c_double * 2)()
        alpha = None if g.fmt in q.GROUP_SCALED else g.alpha.data_ptr()
        ws = None if g.ws is None else g.ws.data_ptr()
        wsb = 0 if g.ws is None else g.ws.numel()
        n = iters if g.M <= 16 else 20
        st = lib.qgemm_probe_host_ns(ctypes.addressof(g.p), g.A.data_ptr(), g.w[0].data_ptr(),
                                     None if g.s[0] is None else g.s[0].data_ptr(), alpha, g.out.data_ptr(),
                                     ws, wsb, torch.cuda.current_stream().cuda_stream, n, ns)
        torch.cuda.synchronize()
        assert st == 0, q.last_error()
        rows.append({"gemm": g.label, "validate_plan_us": round(ns[0] / 1e3, 3),
                     "qgemm_run_us": round(ns[1] / 1e3, 3), "calls": n})
    return rows


def comparator_row(q, torch, fmt, M, N, K, G, key, rot_bytes, qgemm_us):
    """Vendor paths on one shape, timed like the library (graphs over rotating copies):
    the 16-bit GEMM on a resident 16-bit weight, and the cast-copy path (dequantize the whole
    weight into HBM, then the same GEMM).  qgemm_us is the library's time on the shape."""
    import comparators
    import synthetic
    pq = q.problem(1, N, K, fmt, group_size=G if fmt in q.GROUP_SCALED else None)
    w = synthetic.weights(N, K, 0.05 if fmt in ("fp8", "fp8h") else 0.02, key)
    codes, scales, alpha = q.quantize(pq, w)
    cbytes = codes.nbytes + (0 if scales is None else scales.nbytes)
    cc = [comparators.CastCopy(torch, fmt, N, K, G, codes, scales, alpha)
          for _ in range(max(2, -(-rot_bytes // cbytes)))]
    w16 = cc[0].dequantize()
    dense = [w16] + [w16.clone() for _ in range(max(2, -(-rot_bytes // (w16.numel() * 2))) - 1)]
    kind = "f16" if w16.dtype == torch.float16 else "bf16"
    A = synthetic.activations(M, K, kind, key).cuda()
    n = 10 if M >= 128 else 64
    st = {"i": 0, "j": 0}

    def run_dense():
        comparators.dense_gemm(torch, A, dense[st["i"] % len(dense)])
        st["i"] += 1

    def run_cast():
        cc[st["j"] % len(cc)].run(A)
        st["j"] += 1

    g1 = graph_of(torch, run_dense, n)
    us_dense = time_graph(torch, g1, 3) * 1e3 / n
    del g1
    g2 = graph_of(torch, run_cast, n)
    us_cast = time_graph(torch, g2, 3) * 1e3 / n
    del g2, cc, dense, w16
    torch.cuda.empty_cache()
    return {"gemm": f"{fmt} M={M} N={N} K={K}" + (f" G={G}" if fmt in q.GROUP_SCALED else ""),
            "qgemm_us": round(qgemm_us, 3), "vendor_16bit_gemm_us": round(us_dense, 3),
            "cast_copy_us": round(us_cast, 3), "speedup_vs_16bit": round(us_dense / qgemm_us, 2),
            "speedup_vs_cast_copy": round(us_cast / qgemm_us, 2)}


KERNEL_SOURCES = {"decode": ["qgemm_device.h", "qgemm_decode.hip"],
                  "prefill": ["qgemm_device.h", "qgemm_prefill.hip"]}


def kernel_sha(kind):
    """sha256[:16] over the sources that make up one kernel (recorded in the profiles)."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "weight_only_quantized_qgemm_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per decode launch from the committed counter summary, if it still applies.

    The summary records the kernel source hash it was measured with; a changed kernel makes
    the figure stale, and then None is reported.
    """
    prof = os.path.join(ROOT, "profiles", "qgemm_decode_int4_traffic.txt")
    try:
        sha = kernel_sha("decode")
        text = open(prof).read()
    except OSError:
        return None
    tag = "Decode kernel sources sha256[:16]:"
    rec_sha = text.split(tag, 1)[1].split()[0] if tag in text else ""
    if rec_sha != sha or "traffic_bytes_per_launch =" not in text:
        return None
    return int(text.split("traffic_bytes_per_launch =", 1)[1].split()[0])


def cpu_baseline(budget_s=12.0):
    """The oracle (dequant in fp32 + fp64 matmul) on the decode step, timed on the host."""
    import synthetic
    from oracle import quant, reference
    try:
        from threadpoolctl import threadpool_info
        threads = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    wi = synthetic.WORKLOAD_INDEX["int4_decode"]
    prepared = []
    quant_s = 0.0
    for si, (M, N, K) in enumerate(DECODE_SHAPES):
        w = synthetic.weights(N, K, 0.02, (wi, si))
        tq = time.perf_counter()
        codes, sbits = quant.quantize_int4(w, 128)
        quant_s += time.perf_counter() - tq
        a = synthetic.activations(M, K, "f16", (wi, si)).float().numpy()
        prepared.append((codes, sbits, a, weight_bytes("int4", N, K, 128), 2.0 * M * N * K))
    t0 = time.perf_counter()
    done_bytes, done_flops, steps = 0, 0.0, 0
    while True:
        for codes, sbits, a, nb, fl in prepared:
            wdq = reference.dequant_int4(codes, sbits, 128)
            reference.gemm_fp64(a, wdq)
            done_bytes += nb
            done_flops += fl
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or steps >= 64:
            break
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:  # pragma: no cover
        pass
    return {"value": done_bytes / el / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{steps} full decode steps (4 GEMMs each: fp32 dequant + fp64 matmul), "
                      f"{el:.1f} s, host cores available {len(os.sched_getaffinity(0))}",
            "seconds": round(el, 3), "gflops": round(done_flops / el / 1e9, 3), "blas_threads": int(threads),
            "cpu_model": model, "quantize_s": round(quant_s, 3),
            "quantize_note": "oracle INT4 quantizer (absmax/7, group 128) over the four weights, outside the timed loop"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--all", action="store_true",
                    help="also time the comparators of the FP8 / FP4 shapes and the INT4 prefill")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--rotate-mb", type=int, default=1024)
    ap.add_argument("--counter-pass", nargs="?", const="decode", choices=("decode", "prefill"),
                    help="for rocprofv3 --pmc: run each decode GEMM 20 times (or each prefill workload "
                         "3 times) eagerly, print nothing else")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="for rocprofv3 --pmc: copy a MIB-sized device buffer 5 times (known traffic)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the GEMM would shard "
              "by output columns, each rank holding its columns' packed weights, with no exchange). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import weight_only_quantized_qgemm_amd as q
    import synthetic
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.init()
    rot = args.rotate_mb << 20

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_dispatch": n, "dispatches": 5}))
        return

    if args.counter_pass == "prefill":
        # the prefill workloads with the planned launch, then FP8 32768 x 3200 x 5120 with the
        # persistent stream-K schedule (kernel_hint PREFILL_STREAMK) and with one tile per
        # workgroup (kernel_hint PREFILL), then FP4 M = 128 (the 64 x 128 tile, split K)
        done = []
        for name, si, G, hint in (("int4_prefill", 0, 128, 0), ("fp8", 2, 0, 0), ("fp4", 2, 0, 0),
                                  ("fp8", 3, 0, q.KERNEL_PREFILL_STREAMK), ("fp8", 3, 0, q.KERNEL_PREFILL),
                                  ("fp4", 1, 0, 0)):
            wk = synthetic.WORKLOADS[name]
            M, N, K = wk["shapes"][si]
            g = Gemm(q, torch, wk["fmt"], M, N, K, G, (synthetic.WORKLOAD_INDEX[name], si), rot // 2)
            if hint:
                g.p = q.problem(M, N, K, wk["fmt"], group_size=G or None, kernel_hint=hint)
                g.ws = q.alloc_workspace(g.p)
            for _ in range(3):
                g.launch()
            torch.cuda.synchronize()
            done.append(f"{wk['fmt']} M={M} N={N} K={K}" + (f" kernel_hint={hint}" if hint else ""))
            del g
            torch.cuda.empty_cache()
        print(json.dumps({"counter_pass": done, "launches_each": 3}))
        return

    wi = synthetic.WORKLOAD_INDEX["int4_decode"]
    log("bench: preparing decode workload")
    gemms = [Gemm(q, torch, "int4", M, N, K, 128, (wi, si), rot // 2) for si, (M, N, K) in enumerate(DECODE_SHAPES)]

    def step():
        for g in gemms:
            g.launch()

    if args.counter_pass:
        for g in gemms:
            for _ in range(20):
                g.launch()
        torch.cuda.synchronize()
        print(json.dumps({"counter_pass": [f"int4 M={g.M} N={g.N} K={g.K}" for g in gemms],
                          "launches_each": 20, "weight_bytes": [g.wbytes for g in gemms]}))
        return

    step_bytes = sum(g.wbytes for g in gemms)
    # warmup: eager steps, then a captured graph of exactly `steps` steps
    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    log(f"bench: capturing {args.steps} steps")
    graph = graph_of(torch, step, args.steps)
    graph.replay()                        # untimed warm replay
    torch.cuda.synchronize()

    log("bench: timed region")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = e0.elapsed_time(e1)
    ms_per_step = wall * 1e3 / args.steps
    value = step_bytes * args.steps / wall / 1e9
    launches = 4 * args.steps
    avg_launch_us = ev_ms * 1e3 / launches
    avg_bytes = step_bytes / 4
    achieved = avg_bytes / (avg_launch_us * 1e-6) / 1e9
    del graph

    # per-shape breakdown (graphs of one GEMM repeated; not part of the timed steps)
    secondary = [measure(torch, g, 64) for g in gemms]
    host = host_overhead(q, torch, gemms[:2], iters=500)
    hcases = [(f"int4 N={g.N} K={g.K}", g.wbytes - g.s[0].numel(), g.s[0].numel()) for g in gemms[::2]]
    hcases = [(lab + " weights", w, 0) for lab, w, _ in hcases] + [(lab + " weights+scales", w, sb)
                                                                   for lab, w, sb in hcases]
    del gemms
    torch.cuda.empty_cache()
    hbm = hbm_context(torch, hcases + [("2 GiB", 2 << 30, 0)], rot // 2)

    # vendor comparators on the decode shapes (hipBLASLt through torch; context, not target)
    comps = []
    for si, (M, N, K) in enumerate(DECODE_SHAPES):
        comps.append(comparator_row(q, torch, "int4", M, N, K, 128, (wi, si), rot // 2,
                                    secondary[si]["us_per_launch"]))

    # every other workload shape, each on >= rot / 2 bytes of rotating weight copies: the INT4
    # prefill over the group-size sweep, the FP8 and FP4 layer shapes, the FP8 fp16-activation +
    # bias, INT2 and NF4 workloads
    wi2 = synthetic.WORKLOAD_INDEX["int4_prefill"]
    for G in PREFILL_G:
        log(f"bench: int4 prefill G={G}")
        g = Gemm(q, torch, "int4", 4096, 4096, 4096, G, (wi2, 0), rot // 2)
        secondary.append(measure(torch, g, 20))
        if G == 128:
            host += host_overhead(q, torch, [g], iters=20)
        if args.all and G == 128:
            comps.append(comparator_row(q, torch, "int4", 4096, 4096, 4096, G, (wi2, 0), rot // 2,
                                        secondary[-1]["us_per_launch"]))
        del g
        torch.cuda.empty_cache()
    names = ("fp8", "fp4", "fp8h", "int2", "nf4")
    for name in names:
        wk = synthetic.WORKLOADS[name]
        wix = synthetic.WORKLOAD_INDEX[name]
        for si, (M, N, K) in enumerate(wk["shapes"]):
            log(f"bench: {name} M={M} N={N} K={K}")
            g = Gemm(q, torch, name, M, N, K, wk["group_sizes"][0], (wix, si), rot // 2, with_bias=name == "fp8h")
            secondary.append(measure(torch, g, 10 if M >= 128 else 64))
            del g
            torch.cuda.empty_cache()
            if args.all and name in ("fp8", "fp4", "fp8h"):
                comps.append(comparator_row(q, torch, name, M, N, K, 0, (wix, si), rot // 2,
                                            secondary[-1]["us_per_launch"]))

    cpu = None if args.no_cpu else cpu_baseline()

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "W4A16 decode: fp16 A ~N(0,1); int4 W ~N(0,0.02), group 128, fp16 scales; "
                               "M in {1,16} x (N,K) in {(4096,4096),(11008,4096)}; rotating weight copies",
                   "gemms_per_step": 4, "weight_bytes_per_step": step_bytes},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": recorded_traffic(),
                     "kernel": "qgemm_decode (int4)", "avg_launch_us": round(avg_launch_us, 3),
                     "algorithmic_bytes_per_launch": avg_bytes},
        "cpu_baseline": cpu,
        "hbm_context": hbm,
        "host_overhead": host,
        "secondary": secondary,
        "comparators": comps,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

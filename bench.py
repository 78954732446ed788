"""Benchmark of the 4-bit weight-quantized matmul path on one MI355X.

Metric: Q4 GEMV effective HBM GB/s (M=1) + MMQ prefill TOPS (M=512/2048).

One timed step = one pass of the whole hot path over synthetic inputs already
resident in HBM:
  decode leg  -- one decoded token of a ~4B dense transformer at M = 1: the
                 projection set q, k, v (2560 -> 4096/1024/1024), o
                 (4096 -> 2560), gate, up (2560 -> 9216), down (9216 -> 2560)
                 for each of 36 layers with distinct weights (q/k/v and gate/up
                 as row-concatenated matrices, 4 launches per layer), replayed
                 as one HIP graph, then the lm_head GEMV (2560 -> 151936)
                 launched on its own between HIP events.  2.01 GB of packed weights per
                 token, far above the 256 MB Infinity Cache.
  prefill leg -- Q8_1 quantization of the activations followed by the MMQ
                 GEMM for M = 2048 tokens on a ~9B-shaped layer pair
                 (4096 -> 12288 and 12288 -> 4096, 1 % outliers at 20x) and for
                 M = 512 (2560 -> 9216).
value = algorithmic bytes of the decode leg / decode leg time (GB/s);
the MMQ TOPS (2 M N K / kernel time) are reported under "mmq_prefill".
Algorithmic bytes of a GEMV: packed weights N*K/2 + scales N*K/256*4 + x M*K*4
+ y M*N*4.  Packing (q4_pack) is setup and is not timed.

Both MMQ designs run in the step: q4_mmq_gemm as routed (the fp16 matrix-core
design at these shapes) and q4_mmq_gemm_int8 (int8 matrix cores, exact int32
block dots); each is reported against its own matrix-core peak.  For context
only, "vendor_gemm" times the vendor BLAS's plain GEMMs (torch.mm on fp16,
torch._int_mm on int8 operands, no quantization scales) at the same shapes.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--sustain-ms T]
       python bench.py --pmc-mmq        (Q8_1 + MMQ, M=2048 4096->12288, 3 launches;
                                         nothing printed)
       python bench.py --pmc-mmq-int8   (the same through q4_mmq_gemm_int8)
       python bench.py --pmc-tiny-m M   (tiny-M GEMV at M rows, two weight copies in turn,
                                         4 launches)
       python bench.py --pmc-workload   (lm_head GEMV over two weight copies in turn,
                                         4 launches, and a 256 MiB copy, 3 launches,
                                         for hardware-counter runs; prints nothing)
"""
import hashlib
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
I8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA, TOP/s
F16_PEAK_TFLOPS = 2500.0     # MI355X dense fp16 MFMA, TFLOP/s
LAYERS = 36


def gemv_bytes(M, N, K):
    return N * K // 2 + N * (K // 256) * 4 + M * K * 4 + M * N * 4


def mmq_bytes(M, N, K):
    return N * K // 2 + N * (K // 256) * 4 + M * K + M * (K // 32) * 4 + M * N * 4


def f16_tile_rows(M, N):
    """Activation rows per tile of the fp16 design: 192 where the grid of
    256-row tiles fills at most two rounds of 256 CUs and 192-row tiles take
    fewer rows x rounds, else 256."""
    nt = (N + 127) // 128
    t256, t192 = (M + 255) // 256 * nt, (M + 191) // 192 * nt
    if t256 > 512:
        return 256
    return 192 if (t192 + 255) // 256 * 192 < (t256 + 255) // 256 * 256 else 256


def f16_workspace_bytes(M, N, K):
    """Workspace of q4_mmq_gemm's fp16 design: the fp16 activation image (rows
    padded to whole tiles), row factors and the weight rows' exponents."""
    fm = f16_tile_rows(M, N)
    rows = (M + fm - 1) // fm * fm
    return rows * K * 2 + rows * 4 + (N + 127) // 128 * 128 * 8


def q8_bytes(M, K):
    return M * K * 4 + M * K + M * (K // 32) * 4


# Figures timed outside the step first run their launch back to back for this
# long (discarded): the GPU's clocks ramp on a millisecond scale, and a few
# warm calls after an idle moment leave the timed launches mid-ramp (tiny-M
# M = 8 measured 82 us after 1.5 s idle and 5 ms of calls, 62 us after 20 ms).
SUSTAIN_MS = 100.0
_SUSTAIN_SCALE = [1.0]  # --sustain-ms / SUSTAIN_MS (shorter under a profiler)


def log(msg):
    """Progress line on stderr (stdout carries only the JSON line)."""
    print("bench: " + msg, file=sys.stderr, flush=True)


def sustain(fn, ms=SUSTAIN_MS):
    """Call fn(i) back to back for at least ms of wall time (warm-up)."""
    import torch
    ms *= _SUSTAIN_SCALE[0]
    torch.cuda.synchronize()
    t0, i = time.perf_counter(), 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            fn(i)
            i += 1
        torch.cuda.synchronize()


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sustain-ms", type=float, default=SUSTAIN_MS,
                    help="warm-up of each figure timed outside the step (shorter for profiled runs)")
    ap.add_argument("--no-graph", action="store_true", help="launch the decode layers one by one")
    ap.add_argument("--no-tiny-m", action="store_true", help="skip the tiny-M GEMV sweep")
    ap.add_argument("--no-prefill-sweep", action="store_true",
                    help="skip the pp = 256..2048 MMQ sweep and the GEMV/MMQ crossover")
    ap.add_argument("--pmc-workload", action="store_true",
                    help="only launch the lm_head GEMV and a 256 MiB copy (for rocprofv3 --pmc)")
    ap.add_argument("--pmc-mmq", action="store_true",
                    help="only launch Q8_1 + MMQ on the M=2048, 4096 -> 12288 layer, 3 times (for rocprofv3 --pmc)")
    ap.add_argument("--pmc-mmq-int8", action="store_true",
                    help="as --pmc-mmq through q4_mmq_gemm_int8 (the int8 matrix-core design)")
    ap.add_argument("--pmc-tiny-m", type=int, default=0, metavar="M",
                    help="only launch the tiny-M GEMV (K=4096, N=151936) at M rows, 4 times over two "
                         "weight copies in turn (for rocprofv3 --pmc)")
    return ap.parse_args()


# HBM bytes of the lm_head GEMV launch from rocprofv3 counters (FETCH_SIZE and
# WRITE_SIZE runs over --pmc-workload, scaled by the same counters on the copy).
# They describe the kernel source they were taken on; a changed source has not
# been measured, so the figure is then withheld.
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "lm_head_gemv_hbm_counters.md")
GEMV_SOURCES = [os.path.join(ROOT, "bit_quantized_matmul_q4_amd", "csrc", f)
                for f in ("gemv.hip", "q4mi_device.h")]


def gemv_source_hash():
    h = hashlib.sha256()
    for f in GEMV_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def measured_traffic():
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        if line.startswith("traffic-record "):
            for kv in line.split()[1:]:
                k, _, v = kv.partition("=")
                fields[k] = v
    if fields.get("gemv_sha256") != gemv_source_hash() or "bytes_per_launch" not in fields:
        return None
    return int(fields["bytes_per_launch"])


def pmc_workload():
    """lm_head GEMV over two weight copies in turn (402 MB together, beyond the
    256 MB Infinity Cache) x4 and a 256 MiB device copy x3; nothing timed or
    printed."""
    import torch
    import bit_quantized_matmul_q4_amd as q4
    from bit_quantized_matmul_q4_amd import workloads as wl
    dev = torch.device("cuda:0")
    _, K, N = wl.DECODE_PROJECTIONS[7]
    copies = []
    for i in range(2):
        W = wl.draw_weights(wl.generator(7 + 100 * i, dev), N, K, dev)
        copies.append(q4.q4_pack(W))
        del W
    x = wl.draw_activations(wl.generator(12345, dev), 1, K, False, dev)
    y = torch.empty((1, N), dtype=torch.float32, device=dev)
    for i in range(4):
        q4.q4_gemv(x, *copies[i % 2], y=y)
    src = torch.ones((64 << 20,), dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 2.0, out=dst)
    torch.cuda.synchronize()


def pmc_mmq(int8=False):
    """Q8_1 + MMQ on the M = 2048, 4096 -> 12288 prefill layer x3 (q4_mmq_gemm,
    or q4_mmq_gemm_int8), nothing timed or printed."""
    import torch
    import bit_quantized_matmul_q4_amd as q4
    from bit_quantized_matmul_q4_amd import workloads as wl
    dev = torch.device("cuda:0")
    c = wl.MMQ_2048[0]
    W, x = wl.mmq_case(c["seed"], c["M"], c["N"], c["K"], c["outliers"], dev)
    qs, sm = q4.q4_pack(W)
    del W
    y = torch.empty((c["M"], c["N"]), dtype=torch.float32, device=dev)
    gemm = q4.q4_mmq_gemm_int8 if int8 else q4.q4_mmq_gemm
    for _ in range(3):
        qa, ds = q4.q8_1_quantize(x)
        gemm(qa, ds, qs, sm, y=y)
    torch.cuda.synchronize()


def pmc_tiny_m(M):
    """The tiny-M GEMV (K = 4096, N = 151936) at M rows x4, alternating two
    weight copies (642 MB together, beyond the Infinity Cache); nothing timed
    or printed."""
    import torch
    import bit_quantized_matmul_q4_amd as q4
    from bit_quantized_matmul_q4_amd import workloads as wl
    dev = torch.device("cuda:0")
    c = wl.TINY_M
    K, N = c["K"], c["N"]
    copies = []
    for i in range(2):
        W = wl.draw_weights(wl.generator(c["seed"] + 100 * i, dev), N, K, dev)
        copies.append(q4.q4_pack(W))
        del W
    x = wl.draw_activations(wl.generator(M, dev), M, K, False, dev)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    ws = torch.empty((max(1, q4.q4_gemv_workspace_bytes(M, N, K)),), dtype=torch.uint8, device=dev)
    for i in range(4):
        q4.q4_gemv(x, *copies[i % 2], y=y, workspace=ws)
    torch.cuda.synchronize()


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl):
    """Time the CPU oracle on a bounded sample of the same workloads."""
    import numpy as np
    from oracle import oracle as orc
    threads = orc.get_threads()
    out = {"kind": "oracle", "cores": threads, "cpu_model": cpu_model(),
           "affinity_cpus": len(os.sched_getaffinity(0))}
    # GEMV: the oracle's fp64 GEMV on a sample of the decode projection set (one
    # layer's q, k, v, o, gate, up, down at M = 1), packing excluded from timing
    cases = []
    for idx, (name, K, N) in enumerate(wl.DECODE_PROJECTIONS[:7]):
        W, x = wl.gemv_case(idx, 1, N, K)
        qs, sm = orc.q4_pack(W.numpy())
        cases.append((x.numpy(), qs, sm, K, gemv_bytes(1, N, K)))
    nbytes, secs, passes = 0, 0.0, 0
    while passes < 3 or secs < 8.0:   # whole passes over the layer, >= 8 s of work
        for (xn, qs, sm, K, b) in cases:
            t0 = time.perf_counter()
            orc.q4_gemv(xn, qs, sm, K)
            secs += time.perf_counter() - t0
            nbytes += b
        passes += 1
    gemv_gbs = nbytes / secs / 1e9
    # MMQ: the oracle's fp64 MMQ on 256 of the 2048 activation rows of the
    # 4096 -> 12288 layer (ops counted for those rows only)
    c = wl.MMQ_2048[0]
    rows = 256
    W, x = wl.mmq_case(c["seed"], rows, c["N"], c["K"], True)
    qs, sm = orc.q4_pack(W.numpy())
    qa, ds = orc.q8_1_quantize(x.numpy())
    t0 = time.perf_counter()
    orc.q4_mmq(qa, ds, qs, sm, c["K"])
    ms = time.perf_counter() - t0
    out.update({
        "value": round(gemv_gbs, 3), "unit": "GB/s",
        "sample": "oracle q4_gemv (fp64) over %d passes of one layer of the decode projection "
                  "set (q,k,v,o,gate,up,down, M=1, %.1f MB per pass) in %.2f s; oracle q4_mmq on "
                  "%d of 2048 rows of the 4096->12288 prefill layer in %.2f s"
                  % (passes, nbytes / passes / 1e6, secs, rows, ms),
        "mmq_tops": round(2.0 * rows * c["N"] * c["K"] / ms / 1e12, 6),
    })
    return out


def tiny_m_sweep(q4, wl, dev, stream, reps=12):
    """GEMV at M = 1..16 on the lm_head shape (K=4096, N=151936), outside the
    timed step: two weight copies (2 x 321 MB) alternate so the Infinity Cache
    cannot serve them; after the sustained warm-up, median of per-launch
    HIP-event times."""
    import torch
    c = wl.TINY_M
    K, N = c["K"], c["N"]
    copies = []
    for i in range(2):
        g = wl.generator(c["seed"] + 100 * i, dev)
        W = wl.draw_weights(g, N, K, dev)
        copies.append(q4.q4_pack(W))
        del W
    res = {}
    for M in c["Ms"]:
        x = wl.draw_activations(wl.generator(M, dev), M, K, False, dev)
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
        ws_n = q4.q4_gemv_workspace_bytes(M, N, K)
        ws = torch.empty((max(ws_n, 1),), dtype=torch.uint8, device=dev)
        sustain(lambda i: q4.q4_gemv(x, *copies[i % 2], y=y, workspace=ws))
        times = []
        for r in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            q4.q4_gemv(x, *copies[r % 2], y=y, workspace=ws)
            b.record(stream)
            times.append((a, b))
        torch.cuda.synchronize()
        ms = sorted(a.elapsed_time(b) for a, b in times)[len(times) // 2]
        nbytes = gemv_bytes(M, N, K)
        res["M%d" % M] = {"us": round(ms * 1e3, 2), "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                          "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del copies
    return res


def graph_launch_us(fn, n, stream):
    """Median per-launch time (us) of n launches captured by fn() into one graph
    (replayed for the sustained warm-up first)."""
    import torch
    fn()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    sustain(lambda i: g.replay())
    times = []
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        g.replay()
        b.record(stream)
        times.append((a, b))
    torch.cuda.synchronize()
    return sorted(x.elapsed_time(y) for x, y in times)[2] * 1e3 / n


def decode_breakdown(q4, layers, xs, stream):
    """Each projection of the decode set on its own: its 36 per-layer launches
    (distinct weights) replayed as one graph; per-launch time and GB/s."""
    res = {}
    for k in range(len(layers[0])):
        name, K, N = layers[0][k][:3]
        launches = [layers[layer][k] for layer in range(len(layers))]

        def run():
            for (_, K_, N_, qs, sm, y) in launches:
                q4.q4_gemv(xs[K_], qs, sm, y=y)
        us = graph_launch_us(run, len(launches), stream)
        res[name] = {"K": K, "N": N, "us": round(us, 2),
                     "gbs": round(gemv_bytes(1, N, K) / (us * 1e-6) / 1e9, 1)}
    return res


def single_gemv(q4, wl, dev, stream):
    """The 4096 x 4096 GEMV (seed 0) alone: 60 copies of its packed weights
    (521 MB, beyond the Infinity Cache) launched in turn from one graph."""
    import torch
    c = wl.SINGLE_GEMV
    W, x = wl.gemv_case(c["seed"], 1, c["N"], c["K"], dev)
    qs, sm = q4.q4_pack(W)
    del W
    copies = [(qs.clone(), sm.clone()) for _ in range(60)]
    y = torch.empty((1, c["N"]), dtype=torch.float32, device=dev)

    def run():
        for (q, s_) in copies:
            q4.q4_gemv(x, q, s_, y=y)
    us = graph_launch_us(run, len(copies), stream)
    nbytes = gemv_bytes(1, c["N"], c["K"])
    return {"N": c["N"], "K": c["K"], "us": round(us, 2),
            "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
            "frac_hbm": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


def launch_floor_us(stream, n=252):
    """Per-launch time of a one-element fill kernel replayed n times in a graph:
    the dispatch floor every decode launch pays on this system."""
    import torch
    t = [torch.zeros(1, device="cuda") for _ in range(n)]

    def run():
        for v in t:
            v.fill_(1.0)
    return round(graph_launch_us(run, n, stream), 3)


def vendor_gemm(wl, dev, stream, reps=10):
    """Context, not the library: the vendor BLAS's plain GEMMs (torch.mm on fp16
    operands, torch._int_mm on int8 operands; no quantization scales) at the
    MMQ prefill shapes, median of per-launch HIP-event times."""
    import torch
    out = {}
    for c in [wl.MMQ_512] + list(wl.MMQ_2048):
        M, K, N = c["M"], c["K"], c["N"]
        g = torch.Generator(device=dev).manual_seed(0)
        a = torch.randn((M, K), generator=g, device=dev).to(torch.float16)
        b = torch.randn((K, N), generator=g, device=dev).to(torch.float16)  # contiguous K x N
        ai = torch.randint(-127, 128, (M, K), generator=g, device=dev, dtype=torch.int8)
        bi = torch.randint(-8, 8, (K, N), generator=g, device=dev, dtype=torch.int8)
        res = {}
        for name, fn in (("f16_mm", lambda: torch.mm(a, b)), ("i8_int_mm", lambda: torch._int_mm(ai, bi))):
            sustain(lambda i: fn(), ms=30.0)
            ev = []
            for _ in range(reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                ev.append((e0, e1))
            torch.cuda.synchronize()
            us = sorted(x.elapsed_time(y) for x, y in ev)[reps // 2] * 1e3
            res[name] = {"us": round(us, 2), "tops": round(2.0 * M * N * K / us / 1e6, 1)}
        out["M%d_K%d_N%d" % (M, K, N)] = res
    return out


def prefill_sweep(q4, wl, dev, stream):
    """MMQ (with and without its Q8_1 pass; q4_mmq_gemm as routed and, under
    "int8_design", q4_mmq_gemm_int8) at pp = 256..2048 on the ~9B-shaped
    layer pair, and the GEMV/MMQ crossover at M = 16..256 on the 4096 -> 12288
    layer: the GEMV path runs ceil(M/16) launches of 16 rows, the MMQ path
    Q8_1 + MMQ.  Median of 5 event-timed repetitions each, after 30 ms of
    back-to-back calls."""
    import torch

    def timed(fn, reps=5):
        sustain(lambda i: fn(), ms=30.0)
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            ts.append((a, b))
        torch.cuda.synchronize()
        return sorted(x.elapsed_time(y) for x, y in ts)[len(ts) // 2] * 1e3

    out = {"pp": {}, "crossover": {}}
    layers = []
    for c in wl.MMQ_2048:
        g = wl.generator(c["seed"], dev)
        W = wl.draw_weights(g, c["N"], c["K"], dev)
        qs, sm = q4.q4_pack(W)
        del W
        layers.append((c, qs, sm))
    for pp in (256, 512, 1024, 2048):
        row = {}
        for (c, qs, sm) in layers:
            K, N = c["K"], c["N"]
            x = wl.draw_activations(wl.generator(c["seed"], dev), pp, K, True, dev)
            qa = torch.empty((pp, K), dtype=torch.int8, device=dev)
            ds = torch.empty((pp, K // 32, 2), dtype=torch.float16, device=dev)
            y = torch.empty((pp, N), dtype=torch.float32, device=dev)
            q8_us = timed(lambda: q4.q8_1_quantize(x, qa, ds))
            mmq_us = timed(lambda: q4.q4_mmq_gemm(qa, ds, qs, sm, y=y))
            wi = torch.empty((max(1, q4.q4_mmq_int8_workspace_bytes(pp, N, K)),), dtype=torch.uint8, device=dev)
            int8_us = timed(lambda: q4.q4_mmq_gemm_int8(qa, ds, qs, sm, y=y, workspace=wi))
            ops = 2.0 * pp * N * K
            row[c["name"]] = {"mmq_us": round(mmq_us, 1), "q8_1_us": round(q8_us, 1),
                              "tops": round(ops / (mmq_us * 1e-6) / 1e12, 1),
                              "tops_incl_q8_1": round(ops / ((mmq_us + q8_us) * 1e-6) / 1e12, 1),
                              "int8_design": {"us": round(int8_us, 1),
                                              "tops": round(ops / (int8_us * 1e-6) / 1e12, 1),
                                              "frac_i8_peak": round(ops / (int8_us * 1e-6) / 1e12 / I8_PEAK_TOPS, 4)}}
            # handing the result on as Q8_1 (the next layer's input): quantizing
            # in the GEMM epilogue vs the GEMM then a separate Q8_1 pass over y
            qo = torch.empty((pp, N), dtype=torch.int8, device=dev)
            dso = torch.empty((pp, N // 32, 2), dtype=torch.float16, device=dev)
            fused_us = timed(lambda: q4.q4_mmq_gemm_q8_1(qa, ds, qs, sm, qa_out=qo, ds_out=dso))
            sep_us = timed(lambda: (q4.q4_mmq_gemm(qa, ds, qs, sm, y=y), q4.q8_1_quantize(y, qo, dso)))
            row[c["name"]]["q8_1_out"] = {"fused_us": round(fused_us, 1), "separate_us": round(sep_us, 1)}
        tot = sum(v["mmq_us"] + v["q8_1_us"] for v in row.values())
        row["tokens_per_s_layer_pair"] = round(pp / (tot * 1e-6), 1)
        out["pp"][str(pp)] = row
    c, qs, sm = layers[0]
    K, N = c["K"], c["N"]
    for M in (16, 32, 64, 128, 256):
        x = wl.draw_activations(wl.generator(M, dev), M, K, False, dev)
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
        ws = torch.empty((max(1, q4.q4_gemv_workspace_bytes(16, N, K)),), dtype=torch.uint8, device=dev)

        def gemv_path():
            for r in range(0, M, 16):
                q4.q4_gemv(x[r:r + 16], qs, sm, y=y[r:r + 16], workspace=ws)
        qa = torch.empty((M, K), dtype=torch.int8, device=dev)
        ds = torch.empty((M, K // 32, 2), dtype=torch.float16, device=dev)

        def mmq_path():
            q4.q8_1_quantize(x, qa, ds)
            q4.q4_mmq_gemm(qa, ds, qs, sm, y=y)
        g_us, m_us = timed(gemv_path), timed(mmq_path)
        out["crossover"]["M%d" % M] = {"gemv_us": round(g_us, 1), "mmq_us": round(m_us, 1),
                                       "faster": "gemv" if g_us < m_us else "mmq"}
    return out


def group32_figures(q4, wl, dev, stream):
    """The group-32 variant on the same shapes: lm_head GEMV at M = 1 and 8
    (two weight copies in turn), and the M = 2048 gate/up MMQ.  Bytes count the
    group-32 pairs: N*K/2 + N*K/32*4."""
    import torch

    def timed(fn, reps=12):
        sustain(fn)  # both weight copies in turn
        ts = []
        for r in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn(r)
            b.record(stream)
            ts.append((a, b))
        torch.cuda.synchronize()
        return sorted(x.elapsed_time(y) for x, y in ts)[len(ts) // 2] * 1e3

    out = {}
    _, K, N = wl.DECODE_PROJECTIONS[7]
    copies = []
    for i in range(2):
        W = wl.draw_weights(wl.generator(7 + 100 * i, dev), N, K, dev)
        copies.append(q4.q4_pack_g32(W))
        del W
    for M in (1, 8):
        x = wl.draw_activations(wl.generator(M, dev), M, K, False, dev)
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
        ws = torch.empty((max(1, q4.q4_gemv_g32_workspace_bytes(M, N, K)),), dtype=torch.uint8, device=dev)
        us = timed(lambda r=0: q4.q4_gemv_g32(x, *copies[r % 2], y=y, workspace=ws))
        nbytes = N * K // 2 + N * (K // 32) * 4 + M * K * 4 + M * N * 4
        out["gemv_lm_head_M%d" % M] = {"us": round(us, 2), "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
                                       "frac_hbm": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    del copies
    c = wl.MMQ_2048[0]
    W, x = wl.mmq_case(c["seed"], c["M"], c["N"], c["K"], c["outliers"], dev)
    qs, sm = q4.q4_pack_g32(W)
    del W
    qa, ds = q4.q8_1_quantize(x)
    y = torch.empty((c["M"], c["N"]), dtype=torch.float32, device=dev)
    us = timed(lambda r=0: q4.q4_mmq_gemm_g32(qa, ds, qs, sm, y=y))
    ops = 2.0 * c["M"] * c["N"] * c["K"]
    out["mmq_M2048_gate_up"] = {"us": round(us, 1), "tops": round(ops / (us * 1e-6) / 1e12, 1),
                                "frac_i8_peak": round(ops / (us * 1e-6) / 1e12 / I8_PEAK_TOPS, 4)}
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this build runs on one GPU only; --gpus %d is not supported "
              "(the multi-GPU sharding is a design note, not an implementation)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    if args.pmc_mmq or args.pmc_mmq_int8:
        pmc_mmq(int8=args.pmc_mmq_int8)
        return
    if args.pmc_tiny_m:
        pmc_tiny_m(args.pmc_tiny_m)
        return
    if args.pmc_workload:
        pmc_workload()
        return

    import torch
    import bit_quantized_matmul_q4_amd as q4
    from bit_quantized_matmul_q4_amd import workloads as wl

    _SUSTAIN_SCALE[0] = args.sustain_ms / SUSTAIN_MS
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    # ------------------------------------------------------------ setup ----
    def packed(seed, N, K):
        g = wl.generator(seed, dev)
        W = wl.draw_weights(g, N, K, dev)
        qs, sm = q4.q4_pack(W)
        del W
        return qs, sm

    gx = wl.generator(12345, dev)
    xs = {K: wl.draw_activations(gx, 1, K, False, dev) for K in (2560, 4096, 9216)}
    layers = []
    for layer in range(LAYERS):
        projs = []
        for k, (name, K, N) in enumerate(wl.DECODE_PROJECTIONS[:7]):
            qs, sm = packed(8 * layer + k, N, K)
            y = torch.empty((1, N), dtype=torch.float32, device=dev)
            projs.append((name, K, N, qs, sm, y))
        layers.append(projs)
    # The timed step runs each layer in the usual fused layouts: q, k, v as one
    # row-concatenated 2560 -> 6144 matrix and gate, up as one 2560 -> 18432
    # matrix (packing is per row, so the concatenated packed tensors are the
    # packed concatenation), i.e. 4 launches per layer: qkv, o, gate_up, down.
    # The 7-launch stream over the separate matrices is reported beside it.
    fused_layers = []
    for projs in layers:
        by = {p[0]: p for p in projs}

        def cat(names):
            qs = torch.cat([by[n][3] for n in names], 0)
            sm = torch.cat([by[n][4] for n in names], 0)
            return ("_".join(names), by[names[0]][1], qs.shape[0], qs, sm,
                    torch.empty((1, qs.shape[0]), dtype=torch.float32, device=dev))
        fused_layers.append([cat(["q", "k", "v"]), by["o"], cat(["gate", "up"]), by["down"]])
    _, Kl, Nl = wl.DECODE_PROJECTIONS[7]
    lm_qs, lm_sm = packed(7, Nl, Kl)
    lm_y = torch.empty((1, Nl), dtype=torch.float32, device=dev)
    layer_bytes = sum(gemv_bytes(1, N, K) for (_, K, N, *_r) in fused_layers[0])
    unfused_layer_bytes = sum(gemv_bytes(1, N, K) for (_, K, N) in wl.DECODE_PROJECTIONS[:7])
    lm_bytes = gemv_bytes(1, Nl, Kl)
    decode_bytes = LAYERS * layer_bytes + lm_bytes

    pre = []
    for c in wl.MMQ_2048 + [dict(wl.MMQ_512, name="m512")]:
        W, x = wl.mmq_case(c["seed"], c["M"], c["N"], c["K"], c["outliers"], dev)
        qs, sm = q4.q4_pack(W)
        del W
        qa = torch.empty((c["M"], c["K"]), dtype=torch.int8, device=dev)
        ds = torch.empty((c["M"], c["K"] // 32, 2), dtype=torch.float16, device=dev)
        y = torch.empty((c["M"], c["N"]), dtype=torch.float32, device=dev)
        ws_n = q4.q4_mmq_workspace_bytes(c["M"], c["N"], c["K"])
        ws = torch.empty((max(ws_n, 1),), dtype=torch.uint8, device=dev)
        wi_n = q4.q4_mmq_int8_workspace_bytes(c["M"], c["N"], c["K"])
        wi = torch.empty((max(wi_n, 1),), dtype=torch.uint8, device=dev)
        yi = torch.empty((c["M"], c["N"]), dtype=torch.float32, device=dev)
        pre.append((c, x, qa, ds, qs, sm, y, ws, yi, wi))
    # a plain device copy of known size: reference for the HBM byte counters
    cp_src = torch.empty((64 << 20,), dtype=torch.float32, device=dev).fill_(1.0)
    cp_dst = torch.empty_like(cp_src)
    torch.cuda.synchronize()

    def decode_layers():
        for projs in fused_layers:
            for (name, K, N, qs, sm, y) in projs:
                q4.q4_gemv(xs[K], qs, sm, y=y)

    def decode_layers_unfused():
        for projs in layers:
            for (name, K, N, qs, sm, y) in projs:
                q4.q4_gemv(xs[K], qs, sm, y=y)

    def lm_head():
        q4.q4_gemv(xs[Kl], lm_qs, lm_sm, y=lm_y)

    decode_layers()  # warm the per-device property cache before any capture
    graph = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            decode_layers()
        torch.cuda.synchronize()

    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    n_ev = 3 + 4 * len(pre)

    def step(ev):
        ev[0].record(stream)
        if graph is not None:
            graph.replay()
        else:
            decode_layers()
        ev[1].record(stream)
        lm_head()
        ev[2].record(stream)
        i = 3
        for (c, x, qa, ds, qs, sm, y, ws, yi, wi) in pre:
            ev[i].record(stream)
            q4.q8_1_quantize(x, qa, ds)
            ev[i + 1].record(stream)
            q4.q4_mmq_gemm(qa, ds, qs, sm, y=y, workspace=ws)
            ev[i + 2].record(stream)
            q4.q4_mmq_gemm_int8(qa, ds, qs, sm, y=yi, workspace=wi)
            ev[i + 3].record(stream)
            i += 4
        return ev

    log("setup done; warm-up steps")
    for _ in range(args.warmup):
        step([E() for _ in range(n_ev)])
    cp_dst.copy_(cp_src)
    torch.cuda.synchronize()

    # ------------------------------------------------------------ timed ----
    events = [[E() for _ in range(n_ev)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    def med(vals):
        v = sorted(vals)
        return v[len(v) // 2]

    layers_ms = med([e[0].elapsed_time(e[1]) for e in events])
    lm_ms = med([e[1].elapsed_time(e[2]) for e in events])
    decode_ms = med([e[0].elapsed_time(e[2]) for e in events])
    mmq_rep = {}
    for k, (c, *_rest) in enumerate(pre):
        i = 3 + 4 * k
        q_ms = med([e[i].elapsed_time(e[i + 1]) for e in events])
        g_ms = med([e[i + 1].elapsed_time(e[i + 2]) for e in events])
        i_ms = med([e[i + 2].elapsed_time(e[i + 3]) for e in events])
        ops = 2.0 * c["M"] * c["N"] * c["K"]
        mmq_rep["M%d_%s" % (c["M"], c["name"])] = {
            "M": c["M"], "K": c["K"], "N": c["N"],
            "mmq_us": round(g_ms * 1e3, 2), "tops": round(ops / (g_ms * 1e-3) / 1e12, 2),
            "design": "fp16" if q4.q4_mmq_workspace_bytes(c["M"], c["N"], c["K"]) == f16_workspace_bytes(c["M"], c["N"], c["K"])
                      else "int8",
            "frac_i8_peak": round(ops / (g_ms * 1e-3) / 1e12 / I8_PEAK_TOPS, 4),
            "frac_f16_peak": round(ops / (g_ms * 1e-3) / 1e12 / F16_PEAK_TFLOPS, 4),
            "q8_1_us": round(q_ms * 1e3, 2),
            "q8_1_gbs": round(q8_bytes(c["M"], c["K"]) / (q_ms * 1e-3) / 1e9, 1),
            "tops_incl_q8_1": round(ops / ((g_ms + q_ms) * 1e-3) / 1e12, 2),
            "int8_design": {"mmq_us": round(i_ms * 1e3, 2), "tops": round(ops / (i_ms * 1e-3) / 1e12, 2),
                            "frac_i8_peak": round(ops / (i_ms * 1e-3) / 1e12 / I8_PEAK_TOPS, 4)},
        }
    step_ms = wall / args.steps * 1e3
    value = decode_bytes / (decode_ms * 1e-3) / 1e9
    lm_gbs = lm_bytes / (lm_ms * 1e-3) / 1e9
    big = mmq_rep["M2048_gate_up"]

    out = {
        "metric": "Q4 GEMV effective HBM GB/s (M=1) + MMQ prefill TOPS (M=512/2048)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u4 x f16 -> f32 (GEMV); MMQ: f16 x f16 -> f32 (q4_mmq_gemm at these shapes: Q8_1 and u4 "
                 "operands scaled into fp16) and i8 x i4 -> i32 -> f32 (q4_mmq_gemm_int8: exact block dots)",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) activations; random weights of the stated shapes)",
        "config": {
            "workload": "decode token of a ~4B dense transformer at M=1: 36 layers x "
                        "{q,k,v 2560->4096/1024/1024, o 4096->2560, gate,up 2560->9216, down 9216->2560} "
                        "+ lm_head 2560->151936, 4-bit group-256, q/k/v and gate/up as row-concatenated "
                        "fused matrices (4 launches per layer); plus MMQ prefill M=2048 "
                        "(4096->12288, 12288->4096) and M=512 (2560->9216)",
            "decode_bytes_per_step": decode_bytes,
            "graph": graph is not None,
        },
        "decode": {
            "layers_us": round(layers_ms * 1e3, 1),
            "layers_gbs": round(LAYERS * layer_bytes / (layers_ms * 1e-3) / 1e9, 1),
            "lm_head_us": round(lm_ms * 1e3, 2),
            "lm_head_gbs": round(lm_gbs, 1),
            "tokens_per_s_weights_only": round(1e3 / decode_ms, 1),
            "frac_hbm": round(value / HBM_PEAK_GBS, 4),
        },
        "roofline": {
            "kernel": "k_gemv_dot2 (lm_head launch, M=1, K=2560, N=151936)",
            "bound": "hbm",
            "achieved": round(lm_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(lm_gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(),
        },
        "mmq_prefill": dict(mmq_rep, roofline={
            "kernel": "q4_mmq_gemm, fp16 design: k_mmqf_rowscale + k_mmqf_image + k_mmqf "
                      "(M=2048, K=4096, N=12288)", "bound": "mfma",
            "achieved": big["tops"], "peak": F16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(big["tops"] / F16_PEAK_TFLOPS, 4)},
            roofline_int8={
                "kernel": "q4_mmq_gemm_int8: k_mmqi_prep + k_mmqi (M=2048, K=4096, N=12288)", "bound": "mfma",
                "achieved": big["int8_design"]["tops"], "peak": I8_PEAK_TOPS, "unit": "TOP/s",
                "frac": big["int8_design"]["frac_i8_peak"]}),
    }
    log("timed steps done")
    n_unfused = LAYERS * len(layers[0])
    unf_us = graph_launch_us(decode_layers_unfused, n_unfused, stream) * n_unfused
    out["decode_unfused"] = {
        "launches_per_layer": len(layers[0]),
        "layers_us": round(unf_us, 1),
        "layers_gbs": round(LAYERS * unfused_layer_bytes / (unf_us * 1e-6) / 1e9, 1),
        "gbs_with_lm_head": round((LAYERS * unfused_layer_bytes + lm_bytes) /
                                  ((unf_us + lm_ms * 1e3) * 1e-6) / 1e9, 1),
    }
    out["decode_projections"] = decode_breakdown(q4, layers, xs, stream)
    out["decode_projections_fused"] = decode_breakdown(q4, fused_layers, xs, stream)
    out["graph_launch_floor_us"] = launch_floor_us(stream)
    out["gemv_single_4096"] = single_gemv(q4, wl, dev, stream)
    log("decode breakdown done")
    if not args.no_tiny_m:
        out["gemv_tiny_m"] = tiny_m_sweep(q4, wl, dev, stream)
        log("tiny-M sweep done")
    if not args.no_prefill_sweep:
        out["prefill_sweep"] = prefill_sweep(q4, wl, dev, stream)
        log("prefill sweep done")
    out["group32"] = group32_figures(q4, wl, dev, stream)
    out["vendor_gemm"] = vendor_gemm(wl, dev, stream)
    log("group-32 and vendor GEMM done")
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

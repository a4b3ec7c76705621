"""Benchmark of the ZeRO++ quantized-communication hot path on one MI355X.

One step is one rank's pass through every kernel of the path, at full size:
  qwZ  (GPT layer at hidden 8192, fp16, block 256, 16 ranks)
    K1 zpq_quant_i8             quantize this rank's 1/16 weight shard
    K2 zpq_dequant_i8           dequantize the gathered buffer (16 shards)
  qgZ  (138B-model layer gradient: FFN 12288x49152 + QKV 12288x36864, fp16,
        INT4 block 64, L = 8 local ranks, N = 48 nodes)
    K3 zpq_qgz_reorder_quant_i4             slice reorder + INT4 quantize
    K4 zpq_qgz_dequant_reduce_requant_i4    hop 1: 8 received chunks -> INT4
    K5 zpq_qgz_dequant_reduce_requant_i4    hop 2: 48 received chunks -> fp16 average
The all-gather and all-to-alls are simulated: the receive buffers are filled
once before timing (gathered buffer = the 16 shards' quantization; hop-1
receive = this rank's own 8 send chunks; hop-2 receive = the 48 send positions
of its own hop-1 result), so each kernel reads a buffer the previous kernel
did not just write and nothing is served from the 256 MB MALL.

Prints one JSON line.  `value` is the step's effective HBM bandwidth:
algorithmic bytes of all five kernels / wall time per step.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "effective HBM GB/s per kernel and % of MI355X peak (qwZ quant/dequant, qgZ hop)"

# Kernel time, everywhere in this file: the per-launch time of launches issued
# back to back on one stream (one HIP event pair around `LAUNCHES` launches,
# median over groups), cycling through enough distinct buffer sets that no
# launch finds its data in the 256 MB last-level cache.  Back-to-back launches
# hide the dispatch of each kernel behind the previous one, as in a pipeline:
# this is the duration the rocprofv3 kernel trace reports, while an event pair
# around a single launch adds 2-4 us of command-processor time.
LAUNCHES = 20
ROTATE_BYTES = 640 << 20          # data touched between two uses of a buffer set


def kernel_code_digest():
    """SHA-256 of libzpq's kernel source with comments and blank lines removed:
    the HBM traffic recorded by the counter passes stays valid while this is
    unchanged."""
    import hashlib
    import re
    path = os.path.join(ROOT, "block_quantized_communication_amd", "csrc", "zpq.hip")
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = [re.sub(r"//.*$", "", l).rstrip() for l in text.splitlines()]
    return hashlib.sha256("\n".join(l for l in lines if l).encode()).hexdigest()


def n_sets(bytes_per_launch):
    """Buffer sets needed so that ROTATE_BYTES pass between two uses of one."""
    return max(1, -(-ROTATE_BYTES // int(bytes_per_launch)))


def launch_groups_us(torch, fns, groups, settle_s=0.1):
    """Per-launch microseconds of `groups` groups of LAUNCHES back-to-back
    launches cycling through `fns` (one callable per buffer set), each group
    between one pair of HIP events on the current stream."""
    st = torch.cuda.current_stream()
    k = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < settle_s:
        for _ in range(LAUNCHES):
            fns[k % len(fns)]()
            k += 1
        torch.cuda.synchronize()
    us = []
    for _ in range(groups):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        for _ in range(LAUNCHES):
            fns[k % len(fns)]()
            k += 1
        b.record(st)
        torch.cuda.synchronize()
        us.append(a.elapsed_time(b) * 1e3 / LAUNCHES)
    return us


def launch_time_us(np, torch, fns, groups, settle_s=0.1):
    """(median, minimum) of launch_groups_us."""
    us = launch_groups_us(torch, fns, groups, settle_s)
    return float(np.median(us)), float(np.min(us))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="before the warm-up steps, run untimed steps for this long: under "
                         "sustained HBM load the chip's power controller lowers the clocks and "
                         "takes tens of ms to settle, and the timed steps should see the settled "
                         "state")
    ap.add_argument("--kernel-groups", type=int, default=10,
                    help="after the timed steps, time each kernel in this many groups of "
                         f"{LAUNCHES} back-to-back launches over rotating buffer sets; the "
                         "per-kernel figures are the medians over the groups, whatever --steps is")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-check", action="store_true")
    ap.add_argument("--cpu-fraction", type=float, default=0.6)
    ap.add_argument("--per-config", action="store_true",
                    help="time every kernel at every workload size (cache evicted before each "
                         "launch) instead of the step")
    ap.add_argument("--patterns", action="store_true",
                    help="time every kernel at every workload size beside its bare access pattern "
                         "(the same loads and stores without the arithmetic, from "
                         "bench_patterns.hip) and the read / write / copy ceilings")
    ap.add_argument("--valu-rates", action="store_true",
                    help="measure the vector ALU's issue rate per instruction kind and per "
                         "per-element sequence of the hop-receive loop (register-only kernels "
                         "from bench_patterns.hip)")
    ap.add_argument("--study", choices=["hop-count", "blocking", "receive-shapes", "store-policy",
                                        "timeline"],
                    default=None,
                    help="run a study instead of the throughput benchmark: hop-count and "
                         "blocking (quantization error), receive-shapes (launch shapes of the "
                         "receive kernel; needs the variant libraries), store-policy (cache-policy "
                         "bits of streams and of the qgZ quantizer's code stores; needs the "
                         "variant libraries), timeline (every wave's start and end in the receive "
                         "launches and their bare patterns; needs the variant libraries)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after timing, copy 1 GiB with torch (a plain copy kernel of known "
                         "size, to calibrate rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="per-kernel HBM bytes from rocprofv3 counters (optional)")
    args = ap.parse_args()
    if args.steps < 1 or args.warmup < 0:
        ap.error("--steps must be at least 1 and --warmup at least 0")
    return args


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: libzpq has no multi-GPU path "
              "(collectives are simulated in one GPU's memory); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import block_quantized_communication_amd as zpq
    import synth

    if args.study == "hop-count":
        print(json.dumps(hop_count_study(np, torch, zpq, synth)), flush=True)
        return
    if args.study == "blocking":
        print(json.dumps(blocking_study(np, torch, zpq, synth)), flush=True)
        return
    if args.study == "receive-shapes":
        print(json.dumps(receive_shapes_study(np, torch)), flush=True)
        return
    if args.study == "store-policy":
        print(json.dumps(store_policy_study(np, torch)), flush=True)
        return
    if args.study == "timeline":
        print(json.dumps(timeline_study(np, torch)), flush=True)
        return
    if args.per_config:
        print(json.dumps(per_config(np, torch, zpq, synth)), flush=True)
        return
    if args.patterns:
        print(json.dumps(patterns(np, torch, zpq, synth)), flush=True)
        return
    if args.valu_rates:
        print(json.dumps(valu_rates(np, torch)), flush=True)
        return

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    T = torch

    # ---------------- workloads ----------------
    qw = synth.QWZ_LAYER
    Bw, Ww, nw = qw["block"], qw["world"], qw["n"]
    Sw = nw // Ww
    qg = synth.QGZ_FUSED
    L, N, Bg, ng = qg["L"], qg["N"], qg["block"], qg["n"]
    W = L * N
    Sg = ng // W
    chunk = ng // L

    t0 = time.time()
    print(f"[bench] generating qwZ layer ({nw} fp16)", file=sys.stderr, flush=True)
    layer_h = synth.qwz_layer()
    layer = torch.from_numpy(layer_h).to(dev)
    print(f"[bench] generating qgZ gradient ({ng} fp16)", file=sys.stderr, flush=True)
    grad_h = synth.qgz_fused()
    grad = torch.from_numpy(grad_h).to(dev)
    print(f"[bench] inputs ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    import hashlib
    inputs = {"qwz_layer": {"seed": synth.SEEDS["qwz_layer"],
                            "sha256": hashlib.sha256(memoryview(layer_h).cast("B")).hexdigest()},
              "qgz_grad": {"seed": synth.SEEDS["qgz_fused"],
                           "sha256": hashlib.sha256(memoryview(grad_h).cast("B")).hexdigest()}}

    shard = layer[:Sw]
    e = lambda n, dt: torch.empty(n, dtype=dt, device=dev)
    shard_codes, shard_scales = e(Sw, T.int8), e(Sw // Bw, T.float32)
    gath_codes, gath_scales = e(nw, T.int8), e(nw // Bw, T.float32)
    y_layer = e(nw, T.float16)
    send1_c, send1_s = e(ng // 2, T.uint8), e(ng // Bg, T.float32)
    recv1_c, recv1_s = e(ng // 2, T.uint8), e(ng // Bg, T.float32)
    send2_c, send2_s = e(chunk // 2, T.uint8), e(chunk // Bg, T.float32)
    recv2_c, recv2_s = e(chunk // 2, T.uint8), e(chunk // Bg, T.float32)
    y_grad = e(Sg, T.float16)

    # simulated collectives, filled once
    zpq.quant_i8(layer, Bw, out=(gath_codes, gath_scales))          # all-gather of 16 shards
    zpq.qgz_reorder_quant_i4(grad, L, N, Bg, out=(send1_c, send1_s))
    recv1_c.copy_(send1_c)
    recv1_s.copy_(send1_s)                                          # hop-1 all-to-all
    zpq.qgz_dequant_reduce_requant_i4(recv1_c, recv1_s, L, chunk, Bg, out=(send2_c, send2_s))
    recv2_c.copy_(send2_c)
    recv2_s.copy_(send2_s)                                          # hop-2 all-to-all
    torch.cuda.synchronize()

    kernels = [
        ("K1 qwZ quant_i8 (shard 1/16, fp16, B=256)",
         lambda: zpq.quant_i8(shard, Bw, out=(shard_codes, shard_scales)),
         Sw * 2 + Sw + (Sw // Bw) * 4),
        ("K2 qwZ dequant_i8 (gathered 16 shards -> fp16)",
         lambda: zpq.dequant_i8(gath_codes, gath_scales, Bw, out=y_layer),
         nw + (nw // Bw) * 4 + nw * 2),
        ("K3 qgZ reorder_quant_i4 (fp16, L=8, N=48, B=64)",
         lambda: zpq.qgz_reorder_quant_i4(grad, L, N, Bg, out=(send1_c, send1_s)),
         ng * 2 + ng // 2 + (ng // Bg) * 4),
        ("K4 qgZ hop-1 dequant_reduce_requant_i4 (8 x chunk -> INT4)",
         lambda: zpq.qgz_dequant_reduce_requant_i4(recv1_c, recv1_s, L, chunk, Bg,
                                                   out=(send2_c, send2_s)),
         L * (chunk // 2 + (chunk // Bg) * 4) + chunk // 2 + (chunk // Bg) * 4),
        ("K5 qgZ hop-2 dequant_reduce_average (48 x slice -> fp16)",
         lambda: zpq.qgz_dequant_reduce_requant_i4(recv2_c, recv2_s, N, Sg, Bg,
                                                   out_dtype=T.float16, divisor=float(W),
                                                   out=y_grad),
         N * (Sg // 2 + (Sg // Bg) * 4) + Sg * 2),
    ]
    step_bytes = sum(k[2] for k in kernels)

    def step():
        for _, fn, _ in kernels:
            fn()

    settle_steps = 0
    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(10):
            step()
        settle_steps += 10
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # The timed steps: no events inside.
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = wall * 1e3 / args.steps

    # Per-kernel times (after the timed steps): each kernel alone, LAUNCHES
    # back-to-back launches per group, rotating over buffer sets so that no
    # launch finds its data in the last-level cache (set 0 is the step's own).
    def rotation(i):
        name, fn, nbytes = kernels[i]
        k = n_sets(nbytes)
        if k == 1:
            return [fn]
        if i == 0:                      # K1: other ranks' shards, own outputs
            outs = [(e(Sw, T.int8), e(Sw // Bw, T.float32)) for _ in range(k - 1)]
            return [fn] + [lambda r=r, o=o: zpq.quant_i8(layer[r * Sw:(r + 1) * Sw], Bw, out=o)
                           for r, o in zip(range(1, k), outs)]
        if i == 3:                      # K4: copies of the hop-1 receive buffer
            sets = [(recv1_c.clone(), recv1_s.clone(), e(chunk // 2, T.uint8),
                     e(chunk // Bg, T.float32)) for _ in range(k - 1)]
            return [fn] + [lambda q=q: zpq.qgz_dequant_reduce_requant_i4(
                q[0], q[1], L, chunk, Bg, out=(q[2], q[3])) for q in sets]
        if i == 4:                      # K5: copies of the hop-2 receive buffer
            sets = [(recv2_c.clone(), recv2_s.clone(), e(Sg, T.float16)) for _ in range(k - 1)]
            return [fn] + [lambda q=q: zpq.qgz_dequant_reduce_requant_i4(
                q[0], q[1], N, Sg, Bg, out_dtype=T.float16, divisor=float(W), out=q[2])
                for q in sets]
        raise AssertionError(f"no rotation for kernel {i}")
    G = max(1, args.kernel_groups)
    per_kernel = []
    for i in range(len(kernels)):
        fns = rotation(i)
        med, mn = launch_time_us(np, torch, fns, G)
        per_kernel.append((med, mn, len(fns)))
        del fns
    torch.cuda.synchronize()

    if args.copy_probe:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE passes,
    # valid only for the kernel source they were measured on
    traffic = {}
    if args.traffic and os.path.exists(args.traffic):
        with open(args.traffic) as f:
            t = json.load(f)
        if kernel_code_digest() == t.get("kernel_code_sha256"):
            traffic = t.get("bytes_per_launch", {})

    rows = []
    for (name, _, nbytes), (med, mn, nset) in zip(kernels, per_kernel):
        gbs = nbytes / med / 1e3
        rows.append({"kernel": name, "bytes": nbytes, "us": round(med, 2),
                     "us_min": round(mn, 2), "buffer_sets": nset,
                     "GBps": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)})
    dom = max(range(len(rows)), key=lambda i: per_kernel[i][0])
    dk = rows[dom]
    tr = traffic.get(dk["kernel"].split(" ")[0])
    roofline = {"bound": "hbm", "kernel": dk["kernel"], "achieved": dk["GBps"],
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": dk["frac_of_peak"],
                "traffic": tr}

    check = None
    if not args.no_check:
        check = verify(zpq, synth, np, torch, layer_h, grad_h, gath_codes, gath_scales, y_layer,
                       shard_codes, shard_scales, send1_c, send1_s, send2_c, send2_s, y_grad)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(np, layer_h, grad_h, args.cpu_fraction)

    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": settle_steps,
        "kernel_times": f"per-launch time of {LAUNCHES} back-to-back launches between one HIP "
                        f"event pair, median of {G} groups, rotating buffer sets (>= "
                        f"{ROTATE_BYTES >> 20} MiB between reuses), after the timed steps",
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "element_types": "fp16 weights and gradients in; INT8 (qwZ) and packed INT4 (qgZ) "
                         "codes with fp32 scales; fp32 sums; fp16 averaged gradient out",
        "data": "synthetic",
        "config": {
            "workload": "one rank's ZeRO++ quantized-communication step: qwZ on a GPT layer at "
                        "hidden 8192 (fp16, INT8 block 256, 16 ranks) + qgZ on a 138B-model "
                        "layer gradient (fp16, INT4 block 64, L=8, N=48, both hops)",
            "qwz_layer_elems": nw, "qwz_shard_elems": Sw, "qgz_grad_elems": ng,
            "inputs": inputs,
            "step_bytes": step_bytes, "frac_of_peak": round(value / HBM_PEAK_GBS, 4),
            "kernels": rows,
            "parity": check,
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def verify(zpq, synth, np, torch, layer_h, grad_h, gath_codes, gath_scales, y_layer,
           shard_codes, shard_scales, send1_c, send1_s, send2_c, send2_s, y_grad):
    """Every output byte of this run against the oracle chain computed from the
    generator's inputs (never from a GPU output).  The oracle runs over
    independent ranges on host threads: ranges of the layer for qwZ; send
    positions, then block ranges of the received chunks, for qgZ."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    t0 = time.time()
    workers = max(1, min(16, os.cpu_count() or 1))
    pool = ThreadPoolExecutor(workers)
    host = lambda t: t.view(torch.int16 if t.dtype == torch.float16 else t.dtype).cpu().numpy()
    same = lambda a, b: bool(np.array_equal(np.ascontiguousarray(a).view(np.uint8),
                                            np.ascontiguousarray(b).view(np.uint8)))
    ok = {}
    qw, qg = synth.QWZ_LAYER, synth.QGZ_FUSED
    Bw, nw = qw["block"], qw["n"]
    Sw = nw // qw["world"]
    R = 1 << 24

    def qwz(r0):
        c, s = oracle.quant_i8(layer_h[r0:r0 + R], "f16", Bw)
        return c, s, oracle.dequant_i8(c, s, Bw, "f16")
    parts = list(pool.map(qwz, range(0, nw, R)))
    ec = np.concatenate([p[0] for p in parts])
    es = np.concatenate([p[1] for p in parts])
    ok["qwz_gathered_codes"] = same(host(gath_codes), ec)
    ok["qwz_gathered_scales"] = same(host(gath_scales), es)
    ok["qwz_dequant"] = same(host(y_layer), np.concatenate([p[2] for p in parts]))
    ok["qwz_shard_codes"] = same(host(shard_codes), ec[:Sw])
    ok["qwz_shard_scales"] = same(host(shard_scales), es[:Sw // Bw])
    del parts, ec, es

    L, N, B, n = qg["L"], qg["N"], qg["block"], qg["n"]
    W = L * N
    S, chunk = n // W, n // L
    src = oracle.reorder(np.arange(W, dtype=np.int64), L, N)
    parts = list(pool.map(lambda p: oracle.qgz_reorder_quant_i4(
        grad_h[src[p] * S:(src[p] + 1) * S], "f16", 1, 1, B), range(W)))
    c1 = np.concatenate([p[0] for p in parts])
    s1 = np.concatenate([p[1] for p in parts])
    ok["qgz_send_codes"] = same(host(send1_c), c1)
    ok["qgz_send_scales"] = same(host(send1_s), s1)

    def receive(codes, scales, K, ch, pieces, out_dtype=None, divisor=1.0):
        r = ch // pieces

        def one(k):
            lo, hi = k * r, (k + 1) * r
            ic = np.concatenate([codes[i * (ch // 2) + lo // 2:i * (ch // 2) + hi // 2]
                                 for i in range(K)])
            isc = np.concatenate([scales[i * (ch // B) + lo // B:i * (ch // B) + hi // B]
                                  for i in range(K)])
            return oracle.qgz_dequant_reduce_requant_i4(ic, isc, K, r, B, out_dtype, divisor)
        return list(pool.map(one, range(pieces)))
    parts = receive(c1, s1, L, chunk, 48)         # hop-1 receive: this rank's own send chunks
    c2 = np.concatenate([p[0] for p in parts])
    s2 = np.concatenate([p[1] for p in parts])
    ok["qgz_hop1_codes"] = same(host(send2_c), c2)
    ok["qgz_hop1_scales"] = same(host(send2_s), s2)
    y = np.concatenate(receive(c2, s2, N, S, 16, "f16", float(W)))
    ok["qgz_hop2_average"] = same(host(y_grad), y)
    pool.shutdown()
    return {"compared": "every output byte of every kernel of this run", "bit_exact": all(ok.values()),
            "parts": ok, "oracle_threads": workers, "seconds": round(time.time() - t0, 1)}


# Build-time defaults of the receive launch (csrc/zpq.hip); the receive-shapes
# study reads each variant's overrides against these to name the kernel a
# launch uses.
RECEIVE_DEFAULTS = {"ZPQ_REDUCE_EPL_I4": 32, "ZPQ_REDUCE_PF_I4": 2, "ZPQ_REDUCE_EPL_FL": 16,
                    "ZPQ_REDUCE_PF_FL": 2, "ZPQ_REDUCE_PF_FL_NARROW": 4,
                    "ZPQ_REDUCE_NARROW_WAVES": 8, "ZPQ_REDUCE_WG3": 0}


def receive_launch(defines, K, c, B, fl, cus):
    """(EPL, PF, threads per workgroup, mangled kernel-name fragment) of the
    receive launch a library built with `defines` makes for K sources of c
    elements, block B (fl: float output, 1 fp16 / 2 bf16; else INT4)."""
    d = dict(RECEIVE_DEFAULTS)
    for x in defines:
        k, v = x[2:].split("=")
        d[k] = int(v)

    def epl_for(e):
        return B if e > B else (e if B // e <= 32 else B // 32)
    if not fl:
        epl, pf, out = epl_for(d["ZPQ_REDUCE_EPL_I4"]), d["ZPQ_REDUCE_PF_I4"], "in1"
    else:
        waves16 = -(-c // (16 * 64))
        if B <= 256 and waves16 < d["ZPQ_REDUCE_NARROW_WAVES"] * 4 * cus:
            epl, pf = 8, d["ZPQ_REDUCE_PF_FL_NARROW"]
        else:
            epl, pf = epl_for(d["ZPQ_REDUCE_EPL_FL"]), d["ZPQ_REDUCE_PF_FL"]
        out = f"i{fl}"
    waves = -(-c // (64 * epl))
    busiest = lambda w: -(-(-(-waves // w)) // cus) * w
    nt = 192 if d["ZPQ_REDUCE_WG3"] and busiest(3) < busiest(4) else 256
    return epl, pf, nt, f"k_dequant_reduceILi{B}ELi{epl}EL{out}ELi{pf}E"


def receive_shapes_study(np, torch, settle_s=0.1):
    """The receive kernel's launch shapes side by side: every library of
    block_quantized_communication_amd/variants/ (built by
    `python -m block_quantized_communication_amd.build --variants`, one
    build-time override each: elements per lane, sources in flight, when the
    average takes 8 per lane, 3-wave workgroups) on the four receive
    workloads, alternating with the default build, each output compared
    byte for byte with the default's, with the registers, LDS and occupancy
    the compiler reported for the kernel the launch uses.  Then the default
    hop-1 kernel at 1..16 sources (block 128),
    whose VALU instructions per wave (a counter pass over this command) give
    the per-source loop and the fixed part of each tile, the epilogue (the
    chunk is 2^25 + 8192 K elements, so that each K has a grid of its own)."""
    import ctypes
    vdir = os.path.join(ROOT, "block_quantized_communication_amd", "variants")
    rpath = os.path.join(vdir, "resources.json")
    if not os.path.exists(rpath):
        raise RuntimeError("no receive variants: run python -m "
                           "block_quantized_communication_amd.build --variants")
    with open(rpath) as f:
        report = json.load(f)
    names = [n for n in report if report[n].get("group", "receive") == "receive" and
             os.path.exists(os.path.join(vdir, f"libzpq_{n}.so"))]
    if "default" not in names:
        raise RuntimeError("the default variant library is missing: run python -m "
                           "block_quantized_communication_amd.build --variants")
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    libs = {}
    for n in names:
        lib = ctypes.CDLL(os.path.join(vdir, f"libzpq_{n}.so"))
        lib.zpq_qgz_dequant_reduce_requant_i4.argtypes = [vp, vp, i32, i64, i32, vp, vp, vp, i32,
                                                          f32, vp]
        libs[n] = lib
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    st = torch.cuda.current_stream().cuda_stream
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)
    # (label, sources, chunk, block, float output: 0 INT4 / 1 fp16 / 2 bf16, divisor)
    W = [("c3 hop 1: 8 x 2^25 -> INT4, B=128", 8, 1 << 25, 128, 0, 1.0),
         ("c4 hop 2: 16 x 2^24 -> bf16 average, B=128", 16, 1 << 24, 128, 2, 16.0),
         ("c5 hop 1: 8 x 132M -> INT4, B=64", 8, 132120576, 64, 0, 1.0),
         ("c5 hop 2: 48 x 2.75M -> fp16 average, B=64", 48, 2752512, 64, 1, 384.0)]

    def buffers(K, c, B, fl):
        nbytes = K * (c // 2 + c // B * 4) + (c * 2 if fl else c // 2 + c // B * 4)
        sets = []
        for _ in range(n_sets(nbytes)):
            codes = torch.randint(0, 256, (K * c // 2,), dtype=torch.uint8, device=dev, generator=gen)
            scales = torch.rand(K * c // B, device=dev, generator=gen) * 1e-3 + 1e-6
            out = ((torch.empty(c, dtype=torch.int16, device=dev),) if fl else
                   (torch.empty(c // 2, dtype=torch.uint8, device=dev),
                    torch.empty(c // B, dtype=torch.float32, device=dev)))
            sets.append((codes, scales, out))
        return nbytes, sets

    def caller(lib, s, K, c, B, fl, div):
        codes, scales, out = s
        if fl:
            a = (codes.data_ptr(), scales.data_ptr(), K, c, B, None, None, out[0].data_ptr(), fl,
                 div, st)
        else:
            a = (codes.data_ptr(), scales.data_ptr(), K, c, B, out[0].data_ptr(),
                 out[1].data_ptr(), None, 0, 1.0, st)
        f = lib.zpq_qgz_dequant_reduce_requant_i4

        def run():
            rc = f(*a)
            if rc != 0:
                raise RuntimeError(f"receive launch failed ({rc})")
        return run

    rows = []
    for label, K, c, B, fl, div in W:
        nbytes, sets = buffers(K, c, B, fl)
        ref = None
        outs = {}
        for n in names:
            caller(libs[n], sets[0], K, c, B, fl, div)()
            torch.cuda.synchronize()
            outs[n] = [t.clone() for t in sets[0][2]]
        times = {n: [] for n in names}
        for rep in range(6):                       # all libraries in turn, then in reverse
            for n in (names if rep % 2 == 0 else names[::-1]):
                times[n] += launch_groups_us(torch, [caller(libs[n], x, K, c, B, fl, div)
                                                     for x in sets], 5, settle_s)
        ref = outs["default"]
        for n in names:
            epl, pf, nt, frag = receive_launch(report[n]["defines"], K, c, B, fl, cus)
            res = next((r for k, r in report[n]["kernels"].items() if frag in k), {})
            us = float(np.median(times[n]))
            rows.append({"workload": label, "variant": n, "defines": report[n]["defines"],
                         "elements_per_lane": epl, "sources_in_flight": pf,
                         "threads_per_workgroup": nt, "kernel_resources": res,
                         "us": round(us, 2), "frac_of_peak": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4),
                         "identical_to_default": all(torch.equal(a.view(torch.uint8), b.view(torch.uint8))
                                                     for a, b in zip(outs[n], ref))})
            print(f"[receive-shapes] {label} {n}: {us:.2f} us (EPL {epl}, {pf} in flight, "
                  f"{nt} threads, {res.get('vgprs')} VGPRs, {res.get('waves_per_simd')} waves/SIMD)",
                  file=sys.stderr, flush=True)
        del sets, outs
        torch.cuda.empty_cache()
    ksweep = []
    for K in (1, 2, 4, 8, 16):
        c, B = (1 << 25) + 8192 * K, 128            # a grid of its own per K, for the counters
        nbytes, sets = buffers(K, c, B, 0)
        us = float(np.median(launch_groups_us(torch, [caller(libs["default"], x, K, c, B, 0, 1.0)
                                                      for x in sets], 10, settle_s)))
        ksweep.append({"sources": K, "chunk": c, "block": B, "bytes": nbytes, "us": round(us, 2),
                       "frac_of_peak": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)})
        print(f"[receive-shapes] hop 1 K={K}: {us:.2f} us", file=sys.stderr, flush=True)
        del sets
        torch.cuda.empty_cache()
    return {"study": "receive-shapes", "rows": rows, "hop1_source_sweep": ksweep,
            "timing": f"per-launch time of {LAUNCHES} back-to-back launches between one HIP event "
                      "pair, buffer sets rotated; the libraries alternate in runs of 5 groups, 6 times "
                      "(forward, then backward); median of the 30 groups", "peak_GBps": HBM_PEAK_GBS}


def store_policy_study(np, torch, settle_s=0.1):
    """The cache-policy bits of streamed loads and stores on this GPU, and of
    the qgZ quantizer's code stores (bit 0 sc0, bit 1 nt, bit 4 sc1).
    (1) Read, write and copy streams of 1 GiB and 64 MiB through buffer
    loads and stores with each of the 8 values (the copy's loads keep nt),
    one and two 16-byte tiles per lane (bench_patterns.hip).  (2) The qgZ
    quantizer's bare access pattern with its code stores as non-temporal
    global stores or as buffer stores with each value.  (3) The quantizer
    itself: the default build (sc0 sc1 nt) against the QGZ_STORE_VARIANTS
    builds in block_quantized_communication_amd/variants/, outputs compared
    byte for byte, writing one output buffer and rotating over enough output
    buffers (>= 768 MiB) that none stays in the 256 MB last-level cache
    between two uses.  (2) and (3) on the 2^28 bf16 (L=8, N=4, B=128) and
    1.06G fp16 (L=8, N=48, B=64) workloads, inputs rotating over two copies."""
    import ctypes
    path = os.path.join(ROOT, "libbench_patterns.so")
    if not os.path.exists(path):
        raise RuntimeError("libbench_patterns.so is missing: run __graft_entry__.build()")
    vdir = os.path.join(ROOT, "block_quantized_communication_amd", "variants")
    rpath = os.path.join(vdir, "resources.json")
    if not os.path.exists(rpath):
        raise RuntimeError("no variant libraries: run python -m "
                           "block_quantized_communication_amd.build --variants")
    with open(rpath) as f:
        report = json.load(f)
    names = ["default"] + [n for n in report if report[n].get("group") == "qgz_store"]
    missing = [n for n in names if not os.path.exists(os.path.join(vdir, f"libzpq_{n}.so"))]
    if missing or len(names) < 2:
        raise RuntimeError(f"variant libraries missing ({missing or 'qgz_store'}): run python -m "
                           "block_quantized_communication_amd.build --variants")
    P = ctypes.CDLL(path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    P.pat_stream_pol.argtypes = [i32, i32, i32, vp, vp, i64, vp, vp]
    P.pat_reorder_quant_i4_pol.argtypes = [i32, vp, i64, i32, i32, i32, vp, vp, vp]
    P.pat_policy_bits.argtypes = [i32]
    libs = {}
    for n in names:
        lib = ctypes.CDLL(os.path.join(vdir, f"libzpq_{n}.so"))
        lib.zpq_qgz_reorder_quant_i4.argtypes = [vp, i32, i64, i32, i32, i32, vp, vp, vp]
        libs[n] = lib
    bits = [P.pat_policy_bits(i) for i in range(8)]

    def pol_name(b):
        return " ".join(x for x, m in (("sc0", 1), ("nt", 2), ("sc1", 16)) if b & m) or "none"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    st = torch.cuda.current_stream().cuda_stream
    sink = torch.zeros(256, dtype=torch.int32, device=dev)

    def check(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed ({rc})")
    # (1) streams
    streams = []
    for size in (1 << 30, 64 << 20):
        # Sources are only read, destinations only written: a line a store
        # leaves in the last-level cache is never read back.
        nbuf = max(1, -(-ROTATE_BYTES // size))
        srcs = [torch.full((size,), 1, dtype=torch.uint8, device=dev) for _ in range(nbuf)]
        dsts = [torch.empty(size, dtype=torch.uint8, device=dev) for _ in range(nbuf)]
        for kind, kname in ((0, "read"), (1, "write"), (2, "copy")):
            for tpl in (1, 2):
                for pol in range(8):
                    def mk(j, kind=kind, tpl=tpl, pol=pol):
                        a = (kind, pol, tpl, srcs[j].data_ptr(), dsts[j].data_ptr(), size,
                             sink.data_ptr(), st)
                        return lambda: check(P.pat_stream_pol(*a), "stream")
                    us = float(np.median(launch_groups_us(
                        torch, [mk(j) for j in range(nbuf)], 7, settle_s)))
                    moved = size * (2 if kind == 2 else 1)
                    streams.append({"stream": kname, "bytes": size, "tiles_per_lane": tpl,
                                    "policy": pol_name(bits[pol]), "us": round(us, 2),
                                    "frac_of_peak": round(moved / us / 1e3 / HBM_PEAK_GBS, 4)})
                print(f"[store-policy] {kname} {size >> 20} MiB, {tpl} tile(s) per lane: "
                      + ", ".join(f"{r['policy']} {r['frac_of_peak']:.3f}" for r in streams[-8:]),
                      file=sys.stderr, flush=True)
        del srcs, dsts
        torch.cuda.empty_cache()
    # (2) and (3) on the two qgZ quantizer workloads
    W = [("2^28 bf16, L=8, N=4, B=128", 1 << 28, 8, 4, 128, 2, 6),
         ("1.06G fp16, L=8, N=48, B=64", 1056964608, 8, 48, 64, 1, 3)]
    pattern_rows, kernel_rows = [], []
    gen = torch.Generator(device=dev)
    gen.manual_seed(12)
    for label, n, L, N, B, dt, nout in W:
        nbytes = n * 2 + n // 2 + n // B * 4
        xs = [(torch.randn(n, device=dev, generator=gen) * 1e-2).to(
            torch.bfloat16 if dt == 2 else torch.float16) for _ in range(2)]
        outs = [(torch.empty(n // 2, dtype=torch.uint8, device=dev),
                 torch.empty(n // B, dtype=torch.float32, device=dev)) for _ in range(nout)]
        # (2) pattern: -1 = non-temporal global stores, 0..7 = policies
        times = {p: [] for p in range(-1, 8)}
        for rep in range(2):
            for p in (range(-1, 8) if rep == 0 else reversed(range(-1, 8))):
                def mkp(i, p=p):
                    x, (cd, sc) = xs[i % 2], outs[i % nout]
                    a = (p, x.data_ptr(), n, L, N, B, cd.data_ptr(), sc.data_ptr(), st)
                    return lambda: check(P.pat_reorder_quant_i4_pol(*a), "pattern")
                times[p] += launch_groups_us(torch, [mkp(i) for i in range(2 * nout)], 5, settle_s)
        for p in range(-1, 8):
            us = float(np.median(times[p]))
            pattern_rows.append({"workload": label, "code_stores": "global nt" if p < 0 else
                                 "buffer " + pol_name(bits[p]), "us": round(us, 2),
                                 "frac_of_peak": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)})
        print(f"[store-policy] pattern {label}: " + ", ".join(
            f"{r['code_stores']} {r['us']}" for r in pattern_rows[-9:]), file=sys.stderr, flush=True)
        # (3) the kernel, per build: one output buffer, then rotating outputs
        ref = None
        same = {}
        for nm in names:
            cd, sc = outs[0]
            cd.zero_()
            sc.zero_()
            check(libs[nm].zpq_qgz_reorder_quant_i4(xs[0].data_ptr(), dt, n, L, N, B, cd.data_ptr(),
                                                    sc.data_ptr(), st), nm)
            torch.cuda.synchronize()
            got = (cd.clone(), sc.clone())
            ref = got if ref is None else ref
            same[nm] = all(torch.equal(a.view(torch.uint8), b.view(torch.uint8))
                           for a, b in zip(ref, got))
            del got
        for rot in (False, True):
            times = {nm: [] for nm in names}
            for rep in range(2):
                for nm in (names if rep == 0 else names[::-1]):
                    def mkk(i, nm=nm):
                        x, (cd, sc) = xs[i % 2], outs[i % nout if rot else 0]
                        a = (x.data_ptr(), dt, n, L, N, B, cd.data_ptr(), sc.data_ptr(), st)
                        f = libs[nm].zpq_qgz_reorder_quant_i4
                        return lambda: check(f(*a), nm)
                    times[nm] += launch_groups_us(torch, [mkk(i) for i in range(2 * nout)], 5,
                                                  settle_s)
            for nm in names:
                us = float(np.median(times[nm]))
                kernel_rows.append({"workload": label, "build": nm,
                                    "defines": report.get(nm, {}).get("defines", []),
                                    "outputs": f"{nout} rotating" if rot else "one",
                                    "us": round(us, 2),
                                    "frac_of_peak": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4),
                                    "identical_to_default": same[nm]})
            print(f"[store-policy] kernel {label}, {'rotating' if rot else 'one'} output(s): " +
                  ", ".join(f"{r['build']} {r['us']}" for r in kernel_rows[-len(names):]),
                  file=sys.stderr, flush=True)
        del xs, outs
        torch.cuda.empty_cache()
    return {"study": "store-policy", "streams": streams, "qgz_pattern": pattern_rows,
            "qgz_kernel": kernel_rows,
            "timing": f"per-launch time of {LAUNCHES} back-to-back launches between one HIP event "
                      "pair over rotating buffers; streams: median of 7 groups; pattern and kernel "
                      "variants alternate in runs of 5 groups, twice, median of the 10 groups",
            "peak_GBps": HBM_PEAK_GBS}


def timeline_summary(np, start_us, end_us, nbytes):
    """Occupancy and progress of one launch from its waves' start and end
    times (us from the first start).  The byte rate over time assumes each
    wave moves its share of the launch's bytes evenly over its lifetime (an
    estimate: a wave issues its loads ahead of its arithmetic)."""
    s, e = np.asarray(start_us, np.float64), np.asarray(end_us, np.float64)
    span, dt = float(e.max()), 0.05
    grid = np.arange(0.0, span + dt, dt)
    conc = np.zeros(len(grid))
    rate = np.zeros(len(grid))
    per = nbytes / len(s)
    i0 = (s / dt).astype(np.int64)
    i1 = (e / dt).astype(np.int64)
    for a, b, ls in zip(i0, i1, np.maximum(e - s, dt)):
        conc[a:b + 1] += 1
        rate[a:b + 1] += per / ls                  # bytes per us
    cum = np.cumsum(rate) * dt
    t90 = float(grid[min(len(grid) - 1, int(np.searchsorted(cum, 0.9 * nbytes)))])
    mid = rate[(grid > 0.2 * span) & (grid < 0.7 * span)]
    life = e - s
    return {"span_us": round(span, 2), "peak_waves": int(conc.max()),
            "mean_waves_over_peak": round(float(conc.mean() / conc.max()), 3),
            "wave_life_us_p10_p50_p90": [round(float(x), 2) for x in np.percentile(life, [10, 50, 90])],
            "last_wave_start_us": round(float(s.max()), 2),
            "last_10pct_of_bytes_us": round(span - t90, 2),
            "mid_launch_rate_frac_of_peak": round(float(np.median(mid)) / 1e3 / HBM_PEAK_GBS, 3),
            "avg_rate_frac_of_peak": round(nbytes / span / 1e3 / HBM_PEAK_GBS, 3)}


def timeline_study(np, torch, settle_s=0.2):
    """Every wave's start and end (the 100 MHz constant clock) in the four
    receive launches and in their bare access patterns: how full the GPU is
    over a launch, how long a wave lives, how fast bytes move mid-launch and
    how long the last tenth of them takes.  The kernel runs from the
    recording builds of block_quantized_communication_amd/variants/
    (timeline_w7 for the INT4 kernel, timeline for the float ones; the study
    reports their registers beside the shipped kernel's and their time with
    recording off beside libzpq's); the pattern is bench_patterns.hip's with
    parts 7.  Each launch is recorded alone and as the last of 20
    back-to-back launches.  First, bench_patterns.hip's residency probes: the
    most waves of one kernel a SIMD holds at once, by the kernel's scalar
    register count (64 VGPRs each)."""
    import ctypes
    vdir = os.path.join(ROOT, "block_quantized_communication_amd", "variants")
    rpath = os.path.join(vdir, "resources.json")
    ppath = os.path.join(ROOT, "libbench_patterns.so")
    if not os.path.exists(ppath):
        raise RuntimeError("libbench_patterns.so is missing: run __graft_entry__.build()")
    if not os.path.exists(rpath):
        raise RuntimeError("no variant libraries: run python -m "
                           "block_quantized_communication_amd.build --variants")
    with open(rpath) as f:
        report = json.load(f)
    for n in ("default", "timeline", "timeline_w7"):
        if n not in report or not os.path.exists(os.path.join(vdir, f"libzpq_{n}.so")):
            raise RuntimeError(f"variant library {n} missing: run python -m "
                               "block_quantized_communication_amd.build --variants")
    vp, i32, i64, f32, u32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_uint32
    libs = {}
    for n in ("default", "timeline", "timeline_w7"):
        lib = ctypes.CDLL(os.path.join(vdir, f"libzpq_{n}.so"))
        lib.zpq_qgz_dequant_reduce_requant_i4.argtypes = [vp, vp, i32, i64, i32, vp, vp, vp, i32,
                                                          f32, vp]
        if n != "default":
            lib.zpq_timeline_set.argtypes = [vp, u32]
        libs[n] = lib
    P = ctypes.CDLL(ppath)
    P.pat_receive.argtypes = [vp, vp, i32, i64, i32, vp, vp, vp, i32, i32, i32, vp]
    P.pat_timeline_set.argtypes = [vp, u32]
    P.pat_residency.argtypes = [i32, vp, u32, i32, vp]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    st = torch.cuda.current_stream().cuda_stream
    gen = torch.Generator(device=dev)
    gen.manual_seed(13)

    def check(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed ({rc})")
    # residency by scalar registers: 16 waves per SIMD of each probe
    residency = []
    rw = 16 * 4 * cus
    rbuf = torch.zeros(2 * rw, dtype=torch.int64, device=dev)
    for i in range(P.pat_residency_count()):
        rbuf.zero_()
        torch.cuda.synchronize()
        check(P.pat_residency(i, rbuf.data_ptr(), rw, 5, st), "residency probe")
        torch.cuda.synchronize()
        t = rbuf.view(rw, 2).cpu().numpy().astype(np.float64)
        if not ((t[:, 0] > 0) & (t[:, 1] >= t[:, 0])).all():
            raise RuntimeError("residency probe: waves not recorded")
        s0, e0 = t[:, 0] - t[:, 0].min(), t[:, 1] - t[:, 0].min()
        ev = np.concatenate([np.stack([s0, np.ones(rw)], 1), np.stack([e0, -np.ones(rw)], 1)])
        ev = ev[np.lexsort((ev[:, 1], ev[:, 0]))]            # ends before starts at equal times
        peak = int(np.cumsum(ev[:, 1]).max())
        residency.append({"sgprs_reported": P.pat_residency_sgprs(i), "vgprs": 64,
                          "peak_waves": peak, "waves_per_simd": round(peak / (4 * cus), 2)})
        print(f"[timeline] residency {residency[-1]}", file=sys.stderr, flush=True)
    del rbuf
    W = [("c3 hop 1: 8 x 2^25 -> INT4, B=128", 8, 1 << 25, 128, 0, 1.0),
         ("c4 hop 2: 16 x 2^24 -> bf16 average, B=128", 16, 1 << 24, 128, 2, 16.0),
         ("c5 hop 1: 8 x 132M -> INT4, B=64", 8, 132120576, 64, 0, 1.0),
         ("c5 hop 2: 48 x 2.75M -> fp16 average, B=64", 48, 2752512, 64, 1, 384.0)]
    rows = []
    for label, K, c, B, fl, div in W:
        nbytes = K * (c // 2 + c // B * 4) + (c * 2 if fl else c // 2 + c // B * 4)
        sets = []
        for _ in range(n_sets(nbytes)):
            codes = torch.randint(0, 256, (K * c // 2,), dtype=torch.uint8, device=dev, generator=gen)
            scales = torch.rand(K * c // B, device=dev, generator=gen) * 1e-3 + 1e-6
            out = ((torch.empty(c, dtype=torch.int16, device=dev),) if fl else
                   (torch.empty(c // 2, dtype=torch.uint8, device=dev),
                    torch.empty(c // B, dtype=torch.float32, device=dev)))
            sets.append((codes, scales, out))
        epl, pf, nt, frag = receive_launch([], K, c, B, fl, cus)
        probe = "timeline" if fl else "timeline_w7"
        waves = -(-c // (64 * epl))

        def kern(lib, x):
            codes, scales, out = x
            if fl:
                a = (codes.data_ptr(), scales.data_ptr(), K, c, B, None, None, out[0].data_ptr(),
                     fl, div, st)
            else:
                a = (codes.data_ptr(), scales.data_ptr(), K, c, B, out[0].data_ptr(),
                     out[1].data_ptr(), None, 0, 1.0, st)
            f = lib.zpq_qgz_dequant_reduce_requant_i4
            return lambda: check(f(*a), "receive")

        def pat(x):
            codes, scales, out = x
            a = (codes.data_ptr(), scales.data_ptr(), K, c, B, None if fl else out[0].data_ptr(),
                 None if fl else out[1].data_ptr(), out[0].data_ptr() if fl else None, epl, pf, 7, st)
            return lambda: check(P.pat_receive(*a), "pattern")
        res_of = lambda n: next((r for k, r in report[n]["kernels"].items() if frag in k), {})
        row = {"workload": label, "waves": waves, "elements_per_lane": epl, "sources_in_flight": pf,
               "bytes": nbytes, "probe_build": probe,
               "registers_shipped": res_of("default"), "registers_probe": res_of(probe)}
        times = {"default": [], probe: []}
        for rep in range(4):
            for n in (("default", probe) if rep % 2 == 0 else (probe, "default")):
                times[n] += launch_groups_us(torch, [kern(libs[n], x) for x in sets], 5, settle_s)
        row["libzpq_us"] = round(float(np.median(times["default"])), 2)
        row["probe_us_recording_off"] = round(float(np.median(times[probe])), 2)
        buf = torch.zeros(2 * waves, dtype=torch.int64, device=dev)
        for what, setter, fns in (("kernel", libs[probe].zpq_timeline_set,
                                   [kern(libs[probe], x) for x in sets]),
                                  ("pattern", P.pat_timeline_set, [pat(x) for x in sets])):
            check(setter(None, 0), "timeline reset")
            launch_groups_us(torch, fns, 1, settle_s)          # warm, recording off
            for mode in ("alone", "last_of_20"):
                buf.zero_()
                torch.cuda.synchronize()
                check(setter(ctypes.c_void_p(buf.data_ptr()), waves), "timeline set")
                for i in range(1 if mode == "alone" else LAUNCHES):
                    fns[i % len(fns)]()
                torch.cuda.synchronize()
                check(setter(None, 0), "timeline reset")
                t = buf.view(waves, 2).cpu().numpy().astype(np.float64)
                ok = (t[:, 0] > 0) & (t[:, 1] >= t[:, 0])
                if not ok.all():
                    raise RuntimeError(f"{label} {what}: {int((~ok).sum())} waves not recorded")
                t0 = t[:, 0].min()
                row[f"{what}_{mode}"] = timeline_summary(np, (t[:, 0] - t0) / 100.0,
                                                         (t[:, 1] - t0) / 100.0, nbytes)
            print(f"[timeline] {label} {what}: " + json.dumps(row[f"{what}_last_of_20"]),
                  file=sys.stderr, flush=True)
        rows.append(row)
        del sets, buf
        torch.cuda.empty_cache()
    return {"study": "timeline", "residency_by_sgprs": residency, "rows": rows, "clock_MHz": 100,
            "peak_GBps": HBM_PEAK_GBS}


def hop_count_study(np, torch, zpq, synth, S=1 << 20, B=128, seed=40):
    """Error of INT4 gradient averaging against the exact mean, as the world
    size W grows: qgZ's two hops (L = min(W, 8) local ranks, N = W/L nodes:
    every value is quantized twice) against a compressed ring reduce-scatter
    (the running partial sum is requantized at each of the W - 1 hops).  One
    slice of S elements per rank, gradients N(0, 1e-3) with a per-block
    variance multiplier 10^U(-2, 2) (the qgZ hop-1 workload's law), INT4 with
    block B, all steps on the GPU kernels.  The claim being measured: error
    that compounds with the hop count is why the pages replace reduce-scatter
    by an all-to-all (LIT-102 anthology record, Key takeaways)."""
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    rows = []
    for W in (2, 4, 8, 16, 32, 64, 128, 384):
        g = np.stack([synth.blockvar_normal(seed, 1000 + r, S, B, 1e-3, -2.0, 2.0)
                      for r in range(W)])                               # [W][S] fp32
        exact = g.astype(np.float64).mean(axis=0)
        gd = torch.from_numpy(g).to(dev)
        # every rank's slice quantized once (the send-side kernel, L = N = 1)
        q = [zpq.qgz_reorder_quant_i4(gd[r], 1, 1, B) for r in range(W)]
        # compressed ring: partial = requant(dequant(partial) + dequant(own)), W - 1 hops
        pc, ps = q[0]
        for r in range(1, W):
            cc = torch.cat([pc, q[r][0]])
            sc = torch.cat([ps, q[r][1]])
            pc, ps = zpq.qgz_dequant_reduce_requant_i4(cc, sc, 2, S, B)
        ring = zpq.qgz_dequant_reduce_requant_i4(pc, ps, 1, S, B, out_dtype=torch.float32,
                                                 divisor=float(W))
        # qgZ: hop 1 over L local ranks (requantize), hop 2 over N nodes (average)
        L = min(W, 8)
        N = W // L
        hop1 = []
        for m in range(N):
            cc = torch.cat([q[m * L + i][0] for i in range(L)])
            sc = torch.cat([q[m * L + i][1] for i in range(L)])
            hop1.append(zpq.qgz_dequant_reduce_requant_i4(cc, sc, L, S, B))
        cc = torch.cat([h[0] for h in hop1])
        sc = torch.cat([h[1] for h in hop1])
        qgz = zpq.qgz_dequant_reduce_requant_i4(cc, sc, N, S, B, out_dtype=torch.float32,
                                                divisor=float(W))
        torch.cuda.synchronize()
        scale = float(np.sqrt(np.mean(exact ** 2)))

        def err(y):
            d = y.cpu().numpy().astype(np.float64) - exact
            return round(float(np.sqrt(np.mean(d ** 2)) / scale), 5)
        rows.append({"W": W, "L": L, "N": N, "quantizations_qgz": 2,
                     "quantizations_ring": W, "rel_rms_err_qgz": err(qgz),
                     "rel_rms_err_ring": err(ring)})
        print(f"[study] W={W}: qgZ {rows[-1]['rel_rms_err_qgz']}, ring "
              f"{rows[-1]['rel_rms_err_ring']}", file=sys.stderr, flush=True)
    return {"study": "hop-count error: qgZ two-hop all-to-all vs compressed ring "
                     "reduce-scatter (INT4, block 128)", "slice_elems": S, "rows": rows,
            "error": "RMS(y - exact mean) / RMS(exact mean), fp64 reference"}


def per_config(np, torch, zpq, synth, groups=10):
    """Every kernel at every workload size, alone: kernel time as everywhere
    in this file (LAUNCHES back-to-back launches per HIP event pair, median
    over `groups`), each launch on its own buffer set among enough copies
    that ROTATE_BYTES pass between two uses of one.  Inputs are the
    workloads' generators; the receive buffers of the hop kernels are filled
    by the send-side kernels (timing needs realistic codes, not oracle
    values: parity at these sizes is the GPU tests' job)."""
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    T = torch
    rows = []
    e = lambda n, dt: torch.empty(n, dtype=dt, device=dev)

    def timed(label, nbytes, make):
        """make(i) -> a callable launching on buffer set i (set 0 may reuse inputs)."""
        fns = [make(i) for i in range(n_sets(nbytes))]
        med, mn = launch_time_us(np, torch, fns, groups)
        rows.append({"kernel": label, "bytes": int(nbytes), "us_median": round(med, 2),
                     "us_min": round(mn, 2), "buffer_sets": len(fns),
                     "GBps": round(nbytes / med / 1e3, 1),
                     "frac_of_peak": round(nbytes / med / 1e3 / HBM_PEAK_GBS, 4)})
        print(f"[per-config] {label}: {med:.2f} us, {nbytes / med / 1e3:.0f} GB/s "
              f"({len(fns)} buffer sets)", file=sys.stderr, flush=True)
        del fns
        torch.cuda.empty_cache()

    def copy_of(t, i):
        return t if i == 0 else t.clone()

    # c1: qwZ round trip, 2^20 fp16, B = 256 (launch-bound)
    c = synth.QWZ_ROUNDTRIP
    n, B = c["n"], c["block"]
    x = torch.from_numpy(synth.qwz_roundtrip()).to(dev)
    cc, cs = zpq.quant_i8(x, B)
    nb = n * 2 + n + n // B * 4

    def c1_quant(i):
        xi, o = copy_of(x, i), (e(n, T.int8), e(n // B, T.float32))
        return lambda: zpq.quant_i8(xi, B, out=o)

    def c1_dequant(i):
        ci, si, y = copy_of(cc, i), copy_of(cs, i), e(n, T.float16)
        return lambda: zpq.dequant_i8(ci, si, B, out=y)
    timed("c1 K1 quant_i8 2^20 fp16 B=256", nb, c1_quant)
    timed("c1 K2 dequant_i8 2^20 -> fp16", nb, c1_dequant)
    del x, cc, cs
    # c2: qwZ on the h8192 layer, 16 ranks
    c = synth.QWZ_LAYER
    n, B, W = c["n"], c["block"], c["world"]
    S = n // W
    layer = torch.from_numpy(synth.qwz_layer()).to(dev)

    def c2_quant(i):                    # rank i's shard
        o = (e(S, T.int8), e(S // B, T.float32))
        return lambda: zpq.quant_i8(layer[i * S:(i + 1) * S], B, out=o)
    timed("c2 K1 quant_i8 shard 50.3M fp16 B=256", S * 3 + S // B * 4, c2_quant)
    gc, gs = zpq.quant_i8(layer, B)
    del layer
    y = e(n, T.float16)
    timed("c2 K2 dequant_i8 gathered 805M -> fp16", n * 3 + n // B * 4,
          lambda i: (lambda: zpq.dequant_i8(gc, gs, B, out=y)))
    del gc, gs, y
    # c3: qgZ hop 1, bf16 2^28, L = 8, N = 4, B = 128
    c = synth.QGZ_HOP1
    n, B, L, N = c["n"], c["block"], c["L"], c["N"]
    chunk = n // L
    g = torch.from_numpy(synth.qgz_hop1()).view(T.bfloat16).to(dev)
    c1, s1 = e(n // 2, T.uint8), e(n // B, T.float32)
    timed("c3 K3 reorder_quant_i4 2^28 bf16 L=8 N=4 B=128", n * 2 + n // 2 + n // B * 4,
          lambda i: (lambda: zpq.qgz_reorder_quant_i4(g, L, N, B, out=(c1, s1))))
    del g

    def c3_hop1(i):
        ci, si = copy_of(c1, i), copy_of(s1, i)
        o = (e(chunk // 2, T.uint8), e(chunk // B, T.float32))
        return lambda: zpq.qgz_dequant_reduce_requant_i4(ci, si, L, chunk, B, out=o)
    timed("c3 K4 hop-1 8 x 2^25 -> INT4",
          L * (chunk // 2 + chunk // B * 4) + chunk // 2 + chunk // B * 4, c3_hop1)
    del c1, s1
    # c4: qgZ hop 2, 16 sources x 2^24, bf16 average
    c = synth.QGZ_HOP2
    K, chunk, B = c["sources"], c["chunk"], c["block"]
    src = torch.from_numpy(np.concatenate([synth.qgz_hop2_source(i) for i in range(K)])).to(dev)
    ic, isc = zpq.qgz_reorder_quant_i4(src, 1, 1, B)
    del src

    def c4_hop2(i):
        ci, si, yv = copy_of(ic, i), copy_of(isc, i), e(chunk, T.bfloat16)
        return lambda: zpq.qgz_dequant_reduce_requant_i4(ci, si, K, chunk, B,
                                                         out_dtype=T.bfloat16,
                                                         divisor=c["divisor"], out=yv)
    timed("c4 K5 hop-2 16 x 2^24 -> bf16 average", K * (chunk // 2 + chunk // B * 4) + chunk * 2,
          c4_hop2)
    del ic, isc
    # c5: fused qgZ on the 138B-model layer gradient, L = 8, N = 48, B = 64
    c = synth.QGZ_FUSED
    n, B, L, N = c["n"], c["block"], c["L"], c["N"]
    W = L * N
    S, chunk = n // W, n // L
    g = torch.from_numpy(synth.qgz_fused()).to(dev)
    c1, s1 = e(n // 2, T.uint8), e(n // B, T.float32)
    timed("c5 K3 reorder_quant_i4 1.06G fp16 L=8 N=48 B=64", n * 2 + n // 2 + n // B * 4,
          lambda i: (lambda: zpq.qgz_reorder_quant_i4(g, L, N, B, out=(c1, s1))))
    del g
    c2, s2 = zpq.qgz_dequant_reduce_requant_i4(c1, s1, L, chunk, B)

    def c5_hop1(i):
        ci, si = copy_of(c1, i), copy_of(s1, i)
        o = (e(chunk // 2, T.uint8), e(chunk // B, T.float32))
        return lambda: zpq.qgz_dequant_reduce_requant_i4(ci, si, L, chunk, B, out=o)
    timed("c5 K4 hop-1 8 x 132M -> INT4",
          L * (chunk // 2 + chunk // B * 4) + chunk // 2 + chunk // B * 4, c5_hop1)
    del c1, s1

    def c5_hop2(i):
        ci, si, yv = copy_of(c2, i), copy_of(s2, i), e(S, T.float16)
        return lambda: zpq.qgz_dequant_reduce_requant_i4(ci, si, N, S, B, out_dtype=T.float16,
                                                         divisor=float(W), out=yv)
    timed("c5 K5 hop-2 48 x 2.75M -> fp16 average", N * (S // 2 + S // B * 4) + S * 2, c5_hop2)
    return {"per_config": rows,
            "timing": f"per-launch time of {LAUNCHES} back-to-back launches between one HIP event "
                      f"pair, median of {groups} groups; launches rotate over buffer sets so that "
                      f">= {ROTATE_BYTES >> 20} MiB pass between two uses of one",
            "peak_GBps": HBM_PEAK_GBS}


def patterns(np, torch, zpq, synth, settle_s=0.1):
    """Each kernel at each workload size beside its bare access pattern, and
    the streaming ceilings.  The pattern kernels (bench_patterns.hip) issue
    the same per-lane loads and stores as the kernel -- widths, cache hints,
    lane layout, tiles per lane, sources in flight, grid, slice reorder --
    with XOR in place of the arithmetic.  Timing as --per-config (back-to-back
    launches over rotating buffer sets); kernel and pattern alternate in runs
    of 5 groups, twice, so that both see the same clock state."""
    import ctypes
    path = os.path.join(ROOT, "libbench_patterns.so")
    if not os.path.exists(path):
        raise RuntimeError("libbench_patterns.so is missing: run __graft_entry__.build()")
    P = ctypes.CDLL(path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    P.pat_read.argtypes = [vp, i64, vp, vp]
    P.pat_write.argtypes = [vp, i64, vp]
    P.pat_copy.argtypes = [vp, vp, i64, vp]
    P.pat_quant_i8.argtypes = [vp, i64, vp, vp, vp]
    P.pat_dequant_i8.argtypes = [vp, vp, i64, vp, vp]
    P.pat_reorder_quant_i4.argtypes = [vp, i64, i32, i32, i32, vp, vp, vp]
    P.pat_receive.argtypes = [vp, vp, i32, i64, i32, vp, vp, vp, i32, i32, i32, vp]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    T = torch
    st = torch.cuda.current_stream()
    S_ = ctypes.c_void_p(st.cuda_stream)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    null = ctypes.c_void_p(0)
    e = lambda n, dt: torch.empty(n, dtype=dt, device=dev)
    cus = torch.cuda.get_device_properties(0).multi_processor_count

    def ok(rc):
        if rc != 0:
            raise RuntimeError(f"pattern launch failed ({rc})")

    def time_pair(makes, nbytes):
        """Median per-launch microseconds of each of the given launch families
        (make(i) -> callable on buffer set i), alternating 5 groups each, twice."""
        fam = [[m(i) for i in range(n_sets(nbytes))] for m in makes]
        us = [[] for _ in fam]
        for _ in range(2):
            for k, fns in enumerate(fam):
                us[k] += launch_groups_us(torch, fns, 5, settle_s)
        del fam
        return [float(np.median(u)) for u in us]

    rows = []

    def read_stream(nbytes):
        """A plain read stream of (about) `nbytes` -- the streaming ceiling at
        the kernel's own size, where the launch's ramp-up and drain weigh as
        much as they do for the kernel -- on its own buffer sets."""
        n16 = -(-int(nbytes) // (16 * 2 * 256)) * (2 * 256)
        bufs = [e(n16 * 4, T.float32).fill_(1.0) for _ in range(n_sets(n16 * 16))]
        return n16 * 16, [(lambda b=b: ok(P.pat_read(ptr(b), n16 * 16, ptr(sink), S_))) for b in bufs]

    def row(label, nbytes, make_k, make_p, parts=None):
        """parts: for the receive kernels, make(i, parts) of the pattern with
        only some of its accesses (bit 0 the scale loads, bit 1 the stores)."""
        fams = [make_k, make_p]
        if parts:
            fams += [lambda i, b=b: parts(i, b) for b in (2, 1, 0)]
        us = time_pair(fams, nbytes)
        k_us, p_us = us[0], us[1]
        rb, fns = read_stream(nbytes)
        r_us = float(np.median(launch_groups_us(torch, fns, 10, settle_s)))
        del fns
        r = {"kernel": label, "bytes": int(nbytes), "kernel_us": round(k_us, 2),
             "pattern_us": round(p_us, 2),
             "kernel_frac_of_peak": round(nbytes / k_us / 1e3 / HBM_PEAK_GBS, 4),
             "pattern_frac_of_peak": round(nbytes / p_us / 1e3 / HBM_PEAK_GBS, 4),
             "kernel_over_pattern": round(k_us / p_us, 3),
             "read_stream_bytes": rb, "read_stream_us": round(r_us, 2),
             "read_stream_frac_of_peak": round(rb / r_us / 1e3 / HBM_PEAK_GBS, 4)}
        if parts:
            r.update({"pattern_without_scale_loads_us": round(us[2], 2),
                      "pattern_without_stores_us": round(us[3], 2),
                      "pattern_code_loads_only_us": round(us[4], 2)})
        rows.append(r)
        extra = (f"; without scale loads {us[2]:.2f}, without stores {us[3]:.2f}, code loads "
                 f"only {us[4]:.2f}") if parts else ""
        print(f"[patterns] {label}: kernel {k_us:.2f} us, pattern {p_us:.2f} us, "
              f"read stream of the same size {r_us:.2f} us{extra}", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()

    cp = lambda t, i: t if i == 0 else t.clone()

    def receive_shape(c, K, fl):
        if not fl:
            return 32, 2
        waves16 = (c + 16 * 64 - 1) // (16 * 64)
        return (8, 4) if waves16 < 8 * 4 * cus else (16, 2)

    # ceilings: 1 GiB streams (no reuse within the last-level cache)
    nb = 1 << 30
    a, b = e(nb // 4, T.float32), e(nb // 4, T.float32)
    a.fill_(1.0)
    sink = e(256, T.int32)
    ceil = {}
    for name, f, moved in (("read", lambda i: (lambda: ok(P.pat_read(ptr(a), nb, ptr(sink), S_))), nb),
                           ("write", lambda i: (lambda: ok(P.pat_write(ptr(b), nb, S_))), nb),
                           ("copy", lambda i: (lambda: ok(P.pat_copy(ptr(a), ptr(b), nb, S_))),
                            2 * nb)):
        (us,) = time_pair([f], moved)
        ceil[name] = {"bytes": moved, "us": round(us, 2), "GBps": round(moved / us / 1e3, 1),
                      "frac_of_peak": round(moved / us / 1e3 / HBM_PEAK_GBS, 4)}
        print(f"[patterns] {name} ceiling: {moved / us / 1e3:.0f} GB/s", file=sys.stderr, flush=True)
    del a, b

    # c2: qwZ on the h8192 layer (buffer set i: rank i's shard)
    c = synth.QWZ_LAYER
    n, B, W = c["n"], c["block"], c["world"]
    S = n // W
    layer = torch.from_numpy(synth.qwz_layer()).to(dev)

    def k1_kernel(i):
        o = (e(S, T.int8), e(S // B, T.float32))
        return lambda: zpq.quant_i8(layer[i * S:(i + 1) * S], B, out=o)

    def k1_pattern(i):
        o = (e(S, T.int8), e(S // B, T.float32))
        return lambda: ok(P.pat_quant_i8(ptr(layer[i * S:]), S, ptr(o[0]), ptr(o[1]), S_))
    row("c2 K1 quant_i8 shard 50.3M fp16 B=256", S * 3 + S // B * 4, k1_kernel, k1_pattern)
    gc, gs = zpq.quant_i8(layer, B)
    del layer
    y, py = e(n, T.float16), e(n, T.float16)
    row("c2 K2 dequant_i8 gathered 805M -> fp16", n * 3 + n // B * 4,
        lambda i: (lambda: zpq.dequant_i8(gc, gs, B, out=y)),
        lambda i: (lambda: ok(P.pat_dequant_i8(ptr(gc), ptr(gs), n, ptr(py), S_))))
    del gc, gs, y, py

    def qgz_rows(g, dt_bytes, L, N, B, out_dt, fl2_label, fl1_label, k3_label):
        n = g.numel()
        W = L * N
        S, chunk = n // W, n // L
        c1, s1, p1, q1 = e(n // 2, T.uint8), e(n // B, T.float32), e(n // 2, T.uint8), e(n // B, T.float32)
        row(k3_label, n * dt_bytes + n // 2 + n // B * 4,
            lambda i: (lambda: zpq.qgz_reorder_quant_i4(g, L, N, B, out=(c1, s1))),
            lambda i: (lambda: ok(P.pat_reorder_quant_i4(ptr(g), n, L, N, B, ptr(p1), ptr(q1), S_))))
        del p1, q1
        c2, s2 = zpq.qgz_dequant_reduce_requant_i4(c1, s1, L, chunk, B)
        epl, pf = receive_shape(chunk, L, False)

        def h1_kernel(i):
            ci, si = cp(c1, i), cp(s1, i)
            o = (e(chunk // 2, T.uint8), e(chunk // B, T.float32))
            return lambda: zpq.qgz_dequant_reduce_requant_i4(ci, si, L, chunk, B, out=o)

        def h1_pattern(i, parts=3):
            ci, si = cp(c1, i), cp(s1, i)
            o = (e(chunk // 2, T.uint8), e(chunk // B, T.float32))
            return lambda: ok(P.pat_receive(ptr(ci), ptr(si), L, chunk, B, ptr(o[0]), ptr(o[1]),
                                            null, epl, pf, parts, S_))
        row(fl1_label, L * (chunk // 2 + chunk // B * 4) + chunk // 2 + chunk // B * 4,
            h1_kernel, h1_pattern, h1_pattern)
        if fl2_label:
            epl2, pf2 = receive_shape(S, N, True)

            def h2_kernel(i):
                ci, si, yv = cp(c2, i), cp(s2, i), e(S, out_dt)
                return lambda: zpq.qgz_dequant_reduce_requant_i4(ci, si, N, S, B, out_dtype=out_dt,
                                                                 divisor=float(W), out=yv)

            def h2_pattern(i, parts=3):
                ci, si, yv = cp(c2, i), cp(s2, i), e(S, out_dt)
                return lambda: ok(P.pat_receive(ptr(ci), ptr(si), N, S, B, null, null, ptr(yv),
                                                epl2, pf2, parts, S_))
            row(fl2_label, N * (S // 2 + S // B * 4) + S * 2, h2_kernel, h2_pattern, h2_pattern)

    # c3: qgZ hop 1
    c = synth.QGZ_HOP1
    g = torch.from_numpy(synth.qgz_hop1()).view(T.bfloat16).to(dev)
    qgz_rows(g, 2, c["L"], c["N"], c["block"], None, None,
             "c3 K4 hop-1 8 x 2^25 -> INT4", "c3 K3 reorder_quant_i4 2^28 bf16 L=8 N=4 B=128")
    del g
    # c4: qgZ hop 2, 16 x 2^24 -> bf16
    c = synth.QGZ_HOP2
    K, chunk, B = c["sources"], c["chunk"], c["block"]
    src = torch.from_numpy(np.concatenate([synth.qgz_hop2_source(i) for i in range(K)])).to(dev)
    ic, isc = zpq.qgz_reorder_quant_i4(src, 1, 1, B)
    del src
    epl, pf = receive_shape(chunk, K, True)

    def c4_kernel(i):
        ci, si, yv = cp(ic, i), cp(isc, i), e(chunk, T.bfloat16)
        return lambda: zpq.qgz_dequant_reduce_requant_i4(ci, si, K, chunk, B, out_dtype=T.bfloat16,
                                                         divisor=c["divisor"], out=yv)

    def c4_pattern(i, parts=3):
        ci, si, yv = cp(ic, i), cp(isc, i), e(chunk, T.bfloat16)
        return lambda: ok(P.pat_receive(ptr(ci), ptr(si), K, chunk, B, null, null, ptr(yv), epl, pf,
                                        parts, S_))
    row("c4 K5 hop-2 16 x 2^24 -> bf16 average", K * (chunk // 2 + chunk // B * 4) + chunk * 2,
        c4_kernel, c4_pattern, c4_pattern)
    del ic, isc
    # c5: fused qgZ
    c = synth.QGZ_FUSED
    g = torch.from_numpy(synth.qgz_fused()).to(dev)
    qgz_rows(g, 2, c["L"], c["N"], c["block"], T.float16,
             "c5 K5 hop-2 48 x 2.75M -> fp16 average", "c5 K4 hop-1 8 x 132M -> INT4",
             "c5 K3 reorder_quant_i4 1.06G fp16 L=8 N=48 B=64")
    return {"patterns": rows, "ceilings_1GiB": ceil,
            "read_stream": "per row, a plain read stream (16-byte non-temporal loads, two tiles "
                           "per lane) of the kernel's algorithmic bytes, timed the same way",
            "timing": f"per-launch time of {LAUNCHES} back-to-back launches between one HIP event "
                      f"pair; launches rotate over buffer sets (>= {ROTATE_BYTES >> 20} MiB between "
                      "two uses of one); kernel and pattern alternate in runs of 5 groups, twice; "
                      "median of the 10 groups", "peak_GBps": HBM_PEAK_GBS}


VALU_KINDS = [
    ("v_add_f32", "op"), ("v_mul_f32", "op"), ("v_fma_f32", "op"), ("v_cvt_f32_ubyte1", "op"),
    ("v_cvt_off_f32_i4", "op"), ("v_cvt_f32_i32 (SDWA byte select)", "op"), ("v_and_b32", "op"),
    ("v_lshrrev_b32", "op"), ("v_bitop3_b32", "op"), ("v_perm_b32", "op"), ("v_max3_f32", "op"),
    ("v_fma_mix_f32", "op"), ("v_cvt_pk_f32_fp8 (two results)", "op"), ("v_mul_f64", "op"),
    ("cvt_f32_ubyte + fma + add (the receive loop's form)", "seq"),
    ("cvt_f32_ubyte + mul + add", "seq"),
    ("cvt_off_f32_i4 (SDWA byte select) + mul + add", "seq"),
    ("fma_mix (16-bit operand) + add", "seq"),
    ("mov + mul + add (no conversion)", "seq"),
]


def valu_rates(np, torch, waves_per_simd=(4, 8), iters=2000):
    """Issue rate of the vector ALU per instruction kind, and per element for
    the per-element instruction sequences a dequantize-and-add loop can use.
    Register-only kernels (bench_patterns.hip): 8 independent chains per
    lane, nothing but the measured instructions in the loop.  One launch per
    kind and occupancy, HIP events around it, best of 3 (each launch runs
    for a millisecond or more, so the event overhead is negligible)."""
    import ctypes
    path = os.path.join(ROOT, "libbench_patterns.so")
    if not os.path.exists(path):
        raise RuntimeError("libbench_patterns.so is missing: run __graft_entry__.build()")
    P = ctypes.CDLL(path)
    P.pat_valu.argtypes = [ctypes.c_int, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                           ctypes.c_void_p]
    P.pat_valu_instr_per_step.argtypes = [ctypes.c_int]
    nk = P.pat_valu_kinds()
    if nk != len(VALU_KINDS):
        raise RuntimeError(f"bench_patterns.hip has {nk} VALU kinds, bench.py names {len(VALU_KINDS)}")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    simds = cus * 4
    st = torch.cuda.current_stream()
    rows = []
    for wps in waves_per_simd:
        wgs = simds * wps // 4                      # 4 waves per 256-thread workgroup
        out = torch.empty(wgs * 256, dtype=torch.int32, device=dev)
        for k, (name, kind) in enumerate(VALU_KINDS):
            ips = P.pat_valu_instr_per_step(k)
            rc = P.pat_valu(k, wgs, 10, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(st.cuda_stream))
            if rc != 0:
                raise RuntimeError(f"VALU kernel {k} failed to launch ({rc})")
            torch.cuda.synchronize()
            best = None
            for _ in range(3):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(st)
                P.pat_valu(k, wgs, iters, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(st.cuda_stream))
                b.record(st)
                torch.cuda.synchronize()
                ms = a.elapsed_time(b)
                best = ms if best is None else min(best, ms)
            steps_per_simd = wps * iters * 32          # inner steps (one element each) per SIMD
            ns = best * 1e6
            row = {"kind": name, "what": kind, "waves_per_simd": wps, "ms": round(best, 4),
                   "instr_per_ns_per_simd": round(steps_per_simd * ips / ns, 4),
                   "cycles_per_instr_at_2p4GHz": round(ns * 2.4 / (steps_per_simd * ips), 3)}
            if kind == "seq":
                row["cycles_per_element_at_2p4GHz"] = round(ns * 2.4 / steps_per_simd, 3)
            rows.append(row)
            print(f"[valu] {wps} waves/SIMD  {name}: {row['cycles_per_instr_at_2p4GHz']} cycles/instr",
                  file=sys.stderr, flush=True)
        del out
    return {"valu_rates": rows, "simds": simds,
            "note": "a wave64 instruction on a 16-lane SIMD takes 4 cycles when issued alone; "
                    "fewer cycles per instruction mean two waves' instructions issued together"}


def blocking_study(np, torch, zpq, synth):
    """INT8 weight quantization with one scale per tensor against one scale
    per block (the summary page's ablation: non-blocked quantization of the
    weights hurt, block-based did not).  Reconstruction error of both on the
    outlier tensor (fp16 N(0, 0.02) with 0.1% N(0, 1) outliers) and on the
    layer shard (fp16 N(0, 0.02)); kernel throughput of both on the shard.
    The GPU kernels quantize and dequantize; the error is taken in fp64."""
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cases = {"outliers_2^20": synth.qwz_roundtrip(), "layer_shard": synth.qwz_shard(0)}
    rows = []
    for name, x in cases.items():
        xd = torch.from_numpy(x).to(dev)
        ref = x.astype(np.float64)
        scale = float(np.sqrt(np.mean(ref ** 2)))

        def err(y):
            d = y.cpu().numpy().astype(np.float64) - ref
            return {"rel_rms_err": round(float(np.sqrt(np.mean(d ** 2)) / scale), 6),
                    "max_abs_err": float(np.abs(d).max())}
        c, s1 = zpq.quant_i8_tensor(xd)
        r = {"tensor": name, "n": int(x.size),
             # the one scale repeated per 256-block: the same products fl32(q * s)
             "per_tensor": err(zpq.dequant_i8(c, s1.expand(x.size // 256).contiguous(), 256,
                                              torch.float16))}
        for B in (32, 64, 128, 256, 512):
            c, s = zpq.quant_i8(xd, B)
            r[f"block_{B}"] = err(zpq.dequant_i8(c, s, B, torch.float16))
        rows.append(r)
        print(f"[study] {name}: per-tensor {r['per_tensor']['rel_rms_err']}, block 256 "
              f"{r['block_256']['rel_rms_err']}", file=sys.stderr, flush=True)
    x = torch.from_numpy(cases["layer_shard"]).to(dev)
    n = x.numel()
    timing = {}
    for label, nbytes, make in (
            ("block_256", 3 * n + n // 64,
             lambda i: (lambda xi=x if i == 0 else x.clone(),
                        o=(torch.empty(n, dtype=torch.int8, device=dev),
                           torch.empty(n // 256, dtype=torch.float32, device=dev)):
                        zpq.quant_i8(xi, 256, out=o))),
            ("per_tensor", 3 * n,
             lambda i: (lambda xi=x if i == 0 else x.clone(),
                        o=(torch.empty(n, dtype=torch.int8, device=dev),
                           torch.empty(1, dtype=torch.float32, device=dev)):
                        zpq.quant_i8_tensor(xi, out=o)))):
        fns = [make(i) for i in range(n_sets(nbytes))]
        us, _ = launch_time_us(np, torch, fns, 10)
        del fns
        timing[label] = {"us_per_call": round(us, 2),
                         "effective_GBps": round(nbytes / us / 1e3, 1)}
    return {"study": "INT8 weight quantization: per-tensor scale vs per-block scales",
            "rows": rows, "quantize_timing_layer_shard": timing,
            "effective_bytes": "2n read + n codes written (+ scales), whatever the passes",
            "error": "RMS(dequant(quant(x)) - x) / RMS(x) in fp64; max |error|"}


def host_cpu():
    """CPU model and core counts of the host the oracle ran on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = None
    return {"cpu_model": model, "nproc": usable, "os_cpu_count": os.cpu_count(),
            "threads_used": 1}


def cpu_baseline(np, layer_h, grad_h, frac):
    """The oracle (plain single-threaded C) on a fraction of every kernel's
    step work, same block sizes and the same L, N; GB/s over the same
    algorithmic bytes as the GPU step."""
    import oracle
    import synth
    qw, qg = synth.QWZ_LAYER, synth.QGZ_FUSED
    Bw = qw["block"]
    L, N, B = qg["L"], qg["N"], qg["block"]
    W = L * N
    n1 = int(qw["n"] // qw["world"] * frac) // Bw * Bw
    n2 = int(qw["n"] * frac) // Bw * Bw
    n3 = int(qg["n"] * frac) // (W * B) * (W * B)
    c4, c5 = n3 // L, n3 // W
    gc, gs = oracle.quant_i8(layer_h[:n2], "f16", Bw)        # K2's input: not timed

    def timed(fn):
        t = time.perf_counter()
        r = fn()
        return r, time.perf_counter() - t

    secs = 0.0
    _, dt = timed(lambda: oracle.quant_i8(layer_h[:n1], "f16", Bw))
    secs += dt
    _, dt = timed(lambda: oracle.dequant_i8(gc, gs, Bw, "f16"))
    secs += dt
    (c1, s1), dt = timed(lambda: oracle.qgz_reorder_quant_i4(grad_h[:n3], "f16", L, N, B))
    secs += dt
    (c2, s2), dt = timed(lambda: oracle.qgz_dequant_reduce_requant_i4(c1, s1, L, c4, B))
    secs += dt
    _, dt = timed(lambda: oracle.qgz_dequant_reduce_requant_i4(c2, s2, N, c5, B, "f16",
                                                               float(W)))
    secs += dt
    nbytes = ((n1 * 2 + n1 + (n1 // Bw) * 4) + (n2 + (n2 // Bw) * 4 + n2 * 2) +
              (n3 * 2 + n3 // 2 + (n3 // B) * 4) +
              (L * (c4 // 2 + (c4 // B) * 4) + c4 // 2 + (c4 // B) * 4) +
              (N * (c5 // 2 + (c5 // B) * 4) + c5 * 2))
    return {"value": round(nbytes / secs / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "host": host_cpu(),
            "sample": f"{frac:.4g} of every kernel's step work (qwZ shard {n1} and gathered "
                      f"{n2} elements, qgZ gradient {n3} elements, hop-1 chunk {c4}, hop-2 "
                      f"slice {c5}; same blocks, L, N); {secs:.1f} s of single-threaded oracle "
                      f"time"}


if __name__ == "__main__":
    main()

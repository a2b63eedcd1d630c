#!/usr/bin/env python3
"""Benchmark: affine Q4 group-32 weight stream of the 32-layer temporal step, M=1.

One "step" is one pass of the whole hot path over one synthetic frame: the 32
temporal layers' 224 quantized GEMVs (per layer q, k, v, o 4096x4096; gate, up
11264x4096; down 4096x11264), run as 128 ordered stages (q/k/v share the
attention input, gate/up share the FFN input). Weights and activations are
seeded synthetic stand-ins for the model's (``workloads``), packed on the GPU
before timing; the timed region starts with everything resident in HBM.

Prints ONE JSON line (rank 0, N=1):
  value        packed-weight GB/s over the step (algorithmic bytes: 4-bit codes
               + bf16 scale + bf16 bias per 32 weights = 0.625 B/weight)
  ms_per_step  wall time per step (HIP events on the launch stream)
  roofline     the dominant kernel (the persistent chain kernel: one launch
               per step) against the 8 TB/s HBM peak
  cpu_baseline the CPU oracle on a bounded sample of the same workload

Executors: ``--mode chain`` (default: one persistent launch per step) or
``--mode launches`` (224 q4_gemv launches per step, replayed as a HIP graph).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0

# HBM traffic of one chain_kernel launch over the full step, from two rocprofv3
# --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch),
# each scaled by what the same counter reads for a plain 1 GiB copy
# (``--calibrate-copy 1024``: FETCH_SIZE reads 524301.6 KiB for 1 GiB fetched,
# WRITE_SIZE 1048576.0 KiB for 1 GiB written). Valid only for the kernel sources
# whose hash is recorded: any change to them reports traffic as null until the
# counters are taken again (profiles/chain_kernel_temporal_step_m1_pmc.md).
CHAIN_TRAFFIC = {
    "sources_sha256_16": "28a53d59b1e310e0",
    "fetch_kib": 2013940.8, "fetch_scale": 1048576.0 / 524301.6,
    "write_kib": 3072.0, "write_scale": 1048576.0 / 1048576.0,
}
KERNEL_SOURCES = ("q4_chain.h", "q4_kernels.h", "q4_api.hip")
METRIC = "packed-weight GB/s (% HBM peak) + us per 32-layer Q4 temporal step, M=1"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def packed_bytes(n: int, k: int) -> int:
    """Stored bytes of an [n, k] Q4 matrix: k/2 code bytes + 2 bf16 per 32 per row."""
    return n * k // 2 + 2 * 2 * n * (k // 32)


def kernel_sources_hash() -> str:
    """sha256[:16] of the kernel sources with // comments and blank space
    removed (an edit to a comment does not change the kernels)."""
    import hashlib
    import re

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "bit_group_quantized_amd", "csrc", f), encoding="utf-8") as fh:
            text = fh.read()
        code = [re.sub(r"//.*$", "", line).strip() for line in text.splitlines()]
        h.update("\n".join(line for line in code if line).encode())
    return h.hexdigest()[:16]


def chain_traffic_bytes(full_step: bool):
    """Measured HBM bytes per chain launch, or None when the counters do not
    belong to this kernel build or this workload."""
    t = CHAIN_TRAFFIC
    if not full_step or kernel_sources_hash() != t["sources_sha256_16"]:
        return None
    return int(round(1024 * (t["fetch_kib"] * t["fetch_scale"] + t["write_kib"] * t["write_scale"])))


def make_temporal_chain(seed: int = 0, layers: int = workloads.TEMPORAL_LAYERS,
                        config: int = workloads.CFG_STEP, out_dtype=None, device=None):
    """Build the temporal-step chain on the GPU: weights drawn on the host (seeded),
    quantized and packed by q4_pack on the GPU; activations drawn per layer and stage."""
    import torch

    import bit_group_quantized_amd as q4
    from bit_group_quantized_amd.step import Chain, Q4Matrix, Stage

    device = device or torch.device("cuda:0")
    out_dtype = out_dtype or torch.bfloat16
    lin = workloads.temporal_layer()
    stages = []
    t0 = time.time()
    for layer in range(layers):
        ws = workloads.weights_many([(seed, config, layer, li.item, li.n, li.k) for li in lin])
        mats = []
        for w in ws:
            wt = torch.from_numpy(w).to(device)
            mats.append(Q4Matrix(*q4.q4_pack(wt)))
            del wt
        del ws
        by_stage = {}
        for li, m in zip(lin, mats):
            by_stage.setdefault(li.stage, []).append((li, m))
        for st in sorted(by_stage):
            k = by_stage[st][0][0].k
            x = workloads.activations(seed, config, layer, 100 + st, 1, k)[0]
            xt = torch.from_numpy(x.view(np.int16)).to(device).view(torch.bfloat16)
            stages.append(Stage(xt, [m for _, m in by_stage[st]]))
        if layer % 8 == 7:
            log(f"[bench] built {layer + 1}/{layers} layers ({time.time() - t0:.1f}s)")
    torch.cuda.synchronize()
    return Chain(stages, out_dtype)


def fused_stages(chain, seed: int = 0):
    """The temporal step's stages with the model's data flow and the decoder
    layer's parts fused in, on the same matrices: per layer
      norm(h) -> q, k, v;   o(q) + h -> h;   norm(h) -> silu(gate) * up -> mid;
      down(mid) + h -> h
    (h: the bf16 hidden state, updated in place; q stands in for the attention
    output, which this chain does not compute). RMSNorm weights are drawn
    around 1 (seeded), eps 1e-5."""
    import torch

    from bit_group_quantized_amd.step import Stage

    dev = chain.stages[0].x.device
    d, f = workloads.HIDDEN, workloads.FFN
    h = torch.from_numpy(workloads.activations(seed, workloads.CFG_STEP, 0, 200, 1, d)[0].view(np.int16)).to(dev)
    h = h.view(torch.bfloat16)
    out = []
    for layer in range(len(chain.stages) // 4):
        qkv, o, gu, down = chain.stages[4 * layer:4 * layer + 4]
        r = np.random.default_rng([seed, layer, 7])
        gam = [torch.from_numpy(workloads.bf16_bits_rne((1 + 0.1 * r.standard_normal(d)).astype(np.float32))
                                .view(np.int16)).to(dev).view(torch.bfloat16) for _ in range(2)]
        q = torch.empty(d, dtype=torch.bfloat16, device=dev)
        kk = torch.empty(d, dtype=torch.bfloat16, device=dev)
        v = torch.empty(d, dtype=torch.bfloat16, device=dev)
        mid = torch.empty(f, dtype=torch.bfloat16, device=dev)
        out += [Stage(h, qkv.mats, [q, kk, v], norm=gam[0], eps=1e-5),
                Stage(q, o.mats, [h], residuals=[h]),
                Stage(h, gu.mats, [mid, None], norm=gam[1], eps=1e-5, gated=True),
                Stage(mid, down.mats, [h], residuals=[h])]
    return out, h


def make_small_gemm(chain, m: int, seed: int = 0, device=None):
    """The small-GEMM workload: every stage of the temporal step (its packed
    matrices reused) against m activation rows, drawn per layer and stage on the
    host (seeded) as for the step. Returns the stages, x [m, k] and outputs
    [m, n] bf16 on the device."""
    import torch

    from bit_group_quantized_amd.step import Stage

    device = device or torch.device("cuda:0")
    keys = sorted({li.stage for li in workloads.temporal_layer()})
    stages = []
    for si, st in enumerate(chain.stages):
        layer, key = si // len(keys), keys[si % len(keys)]
        k = st.x.shape[-1]
        x = workloads.activations(seed, workloads.CFG_SMALL_GEMM, layer, 100 + key, m, k)
        xt = torch.from_numpy(x.view(np.int16)).to(device).view(torch.bfloat16)
        outs = [torch.empty((m, mt.n), dtype=torch.bfloat16, device=device) for mt in st.mats]
        stages.append(Stage(xt, st.mats, outs))
    return stages


def make_depformer(seed: int = 0, device=None):
    """The Depformer's 6 layers x 7 linears, each stored as one stacked packed tensor
    [16 * out, in] (weights drawn on the host, seeded, quantized and packed by q4_pack
    on the GPU). Returns {(layer, name): Q4Matrix}."""
    import torch

    import bit_group_quantized_amd as q4
    from bit_group_quantized_amd.step import Q4Matrix

    mats = {}
    for layer in range(workloads.DEP_LAYERS):
        lin = workloads.depformer_layer()
        ws = workloads.weights_many([(seed, workloads.CFG_DEPFORMER, layer, li.item, workloads.DEP_STEPS * li.n, li.k)
                                     for li in lin])
        for li, w in zip(lin, ws):
            wt = torch.from_numpy(w).to(device)
            mats[(layer, li.name)] = Q4Matrix(*q4.q4_pack(wt))
            del wt
        del ws
    torch.cuda.synchronize()
    return mats


def make_depformer_frame(mats, seed: int = 0, out_dtype=None, device=None):
    """One frame of the Depformer as one chain: 16 codebook steps x 6 layers x 4
    stages, each matrix the step's row slice of its stacked tensor; activations
    drawn per (step, layer, stage)."""
    import torch

    from bit_group_quantized_amd.step import Chain, Stage

    out_dtype = out_dtype or torch.bfloat16
    lin = workloads.depformer_layer()
    stages = []
    for step in range(workloads.DEP_STEPS):
        for layer in range(workloads.DEP_LAYERS):
            by_stage = {}
            for li in lin:
                by_stage.setdefault(li.stage, []).append(li)
            for st in sorted(by_stage):
                k = by_stage[st][0].k
                x = workloads.activations(seed, workloads.CFG_DEPFORMER, layer, 1000 + 4 * step + st, 1, k)[0]
                xt = torch.from_numpy(x.view(np.int16)).to(device).view(torch.bfloat16)
                stages.append(Stage(xt, [mats[(layer, li.name)].rows(step * li.n, li.n) for li in by_stage[st]]))
    return Chain(stages, out_dtype)


def cpu_baseline(seed: int, budget_s: float, sample_layers: int = 2, threads: int = 0):
    """The oracle (plain C, OpenMP over rows) on a bounded sample of the step: the
    first ``sample_layers`` temporal layers (7 GEMVs each, M=1), quantized once
    (not timed), then their products run pass after pass until the time budget is
    spent. Reported as packed-weight GB/s and the implied us per 32-layer step.
    threads > 0 sets the oracle's thread count (0: its default, one per core)."""
    import oracle

    default_threads = oracle.threads()
    if threads > 0:
        oracle.set_threads(threads)

    lin = workloads.temporal_layer()
    layers = []
    for layer in range(sample_layers):
        ws = workloads.weights_many([(seed, workloads.CFG_STEP, layer, li.item, li.n, li.k) for li in lin])
        qs = [oracle.quantize(w) for w in ws]
        del ws
        xs = {st: workloads.activations(seed, workloads.CFG_STEP, layer, 100 + st, 1, k)
              for st, k in {(li.stage, li.k) for li in lin}}
        layers.append((qs, xs))
    layer_bytes = sum(packed_bytes(li.n, li.k) for li in lin)
    elapsed, bytes_done, passes = 0.0, 0, 0
    while elapsed < budget_s:
        t0 = time.perf_counter()
        for qs, xs in layers:
            for li, (P, S, B) in zip(lin, qs):
                oracle.matmul(xs[li.stage], P, S, B, li.k)
        elapsed += time.perf_counter() - t0
        bytes_done += layer_bytes * len(layers)
        passes += 1
    gbs = bytes_done / elapsed / 1e9
    us_step = elapsed / (passes * len(layers)) * workloads.TEMPORAL_LAYERS * 1e6
    used = oracle.threads()
    oracle.set_threads(default_threads)
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": used, "kind": "oracle",
            "sample": f"temporal layers 0..{sample_layers - 1} of 32 (7 GEMVs each, M=1, "
                      f"{layer_bytes * len(layers) / 1e6:.0f} MB packed), {passes} passes, oracle product "
                      f"timed ({elapsed:.1f} s); quantization not timed",
            "us_per_step": round(us_step, 1)}


def stream_ceiling(dev, nbytes: int, reps: int = 3):
    """HBM stream-read ceiling for nbytes: a plain read-and-fold kernel
    (libq4_ceiling.so) over a buffer of the same size as the workload's packed
    weights, at a small sweep of launch shapes; the best median rate wins."""
    import ctypes

    import torch

    from bit_group_quantized_amd import build as q4_build

    lib = ctypes.CDLL(q4_build.CEILING_LIB)
    lib.q4_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_void_p]
    nbytes = nbytes // 16 * 16
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device=dev)
    buf.random_()
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.empty(cus * 32, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    best = None
    for per_cu in (4, 8, 16, 32):
        for unroll in (2, 4, 8):
            for nt in (0, 1):
                blocks = cus * per_cu

                def once():
                    rc = lib.q4_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(out.data_ptr()),
                                            blocks, unroll, nt, ctypes.c_void_p(stream.cuda_stream))
                    if rc != 0:
                        raise RuntimeError(f"q4_stream_read failed ({rc})")

                once()
                ts = []
                for _ in range(reps):
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record(stream)
                    once()
                    b.record(stream)
                    b.synchronize()
                    ts.append(a.elapsed_time(b))
                gbs = nbytes / (float(np.median(ts)) * 1e-3) / 1e9
                if best is None or gbs > best["gbs"]:
                    best = {"gbs": round(gbs, 1), "blocks_per_cu": per_cu, "loads_in_flight_per_lane": unroll,
                            "nontemporal": bool(nt)}
    del buf
    best["bytes"] = nbytes
    best["kernel"] = "stream_read_kernel"
    return best


def pack_timing(dev, seed: int):
    """q4_pack on the GPU against the oracle's quantizer on the host, on one
    11264x4096 temporal matrix (input fp32 bytes per second)."""
    import torch

    import bit_group_quantized_amd as q4
    import oracle

    n, k = workloads.FFN, workloads.HIDDEN
    w = workloads.weights(seed, workloads.CFG_STEP, 0, 4, n, k)
    wt = torch.from_numpy(w).to(dev)
    outs = q4.q4_pack(wt)
    stream = torch.cuda.current_stream(dev)
    reps = 20
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        q4.q4_pack(wt, *outs)
    b.record(stream)
    b.synchronize()
    gpu_s = a.elapsed_time(b) * 1e-3 / reps
    t0 = time.perf_counter()
    oracle.quantize(w)
    cpu_s = time.perf_counter() - t0
    return {"matrix": f"{n}x{k} fp32 ({w.nbytes / 1e6:.0f} MB)", "q4_pack_us": round(gpu_s * 1e6, 1),
            "q4_pack_gbs": round(w.nbytes / gpu_s / 1e9, 1), "oracle_quantize_ms": round(cpu_s * 1e3, 1),
            "oracle_quantize_gbs": round(w.nbytes / cpu_s / 1e9, 3), "oracle_threads": oracle.threads()}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--spin-up", type=float, default=2.0, metavar="SECONDS",
                    help="untimed calls for this long before the warmup steps of each timed workload: the "
                         "GPU raises its clocks over ~0.1 s of sustained load (steps timed right after the "
                         "host-side set-up run up to 15%% slower; once, right after a long test run, a "
                         "headline timed after 0.5 s ran 13%% slow with a wide spread while the same run's "
                         "later workloads were normal)")
    ap.add_argument("--mode", choices=("chain", "launches", "batch"), default="chain",
                    help="chain: one persistent launch (--workload gemm: m <= 4); launches: one call per matrix; "
                         "batch (--workload gemm, m = 5..16): q4_gemm_batch_run, one launch per distinct k")
    ap.add_argument("--workload", choices=("step", "depformer", "gemm", "gemv", "layer", "embed", "attn"),
                    default="step",
                    help="step: the 32-layer temporal step at M=1 (the headline); depformer: one "
                         "Depformer frame (16 codebook steps x 6 layers, M=1); gemm: the temporal "
                         "step's 224 matrices against X [M, k] (--m rows; one persistent chain launch for "
                         "M <= 4 in --mode chain, else one q4_gemm_small call per matrix); gemv: "
                         "one 4096x4096 GEMV, M=1, over 64 distinct matrices in turn (671 MB, past "
                         "the 256 MB last-level cache); layer: one temporal layer's 7 GEMVs (4 stages), "
                         "8 distinct layers in turn (1.03 GB, past the last-level cache); embed: the "
                         "packed-embedding gather and 17-stream sum of --m frames (text table 32000 x 4096, "
                         "16 audio tables 2048 x 4096), 64 token sets in turn; attn: one decoding step's "
                         "attention for the 32 layers (32 heads x 128, --ctx cached positions, bf16 caches "
                         "of every layer in turn)")
    ap.add_argument("--ctx", type=int, default=4096, help="cached positions for --workload attn")
    ap.add_argument("--m", type=int, default=4, help="rows of X for --workload gemm (1..64; 17..64: prefill), "
                                                     "frames for --workload embed")
    ap.add_argument("--dependent", action="store_true",
                    help="step: every stage's activation is the previous stage's first output (q -> o "
                         "-> gate/up -> down -> next q): each stage stores its outputs before the "
                         "barrier and the next stage loads them after it")
    ap.add_argument("--layers", type=int, default=workloads.TEMPORAL_LAYERS,
                    help="temporal layers (32 = the full step; fewer only for profiling runs)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="step: skip the dependent step, the stream-read ceiling and the pack timing; gemv and "
                         "gemm by per-call launches: skip the per-call read floor")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="instead of the step, run 5 plain device copies of MIB MiB (int32 "
                         "bitwise_not, MIB MiB read + MIB MiB written each) so that HBM byte "
                         "counters can be scaled against a kernel of known traffic")
    args = ap.parse_args(argv)
    global SPIN_UP_S
    SPIN_UP_S = max(0.0, args.spin_up)

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); the step "
              "shards as described in the design notes but no multi-GPU path is built.", file=sys.stderr)
        return 2

    import torch

    import bit_group_quantized_amd as q4

    q4.load()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.randint(-2**31, 2**31 - 1, (n,), dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.bitwise_not(src, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": 4 * n, "calibrate_copy_bytes_written": 4 * n,
                          "dispatches": 5}), flush=True)
        return 0
    if args.workload != "step":
        return bench_other(args, dev)
    chain = make_temporal_chain(args.seed, args.layers, device=dev)
    if args.dependent:
        # (the sizes line up: q, o and down give 4096 outputs, gate 11264)
        for prev, st in zip(chain.stages, chain.stages[1:]):
            assert prev.outs[0].numel() == st.x.numel()
            st.x = prev.outs[0]
    wbytes = chain.weight_bytes()
    launches_per_step = 1 if args.mode == "chain" else chain.num_matrices()

    if args.mode == "chain":
        chain.prepare_chain()
        run = chain.run_chain
    else:
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            chain.run_launches()  # warm the kernels outside capture
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            chain.run_launches()
        run = g.replay

    spin_up(run, args.spin_up)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    if args.mode == "chain" and chain.chain_status() != 0:
        print(f"chain executor reported status {chain.chain_status()}", file=sys.stderr)
        return 1

    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(args.steps):
        run()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]  # ms
    total_ms = ev[0].elapsed_time(ev[-1])
    if args.mode == "chain" and chain.chain_status() != 0:
        print(f"chain executor reported status {chain.chain_status()}", file=sys.stderr)
        return 1

    ms_per_step = total_ms / args.steps
    gbs = wbytes / (ms_per_step * 1e-3) / 1e9
    extra = {}
    if args.mode == "chain" and not args.dependent and not args.no_extras:
        # the same step with the model's data flow: every stage reads the
        # previous stage's first output (stores before the barrier, coherent
        # activation loads after it)
        for prev, st in zip(chain.stages, chain.stages[1:]):
            st.x = prev.outs[0]
        chain._plan = None
        chain.prepare_chain()
        dms, dper = time_replays(chain.run_chain, args.steps, args.warmup)
        if chain.chain_status() != 0:
            print(f"chain executor reported status {chain.chain_status()} (dependent step)", file=sys.stderr)
            return 1
        extra["dependent_step"] = {"us_per_step": round(dms * 1e3, 1),
                                   "gbs": round(wbytes / (dms * 1e-3) / 1e9, 1),
                                   "pct_hbm_peak": round(100 * wbytes / (dms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                                   "step_ms_p10_p50_p90": [round(float(np.percentile(dper, q)), 4)
                                                           for q in (10, 50, 90)]}
        # and with the decoder layer's RMSNorm, SwiGLU gate and residual sums
        # fused in (the hidden state updated in place)
        from bit_group_quantized_amd.step import Chain
        # (h keeps accumulating over the replays: a random walk of O(1) terms
        # that stays far from the bf16 range over any run length used here)
        fst, _ = fused_stages(chain, args.seed)
        fchain = Chain(fst, torch.bfloat16)
        fchain.prepare_chain()
        fms, fper = time_replays(fchain.run_chain, args.steps, args.warmup)
        if fchain.chain_status() != 0:
            print(f"chain executor reported status {fchain.chain_status()} (fused step)", file=sys.stderr)
            return 1
        extra["fused_step"] = {"us_per_step": round(fms * 1e3, 1),
                               "gbs": round(wbytes / (fms * 1e-3) / 1e9, 1),
                               "pct_hbm_peak": round(100 * wbytes / (fms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                               "step_ms_p10_p50_p90": [round(float(np.percentile(fper, q)), 4)
                                                       for q in (10, 50, 90)],
                               "stages": "per layer: norm->qkv, o+residual, norm->gate/up gated, down+residual"}
        del fchain, fst
        log("[bench] stream ceiling ...")
        extra["stream_ceiling"] = stream_ceiling(dev, wbytes)
        extra["pack"] = pack_timing(dev, args.seed)
    # dominant kernel: in chain mode the single launch per step; its duration is
    # the per-step event interval on the launch stream
    kernel_ms = ms_per_step / launches_per_step
    achieved = (wbytes / launches_per_step) / (kernel_ms * 1e-3) / 1e9
    full = args.layers == workloads.TEMPORAL_LAYERS
    result = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup, "spin_up_s": args.spin_up,
        "ms_per_step": round(ms_per_step, 4),
        "us_per_step": round(ms_per_step * 1e3, 1),
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": ("temporal_step_m1" if full else f"temporal_{args.layers}_layers_m1")
                   + ("_dependent" if args.dependent else ""),
                   "layers": args.layers, "hidden": workloads.HIDDEN, "ffn": workloads.FFN, "m": 1,
                   "group": 32, "weights_per_step": sum(li.n * li.k for li in workloads.temporal_layer()) * args.layers,
                   "packed_bytes_per_step": wbytes, "executor": args.mode,
                   "launches_per_step": launches_per_step, "stages_per_step": len(chain.stages)},
        "step_ms_p10_p50_p90": [round(float(np.percentile(per, q)), 4) for q in (10, 50, 90)],
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": chain_traffic_bytes(full and not args.dependent) if args.mode == "chain" else None,
                     "traffic_unit": "bytes per launch",
                     "kernel": "chain_kernel" if args.mode == "chain" else "gemv_kernel",
                     "bytes_per_launch": wbytes // launches_per_step,
                     "timing": "HIP events on the launch stream around each launch, mean over the timed steps"},
    }
    if "stream_ceiling" in extra:
        c = extra["stream_ceiling"]["gbs"]
        result["roofline"]["stream_ceiling_gbs"] = c
        result["roofline"]["frac_of_stream_ceiling"] = round(achieved / c, 4)
    result.update(extra)
    if not args.no_cpu:
        log("[bench] cpu baseline ...")
        result["cpu_baseline"] = cpu_baseline(args.seed, args.cpu_seconds)
        one = cpu_baseline(args.seed, args.cpu_seconds / 2, sample_layers=1, threads=1)
        result["cpu_baseline"]["single_thread"] = {"value": one["value"], "unit": "GB/s", "cores": one["cores"],
                                                   "sample": one["sample"], "us_per_step": one["us_per_step"]}
    print(json.dumps(result), flush=True)
    return 0


def spin_up(run, seconds: float) -> None:
    """Call run() for `seconds` of wall time (untimed; at least once)."""
    import torch

    t_end = time.time() + seconds
    while True:
        for _ in range(8):
            run()
        torch.cuda.synchronize()
        if time.time() >= t_end:
            return


SPIN_UP_S = 2.0  # set from --spin-up in main()


def time_replays(run, steps: int, warmup: int):
    """HIP events on the launch stream around each of `steps` calls of run(),
    after SPIN_UP_S seconds of untimed calls and `warmup` more."""
    import torch

    spin_up(run, SPIN_UP_S)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        run()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return ev[0].elapsed_time(ev[-1]) / steps, per


def per_call_read_floor(dev, sizes, steps: int, warmup: int):
    """What launches that only read the same bytes cost in a per-call
    workload's conditions: the plain read-and-fold kernel (libq4_ceiling.so)
    over one distinct buffer per entry of `sizes` (bytes) in turn (past the
    last-level cache), one launch each, replayed as a graph and timed like the
    workload; the best of a few launch shapes."""
    import ctypes

    import torch

    from bit_group_quantized_amd import build as q4_build

    lib = ctypes.CDLL(q4_build.CEILING_LIB)
    lib.q4_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_void_p]
    sizes = [int(b) // 16 * 16 for b in sizes]
    bufs = [torch.empty(b // 4, dtype=torch.int32, device=dev) for b in sizes]
    for b in bufs:
        b.random_()
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.empty(cus * 32, dtype=torch.int32, device=dev)
    best = None
    for per_cu in (2, 4, 8):
        for unroll in (2, 4):
            for nt in (0, 1):
                def calls():
                    st = torch.cuda.current_stream().cuda_stream
                    for b, nb in zip(bufs, sizes):
                        if lib.q4_stream_read(ctypes.c_void_p(b.data_ptr()), nb, ctypes.c_void_p(out.data_ptr()),
                                              cus * per_cu, unroll, nt, ctypes.c_void_p(st)) != 0:
                            raise RuntimeError("q4_stream_read failed")
                g = graph_of(calls)
                ms, _ = time_replays(g.replay, steps, warmup)
                us = ms * 1e3
                if best is None or us < best["us_total"]:
                    best = {"us_total": round(us, 1), "us_per_launch": round(us / len(sizes), 2),
                            "gbs": round(sum(sizes) / (us * 1e-6) / 1e9, 1),
                            "blocks_per_cu": per_cu, "loads_in_flight_per_lane": unroll, "nontemporal": bool(nt)}
    del bufs
    best.update({"bytes": sum(sizes), "launches": len(sizes), "kernel": "stream_read_kernel"})
    return best


def graph_of(fn):
    """Capture fn (a sequence of launches on the current stream) into a HIP graph."""
    import torch

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm the kernels outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    return g


def bench_other(args, dev) -> int:
    """The Depformer frame and the small-GEMM step (one JSON line each); no
    oracle baseline and no byte counters for these."""
    import torch

    import bit_group_quantized_amd as q4

    if args.workload == "gemv":
        from bit_group_quantized_amd.step import Q4Matrix

        copies, n, k = 64, workloads.HIDDEN, workloads.HIDDEN
        mats = []
        for c in range(copies):
            w = workloads.weights(args.seed, workloads.CFG_GEMV, 0, c, n, k)
            wt = torch.from_numpy(w).to(dev)
            mats.append(Q4Matrix(*q4.q4_pack(wt)))
            del wt
        x = workloads.activations(args.seed, workloads.CFG_GEMV, 0, 0, 1, k)[0]
        xt = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        ys = [torch.empty((n,), dtype=torch.bfloat16, device=dev) for _ in range(copies)]

        def calls():
            for mt, y in zip(mats, ys):
                q4.q4_gemv(xt, mt.packed, mt.scales, mt.biases, out=y)

        g = graph_of(calls)
        ms, per = time_replays(g.replay, args.steps, args.warmup)
        wbytes = sum(mt.nbytes() for mt in mats)
        per_call_us = ms * 1e3 / copies
        achieved = (wbytes / copies) / (per_call_us * 1e-6) / 1e9
        result = {
            "metric": "packed-weight GB/s (% HBM peak) + us per 4096x4096 GEMV, M=1",
            "value": round(achieved, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "spin_up_s": args.spin_up,
            "us_per_gemv": round(per_call_us, 2), "pct_hbm_peak": round(100 * achieved / HBM_PEAK_GBS, 2),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "gemv_4096x4096_m1", "n": n, "k": k, "m": 1, "group": 32, "copies": copies,
                       "packed_bytes_per_gemv": wbytes // copies, "executor": "graph of 64 launches"},
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "traffic_unit": "bytes per launch",
                         "kernel": "gemv_kernel", "bytes_per_launch": wbytes // copies},
        }
        if not args.no_extras:
            # (the same bytes per launch, only read: the floor of a per-call kernel)
            log("[bench] per-call read floor ...")
            result["read_floor"] = per_call_read_floor(dev, [wbytes // copies] * copies, args.steps, args.warmup)
        print(json.dumps(result), flush=True)
        return 0
    if args.workload == "embed":
        import torch as _t

        frames, sets = max(1, args.m), 64
        shapes = [(workloads.TEXT_VOCAB, workloads.HIDDEN)] + [(workloads.AUDIO_CODEBOOK, workloads.HIDDEN)] * 16
        tables = []
        for t, (rows, dim) in enumerate(shapes):
            w = workloads.weights(args.seed, 6, 1, t, rows, dim)
            wt = _t.from_numpy(w).to(dev)
            tables.append(q4.q4_pack(wt))
            del wt
        r = np.random.default_rng(args.seed)
        toks = [_t.from_numpy(np.stack([[r.integers(0, n) for n, _ in shapes] for _ in range(frames)])
                              .astype(np.int32)).to(dev) for _ in range(sets)]
        ys = [_t.empty((frames, workloads.HIDDEN), dtype=_t.bfloat16, device=dev) for _ in range(sets)]

        def calls():
            for tk, y in zip(toks, ys):
                q4.q4_embed_sum(tk, tables, out=y)

        g = graph_of(calls)
        ms, per = time_replays(g.replay, args.steps, args.warmup)
        us = ms * 1e3 / sets
        gathered = frames * len(shapes) * workloads.HIDDEN * 5 // 8  # packed bytes read per call
        gbs = gathered / (us * 1e-6) / 1e9
        result = {
            "metric": "us per packed-embedding gather + 17-stream sum (GB/s of packed rows read)",
            "value": round(us, 3), "unit": "us", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "spin_up_s": args.spin_up,
            "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": f"embed_sum_{frames}_frames", "streams": len(shapes), "dim": workloads.HIDDEN,
                       "text_rows": workloads.TEXT_VOCAB, "audio_rows": workloads.AUDIO_CODEBOOK, "frames": frames,
                       "packed_bytes_per_call": gathered, "executor": f"graph of {sets} q4_embed_sum calls"},
            "roofline": {"bound": "latency", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 6), "traffic": None, "kernel": "embed_sum_kernel",
                         "bytes_per_launch": gathered,
                         "timing": "HIP events on the launch stream around graph replays of 64 calls"},
        }
        print(json.dumps(result), flush=True)
        return 0
    if args.workload == "attn":
        import torch as _t

        heads, d, npos, layers = 32, 128, max(1, args.ctx), workloads.TEMPORAL_LAYERS
        cap, pos = npos, npos - 1
        g = _t.Generator(device=dev)
        g.manual_seed(args.seed)
        ks = [(_t.randn((heads, cap, d), generator=g, device=dev)).to(_t.bfloat16) for _ in range(layers)]
        vs = [(_t.randn((heads, cap, d), generator=g, device=dev)).to(_t.bfloat16) for _ in range(layers)]
        qs = [(_t.randn((3, heads, d), generator=g, device=dev)).to(_t.bfloat16) for _ in range(layers)]
        outs = [_t.empty((heads, d), dtype=_t.bfloat16, device=dev) for _ in range(layers)]
        ws = _t.zeros(q4.q4_attn_workspace_bytes(heads, d), dtype=_t.uint8, device=dev)

        def calls():
            for li in range(layers):
                q4.q4_attn_decode(qs[li][0], qs[li][1], qs[li][2], ks[li], vs[li], pos, out=outs[li], workspace=ws)

        gr = graph_of(calls)
        ms, per = time_replays(gr.replay, args.steps, args.warmup)
        kv = 2 * heads * npos * d * 2  # K and V bytes read per layer
        us = ms * 1e3 / layers
        gbs = kv / (us * 1e-6) / 1e9
        result = {
            "metric": "KV-cache GB/s (% HBM peak) + us per layer of decode attention, M=1",
            "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "spin_up_s": args.spin_up,
            "us_per_layer": round(us, 2), "us_per_step": round(ms * 1e3, 1),
            "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": f"attn_decode_{npos}_positions", "layers": layers, "heads": heads, "head_dim": d,
                       "cached_positions": npos, "kv_bytes_per_layer": kv,
                       "executor": f"graph of {layers} x 3 launches (rope + append, partial, combine)"},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "attn_decode_kernel",
                         "bytes_per_launch": kv,
                         "timing": "HIP events on the launch stream around graph replays; per layer = step / 32"},
        }
        print(json.dumps(result), flush=True)
        return 0
    if args.workload == "layer":
        # 8 layers (1.03 GB, past the 256 MB last-level cache) run in turn, each
        # layer's 7 GEMVs as one launch of its own: every launch starts cold
        from bit_group_quantized_amd.step import Chain

        rot = 8
        chain = make_temporal_chain(args.seed, rot, config=workloads.CFG_LAYER, device=dev)
        wbytes = chain.weight_bytes()
        per_layer = len(chain.stages) // rot
        if args.mode == "chain":
            chains = [Chain(chain.stages[per_layer * i:per_layer * (i + 1)], chain.out_dtype) for i in range(rot)]
            for c in chains:
                c.prepare_chain()

            def run():
                for c in chains:
                    c.run_chain()
            launches, kernel = rot, "chain_kernel"
        else:
            chains = []
            g = graph_of(chain.run_launches)
            run, launches, kernel = g.replay, chain.num_matrices(), "gemv_kernel"
        ms, per = time_replays(run, args.steps, args.warmup)
        if any(c.chain_status() != 0 for c in chains):
            print("chain executor reported a failure", file=sys.stderr)
            return 1
        per_layer_us = ms * 1e3 / rot
        gbs = wbytes / (ms * 1e-3) / 1e9
        result = {
            "metric": "packed-weight GB/s (% HBM peak) + us per temporal layer (7 GEMVs), M=1",
            "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "spin_up_s": args.spin_up,
            "us_per_layer": round(per_layer_us, 2), "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "temporal_layer_m1", "hidden": workloads.HIDDEN, "ffn": workloads.FFN, "m": 1,
                       "group": 32, "layers_in_turn": rot, "packed_bytes_per_layer": wbytes // rot,
                       "executor": args.mode, "launches_per_layer": launches / rot, "stages_per_layer": 4},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "traffic_unit": "bytes per launch",
                         "kernel": kernel, "bytes_per_launch": wbytes // launches,
                         "timing": "HIP events on the launch stream, mean over the timed replays"},
        }
        print(json.dumps(result), flush=True)
        return 0
    if args.workload == "depformer":
        mats = make_depformer(args.seed, dev)
        chain = make_depformer_frame(mats, args.seed, device=dev)
        wbytes = chain.weight_bytes()
        if args.mode == "chain":
            chain.prepare_chain()
            run, launches, kernel = chain.run_chain, 1, "chain_kernel"
        else:
            # one q4_multilinear_step call per linear, on the stacked tensor
            lin = workloads.depformer_layer()
            calls = []
            si = 0
            for step in range(workloads.DEP_STEPS):
                for layer in range(workloads.DEP_LAYERS):
                    by_stage = {}
                    for li in lin:
                        by_stage.setdefault(li.stage, []).append(li)
                    for st in sorted(by_stage):
                        stage = chain.stages[si]
                        si += 1
                        for li, y in zip(by_stage[st], stage.outs):
                            calls.append((stage.x, mats[(layer, li.name)], step, y))

            def run_calls():
                for x, mt, step, y in calls:
                    q4.q4_multilinear_step(x, mt.packed, mt.scales, mt.biases, workloads.DEP_STEPS, step, out=y)

            g = graph_of(run_calls)
            run, launches, kernel = g.replay, len(calls), "gemv_kernel"
        ms, per = time_replays(run, args.steps, args.warmup)
        if args.mode == "chain" and chain.chain_status() != 0:
            print(f"chain executor reported status {chain.chain_status()}", file=sys.stderr)
            return 1
        config = {"workload": "depformer_frame_m1", "layers": workloads.DEP_LAYERS, "codebook_steps": workloads.DEP_STEPS,
                  "dim": workloads.DEP_DIM, "ffn": workloads.DEP_FFN, "m": 1, "group": 32,
                  "packed_bytes_per_frame": wbytes, "executor": args.mode, "launches_per_frame": launches,
                  "stages_per_frame": len(chain.stages)}
        unit_name = "frame"
    else:
        if not 1 <= args.m <= 64:
            print("--m must be in 1..64", file=sys.stderr)
            return 2
        from bit_group_quantized_amd.step import Chain

        chain = make_temporal_chain(args.seed, args.layers, device=dev)
        wbytes = chain.weight_bytes()
        rows_chain = Chain(make_small_gemm(chain, args.m, args.seed, dev))
        use_chain = args.mode == "chain" and args.m <= 4
        use_batch = args.mode == "batch"
        if use_batch and not 5 <= args.m <= 16:
            print("--mode batch needs --m in 5..16", file=sys.stderr)
            return 2
        if use_chain:
            # the step's weights and the m activation rows through one persistent launch
            rows_chain.prepare_chain()
            run, launches, kernel = rows_chain.run_chain, 1, "chain_kernel"
        elif use_batch:
            # every product of one k in one launch (the step: k = 4096 and k = 11264)
            rows_chain.prepare_batches()
            g = graph_of(rows_chain.run_batches)
            run, launches, kernel = g.replay, len(rows_chain._batches), "gemm_batch_kernel"
        else:
            g = graph_of(rows_chain.run_launches)
            run, launches = g.replay, chain.num_matrices()
            kernel = "gemv_kernel" if args.m <= 4 else "gemm_mfma_kernel"
        ms, per = time_replays(run, args.steps, args.warmup)
        if use_chain and rows_chain.chain_status() != 0:
            print(f"chain executor reported status {rows_chain.chain_status()}", file=sys.stderr)
            return 1
        floor = None
        if not use_chain and not use_batch and not args.no_extras:
            # (the same matrices' bytes, only read, one launch each: the floor of a per-call step)
            log("[bench] per-call read floor ...")
            floor = per_call_read_floor(dev, [m.nbytes() for st in chain.stages for m in st.mats], args.steps,
                                        args.warmup)
        config = {"workload": f"small_gemm_m{args.m}_temporal_step", "layers": args.layers, "hidden": workloads.HIDDEN,
                  "ffn": workloads.FFN, "m": args.m, "group": 32, "packed_bytes_per_step": wbytes,
                  "executor": "chain" if use_chain else ("batch" if use_batch else "launches"),
                  "launches_per_step": launches}
        unit_name = "step"
    gbs = wbytes / (ms * 1e-3) / 1e9
    achieved = (wbytes / launches) / ((ms / launches) * 1e-3) / 1e9
    result = {
        "metric": f"packed-weight GB/s (% HBM peak) + us per {unit_name}",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "spin_up_s": args.spin_up,
        f"ms_per_{unit_name}": round(ms, 4), f"us_per_{unit_name}": round(ms * 1e3, 1),
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic", "config": config,
        f"{unit_name}_ms_p10_p50_p90": [round(float(np.percentile(per, q)), 4) for q in (10, 50, 90)],
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "traffic_unit": "bytes per launch",
                     "kernel": kernel, "bytes_per_launch": wbytes // launches},
    }
    if unit_name == "step" and floor is not None:
        result["read_floor"] = floor
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

"""Benchmark: paged single-token decode attention on one MI355X.

Default workload (one line of JSON on stdout): 70B-class GQA decode step,
64 sequences x 8192 tokens, 64 query / 8 KV heads, d_head 128, block size 16,
bf16 KV in 80 per-layer pools (160 GiB), randomly permuted blocks. One step is,
for every layer: kv_append of one new token per sequence (position 8191),
then paged decode attention over 8192 tokens (partition kernel + split-K
reduce). Inputs are resident in HBM before timing starts.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--partition P]

value = KV bytes read per step / step time (GB/s, 1e9 B/s). The roofline
entry is for the dominant kernel (the decode partition kernel): its
algorithmic bytes per launch over its average duration, measured with HIP
events recorded on the stream it runs on, against MI355X's 8 TB/s HBM peak.
cpu_baseline times the float64 oracle on a bounded sample of the same
workload in one process with one BLAS thread; cpu_baseline_procs times it in
several processes (up to 16) over whole sequences of the same layer.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0          # dense bf16
METRIC = "paged decode attention: KV GB/s and % of HBM peak; decode tokens/s"
COUNTERS = os.path.join(ROOT, "profiles", "decode_partition_counters.json")
KERNEL_SOURCES = ["paged_kv_cache_217_amd/csrc/decode_mfma.hip",
                  "paged_kv_cache_217_amd/csrc/mfma_common.h",
                  "paged_kv_cache_217_amd/csrc/pkv_device.h",
                  "paged_kv_cache_217_amd/csrc/pkv_internal.h"]
MQ_COUNTERS = os.path.join(ROOT, "profiles", "multi_query_counters.json")
CASCADE_COUNTERS = os.path.join(ROOT, "profiles", "cascade_counters.json")
CASCADE_KERNEL_SOURCES = ["paged_kv_cache_217_amd/csrc/decode_mfma.hip",
                          "paged_kv_cache_217_amd/csrc/multi_query_lds.hip",
                          "paged_kv_cache_217_amd/csrc/decode_attention.hip",
                          "paged_kv_cache_217_amd/csrc/schedule.hip",
                          "paged_kv_cache_217_amd/csrc/api.cpp",
                          "paged_kv_cache_217_amd/csrc/mfma_common.h",
                          "paged_kv_cache_217_amd/csrc/pkv_device.h",
                          "paged_kv_cache_217_amd/csrc/pkv_internal.h"]
MQ_KERNEL_SOURCES = ["paged_kv_cache_217_amd/csrc/multi_query_mfma.hip",
                     "paged_kv_cache_217_amd/csrc/multi_query_lds.hip",
                     "paged_kv_cache_217_amd/csrc/mfma_common.h",
                     "paged_kv_cache_217_amd/csrc/pkv_device.h",
                     "paged_kv_cache_217_amd/csrc/pkv_internal.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_hash(sources=KERNEL_SOURCES):
    h = hashlib.sha256()
    for f in sources:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=0,
                    help="timed steps (0: 10 for a multi-layer workload, 20 for a single layer)")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="gqa_70b",
                    choices=["gqa_70b", "mha_7b", "gqa_70b_fp8", "gqa_70b_fp4", "long_prefix", "tiny",
                             "spec_verify_70b", "chunked_prefill_70b", "shared_prompt_70b"])
    ap.add_argument("--layers", type=int, default=0, help="override layer count (0: workload's)")
    ap.add_argument("--partition", type=int, default=0, help="split-K partition (0: library)")
    ap.add_argument("--schedule", type=int, default=1,
                    help="1: longest-first work list built once per step (pkv_decode_schedule)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget for the oracle CPU baseline (0 disables it)")
    ap.add_argument("--cpu-procs", type=int, default=min(16, os.cpu_count() or 1),
                    help="also time the oracle in this many processes (one BLAS thread each) "
                         "over whole sequences, reported as cpu_baseline_procs (1 disables it)")
    ap.add_argument("--swap", type=int, default=0, metavar="N",
                    help="measure swapping N sequences of the 70B layer to host memory and back")
    ap.add_argument("--prefix-partition", type=int, default=0,
                    help="shared-prefix workload: prefix partition size (0: library)")
    ap.add_argument("--plain", type=int, default=1,
                    help="shared-prefix workload: also time plain decode on the same tables "
                         "(0: the cascade alone, e.g. for counter runs)")
    ap.add_argument("--bf16-weights", action="store_true",
                    help="multi-query and shared-prompt workloads: PKV_BF16_WEIGHTS (one bf16 "
                         "weight per product with V in the multi-query kernels, ~1e-3 relative "
                         "error)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 1 GiB block copy (for scaling HBM counters) and exit")
    return ap.parse_args()


def copy_calibration(pkv, torch):
    """pkv_copy_blocks over 16384 pairs of 64 KiB blocks: 1 GiB read + 1 GiB written."""
    n_kv, bs, d = 8, 16, 128
    nb = 2 * 16384
    k = torch.empty((nb, n_kv, bs, d), dtype=torch.bfloat16, device="cuda")
    v = torch.empty_like(k)
    k.fill_(1.0)
    v.fill_(2.0)
    pairs = torch.stack([torch.arange(16384), torch.arange(16384) + 16384], 1).to(
        torch.int32).cuda().contiguous()
    for _ in range(3):
        pkv.copy_blocks(k, v, pairs)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": 2 * 16384 * 32768,
                                           "bytes_written": 2 * 16384 * 32768,
                                           "launches": 3}}), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads as W

    w = W.ALL[args.workload]()
    if args.steps <= 0:
        # at least 20 timed launches of every kernel
        args.steps = 10 if (args.layers or w.layers) > 1 else 20
    decode = not (args.copy_calibration or args.swap or w.Q > 1 or w.notes.get("prefix_len"))
    # The processes of the multi-process oracle baseline are started here,
    # before anything touches the GPU (libpkv is not loaded yet, and
    # torch.cuda is first used below): they are new interpreters, and a
    # process that has initialised the GPU must not start programs that way.
    pool = None
    if decode and args.cpu_seconds > 0 and args.cpu_procs > 1:
        import multiprocessing as mp
        pool = mp.get_context("spawn").Pool(args.cpu_procs)
    try:
        run(args, w, pool, np, torch, W)
    finally:
        if pool is not None:
            pool.terminate()
            pool.join()


def run(args, w, pool, np, torch, W):
    import paged_kv_cache_217_amd as pkv

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        copy_calibration(pkv, torch)
        return
    if args.swap:
        bench_swap(args, pkv, W, np, torch, dev)
        return
    if w.Q > 1:
        bench_multi_query(args, w, pkv, W, np, torch, dev)
        return
    if w.notes.get("prefix_len"):
        bench_cascade(args, w, pkv, W, np, torch, dev)
        return
    layers = args.layers or w.layers
    B, n_q, n_kv, d, bs = w.B, w.n_q, w.n_kv, w.d, w.bs
    max_ctx = int(w.context_lens.max())
    log(f"[bench] workload {w.name}: B={B} n_q={n_q} n_kv={n_kv} d={d} bs={bs} "
        f"{w.kv_dtype} layers={layers} tokens={w.total_tokens} pool={w.num_blocks} blocks/layer")

    # ---------------------------------------------------------------- resident inputs
    t_setup = time.perf_counter()
    caches = []
    for layer in range(layers):
        kc, vc, ks, vs = W.make_cache(w, device=dev, seed_offset=1000 * layer,
                                      poison_unused=False)
        caches.append((kc, vc, ks, vs))
        if layer % 10 == 9:
            log(f"[bench] generated {layer + 1}/{layers} layer pools")
    q = W.make_query(w, device=dev, layers=layers) if layers > 1 else \
        W.make_query(w, device=dev)[None]
    k_new, v_new = W.make_new_tokens(w, T=layers * B, device=dev)
    k_new = k_new.view(layers, B, n_kv, d)
    v_new = v_new.view(layers, B, n_kv, d)
    bt = torch.from_numpy(w.block_tables).to(dev)
    cl = torch.from_numpy(w.context_lens).to(dev)
    pos = torch.from_numpy((w.context_lens - 1).astype(np.int32)).to(dev)
    P = args.partition or w.partition_size or \
        pkv.default_partition_size(caches[0][0], B, n_q, max_ctx)
    P_max = max(1, -(-max_ctx // P))
    ws, _ = pkv.make_workspace(caches[0][0], B, n_q, max_ctx, P)
    m_, l_, o_ = pkv.partial_views(ws, B, n_q, d, P_max)
    out = torch.empty((B, n_q, d), dtype=torch.float32, device=dev)
    slots = torch.empty(B, dtype=torch.int64, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] setup {time.perf_counter() - t_setup:.1f}s; partition {P} tokens, "
        f"{P_max} partitions/seq")

    stream = torch.cuda.current_stream()
    split = P_max > 1

    sched_buf = None
    if args.schedule:
        sched_buf = torch.empty(max(32, pkv.lib().pkv_decode_schedule_bytes(B, max_ctx, P)) // 4,
                                dtype=torch.int32, device=dev)

    def step(ev=None):
        pkv.slot_mapping(bt, pos, bs, out=slots)
        sched = pkv.decode_schedule(cl, max_ctx, P, out=sched_buf) if args.schedule else None
        for layer in range(layers):
            kc, vc, ks, vs = caches[layer]
            if ev is not None:
                ev[layer][0].record(stream)
            pkv.kv_append(kc, vc, k_new[layer], v_new[layer], slots, ks, vs)
            if ev is not None:
                ev[layer][1].record(stream)
            if split:
                pkv.paged_decode_partials(q[layer], kc, vc, bt, cl, w.scale, max_ctx, P,
                                          k_scale=ks, v_scale=vs, workspace=ws, schedule=sched)
                if ev is not None:
                    ev[layer][2].record(stream)
                pkv.splitk_reduce(m_, l_, o_, cl, P, out=out)
            else:
                pkv.paged_decode_attention(q[layer], kc, vc, bt, cl, w.scale, max_ctx,
                                           k_scale=ks, v_scale=vs, partition_size=P, out=out,
                                           workspace=ws, schedule=sched)
                if ev is not None:
                    ev[layer][2].record(stream)
            if ev is not None:
                ev[layer][3].record(stream)

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"[bench] warmup step {i + 1}/{args.warmup} done")

    # timed region 1: exactly K steps, nothing but the work between the events
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for s in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(stop) / args.steps
    log(f"[bench] {args.steps} timed steps: {ms_step:.3f} ms/step (host wall {wall:.3f}s)")

    # timed region 2: the same K steps with HIP events on the launch stream around
    # every kernel (an event pair costs a few microseconds, so region 1 gives the
    # step time and this one the per-kernel durations)
    events = [[[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(layers)]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    t_append, t_part, t_reduce = [], [], []
    for s in range(args.steps):
        for layer in range(layers):
            e = events[s][layer]
            t_append.append(e[0].elapsed_time(e[1]))
            t_part.append(e[1].elapsed_time(e[2]))
            t_reduce.append(e[2].elapsed_time(e[3]))
    avg = lambda x: sum(x) / len(x)
    ms_part = avg(t_part)

    # ---------------------------------------------------------------- accounting
    tokens = w.total_tokens
    kv_bytes_layer = kv_bytes(w)
    part_bytes = partition_bytes(w, P)
    achieved = part_bytes / (ms_part * 1e-3) / 1e9
    kv_gbs = kv_bytes_layer * layers / (ms_step * 1e-3) / 1e9
    tok_s = B / (ms_step * 1e-3)

    traffic = counter_traffic(w.name, P)

    result = {
        "metric": METRIC,
        "value": round(kv_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.kv_dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "context": max_ctx if len(set(
            w.context_lens.tolist())) == 1 else "varied", "tokens_per_layer": tokens,
            "n_q": n_q, "n_kv": n_kv, "d_head": d, "block_size": bs, "layers": layers,
            "kv_dtype": w.kv_dtype, "partition_size": P, "accumulate": "fp32",
            "schedule": "longest-first" if args.schedule else "grid order"},
        "hbm_peak_frac": round(kv_gbs / HBM_PEAK_GBS, 4),
        "decode_tokens_per_s": round(tok_s, 1),
        "kernels_ms": {"kv_append": round(avg(t_append), 5),
                       "decode_partition": round(ms_part, 5),
                       "splitk_reduce": round(avg(t_reduce), 5) if split else None},
        # spread of the per-launch event timings of the partition kernel
        "decode_partition_ms_p10_p50_p90": [round(float(np.percentile(t_part, p)), 5)
                                            for p in (10, 50, 90)],
        "roofline": {"bound": "hbm", "kernel": "decode_partition",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "bytes_per_launch": part_bytes,
                     "traffic": traffic["total"] if traffic else None,
                     "traffic_read": traffic["read"] if traffic else None,
                     "traffic_written": traffic["written"] if traffic else None},
    }

    # ---------------------------------------------------------------- oracle on the CPU
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(w, caches[0], q[0], args.cpu_seconds)
        if layers > 1:
            # the oracle's time for one whole step at the measured rate: layer 0
            # only was sampled, so this is extrapolated to every layer
            cb = result["cpu_baseline"]
            cb["step_seconds_extrapolated"] = round(kv_bytes_layer * layers / (cb["value"] * 1e9), 1)
            cb["extrapolation"] = f"rate on layer 0 x {layers} layers"
        if pool is not None:
            try:
                result["cpu_baseline_procs"] = cpu_baseline_procs(
                    w, caches[0], q[0], args.cpu_seconds, args.cpu_procs, pool)
            except Exception as e:           # the GPU figures stand without it
                log(f"[bench] multi-process oracle baseline failed: {e!r}")
    print(json.dumps(result), flush=True)


def counter_traffic(name, P):
    """HBM bytes per launch of the partition kernel for workload `name` at
    partition size P, from the committed rocprofv3 counters, or None when
    none were taken for it or the kernel sources changed since."""
    if not os.path.exists(COUNTERS):
        return None
    c = json.load(open(COUNTERS))
    if c.get("kernel_hash") != kernel_hash():
        return None
    e = c.get("workloads", {}).get(name, {})
    return e.get("traffic_bytes_per_launch") if e.get("partition") == P else None


def mq_counter_traffic(name, P):
    """HBM bytes per launch of the multi-query kernel for workload `name` at
    partition size P, from the committed rocprofv3 counters, or None as for
    counter_traffic (the source hash is kept once, for every workload)."""
    if not os.path.exists(MQ_COUNTERS):
        return None
    c = json.load(open(MQ_COUNTERS))
    if c.get("kernel_hash") != kernel_hash(MQ_KERNEL_SOURCES):
        return None
    e = c.get(name, {})
    return e.get("traffic_bytes_per_launch") if e.get("partition") == P else None


def kv_bytes(w):
    """K and V bytes one layer's attention reads: every attended token's K and
    V rows of every KV head (2 * n_kv * d_head * bytes per element)."""
    return int(w.total_tokens * w.n_kv * w.d * w.p * 2)


def partition_bytes(w, P):
    """Algorithmic bytes of one launch of the decode partition kernel over the
    workload's batch with partition size P: the K/V it reads, the queries, the
    block-table entries of the attended blocks, the FP8/FP4 scales, and what it
    writes (the output in fp32 in a single pass, else (m, l, o) per
    partition)."""
    ctx = [int(c) for c in w.context_lens]
    max_ctx = max(ctx) if ctx else 0
    split = -(-max_ctx // P) > 1
    n_part = sum(-(-c // P) for c in ctx if c > 0)
    return (kv_bytes(w)
            + w.B * w.n_q * w.d * 2                                    # q, bf16
            + sum(-(-c // w.bs) for c in ctx) * 4                      # block-table entries
            + (n_part * w.n_q * (w.d + 2) * 4 if split else w.B * w.n_q * w.d * 4)
            + (2 * w.n_kv * 4 if w.kv_dtype != "bf16" else 0))         # per-head scales


def multi_query_work(w, P_max):
    """Algorithmic work of one multi-token-query attention call (the kernel and,
    with P_max > 1, the reduce): every (sequence, KV head) reads its context's K
    and V once, plus the bf16 queries, the fp32 outputs, the table entries of
    the attended blocks and, when split, the partials written and read back.
    Query i of a sequence with c tokens and q new ones sees c - q + i + 1
    tokens, and each visible (query row, token) costs 4 d flops (2 d for the
    score, 2 d for the weighted value). Returns (flops, bytes)."""
    ctx = [int(c) for c in w.context_lens]
    ql = [int(x) for x in w.query_lens]
    visible = sum(c * q - q * (q - 1) // 2 for c, q in zip(ctx, ql))
    flops = 4 * w.d * w.n_q * visible
    nbytes = (kv_bytes(w) + w.B * w.Q * w.n_q * w.d * (2 + 4)
              + sum(-(-c // w.bs) for c in ctx) * 4)
    if P_max > 1:
        nbytes += 2 * w.B * w.Q * w.n_q * P_max * (w.d + 2) * 4
    return flops, nbytes


def bench_swap(args, pkv, W, np, torch, dev):
    """Swap args.swap sequences of one 70B-GQA layer pool (8192 tokens each,
    512 blocks of 8 heads x 16 tokens x 128 dims) to pinned host memory and
    back into other blocks, timed with HIP events on the stream the calls run
    on (pkv_swap_out = pack kernel + device-to-host copy, pkv_swap_in =
    host-to-device copy + unpack kernel; the kernels' share is in the
    rocprofv3 trace)."""
    w = W.gqa_70b(layers=1)
    kc, vc, _, _ = W.make_cache(w, device=dev, poison_unused=False)
    n_seq = min(args.swap, w.B)
    ids = np.concatenate([w.block_tables[b, :512] for b in range(n_seq)]).astype(np.int32)
    n = len(ids)
    ids_d = torch.from_numpy(ids).to(dev)
    back = torch.from_numpy(ids[::-1].copy()).to(dev)      # other blocks on the way back
    nbytes = pkv.swap_bytes(kc, n)
    staging = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    host = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    desc = pkv.cache_desc(kc)
    L = pkv.lib()
    import ctypes
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)

    def phases(ev):                  # events: 0 start, 2 after swap-out, 4 after swap-in
        ev[0].record(stream)
        assert L.pkv_swap_out(ctypes.byref(desc), ctypes.c_void_p(kc.data_ptr()),
                              ctypes.c_void_p(vc.data_ptr()), ctypes.c_void_p(ids_d.data_ptr()),
                              n, ctypes.c_void_p(staging.data_ptr()),
                              ctypes.c_void_p(host.data_ptr()), sp) == 0
        ev[2].record(stream)
        assert L.pkv_swap_in(ctypes.byref(desc), ctypes.c_void_p(kc.data_ptr()),
                             ctypes.c_void_p(vc.data_ptr()), ctypes.c_void_p(back.data_ptr()),
                             n, ctypes.c_void_p(staging.data_ptr()),
                             ctypes.c_void_p(host.data_ptr()), sp) == 0
        ev[4].record(stream)

    for _ in range(args.warmup):
        phases([torch.cuda.Event(enable_timing=True) for _ in range(5)])
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    for e in evs:
        phases(e)
    torch.cuda.synchronize()
    t_out = sum(e[0].elapsed_time(e[2]) for e in evs) / len(evs)
    t_in = sum(e[2].elapsed_time(e[4]) for e in evs) / len(evs)
    gb = nbytes / 1e9
    result = {
        "metric": "KV swap to host memory and back: GB/s of KV image per direction",
        "value": round(2 * gb / ((t_out + t_in) * 1e-3), 2), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(t_out + t_in, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "swap of 70B-GQA sequences (one layer pool)", "sequences": n_seq,
                   "blocks": n, "image_bytes": nbytes},
        "swap_out_ms": round(t_out, 4), "swap_in_ms": round(t_in, 4),
        "swap_out_gbs": round(gb / (t_out * 1e-3), 2), "swap_in_gbs": round(gb / (t_in * 1e-3), 2),
        "roofline": {"bound": "host link", "achieved": round(gb / (t_out * 1e-3), 2),
                     "peak": 64.0, "unit": "GB/s", "frac": round(gb / (t_out * 1e-3) / 64.0, 4),
                     "note": "peak = PCIe 5.0 x16 nominal per direction", "traffic": None},
    }
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline_swap(kc, vc, ids, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def cpu_baseline_swap(kc, vc, ids, budget):
    """The oracle's swap (the listed blocks' bytes packed into a host image,
    then unpacked into other blocks) on host copies of the pools, repeated
    until the budget is spent; GB/s of image per direction."""
    import workloads as W
    from oracle import paged as ref

    log("[bench] copying the pools to the host for the oracle")
    kb, vb = W.bits(kc), W.bits(vc)
    back = ids[::-1].copy()
    n = 0
    t0 = time.perf_counter()
    while n == 0 or time.perf_counter() - t0 < budget:
        image = ref.swap_out(kb, vb, ids)
        kb, vb = ref.swap_in(kb, vb, back, image)
        n += 1
    dt = time.perf_counter() - t0
    gb = 2 * n * image.nbytes / 1e9
    log(f"[bench] oracle: {n} swap round trips in {dt:.1f}s")
    return {"value": round(gb / dt, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} round trips of a {image.nbytes / 1e6:.0f} MB image ({len(ids)} blocks; "
                      f"the oracle's swap-in returns new copies of the whole pools), numpy, 1 process, "
                      f"{dt:.1f} s; host has {os.cpu_count()} logical CPUs"}


def bench_cascade(args, w, pkv, W, np, torch, dev):
    """A batch sharing a prompt prefix: per layer, kv_append of the new token,
    then decode attention through pkv_cascade_decode_attention (prefix read
    once) and, for comparison, through plain decode on the same full tables."""
    layers = args.layers or w.layers
    B, n_q, n_kv, d, bs = w.B, w.n_q, w.n_kv, w.d, w.bs
    plen = w.notes["prefix_len"]
    pb = plen // bs
    caches = [W.make_cache(w, device=dev, seed_offset=1000 * layer, poison_unused=False)
              for layer in range(layers)]
    q = W.make_query(w, device=dev, layers=layers) if layers > 1 else W.make_query(w, device=dev)[None]
    k_new, v_new = W.make_new_tokens(w, T=layers * B, device=dev)
    k_new = k_new.view(layers, B, n_kv, d)
    v_new = v_new.view(layers, B, n_kv, d)
    bt = torch.from_numpy(w.block_tables).to(dev)
    cl = torch.from_numpy(w.context_lens).to(dev)
    pt = torch.from_numpy(w.block_tables[0, :pb].copy()).to(dev)
    st = torch.from_numpy(np.ascontiguousarray(w.block_tables[:, pb:])).to(dev)
    slen_np = (w.context_lens - plen).astype(np.int32)
    slen = torch.from_numpy(slen_np).to(dev)
    max_ctx, max_s = int(w.context_lens.max()), int(slen_np.max())
    pos = torch.from_numpy((w.context_lens - 1).astype(np.int32)).to(dev)
    slots = torch.empty(B, dtype=torch.int64, device=dev)
    out = torch.empty((B, n_q, d), dtype=torch.float32, device=dev)
    desc = pkv.cache_desc(caches[0][0])
    import ctypes
    cws = torch.empty(max(16, pkv.lib().pkv_cascade_workspace_bytes(
        ctypes.byref(desc), B, n_q, plen, args.prefix_partition, max_s, args.partition)),
        dtype=torch.uint8, device=dev)
    P = pkv.default_partition_size(caches[0][0], B, n_q, max_ctx)
    dws, _ = pkv.make_workspace(caches[0][0], B, n_q, max_ctx, P)
    # longest-first lists, built once per step for all layers (as the decode
    # step does): the suffix partitions' for the cascade, the sequences' for
    # plain decode
    Ps = pkv.cascade_suffix_partition(caches[0][0], B, n_q, plen, max_s, args.prefix_partition,
                                      args.partition)
    c_sched = torch.empty(max(32, pkv.lib().pkv_decode_schedule_bytes(B, max_s, max(Ps, 16))) // 4,
                          dtype=torch.int32, device=dev)
    d_sched = torch.empty(max(32, pkv.lib().pkv_decode_schedule_bytes(B, max_ctx, P)) // 4,
                          dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    log(f"[bench] workload {w.name}: B={B} prefix={plen} suffix {slen_np.min()}..{max_s} "
        f"(partition {Ps}) layers={layers}")

    def step(cascade, ev=None):
        pkv.slot_mapping(bt, pos, bs, out=slots)
        if cascade:
            sched = pkv.cascade_schedule(caches[0][0], slen, n_q, plen, max_s,
                                         args.prefix_partition, args.partition,
                                         out=c_sched) if args.schedule else None
        else:
            sched = pkv.decode_schedule(cl, max_ctx, P, out=d_sched) if args.schedule else None
        for layer in range(layers):
            kc, vc, ks, vs = caches[layer]
            pkv.kv_append(kc, vc, k_new[layer], v_new[layer], slots, ks, vs)
            if ev is not None:
                ev[layer][0].record(stream)
            if cascade:
                pkv.cascade_decode_attention(q[layer], kc, vc, pt, plen, st, slen, w.scale, max_s,
                                             prefix_partition=args.prefix_partition,
                                             suffix_partition=args.partition, out=out,
                                             workspace=cws, schedule=sched,
                                             bf16_weights=args.bf16_weights)
            else:
                pkv.paged_decode_attention(q[layer], kc, vc, bt, cl, w.scale, max_ctx,
                                           partition_size=P, out=out, workspace=dws,
                                           schedule=sched)
            if ev is not None:
                ev[layer][1].record(stream)

    res = {}
    for cascade in ((True, False) if args.plain else (True,)):
        for _ in range(args.warmup):
            step(cascade)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            step(cascade)
        e1.record(stream)
        torch.cuda.synchronize()
        ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(layers)]
              for _ in range(args.steps)]
        for s_ in range(args.steps):
            step(cascade, ev[s_])
        torch.cuda.synchronize()
        att = [e[0].elapsed_time(e[1]) for st_ in ev for e in st_]
        res[cascade] = (e0.elapsed_time(e1) / args.steps, sum(att) / len(att))
        log(f"[bench] {'cascade' if cascade else 'plain'}: {res[cascade][0]:.3f} ms/step, "
            f"attention {res[cascade][1] * 1000:.1f} us/layer")
    ms_step, ms_att = res[True]
    row = n_kv * d * w.p * 2
    unique = (plen + int(slen_np.sum())) * row          # prefix once + every suffix
    logical = int(w.context_lens.sum()) * row            # what each sequence attends over
    att_bytes = unique + B * n_q * d * (2 + 4) + (pb + sum(-(-int(x) // bs) for x in slen_np)) * 4
    achieved = att_bytes / (ms_att * 1e-3) / 1e9
    result = {
        "metric": "shared-prefix decode attention: decode tokens/s",
        "value": round(B / (ms_step * 1e-3 / layers), 1), "unit": "decode tokens/s per layer",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "B": B, "prefix_len": plen,
                   "suffix_partition": args.partition or "library default",
                   "suffix_len": [int(slen_np.min()), max_s], "n_q": n_q, "n_kv": n_kv,
                   "d_head": d, "block_size": bs, "layers": layers, "kv_dtype": w.kv_dtype,
                   "prefix_weights": "bf16" if args.bf16_weights else "bf16 head + tail"},
        "attention_us_per_layer": {"cascade": round(ms_att * 1000, 1),
                                   "plain_decode": round(res[False][1] * 1000, 1)
                                   if False in res else None},
        "speedup_vs_plain_decode": round(res[False][1] / ms_att, 2) if False in res else None,
        "logical_kv_gbs": round(logical / (ms_att * 1e-3) / 1e9, 1),
        "roofline": {"bound": "hbm", "kernel": "cascade (prefix pass + suffix partitions + merge)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "bytes_per_launch": att_bytes,
                     "traffic": None},
    }
    # HBM bytes of one call (all its launches), from the committed counters,
    # while the sources they were taken on are unchanged and the call is the
    # library's default one
    if (os.path.exists(CASCADE_COUNTERS) and not args.partition and not args.prefix_partition
            and not args.bf16_weights):
        c = json.load(open(CASCADE_COUNTERS))
        if c.get("kernel_hash") == kernel_hash(CASCADE_KERNEL_SOURCES):
            t = c["traffic_bytes_per_call"]
            result["roofline"].update(traffic=t["total"], traffic_read=t["read"],
                                      traffic_written=t["written"])
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline_cascade(w, caches[0], q[0], plen, slen_np,
                                                      args.cpu_seconds)
    print(json.dumps(result), flush=True)


def multi_query_kernel_name(w, Q):
    """The kernel the library dispatches a multi-token query batch to: 128 or
    more (query, head) rows per KV head run on the LDS-shared kernel, in its
    ping-pong form at d 128 unless 256-row groups pad the rows by more than a
    tenth beyond 128-row ones; fewer rows on the register kernel."""
    rows = Q * (w.n_q // w.n_kv)
    if rows < 128:
        return "multi_query_partition_mfma"
    if w.d == 128 and rows >= 256 and 10 * 2 * -(-rows // 256) <= 11 * -(-rows // 128):
        return "multi_query_lds_pp"
    return "multi_query_lds_mfma"


def bench_multi_query(args, w, pkv, W, np, torch, dev):
    """Several query tokens per sequence: per layer, kv_append of the Q new
    tokens of every sequence, then causal multi-query paged attention."""
    layers = args.layers or w.layers
    B, Q, n_q, n_kv, d, bs = w.B, w.Q, w.n_q, w.n_kv, w.d, w.bs
    ql = w.query_lens
    max_ctx = int(w.context_lens.max())
    log(f"[bench] workload {w.name}: B={B} Q={Q} n_q={n_q} n_kv={n_kv} d={d} bs={bs} "
        f"layers={layers} tokens={w.total_tokens}")
    caches = [W.make_cache(w, device=dev, seed_offset=1000 * layer, poison_unused=False)
              for layer in range(layers)]
    q = torch.stack([W.make_multi_query(w, Q, device=dev, seed_offset=1000 * layer)
                     for layer in range(layers)])
    k_new, v_new = W.make_new_tokens(w, T=layers * B * Q, device=dev)
    k_new = k_new.view(layers, B * Q, n_kv, d)
    v_new = v_new.view(layers, B * Q, n_kv, d)
    bt = torch.from_numpy(w.block_tables).to(dev)
    cl = torch.from_numpy(w.context_lens).to(dev)
    qld = torch.from_numpy(ql).to(dev)
    # one table row and one position per new token (padding rows: position -1)
    pos_np = np.full((B, Q), -1, dtype=np.int32)
    for b in range(B):
        pos_np[b, :ql[b]] = w.context_lens[b] - ql[b] + np.arange(ql[b])
    bt_tok = bt.repeat_interleave(Q, dim=0).contiguous()
    pos = torch.from_numpy(pos_np.reshape(-1)).to(dev)
    slots = torch.empty(B * Q, dtype=torch.int64, device=dev)
    P = args.partition or pkv.multi_query_partition_size(caches[0][0], B, Q, n_q, max_ctx)
    P_max = max(1, -(-max_ctx // P))
    nbytes = pkv.lib().pkv_multi_query_workspace_bytes(B, Q, n_q, d, max_ctx, P)
    ws = torch.empty(max(16, nbytes), dtype=torch.uint8, device=dev)
    out = torch.empty((B, Q, n_q, d), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    log(f"[bench] partition {P} tokens, {P_max} partitions/seq")

    def step(ev=None):
        pkv.slot_mapping(bt_tok, pos, bs, out=slots)
        for layer in range(layers):
            kc, vc, ks, vs = caches[layer]
            if ev is not None:
                ev[layer][0].record(stream)
            pkv.kv_append(kc, vc, k_new[layer], v_new[layer], slots, ks, vs)
            if ev is not None:
                ev[layer][1].record(stream)
            pkv.paged_multi_query_attention(q[layer], qld, kc, vc, bt, cl, w.scale, max_ctx,
                                            k_scale=ks, v_scale=vs, partition_size=P, out=out,
                                            workspace=ws, bf16_weights=args.bf16_weights)
            if ev is not None:
                ev[layer][2].record(stream)

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"[bench] warmup step {i + 1}/{args.warmup} done")
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / args.steps
    log(f"[bench] {args.steps} timed steps: {ms_step:.3f} ms/step")
    events = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(layers)]
              for _ in range(args.steps)]
    for s_ in range(args.steps):
        step(events[s_])
    torch.cuda.synchronize()
    t_app = [e[0].elapsed_time(e[1]) for st in events for e in st]
    t_att = [e[1].elapsed_time(e[2]) for st in events for e in st]
    avg = lambda x: sum(x) / len(x)
    ms_att = avg(t_att)

    kv_bytes_layer = kv_bytes(w)
    flops, att_bytes = multi_query_work(w, P_max)
    intensity = flops / att_bytes
    kname = multi_query_kernel_name(w, Q)
    if args.bf16_weights and kname == "multi_query_lds_pp":
        kname += " (single bf16 weights)"
    if P_max > 1:
        kname += " + splitk_reduce"
    mfma_bound = intensity > MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if mfma_bound:
        achieved = flops / (ms_att * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": kname, "achieved": round(achieved, 2),
                "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_PEAK_TFLOPS, 4), "flops_per_launch": flops,
                "bytes_per_launch": att_bytes, "traffic": None}
    else:
        achieved = att_bytes / (ms_att * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": kname, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "bytes_per_launch": att_bytes, "traffic": None}
    traffic = None
    if os.path.exists(MQ_COUNTERS) and not args.bf16_weights:
        traffic = mq_counter_traffic(w.name, P)
    roof["traffic"] = traffic["total"] if traffic else None
    roof["traffic_read"] = traffic["read"] if traffic else None
    roof["traffic_written"] = traffic["written"] if traffic else None
    new_tokens = int(ql.sum())
    result = {
        "metric": "multi-query paged attention: query tokens/s, KV GB/s",
        "value": round(new_tokens / (ms_step * 1e-3), 1),
        "unit": "query tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "B": B, "Q": Q, "query_tokens": new_tokens,
                   "tokens_per_layer": w.total_tokens, "n_q": n_q, "n_kv": n_kv, "d_head": d,
                   "block_size": bs, "layers": layers, "kv_dtype": w.kv_dtype,
                   "partition_size": P, "accumulate": "fp32",
                   "weights": "bf16" if args.bf16_weights else "bf16 head + tail"},
        "kv_gbs": round(kv_bytes_layer * layers / (ms_step * 1e-3) / 1e9, 2),
        "attention_tflops": round(flops / (ms_att * 1e-3) / 1e12, 2),
        "kernels_ms": {"kv_append": round(avg(t_app), 5),
                       "multi_query_attention": round(ms_att, 5)},
        "roofline": roof,
    }
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline_mq(w, caches[0], q[0], args.cpu_seconds, layers)
    print(json.dumps(result), flush=True)


def cpu_baseline_mq(w, layer_cache, q0, budget, layers):
    """The float64 oracle on layer 0, one (sequence, query) at a time with all
    heads (query i of sequence b is the one-query problem over its visible
    tokens 0..p), taking query 0 of every sequence, then query 1, ..., until
    the budget is spent; the rate is divided by the layer count to compare
    with the step's query tokens/s."""
    import numpy as np
    import threadpoolctl

    import workloads as W
    from oracle import paged as ref

    kc, vc, ks, vs = layer_cache
    log("[bench] copying layer 0 to the host for the oracle")
    kb, vb, qb = W.bits(kc), W.bits(vc), W.bits(q0)
    ksn = None if ks is None else ks.cpu().numpy()
    vsn = None if vs is None else vs.cpu().numpy()
    ql = w.query_lens
    units = [(b, i) for i in range(w.Q) for b in range(w.B) if i < ql[b]]
    n = tokens = 0
    with threadpoolctl.threadpool_limits(1):
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < budget and n < len(units):
            b, i = units[n]
            p = int(w.context_lens[b]) - int(ql[b]) + i            # the query's position
            ref.multi_query_attention(qb[b:b + 1, i:i + 1], kb, vb, w.block_tables[b:b + 1],
                                      np.array([p + 1], dtype=np.int32),
                                      np.array([1], dtype=np.int32), w.scale, w.kv_dtype,
                                      ksn, vsn)
            tokens += p + 1
            n += 1
        dt = time.perf_counter() - t0
    rate = n / dt
    log(f"[bench] oracle: {n} queries in {dt:.1f}s")
    return {"value": round(rate / layers, 3), "unit": "query tokens/s", "cores": 1,
            "kind": "oracle", "per_layer_value": round(rate, 3),
            "extrapolation": f"rate on layer 0 / {layers} layers",
            "sample": f"{n} queries of layer 0 (query 0 of every sequence, then query 1, ...; "
                      f"{tokens} visible tokens, all {w.n_q} heads), numpy float64, 1 process, "
                      f"1 BLAS thread, {dt:.1f} s; host has {os.cpu_count()} logical CPUs"}


def cpu_baseline_cascade(w, layer_cache, q0, plen, slen_np, budget):
    """The float64 cascade oracle on layer 0, whole sequences (index mod B)
    until the budget is spent: sequences per second is decode tokens/s per
    layer, the metric's unit."""
    import numpy as np
    import threadpoolctl

    import workloads as W
    from oracle import paged as ref

    kc, vc, ks, vs = layer_cache
    log("[bench] copying layer 0 to the host for the oracle")
    kb, vb, qb = W.bits(kc), W.bits(vc), W.bits(q0)
    pb = plen // w.bs
    prefix = np.ascontiguousarray(w.block_tables[0, :pb])
    tables = np.ascontiguousarray(w.block_tables[:, pb:])
    n = tokens = 0
    with threadpoolctl.threadpool_limits(1):
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < budget and n < 64 * w.B:
            b = n % w.B
            ref.cascade_decode_attention(qb[b:b + 1], kb, vb, prefix, plen, tables[b:b + 1],
                                         slen_np[b:b + 1], w.scale)
            tokens += plen + int(slen_np[b])
            n += 1
        dt = time.perf_counter() - t0
    log(f"[bench] oracle: {n} sequences in {dt:.1f}s")
    return {"value": round(n / dt, 3), "unit": "decode tokens/s per layer", "cores": 1,
            "kind": "oracle",
            "sample": f"{n} whole sequences of layer 0 (sequence index mod {w.B}; {tokens} tokens "
                      f"attended, all {w.n_q} heads), numpy float64, 1 process, 1 BLAS thread, "
                      f"{dt:.1f} s; host has {os.cpu_count()} logical CPUs"}


def cpu_baseline(w, layer_cache, q0, budget):
    """The float64 oracle, as it stands, on whole sequences of layer 0 until the budget is spent."""
    import numpy as np
    import threadpoolctl

    import workloads as W
    from oracle import paged as ref

    kc, vc, ks, vs = layer_cache
    log("[bench] copying layer 0 to the host for the oracle")
    kb, vb, qb = W.bits(kc), W.bits(vc), W.bits(q0)
    ksn = None if ks is None else ks.cpu().numpy()
    vsn = None if vs is None else vs.cpu().numpy()
    done_tokens = 0
    n = 0
    # one BLAS thread: the oracle's per-head products are matrix-vector
    # products, which a larger BLAS pool measured no faster on
    with threadpoolctl.threadpool_limits(1):
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < budget and n < 64 * w.B:
            b = n % w.B                  # whole sequences of layer 0, cycling if time remains
            ref.decode_attention(qb[b:b + 1], kb, vb, w.block_tables[b:b + 1],
                                 w.context_lens[b:b + 1], w.scale, w.kv_dtype, ksn, vsn)
            done_tokens += int(w.context_lens[b])
            n += 1
        dt = time.perf_counter() - t0
    kv = done_tokens * w.n_kv * w.d * w.p * 2
    log(f"[bench] oracle: {n} sequences in {dt:.1f}s")
    return {"value": round(kv / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{n} whole sequences of layer 0 (sequence index mod {w.B}; {done_tokens} "
                      f"tokens, all {w.n_q} query heads), numpy float64, 1 process, 1 BLAS "
                      f"thread, {dt:.1f} s; host has {os.cpu_count()} logical CPUs"}


def _oracle_worker(job):
    """One process of the multi-process oracle baseline: whole sequences of the
    shared layer, one BLAS thread, until the budget is spent."""
    import numpy as np
    import threadpoolctl

    from oracle import paged as ref

    d, seqs, budget = job
    with threadpoolctl.threadpool_limits(1):
        kb = np.load(d["k"], mmap_mode="r")
        vb = np.load(d["v"], mmap_mode="r")
        qb = np.load(d["q"])
        bt = np.load(d["bt"])
        cl = np.load(d["cl"])
        ks = np.load(d["ks"]) if d.get("ks") else None
        vs = np.load(d["vs"]) if d.get("vs") else None
        tokens = 0
        t0 = time.perf_counter()
        for b in seqs:
            if time.perf_counter() - t0 >= budget:
                break
            ref.decode_attention(qb[b:b + 1], kb, vb, bt[b:b + 1], cl[b:b + 1], d["scale"],
                                 d["kv_dtype"], ks, vs)
            tokens += int(cl[b])
        return tokens, time.perf_counter() - t0


def cpu_baseline_procs(w, layer_cache, q0, budget, procs, pool):
    """The same oracle in `procs` processes (`pool`, started before the GPU was
    touched), each with one BLAS thread, over whole sequences of layer 0
    (sequence i goes to process i mod procs). The layer is shared through
    read-only memory-mapped files."""
    import shutil
    import tempfile

    import numpy as np

    import workloads as W

    kc, vc, ks, vs = layer_cache
    root = tempfile.mkdtemp(prefix="pkv_oracle_", dir="/dev/shm" if os.path.isdir("/dev/shm")
                            else None)
    try:
        d = {"scale": w.scale, "kv_dtype": w.kv_dtype}
        arrays = {"k": W.bits(kc), "v": W.bits(vc), "q": W.bits(q0), "bt": w.block_tables,
                  "cl": w.context_lens}
        if ks is not None:
            arrays["ks"] = ks.cpu().numpy()
            arrays["vs"] = vs.cpu().numpy()
        for name, arr in arrays.items():
            d[name] = os.path.join(root, name + ".npy")
            np.save(d[name], arr)
        del arrays
        seqs = [list(range(i, 64 * w.B, procs)) for i in range(procs)]
        jobs = [(d, [b % w.B for b in s], budget) for s in seqs]
        log(f"[bench] oracle in {procs} processes")
        res = pool.map(_oracle_worker, jobs, chunksize=1)
    finally:
        shutil.rmtree(root, ignore_errors=True)
    tokens = sum(r[0] for r in res)
    dt = max(r[1] for r in res)
    kv = tokens * w.n_kv * w.d * w.p * 2
    log(f"[bench] oracle, {procs} processes: {tokens} tokens in {dt:.1f}s")
    return {"value": round(kv / dt / 1e9, 4), "unit": "GB/s", "cores": procs, "kind": "oracle",
            "sample": f"whole sequences of layer 0 split over {procs} processes (one BLAS "
                      f"thread each; {tokens} tokens, all {w.n_q} query heads), numpy float64, "
                      f"{dt:.1f} s; host has {os.cpu_count()} logical CPUs"}


if __name__ == "__main__":
    main()

"""The algorithmic byte counts behind bench.py's roofline, pinned on the CPU.

The KV term must reproduce the pages' closed form for KV bytes per token,
2 * L * n_kv * d_head * p ([SMTS] "Quantifying the KV-Cache Memory Wall";
[MTKV] "The Anatomy of the KV-Cache Memory Wall"; [LLMI] "5. Mathematics:
Sizing the KV Cache"): 327,680 B per token at L = 80, n_kv = 8, d = 128,
2-byte elements. The partition kernel's launch total must be that term plus
exactly the queries, table entries, scales and outputs it moves.
"""

import bench
import workloads as W
from oracle import sizing


def test_70b_step_reads_the_closed_form_kv_bytes():
    w = W.gqa_70b()
    per_token = sizing.kv_bytes_per_token(80, 8, 128, 2)
    assert per_token == 327_680
    # one decode step attends 64 x 8192 tokens in each of the 80 layers
    assert bench.kv_bytes(w) * w.layers == 64 * 8192 * per_token == 171_798_691_840


def test_70b_layer_launch_bytes():
    w = W.gqa_70b()
    kv = 64 * 8192 * 8 * 128 * 2 * 2            # K and V of one layer
    q = 64 * 64 * 128 * 2                        # bf16 queries
    table = 64 * (8192 // 16) * 4                # one int32 entry per attended block
    out = 64 * 64 * 128 * 4                      # fp32 output, single pass
    assert bench.partition_bytes(w, 8192) == kv + q + table + out == 2_150_760_448


def test_split_launch_writes_partials_instead_of_the_output():
    w = W.gqa_70b()
    single = bench.partition_bytes(w, 8192)
    split = bench.partition_bytes(w, 4096)      # 2 partitions of every sequence
    out = 64 * 64 * 128 * 4
    partials = 64 * 2 * 64 * (128 + 2) * 4      # (m, l, o) per partition and head
    assert split - single == partials - out


def test_quantised_launch_counts_bytes_per_element_and_scales():
    w = W.gqa_70b_fp8()
    ctx = [int(c) for c in w.context_lens]
    kv = sum(ctx) * 8 * 128 * 1 * 2
    assert bench.kv_bytes(w) == kv
    P = 16384
    n_part = sum(-(-c // P) for c in ctx)
    expect = (kv + w.B * 64 * 128 * 2 + sum(-(-c // 32) for c in ctx) * 4
              + n_part * 64 * 130 * 4 + 2 * 8 * 4)
    assert bench.partition_bytes(w, P) == expect
    # FP4: half a byte per element
    w4 = W.gqa_70b_fp4(layers=1)
    assert bench.kv_bytes(w4) * 4 == bench.kv_bytes(W.gqa_70b(layers=1))


def test_prompt_chunk_flops_count_every_visible_pair_once():
    w = W.chunked_prefill_70b()
    # 512 new tokens at the end of each of the 4096/16384/32768/65536-token
    # contexts: query i sees c - 512 + i + 1 tokens
    visible = sum(sum(c - 512 + i + 1 for i in range(512)) for c in (4096, 16384, 32768, 65536))
    flops, _ = bench.multi_query_work(w, 1)
    assert flops == 4 * 128 * 64 * visible == 1_975_718_510_592


def test_verification_bytes_read_the_context_once():
    w = W.spec_verify_70b()
    _, single = bench.multi_query_work(w, 1)
    kv = 64 * 8192 * 8 * 128 * 2 * 2
    qo = 64 * 4 * 64 * 128 * (2 + 4)              # bf16 queries in, fp32 outputs out
    assert single == kv + qo + 64 * 512 * 4 == 2_160_197_632
    _, split = bench.multi_query_work(w, 2)
    assert split - single == 2 * 64 * 4 * 64 * 2 * 130 * 4
    flops, _ = bench.multi_query_work(w, 1)
    assert flops == 4 * 128 * 64 * 64 * (4 * 8192 - 6)


def test_more_than_one_gpu_exits_with_a_message():
    """The library has no multi-GPU path: --gpus N > 1 stops before any work."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_counter_traffic_is_reported_only_for_measured_configurations():
    """While the kernel sources match the committed counters, each decode
    workload at its bench partition has HBM traffic close to its algorithmic
    bytes (no re-reads); other partitions, and changed sources, give None."""
    cases = [(W.gqa_70b(), 8192, 0.01), (W.gqa_70b_fp4(), 8192, 0.01),
             (W.gqa_70b_fp8(), 16384, 0.01), (W.mha_7b(), 8192, 0.01),
             (W.long_shared_prefix(), 512, 0.03)]       # prefix blocks shared: cache hits
    current = bench.counter_traffic(cases[0][0].name, 8192) is not None
    for w, P, tol in cases:
        t = bench.counter_traffic(w.name, P)
        if not current:
            assert t is None
            continue
        algo = bench.partition_bytes(w, P)
        assert abs(t["total"] - algo) <= tol * algo, (w.name, t["total"], algo)
        assert t["total"] == t["read"] + t["written"]
        assert bench.counter_traffic(w.name, P // 2) is None


def test_multi_query_counter_traffic_resolves_while_sources_match():
    """The multi-query workloads' committed counters are found at their bench
    partition while the sources match (verification reads its context once,
    within 1% of its algorithmic bytes); other partitions give None."""
    current = bench.kernel_hash(bench.MQ_KERNEL_SOURCES)
    import json
    committed = json.load(open(bench.MQ_COUNTERS))["kernel_hash"]
    for w in (W.spec_verify_70b(), W.chunked_prefill_70b()):
        t = bench.mq_counter_traffic(w.name, 8192)
        if committed != current:
            assert t is None
            continue
        assert t is not None, w.name
        assert t["total"] == t["read"] + t["written"]
        assert bench.mq_counter_traffic(w.name, 4096) is None
    t = bench.mq_counter_traffic(W.spec_verify_70b().name, 8192)
    if t is not None:
        _, algo = bench.multi_query_work(W.spec_verify_70b(), 1)
        assert abs(t["total"] - algo) <= 0.01 * algo, (t["total"], algo)

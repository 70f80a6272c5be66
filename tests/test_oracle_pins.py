"""Pins of the float64 oracle against facts that do not come from the oracle.

CPU only. Each test names what fixes the expected value: a number the pages
print (tests/golden/), a closed form, a special case with a known answer, a
library routine computing the same definition independently, or an
invariant of the method.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import bf16, paged, sizing
from oracle.block_manager import BlockManagerModel, OutOfBlocks

RNG = np.random.default_rng(2170)


def bf16_bits(x):
    """float array -> bfloat16 patterns via torch's round-to-nearest cast (input helper)."""
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def scatter_to_pool(dense, table, num_blocks, bs, fill=0x7FC0):
    """Test helper: place dense [ctx, n_kv, d] rows into a paged pool (inverse of gather)."""
    ctx, n_kv, d = dense.shape
    pool = np.full((num_blocks, n_kv, bs, d), fill, dtype=dense.dtype)
    for t in range(ctx):
        pool[table[t // bs], :, t % bs, :] = dense[t]
    return pool


# ------------------------------------------------------------------ bf16

def test_bf16_widening_matches_torch_for_all_patterns():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = bf16.to_f64(pats)
    ref = torch.from_numpy(pats.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_bf16_named_values():
    v = bf16.to_f64(np.array([0x3F80, 0xC000, 0x0001, 0x7F80], dtype=np.uint16))
    assert v[0] == 1.0 and v[1] == -2.0 and v[2] == 2.0 ** -133 and v[3] == math.inf


# ------------------------------------------------------------------ sizing (printed values)

def test_kv_bytes_per_token_closed_form(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "kv_sizing.json")))
    bpt = g["bytes_per_token"]
    assert sizing.kv_bytes_per_token(bpt["L"], bpt["n_kv"], bpt["d"], bpt["p"]) == bpt["value"]
    assert f"{sizing.kv_bytes_per_token(80, 8, 128, 2) / 1024:.1f}" == g["kb_per_token_fp16_printed"]
    assert f"{sizing.kv_bytes_per_token(80, 8, 128, 1) / 1024:.1f}" == g["kb_per_token_fp8_printed"]
    # 64 sequences x 8192 tokens at this geometry: the per-step KV read of the 80-layer workload
    assert sizing.kv_bytes(80, 8, 128, 2, S=8192, B=64) == 64 * 8192 * 327680


def test_capacity_model_reproduces_printed_run(golden_dir):
    c = json.load(open(os.path.join(golden_dir, "kv_sizing.json")))["capacity_fp16"]
    r = sizing.capacity(c["params_billion"], c["L"], c["n_kv"], c["d"], c["p"], c["gpu_count"],
                        c["vram_per_gpu_gb"], c["overhead_per_gpu_gb"], c["avg_ctx"], c["max_ctx"])
    assert r["weights_gb"] == c["weights_gb"]
    assert r["usable_gb"] == c["usable_gb"]
    assert r["streams_contiguous"] == c["streams_contiguous"]
    assert r["streams_paged"] == c["streams_paged"]
    assert r["gain_percent"] == c["gain_percent"]


def test_sizing_catches_a_dropped_factor():
    # a plausible slip (forgetting the K+V factor 2, or using n_q instead of n_kv) changes the pin
    assert sizing.kv_bytes_per_token(80, 8, 128, 2) != 80 * 8 * 128 * 2
    assert sizing.kv_bytes_per_token(80, 8, 128, 2) != 2 * 80 * 64 * 128 * 2


# ------------------------------------------------------------------ mapping and gather

def test_block_table_example_from_page(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "block_table_example.json")))
    bs = g["block_size"]
    table = np.array(g["physical"], dtype=np.int32)
    # block b holds the value b in every element: gather must read 7, 2, 19, 4 in order
    pool = np.zeros((24, 1, bs, 8), dtype=np.uint16)
    for b in range(24):
        pool[b] = bf16_bits(np.float32(b))
    out = bf16.to_f64(paged.gather(pool, table, 4 * bs))
    for t in range(4 * bs):
        assert np.all(out[t] == g["physical"][t // bs])
    for pos, slot in g["slots"].items():
        assert paged.slot_of(table, int(pos), bs) == slot
    assert list(paged.slot_mapping(table[None, :].repeat(2, 0), [16, -1], bs)) == [32, -1]


def test_gather_inverts_scatter_and_refuses_out_of_pool_ids():
    bs, n_kv, d, ctx = 4, 2, 8, 23
    dense = RNG.integers(0, 2 ** 16, size=(ctx, n_kv, d)).astype(np.uint16)
    table = RNG.permutation(10)[:6].astype(np.int32)
    pool = scatter_to_pool(dense, table, 10, bs)
    assert np.array_equal(paged.gather(pool, table, ctx), dense)
    bad = table.copy()
    bad[2] = 10
    with pytest.raises(IndexError):
        paged.gather(pool, bad, ctx)


# ------------------------------------------------------------------ attention: special cases

def _one_seq(ctx, n_q, n_kv, d, bs, k_dense, v_dense, q, scale, pool_extra=3):
    nb = (ctx + bs - 1) // bs
    table = RNG.permutation(nb + pool_extra)[:nb].astype(np.int32)
    kp = scatter_to_pool(k_dense, table, nb + pool_extra, bs)
    vp = scatter_to_pool(v_dense, table, nb + pool_extra, bs)
    return paged.decode_attention(q[None], kp, vp, table[None], np.array([ctx]), scale)[0]


def test_single_token_returns_its_value_exactly():
    n_q, n_kv, d = 4, 2, 16
    k = bf16_bits(RNG.standard_normal((1, n_kv, d)))
    v = bf16_bits(RNG.standard_normal((1, n_kv, d)))
    q = bf16_bits(RNG.standard_normal((n_q, d)))
    out = _one_seq(1, n_q, n_kv, d, 16, k, v, q, 0.25)
    for h in range(n_q):
        assert np.array_equal(out[h], bf16.to_f64(v[0, h // 2]))


def test_zero_query_gives_mean_of_values():
    ctx, n_q, n_kv, d = 29, 2, 1, 8
    k = bf16_bits(RNG.standard_normal((ctx, n_kv, d)))
    v = bf16_bits(RNG.standard_normal((ctx, n_kv, d)))
    q = bf16_bits(np.zeros((n_q, d)))
    out = _one_seq(ctx, n_q, n_kv, d, 8, k, v, q, 0.3)
    np.testing.assert_allclose(out[0], np.mean(bf16.to_f64(v[:, 0]), axis=0), rtol=0, atol=1e-14)


def test_constant_values_give_constant_output_and_head_mapping():
    # V of KV head g is the constant g+1: query head h must output h // G + 1
    ctx, n_q, n_kv, d = 45, 8, 4, 16
    k = bf16_bits(RNG.standard_normal((ctx, n_kv, d)))
    v = bf16_bits(np.broadcast_to((np.arange(n_kv) + 1.0)[None, :, None], (ctx, n_kv, d)))
    q = bf16_bits(RNG.standard_normal((n_q, d)))
    out = _one_seq(ctx, n_q, n_kv, d, 16, k, v, q, 0.2)
    for h in range(n_q):
        np.testing.assert_allclose(out[h], h // (n_q // n_kv) + 1.0, rtol=0, atol=1e-13)


def test_power_of_two_weights_closed_form():
    # k_t = a_t e_0, q = e_0, scale = ln 2  =>  weights = 2**a_t / sum 2**a_j; one-hot V reads them out
    ctx, d = 20, 32
    a = RNG.integers(-6, 7, size=ctx).astype(np.float64)
    k = np.zeros((ctx, 1, d))
    k[:, 0, 0] = a
    v = np.zeros((ctx, 1, d))
    v[np.arange(ctx), 0, np.arange(ctx)] = 1.0
    q = np.zeros((1, d))
    q[0, 0] = 1.0
    out = _one_seq(ctx, 1, 1, d, 8, bf16_bits(k), bf16_bits(v), bf16_bits(q), math.log(2.0))
    expect = 2.0 ** a / np.sum(2.0 ** a)
    np.testing.assert_allclose(out[0, :ctx], expect, rtol=1e-14, atol=0)
    assert np.all(out[0, ctx:] == 0)


def test_two_tokens_logistic_closed_form():
    d = 4
    k = np.array([[[1, 0, 2, 0]], [[0, 1, 0, -1]]], dtype=np.float64)
    v = np.array([[[1, 2, 3, 4]], [[-1, 0, 5, 2]]], dtype=np.float64)
    q = np.array([[0.5, -1.0, 1.0, 2.0]])
    scale = 0.75
    s0 = scale * (0.5 + 2.0)
    s1 = scale * (-1.0 - 2.0)
    w0 = 1.0 / (1.0 + math.exp(s1 - s0))
    out = _one_seq(2, 1, 1, d, 16, bf16_bits(k), bf16_bits(v), bf16_bits(q), scale)
    np.testing.assert_allclose(out[0], w0 * v[0, 0] + (1 - w0) * v[1, 0], rtol=1e-15, atol=1e-15)


def test_large_scale_becomes_hard_attention():
    ctx, d = 33, 16
    k = bf16_bits(RNG.standard_normal((ctx, 1, d)))
    v = bf16_bits(RNG.standard_normal((ctx, 1, d)))
    q = bf16_bits(RNG.standard_normal((1, d)))
    s = bf16.to_f64(k[:, 0]) @ bf16.to_f64(q[0])
    out = _one_seq(ctx, 1, 1, d, 8, k, v, q, 1e6)
    np.testing.assert_array_equal(out[0], bf16.to_f64(v[int(np.argmax(s)), 0]))


def test_empty_sequence_outputs_zeros():
    pool = np.zeros((2, 1, 16, 8), dtype=np.uint16)
    q = bf16_bits(np.ones((1, 1, 8)))
    out = paged.decode_attention(q, pool, pool, np.zeros((1, 1), np.int32), np.array([0]), 1.0)
    assert np.array_equal(out, np.zeros((1, 1, 8)))


@pytest.mark.parametrize("ctx,n_q,n_kv,d,bs", [(37, 4, 2, 64, 16), (100, 4, 2, 64, 16),
                                               (70, 8, 1, 32, 32), (51, 6, 6, 16, 16),
                                               (129, 16, 2, 128, 16)])
def test_matches_torch_sdpa_on_dense_copies(ctx, n_q, n_kv, d, bs):
    """Library routine: torch's float64 scaled_dot_product_attention with GQA expansion."""
    k = bf16_bits(RNG.standard_normal((ctx, n_kv, d)))
    v = bf16_bits(RNG.standard_normal((ctx, n_kv, d)))
    q = bf16_bits(RNG.standard_normal((n_q, d)))
    scale = 1.0 / math.sqrt(d)
    out = _one_seq(ctx, n_q, n_kv, d, bs, k, v, q, scale)
    qt = torch.from_numpy(bf16.to_f64(q))[None, :, None, :]            # [1, n_q, 1, d]
    kt = torch.from_numpy(bf16.to_f64(k)).permute(1, 0, 2)[None]        # [1, n_kv, ctx, d]
    vt = torch.from_numpy(bf16.to_f64(v)).permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale,
                                                           enable_gqa=True)[0, :, 0, :]
    np.testing.assert_allclose(out, ref.numpy(), rtol=0, atol=1e-12)


def test_c1_tiny_workload_matches_sdpa():
    import workloads as W
    w = W.tiny()
    kc, vc, _, _ = W.make_cache(w)
    q = W.make_query(w)
    out = paged.decode_attention(W.bits(q), W.bits(kc), W.bits(vc), w.block_tables,
                                 w.context_lens, w.scale)
    assert np.all(np.isfinite(out))
    for b in range(w.B):
        ctx = int(w.context_lens[b])
        kd = torch.from_numpy(bf16.to_f64(paged.gather(W.bits(kc), w.block_tables[b], ctx)))
        vd = torch.from_numpy(bf16.to_f64(paged.gather(W.bits(vc), w.block_tables[b], ctx)))
        qt = torch.from_numpy(bf16.to_f64(W.bits(q)[b]))[None, :, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt, kd.permute(1, 0, 2)[None], vd.permute(1, 0, 2)[None], scale=w.scale,
            enable_gqa=True)[0, :, 0, :]
        np.testing.assert_allclose(out[b], ref.numpy(), rtol=0, atol=1e-12)


# ------------------------------------------------------------------ invariants

def _random_batch(B=3, n_q=4, n_kv=2, d=16, bs=8, lens=(5, 17, 40), extra=4):
    ctx = np.array(lens, dtype=np.int32)
    nb = [(c + bs - 1) // bs for c in ctx]
    pool_n = sum(nb) + extra
    perm = RNG.permutation(pool_n).astype(np.int32)
    bt = np.zeros((B, max(nb)), dtype=np.int32)
    pos = 0
    for b in range(B):
        bt[b, :nb[b]] = perm[pos:pos + nb[b]]
        pos += nb[b]
    kc = bf16_bits(RNG.standard_normal((pool_n, n_kv, bs, d)))
    vc = bf16_bits(RNG.standard_normal((pool_n, n_kv, bs, d)))
    q = bf16_bits(RNG.standard_normal((B, n_q, d)))
    return q, kc, vc, bt, ctx


def test_permuting_physical_blocks_is_invisible():
    q, kc, vc, bt, ctx = _random_batch()
    ref = paged.decode_attention(q, kc, vc, bt, ctx, 0.3)
    sigma = RNG.permutation(kc.shape[0])              # block i moves to sigma[i]
    kp = np.empty_like(kc)
    vp = np.empty_like(vc)
    kp[sigma] = kc
    vp[sigma] = vc
    out = paged.decode_attention(q, kp, vp, sigma[bt].astype(np.int32), ctx, 0.3)
    assert np.array_equal(out, ref)


def test_shared_prefix_equals_private_copies():
    bs, d, n_kv, n_q = 8, 16, 2, 4
    prefix_blocks, B = 3, 3
    lens = np.array([30, 41, 24], dtype=np.int32)
    nb = [(c + bs - 1) // bs for c in lens]
    own = [n - prefix_blocks for n in nb]
    shared_pool = prefix_blocks + sum(own)
    kc = bf16_bits(RNG.standard_normal((shared_pool, n_kv, bs, d)))
    vc = bf16_bits(RNG.standard_normal((shared_pool, n_kv, bs, d)))
    bt = np.zeros((B, max(nb)), dtype=np.int32)
    pos = prefix_blocks
    for b in range(B):
        bt[b, :prefix_blocks] = np.arange(prefix_blocks)
        bt[b, prefix_blocks:nb[b]] = np.arange(pos, pos + own[b])
        pos += own[b]
    q = bf16_bits(RNG.standard_normal((B, n_q, d)))
    shared = paged.decode_attention(q, kc, vc, bt, lens, 0.25)
    # private copies: every sequence gets its own copy of the prefix blocks
    kp = [kc]
    vp = [vc]
    bt2 = bt.copy()
    nxt = shared_pool
    for b in range(1, B):
        kp.append(kc[:prefix_blocks])
        vp.append(vc[:prefix_blocks])
        bt2[b, :prefix_blocks] = np.arange(nxt, nxt + prefix_blocks)
        nxt += prefix_blocks
    private = paged.decode_attention(q, np.concatenate(kp), np.concatenate(vp), bt2, lens, 0.25)
    assert np.array_equal(shared, private)


def test_weights_sum_to_one():
    q, kc, vc, bt, ctx = _random_batch()
    _, w = paged.decode_attention(q, kc, vc, bt, ctx, 0.7, return_weights=True)
    for (b, h), wv in w.items():
        assert len(wv) == ctx[b]
        assert abs(wv.sum() - 1.0) < 1e-12
        assert np.all(wv > 0)


def test_nan_in_unused_blocks_and_tail_slots_is_invisible():
    q, kc, vc, bt, ctx = _random_batch()
    ref = paged.decode_attention(q, kc, vc, bt, ctx, 0.3)
    kn, vn = kc.copy(), vc.copy()
    bs = kc.shape[2]
    used = set()
    for b in range(len(ctx)):
        n = (ctx[b] + bs - 1) // bs
        used.update(bt[b, :n].tolist())
        if ctx[b] % bs:
            last = bt[b, n - 1]
            kn[last, :, ctx[b] % bs:] = 0x7FC0
            vn[last, :, ctx[b] % bs:] = 0x7FC0
    for blk in range(kc.shape[0]):
        if blk not in used:
            kn[blk] = 0x7FC0
            vn[blk] = 0x7FC0
    out = paged.decode_attention(q, kn, vn, bt, ctx, 0.3)
    assert np.all(np.isfinite(out))
    assert np.array_equal(out, ref)


@pytest.mark.parametrize("partition", [1, 7, 8, 16, 512, 10 ** 6])
def test_split_partials_merge_to_the_definition(partition):
    ctx, d = 61, 16
    k = bf16.to_f64(bf16_bits(RNG.standard_normal((ctx, d))))
    v = bf16.to_f64(bf16_bits(RNG.standard_normal((ctx, d))))
    q = bf16.to_f64(bf16_bits(RNG.standard_normal(d)))
    full, _ = paged.attention_one(q, k, v, 0.4)
    m, l, o = paged.split_partials(q, k, v, 0.4, partition)
    assert len(m) == (ctx + partition - 1) // partition
    np.testing.assert_allclose(paged.merge_partials(m, l, o), full, rtol=0, atol=1e-13)


def test_merge_ignores_empty_partitions_and_empty_input():
    m = np.array([0.5, -np.inf, 1.5])
    l = np.array([2.0, 0.0, 3.0])
    o = np.array([[1.0, 0.0], [np.nan, np.nan], [0.0, 1.0]])
    w0, w2 = 2.0 * math.exp(0.5 - 1.5), 3.0
    np.testing.assert_allclose(paged.merge_partials(m, l, o), [w0 / (w0 + w2), w2 / (w0 + w2)],
                               rtol=1e-15)
    assert np.array_equal(paged.merge_partials([-np.inf], [0.0], [[np.nan, 1.0]]), [0.0, 0.0])


# ------------------------------------------------------------------ cache writes

def test_kv_append_writes_only_the_slots():
    bs, n_kv, d, nb = 16, 2, 8, 6
    kc = RNG.integers(0, 2 ** 16, size=(nb, n_kv, bs, d)).astype(np.uint16)
    vc = RNG.integers(0, 2 ** 16, size=(nb, n_kv, bs, d)).astype(np.uint16)
    kn = RNG.integers(0, 2 ** 16, size=(3, n_kv, d)).astype(np.uint16)
    vn = RNG.integers(0, 2 ** 16, size=(3, n_kv, d)).astype(np.uint16)
    slots = np.array([5 * bs + 3, -1, 0], dtype=np.int64)
    k2, v2 = paged.kv_append(kc, vc, kn, vn, slots)
    assert np.array_equal(k2[5, :, 3], kn[0]) and np.array_equal(v2[0, :, 0], vn[2])
    k2[5, :, 3] = kc[5, :, 3]
    k2[0, :, 0] = kc[0, :, 0]
    v2[5, :, 3] = vc[5, :, 3]
    v2[0, :, 0] = vc[0, :, 0]
    assert np.array_equal(k2, kc) and np.array_equal(v2, vc)


def test_kv_append_then_attend_reads_the_new_token():
    # append-then-attend: with ctx = 1 after the append the output is the appended value
    bs, n_kv, d = 16, 1, 8
    kc = np.zeros((2, n_kv, bs, d), dtype=np.uint16)
    vc = np.zeros((2, n_kv, bs, d), dtype=np.uint16)
    table = np.array([[1]], dtype=np.int32)
    slot = paged.slot_mapping(table, [0], bs)
    kn = bf16_bits(RNG.standard_normal((1, n_kv, d)))
    vn = bf16_bits(RNG.standard_normal((1, n_kv, d)))
    k2, v2 = paged.kv_append(kc, vc, kn, vn, slot)
    q = bf16_bits(RNG.standard_normal((1, 1, d)))
    out = paged.decode_attention(q, k2, v2, table, np.array([1]), 1.0)
    assert np.array_equal(out[0, 0], bf16.to_f64(vn[0, 0]))


def test_copy_blocks_reads_the_original_cache():
    c = RNG.integers(0, 255, size=(5, 2, 4, 3)).astype(np.uint8)
    out = paged.copy_blocks(c, [[0, 3], [3, 4]])
    assert np.array_equal(out[3], c[0]) and np.array_equal(out[4], c[3])
    assert np.array_equal(out[:3], c[:3])


# ------------------------------------------------------------------ block manager model

def test_allocator_pops_the_end_of_the_pool_and_counts_references():
    bm = BlockManagerModel(4, 16)
    slot, src, dst = bm.append_slot(7)
    assert (slot, src, dst) == (3 * 16, -1, -1)          # first block handed out is the last one
    assert bm.ref[3] == 1 and bm.free_pool == [0, 1, 2]
    for _ in range(15):
        bm.append_slot(7)
    slot, _, _ = bm.append_slot(7)                      # token 16 opens a new block
    assert slot == 2 * 16 and bm.tables[7] == [3, 2]


def test_allocator_exhaustion_raises_and_changes_nothing():
    bm = BlockManagerModel(1, 4)
    bm.append_slot(0)
    for _ in range(3):
        bm.append_slot(0)
    with pytest.raises(OutOfBlocks):
        bm.append_slot(0)
    assert bm.lens[0] == 4 and bm.tables[0] == [0]


def test_fork_shares_and_append_copies_on_write():
    bm = BlockManagerModel(8, 4)
    for _ in range(6):                                   # 1.5 blocks: [7, 6]
        bm.append_slot("a")
    bm.fork("a", "b")
    assert bm.ref[7] == 2 and bm.ref[6] == 2
    slot, src, dst = bm.append_slot("b")                 # partial last block is shared -> CoW
    assert (src, dst) == (6, 5) and slot == 5 * 4 + 2
    assert bm.tables["b"] == [7, 5] and bm.tables["a"] == [7, 6]
    assert bm.ref[6] == 1 and bm.ref[5] == 1
    slot, src, dst = bm.append_slot("a")                 # 'a' owns block 6 alone now: no copy
    assert (src, dst) == (-1, -1) and slot == 6 * 4 + 2
    bm.free("a")
    assert bm.ref[7] == 1 and 6 in bm.free_pool and 7 not in bm.free_pool
    bm.free("b")
    assert sorted(bm.free_pool) == list(range(8))

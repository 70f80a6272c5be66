"""Debug mode: caller errors in device data reported at the next call.

Every input below is memory-safe for the kernels in normal mode (an
out-of-range block id reads block 0, an out-of-pool slot or copy pair is
skipped, query counts are clamped), so these tests only check that debug mode
reports them, clears the report, and leaves valid calls untouched.
"""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import paged as ref

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def pkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_217_amd as m
    return m


@pytest.fixture
def dbg(pkv):
    pkv.set_debug(True)
    try:
        pkv.debug_check()
    except pkv.PkvError:
        pass
    yield pkv
    try:
        pkv.debug_check()
    finally:
        pkv.set_debug(False)


def reported(pkv):
    """True if a caller error is pending; the report is cleared either way."""
    try:
        pkv.debug_check()
    except pkv.PkvError as e:
        assert e.status == 1          # PKV_ERR_INVALID_ARG
        pkv.debug_check()             # cleared
        return True
    return False


def setup(w):
    kc, vc, ks, vs = W.make_cache(w, poison_unused=False)
    q = W.make_query(w)
    return (kc.to(DEV), vc.to(DEV), q.to(DEV), torch.from_numpy(w.block_tables).to(DEV),
            torch.from_numpy(w.context_lens).to(DEV), kc, vc, q)


def test_valid_calls_report_nothing_and_match_normal_mode(pkv, dbg):
    w = W.custom("dbg_ok", [5, 40, 300], 16, 2, 128, 16, W.BF16, seed=60)
    kd, vd, qd, bt, cl, kc, vc, q = setup(w)
    pkv.set_debug(False)
    out0 = pkv.paged_decode_attention(qd, kd, vd, bt, cl, w.scale, 300, partition_size=32)
    pkv.set_debug(True)
    out1 = pkv.paged_decode_attention(qd, kd, vd, bt, cl, w.scale, 300, partition_size=32)
    torch.cuda.synchronize()
    assert not reported(pkv)
    assert torch.equal(out0, out1)
    expect = ref.decode_attention(W.bits(q), W.bits(kc), W.bits(vc), w.block_tables,
                                  w.context_lens, w.scale)
    assert np.max(np.abs(out1.cpu().double().numpy() - expect)) <= 1e-2


@pytest.mark.parametrize("bad", [-1, "pool"])
def test_out_of_pool_table_entry_is_reported_at_the_next_call(pkv, dbg, bad):
    w = W.custom("dbg_tab", [40, 100], 8, 2, 64, 16, W.BF16, seed=61)
    kd, vd, qd, bt, cl, *_ = setup(w)
    bt[1, 3] = w.num_blocks if bad == "pool" else bad     # a live entry (100 tokens: 7 blocks)
    pkv.paged_decode_attention(qd, kd, vd, bt, cl, w.scale, 100)
    # the next call that takes device data reports it and enqueues nothing
    slots = torch.tensor([0], dtype=torch.int64, device=DEV)
    k_new = torch.zeros((1, 2, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(pkv.PkvError) as e:
        pkv.kv_append(kd, vd, k_new, k_new, slots)
    assert e.value.status == 1
    assert not reported(pkv)                               # the report was cleared


def test_entries_past_the_length_are_not_checked(pkv, dbg):
    w = W.custom("dbg_tail", [20, 33], 8, 2, 64, 16, W.BF16, seed=62, extra_blocks=0)
    kd, vd, qd, bt, cl, *_ = setup(w)
    bt[0, 2:] = -7                                          # 20 tokens use entries 0 and 1
    bt[1, 3:] = 1 << 30                                     # 33 tokens use entries 0..2
    pkv.paged_decode_attention(qd, kd, vd, bt, cl, w.scale, 33)
    assert not reported(pkv)


def test_length_above_the_stated_bound_is_reported(pkv, dbg):
    w = W.custom("dbg_len", [64, 64], 8, 2, 64, 16, W.BF16, seed=63)
    kd, vd, qd, bt, cl, *_ = setup(w)
    pkv.paged_decode_attention(qd, kd, vd, bt, cl, w.scale, 48)     # bound below 64
    assert reported(pkv)
    cl[0] = -1
    pkv.paged_decode_attention(qd, kd, vd, bt, cl, w.scale, 64)
    assert reported(pkv)


def test_kv_append_slots(pkv, dbg):
    w = W.custom("dbg_slots", [10], 4, 2, 64, 16, W.BF16, seed=64)
    kd, vd, *_ = setup(w)
    pool = w.num_blocks * w.bs
    k_new = torch.zeros((3, 2, 64), dtype=torch.bfloat16, device=DEV)
    for slots, bad in (([5, 9, -1], False), ([5, 9, 5], True), ([5, pool, 1], True),
                       ([-1, -1, 3], False)):
        pkv.kv_append(kd, vd, k_new, k_new,
                      torch.tensor(slots, dtype=torch.int64, device=DEV))
        assert reported(pkv) == bad, slots


def test_copy_pairs(pkv, dbg):
    w = W.custom("dbg_copy", [10], 4, 2, 64, 16, W.BF16, seed=65, extra_blocks=8)
    kd, vd, *_ = setup(w)
    n = w.num_blocks
    for pairs, bad in (([[1, 2], [3, 4]], False), ([[1, n], [3, 4]], True),
                       ([[1, 2], [3, 2]], True), ([[1, 2], [2, 3]], True),
                       ([[-1, 2]], True)):
        pkv.copy_blocks(kd, vd, torch.tensor(pairs, dtype=torch.int32, device=DEV))
        assert reported(pkv) == bad, pairs


def test_multi_query_counts_and_tables(pkv, dbg):
    w = W.custom("dbg_mq", [30, 50], 16, 2, 128, 16, W.BF16, seed=66)
    kd, vd, _, bt, cl, *_ = setup(w)
    Q = 4
    q = torch.zeros((2, Q, 16, 128), dtype=torch.bfloat16, device=DEV)
    for ql, bad in (([4, 2], False), ([5, 2], True), ([-1, 0], True)):
        qlt = torch.tensor(ql, dtype=torch.int32, device=DEV)
        pkv.paged_multi_query_attention(q, qlt, kd, vd, bt, cl, w.scale, 50)
        assert reported(pkv) == bad, ql
    bt[0, 0] = w.num_blocks
    pkv.paged_multi_query_attention(q, torch.tensor([4, 2], dtype=torch.int32, device=DEV),
                                    kd, vd, bt, cl, w.scale, 50)
    assert reported(pkv)


def test_shared_prefix_table(pkv, dbg):
    bs, B, n_q, n_kv, d = 16, 4, 16, 2, 128
    w = W.custom("dbg_cas", [64 + 20] * B, n_q, n_kv, d, bs, W.BF16, seed=67)
    kd, vd, qd, bt, cl, *_ = setup(w)
    prefix = bt[0, :4].contiguous()                         # 64 tokens
    suffix_tables = bt[:, 4:].contiguous()
    suffix_lens = torch.full((B,), 20, dtype=torch.int32, device=DEV)
    pkv.cascade_decode_attention(qd, kd, vd, prefix, 64, suffix_tables, suffix_lens, w.scale, 20)
    assert not reported(pkv)
    prefix[2] = -3
    pkv.cascade_decode_attention(qd, kd, vd, prefix, 64, suffix_tables, suffix_lens, w.scale, 20)
    assert reported(pkv)


def test_gather_row(pkv, dbg):
    w = W.custom("dbg_gather", [40], 4, 2, 64, 16, W.BF16, seed=68)
    kd, vd, _, bt, *_ = setup(w)
    row = bt[0].contiguous()
    pkv.gather_kv(kd, vd, row, 40)
    assert not reported(pkv)
    row[1] = w.num_blocks + 5
    pkv.gather_kv(kd, vd, row, 40)
    assert reported(pkv)


def test_debug_off_reports_nothing(pkv):
    pkv.set_debug(False)
    w = W.custom("dbg_off", [40, 100], 8, 2, 64, 16, W.BF16, seed=69)
    kd, vd, qd, bt, cl, *_ = setup(w)
    bt[1, 3] = w.num_blocks
    out = pkv.paged_decode_attention(qd, kd, vd, bt, cl, w.scale, 100)
    torch.cuda.synchronize()
    pkv.debug_check()                                        # off: always OK
    assert torch.isfinite(out).all()


def test_schedule_for_other_geometry_or_items_is_reported(pkv, dbg):
    # A schedule built for this call is accepted; one built for other lengths
    # (another item count), another partition size or another batch, or one
    # whose items name a sequence outside the call, is reported. In normal
    # mode the kernel reads no item of a list whose header does not match and
    # skips items outside the call, so these calls stay inside the arrays.
    w = W.custom("dbg_sched", [40, 700, 300, 1], 16, 2, 128, 16, W.BF16, seed=66)
    kd, vd, qd, bt, cl, kc, vc, q = setup(w)
    P = 64
    good = pkv.decode_schedule(cl, 700, P)
    pkv.paged_decode_attention(qd, kd, vd, bt, cl, w.scale, 700, partition_size=P, schedule=good)
    torch.cuda.synchronize()
    assert not reported(pkv)

    other_lens = cl.clone()
    other_lens[1] = 600                                  # one partition fewer
    bad_count = pkv.decode_schedule(other_lens, 700, P)
    other_P = pkv.decode_schedule(cl, 700, 2 * P)        # 11 partitions of 128, not 64
    bad_items = good.clone()
    bad_items[8] = 9                                     # first item's sequence: not in the call
    cases = [("count", bad_count, 700), ("partition", other_P, 700),
             ("items", bad_items, 700)]
    for what, sched, max_ctx in cases:
        print(f"[schedule check] {what}", flush=True)
        pkv.paged_decode_attention(qd, kd, vd, bt, cl, w.scale, max_ctx, partition_size=P,
                                   schedule=sched)
        torch.cuda.synchronize()
        assert reported(pkv), what
    # a header recording another batch size
    half = pkv.decode_schedule(cl[:2].contiguous(), 700, P)
    pkv.paged_decode_attention(qd, kd, vd, bt, cl, w.scale, 700, partition_size=P,
                               schedule=torch.cat([half, torch.zeros_like(good)])[:good.numel()])
    torch.cuda.synchronize()
    assert reported(pkv), "batch"

    # normal mode: the same calls complete, and a valid one afterwards is unaffected
    pkv.set_debug(False)
    for _, sched, max_ctx in cases:
        pkv.paged_decode_attention(qd, kd, vd, bt, cl, w.scale, max_ctx, partition_size=P,
                                   schedule=sched)
    ok = pkv.paged_decode_attention(qd, kd, vd, bt, cl, w.scale, 700, partition_size=P,
                                    schedule=good)
    torch.cuda.synchronize()
    pkv.set_debug(True)
    expect = ref.decode_attention(W.bits(q), W.bits(kc), W.bits(vc), w.block_tables,
                                  w.context_lens, w.scale)
    got = ok.cpu().double().numpy()
    assert np.max(np.abs(got - expect)) <= 1e-2
    assert np.linalg.norm(got - expect) / np.linalg.norm(expect) <= 1e-4


def test_cascade_suffix_schedule_for_other_lengths_is_reported(pkv, dbg):
    # The suffixes' longest-first list a caller builds once per step: one
    # built for these suffix lengths is accepted, one built for other lengths
    # (another item count) is reported.
    bs, B, n_q, n_kv, d = 16, 4, 16, 2, 128
    w = W.custom("dbg_cas_sched", [64 + 300, 64 + 20, 64 + 180, 64 + 5], n_q, n_kv, d, bs,
                 W.BF16, seed=68)
    kd, vd, qd, bt, cl, *_ = setup(w)
    prefix = bt[0, :4].contiguous()                         # 64 tokens
    suffix_tables = bt[:, 4:].contiguous()
    suffix_lens = (cl - 64).contiguous()
    Ps = 64
    good = pkv.cascade_schedule(kd, suffix_lens, n_q, 64, 300, 0, Ps)
    assert good is not None
    pkv.cascade_decode_attention(qd, kd, vd, prefix, 64, suffix_tables, suffix_lens, w.scale, 300,
                                 suffix_partition=Ps, schedule=good)
    torch.cuda.synchronize()
    assert not reported(pkv)
    other = suffix_lens.clone()
    other[0] = 200                                          # two partitions fewer
    bad = pkv.cascade_schedule(kd, other, n_q, 64, 300, 0, Ps)
    pkv.cascade_decode_attention(qd, kd, vd, prefix, 64, suffix_tables, suffix_lens, w.scale, 300,
                                 suffix_partition=Ps, schedule=bad)
    torch.cuda.synchronize()
    assert reported(pkv)

"""Pins of the oracle's swap to host memory and the allocator's swap
lifecycle (CPU only).

A swap moves bytes, so the data side is pinned by what a copy must satisfy:
out-then-in to the same blocks is the identity; in to fresh blocks leaves
every logical block, and hence attention through the new table, unchanged;
ids outside the pool read as zeros and are skipped on the way in. The
allocator side is pinned by conservation of blocks and reference counts, by
sharing surviving a sharer's swap-out, and by an exhausted pool changing
nothing.
"""

import numpy as np
import pytest

from oracle import paged
from oracle.block_manager import BlockManagerModel, OutOfBlocks

RNG = np.random.default_rng(21708)


def caches(nb=12, n_kv=2, bs=4, d=8):
    k = RNG.integers(0, 2**16, size=(nb, n_kv, bs, d), dtype=np.uint16)
    v = RNG.integers(0, 2**16, size=(nb, n_kv, bs, d), dtype=np.uint16)
    return k, v


def test_out_then_in_to_the_same_blocks_is_the_identity():
    k, v = caches()
    ids = [3, 0, 11, 7]
    host = paged.swap_out(k, v, ids)
    assert host.shape == (2, 4) + k.shape[1:]
    assert np.array_equal(host[0, 2], k[11]) and np.array_equal(host[1, 0], v[3])
    scrambled_k, scrambled_v = k.copy(), v.copy()
    scrambled_k[ids] = 0
    scrambled_v[ids] = 0xFFFF
    k2, v2 = paged.swap_in(scrambled_k, scrambled_v, ids, host)
    assert np.array_equal(k2, k) and np.array_equal(v2, v)


def test_ids_outside_the_pool():
    k, v = caches()
    host = paged.swap_out(k, v, [1, -1, 12])
    assert not host[:, 1:].any()
    k2, v2 = paged.swap_in(k, v, [-5, 40], np.ones((2, 2) + k.shape[1:], dtype=k.dtype))
    assert np.array_equal(k2, k) and np.array_equal(v2, v)


def bf16_bits(x):
    import torch
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_attention_through_fresh_blocks_is_unchanged():
    # a sequence of 10 tokens (3 blocks of 4) is swapped out, its blocks are
    # overwritten by someone else, and it comes back in three other blocks
    nb, n_kv, bs, d, n_q = 16, 2, 4, 8, 4
    k = bf16_bits(RNG.standard_normal((nb, n_kv, bs, d)))
    v = bf16_bits(RNG.standard_normal((nb, n_kv, bs, d)))
    q = bf16_bits(RNG.standard_normal((1, n_q, d)))
    old = [5, 9, 2]
    before = paged.decode_attention(q, k, v, np.array([old], np.int32), np.array([10], np.int32),
                                    0.35)
    host = paged.swap_out(k, v, old)
    k[old] = bf16_bits(RNG.standard_normal((3, n_kv, bs, d)))
    new = [14, 0, 7]
    k2, v2 = paged.swap_in(k, v, new, host)
    after = paged.decode_attention(q, k2, v2, np.array([new], np.int32),
                                   np.array([10], np.int32), 0.35)
    assert np.array_equal(before, after)


def test_swap_lifecycle_of_the_allocator():
    bm = BlockManagerModel(8, 4)
    for _ in range(6):
        bm.append_slot("a")                   # 2 blocks
    bm.fork("a", "b")                         # shared, ref 2
    for _ in range(3):
        bm.append_slot("c")                   # 1 block
    shared = list(bm.tables["a"])
    out = bm.swap_out("b")
    assert out == shared                      # logical order, for the copy
    assert all(bm.ref[x] == 1 for x in shared)   # still resident for "a"
    assert bm.lens["b"] == 6 and "b" in bm.swapped
    with pytest.raises(ValueError):
        bm.append_slot("b")
    with pytest.raises(ValueError):
        bm.export_table(["b"], 4)
    with pytest.raises(KeyError):
        bm.fork("b", "z")
    free_before = list(bm.free_pool)
    new = bm.swap_in("b")
    assert len(new) == 2 and not set(new) & set(shared)   # private copies
    assert new == [free_before[-1], free_before[-2]]      # popped in logical order
    assert bm.export_table(["b"], 2) == [new]
    # conservation: every block is free or referenced exactly ref times
    held = sum(len(t) for t in bm.tables.values())
    assert sum(bm.ref) == held and len(bm.free_pool) + len({x for t in bm.tables.values() for x in t}) == 8


def test_swap_in_needs_room_and_changes_nothing_without_it():
    bm = BlockManagerModel(3, 4)
    for _ in range(9):
        bm.append_slot("a")                   # 3 blocks: the whole pool
    bm.swap_out("a")
    bm.append_slot("b")
    bm.append_slot("c")
    bm.append_slot("c")
    state = (list(bm.free_pool), list(bm.ref), dict(bm.tables))
    with pytest.raises(OutOfBlocks):
        bm.swap_in("a")                       # needs 3, 2 left... 1 left
    assert (list(bm.free_pool), list(bm.ref), dict(bm.tables)) == state
    assert "a" in bm.swapped
    bm.free("a")                              # a swapped sequence can be dropped
    assert "a" not in bm.lens and "a" not in bm.swapped

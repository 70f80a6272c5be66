"""GPU parity of KV swap to host memory and back, through the C ABI.

Bars: the host image and the caches after swap-in are bit-exact against the
oracle's copy (ids outside the pool included); a preempted sequence whose
blocks were reused while it was on the host attends bit-identically after
coming back in fresh blocks (the kernels' arithmetic does not depend on
physical block ids); the swap runs on a second stream of default priority.
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


def buffers(pkv, kc, n):
    nbytes = pkv.swap_bytes(kc, n)
    staging = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=DEV)
    host = torch.empty(max(nbytes, 16), dtype=torch.uint8, pin_memory=True)
    return staging, host, nbytes


@pytest.mark.parametrize("dtype,bs,d,n_kv", [(W.BF16, 16, 128, 8), (W.FP8, 32, 128, 8),
                                             (W.BF16, 32, 64, 2)])
def test_swap_round_trip_bit_exact(pkv, dtype, bs, d, n_kv):
    w = W.custom("swap", [700, 1300, 45], 2 * n_kv, n_kv, d, bs, dtype, seed=90)
    kc, vc, _, _ = W.make_cache(w)
    nb = kc.shape[0]
    ids = np.array([5, nb - 1, 0, -3, nb + 7, 17, 33], dtype=np.int32)
    kd, vd = kc.to(DEV), vc.to(DEV)
    staging, host, nbytes = buffers(pkv, kd, len(ids))
    ids_d = torch.from_numpy(ids).to(DEV)
    pkv.swap_out(kd, vd, ids_d, staging, host)
    torch.cuda.synchronize()
    expect = ref.swap_out(W.bits(kc), W.bits(vc), ids)
    got = host[:nbytes].numpy().view(expect.dtype).reshape(expect.shape)
    assert np.array_equal(got, expect)
    # back into other blocks (one id outside the pool, skipped)
    dst = np.array([40, 41, 2, 44, -1, 46, 47], dtype=np.int32)
    pkv.swap_in(kd, vd, torch.from_numpy(dst).to(DEV), staging, host)
    torch.cuda.synchronize()
    k2, v2 = ref.swap_in(W.bits(kc), W.bits(vc), dst, expect)
    assert np.array_equal(W.bits(kd), k2) and np.array_equal(W.bits(vd), v2)


def test_preempted_sequence_comes_back_identical(pkv):
    """Three sequences grow through the block manager; one is swapped out on a
    second stream, its blocks are taken over by a new sequence, it is swapped
    back into fresh blocks and attends exactly as before."""
    n_kv, n_q, d, bs, nb = 8, 64, 128, 16, 128
    bm = pkv.BlockManager(nb, bs)
    kd = torch.zeros((nb, n_kv, bs, d), dtype=torch.bfloat16, device=DEV)
    vd = torch.zeros_like(kd)
    g = torch.Generator(device="cpu").manual_seed(2172)

    def grow(seq, n):
        slots = []
        for _ in range(n):
            slot, src, dst = bm.append_slot(seq)
            assert src == -1
            slots.append(slot)
        k = torch.randn((n, n_kv, d), generator=g).to(torch.bfloat16).to(DEV)
        v = torch.randn((n, n_kv, d), generator=g).to(torch.bfloat16).to(DEV)
        pkv.kv_append(kd, vd, k, v, torch.tensor(slots, dtype=torch.int64, device=DEV))

    lens = {1: 300, 2: 333, 3: 401}      # 19 + 21 + 26 of 128 blocks
    for s, n in lens.items():
        grow(s, n)
    q = torch.randn((3, n_q, d), generator=g).to(torch.bfloat16).to(DEV)
    mb = 64

    def attend(seqs):
        bt = torch.tensor(bm.export_table(seqs, mb), dtype=torch.int32, device=DEV)
        cl = torch.tensor([bm.seq_len(s) for s in seqs], dtype=torch.int32, device=DEV)
        return pkv.paged_decode_attention(q[:len(seqs)], kd, vd, bt, cl, 0.0884,
                                          int(cl.max()), partition_size=256)

    before = attend([1, 2, 3])
    side = torch.cuda.Stream()                      # default priority
    blocks = bm.swap_out(2)
    staging, host, _ = buffers(pkv, kd, len(blocks))
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        pkv.swap_out(kd, vd, torch.tensor(blocks, dtype=torch.int32, device=DEV), staging, host,
                     stream=side)
    torch.cuda.current_stream().wait_stream(side)   # reuse of the blocks is ordered after
    grow(4, 500)                                    # takes over sequence 2's blocks
    assert set(bm.export_table([4], mb)[0][:len(blocks)]) & set(blocks)
    fresh = bm.swap_in(2)
    assert len(fresh) == len(blocks) and not set(fresh) & set(blocks)
    with torch.cuda.stream(side):
        side.wait_stream(torch.cuda.current_stream())
        pkv.swap_in(kd, vd, torch.tensor(fresh, dtype=torch.int32, device=DEV), staging, host,
                    stream=side)
    torch.cuda.current_stream().wait_stream(side)
    after = attend([1, 2, 3])
    torch.cuda.synchronize()
    assert torch.equal(before, after)
    # and against the oracle on the final cache
    bt = np.array(bm.export_table([1, 2, 3], mb), dtype=np.int32)
    cl = np.array([lens[1], lens[2], lens[3]], dtype=np.int32)
    expect = ref.decode_attention(W.bits(q), W.bits(kd), W.bits(vd), bt, cl, 0.0884)
    assert np.max(np.abs(after.cpu().double().numpy() - expect)) <= 1e-2
    bm.close()

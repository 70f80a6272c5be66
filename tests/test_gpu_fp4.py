"""GPU parity of FP4 E2M1 KV (two codes per byte, per-head scales) against the
oracle, through the C ABI.

Bars: kv_append, copies, gathers and swaps are bit-exact; attention max abs
error <= 3e-2 (as FP8: the oracle dequantises the same codes with the same
scales) and relative L2 <= 1e-4. With one cached token the output is exactly
that token's dequantised V row, which pins the hardware conversion's nibble
order on all 256 byte patterns. Decode, multi-token queries (both kernels:
fewer and more than 128 rows per KV head) and shared-prefix attention run on
FP4 caches.
"""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import fp4_e2m1 as fp4
from oracle import paged as ref

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
F4 = torch.float4_e2m1fn_x2


@pytest.fixture(scope="module")
def pkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_217_amd as m
    return m


def test_single_token_reads_every_byte_pattern(pkv):
    n_kv, bs, d, B, n_q = 2, 16, 128, 4, 4
    nb = 8
    k = torch.zeros((nb, n_kv, bs, d // 2), dtype=torch.uint8)
    v = torch.zeros_like(k)
    pat = torch.arange(256, dtype=torch.uint8).view(4, 64)
    for b in range(B):
        v[b, :, 0, :] = pat[b]                     # sequence b's only token
        k[b, :, 0, :] = pat[(b + 1) % 4]
    ks = torch.tensor([0.5, 0.375])
    vs = torch.tensor([0.25, 0.4375])
    q = torch.randn((B, n_q, d)).to(torch.bfloat16)
    bt = torch.arange(B, dtype=torch.int32).view(B, 1)
    cl = torch.ones(B, dtype=torch.int32)
    out = pkv.paged_decode_attention(q.to(DEV), k.view(F4).to(DEV), v.view(F4).to(DEV),
                                     bt.to(DEV), cl.to(DEV), 0.1, 1, k_scale=ks.to(DEV),
                                     v_scale=vs.to(DEV))
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for b in range(B):
        for h in range(n_q):
            g = h // 2
            row = fp4.decode(fp4.unpack(pat[b].numpy())) * np.float64(vs[g])
            assert np.allclose(got[b, h], row, rtol=2e-7, atol=0), (b, h)


@pytest.mark.parametrize("bs,n_kv", [(16, 8), (32, 2)])
def test_kv_append_fp4_every_bf16_pattern(pkv, bs, n_kv):
    d = 128
    T = 65536 // (n_kv * d)                         # every bf16 pattern once per scale set
    pats = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(T, n_kv, d)
    for scale_set in ([1.0, 0.5, 3.0, 1e-3, 7.0, 0.1, 2.0, 1e4][:n_kv],
                      [0.0625] * n_kv):
        ks = torch.tensor(scale_set, dtype=torch.float32)
        vs = ks.flip(0).contiguous()
        nb = T // bs + 1
        k = torch.zeros((nb, n_kv, bs, d // 2), dtype=torch.uint8)
        v = torch.zeros_like(k)
        slots = torch.arange(T, dtype=torch.int64)
        knew = pats.view(torch.bfloat16)
        vnew = pats.flip(0).contiguous().view(torch.bfloat16)
        kd, vd = k.view(F4).to(DEV), v.view(F4).to(DEV)
        pkv.kv_append(kd, vd, knew.to(DEV), vnew.to(DEV), slots.to(DEV), ks.to(DEV), vs.to(DEV))
        torch.cuda.synchronize()
        ek, ev = ref.kv_append(k.numpy(), v.numpy(), W.bits(knew), W.bits(vnew), slots.numpy(),
                               ref.FP4, ks.numpy(), vs.numpy())
        assert np.array_equal(W.bits(kd), ek) and np.array_equal(W.bits(vd), ev)


SHAPES = [
    # lengths, n_q, n_kv, bs, partition
    ([1, 15, 16, 17, 200], 8, 8, 16, 0),
    ([1, 15, 16, 17, 200], 8, 8, 16, 16),
    ([33, 64, 700, 129], 64, 8, 32, 0),
    ([33, 64, 700, 129], 64, 8, 32, 64),
    ([1000, 7, 4096], 32, 2, 16, 512),               # G = 16
    ([100, 333], 64, 1, 16, 128),                    # MQA
    ([0, 5, 3000], 16, 8, 32, 1024),                 # an empty sequence
]


@pytest.mark.parametrize("case", SHAPES, ids=[str(i) for i in range(len(SHAPES))])
def test_fp4_decode_shapes(pkv, case):
    lens, n_q, n_kv, bs, P = case
    w = W.custom("fp4", lens, n_q, n_kv, 128, bs, W.FP4, seed=120 + SHAPES.index(case))
    kc, vc, ks, vs = W.make_cache(w)
    q = W.make_query(w)
    out = pkv.paged_decode_attention(q.to(DEV), kc.to(DEV), vc.to(DEV),
                                     torch.from_numpy(w.block_tables).to(DEV),
                                     torch.from_numpy(w.context_lens).to(DEV), w.scale,
                                     int(w.context_lens.max()), k_scale=ks.to(DEV),
                                     v_scale=vs.to(DEV), partition_size=P)
    torch.cuda.synchronize()
    expect = ref.decode_attention(W.bits(q), W.bits(kc), W.bits(vc), w.block_tables,
                                  w.context_lens, w.scale, ref.FP4, ks.numpy(), vs.numpy())
    got = out.cpu().double().numpy()
    assert np.all(np.isfinite(got))
    err = np.max(np.abs(got - expect))
    rel = np.linalg.norm(got - expect) / max(np.linalg.norm(expect), 1e-30)
    assert err <= 3e-2 and rel <= 1e-4, (err, rel)


def test_fp4_decode_query_dynamic_range(pkv):
    # FP4 K is widened exactly to bf16 and multiplied with the bf16 query as
    # given: query elements over a wide range of magnitudes (far below the
    # head's largest, zeros, negative zeros) must give the oracle's result
    w = W.custom("fp4q", [700, 33, 2048], 64, 8, 128, 32, W.FP4, seed=135)
    kc, vc, ks, vs = W.make_cache(w)
    g = torch.Generator().manual_seed(136)
    q = torch.randn((w.B, w.n_q, 128), generator=g)
    q = q * torch.exp2(torch.randint(-24, 4, (w.B, w.n_q, 128), generator=g).float())
    q[:, :, 5] = 900.0                          # one large element per head
    q[:, 3, :] = 0.0                            # an all-zero head
    q[:, 4, 7] = -0.0
    q = q.to(torch.bfloat16)
    out = pkv.paged_decode_attention(q.to(DEV), kc.to(DEV), vc.to(DEV),
                                     torch.from_numpy(w.block_tables).to(DEV),
                                     torch.from_numpy(w.context_lens).to(DEV), w.scale,
                                     int(w.context_lens.max()), k_scale=ks.to(DEV),
                                     v_scale=vs.to(DEV))
    torch.cuda.synchronize()
    expect = ref.decode_attention(W.bits(q), W.bits(kc), W.bits(vc), w.block_tables,
                                  w.context_lens, w.scale, ref.FP4, ks.numpy(), vs.numpy())
    got = out.cpu().double().numpy()
    assert np.all(np.isfinite(got))
    err = np.max(np.abs(got - expect))
    rel = np.linalg.norm(got - expect) / max(np.linalg.norm(expect), 1e-30)
    assert err <= 3e-2 and rel <= 1e-4, (err, rel)


def test_fp4_byte_movers(pkv):
    w = W.custom("fp4mv", [300, 45], 16, 8, 128, 16, W.FP4, seed=130)
    kc, vc, _, _ = W.make_cache(w)
    kd, vd = kc.to(DEV), vc.to(DEV)
    # gather: raw rows of one sequence
    ko, vo = pkv.gather_kv(kd, vd, torch.from_numpy(w.block_tables[0]).to(DEV), 300)
    torch.cuda.synchronize()
    assert np.array_equal(W.bits(ko), ref.gather(W.bits(kc), w.block_tables[0], 300))
    # copy-on-write copy of two blocks
    pairs = np.array([[int(w.block_tables[0][0]), w.num_blocks - 1],
                      [int(w.block_tables[1][1]), w.num_blocks - 2]], dtype=np.int32)
    pkv.copy_blocks(kd, vd, torch.from_numpy(pairs).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(W.bits(kd), ref.copy_blocks(W.bits(kc), pairs))
    # swap out and back into other blocks
    ids = np.array([int(x) for x in w.block_tables[0][:5]], dtype=np.int32)
    n = pkv.swap_bytes(kd, len(ids))
    staging = torch.empty(n, dtype=torch.uint8, device=DEV)
    host = torch.empty(n, dtype=torch.uint8, pin_memory=True)
    pkv.swap_out(kd, vd, torch.from_numpy(ids).to(DEV), staging, host)
    torch.cuda.synchronize()
    expect = ref.swap_out(W.bits(kd), W.bits(vd), ids)
    assert np.array_equal(host.numpy().reshape(expect.shape), expect)


def close(got, expect, what):
    assert np.all(np.isfinite(got)), what
    err = np.max(np.abs(got - expect)) if got.size else 0.0
    rel = np.linalg.norm(got - expect) / max(np.linalg.norm(expect), 1e-30)
    assert err <= 3e-2 and rel <= 1e-4, (what, err, rel)


MQ_SHAPES = [
    # lengths, query lengths, Q, n_q, n_kv, bs, partition
    ([40, 97, 600], [3, 4, 5], 5, 64, 8, 32, 0),         # 40 rows: register kernel
    ([40, 97, 600], [3, 4, 5], 5, 64, 8, 16, 64),
    ([1, 2, 31, 32, 33], [1, 2, 9, 16, 33], 33, 8, 4, 16, 32),
    ([300, 1025], [40, 200], 200, 16, 2, 32, 0),         # 1600 rows: LDS kernel
    ([300, 1025], [40, 200], 200, 16, 2, 16, 256),
    ([77, 640, 5], [77, 130, 5], 130, 8, 8, 16, 96),     # 130 rows, mid-chunk partitions
    ([300, 1025, 64], [40, 64, 64], 64, 64, 8, 16, 0),   # 512 rows: ping-pong kernel
    ([2050, 99], [64, 31], 64, 64, 8, 32, 160),
]


@pytest.mark.parametrize("case", MQ_SHAPES, ids=[str(i) for i in range(len(MQ_SHAPES))])
def test_fp4_multi_query_shapes(pkv, case):
    lens, qlens, Q, n_q, n_kv, bs, P = case
    w = W.custom("fp4mq", lens, n_q, n_kv, 128, bs, W.FP4, seed=140 + MQ_SHAPES.index(case))
    kc, vc, ks, vs = W.make_cache(w)
    q = W.make_multi_query(w, Q)
    ql = np.asarray(qlens, dtype=np.int32)
    out = pkv.paged_multi_query_attention(
        q.to(DEV), torch.from_numpy(ql).to(DEV), kc.to(DEV), vc.to(DEV),
        torch.from_numpy(w.block_tables).to(DEV), torch.from_numpy(w.context_lens).to(DEV),
        w.scale, int(w.context_lens.max()), k_scale=ks.to(DEV), v_scale=vs.to(DEV),
        partition_size=P)
    torch.cuda.synchronize()
    expect = ref.multi_query_attention(W.bits(q), W.bits(kc), W.bits(vc), w.block_tables,
                                       w.context_lens, ql, w.scale, ref.FP4, ks.numpy(),
                                       vs.numpy())
    got = out.cpu().double().numpy()
    for b, n in enumerate(ql):
        assert not np.any(got[b, n:]), f"rows past query length {n} of seq {b} not zero"
    close(got, expect, str(case))


@pytest.mark.parametrize("rows", [16, 512])
def test_fp4_cascade(pkv, rows):
    # the prefix pass on the register kernel (2 sequences x G 8) or on the LDS
    # kernel (64 x 8 rows)
    B = rows // 8
    suffix = [(37 * i) % 300 + (i % 3 == 0) * 700 for i in range(B)]
    plen, n_q, n_kv, bs = 1024, 64, 8, 16
    w = W.custom("fp4cas", [plen] + suffix, n_q, n_kv, 128, bs, W.FP4, seed=150 + rows)
    kc, vc, ks, vs = W.make_cache(w)
    pt = w.block_tables[0, :plen // bs].copy()
    tables = np.ascontiguousarray(w.block_tables[1:])
    slen = np.array(suffix, dtype=np.int32)
    g = torch.Generator().manual_seed(151 + rows)
    q = torch.randn((B, n_q, 128), generator=g).to(torch.bfloat16)
    out = pkv.cascade_decode_attention(
        q.to(DEV), kc.to(DEV), vc.to(DEV), torch.from_numpy(pt).to(DEV), plen,
        torch.from_numpy(tables).to(DEV), torch.from_numpy(slen).to(DEV), w.scale,
        int(slen.max()), k_scale=ks.to(DEV), v_scale=vs.to(DEV))
    torch.cuda.synchronize()
    expect = ref.cascade_decode_attention(W.bits(q), W.bits(kc), W.bits(vc), pt, plen, tables,
                                          slen, w.scale, ref.FP4, ks.numpy(), vs.numpy())
    close(out.cpu().double().numpy(), expect, f"cascade rows={rows}")

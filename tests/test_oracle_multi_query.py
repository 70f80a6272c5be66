"""Pins of the oracle's multi-token-query attention (CPU only).

- one query per sequence is exactly decode attention (already pinned);
- every row equals decode attention over the sequence cut at that row's
  position (the causal prefix property);
- torch's float64 scaled_dot_product_attention with an explicit boolean mask
  (prefix visible, causal among the new tokens) on dense copies.
"""

import math

import numpy as np
import torch

from oracle import bf16, paged

RNG = np.random.default_rng(21707)


def bf16_bits(x):
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def make(B=3, Q=5, n_q=8, n_kv=2, d=32, bs=8, lens=(9, 40, 5), qlens=(5, 3, 1), extra=3):
    ctx = np.array(lens, dtype=np.int32)
    ql = np.array(qlens, dtype=np.int32)
    nb = [(c + bs - 1) // bs for c in ctx]
    pool = sum(nb) + extra
    perm = RNG.permutation(pool).astype(np.int32)
    bt = np.zeros((B, max(nb)), dtype=np.int32)
    pos = 0
    for b in range(B):
        bt[b, :nb[b]] = perm[pos:pos + nb[b]]
        pos += nb[b]
    kc = bf16_bits(RNG.standard_normal((pool, n_kv, bs, d)))
    vc = bf16_bits(RNG.standard_normal((pool, n_kv, bs, d)))
    q = bf16_bits(RNG.standard_normal((B, Q, n_q, d)))
    return q, kc, vc, bt, ctx, ql


def test_single_query_is_decode_attention():
    q, kc, vc, bt, ctx, _ = make(Q=1, qlens=(1, 1, 1))
    got = paged.multi_query_attention(q, kc, vc, bt, ctx, np.ones(3, np.int32), 0.3)
    want = paged.decode_attention(q[:, 0], kc, vc, bt, ctx, 0.3)
    assert np.array_equal(got[:, 0], want)


def test_each_row_is_decode_attention_on_its_prefix():
    q, kc, vc, bt, ctx, ql = make()
    got = paged.multi_query_attention(q, kc, vc, bt, ctx, ql, 0.25)
    for b in range(3):
        for i in range(int(ql[b])):
            p = int(ctx[b] - ql[b] + i)
            want = paged.decode_attention(q[b:b + 1, i], kc, vc, bt[b:b + 1],
                                          np.array([p + 1]), 0.25)
            np.testing.assert_array_equal(got[b, i], want[0])
        assert np.all(got[b, int(ql[b]):] == 0)


def test_matches_torch_sdpa_with_causal_mask():
    q, kc, vc, bt, ctx, ql = make(lens=(37, 64, 20), qlens=(5, 4, 5), n_q=8, n_kv=4)
    scale = 1 / math.sqrt(32)
    got = paged.multi_query_attention(q, kc, vc, bt, ctx, ql, scale)
    for b in range(3):
        c, n = int(ctx[b]), int(ql[b])
        K = torch.from_numpy(bf16.to_f64(paged.gather(kc, bt[b], c))).permute(1, 0, 2)[None]
        V = torch.from_numpy(bf16.to_f64(paged.gather(vc, bt[b], c))).permute(1, 0, 2)[None]
        Qt = torch.from_numpy(bf16.to_f64(q[b, :n])).permute(1, 0, 2)[None]   # [1, n_q, n, d]
        pos = torch.arange(c - n, c)[:, None]
        mask = torch.arange(c)[None, :] <= pos                                 # [n, c]
        ref = torch.nn.functional.scaled_dot_product_attention(
            Qt, K, V, attn_mask=mask, scale=scale, enable_gqa=True)[0].permute(1, 0, 2)
        np.testing.assert_allclose(got[b, :n], ref.numpy(), rtol=0, atol=1e-12)

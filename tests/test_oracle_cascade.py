"""Pins of the oracle's shared-prefix (cascade) decode attention (CPU only).

The oracle is decode attention on each sequence's concatenated table. It is
pinned by the log-sum-exp identity the GPU path relies on: attention over
prefix ++ suffix equals the fp64 merge of attention over the prefix alone and
over the suffix alone, each weighted by its sum of exponentials; and by the
two degenerate splits (no prefix, no suffix).
"""

import numpy as np
import torch

from oracle import bf16, paged

RNG = np.random.default_rng(21709)


def bits(x):
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def part(q, K, V, scale):
    s = scale * K @ q
    m = s.max()
    w = np.exp(s - m)
    return m, w.sum(), (w @ V) / w.sum()


def setup(B=3, n_q=4, n_kv=2, d=16, bs=4, nb=40, prefix_blocks=3, suffix=(5, 0, 9)):
    k = bits(RNG.standard_normal((nb, n_kv, bs, d)))
    v = bits(RNG.standard_normal((nb, n_kv, bs, d)))
    q = bits(RNG.standard_normal((B, n_q, d)))
    perm = RNG.permutation(nb).astype(np.int32)
    prefix = perm[:prefix_blocks]
    mb = max(1, max(-(-s // bs) for s in suffix))
    tables = np.zeros((B, mb), dtype=np.int32)
    at = prefix_blocks
    for b, s in enumerate(suffix):
        n = -(-s // bs)
        tables[b, :n] = perm[at:at + n]
        at += n
    return q, k, v, prefix, prefix_blocks * bs, tables, np.array(suffix, dtype=np.int32)


def test_prefix_and_suffix_merge_to_the_whole():
    q, k, v, prefix, plen, tables, slen = setup()
    out = paged.cascade_decode_attention(q, k, v, prefix, plen, tables, slen, 0.4)
    qf, kf, vf = bf16.to_f64(q), bf16.to_f64(k), bf16.to_f64(v)
    bs = k.shape[2]
    G = q.shape[1] // k.shape[1]
    for b in range(q.shape[0]):
        kp = paged.gather(kf, prefix, plen)
        vp = paged.gather(vf, prefix, plen)
        ks = paged.gather(kf, tables[b], int(slen[b]))
        vs = paged.gather(vf, tables[b], int(slen[b]))
        for h in range(q.shape[1]):
            g = h // G
            m1, l1, o1 = part(qf[b, h], kp[:, g], vp[:, g], 0.4)
            if slen[b] == 0:
                expect = o1
            else:
                m2, l2, o2 = part(qf[b, h], ks[:, g], vs[:, g], 0.4)
                M = max(m1, m2)
                w1, w2 = l1 * np.exp(m1 - M), l2 * np.exp(m2 - M)
                expect = (w1 * o1 + w2 * o2) / (w1 + w2)
            assert np.allclose(out[b, h], expect, rtol=1e-12, atol=1e-12)


def test_degenerate_splits():
    q, k, v, prefix, plen, tables, slen = setup()
    none = paged.cascade_decode_attention(q, k, v, prefix, 0, tables, slen, 0.4)
    assert np.array_equal(none, paged.decode_attention(q, k, v, tables, slen, 0.4))
    only = paged.cascade_decode_attention(q, k, v, prefix, plen, tables, np.zeros(3, np.int32),
                                          0.4)
    pt = np.tile(prefix, (3, 1)).astype(np.int32)
    assert np.array_equal(only, paged.decode_attention(q, k, v, pt, np.full(3, plen, np.int32),
                                                       0.4))

"""Seeded random sweep of decode and multi-token-query attention against the
float64 oracle, through the C ABI.

Each case draws its geometry (head grouping G from 1 to 64, powers of two
and others, 1 to 8 KV heads,
d_head 64 or 128, 16- or 32-token blocks, bf16 / FP8 / FP4 cache), its batch
(1..8 sequences, lengths 0..1500 with block-boundary and empty ones), its
split-K partition (library default or a random block multiple) and, for the
multi-query half, the query count and per-sequence query lengths; a third
set has contexts to 20,000 tokens and up to 520 queries. Bars as in
the other parity tests: max abs error 1e-2 (bf16) / 3e-2 (FP8, FP4),
relative L2 1e-4, rows past a query length exactly zero.
"""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import paged as ref

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
MAX_ABS = {W.BF16: 1e-2, W.FP8: 3e-2, W.FP4: 3e-2}
REL_L2 = 1e-4


def draw_cases(n, seed, groups=(1, 2, 4, 8, 16, 32, 64)):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        dt = [W.BF16, W.FP8, W.FP4][int(rng.integers(0, 3 if d == 128 else 2))]
        bs = int(rng.choice([16, 32]))
        n_kv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice(groups))
        B = int(rng.integers(1, 9))
        lens = [int(x) for x in rng.integers(1, 1501, size=B)]
        special = [0, 1, bs - 1, bs, bs + 1, 2 * bs]
        for j in range(B):
            if rng.random() < 0.3:
                lens[j] = int(rng.choice(special))
        if max(lens) == 0:
            lens[0] = 1
        P = 0 if rng.random() < 0.4 else bs * int(rng.integers(1, 33))
        Q = int(rng.integers(1, 41))
        qlens = [int(min(Q, L, rng.integers(0, Q + 1))) for L in lens]
        cases.append((i, lens, G * n_kv, n_kv, d, bs, dt, P, Q, qlens))
    return cases


CASES = draw_cases(24, 2170)
# head groups that are not powers of two: partly filled head tiles (decode)
# and row groups that split a query's heads (multi-query)
CASES += [(24 + c[0],) + c[1:] for c in draw_cases(12, 2171, (3, 5, 6, 7, 12, 20, 24, 40))]



def draw_long_cases(n, seed):
    """Longer contexts (to 20,000 tokens) and larger query counts (to 520),
    d 128, so the LDS kernels and their partitions see many chunks."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dt = [W.BF16, W.FP8, W.FP4][i % 3]
        bs = int(rng.choice([16, 32]))
        n_kv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 2, 3, 4, 5, 8, 12, 16, 32, 64]))
        while G * n_kv > 64 and n_kv > 1:
            n_kv //= 2
        B = int(rng.integers(1, 3))
        lens = [int(x) for x in rng.integers(1, 20001, size=B)]
        P = 0 if rng.random() < 0.5 else bs * int(rng.integers(1, 300))
        Q = int(rng.choice([1, 4, 20, 64, 96, 128, 300, 520]))
        qlens = [int(min(Q, L, rng.integers(0, Q + 1))) for L in lens]
        cases.append((i, lens, G * n_kv, n_kv, 128, bs, dt, P, Q, qlens))
    return cases


CASES += [(100 + c[0],) + c[1:] for c in draw_long_cases(12, 2172)]


@pytest.fixture(scope="module")
def pkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_217_amd as m
    return m


def close(out, expect, dt, what):
    got = out.detach().cpu().double().numpy()
    assert got.shape == expect.shape, what
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.max(np.abs(got - expect)) if got.size else 0.0
    rel = np.linalg.norm(got - expect) / max(np.linalg.norm(expect), 1e-30)
    assert err <= MAX_ABS[dt], f"{what}: max abs error {err:.3e}"
    assert rel <= REL_L2, f"{what}: relative L2 {rel:.3e} (max abs {err:.3e})"
    return got


def scales(ks, vs):
    t = lambda x: None if x is None else x.to(DEV)
    return t(ks), t(vs), (None if ks is None else ks.numpy()), (None if vs is None else vs.numpy())


@pytest.mark.parametrize("case", CASES, ids=[str(c[0]) for c in CASES])
def test_sweep_decode(pkv, case):
    i, lens, n_q, n_kv, d, bs, dt, P, _, _ = case
    w = W.custom("sweep", lens, n_q, n_kv, d, bs, dt, seed=300 + i)
    kc, vc, ks, vs = W.make_cache(w)
    q = W.make_query(w)
    ksd, vsd, ksn, vsn = scales(ks, vs)
    out = pkv.paged_decode_attention(q.to(DEV), kc.to(DEV), vc.to(DEV),
                                     torch.from_numpy(w.block_tables).to(DEV),
                                     torch.from_numpy(w.context_lens).to(DEV), w.scale,
                                     int(w.context_lens.max()), k_scale=ksd, v_scale=vsd,
                                     partition_size=P)
    torch.cuda.synchronize()
    expect = ref.decode_attention(W.bits(q), W.bits(kc), W.bits(vc), w.block_tables,
                                  w.context_lens, w.scale, dt, ksn, vsn)
    close(out, expect, dt, str(case))


@pytest.mark.parametrize("case", CASES, ids=[str(c[0]) for c in CASES])
def test_sweep_multi_query(pkv, case):
    i, lens, n_q, n_kv, d, bs, dt, P, Q, qlens = case
    w = W.custom("sweepmq", lens, n_q, n_kv, d, bs, dt, seed=400 + i)
    kc, vc, ks, vs = W.make_cache(w)
    q = W.make_multi_query(w, Q)
    ql = np.asarray(qlens, dtype=np.int32)
    ksd, vsd, ksn, vsn = scales(ks, vs)
    out = pkv.paged_multi_query_attention(
        q.to(DEV), torch.from_numpy(ql).to(DEV), kc.to(DEV), vc.to(DEV),
        torch.from_numpy(w.block_tables).to(DEV), torch.from_numpy(w.context_lens).to(DEV),
        w.scale, int(w.context_lens.max()), k_scale=ksd, v_scale=vsd, partition_size=P)
    torch.cuda.synchronize()
    expect = ref.multi_query_attention(W.bits(q), W.bits(kc), W.bits(vc), w.block_tables,
                                       w.context_lens, ql, w.scale, dt, ksn, vsn)
    got = close(out, expect, dt, str(case))
    for b, n in enumerate(ql):
        assert not np.any(got[b, n:]), f"{case}: rows past query length {n} of seq {b}"

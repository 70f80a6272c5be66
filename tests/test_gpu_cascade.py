"""GPU parity of shared-prefix (cascade) decode attention against the oracle.

Bars as for decode (max abs 1e-2 BF16 / 3e-2 FP8, relative L2 1e-4), and
agreement with plain decode attention over the concatenated tables. Cases
put the prefix rows (sequences x G) on each multi-query kernel (fewer than
128 rows per KV head, 128 or more, and the ping-pong form at 512, bf16 and
FP8), cover MQA, an empty prefix, empty suffixes, ragged suffixes with
NaN-poisoned tails, and explicit partitions; each call is repeated with
the suffixes' longest-first list built by the caller.
"""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import paged as ref

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
MAX_ABS = {W.BF16: 1e-2, W.FP8: 3e-2}


@pytest.fixture(scope="module")
def pkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_217_amd as m
    return m


def shared_prefix_case(suffix, prefix_len, n_q, n_kv, d, bs, dtype, seed):
    """Sequence 0 of the generated structure is the prefix; the rest are suffixes."""
    w = W.custom("cascade", [prefix_len] + list(suffix), n_q, n_kv, d, bs, dtype, seed=seed)
    kc, vc, ks, vs = W.make_cache(w)
    prefix_table = w.block_tables[0, :max(1, prefix_len // bs)].copy()
    tables = np.ascontiguousarray(w.block_tables[1:])
    slen = np.array(suffix, dtype=np.int32)
    B = len(suffix)
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, n_q, d), generator=g).to(torch.bfloat16)
    return w, kc, vc, ks, vs, prefix_table, tables, slen, q


CASES = [
    # suffix lengths, prefix_len, n_q, n_kv, d, bs, dtype, prefix partition, suffix partition
    ([5, 0, 40, 129], 64, 8, 2, 64, 16, W.BF16, 0, 0),           # 16 prefix rows: register kernel
    ([300, 17, 1000], 4096, 64, 8, 128, 16, W.BF16, 0, 0),
    ([1, 50, 260, 33, 7, 900, 64, 12, 300, 5, 120, 77, 1, 2, 3, 400, 18, 19, 20, 21],
     2048, 64, 8, 128, 16, W.BF16, 0, 0),                        # 160 prefix rows: LDS kernel
    ([100, 0, 700], 1024, 64, 8, 128, 32, W.FP8, 256, 64),
    ([33, 1], 512, 64, 1, 128, 16, W.BF16, 128, 0),              # MQA: 128 rows
    ([40, 97], 0, 16, 8, 128, 16, W.BF16, 0, 0),                 # no prefix
    ([0, 0, 0], 1024, 64, 8, 128, 16, W.BF16, 0, 0),             # no suffix
    (list(range(3, 3 + 36 * 29, 29)), 2048, 64, 8, 128, 16, W.BF16, 0, 0),   # 288 rows
    (list(range(2, 2 + 64 * 17, 17)), 3072, 64, 8, 128, 32, W.BF16, 1024, 0),  # 512 rows
    (list(range(1, 1 + 40 * 13, 13)), 1024, 64, 8, 128, 32, W.FP8, 512, 0),  # 320 rows
    (list(range(5, 5 + 64 * 11, 11)), 2048, 64, 8, 128, 16, W.FP8, 0, 0),    # 512 rows
]


@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
def test_cascade_matches_oracle_and_plain_decode(pkv, case):
    suffix, plen, n_q, n_kv, d, bs, dt, Pp, Ps = case
    w, kc, vc, ks, vs, pt, tables, slen, q = shared_prefix_case(
        suffix, plen, n_q, n_kv, d, bs, dt, seed=100 + CASES.index(case))
    t = lambda x: None if x is None else x.to(DEV)
    kd, vd = kc.to(DEV), vc.to(DEV)
    max_s = int(slen.max())
    args = (q.to(DEV), kd, vd, torch.from_numpy(pt).to(DEV), plen,
            torch.from_numpy(tables).to(DEV), torch.from_numpy(slen).to(DEV), w.scale, max_s)
    kw = dict(k_scale=t(ks), v_scale=t(vs), prefix_partition=Pp, suffix_partition=Ps)
    out = pkv.cascade_decode_attention(*args, **kw)
    # the suffixes' longest-first list built by the caller (once per step in
    # a model) instead of by the call: the same work, so the same bits
    sched = pkv.cascade_schedule(kd, args[6], n_q, plen, max_s, Pp, Ps)
    out_sched = pkv.cascade_decode_attention(*args, schedule=sched, **kw)
    # the same attention through plain decode on the concatenated tables
    full = np.concatenate([np.tile(pt[:plen // bs], (len(suffix), 1)), tables], axis=1)
    cl = (plen + slen).astype(np.int32)
    plain = pkv.paged_decode_attention(q.to(DEV), kd, vd, torch.from_numpy(full).to(DEV),
                                       torch.from_numpy(cl).to(DEV), w.scale, int(cl.max()),
                                       k_scale=t(ks), v_scale=t(vs))
    torch.cuda.synchronize()
    expect = ref.cascade_decode_attention(W.bits(q), W.bits(kc), W.bits(vc), pt, plen, tables,
                                          slen, w.scale, dt,
                                          None if ks is None else ks.numpy(),
                                          None if vs is None else vs.numpy())
    assert torch.equal(out, out_sched)
    got = out.cpu().double().numpy()
    assert np.all(np.isfinite(got))
    err = np.max(np.abs(got - expect))
    rel = np.linalg.norm(got - expect) / max(np.linalg.norm(expect), 1e-30)
    assert err <= MAX_ABS[dt], f"max abs error {err:.3e}"
    assert rel <= 1e-4, f"relative L2 {rel:.3e}"
    assert np.max(np.abs(got - plain.cpu().double().numpy())) <= 2 * MAX_ABS[dt] / 10


def test_prefix_cache_feeds_cascade_attention(pkv):
    """Sequences start from a cached system prompt (pkv_bm_match_prefix), add
    their own tokens, and attend through the cascade path; the result equals
    plain decode over the block manager's tables and the oracle."""
    n_kv, n_q, d, bs, nb = 8, 64, 128, 16, 512
    bm = pkv.BlockManager(nb, bs)
    kd = torch.zeros((nb, n_kv, bs, d), dtype=torch.bfloat16, device=DEV)
    vd = torch.zeros_like(kd)
    g = torch.Generator(device="cpu").manual_seed(2175)

    def write(seq, n):
        slots = [bm.append_slot(seq)[0] for _ in range(n)]
        k = torch.randn((n, n_kv, d), generator=g).to(torch.bfloat16).to(DEV)
        v = torch.randn((n, n_kv, d), generator=g).to(torch.bfloat16).to(DEV)
        pkv.kv_append(kd, vd, k, v, torch.tensor(slots, dtype=torch.int64, device=DEV))

    system = [int(x) for x in torch.randint(0, 32000, (1000,), generator=g)]
    assert bm.match_prefix(0, system) == 0
    write(0, len(system))
    bm.cache_prefix(0, system)
    B = 12
    for s in range(1, B + 1):
        assert bm.match_prefix(s, system + [s]) == 992          # 62 whole blocks
        write(s, 8 + 37 * s)                                    # the rest, then private tokens
    seqs = list(range(1, B + 1))
    mb = 96
    full = np.array(bm.export_table(seqs, mb), dtype=np.int32)
    lens = np.array([bm.seq_len(s) for s in seqs], dtype=np.int32)
    pb = 992 // bs
    assert (full[:, :pb] == full[0, :pb]).all()                 # the shared chain
    prefix_table = np.ascontiguousarray(full[0, :pb])
    suffix = np.ascontiguousarray(full[:, pb:])
    slen = (lens - 992).astype(np.int32)
    q = torch.randn((B, n_q, d), generator=g).to(torch.bfloat16).to(DEV)
    out = pkv.cascade_decode_attention(q, kd, vd, torch.from_numpy(prefix_table).to(DEV), 992,
                                       torch.from_numpy(suffix).to(DEV),
                                       torch.from_numpy(slen).to(DEV), 0.0884, int(slen.max()))
    plain = pkv.paged_decode_attention(q, kd, vd, torch.from_numpy(full).to(DEV),
                                       torch.from_numpy(lens).to(DEV), 0.0884, int(lens.max()))
    torch.cuda.synchronize()
    expect = ref.decode_attention(W.bits(q), W.bits(kd), W.bits(vd), full, lens, 0.0884)
    got = out.cpu().double().numpy()
    assert np.max(np.abs(got - expect)) <= 1e-2
    assert np.linalg.norm(got - expect) / np.linalg.norm(expect) <= 1e-4
    assert np.max(np.abs(got - plain.cpu().double().numpy())) <= 2e-3
    bm.close()


def test_bf16_output_is_the_rounded_fp32_output(pkv):
    # the two-source merge writes bf16 from the same fp32 values it would
    # write as fp32
    suffix, plen, n_q, n_kv, d, bs = [30, 0, 700, 129], 2048, 64, 8, 128, 16
    w, kc, vc, ks, vs, pt, tables, slen, q = shared_prefix_case(
        suffix, plen, n_q, n_kv, d, bs, W.BF16, seed=150)
    args = (q.to(DEV), kc.to(DEV), vc.to(DEV), torch.from_numpy(pt).to(DEV), plen,
            torch.from_numpy(tables).to(DEV), torch.from_numpy(slen).to(DEV), w.scale,
            int(slen.max()))
    out32 = pkv.cascade_decode_attention(*args)
    out16 = pkv.cascade_decode_attention(*args, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert out16.dtype == torch.bfloat16
    assert torch.equal(out16, out32.to(torch.bfloat16))


# PKV_BF16_WEIGHTS through the cascade: the prefix pass takes single bf16
# weights where it runs on an LDS kernel (128 or more prefix rows, B x G);
# about 1e-3 relative error, the max abs bars still hold. With fewer rows the
# register kernel runs and the result is the default one bit for bit.
BF16_WEIGHT_CASES = [0, 2, 3, 7, 8, 10]


@pytest.mark.parametrize("ci", BF16_WEIGHT_CASES)
def test_cascade_bf16_weights_option(pkv, ci):
    suffix, plen, n_q, n_kv, d, bs, dt, Pp, Ps = CASES[ci]
    w, kc, vc, ks, vs, pt, tables, slen, q = shared_prefix_case(
        suffix, plen, n_q, n_kv, d, bs, dt, seed=100 + ci)
    t = lambda x: None if x is None else x.to(DEV)
    kd, vd = kc.to(DEV), vc.to(DEV)
    max_s = int(slen.max())
    args = (q.to(DEV), kd, vd, torch.from_numpy(pt).to(DEV), plen,
            torch.from_numpy(tables).to(DEV), torch.from_numpy(slen).to(DEV), w.scale, max_s)
    kw = dict(k_scale=t(ks), v_scale=t(vs), prefix_partition=Pp, suffix_partition=Ps)
    out = pkv.cascade_decode_attention(*args, **kw)
    outw = pkv.cascade_decode_attention(*args, bf16_weights=True, **kw)
    torch.cuda.synchronize()
    rows = len(suffix) * (n_q // n_kv)
    if plen == 0 or -(-rows // 16) < 8:
        assert torch.equal(outw, out)
        return
    expect = ref.cascade_decode_attention(W.bits(q), W.bits(kc), W.bits(vc), pt, plen, tables,
                                          slen, w.scale, dt,
                                          None if ks is None else ks.numpy(),
                                          None if vs is None else vs.numpy())
    got = outw.cpu().double().numpy()
    assert np.all(np.isfinite(got))
    err = np.max(np.abs(got - expect))
    rel = np.linalg.norm(got - expect) / max(np.linalg.norm(expect), 1e-30)
    print(f"[cascade bf16 weights] case {ci} {dt}: max abs {err:.2e}, relative L2 {rel:.2e}",
          flush=True)
    assert err <= MAX_ABS[dt] and rel <= 4e-3, (err, rel)
    assert not torch.equal(outw, out)                       # the option took effect

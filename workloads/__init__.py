"""Seeded synthetic inputs for paged decode attention.

This module only draws random numbers and lays them out: sequence lengths,
block permutations, block tables, bfloat16 / FP8 cache contents, queries and
new-token keys/values. It holds none of the attention arithmetic, and both
the HIP library's tests and the oracle receive the same tensors from it.

Seeds: the structure of workload k = 1..5 (lengths, permutations, prefix
layout) comes from a CPU torch generator seeded 217000 + k, its values from
generators seeded 217100 + k (+50 for queries, +70 for multi-token
queries, +90 for new tokens) on the device where they are created. Test-only shapes use their own small k.

FP8 caches are produced from N(0,1) data with one float32 scale per
(K or V, KV head) equal to absmax / 448; the quotient is clamped to +-448 and
cast with torch's float8_e4m3fn conversion (round to nearest even). FP4
caches hold uniformly random bytes (two E2M1 codes each, every pattern
valid; torch has no FP4 cast) with per-(K or V, KV head) scales U[0.25, 0.5).

Poisoning: with `poison=True`, pool blocks that no table references and the
slots of a sequence's last block past its length hold NaN (bfloat16 0x7FC0,
FP8 0x7F), or for FP4, which has no NaN, the largest magnitude (0x77). Table entries past a sequence's last block point at block 0 and
are never read.
"""

from dataclasses import dataclass, field
from typing import Optional
import math

import numpy as np
import torch

BF16 = "bf16"
FP8 = "fp8_e4m3"
FP4 = "fp4_e2m1"

STRUCT_SEED = 217000
VALUE_SEED = 217100


@dataclass
class Workload:
    name: str
    B: int
    n_q: int
    n_kv: int
    d: int
    bs: int
    kv_dtype: str
    context_lens: np.ndarray          # int32 [B]
    block_tables: np.ndarray          # int32 [B, max_blocks]
    num_blocks: int
    scale: float
    layers: int = 1
    partition_size: int = 0           # 0: the library's default; else fixed by the workload
    shared_prefix_blocks: int = 0
    notes: dict = field(default_factory=dict)
    Q: int = 1                        # query tokens per sequence (1: single-token decode)
    query_lens: Optional[np.ndarray] = None   # int32 [B] when Q > 1

    @property
    def G(self):
        return self.n_q // self.n_kv

    @property
    def max_blocks(self):
        return self.block_tables.shape[1]

    @property
    def p(self):
        return 0.5 if self.kv_dtype == FP4 else 1 if self.kv_dtype == FP8 else 2

    @property
    def total_tokens(self):
        return int(np.sum(self.context_lens.astype(np.int64)))

    def kv_bytes_per_layer(self):
        """Bytes of K and V the attention reads for one layer (logical)."""
        return self.total_tokens * self.n_kv * self.d * self.p * 2


def _gen(seed, device="cpu"):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _tables_from_perm(ctx, bs, perm, max_blocks=None):
    need = [(int(c) + bs - 1) // bs for c in ctx]
    mb = max(need) if max_blocks is None else max_blocks
    mb = max(mb, 1)
    bt = np.zeros((len(ctx), mb), dtype=np.int32)
    pos = 0
    for b, n in enumerate(need):
        bt[b, :n] = perm[pos:pos + n]
        pos += n
    return bt


def make_structure(context_lens, bs, seed, pool_factor=1.2, extra_blocks=0,
                   max_blocks=None):
    """Block tables for the given lengths over a randomly permuted pool.

    The pool holds ceil(pool_factor * need) + extra_blocks blocks; the first
    `need` entries of a seeded permutation of the pool are handed out to the
    sequences' logical blocks in order.
    """
    ctx = np.asarray(context_lens, dtype=np.int32)
    need = int(sum((int(c) + bs - 1) // bs for c in ctx))
    pool = int(math.ceil(pool_factor * need)) + extra_blocks
    pool = max(pool, 1)
    perm = torch.randperm(pool, generator=_gen(seed)).numpy().astype(np.int32)
    return ctx, _tables_from_perm(ctx, bs, perm, max_blocks), pool


def custom(name, context_lens, n_q, n_kv, d, bs, kv_dtype=BF16, seed=0,
           pool_factor=1.2, extra_blocks=0, scale=None, partition_size=0):
    ctx, bt, pool = make_structure(context_lens, bs, STRUCT_SEED + seed,
                                   pool_factor, extra_blocks)
    return Workload(name, len(ctx), n_q, n_kv, d, bs, kv_dtype, ctx, bt, pool,
                    scale if scale is not None else 1.0 / math.sqrt(d),
                    partition_size=partition_size, notes={"seed": seed})


# ---------------------------------------------------------------- the five workloads

def tiny():
    """B=2, lengths {37, 100}, 4 query / 2 KV heads, d=64, bs=16, pool of 32."""
    ctx = np.array([37, 100], dtype=np.int32)
    perm = torch.randperm(32, generator=_gen(STRUCT_SEED + 1)).numpy().astype(np.int32)
    bt = _tables_from_perm(ctx, 16, perm)
    return Workload("tiny_paged_decode", 2, 4, 2, 64, 16, BF16, ctx, bt, 32, 1.0 / 8.0,
                    notes={"seed": 1})


def mha_7b():
    """B=32, lengths uniform in [512, 4096], 32/32 heads, d=128, bs=16, pool 1.2x."""
    g = _gen(STRUCT_SEED + 2)
    ctx = torch.randint(512, 4097, (32,), generator=g).numpy().astype(np.int32)
    need = int(sum((int(c) + 15) // 16 for c in ctx))
    pool = int(math.ceil(1.2 * need))
    perm = torch.randperm(pool, generator=g).numpy().astype(np.int32)
    bt = _tables_from_perm(ctx, 16, perm)
    return Workload("mha_7b_single_layer", 32, 32, 32, 128, 16, BF16, ctx, bt, pool,
                    1.0 / math.sqrt(128), notes={"seed": 2})


def gqa_70b(layers=80):
    """B=64 x 8192 tokens, 64/8 heads, d=128, bs=16; one table, 80 layer pools."""
    ctx = np.full(64, 8192, dtype=np.int32)
    pool = 64 * 512
    perm = torch.randperm(pool, generator=_gen(STRUCT_SEED + 3)).numpy().astype(np.int32)
    bt = _tables_from_perm(ctx, 16, perm)
    return Workload("gqa_70b_80_layers", 64, 64, 8, 128, 16, BF16, ctx, bt, pool,
                    1.0 / math.sqrt(128), layers=layers, notes={"seed": 3})


def gqa_70b_fp4(layers=80):
    """The 70B decode step with an FP4 E2M1 cache: B=64 x 8192 tokens, 64/8
    heads, d=128, bs=32 (2 KiB per (block, head) tile), 80 layer pools."""
    ctx = np.full(64, 8192, dtype=np.int32)
    pool = 64 * 256
    perm = torch.randperm(pool, generator=_gen(STRUCT_SEED + 9)).numpy().astype(np.int32)
    bt = _tables_from_perm(ctx, 32, perm)
    return Workload("gqa_70b_fp4_80_layers", 64, 64, 8, 128, 32, FP4, ctx, bt, pool,
                    1.0 / math.sqrt(128), layers=layers, notes={"seed": 9})


def lognormal_lengths(n, median, sigma, cap, g):
    z = torch.randn(n, generator=g, dtype=torch.float64).numpy()
    ctx = np.rint(np.exp(np.log(median) + sigma * z))
    return np.clip(ctx, 1, cap).astype(np.int32)


def gqa_70b_fp8():
    """B=256, lognormal lengths (median 2048, sigma 1, cap 32768), FP8 KV, bs=32."""
    g = _gen(STRUCT_SEED + 4)
    ctx = lognormal_lengths(256, 2048, 1.0, 32768, g)
    need = int(sum((int(c) + 31) // 32 for c in ctx))
    pool = int(math.ceil(1.2 * need))
    perm = torch.randperm(pool, generator=g).numpy().astype(np.int32)
    bt = _tables_from_perm(ctx, 32, perm)
    return Workload("gqa_70b_fp8_single_layer", 256, 64, 8, 128, 32, FP8, ctx, bt, pool,
                    1.0 / math.sqrt(128), notes={"seed": 4, "lognormal_sigma": 1.0})


def long_shared_prefix():
    """B=16 x 131072 tokens; logical blocks 0..255 shared by all 16 sequences."""
    B, ctx_len, bs, shared = 16, 131072, 16, 256
    per_seq = ctx_len // bs - shared
    pool = shared + B * per_seq
    perm = torch.randperm(pool, generator=_gen(STRUCT_SEED + 5)).numpy().astype(np.int32)
    bt = np.zeros((B, ctx_len // bs), dtype=np.int32)
    bt[:, :shared] = perm[:shared]
    for b in range(B):
        lo = shared + b * per_seq
        bt[b, shared:] = perm[lo:lo + per_seq]
    ctx = np.full(B, ctx_len, dtype=np.int32)
    return Workload("long_context_shared_prefix", B, 64, 8, 128, bs, BF16, ctx, bt, pool,
                    1.0 / math.sqrt(128), partition_size=512, shared_prefix_blocks=shared,
                    notes={"seed": 5, "ref_count": B})


def spec_verify_70b(layers=80):
    """The 70B decode batch verifying 4 draft tokens per sequence: B=64, each
    context 8192 tokens including the 4 candidates, 64/8 heads, d=128, bs=16."""
    ctx = np.full(64, 8192, dtype=np.int32)
    pool = 64 * 512
    perm = torch.randperm(pool, generator=_gen(STRUCT_SEED + 6)).numpy().astype(np.int32)
    bt = _tables_from_perm(ctx, 16, perm)
    return Workload("spec_verify_70b_80_layers", 64, 64, 8, 128, 16, BF16, ctx, bt, pool,
                    1.0 / math.sqrt(128), layers=layers, notes={"seed": 6}, Q=4,
                    query_lens=np.full(64, 4, dtype=np.int32))


def chunked_prefill_70b(layers=4):
    """One 512-token prompt chunk per sequence at four depths of a 64K-token
    prompt (contexts 4096, 16384, 32768, 65536 including the chunk), 64/8
    heads, d=128, bs=16."""
    ctx = np.array([4096, 16384, 32768, 65536], dtype=np.int32)
    need = int(sum(int(c) // 16 for c in ctx))
    perm = torch.randperm(need, generator=_gen(STRUCT_SEED + 7)).numpy().astype(np.int32)
    bt = _tables_from_perm(ctx, 16, perm)
    return Workload("chunked_prefill_70b", 4, 64, 8, 128, 16, BF16, ctx, bt, need,
                    1.0 / math.sqrt(128), layers=layers, notes={"seed": 7}, Q=512,
                    query_lens=np.full(4, 512, dtype=np.int32))


def shared_prompt_70b(layers=8):
    """64 sequences sharing a 16384-token prompt (1024 blocks, the same physical
    blocks in every table) followed by private suffixes of U{256..4096} tokens;
    64/8 heads, d=128, bs=16, bf16."""
    g = _gen(STRUCT_SEED + 8)
    B, bs, prefix = 64, 16, 16384
    suffix = torch.randint(256, 4097, (B,), generator=g).numpy().astype(np.int32)
    pb = prefix // bs
    need = [-(-int(x) // bs) for x in suffix]
    pool = pb + sum(need)
    perm = torch.randperm(pool, generator=g).numpy().astype(np.int32)
    mb = pb + max(need)
    bt = np.zeros((B, mb), dtype=np.int32)
    bt[:, :pb] = perm[:pb]
    at = pb
    for b, n in enumerate(need):
        bt[b, pb:pb + n] = perm[at:at + n]
        at += n
    ctx = (prefix + suffix).astype(np.int32)
    return Workload("shared_prompt_70b", B, 64, 8, 128, bs, BF16, ctx, bt, pool,
                    1.0 / math.sqrt(128), layers=layers, shared_prefix_blocks=pb,
                    notes={"seed": 8, "prefix_len": prefix})


ALL = {"tiny": tiny, "mha_7b": mha_7b, "gqa_70b": gqa_70b, "gqa_70b_fp8": gqa_70b_fp8,
       "long_prefix": long_shared_prefix, "spec_verify_70b": spec_verify_70b,
       "chunked_prefill_70b": chunked_prefill_70b, "shared_prompt_70b": shared_prompt_70b,
       "gqa_70b_fp4": gqa_70b_fp4}


# ---------------------------------------------------------------- values

def _bf16_randn(shape, g, device):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def fp8_from_normal(x):
    """FP8 E4M3FN codes and per-head scales from N(0,1) data [N, n_kv, bs, d]."""
    absmax = x.abs().amax(dim=(0, 2, 3)).float()
    s = absmax / 448.0
    y = (x / s[None, :, None, None]).clamp(-448.0, 448.0)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, s


def fp4_codes(shape, g, device):
    """Uniformly random FP4 E2M1 bytes (two codes each; every pattern is a
    valid pair) and per-head scales, for caches whose last dimension is d / 2."""
    codes = torch.randint(0, 256, shape, generator=g, device=device, dtype=torch.int32)
    scale = 0.25 + torch.rand((shape[1],), generator=g, device=device, dtype=torch.float32) / 4
    return codes.to(torch.uint8), scale


def used_mask(w):
    """bool [num_blocks]: blocks referenced by some sequence's live entries."""
    used = np.zeros(w.num_blocks, dtype=bool)
    for b in range(w.B):
        n = (int(w.context_lens[b]) + w.bs - 1) // w.bs
        used[w.block_tables[b, :n]] = True
    return used


def poison(w, k_cache, v_cache):
    """Set unused blocks and tail slots to NaN in place (bf16 or FP8 patterns)."""
    if w.kv_dtype == FP8:
        kv_k, kv_v, nanval = k_cache, v_cache, 0x7F
    elif w.kv_dtype == FP4:
        # E2M1 has no NaN: the largest magnitude in both nibbles instead
        kv_k, kv_v, nanval = k_cache.view(torch.uint8), v_cache.view(torch.uint8), 0x77
    else:
        kv_k, kv_v, nanval = k_cache.view(torch.int16), v_cache.view(torch.int16), 0x7FC0
    unused = torch.from_numpy(~used_mask(w)).to(k_cache.device)
    kv_k[unused] = nanval
    kv_v[unused] = nanval
    for b in range(w.B):
        c = int(w.context_lens[b])
        if c % w.bs == 0:
            continue
        last = int(w.block_tables[b, (c - 1) // w.bs])
        kv_k[last, :, c % w.bs:, :] = nanval
        kv_v[last, :, c % w.bs:, :] = nanval


def make_cache(w, device="cpu", seed_offset=0, poison_unused=True):
    """Random K/V pools [num_blocks, n_kv, bs, d] (bf16, or uint8 FP8 codes + scales)."""
    g = _gen(VALUE_SEED + w.notes.get("seed", 0) + seed_offset, device)
    shape = (w.num_blocks, w.n_kv, w.bs, w.d)
    if w.kv_dtype == FP4:
        half = shape[:3] + (w.d // 2,)
        k_cache, k_scale = fp4_codes(half, g, device)
        v_cache, v_scale = fp4_codes(half, g, device)
        k_cache = k_cache.view(torch.float4_e2m1fn_x2)
        v_cache = v_cache.view(torch.float4_e2m1fn_x2)
    elif w.kv_dtype == FP8:
        kx = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        k_cache, k_scale = fp8_from_normal(kx)
        del kx
        vx = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        v_cache, v_scale = fp8_from_normal(vx)
        del vx
    else:
        k_cache = _bf16_randn(shape, g, device)
        v_cache = _bf16_randn(shape, g, device)
        k_scale = v_scale = None
    if poison_unused:
        poison(w, k_cache, v_cache)
    return k_cache, v_cache, k_scale, v_scale


def make_query(w, device="cpu", seed_offset=0, layers=1):
    g = _gen(VALUE_SEED + 50 + w.notes.get("seed", 0) + seed_offset, device)
    shape = (w.B, w.n_q, w.d) if layers == 1 else (layers, w.B, w.n_q, w.d)
    return _bf16_randn(shape, g, device)


def make_multi_query(w, Q, device="cpu", seed_offset=0):
    """bf16 [B, Q, n_q, d] queries for several new tokens per sequence."""
    g = _gen(VALUE_SEED + 70 + w.notes.get("seed", 0) + seed_offset, device)
    return _bf16_randn((w.B, Q, w.n_q, w.d), g, device)


def make_new_tokens(w, T=None, device="cpu", seed_offset=0):
    """bf16 [T, n_kv, d] keys and values for kv_append."""
    T = w.B if T is None else T
    g = _gen(VALUE_SEED + 90 + w.notes.get("seed", 0) + seed_offset, device)
    return (_bf16_randn((T, w.n_kv, w.d), g, device),
            _bf16_randn((T, w.n_kv, w.d), g, device))


def bits(t):
    """Raw patterns of a CPU/GPU tensor as numpy (uint16 for bf16, uint8 for FP8)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.uint8:
        return t.numpy()
    if t.dtype in (torch.float8_e4m3fn, torch.float4_e2m1fn_x2):
        return t.view(torch.uint8).numpy()
    raise TypeError(t.dtype)

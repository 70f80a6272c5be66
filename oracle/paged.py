"""Paged KV cache and single-token decode attention, plain float64 (TEST INFRASTRUCTURE, oracle).

What the decode path computes, in the order the pages give it:

  1. Logical -> physical mapping. A sequence's token t lives in physical block
     table[t // bs] at offset t % bs ([LLMI] section "PagedAttention & Memory
     Management (vLLM)", block-table diagram; [MTKV] section "High-Throughput
     Paged Attention Kernel Integration", the per-block table lookup).
  2. Cache layout [num_blocks, n_kv, bs, d] for both K and V ([MTKV], same
     section, the K_Buffer / V_Buffer shape comments).
  3. GQA: query head h reads KV head h // G with G = n_q / n_kv ([MTKV], same
     section, cur_head_kv; [LLMI] section "Attention Architectures: MHA vs.
     MQA vs. GQA").
  4. Attention weights A = softmax(scale * q . k) over the sequence's cached
     tokens ([MTKV] section "Mathematical Formulation of Block Salience", the
     definition of A with scale 1/sqrt(D)); output = sum_t A_t v_t.
  5. Append-then-attend: the new token's K/V is written to the cache first and
     attended to in the same step ([LLMI] section "Why We Need the Key-Value
     (KV) Cache" and flow step 5).
  6. Several new tokens at once (chunked prefill, draft verification): each
     attends causally to the positions up to its own (`multi_query_attention`).

The oracle computes the plain definition (4) with a two-pass softmax in
float64. Online softmax and split-K partitions are exact reformulations; the
oracle states them separately (`split_partials`, `merge_partials`) only so
that partial results can be checked, and pins the merge against (4).

Inputs are raw bit patterns: bfloat16 as uint16, FP8 E4M3FN codes as uint8.
Readings where the pages are silent (each also listed in the design notes):
  * context_len == 0: output is defined as zeros (the printed kernel returns
    without writing).
  * masked positions contribute exactly nothing, even if the slot holds NaN.
  * FP8 dequantisation: value = decode(code) * scale[kv_head], separately for
    K and V, in float64 (exact).
"""

import numpy as np

from . import bf16 as _bf16
from . import fp4_e2m1 as _fp4
from . import fp8_e4m3 as _fp8

BF16 = "bf16"
FP8 = "fp8_e4m3"
FP4 = "fp4_e2m1"


# --------------------------------------------------------------------------
# 1. mapping and gather
# --------------------------------------------------------------------------

def slot_of(block_table_row, pos, block_size):
    """Physical slot of logical position `pos`: block * bs + offset.

    [LLMI] "PagedAttention & Memory Management (vLLM)": the block table maps
    logical block pos // bs to a physical block; the offset inside it is
    pos % bs.
    """
    blk = int(block_table_row[pos // block_size])
    return blk * block_size + pos % block_size


def slot_mapping(block_tables, positions, block_size):
    """int64 slot for each sequence's position (negative position -> -1)."""
    bt = np.asarray(block_tables)
    out = np.empty(len(positions), dtype=np.int64)
    for b, pos in enumerate(positions):
        pos = int(pos)
        out[b] = -1 if pos < 0 else slot_of(bt[b], pos, block_size)
    return out


def gather(cache, block_table_row, context_len):
    """Dense [ctx, n_kv, d] copy of one sequence's cache rows, bit for bit.

    cache: [num_blocks, n_kv, bs, d] of raw patterns. Raises IndexError on a
    block id outside the pool (the oracle refuses what the GPU path must not
    read).
    """
    num_blocks, n_kv, bs, d = cache.shape
    out = np.empty((context_len, n_kv, d), dtype=cache.dtype)
    for i in range((context_len + bs - 1) // bs):
        blk = int(block_table_row[i])
        if not (0 <= blk < num_blocks):
            raise IndexError(f"block id {blk} outside pool of {num_blocks}")
        n = min(bs, context_len - i * bs)       # tokens of this block in use
        # tokens i*bs .. i*bs+n-1 are offsets 0..n-1 of block `blk`
        out[i * bs:i * bs + n] = cache[blk, :, :n, :].transpose(1, 0, 2)
    return out


def dequantize(raw, kv_dtype, scale=None):
    """Raw cache patterns [.., n_kv, d] -> float64 values.

    BF16: exact widening. FP8: decode(code) * scale[kv_head] (scale is a
    per-KV-head float32 array; [SMTS] "Technical Q&A", per-head scaling).
    """
    if kv_dtype == BF16:
        return _bf16.to_f64(raw)
    if kv_dtype == FP8:
        vals = _fp8.decode(raw)
        s = np.asarray(scale, dtype=np.float32).astype(np.float64)
        return vals * s[:, None]
    if kv_dtype == FP4:
        # raw rows are packed bytes [..., d / 2]
        vals = _fp4.decode(_fp4.unpack(raw))
        s = np.asarray(scale, dtype=np.float32).astype(np.float64)
        return vals * s[:, None]
    raise ValueError(kv_dtype)


# --------------------------------------------------------------------------
# 2. attention (the plain definition)
# --------------------------------------------------------------------------

def attention_one(q, k, v, scale):
    """softmax(scale * q . k_t) weighted sum of v_t, two-pass, float64.

    q: [d]; k, v: [ctx, d]. Returns (out [d], weights [ctx]).
    [MTKV] "Mathematical Formulation of Block Salience": A_j is
    exp(q.k_j * scale) / sum_k exp(q.k_k * scale). The maximum is subtracted
    before exponentiating, which leaves A unchanged.
    """
    ctx = k.shape[0]
    if ctx == 0:
        return np.zeros(q.shape[0]), np.zeros(0)
    s = scale * (k @ q)
    m = np.max(s)
    e = np.exp(s - m)
    w = e / np.sum(e)
    return w @ v, w


def decode_attention(q_bits, k_cache, v_cache, block_tables, context_lens, scale,
                     kv_dtype=BF16, k_scale=None, v_scale=None, return_weights=False):
    """Paged single-token decode attention for a batch, float64 output.

    q_bits:        uint16 [B, n_q, d] bfloat16 patterns
    k/v_cache:     [num_blocks, n_kv, bs, d] uint16 (BF16) or uint8 (FP8), or
                   [num_blocks, n_kv, bs, d / 2] packed uint8 (FP4)
    block_tables:  int32 [B, max_blocks]
    context_lens:  int32 [B]
    scale:         softmax scale (float)
    Returns out [B, n_q, d] float64 (and per-(b, h) weight vectors if asked).
    """
    B, n_q, d = q_bits.shape
    n_kv = k_cache.shape[1]
    if n_q % n_kv:
        raise ValueError("n_q must be a multiple of n_kv")
    G = n_q // n_kv
    q = _bf16.to_f64(q_bits)
    out = np.zeros((B, n_q, d))
    weights = {}
    for b in range(B):
        ctx = int(context_lens[b])
        kd = dequantize(gather(k_cache, block_tables[b], ctx), kv_dtype, k_scale)
        vd = dequantize(gather(v_cache, block_tables[b], ctx), kv_dtype, v_scale)
        for h in range(n_q):
            g = h // G
            out[b, h], w = attention_one(q[b, h], kd[:, g, :], vd[:, g, :], scale)
            if return_weights:
                weights[(b, h)] = w
    if return_weights:
        return out, weights
    return out


# --------------------------------------------------------------------------
# 3. split-K partials and their log-sum-exp merge
# --------------------------------------------------------------------------

def split_partials(q, k, v, scale, partition):
    """Per-partition (m, l, o) of one query head over [ctx, d] keys/values.

    Partition j covers tokens [j*P, min((j+1)*P, ctx)). For it:
      m_j = max scale*q.k_t,  l_j = sum exp(scale*q.k_t - m_j),
      o_j = sum exp(scale*q.k_t - m_j) v_t / l_j.
    These are the running statistics of [MTKV] "High-Throughput Paged
    Attention Kernel Integration" (running max, running sum, accumulator,
    final division) evaluated over one partition.
    """
    ctx = k.shape[0]
    n_part = (ctx + partition - 1) // partition
    m = np.full(n_part, -np.inf)
    l = np.zeros(n_part)
    o = np.zeros((n_part, q.shape[0]))
    for j in range(n_part):
        ks = k[j * partition:(j + 1) * partition]
        vs = v[j * partition:(j + 1) * partition]
        s = scale * (ks @ q)
        m[j] = np.max(s)
        e = np.exp(s - m[j])
        l[j] = np.sum(e)
        o[j] = (e @ vs) / l[j]
    return m, l, o


def merge_partials(m, l, o):
    """out = sum_j w_j o_j / sum_j w_j with w_j = l_j exp(m_j - max m).

    Partitions with l_j == 0 (no tokens) carry no weight. With no weight at
    all the output is zeros (the empty-sequence reading).
    """
    m = np.asarray(m, dtype=np.float64)
    l = np.asarray(l, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    live = l > 0
    if not np.any(live):
        return np.zeros(o.shape[-1])
    M = np.max(m[live])
    w = np.where(live, l * np.exp(np.where(live, m, M) - M), 0.0)
    return (w[:, None] * np.where(live[:, None], o, 0.0)).sum(axis=0) / w.sum()


# --------------------------------------------------------------------------
# 4. writes into the cache
# --------------------------------------------------------------------------

def kv_append(k_cache, v_cache, k_new_bits, v_new_bits, slots, kv_dtype=BF16,
              k_scale=None, v_scale=None):
    """Return copies of the caches with token i's K/V stored at slots[i].

    k/v_new_bits: uint16 [T, n_kv, d] bfloat16 patterns. A negative slot is
    skipped. BF16 caches store the pattern unchanged. FP8 caches store
    encode(float32(x) / float32(scale[kv_head])) per element; FP4 caches
    store the same with the E2M1 encoder, two codes per byte.
    [LLMI] flow step 5 and "Why We Need the Key-Value (KV) Cache": the new
    token's key and value are appended to the cache.
    """
    kc = k_cache.copy()
    vc = v_cache.copy()
    num_blocks, n_kv, bs, d = kc.shape
    for i, slot in enumerate(np.asarray(slots, dtype=np.int64)):
        if slot < 0:
            continue
        blk, off = divmod(int(slot), bs)
        if blk >= num_blocks:
            raise IndexError("slot outside pool")
        if kv_dtype == BF16:
            kc[blk, :, off, :] = k_new_bits[i]
            vc[blk, :, off, :] = v_new_bits[i]
        elif kv_dtype == FP4:
            ks = np.asarray(k_scale, dtype=np.float32)
            vs = np.asarray(v_scale, dtype=np.float32)
            kc[blk, :, off, :] = _fp4.pack(
                _fp4.quantize_f32_div(_bf16.to_f32(k_new_bits[i]), ks[:, None]))
            vc[blk, :, off, :] = _fp4.pack(
                _fp4.quantize_f32_div(_bf16.to_f32(v_new_bits[i]), vs[:, None]))
        else:
            ks = np.asarray(k_scale, dtype=np.float32)
            vs = np.asarray(v_scale, dtype=np.float32)
            kc[blk, :, off, :] = _fp8.quantize_f32_div(_bf16.to_f32(k_new_bits[i]), ks[:, None])
            vc[blk, :, off, :] = _fp8.quantize_f32_div(_bf16.to_f32(v_new_bits[i]), vs[:, None])
    return kc, vc


def copy_blocks(cache, pairs):
    """Copy whole physical blocks src -> dst (copy-on-write).

    [SMTS] "Paged KV-Cache with Radix Tree Prefix Cache": sequences that share
    a prefix point at the same blocks through copy-on-write pointers; before a
    shared block is written it is copied to a private block. Every pair reads
    the cache as it was before the call (destinations must be distinct and
    must not be sources).
    """
    out = cache.copy()
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        out[dst] = cache[src]
    return out


# --------------------------------------------------------------------------
# 5. several new query tokens per sequence (chunked prefill, draft verification)
# --------------------------------------------------------------------------

def multi_query_attention(q_bits, k_cache, v_cache, block_tables, context_lens, query_lens,
                          scale, kv_dtype=BF16, k_scale=None, v_scale=None):
    """Causal attention of the last query_lens[b] tokens of each sequence.

    q_bits: uint16 [B, Q, n_q, d] bfloat16 patterns (query i of sequence b is
    row i; rows i >= query_lens[b] are unused and left zero in the output).
    The K/V of the new tokens are already in the cache (append-then-attend), so
    sequence b holds context_lens[b] tokens and its query i sits at position
    p = context_lens[b] - query_lens[b] + i. That query attends to tokens
    0..p: causal self-attention over the new tokens ([LLMI] "4. Internal
    workings", flow step 2) on top of the cached prefix. [LLMI] "9. Failure
    modes and limitations" (chunked prefill) and "7. Practical applications"
    (speculative decoding verifies several draft tokens in one pass) are the
    two uses. Returns float64 [B, Q, n_q, d].
    """
    B, Q, n_q, d = q_bits.shape
    n_kv = k_cache.shape[1]
    G = n_q // n_kv
    q = _bf16.to_f64(q_bits)
    out = np.zeros((B, Q, n_q, d))
    for b in range(B):
        ctx = int(context_lens[b])
        ql = int(query_lens[b])
        if ql > ctx or ql > Q:
            raise ValueError("query_lens must be <= context_lens and <= Q")
        kd = dequantize(gather(k_cache, block_tables[b], ctx), kv_dtype, k_scale)
        vd = dequantize(gather(v_cache, block_tables[b], ctx), kv_dtype, v_scale)
        for i in range(ql):
            p = ctx - ql + i
            for h in range(n_q):
                g = h // G
                out[b, i, h], _ = attention_one(q[b, i, h], kd[:p + 1, g, :], vd[:p + 1, g, :],
                                                scale)
    return out


# ---------------------------------------------------------------------------
# Swap to host memory ([LLMI] "9. Failure modes and limitations": preemption
# evicts a request's KV blocks to host RAM over PCIe; [MTKV] "C++ Block
# Scheduler and Asynchronous Fetch Kernel": demotion of a block to pinned host
# memory and promotion back to HBM are plain asynchronous copies of the
# block's bytes). A swap moves bytes and nothing else, so the oracle is the
# copy written out.

def swap_out(k_cache, v_cache, block_ids):
    """Host image of the listed blocks: raw patterns [2, n, n_kv, bs, d]
    (K blocks, then V blocks, in list order). An id outside the pool gives
    a block of zero bytes."""
    nb = k_cache.shape[0]
    n = len(block_ids)
    out = np.zeros((2, n) + k_cache.shape[1:], dtype=k_cache.dtype)
    for i, blk in enumerate(block_ids):
        if 0 <= blk < nb:
            out[0, i] = k_cache[blk]
            out[1, i] = v_cache[blk]
    return out


def swap_in(k_cache, v_cache, block_ids, host):
    """Caches with the listed blocks overwritten from a host image laid out
    as swap_out() returns it; an id outside the pool is skipped."""
    k = k_cache.copy()
    v = v_cache.copy()
    nb = k.shape[0]
    for i, blk in enumerate(block_ids):
        if 0 <= blk < nb:
            k[blk] = host[0, i]
            v[blk] = host[1, i]
    return k, v


# ---------------------------------------------------------------------------
# A batch sharing a prompt prefix ([SMTS] "Paged KV-Cache with Radix Tree
# Prefix Cache": requests with the same system prompt reference the same
# physical blocks). Attention is defined on each sequence's whole table, the
# shared prefix blocks followed by its own, so the oracle is decode attention
# on the concatenated tables.

def cascade_decode_attention(q_bits, k_cache, v_cache, prefix_table, prefix_len, block_tables,
                             suffix_lens, scale, kv_dtype=BF16, k_scale=None, v_scale=None):
    bs = k_cache.shape[2]
    if prefix_len % bs:
        raise ValueError("prefix_len must be a multiple of the block size")
    pre = np.asarray(prefix_table[:prefix_len // bs], dtype=np.int32)
    B = block_tables.shape[0]
    tables = np.concatenate([np.tile(pre, (B, 1)), block_tables], axis=1).astype(np.int32)
    ctx = (prefix_len + np.asarray(suffix_lens)).astype(np.int32)
    return decode_attention(q_bits, k_cache, v_cache, tables, ctx, scale, kv_dtype, k_scale,
                            v_scale)

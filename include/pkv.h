/*
 * pkv.h -- C ABI of libpkv: single-token decode attention over a paged KV cache
 * on AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages), cited by tag and section:
 *   [SMTS] "Sub-Millisecond Token Scheduling: Inside Disaggregated KV-Cache
 *          Paging for Frontier LLMs" (factnode.online)
 *   [LLMI] "LLM inference: prefill, decode, KV cache" (systemcraft.online, c03)
 *   [MTKV] "Architecting Multi-Tier Disaggregated KV-Cache Hierarchies for
 *          Terabyte-Scale LLM Inference" (ultrainstinct.tech)
 *
 * Conventions shared by every entry point:
 *   - Tensors are caller-owned, contiguous, row-major device memory. The
 *     library never allocates device memory in these calls and never
 *     synchronises: each call enqueues kernels on `stream` (a hipStream_t
 *     passed as void*; NULL means the null stream) and returns.
 *   - Results are status codes; no exception crosses the ABI.
 *     pkv_status_string() gives text. Arguments are validated on the host
 *     before anything is enqueued; an invalid call enqueues nothing.
 *   - Values living in device memory (block ids, slots, lengths, scales) cannot
 *     be validated on the host. The kernels never access memory outside the
 *     caches for an out-of-range block id or slot: a write to one is skipped,
 *     and a read of one reads block 0 instead; results for such inputs are
 *     unspecified.
 *   - Launch errors reported by the HIP runtime are returned as PKV_ERR_HIP.
 *
 * Cache layout ([MTKV] "High-Throughput Paged Attention Kernel Integration",
 * K_Buffer / V_Buffer shape): K and V caches are separate arrays
 * [num_blocks, n_kv, block_size, d_head]; element type bfloat16, or OCP FP8
 * E4M3FN codes (one byte) with one fp32 scale per KV head for K and one for
 * V ([SMTS] "Technical Q&A", per-head scaling factors), or FP4 E2M1 codes
 * (half a byte per element, as [MTKV] "The Anatomy of the KV-Cache Memory
 * Wall" prices 4-bit KV; two codes per byte, element 2i in the low nibble,
 * so a row is d_head / 2 bytes) with the same per-head scales. One (block,
 * head) tile of block_size * d_head elements is contiguous.
 *
 * Supported geometry: block_size in {16, 32}; d_head in {64, 128} (FP4:
 * 128); n_q = G * n_kv for any G >= 1, from MHA (G = 1) to MQA (n_kv = 1).
 * Other block sizes, widths or element types return PKV_ERR_UNSUPPORTED; an
 * n_q that is not a multiple of n_kv returns PKV_ERR_INVALID_ARG.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = 1,
  PKV_ERR_UNSUPPORTED = 2,
  PKV_ERR_OUT_OF_BLOCKS = 3,
  PKV_ERR_WORKSPACE_TOO_SMALL = 4,
  PKV_ERR_HIP = 5
} pkv_status;

typedef enum { PKV_BF16 = 0, PKV_FP8_E4M3 = 1, PKV_FP32 = 2, PKV_FP4_E2M1 = 3 } pkv_dtype;

/* Geometry of one layer's K/V pools (both share it). kv_dtype is a pkv_dtype:
 * PKV_BF16, PKV_FP8_E4M3 or PKV_FP4_E2M1. */
typedef struct {
  int32_t num_blocks;
  int32_t block_size;
  int32_t n_kv;
  int32_t d_head;
  int32_t kv_dtype;
} pkv_cache_desc;

/* Text for a status code (static storage). */
const char* pkv_status_string(pkv_status s);

/* Library version string, e.g. "pkv 0.1 gfx950". */
const char* pkv_version(void);

/* ---------------------------------------------------------------------------
 * Debug mode: checks of the caller errors the interface leaves unspecified
 * because their data lives in device memory. Normal mode never reads device
 * data back and stays memory-safe for any such values, but the results are
 * unspecified.
 *
 * pkv_set_debug(1) turns the mode on for the process (0 turns it off). It
 * allocates one int32 flag on the current device (kept until the process
 * ends) and clears it, and allocates one on each further device at its first
 * debug call. Returns PKV_ERR_HIP, with the mode left off, if that fails.
 *
 * While it is on, each entry point that takes device data and a stream:
 *   1. validates its host arguments as always;
 *   2. synchronises `stream` and reports a flag raised by an earlier call's
 *      checks on this device as PKV_ERR_INVALID_ARG, clearing the flag and
 *      enqueuing nothing;
 *   3. enqueues checks of its own device inputs ahead of its work. The work
 *      still runs, with its normal-mode behaviour.
 * The checks:
 *   - decode, partials, multi-token, shared-prefix and gather calls: every
 *     live table entry (the first cdiv(len, block_size) of a row) names a
 *     block in [0, num_blocks); every length lies in [0, the max length
 *     passed]; every query count lies in [0, min(Q, length)];
 *   - kv_append: every non-negative slot lies in the pool
 *     (< num_blocks * block_size) and appears once;
 *   - copy_blocks: ids in the pool, distinct destinations, no destination
 *     that is also a source.
 * Swap ids outside the pool are not errors (see the swap calls).
 *
 * pkv_debug_check(stream) does step 2 alone: PKV_OK, PKV_ERR_INVALID_ARG (a
 * raised flag, now cleared) or PKV_ERR_HIP. With the mode off it returns
 * PKV_OK at once.
 *
 * The mode synchronises at every call. It is for development, not for timing
 * or HIP graph capture. The switch is process-wide and not thread-safe: set it
 * before other threads call the library.
 * ------------------------------------------------------------------------- */
pkv_status pkv_set_debug(int32_t enable);
pkv_status pkv_debug_check(void* stream);

/* ---------------------------------------------------------------------------
 * Slot mapping ([LLMI] "PagedAttention & Memory Management (vLLM)": logical
 * block pos / block_size of a sequence maps through its block-table row to a
 * physical block; the token sits at offset pos % block_size).
 *
 *   slots_out[b] = block_tables[b * max_blocks_per_seq + positions[b] / bs] * bs
 *                  + positions[b] % bs                       (int64)
 * positions[b] < 0, or positions[b] / bs >= max_blocks_per_seq, gives -1.
 * block_tables: int32 [B, max_blocks_per_seq]; positions: int32 [B];
 * slots_out: int64 [B]. All device pointers. B == 0 is a no-op.
 * ------------------------------------------------------------------------- */
pkv_status pkv_slot_mapping(const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* positions, int32_t B, int32_t block_size,
                            int64_t* slots_out, void* stream);

/* ---------------------------------------------------------------------------
 * kv_append ([LLMI] flow step 5 and "Why We Need the Key-Value (KV) Cache":
 * the new token's key and value are appended to the cache before attention).
 *
 * For each token t < T and head h < n_kv:
 *   k_cache[slot / bs, h, slot % bs, :] = store(k_new[t, h, :], k_scale[h])
 *   (same for V), with slot = slot_mapping[t] (int64, device).
 * store() copies the bfloat16 pattern for a BF16 cache; for an FP8 cache it is
 * E4M3FN(round-to-nearest-even, saturating at +-448)(float32(x) / k_scale[h]),
 * the division in IEEE binary32; NaN stores 0x7F. For an FP4 cache it is
 * E2M1(round-to-nearest-even, saturating at +-6)(float32(x) / k_scale[h])
 * (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; sign kept, -0 included); NaN
 * stores +0.
 * k_new, v_new: bfloat16 [T, n_kv, d_head] (device). k_scale, v_scale: fp32
 * [n_kv] device pointers, required for FP8 and FP4, ignored for BF16.
 * A negative slot is skipped (padding). A slot >= num_blocks * bs is skipped.
 * Two tokens with the same slot: the stored value is unspecified.
 * ------------------------------------------------------------------------- */
pkv_status pkv_kv_append(const pkv_cache_desc* desc, void* k_cache, void* v_cache,
                         const void* k_new, const void* v_new,
                         const int64_t* slot_mapping, int32_t T,
                         const float* k_scale, const float* v_scale, void* stream);

/* ---------------------------------------------------------------------------
 * Paged decode attention ([MTKV] "High-Throughput Paged Attention Kernel
 * Integration": one query token per sequence attends over its cached tokens
 * through the block table; query head h reads KV head h / G; [MTKV]
 * "Mathematical Formulation of Block Salience": weights are
 * softmax(scale * q . k)).
 *
 *   out[b, h, :] = sum_{t < ctx_b} w_t * V_b[t, h / G, :],
 *   w = softmax_t(scale * q[b, h, :] . K_b[t, h / G, :]),
 * with K_b[t, g, :] = k_cache[block_tables[b, t / bs], g, t % bs, :]
 * (decoded and times k_scale[g] for FP8 and FP4; likewise V with v_scale).
 * ctx_b == 0 gives zeros.
 * Slots past ctx_b in a sequence's last block never contribute, whatever they
 * hold (NaN included); table entries past cdiv(ctx_b, bs) are never read.
 *
 * q: bfloat16 [B, n_q, d_head]. out: [B, n_q, d_head] of out_dtype (PKV_FP32
 * or PKV_BF16). block_tables: int32 [B, max_blocks_per_seq].
 * context_lens: int32 [B]. max_context_len: an upper bound of context_lens
 * supplied by the host (no device-to-host read is made); it must satisfy
 * max_context_len <= max_blocks_per_seq * block_size.
 *
 * Split-K: the context is cut into partitions of partition_size tokens (a
 * multiple of block_size; 0 picks a size from the geometry and the GPU). With
 * more than one partition, per-partition statistics go to `workspace` and a
 * log-sum-exp merge (pkv_splitk_reduce) runs after; `workspace_bytes` must be
 * at least pkv_decode_workspace_bytes(...) for the same arguments, else
 * PKV_ERR_WORKSPACE_TOO_SMALL. With one partition the workspace is unused and
 * may be NULL.
 * Accumulation is fp32. Calls that share a workspace must not overlap.
 * ------------------------------------------------------------------------- */
size_t pkv_decode_workspace_bytes(int32_t B, int32_t n_q, int32_t d_head,
                                  int32_t max_context_len, int32_t partition_size);

/* The partition size partition_size == 0 resolves to (a multiple of the block
 * size), for inspection and for sizing the workspace. */
int32_t pkv_default_partition_size(const pkv_cache_desc* desc, int32_t B, int32_t n_q,
                                   int32_t max_context_len);

pkv_status pkv_paged_decode_attention(const pkv_cache_desc* desc, void* out, int32_t out_dtype,
                                      const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* context_lens, int32_t B, int32_t n_q,
                                      int32_t max_context_len, float scale,
                                      const float* k_scale, const float* v_scale,
                                      int32_t partition_size, void* workspace,
                                      size_t workspace_bytes, const void* schedule,
                                      void* stream);

/* ---------------------------------------------------------------------------
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * pkv_paged_decode_attention_static computes exactly what
 * pkv_paged_decode_attention computes, with the same kernels and the same
 * arguments except the workspace: its split-K partials live in a file-scope
 * device array of PKV_STATIC_SCRATCH_BYTES (64 MiB) that every GPU the
 * library runs on holds from the loading of the library's code until the
 * process ends. The call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine); the caller passes inputs and outputs.
 *   - A call whose partials, pkv_decode_workspace_bytes(B, n_q, d_head,
 *     max_context_len, P) for the resolved partition size P, exceed
 *     PKV_STATIC_SCRATCH_BYTES returns PKV_ERR_WORKSPACE_TOO_SMALL and
 *     launches nothing; a single-pass call (one partition) uses none.
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents (each call writes every partial it reads). Calls that
 *     overlap on one GPU (other streams or threads) race on it: serialise them.
 *   - Debug mode does not apply to this entry point (its checks allocate a
 *     flag); the normal-mode memory safety of pkv_paged_decode_attention does.
 *   - Other errors as for pkv_paged_decode_attention; the first call on a
 *     device looks up the array's device address (PKV_ERR_HIP if that fails).
 * ------------------------------------------------------------------------- */
#define PKV_STATIC_SCRATCH_BYTES ((size_t)64 << 20)

pkv_status pkv_paged_decode_attention_static(const pkv_cache_desc* desc, void* out,
                                             int32_t out_dtype, const void* q,
                                             const void* k_cache, const void* v_cache,
                                             const int32_t* block_tables,
                                             int32_t max_blocks_per_seq,
                                             const int32_t* context_lens, int32_t B, int32_t n_q,
                                             int32_t max_context_len, float scale,
                                             const float* k_scale, const float* v_scale,
                                             int32_t partition_size, const void* schedule,
                                             void* stream);

/* ---------------------------------------------------------------------------
 * The two halves of pkv_paged_decode_attention, callable on their own (for
 * timing each kernel and checking partial statistics).
 *
 * pkv_paged_decode_partials writes, for every sequence b, head h and
 * partition j < cdiv(ctx_b, P) (P = the resolved partition size):
 *   m[b, h, j]    = log2(e) * max_{t in j} scale * q . k_t     (fp32)
 *   l[b, h, j]    = sum_{t in j} exp(scale * q . k_t - m / log2(e))
 *   o[b, h, j, :] = sum_{t in j} exp(...) v_t / l[b, h, j]
 * into three arrays carved from `workspace` in that order (m, then l, each
 * fp32 [B, n_q, P_max], then o fp32 [B, n_q, P_max, d_head], with
 * P_max = cdiv(max_context_len, P)). Entries j >= cdiv(ctx_b, P) are not
 * written. pkv_splitk_reduce merges them ([MTKV] kernel's running max / sum /
 * rescaled accumulator, applied across partitions):
 *   M = max_j m_j,  w_j = l_j * 2^(m_j - M),  out = sum_j w_j o_j / sum_j w_j
 * over j < cdiv(ctx_b, partition_size); ctx_b == 0 gives zeros.
 * ------------------------------------------------------------------------- */
pkv_status pkv_paged_decode_partials(const pkv_cache_desc* desc, const void* q,
                                     const void* k_cache, const void* v_cache,
                                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                                     const int32_t* context_lens, int32_t B, int32_t n_q,
                                     int32_t max_context_len, float scale,
                                     const float* k_scale, const float* v_scale,
                                     int32_t partition_size, void* workspace,
                                     size_t workspace_bytes, const void* schedule,
                                     void* stream);

pkv_status pkv_splitk_reduce(void* out, int32_t out_dtype, const float* m, const float* l,
                             const float* o, const int32_t* context_lens, int32_t B,
                             int32_t n_q, int32_t d_head, int32_t max_partitions,
                             int32_t partition_size, void* stream);

/* ---------------------------------------------------------------------------
 * Paged attention for several new query tokens per sequence (chunked
 * prefill, verification of draft tokens): [LLMI] "4. Internal workings"
 * (causal self-attention while a prompt is ingested), "9. Failure modes and
 * limitations" (prompts taken in chunks) and "7. Practical applications"
 * (speculative decoding checks several proposed tokens in one pass); the
 * K/V reads go through the block table exactly as in decode ([MTKV]
 * "High-Throughput Paged Attention Kernel Integration").
 *
 * The new tokens' K/V are already in the cache (append first, as in decode),
 * so sequence b holds ctx_b = context_lens[b] tokens, its last
 * q_b = query_lens[b] of them are the queries, and query i < q_b sits at
 * position p = ctx_b - q_b + i and attends to tokens 0..p:
 *   out[b, i, h, :] = sum_{t <= p} w_t V_b[t, h / G, :],
 *   w = softmax_{t <= p}(scale * q[b, i, h, :] . K_b[t, h / G, :]),
 * K_b/V_b, FP8 scales and G as in pkv_paged_decode_attention. Rows
 * i >= q_b of out are written as zeros.
 *
 * q: bfloat16 [B, Q, n_q, d_head] (query-major within a sequence). out:
 * [B, Q, n_q, d_head] of out_dtype. query_lens: int32 [B] on the device,
 * 0 <= query_lens[b] <= min(Q, ctx_b); a value outside that range is clamped
 * into it. Q >= 1. Every other argument is as for pkv_paged_decode_attention,
 * and Q == 1 with query_lens[b] == 1 computes the same thing as it.
 * Split-K runs as in decode; a query's partitions end at its own position.
 * workspace_bytes must be at least pkv_multi_query_workspace_bytes(...) for
 * the same arguments when more than one partition results (else
 * PKV_ERR_WORKSPACE_TOO_SMALL); with one partition it may be NULL.
 * ------------------------------------------------------------------------- */
size_t pkv_multi_query_workspace_bytes(int32_t B, int32_t Q, int32_t n_q, int32_t d_head,
                                       int32_t max_context_len, int32_t partition_size);

/* The partition size partition_size == 0 resolves to for multi-query calls. */
int32_t pkv_multi_query_partition_size(const pkv_cache_desc* desc, int32_t B, int32_t Q,
                                       int32_t n_q, int32_t max_context_len);

pkv_status pkv_paged_multi_query_attention(const pkv_cache_desc* desc, void* out,
                                           int32_t out_dtype, const void* q, int32_t Q,
                                           const int32_t* query_lens, const void* k_cache,
                                           const void* v_cache, const int32_t* block_tables,
                                           int32_t max_blocks_per_seq,
                                           const int32_t* context_lens, int32_t B, int32_t n_q,
                                           int32_t max_context_len, float scale,
                                           const float* k_scale, const float* v_scale,
                                           int32_t partition_size, void* workspace,
                                           size_t workspace_bytes, void* stream);

/* The same with option flags (pkv_paged_multi_query_attention is this with
 * flags == 0). A flag bit other than these returns PKV_ERR_INVALID_ARG.
 *
 * PKV_BF16_WEIGHTS: the softmax weights may enter the products with V as one
 * bf16 value each instead of a bf16 head and tail (the row sums keep the
 * fp32 weights): a relative error of about 1e-3 instead of about 1e-6, well
 * inside a max abs error of 1e-2 on N(0,1) data, for a third fewer matrix
 * products. The kernels for 128 or more query rows per KV head (Q times
 * n_q / n_kv), which share K/V through LDS, take it (measured 1.2-1.4x
 * faster on prompt chunks); the kernel for fewer rows is bound by memory,
 * keeps the head and tail, and returns the flag-free result.
 */
#define PKV_BF16_WEIGHTS 1

pkv_status pkv_paged_multi_query_attention_ex(const pkv_cache_desc* desc, void* out,
                                              int32_t out_dtype, const void* q, int32_t Q,
                                              const int32_t* query_lens, const void* k_cache,
                                              const void* v_cache, const int32_t* block_tables,
                                              int32_t max_blocks_per_seq,
                                              const int32_t* context_lens, int32_t B,
                                              int32_t n_q, int32_t max_context_len, float scale,
                                              const float* k_scale, const float* v_scale,
                                              int32_t partition_size, void* workspace,
                                              size_t workspace_bytes, int32_t flags,
                                              void* stream);

/* ---------------------------------------------------------------------------
 * Longest-first schedule (optional; a performance aid, not part of the
 * method). Sequences of very different lengths leave a long tail when their
 * partitions run in index order. pkv_decode_schedule writes, into a caller
 * buffer of pkv_decode_schedule_bytes(B, max_context_len, partition_size)
 * bytes (device memory), the list of (sequence, partition) work items in
 * decreasing size: every full partition, then each sequence's last partition
 * bucketed by size. It depends only on context_lens and the partition size,
 * so one schedule serves every layer of a decode step.
 *
 * Passing it as `schedule` to pkv_paged_decode_attention / _partials makes
 * the partition kernel take its work in that order. The call must use the
 * same context_lens contents, B, max_context_len and resolved partition size
 * the schedule was built with; NULL keeps the static grid order.
 * partition_size must be > 0 (resolve 0 with pkv_default_partition_size
 * first). B above 65535 is unsupported.
 * A schedule whose recorded partition size, B or partition count differs from
 * the call's is not followed: the partition kernel computes nothing and the
 * results are unspecified, but nothing outside the call's arrays is read or
 * written; items naming a sequence or partition outside the call are
 * skipped. Debug mode (pkv_set_debug) checks the schedule ahead of the work
 * and reports such a mismatch, an item count other than the call's number of
 * partitions, or an item outside the call, as PKV_ERR_INVALID_ARG.
 * ------------------------------------------------------------------------- */
size_t pkv_decode_schedule_bytes(int32_t B, int32_t max_context_len, int32_t partition_size);

pkv_status pkv_decode_schedule(const int32_t* context_lens, int32_t B, int32_t max_context_len,
                               int32_t partition_size, void* schedule, size_t schedule_bytes,
                               void* stream);

/* ---------------------------------------------------------------------------
 * Copy-on-write block copy ([SMTS] "Paged KV-Cache with Radix Tree Prefix
 * Cache": sequences sharing a prefix point at the same physical blocks through
 * copy-on-write pointers; a shared block is copied before it is written).
 * pairs: int32 [n_pairs, 2] (src, dst) on the device. Every head's tile of
 * block src is copied to block dst in both caches. Destinations must be
 * distinct and must not be sources of the same call. Ids outside the pool are
 * skipped.
 * ------------------------------------------------------------------------- */
pkv_status pkv_copy_blocks(const pkv_cache_desc* desc, void* k_cache, void* v_cache,
                           const int32_t* pairs, int32_t n_pairs, void* stream);

/* ---------------------------------------------------------------------------
 * Gather (test export): dense copies of one sequence's cache rows,
 *   k_out[t, h, :] = k_cache[block_table_row[t / bs], h, t % bs, :]
 * for t < context_len (raw element patterns, no conversion).
 * k_out, v_out: [context_len, n_kv, d_head] of the cache's element type.
 * block_table_row: int32 [>= cdiv(context_len, bs)] on the device.
 * ------------------------------------------------------------------------- */
pkv_status pkv_gather_kv(const pkv_cache_desc* desc, void* k_out, void* v_out,
                         const void* k_cache, const void* v_cache,
                         const int32_t* block_table_row, int32_t context_len, void* stream);

/* ---------------------------------------------------------------------------
 * Decode attention for a batch that shares a prompt prefix ([SMTS] "Paged
 * KV-Cache with Radix Tree Prefix Cache": requests sharing a system prompt,
 * tool definitions or few-shot examples point at the same physical blocks;
 * [LLMI] "7. Practical applications": identical document prefixes shared
 * across requests). Computes exactly pkv_paged_decode_attention for
 * sequences whose tables are prefix_table ++ block_tables[b]:
 *   K_b[t] = prefix block prefix_table[t / bs]            for t < prefix_len,
 *            block block_tables[b][(t - prefix_len) / bs]  otherwise,
 * over ctx_b = prefix_len + suffix_lens[b] tokens, but reads the prefix's
 * K/V once for all B sequences: the sharers' (sequence, head) rows attend to
 * the prefix together on the matrix cores (split over prefix_partition-token
 * partitions), each sequence's own suffix runs through the decode partition
 * kernel (longest partitions first when there are several per sequence), and
 * one log-sum-exp merge combines both.
 *
 * prefix_table: int32 [prefix_len / bs] on the device; prefix_len must be a
 * multiple of the block size (0: no prefix, plain decode). block_tables:
 * int32 [B, max_blocks_per_seq] of suffix blocks; suffix_lens: int32 [B]
 * <= max_suffix_len <= max_blocks_per_seq * bs. Partition sizes are block
 * multiples; 0 picks them. workspace: at least
 * pkv_cascade_workspace_bytes(...) for the same arguments. Other arguments
 * as for pkv_paged_decode_attention.
 *
 * suffix_schedule (optional): when the suffixes take more than one partition
 * the call runs them longest first, from a list it builds in its workspace,
 * or from this one: pkv_decode_schedule(suffix_lens, B, max_suffix_len,
 * pkv_cascade_suffix_partition(...), ...) built once per step, since the list
 * depends only on the suffix lengths, serves every layer (the rules of
 * pkv_paged_decode_attention's schedule apply). Ignored when the suffixes take
 * one partition. pkv_cascade_suffix_partition returns the suffix partition
 * size the call resolves for the same arguments, or 0 when there is no suffix
 * or the arguments are invalid.
 * ------------------------------------------------------------------------- */
size_t pkv_cascade_workspace_bytes(const pkv_cache_desc* desc, int32_t B, int32_t n_q,
                                   int32_t prefix_len, int32_t prefix_partition,
                                   int32_t max_suffix_len, int32_t suffix_partition);

int32_t pkv_cascade_suffix_partition(const pkv_cache_desc* desc, int32_t B, int32_t n_q,
                                     int32_t prefix_len, int32_t prefix_partition,
                                     int32_t max_suffix_len, int32_t suffix_partition);

pkv_status pkv_cascade_decode_attention(
    const pkv_cache_desc* desc, void* out, int32_t out_dtype, const void* q, const void* k_cache,
    const void* v_cache, const int32_t* prefix_table, int32_t prefix_len,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* suffix_lens,
    int32_t B, int32_t n_q, int32_t max_suffix_len, float scale, const float* k_scale,
    const float* v_scale, int32_t prefix_partition, int32_t suffix_partition,
    const void* suffix_schedule, void* workspace, size_t workspace_bytes, void* stream);

/* The same with option flags (pkv_cascade_decode_attention is this with
 * flags == 0); a flag bit other than PKV_BF16_WEIGHTS returns
 * PKV_ERR_INVALID_ARG. PKV_BF16_WEIGHTS applies to the prefix pass, which
 * runs on the multi-token-query kernels, as it does to
 * pkv_paged_multi_query_attention_ex (about 1e-3 relative error on the
 * prefix's share of the output); the suffix pass and the merge are
 * unchanged. */
pkv_status pkv_cascade_decode_attention_ex(
    const pkv_cache_desc* desc, void* out, int32_t out_dtype, const void* q, const void* k_cache,
    const void* v_cache, const int32_t* prefix_table, int32_t prefix_len,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* suffix_lens,
    int32_t B, int32_t n_q, int32_t max_suffix_len, float scale, const float* k_scale,
    const float* v_scale, int32_t prefix_partition, int32_t suffix_partition,
    const void* suffix_schedule, void* workspace, size_t workspace_bytes, int32_t flags,
    void* stream);

/* ---------------------------------------------------------------------------
 * Swap of KV blocks to host memory and back ([LLMI] "9. Failure modes and
 * limitations": under memory pressure a request is preempted by evicting its
 * KV blocks to host RAM over PCIe and restoring them later; [MTKV] "C++ Block
 * Scheduler and Asynchronous Fetch Kernel": demotion to pinned host memory and
 * promotion back to HBM are asynchronous copies on a stream of their own).
 *
 * Host image of n blocks: raw cache bytes [2][n][n_kv][block_size][d_head]
 * (K blocks, then V blocks, in block_ids order), pkv_swap_bytes(desc, n)
 * bytes. pkv_swap_out packs the listed blocks into `staging` (device, at
 * least that size) and copies the image to `host`; pkv_swap_in copies `host`
 * into `staging` and unpacks it into the listed blocks. block_ids: int32 [n]
 * on the device. An id outside the pool packs as zero bytes and is skipped on
 * unpacking. `host` should be pinned (hipHostMalloc) for the copies to be
 * asynchronous; both calls are stream-ordered on `stream` (use a second
 * stream to overlap them with attention), the host image is complete once
 * the stream reaches the end of pkv_swap_out, and `staging` must not be
 * reused before then. Blocks released by pkv_bm_swap_out may be reallocated
 * only by work ordered after the pkv_swap_out that reads them.
 * ------------------------------------------------------------------------- */
size_t pkv_swap_bytes(const pkv_cache_desc* desc, int32_t n_blocks);

pkv_status pkv_swap_out(const pkv_cache_desc* desc, const void* k_cache, const void* v_cache,
                        const int32_t* block_ids, int32_t n_blocks, void* staging, void* host,
                        void* stream);

pkv_status pkv_swap_in(const pkv_cache_desc* desc, void* k_cache, void* v_cache,
                       const int32_t* block_ids, int32_t n_blocks, void* staging,
                       const void* host, void* stream);

/* ---------------------------------------------------------------------------
 * Host block manager ([SMTS] "Paged KV-Cache with Radix Tree Prefix Cache":
 * physical blocks with reference counts, slot allocation popping the free
 * pool, exhaustion asking the scheduler to preempt; copy-on-write sharing).
 * Host memory only, owned by the handle. Not thread-safe.
 *
 * Pool of num_blocks blocks starts as [0, 1, ..., num_blocks-1]; allocation
 * pops the last entry; freed blocks are pushed back in the sequence's logical
 * order. Sequences are named by caller-chosen int64 ids.
 *
 * append_slot(seq): reserves the sequence's next token position (creating the
 * sequence on first use). At a block boundary a fresh block is allocated;
 * otherwise the last block is written, and if it is shared (ref_count > 1) a
 * private block is allocated first and *cow_src / *cow_dst name the copy to
 * make (pkv_copy_blocks) -- else both are -1. *slot receives the token's slot.
 * On exhaustion nothing changes and PKV_ERR_OUT_OF_BLOCKS is returned.
 * fork(parent, child): child shares every block of parent (ref_count + 1).
 * free(seq): ref_count - 1 on each block; blocks reaching 0 return to the pool.
 * export_table: rows of block ids for `seqs`, padded with 0 (never read),
 * into host int32 [B, max_blocks]; a sequence wider than max_blocks is an
 * invalid argument.
 * swap_out(seq): writes the resident sequence's blocks in logical order to
 * blocks_out (the blocks to pass to pkv_swap_out), then releases its
 * references as free() does; shared blocks stay resident for their other
 * sharers. The sequence keeps its length and is marked swapped: it cannot
 * append, fork or be exported until swapped in; free() drops it.
 * swap_in(seq): allocates cdiv(len, block_size) fresh blocks, popped in
 * logical order, makes them the sequence's table and writes them to
 * blocks_out (the blocks to pass to pkv_swap_in); sharing is not restored.
 * Too few free blocks return PKV_ERR_OUT_OF_BLOCKS and change nothing.
 * For both, *n_blocks receives the block count; blocks_out == NULL only
 * queries it; capacity below it is an invalid argument (no change).
 * is_swapped: 1 swapped, 0 resident, -1 unknown sequence.
 *
 * Prefix cache ([LLMI] "8. Design Alternatives": hash prefix caching and an
 * LRU radix tree over paged blocks): a radix tree of full blocks, each keyed
 * under its parent by its block_size token ids (int32, caller's vocabulary).
 * match_prefix(seq, tokens): seq must be new; it starts as the longest chain
 * of cached blocks equal to whole blocks of `tokens`, shared (ref_count + 1)
 * -- *matched_tokens receives their token count; the caller appends the rest.
 * cache_prefix(seq, tokens): registers seq's first n_tokens / block_size
 * blocks (all full, n_tokens <= its length) under that chain; a key already
 * cached by another block ends the registration there (first copy wins).
 * A cached block whose count drops to 0 keeps its contents and key and is
 * evictable; a match revives it. When the free pool is empty, allocation
 * evicts the least recently used evictable block that has no cached
 * children ("use": a match, a registration, or the release to count 0).
 * num_free counts the pool only; num_cached all cached blocks; num_evictable
 * the cached leaves with count 0 now.
 * ------------------------------------------------------------------------- */
typedef struct pkv_bm pkv_bm;

pkv_status pkv_bm_create(int32_t num_blocks, int32_t block_size, pkv_bm** out);
void pkv_bm_destroy(pkv_bm* bm);
pkv_status pkv_bm_append_slot(pkv_bm* bm, int64_t seq, int64_t* slot, int32_t* cow_src,
                              int32_t* cow_dst);
pkv_status pkv_bm_fork(pkv_bm* bm, int64_t parent, int64_t child);
pkv_status pkv_bm_free(pkv_bm* bm, int64_t seq);
pkv_status pkv_bm_export_table(const pkv_bm* bm, const int64_t* seqs, int32_t B,
                               int32_t max_blocks, int32_t* host_table);
/* Token count of a sequence (-1 if unknown), free-pool size, a block's count. */
int64_t pkv_bm_seq_len(const pkv_bm* bm, int64_t seq);
pkv_status pkv_bm_swap_out(pkv_bm* bm, int64_t seq, int32_t* blocks_out, int32_t capacity,
                           int32_t* n_blocks);
pkv_status pkv_bm_swap_in(pkv_bm* bm, int64_t seq, int32_t* blocks_out, int32_t capacity,
                          int32_t* n_blocks);
int32_t pkv_bm_is_swapped(const pkv_bm* bm, int64_t seq);
pkv_status pkv_bm_match_prefix(pkv_bm* bm, int64_t seq, const int32_t* tokens, int64_t n_tokens,
                               int64_t* matched_tokens);
pkv_status pkv_bm_cache_prefix(pkv_bm* bm, int64_t seq, const int32_t* tokens,
                               int64_t n_tokens);
int32_t pkv_bm_num_cached(const pkv_bm* bm);
int32_t pkv_bm_num_evictable(const pkv_bm* bm);
int32_t pkv_bm_num_free(const pkv_bm* bm);
int32_t pkv_bm_ref_count(const pkv_bm* bm, int32_t block);
/* Invariant check of the manager's state, O(blocks + table entries + cache):
 * the free pool holds distinct, unreferenced, uncached blocks of the pool;
 * a block's count equals its number of occurrences in resident sequences;
 * each block is free, referenced, or cached with count 0; a resident
 * sequence holds cdiv(length, block_size) blocks and a swapped one none; the
 * radix cache's keys, parents and child counts agree with its child map; the
 * evictable set is exactly the cached leaves with count 0. PKV_OK, or
 * PKV_ERR_INVALID_ARG if any fails (or bm is NULL). Changes nothing. */
pkv_status pkv_bm_check(const pkv_bm* bm);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */

// Launchers shared between the kernel files and the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv {

// Largest partition count per sequence the split-K reduce accepts (its LDS
// holds one weight per partition).
constexpr int kMaxReducePartitions = 8192;

// Arguments of one decode launch after host-side validation.
struct DecodeArgs {
  const uint16_t* q;          // bf16 [B, n_q, d]
  const uint8_t* k_cache;     // raw bytes [num_blocks, n_kv, bs, d]
  const uint8_t* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const float* k_scale;       // FP8 / FP4 only
  const float* v_scale;
  float* ws_m;                // [B, n_q, P_max] (partials mode)
  float* ws_l;
  float* ws_o;                // [B, n_q, P_max, d]
  void* out;                  // final output (single-partition mode)
  int out_dtype;
  int B, n_q, n_kv, d, bs, num_blocks, max_blocks;
  int kv_dtype;
  int partition;              // tokens per partition (multiple of bs)
  int P_max;                  // partitions launched per sequence
  float scale;
  bool write_partials;        // true: (m, l, o) to workspace; false: out directly
  bool wave_partitions;       // partials mode only: one wave per partition
  const int32_t* schedule;    // optional longest-first work list (see schedule.hip)
  // several query tokens per sequence (multi-query kernel and reduce only):
  // q is [B, Q, n_q, d], out and partial rows are (sequence, query, head)
  int Q;                      // 1 for single-token decode
  const int32_t* query_lens;  // [B]; nullptr for single-token decode
  bool non_causal;            // multi-query only: every row sees the whole context
  int fixed_ctx;              // context length of every sequence when context_lens is null
  bool bf16_weights;          // multi-query only: weights may enter P V as one bf16 value
};

// Schedule buffer: int32 header of kScheduleHeader words, then int2 items.
constexpr int kScheduleHeader = 8;
hipError_t launch_decode_schedule(const int32_t* context_lens, int B, int P, int P_max,
                                  int32_t* sched, hipStream_t stream);

// Partition kernel (matrix cores, decode_mfma.hip).
hipError_t launch_decode_partition(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_partition_mfma(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_splitk_reduce(void* out, int out_dtype, const float* m, const float* l,
                                const float* o, const int32_t* context_lens, int B, int n_q,
                                int d, int P_max, int partition, hipStream_t stream,
                                int Q = 1, const int32_t* query_lens = nullptr,
                                int ctx_cap = INT32_MAX, const float* m2 = nullptr,
                                const float* l2 = nullptr, const float* o2 = nullptr,
                                int P2 = 0);
hipError_t launch_multi_query_partition(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_multi_query_lds(const DecodeArgs& a, hipStream_t stream);

hipError_t launch_slot_mapping(const int32_t* block_tables, int max_blocks,
                               const int32_t* positions, int B, int bs, int64_t* slots,
                               hipStream_t stream);
hipError_t launch_kv_append(const pkv_cache_desc& d, void* k_cache, void* v_cache,
                            const void* k_new, const void* v_new, const int64_t* slots, int T,
                            const float* k_scale, const float* v_scale, hipStream_t stream);
hipError_t launch_copy_blocks(const pkv_cache_desc& d, void* k_cache, void* v_cache,
                              const int32_t* pairs, int n_pairs, hipStream_t stream);
hipError_t launch_gather(const pkv_cache_desc& d, void* k_out, void* v_out, const void* k_cache,
                         const void* v_cache, const int32_t* table, int ctx, hipStream_t stream);

// Swap to host memory: bytes of one block's K (or V) for every head, and the
// pack / unpack kernels around the DMA copy.
int64_t swap_block_bytes(const pkv_cache_desc& d);
hipError_t launch_swap_pack(const pkv_cache_desc& d, const void* k_cache, const void* v_cache,
                            const int32_t* block_ids, int n, void* staging, hipStream_t stream);
hipError_t launch_swap_unpack(const pkv_cache_desc& d, void* k_cache, void* v_cache,
                              const int32_t* block_ids, int n, const void* staging,
                              hipStream_t stream);

// pkv_paged_decode_attention (validation, launches) on `workspace_bytes` of
// workspace: `workspace` itself, or, when `lookup` is given, the address it
// returns, asked for only when a valid call needs partials that fit.
// debug_checks false leaves out the debug-mode checks.
using WorkspaceLookup = pkv_status (*)(void** workspace);
pkv_status decode_attention(const pkv_cache_desc* desc, void* out, int32_t out_dtype,
                            const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, int32_t B, int32_t n_q,
                            int32_t max_context_len, float scale, const float* k_scale,
                            const float* v_scale, int32_t partition_size, void* workspace,
                            size_t workspace_bytes, WorkspaceLookup lookup,
                            const void* schedule, void* stream, bool debug_checks);

// Whether the decode kernels were built for this (d, bs, G, dtype) combination.
bool decode_supported(int d, int bs, int G, int kv_dtype);

}  // namespace pkv

// C ABI of libpkv: host-side validation, workspace carving, launch geometry.
// The operations and their sources are documented in include/pkv.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "pkv.h"
#include "pkv_internal.h"
#include "debug_checks.h"

namespace {

using pkv::kMaxReducePartitions;

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

pkv_status from_hip(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ERR_HIP; }

// ------------------------------------------------------------ debug mode
// Process-wide switch (set before use; not thread-safe). When on, calls that
// take device data first report a caller error raised by an earlier call's
// checks (synchronising the stream to read the flag), then enqueue the checks
// of their own device inputs ahead of the work. One int32 flag per device,
// allocated on first use.
constexpr int kMaxDevices = 64;
bool g_debug = false;
int* g_flag[kMaxDevices] = {};

// The current device's flag (allocated and cleared on first use), or null
// when debug mode is off or the allocation failed.
int* debug_flag() {
  if (!g_debug) return nullptr;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  if (!g_flag[dev]) {
    int* f = nullptr;
    if (hipMalloc(&f, sizeof(int)) != hipSuccess) return nullptr;
    if (hipMemset(f, 0, sizeof(int)) != hipSuccess) return nullptr;
    g_flag[dev] = f;
  }
  return g_flag[dev];
}

// Reports (and clears) a flag raised by earlier checks on this device.
pkv_status debug_take(hipStream_t s) {
  if (!g_debug) return PKV_OK;
  int* f = debug_flag();
  if (!f) return PKV_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return PKV_ERR_HIP;
  int h = 0;
  if (hipMemcpy(&h, f, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess) return PKV_ERR_HIP;
  if (h == 0) return PKV_OK;
  if (hipMemset(f, 0, sizeof(int)) != hipSuccess) return PKV_ERR_HIP;
  return PKV_ERR_INVALID_ARG;
}

// Live block-table entries and lengths of a call (debug mode only).
pkv_status debug_tables(hipStream_t s, const int32_t* tables, int max_blocks,
                        const int32_t* lens, int fixed_len, int max_len, const int32_t* qlens,
                        int Q, int B, const pkv_cache_desc* d) {
  if (!g_debug) return PKV_OK;
  return from_hip(pkv::launch_check_tables(tables, max_blocks, lens, fixed_len, max_len, qlens, Q,
                                           B, d->block_size, d->num_blocks, debug_flag(), s));
}

// The longest-first schedule a call follows, if any (debug mode only).
pkv_status debug_schedule(hipStream_t s, const pkv::DecodeArgs& a) {
  if (!g_debug || a.schedule == nullptr) return PKV_OK;
  return from_hip(pkv::launch_check_schedule(a.schedule, a.context_lens, a.B, a.partition,
                                             a.P_max, debug_flag(), s));
}

pkv_status check_desc(const pkv_cache_desc* d) {
  if (!d || d->num_blocks <= 0 || d->n_kv <= 0) return PKV_ERR_INVALID_ARG;
  if (d->kv_dtype != PKV_BF16 && d->kv_dtype != PKV_FP8_E4M3 && d->kv_dtype != PKV_FP4_E2M1)
    return PKV_ERR_UNSUPPORTED;
  if (d->block_size != 16 && d->block_size != 32) return PKV_ERR_UNSUPPORTED;
  if (d->d_head != 64 && d->d_head != 128) return PKV_ERR_UNSUPPORTED;
  return PKV_OK;
}

// Heads served by one workgroup of the decode kernel for a group of G
// (the matrix-core kernel's head tile is 16 wide).
int head_tile(int G) { return G <= 16 ? G : 16; }

int32_t pick_partition_units(int64_t units, int32_t max_ctx, int64_t row_bytes);

// bytes of K and V of one token of one KV head
int64_t kv_row_bytes(const pkv_cache_desc* d) {
  const int64_t elems = 2 * static_cast<int64_t>(d->d_head);
  return d->kv_dtype == PKV_BF16 ? 2 * elems : d->kv_dtype == PKV_FP4_E2M1 ? elems / 2 : elems;
}

int32_t pick_partition_mq(const pkv_cache_desc* d, int32_t B, int32_t Q, int32_t n_q,
                          int32_t max_ctx);

// More than 16 query heads per KV head: decode runs as a one-token multi-query
// launch (see decode_on_multi_query), and its partition rule applies.
bool decode_on_multi_query(int G) { return G > 16; }

int32_t pick_partition(const pkv_cache_desc* d, int32_t B, int32_t n_q, int32_t max_ctx) {
  const int G = n_q / d->n_kv;
  if (decode_on_multi_query(G)) return pick_partition_mq(d, B, 1, n_q, max_ctx);
  return pick_partition_units(
      static_cast<int64_t>(B) * d->n_kv * ((G + head_tile(G) - 1) / head_tile(G)), max_ctx,
      kv_row_bytes(d));
}

// Workgroups of a multi-query launch per partition: the LDS kernel takes 128
// (query, head) rows of a KV head per workgroup (its ping-pong form 256, at
// one workgroup per CU instead of two: the same share of a round), the
// register kernel 32 (two 16-row tiles) or one tile. A launch that fills a
// round of the chip this way needs no split to fill it. On the register
// kernel it runs in a single pass: splitting would only add partials (fp32,
// d_head + 2 words per row and partition), which outweigh the K/V it reads.
// On the LDS kernels a workgroup's time is its compute, proportional to the
// tokens it attends to, so a batch of different context lengths would end
// with a tail of its longest sequences; partitions of at most kLdsPartition
// tokens, dispatched deepest first, spread that work at a cost in partials
// that is small next to the compute. Measured on a 512-token prompt chunk at
// contexts 4K..64K: 3.33 ms in one pass and 2.98-3.01 ms with partitions of
// 4096-32768 tokens (128-row kernel); with the ping-pong kernel 2.39 ms at
// 8192, 2.43-2.53 ms at 16384, 2.44-2.47 at 24576, 2.49-2.52 at 4096 and
// 2.87-2.95 in one pass (one box). Fewer workgroups split the context as
// decode does.
constexpr int32_t kLdsPartition = 8192;

int32_t pick_partition_mq(const pkv_cache_desc* d, int32_t B, int32_t Q, int32_t n_q,
                          int32_t max_ctx) {
  const int64_t rows = static_cast<int64_t>(Q) * (n_q / d->n_kv);
  const int64_t tiles = cdiv(rows, 16);
  const bool lds = tiles >= 8;
  const int64_t per_head = lds ? cdiv(rows, 128) : (tiles >= 2 ? cdiv(tiles, 2) : 1);
  const int64_t units = static_cast<int64_t>(B) * d->n_kv * per_head;
  if (units >= 512) {
    const int64_t whole = std::max<int64_t>(32, cdiv(max_ctx, 32) * 32);
    return static_cast<int32_t>(lds ? std::min<int64_t>(whole, kLdsPartition) : whole);
  }
  return pick_partition_units(units, max_ctx, kv_row_bytes(d));
}

int32_t pick_partition_units(int64_t units, int32_t max_ctx, int64_t row_bytes) {
  // The partition kernel holds two 4-wave workgroups per CU (its register
  // budget allows two waves per SIMD), so 512 workgroups fill the 256 CUs
  // once. A batch whose (sequence, KV head) pairs alone fill that round and
  // whose longest sequence is at most 8192 tokens runs in a single pass with
  // no reduce. Otherwise a partition holds at most 4 MiB of K+V (8192 tokens
  // of bf16 at d_head 128, 16384 of FP8, 32768 of FP4; at least 4096), which
  // bounds the tail of a launch over sequences of very different lengths,
  // and halves while the grid would not fill one round. Longer partitions
  // carry less per-workgroup overhead: measured on MI355X, 16 x 131072 bf16
  // tokens take 1.33 ms at 4096 and 1.29 ms at 8192, and 256 FP8 sequences
  // of lognormal length 327 us at 4096 and 312 us at 16384 (but 346 us in a
  // single pass, where the longest sequence is the tail).
  constexpr int64_t kOneRound = 256 * 2;
  constexpr int64_t kMaxPartitionBytes = int64_t{4} << 20;
  if (max_ctx <= 8192 && units >= kOneRound) return 8192;
  int64_t P = 4096;
  while (2 * P * row_bytes <= kMaxPartitionBytes) P *= 2;
  while (P > 256 && units * cdiv(max_ctx, P) < kOneRound) P /= 2;
  while (cdiv(max_ctx, P) > kMaxReducePartitions) P *= 2;
  return static_cast<int32_t>(P);
}

// Partials mode runs one wave per partition when partitions are short (each
// wave then keeps a long load pipeline instead of a few chunks).
bool use_wave_partitions(int32_t partition) { return partition <= 1024; }

size_t schedule_bytes(int64_t B, int64_t P_max) {
  return pkv::kScheduleHeader * sizeof(int32_t) + static_cast<size_t>(B * P_max) * 2 * sizeof(int32_t);
}

// A schedule orders the partition kernel's work (see pkv_decode_schedule).
pkv_status attach_schedule(pkv::DecodeArgs* a, const void* schedule) {
  a->schedule = static_cast<const int32_t*>(schedule);
  if (!schedule) return PKV_OK;
  if ((reinterpret_cast<uintptr_t>(schedule) & 7u) != 0) return PKV_ERR_INVALID_ARG;
  const int G = a->n_q / a->n_kv;
  const int64_t grid = static_cast<int64_t>(a->n_kv) * ((G + 15) / 16) * a->B * a->P_max;
  if (grid > 0x7fffffff) return PKV_ERR_UNSUPPORTED;
  return PKV_OK;
}

struct Workspace {
  float* m;
  float* l;
  float* o;
};

size_t workspace_bytes(int64_t B, int64_t n_q, int64_t d, int64_t P_max) {
  const size_t ml = align256(static_cast<size_t>(B * n_q * P_max) * sizeof(float));
  const size_t o = align256(static_cast<size_t>(B * n_q * P_max * d) * sizeof(float));
  return 2 * ml + o;
}

Workspace carve(void* ws, int64_t B, int64_t n_q, int64_t P_max) {
  const size_t ml = align256(static_cast<size_t>(B * n_q * P_max) * sizeof(float));
  char* base = static_cast<char*>(ws);
  return {reinterpret_cast<float*>(base), reinterpret_cast<float*>(base + ml),
          reinterpret_cast<float*>(base + 2 * ml)};
}

// Shared validation of the decode entry points; fills `a` and the resolved
// partition count.
pkv_status prepare_decode(const pkv_cache_desc* desc, const void* q, const void* k_cache,
                          const void* v_cache, const int32_t* block_tables,
                          int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t B,
                          int32_t n_q, int32_t max_context_len, float scale,
                          const float* k_scale, const float* v_scale, int32_t partition_size,
                          pkv::DecodeArgs* a) {
  pkv_status st = check_desc(desc);
  if (st != PKV_OK) return st;
  if (B < 0 || n_q <= 0 || n_q % desc->n_kv != 0) return PKV_ERR_INVALID_ARG;
  if (max_context_len < 0 || max_blocks_per_seq <= 0) return PKV_ERR_INVALID_ARG;
  if (static_cast<int64_t>(max_context_len) >
      static_cast<int64_t>(max_blocks_per_seq) * desc->block_size)
    return PKV_ERR_INVALID_ARG;
  if (partition_size < 0 || (partition_size > 0 && partition_size % desc->block_size != 0))
    return PKV_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return PKV_ERR_INVALID_ARG;
  if (B > 0 && (!q || !k_cache || !v_cache || !block_tables || !context_lens))
    return PKV_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return PKV_ERR_INVALID_ARG;
  if (desc->kv_dtype != PKV_BF16 && (!k_scale || !v_scale)) return PKV_ERR_INVALID_ARG;
  const int G = n_q / desc->n_kv;
  if (!pkv::decode_supported(desc->d_head, desc->block_size, G, desc->kv_dtype))
    return PKV_ERR_UNSUPPORTED;
  if (B > 65535) return PKV_ERR_UNSUPPORTED;

  const int32_t P = partition_size > 0 ? partition_size
                                       : pick_partition(desc, B, n_q, max_context_len);
  const int64_t P_max = std::max<int64_t>(1, cdiv(max_context_len, P));
  if (P_max > kMaxReducePartitions) return PKV_ERR_UNSUPPORTED;

  *a = pkv::DecodeArgs{};
  a->q = static_cast<const uint16_t*>(q);
  a->k_cache = static_cast<const uint8_t*>(k_cache);
  a->v_cache = static_cast<const uint8_t*>(v_cache);
  a->block_tables = block_tables;
  a->context_lens = context_lens;
  a->k_scale = k_scale;
  a->v_scale = v_scale;
  a->B = B;
  a->n_q = n_q;
  a->n_kv = desc->n_kv;
  a->d = desc->d_head;
  a->bs = desc->block_size;
  a->num_blocks = desc->num_blocks;
  a->max_blocks = max_blocks_per_seq;
  a->kv_dtype = desc->kv_dtype;
  a->partition = P;
  a->P_max = static_cast<int>(P_max);
  a->scale = scale;
  return PKV_OK;
}

}  // namespace

namespace pkv {

// The body of pkv_paged_decode_attention, shared with the entry point whose
// partials live in a static device array: there `workspace` is resolved by
// `lookup` only once the arguments are valid and the partials are known to
// fit in `workspace_bytes`. `debug_checks` false skips the debug-mode checks
// (which allocate a device flag on first use).
pkv_status decode_attention(const pkv_cache_desc* desc, void* out, int32_t out_dtype,
                            const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, int32_t B, int32_t n_q,
                            int32_t max_context_len, float scale, const float* k_scale,
                            const float* v_scale, int32_t partition_size, void* workspace,
                            size_t workspace_bytes_, WorkspaceLookup lookup,
                            const void* schedule, void* stream, bool debug_checks) {
  DecodeArgs a;
  pkv_status st = prepare_decode(desc, q, k_cache, v_cache, block_tables, max_blocks_per_seq,
                                 context_lens, B, n_q, max_context_len, scale, k_scale, v_scale,
                                 partition_size, &a);
  if (st != PKV_OK) return st;
  if (out_dtype != PKV_FP32 && out_dtype != PKV_BF16) return PKV_ERR_INVALID_ARG;
  if (B == 0) return PKV_OK;
  if (!out) return PKV_ERR_INVALID_ARG;
  st = attach_schedule(&a, schedule);
  if (st != PKV_OK) return st;
  if (g_debug && debug_checks) {
    st = debug_take(as_stream(stream));
    if (st == PKV_OK)
      st = debug_tables(as_stream(stream), block_tables, max_blocks_per_seq, context_lens, 0,
                        max_context_len, nullptr, 0, B, desc);
    if (st == PKV_OK) st = debug_schedule(as_stream(stream), a);
    if (st != PKV_OK) return st;
  }
  a.out = out;
  a.out_dtype = out_dtype;
  // With more than 16 query heads per KV head the partition kernel would run
  // one workgroup per 16-head tile, each reading the KV head's K/V again. The
  // multi-query kernel with one query per sequence that sees its whole
  // context computes the same attention and applies each K/V chunk to two
  // tiles per wave (a schedule, which only the partition kernel follows,
  // keeps the partition kernel).
  const bool on_mq = decode_on_multi_query(n_q / desc->n_kv) && a.schedule == nullptr;
  if (on_mq) {
    a.Q = 1;
    a.non_causal = true;
  }
  auto launch = [&]() {
    return on_mq ? launch_multi_query_partition(a, as_stream(stream))
                 : launch_decode_partition(a, as_stream(stream));
  };
  if (a.P_max == 1) {
    a.write_partials = false;
    return from_hip(launch());
  }
  const size_t need = workspace_bytes(B, n_q, a.d, a.P_max);
  if (workspace_bytes_ < need) return PKV_ERR_WORKSPACE_TOO_SMALL;
  if (lookup) {
    st = lookup(&workspace);
    if (st != PKV_OK) return st;
  }
  if (!workspace) return PKV_ERR_WORKSPACE_TOO_SMALL;
  if (!aligned16(workspace)) return PKV_ERR_INVALID_ARG;
  const Workspace w = carve(workspace, B, n_q, a.P_max);
  a.ws_m = w.m;
  a.ws_l = w.l;
  a.ws_o = w.o;
  a.write_partials = true;
  a.wave_partitions = !on_mq && a.schedule == nullptr && use_wave_partitions(a.partition);
  hipError_t e = launch();
  if (e != hipSuccess) return PKV_ERR_HIP;
  return from_hip(launch_splitk_reduce(out, out_dtype, w.m, w.l, w.o, context_lens, B, n_q, a.d,
                                       a.P_max, a.partition, as_stream(stream)));
}

}  // namespace pkv

extern "C" {

const char* pkv_status_string(pkv_status s) {
  switch (s) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID_ARG: return "invalid argument";
    case PKV_ERR_UNSUPPORTED: return "unsupported geometry or dtype";
    case PKV_ERR_OUT_OF_BLOCKS: return "KV block pool exhausted (preempt a sequence)";
    case PKV_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case PKV_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* pkv_version(void) { return "pkv 0.1 gfx950"; }

pkv_status pkv_set_debug(int32_t enable) {
  g_debug = enable != 0;
  if (!g_debug) return PKV_OK;
  int* f = debug_flag();
  // a fresh start on this device: nothing pending from an earlier session
  if (!f || hipMemset(f, 0, sizeof(int)) != hipSuccess) {
    g_debug = false;
    return PKV_ERR_HIP;
  }
  return PKV_OK;
}

pkv_status pkv_debug_check(void* stream) { return debug_take(as_stream(stream)); }

pkv_status pkv_slot_mapping(const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* positions, int32_t B, int32_t block_size,
                            int64_t* slots_out, void* stream) {
  if (B < 0 || max_blocks_per_seq <= 0 || block_size <= 0) return PKV_ERR_INVALID_ARG;
  if (B == 0) return PKV_OK;
  if (!block_tables || !positions || !slots_out) return PKV_ERR_INVALID_ARG;
  const pkv_status pend = debug_take(as_stream(stream));
  if (pend != PKV_OK) return pend;
  return from_hip(pkv::launch_slot_mapping(block_tables, max_blocks_per_seq, positions, B,
                                           block_size, slots_out, as_stream(stream)));
}

pkv_status pkv_kv_append(const pkv_cache_desc* desc, void* k_cache, void* v_cache,
                         const void* k_new, const void* v_new, const int64_t* slot_mapping,
                         int32_t T, const float* k_scale, const float* v_scale, void* stream) {
  pkv_status st = check_desc(desc);
  if (st != PKV_OK) return st;
  if (T < 0) return PKV_ERR_INVALID_ARG;
  if (T == 0) return PKV_OK;
  if (!k_cache || !v_cache || !k_new || !v_new || !slot_mapping) return PKV_ERR_INVALID_ARG;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new))
    return PKV_ERR_INVALID_ARG;
  if (desc->kv_dtype != PKV_BF16 && (!k_scale || !v_scale)) return PKV_ERR_INVALID_ARG;
  if (g_debug) {
    st = debug_take(as_stream(stream));
    if (st != PKV_OK) return st;
    st = from_hip(pkv::launch_check_slots(
        slot_mapping, T, static_cast<int64_t>(desc->num_blocks) * desc->block_size, debug_flag(),
        as_stream(stream)));
    if (st != PKV_OK) return st;
  }
  return from_hip(pkv::launch_kv_append(*desc, k_cache, v_cache, k_new, v_new, slot_mapping, T,
                                        k_scale, v_scale, as_stream(stream)));
}

size_t pkv_decode_workspace_bytes(int32_t B, int32_t n_q, int32_t d_head,
                                  int32_t max_context_len, int32_t partition_size) {
  if (B <= 0 || n_q <= 0 || d_head <= 0 || max_context_len < 0 || partition_size <= 0) return 0;
  const int64_t P_max = std::max<int64_t>(1, cdiv(max_context_len, partition_size));
  return workspace_bytes(B, n_q, d_head, P_max);
}

int32_t pkv_default_partition_size(const pkv_cache_desc* desc, int32_t B, int32_t n_q,
                                   int32_t max_context_len) {
  if (check_desc(desc) != PKV_OK || B < 0 || n_q <= 0 || n_q % desc->n_kv != 0 ||
      max_context_len < 0)
    return 0;
  return pick_partition(desc, B, n_q, max_context_len);
}

pkv_status pkv_paged_decode_attention(const pkv_cache_desc* desc, void* out, int32_t out_dtype,
                                      const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* context_lens, int32_t B, int32_t n_q,
                                      int32_t max_context_len, float scale,
                                      const float* k_scale, const float* v_scale,
                                      int32_t partition_size, void* workspace,
                                      size_t workspace_bytes_, const void* schedule,
                                      void* stream) {
  return pkv::decode_attention(desc, out, out_dtype, q, k_cache, v_cache, block_tables,
                               max_blocks_per_seq, context_lens, B, n_q, max_context_len, scale,
                               k_scale, v_scale, partition_size, workspace, workspace_bytes_,
                               nullptr, schedule, stream, true);
}

pkv_status pkv_paged_decode_partials(const pkv_cache_desc* desc, const void* q,
                                     const void* k_cache, const void* v_cache,
                                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                                     const int32_t* context_lens, int32_t B, int32_t n_q,
                                     int32_t max_context_len, float scale,
                                     const float* k_scale, const float* v_scale,
                                     int32_t partition_size, void* workspace,
                                     size_t workspace_bytes_, const void* schedule,
                                     void* stream) {
  pkv::DecodeArgs a;
  pkv_status st = prepare_decode(desc, q, k_cache, v_cache, block_tables, max_blocks_per_seq,
                                 context_lens, B, n_q, max_context_len, scale, k_scale, v_scale,
                                 partition_size, &a);
  if (st != PKV_OK) return st;
  if (B == 0) return PKV_OK;
  st = attach_schedule(&a, schedule);
  if (st != PKV_OK) return st;
  const size_t need = workspace_bytes(B, n_q, a.d, a.P_max);
  if (!workspace || workspace_bytes_ < need) return PKV_ERR_WORKSPACE_TOO_SMALL;
  if (!aligned16(workspace)) return PKV_ERR_INVALID_ARG;
  const Workspace w = carve(workspace, B, n_q, a.P_max);
  a.ws_m = w.m;
  a.ws_l = w.l;
  a.ws_o = w.o;
  a.write_partials = true;
  a.wave_partitions = a.schedule == nullptr && use_wave_partitions(a.partition);
  if (g_debug) {
    st = debug_take(as_stream(stream));
    if (st == PKV_OK)
      st = debug_tables(as_stream(stream), block_tables, max_blocks_per_seq, context_lens, 0,
                        max_context_len, nullptr, 0, B, desc);
    if (st == PKV_OK) st = debug_schedule(as_stream(stream), a);
    if (st != PKV_OK) return st;
  }
  return from_hip(pkv::launch_decode_partition(a, as_stream(stream)));
}

pkv_status pkv_splitk_reduce(void* out, int32_t out_dtype, const float* m, const float* l,
                             const float* o, const int32_t* context_lens, int32_t B,
                             int32_t n_q, int32_t d_head, int32_t max_partitions,
                             int32_t partition_size, void* stream) {
  if (B < 0 || n_q <= 0 || d_head <= 0 || max_partitions <= 0 || partition_size <= 0)
    return PKV_ERR_INVALID_ARG;
  if (out_dtype != PKV_FP32 && out_dtype != PKV_BF16) return PKV_ERR_INVALID_ARG;
  if (max_partitions > kMaxReducePartitions) return PKV_ERR_UNSUPPORTED;
  if (B == 0) return PKV_OK;
  if (!out || !m || !l || !o || !context_lens) return PKV_ERR_INVALID_ARG;
  const pkv_status pend = debug_take(as_stream(stream));
  if (pend != PKV_OK) return pend;
  return from_hip(pkv::launch_splitk_reduce(out, out_dtype, m, l, o, context_lens, B, n_q,
                                            d_head, max_partitions, partition_size,
                                            as_stream(stream)));
}

size_t pkv_multi_query_workspace_bytes(int32_t B, int32_t Q, int32_t n_q, int32_t d_head,
                                       int32_t max_context_len, int32_t partition_size) {
  if (B <= 0 || Q <= 0 || n_q <= 0 || d_head <= 0 || max_context_len < 0 ||
      partition_size <= 0)
    return 0;
  const int64_t P_max = std::max<int64_t>(1, cdiv(max_context_len, partition_size));
  return workspace_bytes(static_cast<int64_t>(B) * Q, n_q, d_head, P_max);
}

int32_t pkv_multi_query_partition_size(const pkv_cache_desc* desc, int32_t B, int32_t Q,
                                       int32_t n_q, int32_t max_context_len) {
  if (check_desc(desc) != PKV_OK || B < 0 || Q <= 0 || n_q <= 0 || n_q % desc->n_kv != 0 ||
      max_context_len < 0)
    return 0;
  return pick_partition_mq(desc, B, Q, n_q, max_context_len);
}

pkv_status pkv_paged_multi_query_attention(const pkv_cache_desc* desc, void* out,
                                           int32_t out_dtype, const void* q, int32_t Q,
                                           const int32_t* query_lens, const void* k_cache,
                                           const void* v_cache, const int32_t* block_tables,
                                           int32_t max_blocks_per_seq,
                                           const int32_t* context_lens, int32_t B, int32_t n_q,
                                           int32_t max_context_len, float scale,
                                           const float* k_scale, const float* v_scale,
                                           int32_t partition_size, void* workspace,
                                           size_t workspace_bytes_, void* stream) {
  return pkv_paged_multi_query_attention_ex(desc, out, out_dtype, q, Q, query_lens, k_cache,
                                            v_cache, block_tables, max_blocks_per_seq,
                                            context_lens, B, n_q, max_context_len, scale,
                                            k_scale, v_scale, partition_size, workspace,
                                            workspace_bytes_, 0, stream);
}

pkv_status pkv_paged_multi_query_attention_ex(const pkv_cache_desc* desc, void* out,
                                              int32_t out_dtype, const void* q, int32_t Q,
                                              const int32_t* query_lens, const void* k_cache,
                                              const void* v_cache, const int32_t* block_tables,
                                              int32_t max_blocks_per_seq,
                                              const int32_t* context_lens, int32_t B,
                                              int32_t n_q, int32_t max_context_len, float scale,
                                              const float* k_scale, const float* v_scale,
                                              int32_t partition_size, void* workspace,
                                              size_t workspace_bytes_, int32_t flags,
                                              void* stream) {
  if (Q <= 0 || (flags & ~PKV_BF16_WEIGHTS) != 0) return PKV_ERR_INVALID_ARG;
  if (desc && check_desc(desc) == PKV_OK && n_q > 0 && n_q % desc->n_kv == 0 &&
      partition_size == 0 && B >= 0 && max_context_len >= 0)
    partition_size = pick_partition_mq(desc, B, Q, n_q, max_context_len);
  pkv::DecodeArgs a;
  pkv_status st = prepare_decode(desc, q, k_cache, v_cache, block_tables, max_blocks_per_seq,
                                 context_lens, B, n_q, max_context_len, scale, k_scale, v_scale,
                                 partition_size, &a);
  if (st != PKV_OK) return st;
  if (out_dtype != PKV_FP32 && out_dtype != PKV_BF16) return PKV_ERR_INVALID_ARG;
  if (B == 0) return PKV_OK;
  if (!out || !query_lens) return PKV_ERR_INVALID_ARG;
  const int64_t rows = static_cast<int64_t>(Q) * (n_q / desc->n_kv);
  if (static_cast<int64_t>(desc->n_kv) * cdiv(rows, 16) > 0x7fffffff / 256)
    return PKV_ERR_UNSUPPORTED;
  a.Q = Q;
  a.query_lens = query_lens;
  a.out = out;
  a.out_dtype = out_dtype;
  a.bf16_weights = (flags & PKV_BF16_WEIGHTS) != 0;
  const hipStream_t s = as_stream(stream);
  if (g_debug) {
    st = debug_take(s);
    if (st == PKV_OK)
      st = debug_tables(s, block_tables, max_blocks_per_seq, context_lens, 0, max_context_len,
                        query_lens, Q, B, desc);
    if (st != PKV_OK) return st;
  }
  if (a.P_max == 1) {
    a.write_partials = false;
    return from_hip(pkv::launch_multi_query_partition(a, s));
  }
  const int64_t BQ = static_cast<int64_t>(B) * Q;
  const size_t need = workspace_bytes(BQ, n_q, a.d, a.P_max);
  if (!workspace || workspace_bytes_ < need) return PKV_ERR_WORKSPACE_TOO_SMALL;
  if (!aligned16(workspace)) return PKV_ERR_INVALID_ARG;
  const Workspace w = carve(workspace, BQ, n_q, a.P_max);
  a.ws_m = w.m;
  a.ws_l = w.l;
  a.ws_o = w.o;
  a.write_partials = true;
  hipError_t e = pkv::launch_multi_query_partition(a, s);
  if (e != hipSuccess) return PKV_ERR_HIP;
  return from_hip(pkv::launch_splitk_reduce(out, out_dtype, w.m, w.l, w.o, context_lens, B, n_q,
                                            a.d, a.P_max, a.partition, s, Q, query_lens,
                                            max_blocks_per_seq * desc->block_size));
}

// ---------------------------------------------------------------- cascade

namespace {

struct CascadePlan {
  int32_t Pp, Pp_max;      // prefix partition size and count (0, 0: no prefix)
  int32_t Ps, Ps_max;      // suffix partition size and count (0, 0: no suffix)
  size_t suffix_bytes, prefix_bytes;
  size_t schedule_bytes;   // longest-first list of the suffix partitions (0: none)
};

pkv_status plan_cascade(const pkv_cache_desc* desc, int32_t B, int32_t n_q, int32_t prefix_len,
                        int32_t prefix_partition, int32_t max_suffix_len,
                        int32_t suffix_partition, CascadePlan* pl) {
  pkv_status st = check_desc(desc);
  if (st != PKV_OK) return st;
  if (B < 0 || n_q <= 0 || n_q % desc->n_kv != 0 || prefix_len < 0 || max_suffix_len < 0 ||
      prefix_partition < 0 || suffix_partition < 0)
    return PKV_ERR_INVALID_ARG;
  if (prefix_len % desc->block_size != 0) return PKV_ERR_INVALID_ARG;
  if ((prefix_partition % desc->block_size) != 0 || (suffix_partition % desc->block_size) != 0)
    return PKV_ERR_INVALID_ARG;
  *pl = CascadePlan{};
  if (prefix_len > 0) {
    // the sharers' (sequence, head) rows are the query rows of one prefix pass
    pl->Pp = prefix_partition > 0 ? prefix_partition
                                  : pick_partition_mq(desc, 1, B, n_q, prefix_len);
    if (pl->Pp >= prefix_len) pl->Pp = prefix_len;
    pl->Pp_max = static_cast<int32_t>(cdiv(prefix_len, pl->Pp));
    pl->prefix_bytes = workspace_bytes(B, n_q, desc->d_head, pl->Pp_max);
  }
  if (max_suffix_len > 0) {
    // Suffixes are ragged: the default splits them into at most 2048-token
    // partitions that run longest first (measured on a 64-sequence batch
    // with 304..3978-token suffixes: 187 us per layer against 203 us for
    // one pass over the whole suffixes).
    pl->Ps = suffix_partition;
    if (pl->Ps == 0) {
      pl->Ps = std::min(pick_partition(desc, B, n_q, max_suffix_len), 2048);
      while (pl->Pp_max + cdiv(max_suffix_len, pl->Ps) > kMaxReducePartitions) pl->Ps *= 2;
    }
    pl->Ps_max = static_cast<int32_t>(cdiv(max_suffix_len, pl->Ps));
    pl->suffix_bytes = workspace_bytes(B, n_q, desc->d_head, pl->Ps_max);
    // suffixes are ragged: with several partitions, the longest go first
    if (pl->Ps_max > 1) pl->schedule_bytes = align256(schedule_bytes(B, pl->Ps_max));
  }
  if (static_cast<int64_t>(pl->Pp_max) + pl->Ps_max > kMaxReducePartitions)
    return PKV_ERR_UNSUPPORTED;
  return PKV_OK;
}

}  // namespace

size_t pkv_cascade_workspace_bytes(const pkv_cache_desc* desc, int32_t B, int32_t n_q,
                                   int32_t prefix_len, int32_t prefix_partition,
                                   int32_t max_suffix_len, int32_t suffix_partition) {
  CascadePlan pl;
  if (plan_cascade(desc, B, n_q, prefix_len, prefix_partition, max_suffix_len,
                   suffix_partition, &pl) != PKV_OK)
    return 0;
  return pl.prefix_bytes + pl.suffix_bytes + pl.schedule_bytes;
}

int32_t pkv_cascade_suffix_partition(const pkv_cache_desc* desc, int32_t B, int32_t n_q,
                                     int32_t prefix_len, int32_t prefix_partition,
                                     int32_t max_suffix_len, int32_t suffix_partition) {
  CascadePlan pl;
  if (plan_cascade(desc, B, n_q, prefix_len, prefix_partition, max_suffix_len,
                   suffix_partition, &pl) != PKV_OK)
    return 0;
  return pl.Ps;
}

pkv_status pkv_cascade_decode_attention(
    const pkv_cache_desc* desc, void* out, int32_t out_dtype, const void* q, const void* k_cache,
    const void* v_cache, const int32_t* prefix_table, int32_t prefix_len,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* suffix_lens,
    int32_t B, int32_t n_q, int32_t max_suffix_len, float scale, const float* k_scale,
    const float* v_scale, int32_t prefix_partition, int32_t suffix_partition,
    const void* suffix_schedule, void* workspace, size_t workspace_bytes_, void* stream) {
  return pkv_cascade_decode_attention_ex(desc, out, out_dtype, q, k_cache, v_cache, prefix_table,
                                         prefix_len, block_tables, max_blocks_per_seq,
                                         suffix_lens, B, n_q, max_suffix_len, scale, k_scale,
                                         v_scale, prefix_partition, suffix_partition,
                                         suffix_schedule, workspace, workspace_bytes_, 0, stream);
}

pkv_status pkv_cascade_decode_attention_ex(
    const pkv_cache_desc* desc, void* out, int32_t out_dtype, const void* q, const void* k_cache,
    const void* v_cache, const int32_t* prefix_table, int32_t prefix_len,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* suffix_lens,
    int32_t B, int32_t n_q, int32_t max_suffix_len, float scale, const float* k_scale,
    const float* v_scale, int32_t prefix_partition, int32_t suffix_partition,
    const void* suffix_schedule, void* workspace, size_t workspace_bytes_, int32_t flags,
    void* stream) {
  if ((flags & ~PKV_BF16_WEIGHTS) != 0) return PKV_ERR_INVALID_ARG;
  CascadePlan pl;
  pkv_status st = plan_cascade(desc, B, n_q, prefix_len, prefix_partition, max_suffix_len,
                               suffix_partition, &pl);
  if (st != PKV_OK) return st;
  if (out_dtype != PKV_FP32 && out_dtype != PKV_BF16) return PKV_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return PKV_ERR_INVALID_ARG;
  if (B == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !suffix_lens || !block_tables)
    return PKV_ERR_INVALID_ARG;
  if (prefix_len > 0 && !prefix_table) return PKV_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return PKV_ERR_INVALID_ARG;
  if (desc->kv_dtype != PKV_BF16 && (!k_scale || !v_scale)) return PKV_ERR_INVALID_ARG;
  if (!pkv::decode_supported(desc->d_head, desc->block_size, n_q / desc->n_kv, desc->kv_dtype))
    return PKV_ERR_UNSUPPORTED;
  if (B > 65535 || max_blocks_per_seq <= 0) return PKV_ERR_INVALID_ARG;
  if (static_cast<int64_t>(max_suffix_len) >
      static_cast<int64_t>(max_blocks_per_seq) * desc->block_size)
    return PKV_ERR_INVALID_ARG;
  const size_t need = pl.prefix_bytes + pl.suffix_bytes + pl.schedule_bytes;
  if (need > 0 && (!workspace || workspace_bytes_ < need)) return PKV_ERR_WORKSPACE_TOO_SMALL;
  if (need > 0 && !aligned16(workspace)) return PKV_ERR_INVALID_ARG;
  const hipStream_t s = as_stream(stream);
  char* ws = static_cast<char*>(workspace);
  if (g_debug) {
    st = debug_take(s);
    if (st == PKV_OK && prefix_len > 0)
      st = debug_tables(s, prefix_table, prefix_len / desc->block_size, nullptr, prefix_len,
                        prefix_len, nullptr, 0, 1, desc);
    if (st == PKV_OK)
      st = debug_tables(s, block_tables, max_blocks_per_seq, suffix_lens, 0, max_suffix_len,
                        nullptr, 0, B, desc);
    if (st != PKV_OK) return st;
  }

  Workspace wp{}, wsuf{};
  if (pl.Pp_max > 0) {
    // prefix pass: one virtual sequence whose B query tokens are the sharers,
    // every row seeing the whole prefix
    wp = carve(ws, B, n_q, pl.Pp_max);
    pkv::DecodeArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.k_cache = static_cast<const uint8_t*>(k_cache);
    a.v_cache = static_cast<const uint8_t*>(v_cache);
    a.block_tables = prefix_table;
    a.context_lens = nullptr;
    a.fixed_ctx = prefix_len;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.B = 1;
    a.Q = B;
    a.non_causal = true;
    a.bf16_weights = (flags & PKV_BF16_WEIGHTS) != 0;
    a.n_q = n_q;
    a.n_kv = desc->n_kv;
    a.d = desc->d_head;
    a.bs = desc->block_size;
    a.num_blocks = desc->num_blocks;
    a.max_blocks = prefix_len / desc->block_size;
    a.kv_dtype = desc->kv_dtype;
    a.partition = pl.Pp;
    a.P_max = pl.Pp_max;
    a.scale = scale;
    a.write_partials = true;
    a.ws_m = wp.m;
    a.ws_l = wp.l;
    a.ws_o = wp.o;
    hipError_t e = pkv::launch_multi_query_partition(a, s);
    if (e != hipSuccess) return PKV_ERR_HIP;
  }
  if (pl.Ps_max > 0) {
    wsuf = carve(ws + pl.prefix_bytes, B, n_q, pl.Ps_max);
    pkv::DecodeArgs a;
    st = prepare_decode(desc, q, k_cache, v_cache, block_tables, max_blocks_per_seq, suffix_lens,
                        B, n_q, max_suffix_len, scale, k_scale, v_scale, pl.Ps, &a);
    if (st != PKV_OK) return st;
    a.ws_m = wsuf.m;
    a.ws_l = wsuf.l;
    a.ws_o = wsuf.o;
    a.write_partials = true;
    if (pl.schedule_bytes > 0) {
      // the caller's longest-first list, or one built here
      const void* sched = suffix_schedule;
      if (!sched) {
        int32_t* own = reinterpret_cast<int32_t*>(ws + pl.prefix_bytes + pl.suffix_bytes);
        hipError_t e = pkv::launch_decode_schedule(suffix_lens, B, pl.Ps, pl.Ps_max, own, s);
        if (e != hipSuccess) return PKV_ERR_HIP;
        sched = own;
      }
      st = attach_schedule(&a, sched);
      if (st == PKV_OK && g_debug && suffix_schedule) st = debug_schedule(s, a);
      if (st != PKV_OK) return st;
    }
    a.wave_partitions = a.schedule == nullptr && use_wave_partitions(a.partition);
    hipError_t e = pkv::launch_decode_partition(a, s);
    if (e != hipSuccess) return PKV_ERR_HIP;
  } else {
    wsuf = wp;                       // no suffix partitions: never read (np = 0)
  }
  return from_hip(pkv::launch_splitk_reduce(
      out, out_dtype, wsuf.m, wsuf.l, wsuf.o, suffix_lens, B, n_q, desc->d_head,
      pl.Ps_max > 0 ? pl.Ps_max : 1, pl.Ps > 0 ? pl.Ps : 1, s, 1, nullptr,
      max_blocks_per_seq * desc->block_size, pl.Pp_max > 0 ? wp.m : nullptr, wp.l, wp.o,
      pl.Pp_max));
}

size_t pkv_swap_bytes(const pkv_cache_desc* desc, int32_t n_blocks) {
  if (check_desc(desc) != PKV_OK || n_blocks < 0) return 0;
  return static_cast<size_t>(2 * static_cast<int64_t>(n_blocks) * pkv::swap_block_bytes(*desc));
}

static pkv_status check_swap(const pkv_cache_desc* desc, const void* k_cache, const void* v_cache,
                             const int32_t* block_ids, int32_t n_blocks, const void* staging,
                             const void* host) {
  pkv_status st = check_desc(desc);
  if (st != PKV_OK) return st;
  if (n_blocks < 0) return PKV_ERR_INVALID_ARG;
  if (n_blocks == 0) return PKV_OK;
  if (!k_cache || !v_cache || !block_ids || !staging || !host) return PKV_ERR_INVALID_ARG;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(staging))
    return PKV_ERR_INVALID_ARG;
  if (static_cast<int64_t>(n_blocks) * pkv::swap_block_bytes(*desc) / 16384 > 0x3fffffff)
    return PKV_ERR_UNSUPPORTED;
  return PKV_OK;
}

pkv_status pkv_swap_out(const pkv_cache_desc* desc, const void* k_cache, const void* v_cache,
                        const int32_t* block_ids, int32_t n_blocks, void* staging, void* host,
                        void* stream) {
  pkv_status st = check_swap(desc, k_cache, v_cache, block_ids, n_blocks, staging, host);
  if (st != PKV_OK || n_blocks == 0) return st;
  const hipStream_t s = as_stream(stream);
  st = debug_take(s);
  if (st != PKV_OK) return st;
  hipError_t e = pkv::launch_swap_pack(*desc, k_cache, v_cache, block_ids, n_blocks, staging, s);
  if (e != hipSuccess) return PKV_ERR_HIP;
  return from_hip(hipMemcpyAsync(host, staging, pkv_swap_bytes(desc, n_blocks),
                                 hipMemcpyDeviceToHost, s));
}

pkv_status pkv_swap_in(const pkv_cache_desc* desc, void* k_cache, void* v_cache,
                       const int32_t* block_ids, int32_t n_blocks, void* staging,
                       const void* host, void* stream) {
  pkv_status st = check_swap(desc, k_cache, v_cache, block_ids, n_blocks, staging, host);
  if (st != PKV_OK || n_blocks == 0) return st;
  const hipStream_t s = as_stream(stream);
  st = debug_take(s);
  if (st != PKV_OK) return st;
  hipError_t e = hipMemcpyAsync(staging, host, pkv_swap_bytes(desc, n_blocks),
                                hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return PKV_ERR_HIP;
  return from_hip(
      pkv::launch_swap_unpack(*desc, k_cache, v_cache, block_ids, n_blocks, staging, s));
}

size_t pkv_decode_schedule_bytes(int32_t B, int32_t max_context_len, int32_t partition_size) {
  if (B <= 0 || max_context_len < 0 || partition_size <= 0) return 0;
  const int64_t P_max = std::max<int64_t>(1, cdiv(max_context_len, partition_size));
  return schedule_bytes(B, P_max);
}

pkv_status pkv_decode_schedule(const int32_t* context_lens, int32_t B, int32_t max_context_len,
                               int32_t partition_size, void* schedule, size_t schedule_bytes_,
                               void* stream) {
  if (B < 0 || max_context_len < 0 || partition_size <= 0) return PKV_ERR_INVALID_ARG;
  if (B == 0) return PKV_OK;
  if (B > 65535) return PKV_ERR_UNSUPPORTED;
  if (!context_lens || !schedule) return PKV_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(schedule) & 7u) != 0) return PKV_ERR_INVALID_ARG;
  const int64_t P_max = std::max<int64_t>(1, cdiv(max_context_len, partition_size));
  if (P_max > kMaxReducePartitions) return PKV_ERR_UNSUPPORTED;
  if (schedule_bytes_ < schedule_bytes(B, P_max)) return PKV_ERR_WORKSPACE_TOO_SMALL;
  const pkv_status pend = debug_take(as_stream(stream));
  if (pend != PKV_OK) return pend;
  return from_hip(pkv::launch_decode_schedule(context_lens, B, partition_size,
                                              static_cast<int>(P_max),
                                              static_cast<int32_t*>(schedule), as_stream(stream)));
}

pkv_status pkv_copy_blocks(const pkv_cache_desc* desc, void* k_cache, void* v_cache,
                           const int32_t* pairs, int32_t n_pairs, void* stream) {
  pkv_status st = check_desc(desc);
  if (st != PKV_OK) return st;
  if (n_pairs < 0) return PKV_ERR_INVALID_ARG;
  if (n_pairs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !pairs) return PKV_ERR_INVALID_ARG;
  if (!aligned16(k_cache) || !aligned16(v_cache)) return PKV_ERR_INVALID_ARG;
  if (g_debug) {
    st = debug_take(as_stream(stream));
    if (st == PKV_OK)
      st = from_hip(pkv::launch_check_pairs(pairs, n_pairs, desc->num_blocks, debug_flag(),
                                            as_stream(stream)));
    if (st != PKV_OK) return st;
  }
  return from_hip(pkv::launch_copy_blocks(*desc, k_cache, v_cache, pairs, n_pairs,
                                          as_stream(stream)));
}

pkv_status pkv_gather_kv(const pkv_cache_desc* desc, void* k_out, void* v_out,
                         const void* k_cache, const void* v_cache,
                         const int32_t* block_table_row, int32_t context_len, void* stream) {
  pkv_status st = check_desc(desc);
  if (st != PKV_OK) return st;
  if (context_len < 0) return PKV_ERR_INVALID_ARG;
  if (context_len == 0) return PKV_OK;
  if (!k_out || !v_out || !k_cache || !v_cache || !block_table_row) return PKV_ERR_INVALID_ARG;
  if (!aligned16(k_out) || !aligned16(v_out) || !aligned16(k_cache) || !aligned16(v_cache))
    return PKV_ERR_INVALID_ARG;
  if (g_debug) {
    st = debug_take(as_stream(stream));
    if (st == PKV_OK)
      st = debug_tables(as_stream(stream), block_table_row,
                        static_cast<int>(cdiv(context_len, desc->block_size)), nullptr,
                        context_len, context_len, nullptr, 0, 1, desc);
    if (st != PKV_OK) return st;
  }
  return from_hip(pkv::launch_gather(*desc, k_out, v_out, k_cache, v_cache, block_table_row,
                                     context_len, as_stream(stream)));
}

}  // extern "C"

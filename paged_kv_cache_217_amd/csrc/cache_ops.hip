// Cache-maintenance kernels: slot mapping, kv_append, copy-on-write block
// copy and the gather used by tests. All are launch- or copy-bound; they move
// whole 16-byte chunks per lane where the layout allows it.
//
// Sources: [LLMI] "LLM inference: prefill, decode, KV cache" (systemcraft.online),
// sections "PagedAttention & Memory Management (vLLM)" (block table, slots) and
// "Why We Need the Key-Value (KV) Cache" (append before attending);
// [SMTS] "Sub-Millisecond Token Scheduling: Inside Disaggregated KV-Cache
// Paging for Frontier LLMs" (factnode.online), sections "Paged KV-Cache with
// Radix Tree Prefix Cache" (copy-on-write) and "Technical Q&A" (FP8 E4M3 with
// per-head scales).
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

// slot = table[b][pos / bs] * bs + pos % bs, int64; -1 for pos < 0 or beyond the row.
__global__ void slot_mapping_kernel(const int32_t* __restrict__ block_tables, int max_blocks,
                                    const int32_t* __restrict__ positions, int B, int bs,
                                    int64_t* __restrict__ slots) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int pos = positions[b];
  int64_t slot = -1;
  if (pos >= 0 && pos / bs < max_blocks) {
    const int64_t blk = block_tables[static_cast<int64_t>(b) * max_blocks + pos / bs];
    slot = blk * bs + pos % bs;
  }
  slots[b] = slot;
}

// One thread per 8 elements of one (token, head) row. FMT: 0 bf16 copy,
// 1 FP8 E4M3 store, 2 FP4 E2M1 store (two codes per byte, low nibble first).
template <int FMT>
__global__ void kv_append_kernel(uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
                                 const uint16_t* __restrict__ k_new,
                                 const uint16_t* __restrict__ v_new,
                                 const int64_t* __restrict__ slots, int T, int n_kv, int d,
                                 int bs, int num_blocks, const float* __restrict__ k_scale,
                                 const float* __restrict__ v_scale) {
  const int chunks = d / 8;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = static_cast<int64_t>(T) * n_kv * chunks;
  if (idx >= total) return;
  const int c = static_cast<int>(idx % chunks);
  const int h = static_cast<int>((idx / chunks) % n_kv);
  const int t = static_cast<int>(idx / (static_cast<int64_t>(chunks) * n_kv));
  const int64_t slot = slots[t];
  if (slot < 0) return;
  const int64_t blk = slot / bs;
  const int off = static_cast<int>(slot % bs);
  if (blk >= num_blocks) return;
  const int64_t src = (static_cast<int64_t>(t) * n_kv + h) * d + c * 8;
  const int64_t dst = ((blk * n_kv + h) * bs + off) * d + c * 8;  // element index
  const uint4 kw = *reinterpret_cast<const uint4*>(k_new + src);
  const uint4 vw = *reinterpret_cast<const uint4*>(v_new + src);
  if constexpr (FMT == 2) {
    const float ks = k_scale[h];
    const float vs = v_scale[h];
    const uint32_t kin[4] = {kw.x, kw.y, kw.z, kw.w};
    const uint32_t vin[4] = {vw.x, vw.y, vw.z, vw.w};
    uint32_t kout = 0, vout = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float k0, k1, v0, v1;
      bf16x2_to_f32(kin[i], k0, k1);
      bf16x2_to_f32(vin[i], v0, v1);
      // IEEE binary32 division, then the saturating encode; element 2i low nibble
      kout |= (f32_to_fp4_e2m1_sat(k0 / ks) | (f32_to_fp4_e2m1_sat(k1 / ks) << 4)) << (8 * i);
      vout |= (f32_to_fp4_e2m1_sat(v0 / vs) | (f32_to_fp4_e2m1_sat(v1 / vs) << 4)) << (8 * i);
    }
    *reinterpret_cast<uint32_t*>(k_cache + dst / 2) = kout;
    *reinterpret_cast<uint32_t*>(v_cache + dst / 2) = vout;
  } else if constexpr (FMT == 0) {
    *reinterpret_cast<uint4*>(k_cache + dst * 2) = kw;
    *reinterpret_cast<uint4*>(v_cache + dst * 2) = vw;
  } else {
    const float ks = k_scale[h];
    const float vs = v_scale[h];
    const uint32_t kin[4] = {kw.x, kw.y, kw.z, kw.w};
    const uint32_t vin[4] = {vw.x, vw.y, vw.z, vw.w};
    uint32_t kout[2] = {0, 0}, vout[2] = {0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float k0, k1, v0, v1;
      bf16x2_to_f32(kin[i], k0, k1);
      bf16x2_to_f32(vin[i], v0, v1);
      // IEEE binary32 division (correctly rounded), then the saturating encode
      const uint32_t kc = f32_to_fp8_e4m3_sat(k0 / ks) | (f32_to_fp8_e4m3_sat(k1 / ks) << 8);
      const uint32_t vc = f32_to_fp8_e4m3_sat(v0 / vs) | (f32_to_fp8_e4m3_sat(v1 / vs) << 8);
      kout[i / 2] |= kc << (16 * (i % 2));
      vout[i / 2] |= vc << (16 * (i % 2));
    }
    *reinterpret_cast<uint2*>(k_cache + dst) = make_uint2(kout[0], kout[1]);
    *reinterpret_cast<uint2*>(v_cache + dst) = make_uint2(vout[0], vout[1]);
  }
}

// bytes of one element row of d_head elements
static int row_bytes_of(const pkv_cache_desc& d) {
  return d.kv_dtype == PKV_FP4_E2M1 ? d.d_head / 2
                                    : d.d_head * (d.kv_dtype == PKV_FP8_E4M3 ? 1 : 2);
}

// Block (src -> dst) copy of every head's tile; grid (pairs, 2 caches).
__global__ void copy_blocks_kernel(uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
                                   const int32_t* __restrict__ pairs, int64_t block_bytes,
                                   int num_blocks) {
  const int p = blockIdx.x;
  const int src = pairs[2 * p];
  const int dst = pairs[2 * p + 1];
  if (src < 0 || dst < 0 || src >= num_blocks || dst >= num_blocks) return;
  uint8_t* cache = blockIdx.y == 0 ? k_cache : v_cache;
  const uint4* s = reinterpret_cast<const uint4*>(cache + src * block_bytes);
  uint4* d = reinterpret_cast<uint4*>(cache + dst * block_bytes);
  const int64_t n = block_bytes / 16;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) d[i] = s[i];
}

// Dense copy of one sequence: out[t, h, :] = cache[table[t / bs], h, t % bs, :].
__global__ void gather_kernel(uint8_t* __restrict__ k_out, uint8_t* __restrict__ v_out,
                              const uint8_t* __restrict__ k_cache,
                              const uint8_t* __restrict__ v_cache,
                              const int32_t* __restrict__ table, int ctx, int n_kv,
                              int row_bytes, int bs, int num_blocks) {
  const int chunks = row_bytes / 16;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = static_cast<int64_t>(ctx) * n_kv * chunks;
  if (idx >= total) return;
  const int c = static_cast<int>(idx % chunks);
  const int h = static_cast<int>((idx / chunks) % n_kv);
  const int t = static_cast<int>(idx / (static_cast<int64_t>(chunks) * n_kv));
  int blk = table[t / bs];
  if (blk < 0 || blk >= num_blocks) blk = 0;
  const int64_t src = ((static_cast<int64_t>(blk) * n_kv + h) * bs + t % bs) * row_bytes + c * 16;
  const int64_t dst = (static_cast<int64_t>(t) * n_kv + h) * row_bytes + c * 16;
  *reinterpret_cast<uint4*>(k_out + dst) = *reinterpret_cast<const uint4*>(k_cache + src);
  *reinterpret_cast<uint4*>(v_out + dst) = *reinterpret_cast<const uint4*>(v_cache + src);
}

// Swap to host: the listed blocks (every head's tile, K then V) are packed
// into a contiguous device staging image before one DMA copy to host memory,
// and unpacked from it after the copy back ([MTKV] "C++ Block Scheduler and
// Asynchronous Fetch Kernel" copies block by block; one batched copy keeps the
// DMA engine at the link's rate). grid: (n blocks x slices of 16 KiB, K/V).
constexpr int kSwapSlice = 16384;
typedef uint32_t swap_u32x4 __attribute__((ext_vector_type(4)));

template <bool PACK>
__global__ __launch_bounds__(256) void swap_blocks_kernel(
    uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
    const int32_t* __restrict__ block_ids, int n_blocks, int64_t block_bytes, int num_blocks,
    uint8_t* __restrict__ staging) {
  const int slices = static_cast<int>((block_bytes + kSwapSlice - 1) / kSwapSlice);
  const int i = blockIdx.x / slices;
  const int64_t off0 = static_cast<int64_t>(blockIdx.x % slices) * kSwapSlice;
  const int blk = block_ids[i];
  const bool valid = blk >= 0 && blk < num_blocks;
  uint8_t* cache = blockIdx.y == 0 ? k_cache : v_cache;
  uint8_t* img = staging + (static_cast<int64_t>(blockIdx.y) * n_blocks + i) * block_bytes;
  const int64_t end = min(off0 + kSwapSlice, block_bytes);
  if (PACK) {
    for (int64_t o = off0 + 16 * threadIdx.x; o < end; o += 16 * blockDim.x) {
      swap_u32x4 w = {0u, 0u, 0u, 0u};                 // an absent block packs as zeros
      if (valid)
        w = __builtin_nontemporal_load(
            reinterpret_cast<const swap_u32x4*>(cache + blk * block_bytes + o));
      *reinterpret_cast<swap_u32x4*>(img + o) = w;
    }
  } else {
    if (!valid) return;                               // an absent block is skipped
    for (int64_t o = off0 + 16 * threadIdx.x; o < end; o += 16 * blockDim.x)
      *reinterpret_cast<swap_u32x4*>(cache + blk * block_bytes + o) =
          __builtin_nontemporal_load(reinterpret_cast<const swap_u32x4*>(img + o));
  }
}

// ------------------------------------------------------------------ launchers

hipError_t launch_slot_mapping(const int32_t* block_tables, int max_blocks,
                               const int32_t* positions, int B, int bs, int64_t* slots,
                               hipStream_t stream) {
  const int threads = 256;
  slot_mapping_kernel<<<(B + threads - 1) / threads, threads, 0, stream>>>(
      block_tables, max_blocks, positions, B, bs, slots);
  return hipGetLastError();
}

hipError_t launch_kv_append(const pkv_cache_desc& d, void* k_cache, void* v_cache,
                            const void* k_new, const void* v_new, const int64_t* slots, int T,
                            const float* k_scale, const float* v_scale, hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(T) * d.n_kv * (d.d_head / 8);
  const int threads = 256;
  const unsigned grid = static_cast<unsigned>((total + threads - 1) / threads);
  auto* kc = static_cast<uint8_t*>(k_cache);
  auto* vc = static_cast<uint8_t*>(v_cache);
  auto* kn = static_cast<const uint16_t*>(k_new);
  auto* vn = static_cast<const uint16_t*>(v_new);
  if (d.kv_dtype == PKV_FP8_E4M3)
    kv_append_kernel<1><<<grid, threads, 0, stream>>>(kc, vc, kn, vn, slots, T, d.n_kv,
                                                      d.d_head, d.block_size, d.num_blocks,
                                                      k_scale, v_scale);
  else if (d.kv_dtype == PKV_FP4_E2M1)
    kv_append_kernel<2><<<grid, threads, 0, stream>>>(kc, vc, kn, vn, slots, T, d.n_kv,
                                                      d.d_head, d.block_size, d.num_blocks,
                                                      k_scale, v_scale);
  else
    kv_append_kernel<0><<<grid, threads, 0, stream>>>(kc, vc, kn, vn, slots, T, d.n_kv,
                                                      d.d_head, d.block_size, d.num_blocks,
                                                      k_scale, v_scale);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(const pkv_cache_desc& d, void* k_cache, void* v_cache,
                              const int32_t* pairs, int n_pairs, hipStream_t stream) {
  const int64_t block_bytes = static_cast<int64_t>(d.n_kv) * d.block_size * row_bytes_of(d);
  copy_blocks_kernel<<<dim3(n_pairs, 2), 256, 0, stream>>>(
      static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache), pairs, block_bytes,
      d.num_blocks);
  return hipGetLastError();
}

hipError_t launch_gather(const pkv_cache_desc& d, void* k_out, void* v_out, const void* k_cache,
                         const void* v_cache, const int32_t* table, int ctx,
                         hipStream_t stream) {
  const int row_bytes = row_bytes_of(d);
  const int64_t total = static_cast<int64_t>(ctx) * d.n_kv * (row_bytes / 16);
  const int threads = 256;
  gather_kernel<<<static_cast<unsigned>((total + threads - 1) / threads), threads, 0, stream>>>(
      static_cast<uint8_t*>(k_out), static_cast<uint8_t*>(v_out),
      static_cast<const uint8_t*>(k_cache), static_cast<const uint8_t*>(v_cache), table, ctx,
      d.n_kv, row_bytes, d.block_size, d.num_blocks);
  return hipGetLastError();
}

int64_t swap_block_bytes(const pkv_cache_desc& d) {
  return static_cast<int64_t>(d.n_kv) * d.block_size * row_bytes_of(d);
}

hipError_t launch_swap_pack(const pkv_cache_desc& d, const void* k_cache, const void* v_cache,
                            const int32_t* block_ids, int n, void* staging, hipStream_t stream) {
  const int64_t bb = swap_block_bytes(d);
  const int slices = static_cast<int>((bb + kSwapSlice - 1) / kSwapSlice);
  swap_blocks_kernel<true><<<dim3(n * slices, 2), 256, 0, stream>>>(
      const_cast<uint8_t*>(static_cast<const uint8_t*>(k_cache)),
      const_cast<uint8_t*>(static_cast<const uint8_t*>(v_cache)), block_ids, n, bb, d.num_blocks,
      static_cast<uint8_t*>(staging));
  return hipGetLastError();
}

hipError_t launch_swap_unpack(const pkv_cache_desc& d, void* k_cache, void* v_cache,
                              const int32_t* block_ids, int n, const void* staging,
                              hipStream_t stream) {
  const int64_t bb = swap_block_bytes(d);
  const int slices = static_cast<int>((bb + kSwapSlice - 1) / kSwapSlice);
  swap_blocks_kernel<false><<<dim3(n * slices, 2), 256, 0, stream>>>(
      static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache), block_ids, n, bb,
      d.num_blocks, const_cast<uint8_t*>(static_cast<const uint8_t*>(staging)));
  return hipGetLastError();
}

}  // namespace pkv

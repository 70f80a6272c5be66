// Split-K log-sum-exp reduce of paged decode attention, and the decode
// dispatch.
//
// The partition kernel (decode_mfma.hip) or the multi-query kernels write one
// (m, l, o) partial per (row, partition): the running max, running sum and
// normalised accumulator of [MTKV] "Architecting Multi-Tier Disaggregated
// KV-Cache Hierarchies for Terabyte-Scale LLM Inference" (ultrainstinct.tech),
// section "High-Throughput Paged Attention Kernel Integration", evaluated over
// one partition of the context. Merging them is exact: with M = max_j m_j and
// w_j = l_j 2^(m_j - M) (scores in base-2 units), the row's output is
// sum_j w_j o_j / sum_j w_j; a partition with no tokens has l = 0 and no
// weight, and a row with no weight at all is written as zeros.
#include <float.h>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

// ---------------------------------------------------------------------------
// Split-K reduce, two shapes chosen by the partition count:
//   <= 32 partitions: one wave per (sequence, query head) (below);
//   more: one 256-thread workgroup per (sequence, query head). Thread t owns
//   output dims 4*(t % (D/4)) .. +4 for the partitions j = t / (D/4)
//   (mod 256 / (D/4)), reading 16 bytes per partition row, so a long list of
//   partitions is read many rows at a time; the weights
//   w_j = l_j 2^(m_j - M) are computed once into LDS.
// ---------------------------------------------------------------------------
constexpr int kWaveReduceMaxPartitions = 32;
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Which partials an output row merges. Rows are (sequence, query, head),
// query-major within a sequence; with one query per sequence (query_lens null)
// a row reads every partition of its context, otherwise query i of q_len sits
// at position ctx - q_len + i and reads only the partitions up to it; rows past
// q_len read none and are written as zeros.
// A second source (m2, l2, o2: P2 partitions per row, all present) is merged
// after a row's own partitions: the shared-prefix partials of a cascade.
struct ReduceRows {
  const int32_t* context_lens;
  const int32_t* query_lens;
  int Q, n_q, P_max, partition, ctx_cap;
  const float* m2;
  const float* l2;
  const float* o2;
  int P2;
};

__device__ __forceinline__ int row_partitions(const ReduceRows& r, int64_t row) {
  const int b = static_cast<int>(row / (static_cast<int64_t>(r.Q) * r.n_q));
  const int ctx = min(r.context_lens[b], r.ctx_cap);
  int last = ctx;                                    // tokens this row sees
  if (r.query_lens) {
    const int i = static_cast<int>((row / r.n_q) % r.Q);
    const int ql = max(0, min(min(r.query_lens[b], r.Q), ctx));
    last = i < ql ? ctx - ql + i + 1 : 0;
  }
  return last > 0 ? min((last + r.partition - 1) / r.partition, r.P_max) : 0;
}

// Few partitions per sequence: one wave per (sequence, query head), lanes own
// output dims, weights broadcast by cross-lane reads (no LDS, no barrier).
template <int D>
__global__ __launch_bounds__(256) void splitk_reduce_wave_kernel(
    void* __restrict__ out, int out_dtype, const float* __restrict__ m,
    const float* __restrict__ l, const float* __restrict__ o,
    ReduceRows rows, int64_t n_rows) {
  constexpr int DL = D / 64;                         // output dims per lane
  const int lane = threadIdx.x & 63;
  const int64_t bh = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (bh >= n_rows) return;                          // whole wave
  const int P_max = rows.P_max;
  const int np1 = row_partitions(rows, bh);
  const int np = np1 + rows.P2;
  const float* mb = m + static_cast<int64_t>(bh) * P_max;
  const float* lb = l + static_cast<int64_t>(bh) * P_max;
  const float* ob = o + static_cast<int64_t>(bh) * P_max * D;
  const float* mb2 = rows.m2 + static_cast<int64_t>(bh) * rows.P2;
  const float* lb2 = rows.l2 + static_cast<int64_t>(bh) * rows.P2;
  const float* ob2 = rows.o2 + static_cast<int64_t>(bh) * rows.P2 * D;
  auto pm = [&](int j) { return j < np1 ? mb[j] : mb2[j - np1]; };
  auto pl = [&](int j) { return j < np1 ? lb[j] : lb2[j - np1]; };
  auto po = [&](int j) { return j < np1 ? ob + static_cast<int64_t>(j) * D
                                        : ob2 + static_cast<int64_t>(j - np1) * D; };

  float mx = -INFINITY;
  for (int jj = lane; jj < np; jj += 64) mx = fmaxf(mx, pm(jj));
  const float M = wave_max(mx);
  float acc[DL];
#pragma unroll
  for (int k = 0; k < DL; ++k) acc[k] = 0.0f;
  float lsum = 0.0f;
  for (int j0 = 0; j0 < np; j0 += 64) {
    const int jl = j0 + lane;
    const float wl = jl < np ? pl(jl) * fast_exp2(pm(jl) - M) : 0.0f;
    lsum += wl;
    const int n = min(64, np - j0);
    for (int jj = 0; jj < n; ++jj) {
      const float wj = __shfl(wl, jj);
      const float* row = po(j0 + jj);
#pragma unroll
      for (int k = 0; k < DL; ++k) acc[k] = fmaf(wj, row[lane + 64 * k], acc[k]);
    }
  }
  const float L = wave_sum(lsum);
#pragma unroll
  for (int k = 0; k < DL; ++k) {
    const float v = np > 0 ? acc[k] / L : 0.0f;
    const int64_t oi = static_cast<int64_t>(bh) * D + lane + 64 * k;
    if (out_dtype == PKV_FP32)
      static_cast<float*>(out)[oi] = v;
    else
      static_cast<uint16_t*>(out)[oi] = f32_to_bf16_rne(v);
  }
}

// Many partitions per sequence: one 256-thread workgroup per (sequence, head).
template <int D>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(
    void* __restrict__ out, int out_dtype, const float* __restrict__ m,
    const float* __restrict__ l, const float* __restrict__ o,
    ReduceRows rows) {
  constexpr int DG = D / 4;                           // 16-byte dim groups
  constexpr int PG = 256 / DG;                        // partition groups
  __shared__ float w[kMaxReducePartitions];
  __shared__ float red[4];
  __shared__ float4 part[PG][DG];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wv = t >> 6;
  const int64_t bh = blockIdx.x;
  const int P_max = rows.P_max;
  const int np1 = row_partitions(rows, bh);
  const int np = np1 + rows.P2;
  const float* mb = m + static_cast<int64_t>(bh) * P_max;
  const float* lb = l + static_cast<int64_t>(bh) * P_max;
  const float* ob = o + static_cast<int64_t>(bh) * P_max * D;
  const float* mb2 = rows.m2 + static_cast<int64_t>(bh) * rows.P2;
  const float* lb2 = rows.l2 + static_cast<int64_t>(bh) * rows.P2;
  const float* ob2 = rows.o2 + static_cast<int64_t>(bh) * rows.P2 * D;
  auto pm = [&](int j) { return j < np1 ? mb[j] : mb2[j - np1]; };
  auto pl = [&](int j) { return j < np1 ? lb[j] : lb2[j - np1]; };
  auto po = [&](int j) { return j < np1 ? ob + static_cast<int64_t>(j) * D
                                        : ob2 + static_cast<int64_t>(j - np1) * D; };

  float mx = -INFINITY;
  for (int jj = t; jj < np; jj += 256) mx = fmaxf(mx, pm(jj));
  mx = wave_max(mx);
  if (lane == 0) red[wv] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float ls = 0.0f;
  for (int jj = t; jj < np; jj += 256) {
    const float wj = pl(jj) * fast_exp2(pm(jj) - M);
    w[jj] = wj;
    ls += wj;
  }
  ls = wave_sum(ls);
  if (lane == 0) red[wv] = ls;
  __syncthreads();
  const float L = red[0] + red[1] + red[2] + red[3];

  const int dg = t % DG;
  const int pg = t / DG;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int jj = pg; jj < np; jj += PG) {
    const float wj = w[jj];
    const float4 v = *reinterpret_cast<const float4*>(po(jj) + 4 * dg);
    acc.x = fmaf(wj, v.x, acc.x);
    acc.y = fmaf(wj, v.y, acc.y);
    acc.z = fmaf(wj, v.z, acc.z);
    acc.w = fmaf(wj, v.w, acc.w);
  }
  part[pg][dg] = acc;
  __syncthreads();
  if (t < D) {
    float s = 0.0f;
    const int g4 = t / 4;
    const int k = t % 4;
#pragma unroll
    for (int q = 0; q < PG; ++q) {
      const float4 v = part[q][g4];
      s += k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
    }
    const float r = np > 0 ? s / L : 0.0f;
    const int64_t oi = static_cast<int64_t>(bh) * D + t;
    if (out_dtype == PKV_FP32)
      static_cast<float*>(out)[oi] = r;
    else
      static_cast<uint16_t*>(out)[oi] = f32_to_bf16_rne(r);
  }
}

// ------------------------------------------------------------------ dispatch

bool decode_supported(int d, int bs, int G, int kv_dtype) {
  if (d != 64 && d != 128) return false;
  if (bs != 16 && bs != 32) return false;
  if (kv_dtype != PKV_BF16 && kv_dtype != PKV_FP8_E4M3 && kv_dtype != PKV_FP4_E2M1) return false;
  if (kv_dtype == PKV_FP4_E2M1 && d != 128) return false;   // 64-byte rows
  // the matrix-core kernels take any number of query heads per KV head: a
  // head tile's unused columns (decode) or a row group's unused rows
  // (multi-query) are zero operands
  return G > 0;
}

hipError_t launch_decode_partition(const DecodeArgs& a, hipStream_t s) {
  return launch_decode_partition_mfma(a, s);
}

hipError_t launch_splitk_reduce(void* out, int out_dtype, const float* m, const float* l,
                                const float* o, const int32_t* context_lens, int B, int n_q,
                                int d, int P_max, int partition, hipStream_t stream, int Q,
                                const int32_t* query_lens, int ctx_cap, const float* m2,
                                const float* l2, const float* o2, int P2) {
  if (P_max + P2 > kMaxReducePartitions || (d != 64 && d != 128)) return hipErrorInvalidValue;
  const ReduceRows rows{context_lens, query_lens, Q, n_q, P_max, partition, ctx_cap,
                        m2, l2, o2, m2 ? P2 : 0};
  const int64_t n_rows = static_cast<int64_t>(B) * Q * n_q;
  if (P_max + rows.P2 <= kWaveReduceMaxPartitions) {
    const unsigned grid = static_cast<unsigned>((n_rows + 3) / 4);
    if (d == 128)
      splitk_reduce_wave_kernel<128><<<grid, 256, 0, stream>>>(out, out_dtype, m, l, o, rows,
                                                               n_rows);
    else
      splitk_reduce_wave_kernel<64><<<grid, 256, 0, stream>>>(out, out_dtype, m, l, o, rows,
                                                              n_rows);
    return hipGetLastError();
  }
  const unsigned grid = static_cast<unsigned>(n_rows);
  if (d == 128)
    splitk_reduce_kernel<128><<<grid, 256, 0, stream>>>(out, out_dtype, m, l, o, rows);
  else
    splitk_reduce_kernel<64><<<grid, 256, 0, stream>>>(out, out_dtype, m, l, o, rows);
  return hipGetLastError();
}

}  // namespace pkv

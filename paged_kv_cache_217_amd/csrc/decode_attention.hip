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
//   <= 32 partitions: D / 4 lanes per (sequence, query head) (below);
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

// Few partitions per sequence: D / 4 lanes per output row (two rows per wave
// at d 128, four at d 64), each lane owning 4 output dims. A lane first loads
// the m and l of up to two of its row's partitions, so the row's maximum and
// weights w_j = l_j 2^(m_j - M) take one memory round trip and a few
// cross-lane steps; the partial outputs are then loaded 16 bytes per lane,
// eight partitions at a time, each weight broadcast from the lane that holds
// it. A row with np partitions thus waits for about 1 + np / 8 round trips
// instead of one per partition.
template <int D>
__global__ __launch_bounds__(256) void splitk_reduce_wave_kernel(
    void* __restrict__ out, int out_dtype, const float* __restrict__ m,
    const float* __restrict__ l, const float* __restrict__ o,
    ReduceRows rows, int64_t n_rows) {
  constexpr int LPR = D / 4;                         // lanes per row
  constexpr int RPW = 64 / LPR;                      // rows per wave
  constexpr int WPR = (kWaveReduceMaxPartitions + LPR - 1) / LPR;   // weights per lane
  constexpr int UNROLL = 8;                          // partition rows loaded together
  const int lane = threadIdx.x & 63;
  const int sub = lane / LPR;                        // the lane's row within the wave
  const int lr = lane % LPR;                         // its dims 4 lr .. 4 lr + 3
  const int64_t bh =
      (static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6)) * RPW + sub;
  const bool live = bh < n_rows;
  const int P_max = rows.P_max;
  const int np1 = live ? row_partitions(rows, bh) : 0;
  const int np = live ? np1 + rows.P2 : 0;
  const int64_t r = live ? bh : 0;
  const float* mb = m + r * P_max;
  const float* lb = l + r * P_max;
  const float* ob = o + r * P_max * D;
  const float* mb2 = rows.m2 + r * rows.P2;
  const float* lb2 = rows.l2 + r * rows.P2;
  const float* ob2 = rows.o2 + r * rows.P2 * D;
  auto po = [&](int j) { return j < np1 ? ob + static_cast<int64_t>(j) * D
                                        : ob2 + static_cast<int64_t>(j - np1) * D; };

  // partitions lr + LPR k of this row: m and l, the row's maximum and weights
  float mj[WPR], lj[WPR];
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < WPR; ++k) {
    const int j = lr + LPR * k;
    mj[k] = -INFINITY;
    lj[k] = 0.0f;
    if (j < np) {
      mj[k] = j < np1 ? mb[j] : mb2[j - np1];
      lj[k] = j < np1 ? lb[j] : lb2[j - np1];
    }
    mx = fmaxf(mx, mj[k]);
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  float w[WPR];
  float ls = 0.0f;
#pragma unroll
  for (int k = 0; k < WPR; ++k) {
    w[k] = lr + LPR * k < np && mj[k] != -INFINITY ? lj[k] * fast_exp2(mj[k] - mx) : 0.0f;
    ls += w[k];
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) ls += __shfl_xor(ls, off);

  // every partition row: weight from lane sub LPR + j % LPR, 16 bytes per lane
  int npw = np;                                      // the wave's largest np
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) npw = max(npw, __shfl_xor(npw, off));
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int j0 = 0; j0 < npw; j0 += UNROLL) {
    float4 v[UNROLL];
    float wj[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int j = j0 + u;
      float wk = 0.0f;
#pragma unroll
      for (int k = 0; k < WPR; ++k)
        if (j / LPR == k) wk = __shfl(w[k], sub * LPR + j % LPR);
      wj[u] = j < np ? wk : 0.0f;
      v[u] = j < np ? *reinterpret_cast<const float4*>(po(j) + 4 * lr)
                    : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      acc.x = fmaf(wj[u], v[u].x, acc.x);
      acc.y = fmaf(wj[u], v[u].y, acc.y);
      acc.z = fmaf(wj[u], v[u].z, acc.z);
      acc.w = fmaf(wj[u], v[u].w, acc.w);
    }
  }
  if (!live) return;
  const float inv = ls > 0.0f ? 1.0f / ls : 0.0f;     // no weight at all: zeros
  const int64_t oi = bh * D + 4 * lr;
  if (out_dtype == PKV_FP32) {
    *reinterpret_cast<float4*>(static_cast<float*>(out) + oi) =
        make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  } else {
    uint16_t* ob16 = static_cast<uint16_t*>(out) + oi;
    ob16[0] = f32_to_bf16_rne(acc.x * inv);
    ob16[1] = f32_to_bf16_rne(acc.y * inv);
    ob16[2] = f32_to_bf16_rne(acc.z * inv);
    ob16[3] = f32_to_bf16_rne(acc.w * inv);
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
    const int64_t rows_per_block = 4 * (64 / (d / 4));
    const unsigned grid = static_cast<unsigned>((n_rows + rows_per_block - 1) / rows_per_block);
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

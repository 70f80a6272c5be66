// Paged single-token decode attention: partition kernel + split-K reduce.
//
// What is computed follows [MTKV] "Architecting Multi-Tier Disaggregated
// KV-Cache Hierarchies for Terabyte-Scale LLM Inference" (ultrainstinct.tech),
// section "High-Throughput Paged Attention Kernel Integration": for each
// sequence and query head, walk the sequence's logical blocks, resolve each
// through the block table, score the block's keys against the query, and
// fold the scores into a running max / running sum / rescaled accumulator
// (online softmax); query head h reads KV head h / G. The weights are the
// softmax of scale * q . k ([MTKV] "Mathematical Formulation of Block
// Salience").
//
// How it is computed here differs from the page's kernel (one program per
// (sequence, query head), which re-reads every KV byte G times):
//   * one workgroup serves all G query heads of a KV head (or a tile of 8 of
//     them), so each K/V byte of the partition is read from HBM once;
//   * the context is cut into partitions (split-K) so that short batches
//     still fill 256 CUs; partial (m, l, o) are merged by a log-sum-exp
//     reduce;
//   * scores live in base-2 units (scale * log2 e folded into q) so the
//     exponentials are single v_exp_f32 instructions;
//   * masked slots (past the sequence length, possibly NaN) are removed by
//     selection, never by multiplying with zero.
#include <float.h>
#include <stdlib.h>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// VALU partition kernel.
//
// Workgroup = 4 waves, one (partition, kv head, head tile, sequence). Within a
// wave, a (block, head) tile of BS tokens x D elements is spread as: lane
// (row r, chunk c) holds elements [8c, 8c+8) of tokens r, r+RPL, r+2RPL, ...
// with LPR = D/8 lanes per token row, so every load instruction reads whole
// contiguous rows (16 B per lane for bf16, 8 B for FP8). Waves take the
// partition's blocks round-robin; their (m, l, acc) merge through LDS.
// ---------------------------------------------------------------------------
template <int D, int BS, int GT, bool FP8>
__global__ __launch_bounds__(256) void decode_partition_valu(DecodeArgs a) {
  constexpr int LPR = D / 8;           // lanes per token row
  constexpr int RPL = kWave / LPR;     // rows per load instruction
  constexpr int NL = BS / RPL;         // loads per lane per tile
  constexpr int NW = 4;                // waves per workgroup
  static_assert(BS % RPL == 0, "tile shape");

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c = lane % LPR;
  const int r = lane / LPR;

  const int j = blockIdx.x;
  const int tiles = (a.n_q / a.n_kv) / GT;
  const int g = blockIdx.y / tiles;
  const int h0 = g * (a.n_q / a.n_kv) + (blockIdx.y % tiles) * GT;
  const int b = blockIdx.z;
  // a length beyond the table row is a caller error; never read past the row
  const int ctx = min(a.context_lens[b], a.max_blocks * BS);
  const int t0 = j * a.partition;

  __shared__ float sm_m[NW][GT];
  __shared__ float sm_l[NW][GT];
  __shared__ float sm_acc[NW][GT][D];

  if (t0 >= ctx) {
    // empty partition; an empty sequence still owes zeros in single-pass mode
    if (!a.write_partials && j == 0) {
      for (int i = threadIdx.x; i < GT * D; i += blockDim.x) {
        const int64_t o = (static_cast<int64_t>(b) * a.n_q + h0 + i / D) * D + i % D;
        if (a.out_dtype == PKV_FP32)
          static_cast<float*>(a.out)[o] = 0.0f;
        else
          static_cast<uint16_t*>(a.out)[o] = 0;
      }
    }
    return;
  }
  const int t1 = min(t0 + a.partition, ctx);
  const int blk0 = t0 / BS;
  const int blk1 = (t1 + BS - 1) / BS;

  // query slice for this lane, pre-scaled into base-2 score units
  float qs = a.scale * kLog2e;
  if constexpr (FP8) qs *= a.k_scale[g];
  float qf[GT][8];
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    const uint4 w = *reinterpret_cast<const uint4*>(
        a.q + (static_cast<int64_t>(b) * a.n_q + h0 + h) * D + c * 8);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bf16x2_to_f32(ws[e], qf[h][2 * e], qf[h][2 * e + 1]);
      qf[h][2 * e] *= qs;
      qf[h][2 * e + 1] *= qs;
    }
  }

  float m[GT], l[GT], acc[GT][8];
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.0f;
  }

  const int32_t* bt = a.block_tables + static_cast<int64_t>(b) * a.max_blocks;
  constexpr int P = FP8 ? 1 : 2;       // bytes per element

  for (int blk = blk0 + wave; blk < blk1; blk += NW) {
    int phys = bt[blk];
    if (phys < 0 || phys >= a.num_blocks) phys = 0;
    const int64_t tile = (static_cast<int64_t>(phys) * a.n_kv + g) * BS * D;   // elements

    float kf[NL][8], vf[NL][8];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int64_t off = (tile + (r + i * RPL) * D + c * 8) * P;
      if constexpr (!FP8) {
        const uint4 kw = *reinterpret_cast<const uint4*>(a.k_cache + off);
        const uint4 vw = *reinterpret_cast<const uint4*>(a.v_cache + off);
        const uint32_t ks[4] = {kw.x, kw.y, kw.z, kw.w};
        const uint32_t vs[4] = {vw.x, vw.y, vw.z, vw.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bf16x2_to_f32(ks[e], kf[i][2 * e], kf[i][2 * e + 1]);
          bf16x2_to_f32(vs[e], vf[i][2 * e], vf[i][2 * e + 1]);
        }
      } else {
        const uint2 kw = *reinterpret_cast<const uint2*>(a.k_cache + off);
        const uint2 vw = *reinterpret_cast<const uint2*>(a.v_cache + off);
        fp8x4_to_f32(kw.x, &kf[i][0]);
        fp8x4_to_f32(kw.y, &kf[i][4]);
        fp8x4_to_f32(vw.x, &vf[i][0]);
        fp8x4_to_f32(vw.y, &vf[i][4]);
      }
    }

    // scores: partial dot over this lane's 8 elements, then across the row's lanes
    float s[GT][NL];
#pragma unroll
    for (int h = 0; h < GT; ++h)
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        float x = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) x = fmaf(qf[h][e], kf[i][e], x);
        s[h][i] = x;
      }
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1)
#pragma unroll
      for (int h = 0; h < GT; ++h)
#pragma unroll
        for (int i = 0; i < NL; ++i) s[h][i] += __shfl_xor(s[h][i], off);

    // mask slots past the partition end (only the sequence's last block has any)
    bool valid[NL];
    const bool tail = (blk + 1) * BS > t1;
#pragma unroll
    for (int i = 0; i < NL; ++i) valid[i] = !tail || (blk * BS + r + i * RPL < t1);

#pragma unroll
    for (int h = 0; h < GT; ++h) {
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < NL; ++i) mx = fmaxf(mx, valid[i] ? s[h][i] : -INFINITY);
#pragma unroll
      for (int off = LPR; off < kWave; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      const float m_new = fmaxf(m[h], mx);
      const float alpha = fast_exp2(m[h] - m_new);
      float psum = 0.0f;
      float p[NL];
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        p[i] = valid[i] ? fast_exp2(s[h][i] - m_new) : 0.0f;
        psum += p[i];
      }
      l[h] = l[h] * alpha + psum;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float x = acc[h][e] * alpha;
#pragma unroll
        for (int i = 0; i < NL; ++i) x = fmaf(p[i], valid[i] ? vf[i][e] : 0.0f, x);
        acc[h][e] = x;
      }
      m[h] = m_new;
    }
  }

  // wave totals: sum l and acc over the rows (lanes with the same chunk c)
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1)
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      l[h] += __shfl_xor(l[h], off);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] += __shfl_xor(acc[h][e], off);
    }
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      if (c == 0) {
        sm_m[wave][h] = m[h];
        sm_l[wave][h] = l[h];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) sm_acc[wave][h][c * 8 + e] = acc[h][e];
    }
  }
  __syncthreads();

  // merge the waves and write (m, l, o) or the final output
  for (int i = threadIdx.x; i < GT * D; i += blockDim.x) {
    const int h = i / D;
    const int e = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w][h]);
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = sm_m[w][h] == -INFINITY ? 0.0f : fast_exp2(sm_m[w][h] - M);
      L = fmaf(sm_l[w][h], f, L);
      O = fmaf(sm_acc[w][h][e], f, O);
    }
    const int hq = h0 + h;
    float o = O / L;
    if constexpr (FP8) o *= a.v_scale[g];
    if (a.write_partials) {
      const int64_t mi = (static_cast<int64_t>(b) * a.n_q + hq) * a.P_max + j;
      if (e == 0) {
        a.ws_m[mi] = M;
        a.ws_l[mi] = L;
      }
      a.ws_o[mi * D + e] = o;
    } else {
      const int64_t oi = (static_cast<int64_t>(b) * a.n_q + hq) * D + e;
      if (a.out_dtype == PKV_FP32)
        static_cast<float*>(a.out)[oi] = o;
      else
        static_cast<uint16_t*>(a.out)[oi] = f32_to_bf16_rne(o);
    }
  }
}

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

template <int D, int BS, bool FP8>
static hipError_t launch_gt(const DecodeArgs& a, int GT, dim3 grid, hipStream_t s) {
  switch (GT) {
    case 1: decode_partition_valu<D, BS, 1, FP8><<<grid, 256, 0, s>>>(a); break;
    case 2: decode_partition_valu<D, BS, 2, FP8><<<grid, 256, 0, s>>>(a); break;
    case 4: decode_partition_valu<D, BS, 4, FP8><<<grid, 256, 0, s>>>(a); break;
    case 8: decode_partition_valu<D, BS, 8, FP8><<<grid, 256, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

static int head_tile(int G) { return G <= 8 ? G : 8; }

bool decode_supported(int d, int bs, int G, int kv_dtype) {
  if (d != 64 && d != 128) return false;
  if (bs != 16 && bs != 32) return false;
  if (kv_dtype != PKV_BF16 && kv_dtype != PKV_FP8_E4M3 && kv_dtype != PKV_FP4_E2M1) return false;
  if (kv_dtype == PKV_FP4_E2M1 && d != 128) return false;   // matrix-core kernel, 64-byte rows
  if (G == 1 || G == 2 || G == 4 || G == 8) return true;
  return G > 0 && G % 8 == 0;
}

hipError_t launch_decode_partition_valu(const DecodeArgs& a, hipStream_t s) {
  if (a.kv_dtype == PKV_FP4_E2M1) return hipErrorInvalidValue;   // matrix-core kernel only
  const int G = a.n_q / a.n_kv;
  const int GT = head_tile(G);
  const dim3 grid(a.P_max, a.n_kv * (G / GT), a.B);
  const bool fp8 = a.kv_dtype == PKV_FP8_E4M3;
  if (a.d == 128) {
    if (a.bs == 16) return fp8 ? launch_gt<128, 16, true>(a, GT, grid, s)
                               : launch_gt<128, 16, false>(a, GT, grid, s);
    return fp8 ? launch_gt<128, 32, true>(a, GT, grid, s) : launch_gt<128, 32, false>(a, GT, grid, s);
  }
  if (a.bs == 16) return fp8 ? launch_gt<64, 16, true>(a, GT, grid, s)
                             : launch_gt<64, 16, false>(a, GT, grid, s);
  return fp8 ? launch_gt<64, 32, true>(a, GT, grid, s) : launch_gt<64, 32, false>(a, GT, grid, s);
}

// The matrix-core kernel serves every supported shape; PKV_DECODE_KERNEL=valu
// selects the vector-ALU kernel instead (kept for A/B measurement).
static bool use_valu() {
  static const bool v = [] {
    const char* e = getenv("PKV_DECODE_KERNEL");
    return e && e[0] == 'v';
  }();
  return v;
}

hipError_t launch_decode_partition(const DecodeArgs& a, hipStream_t s) {
  return use_valu() ? launch_decode_partition_valu(a, s) : launch_decode_partition_mfma(a, s);
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

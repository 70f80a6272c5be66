// Paged attention for several new query tokens per sequence (chunked prefill,
// verification of draft tokens), on the gfx950 matrix cores.
//
// What is computed: query i of sequence b sits at position
// p = ctx_b - q_len_b + i (its own K/V is already in the cache) and attends
// causally to tokens 0..p: the prompt-ingestion case of [LLMI] "LLM
// inference: prefill, decode, KV cache" (systemcraft.online), section
// "4. Internal workings" (causal self-attention over the prompt), processed
// in chunks alongside decode ([LLMI] "9. Failure modes and limitations") or
// as the verification pass of speculative decoding ([LLMI] "7. Practical
// applications"). The K/V gather through the block table and the online
// softmax are the single-token path's ([MTKV] "Architecting Multi-Tier
// Disaggregated KV-Cache Hierarchies for Terabyte-Scale LLM Inference",
// "High-Throughput Paged Attention Kernel Integration").
//
// Same layout as the decode kernel (decode_mfma.hip) with "head" generalised
// to "query row": the rows of a KV head's group are (query i, head h) pairs,
// i-major, 16 per matrix-core tile, so a tile is full as soon as
// q_len x G >= 16 (decode pads G = 8 heads to 16). Lane (c, g4) owns row c's
// softmax state and output slice. Rows differ in how far they may look: a
// chunk that reaches past the tile's smallest position masks each lane's
// scores beyond its own row's position; tokens past the tile's largest
// position are not read at all. Rows that see no token of a partition emit
// an empty partial (l = 0, o = 0) and the reduce skips them.
#include <float.h>

#include "mfma_common.h"
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

using namespace mfma;

template <int D, int BS, bool FP8, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void multi_query_partition_mfma(DecodeArgs a) {
  constexpr int CT = FP8 ? 64 : 32;           // tokens per chunk
  constexpr int NRG = CT / 16;                // 16-token row groups per chunk
  constexpr int NKS = CT / 32;                // 32-token PV k-steps per chunk
  constexpr int NKK = D / 32;                 // QK MFMA steps over d
  constexpr int NKL = FP8 ? NKK / 2 : NKK;    // 16-byte K loads per row group
  constexpr int NJ = D / 16;                  // PV MFMAs per k-step
  constexpr int DPL = D / 16;                 // dims per lane per V row
  constexpr int BPC = CT / BS;                // blocks per chunk
  constexpr int EB = FP8 ? 1 : 2;             // bytes per element
  constexpr int VB = DPL * EB;
  constexpr int NVS = 8 * NKS;
  using VT = typename Vec<VB>::T;
  constexpr int VW = (DPL * 2) / 4;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15;
  const int g4 = lane >> 4;

  // grid: x = (KV head, row tile), y = sequence, z = partition from the end
  const int G = a.n_q / a.n_kv;
  const int rows = a.Q * G;                           // query rows of one KV head
  const int tiles = (rows + 15) / 16;
  const int g = blockIdx.x / tiles;
  const int tile = blockIdx.x % tiles;
  const int b = blockIdx.y;
  const int j = gridDim.z - 1 - blockIdx.z;
  const int ctx = min(a.context_lens[b], a.max_blocks * BS);
  const int ql = max(0, min(min(a.query_lens[b], a.Q), ctx));

  // this lane's row and its position; the tile's position range
  const int row = tile * 16 + c;
  const int qi = row / G;
  const int hq = g * G + row % G;
  const bool live_row = row < rows && qi < ql;
  const int pos = ctx - ql + qi;                      // last token this row may see
  const int i_lo = (tile * 16) / G;
  const int i_hi = min((tile * 16 + 15) / G, ql - 1);
  const int p_lo = ctx - ql + i_lo;
  const int p_hi = ctx - ql + i_hi;
  const int t0 = j * a.partition;

  __shared__ float sm_m[NW][16];
  __shared__ float sm_l[NW][16];
  __shared__ float sm_acc[NW][16][D + 4];

  if (i_lo >= ql || t0 > p_hi) {
    // no row of this tile reads this partition; a single pass still owes the
    // tile's rows their zeros (rows past q_len, or a sequence with none)
    if (!a.write_partials && j == 0) {
      for (int e = threadIdx.x; e < 16 * D; e += blockDim.x) {
        const int r = tile * 16 + e / D;
        if (r >= rows) continue;
        const int64_t oi =
            ((static_cast<int64_t>(b) * a.Q + r / G) * a.n_q + g * G + r % G) * D + e % D;
        if (a.out_dtype == PKV_FP32)
          static_cast<float*>(a.out)[oi] = 0.0f;
        else
          static_cast<uint16_t*>(a.out)[oi] = 0;
      }
    }
    return;
  }
  const int t1 = min(t0 + a.partition, p_hi + 1);    // tokens past p_hi are never read
  const int blk0 = t0 / BS;
  const int blk1 = (t1 + BS - 1) / BS;
  const int n_ch = (blk1 - blk0 + BPC - 1) / BPC;

  auto dimbase = [&](int kk) -> int {
    return FP8 ? 64 * (kk >> 1) + 16 * g4 + 8 * (kk & 1) : 32 * kk + 8 * g4;
  };
  bf16x8_t qop[NKK];
  {
    const int64_t qrow = live_row ? (static_cast<int64_t>(b) * a.Q + qi) * a.n_q + hq : 0;
    const uint16_t* qp = a.q + qrow * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      uint4 w = *reinterpret_cast<const uint4*>(qp + dimbase(kk));
      if (!live_row) w = make_uint4(0, 0, 0, 0);
      qop[kk] = __builtin_bit_cast(bf16x8_t, w);
    }
  }
  float qscale = a.scale * kLog2e;
  if constexpr (FP8) qscale *= a.k_scale[g];

  const int64_t tile_bytes = static_cast<int64_t>(BS) * D * EB;
  const int64_t head_off = static_cast<int64_t>(g) * tile_bytes;
  const int64_t block_stride = static_cast<int64_t>(a.n_kv) * tile_bytes;
  const int32_t* bt = a.block_tables + static_cast<int64_t>(b) * a.max_blocks;

  auto v_tok = [&](int s) -> int {
    const int s8 = s & 7;
    return 16 * (2 * (s >> 3) + (s8 >> 2)) + 4 * g4 + (s8 & 3);
  };

  struct Chunk {
    uint4 k[NRG][NKL];
    VT v[NVS];
  };

  auto load = [&](Chunk& ch, int ci) {
    const uint8_t* kb[BPC];
    const uint8_t* vb[BPC];
    bool have[BPC];
#pragma unroll
    for (int i = 0; i < BPC; ++i) {
      const int blk = blk0 + ci * BPC + i;
      have[i] = blk < blk1;
      int p = have[i] ? bt[blk] : 0;
      if (p < 0 || p >= a.num_blocks) p = 0;
      kb[i] = a.k_cache + p * block_stride + head_off;
      vb[i] = a.v_cache + p * block_stride + head_off;
    }
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg) {
      const int t = 16 * rg + c;
      const int bi = t / BS;
#pragma unroll
      for (int kl = 0; kl < NKL; ++kl) {
        const int dim = FP8 ? 64 * kl + 16 * g4 : 32 * kl + 8 * g4;
        if (have[bi])
          ld_stream(ch.k[rg][kl], kb[bi] + ((t % BS) * D + dim) * EB);
        else
          ch.k[rg][kl] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int s = 0; s < NVS; ++s) {
      const int t = v_tok(s);
      const int bi = t / BS;
      if (have[bi])
        ld_stream(ch.v[s], vb[bi] + ((t % BS) * D + DPL * c) * EB);
      else
        ch.v[s] = VT{};
    }
  };

  float m_ref = -INFINITY;
  float m_true = -INFINITY;
  float l = 0.0f;
  f32x4_t acc[NJ];
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj) acc[jj] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  auto compute = [&](Chunk& ch, int ci) {
    const int tok0 = (blk0 + ci * BPC) * BS;
    float s[4 * NRG];
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg) {
      f32x4_t sc = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        bf16x8_t kop;
        if constexpr (!FP8) {
          kop = __builtin_bit_cast(bf16x8_t, ch.k[rg][kk]);
        } else {
          const uint4 w = ch.k[rg][kk >> 1];
          const uint32_t w0 = (kk & 1) ? w.z : w.x;
          const uint32_t w1 = (kk & 1) ? w.w : w.y;
          kop = as_bf16x8(fp8x2_to_bf16x2<false>(w0), fp8x2_to_bf16x2<true>(w0),
                          fp8x2_to_bf16x2<false>(w1), fp8x2_to_bf16x2<true>(w1));
        }
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[kk], sc, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) s[4 * rg + i] = sc[i] * qscale;
    }
    if (tok0 + CT > min(p_lo + 1, t1)) {
      // causal: each row sees tokens up to its own position, and nothing past
      // the partition's end (such slots were not loaded)
      const int lim = min(pos + 1, t1);
#pragma unroll
      for (int rg = 0; rg < NRG; ++rg)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (tok0 + 16 * rg + 4 * g4 + i >= lim) s[4 * rg + i] = -INFINITY;
    }
    if (tok0 + CT > t1) {
#pragma unroll
      for (int si = 0; si < NVS; ++si)
        if (tok0 + v_tok(si) >= t1) ch.v[si] = VT{};
    }
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < 4 * NRG; ++i) mx = fmaxf(mx, s[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    m_true = fmaxf(m_true, mx);
    // a row may see none of a chunk's tokens (all -inf): it keeps its state
    const bool need = mx > m_ref + kLazyRescale;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      const float alpha = need ? fast_exp2(m_ref - mx) : 1.0f;
      if (need) m_ref = mx;
      l *= alpha;
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) acc[jj] *= alpha;
    }
    const float m_use = m_ref == -INFINITY ? 0.0f : m_ref;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      float p[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        p[i] = fast_exp2(s[8 * ks + i] - m_use);
        l += p[i];
      }
      uint32_t ph[4], pl[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        ph[t] = pack_bf16(p[2 * t], p[2 * t + 1]);
        float h0f, h1f;
        bf16x2_to_f32(ph[t], h0f, h1f);
        pl[t] = pack_bf16(p[2 * t] - h0f, p[2 * t + 1] - h1f);
      }
      const bf16x8_t pop_hi = as_bf16x8(ph[0], ph[1], ph[2], ph[3]);
      const bf16x8_t pop_lo = as_bf16x8(pl[0], pl[1], pl[2], pl[3]);
      uint32_t vw[8][VW];
#pragma unroll
      for (int si = 0; si < 8; ++si) {
        if constexpr (!FP8) {
#pragma unroll
          for (int w = 0; w < VW; ++w) vw[si][w] = word(ch.v[8 * ks + si], w);
        } else {
#pragma unroll
          for (int w = 0; w < VW / 2; ++w) {
            const uint32_t x = word(ch.v[8 * ks + si], w);
            vw[si][2 * w] = fp8x2_to_bf16x2<false>(x);
            vw[si][2 * w + 1] = fp8x2_to_bf16x2<true>(x);
          }
        }
      }
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) {
        const int w = jj >> 1;
        const uint32_t sel = (jj & 1) ? 0x07060302u : 0x05040100u;
        uint32_t t4[4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
          t4[t] = __builtin_amdgcn_perm(vw[2 * t + 1][w], vw[2 * t][w], sel);
        const bf16x8_t vop = as_bf16x8(t4[0], t4[1], t4[2], t4[3]);
        acc[jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop_hi, acc[jj], 0, 0, 0);
        acc[jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop_lo, acc[jj], 0, 0, 0);
      }
    }
  };

  {
    Chunk A, B;
    int ci = wave;
    if (ci < n_ch) load(A, ci);
    for (; ci < n_ch; ci += 2 * NW) {
      if (ci + NW < n_ch) load(B, ci + NW);
      compute(A, ci);
      if (ci + NW >= n_ch) break;
      if (ci + 2 * NW < n_ch) load(A, ci + 2 * NW);
      compute(B, ci + NW);
    }
  }

  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  const float f = m_true == -INFINITY ? 0.0f : fast_exp2(m_ref - m_true);
  l *= f;
  if (g4 == 0) {
    sm_m[wave][c] = m_true;
    sm_l[wave][c] = l;
  }
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
    for (int i = 0; i < 4; ++i) sm_acc[wave][c][DPL * (4 * g4 + i) + jj] = acc[jj][i] * f;
  __syncthreads();

  const float vscale = FP8 ? a.v_scale[g] : 1.0f;
  for (int e = threadIdx.x; e < 16 * D; e += blockDim.x) {
    const int r = e / D;                               // tile row
    const int dd = e % D;
    const int rr = tile * 16 + r;
    if (rr >= rows) continue;
    const int ri = rr / G;
    const int64_t orow = (static_cast<int64_t>(b) * a.Q + ri) * a.n_q + g * G + rr % G;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w][r]);
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float fw = sm_m[w][r] == -INFINITY ? 0.0f : fast_exp2(sm_m[w][r] - M);
      L = fmaf(sm_l[w][r], fw, L);
      O = fmaf(sm_acc[w][r][dd], fw, O);
    }
    const bool live = ri < ql;
    const float o = live && L > 0.0f ? O / L * vscale : 0.0f;
    if (a.write_partials) {
      const int64_t mi = orow * a.P_max + j;
      if (dd == 0) {
        a.ws_m[mi] = M;
        a.ws_l[mi] = live ? L : 0.0f;
      }
      a.ws_o[mi * D + dd] = o;
    } else {
      const int64_t oi = orow * D + dd;
      if (a.out_dtype == PKV_FP32)
        static_cast<float*>(a.out)[oi] = o;
      else
        static_cast<uint16_t*>(a.out)[oi] = f32_to_bf16_rne(o);
    }
  }
}

constexpr int kMqWaves = 4;

template <int D, int BS, bool FP8>
static hipError_t launch_mq(const DecodeArgs& a, dim3 grid, hipStream_t s) {
  multi_query_partition_mfma<D, BS, FP8, kMqWaves><<<grid, kMqWaves * 64, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_multi_query_partition(const DecodeArgs& a, hipStream_t s) {
  const int G = a.n_q / a.n_kv;
  const int tiles = (a.Q * G + 15) / 16;
  const dim3 grid(a.n_kv * tiles, a.B, a.P_max);
  const bool fp8 = a.kv_dtype == PKV_FP8_E4M3;
  if (a.d == 128) {
    if (a.bs == 16) return fp8 ? launch_mq<128, 16, true>(a, grid, s)
                               : launch_mq<128, 16, false>(a, grid, s);
    return fp8 ? launch_mq<128, 32, true>(a, grid, s) : launch_mq<128, 32, false>(a, grid, s);
  }
  if (a.bs == 16) return fp8 ? launch_mq<64, 16, true>(a, grid, s)
                             : launch_mq<64, 16, false>(a, grid, s);
  return fp8 ? launch_mq<64, 32, true>(a, grid, s) : launch_mq<64, 32, false>(a, grid, s);
}

}  // namespace pkv

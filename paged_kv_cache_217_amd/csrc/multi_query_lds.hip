// Paged multi-query attention for many query rows per KV head (a prompt
// chunk: [LLMI] "LLM inference: prefill, decode, KV cache"
// (systemcraft.online), "4. Internal workings" and "9. Failure modes and
// limitations"), on the gfx950 matrix cores with the K/V chunk shared
// through LDS.
//
// Same arithmetic and outputs as multi_query_mfma.hip (query i of sequence b
// at position ctx - q_len + i attends causally to tokens 0..p through the
// block table; [MTKV] "Architecting Multi-Tier Disaggregated KV-Cache
// Hierarchies for Terabyte-Scale LLM Inference", "High-Throughput Paged
// Attention Kernel Integration"). There a wave streams K/V from HBM into its
// own registers, which suits a few rows per KV head. A 512-token chunk with
// 8 query heads per KV head has 4096 rows per KV head; each K/V byte then
// feeds thousands of rows and the work is a dense contraction, so here:
//  - a workgroup owns 128 rows (4 waves x 2 tiles of 16) of one KV head and
//    walks the context in chunks; each chunk is fetched once by the whole
//    workgroup (a wave fetches one 1 KiB slice of one (block, head) tile per
//    load) into an LDS double buffer and every wave reads it from there;
//  - the chunk sits in LDS as bf16: FP8 and FP4 codes are widened exactly
//    (scale 1) by the thread that writes them, once per chunk, so the inner
//    loop is the same for every format and holds no conversions (the
//    per-head scales go into the score scale and the output);
//  - LDS rows are padded (K by 16 bytes, V by 32), so the 16 lanes that read
//    the same 16-byte column of 16 consecutive tokens hit 16 different
//    4-bank groups, and every LDS address is one per-lane register plus an
//    immediate;
//  - each wave keeps its rows' softmax state and output in registers for the
//    whole context, so there is no merge between waves;
//  - the row groups of one (sequence, KV head) run on one XCD (blocks are
//    handed to the 8 XCDs round-robin), so the K/V they all read is fetched
//    into that XCD's L2 once.
// A second form at d = 128 (multi_query_lds_pp, below) takes 256 rows per
// workgroup and splits each chunk's work into a matrix phase and a vector
// phase that the two waves of a SIMD run in opposite order.
// In both, SPLIT_P false (PKV_BF16_WEIGHTS) feeds each weight to the P V
// products as one bf16 value instead of a bf16 head and tail: half the
// products with V, while the row sums keep the fp32 weights.
#include <float.h>

#include <type_traits>

#include "mfma_common.h"
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

using namespace mfma;

// One thread's piece of a chunk, stored into LDS as bf16: bf16 bytes as they
// are, FP8 or FP4 codes widened exactly (scale 1) into twice or four times
// the bytes (a zero code widens to +0).
template <int FMT, typename T>
__device__ __forceinline__ void store_bf16(uint8_t* dst, const T& w) {
  constexpr int NIN = sizeof(T) / 4;                  // input words
  constexpr int NOUT = FMT == kFmtBf16 ? NIN : FMT == kFmtFp8 ? 2 * NIN : 4 * NIN;
  static_assert(NOUT % 4 == 0, "whole 16-byte stores");
  uint32_t h[NOUT];
#pragma unroll
  for (int i = 0; i < NIN; ++i) {
    const uint32_t x = word(w, i);
    if constexpr (FMT == kFmtBf16) {
      h[i] = x;
    } else if constexpr (FMT == kFmtFp8) {
      h[2 * i] = fp8x2_to_bf16x2<false>(x);
      h[2 * i + 1] = fp8x2_to_bf16x2<true>(x);
    } else {
      h[4 * i] = fp4x2_to_bf16x2<0>(x);
      h[4 * i + 1] = fp4x2_to_bf16x2<1>(x);
      h[4 * i + 2] = fp4x2_to_bf16x2<2>(x);
      h[4 * i + 3] = fp4x2_to_bf16x2<3>(x);
    }
  }
#pragma unroll
  for (int q = 0; q < NOUT / 4; ++q)
    *reinterpret_cast<uint4*>(dst + 16 * q) =
        make_uint4(h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3]);
}

// w, or zeros where z holds, word by word (no select of whole vectors, which
// the compiler can route through scratch memory)
__device__ __forceinline__ uint4 zero_if(const uint4& w, bool z) {
  return make_uint4(z ? 0u : w.x, z ? 0u : w.y, z ? 0u : w.z, z ? 0u : w.w);
}
__device__ __forceinline__ uint2 zero_if(const uint2& w, bool z) {
  return make_uint2(z ? 0u : w.x, z ? 0u : w.y);
}

template <int D, int BS, int FMT, bool SPLIT_P = true>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void multi_query_lds_mfma(DecodeArgs a) {
  constexpr bool FP8 = FMT == kFmtFp8;
  constexpr bool FP4 = FMT == kFmtFp4;        // two E2M1 codes per byte, d = 128 only
  constexpr bool QNT = FMT != kFmtBf16;       // per-head scales
  constexpr int NW = 4;                       // waves
  constexpr int TPW = 2;                      // 16-row tiles per wave
  constexpr int GR = NW * TPW * 16;           // rows per workgroup
  constexpr int CT = 32;                      // tokens per chunk
  constexpr int NRG = CT / 16;                // 16-token row groups per chunk
  constexpr int NKS = CT / 32;                // 32-token PV k-steps per chunk
  constexpr int NKK = D / 32;                 // QK MFMA steps over d
  constexpr int NJ = D / 16;                  // PV MFMAs per k-step
  static_assert(!FP4 || D == 128, "FP4 is built for d = 128");
  constexpr int RB = 2 * D;                   // bytes per bf16 token row (LDS)
  constexpr int RBS = FP4 ? D / 2 : FP8 ? D : 2 * D;   // bytes per token row in the cache
  constexpr int LR = RB + 16;                 // padded LDS row of K
  // padded LDS row of V: V is read transposed, 4 rows of 32 bytes per 16
  // lanes, which a 32-byte pad puts on 32 different banks (a 16-byte pad
  // overlaps consecutive rows by 4 banks)
  constexpr int LRV = RB + 32;
  constexpr int CB = CT * RBS;                // cache bytes of K (or V) per chunk
  constexpr int LB = CT * LR;                 // LDS bytes of K per chunk
  constexpr int LBV = CT * LRV;               // LDS bytes of V per chunk
  constexpr int TB = BS * RBS;                // bytes of one (block, head) tile
  constexpr int PB = CB / 256 >= 16 ? 16 : CB / 256;   // bytes per thread piece
  constexpr int PIECES = CB / (PB * 256);     // pieces per thread
  using PT = typename Vec<PB>::T;
  static_assert(PIECES >= 1 && CB % (PB * 256) == 0, "chunk must split into thread pieces");
  static_assert(TB % (64 * PB) == 0, "a wave's slice of a chunk must lie in one tile");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15;
  const int g4 = lane >> 4;

  // grid: x = (KV head, group of GR rows), y = sequence, z = partition from
  // the end. Consecutive blocks go to different XCDs; when the x extent is a
  // multiple of 8 the index is permuted so that an XCD receives consecutive
  // work items, i.e. the row groups of one KV head.
  const int G = a.n_q / a.n_kv;
  const int rows = a.Q * G;
  const int groups = (rows + GR - 1) / GR;
  int wid = blockIdx.x;
  if (gridDim.x % 8 == 0) wid = (blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8;
  const int g = wid / groups;
  const int row0 = (wid % groups) * GR;
  const int b = blockIdx.y;
  const int j = gridDim.z - 1 - blockIdx.z;
  const int ctx = min(a.context_lens ? a.context_lens[b] : a.fixed_ctx, a.max_blocks * BS);
  // causal: query i of q_len sits at position ctx - q_len + i; non-causal
  // (a shared prefix read for many sequences' queries): every row sees all
  const int ql = a.non_causal ? (ctx > 0 ? a.Q : 0)
                              : max(0, min(min(a.query_lens[b], a.Q), ctx));
  auto qpos = [&](int i) -> int { return a.non_causal ? ctx - 1 : ctx - ql + i; };
  const int t0 = j * a.partition;

  // last position among rows [r0, r1), or -1 if none of them has a query
  auto last_pos = [&](int r0, int r1) -> int {
    const int i_hi = min((min(r1, rows) - 1) / G, ql - 1);
    return r0 / G < ql && r0 < rows ? qpos(i_hi) : -1;
  };
  const int p_grp = last_pos(row0, row0 + GR);
  if (t0 > p_grp) {
    // no row of this group reads this partition; a single pass still owes the
    // group's rows their zeros
    if (!a.write_partials && j == 0) {
      for (int e = threadIdx.x; e < GR * D; e += blockDim.x) {
        const int r = row0 + e / D;
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
  const int t1 = min(t0 + a.partition, p_grp + 1);   // tokens past the group's last are not read
  const int blk0 = t0 / BS;
  const int blk1 = (t1 + BS - 1) / BS;
  const int n_ch = (t1 - t0 + CT - 1) / CT;

  // this wave's rows
  const int wrow0 = row0 + wave * TPW * 16;
  const int p_lo = qpos(wrow0 / G);
  // dims of MFMA step kk used by lane (c, g4), as in the bf16 K rows in LDS
  auto dimbase = [&](int kk) -> int { return 32 * kk + 8 * g4; };
  bf16x8_t qop[TPW][NKK];
  int pos[TPW];
  // Scores stay unscaled (q . k) until the exponent, where 2^(s qscale - m)
  // is one fused multiply-add. That needs qscale > 0, so that the row maximum
  // of the unscaled scores is that of the scaled ones: a negative product is
  // made positive by negating Q (exact in bf16), a zero one by zeroing Q
  // (every score is then 0, as 0 . q . k would be).
  float qscale = a.scale * kLog2e;
  if constexpr (QNT) qscale *= a.k_scale[g];
  const uint32_t qflip = qscale < 0.0f ? 0x80008000u : 0u;
  const bool qzero = qscale == 0.0f;
  qscale = qzero ? 1.0f : fabsf(qscale);
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int row = wrow0 + 16 * t + c;
    const int qi = row / G;
    const bool live_row = row < rows && qi < ql && !qzero;
    pos[t] = qpos(qi);
    const int64_t qrow =
        live_row ? (static_cast<int64_t>(b) * a.Q + qi) * a.n_q + g * G + row % G : 0;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      uint4 w = *reinterpret_cast<const uint4*>(a.q + qrow * D + dimbase(kk));
      w = make_uint4(w.x ^ qflip, w.y ^ qflip, w.z ^ qflip, w.w ^ qflip);
      if (!live_row) w = make_uint4(0, 0, 0, 0);
      qop[t][kk] = __builtin_bit_cast(bf16x8_t, w);
    }
  }

  __shared__ __align__(16) uint8_t sk[4][LB];
  __shared__ __align__(16) uint8_t sv[4][LBV];

  // chunk ci into registers: piece e = threadIdx + 256 k is cache bytes
  // [PB e, PB e + PB) of the chunk; a wave's 64 pieces lie in one tile
  const int64_t tile_bytes = TB;
  const int64_t head_off = static_cast<int64_t>(g) * tile_bytes;
  const int64_t block_stride = static_cast<int64_t>(a.n_kv) * tile_bytes;
  const int32_t* bt = a.block_tables + static_cast<int64_t>(b) * a.max_blocks;
  // two register stage sets, filled together at the top of a step that
  // computes two chunks: a load has two chunks of compute to land
  struct Stage {
    PT k[PIECES], v[PIECES];
  };
  auto fetch = [&](Stage& st, int ci) {
#pragma unroll
    for (int k = 0; k < PIECES; ++k) {
      const int wbyte = (256 * k + 64 * wave) * PB;   // first byte of the wave's slice
      const int blk = blk0 + ci * (CT / BS) + wbyte / TB;
      const bool have = blk < blk1;
      int p = __builtin_amdgcn_readfirstlane(have ? bt[blk] : 0);
      if (p < 0 || p >= a.num_blocks) p = 0;
      const int bytes = have ? TB : 0;                // absent: loads give 0
      const uint32_t off = static_cast<uint32_t>(wbyte % TB + PB * lane);
      ld_stream(st.k[k], tile_rsrc(a.k_cache + p * block_stride + head_off, bytes), off, 0);
      ld_stream(st.v[k], tile_rsrc(a.v_cache + p * block_stride + head_off, bytes), off, 0);
    }
  };
  // into LDS as bf16. V slots past t1 may hold anything (NaN in a tail
  // block): they are zeroed here, once per chunk, so that P = 0 times them
  // gives 0. K needs nothing: the scores of those slots are replaced by -inf.
  auto commit = [&](Stage& st, int buf, int ci) {
    const int tok0 = t0 + ci * CT;
#pragma unroll
    for (int k = 0; k < PIECES; ++k) {
      if constexpr (FMT == kFmtBf16) {
        // 16 bytes of bf16 at bytes 16 e of the chunk, stored as loaded
        const int e = threadIdx.x + 256 * k;
        if (tok0 + CT > t1 && tok0 + (16 * e) / RB >= t1) st.v[k] = make_uint4(0, 0, 0, 0);
        const int row = (16 * e) / RB, col = (16 * e) % RB;
        *reinterpret_cast<uint4*>(&sk[buf][row * LR + col]) = st.k[k];
        *reinterpret_cast<uint4*>(&sv[buf][row * LRV + col]) = st.v[k];
      } else {
        const int src = PB * (threadIdx.x + 256 * k);   // cache byte within the chunk
        const int row = src / RBS;
        const int col = (src % RBS) * (RB / RBS);       // its bf16 byte within the row
        if (tok0 + CT > t1 && tok0 + row >= t1) st.v[k] = PT{};
        store_bf16<FMT>(&sk[buf][row * LR + col], st.k[k]);
        store_bf16<FMT>(&sv[buf][row * LRV + col], st.v[k]);
      }
    }
  };

  float m_ref[TPW], m_raw[TPW], l[TPW];
  f32x4_t acc[TPW][NJ];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    m_ref[t] = -INFINITY;
    m_raw[t] = -INFINITY;
    l[t] = 0.0f;
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) acc[t][jj] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }

  // per-lane LDS offsets: K token c at dims of lane group g4; V is read
  // transposed: lane (c, g4) addresses token 4 g4 + c / 4, dims 4 (c % 4) ..
  // of a 16-dim column block
  const int k_lane = c * LR + 16 * g4;
  const int v_tr = (4 * g4 + c / 4) * LRV + 8 * (c % 4);
  // A step's chunks go through three phases: the scores of every chunk (K Q^T
  // on the matrix cores, masked), one lazy-rescale check over all of them,
  // then the weights and P V of each chunk. With the rare rescale branch out
  // of the way, the weights of one chunk and the P V products of the other
  // are in one basic block, where the compiler can pair vector instructions
  // with matrix-core work.
  auto scores = [&](int buf, int ci, float (&s)[TPW][4 * NRG]) {
    const uint8_t* kl_ = sk[buf];
    const int tok0 = t0 + ci * CT;
    // K Q^T for every (row group, tile): kk outermost so that the NRG x TPW
    // accumulation chains interleave
    f32x4_t sc[NRG][TPW];
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg)
#pragma unroll
      for (int t = 0; t < TPW; ++t) sc[rg][t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
      for (int rg = 0; rg < NRG; ++rg) {
        const uint8_t* kt = kl_ + k_lane + 16 * rg * LR;   // this lane's K token 16 rg + c
        const bf16x8_t kop =
            __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(kt + 64 * kk));
#pragma unroll
        for (int t = 0; t < TPW; ++t)
          sc[rg][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[t][kk], sc[rg][t], 0, 0, 0);
      }
    }
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg)
#pragma unroll
      for (int t = 0; t < TPW; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[t][4 * rg + i] = sc[rg][t][i];
    if (tok0 + CT > min(p_lo + 1, t1)) {
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int lim = min(pos[t] + 1, t1);
#pragma unroll
        for (int rg = 0; rg < NRG; ++rg)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (tok0 + 16 * rg + 4 * g4 + i >= lim) s[t][4 * rg + i] = -INFINITY;
      }
    }
  };

  // Lazy rescaling, checked per lane: the row's reference m_ref only has to
  // stay within 2^8 of every weight, so each lane compares the largest of its
  // own scores (of all the step's chunks) with it, and the row maximum (a
  // cross-lane reduction) is taken only in the rare step where some lane
  // exceeds it. The true maximum is kept per lane (raw q . k units) and
  // reduced once at the end.
  auto rescale = [&](auto NC, float (&s)[decltype(NC)::value][TPW][4 * NRG]) {
    constexpr int N = decltype(NC)::value;
    float lmax[TPW];
    bool need_any = false;
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      float mx = s[0][t][0];
#pragma unroll
      for (int n = 0; n < N; ++n)
#pragma unroll
        for (int i = (n == 0 ? 1 : 0); i < 4 * NRG; ++i) mx = vmax(mx, s[n][t][i]);
      lmax[t] = mx;
      m_raw[t] = vmax(m_raw[t], mx);
      need_any |= mx * qscale > m_ref[t] + kLazyRescale;
    }
    if (__builtin_amdgcn_ballot_w64(need_any) != 0) {
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const float mx = max_xor32(max_xor16(lmax[t])) * qscale;   // the row's, base-2 units
        const bool need = mx > m_ref[t] + kLazyRescale;
        const float alpha = need ? fast_exp2(m_ref[t] - mx) : 1.0f;
        if (need) m_ref[t] = mx;
        l[t] *= alpha;
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj) acc[t][jj] *= alpha;
      }
    }
  };

  auto accumulate = [&](int buf, const float (&s)[TPW][4 * NRG]) {
    const uint8_t* vl_ = sv[buf];
    float m_use[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) m_use[t] = m_ref[t] == -INFINITY ? 0.0f : m_ref[t];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      bf16x8_t pop_hi[TPW], pop_lo[TPW];
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        float p[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          p[i] = fast_exp2(fmaf(s[t][8 * ks + i], qscale, -m_use[t]));
          l[t] += p[i];
        }
        uint32_t ph[4], pl[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if constexpr (SPLIT_P) {
            const Bf16Split sp = split_bf16(p[2 * u], p[2 * u + 1]);
            ph[u] = sp.hi;
            pl[u] = sp.lo;
          } else {
            ph[u] = pack_bf16(p[2 * u], p[2 * u + 1]);
            pl[u] = 0u;
          }
        }
        pop_hi[t] = as_bf16x8(ph[0], ph[1], ph[2], ph[3]);
        pop_lo[t] = as_bf16x8(pl[0], pl[1], pl[2], pl[3]);
      }
      // V^T operand of dims 16 jj ..: tokens 4 g4 .. (first half) and
      // 16 + 4 g4 .. (second half) of the k-step, straight from LDS
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) {
        const uint8_t* vt = vl_ + v_tr + 32 * ks * LRV + 32 * jj;
        const uint2 v0 = lds_read_tr16(vt);
        const uint2 v1 = lds_read_tr16(vt + 16 * LRV);
        const bf16x8_t vop = as_bf16x8(v0.x, v0.y, v1.x, v1.y);
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
          acc[t][jj] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop_hi[t], acc[t][jj], 0, 0, 0);
          if constexpr (SPLIT_P)
            acc[t][jj] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop_lo[t], acc[t][jj], 0, 0, 0);
        }
      }
    }
  };

  // walk in steps of two chunks: LDS buffers 2h, 2h + 1 (h = step % 2) hold
  // chunks ci, ci + 1 while ci + 2, ci + 3 arrive in the stage registers and
  // are then written to the other pair, which was last read in the previous
  // step, before the barrier that ended it
  {
    Stage sa, sb;
    fetch(sa, 0);
    if (n_ch > 1) fetch(sb, 1);
    commit(sa, 0, 0);
    if (n_ch > 1) commit(sb, 1, 1);
    __syncthreads();
    for (int ci = 0, h = 0; ci < n_ch; ci += 2, h ^= 1) {
      const bool more = ci + 2 < n_ch;
      if (more) fetch(sa, ci + 2);
      if (ci + 3 < n_ch) fetch(sb, ci + 3);
      const bool two = ci + 1 < n_ch;
      float sa_[1][TPW][4 * NRG], sb_[1][TPW][4 * NRG];
      scores(2 * h, ci, sa_[0]);
      rescale(std::integral_constant<int, 1>{}, sa_);
      // the second chunk's scores are issued beside the first chunk's
      // weights and P V products (one basic block)
      if (two) scores(2 * h + 1, ci + 1, sb_[0]);
      accumulate(2 * h, sa_[0]);
      if (two) {
        rescale(std::integral_constant<int, 1>{}, sb_);
        accumulate(2 * h + 1, sb_[0]);
      }
      if (more) commit(sa, 2 * (h ^ 1), ci + 2);
      if (ci + 3 < n_ch) commit(sb, 2 * (h ^ 1) + 1, ci + 3);
      __syncthreads();
    }
  }

  // outputs: lane (c, g4) holds, of row 16 t + c, dims 16 jj + 4 g4 + i
  auto odim = [&](int jj, int i) -> int { return 16 * jj + 4 * g4 + i; };
  const float vscale = QNT ? a.v_scale[g] : 1.0f;
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    float lt = l[t];
    lt = sum_xor32(sum_xor16(lt));
    const float m_true = max_xor32(max_xor16(m_raw[t])) * qscale;   // the row's true maximum
    const float f = m_true == -INFINITY ? 0.0f : fast_exp2(m_ref[t] - m_true);
    const float L = lt * f;
    const int rr = wrow0 + 16 * t + c;
    if (rr >= rows) continue;
    const int ri = rr / G;
    const bool live = ri < ql;
    const int64_t orow = (static_cast<int64_t>(b) * a.Q + ri) * a.n_q + g * G + rr % G;
    const float inv = live && L > 0.0f ? f * vscale / L : 0.0f;
    if (a.write_partials) {
      const int64_t mi = orow * a.P_max + j;
      if (g4 == 0) {
        a.ws_m[mi] = m_true;
        a.ws_l[mi] = live ? L : 0.0f;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj)
          a.ws_o[mi * D + odim(jj, i)] = acc[t][jj][i] * inv;
    } else if (a.out_dtype == PKV_FP32) {
      float* o = static_cast<float*>(a.out) + orow * D;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj) o[odim(jj, i)] = acc[t][jj][i] * inv;
    } else {
      uint16_t* o = static_cast<uint16_t*>(a.out) + orow * D;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj)
          o[odim(jj, i)] = f32_to_bf16_rne(acc[t][jj][i] * inv);
    }
  }
}

// Ping-pong form of the kernel above, for d = 128 with 256 or more rows per KV
// head. Two waves share each SIMD; in the form above they
// belong to different workgroups, drift into the same phase and take turns
// on the matrix core and the vector ALU rather than using both at once. Here
// a workgroup has 8 waves (256 rows), so one workgroup fills a CU with two
// waves per SIMD, and the two waves of a SIMD take opposite roles. The work
// on a 64-token chunk is split into a matrix phase (the previous chunk's
// P V products, then this chunk's K Q^T) and a vector phase (masks, the
// rescale check, the weights and their bf16 head/tail split), and the second
// role runs one phase behind the first. Every phase ends at a workgroup
// barrier, so while one wave of a SIMD issues products the other computes
// weights. The role is taken per SIMD from an LDS counter (the first wave of
// a SIMD to arrive leads); every wave runs the same code and the same number
// of barriers, so the roles only decide timing, never the result.
//
// LDS: K and V of a chunk are held in separate two-deep rings as bf16, rows
// padded by 32 bytes (K and V both: no bank conflicts left, measured). FP8 and
// FP4 codes are widened exactly to bf16 by the thread that writes them into
// LDS, once per chunk, so the matrix phase is the same for every format and
// holds no conversions (the per-head scales go into the score scale and the
// output, as in the kernel above). K of chunk n is
// read in phases 2n, 2n + 1 (scores) and V of chunk n in phases 2n + 2,
// 2n + 3 (its P V products, one phase later than its weights); at the start
// of phase 2k the workgroup writes K of chunk k + 1 and V of chunk k from
// registers loaded two phases earlier. In the matrix phase the LDS reads are
// interleaved with the products (a dozen reads ahead, then one read per two
// products), so that the reads' latency is covered.
//
// SPLIT_P false: 64 products per matrix phase instead of 96.

template <int BS, int FMT, bool SPLIT_P = true>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void multi_query_lds_pp(DecodeArgs a) {
  constexpr int D = 128;
  constexpr bool FP8 = FMT == kFmtFp8;
  constexpr bool FP4 = FMT == kFmtFp4;
  constexpr bool QNT = FMT != kFmtBf16;       // per-head scales
  constexpr int NW = 8;                       // waves
  constexpr int NT = NW * 64;                 // threads
  constexpr int TPW = 2;                      // 16-row tiles per wave
  constexpr int GR = NW * TPW * 16;           // rows per workgroup
  constexpr int CT = 64;                      // tokens per chunk
  constexpr int NRG = CT / 16;                // 16-token row groups per chunk
  constexpr int NKS = CT / 32;                // 32-token PV k-steps per chunk
  constexpr int NKK = D / 32;                 // QK MFMA steps over d
  constexpr int NJ = D / 16;                  // PV MFMAs per k-step
  constexpr int RB = 2 * D;                   // bytes per bf16 token row (LDS)
  constexpr int LR = RB + 32;                 // padded LDS row (K and V)
  constexpr int RBS = FP4 ? D / 2 : FP8 ? D : 2 * D;   // bytes per token row in the cache
  constexpr int CB = CT * RBS;                // cache bytes of K (or V) per chunk
  constexpr int TB = BS * RBS;                // bytes of one (block, head) tile
  constexpr int PB = FP4 ? 8 : 16;            // bytes of one piece (16 elements for FP8/FP4)
  constexpr int PIECES = CB / (PB * NT);      // pieces of a chunk's K per thread
  using VT = typename Vec<PB>::T;
  static_assert(PIECES >= 1 && CB % (PB * NT) == 0, "chunk must split into thread pieces");
  static_assert(TB % (64 * PB) == 0, "a wave's slice of a chunk must lie in one tile");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15;
  const int g4 = lane >> 4;

  // grid as for the kernel above, GR rows per workgroup
  const int G = a.n_q / a.n_kv;
  const int rows = a.Q * G;
  const int groups = (rows + GR - 1) / GR;
  int wid = blockIdx.x;
  if (gridDim.x % 8 == 0) wid = (blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8;
  const int g = wid / groups;
  const int row0 = (wid % groups) * GR;
  const int b = blockIdx.y;
  const int j = gridDim.z - 1 - blockIdx.z;
  const int ctx = min(a.context_lens ? a.context_lens[b] : a.fixed_ctx, a.max_blocks * BS);
  const int ql = a.non_causal ? (ctx > 0 ? a.Q : 0)
                              : max(0, min(min(a.query_lens[b], a.Q), ctx));
  auto qpos = [&](int i) -> int { return a.non_causal ? ctx - 1 : ctx - ql + i; };
  const int t0 = j * a.partition;
  auto last_pos = [&](int r0, int r1) -> int {
    const int i_hi = min((min(r1, rows) - 1) / G, ql - 1);
    return r0 / G < ql && r0 < rows ? qpos(i_hi) : -1;
  };
  const int p_grp = last_pos(row0, row0 + GR);
  if (t0 > p_grp) {                           // the whole workgroup leaves here
    if (!a.write_partials && j == 0) {
      for (int e = threadIdx.x; e < GR * D; e += blockDim.x) {
        const int r = row0 + e / D;
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
  const int t1 = min(t0 + a.partition, p_grp + 1);
  const int blk0 = t0 / BS;
  const int blk1 = (t1 + BS - 1) / BS;
  const int n_ch = (t1 - t0 + CT - 1) / CT;

  // role: 0 for the first wave of its SIMD to get here, 1 for the second
  __shared__ int simd_count[4];
  if (threadIdx.x < 4) simd_count[threadIdx.x] = 0;
  __syncthreads();
  int role;
  {
    // HW_ID bits 5:4 are the wave's SIMD
    const int simd = __builtin_amdgcn_s_getreg((1 << 11) | (4 << 6) | 4) & 3;
    int r = 0;
    if (lane == 0) r = atomicAdd(&simd_count[simd], 1);
    role = __builtin_amdgcn_readfirstlane(r) & 1;
  }

  // this wave's rows and their Q^T operands, as in the kernel above
  const int wrow0 = row0 + wave * TPW * 16;
  const int p_lo = qpos(wrow0 / G);
  bf16x8_t qop[TPW][NKK];
  int pos[TPW];
  float qscale = a.scale * kLog2e;
  if constexpr (QNT) qscale *= a.k_scale[g];
  const uint32_t qflip = qscale < 0.0f ? 0x80008000u : 0u;
  const bool qzero = qscale == 0.0f;
  qscale = qzero ? 1.0f : fabsf(qscale);
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int row = wrow0 + 16 * t + c;
    const int qi = row / G;
    const bool live_row = row < rows && qi < ql && !qzero;
    pos[t] = qpos(qi);
    const int64_t qrow =
        live_row ? (static_cast<int64_t>(b) * a.Q + qi) * a.n_q + g * G + row % G : 0;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      uint4 w = *reinterpret_cast<const uint4*>(a.q + qrow * D + 32 * kk + 8 * g4);
      w = make_uint4(w.x ^ qflip, w.y ^ qflip, w.z ^ qflip, w.w ^ qflip);
      if (!live_row) w = make_uint4(0, 0, 0, 0);
      qop[t][kk] = __builtin_bit_cast(bf16x8_t, w);
    }
  }

  __shared__ __align__(16) uint8_t sk[2][CT * LR];
  __shared__ __align__(16) uint8_t sv[2][CT * LR];

  const int64_t tile_bytes = TB;
  const int64_t head_off = static_cast<int64_t>(g) * tile_bytes;
  const int64_t block_stride = static_cast<int64_t>(a.n_kv) * tile_bytes;
  const int32_t* bt = a.block_tables + static_cast<int64_t>(b) * a.max_blocks;
  // Piece e = threadIdx + NT x of a chunk's K (or V) is cache bytes [PB e,
  // PB e + PB); a wave's 64 pieces lie in one tile. A chunk past the partition reads
  // nothing (its blocks get size-0 resources), so every fetch is issued
  // unconditionally and the outstanding-load count is the same in every phase.
  // The physical blocks of a fetch are resolved a phase ahead, in a vector
  // phase: a scalar load in flight would make every LDS wait of the matrix
  // phase a wait for all of them.
  using Piece = VT[PIECES];
  using Blocks = int[PIECES];
  auto resolve = [&](Blocks& pb, int ci) __attribute__((always_inline)) {
#pragma unroll
    for (int x = 0; x < PIECES; ++x) {
      const int blk = blk0 + ci * (CT / BS) + (PB * (NT * x + 64 * wave)) / TB;
      int p = ld_uniform(bt + min(blk, blk1 - 1));    // always a valid entry
      if (blk >= blk1 || p < 0 || p >= a.num_blocks) p = 0;
      pb[x] = p;
    }
  };
  auto fetch = [&](Piece& out, const uint8_t* cache, int ci, const Blocks& pb)
                   __attribute__((always_inline)) {
#pragma unroll
    for (int x = 0; x < PIECES; ++x) {
      const int wbyte = PB * (NT * x + 64 * wave);
      const bool have = blk0 + ci * (CT / BS) + wbyte / TB < blk1;
      ld_stream(out[x], tile_rsrc(cache + pb[x] * block_stride + head_off, have ? TB : 0),
                static_cast<uint32_t>(wbyte % TB + PB * lane), 0);
    }
  };
  // piece x of this thread: its token row within the chunk and its LDS offset
  auto st_row = [&](int x) -> int { return (PB * (threadIdx.x + NT * x)) / RBS; };
  auto st_off = [&](int x) -> int {
    const int byte = (PB * (threadIdx.x + NT * x)) % RBS;       // cache byte within the row
    return st_row(x) * LR + (FP4 ? 4 * byte : FP8 ? 2 * byte : byte);
  };
  // into LDS as bf16 (store_bf16); V slots past t1 may hold anything (NaN in
  // a tail block) and are zeroed so that P = 0 times them gives 0. K needs
  // nothing: those scores become -inf.
  auto commit_k = [&](const Piece& w, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int x = 0; x < PIECES; ++x) store_bf16<FMT>(&sk[buf][st_off(x)], w[x]);
  };
  auto commit_v = [&](const Piece& w, int buf, int ci) __attribute__((always_inline)) {
#pragma unroll
    for (int x = 0; x < PIECES; ++x)
      store_bf16<FMT>(&sv[buf][st_off(x)], zero_if(w[x], t0 + ci * CT + st_row(x) >= t1));
  };

  float m_ref[TPW], m_raw[TPW], l[TPW];
  f32x4_t acc[TPW][NJ];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    m_ref[t] = -INFINITY;
    m_raw[t] = -INFINITY;
    l[t] = 0.0f;
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) acc[t][jj] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }
  // per-lane LDS offsets: K token c at dims of lane group g4; V read
  // transposed, lane (c, g4) addressing token 4 g4 + c / 4, dims 4 (c % 4) ..
  // of a 16-dim column block
  const int k_lane = c * LR + 16 * g4;
  const int v_tr = (4 * g4 + c / 4) * LR + 8 * (c % 4);

  // carried between phases: the scores of the chunk whose weights come next
  // and the weights (bf16 head and tail) of the chunk whose products come next
  float s[TPW][4 * NRG];
  bf16x8_t pop_hi[TPW][NKS], pop_lo[TPW][NKS];
  // A phase's results are taken as read by an empty volatile asm at its end.
  // Arithmetic is otherwise free to move across a barrier, and the compiler
  // does sink the weights into the next phase, beside their products, which
  // would undo the split into phases.
  auto pin_scores = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int i = 0; i < 4 * NRG; ++i) asm volatile("" : "+v"(s[t][i]));
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) asm volatile("" : "+v"(acc[t][jj]));
  };
  auto pin_weights = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        asm volatile("" : "+v"(pop_hi[t][ks]));
        if constexpr (SPLIT_P) asm volatile("" : "+v"(pop_lo[t][ks]));
      }
      asm volatile("" : "+v"(l[t]));
    }
  };

  // matrix phase: products of P with the V buffer vb, then K Q^T of the K
  // buffer kb into s
  auto pv = [&](int vb) __attribute__((always_inline)) {
    const uint8_t* vl_ = sv[vb];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) {
        // V^T operand of dims 16 jj ..: tokens 4 g4 .. and 16 + 4 g4 .. of
        // the k-step
        const uint8_t* vt = vl_ + v_tr + 32 * ks * LR + 32 * jj;
        const uint2 v0 = lds_read_tr16(vt);
        const uint2 v1 = lds_read_tr16(vt + 16 * LR);
        const bf16x8_t vop = as_bf16x8(v0.x, v0.y, v1.x, v1.y);
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
          acc[t][jj] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop_hi[t][ks], acc[t][jj], 0, 0, 0);
          if constexpr (SPLIT_P)
            acc[t][jj] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop_lo[t][ks], acc[t][jj], 0, 0, 0);
        }
      }
    }
  };
  auto qk = [&](int kb) __attribute__((always_inline)) {
    const uint8_t* kl_ = sk[kb];
    f32x4_t sc[NRG][TPW];
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg)
#pragma unroll
      for (int t = 0; t < TPW; ++t) sc[rg][t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
      for (int rg = 0; rg < NRG; ++rg) {
        const bf16x8_t kop = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const uint4*>(kl_ + k_lane + 16 * rg * LR + 64 * kk));
#pragma unroll
        for (int t = 0; t < TPW; ++t)
          sc[rg][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[t][kk], sc[rg][t], 0, 0, 0);
      }
    }
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg)
#pragma unroll
      for (int t = 0; t < TPW; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[t][4 * rg + i] = sc[rg][t][i];
  };
  // the matrix phase's order: 12 LDS reads, then one read per two products
  // (48 reads and 96 products in all; one read per product and 64 products
  // with single bf16 weights). bf16 writes its share of the next
  // chunks into LDS first; FP8 and FP4 write (and widen) theirs after the
  // products, where the widening overlaps the last products and the wait for
  // the staged loads comes later (2-4% faster than first, measured; bf16 1%
  // slower there).
  auto matrix_order = [&]() __attribute__((always_inline)) {
    constexpr int MPR = SPLIT_P ? 2 : 1;      // products per LDS read in the middle
    constexpr int NMF = SPLIT_P ? 96 : 64;    // products per phase
    if constexpr (FMT == kFmtBf16) __builtin_amdgcn_sched_group_barrier(0x200, 2 * PIECES, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
#pragma unroll
    for (int i = 0; i < 36; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, MPR, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NMF - 36 * MPR, 0);
    if constexpr (FMT != kFmtBf16) {
      __builtin_amdgcn_sched_group_barrier(0x200, 4 * PIECES, 0);   // two 16-byte stores a piece
      __builtin_amdgcn_sched_group_barrier(0x020, 2 * PIECES, 0);
    }
  };

  // vector phase for chunk n: masks, the lazy-rescale check (as in the kernel
  // above), then the weights, split into bf16 head and tail
  auto weights = [&](int n) __attribute__((always_inline)) {
    const int tok0 = t0 + n * CT;
    if (tok0 + CT > min(p_lo + 1, t1)) {
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int lim = min(pos[t] + 1, t1);
#pragma unroll
        for (int rg = 0; rg < NRG; ++rg)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (tok0 + 16 * rg + 4 * g4 + i >= lim) s[t][4 * rg + i] = -INFINITY;
      }
    }
    float lmax[TPW];
    bool need_any = false;
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      float mx = s[t][0];
#pragma unroll
      for (int i = 1; i < 4 * NRG; ++i) mx = vmax(mx, s[t][i]);
      lmax[t] = mx;
      m_raw[t] = vmax(m_raw[t], mx);
      need_any |= mx * qscale > m_ref[t] + kLazyRescale;
    }
    if (__builtin_amdgcn_ballot_w64(need_any) != 0) {
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const float mx = max_xor32(max_xor16(lmax[t])) * qscale;
        const bool need = mx > m_ref[t] + kLazyRescale;
        const float alpha = need ? fast_exp2(m_ref[t] - mx) : 1.0f;
        if (need) m_ref[t] = mx;
        l[t] *= alpha;
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj) acc[t][jj] *= alpha;
      }
    }
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const float m_use = m_ref[t] == -INFINITY ? 0.0f : m_ref[t];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        float p[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          p[i] = fast_exp2(fmaf(s[t][8 * ks + i], qscale, -m_use));
          l[t] += p[i];
        }
        uint32_t ph[4], pl[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if constexpr (SPLIT_P) {
            const Bf16Split sp = split_bf16(p[2 * u], p[2 * u + 1]);
            ph[u] = sp.hi;
            pl[u] = sp.lo;
          } else {
            ph[u] = pack_bf16(p[2 * u], p[2 * u + 1]);
            pl[u] = 0;
          }
        }
        pop_hi[t][ks] = as_bf16x8(ph[0], ph[1], ph[2], ph[3]);
        pop_lo[t][ks] = as_bf16x8(pl[0], pl[1], pl[2], pl[3]);
      }
    }
  };

  // A wave's phases are M0 W0 M1 W1 ... W(N-1) MN, where Mk is the products
  // of chunk k - 1 (k >= 1) and the scores of chunk k (k < N), and Wk the
  // weights of chunk k; each phase ends at a barrier. Role 1 passes one
  // barrier before its first phase and role 0 one after its last, so role 1
  // runs one phase behind: while one wave of a SIMD is in Mk the other is in
  // W(k-1) or Wk. Both roles run the same code. Those two extra barriers sit
  // under a condition that is uniform within a wave but not across the
  // workgroup: s_barrier counts one arrival per wave, whatever instruction it
  // is reached at, and every wave reaches the same number of barriers
  // (2 N + 3 after the role set-up), so each barrier releases all 8 waves.
  //
  // K of chunk n sits in sk[n % 2] and V of chunk n in sv[n % 2]. A wave
  // writes its slice of K of chunk k + 1 and of V of chunk k during Mk (bf16
  // at its start, FP8 and FP4 after its products). With the lag, K of chunk
  // k is complete one phase before role 0 reads it and V of chunk k one phase
  // before role 0's M(k+1), and neither overwrites a buffer before role 1's
  // last read of its previous contents (K of chunk N, written by M(N-1), is
  // zeros that nobody reads). The staged registers are refilled right after
  // they are written out, so a load has a whole step (two phases) to land.
  // The first and last phases are peeled so that the loop's phases have no
  // branches around their products.
  {
    const int N = n_ch;                       // >= 1
    Piece stk, stv;             // staged K of chunk k + 1 and V of chunk k
    Blocks bk, bv;              // blocks of the next K and V fetches
    resolve(bk, 0);
    fetch(stv, a.k_cache, 0, bk);             // K of chunk 0, through stv
    resolve(bk, 1);
    fetch(stk, a.k_cache, 1, bk);
    commit_k(stv, 0);
    resolve(bv, 0);
    fetch(stv, a.v_cache, 0, bv);
    resolve(bk, 2);
    resolve(bv, 1);
    __syncthreads();
    if (role == 1) __syncthreads();
    // M0, W0
    commit_k(stk, 1);
    commit_v(stv, 0, 0);
    fetch(stk, a.k_cache, 2, bk);
    fetch(stv, a.v_cache, 1, bv);
    qk(0);
    pin_scores();
    __syncthreads();
    weights(0);
    resolve(bk, 3);
    resolve(bv, 2);
    pin_weights();
    __syncthreads();
    // Mk and Wk for 1 <= k < N: write K of chunk k + 1 and V of chunk k, fetch
    // K of chunk k + 2 and V of chunk k + 1 into the registers just freed,
    // then the products; the weights, then the blocks of the next fetches
    for (int k = 1; k < N; ++k) {
      const int par = k & 1;
      if constexpr (FMT == kFmtBf16) {
        commit_k(stk, par ^ 1);
        commit_v(stv, par, k);
        fetch(stk, a.k_cache, k + 2, bk);
        fetch(stv, a.v_cache, k + 1, bv);
      }
      pv(par ^ 1);
      qk(par);
      if constexpr (FMT != kFmtBf16) {
        commit_k(stk, par ^ 1);
        commit_v(stv, par, k);
        fetch(stk, a.k_cache, k + 2, bk);
        fetch(stv, a.v_cache, k + 1, bv);
      }
      matrix_order();
      pin_scores();
      __syncthreads();
      weights(k);
      resolve(bk, k + 3);
      resolve(bv, k + 2);
      pin_weights();
      __syncthreads();
    }
    // MN: the last chunk's products (V of chunk N - 1 in sv[(N - 1) % 2])
    pv((N - 1) & 1);
    __syncthreads();
    if (role == 0) __syncthreads();
  }

  // outputs as in the kernel above: lane (c, g4) holds, of row 16 t + c, dims
  // 16 jj + 4 g4 + i
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    float lt = l[t];
    lt = sum_xor32(sum_xor16(lt));
    const float m_true = max_xor32(max_xor16(m_raw[t])) * qscale;
    const float f = m_true == -INFINITY ? 0.0f : fast_exp2(m_ref[t] - m_true);
    const float L = lt * f;
    const int rr = wrow0 + 16 * t + c;
    if (rr >= rows) continue;
    const int ri = rr / G;
    const bool live = ri < ql;
    const int64_t orow = (static_cast<int64_t>(b) * a.Q + ri) * a.n_q + g * G + rr % G;
    const float vscale = QNT ? a.v_scale[g] : 1.0f;
    const float inv = live && L > 0.0f ? f * vscale / L : 0.0f;
    if (a.write_partials) {
      const int64_t mi = orow * a.P_max + j;
      if (g4 == 0) {
        a.ws_m[mi] = m_true;
        a.ws_l[mi] = live ? L : 0.0f;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj)
          a.ws_o[mi * D + 16 * jj + 4 * g4 + i] = acc[t][jj][i] * inv;
    } else if (a.out_dtype == PKV_FP32) {
      float* o = static_cast<float*>(a.out) + orow * D;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj) o[16 * jj + 4 * g4 + i] = acc[t][jj][i] * inv;
    } else {
      uint16_t* o = static_cast<uint16_t*>(a.out) + orow * D;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj)
          o[16 * jj + 4 * g4 + i] = f32_to_bf16_rne(acc[t][jj][i] * inv);
    }
  }
}

template <int D, int BS, int FMT>
static hipError_t launch_lds(const DecodeArgs& a, hipStream_t s) {
  const int rows = a.Q * (a.n_q / a.n_kv);
  if constexpr (D == 128) {
    // the ping-pong form unless its 256-row workgroups pad the rows by more
    // than a tenth beyond what 128-row ones do (its ~10% speed-up per row is
    // then lost: 320 rows, padded to 512 instead of 384, measured slower)
    const int groups = (rows + 255) / 256;
    if (rows >= 256 && 10 * (2 * groups) <= 11 * ((rows + 127) / 128)) {
      const dim3 grid(a.n_kv * groups, a.B, a.P_max);
      if (a.bf16_weights)
        multi_query_lds_pp<BS, FMT, false><<<grid, 512, 0, s>>>(a);
      else
        multi_query_lds_pp<BS, FMT, true><<<grid, 512, 0, s>>>(a);
      return hipGetLastError();
    }
  }
  const int groups = (rows + 127) / 128;
  const dim3 grid(a.n_kv * groups, a.B, a.P_max);
  if (a.bf16_weights)
    multi_query_lds_mfma<D, BS, FMT, false><<<grid, 256, 0, s>>>(a);
  else
    multi_query_lds_mfma<D, BS, FMT, true><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

template <int D, int BS>
static hipError_t launch_lds_fmt(const DecodeArgs& a, hipStream_t s) {
  if (a.kv_dtype == PKV_FP8_E4M3) return launch_lds<D, BS, kFmtFp8>(a, s);
  if constexpr (D == 128)
    if (a.kv_dtype == PKV_FP4_E2M1) return launch_lds<D, BS, kFmtFp4>(a, s);
  if (a.kv_dtype != PKV_BF16) return hipErrorInvalidValue;
  return launch_lds<D, BS, kFmtBf16>(a, s);
}

hipError_t launch_multi_query_lds(const DecodeArgs& a, hipStream_t s) {
  if (a.d == 128) return a.bs == 16 ? launch_lds_fmt<128, 16>(a, s) : launch_lds_fmt<128, 32>(a, s);
  return a.bs == 16 ? launch_lds_fmt<64, 16>(a, s) : launch_lds_fmt<64, 32>(a, s);
}

}  // namespace pkv

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

// Each wave owns TPW row tiles and applies every K operand and transposed V
// operand it loads to all of them; R such waves share a workgroup, S waves
// (chunk streams) per tile set. The R waves of one stream read the same K/V
// chunk at the same time, so a KV head's context crosses HBM once for all of
// the group's tiles.
template <int D, int BS, int FMT, int TPW, int R, int S>
__global__ __launch_bounds__(R * S * 64) __attribute__((amdgpu_waves_per_eu(2)))
void multi_query_partition_mfma(DecodeArgs a) {
  constexpr bool FP8 = FMT == kFmtFp8;
  constexpr bool FP4 = FMT == kFmtFp4;        // two E2M1 codes per byte, d = 128 only
  constexpr bool QNT = FMT != kFmtBf16;       // per-head scales
  constexpr int NW = R * S;
  constexpr int GR = 16 * TPW * R;            // rows per workgroup
  // tokens per chunk: quantised rows are narrower, so a single-tile wave
  // takes twice the tokens per load; with two tiles the scores would not fit
  constexpr int CT = QNT && TPW == 1 ? 64 : 32;
  constexpr int NRG = CT / 16;                // 16-token row groups per chunk
  constexpr int NKS = CT / 32;                // 32-token PV k-steps per chunk
  constexpr int NKK = D / 32;                 // QK MFMA steps over d
  // 16-byte K loads per row group (FP4: one load holds a lane's 32 dims)
  constexpr int NKL = FP4 ? 1 : FP8 ? NKK / 2 : NKK;
  constexpr int NJ = D / 16;                  // PV MFMAs per k-step
  constexpr int DPL = D / 16;                 // dims per lane per V row
  constexpr int BPC = CT / BS;                // blocks per chunk
  constexpr int RB = FP4 ? D / 2 : FP8 ? D : 2 * D;   // bytes per token row
  constexpr int VB = FP4 ? DPL / 2 : FP8 ? DPL : 2 * DPL;   // bytes of a lane's V slice
  constexpr int NVS = 8 * NKS;
  using VT = typename Vec<VB>::T;
  constexpr int VW = (DPL * 2) / 4;
  static_assert(!FP4 || D == 128, "FP4 is built for d = 128");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15;
  const int g4 = lane >> 4;

  // grid: x = (KV head, group of GR rows), y = sequence, z = partition from
  // the end
  const int G = a.n_q / a.n_kv;
  const int rows = a.Q * G;                           // query rows of one KV head
  const int groups = (rows + GR - 1) / GR;
  const int g = blockIdx.x / groups;
  const int row0 = (blockIdx.x % groups) * GR;        // first row of the group
  const int b = blockIdx.y;
  const int j = gridDim.z - 1 - blockIdx.z;
  const int ctx = min(a.context_lens ? a.context_lens[b] : a.fixed_ctx, a.max_blocks * BS);
  // causal: query i of q_len sits at position ctx - q_len + i; non-causal
  // (a shared prefix read for many sequences' queries): every row sees all
  const int ql = a.non_causal ? (ctx > 0 ? a.Q : 0)
                              : max(0, min(min(a.query_lens[b], a.Q), ctx));
  auto qpos = [&](int i) -> int { return a.non_causal ? ctx - 1 : ctx - ql + i; };
  const int t0 = j * a.partition;

  __shared__ float sm_m[NW][TPW * 16];
  __shared__ float sm_l[NW][TPW * 16];
  __shared__ float sm_acc[NW][TPW * 16][D + 4];
  // with several tiles per wave the query operands are staged in LDS and read
  // per chunk: held in registers for the whole loop they would not fit
  constexpr bool QLDS = TPW > 1;
  constexpr int QLD = D + 8;                          // padded row (bf16 elements)
  __shared__ __align__(16) uint16_t sm_q[QLDS ? R * TPW * 16 : 1][QLD];

  // last position of the query among rows [r0, r1) (r1 > r0), or -1 if none
  auto last_pos = [&](int r0, int r1) -> int {
    const int i_hi = min((min(r1, rows) - 1) / G, ql - 1);
    return r0 / G < ql && r0 < rows ? qpos(i_hi) : -1;
  };
  if (t0 > last_pos(row0, row0 + GR)) {
    // no row of this group reads this partition; a single pass still owes the
    // group's rows their zeros (rows past q_len, or a sequence with none)
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

  // this wave's tiles and chunk stream; this lane's rows and their positions
  const int tl = wave % R;
  const int st = wave / R;
  const int wrow0 = row0 + tl * TPW * 16;             // first row of the wave
  const int p_lo = qpos(wrow0 / G);              // smallest position of the wave
  const int p_hi = last_pos(wrow0, wrow0 + TPW * 16); // largest (-1: none)
  const int t1 = min(t0 + a.partition, p_hi + 1);    // tokens past p_hi are never read
  const int blk0 = t0 / BS;
  const int blk1 = (t1 + BS - 1) / BS;
  const int n_ch = t0 < t1 ? (blk1 - blk0 + BPC - 1) / BPC : 0;

  auto dimbase = [&](int kk) -> int {
    if constexpr (FP4) return 32 * g4 + 8 * kk;
    return FP8 ? 64 * (kk >> 1) + 16 * g4 + 8 * (kk & 1) : 32 * kk + 8 * g4;
  };
  // Scores and the softmax reference stay in raw q . k units; the weight of a
  // score s is 2^((s - m) qscale), so a row's largest score weighs exactly 1,
  // as in the decode kernel. That needs qscale > 0, so that the row maximum of
  // the raw scores is that of the scaled ones: a negative product is made
  // positive by negating Q (exact in bf16), a zero one by zeroing Q (every
  // score is then 0, as 0 . q . k would be).
  float qscale = a.scale * kLog2e;
  if constexpr (QNT) qscale *= a.k_scale[g];
  const uint32_t qflip = qscale < 0.0f ? 0x80008000u : 0u;
  const bool qzero = qscale == 0.0f;
  qscale = qzero ? 1.0f : fabsf(qscale);
  bf16x8_t qop[QLDS ? 1 : TPW][NKK];
  int pos[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int row = wrow0 + 16 * t + c;
    pos[t] = qpos(row / G);                      // last token this row may see
  }
  if constexpr (QLDS) {
    // the workgroup's rows (zeros for rows without a query), then a barrier
    for (int e = threadIdx.x; e < R * TPW * 16 * (D / 8); e += blockDim.x) {
      const int r = e / (D / 8);
      const int col = 8 * (e % (D / 8));
      const int row = row0 + r;
      uint4 w = make_uint4(0, 0, 0, 0);
      if (row < rows && row / G < ql && !qzero) {
        w = *reinterpret_cast<const uint4*>(
            a.q + ((static_cast<int64_t>(b) * a.Q + row / G) * a.n_q + g * G + row % G) * D +
            col);
        w = make_uint4(w.x ^ qflip, w.y ^ qflip, w.z ^ qflip, w.w ^ qflip);
      }
      *reinterpret_cast<uint4*>(&sm_q[r][col]) = w;
    }
    __syncthreads();
  } else {
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int row = wrow0 + 16 * t + c;
      const int qi = row / G;
      const bool live_row = row < rows && qi < ql && !qzero;
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
  }
  // query operand of tile t, step kk; `salt` is 0 for every real token index
  // but not provably so, which keeps the LDS reads inside the chunk loop
  auto q_operand = [&](int t, int kk, int salt) -> bf16x8_t {
    if constexpr (!QLDS) {
      return qop[t][kk];
    } else {
      const char* base = reinterpret_cast<const char*>(&sm_q[tl * TPW * 16 + 16 * t + c][0]);
      return __builtin_bit_cast(
          bf16x8_t, *reinterpret_cast<const uint4*>(base + 2 * dimbase(kk) + salt));
    }
  };

  const int64_t tile_bytes = static_cast<int64_t>(BS) * RB;
  const int64_t head_off = static_cast<int64_t>(g) * tile_bytes;
  const int64_t block_stride = static_cast<int64_t>(a.n_kv) * tile_bytes;
  const int32_t* bt = a.block_tables + static_cast<int64_t>(b) * a.max_blocks;

  auto v_tok = [&](int s) -> int {
    const int s8 = s & 7;
    return 16 * (2 * (s >> 3) + (s8 >> 2)) + 4 * g4 + (s8 & 3);
  };

  // K and V of a chunk are separate buffers: the next chunk's V is requested
  // only once this chunk's K has been consumed, so at most three of the four
  // buffers hold data at any time.
  struct KChunk {
    uint4 k[NRG][NKL];
  };
  struct VChunk {
    VT v[NVS];
  };

  // block i of chunk ci as a buffer resource (size 0 when absent: loads give 0)
  auto rsrc = [&](const uint8_t* cache, int ci, int i) -> __amdgpu_buffer_rsrc_t {
    const int blk = blk0 + ci * BPC + i;
    const bool have = blk < blk1;
    int p = __builtin_amdgcn_readfirstlane(have ? bt[blk] : 0);
    if (p < 0 || p >= a.num_blocks) p = 0;
    return tile_rsrc(cache + p * block_stride + head_off, have ? static_cast<int>(tile_bytes) : 0);
  };
  // lane (c, g4): K row c at 16 bytes per lane group (bf16: dims 8 g4 + 32 kl;
  // FP8: 16 g4 + 64 kl; FP4: dims 32 g4 ..), V row 4 g4 at dims DPL c
  const uint32_t k_lane = static_cast<uint32_t>(c * RB + 16 * g4);
  const uint32_t v_lane = static_cast<uint32_t>(4 * g4 * RB + VB * c);
  auto load_k = [&](KChunk& kc, int ci) {
    __amdgpu_buffer_rsrc_t r[BPC];
#pragma unroll
    for (int i = 0; i < BPC; ++i) r[i] = rsrc(a.k_cache, ci, i);
    // token 16 rg + c of the chunk is row (16 rg) % BS + c of block 16 rg / BS
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg)
#pragma unroll
      for (int kl = 0; kl < NKL; ++kl)
        ld_stream(kc.k[rg][kl], r[16 * rg / BS], k_lane, ((16 * rg) % BS) * RB + 64 * kl);
  };
  auto load_v = [&](VChunk& vc, int ci) {
    __amdgpu_buffer_rsrc_t r[BPC];
#pragma unroll
    for (int i = 0; i < BPC; ++i) r[i] = rsrc(a.v_cache, ci, i);
    // token v_tok(s) = 16 X + 4 g4 + (s & 3), X = 2 (s / 8) + (s % 8) / 4
#pragma unroll
    for (int s = 0; s < NVS; ++s) {
      const int X = 2 * (s >> 3) + ((s & 7) >> 2);
      ld_stream(vc.v[s], r[16 * X / BS], v_lane, ((16 * X) % BS + (s & 3)) * RB);
    }
  };

  float m_ref[TPW], m_raw[TPW], l[TPW];     // reference and own maximum in raw units
  const float thr = kLazyRescale / qscale;   // the rescale threshold in raw units
  f32x4_t acc[TPW][NJ];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    m_ref[t] = -INFINITY;
    m_raw[t] = -INFINITY;
    l[t] = 0.0f;
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) acc[t][jj] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }

  using Scores = float[TPW][4 * NRG];
  // scores of chunk ci (base-2 units), masked causally and at the partition end
  auto qk = [&](const KChunk& kc, int ci, Scores& s) {
    const int tok0 = (blk0 + ci * BPC) * BS;
    const int salt = (tok0 >> 31) & 16;
    // d-step outermost: each query operand is read once per chunk and applied
    // to every row group while it is live
    f32x4_t sc[NRG][TPW];
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg)
#pragma unroll
      for (int t = 0; t < TPW; ++t) sc[rg][t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      bf16x8_t qo[TPW];
#pragma unroll
      for (int t = 0; t < TPW; ++t) qo[t] = q_operand(t, kk, salt);
#pragma unroll
      for (int rg = 0; rg < NRG; ++rg) {
        bf16x8_t kop;
        if constexpr (FMT == kFmtBf16) {
          kop = __builtin_bit_cast(bf16x8_t, kc.k[rg][kk]);
        } else if constexpr (FP4) {
          // 8 codes at dims 32 g4 + 8 kk
          const uint32_t w = word(kc.k[rg][0], kk);
          kop = as_bf16x8(fp4x2_to_bf16x2<0>(w), fp4x2_to_bf16x2<1>(w),
                          fp4x2_to_bf16x2<2>(w), fp4x2_to_bf16x2<3>(w));
        } else {
          const uint4 w = kc.k[rg][kk >> 1];
          const uint32_t w0 = (kk & 1) ? w.z : w.x;
          const uint32_t w1 = (kk & 1) ? w.w : w.y;
          kop = as_bf16x8(fp8x2_to_bf16x2<false>(w0), fp8x2_to_bf16x2<true>(w0),
                          fp8x2_to_bf16x2<false>(w1), fp8x2_to_bf16x2<true>(w1));
        }
#pragma unroll
        for (int t = 0; t < TPW; ++t)
          sc[rg][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qo[t], sc[rg][t], 0, 0, 0);
      }
    }
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg)
#pragma unroll
      for (int t = 0; t < TPW; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[t][4 * rg + i] = sc[rg][t][i];
    if (tok0 + CT > min(p_lo + 1, t1)) {
      // causal: each row sees tokens up to its own position, and nothing past
      // the partition's end (such slots were not loaded)
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

  // online softmax update with the scores of chunk ci, then O += P V
  auto pv = [&](VChunk& vc, int ci, Scores& s) {
    const int tok0 = (blk0 + ci * BPC) * BS;
    if (tok0 + CT > t1) {
#pragma unroll
      for (int si = 0; si < NVS; ++si)
        if (tok0 + v_tok(si) >= t1) vc.v[si] = VT{};
    }
    // Lazy rescaling, checked per lane: a row's reference m_ref only has to
    // stay within 2^8 of every weight, so each lane compares its own largest
    // score with it, and the row maximum (a cross-lane reduction) is taken
    // only in the rare chunk where some lane exceeds it. A row may see none
    // of a chunk's tokens (all -inf): it keeps its state.
    float lmax[TPW];
    bool need_any = false;
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      float mx = s[t][0];
#pragma unroll
      for (int i = 1; i < 4 * NRG; ++i) mx = vmax(mx, s[t][i]);
      lmax[t] = mx;
      m_raw[t] = vmax(m_raw[t], mx);
      need_any |= mx > m_ref[t] + thr;
    }
    if (__builtin_amdgcn_ballot_w64(need_any) != 0) {
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const float mx = max_xor32(max_xor16(lmax[t]));   // the row's maximum
        const bool need = mx > m_ref[t] + thr;
        const float alpha = need ? fast_exp2((m_ref[t] - mx) * qscale) : 1.0f;
        if (need) m_ref[t] = mx;
        l[t] *= alpha;
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj) acc[t][jj] *= alpha;
      }
    }
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
          p[i] = fast_exp2((s[t][8 * ks + i] - m_use[t]) * qscale);
          l[t] += p[i];
        }
        uint32_t ph[4], pl[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const Bf16Split sp = split_bf16(p[2 * u], p[2 * u + 1]);
          ph[u] = sp.hi;
          pl[u] = sp.lo;
        }
        pop_hi[t] = as_bf16x8(ph[0], ph[1], ph[2], ph[3]);
        pop_lo[t] = as_bf16x8(pl[0], pl[1], pl[2], pl[3]);
      }
      uint32_t vw[8][FP4 ? 1 : VW];
      Fp4Pair vp[4];                     // FP4: slots 2t, 2t + 1 interleaved
#pragma unroll
      for (int si = 0; si < 8; ++si) {
        if constexpr (FMT == kFmtBf16) {
#pragma unroll
          for (int w = 0; w < VW; ++w) vw[si][w] = word(vc.v[8 * ks + si], w);
        } else if constexpr (FP4) {
          if (si % 2 == 1)
            vp[si / 2] = fp4_interleave(word(vc.v[8 * ks + si - 1], 0), word(vc.v[8 * ks + si], 0));
        } else {
#pragma unroll
          for (int w = 0; w < VW / 2; ++w) {
            const uint32_t x = word(vc.v[8 * ks + si], w);
            vw[si][2 * w] = fp8x2_to_bf16x2<false>(x);
            vw[si][2 * w + 1] = fp8x2_to_bf16x2<true>(x);
          }
        }
      }
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) {
        uint32_t t4[4];
        if constexpr (FP4) {
#pragma unroll
          for (int u = 0; u < 4; ++u) t4[u] = fp4_pair_dim(vp[u], jj);
        } else {
          const int w = jj >> 1;
          const uint32_t sel = (jj & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
          for (int u = 0; u < 4; ++u)
            t4[u] = __builtin_amdgcn_perm(vw[2 * u + 1][w], vw[2 * u][w], sel);
        }
        const bf16x8_t vop = as_bf16x8(t4[0], t4[1], t4[2], t4[3]);
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
          acc[t][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop_hi[t], acc[t][jj], 0, 0, 0);
          acc[t][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop_lo[t], acc[t][jj], 0, 0, 0);
        }
      }
    }
  };

  {
    KChunk kA, kB;
    VChunk vA, vB;
    Scores sc;
    int ci = st;
    if (ci < n_ch) {
      load_k(kA, ci);
      load_v(vA, ci);
    }
    for (; ci < n_ch; ci += 2 * S) {
      const bool nb = ci + S < n_ch;
      if (nb) load_k(kB, ci + S);
      qk(kA, ci, sc);
      if (nb) load_v(vB, ci + S);
      pv(vA, ci, sc);
      if (!nb) break;
      const bool na = ci + 2 * S < n_ch;
      if (na) load_k(kA, ci + 2 * S);
      qk(kB, ci + S, sc);
      if (na) load_v(vA, ci + 2 * S);
      pv(vB, ci + S, sc);
    }
  }

#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    float lt = l[t];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    const float m_true = max_xor32(max_xor16(m_raw[t]));   // the row's true maximum
    const float f = m_true == -INFINITY ? 0.0f : fast_exp2((m_ref[t] - m_true) * qscale);
    if (g4 == 0) {
      sm_m[wave][16 * t + c] = m_true * qscale;           // base-2 units
      sm_l[wave][16 * t + c] = lt * f;
    }
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sm_acc[wave][16 * t + c][DPL * (4 * g4 + i) + jj] = acc[t][jj][i] * f;
  }
  __syncthreads();

  const float vscale = QNT ? a.v_scale[g] : 1.0f;
  for (int e = threadIdx.x; e < GR * D; e += blockDim.x) {
    const int r = e / D;                               // group row
    const int dd = e % D;
    const int rr = row0 + r;
    if (rr >= rows) continue;
    const int ri = rr / G;
    const int64_t orow = (static_cast<int64_t>(b) * a.Q + ri) * a.n_q + g * G + rr % G;
    const int rt = r / (16 * TPW);                     // its waves: rt + R * s
    const int rc = r % (16 * TPW);
    float M = -INFINITY;
#pragma unroll
    for (int s2 = 0; s2 < S; ++s2) M = fmaxf(M, sm_m[rt + R * s2][rc]);
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int s2 = 0; s2 < S; ++s2) {
      const int w = rt + R * s2;
      const float fw = sm_m[w][rc] == -INFINITY ? 0.0f : fast_exp2(sm_m[w][rc] - M);
      L = fmaf(sm_l[w][rc], fw, L);
      O = fmaf(sm_acc[w][rc][dd], fw, O);
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

template <int D, int BS, int FMT, int TPW, int R, int S>
static hipError_t launch_g(const DecodeArgs& a, int tiles, hipStream_t s) {
  constexpr int tpg = TPW * R;
  const dim3 grid(a.n_kv * ((tiles + tpg - 1) / tpg), a.B, a.P_max);
  multi_query_partition_mfma<D, BS, FMT, TPW, R, S><<<grid, R * S * 64, 0, s>>>(a);
  return hipGetLastError();
}

// Two or more row tiles per KV head: each wave applies every K/V chunk to two
// tiles (one 4-wave workgroup per pair); a single tile runs one per wave.
template <int D, int BS, int FMT>
static hipError_t launch_mq(const DecodeArgs& a, int tiles, hipStream_t s) {
  if (tiles >= 2) return launch_g<D, BS, FMT, 2, 1, 4>(a, tiles, s);
  return launch_g<D, BS, FMT, 1, 1, 4>(a, tiles, s);
}

template <int D, int BS>
static hipError_t launch_mq_fmt(const DecodeArgs& a, int tiles, hipStream_t s) {
  if (a.kv_dtype == PKV_FP8_E4M3) return launch_mq<D, BS, kFmtFp8>(a, tiles, s);
  if constexpr (D == 128)
    if (a.kv_dtype == PKV_FP4_E2M1) return launch_mq<D, BS, kFmtFp4>(a, tiles, s);
  if (a.kv_dtype != PKV_BF16) return hipErrorInvalidValue;
  return launch_mq<D, BS, kFmtBf16>(a, tiles, s);
}

// Many rows per KV head (128 or more) share each K/V chunk through LDS
// (multi_query_lds.hip); fewer stream it into registers here.
hipError_t launch_multi_query_partition(const DecodeArgs& a, hipStream_t s) {
  if (a.kv_dtype == PKV_FP4_E2M1 && a.d != 128) return hipErrorInvalidValue;
  const int G = a.n_q / a.n_kv;
  const int tiles = (a.Q * G + 15) / 16;
  if (tiles >= 8) return launch_multi_query_lds(a, s);
  if (a.d == 128)
    return a.bs == 16 ? launch_mq_fmt<128, 16>(a, tiles, s) : launch_mq_fmt<128, 32>(a, tiles, s);
  return a.bs == 16 ? launch_mq_fmt<64, 16>(a, tiles, s) : launch_mq_fmt<64, 32>(a, tiles, s);
}

}  // namespace pkv

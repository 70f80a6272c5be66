// Paged decode attention, partition kernel on the gfx950 matrix cores.
//
// What is computed follows [MTKV] "Architecting Multi-Tier Disaggregated
// KV-Cache Hierarchies for Terabyte-Scale LLM Inference", section
// "High-Throughput Paged Attention Kernel Integration": per (sequence, KV
// head, partition), online softmax of scale * q . k over the partition's
// tokens for all query heads of the group (query head h reads KV head h / G),
// accumulating the weighted sum of V, with the K/V tiles fetched through the
// block table; the weights are the softmax of [MTKV] "Mathematical
// Formulation of Block Salience". The page's kernel runs one program per
// (sequence, query head) and so reads every KV byte G times; here one
// workgroup serves all query heads of a KV head (up to 16 per head tile), so
// each byte of the partition is read once, and short batches are split over
// the context (split-K) and merged by the log-sum-exp reduce.
//
// Why MFMA: with G = 8 query heads per KV head every bf16 K/V element feeds
// 8 fp32 FMAs plus a conversion; on the vector ALU that is ~80% of its issue
// rate at 70% of HBM bandwidth (a vector-ALU form of this kernel measured
// 944 us on the 70B layer against 368 us for the first matrix-core form). v_mfma_f32_16x16x32_bf16 consumes the bf16
// tiles as loaded (no conversion) and does the contraction of 16 heads in one
// instruction; heads beyond G are zero columns.
//
// Register layout (lane l: column c = l % 16, k-group g4 = l / 16):
//   scores  S = K . Q^T : A = K tile (m = token c of a 16-token row group,
//           k = 8 dims 32kk + 8*g4), B = Q^T (n = head c). The result puts
//           head c's scores for tokens 4*g4 .. 4*g4+3 in lane l.
//   output  O^T = V^T . P^T : B = P^T (n = head c, k = those same 8 tokens of
//           the two row groups) -- already in the lane, no data movement;
//           A = V^T (m = dim DPL*c + j, k = the 8 tokens), built by loading
//           8 token rows of DPL dims (whole rows per load instruction across
//           16 lanes) and transposing 16-bit pairs with v_perm_b32.
//   Every lane therefore owns one head's softmax state (its 4 k-group lanes
//   share a max through two row-swap moves, v_permlane16/32_swap) and that
//   head's output
//   accumulator for D/4 dims.
// P is fed to the matrix core as bf16 hi + lo parts (two MFMAs), which keeps
// the weights to ~16 significant bits; the row sums use the fp32 weights.
// The running max is refreshed lazily: only when a chunk's max exceeds the
// reference by more than 2^8 are the accumulators rescaled (weights stay
// <= 256, far inside bf16 and fp32 range); the true max is tracked and the
// partition's statistics are rebased on it at the end.
//
// A chunk is 32 tokens for bf16 and 64 for FP8 (16 KiB of K+V either way),
// i.e. 2 or 4 row groups of 16 tokens. K loads are 16 B per lane: for bf16
// lane (c, g4) reads dims 32kk + 8*g4 of token c (one MFMA step per load);
// for FP8 it reads 16 dims at 64h + 16*g4 (two MFMA steps per load). Either
// way a load instruction covers 64 contiguous bytes of 16 token rows; the
// query operand uses the same dim assignment, so the dot products are
// unchanged.
//
// Two work decompositions:
//   interleaved (default): one workgroup per (partition, KV head, sequence);
//     its 4 waves take the partition's chunks round-robin and merge their
//     softmax states through LDS;
//   wave-per-partition (short partitions): one workgroup per 4 consecutive
//     partitions of a (KV head, sequence); each wave runs one partition end
//     to end, so the load pipeline stays long, and writes its own partial.
#include <float.h>

#include "mfma_common.h"
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

using namespace mfma;

// Two waves per SIMD: the register budget is 256 per lane (arch + acc).
// DEPTH chunk buffers rotate through the main loop: DEPTH - 1 chunks are in
// flight while one is computed. With DEPTH = 4 a chunk is half as long, so the
// four buffers take the registers of two full chunks.
template <int D, int BS, int FMT, int NW, bool SPLIT_P, int DEPTH>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void decode_partition_mfma(DecodeArgs a) {
  constexpr bool FP8 = FMT == kFmtFp8;
  constexpr bool FP4 = FMT == kFmtFp4;        // two E2M1 codes per byte, d = 128 only
  constexpr bool QNT = FMT != kFmtBf16;       // per-head scales
  static_assert(DEPTH == 2 || (DEPTH == 4 && FMT != kFmtBf16), "pipeline depth");
  // tokens per chunk: 16 KiB of K+V with two buffers, 8 KiB with four
  constexpr int CT = (FP4 ? 128 : FP8 ? 64 : 32) / (DEPTH / 2);
  constexpr int NRG = CT / 16;                // 16-token row groups per chunk
  constexpr int NKS = CT / 32;                // 32-token PV k-steps per chunk
  constexpr int NKK = D / 32;                 // QK MFMA steps over d
  constexpr int NKL = FP4 ? 1 : FP8 ? NKK / 2 : NKK;   // 16-byte K loads per row group
  constexpr int NJ = D / 16;                  // PV MFMAs per k-step (16 dims each)
  constexpr int DPL = D / 16;                 // dims per lane per V row
  constexpr int BPC = CT / BS;                // blocks per chunk
  constexpr int EB = FP8 ? 1 : 2;             // bytes per element (bf16, FP8)
  constexpr int RB = FP4 ? D / 2 : D * EB;    // bytes per token row
  constexpr int VB = FP4 ? DPL / 2 : FP8 ? DPL : 2 * DPL;   // bytes per V load (DPL dims)
  constexpr int NVS = 8 * NKS;                // V token slots per chunk
  using VT = typename Vec<VB>::T;
  constexpr int VW = (DPL * 2) / 4;           // bf16 words per V row slice (after conversion)
  // a chunk is computed in sub-chunks of at most 4 row groups (64 tokens),
  // which bounds the score registers
  constexpr int NSUB = NRG > 4 ? NRG / 4 : 1;
  constexpr int RGS = NRG / NSUB;
  constexpr int KSS = NKS / NSUB;
  static_assert(CT % BS == 0 && NKL >= 1, "chunk shape");
  static_assert(!FP4 || D == 128, "FP4 rows are 64 bytes: one 16-byte load per lane group");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15;
  const int g4 = lane >> 4;

  // grid: x = (KV head, head tile), y = sequence, z = partition group counted
  // from the end, so the partitions that only long sequences have are
  // dispatched first and the short tail of the launch is made of first
  // partitions
  // With a schedule, x = item * (KV heads x tiles) + head slot, and the item
  // names (sequence, partition) in longest-first order. Workgroups go to the
  // 8 XCDs round-robin, so with 8 KV heads head g runs on XCD g and the 8
  // XCDs read the 8 head tiles of the same blocks at about the same time;
  // placing a sequence's heads on one XCD instead measured slower.
  const int G = a.n_q / a.n_kv;
  const int tiles = (G + 15) / 16;
  int hx, b, pz;
  if (a.schedule != nullptr) {
    const int hxn = a.n_kv * tiles;
    const int item = blockIdx.x / hxn;
    // A list built for another geometry is not followed (and its items may lie
    // past the caller's buffer). The header is read whole and tested without
    // short-circuits, so its words arrive in one round trip.
    const int2 h01 = reinterpret_cast<const int2*>(a.schedule)[0];
    const int2 h23 = reinterpret_cast<const int2*>(a.schedule)[1];
    const bool stale = (h01.y != a.partition) | (h23.x != a.B) | (h23.y != a.P_max);
    if (stale | (item >= h01.x)) return;               // or past the list: nothing to do
    const int2 it = reinterpret_cast<const int2*>(a.schedule + kScheduleHeader)[item];
    if (it.x < 0 || it.x >= a.B || it.y < 0 || it.y >= a.P_max) return;
    hx = blockIdx.x % hxn;
    b = it.x;
    pz = it.y;
  } else {
    hx = blockIdx.x;
    b = blockIdx.y;
    pz = gridDim.z - 1 - blockIdx.z;
  }
  const int g = hx / tiles;
  const int tile = hx % tiles;
  const int h0 = g * G + tile * 16;
  const int nh = min(16, G - tile * 16);
  const int ctx = min(a.context_lens[b], a.max_blocks * BS);
  const bool wave_parts = a.wave_partitions;
  // interleaved: the workgroup's partition; wave-per-partition: this wave's
  const int j = wave_parts ? pz * NW + wave : pz;
  const int t0 = j * a.partition;

  __shared__ float sm_m[NW][16];
  __shared__ float sm_l[NW][16];
  __shared__ float sm_acc[NW][16][D + 4];

  const int first_t0 = (wave_parts ? pz * NW : pz) * a.partition;
  if (first_t0 >= ctx) {
    // nothing to read; an empty sequence still owes zeros in single-pass mode
    if (!a.write_partials && pz == 0) {
      for (int i = threadIdx.x; i < nh * D; i += blockDim.x) {
        const int64_t o = (static_cast<int64_t>(b) * a.n_q + h0 + i / D) * D + i % D;
        if (a.out_dtype == PKV_FP32)
          static_cast<float*>(a.out)[o] = 0.0f;
        else
          static_cast<uint16_t*>(a.out)[o] = 0;
      }
    }
    return;
  }
  const int t1 = min(t0 + a.partition, ctx);         // may be <= t0 for an idle wave
  const int blk0 = t0 / BS;
  const int blk1 = t1 > t0 ? (t1 + BS - 1) / BS : blk0;
  const int n_ch = (blk1 - blk0 + BPC - 1) / BPC;

  // dims of MFMA step kk used by lane (c, g4); K and Q follow the same map
  auto dimbase = [&](int kk) -> int {
    if constexpr (FP4) return 32 * g4 + 8 * kk;       // lane's 16 bytes hold dims 32 g4 ..
    return FP8 ? 64 * (kk >> 1) + 16 * g4 + 8 * (kk & 1) : 32 * kk + 8 * g4;
  };

  // Scores and the softmax reference stay in raw q . k units; the weight of a
  // score s is 2^((s - m) qscale), so the largest score's weight is exactly 1
  // (a one-token context returns V exactly). That needs qscale > 0, so that
  // the maximum of the raw scores is that of the scaled ones: a negative
  // product is made positive by negating Q (exact in bf16), a zero one by
  // zeroing Q (every score is then 0, as 0 . q . k would be).
  float qscale = a.scale * kLog2e;
  if constexpr (QNT) qscale *= a.k_scale[g];
  const uint32_t qflip = qscale < 0.0f ? 0x80008000u : 0u;
  const bool qzero = qscale == 0.0f;
  qscale = qzero ? 1.0f : fabsf(qscale);

  // Q^T operand: lane (c, g4) holds q[h0 + c][dimbase(kk) .. +8] for each kk
  bf16x8_t qop[NKK];
  {
    const bool live = c < nh && !qzero;
    const uint16_t* qrow = a.q + (static_cast<int64_t>(b) * a.n_q + h0 + (c < nh ? c : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      uint4 w = *reinterpret_cast<const uint4*>(qrow + dimbase(kk));
      w = make_uint4(w.x ^ qflip, w.y ^ qflip, w.z ^ qflip, w.w ^ qflip);
      if (!live) w = make_uint4(0, 0, 0, 0);
      qop[kk] = __builtin_bit_cast(bf16x8_t, w);
    }
  }

  const int64_t tile_bytes = FP4 ? static_cast<int64_t>(BS) * RB : static_cast<int64_t>(BS) * D * EB;
  const int64_t head_off = static_cast<int64_t>(g) * tile_bytes;
  const int64_t block_stride = static_cast<int64_t>(a.n_kv) * tile_bytes;
  const int32_t* bt = a.block_tables + static_cast<int64_t>(b) * a.max_blocks;

  // chunk token of V slot s: k-step s/8, row group 2*(s/8) + (s%8)/4, token 4*g4 + s%4
  auto v_tok = [&](int s) -> int {
    const int s8 = s & 7;
    return 16 * (2 * (s >> 3) + (s8 >> 2)) + 4 * g4 + (s8 & 3);
  };

  struct Chunk {
    uint4 k[NRG][NKL];
    VT v[NVS];
  };

  // Chunk ci through per-block buffer resources (size 0 when the block is
  // absent: its loads give zeros), one constant lane offset each for K and V
  // and a constant offset per row: no per-load address arithmetic.
  const uint32_t k_lane = static_cast<uint32_t>(c * RB + 16 * g4);   // K row c, lane group g4
  const uint32_t v_lane = static_cast<uint32_t>(4 * g4 * RB + VB * c);  // V row 4 g4, dims DPL c
  auto load = [&](Chunk& ch, int ci) {
    __amdgpu_buffer_rsrc_t rk[BPC], rv[BPC];
#pragma unroll
    for (int i = 0; i < BPC; ++i) {
      const int blk = blk0 + ci * BPC + i;
      const bool have = blk < blk1;
      int p = __builtin_amdgcn_readfirstlane(have ? bt[blk] : 0);
      if (p < 0 || p >= a.num_blocks) p = 0;
      const int bytes = have ? static_cast<int>(tile_bytes) : 0;
      rk[i] = tile_rsrc(a.k_cache + p * block_stride + head_off, bytes);
      rv[i] = tile_rsrc(a.v_cache + p * block_stride + head_off, bytes);
    }
    // K: token 16 rg + c is row (16 rg) % BS + c of block 16 rg / BS; load kl
    // covers bytes 64 kl + 16 g4 of the row (bf16: dims 32 kl + 8 g4; FP8:
    // 64 kl + 16 g4; FP4: the lane group's 32 dims)
#pragma unroll
    for (int rg = 0; rg < NRG; ++rg)
#pragma unroll
      for (int kl = 0; kl < NKL; ++kl)
        ld_stream(ch.k[rg][kl], rk[16 * rg / BS], k_lane, ((16 * rg) % BS) * RB + 64 * kl);
    // V: slot s is token 16 X + 4 g4 + (s & 3), X = 2 (s / 8) + (s % 8) / 4
#pragma unroll
    for (int s = 0; s < NVS; ++s) {
      const int X = 2 * (s >> 3) + ((s & 7) >> 2);
      ld_stream(ch.v[s], rv[16 * X / BS], v_lane, ((16 * X) % BS + (s & 3)) * RB);
    }
  };

  float m_ref = -INFINITY;      // reference max of this lane's head (raw q . k units)
  float m_raw = -INFINITY;      // largest of this lane's own scores
  const float thr = kLazyRescale / qscale;   // the rescale threshold in raw units
  float l = 0.0f;               // this lane's share of the row sum
  f32x4_t acc[NJ];
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj) acc[jj] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  auto compute = [&](Chunk& ch, int ci) {
    const int tok0 = (blk0 + ci * BPC) * BS;           // first token of the chunk
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
    // ---- scores: s[4*r + i] is token 16*(sub*RGS + r) + 4*g4 + i for head c
    float s[4 * RGS];
#pragma unroll
    for (int r = 0; r < RGS; ++r) {
      const int rg = sub * RGS + r;
      f32x4_t sc = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        bf16x8_t kop;
        if constexpr (FMT == kFmtBf16) {
          kop = __builtin_bit_cast(bf16x8_t, ch.k[rg][kk]);
        } else if constexpr (FP8) {
          const uint4 w = ch.k[rg][kk >> 1];
          const uint32_t w0 = (kk & 1) ? w.z : w.x;
          const uint32_t w1 = (kk & 1) ? w.w : w.y;
          kop = as_bf16x8(fp8x2_to_bf16x2<false>(w0), fp8x2_to_bf16x2<true>(w0),
                          fp8x2_to_bf16x2<false>(w1), fp8x2_to_bf16x2<true>(w1));
        } else {
          const uint32_t w = word(ch.k[rg][0], kk);    // 8 codes: dims 32 g4 + 8 kk ..
          kop = as_bf16x8(fp4x2_to_bf16x2<0>(w), fp4x2_to_bf16x2<1>(w),
                          fp4x2_to_bf16x2<2>(w), fp4x2_to_bf16x2<3>(w));
        }
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[kk], sc, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) s[4 * r + i] = sc[i];
    }
    if (tok0 + CT > t1) {                              // only the partition's last chunk
#pragma unroll
      for (int r = 0; r < RGS; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (tok0 + 16 * (sub * RGS + r) + 4 * g4 + i >= t1) s[4 * r + i] = -INFINITY;
#pragma unroll
      for (int si = sub * 8 * KSS; si < (sub + 1) * 8 * KSS; ++si)
        if (tok0 + v_tok(si) >= t1) ch.v[si] = VT{};
    }
    // ---- online softmax for head c (shared by the 4 k-group lanes). Lazy
    // rescaling, checked per lane: the head's reference m_ref only has to stay
    // within 2^8 of every weight, so each lane compares its own largest score
    // with it, and the head's maximum (a cross-lane reduction) is taken only
    // in the rare chunk where some lane exceeds it.
    float lm = s[0];
#pragma unroll
    for (int i = 1; i < 4 * RGS; ++i) lm = vmax(lm, s[i]);
    m_raw = vmax(m_raw, lm);
    if (__builtin_amdgcn_ballot_w64(lm > m_ref + thr) != 0) {
      const float mx = max_xor32(max_xor16(lm));       // the head's maximum
      const bool need = mx > m_ref + thr;
      const float alpha = need ? fast_exp2((m_ref - mx) * qscale) : 1.0f;
      if (need) m_ref = mx;
      l *= alpha;
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) acc[jj] *= alpha;
    }
    const float m_use = m_ref == -INFINITY ? 0.0f : m_ref;
#pragma unroll
    for (int kq = 0; kq < KSS; ++kq) {
      const int ks = sub * KSS + kq;
      // P^T operand of k-step ks: slots 0-3 row group 2ks, 4-7 row group 2ks+1
      float p[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        p[i] = fast_exp2((s[8 * kq + i] - m_use) * qscale);
        l += p[i];
      }
      uint32_t ph[4], pl[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if constexpr (SPLIT_P) {
          const Bf16Split sp = split_bf16(p[2 * t], p[2 * t + 1]);
          ph[t] = sp.hi;
          pl[t] = sp.lo;
        } else {
          ph[t] = pack_bf16(p[2 * t], p[2 * t + 1]);
        }
      }
      const bf16x8_t pop_hi = as_bf16x8(ph[0], ph[1], ph[2], ph[3]);
      bf16x8_t pop_lo;
      if constexpr (SPLIT_P) pop_lo = as_bf16x8(pl[0], pl[1], pl[2], pl[3]);

      // ---- V^T operand: vb[s][w] = bf16 pair (dims DPL*c + 2w, +1) of slot 8ks + s
      uint32_t vw[8][FP4 ? 1 : VW];
      Fp4Pair vp[4];                     // FP4: slots 2t, 2t + 1 interleaved
#pragma unroll
      for (int si = 0; si < 8; ++si) {
        if constexpr (FMT == kFmtBf16) {
#pragma unroll
          for (int w = 0; w < VW; ++w) vw[si][w] = word(ch.v[8 * ks + si], w);
        } else if constexpr (FP8) {
#pragma unroll
          for (int w = 0; w < VW / 2; ++w) {
            const uint32_t x = word(ch.v[8 * ks + si], w);
            vw[si][2 * w] = fp8x2_to_bf16x2<false>(x);
            vw[si][2 * w + 1] = fp8x2_to_bf16x2<true>(x);
          }
        } else if (si % 2 == 1) {       // 8 codes per slot: dims DPL c ..
          vp[si / 2] = fp4_interleave(word(ch.v[8 * ks + si - 1], 0), word(ch.v[8 * ks + si], 0));
        }
      }
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) {
        uint32_t t4[4];
        if constexpr (FP4) {
#pragma unroll
          for (int t = 0; t < 4; ++t) t4[t] = fp4_pair_dim(vp[t], jj);
        } else {
          const int w = jj >> 1;
          const uint32_t sel = (jj & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
          for (int t = 0; t < 4; ++t)
            t4[t] = __builtin_amdgcn_perm(vw[2 * t + 1][w], vw[2 * t][w], sel);
        }
        const bf16x8_t vop = as_bf16x8(t4[0], t4[1], t4[2], t4[3]);
        acc[jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop_hi, acc[jj], 0, 0, 0);
        if constexpr (SPLIT_P)
          acc[jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop_lo, acc[jj], 0, 0, 0);
      }
    }
    }
  };

  // ---- main loop, later chunks' loads in flight while the current one is computed
  {
    const int first = wave_parts ? 0 : wave;
    const int stride = wave_parts ? 1 : NW;
    if constexpr (DEPTH == 2) {
      Chunk A, B;
      int ci = first;
      if (ci < n_ch) load(A, ci);
      for (; ci < n_ch; ci += 2 * stride) {
        if (ci + stride < n_ch) load(B, ci + stride);
        compute(A, ci);
        if (ci + stride >= n_ch) break;
        if (ci + 2 * stride < n_ch) load(A, ci + 2 * stride);
        compute(B, ci + stride);
      }
    } else if (first < n_ch) {
      // A chunk past the partition has only absent blocks (size-0 resources),
      // so its loads return zeros without reading memory and every load can be
      // issued unconditionally: the outstanding-load count stays static.
      Chunk buf[DEPTH];
#pragma unroll
      for (int u = 0; u < DEPTH - 1; ++u) load(buf[u], first + u * stride);
      for (int ci = first; ci < n_ch; ci += DEPTH * stride) {
#pragma unroll
        for (int u = 0; u < DEPTH; ++u) {
          const int cu = ci + u * stride;
          if (cu >= n_ch) break;
          load(buf[(u + DEPTH - 1) % DEPTH], cu + (DEPTH - 1) * stride);
          compute(buf[u], cu);
        }
      }
    }
  }

  // ---- wave totals for head c, rebased on the true max
  l = sum_xor32(sum_xor16(l));
  const float m_true = max_xor32(max_xor16(m_raw));
  const float f = m_true == -INFINITY ? 0.0f : fast_exp2((m_ref - m_true) * qscale);
  l *= f;
  if (g4 == 0) {
    sm_m[wave][c] = m_true * qscale;                  // base-2 units
    sm_l[wave][c] = l;
  }
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
    for (int i = 0; i < 4; ++i) sm_acc[wave][c][DPL * (4 * g4 + i) + jj] = acc[jj][i] * f;
  __syncthreads();

  const float vscale = QNT ? a.v_scale[g] : 1.0f;
  if (wave_parts) {
    // every wave's partition is a partial of its own
    for (int i = threadIdx.x; i < NW * nh * D; i += blockDim.x) {
      const int w = i / (nh * D);
      const int h = (i / D) % nh;
      const int e = i % D;
      const int jw = pz * NW + w;
      if (jw >= a.P_max || jw * a.partition >= ctx) continue;
      const float L = sm_l[w][h];
      const int64_t mi = (static_cast<int64_t>(b) * a.n_q + h0 + h) * a.P_max + jw;
      if (e == 0) {
        a.ws_m[mi] = sm_m[w][h];
        a.ws_l[mi] = L;
      }
      a.ws_o[mi * D + e] = sm_acc[w][h][e] / L * vscale;
    }
    return;
  }

  // ---- interleaved: merge the waves; write (m, l, o) or the final output
  for (int i = threadIdx.x; i < nh * D; i += blockDim.x) {
    const int h = i / D;
    const int e = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w][h]);
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float fw = sm_m[w][h] == -INFINITY ? 0.0f : fast_exp2(sm_m[w][h] - M);
      L = fmaf(sm_l[w][h], fw, L);
      O = fmaf(sm_acc[w][h][e], fw, O);
    }
    const float o = O / L * vscale;
    const int hq = h0 + h;
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

// ------------------------------------------------------------------ dispatch

constexpr int kMfmaWaves = 4;

// Pipeline depth: FP4 runs four half-size chunks (its per-byte conversion
// and softmax work keeps a wave on a chunk long enough that one chunk in
// flight does not cover the load latency: 97.6 -> 94.0 us on the 70B FP4
// layer); bf16 and FP8 run two full chunks (FP8 measured no faster with four).
template <int D, int BS, int FMT>
static hipError_t launch_mfma(const DecodeArgs& a, dim3 grid, hipStream_t s) {
  constexpr int depth = FMT == kFmtFp4 ? 4 : 2;
  decode_partition_mfma<D, BS, FMT, kMfmaWaves, true, depth><<<grid, kMfmaWaves * 64, 0, s>>>(a);
  return hipGetLastError();
}

template <int D, int BS>
static hipError_t launch_mfma_fmt(const DecodeArgs& a, dim3 grid, hipStream_t s) {
  if (a.kv_dtype == PKV_FP8_E4M3) return launch_mfma<D, BS, kFmtFp8>(a, grid, s);
  if (a.kv_dtype == PKV_FP4_E2M1) {
    if constexpr (D == 128) return launch_mfma<D, BS, kFmtFp4>(a, grid, s);
    return hipErrorInvalidValue;
  }
  return launch_mfma<D, BS, kFmtBf16>(a, grid, s);
}

hipError_t launch_decode_partition_mfma(const DecodeArgs& a, hipStream_t s) {
  const int G = a.n_q / a.n_kv;
  const int hxn = a.n_kv * ((G + 15) / 16);
  const int gz = a.wave_partitions ? (a.P_max + kMfmaWaves - 1) / kMfmaWaves : a.P_max;
  const dim3 grid = a.schedule != nullptr
                        ? dim3(static_cast<unsigned>(static_cast<int64_t>(hxn) * a.B * a.P_max), 1, 1)
                        : dim3(hxn, a.B, gz);
  if (a.d == 128)
    return a.bs == 16 ? launch_mfma_fmt<128, 16>(a, grid, s) : launch_mfma_fmt<128, 32>(a, grid, s);
  return a.bs == 16 ? launch_mfma_fmt<64, 16>(a, grid, s) : launch_mfma_fmt<64, 32>(a, grid, s);
}

}  // namespace pkv

// Debug-mode checks of caller data that lives in device memory.
//
// The library cannot validate block ids, slots or lengths on the host without
// reading them back. The attention and cache kernels stay memory-safe for any
// such values (an out-of-range block id reads block 0, an out-of-range slot is
// not written), but the results are unspecified. In debug mode these kernels
// run ahead of the work on the caller's stream and raise a per-device flag for
// the caller errors the interface names; the next call reports it. They only
// read within the arrays the call describes.
#include "debug_checks.h"

namespace pkv {

namespace {

__device__ __forceinline__ void raise(int* flag) { atomicOr(flag, 1); }

// One workgroup per table row b. The row's live entries are the first
// cdiv(len, bs) (never more than max_blocks); each must name a pool block.
// A length must lie in [0, max_len]; with query counts, each must lie in
// [0, min(Q, len)].
__global__ void check_tables_kernel(const int32_t* __restrict__ tables, int max_blocks,
                                    const int32_t* __restrict__ lens, int fixed_len, int max_len,
                                    const int32_t* __restrict__ qlens, int Q, int bs,
                                    int num_blocks, int* flag) {
  const int b = blockIdx.x;
  const int len = lens ? lens[b] : fixed_len;
  if (threadIdx.x == 0) {
    if (len < 0 || len > max_len) raise(flag);
    if (qlens) {
      const int q = qlens[b];
      if (q < 0 || q > Q || q > len) raise(flag);
    }
  }
  if (len <= 0) return;
  const int64_t n = min(static_cast<int64_t>(len / bs + (len % bs != 0)),
                        static_cast<int64_t>(max_blocks));
  const int32_t* row = tables + static_cast<int64_t>(b) * max_blocks;
  for (int64_t e = threadIdx.x; e < n; e += blockDim.x) {
    const int32_t p = row[e];
    if (p < 0 || p >= num_blocks) raise(flag);
  }
}

// kv_append: a non-negative slot must lie in the pool and appear once.
__global__ void check_slots_kernel(const int64_t* __restrict__ slots, int T, int64_t pool_slots,
                                   int* flag) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  const int64_t s = slots[t];
  if (s < 0) return;                                  // padding
  if (s >= pool_slots) {
    raise(flag);
    return;
  }
  for (int u = 0; u < t; ++u)
    if (slots[u] == s) {
      raise(flag);
      return;
    }
}

// Copy pairs (src, dst): both in the pool, destinations distinct, and no
// destination also a source of the same call.
__global__ void check_pairs_kernel(const int32_t* __restrict__ pairs, int n, int num_blocks,
                                   int* flag) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int32_t src = pairs[2 * i], dst = pairs[2 * i + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) {
    raise(flag);
    return;
  }
  for (int j = 0; j < n; ++j) {
    if (j < i && pairs[2 * j + 1] == dst) {
      raise(flag);
      return;
    }
    if (pairs[2 * j] == dst) {
      raise(flag);
      return;
    }
  }
}

// One workgroup. The header is read first; only if it names this call's
// geometry (so the buffer holds B * P_max item slots) are the items read.
// A sequence owns cdiv(len, P) partitions (at most P_max); in a single pass
// (P_max == 1) every sequence, empty or not, has its one item.
__global__ void check_schedule_kernel(const int32_t* __restrict__ sched,
                                      const int32_t* __restrict__ lens, int B, int P, int P_max,
                                      int* flag) {
  __shared__ int total;
  __shared__ int ok;
  if (threadIdx.x == 0) {
    total = 0;
    ok = sched[1] == P && sched[2] == B && sched[3] == P_max;
    if (!ok) raise(flag);
  }
  __syncthreads();
  if (!ok) return;
  auto parts = [&](int b) -> int {
    const int len = lens[b];
    const int np = len > 0 ? min((len + P - 1) / P, P_max) : 0;
    return P_max == 1 ? 1 : np;
  };
  int mine = 0;
  for (int b = threadIdx.x; b < B; b += blockDim.x) mine += parts(b);
  atomicAdd(&total, mine);
  __syncthreads();
  const int n = sched[0];
  if (threadIdx.x == 0 && n != total) raise(flag);
  const int cap = min(n, B * P_max);
  const int2* items = reinterpret_cast<const int2*>(sched + 8);
  for (int i = threadIdx.x; i < cap; i += blockDim.x) {
    const int2 it = items[i];
    if (it.x < 0 || it.x >= B || it.y < 0 || it.y >= parts(it.x)) raise(flag);
  }
}

}  // namespace

hipError_t launch_check_schedule(const int32_t* sched, const int32_t* lens, int B, int P,
                                 int P_max, int* flag, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  check_schedule_kernel<<<1, 1024, 0, s>>>(sched, lens, B, P, P_max, flag);
  return hipGetLastError();
}

hipError_t launch_check_tables(const int32_t* tables, int max_blocks, const int32_t* lens,
                               int fixed_len, int max_len, const int32_t* qlens, int Q, int B,
                               int bs, int num_blocks, int* flag, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  check_tables_kernel<<<B, 256, 0, s>>>(tables, max_blocks, lens, fixed_len, max_len, qlens, Q,
                                        bs, num_blocks, flag);
  return hipGetLastError();
}

hipError_t launch_check_slots(const int64_t* slots, int T, int64_t pool_slots, int* flag,
                              hipStream_t s) {
  if (T <= 0) return hipSuccess;
  check_slots_kernel<<<(T + 255) / 256, 256, 0, s>>>(slots, T, pool_slots, flag);
  return hipGetLastError();
}

hipError_t launch_check_pairs(const int32_t* pairs, int n, int num_blocks, int* flag,
                              hipStream_t s) {
  if (n <= 0) return hipSuccess;
  check_pairs_kernel<<<(n + 255) / 256, 256, 0, s>>>(pairs, n, num_blocks, flag);
  return hipGetLastError();
}

}  // namespace pkv

// Longest-first work list for the partition kernel.
//
// A batch of sequences of very different lengths leaves a long tail when its
// partitions are dispatched in index order: the workgroups still running at
// the end are whichever large partitions happened to come last. The hardware
// dispatcher hands workgroups to free CUs in grid order, so ordering the grid
// longest-first turns it into list scheduling by decreasing size. The list
// depends only on the sequence lengths, so one list serves every layer of a
// decode step.
//
// Items are (sequence, partition) pairs: first every full partition (all of
// the same size, in sequence order), then each sequence's last partition in
// decreasing size, bucketed into 64 size classes by a counting sort. With a
// single partition per sequence (single pass) empty sequences come last, so
// that their zero outputs are still written; in split-K mode they have no
// item (the reduce writes their zeros).
//
// Layout of the schedule buffer (int32): [0] item count, [1] partition size,
// [2] B, [3] partitions per sequence (P_max), [4..7] reserved, then the items
// as (sequence, partition) pairs, capacity B * P_max.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

constexpr int kSchedThreads = 1024;
constexpr int kSchedBuckets = 64;

__global__ __launch_bounds__(kSchedThreads) void decode_schedule_kernel(
    const int32_t* __restrict__ context_lens, int B, int P, int P_max,
    int32_t* __restrict__ sched) {
  __shared__ int hist[kSchedBuckets + 1];
  __shared__ int cursor[kSchedBuckets + 1];
  __shared__ int scan[kSchedThreads];
  const int t = threadIdx.x;
  const bool single = P_max == 1;
  const int nb = single ? kSchedBuckets + 1 : kSchedBuckets;
  if (t <= kSchedBuckets) hist[t] = 0;
  __syncthreads();

  // each thread owns a contiguous run of sequences
  const int per = (B + kSchedThreads - 1) / kSchedThreads;
  const int b_lo = min(B, t * per);
  const int b_hi = min(B, b_lo + per);
  auto parts = [&](int b, int* np, int* bucket) {
    const int ctx = context_lens[b];
    *np = ctx > 0 ? min((ctx + P - 1) / P, P_max) : 0;
    if (*np == 0) {
      *bucket = single ? kSchedBuckets : -1;       // empty: last (single pass) or no item
      return;
    }
    const int r = min(ctx - (*np - 1) * P, P);     // size of the last partition
    *bucket = min(kSchedBuckets - 1,
                  static_cast<int>((static_cast<int64_t>(P - r) * kSchedBuckets) / P));
  };
  int full = 0;
  for (int b = b_lo; b < b_hi; ++b) {
    int np, bucket;
    parts(b, &np, &bucket);
    full += max(np - 1, 0);
    if (bucket >= 0) atomicAdd(&hist[bucket], 1);
  }
  // exclusive scan of the full-partition counts over the threads' runs
  scan[t] = full;
  __syncthreads();
  for (int off = 1; off < kSchedThreads; off <<= 1) {
    const int v = t >= off ? scan[t - off] : 0;
    __syncthreads();
    scan[t] += v;
    __syncthreads();
  }
  const int full_before = scan[t] - full;
  const int total_full = scan[kSchedThreads - 1];
  if (t == 0) {
    int acc = total_full;
    for (int k = 0; k < nb; ++k) {
      cursor[k] = acc;
      acc += hist[k];
    }
    sched[0] = acc;
    sched[1] = P;
    sched[2] = B;
    sched[3] = P_max;
  }
  __syncthreads();
  int2* items = reinterpret_cast<int2*>(sched + 8);
  int pos = full_before;
  for (int b = b_lo; b < b_hi; ++b) {
    int np, bucket;
    parts(b, &np, &bucket);
    for (int j = 0; j + 1 < np; ++j) items[pos++] = make_int2(b, j);
    if (bucket >= 0) items[atomicAdd(&cursor[bucket], 1)] = make_int2(b, max(np - 1, 0));
  }
}

hipError_t launch_decode_schedule(const int32_t* context_lens, int B, int P, int P_max,
                                  int32_t* sched, hipStream_t stream) {
  decode_schedule_kernel<<<1, kSchedThreads, 0, stream>>>(context_lens, B, P, P_max, sched);
  return hipGetLastError();
}

}  // namespace pkv

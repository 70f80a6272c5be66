// Launchers of the debug-mode checks (debug_checks.hip) used by the C ABI
// layer. Each raises *flag on a violation and reads only within the arrays
// described.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// Live block-table entries, lengths and query counts of B table rows.
hipError_t launch_check_tables(const int32_t* tables, int max_blocks, const int32_t* lens,
                               int fixed_len, int max_len, const int32_t* qlens, int Q, int B,
                               int bs, int num_blocks, int* flag, hipStream_t stream);
// kv_append slots: in the pool and distinct (negative ones are padding).
hipError_t launch_check_slots(const int64_t* slots, int T, int64_t pool_slots, int* flag,
                              hipStream_t stream);
// Copy pairs: in the pool, distinct destinations, no destination a source.
hipError_t launch_check_pairs(const int32_t* pairs, int n, int num_blocks, int* flag,
                              hipStream_t stream);

// Longest-first schedule: header (partition size, B, partition count) equal
// to the call's, item count equal to the call's number of partitions, every
// item a (sequence, partition) of the call.
hipError_t launch_check_schedule(const int32_t* sched, const int32_t* lens, int B, int P,
                                 int P_max, int* flag, hipStream_t stream);

}  // namespace pkv

// pkv_paged_decode_attention_static: decode attention for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// It is pkv_paged_decode_attention with the split-K partials in `scratch`, a
// file-scope device array of PKV_STATIC_SCRATCH_BYTES, instead of a caller
// workspace; the kernels are the same. Each GPU holds its own copy of the
// array (loaded with the library's code object, kept until the process
// ends). In host code `scratch` is only a stand-in for the symbol, so its
// device address is looked up once per device with hipGetSymbolAddress, with
// that device current, and only that address is ever handed to a kernel.
//
// Every call on one GPU uses that GPU's array: the partials of a call are
// written and read back by the same call, so nothing needs clearing between
// calls, but two calls that overlap on one GPU (other streams, other
// threads) race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pkv.h"
#include "pkv_internal.h"

namespace {

constexpr size_t kScratchBytes = PKV_STATIC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices] = {};
std::mutex g_scratch_mu;

// Device address of the current device's scratch array, looked up on the
// first call on that device.
pkv_status scratch_address(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return PKV_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return PKV_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return PKV_ERR_HIP;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return PKV_OK;
}

}  // namespace

extern "C" pkv_status pkv_paged_decode_attention_static(
    const pkv_cache_desc* desc, void* out, int32_t out_dtype, const void* q, const void* k_cache,
    const void* v_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
    const int32_t* context_lens, int32_t B, int32_t n_q, int32_t max_context_len, float scale,
    const float* k_scale, const float* v_scale, int32_t partition_size, const void* schedule,
    void* stream) {
  // Arguments are validated and partials larger than the array refused
  // (PKV_ERR_WORKSPACE_TOO_SMALL) before the array's address is looked up or
  // anything is launched; a single-pass call never needs it.
  return pkv::decode_attention(desc, out, out_dtype, q, k_cache, v_cache, block_tables,
                               max_blocks_per_seq, context_lens, B, n_q, max_context_len, scale,
                               k_scale, v_scale, partition_size, nullptr, kScratchBytes,
                               scratch_address, schedule, stream, false);
}

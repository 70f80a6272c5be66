// A consumer of libpkv's C ABI with no Python and no torch: one decode step
// (slot mapping, kv_append, the longest-first schedule, split-K decode
// attention) on device buffers and a stream of its own, from raw input files
// written by tests/test_gpu_abi_consumer.py, which compares what it writes
// back with the oracle. It also checks that host validation refuses bad
// arguments before anything is enqueued.
//
// usage: abi_decode DIR   (reads DIR/header.bin etc., writes DIR/out.bin,
//                          DIR/k_out.bin, DIR/v_out.bin)
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "pkv.h"

namespace {

// header.bin: 11 int32 then the float32 scale
struct Header {
  int32_t B, n_q, n_kv, d, bs, num_blocks, max_blocks, kv_dtype, partition, max_ctx, fp8;
  float scale;
};

bool read_file(const std::string& path, std::vector<unsigned char>* out, size_t expect) {
  FILE* f = std::fopen(path.c_str(), "rb");
  if (!f) return false;
  out->resize(expect);
  const size_t got = expect ? std::fread(out->data(), 1, expect, f) : 0;
  const bool at_end = std::fgetc(f) == EOF;
  std::fclose(f);
  return got == expect && at_end;
}

bool write_file(const std::string& path, const void* data, size_t n) {
  FILE* f = std::fopen(path.c_str(), "wb");
  if (!f) return false;
  const size_t put = std::fwrite(data, 1, n, f);
  return std::fclose(f) == 0 && put == n;
}

int fail(const char* what, int code = 1) {
  std::fprintf(stderr, "abi consumer: %s\n", what);
  return code;
}

#define HIP_OK(x)                                                                  \
  do {                                                                             \
    if ((x) != hipSuccess) return fail(#x);                                        \
  } while (0)

#define PKV_OK_OR_FAIL(x)                                                          \
  do {                                                                             \
    const pkv_status st_ = (x);                                                    \
    if (st_ != PKV_OK) {                                                           \
      std::fprintf(stderr, "abi consumer: %s -> %s\n", #x, pkv_status_string(st_)); \
      return 1;                                                                    \
    }                                                                              \
  } while (0)

}  // namespace

int main(int argc, char** argv) {
  if (argc != 2) return fail("usage: abi_decode DIR", 2);
  const std::string dir = argv[1];
  std::vector<unsigned char> hb;
  if (!read_file(dir + "/header.bin", &hb, sizeof(Header))) return fail("header.bin");
  Header h;
  std::memcpy(&h, hb.data(), sizeof(Header));
  if (h.B <= 0 || h.n_q <= 0 || h.n_kv <= 0 || h.d <= 0 || h.bs <= 0 || h.num_blocks <= 0 ||
      h.max_blocks <= 0)
    return fail("header values");

  const size_t elem = h.kv_dtype == PKV_BF16 ? 2 : 1;            // bf16 or FP8 codes
  const size_t pool = static_cast<size_t>(h.num_blocks) * h.n_kv * h.bs * h.d * elem;
  const size_t qn = static_cast<size_t>(h.B) * h.n_q * h.d;
  const size_t newn = static_cast<size_t>(h.B) * h.n_kv * h.d;
  std::vector<unsigned char> q, k, v, bt, cl, kn, vn, ks, vs;
  if (!read_file(dir + "/q.bin", &q, qn * 2) || !read_file(dir + "/k.bin", &k, pool) ||
      !read_file(dir + "/v.bin", &v, pool) ||
      !read_file(dir + "/bt.bin", &bt, static_cast<size_t>(h.B) * h.max_blocks * 4) ||
      !read_file(dir + "/cl.bin", &cl, static_cast<size_t>(h.B) * 4) ||
      !read_file(dir + "/k_new.bin", &kn, newn * 2) || !read_file(dir + "/v_new.bin", &vn, newn * 2))
    return fail("input files");
  if (h.fp8 && (!read_file(dir + "/k_scale.bin", &ks, h.n_kv * 4u) ||
                !read_file(dir + "/v_scale.bin", &vs, h.n_kv * 4u)))
    return fail("scale files");
  std::vector<int32_t> pos(h.B);
  for (int b = 0; b < h.B; ++b) {
    int32_t c;
    std::memcpy(&c, cl.data() + 4 * b, 4);
    pos[b] = c - 1;                                              // the appended token
  }

  const pkv_cache_desc desc{h.num_blocks, h.bs, h.n_kv, h.d, h.kv_dtype};
  hipStream_t s;
  HIP_OK(hipStreamCreateWithFlags(&s, hipStreamNonBlocking));
  void *dq, *dk, *dv, *dbt, *dcl, *dkn, *dvn, *dpos, *dslots, *dout, *dks = nullptr, *dvs = nullptr;
  HIP_OK(hipMalloc(&dq, q.size()));
  HIP_OK(hipMalloc(&dk, pool));
  HIP_OK(hipMalloc(&dv, pool));
  HIP_OK(hipMalloc(&dbt, bt.size()));
  HIP_OK(hipMalloc(&dcl, cl.size()));
  HIP_OK(hipMalloc(&dkn, kn.size()));
  HIP_OK(hipMalloc(&dvn, vn.size()));
  HIP_OK(hipMalloc(&dpos, pos.size() * 4));
  HIP_OK(hipMalloc(&dslots, pos.size() * 8));
  HIP_OK(hipMalloc(&dout, qn * 4));
  if (h.fp8) {
    HIP_OK(hipMalloc(&dks, ks.size()));
    HIP_OK(hipMalloc(&dvs, vs.size()));
    HIP_OK(hipMemcpyAsync(dks, ks.data(), ks.size(), hipMemcpyHostToDevice, s));
    HIP_OK(hipMemcpyAsync(dvs, vs.data(), vs.size(), hipMemcpyHostToDevice, s));
  }
  HIP_OK(hipMemcpyAsync(dq, q.data(), q.size(), hipMemcpyHostToDevice, s));
  HIP_OK(hipMemcpyAsync(dk, k.data(), pool, hipMemcpyHostToDevice, s));
  HIP_OK(hipMemcpyAsync(dv, v.data(), pool, hipMemcpyHostToDevice, s));
  HIP_OK(hipMemcpyAsync(dbt, bt.data(), bt.size(), hipMemcpyHostToDevice, s));
  HIP_OK(hipMemcpyAsync(dcl, cl.data(), cl.size(), hipMemcpyHostToDevice, s));
  HIP_OK(hipMemcpyAsync(dkn, kn.data(), kn.size(), hipMemcpyHostToDevice, s));
  HIP_OK(hipMemcpyAsync(dvn, vn.data(), vn.size(), hipMemcpyHostToDevice, s));
  HIP_OK(hipMemcpyAsync(dpos, pos.data(), pos.size() * 4, hipMemcpyHostToDevice, s));

  // host validation: refused before anything is enqueued
  if (pkv_paged_decode_attention(&desc, dout, PKV_FP32, dq, dk, dv,
                                 static_cast<const int32_t*>(dbt), h.max_blocks,
                                 static_cast<const int32_t*>(dcl), h.B, h.n_q + 1, h.max_ctx,
                                 h.scale, static_cast<const float*>(dks),
                                 static_cast<const float*>(dvs), h.partition, nullptr, 0, nullptr,
                                 s) != PKV_ERR_INVALID_ARG)
    return fail("n_q not a multiple of n_kv was accepted");
  const size_t ws_bytes = pkv_decode_workspace_bytes(h.B, h.n_q, h.d, h.max_ctx, h.partition);
  if (ws_bytes == 0) return fail("the case must take several partitions");
  if (pkv_paged_decode_attention(&desc, dout, PKV_FP32, dq, dk, dv,
                                 static_cast<const int32_t*>(dbt), h.max_blocks,
                                 static_cast<const int32_t*>(dcl), h.B, h.n_q, h.max_ctx, h.scale,
                                 static_cast<const float*>(dks), static_cast<const float*>(dvs),
                                 h.partition, nullptr, 0, nullptr,
                                 s) != PKV_ERR_WORKSPACE_TOO_SMALL)
    return fail("a missing workspace was accepted");

  // the step
  void *dws, *dsched;
  const size_t sched_bytes = pkv_decode_schedule_bytes(h.B, h.max_ctx, h.partition);
  HIP_OK(hipMalloc(&dws, ws_bytes));
  HIP_OK(hipMalloc(&dsched, sched_bytes));
  PKV_OK_OR_FAIL(pkv_slot_mapping(static_cast<const int32_t*>(dbt), h.max_blocks,
                                  static_cast<const int32_t*>(dpos), h.B, h.bs,
                                  static_cast<int64_t*>(dslots), s));
  PKV_OK_OR_FAIL(pkv_kv_append(&desc, dk, dv, dkn, dvn, static_cast<const int64_t*>(dslots), h.B,
                               static_cast<const float*>(dks), static_cast<const float*>(dvs), s));
  PKV_OK_OR_FAIL(pkv_decode_schedule(static_cast<const int32_t*>(dcl), h.B, h.max_ctx, h.partition,
                                     dsched, sched_bytes, s));
  PKV_OK_OR_FAIL(pkv_paged_decode_attention(
      &desc, dout, PKV_FP32, dq, dk, dv, static_cast<const int32_t*>(dbt), h.max_blocks,
      static_cast<const int32_t*>(dcl), h.B, h.n_q, h.max_ctx, h.scale,
      static_cast<const float*>(dks), static_cast<const float*>(dvs), h.partition, dws, ws_bytes,
      dsched, s));
  HIP_OK(hipStreamSynchronize(s));

  std::vector<float> out(qn);
  HIP_OK(hipMemcpy(out.data(), dout, qn * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(k.data(), dk, pool, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(v.data(), dv, pool, hipMemcpyDeviceToHost));
  if (!write_file(dir + "/out.bin", out.data(), qn * 4) ||
      !write_file(dir + "/k_out.bin", k.data(), pool) ||
      !write_file(dir + "/v_out.bin", v.data(), pool))
    return fail("output files");
  for (void* p : {dq, dk, dv, dbt, dcl, dkn, dvn, dpos, dslots, dout, dws, dsched}) HIP_OK(hipFree(p));
  if (h.fp8) {
    HIP_OK(hipFree(dks));
    HIP_OK(hipFree(dvs));
  }
  HIP_OK(hipStreamDestroy(s));
  std::printf("abi consumer: ok (%s, %s)\n", pkv_version(), pkv_status_string(PKV_OK));
  return 0;
}

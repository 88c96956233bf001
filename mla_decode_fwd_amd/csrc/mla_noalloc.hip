// Split-KV decode without a workspace argument and without any allocation,
// for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The chunk partials of a split decode live in `scratch`, one file-scope
// device array of MLA_NOALLOC_SCRATCH_BYTES (64 MiB). Every GPU the library
// runs on holds its own copy of it from the first call on that GPU until the
// process ends. The array's name is only a host-side handle: the device address of each GPU's
// copy is looked up once per device (hipGetSymbolAddress with that device
// current) and kept; kernels receive that address, never the name.
//
// Partial layout in the array (compact, unlike the workspace layout of
// mla_decode_workspace_size, so that the B = 64 x 4096 plan fits): o_part
// [total_splits, s_q, H, 512] in the decode dtype, then lse_part
// [total_splits, s_q, H] fp32 at the next 256-byte boundary. Every chunk
// writes its whole partial before the merge reads it, so nothing needs
// clearing between calls.

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <mutex>

#include "mla_decode.h"
#include "mla_internal.h"

static __device__ __align__(256) unsigned char scratch[MLA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`, looked up on
// the first call on that device.
mla_status_t scratch_address(int dev, void** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MLA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MLA_OK;
}

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

}  // namespace

extern "C" {

size_t mla_decode_noalloc_scratch_bytes(int total_splits, int s_q, int H, mla_dtype_t dtype) {
  if (total_splits <= 0 || s_q <= 0 || H <= 0) return 0;
  if (dtype != MLA_BF16 && dtype != MLA_FP32) return 0;
  const size_t rows = (size_t)total_splits * (size_t)s_q * (size_t)H;
  const size_t elem = dtype == MLA_BF16 ? 2 : 4;
  return align256(rows * (size_t)MLA_D_V * elem) + align256(rows * sizeof(float));
}

mla_status_t mla_decode_fwd_noalloc(const void* q_lat, const void* kv_cache, const int32_t* block_table,
                                    const int32_t* seqlens, const int32_t* split_offsets, int total_splits, int B,
                                    int s_q, int H, int d_qk, int d_v, int page_size, int max_pages_per_seq,
                                    int num_pages, float softmax_scale, int causal, mla_dtype_t dtype, void* o_lat,
                                    float* lse, void* stream) {
  // Outputs are required: the partials stay in the library's array, which
  // the caller cannot address.
  if (!o_lat || !lse) return MLA_ERR_INVALID_ARG;
  if (split_offsets == nullptr)  // one chunk per sequence: no partials at all
    return mla::run_decode(q_lat, kv_cache, nullptr, block_table, seqlens, nullptr, 0, nullptr, total_splits, B, s_q,
                           H, d_qk, d_v, page_size, max_pages_per_seq, num_pages, softmax_scale, causal, dtype,
                           nullptr, 0, o_lat, lse, stream, nullptr);
  const size_t need = mla_decode_noalloc_scratch_bytes(total_splits, s_q, H, dtype);
  if (need == 0) return (dtype != MLA_BF16 && dtype != MLA_FP32) ? MLA_ERR_UNSUPPORTED : MLA_ERR_INVALID_ARG;
  if (need > (size_t)MLA_NOALLOC_SCRATCH_BYTES) return MLA_ERR_WORKSPACE;
  // Every other check that needs no HIP call runs before the lookup: the
  // shared body in check-only mode returns the status the real call would.
  mla::PartialBuffers check{nullptr, nullptr, true};
  const mla_status_t pre = mla::run_decode(q_lat, kv_cache, nullptr, block_table, seqlens, nullptr, 0, split_offsets,
                                           total_splits, B, s_q, H, d_qk, d_v, page_size, max_pages_per_seq,
                                           num_pages, softmax_scale, causal, dtype, nullptr, 0, o_lat, lse, stream,
                                           &check);
  if (pre != MLA_OK) return pre;

  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLA_ERR_HIP;
  if (stream != nullptr) {
    int sdev = -1;
    if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess) return MLA_ERR_HIP;
    if (sdev != dev) return MLA_ERR_INVALID_ARG;  // the array is looked up on the current device
  }
  void* base = nullptr;
  const mla_status_t st = scratch_address(dev, &base);
  if (st != MLA_OK) return st;
  const size_t rows = (size_t)total_splits * (size_t)s_q * (size_t)H;
  const size_t elem = dtype == MLA_BF16 ? 2 : 4;
  mla::PartialBuffers parts{base,
                            reinterpret_cast<float*>(static_cast<unsigned char*>(base) +
                                                     align256(rows * MLA_D_V * elem)),
                            false};
  return mla::run_decode(q_lat, kv_cache, nullptr, block_table, seqlens, nullptr, 0, split_offsets, total_splits, B,
                         s_q, H, d_qk, d_v, page_size, max_pages_per_seq, num_pages, softmax_scale, causal, dtype,
                         nullptr, 0, o_lat, lse, stream, &parts);
}

}  // extern "C"

// Absorbed-MLA decode for fp32 inputs (fp32 storage and arithmetic), gfx950.
//
// Same operation, chunking and partial layout as the bf16 kernel
// ("MLA 推理：两条计算路径与 FlashMLA", sections "两条等价的路径" and
// "decode 注意力变成了计算问题"), written for full fp32 accuracy rather than
// speed: one wave per (chunk, row), keys visited one at a time in token order
// with an exact online softmax (natural exponent, running max updated every
// token). Used for fp32 callers and small fp32 problems.

#include <hip/hip_runtime.h>
#include <cmath>
#include <cstdint>

#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kWaves = 4;  // rows per workgroup

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__global__ __launch_bounds__(64 * kWaves) void mla_decode_fp32_kernel(DecodeArgs a) {
  const int lane = threadIdx.x & 63;
  const int rows = a.s_q * a.H;
  const int row = blockIdx.y * kWaves + (threadIdx.x >> 6);
  const int g = blockIdx.x;
  if (row >= rows || g >= a.total_splits) return;

  int b = g, kk = 0, n = 1;
  if (a.split_offsets != nullptr) {
    int lo = 0, hi = a.B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.split_offsets[mid] <= g) lo = mid; else hi = mid - 1;
    }
    b = lo;
    kk = g - a.split_offsets[lo];
    n = a.split_offsets[lo + 1] - a.split_offsets[lo];
  }
  n = max(n, 1);
  kk = min(max(kk, 0), n - 1);
  int L = a.seqlens[b];
  L = max(a.s_q, min(L, a.max_pages * kPage));
  const int P = (L + kPage - 1) / kPage;
  const int t0 = (int)(((long long)kk * P) / n) * kPage;
  int t1 = (int)(((long long)(kk + 1) * P) / n) * kPage;
  const int qi = row / a.H;
  const int n_allowed = a.causal ? (L - a.s_q + qi + 1) : L;
  t1 = min(t1, n_allowed);

  const float* qrow = reinterpret_cast<const float*>(a.q_lat) + ((size_t)b * rows + row) * kDqk;
  float q[9];
#pragma unroll
  for (int e = 0; e < 9; ++e) q[e] = qrow[lane + 64 * e];
  float o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;
  float m = -INFINITY, l = 0.f;
  const float* cache = reinterpret_cast<const float*>(a.kv_cache);
  const int32_t* btab = a.block_table + (size_t)b * a.max_pages;
  for (int t = t0; t < t1; ++t) {
    const int phys = min(max(btab[t / kPage], 0), a.num_pages - 1);
    const float* krow = cache + ((size_t)phys * kPage + (t % kPage)) * kDqk;
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < 9; ++e) part = fmaf(q[e], krow[lane + 64 * e], part);
    const float s = wave_sum(part) * a.scale;
    const float m_new = fmaxf(m, s);
    const float alpha = expf(m - m_new);  // m = -inf on the first key gives 0
    const float p = expf(s - m_new);
    l = l * alpha + p;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = fmaf(p, krow[lane + 64 * e], o[e] * alpha);
    m = m_new;
  }
  const bool any = l > 0.f;
  const float inv = any ? 1.f / l : 0.f;
  const float lse_v = any ? m + logf(l) : -INFINITY;
  if (n == 1 && a.o_lat != nullptr) {
    float* orow = reinterpret_cast<float*>(a.o_lat) + ((size_t)b * rows + row) * kDv;
#pragma unroll
    for (int e = 0; e < 8; ++e) orow[lane + 64 * e] = o[e] * inv;
    if (lane == 0) a.lse[(size_t)b * rows + row] = lse_v;
  } else {
    float* orow = static_cast<float*>(a.o_part) + ((size_t)g * rows + row) * kDv;
#pragma unroll
    for (int e = 0; e < 8; ++e) orow[lane + 64 * e] = o[e] * inv;
    if (lane == 0) a.lse_part[(size_t)g * rows + row] = lse_v;
  }
}

}  // namespace

hipError_t launch_decode_fp32(const DecodeArgs& a, hipStream_t stream) {
  const int rows = a.s_q * a.H;
  const dim3 grid((unsigned)a.total_splits, (unsigned)((rows + kWaves - 1) / kWaves));
  hipLaunchKernelGGL(mla_decode_fp32_kernel, grid, dim3(64 * kWaves), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla

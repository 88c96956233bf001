// Per-head products around absorbed-MLA decode, gfx950.
//
// "MLA 推理：两条计算路径与 FlashMLA", section "两条等价的路径": the absorbed path
// moves each head's query into latent space (q~ = W_UK q^N) before attention
// and applies W_UV to the latent output afterwards. "DeepSeekV2之MLA", section
// 4.5, does both as batched matrix products over heads.
//
//   absorb_q: q_lat[n,h,0:dc] = sum_d q_nope[n,h,d] * w_uk[h,c,d],
//             q_lat[n,h,dc:dc+dr] = q_rope[n,h,:]
//   out_uv:   out[n,h,e]      = sum_c o_lat[n,h,c] * w_uv[h,c,e]
//
// One kernel serves both: out[n,h,j] = sum_k A[n,h,k] * W(h,k,j), with W read
// either as [H, J, K] (absorb, the weight row is the output index) or as
// [H, K, J] (out_uv). A workgroup computes a 64 x 64 output tile of one head,
// staging 32-deep slices of A and W through LDS in fp32; each thread owns a
// 4 x 4 block of the tile. Accumulation is fp32 for both storage types.

#include <hip/hip_runtime.h>
#include <cstdint>

#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kTN = 64, kTJ = 64, kTK = 32;

template <typename T>
__device__ __forceinline__ float ld(const T* p) { return (float)*p; }
template <typename T>
__device__ __forceinline__ void st(T* p, float v) { *p = (T)v; }

// W_JK: W is [H, J, K] (true) or [H, K, J] (false).
template <typename T, bool W_JK>
__global__ __launch_bounds__(256) void head_bmm_kernel(const T* __restrict__ A, const T* __restrict__ W,
                                                       int N, int H, int K, int J, T* __restrict__ out,
                                                       int out_stride, const T* __restrict__ tail_src,
                                                       int tail) {
  __shared__ float sa[kTK][kTN + 1];
  __shared__ float sw[kTK][kTJ + 1];
  const int h = blockIdx.z;
  const int n0 = blockIdx.y * kTN;
  const int j0 = blockIdx.x * kTJ;
  const int tid = threadIdx.x;
  const int tn = (tid / 16) * 4;  // 16 x 16 threads, 4 x 4 outputs each
  const int tj = (tid % 16) * 4;
  float acc[4][4] = {};
  const T* Wh = W + (size_t)h * J * K;
  for (int k0 = 0; k0 < K; k0 += kTK) {
    for (int idx = tid; idx < kTK * kTN; idx += 256) {
      const int kk = idx % kTK, nn = idx / kTK;
      const int n = n0 + nn, k = k0 + kk;
      sa[kk][nn] = (n < N && k < K) ? ld(A + ((size_t)n * H + h) * K + k) : 0.f;
    }
    for (int idx = tid; idx < kTK * kTJ; idx += 256) {
      int kk, jj;
      if (W_JK) { kk = idx % kTK; jj = idx / kTK; } else { jj = idx % kTJ; kk = idx / kTJ; }
      const int j = j0 + jj, k = k0 + kk;
      float v = 0.f;
      if (j < J && k < K) v = W_JK ? ld(Wh + (size_t)j * K + k) : ld(Wh + (size_t)k * J + j);
      sw[kk][jj] = v;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < kTK; ++kk) {
      float a[4], w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) { a[u] = sa[kk][tn + u]; w[u] = sw[kk][tj + u]; }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = fmaf(a[u], w[v], acc[u][v]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int n = n0 + tn + u;
    if (n >= N) continue;
    T* orow = out + ((size_t)n * H + h) * out_stride;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int j = j0 + tj + v;
      if (j < J) st(orow + j, acc[u][v]);
    }
  }
  // absorb_q: the first column tile also copies the RoPE tail of its rows.
  if (tail > 0 && blockIdx.x == 0) {
    for (int idx = tid; idx < kTN * tail; idx += 256) {
      const int nn = idx / tail, e = idx % tail;
      const int n = n0 + nn;
      if (n < N) out[((size_t)n * H + h) * out_stride + J + e] = tail_src[((size_t)n * H + h) * tail + e];
    }
  }
}

template <typename T, bool W_JK>
hipError_t launch_head_bmm(const void* A, const void* W, int N, int H, int K, int J, void* out,
                           int out_stride, const void* tail_src, int tail, hipStream_t stream) {
  const dim3 grid((unsigned)((J + kTJ - 1) / kTJ), (unsigned)((N + kTN - 1) / kTN), (unsigned)H);
  hipLaunchKernelGGL((head_bmm_kernel<T, W_JK>), grid, dim3(256), 0, stream,
                     static_cast<const T*>(A), static_cast<const T*>(W), N, H, K, J,
                     static_cast<T*>(out), out_stride, static_cast<const T*>(tail_src), tail);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_absorb_q(const void* q_nope, const void* q_rope, const void* w_uk, int N, int H,
                           int dn, int dr, int dc, bool bf16, void* q_lat, hipStream_t stream) {
  if (bf16)
    return launch_head_bmm<__bf16, true>(q_nope, w_uk, N, H, dn, dc, q_lat, dc + dr, q_rope, dr, stream);
  return launch_head_bmm<float, true>(q_nope, w_uk, N, H, dn, dc, q_lat, dc + dr, q_rope, dr, stream);
}

hipError_t launch_out_uv(const void* o_lat, const void* w_uv, int N, int H, int dc, int dv,
                         bool bf16, void* out, hipStream_t stream) {
  if (bf16)
    return launch_head_bmm<__bf16, false>(o_lat, w_uv, N, H, dc, dv, out, dv, nullptr, 0, stream);
  return launch_head_bmm<float, false>(o_lat, w_uv, N, H, dc, dv, out, dv, nullptr, 0, stream);
}

}  // namespace mla

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
#include "mla_launch_aux.h"

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

// bf16 MFMA form, used when K is a multiple of 16 and J a multiple of 4 (the
// DeepSeek shapes): out^T[j][n] = sum_k W(h,j,k) A[n,h,k] with
// v_mfma_f32_32x32x16_bf16, one wave per 32 (j) x 32 (n) tile, four waves per
// workgroup covering 128 consecutive j. B = A rows (8 consecutive k per lane,
// 16-byte loads). A = the weight rows: for W as [H, J, K] 16-byte loads; for
// W as [H, K, J] a 64 x 128 slice of W is staged in LDS (320-byte rows) and
// read transposed with ds_read_b64_tr_b16. fp32 accumulation, bf16 result.
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;
constexpr int kMSlice = 64;                 // k rows of W per staged slice
constexpr int kMStride = 128 * 2 + 64;      // 320-byte LDS rows of a 128-column slice

template <bool W_JK>
__global__ __launch_bounds__(256) void head_bmm_mfma_kernel(const __bf16* __restrict__ A, const __bf16* __restrict__ W,
                                                           int N, int H, int K, int J, __bf16* __restrict__ out,
                                                           int out_stride, const __bf16* __restrict__ tail_src,
                                                           int tail) {
  __shared__ __attribute__((aligned(16))) char smem[W_JK ? 16 : kMSlice * kMStride];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r32 = lane & 31, hi32 = lane >> 5;
  const int h = blockIdx.z;
  const int n0 = blockIdx.y * 32;
  const int jb = blockIdx.x * 128;            // the workgroup's first column
  const int j0 = jb + wave * 32;
  const int n = n0 + r32;
  const int nc = min(n, N - 1);
  const __bf16* xa = A + ((size_t)nc * H + h) * K + 8 * hi32;
  const __bf16* Wh = W + (size_t)h * J * K;
  f32x16_t acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  if constexpr (W_JK) {
    const __bf16* wa = Wh + (size_t)min(j0 + r32, J - 1) * K + 8 * hi32;
    int k = 0;
    for (; k + 128 <= K; k += 128) {  // eight k-steps per round, loads first
      bf16x8_t a[8], b[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        a[u] = *reinterpret_cast<const bf16x8_t*>(wa + k + 16 * u);
        b[u] = *reinterpret_cast<const bf16x8_t*>(xa + k + 16 * u);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u], b[u], acc, 0, 0, 0);
    }
    for (; k < K; k += 16) {
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(wa + k);
      const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(xa + k);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
    }
  } else {
    // Transposed read of the staged slice: 16-lane group g, input lane
    // 4jj + q gives k row 8(g>>1) + 4rd + jj and columns 16(g&1) + 4q .. +4
    // of the wave's 32 columns.
    const int g = lane >> 4, jj = (lane >> 2) & 3, q = lane & 3;
    const int tr_off = kMStride * (8 * (g >> 1) + jj) + 2 * (16 * (g & 1) + 4 * q) + 64 * wave;
    // W[k0 .. k0+63][jb .. jb+127], four 16-byte pieces per thread (columns
    // past J read as column J-1, rows past K as zero); the next slice is
    // loaded into registers while the current one is used.
    auto load_slice = [&](int k0, bf16x8_t (&v)[4]) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int idx = u * 256 + (int)threadIdx.x;
        const int row = idx >> 4, c16 = idx & 15;
        const int k = k0 + row;
        if (k < K && jb + 8 * c16 + 7 < J) {
          v[u] = *reinterpret_cast<const bf16x8_t*>(Wh + (size_t)k * J + jb + 8 * c16);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            v[u][e] = k < K ? Wh[(size_t)k * J + min(jb + 8 * c16 + e, J - 1)] : (__bf16)0.f;
        }
      }
    };
    bf16x8_t nxt[4];
    load_slice(0, nxt);
    for (int k0 = 0; k0 < K; k0 += kMSlice) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int idx = u * 256 + (int)threadIdx.x;
        *reinterpret_cast<bf16x8_t*>(smem + (idx >> 4) * kMStride + 16 * (idx & 15)) = nxt[u];
      }
      __syncthreads();
      if (k0 + kMSlice < K) load_slice(k0 + kMSlice, nxt);
      const int steps = min(kMSlice, K - k0) / 16;
      for (int s4 = 0; s4 < steps; ++s4) {
        bf16x8_t a;
#pragma unroll
        for (int rd = 0; rd < 2; ++rd) {
          const bf16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (lds_bf16x4_t*)((__attribute__((address_space(3))) char*)smem + tr_off + kMStride * (16 * s4 + 4 * rd)));
          a[4 * rd + 0] = v[0]; a[4 * rd + 1] = v[1]; a[4 * rd + 2] = v[2]; a[4 * rd + 3] = v[3];
        }
        const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(xa + k0 + 16 * s4);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
      }
      __syncthreads();
    }
  }
  // acc[r] = out^T[j0 + 8(r>>2) + 4*hi32 + (r&3)][n].
  if (n < N) {
    __bf16* orow = out + ((size_t)n * H + h) * out_stride;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int j = j0 + 8 * q4 + 4 * hi32;
      if (j + 3 < J) {
        bf16x4_t v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (__bf16)acc[4 * q4 + e];
        *reinterpret_cast<bf16x4_t*>(orow + j) = v;
      }
    }
    if (tail > 0 && blockIdx.x == 0 && wave == 0)
      for (int e = hi32; e < tail; e += 2) orow[J + e] = tail_src[((size_t)n * H + h) * tail + e];
  }
}

template <bool W_JK>
hipError_t launch_head_bmm_mfma(const void* A, const void* W, int N, int H, int K, int J, void* out, int out_stride,
                                const void* tail_src, int tail, hipStream_t stream) {
  const dim3 grid((unsigned)((J + 127) / 128), (unsigned)((N + 31) / 32), (unsigned)H);
  hipLaunchKernelGGL((head_bmm_mfma_kernel<W_JK>), grid, dim3(256), 0, stream, static_cast<const __bf16*>(A),
                     static_cast<const __bf16*>(W), N, H, K, J, static_cast<__bf16*>(out), out_stride,
                     static_cast<const __bf16*>(tail_src), tail);
  return hipGetLastError();
}

// The MFMA form needs 16-byte aligned rows: K a multiple of 16, J and the
// output row a multiple of 4 (8-byte stores), 16-byte aligned bases.
bool mfma_shape(const void* A, const void* W, const void* out, int K, int J, int out_stride) {
  return K % 16 == 0 && J % 8 == 0 && out_stride % 4 == 0 && ((uintptr_t)A % 16) == 0 && ((uintptr_t)W % 16) == 0 &&
         ((uintptr_t)out % 8) == 0;
}

}  // namespace

hipError_t launch_absorb_q(const void* q_nope, const void* q_rope, const void* w_uk, int N, int H,
                           int dn, int dr, int dc, bool bf16, void* q_lat, hipStream_t stream) {
  if (bf16 && mfma_shape(q_nope, w_uk, q_lat, dn, dc, dc + dr))
    return launch_head_bmm_mfma<true>(q_nope, w_uk, N, H, dn, dc, q_lat, dc + dr, q_rope, dr, stream);
  if (bf16)
    return launch_head_bmm<__bf16, true>(q_nope, w_uk, N, H, dn, dc, q_lat, dc + dr, q_rope, dr, stream);
  return launch_head_bmm<float, true>(q_nope, w_uk, N, H, dn, dc, q_lat, dc + dr, q_rope, dr, stream);
}

hipError_t launch_out_uv(const void* o_lat, const void* w_uv, int N, int H, int dc, int dv,
                         bool bf16, void* out, hipStream_t stream) {
  if (bf16 && mfma_shape(o_lat, w_uv, out, dc, dv, dv))
    return launch_head_bmm_mfma<false>(o_lat, w_uv, N, H, dc, dv, out, dv, nullptr, 0, stream);
  if (bf16)
    return launch_head_bmm<__bf16, false>(o_lat, w_uv, N, H, dc, dv, out, dv, nullptr, 0, stream);
  return launch_head_bmm<float, false>(o_lat, w_uv, N, H, dc, dv, out, dv, nullptr, 0, stream);
}

}  // namespace mla

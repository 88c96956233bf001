// FP8 (e4m3) batched products around absorbed-MLA decode, gfx950.
//
// "MLA 与 torch.compile：v0.3 的两个来源", the weight-absorption passage (the
// code run once the MLA weights are loaded): with FP8 weights w_kc and w_vc, the query absorption and the output projection run as bmm_fp8 of an
// activation quantised to e4m3 on the fly (one scale per tensor) against the
// e4m3 weights and their scale, with a bf16 result.
//
//   amax_kernel      per-workgroup max |x| of a bf16 tensor
//   quantize_kernel  r = 448 / max|x| (max|x| at least 2^-100; r = 1 for an
//                    all-zero tensor), codes = e4m3(x * r), nearest with ties
//                    to even, |x * r| clamped to 448 (v_cvt_pk_fp8_f32 on the
//                    fp32 product), dequantisation scale s = 1 / r
//   bmm_kernel       out[n,h,j] = s_x * s_w * sum_k X[n,h,k] W[h,j,k] over
//                    e4m3 codes (X quantised as it is loaded, from the
//                    partial maxima), v_mfma_f32_32x32x16_fp8_fp8 with fp32
//                    accumulation, bf16 result; optionally a bf16 tail copied
//                    after the j columns of each row (the RoPE part of q_lat).

#include <hip/hip_runtime.h>

#include <cstdint>

#include "mla_internal.h"
#include "mla_launch_aux.h"

namespace mla {
namespace {

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;

constexpr int kAmaxThreads = 256;

__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float m = 0.f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) m = fmaxf(m, red[w]);
  return m;
}

// partials[blockIdx.x] = max |x| over the elements this workgroup visits.
__global__ __launch_bounds__(kAmaxThreads) void amax_kernel(const __bf16* __restrict__ x, size_t n,
                                                           float* __restrict__ partials) {
  __shared__ float red[kAmaxThreads / 64];
  float m = 0.f;
  const size_t stride = (size_t)gridDim.x * kAmaxThreads;
  const size_t n8 = n / 8;
  for (size_t i = (size_t)blockIdx.x * kAmaxThreads + threadIdx.x; i < n8; i += stride) {
    const bf16x8_t v = *reinterpret_cast<const bf16x8_t*>(x + 8 * i);
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf((float)v[e]));
  }
  for (size_t i = 8 * n8 + (size_t)blockIdx.x * kAmaxThreads + threadIdx.x; i < n; i += stride)
    m = fmaxf(m, fabsf((float)x[i]));
  m = block_max(m, red);
  if (threadIdx.x == 0) partials[blockIdx.x] = m;
}

__device__ __forceinline__ uint32_t e4m3_pair(float a, float b) {
  a = fminf(fmaxf(a, -448.f), 448.f);
  b = fminf(fmaxf(b, -448.f), 448.f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// codes[i] = e4m3(x[i] * r) with r from the partial maxima; workgroup 0 writes s = 1 / r.
__global__ __launch_bounds__(kAmaxThreads) void quantize_kernel(const __bf16* __restrict__ x, size_t n,
                                                               const float* __restrict__ partials, int n_parts,
                                                               uint8_t* __restrict__ codes,
                                                               float* __restrict__ scale_out) {
  __shared__ float red[kAmaxThreads / 64];
  float m = (int)threadIdx.x < n_parts ? partials[threadIdx.x] : 0.f;
  m = block_max(m, red);
  const float r = m > 0.f ? 448.f / fmaxf(m, 0x1p-100f) : 1.f;
  if (blockIdx.x == 0 && threadIdx.x == 0) *scale_out = 1.f / r;
  const size_t stride = (size_t)gridDim.x * kAmaxThreads;
  const size_t n8 = n / 8;
  for (size_t i = (size_t)blockIdx.x * kAmaxThreads + threadIdx.x; i < n8; i += stride) {
    const bf16x8_t v = *reinterpret_cast<const bf16x8_t*>(x + 8 * i);
    uint32_t lo = e4m3_pair((float)v[0] * r, (float)v[1] * r) | (e4m3_pair((float)v[2] * r, (float)v[3] * r) << 16);
    uint32_t hi = e4m3_pair((float)v[4] * r, (float)v[5] * r) | (e4m3_pair((float)v[6] * r, (float)v[7] * r) << 16);
    *reinterpret_cast<uint2*>(codes + 8 * i) = make_uint2(lo, hi);
  }
  for (size_t i = 8 * n8 + (size_t)blockIdx.x * kAmaxThreads + threadIdx.x; i < n; i += stride)
    codes[i] = (uint8_t)e4m3_pair((float)x[i] * r, 0.f);
}

// One wave per 32 (j) x 32 (n) output tile of one head; four waves per
// workgroup cover 128 consecutive j. A = W rows (j), B = X rows (n), both as
// 8 consecutive codes per lane (k = 8 * (lane >> 5) .. +8 of a 16-deep step).
// The activation arrives in bf16 and is quantised as it is loaded: every
// workgroup first reduces the partial maxima to the tensor's scale s, then
// converts its operand exactly as quantize_kernel does (so the codes equal
// mla_quantize_e4m3's).
__global__ __launch_bounds__(256) void bmm_kernel(const __bf16* __restrict__ X, const float* __restrict__ partials,
                                                 int n_parts, const uint8_t* __restrict__ W, float w_scale, int N,
                                                 int H, int K, int J, __bf16* __restrict__ out, int out_stride,
                                                 const __bf16* __restrict__ tail_src, int tail) {
  __shared__ float red[4];
  float m = (int)threadIdx.x < n_parts ? partials[threadIdx.x] : 0.f;
  m = block_max(m, red);
  const float r = m > 0.f ? 448.f / fmaxf(m, 0x1p-100f) : 1.f;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r32 = lane & 31, hi32 = lane >> 5;
  const int h = blockIdx.z;
  const int n0 = blockIdx.y * 32;
  const int j0 = blockIdx.x * 128 + wave * 32;
  const int n = n0 + r32;
  const int nc = min(n, N - 1);
  const int jc = min(j0 + r32, J - 1);
  const __bf16* xa = X + ((size_t)nc * H + h) * K + 8 * hi32;
  const uint8_t* wa = W + ((size_t)h * J + jc) * K + 8 * hi32;
  f32x16_t acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  // Eight k-steps per round, all loads of a round issued before its
  // products, so that the round waits on memory once.
  auto step = [&](long a, const bf16x8_t& v) {
    const uint32_t lo = e4m3_pair((float)v[0] * r, (float)v[1] * r) | (e4m3_pair((float)v[2] * r, (float)v[3] * r) << 16);
    const uint32_t hi = e4m3_pair((float)v[4] * r, (float)v[5] * r) | (e4m3_pair((float)v[6] * r, (float)v[7] * r) << 16);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(a, (long)(((uint64_t)hi << 32) | lo), acc, 0, 0, 0);
  };
  int k = 0;
  for (; k + 128 <= K; k += 128) {
    long a[8];
    bf16x8_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      a[u] = *reinterpret_cast<const long*>(wa + k + 16 * u);
      v[u] = *reinterpret_cast<const bf16x8_t*>(xa + k + 16 * u);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) step(a[u], v[u]);
  }
  for (; k < K; k += 16) step(*reinterpret_cast<const long*>(wa + k), *reinterpret_cast<const bf16x8_t*>(xa + k));
  const float sc = (1.f / r) * w_scale;
  // acc[r] = out^T[j0 + 8(r>>2) + 4*hi32 + (r&3)][n].
  if (n < N) {
    __bf16* orow = out + ((size_t)n * H + h) * out_stride;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int j = j0 + 8 * q4 + 4 * hi32;
      if (j + 3 < J) {
        bf16x4_t v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (__bf16)(acc[4 * q4 + e] * sc);
        *reinterpret_cast<bf16x4_t*>(orow + j) = v;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (j + e < J) orow[j + e] = (__bf16)(acc[4 * q4 + e] * sc);
      }
    }
    // The tail (q_lat's RoPE part) once per row, by the first column block.
    if (tail > 0 && blockIdx.x == 0 && wave == 0)
      for (int e = hi32; e < tail; e += 2) orow[J + e] = tail_src[((size_t)n * H + h) * tail + e];
  }
}

// The same product with both operands staged in LDS, for K a multiple of 16
// up to 512 (the DeepSeek shapes: K = 128 for the absorption, 512 for the
// output projection). A workgroup owns one head's weight rows jb .. jb+JS-1
// (JS = 128 for K <= 256, else 64, so the slab stays within 32 KB of codes),
// reads them from HBM once with whole-line 16-byte loads and applies them to
// every token; the token rows, 64 at a time, are loaded the same way and
// quantised once per workgroup as they are staged. The grid runs head-major
// (blockIdx.x = head), so the workgroups of one head share an XCD's L2 for
// the token rows. Rows are padded by 8 bytes: the 32 rows of an 8-byte
// operand read pass then start on 32 different bank pairs (for K a multiple
// of 128). Output tiles (JS/32 row tiles x two token tiles) are dealt to the
// four waves.
constexpr int kF8MaxK = 512;
constexpr int kF8Tokens = 64;
constexpr int kF8SlabBytes = 128 * (256 + 8);      // >= 64 x (512 + 8)
constexpr int kF8TokBytes = kF8Tokens * (kF8MaxK + 8);

// kK: the contracted length when it is fixed at compile time (128 or 512:
// the index arithmetic of the staging then reduces to shifts), 0 otherwise.
template <int kK>
__global__ __launch_bounds__(256) void bmm_lds_kernel(const __bf16* __restrict__ X, const float* __restrict__ partials,
                                                     int n_parts, const uint8_t* __restrict__ W, float w_scale, int N,
                                                     int H, int K_arg, int J, int JS_arg, __bf16* __restrict__ out,
                                                     int out_stride, const __bf16* __restrict__ tail_src, int tail,
                                                     int vec_out) {
  const int K = kK ? kK : K_arg;
  const int JS = kK ? (kK <= 256 ? 128 : 64) : JS_arg;
  __shared__ float red[4];
  __shared__ __attribute__((aligned(16))) char sw[kF8SlabBytes];
  __shared__ __attribute__((aligned(16))) char sx[kF8TokBytes];
  float r = 1.f;  // the activation's quantisation factor, reduced once the first loads are in flight

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r32 = lane & 31, hi32 = lane >> 5;
  const int h = blockIdx.x;
  const int jb = blockIdx.y * JS;
  const int S = K + 8;        // LDS row stride of both operands, bytes
  const int wp = K / 16;      // 16-byte pieces per weight row (16 codes each)
  const int xp = K / 8;       // 16-byte pieces per token row (8 bf16 each)

  // Staging, all loads of a round issued before any LDS write: the weight
  // slab (at most 2048 pieces of 16 bytes, 8 per thread) and the token rows
  // (at most 64 x 64 pieces, 16 per thread).
  auto load_tokens = [&](int n0, bf16x8_t (&v)[16]) {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int idx = u * 256 + tid;
      if (idx < kF8Tokens * xp) {
        const int row = idx / xp, p = idx - (idx / xp) * xp;
        v[u] = *reinterpret_cast<const bf16x8_t*>(X + ((size_t)min(n0 + row, N - 1) * H + h) * K + 8 * p);
      }
    }
  };
  // Quantised exactly as quantize_kernel does.
  auto store_tokens = [&](const bf16x8_t (&v)[16]) {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int idx = u * 256 + tid;
      if (idx < kF8Tokens * xp) {
        const int row = idx / xp, p = idx - (idx / xp) * xp;
        const uint32_t lo =
            e4m3_pair((float)v[u][0] * r, (float)v[u][1] * r) | (e4m3_pair((float)v[u][2] * r, (float)v[u][3] * r) << 16);
        const uint32_t hi =
            e4m3_pair((float)v[u][4] * r, (float)v[u][5] * r) | (e4m3_pair((float)v[u][6] * r, (float)v[u][7] * r) << 16);
        *reinterpret_cast<uint2*>(sx + row * S + 8 * p) = make_uint2(lo, hi);
      }
    }
  };
  {
    // Weight rows jb .. jb+JS-1 (past J: row J-1, outputs dropped).
    uint4 wv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int idx = u * 256 + tid;
      if (idx < JS * wp) {
        const int row = idx / wp, p = idx - (idx / wp) * wp;
        wv[u] = *reinterpret_cast<const uint4*>(W + ((size_t)h * J + min(jb + row, J - 1)) * K + 16 * p);
      }
    }
    bf16x8_t xv[16];
    load_tokens(0, xv);
    float m = (int)threadIdx.x < n_parts ? partials[threadIdx.x] : 0.f;
    m = block_max(m, red);
    r = m > 0.f ? 448.f / fmaxf(m, 0x1p-100f) : 1.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int idx = u * 256 + tid;
      if (idx < JS * wp) {
        const int row = idx / wp, p = idx - (idx / wp) * wp;
        *reinterpret_cast<uint2*>(sw + row * S + 16 * p) = make_uint2(wv[u].x, wv[u].y);
        *reinterpret_cast<uint2*>(sw + row * S + 16 * p + 8) = make_uint2(wv[u].z, wv[u].w);
      }
    }
    store_tokens(xv);
  }
  const float sc = (1.f / r) * w_scale;
  const int row_tiles = JS / 32;
  // vec_out (J, the output row and the base 16-byte multiples, the tail a
  // multiple of 8 of at most 128): a round's outputs are staged in sx once
  // its products are done and leave as whole 16-byte pieces of contiguous
  // row segments, and the RoPE tail moves in 16-byte pieces too; otherwise
  // each lane stores its 8-byte pieces directly.
  const int SO = 2 * JS + 16;  // staged output row stride, bytes (<= 272: fits in sx)
  const bool copy_tail = vec_out && tail > 0 && blockIdx.y == 0;
  const int tp = tail / 8;
  for (int n0 = 0; n0 < N; n0 += kF8Tokens) {
    if (n0 > 0) {
      bf16x8_t xv[16];
      load_tokens(n0, xv);
      store_tokens(xv);
    }
    constexpr int kTailPer = 4;  // 64 rows x up to 16 pieces
    bf16x8_t tv[kTailPer];
    if (copy_tail) {
#pragma unroll
      for (int u = 0; u < kTailPer; ++u) {
        const int idx = u * 256 + tid;
        const int rr = idx / 16, p = idx % 16;
        if (p < tp && n0 + rr < N)
          tv[u] = *reinterpret_cast<const bf16x8_t*>(tail_src + ((size_t)(n0 + rr) * H + h) * tail + 8 * p);
      }
    }
    __syncthreads();
    const int n_tiles = min(N - n0 + 31, kF8Tokens) / 32;
    f32x16_t outs[2];  // vec_out: this wave's tiles (at most 4 x 2 / 4 per round)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int t = wave + 4 * i;
      if (t >= row_tiles * n_tiles) break;
      const int rt = t % row_tiles, nt = t / row_tiles;
      const int j0 = jb + 32 * rt;
      const int n = n0 + 32 * nt + r32;
      if (j0 >= J) continue;
      const char* wa = sw + (32 * rt + r32) * S + 8 * hi32;
      const char* xa = sx + (32 * nt + r32) * S + 8 * hi32;
      f32x16_t acc;
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[q] = 0.f;
#pragma unroll 4
      for (int k = 0; k < K; k += 16)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(*reinterpret_cast<const long*>(wa + k),
                                                         *reinterpret_cast<const long*>(xa + k), acc, 0, 0, 0);
      if (vec_out) {
        outs[i] = acc;  // staged after every wave has read sx
      } else if (n < N) {
        __bf16* orow = out + ((size_t)n * H + h) * out_stride;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int j = j0 + 8 * q4 + 4 * hi32;
          if (j + 3 < J) {
            bf16x4_t v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (__bf16)(acc[4 * q4 + e] * sc);
            *reinterpret_cast<bf16x4_t*>(orow + j) = v;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (j + e < J) orow[j + e] = (__bf16)(acc[4 * q4 + e] * sc);
          }
        }
      }
    }
    if (vec_out) {
      __syncthreads();  // every wave has read its token rows: sx takes the outputs
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int t = wave + 4 * i;
        if (t >= row_tiles * n_tiles) break;
        const int rt = t % row_tiles, nt = t / row_tiles;
        if (jb + 32 * rt >= J) continue;
        char* const srow = sx + (32 * nt + r32) * SO + 64 * rt;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          bf16x4_t v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (__bf16)(outs[i][4 * q4 + e] * sc);
          *reinterpret_cast<bf16x4_t*>(srow + 2 * (8 * q4 + 4 * hi32)) = v;
        }
      }
      __syncthreads();
      const int pieces = JS / 8;  // 16-byte pieces per staged row
#pragma unroll
      for (int u = 0; u < kF8Tokens * 16 / 256; ++u) {
        const int idx = u * 256 + tid;
        const int rr = idx / 16, p = idx % 16;
        if (p < pieces && n0 + rr < N && jb + 8 * p < J)
          *reinterpret_cast<bf16x8_t*>(out + ((size_t)(n0 + rr) * H + h) * out_stride + jb + 8 * p) =
              *reinterpret_cast<const bf16x8_t*>(sx + rr * SO + 16 * p);
      }
      if (copy_tail) {
#pragma unroll
        for (int u = 0; u < kTailPer; ++u) {
          const int idx = u * 256 + tid;
          const int rr = idx / 16, p = idx % 16;
          if (p < tp && n0 + rr < N)
            *reinterpret_cast<bf16x8_t*>(out + ((size_t)(n0 + rr) * H + h) * out_stride + J + 8 * p) = tv[u];
        }
      }
    }
    __syncthreads();  // before the next token rows overwrite sx
  }
  if (tail > 0 && !vec_out && blockIdx.y == 0)
    for (int idx = tid; idx < N * tail; idx += 256) {
      const int n = idx / tail, e = idx - (idx / tail) * tail;
      out[((size_t)n * H + h) * out_stride + J + e] = tail_src[((size_t)n * H + h) * tail + e];
    }
}

}  // namespace

int amax_parts(size_t n);

hipError_t launch_quantize_e4m3(const void* x, size_t n, float* partials, uint8_t* codes, float* scale,
                                hipStream_t stream) {
  const int parts = amax_parts(n);
  hipLaunchKernelGGL(amax_kernel, dim3((unsigned)parts), dim3(kAmaxThreads), 0, stream,
                     static_cast<const __bf16*>(x), n, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)parts), dim3(kAmaxThreads), 0, stream,
                     static_cast<const __bf16*>(x), n, partials, parts, codes, scale);
  return hipGetLastError();
}

int amax_parts(size_t n) {
  const size_t groups = (n / 8 + kAmaxThreads - 1) / kAmaxThreads;
  return (int)(groups < 1 ? 1 : (groups > kFp8QuantParts ? kFp8QuantParts : groups));
}

hipError_t launch_bmm_fp8(const void* X, float* partials, const uint8_t* W, float w_scale, int N, int H, int K, int J,
                          void* out, int out_stride, const void* tail_src, int tail, hipStream_t stream) {
  const size_t n = (size_t)N * H * K;
  const int parts = amax_parts(n);
  hipLaunchKernelGGL(amax_kernel, dim3((unsigned)parts), dim3(kAmaxThreads), 0, stream,
                     static_cast<const __bf16*>(X), n, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (K % 16 == 0 && K <= kF8MaxK && ((uintptr_t)W % 16) == 0 && ((uintptr_t)X % 16) == 0 &&
      ((uintptr_t)out % 8) == 0 && out_stride % 4 == 0) {
    const int JS = K <= 256 ? 128 : 64;
    const dim3 grid((unsigned)H, (unsigned)((J + JS - 1) / JS));
    auto kern = K == 128 ? bmm_lds_kernel<128> : K == 512 ? bmm_lds_kernel<512> : bmm_lds_kernel<0>;
    const int vec_out = J % 8 == 0 && out_stride % 8 == 0 && ((uintptr_t)out % 16) == 0 && tail % 8 == 0 &&
                        tail <= 128 && (tail == 0 || ((uintptr_t)tail_src % 16) == 0);
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, stream, static_cast<const __bf16*>(X), partials, parts, W, w_scale, N,
                       H, K, J, JS, static_cast<__bf16*>(out), out_stride, static_cast<const __bf16*>(tail_src), tail,
                       vec_out);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((J + 127) / 128), (unsigned)((N + 31) / 32), (unsigned)H);
  hipLaunchKernelGGL(bmm_kernel, grid, dim3(256), 0, stream, static_cast<const __bf16*>(X), partials, parts, W,
                     w_scale, N, H, K, J, static_cast<__bf16*>(out), out_stride,
                     static_cast<const __bf16*>(tail_src), tail);
  return hipGetLastError();
}

}  // namespace mla

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
// Both are out[n,h,j] = sum_k A[n,h,k] * W(h,k,j), with W read either as
// [H, J, K] (absorb, the weight row is the output index) or as [H, K, J]
// (out_uv). Three forms, chosen by shape:
//   * bf16 MFMA, operands staged in LDS (absorb at d_nope = 128, out_uv at
//     d_c <= 512): a head-major workgroup reads a slab of one head's weights
//     once and applies it to every token;
//   * bf16 MFMA with operands loaded straight from global memory (absorb at
//     other d_nope, a multiple of 16);
//   * a general fp32-LDS tile kernel for every other shape and for fp32: a
//     workgroup computes a 64 x 64 output tile of one head, staging 32-deep
//     slices of A and W in fp32; each thread owns a 4 x 4 block.
// Accumulation is fp32 in all of them.

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

// bf16 MFMA forms, used when K is a multiple of 16, J of 8 and the rows are
// 16-byte aligned (the DeepSeek shapes). Both compute out^T[j][n] =
// sum_k W(h,j,k) A[n,h,k] with v_mfma_f32_32x32x16_bf16 (A operand: 32 j x
// 16 k of W; B operand: 16 k x 32 n of the activations, 8 consecutive k per
// lane, 16-byte loads), fp32 accumulation and a bf16 result. At decode sizes
// (N = B * s_q new tokens, tens) both products are bound by reading the
// weights (16 MiB each at H = 128), so a workgroup owns a slab of one head's
// weights, reads it from HBM once and applies it to every token; the grid
// runs head-major (blockIdx.x = head), so the workgroups of one head sit on
// one XCD and share its L2 for the activations.
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

// acc[r] = out^T[j0 + 8(r>>2) + 4*hi32 + (r&3)][n]: 8-byte stores of four
// consecutive j of row n.
__device__ __forceinline__ void store_tile(const f32x16_t& acc, __bf16* orow, int j0, int hi32, int J) {
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
}

// acc (as in store_tile) into an LDS row of bf16 outputs: the lane's four
// 8-byte pieces at columns 8q4 + 4*hi32 of the tile's 32.
__device__ __forceinline__ void stage_tile(const f32x16_t& acc, char* srow, int hi32) {
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    bf16x4_t v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (__bf16)acc[4 * q4 + e];
    *reinterpret_cast<bf16x4_t*>(srow + 2 * (8 * q4 + 4 * hi32)) = v;
  }
}

// absorb_q, W as [H, J, K] (a weight row per output j, k contiguous): grid
// (H, ceil(J/128)), wave w owns rows jb + 32w .. +31 and walks the tokens 32
// at a time. Its A fragments are 16-byte loads straight from the weight rows
// (re-read per token tile from L1/L2; HBM sees each weight once). The first
// column slab of a head also copies the RoPE tail of its rows.
__global__ __launch_bounds__(256) void absorb_mfma_kernel(const __bf16* __restrict__ A, const __bf16* __restrict__ W,
                                                         int N, int H, int K, int J, __bf16* __restrict__ out,
                                                         int out_stride, const __bf16* __restrict__ tail_src,
                                                         int tail) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r32 = lane & 31, hi32 = lane >> 5;
  const int h = blockIdx.x;
  const int j0 = blockIdx.y * 128 + wave * 32;
  if (j0 < J) {
    const __bf16* wa = W + ((size_t)h * J + min(j0 + r32, J - 1)) * K + 8 * hi32;
    for (int n0 = 0; n0 < N; n0 += 32) {
      const int n = n0 + r32;
      const __bf16* xa = A + ((size_t)min(n, N - 1) * H + h) * K + 8 * hi32;
      f32x16_t acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
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
      if (n < N) store_tile(acc, out + ((size_t)n * H + h) * out_stride, j0, hi32, J);
    }
  }
  if (tail > 0 && blockIdx.y == 0)
    for (int idx = threadIdx.x; idx < N * tail; idx += 256) {
      const int n = idx / tail, e = idx - (idx / tail) * tail;
      out[((size_t)n * H + h) * out_stride + J + e] = tail_src[((size_t)n * H + h) * tail + e];
    }
}

// absorb_q at d_nope = 128 (K = 128, the DeepSeek shape): the same grid, but
// the workgroup stages its 128 weight rows (256 bytes each) and the token
// rows, 64 at a time, in LDS with whole-line loads (16 lanes per row) and
// reads the MFMA operands from there: the direct form above issues 32 rows x
// 32 bytes per load instruction, and its address unit, not HBM, sets its
// pace. Rows are padded to 272 bytes, so the 16 rows of a 16-byte read pass
// start on 16 different 4-bank groups.
constexpr int kAbK = 128;
constexpr int kAbStride = kAbK * 2 + 16;  // 272
constexpr int kAbTokens = 64;             // token rows staged per round

__global__ __launch_bounds__(256) void absorb_lds_kernel(const __bf16* __restrict__ A, const __bf16* __restrict__ W,
                                                        int N, int H, int J, __bf16* __restrict__ out,
                                                        int out_stride, const __bf16* __restrict__ tail_src,
                                                        int tail, int tail_vec) {
  __shared__ __attribute__((aligned(16))) char sw[128 * kAbStride];
  __shared__ __attribute__((aligned(16))) char sa[kAbTokens * kAbStride];
  __shared__ __attribute__((aligned(16))) char so[kAbTokens * kAbStride];  // the round's output rows, 128 columns
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r32 = lane & 31, hi32 = lane >> 5;
  const int h = blockIdx.x;
  const int jb = blockIdx.y * 128;
  // Token rows n0 .. n0+63 of head h (past N: row N-1, outputs dropped):
  // 16 pieces of 16 bytes per row, 4 per thread.
  constexpr int kAPieces = kAbTokens * 16 / 256;
  auto load_tokens = [&](int n0, bf16x8_t (&v)[kAPieces]) {
#pragma unroll
    for (int u = 0; u < kAPieces; ++u) {
      const int idx = u * 256 + tid;
      const int r = idx >> 4, p = idx & 15;
      v[u] = *reinterpret_cast<const bf16x8_t*>(A + ((size_t)min(n0 + r, N - 1) * H + h) * kAbK + 8 * p);
    }
  };
  auto store_tokens = [&](const bf16x8_t (&v)[kAPieces]) {
#pragma unroll
    for (int u = 0; u < kAPieces; ++u) {
      const int idx = u * 256 + tid;
      *reinterpret_cast<bf16x8_t*>(sa + (idx >> 4) * kAbStride + 16 * (idx & 15)) = v[u];
    }
  };
  // Weight rows jb .. jb+127 of head h (rows past J repeat row J-1; their
  // outputs are dropped), 8 pieces per thread, requested together with the
  // first token rows: one memory round trip before the first products.
  {
    bf16x8_t wv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int idx = u * 256 + tid;
      wv[u] = *reinterpret_cast<const bf16x8_t*>(W + ((size_t)h * J + min(jb + (idx >> 4), J - 1)) * kAbK +
                                                 8 * (idx & 15));
    }
    bf16x8_t av[kAPieces];
    load_tokens(0, av);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int idx = u * 256 + tid;
      *reinterpret_cast<bf16x8_t*>(sw + (idx >> 4) * kAbStride + 16 * (idx & 15)) = wv[u];
    }
    store_tokens(av);
  }
  const int j0 = jb + 32 * wave;
  const int w_off = (32 * wave + r32) * kAbStride + 16 * hi32;  // A operand: row j0 + r32, k 16s + 8hi32
  // The RoPE tail of the round's token rows, copied by the first column slab
  // in 16-byte pieces (tail_vec: tail a multiple of 8, 16-byte aligned rows),
  // requested before the round's products and stored after them.
  const int tp = tail_vec ? tail / 8 : 0;  // 16-byte pieces per tail row
  const bool copy_tail = tail_vec && blockIdx.y == 0;
  for (int n0 = 0; n0 < N; n0 += kAbTokens) {
    if (n0 > 0) {
      bf16x8_t av[kAPieces];
      load_tokens(n0, av);
      store_tokens(av);
    }
    constexpr int kTailPer = 4;  // pieces per thread per round: 64 rows x up to 16 pieces
    bf16x8_t tv[kTailPer];
    if (copy_tail) {
#pragma unroll
      for (int u = 0; u < kTailPer; ++u) {
        const int idx = u * 256 + tid;
        const int r = idx / 16, p = idx % 16;
        if (p < tp && n0 + r < N)
          tv[u] = *reinterpret_cast<const bf16x8_t*>(tail_src + ((size_t)(n0 + r) * H + h) * tail + 8 * p);
      }
    }
    __syncthreads();
    if (j0 < J) {
      bf16x8_t wf[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) wf[s] = *reinterpret_cast<const bf16x8_t*>(sw + w_off + 32 * s);
#pragma unroll
      for (int t = 0; t < kAbTokens / 32; ++t) {
        if (n0 + 32 * t >= N) break;
        f32x16_t acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(sa + (32 * t + r32) * kAbStride + 16 * hi32 + 32 * s);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[s], b, acc, 0, 0, 0);
        }
        stage_tile(acc, so + (32 * t + r32) * kAbStride + 64 * wave, hi32);
      }
    }
    __syncthreads();
    // The round's output rows leave as whole 16-byte pieces, 256 contiguous
    // bytes per token row (written from the MFMA layout, each store would
    // cover 32 rows with 16 bytes each: measured 2.8 us slower at N = 64).
#pragma unroll
    for (int u = 0; u < kAbTokens * 16 / 256; ++u) {
      const int idx = u * 256 + tid;
      const int r = idx >> 4, p = idx & 15;
      if (n0 + r < N && jb + 8 * p < J)
        *reinterpret_cast<bf16x8_t*>(out + ((size_t)(n0 + r) * H + h) * out_stride + jb + 8 * p) =
            *reinterpret_cast<const bf16x8_t*>(so + r * kAbStride + 16 * p);
    }
    if (copy_tail) {
#pragma unroll
      for (int u = 0; u < kTailPer; ++u) {
        const int idx = u * 256 + tid;
        const int r = idx / 16, p = idx % 16;
        if (p < tp && n0 + r < N)
          *reinterpret_cast<bf16x8_t*>(out + ((size_t)(n0 + r) * H + h) * out_stride + J + 8 * p) = tv[u];
      }
    }
    __syncthreads();  // before the next token rows overwrite sa
  }
  if (tail > 0 && !tail_vec && blockIdx.y == 0)
    for (int idx = tid; idx < N * tail; idx += 256) {
      const int n = idx / tail, e = idx - (idx / tail) * tail;
      out[((size_t)n * H + h) * out_stride + J + e] = tail_src[((size_t)n * H + h) * tail + e];
    }
}

// out_uv, W as [H, K, J] (a weight row per contracted k, j contiguous): grid
// (H, ceil(J/64)). The workgroup stages its 64-column slab of the head's
// weights (K <= 512 rows of 128 bytes, 64 KB) and the token rows (up to 64
// at a time, K elements each) in LDS, both with whole-line 16-byte loads
// issued in one round, then reads the weights transposed
// (ds_read_b64_tr_b16) as the A operand and the token rows as the B operand.
// Weight row r keeps its two 64-byte halves swapped when bit 1 of r is set,
// so the four rows of a 32-lane transposed read start on four different
// 16-bank groups; token rows are padded to K*2 + 16 bytes. Output tiles (two
// 32-column halves x token tiles of 32) are dealt to the four waves.
constexpr int kUvRows = 512;    // weight rows (contracted k) one workgroup stages
constexpr int kUvTokens = 64;   // token rows staged per round
constexpr int kUvAStride = kUvRows * 2 + 16;  // 1040
constexpr int kUvOStride = 64 * 2 + 16;       // 144: a staged output row

__global__ __launch_bounds__(256) void out_uv_mfma_kernel(const __bf16* __restrict__ A, const __bf16* __restrict__ W,
                                                         int N, int H, int K, int J, __bf16* __restrict__ out,
                                                         int out_stride) {
  __shared__ __attribute__((aligned(16))) char smem[kUvRows * 128 + kUvTokens * kUvAStride + kUvTokens * kUvOStride];
  char* const sa = smem + kUvRows * 128;
  char* const so = sa + kUvTokens * kUvAStride;  // the round's output rows, 64 columns
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r32 = lane & 31, hi32 = lane >> 5;
  const int h = blockIdx.x;
  const int jb = blockIdx.y * 64;
  const __bf16* Wh = W + (size_t)h * K * J;
  const int kp = K / 8;  // 16-byte pieces per token row (K is a multiple of 16)

  // Token rows n0 .. n0+63 of head h (past N: row N-1, outputs dropped).
  constexpr int kAPieces = kUvTokens * (kUvRows / 8) / 256;  // 16 per thread at K = 512
  auto load_tokens = [&](int n0, bf16x8_t (&v)[kAPieces]) {
#pragma unroll
    for (int u = 0; u < kAPieces; ++u) {
      const int idx = u * 256 + tid;
      const int r = idx / (kUvRows / 8), p = idx % (kUvRows / 8);
      if (p < kp) v[u] = *reinterpret_cast<const bf16x8_t*>(A + ((size_t)min(n0 + r, N - 1) * H + h) * K + 8 * p);
    }
  };
  auto store_tokens = [&](const bf16x8_t (&v)[kAPieces]) {
#pragma unroll
    for (int u = 0; u < kAPieces; ++u) {
      const int idx = u * 256 + tid;
      const int r = idx / (kUvRows / 8), p = idx % (kUvRows / 8);
      if (p < kp) *reinterpret_cast<bf16x8_t*>(sa + r * kUvAStride + 16 * p) = v[u];
    }
  };
  // Weight slab: piece p (16 bytes, columns jb + 8p .. +7) of row k; rows
  // past K are zero, columns past J repeat column J-1 (their outputs are
  // dropped). Requested together with the first token rows.
  {
    constexpr int kWPieces = kUvRows * 8 / 256;  // 16 per thread
    bf16x8_t wv[kWPieces];
#pragma unroll
    for (int u = 0; u < kWPieces; ++u) {
      const int idx = u * 256 + tid;
      const int k = idx >> 3, p = idx & 7;
      if (k < K && jb + 8 * p + 7 < J) {
        wv[u] = *reinterpret_cast<const bf16x8_t*>(Wh + (size_t)k * J + jb + 8 * p);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) wv[u][e] = k < K ? Wh[(size_t)k * J + min(jb + 8 * p + e, J - 1)] : (__bf16)0.f;
      }
    }
    bf16x8_t av[kAPieces];
    load_tokens(0, av);
#pragma unroll
    for (int u = 0; u < kWPieces; ++u) {
      const int idx = u * 256 + tid;
      const int k = idx >> 3, p = idx & 7;
      *reinterpret_cast<bf16x8_t*>(smem + 128 * k + 64 * ((p >> 2) ^ ((k >> 1) & 1)) + 16 * (p & 3)) = wv[u];
    }
    store_tokens(av);
  }

  // Transposed read: 16-lane group g, lane 4jj + q of the group gives k row
  // 8(g>>1) + 4rd + jj (+16 per k-step) and columns 16(g&1) + 4q .. +4 of the
  // tile's 32 columns; bit 1 of the row is bit 1 of jj.
  const int g = lane >> 4, jj = (lane >> 2) & 3, q = lane & 3;
  const int row_in = 8 * (g >> 1) + jj;
  const int col_b = 2 * (16 * (g & 1) + 4 * q);
  const int steps = K / 16;
  for (int n0 = 0; n0 < N; n0 += kUvTokens) {
    if (n0 > 0) {
      bf16x8_t av[kAPieces];
      load_tokens(n0, av);
      store_tokens(av);
    }
    __syncthreads();
    const int n_tiles = min(N - n0 + 31, kUvTokens) / 32;
    for (int t = wave; t < 2 * n_tiles; t += 4) {
      const int c = t & 1, nt = t >> 1;
      const int tr_off = 128 * row_in + 64 * (c ^ ((jj >> 1) & 1)) + col_b;
      const char* const bsrc = sa + (32 * nt + r32) * kUvAStride + 16 * hi32;  // B operand: token n, k 16s + 8hi32
      f32x16_t acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll 4
      for (int s4 = 0; s4 < steps; ++s4) {
        bf16x8_t a;
#pragma unroll
        for (int rd = 0; rd < 2; ++rd) {
          const bf16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (lds_bf16x4_t*)((__attribute__((address_space(3))) char*)smem + tr_off + 128 * (16 * s4 + 4 * rd)));
          a[4 * rd + 0] = v[0]; a[4 * rd + 1] = v[1]; a[4 * rd + 2] = v[2]; a[4 * rd + 3] = v[3];
        }
        const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(bsrc + 32 * s4);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
      }
      stage_tile(acc, so + (32 * nt + r32) * kUvOStride + 64 * c, hi32);
    }
    __syncthreads();
    // Whole 16-byte pieces, 128 contiguous bytes per token row.
#pragma unroll
    for (int u = 0; u < kUvTokens * 8 / 256; ++u) {
      const int idx = u * 256 + tid;
      const int r = idx >> 3, p = idx & 7;
      if (n0 + r < N && jb + 8 * p < J)
        *reinterpret_cast<bf16x8_t*>(out + ((size_t)(n0 + r) * H + h) * out_stride + jb + 8 * p) =
            *reinterpret_cast<const bf16x8_t*>(so + r * kUvOStride + 16 * p);
    }
    __syncthreads();  // before the next token rows overwrite sa and so
  }
}

// The MFMA forms need 16-byte aligned rows: K a multiple of 16, J and the
// output row a multiple of 8 (whole 16-byte output pieces), 16-byte aligned
// bases.
bool mfma_shape(const void* A, const void* W, const void* out, int K, int J, int out_stride) {
  return K % 16 == 0 && J % 8 == 0 && out_stride % 8 == 0 && ((uintptr_t)A % 16) == 0 && ((uintptr_t)W % 16) == 0 &&
         ((uintptr_t)out % 16) == 0;
}

}  // namespace

hipError_t launch_absorb_q(const void* q_nope, const void* q_rope, const void* w_uk, int N, int H,
                           int dn, int dr, int dc, bool bf16, void* q_lat, hipStream_t stream) {
  if (bf16 && mfma_shape(q_nope, w_uk, q_lat, dn, dc, dc + dr) && dn == kAbK) {
    const dim3 grid((unsigned)H, (unsigned)((dc + 127) / 128));
    // 16-byte tail pieces: whole pieces per row (at most 16), 16-byte aligned bases and row starts.
    const int tail_vec = dr > 0 && dr % 8 == 0 && dr <= 128 && dc % 8 == 0 && (dc + dr) % 8 == 0 &&
                         ((uintptr_t)q_rope % 16) == 0 && ((uintptr_t)q_lat % 16) == 0;
    hipLaunchKernelGGL(absorb_lds_kernel, grid, dim3(256), 0, stream, static_cast<const __bf16*>(q_nope),
                       static_cast<const __bf16*>(w_uk), N, H, dc, static_cast<__bf16*>(q_lat), dc + dr,
                       static_cast<const __bf16*>(q_rope), dr, tail_vec);
    return hipGetLastError();
  }
  if (bf16 && mfma_shape(q_nope, w_uk, q_lat, dn, dc, dc + dr)) {
    const dim3 grid((unsigned)H, (unsigned)((dc + 127) / 128));
    hipLaunchKernelGGL(absorb_mfma_kernel, grid, dim3(256), 0, stream, static_cast<const __bf16*>(q_nope),
                       static_cast<const __bf16*>(w_uk), N, H, dn, dc, static_cast<__bf16*>(q_lat), dc + dr,
                       static_cast<const __bf16*>(q_rope), dr);
    return hipGetLastError();
  }
  if (bf16)
    return launch_head_bmm<__bf16, true>(q_nope, w_uk, N, H, dn, dc, q_lat, dc + dr, q_rope, dr, stream);
  return launch_head_bmm<float, true>(q_nope, w_uk, N, H, dn, dc, q_lat, dc + dr, q_rope, dr, stream);
}

hipError_t launch_out_uv(const void* o_lat, const void* w_uv, int N, int H, int dc, int dv,
                         bool bf16, void* out, hipStream_t stream) {
  if (bf16 && mfma_shape(o_lat, w_uv, out, dc, dv, dv) && dc <= kUvRows) {
    const dim3 grid((unsigned)H, (unsigned)((dv + 63) / 64));
    hipLaunchKernelGGL(out_uv_mfma_kernel, grid, dim3(256), 0, stream, static_cast<const __bf16*>(o_lat),
                       static_cast<const __bf16*>(w_uv), N, H, dc, dv, static_cast<__bf16*>(out), dv);
    return hipGetLastError();
  }
  if (bf16)
    return launch_head_bmm<__bf16, false>(o_lat, w_uv, N, H, dc, dv, out, dv, nullptr, 0, stream);
  return launch_head_bmm<float, false>(o_lat, w_uv, N, H, dc, dv, out, dv, nullptr, 0, stream);
}

}  // namespace mla

// LSE merge of split-KV partial results, gfx950.
//
// "MLA 推理：两条计算路径与 FlashMLA", sections "谁快：看新 token 和缓存 token 的
// 数量" and "decode 注意力变成了计算问题": chunk results are merged by their
// log-sum-exp. For one (sequence, token, head) row with chunks k:
//   M = max_k lse_k, lse = M + ln sum_k exp(lse_k - M),
//   o = sum_k exp(lse_k - lse) o_k,
// and a chunk with lse_k = -inf (no allowed key) adds nothing.
//
// One wave per row: lane k < n reads lse_k, two wave reductions give M and
// the sum, and every lane owns 8 of the 512 columns of the chunks' partial
// rows (in the output dtype: bf16 or fp32), read eight chunks at a time, the
// first eight together with the LSEs.

#include <hip/hip_runtime.h>
#include <cmath>
#include <cstdint>

#include "mla_internal.h"

namespace mla {
namespace {

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;

constexpr int kWaves = 4;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <bool kBf16>
__global__ __launch_bounds__(64 * kWaves) void combine_kernel(const void* __restrict__ o_part,
                                                              const float* __restrict__ lse_part,
                                                              const int32_t* __restrict__ split_offsets,
                                                              int rows, int total_splits,
                                                              int skip_single, void* o_lat, float* lse) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x;
  const int row = blockIdx.y * kWaves + (threadIdx.x >> 6);
  if (row >= rows) return;
  // Clamp so that malformed offsets can never index outside the partials.
  const int s0 = min(max(split_offsets[b], 0), total_splits);
  const int n = min(min(max(split_offsets[b + 1] - s0, 0), kMaxSplits), total_splits - s0);
  if (n == 0 || (skip_single && n == 1)) return;

  // Lane l owns columns 8l .. 8l+7. The first eight chunks' rows are
  // requested together with the LSEs (they do not depend on the weights),
  // so the two loads' latencies overlap; later chunks follow eight at a time.
  float v[8][8];
  const auto load_round = [&](int k0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = k0 + j;
      if (k < n) {
        const size_t off = ((size_t)(s0 + k) * rows + row) * kDv + 8 * lane;
        if (kBf16) {
          const bf16x8_t x = *reinterpret_cast<const bf16x8_t*>(static_cast<const __bf16*>(o_part) + off);
#pragma unroll
          for (int e = 0; e < 8; ++e) v[j][e] = (float)x[e];
        } else {
          const f32x4_t* src = reinterpret_cast<const f32x4_t*>(static_cast<const float*>(o_part) + off);
          const f32x4_t x0 = src[0], x1 = src[1];
#pragma unroll
          for (int e = 0; e < 4; ++e) { v[j][e] = x0[e]; v[j][4 + e] = x1[e]; }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[j][e] = 0.f;
      }
    }
  };
  const float lk = lane < n ? lse_part[(size_t)(s0 + lane) * rows + row] : -INFINITY;
  load_round(0);
  const float M = wave_max(lk);
  const float Mf = (M == -INFINITY) ? 0.f : M;
  const float w = (lane < n) ? expf(lk - Mf) : 0.f;
  const float S = wave_sum(w);
  const float lse_v = (S > 0.f) ? Mf + logf(S) : -INFINITY;
  const float wn = (S > 0.f) ? w / S : 0.f;  // exp(lse_k - lse); lanes >= n hold 0

  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < n; k0 += 8) {
    if (k0 > 0) load_round(k0);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float wk = __shfl(wn, (k0 + j) & 63, 64);  // 0 past n
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(wk, v[j][e], acc[e]);
    }
  }
  if (kBf16) {
    bf16x8_t o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (__bf16)acc[e];
    *(reinterpret_cast<bf16x8_t*>(reinterpret_cast<__bf16*>(o_lat) + ((size_t)b * rows + row) * kDv) + lane) = o;
  } else {
    f32x4_t* dst = reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(o_lat) + ((size_t)b * rows + row) * kDv) + 2 * lane;
    dst[0] = f32x4_t{acc[0], acc[1], acc[2], acc[3]};
    dst[1] = f32x4_t{acc[4], acc[5], acc[6], acc[7]};
  }
  if (lane == 0) lse[(size_t)b * rows + row] = lse_v;
}

// Many chunks per sequence (long contexts, small batches): one workgroup per
// row, its four waves take every fourth chunk (eight per round, the first
// round issued with the LSE loads), and the four partial sums meet in LDS. Each wave then waits on a quarter of the chunk loads, and the
// grid has four times the waves of the row-per-wave form. The weights and
// the summation order of each wave's share are those of the row-per-wave
// form; only the final four-way sum is added.
template <bool kBf16>
__global__ __launch_bounds__(64 * kWaves) void combine_wide_kernel(const void* __restrict__ o_part,
                                                                   const float* __restrict__ lse_part,
                                                                   const int32_t* __restrict__ split_offsets,
                                                                   int rows, int total_splits, int skip_single,
                                                                   void* o_lat, float* lse) {
  __shared__ float part[kWaves - 1][kDv];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int b = blockIdx.x;
  const int row = blockIdx.y;
  const int s0 = min(max(split_offsets[b], 0), total_splits);
  const int n = min(min(max(split_offsets[b + 1] - s0, 0), kMaxSplits), total_splits - s0);
  if (n == 0 || (skip_single && n == 1)) return;  // uniform over the workgroup

  // This wave's chunks: wave, wave + 4, ..., eight per round, the first
  // round requested together with the LSEs.
  constexpr int kPer = 8;
  float v[kPer][8];
  const auto load_round = [&](int k0) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int k = k0 + kWaves * j;
      if (k < n) {
        const size_t off = ((size_t)(s0 + k) * rows + row) * kDv + 8 * lane;
        if (kBf16) {
          const bf16x8_t x = *reinterpret_cast<const bf16x8_t*>(static_cast<const __bf16*>(o_part) + off);
#pragma unroll
          for (int e = 0; e < 8; ++e) v[j][e] = (float)x[e];
        } else {
          const f32x4_t* src = reinterpret_cast<const f32x4_t*>(static_cast<const float*>(o_part) + off);
          const f32x4_t x0 = src[0], x1 = src[1];
#pragma unroll
          for (int e = 0; e < 4; ++e) { v[j][e] = x0[e]; v[j][4 + e] = x1[e]; }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[j][e] = 0.f;
      }
    }
  };
  const float lk = lane < n ? lse_part[(size_t)(s0 + lane) * rows + row] : -INFINITY;
  load_round(wave);
  const float M = wave_max(lk);
  const float Mf = (M == -INFINITY) ? 0.f : M;
  const float w = (lane < n) ? expf(lk - Mf) : 0.f;
  const float S = wave_sum(w);
  const float lse_v = (S > 0.f) ? Mf + logf(S) : -INFINITY;
  const float wn = (S > 0.f) ? w / S : 0.f;

  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int k0 = wave; k0 < n; k0 += kPer * kWaves) {
    if (k0 != wave) load_round(k0);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const float wk = __shfl(wn, (k0 + kWaves * j) & 63, 64);  // 0 past n
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(wk, v[j][e], acc[e]);
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) part[wave - 1][8 * lane + e] = acc[e];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int q = 0; q < kWaves - 1; ++q)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += part[q][8 * lane + e];
  if (kBf16) {
    bf16x8_t o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (__bf16)acc[e];
    *(reinterpret_cast<bf16x8_t*>(reinterpret_cast<__bf16*>(o_lat) + ((size_t)b * rows + row) * kDv) + lane) = o;
  } else {
    f32x4_t* dst = reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(o_lat) + ((size_t)b * rows + row) * kDv) + 2 * lane;
    dst[0] = f32x4_t{acc[0], acc[1], acc[2], acc[3]};
    dst[1] = f32x4_t{acc[4], acc[5], acc[6], acc[7]};
  }
  if (lane == 0) lse[(size_t)b * rows + row] = lse_v;
}

}  // namespace

hipError_t launch_combine(const void* o_part, const float* lse_part, const int32_t* split_offsets,
                          int total_splits, int B, int s_q, int H, bool out_bf16, bool skip_single,
                          void* o_lat, float* lse, hipStream_t stream) {
  const int rows = s_q * H;
  if (total_splits >= 8 * B && rows <= 65535) {
    // Eight or more chunks per sequence on average: one workgroup per row.
    const dim3 grid((unsigned)B, (unsigned)rows);
    if (out_bf16)
      hipLaunchKernelGGL(combine_wide_kernel<true>, grid, dim3(64 * kWaves), 0, stream, o_part, lse_part,
                         split_offsets, rows, total_splits, skip_single ? 1 : 0, o_lat, lse);
    else
      hipLaunchKernelGGL(combine_wide_kernel<false>, grid, dim3(64 * kWaves), 0, stream, o_part, lse_part,
                         split_offsets, rows, total_splits, skip_single ? 1 : 0, o_lat, lse);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)B, (unsigned)((rows + kWaves - 1) / kWaves));
  if (out_bf16)
    hipLaunchKernelGGL(combine_kernel<true>, grid, dim3(64 * kWaves), 0, stream, o_part, lse_part,
                       split_offsets, rows, total_splits, skip_single ? 1 : 0, o_lat, lse);
  else
    hipLaunchKernelGGL(combine_kernel<false>, grid, dim3(64 * kWaves), 0, stream, o_part, lse_part,
                       split_offsets, rows, total_splits, skip_single ? 1 : 0, o_lat, lse);
  return hipGetLastError();
}

}  // namespace mla

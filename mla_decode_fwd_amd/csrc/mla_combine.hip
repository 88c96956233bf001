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
// first eight together with the LSEs. The loaded rows are kept as raw 16-byte
// words and widened to fp32 only where they are summed, so that the wave
// does not wait on a chunk's load until its weight is known (widening at the
// load made the compiler wait on each load in turn: ~1 us more per merge on
// MI355X for 4 chunks per row, ~2 us for 64).

#include <hip/hip_runtime.h>
#include <cmath>
#include <cstdint>

#include "mla_internal.h"

namespace mla {
namespace {

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;

constexpr int kWaves = 4;
constexpr int kRound = 8;  // chunk rows requested together by one wave

typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4_t;

// One chunk's 8 columns of this lane: one 16-byte word (bf16) or two (fp32).
template <bool kBf16>
struct RawRow {
  u32x4_t w[kBf16 ? 1 : 2];
};

// Each partial is read exactly once, so the loads are non-temporal (measured
// on MI355X: the long-context step, decode plus merge, is 1.8-2.2 us shorter,
// the single-sequence step 0.5 us; B=64 x 4096 unchanged).
template <bool kBf16>
__device__ __forceinline__ RawRow<kBf16> load_row(const void* o_part, size_t off) {
  RawRow<kBf16> r;
  if constexpr (kBf16) {
    r.w[0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(static_cast<const __bf16*>(o_part) + off));
  } else {
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(static_cast<const float*>(o_part) + off);
    r.w[0] = __builtin_nontemporal_load(src);
    r.w[1] = __builtin_nontemporal_load(src + 1);
  }
  return r;
}

template <bool kBf16>
__device__ __forceinline__ RawRow<kBf16> zero_row() {
  RawRow<kBf16> r;
#pragma unroll
  for (int i = 0; i < (kBf16 ? 1 : 2); ++i) r.w[i] = u32x4_t{0u, 0u, 0u, 0u};
  return r;
}

// acc += wk * row, the row widened to fp32 (a bf16 is the high half of its fp32).
template <bool kBf16>
__device__ __forceinline__ void fma_row(float (&acc)[8], float wk, const RawRow<kBf16>& r) {
  float x[8];
  if constexpr (kBf16) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __uint_as_float(r.w[0][e] << 16);
      x[2 * e + 1] = __uint_as_float(r.w[0][e] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = __uint_as_float(r.w[0][e]);
      x[4 + e] = __uint_as_float(r.w[1][e]);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = fmaf(wk, x[e], acc[e]);
}

template <bool kBf16>
__device__ __forceinline__ void store_row(void* o_lat, size_t row_off, int lane, const float (&acc)[8]) {
  if constexpr (kBf16) {
    bf16x8_t o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (__bf16)acc[e];
    *(reinterpret_cast<bf16x8_t*>(reinterpret_cast<__bf16*>(o_lat) + row_off) + lane) = o;
  } else {
    f32x4_t* dst = reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(o_lat) + row_off) + 2 * lane;
    dst[0] = f32x4_t{acc[0], acc[1], acc[2], acc[3]};
    dst[1] = f32x4_t{acc[4], acc[5], acc[6], acc[7]};
  }
}

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
                                                              int skip_single, int rows_fast, void* o_lat,
                                                              float* lse) {
  const int lane = threadIdx.x & 63;
  const int b = rows_fast ? blockIdx.y : blockIdx.x;
  const int row = (rows_fast ? blockIdx.x : blockIdx.y) * kWaves + (threadIdx.x >> 6);
  if (row >= rows) return;
  // Clamp so that malformed offsets can never index outside the partials.
  const int s0 = min(max(split_offsets[b], 0), total_splits);
  const int n = min(min(max(split_offsets[b + 1] - s0, 0), kMaxSplits), total_splits - s0);
  if (n == 0 || (skip_single && n == 1)) return;

  // Lane l owns columns 8l .. 8l+7. The first round's chunk rows are
  // requested together with the LSEs (they do not depend on the weights),
  // so the two loads' latencies overlap; later chunks follow a round at a time.
  RawRow<kBf16> v[kRound];
  const auto load_round = [&](int k0) {
#pragma unroll
    for (int j = 0; j < kRound; ++j) {
      const int k = k0 + j;
      v[j] = k < n ? load_row<kBf16>(o_part, ((size_t)(s0 + k) * rows + row) * kDv + 8 * lane) : zero_row<kBf16>();
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
  for (int k0 = 0; k0 < n; k0 += kRound) {
    if (k0 > 0) load_round(k0);
#pragma unroll
    for (int j = 0; j < kRound; ++j) fma_row<kBf16>(acc, __shfl(wn, (k0 + j) & 63, 64), v[j]);  // 0 past n
  }
  store_row<kBf16>(o_lat, ((size_t)b * rows + row) * kDv, lane, acc);
  if (lane == 0) lse[(size_t)b * rows + row] = lse_v;
}

// Many chunks per sequence (long contexts, small batches): one workgroup per
// row, its four waves take every fourth chunk (a round of eight at a time,
// the first round issued with the LSE loads), and the four partial sums meet
// in LDS. Each wave then waits on a quarter of the chunk loads, and the grid
// has four times the waves of the row-per-wave form. The weights and the
// summation order of each wave's share are those of the row-per-wave form;
// only the final four-way sum is added.
template <bool kBf16>
__global__ __launch_bounds__(64 * kWaves) void combine_wide_kernel(const void* __restrict__ o_part,
                                                                   const float* __restrict__ lse_part,
                                                                   const int32_t* __restrict__ split_offsets,
                                                                   int rows, int total_splits, int skip_single,
                                                                   int rows_fast, void* o_lat, float* lse) {
  __shared__ float part[kWaves - 1][kDv];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int b = rows_fast ? blockIdx.y : blockIdx.x;
  const int row = rows_fast ? blockIdx.x : blockIdx.y;
  const int s0 = min(max(split_offsets[b], 0), total_splits);
  const int n = min(min(max(split_offsets[b + 1] - s0, 0), kMaxSplits), total_splits - s0);
  if (n == 0 || (skip_single && n == 1)) return;  // uniform over the workgroup

  // This wave's chunks: wave, wave + 4, ..., a round of eight at a time.
  RawRow<kBf16> v[kRound];
  const auto load_round = [&](int k0) {
#pragma unroll
    for (int j = 0; j < kRound; ++j) {
      const int k = k0 + kWaves * j;
      v[j] = k < n ? load_row<kBf16>(o_part, ((size_t)(s0 + k) * rows + row) * kDv + 8 * lane) : zero_row<kBf16>();
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
  for (int k0 = wave; k0 < n; k0 += kRound * kWaves) {
    if (k0 != wave) load_round(k0);
#pragma unroll
    for (int j = 0; j < kRound; ++j) fma_row<kBf16>(acc, __shfl(wn, (k0 + kWaves * j) & 63, 64), v[j]);
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
  store_row<kBf16>(o_lat, ((size_t)b * rows + row) * kDv, lane, acc);
  if (lane == 0) lse[(size_t)b * rows + row] = lse_v;
}

}  // namespace

hipError_t launch_combine(const void* o_part, const float* lse_part, const int32_t* split_offsets,
                          int total_splits, int B, int s_q, int H, bool out_bf16, bool skip_single,
                          void* o_lat, float* lse, hipStream_t stream) {
  const int rows = s_q * H;
  // Grid: (row block, sequence), rows fastest. Workgroups are dealt to the
  // eight XCDs round robin in launch order, so the rows of one sequence
  // spread over all of them; with the sequence fastest, every row of
  // sequence b would go to XCD b mod 8, and one long sequence with many
  // chunks would load a single XCD (measured on MI355X: the merge of eight
  // sequences of 65536 ... 513 tokens took 9.6 us that way). The sequence
  // index goes in y while it fits there (B <= 65535), else in x.
  const bool wide = total_splits >= 8 * B && rows <= 65535;  // >= 8 chunks per sequence on average
  const unsigned row_blocks = wide ? (unsigned)rows : (unsigned)((rows + kWaves - 1) / kWaves);
  const bool rows_fast = B <= 65535;
  const dim3 grid = rows_fast ? dim3(row_blocks, (unsigned)B) : dim3((unsigned)B, row_blocks);
  const int rf = rows_fast ? 1 : 0, ss = skip_single ? 1 : 0;
  if (wide) {
    // One workgroup per row.
    if (out_bf16)
      hipLaunchKernelGGL(combine_wide_kernel<true>, grid, dim3(64 * kWaves), 0, stream, o_part, lse_part,
                         split_offsets, rows, total_splits, ss, rf, o_lat, lse);
    else
      hipLaunchKernelGGL(combine_wide_kernel<false>, grid, dim3(64 * kWaves), 0, stream, o_part, lse_part,
                         split_offsets, rows, total_splits, ss, rf, o_lat, lse);
    return hipGetLastError();
  }
  if (out_bf16)
    hipLaunchKernelGGL(combine_kernel<true>, grid, dim3(64 * kWaves), 0, stream, o_part, lse_part,
                       split_offsets, rows, total_splits, ss, rf, o_lat, lse);
  else
    hipLaunchKernelGGL(combine_kernel<false>, grid, dim3(64 * kWaves), 0, stream, o_part, lse_part,
                       split_offsets, rows, total_splits, ss, rf, o_lat, lse);
  return hipGetLastError();
}

}  // namespace mla

// The expanded path of MLA for prefill and extend, gfx950.
//
// "MLA 推理：两条计算路径与 FlashMLA", section "两条等价的路径" (path one: expand
// the cached latent into per-head keys k^N = c W_UK[h] and values
// v = c W_UV[h], attach the shared RoPE key, run ordinary multi-head
// attention with scale 1/sqrt(nope + rope)) and section "谁快：看新 token 和缓存
// token 的数量" (prefill and extend pay the expansion once per cached token;
// with a long prefix the prefix is expanded chunk by chunk, attention runs
// per chunk, and the chunk results are merged by their LSE).
//
// Three kernels; the host walks a sequence's cached tokens in chunks:
//   expand_kernel   K[h, j, 0:128] = c_j W_UK[h],  K[h, j, 128:192] = k^R_j,
//                   V[h, j, 0:128] = c_j W_UV[h]   for the chunk's tokens j
//                   (c_j and k^R_j read from the paged cache).
//   attn_kernel     causal attention of the s_q new tokens (the last s_q of
//                   the sequence) over the chunk's keys, per head: o and LSE,
//                   or the chunk's partial o and LSE.
//   merge_kernel    LSE merge of the chunk partials.
// All products are v_mfma_f32_32x32x16_bf16 with fp32 accumulation.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "mla_decode_common.h"
#include "mla_internal.h"

namespace mla {
namespace {

using namespace dec;

typedef __attribute__((address_space(3))) bf16x4_t lds_b4_t;

constexpr int kNope = 128;             // per-head key (no RoPE) and value widths
constexpr int kRope = 64;
constexpr int kHeadK = kNope + kRope;  // 192
constexpr int kHeadV = 128;
constexpr int kLat = 512;              // latent width d_c

// ---------------------------------------------------------------------------
// expand_kernel: one workgroup per (128 tokens, head, K or V). Wave w takes
// tokens 32w..32w+31 and all 128 output columns. The latent rows are the B
// operand (k-steps of 16 over 512, in registers: 32 x 4 VGPRs); the weight
// slice of 64 latent rows x 128 columns is staged in LDS (320-byte rows) and
// read transposed (ds_read_b64_tr_b16) as the A operand, giving
// D^T[column][token].
// ---------------------------------------------------------------------------
constexpr int kExpRows = 128;
constexpr int kWSlice = 64;                    // latent rows per weight slice
constexpr int kWStride = kNope * 2 + 64;       // 320: LDS row stride of a slice
constexpr int kWBuf = kWSlice * kWStride;      // 20,480

__global__ __launch_bounds__(kThreads, 1) void expand_kernel(const __bf16* __restrict__ cache,
                                                            const int32_t* __restrict__ btab_row, int t0, int n,
                                                            int num_pages, const __bf16* __restrict__ w_uk,
                                                            const __bf16* __restrict__ w_uv, int H,
                                                            __bf16* __restrict__ k_out, __bf16* __restrict__ v_out,
                                                            int n_stride) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kWBuf];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r32 = lane & 31, hi32 = lane >> 5;
  const int h = blockIdx.y;
  const bool is_v = blockIdx.z == 1;
  const __bf16* W = (is_v ? w_uv : w_uk) + (size_t)h * kLat * kNope;  // [512][128]

  const int j = blockIdx.x * kExpRows + wave * kWaveRows + r32;  // chunk-local token of this lane
  const int jc = min(j, n - 1);
  const int pos = t0 + jc;                                          // position in the sequence
  const int phys = min(max(btab_row[pos / kPage], 0), num_pages - 1);
  const __bf16* crow = cache + ((size_t)phys * kPage + (pos % kPage)) * kDqk;

  bf16x8_t af[kLat / 16];
#pragma unroll
  for (int s = 0; s < kLat / 16; ++s) af[s] = *reinterpret_cast<const bf16x8_t*>(crow + 16 * s + 8 * hi32);

  // Weight slice staging: 64 rows x 256 bytes = 1024 chunks of 16 bytes, 4 per thread.
  auto load_slice = [&](int ks, u32x4_t (&r)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = u * kThreads + (int)threadIdx.x;
      const int row = idx >> 4, c16 = idx & 15;
      r[u] = *reinterpret_cast<const u32x4_t*>(W + (size_t)(ks * kWSlice + row) * kNope + 8 * c16);
    }
  };
  auto store_slice = [&](char* buf, const u32x4_t (&r)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = u * kThreads + (int)threadIdx.x;
      const int row = idx >> 4, c16 = idx & 15;
      *reinterpret_cast<u32x4_t*>(buf + row * kWStride + 16 * c16) = r[u];
    }
  };

  f32x16_t acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;

  // Transposed read: 16-lane group g, input lane 4jj + q: latent row
  // 16s + 8(g>>1) + 4rd + jj, columns 32ct + 16(g&1) + 4q .. +4.
  const int g = lane >> 4, jj = (lane >> 2) & 3, q = lane & 3;
  const int tr_off = kWStride * (8 * (g >> 1) + jj) + 2 * (16 * (g & 1) + 4 * q);

  u32x4_t pre[4];
  load_slice(0, pre);
  constexpr int kSlices = kLat / kWSlice;  // 8
  for (int ks = 0; ks < kSlices; ++ks) {
    char* buf = smem + (ks & 1) * kWBuf;
    store_slice(buf, pre);
    __syncthreads();
    if (ks + 1 < kSlices) load_slice(ks + 1, pre);
#pragma unroll
    for (int s4 = 0; s4 < kWSlice / 16; ++s4) {
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        bf16x8_t wf;
#pragma unroll
        for (int rd = 0; rd < 2; ++rd) {
          const bf16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (lds_b4_t*)((__attribute__((address_space(3))) char*)buf + tr_off + kWStride * (16 * s4 + 4 * rd) +
                          64 * ct));
          wf[4 * rd + 0] = v[0]; wf[4 * rd + 1] = v[1]; wf[4 * rd + 2] = v[2]; wf[4 * rd + 3] = v[3];
        }
        acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf, af[ks * 4 + s4], acc[ct], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  if (j >= n) return;
  // acc[ct][r] = D^T[32ct + 8(r>>2) + 4*hi32 + (r&3)][token j].
  __bf16* orow = is_v ? v_out + ((size_t)h * n_stride + j) * kHeadV : k_out + ((size_t)h * n_stride + j) * kHeadK;
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      bf16x4_t v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (__bf16)acc[ct][4 * q4 + e];
      *reinterpret_cast<bf16x4_t*>(orow + 32 * ct + 8 * q4 + 4 * hi32) = v;
    }
  if (!is_v) {
    // The shared RoPE key: 64 elements, 32 per lane half.
#pragma unroll
    for (int u = 0; u < 4; ++u)
      *reinterpret_cast<u32x4_t*>(orow + kNope + 32 * hi32 + 8 * u) =
          *reinterpret_cast<const u32x4_t*>(crow + kLat + 32 * hi32 + 8 * u);
  }
}

// ---------------------------------------------------------------------------
// attn_kernel: one workgroup per (128 new tokens, head); wave w takes 32 query
// rows. Q^T (12 k-steps over 192) stays in VGPRs, O^T (128 columns) in four
// 32x32 accumulators. Keys come in tiles of 32: S^T = K Q^T, base-2 online
// softmax with a lazily moved reference (as the decode kernel), O^T += V^T P^T
// with P^T taken from the score registers and V^T read transposed.
// ---------------------------------------------------------------------------
constexpr int kKStride = kHeadK * 2 + 16;   // 400: 16 consecutive keys on 16 bank groups
constexpr int kVStride = kHeadV * 2 + 64;   // 320
constexpr int kKTile = 32;
constexpr int kKBuf = kKTile * kKStride;    // 12,800
constexpr int kVBuf = kKTile * kVStride;    // 10,240
constexpr int kStage = kKBuf + kVBuf;

__global__ __launch_bounds__(kThreads, 1) void attn_kernel(const __bf16* __restrict__ q_nope,
                                                          const __bf16* __restrict__ q_rope, int s_q, int H,
                                                          const __bf16* __restrict__ K, const __bf16* __restrict__ V,
                                                          int n, int n_stride, int k_pos0, int q_pos0, int causal,
                                                          float scale, __bf16* __restrict__ o, float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kStage];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r32 = lane & 31, hi32 = lane >> 5;
  const int h = blockIdx.y;
  const int qb = blockIdx.x * kRowsPerGroup;
  const int qrow = qb + wave * kWaveRows + r32;
  const int qc = min(qrow, s_q - 1);
  const int qpos = q_pos0 + qc;

  // Q^T: k-steps 0..7 from q_nope, 8..11 from q_rope.
  bf16x8_t qf[kHeadK / 16];
  {
    const __bf16* qn = q_nope + ((size_t)qc * H + h) * kNope + 8 * hi32;
    const __bf16* qr = q_rope + ((size_t)qc * H + h) * kRope + 8 * hi32;
#pragma unroll
    for (int s = 0; s < kNope / 16; ++s) qf[s] = *reinterpret_cast<const bf16x8_t*>(qn + 16 * s);
#pragma unroll
    for (int s = 0; s < kRope / 16; ++s) qf[kNope / 16 + s] = *reinterpret_cast<const bf16x8_t*>(qr + 16 * s);
  }

  // Keys this workgroup may need: up to the last query's position.
  const int q_last = q_pos0 + min(s_q, qb + kRowsPerGroup) - 1;
  const int n_vis = causal ? max(0, min(n, q_last - k_pos0 + 1)) : n;
  const int tiles = (n_vis + kKTile - 1) / kKTile;
  const int q_first_wave = q_pos0 + min(qb + wave * kWaveRows, s_q - 1);  // smallest position in this wave

  const __bf16* Kh = K + (size_t)h * n_stride * kHeadK;
  const __bf16* Vh = V + (size_t)h * n_stride * kHeadV;
  // Tile loads: K 32 rows x 24 chunks (3 per thread), V 32 rows x 16 chunks (2 per thread).
  auto load_tile = [&](int kt, u32x4_t (&kr)[3], u32x4_t (&vr)[2]) {
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      const int idx = u * kThreads + (int)threadIdx.x;
      const int row = idx / 24, c16 = idx % 24;
      const int key = min(kt * kKTile + row, n - 1);
      kr[u] = *reinterpret_cast<const u32x4_t*>(Kh + (size_t)key * kHeadK + 8 * c16);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int idx = u * kThreads + (int)threadIdx.x;
      const int row = idx >> 4, c16 = idx & 15;
      const int key = min(kt * kKTile + row, n - 1);
      vr[u] = *reinterpret_cast<const u32x4_t*>(Vh + (size_t)key * kHeadV + 8 * c16);
    }
  };
  auto store_tile = [&](char* buf, const u32x4_t (&kr)[3], const u32x4_t (&vr)[2]) {
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      const int idx = u * kThreads + (int)threadIdx.x;
      *reinterpret_cast<u32x4_t*>(buf + (idx / 24) * kKStride + 16 * (idx % 24)) = kr[u];
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int idx = u * kThreads + (int)threadIdx.x;
      *reinterpret_cast<u32x4_t*>(buf + kKBuf + (idx >> 4) * kVStride + 16 * (idx & 15)) = vr[u];
    }
  };

  f32x16_t acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
  float m_ref = -INFINITY, l_loc = 0.f;
  const float sl2 = scale * 1.4426950408889634f;

  const int qk_off = kKStride * r32 + 16 * hi32;
  const int g = lane >> 4, jj = (lane >> 2) & 3, qq = lane & 3;
  // V^T read for k-step u, half rd: keys 16u + 8rd + 4(g>>1) + jj, columns
  // 32ct + 16(g&1) + 4qq (the key order of the score registers).
  const int pv_off = kVStride * (4 * (g >> 1) + jj) + 2 * (16 * (g & 1) + 4 * qq);

  u32x4_t kr[3], vr[2];
  if (tiles > 0) load_tile(0, kr, vr);
  for (int kt = 0; kt < tiles; ++kt) {
    char* buf = smem + (kt & 1) * kStage;
    store_tile(buf, kr, vr);
    __syncthreads();
    if (kt + 1 < tiles) load_tile(kt + 1, kr, vr);
    const int key0 = k_pos0 + kt * kKTile;  // position of the tile's first key
    if (!causal || key0 <= q_pos0 + min(qb + wave * kWaveRows + kWaveRows, s_q) - 1) {
      f32x16_t st;
#pragma unroll
      for (int r = 0; r < 16; ++r) st[r] = 0.f;
#pragma unroll
      for (int s = 0; s < kHeadK / 16; ++s) {
        const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(buf + qk_off + 32 * s);
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], st, 0, 0, 0);
      }
      // Mask keys past the chunk or past the query's position.
      const bool full = kt * kKTile + kKTile <= n_vis && (!causal || key0 + kKTile - 1 <= q_first_wave);
      if (!full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kl = kt * kKTile + 8 * (r >> 2) + 4 * hi32 + (r & 3);
          if (kl >= n_vis || (causal && k_pos0 + kl > qpos)) st[r] = -INFINITY;
        }
      }
      float mx = st[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, st[r]);
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(mx, __uint_as_float(hi32 ? sw[0] : sw[1])) * sl2;
      const float m_new = (mx > m_ref + 8.0f || m_ref == -INFINITY) ? mx : m_ref;
      if (m_new > m_ref && m_ref != -INFINITY) {
        const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][r] *= alpha;
        l_loc *= alpha;
      }
      m_ref = m_new;
      const float neg = (m_ref == -INFINITY) ? 0.f : -m_ref;
      bf16x8_t pf[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(st[r], sl2, neg));
        l_loc += p;
        pf[r >> 3][r & 7] = (__bf16)p;
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          bf16x8_t vf;
#pragma unroll
          for (int rd = 0; rd < 2; ++rd) {
            const bf16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (lds_b4_t*)((__attribute__((address_space(3))) char*)buf + kKBuf + pv_off +
                            kVStride * (16 * u + 8 * rd) + 64 * ct));
            vf[4 * rd + 0] = v[0]; vf[4 * rd + 1] = v[1]; vf[4 * rd + 2] = v[2]; vf[4 * rd + 3] = v[3];
          }
          acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[u], acc[ct], 0, 0, 0);
        }
    }
    __syncthreads();
  }

  const auto sl = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_loc), __float_as_uint(l_loc), false, false);
  const float l_tot = l_loc + __uint_as_float(hi32 ? sl[0] : sl[1]);
  const bool any = l_tot > 0.f;
  const float inv = any ? 1.f / l_tot : 0.f;
  if (qrow >= s_q) return;
  __bf16* orow = o + ((size_t)qrow * H + h) * kHeadV;
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      bf16x4_t v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (__bf16)(acc[ct][4 * q4 + e] * inv);
      *reinterpret_cast<bf16x4_t*>(orow + 32 * ct + 8 * q4 + 4 * hi32) = v;
    }
  if (hi32 == 0) lse[(size_t)qrow * H + h] = any ? (m_ref + __log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
}

// ---------------------------------------------------------------------------
// merge_kernel: one wave per (token, head) row; lanes 0..15 own 8 of the 128
// columns; chunk k's weight exp(lse_k - lse).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void merge_kernel(const __bf16* __restrict__ o_part, const float* __restrict__ lse_part,
                                                   int n_parts, int rows, __bf16* __restrict__ o,
                                                   float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  float lk = -INFINITY;
  if (lane < n_parts) lk = lse_part[(size_t)lane * rows + row];
  float M = lk;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  const float Mf = (M == -INFINITY) ? 0.f : M;
  float w = lane < n_parts ? expf(lk - Mf) : 0.f;
  float S = w;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) S += __shfl_xor(S, off, 64);
  const float wn = S > 0.f ? w / S : 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < n_parts; ++k) {
    const float wk = __shfl(wn, k, 64);
    if (lane < 16) {
      const bf16x8_t x = *reinterpret_cast<const bf16x8_t*>(o_part + ((size_t)k * rows + row) * kHeadV + 8 * lane);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(wk, (float)x[e], acc[e]);
    }
  }
  if (lane < 16) {
    bf16x8_t v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (__bf16)acc[e];
    *reinterpret_cast<bf16x8_t*>(o + (size_t)row * kHeadV + 8 * lane) = v;
  }
  if (lane == 0) lse[row] = S > 0.f ? Mf + logf(S) : -INFINITY;
}

}  // namespace

hipError_t launch_expand(const void* cache, const int32_t* btab_row, int t0, int n, int num_pages, const void* w_uk,
                         const void* w_uv, int H, void* k_out, void* v_out, int n_stride, hipStream_t stream) {
  const dim3 grid((unsigned)((n + kExpRows - 1) / kExpRows), (unsigned)H, 2u);
  hipLaunchKernelGGL(expand_kernel, grid, dim3(kThreads), 0, stream, static_cast<const __bf16*>(cache), btab_row,
                     t0, n, num_pages, static_cast<const __bf16*>(w_uk), static_cast<const __bf16*>(w_uv), H,
                     static_cast<__bf16*>(k_out), static_cast<__bf16*>(v_out), n_stride);
  return hipGetLastError();
}

hipError_t launch_prefill_attn(const void* q_nope, const void* q_rope, int s_q, int H, const void* K, const void* V,
                               int n, int n_stride, int k_pos0, int q_pos0, int causal, float scale, void* o,
                               float* lse, hipStream_t stream) {
  const dim3 grid((unsigned)((s_q + kRowsPerGroup - 1) / kRowsPerGroup), (unsigned)H);
  hipLaunchKernelGGL(attn_kernel, grid, dim3(kThreads), 0, stream, static_cast<const __bf16*>(q_nope),
                     static_cast<const __bf16*>(q_rope), s_q, H, static_cast<const __bf16*>(K),
                     static_cast<const __bf16*>(V), n, n_stride, k_pos0, q_pos0, causal, scale,
                     static_cast<__bf16*>(o), lse);
  return hipGetLastError();
}

hipError_t launch_prefill_merge(const void* o_part, const float* lse_part, int n_parts, int rows, void* o, float* lse,
                                hipStream_t stream) {
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream,
                     static_cast<const __bf16*>(o_part), lse_part, n_parts, rows, static_cast<__bf16*>(o), lse);
  return hipGetLastError();
}

}  // namespace mla

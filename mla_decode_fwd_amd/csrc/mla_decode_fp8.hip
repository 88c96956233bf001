// Absorbed-MLA decode on an FP8 (e4m3) latent cache, bf16 queries and
// outputs, fp32 accumulation, for gfx950 (MI355X).
//
// What it computes: the decode of mla_decode_bf16.hip ("MLA 推理：两条计算路径与
// FlashMLA", sections "两条等价的路径" and "decode 注意力变成了计算问题") on a cache
// whose rows are 576 e4m3 codes plus one fp32 scale each (the FP8 latent
// cache of that page's exercise 2, which counts 576 bytes per token besides
// the scale factors): row value = scale * e4m3 value.
//
// Same work decomposition as the bf16 kernel (128 rows per workgroup, four
// waves of 32 rows, Q^T in VGPRs, O^T in the AGPR file, pages of 64 tokens
// double-buffered in LDS, two staggered 32-token tiles per page, split-KV
// partials). What differs:
//   * A page is 36,864 bytes in HBM (half the bf16 page) and sits in LDS
//     row-major with one 16-byte padding chunk per row (592-byte rows), the
//     64 row scales after it. Each direct-load instruction copies 64
//     consecutive 16-byte LDS slots, i.e. nearly 1 KB of consecutive HBM.
//   * QK: one 16-byte LDS read per lane feeds two MFMA k-steps. The 576
//     contraction elements are visited in a permuted order, the same for K
//     and Q: k-step 2s+e, lane half h, element i <-> element 32s + 16h + 8e + i.
//     Lane (token t, half h) thus reads chunk 2s+h of row t, and the 592-byte
//     row stride (37 chunks, 37 = 5 mod 16) puts 16 consecutive tokens on 16
//     different bank groups. The codes are widened to bf16 exactly
//     (v_cvt_scalef32_pk_bf16_fp8 with scale 1) and each score is multiplied
//     by its row's scale before the softmax.
//   * PV: one ds_read_b64_tr_b8 per lane gives an 8-token x 1-column piece of
//     V^T (within a 16-lane group, input lane 2j+q names token j's 8 columns
//     8q..8q+7 and output lane c receives column c of the 8 tokens), widened
//     to bf16 without scale; the row scale goes into P instead (P * scale is
//     the PV operand, the sum l keeps P). MFMA rows of column tile i are
//     columns 16a..16a+15 and 16(a+4)..16(a+4)+15, a = (i&3) + 8(i>>2): with
//     the 37-chunk stride the two chunks a and a+4 fall on disjoint bank
//     groups for the 8 tokens a group reads.
//   * Tail tokens past the end of the sequence are cleared in LDS, codes and
//     scales, so that unowned slots (which may hold NaN) never reach a product.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "mla_decode_common.h"
#include "mla_internal.h"

namespace mla {
namespace {

using namespace dec;

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2_t;
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2_t;

constexpr int kChunks = kDqk / 16;                   // 36 16-byte chunks per row
constexpr int kRowStride = (kChunks + 1) * 16;       // 592: LDS row stride, one padding chunk
constexpr int kPageRows = kPage * kRowStride;        // 37,888
constexpr int kScaleOff = kPageRows;                 // 64 fp32 row scales follow the rows
constexpr int kBufBytes = 38 * 1024;                 // per page buffer: rows, scales, 1 KB aligned
static_assert(kPageRows + kPage * 4 <= kBufBytes, "page buffer");
constexpr int kSlots = kPage * (kChunks + 1);        // 2368 LDS slots of 16 bytes
constexpr int kLines = kSlots / 64;                  // 37 direct-load instructions per page
static_assert(kSlots % 64 == 0, "whole lines");
constexpr int kQPairs = kQSteps / 2;                 // 18 LDS reads per tile, 2 k-steps each
// The finalize stages each wave's 32 output rows (32 KB) through LDS, so the
// allocation covers that as well as the two page buffers.
constexpr int kStageBytes = kWaves * kWaveRows * kDv * 2;  // 131,072
constexpr int kSmemBytes = 2 * kBufBytes > kStageBytes ? 2 * kBufBytes : kStageBytes;
// The staged query rows (two rounds of 128 rows x 592 bytes) follow the
// first page buffer.
static_assert(kBufBytes + kRowsPerGroup * (kDqk + 16) <= kSmemBytes, "query staging area");

// Line n of a page covers LDS slots 64n .. 64n+63; lane l loads slot 64n + l:
// row t = k / 37, chunk c = k % 37 (the padding chunk re-reads chunk 35).
__device__ __forceinline__ int line_src_offset(int n, int lane) {
  const unsigned k = 64u * (unsigned)n + (unsigned)lane;
  const unsigned t = k / 37u;
  const unsigned c = k - 37u * t;
  return (int)(t * kDqk + 16u * (c < 35u ? c : 35u));
}

struct PageLoad8 {
  uint64_t src;   // page codes (wave-uniform)
  uint64_t scl;   // page row scales (wave-uniform)
  uint32_t lds;   // LDS page buffer (wave-uniform)
};

__device__ __forceinline__ uint64_t uniform_ptr(const void* p) {
  const uint64_t g = (uint64_t)(uintptr_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)g);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(g >> 32));
  return ((uint64_t)hi << 32) | (uint64_t)lo;
}

__device__ __forceinline__ PageLoad8 make_load8(const uint8_t* cache, const float* scales, int phys, char* buf) {
  PageLoad8 p;
  p.src = uniform_ptr(cache + (size_t)phys * (kPage * kDqk));
  p.scl = uniform_ptr(scales + (size_t)phys * kPage);
  p.lds = (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)(uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)buf);
  return p;
}

// The m-th line of this wave: page lines n = wave, wave+4, ... (wave 0 has 10,
// the others 9); m == 9 on wave 1 is the scales line (16 lanes).
__device__ __forceinline__ void issue_line8(const PageLoad8& p, int wave, int lane, int m) {
  const int n = wave + 4 * m;
  if (n < kLines) {
    dma_line(p.src, line_src_offset(n, lane), p.lds + 1024u * (uint32_t)n);
  } else if (wave == 1 && m == 9 && lane < 16) {
    dma_line(p.scl, 16 * lane, p.lds + (uint32_t)kScaleOff);
  }
}

__device__ __forceinline__ void issue_page8(const PageLoad8& p, int wave, int lane) {
#pragma unroll
  for (int m = 0; m < 10; ++m) issue_line8(p, wave, lane, m);
}

// Eight e4m3 codes (two words) to bf16, times s.
__device__ __forceinline__ bf16x8_t widen8(uint32_t w0, uint32_t w1, float s) {
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, s, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, s, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, s, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, s, true);
  bf16x8_t r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

__global__ __launch_bounds__(kThreads, 1) void mla_decode_fp8_kernel(DecodeArgs a, int row_groups) {
  __shared__ __attribute__((aligned(1024))) char smem[kSmemBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r32 = lane & 31;
  const int hi32 = lane >> 5;

  // XCD-aware chunk mapping, as in the bf16 kernel.
  const int x = blockIdx.x;
  const int xcd = x & 7;
  const int rest = x >> 3;
  const int rgrp = rest % row_groups;
  const int per_xcd = (a.total_splits + 7) / 8;
  const int g = xcd * per_xcd + rest / row_groups;
  if (rest / row_groups >= per_xcd || g >= a.total_splits) return;

  const WorkItem wi = find_work(a.split_offsets, a.seqlens, a.B, g, lane);
  const int b = wi.b;
  const int L = max(a.s_q, min(wi.L, a.max_pages * kPage));
  const int P = (L + kPage - 1) / kPage;
  const int n_chunks = min(max(wi.n, 1), kMaxSplits);
  const int kk = min(max(wi.k, 0), n_chunks - 1);
  const int pg0 = (int)((unsigned)kk * (unsigned)P / (unsigned)n_chunks);
  const int pg1 = (int)((unsigned)(kk + 1) * (unsigned)P / (unsigned)n_chunks);

  const int rows = a.s_q * a.H;
  const int row = rgrp * kRowsPerGroup + wave * kWaveRows + r32;
  const int row_c = min(row, rows - 1);
  const int qi = row_c / a.H;
  const int n_allowed = a.causal ? (L - a.s_q + qi + 1) : L;
  const int n_allowed_min = a.causal ? (L - a.s_q + 1) : L;

  const uint8_t* cache = static_cast<const uint8_t*>(a.kv_cache);
  const int32_t* btab = a.block_table + (size_t)b * a.max_pages;
  const int last_phys = a.num_pages - 1;

  const int bt0 = btab[max(min(pg0, pg1 - 1), 0)];
  const int bt1 = btab[max(min(pg0 + 1, pg1 - 1), 0)];
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);

  // Q^T fragments in the permuted contraction order: k-step 2s+e holds
  // q[row][32s + 16*hi32 + 8e .. +8]. The workgroup's 128 rows are staged
  // through LDS (issue_q_round) in two rounds, dims 0..287 (issued ahead of
  // the first page, whose loads go on while it is read) and 288..575, in the
  // area past the first page buffer.
  bf16x8_t qf[kQSteps];
  const char* const q_seq = static_cast<const char*>(a.q_lat) + (size_t)b * rows * (kDqk * 2);
  char* const q_area = smem + kBufBytes;
  issue_q_round(q_seq, rows, rgrp * kRowsPerGroup, kRowsPerGroup, kDqk, 0, q_area, wave, lane);

  int phys_ahead = 0;
  if (pg0 < pg1) {
    issue_page8(make_load8(cache, a.row_scales, min(max(bt0, 0), last_phys), smem), wave, lane);
    phys_ahead = bt1;
    // The query round, not the page (10 loads on waves 0 and 1, 9 on the others).
    if (wave < 2)
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(10));
    else
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(9));
  } else {
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  }
  __syncthreads();
  {
    const char* const src = q_area + (wave * kWaveRows + r32) * (kDqk + 16) + 32 * hi32;
#pragma unroll
    for (int s = 0; s < kQSteps / 2; ++s)
      qf[s] = *reinterpret_cast<const bf16x8_t*>(src + 64 * (s >> 1) + 16 * (s & 1));
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __syncthreads();  // every wave has its first half: the area takes the second
    issue_q_round(q_seq, rows, rgrp * kRowsPerGroup, kRowsPerGroup, kDqk, kDqk, q_area, wave, lane);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
#pragma unroll
    for (int s = kQSteps / 2; s < kQSteps; ++s)
      qf[s] = *reinterpret_cast<const bf16x8_t*>(src + 64 * ((s - kQSteps / 2) >> 1) + 16 * (s & 1));
    // The next page's loads overwrite the area: every read is done before
    // the page loop's first barrier.
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  }

  f32x16_t acc_o[kColTiles];
#pragma unroll
  for (int i = 0; i < kColTiles; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[i][r] = 0.f;
  float m_ref = -INFINITY;
  float l_loc = 0.f;
  const float sl2 = a.scale * 1.4426950408889634f;

  // QK: lane (token 32T + r32, half hi32) reads chunk 2s + hi32 of its row.
  const int qk_off = kRowStride * r32 + 16 * hi32;
  // PV: 16-lane group gg reads, as input lane 2j + q, token 4(gg>>1) + (j&3) +
  // 8(j>>2) (plus 32T + 16u) at columns 16(a + 4(gg&1)) + 8q .. +8.
  const int gg = lane >> 4;
  const int jj = (lane & 15) >> 1;
  const int pv_off = kRowStride * (4 * (gg >> 1) + (jj & 3) + 8 * (jj >> 2)) + 64 * (gg & 1) + 8 * (lane & 1);

  for (int pg = pg0; pg < pg1; ++pg) {
    char* buf = smem + ((pg - pg0) & 1) * kBufBytes;
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    const int phys_next = min(max(phys_ahead, 0), last_phys);
    phys_ahead = btab[min(pg + 2, pg1 - 1)];
    // Issued on every page: on the last one the clamped table index reloads
    // the current page into the idle buffer, which costs less than a branch
    // around each load (as in the bf16 kernel).
    const PageLoad8 next = make_load8(cache, a.row_scales, phys_next, smem + ((pg + 1 - pg0) & 1) * kBufBytes);
    const int valid = L - pg * kPage;
    if (valid < kPage) {
      // Clear the rows (and scales) of tokens past the end of the sequence.
      for (int idx = threadIdx.x; idx < (kPage - valid) * kChunks; idx += kThreads) {
        const int t = valid + idx / kChunks;
        const int c = idx % kChunks;
        *reinterpret_cast<uint4*>(buf + kRowStride * t + 16 * c) = make_uint4(0, 0, 0, 0);
      }
      for (int t = valid + (int)threadIdx.x; t < kPage; t += kThreads)
        reinterpret_cast<float*>(buf + kScaleOff)[t] = 0.f;
      __syncthreads();
    }
    const bool full_page = (pg + 1) * kPage <= n_allowed_min;
    const float* sbuf = reinterpret_cast<const float*>(buf + kScaleOff);

    auto k_raw = [&](int T, int s2) {
      return *reinterpret_cast<const u32x4_t*>(buf + qk_off + kRowStride * 32 * T + 32 * s2);
    };
    auto v_raw = [&](int u, int i) {
      const int a16 = (i & 3) + 8 * (i >> 2);
      const i32x2_t v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (lds_i32x2_t*)((__attribute__((address_space(3))) char*)buf + pv_off + kRowStride * 16 * u + 16 * a16));
      return v;
    };
    auto tile_max = [&](f32x16_t& st, int T) {
      if (!full_page) {
        const int tok0 = pg * kPage + 32 * T + 4 * hi32;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (tok0 + 8 * (r >> 2) + (r & 3) >= n_allowed) st[r] = -INFINITY;
      }
      float mx[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) mx[r] = fmaxf(st[r], st[r + 8]);
#pragma unroll
      for (int r = 0; r < 4; ++r) mx[r] = fmaxf(mx[r], mx[r + 4]);
      const float mt = fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]));
      return fmaxf(mt, other_half(mt)) * sl2;
    };
    auto move_reference = [&](float m_new) {
      if (__any(m_new > m_ref && m_ref != -INFINITY)) {
        const float alpha = (m_new > m_ref && m_ref != -INFINITY) ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.f;
        agpr_fence();
        scale_accumulators(alpha);
        l_loc *= alpha;
      }
      m_ref = m_new;
    };
    // Row scales of this lane's 16 scores of tile T (tokens 8q + 4*hi32 + 0..3).
    auto tile_scales = [&](int T, float* sc) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(sbuf + 32 * T + 8 * q + 4 * hi32);
        sc[4 * q + 0] = v[0]; sc[4 * q + 1] = v[1]; sc[4 * q + 2] = v[2]; sc[4 * q + 3] = v[3];
      }
    };
    // Two P values (scores e, e+1): l takes P, the PV operand P * row scale.
    auto p_pair = [&](const f32x16_t& st, int e, float neg_ref, const float* sc, bf16x8_t* pf, float& psum) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[e], sl2, neg_ref));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[e + 1], sl2, neg_ref));
      pf[e >> 3][e & 7] = (__bf16)(p0 * sc[e]);
      pf[e >> 3][(e & 7) + 1] = (__bf16)(p1 * sc[e + 1]);
      psum += p0 + p1;
    };
    constexpr int kKDepth = 2;   // 16-byte K reads in flight (each feeds two k-steps)
    constexpr int kVDepth = 4;   // 8-byte V^T reads in flight
    // QK of tile T into st, with work(s2) run after each pair of k-steps.
    auto qk_tile = [&](int T, f32x16_t& st, auto&& work) {
      u32x4_t kr[kKDepth];
#pragma unroll
      for (int s2 = 0; s2 < kKDepth; ++s2) kr[s2] = k_raw(T, s2);
#pragma unroll
      for (int s2 = 0; s2 < kQPairs; ++s2) {
        const u32x4_t cur = kr[s2 % kKDepth];
        if (s2 + kKDepth < kQPairs) kr[s2 % kKDepth] = k_raw(T, s2 + kKDepth);
        const bf16x8_t k0 = widen8(cur[0], cur[1], 1.f);
        const bf16x8_t k1 = widen8(cur[2], cur[3], 1.f);
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[2 * s2], st, 0, 0, 0);
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qf[2 * s2 + 1], st, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        work(s2);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // PV of tile T with operand pf, work(n) after each of the 32 MFMAs. The
    // widened V^T pieces are made two MFMAs ahead of use: the asm MFMA is
    // invisible to the hazard tracker, so VALU results it reads must be old.
    auto pv_tile = [&](int T, const bf16x8_t* pf, auto&& work) {
      i32x2_t vr[kVDepth];
#pragma unroll
      for (int n = 0; n < kVDepth; ++n) vr[n] = v_raw(2 * T + (n >> 4), n & 15);
      bf16x8_t vw[3];
      vw[0] = widen8((uint32_t)vr[0][0], (uint32_t)vr[0][1], 1.f);
      vw[1] = widen8((uint32_t)vr[1][0], (uint32_t)vr[1][1], 1.f);
#pragma unroll
      for (int n = 0; n < 2 * kColTiles; ++n) {
        if (n + 2 < 2 * kColTiles) {
          const i32x2_t c2 = vr[(n + 2) % kVDepth];
          vw[(n + 2) % 3] = widen8((uint32_t)c2[0], (uint32_t)c2[1], 1.f);
        }
        if (n + kVDepth < 2 * kColTiles) vr[n % kVDepth] = v_raw(2 * T + ((n + kVDepth) >> 4), (n + kVDepth) & 15);
        if ((n & 15) == 0)
          mfma_pv<true>(acc_o[n & 15], vw[n % 3], pf[n >> 4]);
        else
          mfma_pv<false>(acc_o[n & 15], vw[n % 3], pf[n >> 4]);
        work(n);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // ---- QK(T0), with the first five of this wave's next-page loads.
    f32x16_t st0;
#pragma unroll
    for (int r = 0; r < 16; ++r) st0[r] = 0.f;
    qk_tile(0, st0, [&](int s2) {
      if ((s2 & 1) == 0 && s2 < 10) issue_line8(next, wave, lane, s2 >> 1);
    });
    float sc0[16];
    tile_scales(0, sc0);
#pragma unroll
    for (int r = 0; r < 16; ++r) st0[r] *= sc0[r];
    const float mt0 = tile_max(st0, 0);
    move_reference((mt0 > m_ref + 8.0f) ? mt0 : m_ref);
    const float neg0 = (m_ref == -INFINITY) ? 0.f : -m_ref;

    // ---- QK(T1), with tile 0's P and the rest of the loads.
    f32x16_t st1;
#pragma unroll
    for (int r = 0; r < 16; ++r) st1[r] = 0.f;
    bf16x8_t pf0[2];
    float psum0 = 0.f;
    qk_tile(1, st1, [&](int s2) {
      if ((s2 & 1) == 0 && s2 < 16) {
        p_pair(st0, s2, neg0, sc0, pf0, psum0);
      }
      if ((s2 & 1) == 1 && s2 < 10) issue_line8(next, wave, lane, 5 + (s2 >> 1));
    });
    l_loc += psum0;
    float sc1[16];
    tile_scales(1, sc1);
#pragma unroll
    for (int r = 0; r < 16; ++r) st1[r] *= sc1[r];
    const float mt1 = tile_max(st1, 1);
    const float m1 = (mt1 > m_ref + 8.0f) ? mt1 : m_ref;
    const float neg1 = (m1 == -INFINITY) ? 0.f : -m1;

    // ---- PV(T0), with tile 1's P.
    bf16x8_t pf1[2];
    float psum1 = 0.f;
    pv_tile(0, pf0, [&](int n) {
      if ((n & 3) == 0) p_pair(st1, n >> 1, neg1, sc1, pf1, psum1);
    });
    move_reference(m1);
    l_loc += psum1;

    // ---- PV(T1).
    pv_tile(1, pf1, [&](int) {});
  }

  // The last page's reload is still landing in the idle buffer, which the
  // finalize reuses for staging.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  // ---- finalize, as in the bf16 kernel; MFMA row m of column tile i is
  // column 16a + m (m < 16) or 16(a + 4) + m - 16, a = (i&3) + 8(i>>2).
  agpr_fence();
  const float l_tot = l_loc + other_half(l_loc);
  const bool any = l_tot > 0.f;
  const float inv = any ? 1.f / l_tot : 0.f;
  const float lse_v = any ? (m_ref + __log2f(l_tot)) * 0.6931471805599453f : -INFINITY;

  __syncthreads();
  const int ln = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int r32f = ln & 31, hi32f = ln >> 5;
  const int rowf = rgrp * kRowsPerGroup + wave * kWaveRows + r32f;
  char* stage = smem + wave * (kWaveRows * kDv * 2);
#pragma unroll
  for (int i = 0; i < kColTiles; ++i)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      bf16x4_t v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (__bf16)(acc_o[i][4 * q4 + e] * inv);
      const int a16 = (i & 3) + 8 * (i >> 2);
      const int m0 = 8 * q4 + 4 * hi32f;
      const int col0 = m0 < 16 ? 16 * a16 + m0 : 16 * (a16 + 4) + m0 - 16;
      const int piece = (col0 >> 3) ^ r32f;
      *reinterpret_cast<bf16x4_t*>(stage + r32f * (kDv * 2) + piece * 16 + 2 * (col0 & 4)) = v;
    }
  __syncthreads();

  const bool direct = n_chunks == 1 && a.o_lat != nullptr;
  __bf16* const out = direct ? static_cast<__bf16*>(a.o_lat) + (size_t)b * rows * kDv
                             : static_cast<__bf16*>(a.o_part) + (size_t)g * rows * kDv;
  const int row0 = rgrp * kRowsPerGroup + wave * kWaveRows;
#pragma unroll 4
  for (int r = 0; r < kWaveRows; ++r) {
    if (row0 + r >= rows) break;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stage + r * (kDv * 2) + ((ln ^ r) * 16));
    if (direct)  // final rows: non-temporal; chunk partials: device scope, the merge reads them next
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(out + (size_t)(row0 + r) * kDv + 8 * ln));
    else
      store_device_scope(out + (size_t)(row0 + r) * kDv, 16 * ln, v);
  }
  if (hi32f == 0 && rowf < rows) {
    if (direct)
      a.lse[(size_t)b * rows + rowf] = lse_v;
    else
      store_device_scope(a.lse_part + (size_t)g * rows, 4 * rowf, lse_v);
  }
}

}  // namespace

hipError_t launch_decode_fp8(const DecodeArgs& a, hipStream_t stream) {
  const int rows = a.s_q * a.H;
  const int row_groups = (rows + kRowsPerGroup - 1) / kRowsPerGroup;
  const int padded = (a.total_splits + 7) / 8 * 8;
  const dim3 grid((unsigned)(padded * row_groups));
  hipLaunchKernelGGL(mla_decode_fp8_kernel, grid, dim3(kThreads), 0, stream, a, row_groups);
  return hipGetLastError();
}

}  // namespace mla

// Absorbed-MLA decode, bf16 storage, fp32 accumulation, for gfx950 (MI355X).
//
// What it computes ("MLA 推理：两条计算路径与 FlashMLA", sections "两条等价的路径"
// and "decode 注意力变成了计算问题"): every (query token, head) row attends to
// one shared 576-wide key per cached token and one shared 512-wide value (the
// first 512 elements of the same cache row), i.e. an MQA with a very wide
// head. Rows are the MFMA N dimension, the latent the K dimension.
//
// Work decomposition
//   * A row is (query token i, head h), m = i*H + h, so q_lat[b] is an
//     [s_q*H, 576] matrix. A workgroup holds 64 rows (4 waves x 16 rows, one
//     wave per SIMD with the whole register file) and walks a range of
//     64-token pages of one sequence. The workgroups of the other row groups
//     of the same chunk are mapped to the same XCD and run at the same time,
//     so the second reader of a page finds it in that XCD's L2.
//   * Per page, the 73,728-byte page is copied HBM -> LDS with direct 16-byte
//     loads (global_load_lds_dwordx4), double-buffered so the next page
//     streams in while the current one is consumed by the four waves.
//   * QK^T is computed transposed, S^T[token, row] = K . Q^T, with
//     v_mfma_f32_16x16x32_bf16: A = 16 tokens x 32 latent elements read from
//     LDS, B = Q^T held in registers for the whole walk (18 k-steps). Each
//     lane then owns one row and 16 of the page's 64 token scores; the row
//     max and sum take two cross-lane steps (lane ^ 16, lane ^ 32).
//   * PV is computed transposed too, O^T[col, row] += V^T . P^T: A = V^T read
//     with ds_read_b64_tr_b16 (a 4x16 -> 16x4 transpose within each 16-lane
//     group), B = P^T taken straight from the score registers after a bf16
//     pack. Inside each 32-token k-step the token order is permuted the same
//     way on both sides, so the score registers need no shuffling.
//   * Online softmax in base 2 with a lazily updated reference max: the
//     accumulators are rescaled only when a row's max grows by more than 8
//     (so P <= 2^8); the result is exact because P, l and O always share the
//     same reference.
//   * Split-KV: a workgroup handles chunk k of n_b page-aligned chunks of its
//     sequence. With n_b = 1 it writes bf16 o_lat and the LSE directly;
//     otherwise (or when only partials are asked for) fp32 partials that
//     the combine kernel merges by LSE.
//
// LDS page layout ("line blocks"): the page is split into 72 blocks of 1 KB.
// Block 9m + j holds, for the 8 tokens t = 8m .. 8m+7, the 128-byte line j
// (chunks 8j .. 8j+7 of 8 elements) of each token's row: token t, chunk c
// sits in 16-byte slot 64*(9*(t>>3) + (c>>3)) + 8*(t&7) + ((c&7) ^ F(t)),
// F(t) = T[(t>>1)&3] ^ 4*((t>>3)&1), T = {0, 2, 5, 7}. Every direct-load
// instruction therefore reads 8 whole 128-byte lines (fully coalesced), and
// the XOR keeps the QK reads (16 lanes = 16 tokens of one chunk) and the
// transposed PV reads (4 lane groups x 4 tokens x 2 chunks) free of LDS bank
// conflicts.

#include <hip/hip_runtime.h>

#include <type_traits>
#include <cmath>
#include <cstdint>

#include "mla_internal.h"

namespace mla {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;
typedef __attribute__((address_space(1))) const void gbl_cvoid_t;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 16;
static_assert(kRowsPerWave * kWaves == kRowsPerGroup, "a workgroup covers one row group");
constexpr int kRowBytes = kDqk * 2;               // 1152: one cache row
constexpr int kPageBytes = kPage * kRowBytes;     // 73728: one page
constexpr int kBlocks = kPageBytes / 1024;        // 72 line blocks
constexpr int kBlocksPerWave = kBlocks / kWaves;  // 18: two token octets per wave
constexpr int kQSteps = kDqk / 32;                // 18 k-steps of 32
constexpr int kColTiles = kDv / 16;               // 32 output column tiles
static_assert(kBlocksPerWave == 18, "each wave loads two token octets");
// s_waitcnt immediate for gfx9: vmcnt = 0, expcnt and lgkmcnt left at "no wait".
constexpr int kWaitVmcnt0 = (0xF << 8) | (0x7 << 4);

__device__ __forceinline__ int swz(int t) {
  const int u = (t >> 1) & 3;
  const int tbl = (u == 0) ? 0 : (u == 1) ? 2 : (u == 2) ? 5 : 7;
  return tbl ^ (4 * ((t >> 3) & 1));
}
__device__ __forceinline__ int slot_bytes(int t, int c) {
  return (64 * (9 * (t >> 3) + (c >> 3)) + 8 * (t & 7) + ((c & 7) ^ swz(t))) * 16;
}

// One direct 16-byte-per-lane load: global sbase + voff -> LDS lds + 16*lane.
// Written as inline asm so that the compiler's wait-count bookkeeping does not
// see it: it would otherwise wait for the next page's loads before every LDS
// read of the current page. Completion is awaited explicitly (vmcnt 0 and a
// barrier) before a buffer is read. An SALU write of M0 needs one wait state
// before a load that writes LDS.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // M0 is reserved; nothing else here uses it
__device__ __forceinline__ void dma_line(uint64_t sbase, int voff, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(sbase), "s"(lds)
      : "memory", "m0");
}
#pragma clang diagnostic pop

// The loads of one page into an LDS buffer. Wave w fills blocks 18w .. 18w+17:
// token octets 2w and 2w+1, lines j = 0..8 each. Lane l takes token
// 8m + (l>>3), chunk 8j + ((l&7) ^ F(token)); F depends on the octet's
// parity, hence two per-lane source offsets. Line n (0..17) of the wave is
// octet n/9, line n%9.
struct PageLoad {
  uint64_t sbase;  // page address (wave-uniform)
  uint32_t lds;    // LDS address of the wave's first block (wave-uniform)
  int off0, off1;  // per-lane source offsets of the two octets
};

__device__ __forceinline__ PageLoad make_page_load(const char* page_src, char* lds_buf, int wave, int lane) {
  PageLoad p;
  // Both bases are wave-uniform; readfirstlane keeps them in SGPRs. It returns
  // a signed int, so widen through uint32_t (never sign-extend).
  const uint64_t gp = (uint64_t)(uintptr_t)page_src;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)gp);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(gp >> 32));
  p.sbase = ((uint64_t)hi << 32) | (uint64_t)lo;
  char* dst = lds_buf + wave * (kBlocksPerWave * 1024);
  p.lds = (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)(uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)dst);
  const int t0 = 16 * wave + (lane >> 3);
  p.off0 = t0 * kRowBytes + (((lane & 7) ^ swz(t0)) * 16);
  p.off1 = (t0 + 8) * kRowBytes + (((lane & 7) ^ swz(t0 + 8)) * 16);
  return p;
}

__device__ __forceinline__ void issue_line(const PageLoad& p, int n) {
  const int octet = n / 9, j = n % 9;
  dma_line(p.sbase, (octet ? p.off1 : p.off0) + 128 * j, p.lds + 1024 * (9 * octet + j));
}

__device__ __forceinline__ void issue_page(const PageLoad& p) {
#pragma unroll
  for (int n = 0; n < kBlocksPerWave; ++n) issue_line(p, n);
}

// Reductions over the four lane groups of a row (lanes l, l^16, l^32, l^48)
// with the gfx950 lane-swap instructions (VALU, no LDS round trip). With both
// operands equal, permlane16_swap yields the values of lanes l and l^16 side
// by side, permlane32_swap those of l and l^32.
__device__ __forceinline__ float max4lanes(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum4lanes(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

struct WorkItem {
  int b, k, n;  // sequence, chunk index, chunk count
};

__device__ __forceinline__ WorkItem find_work(const int32_t* split_offsets, int B, int g) {
  WorkItem w;
  if (split_offsets == nullptr) {
    w.b = g; w.k = 0; w.n = 1;
    return w;
  }
  int lo = 0, hi = B - 1;
  while (lo < hi) {  // largest b with split_offsets[b] <= g
    const int mid = (lo + hi + 1) >> 1;
    if (split_offsets[mid] <= g) lo = mid; else hi = mid - 1;
  }
  w.b = lo;
  w.k = g - split_offsets[lo];
  w.n = split_offsets[lo + 1] - split_offsets[lo];
  return w;
}

__global__ __launch_bounds__(kThreads, 1) void mla_decode_bf16_kernel(DecodeArgs a, int row_groups) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * kPageBytes];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g16 = lane >> 4;  // lane group: k slice / token quad
  const int r16 = lane & 15;  // the row this lane owns in MFMA outputs

  // XCD-aware mapping: workgroups x and x+8j run on the same XCD. The row
  // groups of one chunk (which read the same pages) get consecutive j.
  const int x = blockIdx.x;
  const int xcd = x & 7;
  const int rest = x >> 3;
  const int rgrp = rest % row_groups;
  const int g = (rest / row_groups) * 8 + xcd;
  if (g >= a.total_splits) return;

  const WorkItem wi = find_work(a.split_offsets, a.B, g);
  const int b = wi.b;
  int L = a.seqlens[b];
  L = max(a.s_q, min(L, a.max_pages * kPage));
  const int P = (L + kPage - 1) / kPage;
  const int n_chunks = max(wi.n, 1);
  const int kk = min(max(wi.k, 0), n_chunks - 1);
  const int pg0 = (int)(((long long)kk * P) / n_chunks);
  const int pg1 = (int)(((long long)(kk + 1) * P) / n_chunks);

  const int rows = a.s_q * a.H;
  const int wave_row0 = rgrp * kRowsPerGroup + wave * kRowsPerWave;
  const bool wave_active = wave_row0 < rows;
  const int row = wave_row0 + r16;
  const int row_c = min(row, rows - 1);
  const int qi = row_c / a.H;
  const int n_allowed = a.causal ? (L - a.s_q + qi + 1) : L;
  // Smallest allowed count over all rows (query 0's), the same for every wave.
  const int n_allowed_min = a.causal ? (L - a.s_q + 1) : L;

  // Q^T fragments for the whole walk: k-step s holds q[row][32s + 8*g16 .. +8].
  bf16x8_t qf[kQSteps];
  {
    const __bf16* qrow = reinterpret_cast<const __bf16*>(a.q_lat) + ((size_t)b * rows + row_c) * kDqk + 8 * g16;
#pragma unroll
    for (int s = 0; s < kQSteps; ++s) qf[s] = *reinterpret_cast<const bf16x8_t*>(qrow + 32 * s);
  }

  f32x4_t acc_o[kColTiles];
#pragma unroll
  for (int ct = 0; ct < kColTiles; ++ct) acc_o[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY;  // base-2 reference max of this row
  float l_loc = 0.f;        // this lane's share of the row's sum of P
  const float sl2 = a.scale * 1.4426950408889634f;

  const char* cache = reinterpret_cast<const char*>(a.kv_cache);
  const int32_t* btab = a.block_table + (size_t)b * a.max_pages;
  const int last_phys = a.num_pages - 1;

  // Per-lane LDS byte offsets inside a buffer.
  // QK A operand for token tile t, k-step s: token 16t + r16, chunk 4s + g16:
  //   1024*(18t + 9*(r16>>3) + (s>>1)) + 128*(r16&7) + 16*((4*(s&1) + g16) ^ F(r16)).
  const int qk_base = 1024 * 9 * (r16 >> 3) + 128 * (r16 & 7);
  const int qk_x0 = 16 * (g16 ^ swz(r16));
  const int qk_x1 = 16 * ((4 + g16) ^ swz(r16));
  // PV A operand (transposed read) for k-step u, read rd, column tile ct: lane
  // group g16 reads tokens 32u + 16rd + 4*g16 + jj (jj = (lane>>2)&3) and the
  // lane supplies the 4 columns from 16ct + 4*qq (qq = lane&3), i.e. chunk
  // 2ct + (qq>>1), half-chunk qq&1:
  //   1024*(9*(4u + 2rd + (g16>>1)) + (ct>>2)) + 128*(4*(g16&1) + jj)
  //   + 16*((2*(ct&3)) ^ Z) + 8*(qq&1),  Z = (qq>>1) ^ F(token).
  const int jj = (lane >> 2) & 3;
  const int qq = lane & 3;
  const int pv_tok = 4 * g16 + jj;  // token within its 16-token block
  const int pv_base = 1024 * 9 * (g16 >> 1) + 128 * (4 * (g16 & 1) + jj) + 8 * (qq & 1);
  const int pv_z = (qq >> 1) ^ swz(pv_tok);

  if (pg0 < pg1) {
    const int phys = min(max(btab[pg0], 0), last_phys);
    issue_page(make_page_load(cache + (size_t)phys * kPageBytes, smem, wave, lane));
  }

  for (int pg = pg0; pg < pg1; ++pg) {
    char* buf = smem + ((pg - pg0) & 1) * kPageBytes;
    // Page pg has landed: each wave waits for its own direct loads (vmcnt 0;
    // nothing else is outstanding), then the barrier publishes all of them
    // and also guarantees every wave is done with the other buffer.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    // An active wave issues the next page's loads one per QK k-step below,
    // so they drain behind the MFMAs instead of stalling the wave here.
    // (Built unconditionally, from a clamped table index, so that its bases
    // stay plain wave-uniform values in SGPRs.)
    const bool has_next = pg + 1 < pg1;
    const int phys_next = min(max(btab[min(pg + 1, pg1 - 1)], 0), last_phys);
    const PageLoad next = make_page_load(cache + (size_t)phys_next * kPageBytes,
                                         smem + ((pg + 1 - pg0) & 1) * kPageBytes, wave, lane);
    if (has_next && !wave_active) issue_page(next);
    const int valid = L - pg * kPage;  // tokens of this page that exist
    if (valid < kPage) {
      // Zero the token slots past the end of the sequence: their scores are
      // masked, but 0 * NaN in PV would still poison the sum.
      for (int idx = threadIdx.x; idx < (kPage - valid) * 72; idx += kThreads) {
        const int t = valid + idx / 72;
        const int c = idx % 72;
        *reinterpret_cast<uint4*>(buf + slot_bytes(t, c)) = make_uint4(0, 0, 0, 0);
      }
      __syncthreads();
    }
    if (!wave_active) continue;

    // ---- S^T = K Q^T for the 64 tokens: 4 token tiles x 18 k-steps; the
    // K fragments of k-step s+1 are read while the MFMAs of step s run. Two
    // copies (with and without the next page's loads) keep the k-step loop
    // free of branches.
    f32x4_t st[4];
    const char* qa = buf + qk_base;
    auto qk = [&](auto with_loads) {
#pragma unroll
      for (int t = 0; t < 4; ++t) st[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      bf16x8_t kf[2][4];
#pragma unroll
      for (int t = 0; t < 4; ++t) kf[0][t] = *reinterpret_cast<const bf16x8_t*>(qa + 1024 * 18 * t + qk_x0);
#pragma unroll
      for (int s = 0; s < kQSteps; ++s) {
        if constexpr (decltype(with_loads)::value) issue_line(next, s);
        if (s + 1 < kQSteps) {
#pragma unroll
          for (int t = 0; t < 4; ++t)
            kf[(s + 1) & 1][t] = *reinterpret_cast<const bf16x8_t*>(
                qa + 1024 * (18 * t + ((s + 1) >> 1)) + (((s + 1) & 1) ? qk_x1 : qk_x0));
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) st[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[s & 1][t], qf[s], st[t], 0, 0, 0);
      }
    };
    if (has_next) qk(std::true_type{}); else qk(std::false_type{});

    // ---- scale, mask, row max (token of st[t][r] = 64pg + 16t + 4g16 + r).
    // Pages wholly inside every row's allowed range skip the mask.
    const int tok0 = pg * kPage + 4 * g16;
    float mx = -INFINITY;
    if ((pg + 1) * kPage <= n_allowed_min) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          st[t][r] *= sl2;
          mx = fmaxf(mx, st[t][r]);
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = (tok0 + 16 * t + r < n_allowed) ? st[t][r] * sl2 : -INFINITY;
          st[t][r] = v;
          mx = fmaxf(mx, v);
        }
      }
    }
    mx = max4lanes(mx);
    const float m_new = fmaxf(m_ref, mx);
    if (__any(m_new > m_ref + 8.0f)) {
      const float alpha = (m_ref == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_new);
      l_loc *= alpha;
#pragma unroll
      for (int ct = 0; ct < kColTiles; ++ct) acc_o[ct] *= alpha;
      m_ref = m_new;
    }
    const float mref = (m_ref == -INFINITY) ? 0.f : m_ref;

    // ---- P = exp2(v - m_ref), packed to bf16 as the PV B operand:
    // k-step u takes tiles 2u (k 0..3 of each lane group) and 2u+1 (k 4..7).
    bf16x8_t pf[2];
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = __builtin_amdgcn_exp2f(st[t][r] - mref);
        psum += p;
        pf[t >> 1][4 * (t & 1) + r] = (__bf16)p;
      }
    }
    l_loc += psum;

    // ---- O^T += V^T P^T: 2 k-steps of 32 tokens x 32 column tiles; the V^T
    // fragments run 4 MFMAs ahead of their use.
    const char* va = buf + pv_base;
    auto load_v = [&](int i) {
      const int u = i >> 5, ct = i & 31;
      bf16x8_t av;
#pragma unroll
      for (int rd = 0; rd < 2; ++rd) {
        const int off = 1024 * (9 * (4 * u + 2 * rd) + (ct >> 2)) + 16 * ((2 * (ct & 3)) ^ pv_z);
        const bf16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(va + off));
        av[4 * rd + 0] = v[0];
        av[4 * rd + 1] = v[1];
        av[4 * rd + 2] = v[2];
        av[4 * rd + 3] = v[3];
      }
      return av;
    };
    constexpr int kPvDepth = 4;
    bf16x8_t vf[kPvDepth];
#pragma unroll
    for (int i = 0; i < kPvDepth; ++i) vf[i] = load_v(i);
#pragma unroll
    for (int i = 0; i < 2 * kColTiles; ++i) {
      const bf16x8_t cur = vf[i % kPvDepth];
      if (i + kPvDepth < 2 * kColTiles) vf[i % kPvDepth] = load_v(i + kPvDepth);
      acc_o[i & 31] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur, pf[i >> 5], acc_o[i & 31], 0, 0, 0);
    }
  }

  if (!wave_active) return;

  // ---- finalize: o = O / l, lse = ln2 * (m_ref + log2 l)
  const float l_tot = sum4lanes(l_loc);
  const bool any = l_tot > 0.f;
  const float inv = any ? 1.f / l_tot : 0.f;
  const float lse_v = any ? (m_ref + __log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
  if (row >= rows) return;

  // acc_o[ct][r] is O^T[16ct + 4g16 + r][row]: four consecutive columns.
  if (n_chunks == 1 && a.o_lat != nullptr) {
    __bf16* orow = reinterpret_cast<__bf16*>(a.o_lat) + ((size_t)b * rows + row) * kDv + 4 * g16;
#pragma unroll
    for (int ct = 0; ct < kColTiles; ++ct) {
      bf16x4_t v;
      v[0] = (__bf16)(acc_o[ct][0] * inv);
      v[1] = (__bf16)(acc_o[ct][1] * inv);
      v[2] = (__bf16)(acc_o[ct][2] * inv);
      v[3] = (__bf16)(acc_o[ct][3] * inv);
      *reinterpret_cast<bf16x4_t*>(orow + 16 * ct) = v;
    }
    if (g16 == 0) a.lse[(size_t)b * rows + row] = lse_v;
  } else {
    float* orow = a.o_part + ((size_t)g * rows + row) * kDv + 4 * g16;
#pragma unroll
    for (int ct = 0; ct < kColTiles; ++ct) *reinterpret_cast<f32x4_t*>(orow + 16 * ct) = acc_o[ct] * inv;
    if (g16 == 0) a.lse_part[(size_t)g * rows + row] = lse_v;
  }
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream) {
  const int rows = a.s_q * a.H;
  const int row_groups = (rows + kRowsPerGroup - 1) / kRowsPerGroup;
  const int padded = (a.total_splits + 7) / 8 * 8;
  const dim3 grid((unsigned)(padded * row_groups));
  hipLaunchKernelGGL(mla_decode_bf16_kernel, grid, dim3(kThreads), 0, stream, a, row_groups);
  return hipGetLastError();
}

}  // namespace mla

// Absorbed-MLA decode, bf16 storage, fp32 accumulation, for gfx950 (MI355X).
//
// What it computes ("MLA 推理：两条计算路径与 FlashMLA", sections "两条等价的路径"
// and "decode 注意力变成了计算问题"): every (query token, head) row attends to
// one shared 576-wide key per cached token and one shared 512-wide value (the
// first 512 elements of the same cache row), i.e. an MQA with a very wide
// head. Heads are the matrix M dimension, the latent the K dimension, and one
// workgroup holds 128 rows and walks a range of 64-token pages.
//
// Layout of the work
//   * Workgroup = 4 waves x 32 rows. A row is (query token i, head h),
//     m = i*H + h, so q_lat[b] is a [s_q*H, 576] matrix.
//   * Per page, the 73,728-byte page is copied HBM -> LDS with direct 16-byte
//     loads (global_load_lds_dwordx4), double-buffered so the next page
//     streams in while the current one is consumed. The four waves share it.
//   * QK^T is computed transposed, S^T[token, row] = K . Q^T, with
//     v_mfma_f32_32x32x16_bf16: A = 32 tokens x 16 latent elements read from
//     LDS, B = Q^T kept in registers for the whole walk (36 k-steps). In that
//     layout each lane owns one row and 32 of its 64 token scores, so the
//     softmax max/sum need one cross-lane step (lanes l and l^32).
//   * PV is computed transposed too, O^T[col, row] += V^T . P^T: A = V^T read
//     with ds_read_b64_tr_b16 (4x16 -> 16x4 transposes within 16 lanes),
//     B = P^T straight from the score registers after a bf16 pack. The token
//     order inside each 16-token k-step is permuted identically on both sides
//     so the score registers need no shuffling.
//   * Online softmax in base 2 with a lazily updated reference max: the
//     accumulators are rescaled only when a row's max grows by more than 8
//     (then P <= 2^8); the result is exact because P, l and O always share
//     the same reference.
//   * Split-KV: a workgroup handles chunk k of n_b page-aligned chunks of its
//     sequence. With n_b = 1 it writes bf16 o_lat and LSE directly; otherwise
//     fp32 partials that the combine kernel merges by LSE.
//
// LDS tile layout (chunk-major): a page is 64 tokens x 72 chunks of 16 bytes
// (8 elements). Chunk k of token t sits at byte k*1088 + t*16: each chunk
// column holds the 64 tokens contiguously and columns are padded by 64 bytes.
// One direct-load instruction moves chunk k of all 64 tokens (lane = token),
// so every load of a page uses the same per-lane source offset. The QK reads
// (16 lanes = 16 consecutive tokens of one chunk) touch 256 contiguous bytes,
// and the transposed PV reads (4 tokens x 4 chunks per 32 lanes) land in four
// different 64-byte bank windows thanks to the padding: no bank conflicts.

#include <hip/hip_runtime.h>
#include <cmath>
#include <cstdint>

#include "mla_internal.h"

namespace mla {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8_t;
typedef __attribute__((address_space(1))) const void gbl_cvoid_t;

constexpr int kThreads = 256;
constexpr int kRowBytes = kDqk * 2;                  // 1152: one cache row
constexpr int kPageBytes = kPage * kRowBytes;        // 73728: one page in HBM
constexpr int kChunks = kRowBytes / 16;              // 72 chunks of 8 elements
constexpr int kChunkStride = kPage * 16 + 64;        // 1088: padded chunk column
constexpr int kBufBytes = kChunks * kChunkStride;    // 78336: one page in LDS
constexpr int kChunksPerWave = kChunks / 4;          // 18 load instructions
static_assert(kChunksPerWave * 4 == kChunks, "chunks must split evenly over the waves");
// s_waitcnt immediate for gfx9: vmcnt = 0, expcnt and lgkmcnt left at "no wait".
constexpr int kWaitVmcnt0 = (0xF << 8) | (0x7 << 4);

// Copy one page into an LDS buffer. Wave w moves chunks 18w .. 18w+17; for
// chunk k, lane t reads token t's 16 bytes at t*1152 + 16k and the hardware
// writes them to LDS at k*1088 + 16t.
__device__ __forceinline__ void issue_page_load(const char* page_src, char* lds_buf, int wave, int lane) {
  const char* src = page_src + lane * kRowBytes + wave * (kChunksPerWave * 16);
  char* dst = lds_buf + wave * (kChunksPerWave * kChunkStride);
#pragma unroll
  for (int n = 0; n < kChunksPerWave; ++n)
    __builtin_amdgcn_global_load_lds((gbl_cvoid_t*)(src + 16 * n), (lds_void_t*)(dst + n * kChunkStride), 16, 0, 0);
}

__device__ __forceinline__ float wave_xor32(float v) { return __shfl_xor(v, 32, 64); }

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
  __shared__ __attribute__((aligned(1024))) char smem[2 * kBufBytes];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;   // which 8-element k slice / 4-token group the lane holds
  const int lrow = lane & 31;   // the row this lane owns in MFMA outputs

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
  const int wave_row0 = rgrp * kRowsPerGroup + wave * 32;
  const bool wave_active = wave_row0 < rows;
  const int row = wave_row0 + lrow;
  const int row_c = min(row, rows - 1);
  const int qi = row_c / a.H;
  const int n_allowed = a.causal ? (L - a.s_q + qi + 1) : L;

  // Q^T fragments for the whole walk: k-step s holds q[row][16s + 8*half .. +8].
  bf16x8_t qf[36];
  {
    const __bf16* qrow = reinterpret_cast<const __bf16*>(a.q_lat) + ((size_t)b * rows + row_c) * kDqk + 8 * half;
#pragma unroll
    for (int s = 0; s < 36; ++s) qf[s] = *reinterpret_cast<const bf16x8_t*>(qrow + 16 * s);
  }

  f32x16_t acc_o[16];
#pragma unroll
  for (int ct = 0; ct < 16; ++ct) acc_o[ct] = f32x16_t{};
  float m_ref = -INFINITY;  // base-2 reference max of this row
  float l_loc = 0.f;        // this lane's share of the row's sum of P
  const float sl2 = a.scale * 1.4426950408889634f;

  const char* cache = reinterpret_cast<const char*>(a.kv_cache);
  const int32_t* btab = a.block_table + (size_t)b * a.max_pages;
  const int last_phys = a.num_pages - 1;

  // Per-lane LDS byte offsets (relative to a buffer).
  // QK A operand: token lrow (+32 for the second tile), chunk 2s + half.
  const int qk_base = half * kChunkStride + lrow * 16;
  // PV A operand (transposed read): lane group g4 = lane/16 covers 16 columns
  // (column half g4&1) and tokens 4*(g4>>1) + j, j = (lane%16)/4; the lane
  // supplies the address of the 4 columns starting at 4*(lane%4).
  const int g4 = lane >> 4;
  const int jj = (lane >> 2) & 3;
  const int qq = lane & 3;
  const int pv_base = (2 * (g4 & 1) + (qq >> 1)) * kChunkStride + (4 * (g4 >> 1) + jj) * 16 + (qq & 1) * 8;

  if (pg0 < pg1) {
    const int phys = min(max(btab[pg0], 0), last_phys);
    issue_page_load(cache + (size_t)phys * kPageBytes, smem, wave, lane);
  }

  for (int pg = pg0; pg < pg1; ++pg) {
    char* buf = smem + ((pg - pg0) & 1) * kBufBytes;
    // Page pg has landed: each wave waits for its own direct loads (vmcnt 0;
    // nothing else is outstanding), then the barrier publishes all of them.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (pg + 1 < pg1) {
      const int phys = min(max(btab[pg + 1], 0), last_phys);
      issue_page_load(cache + (size_t)phys * kPageBytes, smem + ((pg + 1 - pg0) & 1) * kBufBytes, wave, lane);
    }
    const int valid = L - pg * kPage;  // tokens of this page that exist
    if (valid < kPage) {
      // Zero the token slots past the end of the sequence: their scores are
      // masked, but 0 * NaN in PV would still poison the sum.
      for (int idx = threadIdx.x; idx < (kPage - valid) * kChunks; idx += kThreads) {
        const int t = valid + idx / kChunks;
        const int k = idx % kChunks;
        *reinterpret_cast<uint4*>(buf + k * kChunkStride + t * 16) = make_uint4(0, 0, 0, 0);
      }
      __syncthreads();
    }
    if (!wave_active) continue;

#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {  // two 32-token halves of the page
      // ---- S^T = K Q^T for 32 tokens
      f32x16_t sc = f32x16_t{};
      const char* qa = buf + qk_base + tt * 32 * 16;
#pragma unroll
      for (int s = 0; s < 36; ++s) {
        const bf16x8_t a0 = *reinterpret_cast<const bf16x8_t*>(qa + 2 * s * kChunkStride);
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[s], sc, 0, 0, 0);
      }

      // ---- scale, mask, row max
      const int tok0 = pg * kPage + tt * 32 + 4 * half;
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = tok0 + 8 * (r >> 2) + (r & 3);
        const float v = (t < n_allowed) ? sc[r] * sl2 : -INFINITY;
        sc[r] = v;
        mx = fmaxf(mx, v);
      }
      mx = fmaxf(mx, wave_xor32(mx));
      const float m_new = fmaxf(m_ref, mx);
      if (__any(m_new > m_ref + 8.0f)) {
        const float alpha = (m_ref == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_new);
        l_loc *= alpha;
#pragma unroll
        for (int ct = 0; ct < 16; ++ct) acc_o[ct] *= alpha;
        m_ref = m_new;
      }
      const float mref = (m_ref == -INFINITY) ? 0.f : m_ref;

      // ---- P = exp2(v - m_ref), packed to bf16 as the PV B operand
      bf16x8_t pf[2];
      float psum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(sc[r] - mref);
        psum += p;
        pf[r >> 3][r & 7] = (__bf16)p;
      }
      l_loc += psum;

      // ---- O^T += V^T P^T over these 32 tokens (k-steps 2tt, 2tt+1)
      const char* va = buf + pv_base + tt * 32 * 16;
#pragma unroll
      for (int ct = 0; ct < 16; ++ct) {
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          bf16x8_t av;
#pragma unroll
          for (int rd = 0; rd < 2; ++rd) {
            const int off = 4 * ct * kChunkStride + (16 * k2 + 8 * rd) * 16;
            const bf16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(va + off));
            av[4 * rd + 0] = v[0];
            av[4 * rd + 1] = v[1];
            av[4 * rd + 2] = v[2];
            av[4 * rd + 3] = v[3];
          }
          acc_o[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pf[k2], acc_o[ct], 0, 0, 0);
        }
      }
    }
  }

  if (!wave_active) return;

  // ---- finalize: o = O / l, lse = ln2 * (m_ref + log2 l)
  const float l_tot = l_loc + wave_xor32(l_loc);
  const bool any = l_tot > 0.f;
  const float inv = any ? 1.f / l_tot : 0.f;
  const float lse_v = any ? (m_ref + __log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
  if (row >= rows) return;

  if (n_chunks == 1) {
    __bf16* orow = reinterpret_cast<__bf16*>(a.o_lat) + ((size_t)b * rows + row) * kDv + 4 * half;
#pragma unroll
    for (int ct = 0; ct < 16; ++ct) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4_t v;
        v[0] = (__bf16)(acc_o[ct][4 * r4 + 0] * inv);
        v[1] = (__bf16)(acc_o[ct][4 * r4 + 1] * inv);
        v[2] = (__bf16)(acc_o[ct][4 * r4 + 2] * inv);
        v[3] = (__bf16)(acc_o[ct][4 * r4 + 3] * inv);
        *reinterpret_cast<bf16x4_t*>(orow + 32 * ct + 8 * r4) = v;
      }
    }
    if (half == 0) a.lse[(size_t)b * rows + row] = lse_v;
  } else {
    float* orow = a.o_part + ((size_t)g * rows + row) * kDv + 4 * half;
#pragma unroll
    for (int ct = 0; ct < 16; ++ct) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4_t v;
        v[0] = acc_o[ct][4 * r4 + 0] * inv;
        v[1] = acc_o[ct][4 * r4 + 1] * inv;
        v[2] = acc_o[ct][4 * r4 + 2] * inv;
        v[3] = acc_o[ct][4 * r4 + 3] * inv;
        *reinterpret_cast<f32x4_t*>(orow + 32 * ct + 8 * r4) = v;
      }
    }
    if (half == 0) a.lse_part[(size_t)g * rows + row] = lse_v;
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

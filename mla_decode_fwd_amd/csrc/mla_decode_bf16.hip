// Absorbed-MLA decode, bf16 storage, fp32 accumulation, for gfx950 (MI355X).
//
// What it computes ("MLA 推理：两条计算路径与 FlashMLA", sections "两条等价的路径"
// and "decode 注意力变成了计算问题"): every (query token, head) row attends to
// one shared 576-wide key per cached token and one shared 512-wide value (the
// first 512 elements of the same cache row), i.e. an MQA with a very wide
// head.
//
// Work decomposition
//   * A row is (query token i, head h), m = i*H + h, so q_lat[b] is an
//     [s_q*H, 576] matrix. A workgroup holds 128 rows (all heads of one new
//     token at H = 128) and walks a range of 64-token pages of one sequence,
//     so every page crosses HBM once per chunk and each compute unit has a
//     page of its own in flight.
//   * Each page (73,728 bytes) is copied HBM -> LDS with direct 16-byte loads
//     (global_load_lds_dwordx4), double-buffered: the next page streams in
//     while the four waves consume the current one.
//   * Four waves, one per SIMD, 32 rows each. A wave holds Q^T for its rows
//     in VGPRs (36 k-steps, 144 registers) and O^T for its rows in AGPRs
//     (16 column tiles of 32x32 fp32, the whole AGPR file): every LDS byte a
//     wave reads feeds 32 rows, and the waves never exchange data.
//   * A page is two 32-token tiles. Per tile: S^T = K . Q^T with
//     v_mfma_f32_32x32x16_bf16 (A = 32 tokens x 16 latent elements from LDS,
//     B = Q^T), an online softmax on the 16 scores a lane holds (one row,
//     lanes l and l^32 share a row), then O^T += V^T . P^T (A = V^T read from
//     the same LDS page with ds_read_b64_tr_b16, a 4x16 -> 16x4 transpose
//     within each 16-lane group; B = P^T taken straight from the score
//     registers: the score layout of a 16-token half tile is exactly the B
//     layout of one k-step with the tokens of the k-step permuted, and the
//     V^T reads use the same permutation). The two tiles are staggered in
//     the source: each tile's exponentials run between the MFMAs of the
//     other tile's product, one per MFMA (an exponential issues at quarter
//     rate), held in those slots by empty asm uses (the compiler otherwise
//     sinks them to the first PV MFMA that reads them).
//   * With few sequences, a 64-row variant puts two workgroups on each page
//     range: a wave pair shares 32 rows, each wave takes one 32-token tile
//     of every page, and the pair merges its two (m, l, O) at the end.
//   * Softmax in base 2 with a lazily updated reference max: O and l are
//     rescaled only when a row's max grows by more than 8 (so P <= 2^8); the
//     result is exact because P, l and O always share the reference.
//   * Split-KV: a workgroup handles chunk k of n_b page-aligned chunks of its
//     sequence. With n_b = 1 it writes bf16 o_lat and the LSE directly;
//     otherwise (or when only partials are asked for) bf16 partials and fp32
//     LSEs that the combine kernel merges.
//
// LDS page layout ("line blocks"): the page is split into 72 blocks of 1 KB.
// Block 9m + j holds, for the 8 tokens t = 8m .. 8m+7, the 128-byte line j
// (chunks 8j .. 8j+7 of 8 elements) of each token's row: token t, chunk c
// sits in 16-byte slot 64*(9*(t>>3) + (c>>3)) + 8*(t&7) + ((c&7) ^ F(t)),
// F(t) = ((u&1) << 2) | (u >> 1), u = (t>>1) & 7. Every direct-load
// instruction therefore reads 8 whole 128-byte lines (fully coalesced), and
// the XOR keeps the QK reads (16 lanes = 16 tokens of one chunk) and the
// transposed PV reads (2 x 4 tokens x 16 columns per 32 lanes) free of LDS
// bank conflicts.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "mla_decode_common.h"
#include "mla_internal.h"

namespace mla {
namespace {

using namespace dec;

constexpr int kRowBytes = kDqk * 2;                // 1152: one cache row
constexpr int kPageBytes = kPage * kRowBytes;      // 73728: one page
constexpr int kBlocks = kPageBytes / 1024;         // 72 line blocks
constexpr int kBlocksPerWave = kBlocks / kWaves;   // 18: two token octets per wave
static_assert(2 * kPageBytes >= kWaves * kWaveRows * kDv * 2, "the output staging fits in the page buffers");
static_assert(kBlocksPerWave == 18, "each wave loads two token octets");

__device__ __forceinline__ int swz(int t) {
  const int u = (t >> 1) & 7;
  return ((u & 1) << 2) | (u >> 1);
}
__device__ __forceinline__ int slot_bytes(int t, int c) {
  return (64 * (9 * (t >> 3) + (c >> 3)) + 8 * (t & 7) + ((c & 7) ^ swz(t))) * 16;
}


// The loads of one page into an LDS buffer. Wave w fills blocks 18w .. 18w+17:
// token octets 2w and 2w+1, lines j = 0..8 each. Lane l takes token
// 8m + (l>>3), chunk 8j + ((l&7) ^ F(token)); F depends on the token, hence
// two per-lane source offsets. Line n (0..17) of the wave is octet n/9, line
// n%9.
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
  // Global: page + off + 128j; LDS: block 9*octet + j. The 128j goes in the
  // instruction's immediate, which both addresses take (measured on MI355X:
  // a 128-row page 5820 -> 5720 cycles, the same bits out).
  dma_line_off(p.sbase, octet ? p.off1 : p.off0, p.lds, 1024 * (9 * octet + j) - 128 * j, 128 * j);
}

__device__ __forceinline__ void issue_page(const PageLoad& p) {
#pragma unroll
  for (int n = 0; n < kBlocksPerWave; ++n) issue_line(p, n);
}

// The query rows of a workgroup go to the MFMA operand registers through
// LDS. Loaded straight into the B layout of v_mfma_f32_32x32x16_bf16 (lane
// l: 16 bytes of row l&31), each of the 36 load instructions of a wave would
// touch 32 rows with 32 bytes each, and the address unit spends ~3 us per
// workgroup on them (measured on MI355X: the first page of a chunk landed
// 8.2 us after the chunk began, 5.0 us with a quarter of those loads).
// Direct loads instead fill LDS in 1 KB runs of contiguous row bytes, and
// each wave then reads its operands with one 16-byte LDS read per k-step.
// Rows sit at a stride of their length + 16 bytes, so the 16 rows of a read
// pass start on 16 different 4-bank groups. A 128-row group stages dims
// 0..287 and then 288..575 of every row (two rounds of 74 KB; the first
// overlaps the first page's load); a 64-row group stages whole rows in one
// round (73 KB). The staging area is the second page buffer, extended by
// kQStageExtra bytes. (Loading half of the rows' dims directly instead of a
// second round was measured slower: its address work delays the page.)
constexpr int kQStageExtra = 2048;

// Top-k decode: a "page" is 64 listed tokens whose rows sit anywhere in the
// pool, so each lane carries its own two source addresses (the rows of its
// two tokens, at its chunk) and the load takes a 64-bit VGPR address. The
// LDS side is the page layout above, unchanged.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma_line_addr(uint64_t vaddr, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off nt"
      :
      : "v"(vaddr), "s"(lds)
      : "memory", "m0");
}
#pragma clang diagnostic pop

struct GatherLoad {
  uint64_t src0, src1;  // per-lane row addresses of the wave's two token octets, at the lane's chunk
  uint32_t lds;         // LDS address of the wave's first block (wave-uniform)
};

// row_ids: the 64 physical row numbers (page * 64 + slot) of the listed tokens.
__device__ __forceinline__ GatherLoad make_gather_load(const char* cache, const int32_t* row_ids, char* lds_buf,
                                                       int wave, int lane) {
  GatherLoad p;
  char* dst = lds_buf + wave * (kBlocksPerWave * 1024);
  p.lds = (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)(uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)dst);
  const int t0 = 16 * wave + (lane >> 3);
  p.src0 = (uint64_t)(uintptr_t)(cache + (size_t)row_ids[t0] * kRowBytes + (((lane & 7) ^ swz(t0)) * 16));
  p.src1 = (uint64_t)(uintptr_t)(cache + (size_t)row_ids[t0 + 8] * kRowBytes + (((lane & 7) ^ swz(t0 + 8)) * 16));
  return p;
}

__device__ __forceinline__ void issue_line(const GatherLoad& p, int n) {
  const int octet = n / 9, j = n % 9;
  dma_line_addr((octet ? p.src1 : p.src0) + 128 * j, p.lds + 1024 * (9 * octet + j));
}

__device__ __forceinline__ void issue_page(const GatherLoad& p) {
#pragma unroll
  for (int n = 0; n < kBlocksPerWave; ++n) issue_line(p, n);
}

// One chunk of work: query rows of row group `rgrp` of sequence b against
// pages [pg0, pg1) of the sequence (dense), or against 64-entry "pages"
// [pg0, pg1) of the query token's selected-token list (kSparse: top-k
// decode; the prologue resolves the chunk's entries through the block table
// into physical row numbers, kept in LDS after the page buffers with one
// 64-bit validity mask per page, each page is then gathered row by row, and
// entries outside [0, L_b) are masked out of the softmax; their slot is
// loaded from the sequence's token 0, so P = 0 meets finite values).
//
// kHalf: a 64-row group. Waves w and w^2 hold the same 32 rows; wave w takes
// the 32-token tile w>>1 of every page (its own QK, softmax and PV), and at
// the end the tile-1 wave hands its running max, sum and O to the tile-0
// wave through LDS, which merges them and writes the rows. Every page is
// still loaded whole by all four waves.
//
// part: the partial's index (the chunk's index in the merge layout); direct:
// the chunk is its sequence's only one and outputs go straight to o_lat/lse.
template <bool kSparse, bool kHalf>
__device__ __forceinline__ void decode_chunk(const DecodeArgs& a, char* smem, const int b, const int L, const int pg0,
                                             const int pg1, const int part, const bool direct, const int rgrp,
                                             const int wave) {
  // The lane index and H are made opaque here, so that the per-lane LDS
  // offsets and the row arithmetic derived from them are computed inside
  // each chunk rather than hoisted out of a workgroup's chunk loop, where
  // they would stay live (and spill) across every chunk's page loop.
  const int lane = lane_id();
  const int tid = wave * 64 + lane;
  int H = a.H;
  asm volatile("" : "+s"(H));
  const char* q_base = static_cast<const char*>(a.q_lat);
  asm volatile("" : "+s"(q_base));
  const int r32 = lane & 31;   // the row this lane owns in MFMA outputs
  const int hi32 = lane >> 5;  // upper half of the wave
  constexpr int kGroupRows = kHalf ? kRowsPerGroup / 2 : kRowsPerGroup;
  const int slice = kHalf ? (wave & 1) : wave;  // 32-row slice of the row group
  const int my_tile = wave >> 1;                // kHalf: the page tile this wave takes

  // Rows past the end (H*s_q not a multiple of 32) compute on a clamped row
  // and write nothing.
  const int rows = a.s_q * H;
  const int row = rgrp * kGroupRows + slice * kWaveRows + r32;
  const int row_c = min(row, rows - 1);
  const int qi = row_c / H;
  const int n_allowed = a.causal ? (L - a.s_q + qi + 1) : L;
  // Smallest allowed count over all rows (query 0's), the same for every wave.
  const int n_allowed_min = a.causal ? (L - a.s_q + 1) : L;

  const char* cache = reinterpret_cast<const char*>(a.kv_cache);
  const int32_t* btab = a.block_table + (size_t)b * a.max_pages;
  const int last_phys = a.num_pages - 1;

  int32_t* const s_ids = reinterpret_cast<int32_t*>(smem + 2 * kPageBytes);  // top-k only
  uint64_t* const s_mask = reinterpret_cast<uint64_t*>(smem + 2 * kPageBytes + kSparseMaxTopk * 4);

  // Dense: the first two block-table entries are requested, then the Q loads
  // are issued while they travel, then the first page's loads. Later entries
  // are read one page ahead of their use, so that no page waits on a table
  // read. Top-k: the chunk's list entries, then their table entries, are
  // requested before the Q loads.
  constexpr int kIt = kSparseMaxTopk / kThreads;
  int bt0 = 0, bt1 = 0;
  int lpos[kSparse ? kIt : 1], lphys[kSparse ? kIt : 1];
  if constexpr (kSparse) {
    const int32_t* list = a.indices + ((size_t)b * a.s_q + rgrp) * a.topk;  // H = 128: row group = query token
    const int n_tok = (pg1 - pg0) * kPage;  // <= kSparseMaxTopk
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const int t = it * kThreads + tid;
      const int e = pg0 * kPage + t;
      lpos[it] = (t < n_tok && e < a.topk) ? list[e] : -1;
    }
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const bool valid = lpos[it] >= 0 && lpos[it] < L;
      lphys[it] = btab[(valid ? lpos[it] : 0) >> 6];
    }
  } else {
    bt0 = btab[max(min(pg0, pg1 - 1), 0)];  // an empty chunk (pg0 == pg1) reads entry 0, unused
    bt1 = btab[max(min(pg0 + 1, pg1 - 1), 0)];
  }
  asm volatile("" ::: "memory");  // keep the table reads ahead of the Q loads
  __builtin_amdgcn_sched_barrier(0);

  // Q^T fragments for the whole walk: k-step s holds q[row][16s + 8*hi32 .. +8]
  // (the B layout of v_mfma_f32_32x32x16_bf16: lane l holds k = 8(l>>5) .. +8
  // of column l&31).
  bf16x8_t qf[kQSteps];
  if constexpr (kSparse) {
    const __bf16* qrow = reinterpret_cast<const __bf16*>(q_base) + ((size_t)b * rows + row_c) * kDqk + 8 * hi32;
#pragma unroll
    for (int s = 0; s < kQSteps; ++s) qf[s] = *reinterpret_cast<const bf16x8_t*>(qrow + 16 * s);
  } else {
    // Staged (issue_q_round): the first round goes out now, ahead of the
    // first page, and is read once it has landed; the page keeps loading.
    const char* const q_seq = q_base + (size_t)b * rows * (kDqk * 2);
    constexpr int kRound = kHalf ? 2 * kDqk : kDqk;  // bytes per row per round
    issue_q_round(q_seq, rows, rgrp * kGroupRows, kGroupRows, kRound, 0, smem + kPageBytes, wave, lane);
  }

  int phys_ahead = 0;
  if constexpr (kSparse) {
    // Physical row numbers of the chunk's entries (invalid ones point at the
    // sequence's token 0) and the per-page validity masks.
    const int n_tok = (pg1 - pg0) * kPage;
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const int t = it * kThreads + tid;
      const bool valid = lpos[it] >= 0 && lpos[it] < L;
      const unsigned long long m = __ballot(valid);  // wave w of round it holds page 4*it + w
      if (t < n_tok) {
        s_ids[t] = min(max(lphys[it], 0), last_phys) * kPage + ((valid ? lpos[it] : 0) & (kPage - 1));
        if (lane == 0) s_mask[t >> 6] = m;
      }
    }
    __syncthreads();
    if (pg0 < pg1) issue_page(make_gather_load(cache, s_ids, smem, wave, lane));
  } else {
    if (pg0 < pg1) {
      const int phys = min(max(bt0, 0), last_phys);
      issue_page(make_page_load(cache + (size_t)phys * kPageBytes, smem, wave, lane));
      phys_ahead = bt1;
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(kBlocksPerWave));  // the query round, not the page
    } else {
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    }
    __syncthreads();
    const char* const area = smem + kPageBytes;
    const int R = slice * kWaveRows + r32;  // this lane's row in the staged group
    if constexpr (kHalf) {
      const char* const src = area + R * (2 * kDqk + 16) + 16 * hi32;
#pragma unroll
      for (int s = 0; s < kQSteps; ++s) qf[s] = *reinterpret_cast<const bf16x8_t*>(src + 32 * s);
    } else {
      const char* const src = area + R * (kDqk + 16) + 16 * hi32;
#pragma unroll
      for (int s = 0; s < kQSteps / 2; ++s) qf[s] = *reinterpret_cast<const bf16x8_t*>(src + 32 * s);
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      __syncthreads();  // every wave has its first half: the area takes the second
      const char* const q_seq = q_base + (size_t)b * rows * (kDqk * 2);
      issue_q_round(q_seq, rows, rgrp * kGroupRows, kGroupRows, kDqk, kDqk, smem + kPageBytes, wave, lane);
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __syncthreads();
#pragma unroll
      for (int s = kQSteps / 2; s < kQSteps; ++s)
        qf[s] = *reinterpret_cast<const bf16x8_t*>(src + 32 * (s - kQSteps / 2));
    }
    // The next page's loads overwrite the area: every read must be done
    // before the page loop's first barrier.
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  }

  f32x16_t acc_o[kColTiles];
#pragma unroll
  for (int i = 0; i < kColTiles; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[i][r] = 0.f;
  float m_ref = -INFINITY;  // base-2 reference max of this row
  float l_loc = 0.f;        // this lane's share of the row's sum of P
  const float sl2 = a.scale * 1.4426950408889634f;

  // Per-lane LDS byte offsets inside a page buffer.
  // QK A operand for token tile T, k-step s: token 32T + r32, chunk 2s + hi32:
  //   36864T + 1024*(9*(r32>>3) + (s>>2)) + 128*(r32&7) + 16*((2(s&3) + hi32) ^ F(r32)).
  const int qk_base = 1024 * 9 * (r32 >> 3) + 128 * (r32 & 7);
  int qk_x[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) qk_x[q] = qk_base + 16 * ((2 * q + hi32) ^ swz(r32));
  // PV A operand (transposed read) for k-step u, read rd, column tile i: lane
  // group g = lane>>4 reads tokens 16u + 8rd + 4(g>>1) + j (j = (lane>>2)&3)
  // and supplies the 4 columns from 32i + 16(g&1) + 4q (q = lane&3), i.e.
  // chunk 4i + 2(g&1) + (q>>1), half-chunk q&1:
  //   1024*(9*(2u + rd) + (i>>1)) + 128*(4(g>>1) + j)
  //   + 16*((4(i&1)) ^ Z_rd) + 8*(q&1),  Z_rd = (2(g&1) + (q>>1)) ^ F(token).
  const int g16 = lane >> 4;
  const int jj = (lane >> 2) & 3;
  const int qq = lane & 3;
  const int pv_base = 128 * (4 * (g16 >> 1) + jj) + 8 * (qq & 1);
  int pv_x[2][2];
#pragma unroll
  for (int rd = 0; rd < 2; ++rd) {
    const int z = (2 * (g16 & 1) + (qq >> 1)) ^ swz(8 * rd + 4 * (g16 >> 1) + jj);
    pv_x[rd][0] = pv_base + 16 * z;
    pv_x[rd][1] = pv_base + 16 * (z ^ 4);
  }

  for (int pg = pg0; pg < pg1; ++pg) {
    char* buf = smem + ((pg - pg0) & 1) * kPageBytes;
    // Page pg has landed: each wave waits for its own direct loads (vmcnt 0;
    // nothing else is outstanding), then the barrier publishes all of them
    // and also guarantees every wave is done with the other buffer.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    // The next page's 18 loads per wave are spread over this page's QK
    // k-steps: in a denser burst the four waves' loads queue up in the
    // address unit and stall the MFMA stream behind them. They are issued on
    // every page, the last one included, where the clamped table index makes
    // them reload the current page into the idle buffer: a uniform branch
    // around each load cost more than that one page's reload (measured on
    // MI355X: 200 cycles per page in the 64-row mode; the B=64 x 4096 step
    // 4-5 us and the MTP step 8-10 us shorter without the branches, with the
    // same results bit for bit). The bases stay wave-uniform SGPRs.
    char* const next_buf = smem + ((pg + 1 - pg0) & 1) * kPageBytes;
    const auto next = [&]() {
      if constexpr (kSparse) {
        return make_gather_load(cache, s_ids + (min(pg + 1, pg1 - 1) - pg0) * kPage, next_buf, wave, lane);
      } else {
        const int phys_next = min(max(phys_ahead, 0), last_phys);
        phys_ahead = btab[min(pg + 2, pg1 - 1)];
        return make_page_load(cache + (size_t)phys_next * kPageBytes, next_buf, wave, lane);
      }
    }();
    uint64_t page_mask = ~0ull;  // top-k: valid entries of this page
    if constexpr (kSparse) {
      const uint64_t m = s_mask[pg - pg0];
      page_mask = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(m >> 32)) << 32) |
                  (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)m);
    } else {
      const int valid = L - pg * kPage;  // tokens of this page that exist
      if (valid < kPage) {
        // Zero the token slots past the end of the sequence: their scores are
        // masked, but 0 * NaN in PV would still poison the sum.
        for (int idx = tid; idx < (kPage - valid) * 72; idx += kThreads) {
          const int t = valid + idx / 72;
          const int c = idx % 72;
          *reinterpret_cast<uint4*>(buf + slot_bytes(t, c)) = make_uint4(0, 0, 0, 0);
        }
        __syncthreads();
      }
    }
    const bool full_page = kSparse ? page_mask == ~0ull : (pg + 1) * kPage <= n_allowed_min;

    auto k_frag = [&](int T, int s) {
      return *reinterpret_cast<const bf16x8_t*>(buf + qk_x[s & 3] + 36864 * T + 1024 * (s >> 2));
    };
    auto v_frag = [&](int u, int i) {
      bf16x8_t av;
#pragma unroll
      for (int rd = 0; rd < 2; ++rd) {
        const bf16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4_t*)(buf + pv_x[rd][i & 1] + 1024 * (9 * (2 * u + rd) + (i >> 1))));
        av[4 * rd + 0] = v[0];
        av[4 * rd + 1] = v[1];
        av[4 * rd + 2] = v[2];
        av[4 * rd + 3] = v[3];
      }
      return av;
    };
    // Masked scores to -inf, then the base-2 row max over the tile. st[r]
    // belongs to token 64pg + 32T + 8(r>>2) + 4*hi32 + (r&3). The scale is
    // positive, so the max of the raw scores, scaled, is the max of the
    // scaled scores.
    auto tile_max = [&](f32x16_t& st, int T) {
      if (!full_page) {
        if constexpr (kSparse) {
          const uint32_t mt = (uint32_t)(page_mask >> (32 * T)) >> (4 * hi32);
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (!((mt >> (8 * (r >> 2) + (r & 3))) & 1u)) st[r] = -INFINITY;
        } else {
          const int tok0 = pg * kPage + 32 * T + 4 * hi32;
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (tok0 + 8 * (r >> 2) + (r & 3) >= n_allowed) st[r] = -INFINITY;
        }
      }
      float mx[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) mx[r] = fmaxf(st[r], st[r + 8]);
#pragma unroll
      for (int r = 0; r < 4; ++r) mx[r] = fmaxf(mx[r], mx[r + 4]);
      const float mt = fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]));
      return fmaxf(mt, other_half(mt)) * sl2;
    };
    // O and l to a new reference (nothing to rescale before the first
    // allowed key: O and l are still zero).
    auto move_reference = [&](float m_new) {
      if (__any(m_new > m_ref && m_ref != -INFINITY)) {
        const float alpha = (m_new > m_ref && m_ref != -INFINITY) ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.f;
        agpr_fence();
        scale_accumulators(alpha);
        l_loc *= alpha;
      }
      m_ref = m_new;
    };
    // Two P values of a tile (scores e and e+1), packed into the PV operand:
    // k-step kk of the tile takes scores 8kk .. 8kk+7. The empty asm uses
    // anchor the exponentials and the running sum where the call stands:
    // between the MFMAs they are meant to hide under. Without them the
    // compiler sinks every one of a tile's exponentials into the block of
    // the first MFMA that reads them (the next-page load branches split the
    // unrolled loop into blocks), where they run exposed.
    auto p_pair = [&](const f32x16_t& st, int e, float neg_ref, bf16x8_t* pf, float& psum) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[e], sl2, neg_ref));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[e + 1], sl2, neg_ref));
      asm volatile("" ::"v"(p0), "v"(p1));
      pf[e >> 3][e & 7] = (__bf16)p0;
      pf[e >> 3][(e & 7) + 1] = (__bf16)p1;
      psum += p0 + p1;
      asm volatile("" : "+v"(psum));
    };
    // One exponential per MFMA slot: its quarter-rate issue fits beside an
    // MFMA, two do not. Two slots compute a pair's exponentials, a third
    // packs them (measured on MI355X: a 128-row page 6020 -> 5810 cycles,
    // the same bits out; splitting the max over three slots as well did
    // not help).
    auto p_exp = [&](const f32x16_t& st, int e, float neg_ref) {
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(st[e], sl2, neg_ref));
      asm volatile("" ::"v"(p));
      return p;
    };
    auto p_pack = [&](int e, float p0, float p1, bf16x8_t* pf, float& psum) {
      pf[e >> 3][e & 7] = (__bf16)p0;
      pf[e >> 3][(e & 7) + 1] = (__bf16)p1;
      psum += p0 + p1;
      asm volatile("" : "+v"(psum));
    };
    float pa = 0.f, pb = 0.f;
    constexpr int kKDepth = 3;
    constexpr int kPvDepth = 4;

    if constexpr (kHalf) {
      // ---- One tile per wave: QK(T) with all 18 of the wave's next-page
      // loads (one every two k-steps), then the tile's P (the first k-step's
      // eight values up front, the other eight in PV's first twelve MFMA
      // slots) and PV(T).
      const int T = my_tile;
      f32x16_t st;
#pragma unroll
      for (int r = 0; r < 16; ++r) st[r] = 0.f;
      {
        bf16x8_t kf[kKDepth];
#pragma unroll
        for (int s = 0; s < kKDepth; ++s) kf[s] = k_frag(T, s);
#pragma unroll
        for (int s = 0; s < kQSteps; ++s) {
          const bf16x8_t cur = kf[s % kKDepth];
          if (s + kKDepth < kQSteps) kf[s % kKDepth] = k_frag(T, s + kKDepth);
          st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, qf[s], st, 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
          if ((s & 1) == 0) issue_line(next, s >> 1);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      const float mt = tile_max(st, T);
      move_reference((mt > m_ref + 8.0f) ? mt : m_ref);
      const float neg = (m_ref == -INFINITY) ? 0.f : -m_ref;
      bf16x8_t pf[2];
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; e += 2) p_pair(st, e, neg, pf, psum);
      {
        bf16x8_t vf[kPvDepth];
#pragma unroll
        for (int n = 0; n < kPvDepth; ++n) vf[n] = v_frag(2 * T + (n >> 4), n & 15);
#pragma unroll
        for (int n = 0; n < 2 * kColTiles; ++n) {
          const bf16x8_t cur = vf[n % kPvDepth];
          if (n + kPvDepth < 2 * kColTiles)
            vf[n % kPvDepth] = v_frag(2 * T + ((n + kPvDepth) >> 4), (n + kPvDepth) & 15);
          if ((n & 15) == 0)
            mfma_pv<true>(acc_o[n & 15], cur, pf[n >> 4]);  // first use of this P fragment
          else
            mfma_pv<false>(acc_o[n & 15], cur, pf[n >> 4]);
          if (n < 12) {
            const int k = n / 3, r = n % 3;
            if (r == 0) pa = p_exp(st, 8 + 2 * k, neg);
            else if (r == 1) pb = p_exp(st, 9 + 2 * k, neg);
            else p_pack(8 + 2 * k, pa, pb, pf, psum);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      l_loc += psum;
    } else {
      // A page is two 32-token tiles, staggered in the source so that the
      // softmax work of one tile sits between the MFMAs of the other: QK(T0);
      // QK(T1) with tile 0's exponentials; PV(T0) with tile 1's exponentials;
      // PV(T1) (the compiler gathers each tile's exponentials just before its
      // PV). Tile 1's P uses a provisional reference taken before PV(T0); O
      // and l move to it only after PV(T0) has added tile 0 (which used the
      // old one).

      // ---- QK(T0), with half of the next page's loads.
      f32x16_t st0;
#pragma unroll
      for (int r = 0; r < 16; ++r) st0[r] = 0.f;
      {
        bf16x8_t kf[kKDepth];
#pragma unroll
        for (int s = 0; s < kKDepth; ++s) kf[s] = k_frag(0, s);
#pragma unroll
        for (int s = 0; s < kQSteps; ++s) {
          const bf16x8_t cur = kf[s % kKDepth];
          if (s + kKDepth < kQSteps) kf[s % kKDepth] = k_frag(0, s + kKDepth);
          st0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, qf[s], st0, 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
          if ((s & 3) == 0) issue_line(next, s >> 2);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // ---- QK(T1), with tile 0's max and reference move after its second
      // MFMA, tile 0's P (one exponential per k-step from the fifth, a pair
      // packed every third) and the other half of the next page's loads.
      f32x16_t st1;
#pragma unroll
      for (int r = 0; r < 16; ++r) st1[r] = 0.f;
      bf16x8_t pf0[2];
      float psum0 = 0.f;
      float neg0 = 0.f;
      {
        bf16x8_t kf[kKDepth];
#pragma unroll
        for (int s = 0; s < kKDepth; ++s) kf[s] = k_frag(1, s);
#pragma unroll
        for (int s = 0; s < kQSteps; ++s) {
          const bf16x8_t cur = kf[s % kKDepth];
          if (s + kKDepth < kQSteps) kf[s % kKDepth] = k_frag(1, s + kKDepth);
          st1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, qf[s], st1, 0, 0, 0);
          if (s == 1) {
            const float mt0 = tile_max(st0, 0);
            move_reference((mt0 > m_ref + 8.0f) ? mt0 : m_ref);
            neg0 = (m_ref == -INFINITY) ? 0.f : -m_ref;
          }
          if (s >= 4 && s < 28) {
            const int k = (s - 4) / 3, r = (s - 4) % 3;
            if (r == 0) pa = p_exp(st0, 2 * k, neg0);
            else if (r == 1) pb = p_exp(st0, 2 * k + 1, neg0);
            else p_pack(2 * k, pa, pb, pf0, psum0);
          }
          if ((s & 3) == 2) issue_line(next, 9 + (s >> 2));
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      l_loc += psum0;

      // ---- PV(T0), with tile 1's max (a provisional reference, applied to O
      // and l only after PV(T0) has added tile 0) after its second MFMA and
      // tile 1's P (one exponential per MFMA from the fifth, a pair packed
      // every third).
      bf16x8_t pf1[2];
      float psum1 = 0.f;
      float m1 = m_ref, neg1 = 0.f;
      {
        bf16x8_t vf[kPvDepth];
#pragma unroll
        for (int n = 0; n < kPvDepth; ++n) vf[n] = v_frag(n >> 4, n & 15);
#pragma unroll
        for (int n = 0; n < 2 * kColTiles; ++n) {
          const bf16x8_t cur = vf[n % kPvDepth];
          if (n + kPvDepth < 2 * kColTiles) vf[n % kPvDepth] = v_frag((n + kPvDepth) >> 4, (n + kPvDepth) & 15);
          if ((n & 15) == 0)
            mfma_pv<true>(acc_o[n & 15], cur, pf0[n >> 4]);  // first use of this P fragment
          else
            mfma_pv<false>(acc_o[n & 15], cur, pf0[n >> 4]);
          if (n == 1) {
            const float mt1 = tile_max(st1, 1);
            m1 = (mt1 > m_ref + 8.0f) ? mt1 : m_ref;
            neg1 = (m1 == -INFINITY) ? 0.f : -m1;
          }
          if (n >= 4 && n < 28) {
            const int k = (n - 4) / 3, r = (n - 4) % 3;
            if (r == 0) pa = p_exp(st1, 2 * k, neg1);
            else if (r == 1) pb = p_exp(st1, 2 * k + 1, neg1);
            else p_pack(2 * k, pa, pb, pf1, psum1);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      move_reference(m1);
      l_loc += psum1;

      // ---- PV(T1).
      {
        bf16x8_t vf[kPvDepth];
#pragma unroll
        for (int n = 0; n < kPvDepth; ++n) vf[n] = v_frag(2 + (n >> 4), n & 15);
#pragma unroll
        for (int n = 0; n < 2 * kColTiles; ++n) {
          const bf16x8_t cur = vf[n % kPvDepth];
          if (n + kPvDepth < 2 * kColTiles) vf[n % kPvDepth] = v_frag(2 + ((n + kPvDepth) >> 4), (n + kPvDepth) & 15);
          if ((n & 15) == 0)
            mfma_pv<true>(acc_o[n & 15], cur, pf1[n >> 4]);
          else
            mfma_pv<false>(acc_o[n & 15], cur, pf1[n >> 4]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }

  // The last page's reload is still landing in the idle buffer, which the
  // finalize reuses for staging.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  // ---- finalize: o = O / l, lse = ln2 * (m_ref + log2 l); l is split over
  // the two lanes of a row.
  agpr_fence();
  float l_tot = l_loc + other_half(l_loc);
  __syncthreads();  // every wave is done with the page buffers
  // The lane position is taken afresh (mbcnt) rather than kept live through
  // the page loop, where every VGPR is taken.
  const int ln = lane_id();
  const int r32f = ln & 31, hi32f = ln >> 5;
  const int rowf = rgrp * kGroupRows + slice * kWaveRows + r32f;
  if constexpr (kHalf) {
    // The two waves of a pair hold the same 32 rows with (m, l, O) over
    // complementary halves of every page. Wave t of the pair finalizes
    // columns 256t .. 256t+255: each hands the other half of its O (fp32,
    // lane-contiguous 16-byte pieces) and its m and l to its partner through
    // LDS, merges what it receives with its own half by the textbook
    // two-way rule straight into bf16 registers, then stages 512-byte half
    // rows and stores them.
    // One straight-line copy per t (acc_o is indexed with constants only: a
    // runtime index would move it to scratch); both copies pass the same
    // three barriers.
    const int pair = wave & 1;
    const auto finalize_half = [&](auto tc) {
      constexpr int t = decltype(tc)::value;
      char* const area = smem + pair * 65536;
      float* const give = reinterpret_cast<float*>(area + t * 32768);
      const float* const take = reinterpret_cast<const float*>(area + (t ^ 1) * 32768);
      float* const ml = reinterpret_cast<float*>(smem + 131072 + pair * 512);  // [2][m 32 | l 32]
#pragma unroll
      for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          f32x4_t v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc_o[(t ^ 1) * 8 + k][4 * q4 + e];  // the partner's columns
          *reinterpret_cast<f32x4_t*>(give + ((4 * k + q4) * 64 + ln) * 4) = v;
        }
      if (hi32f == 0) {
        ml[64 * t + r32f] = m_ref;
        ml[64 * t + 32 + r32f] = l_tot;
      }
      __syncthreads();
      const float m_o = ml[64 * (t ^ 1) + r32f];
      const float l_o = ml[64 * (t ^ 1) + 32 + r32f];
      const float m_new = fmaxf(m_ref, m_o);
      const float a_s = (m_ref == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_new);
      const float a_o = (m_o == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_o - m_new);
      const float l_m = l_tot * a_s + l_o * a_o;
      const bool any = l_m > 0.f;
      const float inv = any ? 1.f / l_m : 0.f;
      const float c_s = a_s * inv, c_o = a_o * inv;
      const float lse_v = any ? (m_new + __log2f(l_m)) * 0.6931471805599453f : -INFINITY;
      bf16x4_t res[32];
#pragma unroll
      for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4_t x = *reinterpret_cast<const f32x4_t*>(take + ((4 * k + q4) * 64 + ln) * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            res[4 * k + q4][e] = (__bf16)(acc_o[t * 8 + k][4 * q4 + e] * c_s + x[e] * c_o);  // this wave's columns
        }
      __syncthreads();  // both halves of every pair read; the areas are free
      // Half row r of the wave: 512 bytes at r*512 in its 16 KB staging
      // area, 16-byte piece p at (p ^ r) so a write's 32 rows spread over
      // the banks.
      char* const stage = area + t * 32768;
#pragma unroll
      for (int p = 0; p < 32; ++p)
        *reinterpret_cast<bf16x4_t*>(stage + r32f * 512 + ((p ^ r32f) * 16) + 8 * hi32f) = res[p];
      __syncthreads();
      __bf16* const out = direct ? static_cast<__bf16*>(a.o_lat) + (size_t)b * rows * kDv
                                 : static_cast<__bf16*>(a.o_part) + (size_t)part * rows * kDv;
      const int row0 = rgrp * kGroupRows + slice * kWaveRows;
#pragma unroll 4
      for (int r = 0; r < kWaveRows; r += 2) {
        const int rr = r + hi32f;  // two half rows per store instruction
        if (row0 + rr < rows) {
          const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stage + rr * 512 + (((ln & 31) ^ rr) * 16));
          if (direct)
            __builtin_nontemporal_store(
                v, reinterpret_cast<u32x4_t*>(out + (size_t)(row0 + rr) * kDv + 256 * t + 8 * (ln & 31)));
          else
            store_device_scope(out + (size_t)row0 * kDv + 256 * t, 2 * (rr * kDv + 8 * (ln & 31)), v);
        }
      }
      if (t == 0 && hi32f == 0 && rowf < rows) {
        if (direct)
          a.lse[(size_t)b * rows + rowf] = lse_v;
        else
          store_device_scope(a.lse_part + (size_t)part * rows, 4 * rowf, lse_v);
      }
    };
    if (wave < 2)
      finalize_half(std::integral_constant<int, 0>{});
    else
      finalize_half(std::integral_constant<int, 1>{});
    return;
  }
  const bool any = l_tot > 0.f;
  const float inv = any ? 1.f / l_tot : 0.f;
  const float lse_v = any ? (m_ref + __log2f(l_tot)) * 0.6931471805599453f : -INFINITY;

  // The rows go out through LDS. acc_o[i][r] is O^T[32i + 8(r>>2) + 4*hi32 +
  // (r&3)][row], so a lane holds 8-byte pieces of its row and a direct store
  // would touch 32 rows per instruction, 16 bytes each: partial 128-byte lines
  // that stay dirty in L2 until the end of the kernel and then cost
  // microseconds to write back. Staged, every store instruction writes one
  // whole 1 KB row. A sequence's final rows are stored non-temporally (the
  // next reader is another kernel's, much later); chunk partials and their
  // LSE values are stored at device scope, written through L2 to the memory
  // side where the merge kernel, on any XCD, reads them right after this one,
  // and none of them is left dirty for the end-of-launch write-back
  // (measured on MI355X: the step is 1.5-2.5 us shorter than with
  // non-temporal partial stores, and about 1 us shorter again than with
  // plain cacheable ones). Row r of a wave's 32 KB staging area
  // keeps its 64 16-byte pieces XOR-permuted by r so that the 32 rows of a
  // write do not fall on the same LDS banks.
  char* stage = smem + wave * (kWaveRows * kDv * 2);
#pragma unroll
  for (int i = 0; i < kColTiles; ++i)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      bf16x4_t v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (__bf16)(acc_o[i][4 * q4 + e] * inv);
      const int piece = (4 * i + q4) ^ r32f;  // 16-byte piece of the row, permuted
      *reinterpret_cast<bf16x4_t*>(stage + r32f * (kDv * 2) + piece * 16 + 8 * hi32f) = v;
    }
  __syncthreads();

  __bf16* const out = direct ? static_cast<__bf16*>(a.o_lat) + (size_t)b * rows * kDv
                             : static_cast<__bf16*>(a.o_part) + (size_t)part * rows * kDv;
  const int row0 = rgrp * kGroupRows + slice * kWaveRows;
#pragma unroll 4
  for (int r = 0; r < kWaveRows; ++r) {
    if (row0 + r >= rows) break;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stage + r * (kDv * 2) + ((ln ^ r) * 16));
    if (direct)
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(out + (size_t)(row0 + r) * kDv + 8 * ln));
    else
      store_device_scope(out + (size_t)(row0 + r) * kDv, 16 * ln, v);
  }
  if (hi32f == 0 && rowf < rows) {
    if (direct)
      a.lse[(size_t)b * rows + rowf] = lse_v;
    else
      store_device_scope(a.lse_part + (size_t)part * rows, 4 * rowf, lse_v);
  }
}

// One schedule entry's four words (b, first page, end page, L_b), read by
// four lanes side by side and broadcast.
__device__ __forceinline__ void load_chunk_desc(const int32_t* desc, int c, int& b, int& p0, int& p1, int& L) {
  const int lane = lane_id();
  const int v = lane < 4 ? desc[4 * (size_t)c + lane] : 0;
  b = __builtin_amdgcn_readlane(v, 0);
  p0 = __builtin_amdgcn_readlane(v, 1);
  p1 = __builtin_amdgcn_readlane(v, 2);
  L = __builtin_amdgcn_readlane(v, 3);
}

// Measurement aid (mla_decode_clock_probe): while `buf` is set, workgroup x
// < cap writes its shader-clock cycles and 100 MHz reference ticks from its
// start to its end at buf[2x], buf[2x+1]. One copy per device. The start
// stamps go to the buffer (nothing is held in registers through the kernel,
// where every register is taken) and the end turns them into differences.
struct ClockProbe {
  uint64_t* buf;
  int cap;
};
__device__ ClockProbe g_clock_probe = {nullptr, 0};

__device__ __forceinline__ void clock_begin() {
  const ClockProbe p = g_clock_probe;
  if (p.buf != nullptr && threadIdx.x == 0 && (int)blockIdx.x < p.cap) {
    p.buf[2 * (size_t)blockIdx.x] = __builtin_amdgcn_s_memtime();
    p.buf[2 * (size_t)blockIdx.x + 1] = __builtin_amdgcn_s_memrealtime();
  }
}
__device__ __forceinline__ void clock_end() {
  const ClockProbe p = g_clock_probe;
  if (p.buf != nullptr && threadIdx.x == 0 && (int)blockIdx.x < p.cap) {
    const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    uint64_t* const w = p.buf + 2 * (size_t)blockIdx.x;
    w[0] = t1 - __builtin_nontemporal_load(w);
    w[1] = r1 - __builtin_nontemporal_load(w + 1);
  }
}

template <bool kSparse, bool kHalf>
__global__ __launch_bounds__(kThreads, 1) void mla_decode_bf16_kernel(DecodeArgs a, int row_groups, int n_units) {
  constexpr int kSparseBytes = kSparse ? kSparseMaxTopk * 4 + (kSparseMaxTopk / kPage) * 8 : 0;
  __shared__ __attribute__((aligned(1024))) char smem[2 * kPageBytes + (kSparse ? kSparseBytes : kQStageExtra)];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: keep it in an SGPR

  // XCD-aware mapping: workgroups x and x+8j run on the same XCD (its own
  // L2). Each XCD takes a contiguous range of work units (chunks, or the
  // schedule's segments), so the chunks of one sequence (which load the same
  // Q rows) and the row groups of one unit (which read the same pages) share
  // an L2.
  const int x = blockIdx.x;
  const int xcd = x & 7;
  const int rest = x >> 3;
  const int rgrp = rest % row_groups;
  const int per_xcd = (n_units + 7) / 8;
  const int g = xcd * per_xcd + rest / row_groups;
  if (rest / row_groups >= per_xcd || g >= n_units) return;
  clock_begin();

  if (a.schedule != nullptr) {
    // Balanced schedule: unit g is segment g; its chunks are consecutive
    // entries, each a page range of one sequence with its own partial.
    const int32_t* desc = a.schedule + a.num_segments + 1;
    int c0 = g, c1 = g + 1;
    if (a.num_segments != a.total_splits) {  // some segment holds several chunks
      const int lane = lane_id();
      const int v = lane < 2 ? a.schedule[g + lane] : 0;
      c0 = min(max(__builtin_amdgcn_readlane(v, 0), 0), a.total_splits);
      c1 = min(max(__builtin_amdgcn_readlane(v, 1), c0), a.total_splits);
    }
    for (int c = c0; c < c1; ++c) {
      int b, p0, p1, Ld;
      load_chunk_desc(desc, c, b, p0, p1, Ld);
      b = min(max(b, 0), a.B - 1);
      const int L = max(a.s_q, min(Ld, a.max_pages * kPage));
      const int P = (L + kPage - 1) / kPage;
      p1 = min(max(p1, 0), P);
      p0 = min(max(p0, 0), p1);
      const bool direct = p0 == 0 && p1 == P && a.o_lat != nullptr;
      decode_chunk<false, kHalf>(a, smem, b, L, p0, p1, c, direct, rgrp, wave);
      __syncthreads();  // the staging area is the next chunk's first page buffer
    }
    clock_end();
    return;
  }

  const WorkItem wi = find_work(a.split_offsets, a.seqlens, a.B, g, lane_id());
  // Top-k: the chunks split the list (topk entries); positions must be < L.
  const int L = max(kSparse ? 1 : a.s_q, min(wi.L, a.max_pages * kPage));
  const int P = ((kSparse ? a.topk : L) + kPage - 1) / kPage;
  const int n_chunks = min(max(wi.n, 1), kMaxSplits);
  const int kk = min(max(wi.k, 0), n_chunks - 1);
  // kk * P < 64 * 2^25: exact in 32-bit unsigned arithmetic.
  const int pg0 = (int)((unsigned)kk * (unsigned)P / (unsigned)n_chunks);
  const int pg1 = (int)((unsigned)(kk + 1) * (unsigned)P / (unsigned)n_chunks);
  decode_chunk<kSparse, kHalf>(a, smem, wi.b, L, pg0, pg1, g, n_chunks == 1 && a.o_lat != nullptr, rgrp, wave);
  clock_end();
}

template <bool kSparse, bool kHalf>
hipError_t launch(const DecodeArgs& a, hipStream_t stream) {
  const int rows = a.s_q * a.H;
  const int group_rows = kHalf ? kRowsPerGroup / 2 : kRowsPerGroup;
  const int row_groups = (rows + group_rows - 1) / group_rows;
  const int units = a.schedule != nullptr ? a.num_segments : a.total_splits;
  const int padded = (units + 7) / 8 * 8;
  const dim3 grid((unsigned)(padded * row_groups));
  hipLaunchKernelGGL((mla_decode_bf16_kernel<kSparse, kHalf>), grid, dim3(kThreads), 0, stream, a, row_groups, units);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream) {
  if (a.schedule != nullptr && a.rows_per_group == kRowsPerGroup / 2) return launch<false, true>(a, stream);
  return launch<false, false>(a, stream);
}
hipError_t launch_sparse_decode_bf16(const DecodeArgs& a, hipStream_t stream) { return launch<true, false>(a, stream); }

hipError_t set_clock_probe(uint64_t* buf, int cap) {
  const ClockProbe p = {buf, buf != nullptr ? cap : 0};
  return hipMemcpyToSymbol(HIP_SYMBOL(g_clock_probe), &p, sizeof(p));
}

}  // namespace mla

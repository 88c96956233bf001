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
//     V^T reads use the same permutation). The two tiles are staggered so
//     that each tile's exponentials run between the MFMAs of the other
//     tile's product (MFMA and VALU work of one wave execute together).
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

#include "mla_internal.h"

namespace mla {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kWaveRows = 32;                      // rows per wave
static_assert(kWaveRows * kWaves == kRowsPerGroup, "a workgroup covers one row group");
constexpr int kRowBytes = kDqk * 2;                // 1152: one cache row
constexpr int kPageBytes = kPage * kRowBytes;      // 73728: one page
constexpr int kBlocks = kPageBytes / 1024;         // 72 line blocks
constexpr int kBlocksPerWave = kBlocks / kWaves;   // 18: two token octets per wave
constexpr int kQSteps = kDqk / 16;                 // 36 k-steps of 16
constexpr int kColTiles = kDv / 32;                // 16 column tiles of 32
static_assert(kBlocksPerWave == 18, "each wave loads two token octets");
// s_waitcnt immediate for gfx9: vmcnt = 0, expcnt and lgkmcnt left at "no wait".
constexpr int kWaitVmcnt0 = (0xF << 8) | (0x7 << 4);

__device__ __forceinline__ int swz(int t) {
  const int u = (t >> 1) & 7;
  return ((u & 1) << 2) | (u >> 1);
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
  dma_line(p.sbase, (octet ? p.off1 : p.off0) + 128 * j, p.lds + 1024 * (9 * octet + j));
}

__device__ __forceinline__ void issue_page(const PageLoad& p) {
#pragma unroll
  for (int n = 0; n < kBlocksPerWave; ++n) issue_line(p, n);
}

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
      "global_load_lds_dwordx4 %0, off"
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

// Value of lane l ^ 32 (gfx950 lane swap; VALU, no LDS round trip). With
// both operands equal, permlane32_swap yields the values of lanes l and l^32.
__device__ __forceinline__ float other_half(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// O^T += V^T P^T for one 32x32 column tile, accumulator pinned to AGPRs: the
// 16 tiles of a wave fill the AGPR file exactly, and the compiler left to
// itself places some of them in VGPRs and spills Q. The compiler's hazard
// tracking does not see into this asm, so the caller asks for wait states
// (kFresh) where B was just written by VALU instructions, and any VALU
// access to the accumulators goes through agpr_fence() first.
template <bool kFresh>
__device__ __forceinline__ void mfma_pv(f32x16_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  if constexpr (kFresh)
    asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// Wait states between the last accumulating MFMA (8 passes) and a VALU
// read of its AGPRs; the hazard tracker does not see into the asm above.
__device__ __forceinline__ void agpr_fence() {
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");
}

// O *= alpha for the whole accumulator: every AGPR of a lane belongs to the
// lane's one query row (the column of its O^T tiles), and O occupies the
// AGPR file alone, so all 256 AGPRs are scaled in place. Done in asm so that
// no VALU use of the accumulators is visible to the register allocator
// (which would otherwise stage all of O through VGPRs and spill). Trailing
// wait states cover the AGPR write -> MFMA srcC hazard.
__device__ __forceinline__ void scale_accumulators(float alpha) {
  float t0, t1, t2, t3;
  asm volatile(
      "v_accvgpr_read_b32 %0, a0\n\t"
      "v_accvgpr_read_b32 %1, a1\n\t"
      "v_accvgpr_read_b32 %2, a2\n\t"
      "v_accvgpr_read_b32 %3, a3\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a0, %0\n\t"
      "v_accvgpr_write_b32 a1, %1\n\t"
      "v_accvgpr_write_b32 a2, %2\n\t"
      "v_accvgpr_write_b32 a3, %3\n\t"
      "v_accvgpr_read_b32 %0, a4\n\t"
      "v_accvgpr_read_b32 %1, a5\n\t"
      "v_accvgpr_read_b32 %2, a6\n\t"
      "v_accvgpr_read_b32 %3, a7\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a4, %0\n\t"
      "v_accvgpr_write_b32 a5, %1\n\t"
      "v_accvgpr_write_b32 a6, %2\n\t"
      "v_accvgpr_write_b32 a7, %3\n\t"
      "v_accvgpr_read_b32 %0, a8\n\t"
      "v_accvgpr_read_b32 %1, a9\n\t"
      "v_accvgpr_read_b32 %2, a10\n\t"
      "v_accvgpr_read_b32 %3, a11\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a8, %0\n\t"
      "v_accvgpr_write_b32 a9, %1\n\t"
      "v_accvgpr_write_b32 a10, %2\n\t"
      "v_accvgpr_write_b32 a11, %3\n\t"
      "v_accvgpr_read_b32 %0, a12\n\t"
      "v_accvgpr_read_b32 %1, a13\n\t"
      "v_accvgpr_read_b32 %2, a14\n\t"
      "v_accvgpr_read_b32 %3, a15\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a12, %0\n\t"
      "v_accvgpr_write_b32 a13, %1\n\t"
      "v_accvgpr_write_b32 a14, %2\n\t"
      "v_accvgpr_write_b32 a15, %3\n\t"
      "v_accvgpr_read_b32 %0, a16\n\t"
      "v_accvgpr_read_b32 %1, a17\n\t"
      "v_accvgpr_read_b32 %2, a18\n\t"
      "v_accvgpr_read_b32 %3, a19\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a16, %0\n\t"
      "v_accvgpr_write_b32 a17, %1\n\t"
      "v_accvgpr_write_b32 a18, %2\n\t"
      "v_accvgpr_write_b32 a19, %3\n\t"
      "v_accvgpr_read_b32 %0, a20\n\t"
      "v_accvgpr_read_b32 %1, a21\n\t"
      "v_accvgpr_read_b32 %2, a22\n\t"
      "v_accvgpr_read_b32 %3, a23\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a20, %0\n\t"
      "v_accvgpr_write_b32 a21, %1\n\t"
      "v_accvgpr_write_b32 a22, %2\n\t"
      "v_accvgpr_write_b32 a23, %3\n\t"
      "v_accvgpr_read_b32 %0, a24\n\t"
      "v_accvgpr_read_b32 %1, a25\n\t"
      "v_accvgpr_read_b32 %2, a26\n\t"
      "v_accvgpr_read_b32 %3, a27\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a24, %0\n\t"
      "v_accvgpr_write_b32 a25, %1\n\t"
      "v_accvgpr_write_b32 a26, %2\n\t"
      "v_accvgpr_write_b32 a27, %3\n\t"
      "v_accvgpr_read_b32 %0, a28\n\t"
      "v_accvgpr_read_b32 %1, a29\n\t"
      "v_accvgpr_read_b32 %2, a30\n\t"
      "v_accvgpr_read_b32 %3, a31\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a28, %0\n\t"
      "v_accvgpr_write_b32 a29, %1\n\t"
      "v_accvgpr_write_b32 a30, %2\n\t"
      "v_accvgpr_write_b32 a31, %3\n\t"
      "v_accvgpr_read_b32 %0, a32\n\t"
      "v_accvgpr_read_b32 %1, a33\n\t"
      "v_accvgpr_read_b32 %2, a34\n\t"
      "v_accvgpr_read_b32 %3, a35\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a32, %0\n\t"
      "v_accvgpr_write_b32 a33, %1\n\t"
      "v_accvgpr_write_b32 a34, %2\n\t"
      "v_accvgpr_write_b32 a35, %3\n\t"
      "v_accvgpr_read_b32 %0, a36\n\t"
      "v_accvgpr_read_b32 %1, a37\n\t"
      "v_accvgpr_read_b32 %2, a38\n\t"
      "v_accvgpr_read_b32 %3, a39\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a36, %0\n\t"
      "v_accvgpr_write_b32 a37, %1\n\t"
      "v_accvgpr_write_b32 a38, %2\n\t"
      "v_accvgpr_write_b32 a39, %3\n\t"
      "v_accvgpr_read_b32 %0, a40\n\t"
      "v_accvgpr_read_b32 %1, a41\n\t"
      "v_accvgpr_read_b32 %2, a42\n\t"
      "v_accvgpr_read_b32 %3, a43\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a40, %0\n\t"
      "v_accvgpr_write_b32 a41, %1\n\t"
      "v_accvgpr_write_b32 a42, %2\n\t"
      "v_accvgpr_write_b32 a43, %3\n\t"
      "v_accvgpr_read_b32 %0, a44\n\t"
      "v_accvgpr_read_b32 %1, a45\n\t"
      "v_accvgpr_read_b32 %2, a46\n\t"
      "v_accvgpr_read_b32 %3, a47\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a44, %0\n\t"
      "v_accvgpr_write_b32 a45, %1\n\t"
      "v_accvgpr_write_b32 a46, %2\n\t"
      "v_accvgpr_write_b32 a47, %3\n\t"
      "v_accvgpr_read_b32 %0, a48\n\t"
      "v_accvgpr_read_b32 %1, a49\n\t"
      "v_accvgpr_read_b32 %2, a50\n\t"
      "v_accvgpr_read_b32 %3, a51\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a48, %0\n\t"
      "v_accvgpr_write_b32 a49, %1\n\t"
      "v_accvgpr_write_b32 a50, %2\n\t"
      "v_accvgpr_write_b32 a51, %3\n\t"
      "v_accvgpr_read_b32 %0, a52\n\t"
      "v_accvgpr_read_b32 %1, a53\n\t"
      "v_accvgpr_read_b32 %2, a54\n\t"
      "v_accvgpr_read_b32 %3, a55\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a52, %0\n\t"
      "v_accvgpr_write_b32 a53, %1\n\t"
      "v_accvgpr_write_b32 a54, %2\n\t"
      "v_accvgpr_write_b32 a55, %3\n\t"
      "v_accvgpr_read_b32 %0, a56\n\t"
      "v_accvgpr_read_b32 %1, a57\n\t"
      "v_accvgpr_read_b32 %2, a58\n\t"
      "v_accvgpr_read_b32 %3, a59\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a56, %0\n\t"
      "v_accvgpr_write_b32 a57, %1\n\t"
      "v_accvgpr_write_b32 a58, %2\n\t"
      "v_accvgpr_write_b32 a59, %3\n\t"
      "v_accvgpr_read_b32 %0, a60\n\t"
      "v_accvgpr_read_b32 %1, a61\n\t"
      "v_accvgpr_read_b32 %2, a62\n\t"
      "v_accvgpr_read_b32 %3, a63\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a60, %0\n\t"
      "v_accvgpr_write_b32 a61, %1\n\t"
      "v_accvgpr_write_b32 a62, %2\n\t"
      "v_accvgpr_write_b32 a63, %3\n\t"
      "v_accvgpr_read_b32 %0, a64\n\t"
      "v_accvgpr_read_b32 %1, a65\n\t"
      "v_accvgpr_read_b32 %2, a66\n\t"
      "v_accvgpr_read_b32 %3, a67\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a64, %0\n\t"
      "v_accvgpr_write_b32 a65, %1\n\t"
      "v_accvgpr_write_b32 a66, %2\n\t"
      "v_accvgpr_write_b32 a67, %3\n\t"
      "v_accvgpr_read_b32 %0, a68\n\t"
      "v_accvgpr_read_b32 %1, a69\n\t"
      "v_accvgpr_read_b32 %2, a70\n\t"
      "v_accvgpr_read_b32 %3, a71\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a68, %0\n\t"
      "v_accvgpr_write_b32 a69, %1\n\t"
      "v_accvgpr_write_b32 a70, %2\n\t"
      "v_accvgpr_write_b32 a71, %3\n\t"
      "v_accvgpr_read_b32 %0, a72\n\t"
      "v_accvgpr_read_b32 %1, a73\n\t"
      "v_accvgpr_read_b32 %2, a74\n\t"
      "v_accvgpr_read_b32 %3, a75\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a72, %0\n\t"
      "v_accvgpr_write_b32 a73, %1\n\t"
      "v_accvgpr_write_b32 a74, %2\n\t"
      "v_accvgpr_write_b32 a75, %3\n\t"
      "v_accvgpr_read_b32 %0, a76\n\t"
      "v_accvgpr_read_b32 %1, a77\n\t"
      "v_accvgpr_read_b32 %2, a78\n\t"
      "v_accvgpr_read_b32 %3, a79\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a76, %0\n\t"
      "v_accvgpr_write_b32 a77, %1\n\t"
      "v_accvgpr_write_b32 a78, %2\n\t"
      "v_accvgpr_write_b32 a79, %3\n\t"
      "v_accvgpr_read_b32 %0, a80\n\t"
      "v_accvgpr_read_b32 %1, a81\n\t"
      "v_accvgpr_read_b32 %2, a82\n\t"
      "v_accvgpr_read_b32 %3, a83\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a80, %0\n\t"
      "v_accvgpr_write_b32 a81, %1\n\t"
      "v_accvgpr_write_b32 a82, %2\n\t"
      "v_accvgpr_write_b32 a83, %3\n\t"
      "v_accvgpr_read_b32 %0, a84\n\t"
      "v_accvgpr_read_b32 %1, a85\n\t"
      "v_accvgpr_read_b32 %2, a86\n\t"
      "v_accvgpr_read_b32 %3, a87\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a84, %0\n\t"
      "v_accvgpr_write_b32 a85, %1\n\t"
      "v_accvgpr_write_b32 a86, %2\n\t"
      "v_accvgpr_write_b32 a87, %3\n\t"
      "v_accvgpr_read_b32 %0, a88\n\t"
      "v_accvgpr_read_b32 %1, a89\n\t"
      "v_accvgpr_read_b32 %2, a90\n\t"
      "v_accvgpr_read_b32 %3, a91\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a88, %0\n\t"
      "v_accvgpr_write_b32 a89, %1\n\t"
      "v_accvgpr_write_b32 a90, %2\n\t"
      "v_accvgpr_write_b32 a91, %3\n\t"
      "v_accvgpr_read_b32 %0, a92\n\t"
      "v_accvgpr_read_b32 %1, a93\n\t"
      "v_accvgpr_read_b32 %2, a94\n\t"
      "v_accvgpr_read_b32 %3, a95\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a92, %0\n\t"
      "v_accvgpr_write_b32 a93, %1\n\t"
      "v_accvgpr_write_b32 a94, %2\n\t"
      "v_accvgpr_write_b32 a95, %3\n\t"
      "v_accvgpr_read_b32 %0, a96\n\t"
      "v_accvgpr_read_b32 %1, a97\n\t"
      "v_accvgpr_read_b32 %2, a98\n\t"
      "v_accvgpr_read_b32 %3, a99\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a96, %0\n\t"
      "v_accvgpr_write_b32 a97, %1\n\t"
      "v_accvgpr_write_b32 a98, %2\n\t"
      "v_accvgpr_write_b32 a99, %3\n\t"
      "v_accvgpr_read_b32 %0, a100\n\t"
      "v_accvgpr_read_b32 %1, a101\n\t"
      "v_accvgpr_read_b32 %2, a102\n\t"
      "v_accvgpr_read_b32 %3, a103\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a100, %0\n\t"
      "v_accvgpr_write_b32 a101, %1\n\t"
      "v_accvgpr_write_b32 a102, %2\n\t"
      "v_accvgpr_write_b32 a103, %3\n\t"
      "v_accvgpr_read_b32 %0, a104\n\t"
      "v_accvgpr_read_b32 %1, a105\n\t"
      "v_accvgpr_read_b32 %2, a106\n\t"
      "v_accvgpr_read_b32 %3, a107\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a104, %0\n\t"
      "v_accvgpr_write_b32 a105, %1\n\t"
      "v_accvgpr_write_b32 a106, %2\n\t"
      "v_accvgpr_write_b32 a107, %3\n\t"
      "v_accvgpr_read_b32 %0, a108\n\t"
      "v_accvgpr_read_b32 %1, a109\n\t"
      "v_accvgpr_read_b32 %2, a110\n\t"
      "v_accvgpr_read_b32 %3, a111\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a108, %0\n\t"
      "v_accvgpr_write_b32 a109, %1\n\t"
      "v_accvgpr_write_b32 a110, %2\n\t"
      "v_accvgpr_write_b32 a111, %3\n\t"
      "v_accvgpr_read_b32 %0, a112\n\t"
      "v_accvgpr_read_b32 %1, a113\n\t"
      "v_accvgpr_read_b32 %2, a114\n\t"
      "v_accvgpr_read_b32 %3, a115\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a112, %0\n\t"
      "v_accvgpr_write_b32 a113, %1\n\t"
      "v_accvgpr_write_b32 a114, %2\n\t"
      "v_accvgpr_write_b32 a115, %3\n\t"
      "v_accvgpr_read_b32 %0, a116\n\t"
      "v_accvgpr_read_b32 %1, a117\n\t"
      "v_accvgpr_read_b32 %2, a118\n\t"
      "v_accvgpr_read_b32 %3, a119\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a116, %0\n\t"
      "v_accvgpr_write_b32 a117, %1\n\t"
      "v_accvgpr_write_b32 a118, %2\n\t"
      "v_accvgpr_write_b32 a119, %3\n\t"
      "v_accvgpr_read_b32 %0, a120\n\t"
      "v_accvgpr_read_b32 %1, a121\n\t"
      "v_accvgpr_read_b32 %2, a122\n\t"
      "v_accvgpr_read_b32 %3, a123\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a120, %0\n\t"
      "v_accvgpr_write_b32 a121, %1\n\t"
      "v_accvgpr_write_b32 a122, %2\n\t"
      "v_accvgpr_write_b32 a123, %3\n\t"
      "v_accvgpr_read_b32 %0, a124\n\t"
      "v_accvgpr_read_b32 %1, a125\n\t"
      "v_accvgpr_read_b32 %2, a126\n\t"
      "v_accvgpr_read_b32 %3, a127\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a124, %0\n\t"
      "v_accvgpr_write_b32 a125, %1\n\t"
      "v_accvgpr_write_b32 a126, %2\n\t"
      "v_accvgpr_write_b32 a127, %3\n\t"
      "v_accvgpr_read_b32 %0, a128\n\t"
      "v_accvgpr_read_b32 %1, a129\n\t"
      "v_accvgpr_read_b32 %2, a130\n\t"
      "v_accvgpr_read_b32 %3, a131\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a128, %0\n\t"
      "v_accvgpr_write_b32 a129, %1\n\t"
      "v_accvgpr_write_b32 a130, %2\n\t"
      "v_accvgpr_write_b32 a131, %3\n\t"
      "v_accvgpr_read_b32 %0, a132\n\t"
      "v_accvgpr_read_b32 %1, a133\n\t"
      "v_accvgpr_read_b32 %2, a134\n\t"
      "v_accvgpr_read_b32 %3, a135\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a132, %0\n\t"
      "v_accvgpr_write_b32 a133, %1\n\t"
      "v_accvgpr_write_b32 a134, %2\n\t"
      "v_accvgpr_write_b32 a135, %3\n\t"
      "v_accvgpr_read_b32 %0, a136\n\t"
      "v_accvgpr_read_b32 %1, a137\n\t"
      "v_accvgpr_read_b32 %2, a138\n\t"
      "v_accvgpr_read_b32 %3, a139\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a136, %0\n\t"
      "v_accvgpr_write_b32 a137, %1\n\t"
      "v_accvgpr_write_b32 a138, %2\n\t"
      "v_accvgpr_write_b32 a139, %3\n\t"
      "v_accvgpr_read_b32 %0, a140\n\t"
      "v_accvgpr_read_b32 %1, a141\n\t"
      "v_accvgpr_read_b32 %2, a142\n\t"
      "v_accvgpr_read_b32 %3, a143\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a140, %0\n\t"
      "v_accvgpr_write_b32 a141, %1\n\t"
      "v_accvgpr_write_b32 a142, %2\n\t"
      "v_accvgpr_write_b32 a143, %3\n\t"
      "v_accvgpr_read_b32 %0, a144\n\t"
      "v_accvgpr_read_b32 %1, a145\n\t"
      "v_accvgpr_read_b32 %2, a146\n\t"
      "v_accvgpr_read_b32 %3, a147\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a144, %0\n\t"
      "v_accvgpr_write_b32 a145, %1\n\t"
      "v_accvgpr_write_b32 a146, %2\n\t"
      "v_accvgpr_write_b32 a147, %3\n\t"
      "v_accvgpr_read_b32 %0, a148\n\t"
      "v_accvgpr_read_b32 %1, a149\n\t"
      "v_accvgpr_read_b32 %2, a150\n\t"
      "v_accvgpr_read_b32 %3, a151\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a148, %0\n\t"
      "v_accvgpr_write_b32 a149, %1\n\t"
      "v_accvgpr_write_b32 a150, %2\n\t"
      "v_accvgpr_write_b32 a151, %3\n\t"
      "v_accvgpr_read_b32 %0, a152\n\t"
      "v_accvgpr_read_b32 %1, a153\n\t"
      "v_accvgpr_read_b32 %2, a154\n\t"
      "v_accvgpr_read_b32 %3, a155\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a152, %0\n\t"
      "v_accvgpr_write_b32 a153, %1\n\t"
      "v_accvgpr_write_b32 a154, %2\n\t"
      "v_accvgpr_write_b32 a155, %3\n\t"
      "v_accvgpr_read_b32 %0, a156\n\t"
      "v_accvgpr_read_b32 %1, a157\n\t"
      "v_accvgpr_read_b32 %2, a158\n\t"
      "v_accvgpr_read_b32 %3, a159\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a156, %0\n\t"
      "v_accvgpr_write_b32 a157, %1\n\t"
      "v_accvgpr_write_b32 a158, %2\n\t"
      "v_accvgpr_write_b32 a159, %3\n\t"
      "v_accvgpr_read_b32 %0, a160\n\t"
      "v_accvgpr_read_b32 %1, a161\n\t"
      "v_accvgpr_read_b32 %2, a162\n\t"
      "v_accvgpr_read_b32 %3, a163\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a160, %0\n\t"
      "v_accvgpr_write_b32 a161, %1\n\t"
      "v_accvgpr_write_b32 a162, %2\n\t"
      "v_accvgpr_write_b32 a163, %3\n\t"
      "v_accvgpr_read_b32 %0, a164\n\t"
      "v_accvgpr_read_b32 %1, a165\n\t"
      "v_accvgpr_read_b32 %2, a166\n\t"
      "v_accvgpr_read_b32 %3, a167\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a164, %0\n\t"
      "v_accvgpr_write_b32 a165, %1\n\t"
      "v_accvgpr_write_b32 a166, %2\n\t"
      "v_accvgpr_write_b32 a167, %3\n\t"
      "v_accvgpr_read_b32 %0, a168\n\t"
      "v_accvgpr_read_b32 %1, a169\n\t"
      "v_accvgpr_read_b32 %2, a170\n\t"
      "v_accvgpr_read_b32 %3, a171\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a168, %0\n\t"
      "v_accvgpr_write_b32 a169, %1\n\t"
      "v_accvgpr_write_b32 a170, %2\n\t"
      "v_accvgpr_write_b32 a171, %3\n\t"
      "v_accvgpr_read_b32 %0, a172\n\t"
      "v_accvgpr_read_b32 %1, a173\n\t"
      "v_accvgpr_read_b32 %2, a174\n\t"
      "v_accvgpr_read_b32 %3, a175\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a172, %0\n\t"
      "v_accvgpr_write_b32 a173, %1\n\t"
      "v_accvgpr_write_b32 a174, %2\n\t"
      "v_accvgpr_write_b32 a175, %3\n\t"
      "v_accvgpr_read_b32 %0, a176\n\t"
      "v_accvgpr_read_b32 %1, a177\n\t"
      "v_accvgpr_read_b32 %2, a178\n\t"
      "v_accvgpr_read_b32 %3, a179\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a176, %0\n\t"
      "v_accvgpr_write_b32 a177, %1\n\t"
      "v_accvgpr_write_b32 a178, %2\n\t"
      "v_accvgpr_write_b32 a179, %3\n\t"
      "v_accvgpr_read_b32 %0, a180\n\t"
      "v_accvgpr_read_b32 %1, a181\n\t"
      "v_accvgpr_read_b32 %2, a182\n\t"
      "v_accvgpr_read_b32 %3, a183\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a180, %0\n\t"
      "v_accvgpr_write_b32 a181, %1\n\t"
      "v_accvgpr_write_b32 a182, %2\n\t"
      "v_accvgpr_write_b32 a183, %3\n\t"
      "v_accvgpr_read_b32 %0, a184\n\t"
      "v_accvgpr_read_b32 %1, a185\n\t"
      "v_accvgpr_read_b32 %2, a186\n\t"
      "v_accvgpr_read_b32 %3, a187\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a184, %0\n\t"
      "v_accvgpr_write_b32 a185, %1\n\t"
      "v_accvgpr_write_b32 a186, %2\n\t"
      "v_accvgpr_write_b32 a187, %3\n\t"
      "v_accvgpr_read_b32 %0, a188\n\t"
      "v_accvgpr_read_b32 %1, a189\n\t"
      "v_accvgpr_read_b32 %2, a190\n\t"
      "v_accvgpr_read_b32 %3, a191\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a188, %0\n\t"
      "v_accvgpr_write_b32 a189, %1\n\t"
      "v_accvgpr_write_b32 a190, %2\n\t"
      "v_accvgpr_write_b32 a191, %3\n\t"
      "v_accvgpr_read_b32 %0, a192\n\t"
      "v_accvgpr_read_b32 %1, a193\n\t"
      "v_accvgpr_read_b32 %2, a194\n\t"
      "v_accvgpr_read_b32 %3, a195\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a192, %0\n\t"
      "v_accvgpr_write_b32 a193, %1\n\t"
      "v_accvgpr_write_b32 a194, %2\n\t"
      "v_accvgpr_write_b32 a195, %3\n\t"
      "v_accvgpr_read_b32 %0, a196\n\t"
      "v_accvgpr_read_b32 %1, a197\n\t"
      "v_accvgpr_read_b32 %2, a198\n\t"
      "v_accvgpr_read_b32 %3, a199\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a196, %0\n\t"
      "v_accvgpr_write_b32 a197, %1\n\t"
      "v_accvgpr_write_b32 a198, %2\n\t"
      "v_accvgpr_write_b32 a199, %3\n\t"
      "v_accvgpr_read_b32 %0, a200\n\t"
      "v_accvgpr_read_b32 %1, a201\n\t"
      "v_accvgpr_read_b32 %2, a202\n\t"
      "v_accvgpr_read_b32 %3, a203\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a200, %0\n\t"
      "v_accvgpr_write_b32 a201, %1\n\t"
      "v_accvgpr_write_b32 a202, %2\n\t"
      "v_accvgpr_write_b32 a203, %3\n\t"
      "v_accvgpr_read_b32 %0, a204\n\t"
      "v_accvgpr_read_b32 %1, a205\n\t"
      "v_accvgpr_read_b32 %2, a206\n\t"
      "v_accvgpr_read_b32 %3, a207\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a204, %0\n\t"
      "v_accvgpr_write_b32 a205, %1\n\t"
      "v_accvgpr_write_b32 a206, %2\n\t"
      "v_accvgpr_write_b32 a207, %3\n\t"
      "v_accvgpr_read_b32 %0, a208\n\t"
      "v_accvgpr_read_b32 %1, a209\n\t"
      "v_accvgpr_read_b32 %2, a210\n\t"
      "v_accvgpr_read_b32 %3, a211\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a208, %0\n\t"
      "v_accvgpr_write_b32 a209, %1\n\t"
      "v_accvgpr_write_b32 a210, %2\n\t"
      "v_accvgpr_write_b32 a211, %3\n\t"
      "v_accvgpr_read_b32 %0, a212\n\t"
      "v_accvgpr_read_b32 %1, a213\n\t"
      "v_accvgpr_read_b32 %2, a214\n\t"
      "v_accvgpr_read_b32 %3, a215\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a212, %0\n\t"
      "v_accvgpr_write_b32 a213, %1\n\t"
      "v_accvgpr_write_b32 a214, %2\n\t"
      "v_accvgpr_write_b32 a215, %3\n\t"
      "v_accvgpr_read_b32 %0, a216\n\t"
      "v_accvgpr_read_b32 %1, a217\n\t"
      "v_accvgpr_read_b32 %2, a218\n\t"
      "v_accvgpr_read_b32 %3, a219\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a216, %0\n\t"
      "v_accvgpr_write_b32 a217, %1\n\t"
      "v_accvgpr_write_b32 a218, %2\n\t"
      "v_accvgpr_write_b32 a219, %3\n\t"
      "v_accvgpr_read_b32 %0, a220\n\t"
      "v_accvgpr_read_b32 %1, a221\n\t"
      "v_accvgpr_read_b32 %2, a222\n\t"
      "v_accvgpr_read_b32 %3, a223\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a220, %0\n\t"
      "v_accvgpr_write_b32 a221, %1\n\t"
      "v_accvgpr_write_b32 a222, %2\n\t"
      "v_accvgpr_write_b32 a223, %3\n\t"
      "v_accvgpr_read_b32 %0, a224\n\t"
      "v_accvgpr_read_b32 %1, a225\n\t"
      "v_accvgpr_read_b32 %2, a226\n\t"
      "v_accvgpr_read_b32 %3, a227\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a224, %0\n\t"
      "v_accvgpr_write_b32 a225, %1\n\t"
      "v_accvgpr_write_b32 a226, %2\n\t"
      "v_accvgpr_write_b32 a227, %3\n\t"
      "v_accvgpr_read_b32 %0, a228\n\t"
      "v_accvgpr_read_b32 %1, a229\n\t"
      "v_accvgpr_read_b32 %2, a230\n\t"
      "v_accvgpr_read_b32 %3, a231\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a228, %0\n\t"
      "v_accvgpr_write_b32 a229, %1\n\t"
      "v_accvgpr_write_b32 a230, %2\n\t"
      "v_accvgpr_write_b32 a231, %3\n\t"
      "v_accvgpr_read_b32 %0, a232\n\t"
      "v_accvgpr_read_b32 %1, a233\n\t"
      "v_accvgpr_read_b32 %2, a234\n\t"
      "v_accvgpr_read_b32 %3, a235\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a232, %0\n\t"
      "v_accvgpr_write_b32 a233, %1\n\t"
      "v_accvgpr_write_b32 a234, %2\n\t"
      "v_accvgpr_write_b32 a235, %3\n\t"
      "v_accvgpr_read_b32 %0, a236\n\t"
      "v_accvgpr_read_b32 %1, a237\n\t"
      "v_accvgpr_read_b32 %2, a238\n\t"
      "v_accvgpr_read_b32 %3, a239\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a236, %0\n\t"
      "v_accvgpr_write_b32 a237, %1\n\t"
      "v_accvgpr_write_b32 a238, %2\n\t"
      "v_accvgpr_write_b32 a239, %3\n\t"
      "v_accvgpr_read_b32 %0, a240\n\t"
      "v_accvgpr_read_b32 %1, a241\n\t"
      "v_accvgpr_read_b32 %2, a242\n\t"
      "v_accvgpr_read_b32 %3, a243\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a240, %0\n\t"
      "v_accvgpr_write_b32 a241, %1\n\t"
      "v_accvgpr_write_b32 a242, %2\n\t"
      "v_accvgpr_write_b32 a243, %3\n\t"
      "v_accvgpr_read_b32 %0, a244\n\t"
      "v_accvgpr_read_b32 %1, a245\n\t"
      "v_accvgpr_read_b32 %2, a246\n\t"
      "v_accvgpr_read_b32 %3, a247\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a244, %0\n\t"
      "v_accvgpr_write_b32 a245, %1\n\t"
      "v_accvgpr_write_b32 a246, %2\n\t"
      "v_accvgpr_write_b32 a247, %3\n\t"
      "v_accvgpr_read_b32 %0, a248\n\t"
      "v_accvgpr_read_b32 %1, a249\n\t"
      "v_accvgpr_read_b32 %2, a250\n\t"
      "v_accvgpr_read_b32 %3, a251\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a248, %0\n\t"
      "v_accvgpr_write_b32 a249, %1\n\t"
      "v_accvgpr_write_b32 a250, %2\n\t"
      "v_accvgpr_write_b32 a251, %3\n\t"
      "v_accvgpr_read_b32 %0, a252\n\t"
      "v_accvgpr_read_b32 %1, a253\n\t"
      "v_accvgpr_read_b32 %2, a254\n\t"
      "v_accvgpr_read_b32 %3, a255\n\t"
      "v_mul_f32 %0, %0, %4\n\t"
      "v_mul_f32 %1, %1, %4\n\t"
      "v_mul_f32 %2, %2, %4\n\t"
      "v_mul_f32 %3, %3, %4\n\t"
      "v_accvgpr_write_b32 a252, %0\n\t"
      "v_accvgpr_write_b32 a253, %1\n\t"
      "v_accvgpr_write_b32 a254, %2\n\t"
      "v_accvgpr_write_b32 a255, %3\n\t"
      "s_nop 7"
      : "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3)
      : "v"(alpha)
      : "memory");
}

struct WorkItem {
  int b, k, n, L;  // sequence, chunk index, chunk count, sequence length
};

// The sequence of chunk g: the largest b with split_offsets[b] <= g. A round
// probes 64 evenly spaced entries at once (one load per lane) and narrows the
// range 64-fold until at most 63 sequences remain; the last round loads their
// offsets and lengths side by side, so that the chunk's offsets and its
// sequence length come out of registers (readlane) rather than from a chain
// of dependent loads. B <= 63 takes that one round.
__device__ __forceinline__ WorkItem find_work(const int32_t* split_offsets, const int32_t* seqlens, int B, int g,
                                              int lane) {
  WorkItem w;
  if (split_offsets == nullptr) {
    w.b = g; w.k = 0; w.n = 1; w.L = seqlens[g];
    return w;
  }
  int lo = 0, n = B;  // the answer lies in [lo, lo + n)
  while (n > 63) {
    const int step = (n + 63) / 64;
    const bool le = lane * step < n && split_offsets[lo + lane * step] <= g;
    const int c = max(__popcll(__ballot(le)), 1);
    lo += (c - 1) * step;
    n = min(step, n - (c - 1) * step);
  }
  const int so = lane <= n ? split_offsets[lo + lane] : 0;  // n + 1 <= 64 offsets
  const int sl = lane < n ? seqlens[lo + lane] : 0;
  const int j = max(__popcll(__ballot(lane < n && so <= g)), 1) - 1;
  const int s0 = __builtin_amdgcn_readlane(so, j);
  w.b = lo + j;
  w.k = g - s0;
  w.n = __builtin_amdgcn_readlane(so, j + 1) - s0;
  w.L = __builtin_amdgcn_readlane(sl, j);
  return w;
}

// kSparse: top-k decode. The chunk walks "pages" of 64 consecutive entries of
// the query token's selected-token list instead of the sequence's pages: the
// prologue resolves the chunk's entries through the block table into
// physical row numbers (kept in LDS after the page buffers, with one 64-bit
// validity mask per page), each page is then gathered row by row, and
// entries outside [0, L_b) are masked out of the softmax (their slot is
// loaded from the sequence's token 0, so P = 0 meets finite values).
template <bool kSparse>
__global__ __launch_bounds__(kThreads, 1) void mla_decode_bf16_kernel(DecodeArgs a, int row_groups) {
  constexpr int kSparseBytes = kSparse ? kSparseMaxTopk * 4 + (kSparseMaxTopk / kPage) * 8 : 0;
  __shared__ __attribute__((aligned(1024))) char smem[2 * kPageBytes + kSparseBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: keep it in an SGPR
  const int r32 = lane & 31;   // the row this lane owns in MFMA outputs
  const int hi32 = lane >> 5;  // upper half of the wave

  // XCD-aware mapping: workgroups x and x+8j run on the same XCD (its own
  // L2). Each XCD takes a contiguous range of chunks, so the chunks of one
  // sequence (which load the same Q rows) and the row groups of one chunk
  // (which read the same pages) share an L2.
  const int x = blockIdx.x;
  const int xcd = x & 7;
  const int rest = x >> 3;
  const int rgrp = rest % row_groups;
  const int per_xcd = (a.total_splits + 7) / 8;
  const int g = xcd * per_xcd + rest / row_groups;
  if (rest / row_groups >= per_xcd || g >= a.total_splits) return;

  const WorkItem wi = find_work(a.split_offsets, a.seqlens, a.B, g, lane);
  const int b = wi.b;
  // Top-k: the chunks split the list (topk entries); positions must be < L.
  const int L = max(kSparse ? 1 : a.s_q, min(wi.L, a.max_pages * kPage));
  const int P = ((kSparse ? a.topk : L) + kPage - 1) / kPage;
  const int n_chunks = min(max(wi.n, 1), kMaxSplits);
  const int kk = min(max(wi.k, 0), n_chunks - 1);
  // kk * P < 64 * 2^25: exact in 32-bit unsigned arithmetic.
  const int pg0 = (int)((unsigned)kk * (unsigned)P / (unsigned)n_chunks);
  const int pg1 = (int)((unsigned)(kk + 1) * (unsigned)P / (unsigned)n_chunks);

  // Rows past the end (H*s_q not a multiple of 32) compute on a clamped row
  // and write nothing.
  const int rows = a.s_q * a.H;
  const int row = rgrp * kRowsPerGroup + wave * kWaveRows + r32;
  const int row_c = min(row, rows - 1);
  const int qi = row_c / a.H;
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
      const int t = it * kThreads + (int)threadIdx.x;
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
  {
    const __bf16* qrow = reinterpret_cast<const __bf16*>(a.q_lat) + ((size_t)b * rows + row_c) * kDqk + 8 * hi32;
#pragma unroll
    for (int s = 0; s < kQSteps; ++s) qf[s] = *reinterpret_cast<const bf16x8_t*>(qrow + 16 * s);
  }

  int phys_ahead = 0;
  if constexpr (kSparse) {
    // Physical row numbers of the chunk's entries (invalid ones point at the
    // sequence's token 0) and the per-page validity masks.
    const int n_tok = (pg1 - pg0) * kPage;
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const int t = it * kThreads + (int)threadIdx.x;
      const bool valid = lpos[it] >= 0 && lpos[it] < L;
      const unsigned long long m = __ballot(valid);  // wave w of round it holds page 4*it + w
      if (t < n_tok) {
        s_ids[t] = min(max(lphys[it], 0), last_phys) * kPage + ((valid ? lpos[it] : 0) & (kPage - 1));
        if (lane == 0) s_mask[t >> 6] = m;
      }
    }
    __syncthreads();
    if (pg0 < pg1) issue_page(make_gather_load(cache, s_ids, smem, wave, lane));
  } else if (pg0 < pg1) {
    const int phys = min(max(bt0, 0), last_phys);
    issue_page(make_page_load(cache + (size_t)phys * kPageBytes, smem, wave, lane));
    phys_ahead = bt1;
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
    // The next page's 18 loads per wave are issued one per four QK k-steps
    // over both tiles: in a denser burst the four waves' loads queue up in the
    // address unit and stall the MFMA stream behind them. (Built
    // unconditionally, from a clamped table index, so that its bases stay
    // wave-uniform SGPRs.)
    const bool has_next = pg + 1 < pg1;
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
        for (int idx = threadIdx.x; idx < (kPage - valid) * 72; idx += kThreads) {
          const int t = valid + idx / 72;
          const int c = idx % 72;
          *reinterpret_cast<uint4*>(buf + slot_bytes(t, c)) = make_uint4(0, 0, 0, 0);
        }
        __syncthreads();
      }
    }
    const bool full_page = kSparse ? page_mask == ~0ull : (pg + 1) * kPage <= n_allowed_min;

    // A page is two 32-token tiles, staggered so that the softmax work of
    // one tile runs between the MFMAs of the other: QK(T0); QK(T1) with
    // tile 0's exponentials; PV(T0) with tile 1's exponentials; PV(T1).
    // Tile 1's P uses a provisional reference taken before PV(T0); O and l
    // move to it only after PV(T0) has added tile 0 (which used the old one).
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
    // k-step kk of the tile takes scores 8kk .. 8kk+7.
    auto p_pair = [&](const f32x16_t& st, int e, float neg_ref, bf16x8_t* pf, float& psum) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[e], sl2, neg_ref));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[e + 1], sl2, neg_ref));
      pf[e >> 3][e & 7] = (__bf16)p0;
      pf[e >> 3][(e & 7) + 1] = (__bf16)p1;
      psum += p0 + p1;
    };
    constexpr int kKDepth = 3;
    constexpr int kPvDepth = 4;

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
        if (has_next && (s & 3) == 0) issue_line(next, s >> 2);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    const float mt0 = tile_max(st0, 0);
    move_reference((mt0 > m_ref + 8.0f) ? mt0 : m_ref);
    const float neg0 = (m_ref == -INFINITY) ? 0.f : -m_ref;

    // ---- QK(T1), with tile 0's P (two values every four k-steps) and the
    // other half of the next page's loads.
    f32x16_t st1;
#pragma unroll
    for (int r = 0; r < 16; ++r) st1[r] = 0.f;
    bf16x8_t pf0[2];
    float psum0 = 0.f;
    {
      bf16x8_t kf[kKDepth];
#pragma unroll
      for (int s = 0; s < kKDepth; ++s) kf[s] = k_frag(1, s);
#pragma unroll
      for (int s = 0; s < kQSteps; ++s) {
        const bf16x8_t cur = kf[s % kKDepth];
        if (s + kKDepth < kQSteps) kf[s % kKDepth] = k_frag(1, s + kKDepth);
        st1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, qf[s], st1, 0, 0, 0);
        if ((s & 3) == 0 && s < 32) p_pair(st0, s >> 1, neg0, pf0, psum0);
        if (has_next && (s & 3) == 2) issue_line(next, 9 + (s >> 2));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    l_loc += psum0;
    const float mt1 = tile_max(st1, 1);
    const float m1 = (mt1 > m_ref + 8.0f) ? mt1 : m_ref;  // provisional reference of tile 1
    const float neg1 = (m1 == -INFINITY) ? 0.f : -m1;

    // ---- PV(T0), with tile 1's P.
    bf16x8_t pf1[2];
    float psum1 = 0.f;
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
        if ((n & 3) == 0) p_pair(st1, n >> 1, neg1, pf1, psum1);
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

  // ---- finalize: o = O / l, lse = ln2 * (m_ref + log2 l); l is split over
  // the two lanes of a row.
  agpr_fence();
  const float l_tot = l_loc + other_half(l_loc);
  const bool any = l_tot > 0.f;
  const float inv = any ? 1.f / l_tot : 0.f;
  const float lse_v = any ? (m_ref + __log2f(l_tot)) * 0.6931471805599453f : -INFINITY;

  // The rows go out through LDS. acc_o[i][r] is O^T[32i + 8(r>>2) + 4*hi32 +
  // (r&3)][row], so a lane holds 8-byte pieces of its row and a direct store
  // would touch 32 rows per instruction, 16 bytes each: partial 128-byte lines
  // that stay dirty in L2 until the end of the kernel and then cost
  // microseconds to write back. Staged, every store instruction writes one
  // whole 1 KB row, non-temporal: nothing reads it again in this kernel. Row r of a wave's 32 KB staging area keeps its 64 16-byte
  // pieces XOR-permuted by r so that the 32 rows of a write do not fall on the
  // same LDS banks.
  __syncthreads();  // every wave is done with the page buffers
  // The lane position is taken afresh (mbcnt) rather than kept live through
  // the page loop, where every VGPR is taken.
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
      const int piece = (4 * i + q4) ^ r32f;  // 16-byte piece of the row, permuted
      *reinterpret_cast<bf16x4_t*>(stage + r32f * (kDv * 2) + piece * 16 + 8 * hi32f) = v;
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
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(out + (size_t)(row0 + r) * kDv + 8 * ln));
  }
  if (hi32f == 0 && rowf < rows) {
    if (direct)
      a.lse[(size_t)b * rows + rowf] = lse_v;
    else
      a.lse_part[(size_t)g * rows + rowf] = lse_v;
  }
}

template <bool kSparse>
hipError_t launch(const DecodeArgs& a, hipStream_t stream) {
  const int rows = a.s_q * a.H;
  const int row_groups = (rows + kRowsPerGroup - 1) / kRowsPerGroup;
  const int padded = (a.total_splits + 7) / 8 * 8;
  const dim3 grid((unsigned)(padded * row_groups));
  hipLaunchKernelGGL(mla_decode_bf16_kernel<kSparse>, grid, dim3(kThreads), 0, stream, a, row_groups);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream) { return launch<false>(a, stream); }
hipError_t launch_sparse_decode_bf16(const DecodeArgs& a, hipStream_t stream) { return launch<true>(a, stream); }

}  // namespace mla

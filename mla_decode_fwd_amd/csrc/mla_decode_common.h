// Device helpers shared by the bf16 and FP8 decode kernels (gfx950):
// register types, the direct global->LDS load, the PV MFMA with O pinned in
// AGPRs, the in-place rescale of O, and the chunk -> sequence lookup.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "mla_internal.h"

namespace mla {
namespace dec {

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
constexpr int kQSteps = kDqk / 16;                 // 36 k-steps of 16
constexpr int kColTiles = kDv / 32;                // 16 column tiles of 32
// s_waitcnt immediate for gfx9: vmcnt = 0, expcnt and lgkmcnt left at "no wait".
constexpr int kWaitVmcnt0 = (0xF << 8) | (0x7 << 4);

// One direct 16-byte-per-lane load: global sbase + voff -> LDS lds + 16*lane.
// Non-temporal (nt): every cache page is read once per chunk, and on MI355X a
// stream of nt direct loads with one page in flight per compute unit reaches
// ~6.4 TB/s against ~5.6 TB/s without the hint (a 302 MB read, 256
// workgroups, 72 KB in flight each).
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
      "global_load_lds_dwordx4 %0, %1 nt"
      :
      : "v"(voff), "s"(sbase), "s"(lds)
      : "memory", "m0");
}
// The same load with M0 written by a single SALU add (lds_base + lds_off)
// and an immediate byte offset that the instruction adds to both the global
// and the LDS address: one instruction fewer per line than computing the LDS
// address into an SGPR first, and no VALU add for the global offset (the
// per-lane offset stays the unsigned, non-negative voff).
__device__ __forceinline__ void dma_line_off(uint64_t sbase, int voff, uint32_t lds_base, const int lds_off,
                                             const int imm) {
  asm volatile(
      "s_add_u32 m0, %2, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1 offset:%4 nt"
      :
      : "v"(voff), "s"(sbase), "s"(lds_base), "i"(lds_off), "i"(imm)
      : "memory", "m0", "scc");
}
// The same load without the non-temporal hint (data that other workgroups
// read again soon: the query rows).
__device__ __forceinline__ void dma_line_cached(uint64_t sbase, int voff, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(sbase), "s"(lds)
      : "memory", "m0");
}
#pragma clang diagnostic pop

// A 16-byte store at device scope (cache-policy bit sc1 of a gfx950 buffer
// store): the line is written through this XCD's L2 to the memory side at
// once instead of staying dirty in L2 until the end-of-launch write-back, and
// the next kernel finds it there whichever XCD it runs on. `base` must be
// wave-uniform: it becomes the buffer descriptor, in SGPRs; `off` is the
// lane's byte offset from it (below 2 GiB). Descriptor word 3 selects the
// 32-bit data format that untyped buffer accesses need.
__device__ __forceinline__ void store_device_scope(void* base, uint32_t off, u32x4_t v) {
  typedef uint32_t v4u __attribute__((ext_vector_type(4)));
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7FFFFFFF, 0x00020000);
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v), r, off, 0, 16 /* sc1 */);
}
// The same for one float (a chunk's partial LSE values).
__device__ __forceinline__ void store_device_scope(void* base, uint32_t off, float v) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7FFFFFFF, 0x00020000);
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 16 /* sc1 */);
}

// s_waitcnt immediate for gfx9 waiting until at most n (< 64) vector memory
// operations are outstanding (vmcnt is split over bits 3:0 and 15:14).
constexpr int wait_vmcnt(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0xF << 8) | (0x7 << 4); }
// ... until no LDS operation is outstanding (lgkmcnt 0, vmcnt and expcnt not waited on).
constexpr int kWaitLgkm0 = 0xF | (0x3 << 14) | (0x7 << 4);

// The lane's index in its wave, produced where it is used: the compiler
// cannot hoist an asm result out of a loop, so values derived from it are
// recomputed there instead of being kept live (and spilled) across it.
__device__ __forceinline__ int lane_id() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// One round of staged query rows (both decode kernels stage the rows of a
// workgroup through LDS with coalesced direct loads, then read their
// operands from there): `nrows` rows of `cols` bytes from column byte
// `col0`, row R at R * (cols + 16) bytes of the area, so that the 16 rows of
// a 16-byte read pass start on 16 different bank groups. nrows * (cols + 16)
// must be a multiple of 1024: instruction i of the round fills area bytes
// 1024i .. 1024i + 1023, and the waves take instructions w, w + 4, ... Lanes
// that fall on a row's padding load the row's first piece (never read).
__device__ __forceinline__ void issue_q_round(const char* q_seq, int rows, int row_base, int nrows, int cols,
                                              int col0, char* area, int wave, int lane) {
  const int stride = cols + 16;
  const int n_inst = nrows * stride / 1024;
  const uint64_t gp = (uint64_t)(uintptr_t)q_seq;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)gp);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(gp >> 32));
  const uint64_t sbase = ((uint64_t)hi << 32) | (uint64_t)lo;
  const uint32_t lds0 = (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)(uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)area);
  for (int i = wave; i < n_inst; i += kWaves) {
    const int byte = 1024 * i + 16 * lane;
    const int R = byte / stride, off = byte - R * stride;
    const int row = min(row_base + R, rows - 1);
    dma_line_cached(sbase, row * (kDqk * 2) + col0 + (off < cols ? off : 0), lds0 + 1024 * i);
  }
}

// Value of lane l ^ 32 (gfx950 lane swap; VALU, no LDS round trip). With
// both operands equal, permlane32_swap yields the values of lanes l and l^32.
__device__ __forceinline__ float other_half(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float((lane_id() & 32) ? r[0] : r[1]);
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
// Four AGPRs a(n) .. a(n+3) scaled through the four temporaries.
#define MLA_SCALE4(n0, n1, n2, n3)                                                        \
  "v_accvgpr_read_b32 %0, a" #n0 "\n\tv_accvgpr_read_b32 %1, a" #n1 "\n\t"              \
  "v_accvgpr_read_b32 %2, a" #n2 "\n\tv_accvgpr_read_b32 %3, a" #n3 "\n\t"              \
  "v_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\t"                                    \
  "v_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\t"                                    \
  "v_accvgpr_write_b32 a" #n0 ", %0\n\tv_accvgpr_write_b32 a" #n1 ", %1\n\t"            \
  "v_accvgpr_write_b32 a" #n2 ", %2\n\tv_accvgpr_write_b32 a" #n3 ", %3\n\t"
__device__ __forceinline__ void scale_accumulators(float alpha) {
  float t0, t1, t2, t3;
  asm volatile(
      MLA_SCALE4(0, 1, 2, 3) MLA_SCALE4(4, 5, 6, 7) MLA_SCALE4(8, 9, 10, 11) MLA_SCALE4(12, 13, 14, 15)
      MLA_SCALE4(16, 17, 18, 19) MLA_SCALE4(20, 21, 22, 23) MLA_SCALE4(24, 25, 26, 27) MLA_SCALE4(28, 29, 30, 31)
      MLA_SCALE4(32, 33, 34, 35) MLA_SCALE4(36, 37, 38, 39) MLA_SCALE4(40, 41, 42, 43) MLA_SCALE4(44, 45, 46, 47)
      MLA_SCALE4(48, 49, 50, 51) MLA_SCALE4(52, 53, 54, 55) MLA_SCALE4(56, 57, 58, 59) MLA_SCALE4(60, 61, 62, 63)
      MLA_SCALE4(64, 65, 66, 67) MLA_SCALE4(68, 69, 70, 71) MLA_SCALE4(72, 73, 74, 75) MLA_SCALE4(76, 77, 78, 79)
      MLA_SCALE4(80, 81, 82, 83) MLA_SCALE4(84, 85, 86, 87) MLA_SCALE4(88, 89, 90, 91) MLA_SCALE4(92, 93, 94, 95)
      MLA_SCALE4(96, 97, 98, 99) MLA_SCALE4(100, 101, 102, 103) MLA_SCALE4(104, 105, 106, 107) MLA_SCALE4(108, 109, 110, 111)
      MLA_SCALE4(112, 113, 114, 115) MLA_SCALE4(116, 117, 118, 119) MLA_SCALE4(120, 121, 122, 123) MLA_SCALE4(124, 125, 126, 127)
      MLA_SCALE4(128, 129, 130, 131) MLA_SCALE4(132, 133, 134, 135) MLA_SCALE4(136, 137, 138, 139) MLA_SCALE4(140, 141, 142, 143)
      MLA_SCALE4(144, 145, 146, 147) MLA_SCALE4(148, 149, 150, 151) MLA_SCALE4(152, 153, 154, 155) MLA_SCALE4(156, 157, 158, 159)
      MLA_SCALE4(160, 161, 162, 163) MLA_SCALE4(164, 165, 166, 167) MLA_SCALE4(168, 169, 170, 171) MLA_SCALE4(172, 173, 174, 175)
      MLA_SCALE4(176, 177, 178, 179) MLA_SCALE4(180, 181, 182, 183) MLA_SCALE4(184, 185, 186, 187) MLA_SCALE4(188, 189, 190, 191)
      MLA_SCALE4(192, 193, 194, 195) MLA_SCALE4(196, 197, 198, 199) MLA_SCALE4(200, 201, 202, 203) MLA_SCALE4(204, 205, 206, 207)
      MLA_SCALE4(208, 209, 210, 211) MLA_SCALE4(212, 213, 214, 215) MLA_SCALE4(216, 217, 218, 219) MLA_SCALE4(220, 221, 222, 223)
      MLA_SCALE4(224, 225, 226, 227) MLA_SCALE4(228, 229, 230, 231) MLA_SCALE4(232, 233, 234, 235) MLA_SCALE4(236, 237, 238, 239)
      MLA_SCALE4(240, 241, 242, 243) MLA_SCALE4(244, 245, 246, 247) MLA_SCALE4(248, 249, 250, 251) MLA_SCALE4(252, 253, 254, 255)
      "s_nop 7"
      : "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3)
      : "v"(alpha)
      : "memory");
}
#undef MLA_SCALE4

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

}  // namespace dec
}  // namespace mla

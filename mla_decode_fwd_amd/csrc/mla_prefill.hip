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
#include "mla_launch_aux.h"

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
// expand_kernel: the expansion is one GEMM per head, [tokens x 512] times
// [512 x 256] (W_UK[h] and W_UV[h] side by side). A workgroup of eight waves
// owns one head and one range of the chunk's tokens; wave w keeps the
// transposed weight columns 32(w&3) .. +31 of W_UK[h] (waves 0-3) or W_UV[h]
// (waves 4-7) in registers for the whole range (the A operand, 32 k-steps,
// 128 VGPRs), and the range's latent rows stream through LDS 32 tokens at a
// time (the B operand, read with ds_read_b128). So the weights are read
// once per workgroup, every latent byte in LDS feeds eight MFMAs, and the
// workgroups of one XCD take the same token range (the latent stays in its
// L2). Output: K [H, chunk, 128] and V [H, chunk, 128] bf16 as
// D^T[column][token]; the head-0 workgroup of each range also copies the
// tokens' RoPE keys into R [chunk, 64], which every head shares.
// ---------------------------------------------------------------------------
constexpr int kExpWaves = 8;
constexpr int kExpThreads = 64 * kExpWaves;
constexpr int kTok = 32;                         // tokens per latent tile
constexpr int kLatStride = kLat * 2 + 16;        // 1040: 16 consecutive tokens on 16 bank groups
constexpr int kTileBytes = kTok * kLatStride;    // 33,280
constexpr int kRing = 3;                         // tile buffers: the current tile and two in flight
constexpr int kAhead = kRing - 1;
constexpr int kMaxRangePages = 1040;             // page ids of one token range kept in LDS
constexpr int kOutStride = kNope * 2 + 16;       // 272: staged output row of one tile token
constexpr int kOutBytes = 2 * kTok * kOutStride; // K and V rows of one tile: 17,408
constexpr int kWSlice = 64;                      // latent rows per weight slice
constexpr int kWStride = kNope * 2 + 64;         // 320: LDS row stride of a slice
constexpr int kWMat = kWSlice * kWStride;        // 20,480: one matrix's slice
static_assert(4 * kWMat <= kRing * kTileBytes, "two staged weight slices fit in the tile buffers");
static_assert(kTok == 4 * kExpWaves, "each wave loads four token rows of a tile");

// One direct load of a 1 KB token row: lane l's 16 bytes at vaddr go to LDS
// lds + 16 l. Inline asm, so the compiler's wait counting does not see it;
// the tile loop waits for these loads with explicit vmcnt values.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma_row(uint64_t vaddr, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(vaddr), "s"(lds)
      : "memory", "m0");
}
#pragma clang diagnostic pop

__global__ __launch_bounds__(kExpThreads, 1) void expand_kernel(
    const __bf16* __restrict__ cache, const int32_t* __restrict__ btab_row, int t0, int n, int num_pages,
    const __bf16* __restrict__ w_uk, const __bf16* __restrict__ w_uv, int H, __bf16* __restrict__ k_out,
    __bf16* __restrict__ v_out, __bf16* __restrict__ r_out, int n_stride, int ranges, int range_tokens) {
  __shared__ __attribute__((aligned(16))) char smem[kRing * kTileBytes + kMaxRangePages * 4 + 2 * kOutBytes];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int r32 = lane & 31, hi32 = lane >> 5;

  // Workgroup x runs on XCD x & 7; the XCDs split the token ranges, so the
  // heads on one XCD read the same latent rows.
  const int x = blockIdx.x;
  const int xcd = x & 7;
  const int h = (x >> 3) * (8 / ranges) + xcd / ranges;
  const int rg = xcd % ranges;
  const int tok_begin = rg * range_tokens;
  const int tok_end = min(n, tok_begin + range_tokens);
  if (h >= H || tok_begin >= tok_end) return;  // uniform over the workgroup
  const int ct = wave & 3;
  const bool is_v = wave >= 4;

  // ---- Weight fragments: k-step s holds W[16s + 8*hi32 + j][32ct + r32],
  // j = 0..7, staged 64 latent rows of both matrices at a time and read
  // transposed (16-lane group g, input lane 4jj + q: latent row
  // 8(g>>1) + 4rd + jj, columns 16(g&1) + 4q .. +4 of the 32-column tile).
  bf16x8_t wf[kLat / 16];
  {
    const int g = lane >> 4, jj = (lane >> 2) & 3, q = lane & 3;
    const int tr_off = (is_v ? kWMat : 0) + kWStride * (8 * (g >> 1) + jj) + 2 * (16 * (g & 1) + 4 * q) + 64 * ct;
    const size_t wbase = (size_t)h * kLat * kNope;
    // Two staged slices alternate in LDS and the global loads run two slices
    // ahead, so one barrier per slice suffices and the load latency is paid
    // about half as often.
    u32x4_t pre[2][4];
    auto load_slice = [&](int ks, u32x4_t (&r)[4]) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int idx = u * kExpThreads + t;        // 0 .. 2047
        const int mat = idx >> 10, rem = idx & 1023;
        const int row = rem >> 4, c16 = rem & 15;
        r[u] = *reinterpret_cast<const u32x4_t*>((mat ? w_uv : w_uk) + wbase + (size_t)(ks * kWSlice + row) * kNope +
                                                 8 * c16);
      }
    };
    load_slice(0, pre[0]);
    load_slice(1, pre[1]);
#pragma unroll
    for (int ks = 0; ks < kLat / kWSlice; ++ks) {
      char* const region = smem + (ks & 1) * (2 * kWMat);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int idx = u * kExpThreads + t;
        const int mat = idx >> 10, rem = idx & 1023;
        *reinterpret_cast<u32x4_t*>(region + mat * kWMat + (rem >> 4) * kWStride + 16 * (rem & 15)) = pre[ks & 1][u];
      }
      __syncthreads();  // slice ks staged; every wave is done with slice ks - 2's region
      if (ks + 2 < kLat / kWSlice) load_slice(ks + 2, pre[ks & 1]);
#pragma unroll
      for (int s4 = 0; s4 < kWSlice / 16; ++s4) {
        bf16x8_t w;
#pragma unroll
        for (int rd = 0; rd < 2; ++rd) {
          const bf16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (lds_b4_t*)((__attribute__((address_space(3))) char*)region + tr_off + kWStride * (16 * s4 + 4 * rd)));
          w[4 * rd + 0] = v[0]; w[4 * rd + 1] = v[1]; w[4 * rd + 2] = v[2]; w[4 * rd + 3] = v[3];
        }
        wf[ks * 4 + s4] = w;
      }
    }
    __syncthreads();  // the staging area becomes the tile ring
  }

  // ---- Latent tiles through a ring of kRing LDS buffers, filled by direct
  // loads kAhead tiles ahead: wave w loads token rows 4w .. 4w+3 of a tile,
  // one 1 KB load each. The range's physical page ids are first copied to
  // LDS, so that no global load of the loop depends on another.
  int32_t* const s_pages = reinterpret_cast<int32_t*>(smem + kRing * kTileBytes);
  const int page0 = (t0 + tok_begin) >> 6;
  const int n_pages = ((t0 + tok_end - 1) >> 6) - page0 + 1;  // <= kMaxRangePages (checked by the host)
  for (int i = t; i < n_pages; i += kExpThreads) s_pages[i] = min(max(btab_row[page0 + i], 0), num_pages - 1);
  __syncthreads();
  const int n_tiles = (tok_end - tok_begin + kTok - 1) / kTok;
  const uint32_t lds_ring =
      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem);
  // Sources of a tile's four rows for this wave, prepared one iteration
  // before their loads are issued (the page id comes from LDS).
  uint64_t nsrc[4];
  // The four rows lie in at most two pages; both page ids are read before
  // either is used, so the wave waits on LDS once.
  auto prep_tile = [&](int i) {
    const int slot0 = ((t0 + min(tok_begin + i * kTok + 4 * wave, tok_end - 1)) >> 6) - page0;
    const int id_a = s_pages[slot0];
    const int id_b = s_pages[slot0 + 1];  // < kMaxRangePages; used only when the rows reach the next page
    const int phys_a = __builtin_amdgcn_readfirstlane(id_a);
    const int phys_b = __builtin_amdgcn_readfirstlane(id_b);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int pos = t0 + min(tok_begin + i * kTok + 4 * wave + j, tok_end - 1);  // clamped into the range
      const int phys = ((pos >> 6) - page0 == slot0) ? phys_a : phys_b;
      nsrc[j] = (uint64_t)(uintptr_t)(cache + ((size_t)phys * kPage + (pos & (kPage - 1))) * kDqk) + 16 * (uint32_t)lane;
    }
  };
  auto issue_row = [&](int i, int j) {
    dma_row(nsrc[j], lds_ring + (uint32_t)((i % kRing) * kTileBytes + (4 * wave + j) * kLatStride));
  };
#pragma unroll
  for (int i = 0; i < kAhead; ++i) {
    if (i < n_tiles) {
      prep_tile(i);
#pragma unroll
      for (int j = 0; j < 4; ++j) issue_row(i, j);
    }
  }
  if (kAhead < n_tiles) prep_tile(kAhead);

  const int b_off = r32 * kLatStride + 16 * hi32;
  // Results leave through LDS: each wave writes its 32 x 32 block of D^T
  // into the tile's staged K or V rows (272-byte rows keep the 8-byte writes
  // of 32 tokens on distinct banks), and after the next barrier every thread
  // stores two 16-byte pieces, so each store instruction writes four whole
  // 256-byte rows. Two staging buffers alternate between tiles.
  char* const stage0 = smem + kRing * kTileBytes + kMaxRangePages * 4;
  auto stage_tile = [&](const f32x16_t& acc, int i) {
    char* st = stage0 + (i & 1) * kOutBytes + (is_v ? kTok * kOutStride : 0) + r32 * kOutStride + 2 * (32 * ct + 4 * hi32);
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      bf16x4_t v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (__bf16)acc[4 * q4 + e];
      *reinterpret_cast<bf16x4_t*>(st + 16 * q4) = v;
    }
  };
  auto store_piece = [&](int i, int u) {
    const int p = u * kExpThreads + t;  // 0 .. 1023
    const int mat = p >> 9, tok = (p >> 4) & (kTok - 1), c16 = p & 15;
    const int tk = tok_begin + i * kTok + tok;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stage0 + (i & 1) * kOutBytes + mat * kTok * kOutStride +
                                                        tok * kOutStride + 16 * c16);
    // Non-temporal: the chunk's expanded keys and values (64 KB per token)
    // are far larger than the caches and are read back once, by the
    // attention kernel (extend: 2.73 -> 2.69 ms per call).
    if (tk < tok_end)
      __builtin_nontemporal_store(
          v, reinterpret_cast<u32x4_t*>((mat ? v_out : k_out) + ((size_t)h * n_stride + tk) * kNope + 8 * c16));
  };
  for (int i = 0; i < n_tiles; ++i) {
    // Tile i has landed once at most the 4 loads of the next tile remain in
    // flight (in-order completion; stores issued after tile i's loads only
    // make the wait longer, never too short).
    if (i + 1 < n_tiles)
      __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8) | 4);
    else
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();  // tile i and the previous tile's staged rows visible; tile i-1's buffer free
    const bool issue_next = i + kAhead < n_tiles;
    const char* buf = smem + (i % kRing) * kTileBytes;
    f32x16_t acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    // B fragments read kBDepth k-steps ahead; the previous tile's stores and
    // the loads of tile i + kAhead go out between the first MFMAs.
    constexpr int kBDepth = 8;
    bf16x8_t bq[kBDepth];
#pragma unroll
    for (int s = 0; s < kBDepth; ++s) bq[s] = *reinterpret_cast<const bf16x8_t*>(buf + b_off + 32 * s);
#pragma unroll
    for (int s = 0; s < kLat / 16; ++s) {
      const bf16x8_t bfr = bq[s % kBDepth];
      if (s + kBDepth < kLat / 16) bq[s % kBDepth] = *reinterpret_cast<const bf16x8_t*>(buf + b_off + 32 * (s + kBDepth));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[s], bfr, acc, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (s < 2 && i > 0) store_piece(i - 1, s);
      if (s >= 2 && s < 6 && issue_next) issue_row(i + kAhead, s - 2);
      __builtin_amdgcn_sched_barrier(0);
    }
    // acc[r] = D^T[32ct + 8(r>>2) + 4*hi32 + (r&3)][token r32 of tile i].
    stage_tile(acc, i);
    if (i + kAhead + 1 < n_tiles) prep_tile(i + kAhead + 1);
  }
  __syncthreads();
  store_piece(n_tiles - 1, 0);
  store_piece(n_tiles - 1, 1);

  // ---- The RoPE keys of the range, once per range (head 0).
  if (h == 0) {
    for (int idx = t; idx < (tok_end - tok_begin) * 8; idx += kExpThreads) {
      const int tok = tok_begin + (idx >> 3), c = idx & 7;
      const int pos = t0 + tok;
      const int phys = min(max(btab_row[pos >> 6], 0), num_pages - 1);
      *reinterpret_cast<u32x4_t*>(r_out + (size_t)tok * kRope + 8 * c) = *reinterpret_cast<const u32x4_t*>(
          cache + ((size_t)phys * kPage + (pos & (kPage - 1))) * kDqk + kLat + 8 * c);
    }
  }
}

// ---------------------------------------------------------------------------
// attn_kernel: one workgroup per (256 new tokens, head), eight waves of 32
// query rows (two per SIMD). Q^T (12 k-steps over 192) stays in VGPRs, O^T
// (128 columns) in four 32x32 accumulators. Keys come in tiles of 64,
// double-buffered in LDS (global loads into registers during the previous
// tile's products, one barrier per tile), so every K and V byte in LDS
// feeds the eight waves: S^T = K Q^T per 32-key half, base-2 online softmax
// over the 64 keys with a lazily moved reference (as the decode kernel),
// O^T += V^T P^T with P^T taken from the score registers and V^T read
// transposed. A wave skips the products of tiles that lie wholly past its
// last row's position.
// ---------------------------------------------------------------------------
constexpr int kAttnWaves = 8;
constexpr int kAttnThreads = 64 * kAttnWaves;
constexpr int kQRows = kAttnWaves * kWaveRows;  // 256 query rows per workgroup
constexpr int kKStride = kHeadK * 2 + 16;   // 400: 16 consecutive keys on 16 bank groups
constexpr int kVStride = kHeadV * 2 + 64;   // 320
constexpr int kKTile = 64;
constexpr int kKBuf = kKTile * kKStride;    // 25,600
constexpr int kVBuf = kKTile * kVStride;    // 20,480
constexpr int kStage = kKBuf + kVBuf;
static_assert(kKTile * 24 == 3 * kAttnThreads && kKTile * 16 == 2 * kAttnThreads, "tile loads: 3 + 2 pieces per thread");

__global__ __launch_bounds__(kAttnThreads, 1) void attn_kernel(const __bf16* __restrict__ q_nope,
                                                              const __bf16* __restrict__ q_rope, int s_q, int H,
                                                              const __bf16* __restrict__ K,
                                                              const __bf16* __restrict__ V,
                                                              const __bf16* __restrict__ R, int n, int n_stride,
                                                              int k_pos0, int q_pos0, int causal, float scale,
                                                              __bf16* __restrict__ o, float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kStage];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int r32 = lane & 31, hi32 = lane >> 5;
  // Head-major, XCD-aware order: workgroup x runs on XCD x & 7, which takes
  // heads x & 7, 8 + (x & 7), ... one at a time, heaviest query block first.
  // So the query blocks of one head run together on one XCD and re-read
  // that head's keys and values from its L2 and the last-level cache rather
  // than from HBM.
  const int n_qb = (s_q + kQRows - 1) / kQRows;
  const int xk = blockIdx.x >> 3;
  const int h = (xk / n_qb) * 8 + (blockIdx.x & 7);
  if (h >= H) return;  // uniform over the workgroup, before any barrier
  const int qb = (n_qb - 1 - xk % n_qb) * kQRows;
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
  const int q_last = q_pos0 + min(s_q, qb + kQRows) - 1;
  const int n_vis = causal ? max(0, min(n, q_last - k_pos0 + 1)) : n;
  const int tiles = (n_vis + kKTile - 1) / kKTile;
  const int w_first = q_pos0 + min(qb + wave * kWaveRows, s_q - 1);                   // this wave's first row
  const int w_last = q_pos0 + min(qb + wave * kWaveRows + kWaveRows, s_q) - 1;         // and its last row

  const __bf16* Kh = K + (size_t)h * n_stride * kNope;
  const __bf16* Vh = V + (size_t)h * n_stride * kHeadV;
  // Tile loads: K 64 rows x 24 chunks (3 per thread; chunks 0-15 from the
  // head's expanded keys, 16-23 the shared RoPE key), V 64 rows x 16 chunks
  // (2 per thread).
  auto load_tile = [&](int kt, u32x4_t (&kr)[3], u32x4_t (&vr)[2]) {
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      const int idx = u * kAttnThreads + t;
      const int row = idx / 24, c16 = idx % 24;
      const int key = min(kt * kKTile + row, n - 1);
      kr[u] = *reinterpret_cast<const u32x4_t*>(c16 < 16 ? Kh + (size_t)key * kNope + 8 * c16
                                                         : R + (size_t)key * kRope + 8 * (c16 - 16));
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int idx = u * kAttnThreads + t;
      const int row = idx >> 4, c16 = idx & 15;
      const int key = min(kt * kKTile + row, n - 1);
      vr[u] = *reinterpret_cast<const u32x4_t*>(Vh + (size_t)key * kHeadV + 8 * c16);
    }
  };
  auto store_tile = [&](char* buf, const u32x4_t (&kr)[3], const u32x4_t (&vr)[2]) {
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      const int idx = u * kAttnThreads + t;
      *reinterpret_cast<u32x4_t*>(buf + (idx / 24) * kKStride + 16 * (idx % 24)) = kr[u];
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int idx = u * kAttnThreads + t;
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
    __syncthreads();  // tile kt visible; every wave is done with tile kt-2, whose buffer the next store refills
    if (kt + 1 < tiles) load_tile(kt + 1, kr, vr);
    const int key0 = k_pos0 + kt * kKTile;  // position of the tile's first key
    if (!causal || key0 <= w_last) {
      f32x16_t st[2];
#pragma unroll
      for (int T = 0; T < 2; ++T) {
#pragma unroll
        for (int r = 0; r < 16; ++r) st[T][r] = 0.f;
#pragma unroll
        for (int s = 0; s < kHeadK / 16; ++s) {
          const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(buf + T * 32 * kKStride + qk_off + 32 * s);
          st[T] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], st[T], 0, 0, 0);
        }
      }
      // Mask keys past the chunk or past the query's position.
      const bool full = kt * kKTile + kKTile <= n_vis && (!causal || key0 + kKTile - 1 <= w_first);
      if (!full) {
#pragma unroll
        for (int T = 0; T < 2; ++T)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kl = kt * kKTile + 32 * T + 8 * (r >> 2) + 4 * hi32 + (r & 3);
            if (kl >= n_vis || (causal && k_pos0 + kl > qpos)) st[T][r] = -INFINITY;
          }
      }
      float mx = fmaxf(st[0][0], st[1][0]);
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(st[0][r], st[1][r]));
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
      // k-step u of the tile: keys 16u .. 16u+15 = half T = u >> 1, scores 8(u&1) .. +8.
      bf16x8_t pf[4];
#pragma unroll
      for (int T = 0; T < 2; ++T)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(st[T][r], sl2, neg));
          l_loc += p;
          pf[2 * T + (r >> 3)][r & 7] = (__bf16)p;
        }
#pragma unroll
      for (int u = 0; u < 4; ++u)
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
// merge_kernel: one wave per (token, head) row; its four 16-lane groups split
// the chunks, each lane of a group owns 8 of the 128 columns; chunk k's
// weight is exp(lse_k - lse).
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
  // Lane group g = lane >> 4 takes chunks g, g + 4, ...; its 16 lanes own 8
  // columns each. Sixteen chunks per round, all loads of a round issued
  // before their products; slots past n_parts load nothing and weigh 0. The
  // four groups' sums meet by lane swaps.
  const int sub = lane & 15, grp = lane >> 4;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < n_parts; k0 += 16) {
    bf16x8_t x[4];
    float wk[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = k0 + 4 * j + grp;
      wk[j] = __shfl(wn, min(k, 63), 64);
      if (k < n_parts) {
        x[j] = *reinterpret_cast<const bf16x8_t*>(o_part + ((size_t)k * rows + row) * kHeadV + 8 * sub);
      } else {
        wk[j] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[j][e] = (__bf16)0.f;
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(wk[j], (float)x[j][e], acc[e]);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    acc[e] += __shfl_xor(acc[e], 16, 64);
    acc[e] += __shfl_xor(acc[e], 32, 64);
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
                         const void* w_uv, int H, void* k_out, void* v_out, void* r_out, int n_stride,
                         hipStream_t stream) {
  // About one workgroup per compute unit: ranges (a divisor of 8) split the
  // chunk's tokens so that H * ranges reaches 256 where it can.
  int ranges = 1;
  while (ranges < 8 && H * ranges < 256 && (n + 2 * ranges - 1) / (2 * ranges) >= kTok) ranges *= 2;
  const int range_tokens = ((n + ranges - 1) / ranges + kTok - 1) / kTok * kTok;
  const int groups = (H * ranges + 7) / 8 * 8;
  hipLaunchKernelGGL(expand_kernel, dim3((unsigned)groups), dim3(kExpThreads), 0, stream,
                     static_cast<const __bf16*>(cache), btab_row, t0, n, num_pages, static_cast<const __bf16*>(w_uk),
                     static_cast<const __bf16*>(w_uv), H, static_cast<__bf16*>(k_out), static_cast<__bf16*>(v_out),
                     static_cast<__bf16*>(r_out), n_stride, ranges, range_tokens);
  return hipGetLastError();
}

hipError_t launch_prefill_attn(const void* q_nope, const void* q_rope, int s_q, int H, const void* K, const void* V,
                               const void* R, int n, int n_stride, int k_pos0, int q_pos0, int causal, float scale,
                               void* o, float* lse, hipStream_t stream) {
  const int n_qb = (s_q + kQRows - 1) / kQRows;
  const dim3 grid((unsigned)(n_qb * ((H + 7) / 8) * 8));
  hipLaunchKernelGGL(attn_kernel, grid, dim3(kAttnThreads), 0, stream, static_cast<const __bf16*>(q_nope),
                     static_cast<const __bf16*>(q_rope), s_q, H, static_cast<const __bf16*>(K),
                     static_cast<const __bf16*>(V), static_cast<const __bf16*>(R), n, n_stride, k_pos0, q_pos0,
                     causal, scale, static_cast<__bf16*>(o), lse);
  return hipGetLastError();
}

hipError_t launch_prefill_merge(const void* o_part, const float* lse_part, int n_parts, int rows, void* o, float* lse,
                                hipStream_t stream) {
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream,
                     static_cast<const __bf16*>(o_part), lse_part, n_parts, rows, static_cast<__bf16*>(o), lse);
  return hipGetLastError();
}

}  // namespace mla

// Internal launch interfaces of the absorbed-MLA decode library (gfx950):
// the shapes and arguments of the decode kernels and their merge. The C ABI
// (include/mla_decode.h) validates arguments and then calls these; the other
// kernels' launchers are in mla_launch_aux.h.
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

#include "mla_decode.h"

namespace mla {

constexpr int kDqk = 576;       // key width: latent 512 + RoPE 64
constexpr int kDv = 512;        // value width: the latent
constexpr int kPage = 64;       // tokens per cache page
constexpr int kMaxSplits = 64;  // chunks per sequence at most
constexpr int kRowsPerGroup = 128;  // query rows (token, head) per decode workgroup

// Arguments of one decode launch, already validated on the host.
struct DecodeArgs {
  const void* q_lat;            // [B, s_q, H, 576]
  const void* kv_cache;         // [num_pages, 64, 576]
  const int32_t* block_table;   // [B, max_pages]
  const int32_t* seqlens;       // [B]
  const int32_t* split_offsets; // [B+1] or nullptr (one chunk per sequence)
  int total_splits;
  int B, s_q, H;
  int max_pages;
  int num_pages;
  float scale;
  int causal;
  void* o_part;     // [total_splits, s_q, H, 512] in the output dtype when split, else nullptr
  float* lse_part;  // [total_splits, s_q, H]
  void* o_lat;      // [B, s_q, H, 512]; nullptr: write partials for every chunk
  float* lse;       // [B, s_q, H]; nullptr together with o_lat
  const int32_t* indices = nullptr;  // top-k decode: [B, s_q, topk] token positions
  int topk = 0;
  const float* row_scales = nullptr;  // FP8 cache: [num_pages, 64] fp32, one per cache row
  // Balanced schedule (bf16 dense decode only): [num_segments + 1] first
  // chunk of each segment, then [total_splits][4] = (b, first page, end
  // page, L_b) per chunk. nullptr: one chunk per workgroup, near-equal page
  // counts per sequence (split_offsets alone).
  const int32_t* schedule = nullptr;
  int num_segments = 0;
  int rows_per_group = kRowsPerGroup;  // 128, or 64 (two waves share each 32-row slice)
};

constexpr int kSparseMaxTopk = 2048;  // selected tokens per query token at most

// Chunk partials of a split decode placed by the caller: o_part [total_splits,
// s_q, H, 512] in the decode dtype and lse_part [total_splits, s_q, H] fp32.
struct PartialBuffers {
  void* o_part;
  float* lse_part;
  bool check_only;  // run the argument checks, launch nothing
};

// The decode entry points' shared body (argument checks, then the decode and,
// when outputs are given with split offsets, the merge). parts == nullptr:
// the partials live in the workspace (layout of mla_decode_workspace_size);
// otherwise in *parts and the workspace is not used.
mla_status_t run_decode(const void* q_lat, const void* kv_cache, const float* row_scales,
                        const int32_t* block_table, const int32_t* seqlens, const int32_t* indices, int topk,
                        const int32_t* split_offsets, int total_splits, int B, int s_q, int H, int d_qk,
                        int d_v, int page_size, int max_pages_per_seq, int num_pages, float softmax_scale,
                        int causal, mla_dtype_t dtype, void* workspace, size_t workspace_bytes, void* o_lat,
                        float* lse, void* stream, const PartialBuffers* parts, const int32_t* schedule = nullptr,
                        int num_segments = 0, int rows_per_group = 0);

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_fp32(const DecodeArgs& a, hipStream_t stream);
// Top-k decode (bf16, H = 128): the same kernel over gathered token rows.
hipError_t launch_sparse_decode_bf16(const DecodeArgs& a, hipStream_t stream);
// FP8 (e4m3) cache with per-row fp32 scales, bf16 queries and outputs.
hipError_t launch_decode_fp8(const DecodeArgs& a, hipStream_t stream);

// LSE merge. skip_single: sequences with one chunk were written directly by
// the decode kernel and are left alone.
// o_part holds the output dtype (bf16 when out_bf16, else fp32).
// Sets (buf non-null) or clears the bf16 decode kernel's clock stamps on the
// current device (mla_decode_clock_probe).
hipError_t set_clock_probe(uint64_t* buf, int cap);

hipError_t launch_combine(const void* o_part, const float* lse_part, const int32_t* split_offsets,
                          int total_splits, int B, int s_q, int H, bool out_bf16, bool skip_single,
                          void* o_lat, float* lse, hipStream_t stream);

}  // namespace mla

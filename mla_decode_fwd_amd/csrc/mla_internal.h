// Internal launch interfaces of the absorbed-MLA decode library (gfx950).
// The C ABI (include/mla_decode.h) validates arguments and then calls these.
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

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
};

constexpr int kSparseMaxTopk = 2048;  // selected tokens per query token at most

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_fp32(const DecodeArgs& a, hipStream_t stream);
// Top-k decode (bf16, H = 128): the same kernel over gathered token rows.
hipError_t launch_sparse_decode_bf16(const DecodeArgs& a, hipStream_t stream);
// FP8 (e4m3) cache with per-row fp32 scales, bf16 queries and outputs.
hipError_t launch_decode_fp8(const DecodeArgs& a, hipStream_t stream);

// Expanded path (bf16): per-head K [H, n_stride, 192] and V [H, n_stride, 128]
// for cached tokens t0 .. t0+n-1 of one sequence; causal attention of s_q new
// tokens over them; LSE merge of n_parts chunk partials of width 128.
hipError_t launch_expand(const void* cache, const int32_t* btab_row, int t0, int n, int num_pages, const void* w_uk,
                         const void* w_uv, int H, void* k_out, void* v_out, void* r_out, int n_stride,
                         hipStream_t stream);
hipError_t launch_prefill_attn(const void* q_nope, const void* q_rope, int s_q, int H, const void* K, const void* V,
                               const void* R, int n, int n_stride, int k_pos0, int q_pos0, int causal, float scale,
                               void* o, float* lse, hipStream_t stream);
// FP8 products for the absorption: per-tensor e4m3 quantisation of a bf16
// tensor (partials: kFp8QuantParts floats of scratch) and the per-head e4m3
// product out[n,h,j] = x_scale * w_scale * sum_k X[n,h,k] W[h,j,k].
constexpr int kFp8QuantParts = 256;
hipError_t launch_quantize_e4m3(const void* x, size_t n, float* partials, uint8_t* codes, float* scale,
                                hipStream_t stream);
// X is the bf16 activation, quantised inside (its partial maxima go to
// partials); two kernels on stream.
hipError_t launch_bmm_fp8(const void* X, float* partials, const uint8_t* W, float w_scale, int N, int H, int K, int J,
                          void* out, int out_stride, const void* tail_src, int tail, hipStream_t stream);
hipError_t launch_prefill_merge(const void* o_part, const float* lse_part, int n_parts, int rows, void* o, float* lse,
                                hipStream_t stream);

// LSE merge. skip_single: sequences with one chunk were written directly by
// the decode kernel and are left alone.
// o_part holds the output dtype (bf16 when out_bf16, else fp32).
hipError_t launch_combine(const void* o_part, const float* lse_part, const int32_t* split_offsets,
                          int total_splits, int B, int s_q, int H, bool out_bf16, bool skip_single,
                          void* o_lat, float* lse, hipStream_t stream);

// Per-head small-M products. absorb: out[n,h,0:dc] = A[n,h,:] . W[h,c,:] and
// the RoPE tail copied; out_uv: out[n,h,:] = A[n,h,:] . W[h,:,:].
hipError_t launch_absorb_q(const void* q_nope, const void* q_rope, const void* w_uk, int N, int H,
                           int dn, int dr, int dc, bool bf16, void* q_lat, hipStream_t stream);
hipError_t launch_out_uv(const void* o_lat, const void* w_uv, int N, int H, int dc, int dv,
                         bool bf16, void* out, hipStream_t stream);

}  // namespace mla

// Internal launch interfaces of the library's kernels outside the decode
// kernels: the expanded (prefill / extend) path, the per-head absorption
// products in bf16/fp32 and in FP8. The C ABI (include/mla_decode.h)
// validates arguments and then calls these.
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace mla {

// Expanded path (bf16): per-head K [H, n_stride, 128] and V [H, n_stride, 128]
// and the shared RoPE keys R [n_stride, 64] for cached tokens t0 .. t0+n-1 of
// one sequence; causal attention of s_q new tokens over them; LSE merge of
// n_parts chunk partials of width 128.
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

// Per-head small-M products. absorb: out[n,h,0:dc] = A[n,h,:] . W[h,c,:] and
// the RoPE tail copied; out_uv: out[n,h,:] = A[n,h,:] . W[h,:,:].
hipError_t launch_absorb_q(const void* q_nope, const void* q_rope, const void* w_uk, int N, int H,
                           int dn, int dr, int dc, bool bf16, void* q_lat, hipStream_t stream);
hipError_t launch_out_uv(const void* o_lat, const void* w_uv, int N, int H, int dc, int dv,
                         bool bf16, void* out, hipStream_t stream);

}  // namespace mla

// C ABI of the absorbed-MLA decode library: argument checks, split planning
// and kernel dispatch. Every check that the host can make runs before any HIP
// call, so a rejected call enqueues nothing.

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <vector>

#include "mla_decode.h"
#include "mla_internal.h"
#include "mla_launch_aux.h"

namespace {

constexpr int kMaxHeads = 128;
constexpr int kMaxSq = 16;
constexpr int kMaxBmmHeads = 1024;
constexpr int kMaxBmmDim = 4096;

mla_status_t from_hip(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_HIP; }

bool known_dtype(mla_dtype_t d) { return d == MLA_BF16 || d == MLA_FP32; }

size_t workspace_size(long long total_splits, long long s_q, long long H) {
  if (total_splits <= 0 || s_q <= 0 || H <= 0) return 0;
  const size_t rows = (size_t)total_splits * (size_t)s_q * (size_t)H;
  const size_t bytes = rows * (size_t)mla::kDv * sizeof(float) + rows * sizeof(float);
  return (bytes + 255) / 256 * 256;
}

}  // namespace

extern "C" {

const char* mla_status_string(mla_status_t status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARG: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case MLA_ERR_WORKSPACE: return "workspace missing or too small";
    case MLA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

int mla_abi_version(void) { return 8; }

size_t mla_decode_workspace_size(int total_splits, int s_q, int H) {
  return workspace_size(total_splits, s_q, H);
}

mla_status_t mla_decode_plan(const int32_t* seqlens_host, int B, int s_q, int H, int num_cus,
                             int max_splits, int32_t* num_splits_host,
                             int32_t* split_offsets_host, size_t* workspace_bytes) {
  if (!seqlens_host || !num_splits_host || !split_offsets_host) return MLA_ERR_INVALID_ARG;
  if (B <= 0 || s_q <= 0 || H <= 0) return MLA_ERR_INVALID_ARG;
  if (max_splits < 1 || max_splits > MLA_MAX_SPLITS) return MLA_ERR_INVALID_ARG;
  if (num_cus <= 0) num_cus = 256;
  long long total_pages = 0, max_pages = 0;
  for (int b = 0; b < B; ++b) {
    const long long L = seqlens_host[b];
    if (L < s_q) return MLA_ERR_INVALID_ARG;
    const long long P = (L + MLA_PAGE_SIZE - 1) / MLA_PAGE_SIZE;
    total_pages += P;
    if (P > max_pages) max_pages = P;
  }
  const long long row_groups = ((long long)s_q * H + mla::kRowsPerGroup - 1) / mla::kRowsPerGroup;
  // Pages per chunk: one wave of workgroups over the compute units, but no
  // finer than the split cap allows for the longest sequence.
  long long chunk = (total_pages * row_groups + num_cus - 1) / num_cus;
  const long long floor_by_cap = (max_pages + max_splits - 1) / max_splits;
  if (chunk < floor_by_cap) chunk = floor_by_cap;
  if (chunk < 1) chunk = 1;
  long long total = 0;
  bool any_split = false;
  split_offsets_host[0] = 0;
  for (int b = 0; b < B; ++b) {
    const long long P = ((long long)seqlens_host[b] + MLA_PAGE_SIZE - 1) / MLA_PAGE_SIZE;
    long long n = (P + chunk - 1) / chunk;
    if (n < 1) n = 1;
    if (n > max_splits) n = max_splits;
    if (n > 1) any_split = true;
    num_splits_host[b] = (int32_t)n;
    total += n;
    if (total > INT_MAX) return MLA_ERR_INVALID_ARG;
    split_offsets_host[b + 1] = (int32_t)total;
  }
  if (workspace_bytes) *workspace_bytes = any_split ? workspace_size(total, s_q, H) : 0;
  return MLA_OK;
}

size_t mla_decode_schedule_capacity(int B, int num_cus) {
  if (B <= 0) return 0;
  if (num_cus <= 0) num_cus = 256;
  // Segments <= num_cus; each segment boundary inside a sequence adds one
  // chunk, so chunks <= B + num_cus.
  return (size_t)num_cus + 1 + 4 * ((size_t)B + (size_t)num_cus);
}

mla_status_t mla_decode_schedule(const int32_t* seqlens_host, int B, int s_q, int H, int num_cus, int max_splits,
                                 int rows_per_group, int32_t* split_offsets_host, int32_t* schedule_host,
                                 size_t schedule_capacity, int* num_segments, int* rows_per_group_out,
                                 size_t* workspace_bytes) {
  if (!seqlens_host || !split_offsets_host || !schedule_host || !num_segments || !rows_per_group_out)
    return MLA_ERR_INVALID_ARG;
  if (B <= 0 || s_q <= 0 || H <= 0) return MLA_ERR_INVALID_ARG;
  if (max_splits < 1 || max_splits > MLA_MAX_SPLITS) return MLA_ERR_INVALID_ARG;
  if (rows_per_group != 0 && rows_per_group != 64 && rows_per_group != 128) return MLA_ERR_INVALID_ARG;
  if (num_cus <= 0) num_cus = 256;
  if (num_cus > 65536) return MLA_ERR_INVALID_ARG;
  long long total_pages = 0, max_pages = 0;
  for (int b = 0; b < B; ++b) {
    const long long L = seqlens_host[b];
    if (L < s_q) return MLA_ERR_INVALID_ARG;
    const long long P = (L + MLA_PAGE_SIZE - 1) / MLA_PAGE_SIZE;
    total_pages += P;
    if (P > max_pages) max_pages = P;
  }
  if (total_pages > INT_MAX / 2) return MLA_ERR_INVALID_ARG;
  const long long rows = (long long)s_q * H;
  // Chunks of sequence b for segments of `seg` pages laid end to end over the
  // concatenated pages: the segments overlapping [S_b, S_b + P_b).
  const auto max_chunks = [&](long long seg) {
    long long start = 0, worst = 0;
    for (int b = 0; b < B; ++b) {
      const long long P = ((long long)seqlens_host[b] + MLA_PAGE_SIZE - 1) / MLA_PAGE_SIZE;
      const long long n = (start + P - 1) / seg - start / seg + 1;
      if (n > worst) worst = n;
      start += P;
    }
    return worst;
  };
  // Candidate row-group sizes. A 64-row group halves the rows a workgroup
  // holds, so twice as many workgroups share each page range and the
  // segments are twice as long for the same number of workgroups; it is
  // taken when the chunk cap would otherwise leave compute units idle, and
  // its per-page cost is taken as 0.6 of a 128-row group's (two waves share
  // each page tile's rows and merge at the end).
  long long best_seg = 0;
  int best_rpg = 0;
  double best_cost = 0.0;
  for (int rpg : {128, 64}) {
    if (rows_per_group != 0 && rpg != rows_per_group) continue;
    const long long groups = (rows + rpg - 1) / rpg;
    long long G = num_cus / groups;
    if (G < 1) G = 1;
    long long seg = (total_pages + G - 1) / G;
    if (seg < 1) seg = 1;
    if (max_splits == 1) {
      seg = -1;  // one chunk per sequence: segments are the sequences
    } else if (max_chunks(seg) > max_splits) {
      // The chunk cap binds: lengthen the segments until it holds
      // (ceil(P / seg) + 1 segments can overlap a sequence).
      long long lo = seg, hi = (max_pages + max_splits - 2) / (max_splits - 1);
      if (hi < lo) hi = lo;
      while (lo < hi) {
        const long long mid = lo + (hi - lo) / 2;
        if (max_chunks(mid) <= max_splits) hi = mid; else lo = mid + 1;
      }
      seg = lo;
    }
    const double per_page = rpg == 128 ? 1.0 : 0.6;
    const double cost = (seg < 0 ? (double)max_pages : (double)seg) * per_page;
    if (best_rpg == 0 || cost < best_cost) {
      best_cost = cost;
      best_seg = seg;
      best_rpg = rpg;
    }
  }
  // Segment ends (global page offsets). Every chunk costs a workgroup a
  // fixed prologue and finalize besides its pages (measured on MI355X: one
  // more chunk in a workgroup adds about as much time as kChunkPages pages),
  // so segments are cut to equal cost, pages + kChunkPages * chunks, rather
  // than to equal pages: the smallest cost bound T for which a greedy walk
  // over the concatenated pages needs at most G segments and cuts no
  // sequence into more than max_splits chunks. With uniform lengths that
  // divide evenly this gives the equal segments; with mixed lengths
  // segments that start or cross more sequences get fewer pages.
  std::vector<int64_t> P(B);
  for (int b = 0; b < B; ++b) P[b] = ((long long)seqlens_host[b] + MLA_PAGE_SIZE - 1) / MLA_PAGE_SIZE;
  std::vector<int64_t> ends;
  if (best_seg < 0) {
    long long acc = 0;
    for (int b = 0; b < B; ++b) ends.push_back(acc += P[b]);  // one segment per sequence
  } else {
    const double kChunkPages = best_rpg == 128 ? 2.0 : 3.4;
    const long long groups = (rows + best_rpg - 1) / best_rpg;
    const long long G = num_cus / groups >= 1 ? num_cus / groups : 1;
    // Greedy walk under bound T: segment count, and (if out) the ends; false
    // if some sequence gets more than max_splits chunks.
    const auto walk = [&](double T, long long* n_segs, std::vector<int64_t>* out) {
      long long segs = 0, pos = 0, chunks_b = 0;
      int b = 0;
      long long off = 0;  // pages of sequence b already taken
      while (b < B) {
        double cost = 0.0;
        ++segs;
        for (;;) {
          const long long left = P[b] - off;
          const double room = T - cost - kChunkPages;
          if (cost > 0.0 && room < 1.0) break;  // no room for another chunk
          const long long take = room >= (double)left ? left : (room >= 1.0 ? (long long)room : 1);
          cost += kChunkPages + (double)take;
          pos += take;
          off += take;
          ++chunks_b;
          if (off == P[b]) {
            if (chunks_b > max_splits) return false;
            ++b;
            off = 0;
            chunks_b = 0;
            if (b == B) break;
          } else {
            break;  // the segment ends inside sequence b
          }
        }
        if (out) out->push_back(pos);
      }
      *n_segs = segs;
      return true;
    };
    // Bisection on T between a bound that needs too many segments (or
    // breaks the cap) and one that holds: the equal segments' cost.
    double lo = 0.0, hi = (double)best_seg + kChunkPages * (double)(B + 1) + 1.0;
    long long n = 0;
    if (!walk(hi, &n, nullptr) || n > G) hi = (double)total_pages + kChunkPages * (double)B + 1.0;
    for (int it = 0; it < 60; ++it) {
      const double mid = 0.5 * (lo + hi);
      if (walk(mid, &n, nullptr) && n <= G) hi = mid; else lo = mid;
    }
    if (walk(hi, &n, &ends) && n <= G) {
      // cost-balanced ends
    } else {
      ends.clear();  // fall back to the equal segments
      for (long long e = best_seg; ; e += best_seg) {
        ends.push_back(e < total_pages ? e : total_pages);
        if (e >= total_pages) break;
      }
    }
  }
  // Build the chunks in the global page order (sequence-major): the pieces
  // of each sequence between segment ends.
  const size_t need_segs = ends.size();
  long long total_chunks = 0;
  {
    long long start = 0;
    size_t e = 0;
    for (int b = 0; b < B; ++b) {
      const long long stop = start + P[b];
      while (e < ends.size() && ends[e] <= start) ++e;
      size_t f = e;
      long long n_b = 1;
      while (f < ends.size() && ends[f] < stop) { ++n_b; ++f; }
      total_chunks += n_b;
      start = stop;
    }
  }
  if (total_chunks > INT_MAX / 4) return MLA_ERR_INVALID_ARG;
  if (need_segs + 1 + 4 * (size_t)total_chunks > schedule_capacity) return MLA_ERR_WORKSPACE;
  int32_t* seg_first = schedule_host;             // [segments + 1]
  int32_t* desc = schedule_host + need_segs + 1;  // [chunks][4]: b, first page, end page, L_b
  long long c = 0, start = 0;
  size_t e = 0;  // first segment whose end lies past the current page
  seg_first[0] = 0;
  size_t s = 0;  // segments whose chunk lists are closed
  split_offsets_host[0] = 0;
  for (int b = 0; b < B; ++b) {
    long long p = 0;
    while (p < P[b]) {
      while (e < ends.size() && ends[e] <= start + p) ++e;
      // Segment e holds page start + p: every segment before it is complete.
      while (s < e) seg_first[++s] = (int32_t)c;
      const long long seg_end = e < ends.size() ? ends[e] - start : P[b];
      const long long q = seg_end < P[b] ? seg_end : P[b];
      desc[4 * c + 0] = b;
      desc[4 * c + 1] = (int32_t)p;
      desc[4 * c + 2] = (int32_t)q;
      desc[4 * c + 3] = seqlens_host[b];
      ++c;
      p = q;
    }
    split_offsets_host[b + 1] = (int32_t)c;
    start += P[b];
  }
  while (s < need_segs) seg_first[++s] = (int32_t)c;
  *num_segments = (int)need_segs;
  *rows_per_group_out = best_rpg;
  if (workspace_bytes) *workspace_bytes = workspace_size(total_chunks, s_q, H);
  return MLA_OK;
}

}  // extern "C"

namespace mla {

// Shared by the dense, top-k and FP8 entry points (indices == nullptr: dense)
// and by the entry point without a workspace (parts != nullptr: the chunk
// partials go to parts->o_part / parts->lse_part, already sized by the
// caller, instead of the workspace).
mla_status_t run_decode(const void* q_lat, const void* kv_cache, const float* row_scales,
                        const int32_t* block_table, const int32_t* seqlens, const int32_t* indices, int topk,
                        const int32_t* split_offsets, int total_splits, int B, int s_q, int H, int d_qk,
                        int d_v, int page_size, int max_pages_per_seq, int num_pages, float softmax_scale,
                        int causal, mla_dtype_t dtype, void* workspace, size_t workspace_bytes, void* o_lat,
                        float* lse, void* stream, const PartialBuffers* parts, const int32_t* schedule,
                        int num_segments, int rows_per_group) {
  if (!q_lat || !kv_cache || !block_table || !seqlens) return MLA_ERR_INVALID_ARG;
  // Partials only: no outputs, which needs split offsets and a workspace.
  const bool partials_only = !o_lat && !lse;
  if (!partials_only && (!o_lat || !lse)) return MLA_ERR_INVALID_ARG;
  if (partials_only && !split_offsets) return MLA_ERR_INVALID_ARG;
  if (B <= 0 || s_q <= 0 || H <= 0 || max_pages_per_seq <= 0 || num_pages <= 0)
    return MLA_ERR_INVALID_ARG;
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return MLA_ERR_INVALID_ARG;
  if (!known_dtype(dtype)) return MLA_ERR_UNSUPPORTED;
  if (d_qk != MLA_D_QK || d_v != MLA_D_V || page_size != MLA_PAGE_SIZE) return MLA_ERR_UNSUPPORTED;
  if (H > kMaxHeads || s_q > kMaxSq) return MLA_ERR_UNSUPPORTED;
  if ((long long)max_pages_per_seq * MLA_PAGE_SIZE > INT_MAX) return MLA_ERR_INVALID_ARG;
  if (split_offsets == nullptr) {
    if (total_splits != B) return MLA_ERR_INVALID_ARG;
  } else {
    if (total_splits < B || (long long)total_splits > (long long)B * MLA_MAX_SPLITS)
      return MLA_ERR_INVALID_ARG;
    if (!parts && (!workspace || workspace_bytes < workspace_size(total_splits, s_q, H))) return MLA_ERR_WORKSPACE;
  }
  if (schedule) {
    // Balanced schedule: bf16 dense decode only, with its own launch shape.
    if (!split_offsets) return MLA_ERR_INVALID_ARG;
    if (indices || row_scales || dtype != MLA_BF16) return MLA_ERR_UNSUPPORTED;
    if (rows_per_group != 64 && rows_per_group != 128) return MLA_ERR_INVALID_ARG;
    if (num_segments < 1 || num_segments > total_splits) return MLA_ERR_INVALID_ARG;
    const long long groups = ((long long)s_q * H + rows_per_group - 1) / rows_per_group;
    if (((long long)num_segments + 7) / 8 * 8 * groups > INT_MAX) return MLA_ERR_INVALID_ARG;
  }
  if (parts && parts->check_only) return MLA_OK;
  if (parts && (!parts->o_part || !parts->lse_part)) return MLA_ERR_INVALID_ARG;
  mla::DecodeArgs a{};
  a.q_lat = q_lat;
  a.kv_cache = kv_cache;
  a.block_table = block_table;
  a.seqlens = seqlens;
  a.split_offsets = split_offsets;
  a.total_splits = total_splits;
  a.B = B;
  a.s_q = s_q;
  a.H = H;
  a.max_pages = max_pages_per_seq;
  a.num_pages = num_pages;
  a.scale = softmax_scale;
  a.causal = causal ? 1 : 0;
  a.o_lat = o_lat;
  a.lse = lse;
  a.indices = indices;
  a.topk = topk;
  a.row_scales = row_scales;
  a.schedule = schedule;
  a.num_segments = num_segments;
  a.rows_per_group = schedule ? rows_per_group : mla::kRowsPerGroup;
  if (split_offsets && parts) {
    a.o_part = parts->o_part;
    a.lse_part = parts->lse_part;
  } else if (split_offsets) {
    const size_t rows = (size_t)total_splits * s_q * H;
    // The o_part region is sized for fp32 whatever the dtype, so the LSE
    // partials always start at the same byte offset.
    a.o_part = workspace;
    a.lse_part = reinterpret_cast<float*>(static_cast<char*>(workspace) + rows * mla::kDv * sizeof(float));
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = indices      ? mla::launch_sparse_decode_bf16(a, st)
                 : row_scales ? mla::launch_decode_fp8(a, st)
                 : (dtype == MLA_BF16 ? mla::launch_decode_bf16(a, st) : mla::launch_decode_fp32(a, st));
  if (e != hipSuccess) return MLA_ERR_HIP;
  if (split_offsets && !partials_only) {
    e = mla::launch_combine(a.o_part, a.lse_part, split_offsets, total_splits, B, s_q, H, dtype == MLA_BF16,
                            /*skip_single=*/true, o_lat, lse, st);
  }
  return from_hip(e);
}

}  // namespace mla

using mla::run_decode;

extern "C" {

mla_status_t mla_decode_fwd(const void* q_lat, const void* kv_cache, const int32_t* block_table,
                            const int32_t* seqlens, const int32_t* split_offsets,
                            int total_splits, int B, int s_q, int H, int d_qk, int d_v,
                            int page_size, int max_pages_per_seq, int num_pages,
                            float softmax_scale, int causal, mla_dtype_t dtype, void* workspace,
                            size_t workspace_bytes, void* o_lat, float* lse, void* stream) {
  return run_decode(q_lat, kv_cache, nullptr, block_table, seqlens, nullptr, 0, split_offsets, total_splits, B, s_q, H,
                    d_qk, d_v, page_size, max_pages_per_seq, num_pages, softmax_scale, causal, dtype, workspace,
                    workspace_bytes, o_lat, lse, stream, nullptr);
}

mla_status_t mla_decode_fwd_scheduled(const void* q_lat, const void* kv_cache, const int32_t* block_table,
                                      const int32_t* seqlens, const int32_t* split_offsets,
                                      const int32_t* schedule, int num_segments, int rows_per_group,
                                      int total_splits, int B, int s_q, int H, int d_qk, int d_v,
                                      int page_size, int max_pages_per_seq, int num_pages,
                                      float softmax_scale, int causal, mla_dtype_t dtype, void* workspace,
                                      size_t workspace_bytes, void* o_lat, float* lse, void* stream) {
  if (!schedule) return MLA_ERR_INVALID_ARG;
  return run_decode(q_lat, kv_cache, nullptr, block_table, seqlens, nullptr, 0, split_offsets, total_splits, B, s_q, H,
                    d_qk, d_v, page_size, max_pages_per_seq, num_pages, softmax_scale, causal, dtype, workspace,
                    workspace_bytes, o_lat, lse, stream, nullptr, schedule, num_segments, rows_per_group);
}

mla_status_t mla_sparse_decode_fwd(const void* q_lat, const void* kv_cache, const int32_t* block_table,
                                   const int32_t* seqlens, const int32_t* indices, int topk,
                                   const int32_t* split_offsets, int total_splits, int B, int s_q, int H,
                                   int d_qk, int d_v, int page_size, int max_pages_per_seq, int num_pages,
                                   float softmax_scale, mla_dtype_t dtype, void* workspace,
                                   size_t workspace_bytes, void* o_lat, float* lse, void* stream) {
  if (!indices) return MLA_ERR_INVALID_ARG;
  if (topk < 1 || topk > mla::kSparseMaxTopk) return MLA_ERR_UNSUPPORTED;
  if (!known_dtype(dtype)) return MLA_ERR_UNSUPPORTED;
  if (dtype != MLA_BF16 || H != mla::kRowsPerGroup) return MLA_ERR_UNSUPPORTED;
  return run_decode(q_lat, kv_cache, nullptr, block_table, seqlens, indices, topk, split_offsets, total_splits, B, s_q,
                    H, d_qk, d_v, page_size, max_pages_per_seq, num_pages, softmax_scale, /*causal=*/0, dtype,
                    workspace, workspace_bytes, o_lat, lse, stream, nullptr);
}

mla_status_t mla_decode_fwd_fp8(const void* q_lat, const void* kv_cache_e4m3, const float* row_scales,
                                const int32_t* block_table, const int32_t* seqlens, const int32_t* split_offsets,
                                int total_splits, int B, int s_q, int H, int d_qk, int d_v, int page_size,
                                int max_pages_per_seq, int num_pages, float softmax_scale, int causal,
                                void* workspace, size_t workspace_bytes, void* o_lat, float* lse, void* stream) {
  if (!row_scales) return MLA_ERR_INVALID_ARG;
  return run_decode(q_lat, kv_cache_e4m3, row_scales, block_table, seqlens, nullptr, 0, split_offsets, total_splits,
                    B, s_q, H, d_qk, d_v, page_size, max_pages_per_seq, num_pages, softmax_scale, causal, MLA_BF16,
                    workspace, workspace_bytes, o_lat, lse, stream, nullptr);
}

// ---- expanded path (prefill / extend) ----

namespace {
constexpr int kPrefillMaxChunks = 64;
constexpr int kPrefillMaxChunkTokens = 65536;  // the expansion keeps one range's page ids in LDS
size_t align256(size_t x) { return (x + 255) / 256 * 256; }
// Expanded keys K [H, chunk, 128] and values V [H, chunk, 128], and the
// chunk's RoPE keys R [chunk, 64] that every head shares.
size_t prefill_kv_bytes(int H, int chunk) { return align256((size_t)H * chunk * (128 + 128) * 2 + (size_t)chunk * 64 * 2); }
}  // namespace

size_t mla_prefill_workspace_size(int s_q, int H, int chunk_tokens, int max_chunks) {
  if (s_q <= 0 || H <= 0 || chunk_tokens <= 0 || max_chunks <= 0) return 0;
  const size_t parts = (size_t)max_chunks * s_q * H;
  return prefill_kv_bytes(H, chunk_tokens) + align256(parts * 128 * 2) + align256(parts * 4);
}

int mla_select_path(int s_q, int L) {
  if (s_q <= 0 || L < s_q) return -1;
  // FLOPs of the two paths for s_q new tokens over L keys at the DeepSeek-V3
  // shape (H cancels): expansion per key e and absorption per query b are
  // both d_c (d_nope + d_v) multiply-adds; per (query, key) pair the
  // absorbed path costs 2 d_c + d_rope and the expanded d_nope + d_rope + d_v.
  const double e = 512.0 * 256.0, b = e, p_abs = 1088.0, p_exp = 320.0;
  const double pairs = (double)s_q * L - (double)s_q * (s_q - 1) / 2.0;
  const double absorbed = s_q * b + pairs * p_abs, expanded = L * e + pairs * p_exp;
  return expanded < absorbed ? 1 : 0;
}

mla_status_t mla_prefill_fwd(const void* q_nope, const void* q_rope, const void* kv_cache, const int32_t* block_table,
                             const int32_t* seqlens_host, int B, int s_q, int H, int max_pages_per_seq, int num_pages,
                             const void* w_uk, const void* w_uv, int chunk_tokens, float softmax_scale,
                             void* workspace, size_t workspace_bytes, void* o, float* lse, void* stream) {
  if (!q_nope || !q_rope || !kv_cache || !block_table || !seqlens_host || !w_uk || !w_uv || !o || !lse)
    return MLA_ERR_INVALID_ARG;
  if (B <= 0 || s_q <= 0 || H <= 0 || H > kMaxHeads || max_pages_per_seq <= 0 || num_pages <= 0 || chunk_tokens <= 0)
    return MLA_ERR_INVALID_ARG;
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return MLA_ERR_INVALID_ARG;
  if (chunk_tokens > kPrefillMaxChunkTokens) return MLA_ERR_UNSUPPORTED;
  int max_chunks = 1;
  for (int b = 0; b < B; ++b) {
    const long long L = seqlens_host[b];
    if (L < s_q || L > (long long)max_pages_per_seq * MLA_PAGE_SIZE) return MLA_ERR_INVALID_ARG;
    const long long n = (L + chunk_tokens - 1) / chunk_tokens;
    if (n > kPrefillMaxChunks) return MLA_ERR_UNSUPPORTED;
    if (n > max_chunks) max_chunks = (int)n;
  }
  const size_t need = mla_prefill_workspace_size(s_q, H, chunk_tokens, max_chunks);
  if (!workspace || workspace_bytes < need) return MLA_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  void* K = ws;
  void* V = ws + (size_t)H * chunk_tokens * 128 * 2;
  void* R = ws + (size_t)H * chunk_tokens * 256 * 2;
  const size_t parts = (size_t)max_chunks * s_q * H;
  char* o_part = ws + prefill_kv_bytes(H, chunk_tokens);
  float* lse_part = reinterpret_cast<float*>(o_part + align256(parts * 128 * 2));
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t q_rows = (size_t)s_q * H;
  for (int b = 0; b < B; ++b) {
    const int L = seqlens_host[b];
    const int n_chunks = (L + chunk_tokens - 1) / chunk_tokens;
    const char* qn = static_cast<const char*>(q_nope) + (size_t)b * q_rows * 128 * 2;
    const char* qr = static_cast<const char*>(q_rope) + (size_t)b * q_rows * 64 * 2;
    char* ob = static_cast<char*>(o) + (size_t)b * q_rows * 128 * 2;
    float* lb = lse + (size_t)b * q_rows;
    for (int c = 0; c < n_chunks; ++c) {
      const int t0 = c * chunk_tokens;
      const int n = L - t0 < chunk_tokens ? L - t0 : chunk_tokens;
      hipError_t e = mla::launch_expand(kv_cache, block_table + (size_t)b * max_pages_per_seq, t0, n, num_pages, w_uk,
                                        w_uv, H, K, V, R, chunk_tokens, st);
      if (e != hipSuccess) return MLA_ERR_HIP;
      void* od = n_chunks == 1 ? static_cast<void*>(ob) : static_cast<void*>(o_part + (size_t)c * q_rows * 128 * 2);
      float* ld = n_chunks == 1 ? lb : lse_part + (size_t)c * q_rows;
      e = mla::launch_prefill_attn(qn, qr, s_q, H, K, V, R, n, chunk_tokens, t0, L - s_q, 1, softmax_scale, od, ld,
                                   st);
      if (e != hipSuccess) return MLA_ERR_HIP;
    }
    if (n_chunks > 1) {
      if (mla::launch_prefill_merge(o_part, lse_part, n_chunks, (int)q_rows, ob, lb, st) != hipSuccess)
        return MLA_ERR_HIP;
    }
  }
  return MLA_OK;
}

mla_status_t mla_splitkv_combine(const void* o_part, const float* lse_part,
                                 const int32_t* split_offsets, int total_splits, int B, int s_q,
                                 int H, int d_v, mla_dtype_t out_dtype, void* o_lat, float* lse,
                                 void* stream) {
  if (!o_part || !lse_part || !split_offsets || !o_lat || !lse) return MLA_ERR_INVALID_ARG;
  if (B <= 0 || s_q <= 0 || H <= 0) return MLA_ERR_INVALID_ARG;
  if (total_splits < B || (long long)total_splits > (long long)B * MLA_MAX_SPLITS)
    return MLA_ERR_INVALID_ARG;
  if (!known_dtype(out_dtype)) return MLA_ERR_UNSUPPORTED;
  if (d_v != MLA_D_V) return MLA_ERR_UNSUPPORTED;
  if ((long long)s_q * H > 65535LL * 4) return MLA_ERR_UNSUPPORTED;
  return from_hip(mla::launch_combine(o_part, lse_part, split_offsets, total_splits, B, s_q, H,
                                      out_dtype == MLA_BF16, /*skip_single=*/false, o_lat, lse,
                                      static_cast<hipStream_t>(stream)));
}

mla_status_t mla_absorb_q(const void* q_nope, const void* q_rope, const void* w_uk, int N, int H,
                          int d_nope, int d_rope, int d_c, mla_dtype_t dtype, void* q_lat,
                          void* stream) {
  if (!q_nope || !w_uk || !q_lat || (d_rope > 0 && !q_rope)) return MLA_ERR_INVALID_ARG;
  if (N <= 0 || H <= 0 || d_nope <= 0 || d_c <= 0 || d_rope < 0) return MLA_ERR_INVALID_ARG;
  if (!known_dtype(dtype)) return MLA_ERR_UNSUPPORTED;
  if (H > kMaxBmmHeads || d_nope > kMaxBmmDim || d_c > kMaxBmmDim || d_rope > kMaxBmmDim)
    return MLA_ERR_UNSUPPORTED;
  if ((long long)N > 65535LL * 64) return MLA_ERR_UNSUPPORTED;
  return from_hip(mla::launch_absorb_q(q_nope, q_rope, w_uk, N, H, d_nope, d_rope, d_c,
                                       dtype == MLA_BF16, q_lat, static_cast<hipStream_t>(stream)));
}

mla_status_t mla_out_uv(const void* o_lat, const void* w_uv, int N, int H, int d_c, int d_v,
                        mla_dtype_t dtype, void* out, void* stream) {
  if (!o_lat || !w_uv || !out) return MLA_ERR_INVALID_ARG;
  if (N <= 0 || H <= 0 || d_c <= 0 || d_v <= 0) return MLA_ERR_INVALID_ARG;
  if (!known_dtype(dtype)) return MLA_ERR_UNSUPPORTED;
  if (H > kMaxBmmHeads || d_c > kMaxBmmDim || d_v > kMaxBmmDim) return MLA_ERR_UNSUPPORTED;
  if ((long long)N > 65535LL * 64) return MLA_ERR_UNSUPPORTED;
  return from_hip(mla::launch_out_uv(o_lat, w_uv, N, H, d_c, d_v, dtype == MLA_BF16, out,
                                     static_cast<hipStream_t>(stream)));
}

// ---- FP8 products for the absorption ----

namespace {
constexpr size_t kFp8ScaleOff = (size_t)mla::kFp8QuantParts * 4;  // the partial maxima
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

mla_status_t quantize_into(const void* x, size_t n, void* workspace, uint8_t* codes, float* scale,
                           hipStream_t st) {
  return from_hip(mla::launch_quantize_e4m3(x, n, static_cast<float*>(workspace), codes, scale, st));
}
}  // namespace

size_t mla_fp8_workspace_size(size_t n_elems) {
  if (n_elems == 0) return 0;
  return kFp8ScaleOff;  // the partial maxima; the activation is quantised as the product loads it
}

mla_status_t mla_quantize_e4m3(const void* x, size_t n, void* workspace, size_t workspace_bytes, uint8_t* codes,
                               float* scale, void* stream) {
  if (!x || !codes || !scale || n == 0) return MLA_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(codes, 8)) return MLA_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < kFp8ScaleOff) return MLA_ERR_WORKSPACE;
  return quantize_into(x, n, workspace, codes, scale, static_cast<hipStream_t>(stream));
}

mla_status_t mla_absorb_q_fp8(const void* q_nope, const void* q_rope, const uint8_t* w_uk, float w_scale, int N,
                              int H, int d_nope, int d_rope, int d_c, void* workspace, size_t workspace_bytes,
                              void* q_lat, void* stream) {
  if (!q_nope || !w_uk || !q_lat || (d_rope > 0 && !q_rope)) return MLA_ERR_INVALID_ARG;
  if (N <= 0 || H <= 0 || d_nope <= 0 || d_c <= 0 || d_rope < 0) return MLA_ERR_INVALID_ARG;
  if (!std::isfinite(w_scale) || !(w_scale > 0.f)) return MLA_ERR_INVALID_ARG;
  if (H > kMaxBmmHeads || d_nope > kMaxBmmDim || d_c > kMaxBmmDim || d_rope > kMaxBmmDim) return MLA_ERR_UNSUPPORTED;
  if (d_nope % 16 || d_c % 4 || d_rope % 4) return MLA_ERR_UNSUPPORTED;
  if ((long long)N > 65535LL * 32) return MLA_ERR_UNSUPPORTED;
  if (!aligned(q_nope, 16) || !aligned(w_uk, 8) || !aligned(q_lat, 8)) return MLA_ERR_INVALID_ARG;
  const size_t n = (size_t)N * H * d_nope;
  if (!workspace || workspace_bytes < mla_fp8_workspace_size(n)) return MLA_ERR_WORKSPACE;
  return from_hip(mla::launch_bmm_fp8(q_nope, static_cast<float*>(workspace), w_uk, w_scale, N, H, d_nope, d_c,
                                      q_lat, d_c + d_rope, q_rope, d_rope, static_cast<hipStream_t>(stream)));
}

mla_status_t mla_out_uv_fp8(const void* o_lat, const uint8_t* w_uv_t, float w_scale, int N, int H, int d_c, int d_v,
                            void* workspace, size_t workspace_bytes, void* out, void* stream) {
  if (!o_lat || !w_uv_t || !out) return MLA_ERR_INVALID_ARG;
  if (N <= 0 || H <= 0 || d_c <= 0 || d_v <= 0) return MLA_ERR_INVALID_ARG;
  if (!std::isfinite(w_scale) || !(w_scale > 0.f)) return MLA_ERR_INVALID_ARG;
  if (H > kMaxBmmHeads || d_c > kMaxBmmDim || d_v > kMaxBmmDim) return MLA_ERR_UNSUPPORTED;
  if (d_c % 16 || d_v % 4) return MLA_ERR_UNSUPPORTED;
  if ((long long)N > 65535LL * 32) return MLA_ERR_UNSUPPORTED;
  if (!aligned(o_lat, 16) || !aligned(w_uv_t, 8) || !aligned(out, 8)) return MLA_ERR_INVALID_ARG;
  const size_t n = (size_t)N * H * d_c;
  if (!workspace || workspace_bytes < mla_fp8_workspace_size(n)) return MLA_ERR_WORKSPACE;
  return from_hip(mla::launch_bmm_fp8(o_lat, static_cast<float*>(workspace), w_uv_t, w_scale, N, H, d_c, d_v, out,
                                      d_v, nullptr, 0, static_cast<hipStream_t>(stream)));
}

mla_status_t mla_decode_clock_probe(uint64_t* device_buffer, int capacity) {
  if (device_buffer != nullptr && capacity < 0) return MLA_ERR_INVALID_ARG;
  return from_hip(mla::set_clock_probe(device_buffer, capacity));
}

}  // extern "C"

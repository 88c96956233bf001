/*
 * mla_decode.h - C ABI of the MI355X (gfx950) absorbed-MLA decode library.
 *
 * Multi-head Latent Attention decode on the weight-absorbed path. Every
 * query head attends to ONE shared 576-wide key per cached token (the
 * 512-wide latent c followed by the 64-wide decoupled RoPE key k^R) and ONE
 * shared 512-wide value (the latent c itself, i.e. the first 512 elements of
 * the same cache row).
 *
 * Sources (by page title and section):
 *   [MLA-推理]  "MLA 推理：两条计算路径与 FlashMLA"
 *               - section "两条等价的路径": the absorbed path. The query moves into
 *                 latent space (q~ = W_UK q^N), the score is q~ᵀc + q^Rᵀk^R, the
 *                 weighted sum stays in latent space and W_UV is applied last.
 *                 The cache row per token per layer is 512 + 64 numbers.
 *               - section "decode 注意力变成了计算问题": all heads share the key
 *                 and value (an MQA with a very wide head), paged KV with pages of
 *                 64 tokens, split-KV across compute units with a final merge of
 *                 the partial results.
 *               - section "谁快：看新 token 和缓存 token 的数量": new tokens follow
 *                 the cached ones and the cached count includes them (causal pairs
 *                 q*k - q(q-1)/2); chunk results are merged by their LSE.
 *   [DSV2-MLA]  "DeepSeekV2之MLA", section 4.5 (forward_absorb: bmm of q_nope with
 *               w_kc, attention as an MQA with a 576-wide key and 512-wide value,
 *               bmm of the attention output with w_vc).
 *   [AI-MTP]    "为什么 MLA + MTP 容易吃亏？从 Arithmetic Intensity 看 Attention",
 *               section 6: top-k sparse attention over gathered latents.
 *   [SGL-compile] "MLA 与 torch.compile：v0.3 的两个来源", the weight-absorption
 *               passage: with e4m3 weights w_kc / w_vc both per-head products
 *               run as bmm_fp8 of an activation quantised on the fly.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless the name ends in _host. All tensors
 *     are row-major and contiguous. The caller owns every buffer and the
 *     stream; the library allocates nothing, keeps no state between calls and
 *     may be called from several host threads at once.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). All
 *     device work is enqueued on it asynchronously; no call synchronizes.
 *   - Errors are reported only through the return code. All argument checks
 *     that the host can make run before any HIP call, so an invalid call
 *     enqueues nothing. A failed kernel launch returns MLA_ERR_HIP.
 *   - Device-side data (sequence lengths, block-table entries, split offsets)
 *     is not read by the host. Out-of-range values there give undefined
 *     results, but the kernels clamp every index they derive from them, so
 *     they never read or write outside the buffers the sizes describe.
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1, /* null pointer, negative or inconsistent size    */
  MLA_ERR_UNSUPPORTED = 2, /* valid but not implemented: dims, dtype, page   */
  MLA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required     */
  MLA_ERR_HIP = 4          /* a HIP launch or runtime call failed            */
} mla_status_t;

typedef enum {
  MLA_BF16 = 0, /* bf16 storage, fp32 accumulation, bf16 output (RNE)         */
  MLA_FP32 = 1  /* fp32 storage and arithmetic, fp32 output                   */
} mla_dtype_t;

/* Fixed shapes of the absorbed DeepSeek-V3 layout. */
#define MLA_D_QK 576      /* key width: 512 latent + 64 RoPE                  */
#define MLA_D_V 512       /* value width: the latent                          */
#define MLA_PAGE_SIZE 64  /* tokens per cache page                            */
#define MLA_MAX_SPLITS 64 /* most KV chunks one sequence may be split into    */

/* Human-readable name of a status code (static string, never NULL). */
const char* mla_status_string(mla_status_t status);

/* Library ABI version, currently 8 (2 added mla_sparse_decode_fwd, 3 mla_decode_fwd_fp8,
   4 the expanded path: mla_select_path, mla_prefill_workspace_size, mla_prefill_fwd,
   5 the FP8 products: mla_fp8_workspace_size, mla_quantize_e4m3, mla_absorb_q_fp8,
   mla_out_uv_fp8, 6 mla_decode_noalloc_scratch_bytes and mla_decode_fwd_noalloc, 7 the balanced
   schedule: mla_decode_schedule_capacity, mla_decode_schedule, mla_decode_fwd_scheduled,
   8 mla_decode_clock_probe). */
int mla_abi_version(void);

/*
 * Bytes of workspace mla_decode_fwd needs for `total_splits` work chunks:
 * fp32 partial outputs [total_splits, s_q, H, 512] followed by fp32 partial
 * LSEs [total_splits, s_q, H], rounded up to 256 bytes. Returns 0 for
 * non-positive sizes.
 */
size_t mla_decode_workspace_size(int total_splits, int s_q, int H);

/*
 * Split planner (host only, no HIP call).
 *
 * Chooses how many KV chunks each sequence is cut into ([MLA-推理] section
 * "decode 注意力变成了计算问题": long contexts and small batches are split along
 * the KV axis over the compute units). Chunks are whole pages. The plan
 * balances pages per workgroup over `num_cus` compute units: with P_b pages
 * in sequence b and R = ceil(s_q*H/128) row groups, it targets about one
 * wave of workgroups, giving each chunk close to sum(P_b)*R/num_cus pages,
 * capped at `max_splits` (<= 64) chunks per sequence and at P_b.
 *
 *   seqlens_host[B]      L_b, tokens cached for sequence b INCLUDING its s_q
 *                        new tokens; each must be >= s_q.
 *   num_cus              compute units to fill (256 on MI355X; <= 0 means 256).
 *   num_splits_host[B]   out: chunks per sequence, in [1, max_splits].
 *   split_offsets_host   out: [B+1] exclusive prefix sum of num_splits_host;
 *                        split_offsets_host[B] is total_splits.
 *   workspace_bytes      out (may be NULL): mla_decode_workspace_size of the
 *                        plan, or 0 when no sequence is split.
 */
mla_status_t mla_decode_plan(const int32_t* seqlens_host, int B, int s_q, int H, int num_cus,
                             int max_splits, int32_t* num_splits_host,
                             int32_t* split_offsets_host, size_t* workspace_bytes);

/*
 * Balanced schedule (host only, no HIP call): the analogue of the pages'
 * scheduling metadata ([MLA-推理] section "decode 注意力变成了计算问题":
 * get_mla_metadata decides which KV segments each compute unit processes, so
 * that every unit gets about the same work).
 *
 * The pages of all sequences are laid end to end (sequence 0 first) and cut
 * into contiguous segments, one per workgroup slot; a segment's intersection
 * with one sequence is a chunk (one partial of the LSE merge), so a segment
 * may cover the end of one sequence and the start of the next. Segments are
 * cut to equal cost, pages plus a fixed cost per chunk (2 pages for 128-row
 * groups, 3.4 half pages for 64-row groups: a chunk's prologue and finalize),
 * so a segment that holds more chunks gets fewer pages; uniform batches get
 * equal segments. A workgroup covers one row group of rows_per_group (query token,
 * head) rows: 128 (all heads of one new token), or 64, where two waves share
 * each 32-row slice and take one 32-token half of every page each, merging
 * their softmax states at the end. With R = ceil(s_q*H / rows_per_group) row
 * groups there are at most num_cus / R segments, each processed by R
 * workgroups at once. 64-row groups are chosen when the chunk cap
 * (max_splits per sequence) would otherwise leave compute units idle: with
 * them each segment holds twice the pages of half the rows. If the cap
 * still binds, the cost bound rises until no sequence is cut into more than
 * max_splits chunks.
 *
 *   seqlens_host[B]     L_b, each >= s_q (the same values as the device seqlens
 *                       passed to mla_decode_fwd_scheduled).
 *   num_cus             compute units (<= 0: 256).   max_splits: 1..64.
 *   rows_per_group      0 (choose), 64 or 128 (force).
 *   split_offsets_host  out [B+1]: chunks of sequence b are
 *                       split_offsets_host[b] .. [b+1]-1 (the merge layout).
 *   schedule_host       out: [num_segments + 1] first chunk of each segment,
 *                       then [total_splits][4] = (b, first page, end page, L_b)
 *                       of every chunk. Needs at most
 *                       mla_decode_schedule_capacity(B, num_cus) int32 entries;
 *                       schedule_capacity smaller than what the plan needs is
 *                       MLA_ERR_WORKSPACE.
 *   num_segments, rows_per_group_out   out: launch shape for the decode.
 *   workspace_bytes     out (may be NULL): mla_decode_workspace_size of the plan.
 */
size_t mla_decode_schedule_capacity(int B, int num_cus);
mla_status_t mla_decode_schedule(const int32_t* seqlens_host, int B, int s_q, int H, int num_cus,
                                 int max_splits, int rows_per_group, int32_t* split_offsets_host,
                                 int32_t* schedule_host, size_t schedule_capacity, int* num_segments,
                                 int* rows_per_group_out, size_t* workspace_bytes);

/*
 * Absorbed-MLA decode: o_lat and LSE for every (sequence, new token, head).
 *
 * For sequence b with L_b cached tokens (counting its s_q new ones, which
 * are the last s_q), query token i in [0, s_q) and head h:
 *   K_j = kv_cache[block_table[b, j/64], j%64, 0:576]     (key of token j)
 *   V_j = K_j[0:512]                                      (value of token j)
 *   allowed keys: j < L_b, and j <= L_b - s_q + i if causal
 *   s_j = softmax_scale * sum_k q_lat[b,i,h,k] * K_j[k]
 *   o_lat[b,i,h,:] = sum_j softmax(s)_j * V_j
 *   lse[b,i,h]     = ln sum_j exp(s_j)         (natural log)
 * ([MLA-推理] sections "两条等价的路径" and "decode 注意力变成了计算问题";
 *  softmax_scale is 1/sqrt(d_nope + d_rope) = 1/sqrt(192) for DeepSeek-V3;
 *  it must be finite and > 0.)
 *
 *   q_lat            [B, s_q, H, 576] dtype; q_lat[...,0:512] = W_UK q^N,
 *                    q_lat[...,512:576] = RoPE(q^R) (see mla_absorb_q).
 *   kv_cache         [num_pages, 64, 576] dtype; row = [c (512) ; k^R (64)],
 *                    k^R already rotated. Slots no sequence owns never affect
 *                    the result (the tail of a last page may be loaded, then ignored).
 *   block_table      [B, max_pages_per_seq] int32 physical page ids; entries
 *                    past ceil(L_b/64) are never read. Pages may sit anywhere
 *                    in the pool and in any order.
 *   seqlens          [B] int32 L_b (device), each in [s_q, 64*max_pages_per_seq].
 *   split_offsets    [B+1] int32 (device) from mla_decode_plan, or NULL for one
 *                    chunk per sequence. Sequence b is cut into
 *                    n_b = split_offsets[b+1]-split_offsets[b] page-aligned
 *                    chunks of near-equal page counts.
 *   total_splits     split_offsets[B] (host copy), or B when split_offsets is NULL.
 *   d_qk, d_v        must be 576 and 512.  page_size must be 64.
 *   H                heads, 1..128.  s_q: new tokens per sequence, 1..16.
 *   causal           nonzero: bottom-right causal mask among the s_q new tokens.
 *   workspace        device scratch of at least
 *                    mla_decode_workspace_size(total_splits, s_q, H) bytes when
 *                    split_offsets != NULL (may be NULL otherwise). Its contents
 *                    on entry are ignored; on return it holds the per-chunk
 *                    partials in mla_splitkv_combine's input layout: o_part
 *                    (in the decode dtype) at byte 0, lse_part (fp32) at byte
 *                    total_splits*s_q*H*512*4 for either dtype.
 *   o_lat            out [B, s_q, H, 512] dtype.
 *   lse              out [B, s_q, H] fp32 (natural log).
 *                    o_lat and lse may both be NULL when split_offsets is
 *                    given: then only the per-chunk partials are written (for
 *                    every chunk, including sequences with one chunk) and no
 *                    merge runs; mla_splitkv_combine on the workspace finishes
 *                    the job. One of the two NULL is MLA_ERR_INVALID_ARG.
 * Concurrent calls that share a workspace race; give each its own.
 */
mla_status_t mla_decode_fwd(const void* q_lat, const void* kv_cache, const int32_t* block_table,
                            const int32_t* seqlens, const int32_t* split_offsets,
                            int total_splits, int B, int s_q, int H, int d_qk, int d_v,
                            int page_size, int max_pages_per_seq, int num_pages,
                            float softmax_scale, int causal, mla_dtype_t dtype, void* workspace,
                            size_t workspace_bytes, void* o_lat, float* lse, void* stream);

/*
 * mla_decode_fwd with a split plan but without a workspace, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. The call allocates nothing (no
 * hipMalloc, no hipFree, no allocating library routine); the chunk partials
 * go to a static device array of MLA_NOALLOC_SCRATCH_BYTES that each GPU the
 * library runs on holds from the first call on it until the process ends.
 *
 * Arguments and results are those of mla_decode_fwd, except:
 *   - there is no workspace, and o_lat and lse are required (no
 *     partials-only mode: the partials stay in the library's array);
 *   - the partials need mla_decode_noalloc_scratch_bytes(total_splits, s_q,
 *     H, dtype) bytes; above MLA_NOALLOC_SCRATCH_BYTES the call returns
 *     MLA_ERR_WORKSPACE (e.g. bf16, H = 128, s_q = 1 allows up to 510
 *     chunks: the B = 64 x 4096 plan of 256 chunks fits);
 *   - `stream` must belong to the current device (else MLA_ERR_INVALID_ARG);
 *     the first call on a device looks up that device's copy of the array
 *     (MLA_ERR_HIP if that fails).
 * With split_offsets == NULL it is mla_decode_fwd without a workspace.
 * Every call on one GPU uses the same array and leaves the last call's
 * partials in it (nothing needs clearing: every chunk writes its whole
 * partial before the merge reads it). Calls that overlap in time on one GPU,
 * on any streams or host threads, race on the array: serialize them.
 */
#define MLA_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
size_t mla_decode_noalloc_scratch_bytes(int total_splits, int s_q, int H, mla_dtype_t dtype);
mla_status_t mla_decode_fwd_noalloc(const void* q_lat, const void* kv_cache, const int32_t* block_table,
                                    const int32_t* seqlens, const int32_t* split_offsets, int total_splits,
                                    int B, int s_q, int H, int d_qk, int d_v, int page_size,
                                    int max_pages_per_seq, int num_pages, float softmax_scale, int causal,
                                    mla_dtype_t dtype, void* o_lat, float* lse, void* stream);

/*
 * mla_decode_fwd under a balanced schedule from mla_decode_schedule (bf16
 * only): the same results, with the work laid out by the schedule instead of
 * cut into near-equal chunks per sequence. split_offsets (device, [B+1]) and
 * schedule (device, the schedule_host entries) are the planner's outputs
 * copied to the device; num_segments, rows_per_group (64 or 128) and
 * total_splits = split_offsets[B] come from the planner on the host. The
 * workspace needs mla_decode_workspace_size(total_splits, s_q, H) bytes and
 * holds the partials in the same layout; o_lat = lse = NULL writes only the
 * partials. dtype must be MLA_BF16 (else MLA_ERR_UNSUPPORTED); every other
 * argument and error is as for mla_decode_fwd. Chunk descriptors are
 * clamped to the sequence and the page table, so an inconsistent schedule
 * gives wrong results but never reads or writes outside the buffers.
 */
mla_status_t mla_decode_fwd_scheduled(const void* q_lat, const void* kv_cache, const int32_t* block_table,
                                      const int32_t* seqlens, const int32_t* split_offsets,
                                      const int32_t* schedule, int num_segments, int rows_per_group,
                                      int total_splits, int B, int s_q, int H, int d_qk, int d_v,
                                      int page_size, int max_pages_per_seq, int num_pages,
                                      float softmax_scale, int causal, mla_dtype_t dtype, void* workspace,
                                      size_t workspace_bytes, void* o_lat, float* lse, void* stream);

/*
 * Top-k (sparse) absorbed-MLA decode ([AI-MTP] section 6 "Sparse attention
 * 把方向反过来": a selector keeps index_topk = 2048 history tokens per new
 * token; their latents are gathered by index and the scores and the weighted
 * sum run over those tokens only, so the cost follows topk, not L).
 * For sequence b, query token i and head h, with S = the entries e of
 * indices[b, i, 0:topk] that satisfy 0 <= e < L_b (the others are padding),
 * taken in list order (a repeated entry counts once per occurrence):
 *   K_e = kv_cache[block_table[b, e/64], e%64, 0:576],  V_e = K_e[0:512]
 *   s_e = softmax_scale * sum_k q_lat[b,i,h,k] * K_e[k]          for e in S
 *   o_lat[b,i,h,:] = sum_e softmax(s)_e * V_e,  lse[b,i,h] = ln sum_e exp(s_e)
 * No causal mask: the list is the key set. A row with S empty gets o = 0 and
 * lse = -inf.
 *
 *   indices          [B, s_q, topk] int32 (device), logical token positions.
 *   topk             1..2048.
 *   H                must be 128 (one workgroup row group per new token);
 *                    dtype must be MLA_BF16 (else MLA_ERR_UNSUPPORTED).
 *   seqlens          [B] int32 L_b (device), each in [1, 64*max_pages_per_seq];
 *                    the rows of positions 0..L_b-1 must hold finite values
 *                    (padding entries are loaded from position 0, then masked).
 *   split_offsets    as for mla_decode_fwd, but chunks cut the list: plan with
 *                    mla_decode_plan(seqlens_host = topk for every sequence).
 *   Every other argument, the workspace layout, the partials-only mode and
 *   the error behaviour are those of mla_decode_fwd (causal does not apply).
 */
mla_status_t mla_sparse_decode_fwd(const void* q_lat, const void* kv_cache, const int32_t* block_table,
                                   const int32_t* seqlens, const int32_t* indices, int topk,
                                   const int32_t* split_offsets, int total_splits, int B, int s_q, int H,
                                   int d_qk, int d_v, int page_size, int max_pages_per_seq, int num_pages,
                                   float softmax_scale, mla_dtype_t dtype, void* workspace,
                                   size_t workspace_bytes, void* o_lat, float* lse, void* stream);

/*
 * Absorbed-MLA decode on an FP8 latent cache ([MLA-推理] section "练习",
 * exercise 2: with the latent cache in FP8 a cached token is 576 bytes plus
 * its scale factors, which halves the bytes read per token and doubles the
 * arithmetic intensity to about 484 FLOP/byte). Each cache row holds 576
 * e4m3 codes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no
 * infinities, NaN = 0x7F/0xFF) and has one fp32 scale; its value is
 *   row = row_scales[page, slot] * e4m3(kv_cache_e4m3[page, slot, :]).
 * The result is mla_decode_fwd's on those row values (bf16 q_lat, bf16 o_lat,
 * fp32 LSE, same split, workspace and partials-only rules; partials in bf16).
 *
 *   kv_cache_e4m3    [num_pages, 64, 576] uint8 codes (device).
 *   row_scales       [num_pages, 64] fp32 (device). Rows no sequence owns may
 *                    hold anything, NaN included: they never reach a product.
 *   Every other argument as mla_decode_fwd with dtype MLA_BF16.
 * Compute: the codes are widened to bf16 on the chip (exactly), the bf16 MFMA
 * path runs with fp32 accumulation, and each row's scale multiplies its score
 * and, for the value, its P.
 */
mla_status_t mla_decode_fwd_fp8(const void* q_lat, const void* kv_cache_e4m3, const float* row_scales,
                                const int32_t* block_table, const int32_t* seqlens, const int32_t* split_offsets,
                                int total_splits, int B, int s_q, int H, int d_qk, int d_v, int page_size,
                                int max_pages_per_seq, int num_pages, float softmax_scale, int causal,
                                void* workspace, size_t workspace_bytes, void* o_lat, float* lse, void* stream);

/*
 * Path choice for s_q new tokens over L keys (L counting them)
 * ([MLA-推理] section "谁快：看新 token 和缓存 token 的数量" and [AI-MTP] 5.6):
 * 1 when the expanded path (mla_prefill_fwd) costs fewer FLOPs than the
 * absorbed one (mla_absorb_q + mla_decode_fwd + mla_out_uv) at the
 * DeepSeek-V3 shape (d_c 512, d_nope 128, d_rope 64, d_v 128), else 0;
 * -1 for s_q <= 0 or L < s_q. For L >> s_q the switch is at s_q ≈ 171.
 */
int mla_select_path(int s_q, int L);

/*
 * Workspace bytes of mla_prefill_fwd for chunks of chunk_tokens cached tokens
 * and at most max_chunks chunks per sequence: the expanded keys and values
 * of one chunk (H * chunk_tokens * (128 + 128) bf16, 64 KB per token at
 * H = 128), the chunk's RoPE keys, which every head shares
 * (chunk_tokens * 64 bf16), and the chunk partials
 * (max_chunks * s_q * H * (128 bf16 + 1 fp32)).
 * 0 for non-positive arguments.
 */
size_t mla_prefill_workspace_size(int s_q, int H, int chunk_tokens, int max_chunks);

/*
 * The expanded path (path one of [MLA-推理] "两条等价的路径") for prefill and
 * extend: the s_q new tokens of each sequence (the last s_q of its L_b
 * cached tokens, which the cache already holds) attend causally to all
 * L_b tokens through per-head keys and values expanded from the latent:
 *   k_j^h = [c_j W_UK[h] ; k^R_j],  v_j^h = c_j W_UV[h]
 *   s     = softmax_scale * ([q^N ; q^R] . k_j^h),  o^h = softmax(s) V^h
 * returning per-head outputs o [B, s_q, H, 128] (before W_o) and the
 * natural-log LSE [B, s_q, H]. The cached tokens are expanded
 * chunk_tokens at a time and the chunk results merged by their LSE
 * ([MLA-推理] "谁快": SGLang's MHA_CHUNKED_KV, threshold 8192 by default).
 *
 *   q_nope [B, s_q, H, 128], q_rope [B, s_q, H, 64] (rotated), bf16.
 *   kv_cache [num_pages, 64, 576] bf16 rows [c (512) ; k^R (64)];
 *   block_table [B, max_pages_per_seq] int32 (device);
 *   seqlens_host [B] (HOST) L_b in [s_q, 64 * max_pages_per_seq].
 *   w_uk, w_uv [H, 512, 128] bf16 (latent rows), as for mla_absorb_q/out_uv.
 *   1 <= chunk_tokens <= 65536 and at most 64 chunks per sequence (else
 *   UNSUPPORTED).
 *   H 1..128. softmax_scale finite and > 0 (1/sqrt(192) for DeepSeek-V3).
 *   workspace of at least mla_prefill_workspace_size(s_q, H, chunk_tokens,
 *   max over b of ceil(L_b / chunk_tokens)) bytes, contents ignored.
 * Launches two kernels per chunk and one merge per sequence on stream; the
 * host loop reads seqlens_host only.
 */
mla_status_t mla_prefill_fwd(const void* q_nope, const void* q_rope, const void* kv_cache, const int32_t* block_table,
                             const int32_t* seqlens_host, int B, int s_q, int H, int max_pages_per_seq, int num_pages,
                             const void* w_uk, const void* w_uv, int chunk_tokens, float softmax_scale,
                             void* workspace, size_t workspace_bytes, void* o, float* lse, void* stream);

/*
 * LSE merge of split-KV partial results ([MLA-推理] sections
 * "谁快：看新 token 和缓存 token 的数量" and "decode 注意力变成了计算问题":
 * the chunk results are merged by their log-sum-exp).
 * For each (b, i, h), over the n_b chunks k of sequence b:
 *   M = max_k lse_k;  lse = M + ln sum_k exp(lse_k - M);
 *   o = sum_k exp(lse_k - lse) * o_k
 * A chunk with lse_k = -inf (no allowed key) contributes nothing.
 *
 *   o_part     [total_splits, s_q, H, d_v] in out_dtype (bf16 partials for a
 *              bf16 output, fp32 for fp32), chunk-major: the chunks of
 *              sequence b are rows split_offsets[b] .. split_offsets[b+1]-1.
 *   lse_part   [total_splits, s_q, H] fp32, natural log.
 *   split_offsets [B+1] int32 (device), total_splits = split_offsets[B].
 *   d_v        must be 512.
 *   o_lat      out [B, s_q, H, d_v] in out_dtype;  lse: out [B, s_q, H] fp32.
 */
mla_status_t mla_splitkv_combine(const void* o_part, const float* lse_part,
                                 const int32_t* split_offsets, int total_splits, int B, int s_q,
                                 int H, int d_v, mla_dtype_t out_dtype, void* o_lat, float* lse,
                                 void* stream);

/*
 * Query absorption ([MLA-推理] section "两条等价的路径": q~ = W_UK q^N;
 * [DSV2-MLA] section 4.5: the bmm of q_nope with w_kc):
 *   q_lat[n,h,0:d_c]          = sum_d q_nope[n,h,d] * w_uk[h,c,d]
 *   q_lat[n,h,d_c:d_c+d_rope] = q_rope[n,h,:]   (already rotated; copied)
 *
 *   q_nope [N, H, d_nope], q_rope [N, H, d_rope], w_uk [H, d_c, d_nope]
 *   (the per-head latent-to-key matrix, latent rows), all in dtype;
 *   q_lat out [N, H, d_c + d_rope] in dtype. Accumulation is fp32.
 *   Sizes: N >= 1, 1 <= H <= 1024, 1 <= d_nope, d_c <= 4096, 0 <= d_rope <= 4096.
 */
mla_status_t mla_absorb_q(const void* q_nope, const void* q_rope, const void* w_uk, int N, int H,
                          int d_nope, int d_rope, int d_c, mla_dtype_t dtype, void* q_lat,
                          void* stream);

/*
 * Output un-absorption ([MLA-推理] section "两条等价的路径": W_UV is applied
 * after the weighted sum in latent space; [DSV2-MLA] section 4.5: the bmm of
 * the attention output with w_vc):
 *   out[n,h,e] = sum_c o_lat[n,h,c] * w_uv[h,c,e]
 *
 *   o_lat [N, H, d_c], w_uv [H, d_c, d_v], out [N, H, d_v], all in dtype;
 *   fp32 accumulation. Sizes: N >= 1, 1 <= H <= 1024, 1 <= d_c, d_v <= 4096.
 */
mla_status_t mla_out_uv(const void* o_lat, const void* w_uv, int N, int H, int d_c, int d_v,
                        mla_dtype_t dtype, void* out, void* stream);

/*
 * FP8 (e4m3) products for the absorption ([SGL-compile] "MLA 与 torch.compile：
 * v0.3 的两个来源", the weight-absorption passage: with FP8 weights w_kc and w_vc, both bmm's run as bmm_fp8 of an
 * activation quantised to e4m3 on the fly, one scale per tensor, against the
 * e4m3 weights and their scale, with a bf16 result).
 *
 * Codes are e4m3 "fn" (bias 7, no infinities, NaN 0x7F/0xFF, largest finite
 * 448). Per-tensor dynamic quantisation of a bf16 tensor x:
 *   r = 448 / max|x| (fp32; max|x| taken as at least 2^-100; r = 1 when x is
 *       all zero), code = nearest e4m3 value of the fp32 product x * r, ties
 *       to even, magnitudes clamped to 448; the dequantisation scale is
 *       s = 1 / r (fp32).
 */

/* Workspace bytes of mla_absorb_q_fp8 / mla_out_uv_fp8 for an activation of
   n_elems elements: the partial maxima of the per-tensor scale (1 KB; the
   products quantise the activation as they load it); 0 for 0. */
size_t mla_fp8_workspace_size(size_t n_elems);

/*
 * Per-tensor quantisation on its own: x [n] bf16 (16-byte aligned) ->
 * codes [n] uint8 (8-byte aligned) and *scale (one fp32, device). workspace:
 * at least 1 KB of device scratch (contents ignored). Two kernels on stream.
 */
mla_status_t mla_quantize_e4m3(const void* x, size_t n, void* workspace, size_t workspace_bytes, uint8_t* codes,
                               float* scale, void* stream);

/*
 * mla_absorb_q with FP8 operands:
 *   q_lat[n,h,0:d_c] = bf16( s * w_scale * sum_d e4m3(q_nope)[n,h,d] * w_uk[h,c,d] )
 *   q_lat[n,h,d_c:]  = q_rope[n,h,:]  (copied)
 * where q_nope is quantised per tensor as above.
 *   q_nope [N, H, d_nope] bf16 (16-byte aligned), q_rope [N, H, d_rope] bf16;
 *   w_uk [H, d_c, d_nope] e4m3 codes (8-byte aligned) with scale w_scale
 *   (host float, finite, > 0); q_lat out [N, H, d_c + d_rope] bf16 (8-byte aligned).
 *   d_nope a multiple of 16, d_c and d_rope multiples of 4; H <= 1024; dims <= 4096.
 *   workspace of at least mla_fp8_workspace_size(N * H * d_nope) bytes.
 */
mla_status_t mla_absorb_q_fp8(const void* q_nope, const void* q_rope, const uint8_t* w_uk, float w_scale, int N,
                              int H, int d_nope, int d_rope, int d_c, void* workspace, size_t workspace_bytes,
                              void* q_lat, void* stream);

/*
 * mla_out_uv with FP8 operands:
 *   out[n,h,e] = bf16( s * w_scale * sum_c e4m3(o_lat)[n,h,c] * w_uv_t[h,e,c] )
 * where o_lat is quantised per tensor as above and the weight is W_UV stored
 * transposed, [H, d_v, d_c] e4m3 codes (prepared once, as the pages' history
 * transposes the MLA weights offline), so that both operands run along d_c.
 *   o_lat [N, H, d_c] bf16 (16-byte aligned); out [N, H, d_v] bf16 (8-byte
 *   aligned). d_c a multiple of 16, d_v a multiple of 4; H <= 1024; dims <= 4096.
 *   workspace of at least mla_fp8_workspace_size(N * H * d_c) bytes.
 */
mla_status_t mla_out_uv_fp8(const void* o_lat, const uint8_t* w_uv_t, float w_scale, int N, int H, int d_c, int d_v,
                            void* workspace, size_t workspace_bytes, void* out, void* stream);

/*
 * A measurement aid, not part of the computation: the shader clock at which
 * the bf16 decode kernel runs (mla_decode_fwd and mla_decode_fwd_scheduled
 * with bf16 inputs, dense or top-k). While `device_buffer` is set, every
 * workgroup x < capacity of later launches on the current device writes two
 * uint64 words at device_buffer[2x]: the shader-clock cycles (s_memtime) and
 * the 100 MHz reference-clock ticks (s_memrealtime) from its start to its
 * end, so cycles / ticks * 100 MHz is the clock it ran at. Workgroups with no
 * work write nothing. device_buffer = NULL (capacity ignored) switches the
 * stamps off; the setting is per device and stays until changed. The caller
 * owns the buffer (device memory, 2 * capacity uint64 words) and keeps it
 * alive while the setting is on; launches already queued may or may not see
 * a change, so synchronize around it. capacity < 0 with a non-NULL buffer
 * gives MLA_ERR_INVALID_ARG.
 */
mla_status_t mla_decode_clock_probe(uint64_t* device_buffer, int capacity);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */

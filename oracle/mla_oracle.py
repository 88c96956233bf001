"""Plain fp64 CPU oracle for Multi-head Latent Attention (MLA) decode.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import or
call this module. The GPU library never imports it, and this module imports
nothing from the GPU library: the two share no code. Inputs reach both sides
from the seeded generators in ``mla_inputs``, which hold none of the method's
arithmetic.

Everything here is a direct, unblocked statement of what the pages define,
computed in float64 with numpy. There is no tiling, no online softmax and no
reordering beyond what each definition states.

Sources. Each citation names the page by its title and the section:
  [MLA-推理]  "MLA 推理：两条计算路径与 FlashMLA" (AI infra handbook, serving/moe/mla)
  [DSV2-MLA]  "DeepSeekV2之MLA" (blog post with the DeepSeek-V2 equations and SGLang code)
  [AI-MTP]    "为什么 MLA + MTP 容易吃亏？从 Arithmetic Intensity 看 Attention"
              (section 6 "Sparse attention 把方向反过来" for decode_sparse)
  [SGL-compile] "MLA 与 torch.compile：v0.3 的两个来源" (the weight-absorption
              passage: bmm_fp8 of an e4m3 activation against e4m3 w_kc / w_vc)

Function list and pins:
  rope_adjacent      RoPE on adjacent pairs                 pinned (rotation identities)
  project            hidden -> q_n, q_r, c, k_r             pinned (one-hot hidden rows read back
                                                            weight entries block by block; cos/sin
                                                            of t*theta along the tokens; rope
                                                            scores depend on t - s only)
  expanded_attention path one: per-head K, V, ordinary MHA  pinned (path equivalence, SDPA)
  mla_forward_*      both full tiny MLA paths to y          pinned (the page prints True; a
                                                            selector W_o picks head h, element d
                                                            at column h*DV + d)
  absorb_q           q_lat = [W_UK q^N ; q^R]               pinned (path equivalence)
  out_uv             o = o_lat W_UV[h]                      pinned (path equivalence)
  decode_absorbed    absorbed decode on a paged cache       pinned (brute force, SDPA, closed forms)
  decode_partials    the same over a token chunk            pinned (merge invariant)
  lse_merge          log-sum-exp merge of chunk results     pinned (merge == unsplit)
  decode_sparse      absorbed decode over top-k token lists pinned (full list == dense, brute
                                                            force, closed forms)
  e4m3_decode        FP8 (e4m3, no infinities) code -> value pinned (all 256 codes vs torch,
                                                            hand values)
  decode_absorbed_fp8 absorbed decode on an FP8 cache with  pinned (closed forms, the dequantised
                     one scale per token row                 cache through decode_absorbed)
  prefill_expanded   path one on a paged latent cache: new   pinned (== absorb_q + decode_absorbed
                     tokens after a prefix, per-head K, V    + out_uv; worked example)
  prefill_chunked    the same over prefix chunks + LSE merge pinned (== unchunked)
  crossover_tokens   new-token count where the paths' FLOPs  pinned (the chapter's printed 171)
                     cross, for a given key count
  e4m3_encode        value -> FP8 e4m3 code, nearest, ties   pinned (torch's float8_e4m3fn
                     to even, saturating at 448              conversion on every tie and a dense
                                                            sweep; round trip of all codes)
  quantize_e4m3      per-tensor dynamic quantisation: codes  pinned (max element -> 448, zero
                     of x * 448 / max|x|, scale max|x| / 448 tensor, exact inputs round-trip)
  absorb_q_fp8       absorb_q with an e4m3 query and e4m3    pinned (== absorb_q on exactly
                     weights, both scaled                    representable inputs)
  out_uv_fp8         out_uv with an e4m3 latent output and   pinned (== out_uv on exactly
                     e4m3 weights stored transposed          representable inputs)
No function is left without a pin.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "rope_adjacent",
    "project",
    "expanded_attention",
    "mla_forward_expanded",
    "mla_forward_absorbed",
    "absorb_q",
    "out_uv",
    "gather_tokens",
    "decode_absorbed",
    "decode_partials",
    "lse_merge",
    "decode_sparse",
    "e4m3_decode",
    "decode_absorbed_fp8",
    "prefill_expanded",
    "prefill_chunked",
    "crossover_tokens",
    "e4m3_encode",
    "quantize_e4m3",
    "absorb_q_fp8",
    "out_uv_fp8",
]


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# Full tiny MLA: the worked example of [MLA-推理] §"两条等价的路径".
# ---------------------------------------------------------------------------

def rope_adjacent(x, base: float = 10000.0) -> np.ndarray:
    """Rotary embedding that rotates adjacent element pairs by position.

    [MLA-推理] §"两条等价的路径", the worked example's ``rope``: the second-to-
    last axis of ``x`` is the position t = 0..T-1 and the last axis has R
    (even) elements. Pair i is (x[2i], x[2i+1]) and its angle is
    t / base**(2i/R). The rotated pair is (x1 cos - x2 sin, x1 sin + x2 cos),
    written back interleaved at the same two slots.
    """
    x = _f64(x)
    T, R = x.shape[-2], x.shape[-1]
    if R % 2:
        raise ValueError("RoPE width must be even")
    pos = np.arange(T, dtype=np.float64)[:, None]
    inv = base ** (np.arange(0, R, 2, dtype=np.float64) / R)
    ang = pos / inv  # [T, R/2]
    x1, x2 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x1 * np.cos(ang) - x2 * np.sin(ang)
    out[..., 1::2] = x1 * np.sin(ang) + x2 * np.cos(ang)
    return out


def project(h, W_q, W_dkv, W_kr, H: int, nope: int, rope_dim: int):
    """Projections of the worked example, [MLA-推理] §"两条等价的路径".

    c = h W_dkv (the cached latent), k_r = RoPE(h W_kr) (the RoPE key shared by
    all heads, cached beside c), q = h W_q viewed per head as [nope | rope],
    q_n = its first ``nope`` elements, q_r = RoPE of the remaining ones.

    Returns token-major arrays: q_n [T,H,nope], q_r [T,H,rope], c [T,DC],
    k_r [T,rope].
    """
    h = _f64(h)
    T = h.shape[0]
    c = h @ _f64(W_dkv)
    k_r = rope_adjacent(h @ _f64(W_kr))
    q = (h @ _f64(W_q)).reshape(T, H, nope + rope_dim)
    q_n = q[..., :nope]
    # RoPE runs over the position axis, so rotate in [H, T, rope] order.
    q_r = rope_adjacent(np.transpose(q[..., nope:], (1, 0, 2))).transpose(1, 0, 2)
    return q_n, q_r, c, k_r


def _masked_softmax_rows(s: np.ndarray, allowed: np.ndarray) -> np.ndarray:
    """Row softmax of s over the entries where ``allowed`` is true (two passes)."""
    s = np.where(allowed, s, -np.inf)
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def expanded_attention(q_n, q_r, c, k_r, W_uk, W_uv, causal: bool = True) -> np.ndarray:
    """Path one ("展开"): expand the latent per head, then ordinary MHA.

    [MLA-推理] §"两条等价的路径": k^N = c W_UK[h] per head, concatenated with the
    shared k^R; v = c W_UV[h]; scores use scale 1/sqrt(nope + rope); the mask
    is the lower-triangular causal mask over the T tokens.
    Shapes: q_n [T,H,nope], q_r [T,H,rope], c [T,DC], k_r [T,rope],
    W_uk [H,DC,nope], W_uv [H,DC,DV]. Returns per-head outputs [T,H,DV].
    """
    q_n, q_r, c, k_r = map(_f64, (q_n, q_r, c, k_r))
    W_uk, W_uv = _f64(W_uk), _f64(W_uv)
    T, H, nope = q_n.shape
    rope_dim = q_r.shape[-1]
    scale = 1.0 / math.sqrt(nope + rope_dim)
    k_nope = np.einsum("tc,hcd->htd", c, W_uk)  # [H,T,nope]
    k = np.concatenate([k_nope, np.broadcast_to(k_r, (H, T, rope_dim))], axis=-1)
    v = np.einsum("tc,hcd->htd", c, W_uv)  # [H,T,DV]
    q = np.concatenate([q_n, q_r], axis=-1).transpose(1, 0, 2)  # [H,T,nope+rope]
    s = (q @ k.transpose(0, 2, 1)) * scale  # [H,T,T]
    allowed = np.tril(np.ones((T, T), dtype=bool)) if causal else np.ones((T, T), dtype=bool)
    p = _masked_softmax_rows(s, allowed)
    return (p @ v).transpose(1, 0, 2)  # [T,H,DV]


def mla_forward_expanded(h, W_q, W_dkv, W_kr, W_uk, W_uv, W_o, H, nope, rope_dim, causal=True):
    """Full tiny MLA on path one, output projection included: y = out W_o.

    [MLA-推理] §"两条等价的路径" (worked example, ``out1`` and ``y1``).
    """
    q_n, q_r, c, k_r = project(h, W_q, W_dkv, W_kr, H, nope, rope_dim)
    out = expanded_attention(q_n, q_r, c, k_r, W_uk, W_uv, causal)
    T = out.shape[0]
    return out.reshape(T, -1) @ _f64(W_o)


def absorb_q(q_n, q_r, W_uk) -> np.ndarray:
    """Absorbed query q_lat = [W_UK q^N ; q^R].

    [MLA-推理] §"两条等价的路径" (path two: the query moves into latent space,
    q~ = W_UK q^N, and the RoPE part is carried alongside);
    [DSV2-MLA] §4.5 (the bmm of q_nope with w_kc before attention).
    Shapes: q_n [N,H,nope], q_r [N,H,rope], W_uk [H,DC,nope] -> [N,H,DC+rope].
    """
    q_n, q_r, W_uk = _f64(q_n), _f64(q_r), _f64(W_uk)
    lat = np.einsum("nhd,hcd->nhc", q_n, W_uk)
    return np.concatenate([lat, q_r], axis=-1)


def out_uv(o_lat, W_uv) -> np.ndarray:
    """Per-head up-projection of the latent attention output: o[h] = o_lat[h] W_UV[h].

    [MLA-推理] §"两条等价的路径" (path two multiplies by W_UV last);
    [DSV2-MLA] §4.5 (the bmm of the attention output with w_vc).
    Shapes: o_lat [N,H,DC], W_uv [H,DC,DV] -> [N,H,DV].
    """
    return np.einsum("nhc,hcd->nhd", _f64(o_lat), _f64(W_uv))


def mla_forward_absorbed(h, W_q, W_dkv, W_kr, W_uk, W_uv, W_o, H, nope, rope_dim, causal=True):
    """Full tiny MLA on path two, through the paged absorbed decode.

    [MLA-推理] §"两条等价的路径" (``out2``/``y2``): every query attends to the
    cached rows [c ; k_r] with the absorbed query, the weighted sum stays in
    latent space, and W_UV is applied last. The T tokens are the s_q = T new
    tokens of one sequence of length T, so the causal mask of the example is
    the bottom-right mask of ``decode_absorbed``. One page holds all rows.
    """
    q_n, q_r, c, k_r = project(h, W_q, W_dkv, W_kr, H, nope, rope_dim)
    T = c.shape[0]
    q_lat = absorb_q(q_n, q_r, W_uk)[None]  # [1,T,H,DC+rope]
    cache = np.concatenate([c, k_r], axis=-1)[None]  # [1 page, T rows, DC+rope]
    o_lat, _ = decode_absorbed(
        q_lat, cache, np.zeros((1, 1), np.int64), np.array([T]),
        scale=1.0 / math.sqrt(nope + rope_dim), causal=causal, dv=c.shape[1])
    out = out_uv(o_lat[0], W_uv)  # [T,H,DV]
    return out.reshape(T, -1) @ _f64(W_o)


# ---------------------------------------------------------------------------
# Absorbed decode over a paged latent cache.
# ---------------------------------------------------------------------------

def gather_tokens(cache, block_table_row, L: int) -> np.ndarray:
    """Logical token rows 0..L-1 of one sequence from the page pool.

    Token j sits in physical page block_table_row[j // page] at slot j % page
    ([MLA-推理] §"decode 注意力变成了计算问题": paged KV with pages of 64).
    Returns [L, Dqk] in float64. Slots at or past L are never read.
    """
    page = cache.shape[1]
    j = np.arange(L)
    phys = np.asarray(block_table_row)[j // page]
    return _f64(cache[phys, j % page])


def _allowed_count(L: int, s_q: int, i: int, causal: bool) -> int:
    """Number of keys query i may see: the new tokens are the last s_q of L,
    so under the causal mask query i sees keys 0..L-s_q+i ([MLA-推理]
    §"谁快：看新 token 和缓存 token 的数量": pairs = q*k - q(q-1)/2, k counts
    the new tokens)."""
    return L - s_q + i + 1 if causal else L


def decode_absorbed(q_lat, cache, block_table, seqlens, scale: float, causal: bool, dv: int = 512):
    """Absorbed-MLA decode: softmax attention of each (query token, head) row
    over one shared key row and one shared value row per cached token.

    [MLA-推理] §"两条等价的路径" (path two: scores q~ᵀc + q^Rᵀk^R, weighted sum in
    latent space) and §"decode 注意力变成了计算问题" (the 128 heads share one
    576-wide key and 512-wide value: an MQA with a wide head);
    [AI-MTP] Appendix A (the RoPE part only enters the score; the value is the
    latent alone).

    q_lat [B,s_q,H,Dqk], cache [num_pages,page,Dqk], block_table [B,max_pages],
    seqlens [B] (L_b, counting the s_q new tokens). The key of token j is the
    whole cache row; its value is the first ``dv`` elements of that row.
    For each (b, i, h): s_j = scale * q·K_j over the allowed keys, M = max s,
    Z = sum exp(s_j - M), o = sum exp(s_j - M)/Z * V_j, lse = M + ln Z
    (natural log). Two passes over the full row; no online rescaling.
    Returns o_lat [B,s_q,H,dv] and lse [B,s_q,H], both float64.
    """
    q_lat = _f64(q_lat)
    B, s_q, H, _ = q_lat.shape
    o = np.zeros((B, s_q, H, dv))
    lse = np.zeros((B, s_q, H))
    for b in range(B):
        L = int(seqlens[b])
        if L < s_q:
            raise ValueError("each sequence must hold at least its s_q new tokens")
        K = gather_tokens(cache, block_table[b], L)
        for i in range(s_q):
            n = _allowed_count(L, s_q, i, causal)
            Kb = K[:n]
            s = (q_lat[b, i] @ Kb.T) * scale  # [H, n]
            M = s.max(axis=1, keepdims=True)
            e = np.exp(s - M)
            Z = e.sum(axis=1, keepdims=True)
            o[b, i] = (e / Z) @ Kb[:, :dv]
            lse[b, i] = (M + np.log(Z))[:, 0]
    return o, lse


def decode_partials(q_lat, cache, block_table, seqlens, scale: float, causal: bool,
                    chunks, dv: int = 512):
    """The absorbed decode restricted to token chunks, one partial per chunk.

    [MLA-推理] §"decode 注意力变成了计算问题" (split-KV: split along the KV axis
    and merge the partial results). ``chunks[b]`` lists half-open token ranges
    [a, e) of sequence b. A row with no allowed key inside a chunk has
    o = 0 and lse = -inf, so it drops out of the merge.
    Returns a list over b of (o_part [n_b,s_q,H,dv], lse_part [n_b,s_q,H]).
    """
    q_lat = _f64(q_lat)
    B, s_q, H, _ = q_lat.shape
    out = []
    for b in range(B):
        L = int(seqlens[b])
        K = gather_tokens(cache, block_table[b], L)
        ob = np.zeros((len(chunks[b]), s_q, H, dv))
        lb = np.full((len(chunks[b]), s_q, H), -np.inf)
        for k, (a, e_) in enumerate(chunks[b]):
            for i in range(s_q):
                n = min(e_, _allowed_count(L, s_q, i, causal))
                if n <= a:
                    continue
                Kc = K[a:n]
                s = (q_lat[b, i] @ Kc.T) * scale
                M = s.max(axis=1, keepdims=True)
                ex = np.exp(s - M)
                Z = ex.sum(axis=1, keepdims=True)
                ob[k, i] = (ex / Z) @ Kc[:, :dv]
                lb[k, i] = (M + np.log(Z))[:, 0]
        out.append((ob, lb))
    return out


def lse_merge(o_parts, lse_parts):
    """Merge chunk results by their log-sum-exp.

    [MLA-推理] §"谁快：看新 token 和缓存 token 的数量" (chunk results are merged by
    LSE, the same merge as in context parallelism) and §"decode 注意力变成了计算
    问题" (split-KV merges the partial results). With lse_k the natural-log
    normaliser of chunk k: lse = M + ln sum_k exp(lse_k - M) where
    M = max_k lse_k, and o = sum_k exp(lse_k - lse) o_k. Chunks with
    lse_k = -inf add nothing.
    o_parts [n,...,dv], lse_parts [n,...] -> (o [...,dv], lse [...]).
    """
    o_parts, lse_parts = _f64(o_parts), _f64(lse_parts)
    M = lse_parts.max(axis=0)
    Mf = np.where(np.isfinite(M), M, 0.0)
    w = np.exp(lse_parts - Mf)  # exp(-inf) = 0 for empty chunks
    S = w.sum(axis=0)
    with np.errstate(divide="ignore"):
        lse = Mf + np.log(S)
    o = np.einsum("k...,k...d->...d", w / np.where(S > 0, S, 1.0), o_parts)
    return o, lse


def decode_sparse(q_lat, cache, block_table, seqlens, indices, scale: float, dv: int = 512):
    """Absorbed decode over a selected token list per query token.

    [AI-MTP] §6 "Sparse attention 把方向反过来": a light selector scores the
    history and keeps the top-k tokens (index_topk = 2048 in DeepSeek-V3.2);
    the latents at the selected indices are gathered and the scores and the
    weighted sum are taken over those tokens only, so the cost follows k, not L.

    indices [B,s_q,k] int: logical token positions in sequence b's cache
    (mapped through block_table like every other token). Entries outside
    [0, L_b) are padding and are skipped; the rest are used in list order, a
    repeated position counting once per occurrence (the definition is a sum
    over the list). No causal mask is applied: the list is the key set. A
    row whose list holds no valid entry gives o = 0 and lse = -inf.
    Other arguments and the per-row arithmetic are those of decode_absorbed.
    Returns o_lat [B,s_q,H,dv] and lse [B,s_q,H], float64.
    """
    q_lat = _f64(q_lat)
    B, s_q, H, _ = q_lat.shape
    indices = np.asarray(indices)
    o = np.zeros((B, s_q, H, dv))
    lse = np.full((B, s_q, H), -np.inf)
    for b in range(B):
        L = int(seqlens[b])
        K_all = gather_tokens(cache, block_table[b], L)
        for i in range(s_q):
            sel = indices[b, i]
            sel = sel[(sel >= 0) & (sel < L)]
            if sel.size == 0:
                continue
            K = K_all[sel]
            s = (q_lat[b, i] @ K.T) * scale  # [H, n]
            M = s.max(axis=1, keepdims=True)
            e = np.exp(s - M)
            Z = e.sum(axis=1, keepdims=True)
            o[b, i] = (e / Z) @ K[:, :dv]
            lse[b, i] = (M + np.log(Z))[:, 0]
    return o, lse


def e4m3_decode(codes) -> np.ndarray:
    """Values of FP8 e4m3 codes (the "fn" variant: no infinities), float64.

    Bit layout: sign (bit 7), exponent E (bits 3..6, bias 7), mantissa M
    (bits 0..2). E = 0 is subnormal: M * 2^-9. Otherwise (1 + M/8) * 2^(E-7).
    E = 15 with M = 7 is NaN (the only non-finite code); the largest finite
    magnitude is 448. This is the format the pages name for the FP8 latent
    cache ([MLA-推理] §"练习" exercise 2 and §"decode 注意力变成了计算问题").
    """
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    E = (c >> 3) & 0xF
    M = (c & 0x7).astype(np.float64)
    mag = np.where(E == 0, M * 2.0 ** -9, (1.0 + M / 8.0) * np.exp2(E.astype(np.float64) - 7.0))
    mag = np.where((E == 15) & (M == 7), np.nan, mag)
    return sign * mag


def decode_absorbed_fp8(q_lat, cache_codes, row_scales, block_table, seqlens, scale: float, causal: bool,
                        dv: int = 512):
    """Absorbed decode on an FP8 latent cache.

    [MLA-推理] §"练习" exercise 2: with the latent cache stored in FP8 a cached
    token is 576 bytes plus its scale factors. The reading used here: every
    cache row holds 576 e4m3 codes and one fp32 scale, and its value is
    scale * e4m3_decode(codes); the key is the whole row and the value its
    first ``dv`` elements, exactly as in decode_absorbed, which runs on the
    dequantised rows.
    cache_codes [num_pages, page, 576] uint8, row_scales [num_pages, page].
    """
    rows = e4m3_decode(cache_codes) * _f64(row_scales)[..., None]
    return decode_absorbed(q_lat, rows, block_table, seqlens, scale, causal, dv=dv)


def _prefill_rows(q_nope, q_rope, K_lat, W_uk, W_uv, scale, L, s_q, a, e, causal=True):
    """Path-one attention of the s_q new tokens over cached tokens [a, e) of a
    sequence of L tokens (rows K_lat[j] = [c_j ; k^R_j]). Returns o [s_q,H,dv]
    and lse [s_q,H] (o = 0, lse = -inf where a row sees no key in [a, e))."""
    dc = W_uk.shape[1]
    c = K_lat[a:e, :dc]
    k_r = K_lat[a:e, dc:]
    k_n = np.einsum("tc,hcd->htd", c, W_uk)            # [H, n, nope]
    v = np.einsum("tc,hcd->htd", c, W_uv)              # [H, n, dv]
    H = W_uk.shape[0]
    o = np.zeros((s_q, H, W_uv.shape[2]))
    lse = np.full((s_q, H), -np.inf)
    for i in range(s_q):
        last = (L - s_q + i) if causal else (L - 1)   # the new tokens are the last s_q of L
        n = min(e, last + 1) - a
        if n <= 0:
            continue
        s = (np.einsum("hd,htd->ht", q_nope[i], k_n[:, :n]) + q_rope[i] @ k_r[:n].T) * scale  # [H, n]
        M = s.max(axis=1, keepdims=True)
        w = np.exp(s - M)
        Z = w.sum(axis=1, keepdims=True)
        o[i] = np.einsum("ht,htd->hd", w / Z, v[:, :n])
        lse[i] = (M + np.log(Z))[:, 0]
    return o, lse


def prefill_expanded(q_nope, q_rope, cache, block_table, seqlens, W_uk, W_uv, scale: float, causal: bool = True):
    """Path one ("展开") on a paged latent cache, for new tokens after a prefix.

    [MLA-推理] §"两条等价的路径" (path one: expand the latent into per-head
    keys k^N = c W_UK[h] and values v = c W_UV[h], attach the shared k^R, run
    ordinary multi-head attention with scale 1/sqrt(nope + rope)) and
    §"谁快：看新 token 和缓存 token 的数量" (prefill and extend: the s_q new
    tokens are the last s_q of the L cached ones and see every earlier token).
    q_nope [B,s_q,H,nope], q_rope [B,s_q,H,rope] (rotated), cache rows
    [c ; k^R] [num_pages,page,dc+rope], W_uk [H,dc,nope], W_uv [H,dc,dv].
    Returns per-head outputs o [B,s_q,H,dv] (before W_o) and lse [B,s_q,H].
    """
    q_nope, q_rope = _f64(q_nope), _f64(q_rope)
    W_uk, W_uv = _f64(W_uk), _f64(W_uv)
    B, s_q, H, _ = q_nope.shape
    o = np.zeros((B, s_q, H, W_uv.shape[2]))
    lse = np.zeros((B, s_q, H))
    for b in range(B):
        L = int(seqlens[b])
        K_lat = gather_tokens(cache, block_table[b], L)
        o[b], lse[b] = _prefill_rows(q_nope[b], q_rope[b], K_lat, W_uk, W_uv, scale, L, s_q, 0, L, causal)
    return o, lse


def prefill_chunked(q_nope, q_rope, cache, block_table, seqlens, W_uk, W_uv, scale: float, chunk: int,
                    causal: bool = True):
    """Path one with the cached tokens expanded ``chunk`` at a time.

    [MLA-推理] §"谁快" (SGLang's MHA_CHUNKED_KV: the prefix is expanded chunk by
    chunk, attention runs per chunk, and the chunk results are merged by
    their LSE, as in context parallelism). Partials per chunk, then lse_merge.
    """
    q_nope, q_rope = _f64(q_nope), _f64(q_rope)
    W_uk, W_uv = _f64(W_uk), _f64(W_uv)
    B, s_q, H, _ = q_nope.shape
    o = np.zeros((B, s_q, H, W_uv.shape[2]))
    lse = np.zeros((B, s_q, H))
    for b in range(B):
        L = int(seqlens[b])
        K_lat = gather_tokens(cache, block_table[b], L)
        parts = [_prefill_rows(q_nope[b], q_rope[b], K_lat, W_uk, W_uv, scale, L, s_q, a, min(a + chunk, L), causal)
                 for a in range(0, L, chunk)]
        o[b], lse[b] = lse_merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    return o, lse


def crossover_tokens(L: int, H: int = 128, nope: int = 128, rope: int = 64, dv: int = 128, dc: int = 512) -> float:
    """New-token count above which path one (expanded) costs fewer FLOPs for
    a sequence of L keys counting the new ones.

    [MLA-推理] §"谁快": path one pays the expansion per cached token and the
    cheap pair cost; path two pays the absorption per new token and the
    dearer pair cost. With e = expansion per key, b = absorption per query,
    p1, p2 the pair costs and pairs ≈ q L (q ≪ L), path one wins when
    q (b + (p2 - p1) L) > e L, i.e. q > e L / (b + (p2 - p1) L); for L → ∞
    this is e / (p2 - p1), the chapter's 171.
    """
    e = 2 * dc * H * (nope + dv)
    b = 2 * H * nope * dc + 2 * H * dc * dv
    p1 = 2 * H * (nope + rope) + 2 * H * dv
    p2 = 2 * H * (dc + rope) + 2 * H * dc
    return e * L / (b + (p2 - p1) * L)


# ---------------------------------------------------------------------------
# FP8 batched products for the absorption ([SGL-compile] "MLA 与 torch.compile：
# v0.3 的两个来源", the weight-absorption passage: with FP8 weights w_kc and w_vc the absorbed query and the output
# projection run as bmm_fp8 of an activation quantised to e4m3 on the fly,
# one scale per tensor, against the e4m3 weights and their scale, with a
# bf16 result).
# ---------------------------------------------------------------------------

_E4M3_CODES = np.arange(0x00, 0x7F)            # the 127 non-negative finite codes, increasing values
_E4M3_VALUES = None


def _e4m3_table():
    global _E4M3_VALUES
    if _E4M3_VALUES is None:
        _E4M3_VALUES = e4m3_decode(_E4M3_CODES)
    return _E4M3_VALUES


def e4m3_encode(x) -> np.ndarray:
    """Nearest e4m3 ("fn") code of each value, ties to the even code, magnitudes
    beyond the largest finite value 448 clamped to it; the sign is kept (so -0
    gives 0x80). This is round-to-nearest-even onto the value set e4m3_decode
    defines, taken over the exact float64 values of x."""
    x = np.asarray(x, dtype=np.float64)
    vals = _e4m3_table()
    mag = np.minimum(np.abs(x), vals[-1])
    hi = np.searchsorted(vals, mag, side="left")          # vals[hi-1] < mag <= vals[hi]
    hi = np.clip(hi, 1, len(vals) - 1)
    lo = hi - 1
    d_lo, d_hi = mag - vals[lo], vals[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_E4M3_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _E4M3_CODES[hi], _E4M3_CODES[lo])
    code = np.where(mag == 0.0, 0, code)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def quantize_e4m3(x):
    """Per-tensor dynamic quantisation to e4m3, the activation side of the
    pages' bmm_fp8: the multiplier r = 448 / max|x| (fp32; max|x| taken as at
    least 2^-100, and r = 1 for an all-zero tensor), codes e4m3_encode(x * r)
    with the product taken in fp32 (the precision the kernel decides the
    codes in), and the dequantisation scale s = 1 / r (fp32).
    Returns (codes uint8, s float32)."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0.0)
    r = np.float32(448.0) / np.maximum(amax, np.float32(2.0 ** -100)) if amax > 0 else np.float32(1.0)
    s = np.float32(1.0) / r
    return e4m3_encode((x32 * r).astype(np.float32)), s


def absorb_q_fp8(q_n, q_r, w_uk_codes, w_scale: float) -> np.ndarray:
    """absorb_q with e4m3 operands: q^N quantised per tensor (quantize_e4m3),
    W_UK given as e4m3 codes [H, DC, nope] with one scale, the product scaled
    by both scales, q^R copied. Returns float64 [N, H, DC + rope]."""
    codes, s = quantize_e4m3(q_n)
    q = e4m3_decode(codes) * np.float64(s)
    w = e4m3_decode(w_uk_codes) * float(w_scale)
    return absorb_q(q, q_r, w)


def out_uv_fp8(o_lat, w_uv_t_codes, w_scale: float) -> np.ndarray:
    """out_uv with e4m3 operands: the latent output quantised per tensor, W_UV
    given transposed as e4m3 codes [H, DV, DC] (the weight prepared once, as
    the pages' history transposes the MLA weights offline) with one scale.
    Returns float64 [N, H, DV]."""
    codes, s = quantize_e4m3(o_lat)
    o = e4m3_decode(codes) * np.float64(s)
    w = e4m3_decode(w_uv_t_codes) * float(w_scale)
    return out_uv(o, np.swapaxes(w, 1, 2))

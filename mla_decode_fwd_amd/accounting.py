"""FLOP and byte accounting for absorbed-MLA decode, and the MI355X roofline.

Pure host arithmetic used by the benchmark to turn a measured time into
TFLOP/s, GB/s and a roofline fraction.

Sources:
  [MLA-推理] "MLA 推理：两条计算路径与 FlashMLA", section "谁快：看新 token 和缓存
             token 的数量" (FLOPs per (query, key) pair on both paths, the
             per-key expansion and per-query absorption costs, the causal pair
             count, the decode arithmetic intensity).
  [AI-MTP]   "为什么 MLA + MTP 容易吃亏？从 Arithmetic Intensity 看 Attention",
             Appendix A (F = 2HL(2d_c+d_s), B = bL(d_c+d_s), hence
             AI = H(2d_c+d_s)/(d_c+d_s) for bf16) and section 6 (sparse
             attention: the cost follows the top-k list, not L).
"""
from __future__ import annotations

from typing import Iterable

# MI355X published peaks (dense, no sparsity).
PEAK_HBM_BYTES_PER_S = 8.0e12
PEAK_MFMA_BF16_FLOP_PER_S = 2.5e15
PEAK_MFMA_FP32_FLOP_PER_S = 157.3e12  # fp32 matrix/vector peak used for fp32 inputs

DSV3 = dict(H=128, NOPE=128, ROPE=64, DV=128, DC=512)


def pair_flops_expanded(H: int, nope: int, rope: int, dv: int) -> int:
    """Path one, per (query, key) pair: QK over nope+rope and PV over dv, all heads."""
    return 2 * H * (nope + rope) + 2 * H * dv


def pair_flops_absorbed(H: int, dc: int, rope: int) -> int:
    """Path two, per (query, key) pair: QK over dc+rope and PV over dc, all heads."""
    return 2 * H * (dc + rope) + 2 * H * dc


def expand_flops_per_key(H: int, nope: int, dv: int, dc: int) -> int:
    """Path one's fixed cost per cached token: expanding c into every head's k^N and v."""
    return 2 * dc * H * (nope + dv)


def absorb_flops_per_query(H: int, nope: int, dv: int, dc: int) -> int:
    """Path two's fixed cost per new token: W_UK into the query, W_UV on the output."""
    return 2 * H * nope * dc + 2 * H * dc * dv


def causal_pairs(q: int, k: int) -> float:
    """(query, key) pairs when q new tokens follow k-q cached ones, k counting them."""
    return q * k - q * (q - 1) / 2


def path_flops(q: int, k: int, H=128, nope=128, rope=64, dv=128, dc=512):
    """Total FLOPs of (expanded, absorbed) attention for q new tokens over k keys."""
    pairs = causal_pairs(q, k)
    exp = k * expand_flops_per_key(H, nope, dv, dc) + pairs * pair_flops_expanded(H, nope, rope, dv)
    ab = q * absorb_flops_per_query(H, nope, dv, dc) + pairs * pair_flops_absorbed(H, dc, rope)
    return exp, ab


def crossover_new_tokens(H=128, nope=128, rope=64, dv=128, dc=512) -> float:
    """New-token count past which expansion wins when the prefix is much longer."""
    return expand_flops_per_key(H, nope, dv, dc) / (
        pair_flops_absorbed(H, dc, rope) - pair_flops_expanded(H, nope, rope, dv))


def mla_decode_ai(H: int, dc: int, ds: int, bytes_per_elem: float = 2.0) -> float:
    """Decode arithmetic intensity of absorbed MLA, FLOP per byte of cache read."""
    return 2.0 * H * (2 * dc + ds) / (bytes_per_elem * (dc + ds))


def decode_flops(seqlens: Iterable[int], s_q: int, H: int, d_qk: int = 576, d_v: int = 512) -> float:
    """Algorithmic FLOPs of one decode call: 2 H (d_qk + d_v) per causal pair."""
    return sum(2.0 * H * (d_qk + d_v) * causal_pairs(s_q, int(L)) for L in seqlens)


def decode_bytes(seqlens: Iterable[int], s_q: int, H: int, elem_bytes: int = 2,
                 d_qk: int = 576, d_v: int = 512, page: int = 64) -> float:
    """Algorithmic HBM bytes of one decode call.

    Each cached row read once, plus the query, the output, the fp32 LSE and
    the block-table entries in use.
    """
    seqlens = [int(L) for L in seqlens]
    B = len(seqlens)
    kv = sum(L * d_qk * elem_bytes for L in seqlens)
    q = B * s_q * H * d_qk * elem_bytes
    o = B * s_q * H * d_v * elem_bytes
    lse = B * s_q * H * 4
    table = sum(((L + page - 1) // page) * 4 for L in seqlens)
    return float(kv + q + o + lse + table)


def sparse_valid_counts(indices, seqlens):
    """Selected entries per (sequence, query token): positions in [0, L_b)."""
    import numpy as np
    idx = np.asarray(indices)
    L = np.asarray(seqlens, dtype=np.int64).reshape(-1, 1, 1)
    return ((idx >= 0) & (idx < L)).sum(axis=-1)


def sparse_decode_flops(valid_counts, H: int, d_qk: int = 576, d_v: int = 512) -> float:
    """Algorithmic FLOPs of a top-k decode: 2 H (d_qk + d_v) per selected (row, token)."""
    import numpy as np
    return float(2.0 * H * (d_qk + d_v) * np.asarray(valid_counts, dtype=np.float64).sum())


def sparse_decode_bytes(valid_counts, B: int, s_q: int, H: int, topk: int, elem_bytes: int = 2,
                        d_qk: int = 576, d_v: int = 512) -> float:
    """Algorithmic HBM bytes of a top-k decode: each selected cache row once per
    query token that selects it (counted per list entry), the index lists, the
    block-table entries they map through (one per entry), q, o and the LSE."""
    import numpy as np
    n = float(np.asarray(valid_counts, dtype=np.float64).sum())
    rows = n * d_qk * elem_bytes
    lists = B * s_q * topk * 4 + n * 4
    return rows + lists + B * s_q * H * (d_qk * elem_bytes + d_v * elem_bytes + 4)


def decode_bytes_fp8(seqlens: Iterable[int], s_q: int, H: int, d_qk: int = 576, d_v: int = 512,
                     page: int = 64) -> float:
    """Algorithmic HBM bytes of one decode call on an FP8 latent cache: each
    cached row once as d_qk one-byte codes plus its fp32 scale; bf16 q and o,
    the fp32 LSE and the block-table entries in use."""
    seqlens = [int(L) for L in seqlens]
    B = len(seqlens)
    kv = sum(L * (d_qk + 4) for L in seqlens)
    table = sum(((L + page - 1) // page) * 4 for L in seqlens)
    return float(kv + B * s_q * H * (d_qk * 2 + d_v * 2 + 4) + table)


def kv_bytes(seqlens: Iterable[int], elem_bytes: int = 2, d_qk: int = 576) -> float:
    return float(sum(int(L) * d_qk * elem_bytes for L in seqlens))


def roofline(flops: float, nbytes: float, seconds: float,
             peak_flops: float = PEAK_MFMA_BF16_FLOP_PER_S,
             peak_bw: float = PEAK_HBM_BYTES_PER_S) -> dict:
    """Achieved rates and the fraction of the binding ceiling.

    The bound is whichever ceiling the arithmetic intensity selects
    (AI below peak_flops/peak_bw means HBM); the fraction is achieved/peak on
    that ceiling.
    """
    ai = flops / nbytes
    tflops = flops / seconds / 1e12
    gbs = nbytes / seconds / 1e9
    if ai < peak_flops / peak_bw:
        bound, achieved, peak, unit = "hbm", gbs, peak_bw / 1e9, "GB/s"
    else:
        bound, achieved, peak, unit = "mfma", tflops, peak_flops / 1e12, "TFLOP/s"
    return dict(bound=bound, achieved=achieved, peak=peak, unit=unit, frac=achieved / peak,
                ai=ai, tflops=tflops, gbs=gbs,
                frac_mfma=tflops / (peak_flops / 1e12), frac_hbm=gbs / (peak_bw / 1e9))


def prefill_flops(seqlens: Iterable[int], s_q: int, H: int, nope=128, rope=64, dv=128, dc=512) -> float:
    """Expanded path over a batch: expansion of every cached token plus the
    causal (query, key) pairs of the s_q new tokens of each sequence."""
    return float(sum(path_flops(s_q, int(L), H, nope, rope, dv, dc)[0] for L in seqlens))


def prefill_bytes(seqlens: Iterable[int], s_q: int, H: int, nope=128, rope=64, dv=128, dc=512,
                  elem_bytes: int = 2) -> float:
    """Compulsory HBM bytes of the expanded path: the latent rows, both weight
    stacks and the queries read once, o and the LSE written once."""
    B = 0
    total = 0.0
    for L in seqlens:
        B += 1
        total += int(L) * (dc + rope) * elem_bytes
    total += 2 * H * dc * nope * elem_bytes if nope == dv else H * dc * (nope + dv) * elem_bytes
    total += B * s_q * H * ((nope + rope) * elem_bytes + dv * elem_bytes + 4)
    return total

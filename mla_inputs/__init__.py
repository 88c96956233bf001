"""Seeded synthetic inputs for absorbed-MLA decode.

This module only draws and lays out random data: it holds none of the
method's arithmetic, and both the GPU library's tests and the CPU oracle take
their inputs from here. Nothing in it imports either side.

Recipes (all seeded, all synthetic):

* ``tiny_mla_weights``: the tiny full-MLA instance of the handbook chapter
  "MLA 推理：两条计算路径与 FlashMLA", section "两条等价的路径": torch seed 0,
  T=6, D=64, H=4, nope 8, rope 4, v 8, latent 16, with weights drawn by
  ``torch.randn`` in the chapter's order (W_q, W_dkv, W_kr, W_uk, W_uv, W_o, h)
  and scaled by 1/8 or 1/4 as the chapter does.
* ``make_decode_case``: a paged latent cache and absorbed queries. Cache rows
  and queries are standard normals from ``numpy.random.default_rng(seed)``;
  queries are scaled (default 1/sqrt(576)); both are rounded to bf16 with
  round-to-nearest-even (or kept fp32). Pages hold 64 tokens. Physical pages
  come from one shuffled global pool with about 10% spare pages. Every slot no
  sequence owns (spare pages, the tail of each last page, block-table entries
  past a sequence's pages, which point at a spare page) holds NaN, so any read
  of it shows up in the output. Optionally a fraction of each sequence's token
  rows is multiplied by 8 (exact in bf16) as outliers.
* ``config_case``: the five workload shapes (tiny fp32 case aside) used for
  parity and measurement: single-sequence 4096-token decode, 64 x 4096 batched
  decode, 128-sequence two-token speculative decode with lengths uniform in
  [1024, 8192], and 8-sequence long-context variable-length decode.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Sequence

import math

import numpy as np
import torch

PAGE = 64
D_QK = 576
D_V = 512
SCALE_DS = 1.0 / math.sqrt(192.0)  # 1/sqrt(d_nope + d_rope) with 128 + 64


@dataclass
class DecodeCase:
    """One decode problem, CPU tensors, row-major and contiguous."""

    q_lat: torch.Tensor  # [B, s_q, H, 576] bf16 or fp32
    cache: torch.Tensor  # [num_pages, 64, 576] same dtype
    block_table: torch.Tensor  # [B, max_pages] int32
    seqlens: torch.Tensor  # [B] int32, L_b counting the s_q new tokens
    s_q: int
    H: int
    causal: bool
    scale: float
    name: str = ""
    meta: dict = field(default_factory=dict)

    @property
    def B(self) -> int:
        return int(self.q_lat.shape[0])

    @property
    def dtype(self) -> torch.dtype:
        return self.q_lat.dtype


def _round_to(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(dtype) if dtype != torch.float32 else t.clone()


def make_decode_case(
    seqlens: Sequence[int],
    s_q: int = 1,
    H: int = 128,
    seed: int = 0,
    dtype: torch.dtype = torch.bfloat16,
    q_scale: float = 1.0 / math.sqrt(D_QK),
    causal: Optional[bool] = None,
    scale: float = SCALE_DS,
    spare_frac: float = 0.10,
    outlier_frac: float = 0.0,
    extra_table_cols: int = 1,
    d_qk: int = D_QK,
    name: str = "",
    draw_q: bool = True,
) -> DecodeCase:
    """Draw one paged decode problem.

    Draw order from ``default_rng(seed)``: page permutation, cache normals,
    query normals, then (if ``outlier_frac``) the outlier rows per sequence.
    ``causal`` defaults to ``s_q > 1``. ``draw_q=False`` skips the query
    draw (q_lat is then empty), for callers that draw their own queries.
    """
    seqlens = [int(x) for x in seqlens]
    B = len(seqlens)
    if any(L < s_q for L in seqlens):
        raise ValueError("every sequence must hold its s_q new tokens")
    causal = (s_q > 1) if causal is None else bool(causal)
    pages = [(L + PAGE - 1) // PAGE for L in seqlens]
    used = sum(pages)
    spares = max(1, int(round(spare_frac * used)))
    num_pages = used + spares
    rng = np.random.default_rng(seed)
    perm = rng.permutation(num_pages)
    max_pages = max(pages) + extra_table_cols
    spare_ids = perm[used:]
    table = np.empty((B, max_pages), dtype=np.int32)
    pos = 0
    for b in range(B):
        table[b, : pages[b]] = perm[pos : pos + pages[b]]
        table[b, pages[b] :] = spare_ids[b % len(spare_ids)]
        pos += pages[b]
    cache32 = rng.standard_normal((num_pages, PAGE, d_qk), dtype=np.float32)
    q32 = (rng.standard_normal((B, s_q, H, d_qk), dtype=np.float32) * np.float32(q_scale) if draw_q
           else np.zeros((B, s_q, H, 0), dtype=np.float32))
    cache = _round_to(cache32, dtype)
    del cache32
    if outlier_frac > 0:
        for b in range(B):
            k = int(round(outlier_frac * seqlens[b]))
            if k == 0:
                continue
            rows = rng.choice(seqlens[b], size=k, replace=False)
            phys = torch.from_numpy(table[b, rows // PAGE].astype(np.int64))
            slot = torch.from_numpy((rows % PAGE).astype(np.int64))
            cache[phys, slot] = cache[phys, slot] * 8
    # Poison every slot no sequence owns.
    owned = np.zeros((num_pages, PAGE), dtype=bool)
    for b in range(B):
        full, rem = divmod(seqlens[b], PAGE)
        owned[table[b, :full]] = True
        if rem:
            owned[table[b, full], :rem] = True
    cache[torch.from_numpy(~owned)] = float("nan")
    return DecodeCase(
        q_lat=_round_to(q32, dtype),
        cache=cache,
        block_table=torch.from_numpy(table),
        seqlens=torch.tensor(seqlens, dtype=torch.int32),
        s_q=s_q,
        H=H,
        causal=causal,
        scale=scale,
        name=name,
        meta={"seed": seed, "num_pages": num_pages, "used_pages": used,
              "q_scale": q_scale, "outlier_frac": outlier_frac},
    )


def mtp_lengths(B: int, lo: int, hi: int, seed: int) -> list:
    """Per-sequence cached lengths uniform in [lo, hi] (a separate stream, seed+1000)."""
    rng = np.random.default_rng(seed + 1000)
    return [int(x) for x in rng.integers(lo, hi + 1, size=B)]


LONG_CONTEXT_LENGTHS = [65536, 32768, 16384, 8192, 4096, 2048, 1024, 513]


def config_case(idx: int) -> DecodeCase:
    """The workload shapes, by index 1..4 (index 0 is ``tiny_mla_weights``)."""
    if idx == 1:
        return make_decode_case([4096], s_q=1, seed=1, name="single-seq B=1 ctx=4096",
                                spare_frac=0.25)
    if idx == 2:
        return make_decode_case([4096] * 64, s_q=1, seed=2, name="batched B=64 ctx=4096")
    if idx == 3:
        return make_decode_case(mtp_lengths(128, 1024, 8192, 3), s_q=2, seed=3,
                                name="mtp B=128 s_q=2 ctx~U[1024,8192]")
    if idx == 4:
        return make_decode_case(LONG_CONTEXT_LENGTHS, s_q=1, seed=4, outlier_frac=0.01,
                                name="long-context varlen B=8")
    raise ValueError(f"no decode workload with index {idx}")


def mtp_case(s_q: int, B: int = 0, seed: int = 30) -> DecodeCase:
    """Wider speculative decode: s_q causal new tokens per sequence, H=128,
    lengths uniform in [1024, 8192] like the two-token workload. B defaults
    to 256 // s_q sequences (the two-token workload's 256 query rows per
    head, i.e. B=128 at s_q=2)."""
    B = B or max(1, 256 // s_q)
    return make_decode_case(mtp_lengths(B, 1024, 8192, seed + s_q), s_q=s_q, seed=seed + s_q,
                            name=f"mtp B={B} s_q={s_q} ctx~U[1024,8192]")


def ramp_case(seqlens: Sequence[int], s_q: int = 1, growth: float = 0.5, seed: int = 50,
              H: int = 128) -> DecodeCase:
    """Scores that keep growing along the sequence: unscaled queries, and the
    rows of logical page p multiplied by (1 + growth * p) (re-rounded to
    bf16). The running row max then rises by several units (base 2) every few
    pages, so a decoder that keeps a running reference must move it and
    rescale its accumulators many times per sequence. Unowned slots stay NaN."""
    case = make_decode_case(seqlens, s_q=s_q, H=H, seed=seed, q_scale=1.0,
                            name=f"ramp {list(seqlens)} s_q={s_q} growth={growth}")
    cache = case.cache.float()
    table = case.block_table.numpy()
    for b, L in enumerate(case.seqlens.tolist()):
        for p in range((L + PAGE - 1) // PAGE):
            cache[int(table[b, p])] *= 1.0 + growth * p
    case.cache = cache.to(case.cache.dtype)
    case.meta["growth"] = growth
    return case


def topk_indices(seqlens: Sequence[int], s_q: int, topk: int, seed: int, causal: bool = True,
                 repeat_frac: float = 0.0) -> torch.Tensor:
    """Selected-token lists [B, s_q, topk] int32, as a top-k selector would
    return them: for query token i of sequence b, min(topk, n) distinct
    positions drawn uniformly without replacement from the n positions it may
    see (n = L_b - s_q + i + 1 when causal, else L_b), in random order, the
    rest of the row padded with -1. ``repeat_frac`` replaces that fraction of
    each row's picks by copies of other picks (duplicate entries)."""
    rng = np.random.default_rng(seed)
    B = len(seqlens)
    out = np.full((B, s_q, topk), -1, dtype=np.int32)
    for b, L in enumerate(seqlens):
        for i in range(s_q):
            n = L - s_q + i + 1 if causal else L
            k = min(topk, n)
            pick = rng.choice(n, size=k, replace=False)
            r = int(round(repeat_frac * k))
            if r and k > 1:
                pick[:r] = pick[rng.integers(r, k, size=r)] if k > r else pick[:r]
            rng.shuffle(pick)
            out[b, i, :k] = pick
    return torch.from_numpy(out)


def sparse_case(seqlens: Sequence[int], s_q: int = 1, topk: int = 2048, seed: int = 60, H: int = 128,
                q_scale: float = 1.0 / math.sqrt(D_QK), repeat_frac: float = 0.0):
    """A paged decode problem plus its selected-token lists (seed + 7 for the lists)."""
    case = make_decode_case(seqlens, s_q=s_q, H=H, seed=seed, q_scale=q_scale,
                            name=f"sparse B={len(seqlens)} s_q={s_q} topk={topk}")
    case.meta["indices"] = topk_indices(seqlens, s_q, topk, seed + 7, causal=case.causal or s_q == 1,
                                        repeat_frac=repeat_frac)
    case.meta["topk"] = topk
    return case


FP8_E4M3_MAX = 448.0


def fp8_case(seqlens: Sequence[int], s_q: int = 1, seed: int = 100, H: int = 128,
             q_scale: float = 1.0 / math.sqrt(D_QK), name: str = "") -> DecodeCase:
    """A paged decode problem with an FP8 (e4m3) latent cache and one fp32
    scale per cache row. The rows are drawn as in ``make_decode_case`` (bf16
    values), scaled per row by max|row| / 448 and rounded to e4m3 by torch's
    float8_e4m3fn conversion. ``meta["cache_fp8"]`` holds the codes
    [pages, 64, 576] uint8 and ``meta["row_scales"]`` [pages, 64] fp32; rows
    no sequence owns hold NaN codes (0x7F) and NaN scales. ``cache`` keeps
    the bf16 draw."""
    case = make_decode_case(seqlens, s_q=s_q, H=H, seed=seed, q_scale=q_scale,
                            name=name or f"fp8 B={len(seqlens)} s_q={s_q}")
    x = case.cache.float()
    owned = ~torch.isnan(x).any(dim=-1)
    amax = torch.where(owned, x.abs().amax(dim=-1), torch.ones_like(x[..., 0]))
    scales = torch.where(amax > 0, amax / FP8_E4M3_MAX, torch.ones_like(amax))
    codes = (x / scales[..., None]).to(torch.float8_e4m3fn).view(torch.uint8)
    codes[~owned] = 0x7F
    scales[~owned] = float("nan")
    case.meta["cache_fp8"] = codes.contiguous()
    case.meta["row_scales"] = scales.contiguous()
    return case


def prefill_case(seqlens: Sequence[int], s_q: int, H: int = 128, seed: int = 130, nope: int = 128,
                 rope: int = 64, dv: int = 128) -> DecodeCase:
    """Inputs of the expanded (prefill / extend) path: the paged latent cache of
    ``make_decode_case`` (rows [c ; k^R] ~ N(0,1), bf16), per-head queries
    q^N [B,s_q,H,nope] and rotated q^R [B,s_q,H,rope] ~ N(0,1), and W_UK
    [H,512,nope], W_UV [H,512,dv] ~ N(0, 1/512), all bf16 (meta["q_nope"],
    meta["q_rope"], meta["w_uk"], meta["w_uv"]). Expanded keys and values
    are then ~ N(0,1) and the scores, at scale 1/sqrt(nope+rope), ~ N(0,1)."""
    case = make_decode_case(seqlens, s_q=s_q, H=H, seed=seed, scale=1.0 / math.sqrt(nope + rope),
                            name=f"prefill B={len(seqlens)} s_q={s_q} H={H}", draw_q=False)
    rng = np.random.default_rng(seed + 11)
    B = len(seqlens)
    case.meta["q_nope"] = _round_to(rng.standard_normal((B, s_q, H, nope), dtype=np.float32), torch.bfloat16)
    case.meta["q_rope"] = _round_to(rng.standard_normal((B, s_q, H, rope), dtype=np.float32), torch.bfloat16)
    w = np.float32(1.0 / math.sqrt(512))
    case.meta["w_uk"] = _round_to(rng.standard_normal((H, 512, nope), dtype=np.float32) * w, torch.bfloat16)
    case.meta["w_uv"] = _round_to(rng.standard_normal((H, 512, dv), dtype=np.float32) * w, torch.bfloat16)
    return case


def tiny_mla_weights(seed: int = 0) -> dict:
    """The tiny full-MLA draws of the handbook chapter's worked example.

    ``torch.manual_seed(seed)`` then ``torch.randn`` in the chapter's order:
    W_q [D, H(nope+rope)]/8, W_dkv [D, DC]/8, W_kr [D, rope]/8,
    W_uk [H, DC, nope]/4, W_uv [H, DC, DV]/4, W_o [H DV, D]/8, h [T, D].
    Returns float32 numpy arrays and the dimensions.
    """
    T, D, H = 6, 64, 4
    NOPE, ROPE, DV, DC = 8, 4, 8, 16
    g = torch.Generator().manual_seed(seed)
    W_q = torch.randn(D, H * (NOPE + ROPE), generator=g) / 8
    W_dkv = torch.randn(D, DC, generator=g) / 8
    W_kr = torch.randn(D, ROPE, generator=g) / 8
    W_uk = torch.randn(H, DC, NOPE, generator=g) / 4
    W_uv = torch.randn(H, DC, DV, generator=g) / 4
    W_o = torch.randn(H * DV, D, generator=g) / 8
    h = torch.randn(T, D, generator=g)
    arrays = dict(W_q=W_q, W_dkv=W_dkv, W_kr=W_kr, W_uk=W_uk, W_uv=W_uv, W_o=W_o, h=h)
    out = {k: v.numpy() for k, v in arrays.items()}
    out.update(T=T, D=D, H=H, NOPE=NOPE, ROPE=ROPE, DV=DV, DC=DC)
    return out


def random_tiny_mla(seed: int, T: int = 5, D: int = 32, H: int = 3, NOPE: int = 6,
                    ROPE: int = 4, DV: int = 5, DC: int = 10) -> dict:
    """Other tiny full-MLA instances, same recipe with a numpy stream."""
    rng = np.random.default_rng(seed)
    out = dict(
        W_q=rng.standard_normal((D, H * (NOPE + ROPE))) / 8,
        W_dkv=rng.standard_normal((D, DC)) / 8,
        W_kr=rng.standard_normal((D, ROPE)) / 8,
        W_uk=rng.standard_normal((H, DC, NOPE)) / 4,
        W_uv=rng.standard_normal((H, DC, DV)) / 4,
        W_o=rng.standard_normal((H * DV, D)) / 8,
        h=rng.standard_normal((T, D)),
    )
    out.update(T=T, D=D, H=H, NOPE=NOPE, ROPE=ROPE, DV=DV, DC=DC)
    return out


def fp8_bmm_case(N: int, H: int = 128, d_nope: int = 128, d_rope: int = 64, d_c: int = 512, d_v: int = 128,
                 seed: int = 170) -> dict:
    """Inputs of the FP8 absorption products: bf16 activations q_nope
    [N,H,d_nope], q_rope [N,H,d_rope] ~ N(0,1) and o_lat [N,H,d_c] ~ N(0,1),
    and FP8 weights: W_UK [H,d_c,d_nope] and W_UV [H,d_c,d_v] drawn
    N(0, 1/d_c), each scaled by max|W| / 448 and rounded to e4m3 by torch's
    float8_e4m3fn conversion (the weight stored once, as a serving engine
    loads it). Keys: q_nope, q_rope, o_lat (bf16 tensors), w_uk_codes
    [H,d_c,d_nope], w_uv_t_codes [H,d_v,d_c] (W_UV transposed) uint8, and the
    float scales w_uk_scale, w_uv_scale."""
    rng = np.random.default_rng(seed)

    def weight(shape):
        w = rng.standard_normal(shape, dtype=np.float32) * np.float32(1.0 / math.sqrt(d_c))
        t = torch.from_numpy(w)
        s = float(t.abs().max()) / FP8_E4M3_MAX
        return (t / s).to(torch.float8_e4m3fn).view(torch.uint8).contiguous(), s

    q_nope = _round_to(rng.standard_normal((N, H, d_nope), dtype=np.float32), torch.bfloat16)
    q_rope = _round_to(rng.standard_normal((N, H, d_rope), dtype=np.float32), torch.bfloat16)
    o_lat = _round_to(rng.standard_normal((N, H, d_c), dtype=np.float32), torch.bfloat16)
    w_uk, s_uk = weight((H, d_c, d_nope))
    w_uv, s_uv = weight((H, d_c, d_v))
    return dict(q_nope=q_nope, q_rope=q_rope, o_lat=o_lat, w_uk_codes=w_uk, w_uk_scale=s_uk,
                w_uv_t_codes=w_uv.transpose(1, 2).contiguous(), w_uv_scale=s_uv)

"""Shared helpers for the GPU parity tests: run a decode case through the
library and compare it element by element with the fp64 oracle."""
from __future__ import annotations

import numpy as np
import torch

import mla_decode_fwd_amd as mla
from oracle import mla_oracle as orc

# Tolerances. bf16 inputs: max-abs 2e-2 and relative L2 5e-3 on o_lat. fp32
# inputs: 1e-5. The LSE bound is this suite's own: scores are exact products
# of the bf16 inputs accumulated in fp32, so the LSE carries only fp32
# rounding (measured ~1e-6), and 1e-4 leaves a wide margin.
TOL = {
    torch.bfloat16: dict(max_abs=2e-2, rel_l2=5e-3, lse=1e-4),
    torch.float32: dict(max_abs=1e-5, rel_l2=1e-5, lse=1e-5),
}


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def oracle(case, rows=None):
    """Oracle result for every sequence (or the listed sequence indices)."""
    q = to_np(case.q_lat)
    cache = case.cache  # gathered per sequence inside the oracle
    table = case.block_table.numpy()
    L = case.seqlens.numpy()
    idx = range(case.B) if rows is None else rows
    outs, lses = [], []
    for b in idx:
        npg = (int(L[b]) + 63) // 64
        pages = table[b, :npg]
        sub_cache = to_np(cache[torch.from_numpy(pages.astype(np.int64))])
        sub_table = np.arange(npg)[None, :]
        o, lse = orc.decode_absorbed(q[b:b + 1], sub_cache, sub_table, L[b:b + 1], case.scale, case.causal,
                                     dv=512)
        outs.append(o[0])
        lses.append(lse[0])
    return np.stack(outs), np.stack(lses)


def to_device(case, dev="cuda"):
    return dict(q_lat=case.q_lat.to(dev), kv_cache=case.cache.to(dev),
                block_table=case.block_table.to(dev), seqlens=case.seqlens.to(dev))


def run(case, plan="auto", dev_inputs=None, num_cus=256, max_splits=64, split_offsets=None, rows_per_group=0):
    """Decode on the GPU. plan: "auto" (library planner), None (one chunk per
    sequence), "custom" with explicit host split_offsets, or "schedule" (the
    balanced schedule, mla_decode_fwd_scheduled; rows_per_group 0 lets the
    planner choose 64 or 128)."""
    d = dev_inputs or to_device(case)
    kw = {}
    if plan == "schedule":
        kw = dict(schedule=mla.decode_schedule(case.seqlens.tolist(), case.s_q, case.H, num_cus=num_cus,
                                               max_splits=max_splits, rows_per_group=rows_per_group))
    elif plan == "auto":
        p = mla.decode_plan(case.seqlens.tolist(), case.s_q, case.H, num_cus=num_cus, max_splits=max_splits)
        if p.any_split:
            kw = dict(split_offsets=p.device_offsets("cuda"), total_splits=p.total_splits)
    elif plan == "custom":
        off = np.asarray(split_offsets, dtype=np.int32)
        kw = dict(split_offsets=torch.from_numpy(off).cuda(), total_splits=int(off[-1]))
    o, lse = mla.mla_decode_fwd(d["q_lat"], d["kv_cache"], d["block_table"], d["seqlens"], case.scale,
                                case.causal, **kw)
    torch.cuda.synchronize()
    return o, lse


def compare(o_gpu, lse_gpu, o_ref, lse_ref, dtype, label="", abs_relative=False):
    """Assert parity; return the error statistics. abs_relative: the max-abs
    bound is taken relative to max(1, max|o_ref|) (sharp-softmax cases, whose
    outputs approach single value rows of magnitude ~4, where one bf16 output
    rounding alone is up to 1.6e-2)."""
    o = to_np(o_gpu)
    lse = to_np(lse_gpu)
    assert np.all(np.isfinite(o)), f"{label}: non-finite output"
    assert np.all(np.isfinite(lse)), f"{label}: non-finite lse"
    diff = o - o_ref
    max_abs = float(np.max(np.abs(diff)))
    rel_l2 = float(np.linalg.norm(diff) / max(np.linalg.norm(o_ref), 1e-30))
    lse_err = float(np.max(np.abs(lse - lse_ref)))
    t = TOL[dtype]
    stats = dict(max_abs=max_abs, rel_l2=rel_l2, lse=lse_err)
    print(f"[parity] {label} max_abs={max_abs:.3e} rel_l2={rel_l2:.3e} lse={lse_err:.3e}", flush=True)
    bound = t["max_abs"] * (max(1.0, float(np.max(np.abs(o_ref)))) if abs_relative else 1.0)
    assert max_abs <= bound, (label, stats)
    assert rel_l2 <= t["rel_l2"], (label, stats)
    assert lse_err <= t["lse"], (label, stats)
    return stats


def oracle_sparse(case, rows=None):
    """Oracle result of the top-k decode (case.meta["indices"]) for every
    sequence or the listed sequence indices."""
    q = to_np(case.q_lat)
    table = case.block_table.numpy()
    L = case.seqlens.numpy()
    idx_all = case.meta["indices"].numpy()
    outs, lses = [], []
    for b in (range(case.B) if rows is None else rows):
        npg = (int(L[b]) + 63) // 64
        sub_cache = to_np(case.cache[torch.from_numpy(table[b, :npg].astype(np.int64))])
        o, lse = orc.decode_sparse(q[b:b + 1], sub_cache, np.arange(npg)[None, :], L[b:b + 1],
                                   idx_all[b:b + 1], case.scale, dv=512)
        outs.append(o[0])
        lses.append(lse[0])
    return np.stack(outs), np.stack(lses)


def run_sparse(case, plan="auto", num_cus=256, dev="cuda"):
    """Top-k decode on the GPU through the C ABI."""
    d = to_device(case, dev)
    idx = case.meta["indices"].to(dev)
    kw = {}
    if plan == "auto":
        p = mla.sparse_decode_plan(case.B, case.meta["topk"], case.s_q, case.H, num_cus=num_cus)
        if p.any_split:
            kw = dict(split_offsets=p.device_offsets(dev), total_splits=p.total_splits)
    o, lse = mla.mla_sparse_decode_fwd(d["q_lat"], d["kv_cache"], d["block_table"], d["seqlens"], idx,
                                       case.scale, **kw)
    torch.cuda.synchronize()
    return o, lse


def oracle_fp8(case, rows=None):
    """Oracle result of the FP8-cache decode (case.meta["cache_fp8"] codes and
    case.meta["row_scales"]) for every sequence or the listed ones."""
    q = to_np(case.q_lat)
    table = case.block_table.numpy()
    L = case.seqlens.numpy()
    codes = case.meta["cache_fp8"]
    scales = case.meta["row_scales"]
    outs, lses = [], []
    for b in (range(case.B) if rows is None else rows):
        npg = (int(L[b]) + 63) // 64
        sel = torch.from_numpy(table[b, :npg].astype(np.int64))
        o, lse = orc.decode_absorbed_fp8(q[b:b + 1], codes[sel].numpy(), scales[sel].numpy().astype(np.float64),
                                         np.arange(npg)[None, :], L[b:b + 1], case.scale, case.causal, dv=512)
        outs.append(o[0])
        lses.append(lse[0])
    return np.stack(outs), np.stack(lses)


def run_fp8(case, plan="auto", num_cus=256, dev="cuda"):
    """FP8-cache decode on the GPU through the C ABI."""
    d = to_device(case, dev)
    kw = {}
    if plan == "auto":
        p = mla.decode_plan(case.seqlens.tolist(), case.s_q, case.H, num_cus=num_cus)
        if p.any_split:
            kw = dict(split_offsets=p.device_offsets(dev), total_splits=p.total_splits)
    o, lse = mla.mla_decode_fwd_fp8(d["q_lat"], case.meta["cache_fp8"].to(dev), case.meta["row_scales"].to(dev),
                                    d["block_table"], d["seqlens"], case.scale, case.causal, **kw)
    torch.cuda.synchronize()
    return o, lse


def oracle_prefill(case, chunk=None):
    """Oracle of the expanded path (prefill_expanded, or prefill_chunked when chunk is given)."""
    m = case.meta
    args = (to_np(m["q_nope"]), to_np(m["q_rope"]), to_np(case.cache), case.block_table.numpy(),
            case.seqlens.numpy(), to_np(m["w_uk"]), to_np(m["w_uv"]), case.scale)
    if chunk is None:
        return orc.prefill_expanded(*args)
    return orc.prefill_chunked(*args, chunk)

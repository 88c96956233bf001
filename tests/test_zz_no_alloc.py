"""The decode entry point that allocates nothing (mla_decode_fwd_noalloc),
called through the C ABI, against mla_decode_fwd with a workspace on the same
inputs and the same plan: two calls in a row, the second on a smaller batch,
each bit-identical to the workspace call and within the oracle tolerance."""
import numpy as np
import pytest
import torch

import mla_decode_fwd_amd as mla
from mla_inputs import make_decode_case
from gpu_helpers import compare, oracle, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mla.load_library()


def _both(case, num_cus):
    d = to_device(case)
    p = mla.decode_plan(case.seqlens.tolist(), case.s_q, case.H, num_cus=num_cus)
    assert p.any_split
    offs = p.device_offsets("cuda")
    args = (d["q_lat"], d["kv_cache"], d["block_table"], d["seqlens"], case.scale, case.causal)
    o_ws, l_ws = mla.mla_decode_fwd(*args, split_offsets=offs, total_splits=p.total_splits)
    o = torch.full_like(o_ws, float("nan"))
    lse = torch.full_like(l_ws, float("nan"))
    mla.mla_decode_fwd_noalloc(*args, o, lse, split_offsets=offs, total_splits=p.total_splits)
    torch.cuda.synchronize()
    return (o, lse), (o_ws, l_ws), p


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_noalloc_matches_workspace_call_twice(dtype):
    # First call: the B = 64 x 4096 shape's plan size class (many chunks); second,
    # smaller: the static array still holds the first call's partials.
    big = make_decode_case([4096] * 16 + [3000, 77, 1], s_q=1, H=128, seed=301, dtype=dtype)
    small = make_decode_case([700, 129, 64], s_q=2, H=128, seed=302, dtype=dtype)
    for case, cus in ((big, 256), (small, 16)):
        (o, lse), (o_ws, l_ws), p = _both(case, cus)
        print(f"[noalloc] {dtype} B={case.B} s_q={case.s_q} chunks={p.total_splits} "
              f"scratch={mla.noalloc_scratch_bytes(p.total_splits, case.s_q, case.H, dtype)}", flush=True)
        assert torch.equal(o, o_ws) and torch.equal(lse, l_ws)
        o_ref, l_ref = oracle(case)
        compare(o, lse, o_ref, l_ref, dtype, f"noalloc B={case.B} {dtype}")


def test_noalloc_without_split_and_at_the_limit():
    # No split offsets: the plain one-chunk-per-sequence decode. Then the
    # largest bf16 plan the array holds (510 chunks at H = 128, s_q = 1), and
    # one chunk more, which is refused before any launch.
    case = make_decode_case([300, 64, 129], s_q=1, H=128, seed=303)
    d = to_device(case)
    args = (d["q_lat"], d["kv_cache"], d["block_table"], d["seqlens"], case.scale, case.causal)
    o1, l1 = mla.mla_decode_fwd(*args)
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    mla.mla_decode_fwd_noalloc(*args, o2, l2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)

    lens = [64 * 64] * 8
    case = make_decode_case(lens, s_q=1, H=128, seed=304)
    d = to_device(case)
    args = (d["q_lat"], d["kv_cache"], d["block_table"], d["seqlens"], case.scale, case.causal)
    counts = [64] * 7 + [62]  # 510 chunks
    off = torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32, device="cuda")
    assert mla.noalloc_scratch_bytes(510, 1, 128) <= mla.NOALLOC_SCRATCH_BYTES
    o_ws, l_ws = mla.mla_decode_fwd(*args, split_offsets=off, total_splits=510)
    o, lse = torch.empty_like(o_ws), torch.empty_like(l_ws)
    mla.mla_decode_fwd_noalloc(*args, o, lse, split_offsets=off, total_splits=510)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ws) and torch.equal(lse, l_ws)
    o_ref, l_ref = oracle(case)
    compare(o, lse, o_ref, l_ref, torch.bfloat16, "noalloc 510 chunks")
    counts = [64] * 7 + [63]  # 511 chunks: over the limit
    off = torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32, device="cuda")
    with pytest.raises(mla.MlaError) as e:
        mla.mla_decode_fwd_noalloc(*args, o, lse, split_offsets=off, total_splits=511)
    assert e.value.status == 3

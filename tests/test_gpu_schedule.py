"""GPU parity of the balanced schedule (mla_decode_fwd_scheduled) against
the fp64 oracle: segments that span sequence boundaries, both row-group
sizes (128 rows, and 64 rows where two waves split every page and merge),
causal new tokens, few heads, running-max rescales, and the workload shapes
in the launch configuration the bench uses."""
import numpy as np
import pytest
import torch

import mla_decode_fwd_amd as mla
from mla_inputs import config_case, make_decode_case, mtp_case, ramp_case
from gpu_helpers import compare, oracle, run, to_device, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mla.load_library()


CASES = [
    # (seqlens, s_q, H, num_cus)
    ([300, 64, 129, 7], 1, 128, 8),     # segments span sequences; a 1-page sequence inside one
    ([1], 1, 128, 4),
    ([65, 64, 1000], 1, 128, 16),
    ([130, 5, 64], 2, 128, 8),           # causal, two row groups (four at 64 rows)
    ([200, 3, 77], 3, 64, 8),
    ([513, 100], 4, 32, 16),
    ([70, 70], 1, 16, 4),                # 16 rows: most of a row group clamped
    ([190], 16, 8, 32),
    ([33, 250], 1, 1, 16),
]


@pytest.mark.parametrize("rpg", [128, 64])
@pytest.mark.parametrize("lens,s_q,H,num_cus", CASES)
def test_schedule_small(lens, s_q, H, num_cus, rpg):
    case = make_decode_case(lens, s_q=s_q, H=H, seed=400 + s_q * 7 + H + len(lens))
    o, lse = run(case, plan="schedule", num_cus=num_cus, rows_per_group=rpg)
    o_ref, l_ref = oracle(case)
    compare(o, lse, o_ref, l_ref, torch.bfloat16, f"schedule {lens} s_q={s_q} H={H} cus={num_cus} rpg={rpg}")


@pytest.mark.parametrize("rpg", [128, 64])
def test_schedule_sharp_and_rescale(rpg):
    # Unscaled queries (score std ~1.7), then scores that rise page after page
    # so every row moves its reference and rescales O many times, with long
    # segments (few compute units) crossing sequence boundaries.
    case = make_decode_case([300, 64, 129, 7, 1000], s_q=2, H=128, seed=7, q_scale=1.0)
    o, lse = run(case, plan="schedule", num_cus=8, rows_per_group=rpg)
    o_ref, l_ref = oracle(case)
    compare(o, lse, o_ref, l_ref, torch.bfloat16, f"schedule sharp rpg={rpg}", abs_relative=True)
    case = ramp_case([4096, 1500, 700], s_q=1, growth=0.5)
    o, lse = run(case, plan="schedule", num_cus=8, rows_per_group=rpg)
    o_ref, l_ref = oracle(case)
    og, lg = to_np(o), to_np(lse)
    rel = np.linalg.norm(og - o_ref) / np.linalg.norm(o_ref)
    mabs = np.max(np.abs(og - o_ref)) / np.max(np.abs(o_ref))
    lrel = np.max(np.abs(lg - l_ref) / np.maximum(np.abs(l_ref), 1.0))
    print(f"[parity] schedule ramp rpg={rpg} rel_l2={rel:.3e} max_abs/scale={mabs:.3e} lse_rel={lrel:.3e}", flush=True)
    assert np.all(np.isfinite(og)) and rel <= 5e-3 and mabs <= 2e-2 and lrel <= 1e-5


def test_schedule_partials_then_combine_matches_one_call():
    # Partials only under the schedule, merged by the public combine: the
    # same bits as the one-call path (a one-chunk merge is exact).
    case = make_decode_case([300, 64, 1000, 7, 2500], s_q=2, H=128, seed=41)
    d = to_device(case)
    s = mla.decode_schedule(case.seqlens.tolist(), case.s_q, case.H, num_cus=16)
    args = (d["q_lat"], d["kv_cache"], d["block_table"], d["seqlens"], case.scale, case.causal)
    o1, l1 = mla.mla_decode_fwd(*args, schedule=s)
    ws = torch.empty(s.workspace_bytes, dtype=torch.uint8, device="cuda")
    assert mla.mla_decode_fwd(*args, schedule=s, workspace=ws, partials_only=True) == (None, None)
    o_part, lse_part = mla.workspace_partials(ws, s.total_splits, case.s_q, case.H)
    offs, _ = s.device_arrays("cuda")
    o2, l2 = mla.mla_splitkv_combine(o_part, lse_part, offs, s.total_splits, case.B)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("n", [2, 4])
def test_schedule_workload_shapes(n):
    # B=64 x 4096 (256 segments of 16 pages) and the long-context batch
    # (64-row groups, 128 segments of <= 16 pages, 64 chunks for the 64K
    # sequence), every sequence against the oracle.
    case = config_case(n)
    s = mla.decode_schedule(case.seqlens.tolist(), case.s_q, case.H)
    print(f"[schedule] {case.name}: rows/group {s.rows_per_group}, {s.num_segments} segments, "
          f"{s.total_splits} chunks", flush=True)
    o, lse = run(case, plan="schedule")
    o_ref, l_ref = oracle(case)
    compare(o, lse, o_ref, l_ref, torch.bfloat16, case.name + " (schedule)")


@pytest.mark.parametrize("s_q", [2, 4, 8])
def test_schedule_mtp_workloads(s_q):
    case = config_case(3) if s_q == 2 else mtp_case(s_q)
    o, lse = run(case, plan="schedule")
    o_ref, l_ref = oracle(case)
    compare(o, lse, o_ref, l_ref, torch.bfloat16, case.name + " (schedule)")


@pytest.mark.gpu
def test_clock_probe_stamps_every_workgroup_and_stops_when_off():
    """mla_decode_clock_probe: with a buffer set, every workgroup of a bf16
    decode writes its shader-clock cycles and 100 MHz ticks; the clock they
    give is a plausible MI355X shader clock; the results are unchanged; with
    the probe off the buffer is left alone."""
    case = make_decode_case([300, 64, 129, 7], s_q=1, H=128, seed=31)
    o_ref, l_ref = run(case, plan="schedule")
    stamps = torch.zeros(2 * 1024, dtype=torch.int64, device="cuda")
    mla.decode_clock_probe(stamps)
    try:
        o, lse = run(case, plan="schedule")
    finally:
        mla.decode_clock_probe(None)
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
    st = stamps.view(-1, 2).cpu().numpy()
    n = int((st[:, 1] > 0).sum())
    sched = mla.decode_schedule(case.seqlens.tolist(), case.s_q, case.H)
    groups = -(-(case.s_q * case.H) // sched.rows_per_group)
    assert n == sched.num_segments * groups, (n, sched.num_segments, groups)
    mhz = st[st[:, 1] > 0, 0] / st[st[:, 1] > 0, 1] * 100.0
    assert np.all((mhz > 300) & (mhz < 4000)), mhz
    snap = stamps.clone()
    run(case, plan="schedule")
    assert torch.equal(stamps, snap)

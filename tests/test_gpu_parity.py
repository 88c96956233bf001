"""GPU parity: the HIP library, called through its C ABI, against the fp64
oracle on the same seeded inputs. Every unused cache slot is NaN, so any read
outside a sequence's tokens shows up as a non-finite output."""
import math

import numpy as np
import pytest
import torch

import mla_decode_fwd_amd as mla
from mla_inputs import config_case, make_decode_case, mtp_case, ramp_case, tiny_mla_weights
from oracle import mla_oracle as orc
from gpu_helpers import TOL, compare, oracle, run, to_device, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mla.load_library()


# ---------------------------------------------------------------------------
# Small cases: several pages, ragged tails, every split path.
# ---------------------------------------------------------------------------

SMALL = [
    # (seqlens, s_q, H)
    ([1], 1, 128),
    ([64], 1, 128),
    ([65], 1, 128),
    ([300, 64, 129, 7], 1, 128),
    ([130, 5, 64], 2, 128),
    ([200, 3, 77], 3, 64),
    ([513, 100], 4, 32),
    ([70, 70], 1, 16),
    ([190], 16, 8),
    ([33, 250], 1, 1),
]


@pytest.mark.parametrize("plan", ["auto", None])
@pytest.mark.parametrize("lens,s_q,H", SMALL)
def test_small_bf16(lens, s_q, H, plan):
    case = make_decode_case(lens, s_q=s_q, H=H, seed=100 + s_q * 7 + H + len(lens))
    o, lse = run(case, plan=plan, num_cus=8)
    o_ref, l_ref = oracle(case)
    compare(o, lse, o_ref, l_ref, torch.bfloat16, f"small {lens} s_q={s_q} H={H} plan={plan}")


@pytest.mark.parametrize("lens,s_q,H", [([300, 64, 129, 7], 1, 128), ([130, 5, 64], 2, 128)])
def test_small_bf16_sharp_softmax(lens, s_q, H):
    """Unscaled queries: score std ~1.7, so a wrong or missing key shows."""
    case = make_decode_case(lens, s_q=s_q, H=H, seed=7, q_scale=1.0)
    o, lse = run(case, plan="auto", num_cus=8)
    o_ref, l_ref = oracle(case)
    compare(o, lse, o_ref, l_ref, torch.bfloat16, f"sharp {lens}")


@pytest.mark.parametrize("lens,s_q,plan", [([4096, 1500, 700], 1, "auto"), ([4096, 1500, 700], 1, None),
                                           ([2000, 900, 65], 2, "auto")])
def test_running_max_rescale(lens, s_q, plan):
    # Scores that grow page after page (row max up by ~3 in base 2 per page),
    # so every row moves its softmax reference and rescales O and l dozens of
    # times inside one chunk (few compute units => long chunks). Outputs and
    # LSEs are large here (rows scaled up to ~33x), so the absolute bounds are
    # taken relative to the output's scale: max-abs 2e-2 * max|o_ref| and LSE
    # 1e-5 relative (fp32 accumulation of 576 products of that size); rel-L2
    # keeps the usual 5e-3.
    case = ramp_case(lens, s_q=s_q, growth=0.5)
    o, lse = run(case, plan=plan, num_cus=8)
    o_ref, l_ref = oracle(case)
    og, lg = to_np(o), to_np(lse)
    assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg))
    rel = np.linalg.norm(og - o_ref) / np.linalg.norm(o_ref)
    mabs = np.max(np.abs(og - o_ref)) / np.max(np.abs(o_ref))
    lrel = np.max(np.abs(lg - l_ref) / np.maximum(np.abs(l_ref), 1.0))
    print(f"[parity] {case.name} plan={plan} rel_l2={rel:.3e} max_abs/scale={mabs:.3e} lse_rel={lrel:.3e}")
    assert rel <= 5e-3 and mabs <= 2e-2 and lrel <= 1e-5, (rel, mabs, lrel)


def test_small_fp32():
    case = make_decode_case([300, 64, 129, 7], s_q=2, H=16, seed=9, dtype=torch.float32, q_scale=1.0)
    for plan in ("auto", None):
        o, lse = run(case, plan=plan, num_cus=8)
        o_ref, l_ref = oracle(case)
        compare(o, lse, o_ref, l_ref, torch.float32, f"fp32 plan={plan}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_many_chunks_merge(dtype):
    """Eight or more chunks per sequence on average: the merge takes one
    workgroup per row with the chunks split over its waves."""
    case = make_decode_case([700, 300], s_q=2, H=16, seed=12, dtype=dtype, q_scale=1.0)
    o, lse = run(case, plan="custom", split_offsets=[0, 11, 16])
    o_ref, l_ref = oracle(case)
    compare(o, lse, o_ref, l_ref, dtype, f"many chunks {dtype}", abs_relative=True)


def test_chunks_with_no_pages_and_max_splits():
    """Explicit offsets: 64 chunks over 3 pages (most empty) and 1-page chunks."""
    case = make_decode_case([150, 64 * 64], s_q=1, H=128, seed=11)
    o, lse = run(case, plan="custom", split_offsets=[0, 64, 128])
    o_ref, l_ref = oracle(case)
    compare(o, lse, o_ref, l_ref, torch.bfloat16, "custom splits")


# ---------------------------------------------------------------------------
# The workload shapes at full size, in the launch configuration the bench uses.
# ---------------------------------------------------------------------------

def test_single_sequence_4096():
    case = config_case(1)
    o, lse = run(case)
    o_ref, l_ref = oracle(case)
    compare(o, lse, o_ref, l_ref, torch.bfloat16, case.name)


def test_batched_64x4096():
    case = config_case(2)
    o, lse = run(case)
    o_ref, l_ref = oracle(case)
    compare(o, lse, o_ref, l_ref, torch.bfloat16, case.name)


def test_mtp_two_tokens():
    # Every one of the 128 sequences (both new tokens, all heads) against the oracle.
    case = config_case(3)
    o, lse = run(case)
    o_ref, l_ref = oracle(case)
    compare(o, lse, o_ref, l_ref, torch.bfloat16, case.name)


@pytest.mark.parametrize("plan", ["auto", None])
def test_max_new_tokens_at_128_heads(plan):
    # The largest row count the kernel takes: s_q = 16 causal new tokens at
    # H = 128 (2048 rows, sixteen row groups per chunk), with a sequence that
    # holds nothing but its new tokens (L = s_q: the first query sees one key)
    # and one whose new tokens straddle a page boundary.
    for q_scale in (None, 1.0):
        kw = {} if q_scale is None else dict(q_scale=q_scale)
        case = make_decode_case([16, 17, 100], s_q=16, H=128, seed=230, **kw)
        o, lse = run(case, plan=plan, num_cus=64)
        o_ref, l_ref = oracle(case)
        compare(o, lse, o_ref, l_ref, torch.bfloat16, f"s_q=16 H=128 plan={plan} q_scale={q_scale}",
                abs_relative=True)


@pytest.mark.parametrize("lens,s_q", [([1000, 300, 2000], 4), ([700, 129], 8), ([64, 65], 8)])
def test_wider_mtp_small(lens, s_q):
    # Speculative verify with up to 8 causal new tokens at H=128 (one group of
    # 128 rows per new token), scaled and unscaled queries.
    for q_scale in (None, 1.0):
        kw = {} if q_scale is None else dict(q_scale=q_scale)
        case = make_decode_case(lens, s_q=s_q, H=128, seed=200 + s_q, **kw)
        o, lse = run(case, plan="auto", num_cus=32)
        o_ref, l_ref = oracle(case)
        compare(o, lse, o_ref, l_ref, torch.bfloat16, f"mtp {lens} s_q={s_q} q_scale={q_scale}")


@pytest.mark.parametrize("s_q", [4, 8])
def test_wider_mtp_workload(s_q):
    # The mtp4 / mtp8 bench workloads, every sequence against the oracle.
    case = mtp_case(s_q)
    o, lse = run(case)
    o_ref, l_ref = oracle(case)
    compare(o, lse, o_ref, l_ref, torch.bfloat16, case.name)


def test_long_context_varlen():
    case = config_case(4)
    o, lse = run(case)
    o_ref, l_ref = oracle(case)
    compare(o, lse, o_ref, l_ref, torch.bfloat16, case.name)


# ---------------------------------------------------------------------------
# Invariants on the GPU
# ---------------------------------------------------------------------------

def test_page_permutation_and_determinism_bitwise():
    case = make_decode_case([700, 333, 64], s_q=2, H=128, seed=21)
    o1, l1 = run(case)
    o1b, l1b = run(case)
    assert torch.equal(o1, o1b) and torch.equal(l1, l1b), "two runs differ"
    perm = torch.from_numpy(np.random.default_rng(5).permutation(case.cache.shape[0]).astype(np.int64))
    cache2 = torch.empty_like(case.cache)
    cache2[perm] = case.cache
    table2 = perm[case.block_table.long()].to(torch.int32)
    case2 = make_decode_case([700, 333, 64], s_q=2, H=128, seed=21)
    case2.cache, case2.block_table = cache2, table2
    o2, l2 = run(case2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "page permutation changed the output"


def test_split_invariance():
    case = make_decode_case([2000, 1500, 700], s_q=1, H=128, seed=22)
    o_ref, l_ref = oracle(case)
    outs = []
    for num_cus, ms in [(1, 64), (16, 64), (256, 64), (256, 4)]:
        o, lse = run(case, num_cus=num_cus, max_splits=ms)
        compare(o, lse, o_ref, l_ref, torch.bfloat16, f"num_cus={num_cus} max_splits={ms}")
        outs.append((o.float(), lse))
    for o, lse in outs[1:]:
        assert (o - outs[0][0]).abs().max().item() < 4e-3
        assert (lse - outs[0][1]).abs().max().item() < 1e-4


def test_head_permutation_and_sequence_independence():
    case = make_decode_case([400, 257], s_q=1, H=128, seed=23)
    o1, l1 = run(case)
    hp = torch.from_numpy(np.random.default_rng(6).permutation(128))
    case_p = make_decode_case([400, 257], s_q=1, H=128, seed=23)
    case_p.q_lat = case.q_lat[:, :, hp].contiguous()
    o2, l2 = run(case_p)
    assert torch.equal(o2, o1[:, :, hp]) and torch.equal(l2, l1[:, :, hp])
    case_s = make_decode_case([400, 257], s_q=1, H=128, seed=23)
    case_s.q_lat = case.q_lat.clone()
    case_s.q_lat[1] = -case_s.q_lat[1]
    o3, l3 = run(case_s, plan=None)
    o1n, l1n = run(case, plan=None)
    assert torch.equal(o3[0], o1n[0]) and torch.equal(l3[0], l1n[0])


# ---------------------------------------------------------------------------
# Combine and the bmm helpers
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_splitkv_combine(out_dtype):
    rng = np.random.default_rng(31)
    counts = [1, 3, 64, 2]
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    S, s_q, H = int(off[-1]), 2, 16
    o_part = rng.standard_normal((S, s_q, H, 512)).astype(np.float32)
    lse_part = (rng.standard_normal((S, s_q, H)) * 3).astype(np.float32)
    lse_part[1, 0, :4] = -np.inf  # empty chunks
    lse_part[5:9, 1, 3] = -np.inf
    # The partials come in the output dtype; the reference merges the same
    # (rounded) values in fp64.
    o_part_t = torch.from_numpy(o_part).to(out_dtype)
    o_part = o_part_t.to(torch.float64).numpy()
    o_gpu, l_gpu = mla.mla_splitkv_combine(o_part_t.cuda(), torch.from_numpy(lse_part).cuda(),
                                           torch.from_numpy(off).cuda(), S, len(counts), out_dtype)
    torch.cuda.synchronize()
    o_ref = np.zeros((len(counts), s_q, H, 512))
    l_ref = np.zeros((len(counts), s_q, H))
    for b in range(len(counts)):
        o_ref[b], l_ref[b] = orc.lse_merge(o_part[off[b]:off[b + 1]], lse_part[off[b]:off[b + 1]])
    o = to_np(o_gpu)
    err = np.abs(o - o_ref)
    if out_dtype == torch.float32:
        # fp32 sums of up to 64 weighted unit-size partials: ~64 * 2^-24 absolute.
        assert err.max() <= 1e-5
    else:
        # bf16 output: round-to-nearest-even costs at most half an ulp (2^-9 relative).
        assert np.max(err / (np.abs(o_ref) + 1e-2)) <= 2 ** -8
    assert np.max(np.abs(to_np(l_gpu) - l_ref)) < 1e-5


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_partials_only_then_combine_matches_one_call(dtype):
    # Two-phase use: decode writes only the chunk partials (every chunk, also
    # the sequences with one chunk), the public combine merges them. Both
    # phases run the same kernels as the one-call path, and a one-chunk merge
    # is exact (weight exp(0) = 1, lse + ln 1), so the results are identical.
    case = make_decode_case([300, 64, 1000, 7, 2500], s_q=2, H=128, seed=41, dtype=dtype)
    d = to_device(case)
    p = mla.decode_plan(case.seqlens.tolist(), case.s_q, case.H, num_cus=16)
    assert p.any_split and (p.num_splits == 1).any()
    offs = p.device_offsets("cuda")
    o1, l1 = mla.mla_decode_fwd(d["q_lat"], d["kv_cache"], d["block_table"], d["seqlens"], case.scale,
                                case.causal, split_offsets=offs, total_splits=p.total_splits)
    ws = torch.empty(p.workspace_bytes, dtype=torch.uint8, device="cuda")
    res = mla.mla_decode_fwd(d["q_lat"], d["kv_cache"], d["block_table"], d["seqlens"], case.scale, case.causal,
                             split_offsets=offs, total_splits=p.total_splits, workspace=ws, partials_only=True)
    assert res == (None, None)
    o_part, lse_part = mla.workspace_partials(ws, p.total_splits, case.s_q, case.H, dtype)
    o2, l2 = mla.mla_splitkv_combine(o_part, lse_part, offs, p.total_splits, case.B, dtype)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o_ref, l_ref = oracle(case)
    compare(o2, l2, o_ref, l_ref, dtype, "partials+combine")


def test_prepared_calls_match_plain_calls():
    # A prepared decode + combine (checked and marshalled once) launches the
    # same entry points as the plain calls: identical results, repeatably.
    case = make_decode_case([700, 64, 1500], s_q=1, H=128, seed=43)
    d = to_device(case)
    p = mla.decode_plan(case.seqlens.tolist(), case.s_q, case.H, num_cus=16)
    offs = p.device_offsets("cuda")
    o1, l1 = mla.mla_decode_fwd(d["q_lat"], d["kv_cache"], d["block_table"], d["seqlens"], case.scale,
                                case.causal, split_offsets=offs, total_splits=p.total_splits)
    ws = torch.empty(p.workspace_bytes, dtype=torch.uint8, device="cuda")
    dec, _ = mla.prepare_decode(d["q_lat"], d["kv_cache"], d["block_table"], d["seqlens"], case.scale, case.causal,
                                split_offsets=offs, total_splits=p.total_splits, workspace=ws, partials_only=True)
    o_part, lse_part = mla.workspace_partials(ws, p.total_splits, case.s_q, case.H)
    o2 = torch.empty_like(o1)
    l2 = torch.empty_like(l1)
    comb = mla.prepare_combine(o_part, lse_part, offs, p.total_splits, case.B, torch.bfloat16, o2, l2)
    for _ in range(2):
        o2.zero_()
        dec()
        comb()
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_graph_replays_match_eager():
    # The split decode and its merge (two kernels on the caller's stream)
    # captured once in a HIP graph and replayed several times, with eager
    # calls on the same workspace between the replays: every replay gives
    # the eager call's bits.
    lens = [3000, 700, 130, 4096]
    case = make_decode_case(lens, s_q=1, H=128, seed=52)
    d = to_device(case)
    p = mla.decode_plan(lens, 1, 128, num_cus=32)
    assert p.any_split
    ws = torch.empty(p.workspace_bytes, dtype=torch.uint8, device="cuda")
    args = (d["q_lat"], d["kv_cache"], d["block_table"], d["seqlens"], case.scale, case.causal)
    kw = dict(split_offsets=p.device_offsets("cuda"), total_splits=p.total_splits, workspace=ws)
    o_e, l_e = mla.mla_decode_fwd(*args, **kw)
    torch.cuda.synchronize()
    o = torch.empty_like(o_e)
    lse = torch.empty_like(l_e)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mla.mla_decode_fwd(*args, o_lat=o, lse=lse, **kw)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mla.mla_decode_fwd(*args, o_lat=o, lse=lse, **kw)
    torch.cuda.synchronize()
    for i in range(4):
        o.zero_()
        lse.zero_()
        if i % 2 == 1:
            o3, l3 = mla.mla_decode_fwd(*args, **kw)
            torch.cuda.synchronize()
            assert torch.equal(o3, o_e) and torch.equal(l3, l_e)
        g.replay()
        torch.cuda.synchronize()
        print(f"[graph] replay {i}", flush=True)
        assert torch.equal(o, o_e) and torch.equal(lse, l_e), f"replay {i}"
    o_ref, l_ref = oracle(case)
    compare(o, lse, o_ref, l_ref, torch.bfloat16, "graph replays")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_absorb_q_and_out_uv_deepseek_shape(dtype):
    rng = np.random.default_rng(41)
    N, H, dn, dr, dc, dv = 64, 128, 128, 64, 512, 128
    q_n = torch.from_numpy(rng.standard_normal((N, H, dn), dtype=np.float32)).to(dtype)
    q_r = torch.from_numpy(rng.standard_normal((N, H, dr), dtype=np.float32)).to(dtype)
    w_uk = torch.from_numpy(rng.standard_normal((H, dc, dn), dtype=np.float32) / 11).to(dtype)
    w_uv = torch.from_numpy(rng.standard_normal((H, dc, dv), dtype=np.float32) / 22).to(dtype)
    o_lat = torch.from_numpy(rng.standard_normal((N, H, dc), dtype=np.float32)).to(dtype)
    ql = mla.mla_absorb_q(q_n.cuda(), q_r.cuda(), w_uk.cuda())
    ou = mla.mla_out_uv(o_lat.cuda(), w_uv.cuda())
    torch.cuda.synchronize()
    ql_ref = orc.absorb_q(to_np(q_n), to_np(q_r), to_np(w_uk))
    ou_ref = orc.out_uv(to_np(o_lat), to_np(w_uv))
    for got, ref, name in [(ql, ql_ref, "absorb_q"), (ou, ou_ref, "out_uv")]:
        g = to_np(got)
        rel = np.linalg.norm(g - ref) / np.linalg.norm(ref)
        mx = np.max(np.abs(g - ref))
        print(f"[parity] {name} {dtype} rel_l2={rel:.3e} max_abs={mx:.3e}", flush=True)
        if dtype == torch.float32:
            assert rel < 1e-6 and mx < 1e-4
        else:
            assert rel < 5e-3 and mx < 2e-2 * max(1.0, np.abs(ref).max())
    assert torch.equal(ql[..., dc:].cpu(), q_r)  # the RoPE tail is copied unchanged


@pytest.mark.parametrize("N,H,dn,dr,dc,dv", [(5, 3, 48, 8, 40, 24), (33, 2, 16, 4, 136, 200), (7, 4, 24, 4, 12, 20),
                                            (70, 3, 128, 64, 208, 72), (130, 2, 128, 64, 512, 128),
                                            (9, 2, 128, 136, 64, 24), (21, 2, 128, 4, 60, 24)])
def test_absorb_q_and_out_uv_bf16_odd_shapes(N, H, dn, dr, dc, dv):
    # Partial column blocks, a partial last k slice, and (third case) shapes
    # the MFMA form does not take, which run through the general kernel. The
    # next two take the staged d_nope = 128 absorption with a partial weight
    # slab and partial token rounds, and the staged out_uv with partial
    # column slabs, a k count that is not a multiple of 128 and three token
    # tiles spread over the waves. The sixth has a RoPE tail too long for the
    # staged absorption's 16-byte tail copy (its element-wise copy runs); the
    # last has output rows that are not 16-byte multiples (general kernel).
    rng = np.random.default_rng(42 + N)
    q_n = torch.from_numpy(rng.standard_normal((N, H, dn), dtype=np.float32)).to(torch.bfloat16)
    q_r = torch.from_numpy(rng.standard_normal((N, H, dr), dtype=np.float32)).to(torch.bfloat16)
    w_uk = torch.from_numpy(rng.standard_normal((H, dc, dn), dtype=np.float32) / 7).to(torch.bfloat16)
    w_uv = torch.from_numpy(rng.standard_normal((H, dc, dv), dtype=np.float32) / 7).to(torch.bfloat16)
    o_lat = torch.from_numpy(rng.standard_normal((N, H, dc), dtype=np.float32)).to(torch.bfloat16)
    ql = mla.mla_absorb_q(q_n.cuda(), q_r.cuda(), w_uk.cuda())
    ou = mla.mla_out_uv(o_lat.cuda(), w_uv.cuda())
    torch.cuda.synchronize()
    assert torch.equal(ql[..., dc:].cpu(), q_r)  # the RoPE tail is copied unchanged
    for got, ref, name in [(ql[..., :dc], orc.absorb_q(to_np(q_n), to_np(q_r), to_np(w_uk))[..., :dc], "absorb_q"),
                           (ou, orc.out_uv(to_np(o_lat), to_np(w_uv)), "out_uv")]:
        g = to_np(got)
        rel = np.linalg.norm(g - ref) / np.linalg.norm(ref)
        mx = np.max(np.abs(g - ref))
        print(f"[parity] {name} bf16 N={N} H={H} dn={dn} dc={dc} dv={dv} rel_l2={rel:.3e} max_abs={mx:.3e}", flush=True)
        assert rel < 5e-3 and mx < 2e-2 * max(1.0, np.abs(ref).max())
    assert torch.equal(ql[..., dc:].cpu(), q_r)


def test_tiny_full_mla_fp32_end_to_end():
    """The tiny full MLA of the worked example, absorbed path on the GPU:
    mla_absorb_q -> mla_decode_fwd (fp32, latent and RoPE zero-padded to
    512 + 64) -> mla_out_uv, then W_o; against the oracle's expanded path."""
    w = tiny_mla_weights(0)
    T, H, NOPE, ROPE, DC = w["T"], w["H"], w["NOPE"], w["ROPE"], w["DC"]
    q_n, q_r, c, k_r = orc.project(w["h"], w["W_q"], w["W_dkv"], w["W_kr"], H, NOPE, ROPE)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    q_lat_small = mla.mla_absorb_q(f32(q_n), f32(q_r), f32(w["W_uk"]))  # [T,H,DC+ROPE]
    q_lat = torch.zeros((1, T, H, 576), dtype=torch.float32, device="cuda")
    q_lat[0, :, :, :DC] = q_lat_small[..., :DC]
    q_lat[0, :, :, 512:512 + ROPE] = q_lat_small[..., DC:]
    cache = torch.full((2, 64, 576), float("nan"), dtype=torch.float32, device="cuda")
    cache[1, :T] = 0.0
    cache[1, :T, :DC] = f32(c)
    cache[1, :T, 512:512 + ROPE] = f32(k_r)
    table = torch.tensor([[1]], dtype=torch.int32, device="cuda")
    seqlens = torch.tensor([T], dtype=torch.int32, device="cuda")
    o_lat, lse = mla.mla_decode_fwd(q_lat, cache, table, seqlens, 1 / math.sqrt(NOPE + ROPE), True)
    o_small = o_lat[0, :, :, :DC].contiguous()
    out = mla.mla_out_uv(o_small, f32(w["W_uv"]))  # [T,H,DV]
    torch.cuda.synchronize()
    y_gpu = to_np(out).reshape(T, -1) @ w["W_o"].astype(np.float64)
    y_ref = orc.mla_forward_expanded(w["h"], w["W_q"], w["W_dkv"], w["W_kr"], w["W_uk"], w["W_uv"], w["W_o"],
                                     H, NOPE, ROPE)
    err = np.max(np.abs(y_gpu - y_ref))
    print(f"[parity] tiny full MLA fp32 max_abs={err:.3e}", flush=True)
    assert err <= 1e-5
    assert torch.isfinite(o_lat).all()


# ---------------------------------------------------------------------------
# Top-k (sparse) decode
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("plan", ["auto", None])
@pytest.mark.parametrize("lens,s_q,topk,q_scale", [([3000, 700, 130, 65], 1, 512, None),
                                                   ([3000, 700, 130, 65], 1, 100, 1.0),
                                                   ([2000, 900, 40], 2, 256, 1.0),
                                                   ([5000], 1, 2048, None)])
def test_sparse_small(lens, s_q, topk, q_scale, plan):
    from gpu_helpers import oracle_sparse, run_sparse
    from mla_inputs import sparse_case
    kw = {} if q_scale is None else dict(q_scale=q_scale)
    case = sparse_case(lens, s_q=s_q, topk=topk, seed=70 + topk, **kw)
    o, lse = run_sparse(case, plan=plan, num_cus=32)
    o_ref, l_ref = oracle_sparse(case)
    compare(o, lse, o_ref, l_ref, torch.bfloat16, f"{case.name} lens={lens} q_scale={q_scale} plan={plan}")


def test_sparse_sixteen_query_tokens():
    # Top-k lists for 16 new tokens per sequence (sixteen row groups), lists
    # shorter than a page, sharp scores.
    from gpu_helpers import oracle_sparse, run_sparse
    from mla_inputs import sparse_case
    case = sparse_case([900, 70], s_q=16, topk=40, seed=84, q_scale=1.0)
    o, lse = run_sparse(case, plan="auto", num_cus=16)
    o_ref, l_ref = oracle_sparse(case)
    compare(o, lse, o_ref, l_ref, torch.bfloat16, "sparse s_q=16 topk=40", abs_relative=True)


def test_sparse_padding_duplicates_and_empty_rows():
    # Lists shorter than topk (-1 padding), out-of-range entries, repeated
    # entries, and one query token with nothing selected (o = 0, lse = -inf).
    from gpu_helpers import oracle_sparse, run_sparse
    from mla_inputs import sparse_case
    case = sparse_case([300, 64, 129, 7], s_q=1, topk=200, seed=81, q_scale=1.0, repeat_frac=0.1)
    idx = case.meta["indices"]
    idx[1, 0, 5] = 64      # == L: padding
    idx[2, 0, 0] = 100000  # far out of range
    idx[3, 0, :] = -1      # nothing selected
    o, lse = run_sparse(case, plan="auto", num_cus=8)
    o_ref, l_ref = oracle_sparse(case)
    assert torch.all(o[3].float() == 0) and torch.all(torch.isneginf(lse[3]))
    compare(o[:3], lse[:3], o_ref[:3], l_ref[:3], torch.bfloat16, "sparse padding/duplicates")


def test_sparse_full_list_matches_dense_kernel():
    # Every visible position listed (shuffled): the top-k path equals the
    # dense decode of the same inputs, both within the oracle tolerance.
    from gpu_helpers import run_sparse
    from mla_inputs import topk_indices
    lens = [2048, 1000, 64]
    case = make_decode_case(lens, s_q=1, H=128, seed=82, q_scale=1.0)
    case.meta["indices"] = topk_indices(lens, 1, 2048, seed=9)
    case.meta["topk"] = 2048
    o_s, l_s = run_sparse(case, plan="auto", num_cus=16)
    o_d, l_d = run(case, plan="auto", num_cus=16)
    o_ref, l_ref = oracle(case)
    compare(o_s, l_s, o_ref, l_ref, torch.bfloat16, "sparse full list vs oracle")
    compare(o_d, l_d, o_ref, l_ref, torch.bfloat16, "dense vs oracle")


def test_sparse_dsa_shape():
    # DeepSeek-V3.2 shape: topk 2048 over 8192-token histories, B=16, every
    # sequence against the oracle.
    from gpu_helpers import oracle_sparse, run_sparse
    from mla_inputs import sparse_case
    case = sparse_case([8192] * 16, s_q=1, topk=2048, seed=83)
    o, lse = run_sparse(case)
    o_ref, l_ref = oracle_sparse(case)
    compare(o, lse, o_ref, l_ref, torch.bfloat16, case.name)


# ---------------------------------------------------------------------------
# FP8 (e4m3) latent cache
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("plan", ["auto", None])
@pytest.mark.parametrize("lens,s_q,q_scale", [([300, 64, 129, 7], 1, None), ([300, 64, 129, 7], 1, 1.0),
                                              ([1000, 130, 5], 2, 1.0), ([700, 129], 8, None)])
def test_fp8_small(lens, s_q, q_scale, plan):
    # Rows no sequence owns hold NaN codes and NaN scales; sequence tails end
    # inside pages; causal among the new tokens for s_q > 1.
    from gpu_helpers import oracle_fp8, run_fp8
    from mla_inputs import fp8_case
    kw = {} if q_scale is None else dict(q_scale=q_scale)
    case = fp8_case(lens, s_q=s_q, seed=110 + s_q, **kw)
    o, lse = run_fp8(case, plan=plan, num_cus=32)
    o_ref, l_ref = oracle_fp8(case)
    compare(o, lse, o_ref, l_ref, torch.bfloat16, f"{case.name} {lens} q_scale={q_scale} plan={plan}",
            abs_relative=q_scale is not None)


def test_fp8_batched_64x4096():
    # The fp8 bench workload, every sequence against the oracle.
    from gpu_helpers import oracle_fp8, run_fp8
    from mla_inputs import fp8_case
    case = fp8_case([4096] * 64, s_q=1, seed=120, name="fp8 batched B=64 ctx=4096")
    o, lse = run_fp8(case)
    o_ref, l_ref = oracle_fp8(case)
    compare(o, lse, o_ref, l_ref, torch.bfloat16, case.name)


def test_fp8_partials_then_combine_matches_one_call():
    from gpu_helpers import run_fp8
    from mla_inputs import fp8_case
    case = fp8_case([2000, 700, 64], s_q=1, seed=121)
    d = to_device(case)
    p = mla.decode_plan(case.seqlens.tolist(), 1, 128, num_cus=16)
    offs = p.device_offsets("cuda")
    ws = torch.empty(p.workspace_bytes, dtype=torch.uint8, device="cuda")
    codes, scales = case.meta["cache_fp8"].cuda(), case.meta["row_scales"].cuda()
    mla.mla_decode_fwd_fp8(d["q_lat"], codes, scales, d["block_table"], d["seqlens"], case.scale, False,
                           split_offsets=offs, total_splits=p.total_splits, workspace=ws, partials_only=True)
    o_part, lse_part = mla.workspace_partials(ws, p.total_splits, 1, 128)
    o1, l1 = mla.mla_splitkv_combine(o_part, lse_part, offs, p.total_splits, case.B)
    o2, l2 = mla.mla_decode_fwd_fp8(d["q_lat"], codes, scales, d["block_table"], d["seqlens"], case.scale, False,
                                    split_offsets=offs, total_splits=p.total_splits)
    torch.cuda.synchronize()
    multi = torch.from_numpy(p.num_splits > 1)
    assert torch.equal(o1[multi], o2[multi]) and torch.equal(l1[multi], l2[multi])


# ---------------------------------------------------------------------------
# Expanded path (prefill / extend), chunked prefix, and the path choice
# ---------------------------------------------------------------------------

# The expanded path materialises K and V in bf16 (as any implementation of
# that path does), so each score carries the rounding of its 128 expanded key
# elements (relative 2^-9, uniform): with unit-variance q and k and scale
# 1/sqrt(192) the score error has standard deviation ~2^-9/sqrt(3) * sqrt(128/192)
# ~ 9e-4, and an LSE inherits at most the largest of its scores' errors. The
# bound 1e-2 is ~10 of those deviations, far below a wrong key or scale (an
# error of order 1). Outputs keep rel-L2 5e-3 and max-abs 2e-2 relative to
# their scale.
PREFILL_LSE_TOL = 1e-2


def _prefill_compare(o, lse, o_ref, l_ref, label):
    og, lg = to_np(o), to_np(lse)
    assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg)), label
    rel = np.linalg.norm(og - o_ref) / np.linalg.norm(o_ref)
    mabs = np.max(np.abs(og - o_ref))
    lerr = np.max(np.abs(lg - l_ref))
    print(f"[parity] {label} rel_l2={rel:.3e} max_abs={mabs:.3e} lse={lerr:.3e}", flush=True)
    assert rel <= 5e-3 and mabs <= 2e-2 * max(1.0, np.max(np.abs(o_ref))) and lerr <= PREFILL_LSE_TOL, \
        (label, rel, mabs, lerr)


@pytest.mark.parametrize("lens,s_q,H,chunk", [([300, 1000], 1, 16, 8192), ([300, 1000], 5, 16, 128),
                                              ([1000, 77], 77, 16, 100), ([2000], 300, 32, 512),
                                              ([640, 129], 129, 128, 256),
                                              # More chunks than one merge round of 16 holds: 17
                                              # (a second round of one), 63 and the full 64.
                                              ([1500, 400], 20, 8, 90), ([2000], 5, 16, 32),
                                              ([2048, 31], 3, 8, 32)])
def test_prefill_expanded(lens, s_q, H, chunk):
    from gpu_helpers import oracle_prefill
    from mla_inputs import prefill_case
    case = prefill_case(lens, s_q, H=H, seed=140 + s_q)
    m = case.meta
    d = to_device(case)
    o, lse = mla.mla_prefill_fwd(m["q_nope"].cuda(), m["q_rope"].cuda(), d["kv_cache"], d["block_table"], lens,
                                 m["w_uk"].cuda(), m["w_uv"].cuda(), case.scale, chunk_tokens=chunk)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle_prefill(case)
    _prefill_compare(o, lse, o_ref, l_ref, f"{case.name} lens={lens} chunk={chunk}")


def test_two_paths_agree_and_auto_choice():
    # Both paths on one extend batch (s_q = 8 new tokens): each against the
    # oracle of the expanded path, and "auto" picks the absorbed one here and
    # the expanded one for 300 new tokens (the crossover is ~171).
    from gpu_helpers import oracle_prefill
    from mla_inputs import prefill_case
    case = prefill_case([1000, 300], 8, H=128, seed=150)
    m = case.meta
    d = to_device(case)
    args = (m["q_nope"].cuda(), m["q_rope"].cuda(), d["kv_cache"], d["block_table"], d["seqlens"],
            m["w_uk"].cuda(), m["w_uv"].cuda(), case.scale)
    o_ref, l_ref = oracle_prefill(case)
    for path in ("absorbed", "expanded"):
        o, lse = mla.mla_attention_fwd(*args, path=path, chunk_tokens=512)
        torch.cuda.synchronize()
        _prefill_compare(o, lse, o_ref, l_ref, f"extend s_q=8 via {path}")
    assert mla.select_path(8, 1000) == "absorbed" and mla.select_path(300, 2000) == "expanded"


def _prefill_sampled(L, s_q, chunk, heads, seed):
    """The expanded path at a full workload size, checked on two blocks of 16
    query rows (the first and the last new tokens) for a few heads: each
    block is the last 16 tokens of a prefix of the sequence, which is how
    the oracle states it."""
    from mla_inputs import prefill_case
    case = prefill_case([L], s_q, H=128, seed=seed)
    m = case.meta
    d = to_device(case)
    o, lse = mla.mla_prefill_fwd(m["q_nope"].cuda(), m["q_rope"].cuda(), d["kv_cache"], d["block_table"], [L],
                                 m["w_uk"].cuda(), m["w_uv"].cuda(), case.scale, chunk_tokens=chunk)
    torch.cuda.synchronize()
    og, lg = to_np(o), to_np(lse)
    hs = list(heads)
    for first in (0, s_q - 16):
        rows = slice(first, first + 16)
        Lp = L - s_q + first + 16  # the block's last query sits at position Lp - 1
        o_ref, l_ref = orc.prefill_expanded(to_np(m["q_nope"][:, rows][:, :, hs]), to_np(m["q_rope"][:, rows][:, :, hs]),
                                            to_np(case.cache), case.block_table.numpy(), np.array([Lp]),
                                            to_np(m["w_uk"][hs]), to_np(m["w_uv"][hs]), case.scale)
        _prefill_compare(torch.from_numpy(og[:, rows][:, :, hs].copy()), torch.from_numpy(lg[:, rows][:, :, hs].copy()),
                         o_ref, l_ref, f"L={L} s_q={s_q} chunk={chunk} rows {first}..{first + 15} heads {hs}")


def test_prefill_8k_sampled():
    # The prefill bench workload: a fresh 8K-token prefill, one 8192-token chunk.
    _prefill_sampled(8192, 8192, 8192, (0, 77, 127), seed=160)


def test_extend_32k_sampled():
    # The extend bench workload: 512 new tokens after 32K, five chunks merged by LSE.
    _prefill_sampled(32768 + 512, 512, 8192, (0, 127), seed=161)


# ---------------------------------------------------------------------------
# FP8 products for the absorption
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(3, 5, 16), (64, 128, 128), (7, 3, 37), (1, 1, 1)])
def test_quantize_e4m3_codes_bitexact(shape):
    # The codes are integers decided in fp32 on both sides: compare exactly.
    rng = np.random.default_rng(171 + len(shape) + shape[-1])
    x = rng.standard_normal(shape).astype(np.float32) * np.float32(3.0)
    x.reshape(-1)[::11] *= np.float32(1e-3)   # values in the subnormal codes
    x.reshape(-1)[1::13] = -0.0
    xb = torch.from_numpy(x).to(torch.bfloat16)
    codes, scale = mla.quantize_e4m3(xb.cuda())
    torch.cuda.synchronize()
    ref_codes, ref_scale = orc.quantize_e4m3(xb.float().numpy())
    assert float(scale.item()) == float(ref_scale)
    got = codes.cpu().numpy()
    bad = np.flatnonzero(got.reshape(-1) != ref_codes.reshape(-1))
    assert bad.size == 0, (bad[:8], got.reshape(-1)[bad[:8]], ref_codes.reshape(-1)[bad[:8]])


def _fp8_compare(got, ref, label):
    g = to_np(got)
    rel = np.linalg.norm(g - ref) / np.linalg.norm(ref)
    mabs = np.max(np.abs(g - ref))
    print(f"[parity] {label} rel_l2={rel:.3e} max_abs={mabs:.3e}", flush=True)
    assert np.all(np.isfinite(g)) and rel <= 5e-3 and mabs <= 2e-2 * max(1.0, np.max(np.abs(ref))), (label, rel, mabs)


@pytest.mark.parametrize("N,H,dn,dr,dc,dv", [(37, 3, 48, 8, 208, 72), (9, 2, 128, 64, 640, 40),
                                            (70, 2, 128, 4, 144, 20)])
def test_fp8_products_odd_shapes(N, H, dn, dr, dc, dv):
    # A contracted length other than the staged forms' fixed 128 / 512
    # (generic staging), partial weight slabs, (second case) a contracted
    # length past 512, which takes the direct-load kernel, and (third) a RoPE
    # tail and output rows that are not 16-byte multiples, which the staged
    # kernel stores piece by piece from the MFMA layout, over two token rounds.
    from mla_inputs import fp8_bmm_case
    c = fp8_bmm_case(N, H=H, d_nope=dn, d_rope=dr, d_c=dc, d_v=dv, seed=180 + N)
    q_lat = mla.mla_absorb_q_fp8(c["q_nope"].cuda(), c["q_rope"].cuda(), c["w_uk_codes"].cuda(), c["w_uk_scale"])
    out = mla.mla_out_uv_fp8(c["o_lat"].cuda(), c["w_uv_t_codes"].cuda(), c["w_uv_scale"])
    torch.cuda.synchronize()
    ref_q = orc.absorb_q_fp8(c["q_nope"].float().numpy(), c["q_rope"].float().numpy(), c["w_uk_codes"].numpy(),
                             c["w_uk_scale"])
    ref_o = orc.out_uv_fp8(c["o_lat"].float().numpy(), c["w_uv_t_codes"].numpy(), c["w_uv_scale"])
    _fp8_compare(q_lat[..., :dc], ref_q[..., :dc], f"absorb_q_fp8 N={N} H={H} dn={dn} dc={dc}")
    _fp8_compare(out, ref_o, f"out_uv_fp8 N={N} H={H} dc={dc} dv={dv}")
    assert torch.equal(q_lat[..., dc:].cpu(), c["q_rope"])


@pytest.mark.parametrize("N,H", [(64, 128), (5, 3), (33, 16), (130, 2)])
def test_absorb_q_fp8(N, H):
    from mla_inputs import fp8_bmm_case
    c = fp8_bmm_case(N, H=H, seed=172 + N)
    q_lat = mla.mla_absorb_q_fp8(c["q_nope"].cuda(), c["q_rope"].cuda(), c["w_uk_codes"].cuda(), c["w_uk_scale"])
    torch.cuda.synchronize()
    ref = orc.absorb_q_fp8(c["q_nope"].float().numpy(), c["q_rope"].float().numpy(), c["w_uk_codes"].numpy(),
                           c["w_uk_scale"])
    _fp8_compare(q_lat[..., :512], ref[..., :512], f"absorb_q_fp8 N={N} H={H}")
    assert torch.equal(q_lat[..., 512:].cpu(), c["q_rope"])  # the RoPE part is copied


@pytest.mark.parametrize("N,H", [(64, 128), (5, 3), (33, 16), (130, 2)])
def test_out_uv_fp8(N, H):
    from mla_inputs import fp8_bmm_case
    c = fp8_bmm_case(N, H=H, seed=173 + N)
    out = mla.mla_out_uv_fp8(c["o_lat"].cuda(), c["w_uv_t_codes"].cuda(), c["w_uv_scale"])
    torch.cuda.synchronize()
    ref = orc.out_uv_fp8(c["o_lat"].float().numpy(), c["w_uv_t_codes"].numpy(), c["w_uv_scale"])
    _fp8_compare(out, ref, f"out_uv_fp8 N={N} H={H}")

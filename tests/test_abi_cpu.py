"""CPU checks of the C ABI: the library loads, exports every declared entry
point, and host-side planning and argument validation behave as the header
documents. Nothing here launches device work."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import mla_decode_fwd_amd as mla
from mla_decode_fwd_amd import accounting

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_decode.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return mla.load_library()


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"mla_decode_fwd", "mla_splitkv_combine", "mla_absorb_q", "mla_out_uv",
            "mla_decode_plan"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", mla.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if " T " in line)
    for n in names:
        assert n in exported, n
        assert getattr(lib, n) is not None


def test_status_strings_and_version(lib):
    assert mla.abi_version() == 8
    for code in range(5):
        assert lib.mla_status_string(code)
    assert lib.mla_status_string(99) == b"unknown status"


def test_workspace_size(lib):
    assert mla.decode_workspace_size(256, 1, 128) == 256 * 128 * 513 * 4
    assert mla.decode_workspace_size(0, 1, 128) == 0
    assert mla.decode_workspace_size(3, 2, 5) % 256 == 0


def test_plan_headline_batch_fills_the_chip():
    # A workgroup covers all 128 head rows, so 64 sequences x 64 pages over
    # 256 compute units give chunks of 16 pages: 4 per sequence, 256 chunks =
    # one workgroup per compute unit.
    p = mla.decode_plan([4096] * 64, s_q=1, H=128)
    assert (p.num_splits == 4).all() and p.total_splits == 256
    assert p.workspace_bytes == mla.decode_workspace_size(256, 1, 128)
    assert np.array_equal(p.split_offsets, np.arange(65) * 4)


def test_plan_long_context_respects_cap_and_balances():
    lens = [65536, 32768, 16384, 8192, 4096, 2048, 1024, 513]
    p = mla.decode_plan(lens, s_q=1, H=128)
    assert p.num_splits.max() <= 64 and p.num_splits.min() >= 1
    assert p.num_splits[0] == 64
    pages = [(L + 63) // 64 for L in lens]
    per_chunk = max(-(-P // n) for P, n in zip(pages, p.num_splits))
    assert per_chunk == 16  # the longest sequence bounds the chunk size
    assert p.split_offsets[-1] == p.num_splits.sum()


def test_plan_single_short_sequence_is_not_split():
    p = mla.decode_plan([100], s_q=1, H=128, num_cus=1)
    assert p.total_splits == 1 and p.workspace_bytes == 0 and not p.any_split


def test_plan_invalid_arguments(lib):
    L = np.array([10, 3], dtype=np.int32)
    ns = np.zeros(2, np.int32)
    off = np.zeros(3, np.int32)
    c = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    assert lib.mla_decode_plan(c(L), 2, 4, 128, 256, 64, c(ns), c(off), None) == INVALID  # L < s_q
    assert lib.mla_decode_plan(c(L), 2, 1, 128, 256, 65, c(ns), c(off), None) == INVALID
    assert lib.mla_decode_plan(c(L), 2, 1, 128, 256, 0, c(ns), c(off), None) == INVALID
    assert lib.mla_decode_plan(None, 2, 1, 128, 256, 64, c(ns), c(off), None) == INVALID
    assert lib.mla_decode_plan(c(L), 0, 1, 128, 256, 64, c(ns), c(off), None) == INVALID
    assert lib.mla_decode_plan(c(L), 2, 1, 128, 256, 64, c(ns), c(off), None) == OK


def _fwd(lib, **kw):
    a = dict(q=FAKE, kv=FAKE, bt=FAKE, sl=FAKE, so=None, total=2, B=2, s_q=1, H=128, dqk=576, dv=512,
             page=64, maxp=4, npages=8, scale=0.0722, causal=0, dtype=0, ws=None, wsb=0, o=FAKE,
             lse=FAKE)
    a.update(kw)
    return lib.mla_decode_fwd(a["q"], a["kv"], a["bt"], a["sl"], a["so"], a["total"], a["B"], a["s_q"],
                              a["H"], a["dqk"], a["dv"], a["page"], a["maxp"], a["npages"], a["scale"],
                              a["causal"], a["dtype"], a["ws"], a["wsb"], a["o"], a["lse"], None)


def test_decode_fwd_validation(lib):
    assert _fwd(lib, q=None) == INVALID
    assert _fwd(lib, lse=None) == INVALID
    assert _fwd(lib, o=None) == INVALID
    assert _fwd(lib, o=None, lse=None) == INVALID  # partials only needs split offsets
    assert _fwd(lib, o=None, lse=None, so=FAKE, total=4, ws=None, wsb=0) == WORKSPACE
    assert _fwd(lib, B=0) == INVALID
    assert _fwd(lib, npages=0) == INVALID
    assert _fwd(lib, scale=float("nan")) == INVALID
    assert _fwd(lib, scale=0.0) == INVALID
    assert _fwd(lib, scale=-0.07) == INVALID
    assert _fwd(lib, dqk=128) == UNSUPPORTED
    assert _fwd(lib, dv=128) == UNSUPPORTED
    assert _fwd(lib, page=16) == UNSUPPORTED
    assert _fwd(lib, H=129) == UNSUPPORTED
    assert _fwd(lib, s_q=17) == UNSUPPORTED
    assert _fwd(lib, dtype=7) == UNSUPPORTED
    assert _fwd(lib, total=3) == INVALID  # no split offsets: one chunk per sequence
    assert _fwd(lib, so=FAKE, total=1) == INVALID  # fewer chunks than sequences
    assert _fwd(lib, so=FAKE, total=129) == INVALID  # more than 64 per sequence
    assert _fwd(lib, so=FAKE, total=4, ws=None, wsb=1 << 30) == WORKSPACE
    need = mla.decode_workspace_size(4, 1, 128)
    assert _fwd(lib, so=FAKE, total=4, ws=FAKE, wsb=need - 1) == WORKSPACE


def _noalloc(lib, **kw):
    a = dict(q=FAKE, kv=FAKE, bt=FAKE, sl=FAKE, so=FAKE, total=4, B=2, s_q=1, H=128, dqk=576, dv=512,
             page=64, maxp=4, npages=8, scale=0.0722, causal=0, dtype=0, o=FAKE, lse=FAKE)
    a.update(kw)
    return lib.mla_decode_fwd_noalloc(a["q"], a["kv"], a["bt"], a["sl"], a["so"], a["total"], a["B"], a["s_q"],
                                      a["H"], a["dqk"], a["dv"], a["page"], a["maxp"], a["npages"], a["scale"],
                                      a["causal"], a["dtype"], a["o"], a["lse"], None)


def test_noalloc_validation_and_scratch_size(lib):
    # Every refusal below comes before any HIP call (none is possible here).
    assert mla.NOALLOC_SCRATCH_BYTES == 64 << 20
    bf16_rows = 510 * 128
    assert mla.noalloc_scratch_bytes(510, 1, 128) == bf16_rows * 1024 + bf16_rows * 4
    assert mla.noalloc_scratch_bytes(510, 1, 128) <= mla.NOALLOC_SCRATCH_BYTES
    assert mla.noalloc_scratch_bytes(511, 1, 128) > mla.NOALLOC_SCRATCH_BYTES
    assert lib.mla_decode_noalloc_scratch_bytes(4, 1, 128, 1) == 4 * 128 * 2048 + 4 * 128 * 4
    assert lib.mla_decode_noalloc_scratch_bytes(0, 1, 128, 0) == 0
    assert lib.mla_decode_noalloc_scratch_bytes(4, 1, 128, 9) == 0
    assert _noalloc(lib, o=None) == INVALID          # outputs are required
    assert _noalloc(lib, lse=None) == INVALID
    assert _noalloc(lib, q=None) == INVALID
    assert _noalloc(lib, dqk=128) == UNSUPPORTED
    assert _noalloc(lib, dtype=7) == UNSUPPORTED
    assert _noalloc(lib, H=129) == UNSUPPORTED
    assert _noalloc(lib, total=1) == INVALID         # fewer chunks than sequences
    assert _noalloc(lib, total=129) == INVALID       # more than 64 per sequence
    assert _noalloc(lib, B=16, total=511) == WORKSPACE   # over the static array
    assert _noalloc(lib, B=16, total=256, dtype=1) == WORKSPACE  # fp32 partials: 255 chunks at most
    assert _noalloc(lib, so=None, total=3) == INVALID  # no split offsets: one chunk per sequence


def test_combine_and_bmm_validation(lib):
    assert lib.mla_splitkv_combine(None, FAKE, FAKE, 2, 2, 1, 128, 512, 0, FAKE, FAKE, None) == INVALID
    assert lib.mla_splitkv_combine(FAKE, FAKE, FAKE, 1, 2, 1, 128, 512, 0, FAKE, FAKE, None) == INVALID
    assert lib.mla_splitkv_combine(FAKE, FAKE, FAKE, 2, 2, 1, 128, 256, 0, FAKE, FAKE, None) == UNSUPPORTED
    assert lib.mla_splitkv_combine(FAKE, FAKE, FAKE, 2, 2, 1, 128, 512, 5, FAKE, FAKE, None) == UNSUPPORTED
    assert lib.mla_absorb_q(FAKE, None, FAKE, 4, 128, 128, 64, 512, 0, FAKE, None) == INVALID
    assert lib.mla_absorb_q(FAKE, FAKE, FAKE, 0, 128, 128, 64, 512, 0, FAKE, None) == INVALID
    assert lib.mla_absorb_q(FAKE, FAKE, FAKE, 4, 128, 128, 64, 8192, 0, FAKE, None) == UNSUPPORTED
    assert lib.mla_absorb_q(FAKE, FAKE, FAKE, 4, 128, 128, 64, 512, 9, FAKE, None) == UNSUPPORTED
    assert lib.mla_out_uv(FAKE, None, 4, 128, 512, 128, 0, FAKE, None) == INVALID
    assert lib.mla_out_uv(FAKE, FAKE, 4, 2000, 512, 128, 0, FAKE, None) == UNSUPPORTED


def _sparse(lib, **kw):
    a = dict(q=FAKE, kv=FAKE, bt=FAKE, sl=FAKE, idx=FAKE, topk=2048, so=None, total=2, B=2, s_q=1, H=128,
             dqk=576, dv=512, page=64, maxp=4, npages=8, scale=0.0722, dtype=0, ws=None, wsb=0, o=FAKE,
             lse=FAKE)
    a.update(kw)
    return lib.mla_sparse_decode_fwd(a["q"], a["kv"], a["bt"], a["sl"], a["idx"], a["topk"], a["so"], a["total"],
                                     a["B"], a["s_q"], a["H"], a["dqk"], a["dv"], a["page"], a["maxp"],
                                     a["npages"], a["scale"], a["dtype"], a["ws"], a["wsb"], a["o"], a["lse"],
                                     None)


def test_sparse_decode_validation(lib):
    assert _sparse(lib, idx=None) == INVALID
    assert _sparse(lib, topk=0) == UNSUPPORTED
    assert _sparse(lib, topk=2049) == UNSUPPORTED
    assert _sparse(lib, H=64) == UNSUPPORTED  # one row group per new token needs H = 128
    assert _sparse(lib, dtype=1) == UNSUPPORTED  # bf16 only
    assert _sparse(lib, dtype=7) == UNSUPPORTED
    assert _sparse(lib, q=None) == INVALID
    assert _sparse(lib, scale=0.0) == INVALID
    assert _sparse(lib, total=3) == INVALID
    assert _sparse(lib, so=FAKE, total=4, ws=None, wsb=1 << 30) == WORKSPACE
    assert _sparse(lib, o=None, lse=None) == INVALID


def test_sparse_plan_cuts_the_list():
    p = mla.sparse_decode_plan(64, 2048)
    assert p.total_splits == 256 and int(p.num_splits.max()) == 4
    p1 = mla.sparse_decode_plan(1, 2048)
    assert p1.total_splits == 32  # 32 pages of list, one per chunk at most


def test_fp8_decode_validation(lib):
    def call(**kw):
        a = dict(q=FAKE, kv=FAKE, sc=FAKE, bt=FAKE, sl=FAKE, so=None, total=2, B=2, s_q=1, H=128, dqk=576,
                 dv=512, page=64, maxp=4, npages=8, scale=0.0722, causal=0, ws=None, wsb=0, o=FAKE, lse=FAKE)
        a.update(kw)
        return lib.mla_decode_fwd_fp8(a["q"], a["kv"], a["sc"], a["bt"], a["sl"], a["so"], a["total"], a["B"],
                                      a["s_q"], a["H"], a["dqk"], a["dv"], a["page"], a["maxp"], a["npages"],
                                      a["scale"], a["causal"], a["ws"], a["wsb"], a["o"], a["lse"], None)
    assert call(sc=None) == INVALID
    assert call(kv=None) == INVALID
    assert call(dqk=512) == UNSUPPORTED
    assert call(scale=-1.0) == INVALID
    assert call(so=FAKE, total=4, ws=None, wsb=0) == WORKSPACE
    assert call(o=None) == INVALID


def test_select_path_matches_the_printed_choices(lib):
    # [MLA-推理] "谁快": decode over 8K -> absorbed, prefill 8K -> expanded,
    # 64 new tokens after 32K -> absorbed, 512 after 32K -> expanded.
    assert mla.select_path(1, 8192) == "absorbed"
    assert mla.select_path(8192, 8192) == "expanded"
    assert mla.select_path(64, 32768 + 64) == "absorbed"
    assert mla.select_path(512, 32768 + 512) == "expanded"
    assert lib.mla_select_path(0, 10) == -1 and lib.mla_select_path(5, 4) == -1


def test_prefill_validation(lib):
    L = np.array([100, 200], dtype=np.int32)
    c = L.ctypes.data_as(ctypes.c_void_p)

    def call(**kw):
        a = dict(qn=FAKE, qr=FAKE, kv=FAKE, bt=FAKE, L=c, B=2, s_q=4, H=16, maxp=4, npages=8, wuk=FAKE, wuv=FAKE,
                 chunk=64, scale=0.07, ws=FAKE, wsb=1 << 40, o=FAKE, lse=FAKE)
        a.update(kw)
        return lib.mla_prefill_fwd(a["qn"], a["qr"], a["kv"], a["bt"], a["L"], a["B"], a["s_q"], a["H"], a["maxp"],
                                   a["npages"], a["wuk"], a["wuv"], a["chunk"], a["scale"], a["ws"], a["wsb"],
                                   a["o"], a["lse"], None)
    assert call(qn=None) == INVALID
    assert call(L=None) == INVALID
    assert call(chunk=0) == INVALID
    assert call(scale=0.0) == INVALID
    assert call(H=129) == INVALID
    assert call(s_q=101) == INVALID          # L_0 = 100 < s_q
    assert call(maxp=1) == INVALID           # 200 tokens > 64 * 1
    assert call(chunk=3) == UNSUPPORTED      # 67 chunks > 64
    assert call(ws=None) == WORKSPACE
    need = mla.prefill_workspace_size(4, 16, 64, 4)
    assert call(wsb=need - 1) == WORKSPACE
    assert mla.prefill_workspace_size(0, 16, 64, 4) == 0


def test_fp8_products_validation(lib):
    ws = mla.fp8_workspace_size(4 * 8 * 128)
    assert ws == 1024 and mla.fp8_workspace_size(0) == 0

    def absorb(**kw):
        a = dict(qn=FAKE, qr=FAKE, w=FAKE, s=0.5, N=4, H=8, dn=128, dr=64, dc=512, ws=FAKE, wsb=1 << 30, out=FAKE)
        a.update(kw)
        return lib.mla_absorb_q_fp8(a["qn"], a["qr"], a["w"], a["s"], a["N"], a["H"], a["dn"], a["dr"], a["dc"],
                                    a["ws"], a["wsb"], a["out"], None)
    assert absorb(qn=None) == INVALID
    assert absorb(qr=None) == INVALID
    assert absorb(s=0.0) == INVALID and absorb(s=float("nan")) == INVALID
    assert absorb(N=0) == INVALID
    assert absorb(dn=120) == UNSUPPORTED     # not a multiple of 16
    assert absorb(dc=510) == UNSUPPORTED     # not a multiple of 4
    assert absorb(H=1025) == UNSUPPORTED
    assert absorb(qn=ctypes.c_void_p(0x1008)) == INVALID  # q_nope not 16-byte aligned
    assert absorb(ws=None) == WORKSPACE
    assert absorb(wsb=mla.fp8_workspace_size(4 * 8 * 128) - 1) == WORKSPACE

    def out_uv(**kw):
        a = dict(o=FAKE, w=FAKE, s=0.5, N=4, H=8, dc=512, dv=128, ws=FAKE, wsb=1 << 30, out=FAKE)
        a.update(kw)
        return lib.mla_out_uv_fp8(a["o"], a["w"], a["s"], a["N"], a["H"], a["dc"], a["dv"], a["ws"], a["wsb"],
                                  a["out"], None)
    assert out_uv(w=None) == INVALID
    assert out_uv(dc=100) == UNSUPPORTED
    assert out_uv(out=ctypes.c_void_p(0x1004)) == INVALID
    assert out_uv(wsb=mla.fp8_workspace_size(4 * 8 * 512) - 1) == WORKSPACE
    assert lib.mla_quantize_e4m3(FAKE, 0, FAKE, 1024, FAKE, FAKE, None) == INVALID
    assert lib.mla_quantize_e4m3(FAKE, 64, FAKE, 1023, FAKE, FAKE, None) == WORKSPACE


# ---------------------------------------------------------------------------
# Balanced schedule (mla_decode_schedule)
# ---------------------------------------------------------------------------

def _check_schedule(s, lens, s_q, H, num_cus, max_splits):
    """Structural invariants of a schedule: every sequence's pages are tiled
    by its chunks in order, within the cap; each segment is a run of
    consecutive chunks over consecutive global pages; the launch fits."""
    P = [(int(L) + 63) // 64 for L in lens]
    ch = s.chunks
    off = s.split_offsets
    assert off[0] == 0 and off[-1] == len(ch) == s.total_splits
    for b, L in enumerate(lens):
        mine = ch[off[b]:off[b + 1]]
        assert 1 <= len(mine) <= max_splits
        assert (mine[:, 0] == b).all() and (mine[:, 3] == L).all()
        assert mine[0, 1] == 0 and mine[-1, 2] == P[b]
        assert (mine[1:, 1] == mine[:-1, 2]).all() and (mine[:, 2] > mine[:, 1]).all()
    start = np.concatenate([[0], np.cumsum(P)])
    g0 = start[ch[:, 0]] + ch[:, 1]  # global first page of every chunk
    sf = s.segment_first_chunk
    assert sf[0] == 0 and sf[-1] == len(ch) and (np.diff(sf) >= 1).all()
    seg_pages = []
    for i in range(s.num_segments):
        c = np.arange(sf[i], sf[i + 1])
        assert (g0[c[1:]] == g0[c[:-1]] + (ch[c[:-1], 2] - ch[c[:-1], 1])).all()  # contiguous pages
        seg_pages.append(int((ch[c, 2] - ch[c, 1]).sum()))
    groups = -(-(s_q * H) // s.rows_per_group)
    assert s.num_segments * groups <= max(num_cus, groups)
    return seg_pages


@pytest.mark.parametrize("lens,s_q,H,num_cus", [([4096] * 64, 1, 128, 256), ([65536, 32768, 16384, 8192, 4096, 2048,
                                                                              1024, 513], 1, 128, 256),
                                                 ([4096], 1, 128, 256), ([300, 64, 129, 7], 2, 128, 8),
                                                 ([33, 250], 1, 1, 16), ([190], 16, 8, 64)])
def test_schedule_structure(lens, s_q, H, num_cus):
    s = mla.decode_schedule(lens, s_q, H, num_cus=num_cus)
    _check_schedule(s, lens, s_q, H, num_cus, 64)
    assert s.workspace_bytes == mla.decode_workspace_size(s.total_splits, s_q, H)


def test_schedule_balances_the_workload_shapes():
    # B=64 x 4096: 256 segments of exactly 16 pages, 128-row groups (the
    # equal-split plan's shape).
    s = mla.decode_schedule([4096] * 64, 1, 128)
    assert s.rows_per_group == 128 and s.num_segments == 256 and s.total_splits == 256
    assert set(_check_schedule(s, [4096] * 64, 1, 128, 256, 64)) == {16}
    # Long context: with 128-row groups the 64K sequence would need 128
    # chunks of 8 pages; 64-row groups give 128 segments of <= 16 pages (256
    # workgroups) and exactly 64 chunks for it.
    lens = [65536, 32768, 16384, 8192, 4096, 2048, 1024, 513]
    s = mla.decode_schedule(lens, 1, 128)
    pages = _check_schedule(s, lens, 1, 128, 256, 64)
    assert s.rows_per_group == 64 and s.num_segments == 128 and max(pages) == 16
    assert s.num_splits[0] == 64
    # MTP s_q = 2, lengths U{1024..8192}: 128 segments (two row groups each)
    # cut to equal cost, pages + 2 per chunk (a chunk's fixed work in pages),
    # so segments that start or cross more sequences hold fewer pages. The
    # costliest segment is within a chunk and a page of the mean, and below
    # the costliest of equal-page segments.
    rng = np.random.default_rng(3)
    lens = rng.integers(1024, 8193, 128).tolist()
    s = mla.decode_schedule(lens, 2, 128)
    pages = np.array(_check_schedule(s, lens, 2, 128, 256, 64))
    assert s.rows_per_group == 128 and s.num_segments == 128
    cost = pages + 2.0 * np.diff(s.segment_first_chunk)
    assert cost.max() <= cost.sum() / 128 + 3.0, (cost.max(), cost.sum() / 128)
    assert cost.max() < _equal_page_max_cost(lens, 128), cost.max()


def test_schedule_cap_and_forced_row_groups():
    lens = [64 * 1000, 64]
    for rpg in (64, 128):
        s = mla.decode_schedule(lens, 1, 128, rows_per_group=rpg)
        assert s.rows_per_group == rpg
        _check_schedule(s, lens, 1, 128, 256, 64)
    s = mla.decode_schedule(lens, 1, 128, max_splits=5)
    assert s.num_splits.max() <= 5
    _check_schedule(s, lens, 1, 128, 256, 5)
    s = mla.decode_schedule([500, 70, 3000], 1, 128, max_splits=1)
    assert (s.num_splits == 1).all() and s.num_segments == 3


def test_schedule_invalid_arguments(lib):
    L = np.array([100, 3], np.int32)
    off = np.zeros(3, np.int32)
    sched = np.zeros(64, np.int32)
    n, r = ctypes.c_int(0), ctypes.c_int(0)
    c = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    call = lambda *a: lib.mla_decode_schedule(*a)
    assert call(c(L), 2, 4, 128, 256, 64, 0, c(off), c(sched), 64, ctypes.byref(n), ctypes.byref(r), None) == INVALID
    assert call(c(L), 2, 1, 128, 256, 65, 0, c(off), c(sched), 64, ctypes.byref(n), ctypes.byref(r), None) == INVALID
    assert call(c(L), 2, 1, 128, 256, 64, 32, c(off), c(sched), 64, ctypes.byref(n), ctypes.byref(r), None) == INVALID
    assert call(c(L), 2, 1, 128, 256, 64, 0, c(off), c(sched), 3, ctypes.byref(n), ctypes.byref(r), None) == WORKSPACE
    assert call(c(L), 2, 1, 128, 256, 64, 0, c(off), c(sched), 64, ctypes.byref(n), ctypes.byref(r), None) == OK
    # The scheduled decode's own checks (no launch): bf16 only, a schedule
    # needs split offsets, a known row-group size and a plausible segment count.
    f = lib.mla_decode_fwd_scheduled
    base = dict(so=FAKE, sched=FAKE, nseg=2, rpg=128, total=4, dtype=0)

    def fwd(**kw):
        a = dict(base, **kw)
        return f(FAKE, FAKE, FAKE, FAKE, a["so"], a["sched"], a["nseg"], a["rpg"], a["total"], 2, 1, 128, 576, 512, 64,
                 4, 8, 0.0722, 0, a["dtype"], FAKE, 1 << 30, FAKE, FAKE, None)
    assert fwd(sched=None) == INVALID
    assert fwd(so=None) == INVALID
    assert fwd(dtype=1) == UNSUPPORTED
    assert fwd(rpg=32) == INVALID
    assert fwd(nseg=0) == INVALID
    assert fwd(nseg=5) == INVALID  # more segments than chunks


def test_clock_probe_rejects_a_negative_capacity(lib):
    # Checked before any HIP call: a buffer with a negative capacity.
    assert lib.mla_decode_clock_probe(FAKE, -1) == INVALID


@pytest.mark.parametrize("seed,B,num_cus,max_splits", [(0, 700, 256, 64), (1, 50, 256, 3), (2, 1, 256, 64),
                                                       (3, 300, 16, 64), (4, 9, 1000, 64)])
def test_schedule_random_batches_are_tiled_within_the_cap(seed, B, num_cus, max_splits):
    # Mixed lengths (1 token .. 40K), more or fewer sequences than segments,
    # tight caps: every page is covered once, in order, within the cap and
    # the segment count, and (128-row groups) no segment costs more than the
    # costliest segment of an equal-page cut into as many segments.
    rng = np.random.default_rng(seed)
    lens = np.maximum(1, (rng.pareto(1.2, B) * 2000).astype(int) % 40000).tolist()
    s = mla.decode_schedule(lens, 1, 128, num_cus=num_cus, max_splits=max_splits)
    pages = np.array(_check_schedule(s, lens, 1, 128, num_cus, max_splits))
    assert pages.sum() == sum((L + 63) // 64 for L in lens)
    if s.rows_per_group == 128 and max_splits > 1:
        cost = pages + 2.0 * np.diff(s.segment_first_chunk)
        assert cost.max() <= _equal_page_max_cost(lens, s.num_segments) + 1e-9


def _equal_page_max_cost(lens, G):
    """Costliest segment (pages + 2 per chunk) when the concatenated pages are
    cut into segments of ceil(total / G) pages."""
    P = np.array([(L + 63) // 64 for L in lens])
    seg = -(-int(P.sum()) // G)
    start = np.concatenate([[0], np.cumsum(P)])
    n_seg = -(-int(P.sum()) // seg)
    chunks = np.zeros(n_seg, int)
    for b in range(len(P)):
        for g in range(start[b] // seg, (start[b + 1] - 1) // seg + 1):
            chunks[g] += 1
    return float((np.minimum(seg, P.sum() - seg * np.arange(n_seg)) + 2.0 * chunks).max())

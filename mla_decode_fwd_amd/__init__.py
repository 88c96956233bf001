"""Python binding of the MI355X absorbed-MLA decode library (libmla_decode.so).

Thin ctypes marshalling over the C ABI in include/mla_decode.h: every function
here checks tensor properties, allocates outputs with torch when the caller
does not pass them, and calls the library entry point of the same name. All
computation happens in the library's HIP kernels; there is no fallback. If
the library is not built, every call raises.

Tensors are torch tensors on the current HIP device (row-major, contiguous);
work is enqueued on torch's current stream.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch

__all__ = [
    "MlaError", "library_path", "load_library", "abi_version",
    "decode_plan", "decode_workspace_size", "mla_decode_fwd", "mla_splitkv_combine",
    "mla_absorb_q", "mla_out_uv", "DecodePlan", "workspace_partials",
    "PreparedCall", "prepare_decode", "prepare_combine",
    "mla_sparse_decode_fwd", "sparse_decode_plan", "prepare_sparse_decode",
    "mla_decode_fwd_fp8", "prepare_decode_fp8",
    "select_path", "prefill_workspace_size", "mla_prefill_fwd", "mla_attention_fwd",
    "fp8_workspace_size", "quantize_e4m3", "mla_absorb_q_fp8", "mla_out_uv_fp8",
    "mla_decode_fwd_noalloc", "noalloc_scratch_bytes", "NOALLOC_SCRATCH_BYTES",
    "DecodeSchedule", "decode_schedule", "decode_clock_probe",
    "D_QK", "D_V", "PAGE_SIZE", "MAX_SPLITS", "MAX_DECODE_SQ",
]

D_QK = 576
D_V = 512
PAGE_SIZE = 64
MAX_DECODE_SQ = 16  # query tokens per sequence the decode kernel takes
MAX_SPLITS = 64

MLA_BF16 = 0
MLA_FP32 = 1
_DTYPES = {torch.bfloat16: MLA_BF16, torch.float32: MLA_FP32}

_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported shape or dtype",
           3: "workspace missing or too small", 4: "HIP runtime error"}

_LIB = None


class MlaError(RuntimeError):
    """A library call returned a non-zero status."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {_STATUS.get(status, 'unknown')} (status {status})")


def library_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla_decode.so")


def load_library():
    """Load libmla_decode.so (once). Raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with mla_decode_fwd_amd.build.build_library() "
                           "(hipcc, gfx950); there is no fallback implementation")
    lib = ctypes.CDLL(path)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    sig = {
        "mla_status_string": ([I], ctypes.c_char_p),
        "mla_abi_version": ([], I),
        "mla_decode_workspace_size": ([I, I, I], Z),
        "mla_decode_clock_probe": ([P, I], I),
        "mla_decode_plan": ([P, I, I, I, I, I, P, P, P], I),
        "mla_decode_fwd": ([P, P, P, P, P, I, I, I, I, I, I, I, I, I, F, I, I, P, Z, P, P, P], I),
        "mla_sparse_decode_fwd": ([P, P, P, P, P, I, P, I, I, I, I, I, I, I, I, I, F, I, P, Z, P, P, P], I),
        "mla_decode_fwd_fp8": ([P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, F, I, P, Z, P, P, P], I),
        "mla_select_path": ([I, I], I),
        "mla_prefill_workspace_size": ([I, I, I, I], Z),
        "mla_prefill_fwd": ([P, P, P, P, P, I, I, I, I, I, P, P, I, F, P, Z, P, P, P], I),
        "mla_splitkv_combine": ([P, P, P, I, I, I, I, I, I, P, P, P], I),
        "mla_absorb_q": ([P, P, P, I, I, I, I, I, I, P, P], I),
        "mla_out_uv": ([P, P, I, I, I, I, I, P, P], I),
        "mla_fp8_workspace_size": ([Z], Z),
        "mla_quantize_e4m3": ([P, Z, P, Z, P, P, P], I),
        "mla_absorb_q_fp8": ([P, P, P, F, I, I, I, I, I, P, Z, P, P], I),
        "mla_out_uv_fp8": ([P, P, F, I, I, I, I, P, Z, P, P], I),
        "mla_decode_noalloc_scratch_bytes": ([I, I, I, I], Z),
        "mla_decode_schedule_capacity": ([I, I], Z),
        "mla_decode_schedule": ([P, I, I, I, I, I, I, P, P, Z, P, P, P], I),
        "mla_decode_fwd_scheduled": ([P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, I, I, F, I, I, P, Z, P, P, P], I),
        "mla_decode_fwd_noalloc": ([P, P, P, P, P, I, I, I, I, I, I, I, I, I, F, I, I, P, P, P], I),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _LIB = lib
    return lib


def abi_version() -> int:
    return load_library().mla_abi_version()


def _check(fn: str, status: int):
    if status != 0:
        raise MlaError(fn, status)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t: torch.Tensor, name: str, dtype=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}")


def decode_workspace_size(total_splits: int, s_q: int, H: int) -> int:
    return int(load_library().mla_decode_workspace_size(int(total_splits), int(s_q), int(H)))


def decode_clock_probe(buffer: Optional[torch.Tensor]) -> None:
    """Clock stamps of the bf16 decode kernel (mla_decode_clock_probe): with a
    device int64 tensor of 2 * capacity elements, workgroup x of later launches
    on its device writes [shader cycles, 100 MHz ticks] at buffer[2x:2x+2];
    None switches them off (on the current device)."""
    if buffer is None:
        st = load_library().mla_decode_clock_probe(None, 0)
    else:
        _need(buffer, "buffer", dtype=torch.int64)
        if buffer.dim() != 1 or buffer.numel() % 2:
            raise ValueError("buffer must be a 1-D int64 tensor of 2 * capacity elements")
        st = load_library().mla_decode_clock_probe(_ptr(buffer), buffer.numel() // 2)
    _check("mla_decode_clock_probe", st)


class DecodePlan:
    """A split plan: per-sequence chunk counts, their offsets and workspace size."""

    def __init__(self, num_splits: np.ndarray, split_offsets: np.ndarray, workspace_bytes: int, s_q: int, H: int):
        self.num_splits = num_splits
        self.split_offsets = split_offsets
        self.workspace_bytes = int(workspace_bytes)
        self.s_q = s_q
        self.H = H

    @property
    def total_splits(self) -> int:
        return int(self.split_offsets[-1])

    @property
    def any_split(self) -> bool:
        return bool((self.num_splits > 1).any())

    def device_offsets(self, device) -> torch.Tensor:
        return torch.from_numpy(self.split_offsets).to(device)


def decode_plan(seqlens: Sequence[int], s_q: int, H: int, num_cus: int = 256,
                max_splits: int = MAX_SPLITS) -> DecodePlan:
    """Host split planner (mla_decode_plan)."""
    L = np.ascontiguousarray(np.asarray(seqlens, dtype=np.int32))
    B = int(L.shape[0])
    ns = np.zeros(B, dtype=np.int32)
    off = np.zeros(B + 1, dtype=np.int32)
    ws = ctypes.c_size_t(0)
    st = load_library().mla_decode_plan(L.ctypes.data_as(ctypes.c_void_p), B, int(s_q), int(H), int(num_cus),
                                        int(max_splits), ns.ctypes.data_as(ctypes.c_void_p),
                                        off.ctypes.data_as(ctypes.c_void_p), ctypes.byref(ws))
    _check("mla_decode_plan", st)
    return DecodePlan(ns, off, ws.value, s_q, H)


class DecodeSchedule(DecodePlan):
    """A balanced schedule (mla_decode_schedule): the split offsets of its
    chunks, the schedule entries (segment -> first chunk, then per chunk b,
    first page, end page, L_b), the segment count and the row-group size.
    ``device_arrays(device)`` copies the offsets and the entries to the
    device once and keeps them."""

    def __init__(self, split_offsets: np.ndarray, workspace_bytes: int, s_q: int, H: int, schedule: np.ndarray,
                 num_segments: int, rows_per_group: int):
        super().__init__(np.diff(split_offsets).astype(np.int32), split_offsets, workspace_bytes, s_q, H)
        self.schedule = schedule
        self.num_segments = int(num_segments)
        self.rows_per_group = int(rows_per_group)
        self._dev = {}

    @property
    def chunks(self) -> np.ndarray:
        """[total_splits, 4]: b, first page, end page, L_b of every chunk."""
        return self.schedule[self.num_segments + 1:].reshape(-1, 4)

    @property
    def segment_first_chunk(self) -> np.ndarray:
        return self.schedule[:self.num_segments + 1]

    def device_arrays(self, device):
        key = str(torch.device(device))
        if key not in self._dev:
            self._dev[key] = (torch.from_numpy(self.split_offsets).to(device),
                              torch.from_numpy(self.schedule).to(device))
        return self._dev[key]


def decode_schedule(seqlens: Sequence[int], s_q: int, H: int, num_cus: int = 256, max_splits: int = MAX_SPLITS,
                    rows_per_group: int = 0) -> DecodeSchedule:
    """Host balanced-schedule planner (mla_decode_schedule); rows_per_group 0 lets it choose."""
    lib = load_library()
    L = np.ascontiguousarray(np.asarray(seqlens, dtype=np.int32))
    B = int(L.shape[0])
    cap = int(lib.mla_decode_schedule_capacity(B, int(num_cus)))
    off = np.zeros(B + 1, dtype=np.int32)
    sched = np.zeros(max(cap, 1), dtype=np.int32)
    nseg, rpg, ws = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_size_t(0)
    st = lib.mla_decode_schedule(L.ctypes.data_as(ctypes.c_void_p), B, int(s_q), int(H), int(num_cus),
                                 int(max_splits), int(rows_per_group), off.ctypes.data_as(ctypes.c_void_p),
                                 sched.ctypes.data_as(ctypes.c_void_p), cap, ctypes.byref(nseg), ctypes.byref(rpg),
                                 ctypes.byref(ws))
    _check("mla_decode_schedule", st)
    n = nseg.value + 1 + 4 * int(off[-1])
    return DecodeSchedule(off, ws.value, s_q, H, np.ascontiguousarray(sched[:n]), nseg.value, rpg.value)


def mla_decode_fwd(q_lat: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
                   seqlens: torch.Tensor, softmax_scale: float, causal: bool,
                   split_offsets: Optional[torch.Tensor] = None, total_splits: Optional[int] = None,
                   workspace: Optional[torch.Tensor] = None, o_lat: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None, partials_only: bool = False,
                   schedule: Optional[DecodeSchedule] = None, _prepare: bool = False):
    """Absorbed-MLA decode (mla_decode_fwd). Returns (o_lat [B,s_q,H,512], lse [B,s_q,H] fp32).

    split_offsets: int32 device [B+1] from ``decode_plan`` (or None for one
    chunk per sequence); total_splits: its last entry (host int).
    schedule: a ``decode_schedule`` result instead (mla_decode_fwd_scheduled;
    its own offsets are used, split_offsets and total_splits must be None).
    partials_only (needs split_offsets or a schedule): write only the
    per-chunk partials into ``workspace`` and return (None, None);
    ``workspace_partials`` views them for ``mla_splitkv_combine``.
    """
    sched_t = None
    if schedule is not None:
        if split_offsets is not None or total_splits is not None:
            raise ValueError("a schedule carries its own split offsets")
        split_offsets, sched_t = schedule.device_arrays(q_lat.device)
        total_splits = schedule.total_splits
    if q_lat.dim() != 4 or kv_cache.dim() != 3 or block_table.dim() != 2 or seqlens.dim() != 1:
        raise ValueError("expected q_lat [B,s_q,H,576], kv_cache [pages,64,576], block_table [B,P], seqlens [B]")
    dev = q_lat.device
    dtype = q_lat.dtype
    if dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {dtype}")
    _need(q_lat, "q_lat", device=dev)
    _need(kv_cache, "kv_cache", dtype=dtype, device=dev)
    _need(block_table, "block_table", dtype=torch.int32, device=dev)
    _need(seqlens, "seqlens", dtype=torch.int32, device=dev)
    B, s_q, H, dqk = q_lat.shape
    if block_table.shape[0] != B or seqlens.shape[0] != B:
        raise ValueError("block_table and seqlens must have B rows")
    if split_offsets is not None:
        _need(split_offsets, "split_offsets", dtype=torch.int32, device=dev)
        if split_offsets.shape[0] != B + 1:
            raise ValueError("split_offsets must have B+1 entries")
        if total_splits is None:
            raise ValueError("total_splits (host copy of split_offsets[B]) is required")
        if workspace is None:
            nbytes = decode_workspace_size(total_splits, s_q, H)
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    else:
        total_splits = B
    if workspace is not None:
        _need(workspace, "workspace", device=dev)
    if partials_only:
        if split_offsets is None:
            raise ValueError("partials_only needs split_offsets")
        if o_lat is not None or lse is not None:
            raise ValueError("partials_only writes no o_lat/lse")
    else:
        if o_lat is None:
            o_lat = torch.empty((B, s_q, H, D_V), dtype=dtype, device=dev)
        if lse is None:
            lse = torch.empty((B, s_q, H), dtype=torch.float32, device=dev)
        _need(o_lat, "o_lat", dtype=dtype, device=dev)
        _need(lse, "lse", dtype=torch.float32, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    head = (_ptr(q_lat), _ptr(kv_cache), _ptr(block_table), _ptr(seqlens), _ptr(split_offsets))
    if sched_t is not None:
        fn = "mla_decode_fwd_scheduled"
        head = head + (_ptr(sched_t), schedule.num_segments, schedule.rows_per_group)
    else:
        fn = "mla_decode_fwd"
    args = head + (int(total_splits), B, s_q, H, dqk, D_V if o_lat is None else int(o_lat.shape[-1]),
                   int(kv_cache.shape[1]), int(block_table.shape[1]), int(kv_cache.shape[0]), float(softmax_scale),
                   int(bool(causal)), _DTYPES[dtype], _ptr(workspace), ws_bytes, _ptr(o_lat), _ptr(lse), _stream())
    if _prepare:
        return PreparedCall(fn, args), (o_lat, lse)
    _check(fn, getattr(load_library(), fn)(*args))
    return o_lat, lse


NOALLOC_SCRATCH_BYTES = 64 << 20  # MLA_NOALLOC_SCRATCH_BYTES


def noalloc_scratch_bytes(total_splits: int, s_q: int, H: int, dtype=torch.bfloat16) -> int:
    """Bytes of the library's static array that ``mla_decode_fwd_noalloc`` needs for a plan."""
    return int(load_library().mla_decode_noalloc_scratch_bytes(int(total_splits), int(s_q), int(H),
                                                               _DTYPES[dtype]))


def mla_decode_fwd_noalloc(q_lat: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
                           seqlens: torch.Tensor, softmax_scale: float, causal: bool, o_lat: torch.Tensor,
                           lse: torch.Tensor, split_offsets: Optional[torch.Tensor] = None,
                           total_splits: Optional[int] = None):
    """mla_decode_fwd_noalloc: the split decode and its merge with the chunk partials in the
    library's static device array. The caller passes the outputs; the call allocates nothing."""
    if q_lat.dim() != 4 or kv_cache.dim() != 3 or block_table.dim() != 2 or seqlens.dim() != 1:
        raise ValueError("expected q_lat [B,s_q,H,576], kv_cache [pages,64,576], block_table [B,P], seqlens [B]")
    dev = q_lat.device
    dtype = q_lat.dtype
    if dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {dtype}")
    for t, name, dt in ((q_lat, "q_lat", None), (kv_cache, "kv_cache", dtype), (block_table, "block_table", torch.int32),
                        (seqlens, "seqlens", torch.int32), (o_lat, "o_lat", dtype), (lse, "lse", torch.float32)):
        _need(t, name, dtype=dt, device=dev)
    B, s_q, H, dqk = q_lat.shape
    if split_offsets is not None:
        _need(split_offsets, "split_offsets", dtype=torch.int32, device=dev)
        if split_offsets.shape[0] != B + 1 or total_splits is None:
            raise ValueError("split_offsets must have B+1 entries and total_splits its last one")
    else:
        total_splits = B
    st = load_library().mla_decode_fwd_noalloc(
        _ptr(q_lat), _ptr(kv_cache), _ptr(block_table), _ptr(seqlens), _ptr(split_offsets), int(total_splits), B,
        s_q, H, dqk, int(o_lat.shape[-1]), int(kv_cache.shape[1]), int(block_table.shape[1]),
        int(kv_cache.shape[0]), float(softmax_scale), int(bool(causal)), _DTYPES[dtype], _ptr(o_lat), _ptr(lse),
        _stream())
    _check("mla_decode_fwd_noalloc", st)
    return o_lat, lse


def sparse_decode_plan(B: int, topk: int, s_q: int = 1, H: int = 128, num_cus: int = 256,
                       max_splits: int = MAX_SPLITS) -> DecodePlan:
    """Split plan for ``mla_sparse_decode_fwd``: the chunks cut each query
    token's list of ``topk`` entries, so every sequence plans as length topk."""
    return decode_plan([int(topk)] * int(B), s_q, H, num_cus=num_cus, max_splits=max_splits)


def mla_sparse_decode_fwd(q_lat: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
                          seqlens: torch.Tensor, indices: torch.Tensor, softmax_scale: float,
                          split_offsets: Optional[torch.Tensor] = None, total_splits: Optional[int] = None,
                          workspace: Optional[torch.Tensor] = None, o_lat: Optional[torch.Tensor] = None,
                          lse: Optional[torch.Tensor] = None, partials_only: bool = False,
                          _prepare: bool = False):
    """Top-k decode (mla_sparse_decode_fwd): attention of each (token, head)
    row over the positions listed in ``indices`` [B, s_q, topk] int32 (entries
    outside [0, L_b) are padding). bf16, H = 128. Arguments and results as
    ``mla_decode_fwd``; plan with ``sparse_decode_plan``."""
    if q_lat.dim() != 4 or indices.dim() != 3:
        raise ValueError("expected q_lat [B,s_q,H,576] and indices [B,s_q,topk]")
    B, s_q = q_lat.shape[:2]
    if tuple(indices.shape[:2]) != (B, s_q):
        raise ValueError("indices must be [B, s_q, topk]")
    _need(indices, "indices", dtype=torch.int32, device=q_lat.device)
    call, outs = mla_decode_fwd(q_lat, kv_cache, block_table, seqlens, softmax_scale, False,
                                split_offsets=split_offsets, total_splits=total_splits, workspace=workspace,
                                o_lat=o_lat, lse=lse, partials_only=partials_only, _prepare=True)
    a = call.args
    args = a[:4] + (_ptr(indices), int(indices.shape[2])) + a[4:15] + a[16:]
    if _prepare:
        return PreparedCall("mla_sparse_decode_fwd", args), outs
    _check("mla_sparse_decode_fwd", load_library().mla_sparse_decode_fwd(*args))
    return outs


def mla_decode_fwd_fp8(q_lat: torch.Tensor, kv_cache_e4m3: torch.Tensor, row_scales: torch.Tensor,
                       block_table: torch.Tensor, seqlens: torch.Tensor, softmax_scale: float, causal: bool,
                       split_offsets: Optional[torch.Tensor] = None, total_splits: Optional[int] = None,
                       workspace: Optional[torch.Tensor] = None, o_lat: Optional[torch.Tensor] = None,
                       lse: Optional[torch.Tensor] = None, partials_only: bool = False, _prepare: bool = False):
    """Decode on an FP8 latent cache (mla_decode_fwd_fp8): ``kv_cache_e4m3``
    [pages, 64, 576] uint8 e4m3 codes, ``row_scales`` [pages, 64] fp32, bf16
    q_lat and o_lat. Other arguments and results as ``mla_decode_fwd``."""
    if q_lat.dim() != 4 or kv_cache_e4m3.dim() != 3 or block_table.dim() != 2 or seqlens.dim() != 1:
        raise ValueError("expected q_lat [B,s_q,H,576], kv_cache_e4m3 [pages,64,576], block_table [B,P], seqlens [B]")
    dev = q_lat.device
    _need(q_lat, "q_lat", dtype=torch.bfloat16, device=dev)
    _need(kv_cache_e4m3, "kv_cache_e4m3", dtype=torch.uint8, device=dev)
    _need(row_scales, "row_scales", dtype=torch.float32, device=dev)
    _need(block_table, "block_table", dtype=torch.int32, device=dev)
    _need(seqlens, "seqlens", dtype=torch.int32, device=dev)
    if tuple(row_scales.shape) != tuple(kv_cache_e4m3.shape[:2]):
        raise ValueError("row_scales must be [pages, 64]")
    B, s_q, H, dqk = q_lat.shape
    if block_table.shape[0] != B or seqlens.shape[0] != B:
        raise ValueError("block_table and seqlens must have B rows")
    if split_offsets is not None:
        _need(split_offsets, "split_offsets", dtype=torch.int32, device=dev)
        if split_offsets.shape[0] != B + 1 or total_splits is None:
            raise ValueError("split_offsets must have B+1 entries and total_splits is required")
        if workspace is None:
            workspace = torch.empty(decode_workspace_size(total_splits, s_q, H), dtype=torch.uint8, device=dev)
    else:
        total_splits = B
    if workspace is not None:
        _need(workspace, "workspace", device=dev)
    if partials_only:
        if split_offsets is None or o_lat is not None or lse is not None:
            raise ValueError("partials_only needs split_offsets and no o_lat/lse")
    else:
        o_lat = torch.empty((B, s_q, H, D_V), dtype=torch.bfloat16, device=dev) if o_lat is None else o_lat
        lse = torch.empty((B, s_q, H), dtype=torch.float32, device=dev) if lse is None else lse
        _need(o_lat, "o_lat", dtype=torch.bfloat16, device=dev)
        _need(lse, "lse", dtype=torch.float32, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_ptr(q_lat), _ptr(kv_cache_e4m3), _ptr(row_scales), _ptr(block_table), _ptr(seqlens),
            _ptr(split_offsets), int(total_splits), B, s_q, H, dqk, D_V, int(kv_cache_e4m3.shape[1]),
            int(block_table.shape[1]), int(kv_cache_e4m3.shape[0]), float(softmax_scale), int(bool(causal)),
            _ptr(workspace), ws_bytes, _ptr(o_lat), _ptr(lse), _stream())
    if _prepare:
        return PreparedCall("mla_decode_fwd_fp8", args), (o_lat, lse)
    _check("mla_decode_fwd_fp8", load_library().mla_decode_fwd_fp8(*args))
    return o_lat, lse


def prepare_decode_fp8(*args, **kwargs):
    """Like ``mla_decode_fwd_fp8`` but returns (PreparedCall, (o_lat, lse))."""
    return mla_decode_fwd_fp8(*args, _prepare=True, **kwargs)


def prepare_sparse_decode(*args, **kwargs):
    """Like ``mla_sparse_decode_fwd`` but returns (PreparedCall, (o_lat, lse))."""
    return mla_sparse_decode_fwd(*args, _prepare=True, **kwargs)


def workspace_partials(workspace: torch.Tensor, total_splits: int, s_q: int, H: int,
                       dtype: torch.dtype = torch.bfloat16):
    """Views (o_part [total_splits,s_q,H,512] in the decode dtype, lse_part
    [total_splits,s_q,H] fp32) of a decode workspace. The o_part region is
    sized for fp32 whatever the dtype, so lse_part always starts at byte
    total_splits*s_q*H*512*4."""
    rows = int(total_splits) * s_q * H
    need = rows * (D_V + 1) * 4
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError("workspace is smaller than the partials of this plan")
    raw = workspace.view(torch.uint8)
    esz = torch.empty((), dtype=dtype).element_size()
    o_part = raw[:rows * D_V * esz].view(dtype).view(total_splits, s_q, H, D_V)
    lse_part = raw[rows * D_V * 4:need].view(torch.float32).view(total_splits, s_q, H)
    return o_part, lse_part


def mla_splitkv_combine(o_part: torch.Tensor, lse_part: torch.Tensor, split_offsets: torch.Tensor,
                        total_splits: int, B: int, out_dtype: torch.dtype = torch.bfloat16,
                        o_lat: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
    """LSE merge of chunk partials (mla_splitkv_combine).

    o_part [total_splits, s_q, H, 512] in out_dtype, lse_part [total_splits, s_q, H] fp32.
    Returns (o_lat [B,s_q,H,512] out_dtype, lse [B,s_q,H] fp32).
    """
    dev = o_part.device
    _need(o_part, "o_part", dtype=out_dtype)
    _need(lse_part, "lse_part", dtype=torch.float32, device=dev)
    _need(split_offsets, "split_offsets", dtype=torch.int32, device=dev)
    if o_part.dim() != 4 or lse_part.shape != o_part.shape[:3] or o_part.shape[0] != total_splits:
        raise ValueError("o_part must be [total_splits,s_q,H,512] and lse_part [total_splits,s_q,H]")
    if out_dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {out_dtype}")
    _, s_q, H, dv = o_part.shape
    if o_lat is None:
        o_lat = torch.empty((B, s_q, H, dv), dtype=out_dtype, device=dev)
    if lse is None:
        lse = torch.empty((B, s_q, H), dtype=torch.float32, device=dev)
    _need(o_lat, "o_lat", dtype=out_dtype, device=dev)
    _need(lse, "lse", dtype=torch.float32, device=dev)
    st = load_library().mla_splitkv_combine(_ptr(o_part), _ptr(lse_part), _ptr(split_offsets), int(total_splits),
                                            int(B), s_q, H, dv, _DTYPES[out_dtype], _ptr(o_lat), _ptr(lse),
                                            _stream())
    _check("mla_splitkv_combine", st)
    return o_lat, lse


class PreparedCall:
    """One library call with its arguments validated and marshalled once.

    Calling it launches the same entry point with the same tensors (by
    address) on the stream that was current when it was prepared, without
    re-checking the tensors in Python: the caller keeps them alive and
    unchanged in shape. For launch-rate-bound loops (a decode step per layer).
    """

    def __init__(self, fn: str, args: tuple):
        self.fn = fn
        self.args = args
        self._f = getattr(load_library(), fn)

    def __call__(self) -> None:
        st = self._f(*self.args)
        if st != 0:
            raise MlaError(self.fn, st)


def prepare_decode(*args, **kwargs):
    """Like ``mla_decode_fwd`` but returns (PreparedCall, (o_lat, lse)) instead of launching."""
    return mla_decode_fwd(*args, _prepare=True, **kwargs)


def prepare_combine(o_part: torch.Tensor, lse_part: torch.Tensor, split_offsets: torch.Tensor,
                    total_splits: int, B: int, out_dtype: torch.dtype, o_lat: torch.Tensor,
                    lse: torch.Tensor) -> PreparedCall:
    """A PreparedCall of ``mla_splitkv_combine`` (same checks, run once)."""
    _need(o_part, "o_part", dtype=out_dtype)
    dev = o_part.device
    _need(lse_part, "lse_part", dtype=torch.float32, device=dev)
    _need(split_offsets, "split_offsets", dtype=torch.int32, device=dev)
    _need(o_lat, "o_lat", dtype=out_dtype, device=dev)
    _need(lse, "lse", dtype=torch.float32, device=dev)
    if o_part.dim() != 4 or lse_part.shape != o_part.shape[:3] or o_part.shape[0] != total_splits:
        raise ValueError("o_part must be [total_splits,s_q,H,512] and lse_part [total_splits,s_q,H]")
    _, s_q, H, dv = o_part.shape
    return PreparedCall("mla_splitkv_combine",
                        (_ptr(o_part), _ptr(lse_part), _ptr(split_offsets), int(total_splits), int(B), s_q, H,
                         dv, _DTYPES[out_dtype], _ptr(o_lat), _ptr(lse), _stream()))


def mla_absorb_q(q_nope: torch.Tensor, q_rope: Optional[torch.Tensor], w_uk: torch.Tensor,
                 q_lat: Optional[torch.Tensor] = None) -> torch.Tensor:
    """q_lat [N,H,d_c+d_rope] = [W_UK q_nope ; q_rope] (mla_absorb_q). w_uk is [H, d_c, d_nope]."""
    dtype = q_nope.dtype
    if dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {dtype}")
    dev = q_nope.device
    _need(q_nope, "q_nope", device=dev)
    _need(w_uk, "w_uk", dtype=dtype, device=dev)
    N, H, dn = q_nope.shape
    Hw, dc, dn2 = w_uk.shape
    if Hw != H or dn2 != dn:
        raise ValueError("w_uk must be [H, d_c, d_nope]")
    dr = 0
    if q_rope is not None:
        _need(q_rope, "q_rope", dtype=dtype, device=dev)
        if q_rope.shape[:2] != (N, H):
            raise ValueError("q_rope must be [N, H, d_rope]")
        dr = q_rope.shape[2]
    if q_lat is None:
        q_lat = torch.empty((N, H, dc + dr), dtype=dtype, device=dev)
    _need(q_lat, "q_lat", dtype=dtype, device=dev)
    st = load_library().mla_absorb_q(_ptr(q_nope), _ptr(q_rope), _ptr(w_uk), N, H, dn, dr, dc,
                                     _DTYPES[dtype], _ptr(q_lat), _stream())
    _check("mla_absorb_q", st)
    return q_lat


def mla_out_uv(o_lat: torch.Tensor, w_uv: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out [N,H,d_v] = o_lat [N,H,d_c] . W_UV[h] (mla_out_uv). w_uv is [H, d_c, d_v]."""
    dtype = o_lat.dtype
    if dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {dtype}")
    dev = o_lat.device
    _need(o_lat, "o_lat", device=dev)
    _need(w_uv, "w_uv", dtype=dtype, device=dev)
    N, H, dc = o_lat.shape
    if w_uv.shape[0] != H or w_uv.shape[1] != dc:
        raise ValueError("w_uv must be [H, d_c, d_v]")
    dv = w_uv.shape[2]
    if out is None:
        out = torch.empty((N, H, dv), dtype=dtype, device=dev)
    _need(out, "out", dtype=dtype, device=dev)
    st = load_library().mla_out_uv(_ptr(o_lat), _ptr(w_uv), N, H, dc, dv, _DTYPES[dtype], _ptr(out), _stream())
    _check("mla_out_uv", st)
    return out


# ---------------------------------------------------------------------------
# The expanded path (prefill / extend) and the choice between the two paths.
# ---------------------------------------------------------------------------

PREFILL_CHUNK = 8192  # cached tokens expanded at a time: the prefix-length threshold [MLA-推理] "谁快" gives


def select_path(s_q: int, L: int) -> str:
    """"expanded" or "absorbed": the cheaper path in FLOPs (mla_select_path)."""
    r = load_library().mla_select_path(int(s_q), int(L))
    if r < 0:
        raise ValueError("need 1 <= s_q <= L")
    return "expanded" if r == 1 else "absorbed"


def prefill_workspace_size(s_q: int, H: int, chunk_tokens: int, max_chunks: int) -> int:
    return int(load_library().mla_prefill_workspace_size(int(s_q), int(H), int(chunk_tokens), int(max_chunks)))


def mla_prefill_fwd(q_nope: torch.Tensor, q_rope: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
                    seqlens_host: Sequence[int], w_uk: torch.Tensor, w_uv: torch.Tensor, softmax_scale: float,
                    chunk_tokens: int = PREFILL_CHUNK, workspace: Optional[torch.Tensor] = None,
                    o: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
    """Expanded path (mla_prefill_fwd): per-head outputs o [B,s_q,H,128] bf16 and lse [B,s_q,H] fp32 of
    the s_q new tokens (the last s_q of each sequence's cached tokens), the cache expanded chunk_tokens
    at a time with an LSE merge across chunks."""
    dev = q_nope.device
    if q_nope.dim() != 4 or q_rope.dim() != 4 or tuple(q_rope.shape[:3]) != tuple(q_nope.shape[:3]):
        raise ValueError("expected q_nope [B,s_q,H,128] and q_rope [B,s_q,H,64]")
    B, s_q, H, _ = q_nope.shape
    for t, name in ((q_nope, "q_nope"), (q_rope, "q_rope"), (kv_cache, "kv_cache"), (w_uk, "w_uk"), (w_uv, "w_uv")):
        _need(t, name, dtype=torch.bfloat16, device=dev)
    _need(block_table, "block_table", dtype=torch.int32, device=dev)
    if q_nope.shape[3] != 128 or q_rope.shape[3] != 64:
        raise ValueError("expanded path needs d_nope = d_v = 128 and d_rope = 64")
    for w, name in ((w_uk, "w_uk"), (w_uv, "w_uv")):
        if tuple(w.shape) != (H, 512, 128):
            raise ValueError(f"{name} must be [H,512,128], got {tuple(w.shape)}")
    if kv_cache.dim() != 3 or tuple(kv_cache.shape[1:]) != (PAGE_SIZE, 576):
        raise ValueError("kv_cache must be [num_pages, 64, 576]")
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_pages]")
    L = np.ascontiguousarray(np.asarray(seqlens_host, dtype=np.int32))
    if L.shape != (B,):
        raise ValueError("seqlens_host must have B entries")
    max_chunks = int(max(1, ((L.astype(np.int64) + chunk_tokens - 1) // chunk_tokens).max()))
    if workspace is None:
        workspace = torch.empty(prefill_workspace_size(s_q, H, chunk_tokens, max_chunks), dtype=torch.uint8,
                                device=dev)
    o = torch.empty((B, s_q, H, 128), dtype=torch.bfloat16, device=dev) if o is None else o
    lse = torch.empty((B, s_q, H), dtype=torch.float32, device=dev) if lse is None else lse
    _need(o, "o", dtype=torch.bfloat16, device=dev)
    _need(lse, "lse", dtype=torch.float32, device=dev)
    if tuple(o.shape) != (B, s_q, H, 128) or tuple(lse.shape) != (B, s_q, H):
        raise ValueError("o must be [B,s_q,H,128] and lse [B,s_q,H]")
    st = load_library().mla_prefill_fwd(_ptr(q_nope), _ptr(q_rope), _ptr(kv_cache), _ptr(block_table),
                                        L.ctypes.data_as(ctypes.c_void_p), B, s_q, H, int(block_table.shape[1]),
                                        int(kv_cache.shape[0]), _ptr(w_uk), _ptr(w_uv), int(chunk_tokens),
                                        float(softmax_scale), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _ptr(o), _ptr(lse), _stream())
    _check("mla_prefill_fwd", st)
    return o, lse


def mla_attention_fwd(q_nope: torch.Tensor, q_rope: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
                      seqlens: torch.Tensor, w_uk: torch.Tensor, w_uv: torch.Tensor, softmax_scale: float,
                      path: str = "auto", chunk_tokens: int = PREFILL_CHUNK):
    """Attention of the s_q new tokens of each sequence by either path, per-head outputs
    o [B,s_q,H,128] and lse [B,s_q,H]. path "auto" asks mla_select_path with the longest sequence;
    "absorbed" runs mla_absorb_q, mla_decode_fwd (causal, split by mla_decode_plan) and mla_out_uv
    (s_q <= 16); "expanded" runs mla_prefill_fwd. Both compute the same attention ([MLA-推理]
    "两条等价的路径"); "auto" takes the expanded one also when s_q exceeds the decode kernel's 16."""
    B, s_q, H, _ = q_nope.shape
    L = [int(x) for x in seqlens.cpu().tolist()]
    if path == "auto":
        path = select_path(s_q, max(L)) if s_q <= MAX_DECODE_SQ else "expanded"
    if path == "expanded":
        return mla_prefill_fwd(q_nope, q_rope, kv_cache, block_table, L, w_uk, w_uv, softmax_scale, chunk_tokens)
    if path != "absorbed":
        raise ValueError(f"unknown path {path}")
    q_lat = mla_absorb_q(q_nope.reshape(B * s_q, H, -1), q_rope.reshape(B * s_q, H, -1), w_uk)
    p = decode_plan(L, s_q, H)
    kw = dict(split_offsets=p.device_offsets(q_nope.device), total_splits=p.total_splits) if p.any_split else {}
    o_lat, lse = mla_decode_fwd(q_lat.view(B, s_q, H, -1), kv_cache, block_table, seqlens, softmax_scale, True, **kw)
    o = mla_out_uv(o_lat.view(B * s_q, H, -1), w_uv)
    return o.view(B, s_q, H, -1), lse


# ---- FP8 products for the absorption -------------------------------------

def fp8_workspace_size(n_elems: int) -> int:
    return int(load_library().mla_fp8_workspace_size(int(n_elems)))


def quantize_e4m3(x: torch.Tensor, workspace: Optional[torch.Tensor] = None):
    """Per-tensor e4m3 quantisation (mla_quantize_e4m3): codes (uint8, x's
    shape) and the scale (one-element fp32 tensor) on x's device."""
    _need(x, "x", dtype=torch.bfloat16)
    dev = x.device
    codes = torch.empty(x.shape, dtype=torch.uint8, device=dev)
    scale = torch.empty(1, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(1024, dtype=torch.uint8, device=dev)
    st = load_library().mla_quantize_e4m3(_ptr(x), x.numel(), _ptr(workspace), workspace.numel(), _ptr(codes),
                                          _ptr(scale), _stream())
    _check("mla_quantize_e4m3", st)
    return codes, scale


def mla_absorb_q_fp8(q_nope: torch.Tensor, q_rope: torch.Tensor, w_uk_codes: torch.Tensor, w_scale: float,
                     q_lat: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """q_lat [N,H,d_c+d_rope] bf16 from bf16 q_nope/q_rope and e4m3 W_UK codes [H,d_c,d_nope] (mla_absorb_q_fp8)."""
    N, H, dn = q_nope.shape
    dr = q_rope.shape[2]
    dc = w_uk_codes.shape[1]
    dev = q_nope.device
    _need(q_nope, "q_nope", dtype=torch.bfloat16, device=dev)
    _need(q_rope, "q_rope", dtype=torch.bfloat16, device=dev)
    _need(w_uk_codes, "w_uk_codes", dtype=torch.uint8, device=dev)
    if tuple(w_uk_codes.shape) != (H, dc, dn) or tuple(q_rope.shape[:2]) != (N, H):
        raise ValueError("expected w_uk_codes [H, d_c, d_nope] and q_rope [N, H, d_rope]")
    if q_lat is None:
        q_lat = torch.empty((N, H, dc + dr), dtype=torch.bfloat16, device=dev)
    if workspace is None:
        workspace = torch.empty(fp8_workspace_size(N * H * dn), dtype=torch.uint8, device=dev)
    st = load_library().mla_absorb_q_fp8(_ptr(q_nope), _ptr(q_rope), _ptr(w_uk_codes), float(w_scale), N, H, dn, dr,
                                         dc, _ptr(workspace), workspace.numel(), _ptr(q_lat), _stream())
    _check("mla_absorb_q_fp8", st)
    return q_lat


def mla_out_uv_fp8(o_lat: torch.Tensor, w_uv_t_codes: torch.Tensor, w_scale: float,
                   out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out [N,H,d_v] bf16 from bf16 o_lat [N,H,d_c] and e4m3 W_UV^T codes [H,d_v,d_c] (mla_out_uv_fp8)."""
    N, H, dc = o_lat.shape
    dv = w_uv_t_codes.shape[1]
    dev = o_lat.device
    _need(o_lat, "o_lat", dtype=torch.bfloat16, device=dev)
    _need(w_uv_t_codes, "w_uv_t_codes", dtype=torch.uint8, device=dev)
    if tuple(w_uv_t_codes.shape) != (H, dv, dc):
        raise ValueError("expected w_uv_t_codes [H, d_v, d_c]")
    if out is None:
        out = torch.empty((N, H, dv), dtype=torch.bfloat16, device=dev)
    if workspace is None:
        workspace = torch.empty(fp8_workspace_size(N * H * dc), dtype=torch.uint8, device=dev)
    st = load_library().mla_out_uv_fp8(_ptr(o_lat), _ptr(w_uv_t_codes), float(w_scale), N, H, dc, dv,
                                       _ptr(workspace), workspace.numel(), _ptr(out), _stream())
    _check("mla_out_uv_fp8", st)
    return out

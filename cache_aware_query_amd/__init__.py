"""Python binding of libwavealign, the MI355X cache-aware block-sparse attention library.

Argument marshalling only: every function below checks tensor types and shapes,
allocates outputs with PyTorch on the inputs' device, passes raw device pointers
and the current HIP stream to the C ABI (include/wavealign.h) and raises on a
non-zero status.  All arithmetic runs in the HIP kernels.  There is no fallback:
if the shared library is missing the import of any entry point raises.

Function names follow the C ABI without the ``wa_`` prefix.
"""

from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import torch  # loads the HIP runtime that the library then binds to

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwavealign.so")

WA_SCHED_NATURAL = 0
WA_SCHED_XCD_SLICED = 1
WA_SCHED_HEADS_INTERLEAVED = 2
WA_SCHED_AUTO = 3
WA_SCHED_DEFAULT = 4
WA_SKIP_ADAPTIVE = 0
WA_SKIP_NEVER = 1
WA_SKIP_ALWAYS = 2

EXPORTED = (
    "wa_abi_version", "wa_last_error", "wa_schedule_info", "wa_build_block_index",
    "wa_reorder_rows", "wa_reorder_needs_csc", "wa_minhash_order", "wa_sparse_attn_workspace_size",
    "wa_sparse_attn_fwd", "wa_sparse_attn_fwd_diag", "wa_attn_schedule_select",
    "wa_block_importance", "wa_topp_select", "wa_mask_recall", "wa_gather_blocks",
    "wa_scatter_blocks", "wa_xcd_placement", "wa_sparse_attn_fwd_noalloc", "wa_lsh_order",
    "wa_default_schedule",
)


class WaError(RuntimeError):
    """A libwavealign call returned an error status."""


class _ReorderParams(ctypes.Structure):
    _fields_ = [
        ("wave", ctypes.c_int32), ("n_slices", ctypes.c_int32), ("iters", ctypes.c_int32),
        ("stage1", ctypes.c_int32), ("stage2", ctypes.c_int32), ("skip_mode", ctypes.c_int32),
        ("ws_min_bytes", ctypes.c_double), ("flops_min", ctypes.c_double),
        ("jaccard_max", ctypes.c_double),
    ]


@dataclass
class ReorderParams:
    """Host parameters of reorder_rows (see wa_reorder_params in wavealign.h)."""
    wave: int = 64
    n_slices: int = 8
    iters: int = 10
    stage1: bool = True
    stage2: bool = True
    skip_mode: int = WA_SKIP_ADAPTIVE
    ws_min_bytes: float = 0.0
    flops_min: float = 0.0
    jaccard_max: float = 1.0

    @classmethod
    def calibrated(cls, path: str | None = None, **over) -> "ReorderParams":
        """Adaptive skip with the thresholds that ``python -m cache_aware_query_amd.calibrate``
        measured on this GPU model (raises FileNotFoundError if no calibration exists)."""
        import json

        with open(path or os.path.join(_HERE, "calib_mi355x.json")) as f:
            c = json.load(f)
        kw = dict(skip_mode=WA_SKIP_ADAPTIVE, iters=int(c["iters"]),
                  ws_min_bytes=float(c["ws_min_bytes"]), flops_min=float(c["flops_min"]),
                  jaccard_max=float(c["jaccard_max"]))
        kw.update(over)
        return cls(**kw)

    def _c(self) -> _ReorderParams:
        return _ReorderParams(int(self.wave), int(self.n_slices), int(self.iters),
                              int(bool(self.stage1)), int(bool(self.stage2)), int(self.skip_mode),
                              float(self.ws_min_bytes), float(self.flops_min),
                              float(self.jaccard_max))


_LIB = None
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libwavealign.so and declare its prototypes (raises if it is missing)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
            "or `python cache_aware_query_amd/build.py`")
    lib = ctypes.CDLL(path)
    sig = {
        "wa_abi_version": (ctypes.c_int, []),
        "wa_last_error": (ctypes.c_char_p, []),
        "wa_schedule_info": (ctypes.c_int, [ctypes.c_int, _I32, _P, _P, _P]),
        "wa_build_block_index": (ctypes.c_int, [_P, _I32, _I32, _I32, _P, _P, _I64, _P, _P, _P,
                                                _I64, _P]),
        "wa_reorder_rows": (ctypes.c_int, [_P, _P, _P, _P, _I64, _P, _I32, _I32, _I32, _I32, _I32,
                                           ctypes.POINTER(_ReorderParams), _P, _P, _P, _P, _P,
                                           _P]),
        "wa_reorder_needs_csc": (ctypes.c_int, [_I32, _I32]),
        "wa_lsh_order": (ctypes.c_int, [_P, _P, _I64, _I32, _I32, _I32, _P, _P, _I32, _I32,
                                        _I32, _I32, _P, _P, _P]),
        "wa_minhash_order": (ctypes.c_int, [_P, _P, _I64, _I32, _I32, _I32, _P, _P, _I32, _I32,
                                            _I32, _I32, _P, _P, _P]),
        "wa_sparse_attn_workspace_size": (ctypes.c_int, [_I32, _I32, _I32, _I32,
                                                         ctypes.POINTER(ctypes.c_size_t)]),
        "wa_attn_schedule_select": (ctypes.c_int, [_P, _I32, _P, ctypes.c_size_t, _P]),
        "wa_default_schedule": (ctypes.c_int, [_I32, _I32, _I32, _P]),
        "wa_sparse_attn_fwd": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _I32, _I32, _P, _P, _I64, _P,
                                              _I32, _I32, ctypes.c_float, _P, _P, _P, _P,
                                              ctypes.c_size_t, _P]),
        "wa_sparse_attn_fwd_diag": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _I32, _I32, _P, _P,
                                                   _I64, _P, _I32, _I32, ctypes.c_float, _P, _P,
                                                   _P, _P, _P, _P, ctypes.c_size_t, _P]),
        "wa_xcd_placement": (ctypes.c_int, [_I32, _I32, _P, _P]),
        "wa_sparse_attn_fwd_noalloc": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _I32, _I32, _P, _P,
                                                      _I64, _P, _I32, _I32, _P, ctypes.c_float,
                                                      _P, _P, _P, _P]),
        "wa_block_importance": (ctypes.c_int, [_P, _P, _P, _I64, _I32, _I32, _I32, _I32, _P,
                                               _P]),
        "wa_topp_select": (ctypes.c_int, [_P, _P, _P, _I64, _I32, _I32, _I32, ctypes.c_double,
                                          _P, _P]),
        "wa_mask_recall": (ctypes.c_int, [_P, _P, _P, _I64, _I32, _I32, _I32, _P, _P, _P]),
        "wa_gather_blocks": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _I64, _P]),
        "wa_scatter_blocks": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _I64, _P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


def _check(status: int, what: str) -> None:
    if status != 0:
        msg = _LIB.wa_last_error().decode(errors="replace") if _LIB is not None else ""
        raise WaError(f"{what} failed with status {status}: {msg}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, dtype, name: str, dims=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dims is not None and t.dim() != dims:
        raise ValueError(f"{name} must have {dims} dimensions, got {t.dim()}")


def abi_version() -> int:
    return load_library().wa_abi_version()


def schedule_info(device: int = 0, head_dim: int = 128):
    """(n_xcd, cus_per_xcd, wave): the per-XCD dispatch wave that sizes the buckets."""
    lib = load_library()
    a, b, c = _I32(), _I32(), _I32()
    _check(lib.wa_schedule_info(device, head_dim, ctypes.byref(a), ctypes.byref(b),
                                ctypes.byref(c)), "wa_schedule_info")
    return a.value, b.value, c.value


@dataclass
class BlockIndex:
    row_ptr: torch.Tensor   # int32 [H*MB+1]
    col_idx: torch.Tensor   # int32 [capacity]
    row_nnz: torch.Tensor   # int32 [H*MB]
    csc_ptr: torch.Tensor   # int32 [H*NB+1]
    csc_idx: torch.Tensor   # int32 [capacity]
    heads: int
    mb: int
    nb: int


def build_block_index(mask: torch.Tensor, capacity: int | None = None,
                      with_csc: bool = True) -> BlockIndex:
    """CSR (and CSC) of a uint8 block mask [H, MB, NB]; capacity defaults to H*MB*NB."""
    lib = load_library()
    _need(mask, torch.uint8, "mask", 3)
    H, MB, NB = mask.shape
    cap = H * MB * NB if capacity is None else int(capacity)
    dev = mask.device
    i32 = dict(dtype=torch.int32, device=dev)
    row_ptr = torch.empty(H * MB + 1, **i32)
    row_nnz = torch.empty(H * MB, **i32)
    col_idx = torch.empty(max(cap, 1), **i32)
    csc_ptr = torch.empty(H * NB + 1, **i32) if with_csc else None
    csc_idx = torch.empty(max(cap, 1), **i32) if with_csc else None
    _check(lib.wa_build_block_index(_ptr(mask), H, MB, NB, _ptr(row_ptr), _ptr(col_idx), cap,
                                    _ptr(row_nnz), _ptr(csc_ptr), _ptr(csc_idx),
                                    cap if with_csc else 0, _stream(dev)),
           "wa_build_block_index")
    return BlockIndex(row_ptr, col_idx, row_nnz, csc_ptr, csc_idx, H, MB, NB)


@dataclass
class Reorder:
    perm: torch.Tensor      # int32 [H, MB]
    inv_perm: torch.Tensor  # int32 [H, MB]
    skipped: torch.Tensor   # uint8 [H]
    angles: torch.Tensor    # float64 [H, MB]
    stats: torch.Tensor     # float64 [H, 5]
    n_slices: int = 1       # slices the wave buckets were cut into (params.n_slices)


def reorder_rows(index: BlockIndex, x0: torch.Tensor, block: int, head_dim: int,
                 params: ReorderParams | None = None) -> Reorder:
    """WaveAlign two-stage reordering of every head's query blocks."""
    lib = load_library()
    params = params or ReorderParams()
    _need(x0, torch.float32, "x0", 3)
    H, MB, NB = index.heads, index.mb, index.nb
    if tuple(x0.shape) != (H, MB, 2):
        raise ValueError(f"x0 must be [{H}, {MB}, 2]")
    if index.csc_ptr is None and reorder_needs_csc(MB, NB):
        raise ValueError(f"reorder_rows needs the CSC of the block index for MB={MB}, NB={NB}")
    dev = x0.device
    perm = torch.empty(H, MB, dtype=torch.int32, device=dev)
    inv = torch.empty(H, MB, dtype=torch.int32, device=dev)
    skipped = torch.empty(H, dtype=torch.uint8, device=dev)
    angles = torch.empty(H, MB, dtype=torch.float64, device=dev)
    stats = torch.empty(H, 5, dtype=torch.float64, device=dev)
    cp = params._c()
    cap = index.col_idx.numel()
    if index.csc_idx is not None:
        cap = min(cap, index.csc_idx.numel())
    _check(lib.wa_reorder_rows(_ptr(index.row_ptr), _ptr(index.col_idx), _ptr(index.csc_ptr),
                               _ptr(index.csc_idx), cap, _ptr(x0), H, MB, NB, block, head_dim,
                               ctypes.byref(cp), _ptr(perm), _ptr(inv), _ptr(skipped),
                               _ptr(angles), _ptr(stats), _stream(dev)), "wa_reorder_rows")
    return Reorder(perm, inv, skipped, angles, stats, int(params.n_slices))


def minhash_order(index: BlockIndex, hash_a, hash_b, wave: int, n_slices: int,
                  stage2: bool = True, out: tuple | None = None):
    """The MinHash comparator order (wa_minhash_order): returns (perm, inv_perm)."""
    lib = load_library()
    H, MB, NB = index.heads, index.mb, index.nb
    n = len(hash_a)
    if n != len(hash_b) or n not in (1, 2):
        raise ValueError("hash_a and hash_b must both hold 1 or 2 coefficients")
    dev = index.row_ptr.device
    if out is None:
        perm = torch.empty(H, MB, dtype=torch.int32, device=dev)
        inv = torch.empty(H, MB, dtype=torch.int32, device=dev)
    else:
        perm, inv = out
    a = (ctypes.c_uint32 * n)(*[int(x) for x in hash_a])
    b = (ctypes.c_uint32 * n)(*[int(x) for x in hash_b])
    _check(lib.wa_minhash_order(_ptr(index.row_ptr), _ptr(index.col_idx), index.col_idx.numel(),
                                H, MB, NB, a, b, n, wave, n_slices, 1 if stage2 else 0, _ptr(perm),
                                _ptr(inv), _stream(dev)), "wa_minhash_order")
    return perm, inv


def lsh_order(index: BlockIndex, hash_a, hash_b, wave: int, n_slices: int,
              stage2: bool = True, out: tuple | None = None):
    """The banded LSH comparator order (wa_lsh_order): len(hash_a) / 2 bands of two
    MinHash values each; returns (perm, inv_perm)."""
    lib = load_library()
    H, MB, NB = index.heads, index.mb, index.nb
    n = len(hash_a)
    if n != len(hash_b) or n % 2 or not 2 <= n <= 8:
        raise ValueError("hash_a and hash_b must both hold 2, 4, 6 or 8 coefficients")
    dev = index.row_ptr.device
    if out is None:
        perm = torch.empty(H, MB, dtype=torch.int32, device=dev)
        inv = torch.empty(H, MB, dtype=torch.int32, device=dev)
    else:
        perm, inv = out
    a = (ctypes.c_uint32 * n)(*[int(x) for x in hash_a])
    b = (ctypes.c_uint32 * n)(*[int(x) for x in hash_b])
    _check(lib.wa_lsh_order(_ptr(index.row_ptr), _ptr(index.col_idx), index.col_idx.numel(),
                            H, MB, NB, a, b, n // 2, wave, n_slices, 1 if stage2 else 0,
                            _ptr(perm), _ptr(inv), _stream(dev)), "wa_lsh_order")
    return perm, inv


def reorder_needs_csc(mb: int, nb: int) -> bool:
    """Whether reorder_rows must be given the CSC for an MB x NB mask."""
    r = load_library().wa_reorder_needs_csc(mb, nb)
    _check(0 if r >= 0 else r, "wa_reorder_needs_csc")
    return r == 1


def sparse_attn_workspace_size(heads: int, seq_len: int, head_dim: int, block: int) -> int:
    lib = load_library()
    n = ctypes.c_size_t()
    _check(lib.wa_sparse_attn_workspace_size(heads, seq_len, head_dim, block, ctypes.byref(n)),
           "wa_sparse_attn_workspace_size")
    return n.value


def default_schedule(seq_len: int, head_dim: int, block: int) -> int:
    """The schedule WA_SCHED_DEFAULT runs for these sizes (wa_default_schedule): all
    heads at once for small heads, XCD-sliced in the original order otherwise."""
    lib = load_library()
    out = ctypes.c_int32()
    _check(lib.wa_default_schedule(seq_len, head_dim, block, ctypes.byref(out)),
           "wa_default_schedule")
    return int(out.value)


def attn_schedule_select(skipped: torch.Tensor, workspace: torch.Tensor) -> None:
    """Write the WA_SCHED_AUTO choice for these skip flags into ``workspace``
    (wa_attn_schedule_select): the default path (WA_SCHED_DEFAULT) if every head was
    skipped, else XCD-sliced.  Pass the same workspace to
    sparse_attn_fwd(schedule=WA_SCHED_AUTO)."""
    lib = load_library()
    _need(skipped, torch.uint8, "skipped", 1)
    _need(workspace, torch.uint8, "workspace", 1)
    _check(lib.wa_attn_schedule_select(_ptr(skipped), skipped.numel(), _ptr(workspace),
                                       workspace.numel(), _stream(skipped.device)),
           "wa_attn_schedule_select")


def xcd_placement(n_wg: int, block: int = 128, device=0) -> torch.Tensor:
    """XCD each of n_wg workgroups of the attention kernel's size ran on
    (wa_xcd_placement): the dispatch the XCD-sliced schedule relies on."""
    lib = load_library()
    dev = torch.device("cuda", device) if isinstance(device, int) else torch.device(device)
    out = torch.full((n_wg,), -1, dtype=torch.int32, device=dev)
    _check(lib.wa_xcd_placement(n_wg, block, _ptr(out), _stream(dev)), "wa_xcd_placement")
    return out


def sparse_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, seq_len: int,
                    block: int, row_ptr: torch.Tensor, col_idx: torch.Tensor,
                    perm: torch.Tensor | None = None, schedule: int = WA_SCHED_XCD_SLICED,
                    perm_slices: int | None = None,
                    scale: float | None = None, with_g: bool = False,
                    out: tuple | None = None, workspace: torch.Tensor | None = None,
                    entropy_out: torch.Tensor | None = None,
                    distance_out: torch.Tensor | None = None):
    """Block-sparse attention forward.  Returns (O bf16, LSE fp32, G fp32 or None).

    ``out`` may hold preallocated (O, LSE, G) tensors and ``workspace`` a uint8
    buffer of sparse_attn_workspace_size bytes, so that repeated calls allocate
    nothing and never wait on the device.  Without ``out`` and with ``with_g``, G is
    sized from the CSR's total, ``row_ptr[-1]``, which is read back to the host: that
    call synchronises with the stream (the C entry point itself never does).  With
    ``entropy_out`` and/or ``distance_out`` (float [H, L_pad]) the same
    pass also writes each row's attention entropy and mean attention distance in
    tokens (wa_sparse_attn_fwd_diag).  ``perm_slices`` is the n_slices ``perm`` was
    built with (``Reorder.n_slices``); the XCD-sliced and AUTO schedules need it and
    the library rejects a count other than the device's XCD count.
    """
    lib = load_library()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, torch.bfloat16, n, 3)
    if q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k and v must have the same shape [H, L_pad, d]")
    H, lp, d = q.shape
    mb = -(-seq_len // block)
    if lp != mb * block:
        raise ValueError(f"L_pad must be ceil(L / block) * block = {mb * block}, got {lp}")
    _need(row_ptr, torch.int32, "row_ptr", 1)
    _need(col_idx, torch.int32, "col_idx", 1)
    if row_ptr.numel() != H * mb + 1:
        raise ValueError("row_ptr must have H*MB+1 entries")
    if perm is not None:
        _need(perm, torch.int32, "perm")
        if perm.numel() != H * mb:
            raise ValueError("perm must have H*MB entries")
        if perm_slices is None and schedule in (WA_SCHED_XCD_SLICED, WA_SCHED_AUTO):
            raise ValueError("perm_slices (the n_slices perm was built with) is required with "
                             "the XCD-sliced and AUTO schedules")
    slices = 0 if perm is None or perm_slices is None else int(perm_slices)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dev = q.device
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty(H, lp, dtype=torch.float32, device=dev)
        g = None
        if with_g:
            nnz = int(row_ptr[-1].item())
            g = torch.empty(max(nnz, 1), block, dtype=torch.float32, device=dev)
    else:
        o, lse, g = out
        if not with_g:
            g = None
    ws_bytes = sparse_attn_workspace_size(H, seq_len, d, block)
    if schedule == WA_SCHED_AUTO and workspace is None:
        raise ValueError("WA_SCHED_AUTO reads its choice from the workspace that "
                         "attn_schedule_select wrote; pass that workspace")
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    cap = col_idx.numel() if g is None else min(col_idx.numel(), g.shape[0])
    if entropy_out is not None or distance_out is not None:
        for t, n in ((entropy_out, "entropy_out"), (distance_out, "distance_out")):
            if t is not None:
                _need(t, torch.float32, n, 2)
                if tuple(t.shape) != (H, lp):
                    raise ValueError(f"{n} must be [H, L_pad]")
        _check(lib.wa_sparse_attn_fwd_diag(
            _ptr(q), _ptr(k), _ptr(v), H, seq_len, d, block, _ptr(row_ptr), _ptr(col_idx), cap,
            _ptr(perm), slices, schedule, scale, _ptr(o), _ptr(lse), _ptr(g), _ptr(entropy_out),
            _ptr(distance_out), _ptr(workspace), workspace.numel(), _stream(dev)),
            "wa_sparse_attn_fwd_diag")
        return o, lse, g
    _check(lib.wa_sparse_attn_fwd(_ptr(q), _ptr(k), _ptr(v), H, seq_len, d, block,
                                  _ptr(row_ptr), _ptr(col_idx), cap, _ptr(perm), slices,
                                  schedule, scale,
                                  _ptr(o), _ptr(lse), _ptr(g), _ptr(workspace),
                                  workspace.numel(), _stream(dev)), "wa_sparse_attn_fwd")
    return o, lse, g


def block_importance(g: torch.Tensor, lse: torch.Tensor, row_ptr: torch.Tensor, seq_len: int,
                     block: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """GSRS Phase 2: W [nnz] from G [nnz, block] and the row LSE [H, L_pad]."""
    lib = load_library()
    _need(g, torch.float32, "g", 2)
    _need(lse, torch.float32, "lse", 2)
    _need(row_ptr, torch.int32, "row_ptr", 1)
    H, lp = lse.shape
    mb = lp // block
    w = out if out is not None else torch.empty(g.shape[0], dtype=torch.float32, device=g.device)
    cap = min(g.shape[0], w.numel())
    _check(lib.wa_block_importance(_ptr(g), _ptr(lse), _ptr(row_ptr), cap, H, mb, seq_len, block,
                                   _ptr(w), _stream(g.device)), "wa_block_importance")
    return w


def topp_select(w: torch.Tensor, row_ptr: torch.Tensor, col_idx: torch.Tensor, heads: int,
                mb: int, nb: int, p: float, out: torch.Tensor | None = None) -> torch.Tensor:
    """GSRS Top-p selection: uint8 mask [H, MB, NB] of the kept blocks."""
    lib = load_library()
    _need(w, torch.float32, "w", 1)
    _need(row_ptr, torch.int32, "row_ptr", 1)
    _need(col_idx, torch.int32, "col_idx", 1)
    m = out if out is not None else torch.empty(heads, mb, nb, dtype=torch.uint8, device=w.device)
    cap = min(w.numel(), col_idx.numel())
    _check(lib.wa_topp_select(_ptr(w), _ptr(row_ptr), _ptr(col_idx), cap, heads, mb, nb, float(p),
                              _ptr(m), _stream(w.device)), "wa_topp_select")
    return m


def mask_recall(w: torch.Tensor, row_ptr: torch.Tensor, col_idx: torch.Tensor,
                mask: torch.Tensor) -> torch.Tensor:
    """GSRS attention recall of ``mask`` [H, MB, NB] per query block, float [H, MB], from
    the block weights ``w`` of an evaluated pass (its index row_ptr / col_idx)."""
    lib = load_library()
    _need(w, torch.float32, "w", 1)
    _need(row_ptr, torch.int32, "row_ptr", 1)
    _need(col_idx, torch.int32, "col_idx", 1)
    _need(mask, torch.uint8, "mask", 3)
    heads, mb, nb = mask.shape
    if row_ptr.numel() != heads * mb + 1:
        raise ValueError("row_ptr does not match the mask's H * MB rows")
    out = torch.empty(heads, mb, dtype=torch.float32, device=w.device)
    cap = min(w.numel(), col_idx.numel())
    _check(lib.wa_mask_recall(_ptr(w), _ptr(row_ptr), _ptr(col_idx), cap, heads, mb, nb,
                              _ptr(mask), _ptr(out), _stream(w.device)), "wa_mask_recall")
    return out


def gather_blocks(src: torch.Tensor, perm: torch.Tensor, rows_per_block: int) -> torch.Tensor:
    """dst[h, s-th block] = src[h, perm[h, s]-th block] along dim 1."""
    return _permute(src, perm, rows_per_block, scatter=False)


def scatter_blocks(src: torch.Tensor, perm: torch.Tensor, rows_per_block: int) -> torch.Tensor:
    """dst[h, perm[h, s]-th block] = src[h, s-th block] along dim 1."""
    return _permute(src, perm, rows_per_block, scatter=True)


def _permute(src, perm, rows_per_block, scatter):
    lib = load_library()
    if not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous GPU tensor")
    _need(perm, torch.int32, "perm", 2)
    H, mb = perm.shape
    if src.shape[0] != H or src.shape[1] != mb * rows_per_block:
        raise ValueError("src must be [H, MB*rows_per_block, ...]")
    dst = torch.empty_like(src)
    row_bytes = src[0, 0].numel() * src.element_size()
    fn = lib.wa_scatter_blocks if scatter else lib.wa_gather_blocks
    _check(fn(_ptr(src), _ptr(dst), _ptr(perm), H, mb, rows_per_block * row_bytes,
              _stream(src.device)), "wa_scatter_blocks" if scatter else "wa_gather_blocks")
    return dst

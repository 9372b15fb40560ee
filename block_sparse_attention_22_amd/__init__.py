"""FVAttn block-sparse attention hot path for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI of ``libfvattn.so`` (``include/fvattn.h``):
argument marshalling only.  Every step of the path runs in the library's HIP
kernels; PyTorch only supplies device memory and the current stream.  If the
library has not been built, every call raises - there is no fallback.

    lists = route(q, k, p, kmin, budget, grid=(T, Y, X), tile=(tt, ty, tx))
    o     = sparse_attn(q, k, v, lists)

Blocks are 3D tiles (``tile``) or consecutive 128-token runs of a token order
(``order=hilbert_order(grid, device)`` for the Hilbert-curve organisation).

q, k, v: CUDA (HIP) tensors [B, H, N, d] (bf16 or float32, d in {64, 128},
last dim contiguous) with N = T*Y*X tokens in (t, y, x) raster order.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import threading
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfvattn.so")

FVA_OK, FVA_ERR_INVALID_ARG, FVA_ERR_UNSUPPORTED, FVA_ERR_WORKSPACE, FVA_ERR_HIP = 0, -1, -2, -3, -4
FVA_ERR_SCRATCH = -5
STATIC_SCRATCH_BYTES = 64 << 20     # FVA_STATIC_SCRATCH_BYTES
FVA_BF16, FVA_F32 = 0, 1
BUDGET_MODES = {"none": 0, "frac": 1, "match_max": 2}


class Problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("grid_t", ctypes.c_int32), ("grid_y", ctypes.c_int32), ("grid_x", ctypes.c_int32),
                ("tile_t", ctypes.c_int32), ("tile_y", ctypes.c_int32), ("tile_x", ctypes.c_int32),
                ("dtype", ctypes.c_int32),
                ("stride_b", ctypes.c_int64), ("stride_h", ctypes.c_int64), ("stride_n", ctypes.c_int64),
                ("token_order", ctypes.c_void_p)]


class Budget(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("frac", ctypes.c_double)]


class ListsC(ctypes.Structure):
    _fields_ = [("row_ptr", ctypes.c_void_p), ("col_idx", ctypes.c_void_p), ("base_count", ctypes.c_void_p),
                ("head_kept", ctypes.c_void_p), ("mask", ctypes.c_void_p)]


class AttnOptions(ctypes.Structure):
    _fields_ = [("chunk_blocks", ctypes.c_int32), ("num_ctas", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("reserved", ctypes.c_int32), ("kernel_events", ctypes.c_void_p * 2)]


FVA_ATTN_PREPARED = 1
FVA_ATTN_NO_ROW_PAIRS = 2


class PlanInfo(ctypes.Structure):
    _fields_ = [("n_items", ctypes.c_int32), ("chunk_blocks", ctypes.c_int32), ("n_split_rows", ctypes.c_int32),
                ("n_partials", ctypes.c_int32), ("total_blocks", ctypes.c_int64), ("num_ctas", ctypes.c_int32),
                ("n_row_pairs", ctypes.c_int32), ("kept_pairs", ctypes.c_int64),
                ("predicted_imbalance", ctypes.c_float), ("reserved", ctypes.c_int32)]


class CtaStat(ctypes.Structure):
    _fields_ = [("hw_id", ctypes.c_uint32), ("xcc_id", ctypes.c_uint32), ("items", ctypes.c_uint32),
                ("blocks", ctypes.c_uint32), ("t_start", ctypes.c_uint64), ("t_end", ctypes.c_uint64)]


EXPORTS = ("fva_num_blocks", "fva_block_sizes", "fva_hilbert_order", "fva_lists_capacity", "fva_route_workspace_bytes",
           "fva_route", "fva_route_static",
           "fva_attn_workspace_bytes", "fva_attn_stats_bytes", "fva_attn_prepare", "fva_sparse_attn",
           "fva_layer_workspace_bytes", "fva_layer", "fva_status_string")

_lib = None
_lib_lock = threading.Lock()


class FvaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


def load_library(path: Optional[str] = None):
    """Load libfvattn.so (built by ``__graft_entry__.build()``); raises if absent."""
    global _lib
    with _lib_lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError(f"{p} is not built: run `python -c 'import __graft_entry__ as g; g.build()'`")
        lib = ctypes.CDLL(p)
        P = ctypes.POINTER
        lib.fva_num_blocks.argtypes = [P(Problem), P(ctypes.c_int32), P(ctypes.c_int32)]
        lib.fva_block_sizes.argtypes = [P(Problem), P(ctypes.c_int32)]
        lib.fva_block_sizes.restype = ctypes.c_int
        lib.fva_hilbert_order.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P(ctypes.c_int32)]
        lib.fva_hilbert_order.restype = ctypes.c_int
        lib.fva_num_blocks.restype = ctypes.c_int
        lib.fva_lists_capacity.argtypes = [P(Problem)]
        lib.fva_lists_capacity.restype = ctypes.c_size_t
        lib.fva_route_workspace_bytes.argtypes = [P(Problem)]
        lib.fva_route_workspace_bytes.restype = ctypes.c_size_t
        lib.fva_route.argtypes = [P(Problem), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_double, ctypes.c_int32,
                                  Budget, P(ListsC), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        lib.fva_route.restype = ctypes.c_int
        lib.fva_route_static.argtypes = [P(Problem), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_double,
                                         ctypes.c_int32, Budget, P(ListsC), ctypes.c_void_p]
        lib.fva_route_static.restype = ctypes.c_int
        lib.fva_attn_workspace_bytes.argtypes = [P(Problem), P(AttnOptions)]
        lib.fva_attn_workspace_bytes.restype = ctypes.c_size_t
        lib.fva_attn_stats_bytes.argtypes = [P(Problem), P(AttnOptions)]
        lib.fva_attn_stats_bytes.restype = ctypes.c_size_t
        lib.fva_sparse_attn.argtypes = [P(Problem), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, P(ListsC),
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                        P(AttnOptions), ctypes.c_void_p]
        lib.fva_sparse_attn.restype = ctypes.c_int
        lib.fva_attn_prepare.argtypes = [P(Problem), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_size_t, P(AttnOptions), ctypes.c_void_p]
        lib.fva_attn_prepare.restype = ctypes.c_int
        lib.fva_layer_workspace_bytes.argtypes = [P(Problem), P(AttnOptions)]
        lib.fva_layer_workspace_bytes.restype = ctypes.c_size_t
        lib.fva_layer.argtypes = [P(Problem), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_double,
                                  ctypes.c_int32, P(Budget), P(ListsC), ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_size_t, ctypes.c_void_p, P(AttnOptions), ctypes.c_void_p]
        lib.fva_layer.restype = ctypes.c_int
        lib.fva_status_string.argtypes = [ctypes.c_int]
        lib.fva_status_string.restype = ctypes.c_char_p
        if path is None:
            _lib = lib
        return lib


def status_string(status: int) -> str:
    try:
        return load_library().fva_status_string(status).decode()
    except Exception:  # pragma: no cover - only when the library is absent
        return "unknown"


def _check_order(order, N, device):
    if order is None:
        return None
    if not order.is_cuda or order.dtype != torch.int32 or order.dim() != 1 or order.numel() != N \
            or not order.is_contiguous():
        raise ValueError(f"order must be a contiguous int32 device tensor of the grid's {N} tokens")
    if device is not None and order.device != device:
        raise ValueError("order must live on the device of the activations")
    return order.data_ptr()


def make_problem(x: torch.Tensor, grid, tile, order: Optional[torch.Tensor] = None) -> Problem:
    """Problem descriptor for a [B, H, N, d] tensor laid out like x; blocks are
    tiles, or 128-token runs of ``order`` when it is given."""
    if x.dim() != 4:
        raise ValueError("expected a [B, H, N, d] tensor")
    B, H, N, d = x.shape
    T, Y, X = (int(a) for a in grid)
    if T * Y * X != N:
        raise ValueError(f"grid {grid} has {T * Y * X} tokens but the tensor has N={N}")
    if x.stride(3) != 1:
        raise ValueError("the head dimension must be contiguous")
    if x.dtype == torch.bfloat16:
        dt = FVA_BF16
    elif x.dtype == torch.float32:
        dt = FVA_F32
    else:
        raise ValueError(f"unsupported dtype {x.dtype}")
    tt, ty, tx = (int(a) for a in tile) if tile is not None else (1, 1, 1)
    if tile is None and order is None:
        raise ValueError("give tile or order")
    return Problem(B, H, d, T, Y, X, tt, ty, tx, dt, x.stride(0), x.stride(1), x.stride(2),
                   _check_order(order, N, x.device))


_hilbert_cache = {}


def hilbert_order(grid, device=None) -> torch.Tensor:
    """Tokens of a T x Y x X grid in 3D Hilbert-curve order (fva_hilbert_order,
    computed on the host once per grid and device), as int32 on ``device``."""
    import numpy as np
    T, Y, X = (int(a) for a in grid)
    key = (T, Y, X, str(device))
    t = _hilbert_cache.get(key)
    if t is None:
        host = np.empty(T * Y * X, dtype=np.int32)
        st = load_library().fva_hilbert_order(T, Y, X, host.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
        if st != FVA_OK:
            raise FvaError(st, "fva_hilbert_order")
        t = torch.from_numpy(host)
        if device is not None:
            t = t.to(device)
        _hilbert_cache[key] = t
    return t


def _shape_problem(grid, tile, ordered, B=1, H=1, d=128, dtype=torch.bfloat16) -> Problem:
    """A problem descriptor that carries only a shape (the calls that take it
    compute counts and never touch device memory)."""
    T, Y, X = (int(a) for a in grid)
    return Problem(B, H, d, T, Y, X, *(tile if tile is not None else (1, 1, 1)),
                   FVA_BF16 if dtype == torch.bfloat16 else FVA_F32, H * T * Y * X * d, T * Y * X * d, d,
                   256 if ordered else None)      # any aligned non-null address stands for a token order


def block_sizes(grid, tile, ordered: bool = False):
    """Valid tokens of every block (fva_block_sizes): tile raster order (edge
    tiles hold fewer), or, ``ordered``, 128-token runs of a token order."""
    import numpy as np
    p = _shape_problem(grid, tile, ordered)
    nq = ctypes.c_int32()
    lib = load_library()
    st = lib.fva_num_blocks(ctypes.byref(p), ctypes.byref(nq), ctypes.byref(ctypes.c_int32()))
    if st != FVA_OK:
        raise FvaError(st, "fva_num_blocks")
    out = np.empty(nq.value, dtype=np.int32)
    st = lib.fva_block_sizes(ctypes.byref(p), out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    if st != FVA_OK:
        raise FvaError(st, "fva_block_sizes")
    return out.astype(np.int64)


def num_blocks(grid, tile, *, B=1, H=1, d=128, dtype=torch.bfloat16, ordered: bool = False) -> int:
    p = _shape_problem(grid, tile, ordered, B, H, d, dtype)
    nq, nk = ctypes.c_int32(), ctypes.c_int32()
    st = load_library().fva_num_blocks(ctypes.byref(p), ctypes.byref(nq), ctypes.byref(nk))
    if st != FVA_OK:
        raise FvaError(st, "fva_num_blocks")
    return nq.value


# Workspaces are plain device byte buffers owned here, one per (kind of
# call, device, stream), reused between calls and grown on demand.  Calls on
# one stream run in order, so they can share one; calls on different streams
# get different buffers and never race.  A buffer is allocated while its own
# stream is current, so when it is replaced the caching allocator hands its
# memory to other work only in that stream's order.
_ws_cache = {}


def _workspace(nbytes: int, device, key: str, stream=None) -> torch.Tensor:
    s = stream if stream is not None else torch.cuda.current_stream(device)
    k = (key, device.index if device.index is not None else torch.cuda.current_device(), s.cuda_stream)
    buf = _ws_cache.get(k)
    if buf is None or buf.numel() < nbytes:
        with torch.cuda.stream(s):
            buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _ws_cache[k] = buf
    return buf


def release_workspaces() -> None:
    """Drop every cached workspace (each is freed in its own stream's order)."""
    _ws_cache.clear()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _check_device_tensor(name, t):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


@dataclasses.dataclass
class BlockLists:
    """CSR block lists written by ``route`` (all int32 device tensors)."""
    row_ptr: torch.Tensor        # [B*H*Nq + 1]
    col_idx: torch.Tensor        # [B*H*Nq*Nk] capacity; valid prefix row_ptr[-1]
    base_count: torch.Tensor     # [B*H*Nq]
    head_kept: torch.Tensor      # [B*H]
    mask: Optional[torch.Tensor]  # [B*H*Nq*ceil(Nk/32)] int32 bit words, or None
    nq: int
    nk: int
    grid: Tuple[int, int, int]
    tile: Optional[Tuple[int, int, int]]
    order: Optional[torch.Tensor] = None   # token order of the blocks (device int32), or None for tiles

    def as_c(self) -> ListsC:
        return ListsC(self.row_ptr.data_ptr(), self.col_idx.data_ptr(), self.base_count.data_ptr(),
                      self.head_kept.data_ptr(), self.mask.data_ptr() if self.mask is not None else None)


def _budget(budget) -> Budget:
    if budget is None:
        return Budget(0, 0.0)
    mode, frac = budget
    return Budget(BUDGET_MODES[mode], float(frac))


def _route_setup(q, k, grid, tile, order, want_mask, out):
    _check_device_tensor("q", q)
    _check_device_tensor("k", k)
    if q.shape != k.shape or q.dtype != k.dtype or q.stride() != k.stride():
        raise ValueError("q and k must share shape, dtype and strides")
    lib = load_library()
    prob = make_problem(q, grid, tile, order)
    nb = ctypes.c_int32()
    st = lib.fva_num_blocks(ctypes.byref(prob), ctypes.byref(nb), ctypes.byref(ctypes.c_int32()))
    if st != FVA_OK:
        raise FvaError(st, "fva_route")
    nb = nb.value
    B, H = q.shape[:2]
    R = B * H * nb
    dev = q.device
    if out is None:
        words = (nb + 31) // 32
        out = BlockLists(
            row_ptr=torch.empty(R + 1, dtype=torch.int32, device=dev),
            col_idx=torch.empty(max(1, lib.fva_lists_capacity(ctypes.byref(prob))), dtype=torch.int32, device=dev),
            base_count=torch.empty(max(1, R), dtype=torch.int32, device=dev),
            head_kept=torch.empty(max(1, B * H), dtype=torch.int32, device=dev),
            mask=torch.empty(max(1, R * words), dtype=torch.int32, device=dev) if want_mask else None,
            nq=nb, nk=nb, grid=tuple(grid), tile=tuple(tile) if tile is not None else None, order=order)
    return lib, prob, out


def route(q: torch.Tensor, k: torch.Tensor, p: float, kmin: int, budget=None, *, grid, tile=None,
          order: Optional[torch.Tensor] = None,
          want_mask: bool = False, out: Optional[BlockLists] = None) -> BlockLists:
    """Sparse-routing front end (fva_route): per-head CSR block lists.

    Runs on the current stream with that stream's routing workspace."""
    lib, prob, out = _route_setup(q, k, grid, tile, order, want_mask, out)
    dev = q.device
    wsb = lib.fva_route_workspace_bytes(ctypes.byref(prob))
    ws = _workspace(wsb, dev, "route")
    lc = out.as_c()
    st = lib.fva_route(ctypes.byref(prob), q.data_ptr(), k.data_ptr(), float(p), int(kmin), _budget(budget),
                       ctypes.byref(lc), ws.data_ptr(), ws.numel(), _stream(dev))
    if st != FVA_OK:
        raise FvaError(st, "fva_route")
    return out


def route_static(q: torch.Tensor, k: torch.Tensor, p: float, kmin: int, budget=None, *, grid, tile=None,
                 order: Optional[torch.Tensor] = None, out: BlockLists) -> BlockLists:
    """fva_route_static: ``route`` into caller-allocated ``out`` lists with the
    library's static per-device scratch (no allocation of any kind; problems
    whose routing workspace exceeds STATIC_SCRATCH_BYTES raise FVA_ERR_SCRATCH).
    Calls that overlap on one device race; keep them on one stream."""
    lib, prob, out = _route_setup(q, k, grid, tile, order, False, out)
    lc = out.as_c()
    st = lib.fva_route_static(ctypes.byref(prob), q.data_ptr(), k.data_ptr(), float(p), int(kmin),
                              _budget(budget), ctypes.byref(lc), _stream(q.device))
    if st != FVA_OK:
        raise FvaError(st, "fva_route_static")
    return out


def _event_handle(e) -> int:
    """Raw hipEvent_t of a torch.cuda.Event (created on first use) or an int."""
    if isinstance(e, int):
        return e
    if not e.cuda_event:
        e.record()          # torch creates the underlying event lazily
    return int(e.cuda_event)


def attn_options(chunk_blocks: int = 0, num_ctas: int = 0, kernel_events=None, prepared: bool = False,
                 row_pairs: bool = True) -> AttnOptions:
    o = AttnOptions()
    o.chunk_blocks = int(chunk_blocks)
    o.num_ctas = int(num_ctas)
    o.flags = (FVA_ATTN_PREPARED if prepared else 0) | (0 if row_pairs else FVA_ATTN_NO_ROW_PAIRS)
    if kernel_events is not None:
        e0, e1 = kernel_events
        o.kernel_events[0] = _event_handle(e0)
        o.kernel_events[1] = _event_handle(e1)
    return o


def stats_bytes(q: torch.Tensor, grid, tile=None, chunk_blocks: int = 0, num_ctas: int = 0,
                order: Optional[torch.Tensor] = None) -> int:
    prob = make_problem(q, grid, tile, order)
    opts = attn_options(chunk_blocks, num_ctas)
    return load_library().fva_attn_stats_bytes(ctypes.byref(prob), ctypes.byref(opts))


def _check_qkv(q, k, v):
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_device_tensor(name, t)
    if not (q.shape == k.shape == v.shape) or not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k and v must share shape and dtype")
    if not (q.stride() == k.stride() == v.stride()):
        raise ValueError("q, k and v must share strides")


def attn_prepare(k: torch.Tensor, v: torch.Tensor, *, grid, tile=None, chunk_blocks: int = 0,
                 num_ctas: int = 0, order: Optional[torch.Tensor] = None, stream=None) -> None:
    """The list-independent part of sparse_attn (fva_attn_prepare), enqueued
    on the current stream, into the attention workspace of ``stream`` (the
    stream on which the matching ``sparse_attn(..., prepared=True)`` with the
    same k, v and options will run; default: the current stream).  The
    caller orders the two (and this call after any earlier sparse_attn on
    ``stream`` still reading that workspace), e.g. with
    ``Stream.wait_stream``."""
    _check_qkv(k, k, v)
    lib = load_library()
    prob = make_problem(k, grid, tile, order)
    opts = attn_options(chunk_blocks, num_ctas)
    wsb = lib.fva_attn_workspace_bytes(ctypes.byref(prob), ctypes.byref(opts))
    if wsb == 0:
        raise FvaError(FVA_ERR_INVALID_ARG, "fva_attn_workspace_bytes")
    cur = torch.cuda.current_stream(k.device)
    ws = _workspace(wsb, k.device, "attn", stream)
    if stream is not None and stream.cuda_stream != cur.cuda_stream:
        ws.record_stream(cur)     # the copies are written on this stream
    st = lib.fva_attn_prepare(ctypes.byref(prob), k.data_ptr(), v.data_ptr(), ws.data_ptr(), ws.numel(),
                              ctypes.byref(opts), cur.cuda_stream)
    if st != FVA_OK:
        raise FvaError(st, "fva_attn_prepare")


def sparse_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, lists: BlockLists, *,
                out: Optional[torch.Tensor] = None, stats: Optional[torch.Tensor] = None,
                chunk_blocks: int = 0, num_ctas: int = 0, kernel_events=None,
                prepared: bool = False, row_pairs: bool = True) -> torch.Tensor:
    """Block-sparse attention over the kept blocks (fva_sparse_attn).

    ``stats``: optional uint8 device tensor of ``stats_bytes(...)`` bytes that
    receives the plan header and per-workgroup timing records.
    ``kernel_events``: optional pair of timing-enabled torch.cuda.Event (or raw
    hipEvent_t ints) recorded right before and after the attention kernel.
    ``prepared``: ``attn_prepare(k, v, ..., stream=<this call's stream>)``
    already ran (ordered before this call) with the same tensors and options.
    Runs on the current stream with that stream's attention workspace.
    ``row_pairs``: let neighbouring query blocks of at most 64 tokens share a
    work item (bf16, head_dim 128; off: FVA_ATTN_NO_ROW_PAIRS).
    """
    _check_qkv(q, k, v)
    lib = load_library()
    prob = make_problem(q, lists.grid, lists.tile, lists.order)
    if out is None:
        out = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    if out.stride() != q.stride() or out.dtype != q.dtype:
        raise ValueError("out must match q's strides and dtype")
    opts = attn_options(chunk_blocks, num_ctas, kernel_events, prepared, row_pairs)
    wsb = lib.fva_attn_workspace_bytes(ctypes.byref(prob), ctypes.byref(opts))
    if wsb == 0:
        raise FvaError(FVA_ERR_INVALID_ARG, "fva_attn_workspace_bytes")
    ws = _workspace(wsb, q.device, "attn")
    sp = None
    if stats is not None:
        need = lib.fva_attn_stats_bytes(ctypes.byref(prob), ctypes.byref(opts))
        if stats.numel() * stats.element_size() < need:
            raise ValueError(f"stats buffer needs {need} bytes")
        sp = stats.data_ptr()
    lc = lists.as_c()
    st = lib.fva_sparse_attn(ctypes.byref(prob), q.data_ptr(), k.data_ptr(), v.data_ptr(), ctypes.byref(lc),
                             out.data_ptr(), ws.data_ptr(), ws.numel(), sp, ctypes.byref(opts), _stream(q.device))
    if st != FVA_OK:
        raise FvaError(st, "fva_sparse_attn")
    return out


def layer(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, p: float, kmin: int, budget=None, *, grid, tile=None,
          order: Optional[torch.Tensor] = None, lists: Optional[BlockLists] = None,
          out: Optional[torch.Tensor] = None, stats: Optional[torch.Tensor] = None, chunk_blocks: int = 0,
          num_ctas: int = 0, kernel_events=None, row_pairs: bool = True):
    """route then sparse_attn in one call (fva_layer), sharing one read of q, k
    and v for bf16, head_dim 128; returns (lists, out), bit for bit those of
    the two calls.  Runs on the current stream with that stream's layer
    workspace."""
    _check_qkv(q, k, v)
    lib, prob, lists = _route_setup(q, k, grid, tile, order, False, lists)
    if out is None:
        out = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    if out.stride() != q.stride() or out.dtype != q.dtype:
        raise ValueError("out must match q's strides and dtype")
    opts = attn_options(chunk_blocks, num_ctas, kernel_events, False, row_pairs)
    wsb = lib.fva_layer_workspace_bytes(ctypes.byref(prob), ctypes.byref(opts))
    if wsb == 0:
        raise FvaError(FVA_ERR_INVALID_ARG, "fva_layer_workspace_bytes")
    ws = _workspace(wsb, q.device, "layer")
    sp = None
    if stats is not None:
        need = lib.fva_attn_stats_bytes(ctypes.byref(prob), ctypes.byref(opts))
        if stats.numel() * stats.element_size() < need:
            raise ValueError(f"stats buffer needs {need} bytes")
        sp = stats.data_ptr()
    lc = lists.as_c()
    bud = _budget(budget)
    st = lib.fva_layer(ctypes.byref(prob), q.data_ptr(), k.data_ptr(), v.data_ptr(), float(p), int(kmin),
                       ctypes.byref(bud), ctypes.byref(lc), out.data_ptr(), ws.data_ptr(), ws.numel(), sp,
                       ctypes.byref(opts), _stream(q.device))
    if st != FVA_OK:
        raise FvaError(st, "fva_layer")
    return lists, out


def lists_from_csr(row_ptr, col_idx, *, nq, grid, tile=None, device, order=None) -> BlockLists:
    """Wrap host CSR arrays (e.g. lists made elsewhere) as device BlockLists."""
    rp = torch.as_tensor(row_ptr, dtype=torch.int32).to(device)
    ci = torch.as_tensor(col_idx, dtype=torch.int32)
    if ci.numel() == 0:
        ci = torch.zeros(1, dtype=torch.int32)
    ci = ci.to(device)
    R = rp.numel() - 1
    return BlockLists(row_ptr=rp, col_idx=ci, base_count=torch.empty(max(R, 1), dtype=torch.int32, device=device),
                      head_kept=torch.empty(1, dtype=torch.int32, device=device), mask=None, nq=nq, nk=nq,
                      grid=tuple(grid), tile=tuple(tile) if tile is not None else None, order=order)


def parse_stats(stats: torch.Tensor):
    """Host view of a stats buffer: (PlanInfo, list of CtaStat)."""
    raw = stats.detach().cpu().numpy().tobytes()
    info = PlanInfo.from_buffer_copy(raw[:ctypes.sizeof(PlanInfo)])
    n = info.num_ctas
    off = ctypes.sizeof(PlanInfo)
    sz = ctypes.sizeof(CtaStat)
    ctas = [CtaStat.from_buffer_copy(raw[off + i * sz: off + (i + 1) * sz]) for i in range(n)]
    return info, ctas


def cu_key(st: CtaStat) -> int:
    """A compute unit's identity from HW_ID (CU_ID, SH_ID, SE_ID: bits 8-15) and XCC_ID."""
    return ((st.xcc_id & 0xF) << 8) | ((st.hw_id >> 8) & 0xFF)


def per_cu_imbalance(ctas, num_cus: int):
    """Busy time per compute unit (sum over its workgroups) -> (max/mean, busy dict).

    The mean is over ``num_cus`` compute units, so a CU that ran nothing counts
    as idle."""
    busy = {}
    for c in ctas:
        busy[cu_key(c)] = busy.get(cu_key(c), 0) + (c.t_end - c.t_start)
    if not busy:
        return 1.0, busy
    mean = sum(busy.values()) / max(num_cus, len(busy))
    return (max(busy.values()) / mean if mean > 0 else 1.0), busy


__all__ = ["route", "route_static", "sparse_attn", "layer", "BlockLists", "make_problem", "num_blocks", "block_sizes", "load_library", "FvaError",
           "stats_bytes", "parse_stats", "attn_prepare", "release_workspaces", "FVA_ATTN_PREPARED", "hilbert_order", "per_cu_imbalance", "lists_from_csr", "EXPORTS", "LIB_PATH"]

"""Exact grouped-query attention forward for MI355X (gfx950): a thin binding of ``libattn_gqa.so``.

Every function here only marshals arguments into the C ABI declared in
``include/attn_gqa.h`` (same names); all arithmetic runs in the library's HIP kernels.
PyTorch supplies device memory and the current stream.  If the library is missing the
calls raise ``RuntimeError``: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libattn_gqa.so")

ATTN_OK = 0
ATTN_ERR_NULL = -1
ATTN_ERR_SHAPE = -2
ATTN_ERR_UNSUPPORTED = -3
ATTN_ERR_ALIGN = -4
ATTN_ERR_WORKSPACE = -5
ATTN_ERR_HIP = -6
ATTN_MAX_BATCH = 256
ATTN_MAX_COLUMNS = 64
ATTN_MAX_COLUMN_ELEMS = 8192
ATTN_MAX_CTAS = 4096
ATTN_DECODE_COUNTER_BYTES = 32768
ATTN_DECODE_PLAN_BYTES = 8192
ATTN_NOALLOC_SCRATCH_BYTES = 32 << 20
ATTN_SCHEDULE_AUTO = 0
ATTN_SCHEDULE_STREAM_K = 1
ATTN_SCHEDULE_FIXED_SPLIT = 2
ATTN_KV_BF16 = 0
ATTN_KV_FP8_E4M3 = 1

_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64


class AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


class attn_decode_args(ctypes.Structure):
    _fields_ = [
        ("q", _P), ("k_cache", _P), ("v_cache", _P), ("seqlens", _P), ("out", _P),
        ("B", _I), ("Hq", _I), ("KH", _I), ("Hsz", _I),
        ("kv_stride", _I64), ("scale", ctypes.c_float),
        ("workspace", _P), ("workspace_bytes", ctypes.c_size_t),
        ("tile_keys", _I), ("num_ctas", _I),
        ("ev_tiles_begin", _P), ("ev_tiles_end", _P),
        ("schedule", _I), ("num_splits", _I),
        ("kv_dtype", _I), ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
        ("block_table", _P), ("block_size", _I), ("max_blocks_per_seq", _I), ("num_blocks", _I),
        ("q_len", _I), ("seqlens_on_device", _I), ("out_lse", _P),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m attention_gqa_decode_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    L.attn_decode.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _P, _P]
    L.attn_decode.restype = _I
    L.attn_decode_ex.argtypes = [ctypes.POINTER(attn_decode_args), _P]
    L.attn_decode_ex.restype = _I
    L.attn_decode_noalloc.argtypes = [ctypes.POINTER(attn_decode_args), _P]
    L.attn_decode_noalloc.restype = _I
    L.attn_decode_workspace_bytes.argtypes = [_I, _I, _I, _I, _I]
    L.attn_decode_workspace_bytes.restype = ctypes.c_size_t
    L.attn_decode_multi_workspace_bytes.argtypes = [_I, _I, _I, _I, _I, _I]
    L.attn_decode_multi_workspace_bytes.restype = ctypes.c_size_t
    L.attn_prefill_causal.argtypes = [_P, _P, _P, _I, _I, _I, _I, _I, _P, _P]
    L.attn_prefill_causal.restype = _I
    L.attn_decode_plan.argtypes = [_P, _I, _I, _I, _I, _P, _P, _P, _P]
    L.attn_decode_plan.restype = _I
    L.attn_hbm_copy_probe.argtypes = [_P, _P, ctypes.c_size_t, _P]
    L.attn_hbm_copy_probe.restype = _I
    L.attn_hbm_read_probe.argtypes = [_P, ctypes.c_size_t, _P, _P]
    L.attn_hbm_read_probe.restype = _I
    L.attn_merge_shards.argtypes = [_P, _P, _I, _I64, _I, _P, _P, _P]
    L.attn_merge_shards.restype = _I
    L.attn_device_info.argtypes = [_P, _P]
    L.attn_device_info.restype = _I
    L.attn_release.argtypes = []
    L.attn_release.restype = _I
    L.attn_status_string.argtypes = [_I]
    L.attn_status_string.restype = ctypes.c_char_p
    L.attn_last_error.argtypes = []
    L.attn_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(status: int) -> None:
    if status != ATTN_OK:
        L = lib()
        msg = L.attn_last_error().decode() or L.attn_status_string(status).decode()
        raise AttnError(status, msg)


def _stream_handle(stream=None) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _bf16_cuda(name, t):
    import torch
    if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous bf16 CUDA tensor (got {t.dtype}, {t.device})")


def _kv_cuda(name, t):
    """K/V cache check: bf16, or FP8 E4M3 (torch.float8_e4m3fn or raw uint8 codes).  Returns kv_dtype."""
    import torch
    if not t.is_cuda or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous CUDA tensor (got {t.device})")
    if t.dtype == torch.bfloat16:
        return ATTN_KV_BF16
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return ATTN_KV_FP8_E4M3
    raise TypeError(f"{name} must be bf16 or FP8 E4M3 (float8_e4m3fn / uint8 codes), got {t.dtype}")


def _host_seqlens(seqlens):
    import numpy as np
    import torch
    if isinstance(seqlens, torch.Tensor):
        seqlens = seqlens.detach().cpu().numpy()
    arr = np.ascontiguousarray(np.asarray(seqlens), dtype=np.int32)
    return arr


def _seqlens_arg(seqlens, B):
    """(pointer, on_device, owner) for attn_decode_args.seqlens: a CUDA int32 tensor is
    passed as device seqlens (never read on the host); anything else becomes a host array."""
    import torch
    if isinstance(seqlens, torch.Tensor) and seqlens.is_cuda:
        if seqlens.dtype != torch.int32 or not seqlens.is_contiguous() or seqlens.numel() != B:
            raise TypeError("device seqlens must be a contiguous int32 CUDA tensor with B entries")
        return seqlens.data_ptr(), 1, seqlens
    sl = _host_seqlens(seqlens)
    if len(sl) != B:
        raise ValueError("seqlens must have B entries")
    return sl.ctypes.data, 0, sl


def _f32_cuda(name, t, shape):
    """`t` must be a contiguous fp32 CUDA tensor of the given shape (the library writes it)."""
    import torch
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous fp32 CUDA tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")


def _decode_args(q, k_cache, v_cache, seqlens, out, *, q_len, multi, paged, block_table, scale, tile_keys, num_ctas,
                 schedule, num_splits, k_scale, v_scale, out_lse, workspace):
    """Checks the tensors of one decode call and packs its attn_decode_args.

    Returns (args, keep): `keep` holds the objects whose memory the packed pointers refer to.
    q is [B][Hq][Hsz], or [B][Hq][q_len][Hsz] with `multi`; contiguous caches are
    [B][KH][S][Hsz], paged pools [num_blocks][KH][block_size][Hsz] with an int32 CUDA
    block_table [B][max_blocks]."""
    import torch
    _bf16_cuda("q", q)
    kv_dtype = _kv_cuda("k_cache", k_cache)
    if _kv_cuda("v_cache", v_cache) != kv_dtype:
        raise TypeError("k_cache and v_cache must have the same element type")
    if not multi:
        if q.dim() != 3:
            raise ValueError("q must be [B][Hq][Hsz]")
        B, Hq, Hsz = q.shape
    else:
        if q.dim() != 4 or q.shape[2] != q_len:
            raise ValueError("q must be [B][Hq][q_len][Hsz]")
        B, Hq, _, Hsz = q.shape
    if k_cache.dim() != 4 or v_cache.shape != k_cache.shape or k_cache.shape[3] != Hsz:
        raise ValueError("k_cache/v_cache must share one 4-d shape ending in Hsz")
    KH = k_cache.shape[1]
    if paged:
        if block_table.dtype != torch.int32 or not block_table.is_cuda or not block_table.is_contiguous():
            raise TypeError("block_table must be a contiguous int32 CUDA tensor")
        if block_table.dim() != 2 or block_table.shape[0] != B:
            raise ValueError("pools must be [num_blocks][KH][block_size][Hsz], block_table [B][max_blocks]")
    elif k_cache.shape[0] != B:
        raise ValueError("k_cache/v_cache must be [B][KH][S][Hsz]")
    out_shape = (B, Hq, q_len, Hsz) if multi else (B, Hq, Hsz)
    if out is None:
        out = torch.empty(out_shape, dtype=torch.float32, device=q.device)
    _f32_cuda("out", out, out_shape)
    sl_ptr, on_dev, sl_keep = _seqlens_arg(seqlens, B)
    a = attn_decode_args()
    a.q, a.k_cache, a.v_cache = q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr()
    a.seqlens, a.seqlens_on_device, a.out = sl_ptr, on_dev, out.data_ptr()
    a.B, a.Hq, a.KH, a.Hsz = B, Hq, KH, Hsz
    a.scale = float(scale)
    a.tile_keys, a.num_ctas = int(tile_keys), int(num_ctas)
    a.schedule, a.num_splits = int(schedule), int(num_splits)
    a.kv_dtype, a.k_scale, a.v_scale = kv_dtype, float(k_scale), float(v_scale)
    a.q_len = q_len if q_len > 1 else 0
    keep = [sl_keep, out]
    if paged:
        a.kv_stride = 0
        a.block_table = block_table.data_ptr()
        a.block_size, a.max_blocks_per_seq, a.num_blocks = k_cache.shape[2], block_table.shape[1], k_cache.shape[0]
        keep.append(block_table)
    else:
        a.kv_stride = k_cache.shape[2]
    if out_lse is not None:
        _f32_cuda("out_lse", out_lse, tuple(out_lse.shape))
        if out_lse.numel() != B * Hq * q_len:
            raise ValueError(f"out_lse must hold B*Hq*q_len = {B * Hq * q_len} entries")
        a.out_lse = out_lse.data_ptr()
        keep.append(out_lse)
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda or not workspace.is_contiguous():
            raise TypeError("workspace must be a contiguous CUDA tensor")
        a.workspace = workspace.data_ptr()
        a.workspace_bytes = workspace.numel() * workspace.element_size()
        keep.append(workspace)
    return a, keep


def attn_decode(q, k_cache, v_cache, seqlens, out=None, stream=None):
    """Decode step (``attn_decode``): q [B][Hq][Hsz], caches [B][KH][S][Hsz] bf16, S = max seqlens.

    ``seqlens`` is a host sequence of int32 lengths.  Returns ``out`` fp32 [B][Hq][Hsz].
    """
    import torch
    for n, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _bf16_cuda(n, t)
    B, Hq, Hsz = q.shape
    KH, S = k_cache.shape[1], k_cache.shape[2]
    sl = _host_seqlens(seqlens)
    if len(sl) != B:
        raise ValueError("seqlens must have B entries")
    if k_cache.shape != (B, KH, S, Hsz) or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache/v_cache must be [B][KH][S][Hsz]")
    if S != int(sl.max(initial=0)):
        raise ValueError("attn_decode packs the cache to max(seqlens); use attn_decode_ex for another capacity")
    if out is None:
        out = torch.empty((B, Hq, Hsz), dtype=torch.float32, device=q.device)
    _f32_cuda("out", out, (B, Hq, Hsz))
    _check(lib().attn_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), sl.ctypes.data, B, Hq, KH, Hsz,
                             out.data_ptr(), _stream_handle(stream)))
    return out


def attn_decode_ex(q, k_cache, v_cache, seqlens, out=None, *, scale=0.0, tile_keys=0, num_ctas=0,
                   workspace=None, ev_tiles_begin=None, ev_tiles_end=None, schedule=ATTN_SCHEDULE_AUTO,
                   num_splits=0, k_scale=0.0, v_scale=0.0, out_lse=None, stream=None):
    """Full-control decode (``attn_decode_ex``); the cache capacity is ``k_cache.shape[2]``.

    ``seqlens`` may be host values or a CUDA int32 tensor; the latter is passed as device
    seqlens (the plan is then built on the device and the call can be graph-captured).

    ``workspace`` is an optional CUDA tensor used as the partial-state buffer; its first
    ``ATTN_DECODE_COUNTER_BYTES`` bytes must be zero before its first use (allocate it with
    ``torch.zeros``), and each call leaves them zero.  ``ev_tiles_begin/end`` are optional
    raw ``hipEvent_t`` handles (ints) bound to the start of the tile kernel and the end of
    the call's last decode kernel.  ``out_lse`` (optional) is an fp32 CUDA tensor of B*Hq entries.
    """
    a, _keep = _decode_args(q, k_cache, v_cache, seqlens, out, q_len=1, multi=False, paged=False, block_table=None,
                            scale=scale, tile_keys=tile_keys, num_ctas=num_ctas, schedule=schedule,
                            num_splits=num_splits, k_scale=k_scale, v_scale=v_scale, out_lse=out_lse,
                            workspace=workspace)
    a.ev_tiles_begin = ev_tiles_begin
    a.ev_tiles_end = ev_tiles_end
    _check(lib().attn_decode_ex(ctypes.byref(a), _stream_handle(stream)))
    return _keep[1]


def attn_decode_noalloc(q, k_cache, v_cache, seqlens, out, *, scale=0.0, tile_keys=0, num_ctas=0,
                        schedule=ATTN_SCHEDULE_AUTO, num_splits=0, k_scale=0.0, v_scale=0.0, out_lse=None,
                        stream=None):
    """``attn_decode_noalloc``: ``attn_decode_ex`` with the library's fixed device scratch as
    its workspace (no device allocation in the call).  ``out`` must be given: this call
    allocates nothing, torch tensors included.  ``q`` is [B][Hq][Hsz], or
    [B][Hq][q_len][Hsz] for multi-token decode."""
    if out is None:
        raise ValueError("attn_decode_noalloc needs a preallocated out tensor")
    multi = q.dim() == 4
    a, keep = _decode_args(q, k_cache, v_cache, seqlens, out, q_len=q.shape[2] if multi else 1, multi=multi,
                           paged=False, block_table=None, scale=scale, tile_keys=tile_keys, num_ctas=num_ctas,
                           schedule=schedule, num_splits=num_splits, k_scale=k_scale, v_scale=v_scale,
                           out_lse=out_lse, workspace=None)
    if multi:
        a.q_len = q.shape[2]
    _check(lib().attn_decode_noalloc(ctypes.byref(a), _stream_handle(stream)))
    return keep[1]


def attn_merge_shards(outs, lses, out=None, lse_out=None, stream=None):
    """Merge (``attn_merge_shards``) of S decode outputs over disjoint key ranges of the same
    rows: ``outs`` fp32 [S][rows...][Hsz], ``lses`` fp32 [S][rows...] (each shard's ``out_lse``).
    Returns ``out`` fp32 [rows...][Hsz]; ``lse_out`` (optional) receives the merged lse."""
    import torch
    for n, t in (("outs", outs), ("lses", lses)):
        if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
            raise TypeError(f"{n} must be a contiguous fp32 CUDA tensor")
    S, Hsz = outs.shape[0], outs.shape[-1]
    rows = outs.numel() // (S * Hsz)
    if lses.shape[0] != S or lses.numel() != S * rows:
        raise ValueError("lses must be [S][rows] matching outs [S][rows][Hsz]")
    if out is None:
        out = torch.empty(outs.shape[1:], dtype=torch.float32, device=outs.device)
    _f32_cuda("out", out, tuple(outs.shape[1:]))
    if lse_out is not None:
        _f32_cuda("lse_out", lse_out, tuple(lse_out.shape))
        if lse_out.numel() != rows:
            raise ValueError(f"lse_out must hold {rows} entries")
    _check(lib().attn_merge_shards(outs.data_ptr(), lses.data_ptr(), S, rows, Hsz, out.data_ptr(),
                                   None if lse_out is None else lse_out.data_ptr(), _stream_handle(stream)))
    return out


class PreparedDecode:
    """``attn_decode_ex`` with its argument block marshalled once, for tight launch loops.

    The tensors are validated and their addresses packed when the object is built;
    calling it only passes the packed block and a stream handle to ``attn_decode_ex``.
    The caller keeps the tensors alive and unchanged in shape while the object is used.
    """

    def __init__(self, q, k_cache, v_cache, seqlens, out, *, scale=0.0, tile_keys=0, num_ctas=0,
                 schedule=ATTN_SCHEDULE_AUTO, num_splits=0, k_scale=0.0, v_scale=0.0, block_table=None,
                 out_lse=None, workspace=None):
        a, self._keep = _decode_args(q, k_cache, v_cache, seqlens, out, q_len=1, multi=False, paged=block_table is not None,
                                     block_table=block_table, scale=scale, tile_keys=tile_keys,
                                     num_ctas=num_ctas, schedule=schedule, num_splits=num_splits,
                                     k_scale=k_scale, v_scale=v_scale, out_lse=out_lse, workspace=workspace)
        self._args = a
        self._ref = ctypes.byref(a)
        self._fn = lib().attn_decode_ex

    def set_events(self, begin=None, end=None):
        """Raw ``hipEvent_t`` handles to record around the decode kernel (None = none)."""
        self._args.ev_tiles_begin = begin
        self._args.ev_tiles_end = end

    def __call__(self, stream_handle: int) -> None:
        st = self._fn(self._ref, stream_handle)
        if st != ATTN_OK:
            _check(st)


def attn_decode_workspace_bytes(B: int, Hq: int, KH: int, Hsz: int, num_ctas: int = 0) -> int:
    return int(lib().attn_decode_workspace_bytes(B, Hq, KH, Hsz, num_ctas))


def attn_prefill_causal(q, k, v, out=None, stream=None):
    """Causal prefill (``attn_prefill_causal``): q [B][Hq][ISL][Hsz], k/v [B][KH][ISL][Hsz] bf16 -> bf16."""
    import torch
    for n, t in (("q", q), ("k", k), ("v", v)):
        _bf16_cuda(n, t)
    B, Hq, ISL, Hsz = q.shape
    KH = k.shape[1]
    if k.shape != (B, KH, ISL, Hsz) or v.shape != k.shape:
        raise ValueError("k/v must be [B][KH][ISL][Hsz]")
    if out is None:
        out = torch.empty_like(q)
    _check(lib().attn_prefill_causal(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, ISL, Hq, KH, Hsz, out.data_ptr(),
                                     _stream_handle(stream)))
    return out


def attn_decode_plan(seqlens, KH: int, tile_keys: int, num_ctas: int):
    """Host planner (``attn_decode_plan``): returns (N, P, cta_tile_begin[P+1], seg_tile_begin[B*KH+1])."""
    import numpy as np
    sl = _host_seqlens(seqlens)
    B = len(sl)
    N = ctypes.c_int64()
    P = ctypes.c_int()
    cta = np.zeros(max(num_ctas, 0) + 1, dtype=np.int64)
    seg = np.zeros(B * KH + 1, dtype=np.int64)
    _check(lib().attn_decode_plan(sl.ctypes.data, B, KH, tile_keys, num_ctas, ctypes.byref(N), ctypes.byref(P),
                                  cta.ctypes.data, seg.ctypes.data))
    return N.value, P.value, cta[: P.value + 1], seg


def attn_hbm_copy_probe(src, dst, nbytes=None, stream=None):
    nbytes = src.numel() * src.element_size() if nbytes is None else nbytes
    _check(lib().attn_hbm_copy_probe(src.data_ptr(), dst.data_ptr(), nbytes, _stream_handle(stream)))


def attn_hbm_read_probe(src, sink, nbytes=None, stream=None):
    nbytes = src.numel() * src.element_size() if nbytes is None else nbytes
    _check(lib().attn_hbm_read_probe(src.data_ptr(), nbytes, sink.data_ptr(), _stream_handle(stream)))


def attn_device_info():
    cus, lds = ctypes.c_int(), ctypes.c_int()
    _check(lib().attn_device_info(ctypes.byref(cus), ctypes.byref(lds)))
    return cus.value, lds.value


def attn_release():
    _check(lib().attn_release())


def attn_decode_paged(q, k_pool, v_pool, block_table, seqlens, out=None, *, scale=0.0, tile_keys=0, num_ctas=0,
                      schedule=ATTN_SCHEDULE_AUTO, num_splits=0, k_scale=0.0, v_scale=0.0, stream=None):
    """Decode over a paged KV cache (``attn_decode_ex`` with a block table).

    k_pool, v_pool: [num_blocks][KH][block_size][Hsz] (bf16 or FP8 E4M3 codes);
    block_table: int32 CUDA tensor [B][max_blocks_per_seq] of block ids.  ``q`` is
    [B][Hq][Hsz], or [B][Hq][gamma][Hsz] for multi-token decode (the drafted tokens are the
    last gamma keys of each context; the output is then [B][Hq][gamma][Hsz]).
    """
    multi = q.dim() == 4
    q_len = q.shape[2] if multi else 1
    a, keep = _decode_args(q, k_pool, v_pool, seqlens, out, q_len=q_len, multi=multi, paged=True, block_table=block_table,
                           scale=scale, tile_keys=tile_keys, num_ctas=num_ctas, schedule=schedule,
                           num_splits=num_splits, k_scale=k_scale, v_scale=v_scale, out_lse=None, workspace=None)
    _check(lib().attn_decode_ex(ctypes.byref(a), _stream_handle(stream)))
    return keep[1]


def attn_decode_multi_workspace_bytes(B: int, Hq: int, KH: int, Hsz: int, q_len: int, num_ctas: int = 0) -> int:
    return int(lib().attn_decode_multi_workspace_bytes(B, Hq, KH, Hsz, q_len, num_ctas))


def attn_decode_multi(q, k_cache, v_cache, seqlens, out=None, *, scale=0.0, tile_keys=0, num_ctas=0,
                      schedule=ATTN_SCHEDULE_AUTO, num_splits=0, k_scale=0.0, v_scale=0.0, workspace=None,
                      stream=None):
    """Multi-token decode (``attn_decode_ex`` with q_len = gamma): q [B][Hq][gamma][Hsz] bf16,
    caches [B][KH][S][Hsz] holding the drafted tokens last; query t attends keys
    0 .. L_b - gamma + t.  Returns out fp32 [B][Hq][gamma][Hsz]."""
    if q.dim() != 4:
        raise ValueError("q must be [B][Hq][gamma][Hsz]")
    a, keep = _decode_args(q, k_cache, v_cache, seqlens, out, q_len=q.shape[2], multi=True, paged=False, block_table=None,
                           scale=scale, tile_keys=tile_keys, num_ctas=num_ctas, schedule=schedule,
                           num_splits=num_splits, k_scale=k_scale, v_scale=v_scale, out_lse=None,
                           workspace=workspace)
    a.q_len = q.shape[2]
    _check(lib().attn_decode_ex(ctypes.byref(a), _stream_handle(stream)))
    return keep[1]

"""Python binding of libcsa: compressed sparse attention decode on MI355X (gfx950).

Argument marshalling only.  Every step runs in the HIP kernels of ``libcsa.so``
(built from ``csrc/`` by ``build.build()``); torch supplies device memory and
the current HIP stream.  There is no fallback: if the library is not built,
``lib()`` raises.

Calls (see include/csa.h for the exact semantics of each):

* ``compress_insert`` -- compress + RMSNorm + RoPE + paged insert, rolling
  state append and window-row write; ``compress_insert_many`` runs several
  compressors (main KV and indexer keys) in one launch.
* ``index_topk`` (or ``index_score`` then ``index_select``) -- indexer scores
  and exact top-k over c4a entries.
* ``sparse_attn_decode`` -- attention with K = V over the selected entries
  plus the sliding window, inverse RoPE at the query position.
"""

from __future__ import annotations

import ctypes
import os

import torch

F32, BF16, FP8_E4M3, FP4_E2M1 = 0, 1, 2, 3
OK, EINVAL, ENOTSUP, EWORKSPACE, EHIP = 0, -1, -2, -3, -4
ABI_VERSION = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa.so")


class _CCache(ctypes.Structure):
    _fields_ = [
        ("rows", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("dim", ctypes.c_int32),
        ("rows_per_block", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("block_table", ctypes.c_void_p),
        ("bt_stride", ctypes.c_int32),
    ]


class _CJob(ctypes.Structure):
    """csa_compress_job (include/csa.h)."""
    _fields_ = [
        ("ratio", ctypes.c_int32),
        ("new_raw", ctypes.c_void_p),
        ("raw_dtype", ctypes.c_int32),
        ("cu_entries", ctypes.c_void_p),
        ("total_entries", ctypes.c_int32),
        ("gate_logits", ctypes.c_void_p),
        ("gamma", ctypes.c_void_p),
        ("eps", ctypes.c_float),
        ("rope_base", ctypes.c_float),
        ("rope_dims", ctypes.c_int32),
        ("state", ctypes.POINTER(_CCache)),
        ("out", ctypes.POINTER(_CCache)),
        ("swa", ctypes.POINTER(_CCache)),
    ]


_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_SZ = ctypes.c_size_t
_CP = ctypes.POINTER(_CCache)

_SIGNATURES = {
    "csa_abi_version": (_I, []),
    "csa_status_str": (ctypes.c_char_p, [_I]),
    "csa_num_entries": (ctypes.c_int64, [_I, ctypes.c_int64]),
    "csa_compress_insert": (_I, [_P, _I, _I, _P, _P, _I, _P, _I, _P, _I, _P, _P, _F, _F, _I,
                                 _CP, _CP, _CP]),
    "csa_compress_insert_many": (_I, [_P, _I, _P, _P, _I, _I, ctypes.POINTER(_CJob)]),
    "csa_index_workspace_size": (_SZ, [_I, _I, _I]),
    "csa_index_topk": (_I, [_P, _I, _P, _P, _I, _I, _P, _I, _I, _P, _CP, _I, _P, _P, _P, _SZ]),
    "csa_index_score": (_I, [_P, _I, _P, _P, _I, _I, _P, _I, _I, _P, _CP, _I, _P, _SZ]),
    "csa_index_select": (_I, [_P, _I, _P, _P, _I, _I, _I, _P, _P, _P, _SZ]),
    "csa_q_norm_rope_swa": (_I, [_P, _I, _P, _P, _P, _I, _I, _I, _P, _F, _F, _I, _I, _P, _P, _I,
                                 _P, _I, _CP]),
    "csa_sparse_attn_workspace_size": (_SZ, [_I, _I, _I, _I, _I, _I, _I, _I]),
    "csa_sparse_attn_decode": (_I, [_P, _I, _P, _P, _I, _I, _P, _I, _I, _CP, _I, _P, _I, _CP, _I,
                                    _F, _F, _I, _P, _P, _P, _SZ]),
    "csa_sparse_attn_decode_noalloc": (_I, [_P, _I, _P, _P, _I, _I, _P, _I, _I, _CP, _I, _P, _I, _CP,
                                            _I, _F, _F, _I, _P, _P]),
    "csa_sparse_attn_decode_fp8": (_I, [_P, _I, _P, _P, _I, _I, _P, _I, _I, _CP, _I, _P, _I, _CP,
                                        _I, _F, _F, _I, _P, _P, _P, _P, _P, _SZ]),
    "csa_compress_index_score": (_I, [_P, _I, _P, _P, _I, _I, ctypes.POINTER(_CJob), _I, _P, _P, _I,
                                      _I, _P, _I, _I, _P, _CP, _I, _P, _SZ]),
    "csa_compress_index_score_launches": (_I, [_I, ctypes.POINTER(_CJob), _I, _I, _I, _I, _I]),
    "csa_read_probe": (_I, [_P, _P, _SZ, _P]),
    "csa_read_probe_sink_words": (_I, []),
}
EXPORTED = tuple(_SIGNATURES)

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libcsa.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run compressed_sparse_long_c4a_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        if L.csa_abi_version() != ABI_VERSION:
            raise RuntimeError("libcsa ABI version mismatch")
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().csa_status_str(status).decode()


class CsaError(RuntimeError):
    def __init__(self, what: str, status: int):
        super().__init__(f"{what}: {status_str(status)} ({status})")
        self.status = status


def _check(status: int, what: str) -> None:
    if status != OK:
        raise CsaError(what, status)


def dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return F32
    if t == torch.bfloat16:
        return BF16
    if t in (torch.uint8, torch.float8_e4m3fn):
        return FP8_E4M3
    raise ValueError(f"unsupported element type {t}")


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, name: str, dtype=None, ndim=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got {t.dim()}")
    return t


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


class PagedCache:
    """A paged cache in device memory (layout of ``csa_cache`` in include/csa.h).

    rows:        [num_blocks, rows_per_block, dim] float32 | bfloat16 | uint8 (fp8 E4M3 codes),
                 or [num_blocks, rows_per_block, dim / 2] uint8 (fp4: two E2M1 codes a byte,
                 the lower element in the low nibble)
    block_table: [batch, bt_stride] int32 physical block ids
    scales:      fp8: [num_blocks, rows_per_block] float32; fp4: [num_blocks, rows_per_block,
                 dim / 16] uint8 E8M0 bytes (2^(s - 127)); None otherwise

    uint8 rows with uint8 scales form an fp4 cache, with float32 scales an fp8 cache.
    """

    def __init__(self, rows: torch.Tensor, block_table: torch.Tensor, scales: torch.Tensor | None = None):
        _dev(rows, "rows", ndim=3)
        _dev(block_table, "block_table", torch.int32, 2)
        self.dtype = dtype_code(rows.dtype)
        if self.dtype == FP8_E4M3 and scales is not None and scales.dtype == torch.uint8:
            self.dtype = FP4_E2M1
            _dev(scales, "scales", torch.uint8, 3)
            if tuple(scales.shape) != (rows.shape[0], rows.shape[1], rows.shape[2] // 8) or rows.shape[2] % 8:
                raise ValueError("fp4 scales must be [num_blocks, rows_per_block, dim / 16]")
        elif self.dtype == FP8_E4M3:
            if scales is None:
                raise ValueError("fp8 cache needs scales")
            _dev(scales, "scales", torch.float32, 2)
            if tuple(scales.shape) != tuple(rows.shape[:2]):
                raise ValueError("scales must be [num_blocks, rows_per_block]")
        self.rows, self.block_table, self.scales = rows, block_table, scales

    @property
    def dim(self) -> int:
        """Elements per row (fp4: two per byte)."""
        return self.rows.shape[2] * (2 if self.dtype == FP4_E2M1 else 1)

    @property
    def rows_per_block(self) -> int:
        return self.rows.shape[1]

    def c(self) -> _CCache:
        return _CCache(self.rows.data_ptr(), _ptr(self.scales), self.dtype, self.dim,
                       self.rows.shape[1], self.rows.shape[0], self.block_table.data_ptr(),
                       self.block_table.shape[1])


def _cref(cache: PagedCache | None):
    return None if cache is None else ctypes.pointer(cache.c())


def num_entries(ratio: int, num_tokens: int) -> int:
    """Compressed entries after num_tokens raw tokens (floor(num_tokens / ratio))."""
    return lib().csa_num_entries(ratio, num_tokens)


def compress_insert(ratio: int, ctx_lens: torch.Tensor, cu_new: torch.Tensor, new_raw: torch.Tensor,
                    cu_entries: torch.Tensor, gate_logits: torch.Tensor, state: PagedCache,
                    out: PagedCache, swa: PagedCache | None = None, gamma: torch.Tensor | None = None,
                    eps: float = 1e-6, rope_base: float = 10000.0, rope_dims: int = 64) -> None:
    """Emit the entries completed by new raw rows, append the rolling state, write window rows."""
    _dev(ctx_lens, "ctx_lens", torch.int32, 1)
    _dev(cu_new, "cu_new", torch.int32, 1)
    _dev(cu_entries, "cu_entries", torch.int32, 1)
    _dev(new_raw, "new_raw", (torch.float32, torch.bfloat16), 2)
    _dev(gate_logits, "gate_logits", torch.float32, 2)
    if gamma is not None:
        _dev(gamma, "gamma", torch.float32, 1)
    batch = ctx_lens.shape[0]
    if cu_new.shape[0] != batch + 1 or cu_entries.shape[0] != batch + 1:
        raise ValueError("cu_new and cu_entries need batch + 1 entries")
    st = lib().csa_compress_insert(
        _stream(), ratio, batch, ctx_lens.data_ptr(), cu_new.data_ptr(), new_raw.shape[0],
        _ptr(new_raw), dtype_code(new_raw.dtype), cu_entries.data_ptr(), gate_logits.shape[0],
        _ptr(gate_logits), _ptr(gamma), eps, rope_base, rope_dims, _cref(state), _cref(out), _cref(swa))
    _check(st, "csa_compress_insert")


def q_norm_rope_swa(q_pos: torch.Tensor, q: torch.Tensor, q_out: torch.Tensor | None = None,
                    gamma: torch.Tensor | None = None, eps: float = 1e-6, rope_base: float = 10000.0,
                    rope_dims: int = 64, ctx_lens: torch.Tensor | None = None,
                    cu_new: torch.Tensor | None = None, new_raw: torch.Tensor | None = None,
                    swa: PagedCache | None = None) -> torch.Tensor:
    """Query heads RMS-normalised and rotated at their positions (returned, in q's dtype); with
    a window cache, every new raw row stored there as RoPE_p(x_p).  One launch."""
    _dev(q_pos, "q_pos", torch.int32, 1)
    _dev(q, "q", (torch.float32, torch.bfloat16), 3)
    if q_out is None:
        q_out = torch.empty_like(q)
    _dev(q_out, "q_out", q.dtype, 3)
    if q_out.shape != q.shape or q.shape[0] != q_pos.shape[0]:
        raise ValueError("q_out must match q, and q_pos must have one entry per query")
    if gamma is not None:
        _dev(gamma, "gamma", torch.float32, 1)
    batch, total_new, raw_dt = 0, 0, F32
    if swa is not None:
        _dev(ctx_lens, "ctx_lens", torch.int32, 1)
        _dev(cu_new, "cu_new", torch.int32, 1)
        _dev(new_raw, "new_raw", (torch.float32, torch.bfloat16), 2)
        batch, total_new, raw_dt = ctx_lens.shape[0], new_raw.shape[0], dtype_code(new_raw.dtype)
        if cu_new.shape[0] != batch + 1:
            raise ValueError("cu_new needs batch + 1 entries")
    st = lib().csa_q_norm_rope_swa(
        _stream(), q.shape[0], _ptr(q_pos), _ptr(q), _ptr(q_out), dtype_code(q.dtype), q.shape[1],
        q.shape[2], _ptr(gamma), eps, rope_base, rope_dims, batch, _ptr(ctx_lens), _ptr(cu_new),
        total_new, _ptr(new_raw), raw_dt, _cref(swa))
    _check(st, "csa_q_norm_rope_swa")
    return q_out


class CompressJob:
    """One compressor instance of compress_insert_many (the arguments of compress_insert that
    are not shared by the call)."""

    def __init__(self, ratio: int, new_raw: torch.Tensor, cu_entries: torch.Tensor,
                 gate_logits: torch.Tensor, state: PagedCache, out: PagedCache,
                 swa: PagedCache | None = None, gamma: torch.Tensor | None = None,
                 eps: float = 1e-6, rope_base: float = 10000.0, rope_dims: int = 64):
        _dev(cu_entries, "cu_entries", torch.int32, 1)
        _dev(new_raw, "new_raw", (torch.float32, torch.bfloat16), 2)
        _dev(gate_logits, "gate_logits", torch.float32, 2)
        if gamma is not None:
            _dev(gamma, "gamma", torch.float32, 1)
        self.args = (ratio, new_raw, cu_entries, gate_logits, state, out, swa, gamma, eps, rope_base,
                     rope_dims)
        self._refs = [_cref(state), _cref(out), _cref(swa)]
        self.c = _CJob(ratio, _ptr(new_raw), dtype_code(new_raw.dtype), cu_entries.data_ptr(),
                       gate_logits.shape[0], _ptr(gate_logits), _ptr(gamma), eps, rope_base, rope_dims,
                       *self._refs)


def compress_jobs_array(jobs: list[CompressJob]):
    """A ctypes array of csa_compress_job for compress_insert_many (kept alive by the caller)."""
    arr = (_CJob * len(jobs))(*[j.c for j in jobs])
    return arr


def compress_insert_many(ctx_lens: torch.Tensor, cu_new: torch.Tensor, total_new: int,
                         jobs: list[CompressJob]) -> None:
    """Several compressors (e.g. main KV and indexer keys) over the same new tokens, one launch."""
    _dev(ctx_lens, "ctx_lens", torch.int32, 1)
    _dev(cu_new, "cu_new", torch.int32, 1)
    batch = ctx_lens.shape[0]
    if cu_new.shape[0] != batch + 1:
        raise ValueError("cu_new needs batch + 1 entries")
    for j in jobs:
        if j.args[2].shape[0] != batch + 1:
            raise ValueError("cu_entries needs batch + 1 entries")
        if j.args[1].shape[0] != total_new:
            raise ValueError("new_raw must have total_new rows")
    arr = compress_jobs_array(jobs)
    st = lib().csa_compress_insert_many(_stream(), batch, ctx_lens.data_ptr(), cu_new.data_ptr(), total_new,
                                        len(jobs), arr)
    _check(st, "csa_compress_insert_many")


def index_workspace_size(total_q: int, max_context: int, k: int) -> int:
    return lib().csa_index_workspace_size(total_q, max_context, k)


def _index_common(cu_q, q_pos, q_idx, head_w):
    _dev(cu_q, "cu_q", torch.int32, 1)
    _dev(q_pos, "q_pos", torch.int32, 1)
    _dev(q_idx, "q_idx", (torch.bfloat16, torch.float32), 3)
    _dev(head_w, "head_w", torch.float32, 2)
    total_q, heads, d = q_idx.shape
    if d != 128 or tuple(head_w.shape) != (total_q, heads) or q_pos.shape[0] != total_q:
        raise ValueError("q_idx must be [total_q, heads, 128] and head_w [total_q, heads]")
    return cu_q.shape[0] - 1, total_q, heads


def index_topk(cu_q, q_pos, q_idx, head_w, idx_cache: PagedCache, k: int, max_context: int,
               with_scores: bool = False, workspace: torch.Tensor | None = None,
               workspace_limit: int | None = None):
    """Top-k entry ids [total_q, k] int32 (ascending, -1 padded) and optionally their scores.
    workspace_limit (bytes): allocate at most this much workspace (at least one query's); the
    library then takes the queries in slices that fit."""
    batch, total_q, heads = _index_common(cu_q, q_pos, q_idx, head_w)
    dev = q_idx.device
    topk = torch.empty((total_q, k), dtype=torch.int32, device=dev)
    scores = torch.empty((total_q, k), dtype=torch.float32, device=dev) if with_scores else None
    ws_bytes = index_workspace_size(total_q, max_context, k)
    if workspace_limit is not None and total_q > 0:
        ws_bytes = min(ws_bytes, max(int(workspace_limit), index_workspace_size(1, max_context, k)))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    st = lib().csa_index_topk(_stream(), batch, cu_q.data_ptr(), q_pos.data_ptr(), total_q, max_context,
                              q_idx.data_ptr(), dtype_code(q_idx.dtype), heads, head_w.data_ptr(),
                              _cref(idx_cache), k, topk.data_ptr(), _ptr(scores), workspace.data_ptr(),
                              workspace.numel())
    _check(st, "csa_index_topk")
    return topk, scores


def index_score(cu_q, q_pos, q_idx, head_w, idx_cache: PagedCache, k: int, max_context: int,
                workspace: torch.Tensor) -> None:
    """First half of index_topk: scores and chunk bounds into ``workspace``."""
    batch, total_q, heads = _index_common(cu_q, q_pos, q_idx, head_w)
    st = lib().csa_index_score(_stream(), batch, cu_q.data_ptr(), q_pos.data_ptr(), total_q, max_context,
                               q_idx.data_ptr(), dtype_code(q_idx.dtype), heads, head_w.data_ptr(),
                               _cref(idx_cache), k, workspace.data_ptr(), workspace.numel())
    _check(st, "csa_index_score")


def compress_index_score(ctx_lens: torch.Tensor, cu_new: torch.Tensor, total_new: int,
                         jobs: list[CompressJob], idx_job: int, cu_q, q_pos, q_idx, head_w,
                         idx_cache: PagedCache, k: int, max_context: int,
                         workspace: torch.Tensor) -> None:
    """compress_insert_many followed by index_score, the compressors running in the score's
    launch (jobs[idx_job] writes idx_cache and scores the entries it inserts)."""
    _dev(ctx_lens, "ctx_lens", torch.int32, 1)
    _dev(cu_new, "cu_new", torch.int32, 1)
    batch, total_q, heads = _index_common(cu_q, q_pos, q_idx, head_w)
    if ctx_lens.shape[0] != batch or cu_new.shape[0] != batch + 1:
        raise ValueError("ctx_lens needs batch entries and cu_new batch + 1")
    for j in jobs:
        if j.args[2].shape[0] != batch + 1 or j.args[1].shape[0] != total_new:
            raise ValueError("cu_entries needs batch + 1 entries and new_raw total_new rows")
    arr = compress_jobs_array(jobs)
    st = lib().csa_compress_index_score(
        _stream(), batch, ctx_lens.data_ptr(), cu_new.data_ptr(), total_new, len(jobs), arr, idx_job,
        cu_q.data_ptr(), q_pos.data_ptr(), total_q, max_context, q_idx.data_ptr(), dtype_code(q_idx.dtype),
        heads, head_w.data_ptr(), _cref(idx_cache), k, workspace.data_ptr(), workspace.numel())
    _check(st, "csa_compress_index_score")


def compress_index_score_launches(jobs: list[CompressJob], idx_job: int, total_new: int, total_q: int,
                                  q_dtype: torch.dtype, heads: int) -> int:
    """Kernel launches compress_index_score makes for these arguments (1: the compressors run
    inside the score launch); the library decides, nothing is launched."""
    n = lib().csa_compress_index_score_launches(len(jobs), compress_jobs_array(jobs), idx_job, total_new,
                                                total_q, dtype_code(q_dtype), heads)
    _check(min(n, 0), "csa_compress_index_score_launches")
    return n


def index_select(cu_q, q_pos, k: int, max_context: int, workspace: torch.Tensor,
                 topk: torch.Tensor, scores: torch.Tensor | None = None) -> None:
    """Second half of index_topk: exact selection from the scores in ``workspace``."""
    _dev(topk, "topk", torch.int32, 2)
    st = lib().csa_index_select(_stream(), cu_q.shape[0] - 1, cu_q.data_ptr(), q_pos.data_ptr(),
                                q_pos.shape[0], max_context, k, topk.data_ptr(), _ptr(scores),
                                workspace.data_ptr(), workspace.numel())
    _check(st, "csa_index_select")


def sparse_attn_workspace_size(total_q: int, n_heads: int, dim: int, ratio: int, has_topk: bool,
                               k: int, max_context: int, window: int) -> int:
    return lib().csa_sparse_attn_workspace_size(total_q, n_heads, dim, ratio, int(has_topk), k,
                                                max_context, window)


def sparse_attn_decode(cu_q, q_pos, q, kv: PagedCache, ratio: int, topk_idx, swa: PagedCache,
                       window: int, softmax_scale: float, max_context: int, rope_base: float = 10000.0,
                       rope_dims: int = 64, with_lse: bool = False, out: torch.Tensor | None = None,
                       workspace: torch.Tensor | None = None):
    """out [total_q, H, dim] float32 (inverse-RoPE'd) and optionally lse [total_q, H]."""
    _dev(cu_q, "cu_q", torch.int32, 1)
    _dev(q_pos, "q_pos", torch.int32, 1)
    _dev(q, "q", (torch.bfloat16, torch.float32), 3)
    total_q, heads, dim = q.shape
    k = 0
    if topk_idx is not None:
        _dev(topk_idx, "topk_idx", torch.int32, 2)
        if topk_idx.shape[0] != total_q:
            raise ValueError("topk_idx must have one row per query")
        k = topk_idx.shape[1]
    if out is None:
        out = torch.empty((total_q, heads, dim), dtype=torch.float32, device=q.device)
    lse = torch.empty((total_q, heads), dtype=torch.float32, device=q.device) if with_lse else None
    ws_bytes = sparse_attn_workspace_size(total_q, heads, dim, ratio, topk_idx is not None, k,
                                          max_context, window)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    st = lib().csa_sparse_attn_decode(
        _stream(), cu_q.shape[0] - 1, cu_q.data_ptr(), q_pos.data_ptr(), total_q, max_context,
        q.data_ptr(), dtype_code(q.dtype), heads, _cref(kv), ratio, _ptr(topk_idx), k, _cref(swa),
        window, softmax_scale, rope_base, rope_dims, out.data_ptr(), _ptr(lse), workspace.data_ptr(),
        workspace.numel())
    _check(st, "csa_sparse_attn_decode")
    return out, lse


def sparse_attn_decode_fp8(cu_q, q_pos, q, kv: PagedCache, ratio: int, topk_idx, swa: PagedCache,
                           window: int, softmax_scale: float, max_context: int,
                           rope_base: float = 10000.0, rope_dims: int = 64, with_f32: bool = False,
                           with_lse: bool = False, workspace: torch.Tensor | None = None):
    """The attention output as fp8 rows: (codes [total_q, H, dim] uint8, scales [total_q, H]
    float32, the float32 rows or None, lse or None)."""
    _dev(cu_q, "cu_q", torch.int32, 1)
    _dev(q_pos, "q_pos", torch.int32, 1)
    _dev(q, "q", (torch.bfloat16, torch.float32), 3)
    total_q, heads, dim = q.shape
    k = 0
    if topk_idx is not None:
        _dev(topk_idx, "topk_idx", torch.int32, 2)
        if topk_idx.shape[0] != total_q:
            raise ValueError("topk_idx must have one row per query")
        k = topk_idx.shape[1]
    codes = torch.empty((total_q, heads, dim), dtype=torch.uint8, device=q.device)
    scales = torch.empty((total_q, heads), dtype=torch.float32, device=q.device)
    out = torch.empty((total_q, heads, dim), dtype=torch.float32, device=q.device) if with_f32 else None
    lse = torch.empty((total_q, heads), dtype=torch.float32, device=q.device) if with_lse else None
    ws_bytes = sparse_attn_workspace_size(total_q, heads, dim, ratio, topk_idx is not None, k,
                                          max_context, window)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    st = lib().csa_sparse_attn_decode_fp8(
        _stream(), cu_q.shape[0] - 1, cu_q.data_ptr(), q_pos.data_ptr(), total_q, max_context,
        q.data_ptr(), dtype_code(q.dtype), heads, _cref(kv), ratio, _ptr(topk_idx), k, _cref(swa),
        window, softmax_scale, rope_base, rope_dims, codes.data_ptr(), scales.data_ptr(), _ptr(out),
        _ptr(lse), workspace.data_ptr(), workspace.numel())
    _check(st, "csa_sparse_attn_decode_fp8")
    return codes, scales, out, lse


def read_probe(buf: torch.Tensor, sink: torch.Tensor | None = None) -> torch.Tensor:
    """One launch of the streaming-read probe over every byte of `buf` (a measurement utility:
    time it to get the achievable read bandwidth).  Returns the sink words."""
    _dev(buf, "buf")
    nbytes = buf.numel() * buf.element_size()
    if sink is None:
        sink = torch.empty(lib().csa_read_probe_sink_words(), dtype=torch.int32, device=buf.device)
    _check(lib().csa_read_probe(_stream(), buf.data_ptr(), nbytes, sink.data_ptr()), "csa_read_probe")
    return sink

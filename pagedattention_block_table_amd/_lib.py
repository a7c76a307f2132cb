"""ctypes binding of libpa.so (declared in include/pa.h).

Argument marshalling only: torch tensors are checked for device, dtype, shape and
layout, turned into device pointers, and handed to the C entry points of the same
names on torch's current HIP stream. Every step of the decode runs in the library's
kernels; there is no CPU path. If the library is missing the first call raises.
"""
from __future__ import annotations

import ctypes
import functools
import math
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
# PA_LIBRARY may name another build of the same library (e.g. a tuning variant)
LIB_PATH = os.environ.get("PA_LIBRARY") or os.path.join(_HERE, "libpa.so")

PA_F32, PA_F16, PA_BF16, PA_FP8_E4M3 = 0, 1, 2, 3
PA_OK, PA_ERR_INVALID, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_LAUNCH, PA_ERR_SCRATCH = 0, -1, -2, -3, -4, -5
PA_NOALLOC_SCRATCH_BYTES = 16 << 20
DEFAULT_PARTITION = 512

# name -> (restype, argtypes), mirroring include/pa.h
_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_SZ = ctypes.c_size_t
_DECODE_ARGS = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _I, _F, _F]
SIGNATURES = {
    "pa_decode": (_I, _DECODE_ARGS + [_P, _P]),
    "pa_partitioned_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I]),
    "pa_decode_partitioned": (_I, _DECODE_ARGS + [_I, _I, _P, _SZ, _P, _P]),
    "pa_decode_partitioned_noalloc": (_I, _DECODE_ARGS + [_I, _I, _P, _P]),
    "pa_balanced_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I]),
    "pa_decode_balanced": (_I, _DECODE_ARGS + [_I, _P, _SZ, _P, _P]),
    "pa_grouped_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I]),
    "pa_decode_grouped": (_I, _DECODE_ARGS + [_I, _P, _SZ, _P, _P]),
    "pa_debug_trace_grouped": (_I, _DECODE_ARGS + [_I, _I, _P, _SZ, _P, _P, _P, _P, _P, _P]),
    "pa_ordered_workspace_bytes": (_SZ, [_I]),
    "pa_decode_ordered": (_I, _DECODE_ARGS + [_P, _SZ, _P, _P]),
    "pa_debug_trace": (_I, _DECODE_ARGS + [_I, _I, _I, _P, _SZ, _P, _P, _P, _P, _P]),
    "pa_check_tables": (_I, [_P, _P, _I, _I, _I, _I, _I, _P, _P]),
    "pa_append_kv": (_I, [_P, _P, _P, _P, _I, _P, _I, _I, _P, _P, _I, _I, _I, _I, _I, _I, _F, _F, _P]),
    "pa_copy_blocks": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _P]),
    "pa_extend": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _I, _I, _F, _F, _P, _P]),
    "pa_debug_fp8_to_f32": (_I, [_P, _P, _I, _P]),
    "pa_debug_fp8_to_16bit": (_I, [_P, _P, _I, _I, _P]),
    "pa_debug_stream_read": (_I, [_P, _SZ, _I, _I, _I, _P, _P]),
    "pa_bm_create": (_P, [_I, _I, _I, _I]),
    "pa_bm_destroy": (None, [_P]),
    "pa_bm_num_free": (_I, [_P]),
    "pa_bm_add_sequence": (_I, [_P, _P, _I, _P]),
    "pa_bm_append_token": (_I, [_P, _I, ctypes.c_int32, _P, _P, _P]),
    "pa_bm_fork": (_I, [_P, _I]),
    "pa_bm_free_sequence": (_I, [_P, _I]),
    "pa_bm_context_len": (_I, [_P, _I]),
    "pa_bm_block_table": (_I, [_P, _I, _P, _I]),
    "pa_bm_ref_count": (_I, [_P, _I]),
    "pa_bm_export": (_I, [_P, _P, _I, _I, _P, _P]),
    "pa_status_str": (ctypes.c_char_p, [_I]),
    "pa_version": (_I, []),
}

_lib = None


class PagedAttentionError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {status}: {pa_status_str(status)}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libpa.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                               "(run `python -m pagedattention_block_table_amd.build`)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def pa_status_str(status: int) -> str:
    return lib().pa_status_str(int(status)).decode()


def pa_version() -> int:
    return int(lib().pa_version())


def pa_partitioned_workspace_bytes(num_seqs: int, num_heads: int, head_dim: int,
                                   max_context_len: int, partition_size: int = 0) -> int:
    return int(lib().pa_partitioned_workspace_bytes(num_seqs, num_heads, head_dim,
                                                    max_context_len, partition_size))


def pa_balanced_workspace_bytes(num_seqs: int, num_heads: int, num_kv_heads: int, head_dim: int,
                                num_workgroups: int = 0) -> int:
    return int(lib().pa_balanced_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_dim,
                                                 num_workgroups))


# ----------------------------------------------------------------------------------
# torch-facing wrappers
# ----------------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def dtype_code(t) -> int:
    torch = _torch()
    m = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16,
         torch.uint8: PA_FP8_E4M3}
    if hasattr(torch, "float8_e4m3fn"):
        m[torch.float8_e4m3fn] = PA_FP8_E4M3
    if t.dtype not in m:
        raise TypeError(f"unsupported tensor dtype {t.dtype}")
    return m[t.dtype]


def _check_dev(name, t):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (there is no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(stream) -> int:
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _shapes(q, k_pool, v_pool, block_tables, context_lens):
    torch = _torch()
    for n, t in (("q", q), ("k_pool", k_pool), ("v_pool", v_pool),
                 ("block_tables", block_tables), ("context_lens", context_lens)):
        _check_dev(n, t)
    if q.dim() != 3 or k_pool.dim() != 4 or v_pool.shape != k_pool.shape:
        raise ValueError("q must be [S][H][D]; k_pool and v_pool [NB][Hkv][BS][D] of equal shape")
    if k_pool.dtype != v_pool.dtype:
        raise ValueError("k_pool and v_pool must share a dtype")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    S, H, D = q.shape
    NB, Hkv, BS, D2 = k_pool.shape
    if D2 != D:
        raise ValueError("head_dim of q and pools differ")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_tables must be [S][max_blocks] and context_lens [S]")
    return S, H, D, NB, Hkv, BS, int(block_tables.shape[1])


def _common(q, k_pool, v_pool, block_tables, context_lens, scale, k_scale, v_scale, out):
    torch = _torch()
    S, H, D, NB, Hkv, BS, MB = _shapes(q, k_pool, v_pool, block_tables, context_lens)
    if out is None:
        out = torch.empty_like(q)
    _check_dev("out", out)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q in shape and dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    args = [q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), block_tables.data_ptr(),
            context_lens.data_ptr(), S, MB, NB, H, Hkv, D, BS, float(scale), dtype_code(q),
            dtype_code(k_pool), float(k_scale), float(v_scale)]
    return args, out, (S, H, D, NB, Hkv, BS, MB)


def _raise(fn, rc):
    if rc != PA_OK:
        raise PagedAttentionError(fn, rc)


def pa_decode(q, k_pool, v_pool, block_tables, context_lens, scale: Optional[float] = None,
              k_scale: float = 1.0, v_scale: float = 1.0, out=None, stream=None):
    """Single-pass paged decode; returns out [S][H][D] (q's dtype)."""
    args, out, _ = _common(q, k_pool, v_pool, block_tables, context_lens, scale, k_scale, v_scale, out)
    _raise("pa_decode", lib().pa_decode(*args, out.data_ptr(), _stream(stream)))
    return out


def pa_decode_partitioned(q, k_pool, v_pool, block_tables, context_lens, max_context_len: int,
                          scale: Optional[float] = None, partition_size: int = 0,
                          workspace=None, k_scale: float = 1.0, v_scale: float = 1.0,
                          out=None, stream=None):
    """Split-context paged decode with log-sum-exp merge; returns out."""
    torch = _torch()
    args, out, (S, H, D, *_rest) = _common(q, k_pool, v_pool, block_tables, context_lens, scale,
                                           k_scale, v_scale, out)
    need = pa_partitioned_workspace_bytes(S, H, D, int(max_context_len), int(partition_size))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check_dev("workspace", workspace)
    nbytes = workspace.numel() * workspace.element_size()
    _raise("pa_decode_partitioned",
           lib().pa_decode_partitioned(*args, int(max_context_len), int(partition_size),
                                       workspace.data_ptr(), nbytes, out.data_ptr(), _stream(stream)))
    return out


def pa_decode_partitioned_noalloc(q, k_pool, v_pool, block_tables, context_lens, max_context_len: int,
                                  scale: Optional[float] = None, partition_size: int = 0,
                                  k_scale: float = 1.0, v_scale: float = 1.0, out=None, stream=None):
    """Split-context paged decode whose partition states live in the library's static device
    scratch (no workspace; calls on one GPU must not overlap); returns out. With out given,
    the call allocates nothing."""
    args, out, _ = _common(q, k_pool, v_pool, block_tables, context_lens, scale, k_scale, v_scale, out)
    _raise("pa_decode_partitioned_noalloc",
           lib().pa_decode_partitioned_noalloc(*args, int(max_context_len), int(partition_size),
                                               out.data_ptr(), _stream(stream)))
    return out


def pa_extend(q, k_pool, v_pool, block_tables, context_lens, query_start_loc, max_query_len: int,
              scale: Optional[float] = None, k_scale: float = 1.0, v_scale: float = 1.0,
              out=None, stream=None):
    """Prefill / extend: q [T][H][D] packed by query_start_loc (int32 [S+1]); the new
    tokens are the last Q_s of each context and attend causally. Returns out [T][H][D]."""
    torch = _torch()
    for n, t in (("q", q), ("k_pool", k_pool), ("v_pool", v_pool), ("block_tables", block_tables),
                 ("context_lens", context_lens), ("query_start_loc", query_start_loc)):
        _check_dev(n, t)
    if q.dim() != 3 or k_pool.dim() != 4 or v_pool.shape != k_pool.shape or v_pool.dtype != k_pool.dtype:
        raise ValueError("q must be [T][H][D]; k_pool and v_pool [NB][Hkv][BS][D] of one shape and dtype")
    for n, t in (("block_tables", block_tables), ("context_lens", context_lens),
                 ("query_start_loc", query_start_loc)):
        if t.dtype != torch.int32:
            raise ValueError(f"{n} must be int32")
    T, H, D = q.shape
    NB, Hkv, BS, D2 = k_pool.shape
    S = context_lens.shape[0]
    if D2 != D or block_tables.dim() != 2 or block_tables.shape[0] != S or query_start_loc.shape != (S + 1,):
        raise ValueError("shapes of q, pools, block_tables, context_lens and query_start_loc disagree")
    if out is None:
        out = torch.empty_like(q)
    _check_dev("out", out)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q in shape and dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    _raise("pa_extend",
           lib().pa_extend(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), block_tables.data_ptr(),
                           context_lens.data_ptr(), query_start_loc.data_ptr(), S, block_tables.shape[1],
                           NB, int(max_query_len), H, Hkv, D, BS, float(scale), dtype_code(q),
                           dtype_code(k_pool), float(k_scale), float(v_scale), out.data_ptr(),
                           _stream(stream)))
    return out


def balanced_workspace(q, k_pool, num_workgroups: int = 0):
    """Zero-filled workspace for pa_decode_balanced (the counters must start at zero;
    every completed call leaves them zero, so one workspace serves a whole decode loop)."""
    torch = _torch()
    S, H, D = q.shape
    Hkv = k_pool.shape[1]
    need = pa_balanced_workspace_bytes(S, H, Hkv, D, num_workgroups)
    return torch.zeros(max(need, 16), dtype=torch.uint8, device=q.device)


def pa_decode_balanced(q, k_pool, v_pool, block_tables, context_lens, scale: Optional[float] = None,
                       num_workgroups: int = 0, workspace=None, k_scale: float = 1.0,
                       v_scale: float = 1.0, out=None, stream=None):
    """Work-balanced paged decode (one launch, any length mix); returns out."""
    args, out, _ = _common(q, k_pool, v_pool, block_tables, context_lens, scale, k_scale, v_scale, out)
    if workspace is None:
        workspace = balanced_workspace(q, k_pool, num_workgroups)
    _check_dev("workspace", workspace)
    nbytes = workspace.numel() * workspace.element_size()
    _raise("pa_decode_balanced",
           lib().pa_decode_balanced(*args, int(num_workgroups), workspace.data_ptr(), nbytes,
                                    out.data_ptr(), _stream(stream)))
    return out


def pa_grouped_workspace_bytes(num_seqs: int, num_heads: int, num_kv_heads: int, head_dim: int,
                               num_splits: int = 0) -> int:
    return int(lib().pa_grouped_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_dim,
                                                num_splits))


def grouped_workspace(q, k_pool, num_splits: int = 0):
    """Workspace for pa_decode_grouped (None when the call needs none)."""
    torch = _torch()
    S, H, D = q.shape
    need = pa_grouped_workspace_bytes(S, H, k_pool.shape[1], D, num_splits)
    return torch.empty(need, dtype=torch.uint8, device=q.device) if need else None


def pa_decode_grouped(q, k_pool, v_pool, block_tables, context_lens, scale: Optional[float] = None,
                      num_splits: int = 0, workspace=None, k_scale: float = 1.0,
                      v_scale: float = 1.0, out=None, stream=None):
    """Shared-prefix paged decode: blocks shared by consecutive sequences are read once per
    group and KV head (same result as pa_decode up to rounding order); returns out."""
    args, out, _ = _common(q, k_pool, v_pool, block_tables, context_lens, scale, k_scale, v_scale, out)
    if workspace is None:
        workspace = grouped_workspace(q, k_pool, num_splits)
    ptr, nbytes = None, 0
    if workspace is not None:
        _check_dev("workspace", workspace)
        ptr, nbytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    _raise("pa_decode_grouped",
           lib().pa_decode_grouped(*args, int(num_splits), ptr, nbytes, out.data_ptr(), _stream(stream)))
    return out


def pa_debug_trace_grouped(q, k_pool, v_pool, block_tables, context_lens, max_context_len: int,
                           scale: Optional[float] = None, num_splits: int = 0, k_scale: float = 1.0,
                           v_scale: float = 1.0, stream=None):
    """Instrumented grouped decode; returns (out, k_rows, v_rows, read_counts, block_reads)."""
    torch = _torch()
    args, out, (S, H, D, NB, Hkv, BS, MB) = _common(q, k_pool, v_pool, block_tables, context_lens,
                                                   scale, k_scale, v_scale, None)
    workspace = grouped_workspace(q, k_pool, num_splits)
    ptr = workspace.data_ptr() if workspace is not None else None
    nbytes = workspace.numel() if workspace is not None else 0
    k_rows = torch.zeros((S, Hkv, max_context_len, D), dtype=k_pool.dtype, device=q.device)
    v_rows = torch.zeros_like(k_rows)
    counts = torch.zeros((S, Hkv, max_context_len), dtype=torch.int32, device=q.device)
    block_reads = torch.zeros((NB, Hkv), dtype=torch.int32, device=q.device)
    _raise("pa_debug_trace_grouped",
           lib().pa_debug_trace_grouped(*args, int(max_context_len), int(num_splits), ptr, nbytes,
                                        out.data_ptr(), k_rows.data_ptr(), v_rows.data_ptr(),
                                        counts.data_ptr(), block_reads.data_ptr(), _stream(stream)))
    return out, k_rows, v_rows, counts, block_reads


def pa_ordered_workspace_bytes(num_seqs: int) -> int:
    return int(lib().pa_ordered_workspace_bytes(num_seqs))


def ordered_workspace(q):
    """Workspace for pa_decode_ordered: it needs none (the decode launch derives the order
    itself), so this is None; kept for callers that size one."""
    return None


def pa_decode_ordered(q, k_pool, v_pool, block_tables, context_lens, scale: Optional[float] = None,
                      workspace=None, k_scale: float = 1.0, v_scale: float = 1.0, out=None,
                      stream=None):
    """Longest-first paged decode (same result as pa_decode, one launch); returns out.
    workspace is accepted and ignored (the launch needs none)."""
    args, out, _ = _common(q, k_pool, v_pool, block_tables, context_lens, scale, k_scale, v_scale, out)
    _raise("pa_decode_ordered",
           lib().pa_decode_ordered(*args, None, 0, out.data_ptr(), _stream(stream)))
    return out


def pa_debug_trace(q, k_pool, v_pool, block_tables, context_lens, max_context_len: int,
                   scale: Optional[float] = None, partition_size: int = 0, num_workgroups: int = 0,
                   k_scale: float = 1.0, v_scale: float = 1.0, stream=None):
    """Instrumented decode; returns (out, k_rows, v_rows, read_counts)."""
    torch = _torch()
    args, out, (S, H, D, NB, Hkv, BS, MB) = _common(q, k_pool, v_pool, block_tables, context_lens,
                                                   scale, k_scale, v_scale, None)
    workspace = None
    nbytes = 0
    if num_workgroups:
        workspace = balanced_workspace(q, k_pool, num_workgroups)
        nbytes = workspace.numel()
    elif partition_size:
        need = pa_partitioned_workspace_bytes(S, H, D, int(max_context_len), int(partition_size))
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
        nbytes = need
    k_rows = torch.zeros((S, Hkv, max_context_len, D), dtype=k_pool.dtype, device=q.device)
    v_rows = torch.zeros_like(k_rows)
    counts = torch.zeros((S, Hkv, max_context_len), dtype=torch.int32, device=q.device)
    _raise("pa_debug_trace",
           lib().pa_debug_trace(*args, int(max_context_len), int(partition_size), int(num_workgroups),
                                workspace.data_ptr() if workspace is not None else None, nbytes,
                                out.data_ptr(), k_rows.data_ptr(), v_rows.data_ptr(),
                                counts.data_ptr(), _stream(stream)))
    return out, k_rows, v_rows, counts


class DecodePlan:
    """Arguments of one decode, checked and marshalled once, for calls repeated on the
    same buffers (a decode loop). Calling the plan enqueues the decode on its stream; the
    pools may be swapped per call for others of identical shape and dtype (another
    layer's cache). Marshalling only: the decode itself runs in the library."""

    def __init__(self, q, k_pool, v_pool, block_tables, context_lens, scale=None,
                 k_scale: float = 1.0, v_scale: float = 1.0, out=None,
                 max_context_len: Optional[int] = None, partition_size: int = 0,
                 workspace=None, stream=None, balanced: bool = False, num_workgroups: int = 0,
                 ordered: bool = False, grouped: bool = False, num_splits: int = 0):
        torch = _torch()
        args, out, (S, H, D, *_r) = _common(q, k_pool, v_pool, block_tables, context_lens,
                                            scale, k_scale, v_scale, out)
        self.out = out
        self._kmeta = (tuple(k_pool.shape), k_pool.dtype, k_pool.device)
        self._keep = [q, k_pool, v_pool, block_tables, context_lens, out]
        st = _stream(stream)
        if balanced:
            if workspace is None:
                workspace = balanced_workspace(q, k_pool, num_workgroups)
            _check_dev("workspace", workspace)
            self._keep.append(workspace)
            self._fn = lib().pa_decode_balanced
            tail = [int(num_workgroups), workspace.data_ptr(),
                    workspace.numel() * workspace.element_size(), out.data_ptr(), st]
        elif ordered:
            self._fn = lib().pa_decode_ordered
            tail = [None, 0, out.data_ptr(), st]
        elif grouped:
            if workspace is None:
                workspace = grouped_workspace(q, k_pool, num_splits)
            ptr, nbytes = None, 0
            if workspace is not None:
                _check_dev("workspace", workspace)
                self._keep.append(workspace)
                ptr, nbytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
            self._fn = lib().pa_decode_grouped
            tail = [int(num_splits), ptr, nbytes, out.data_ptr(), st]
        elif max_context_len is None:
            self._fn = lib().pa_decode
            tail = [out.data_ptr(), st]
        else:
            need = pa_partitioned_workspace_bytes(S, H, D, int(max_context_len), int(partition_size))
            if workspace is None:
                workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
            _check_dev("workspace", workspace)
            self._keep.append(workspace)
            self._fn = lib().pa_decode_partitioned
            tail = [int(max_context_len), int(partition_size), workspace.data_ptr(),
                    workspace.numel() * workspace.element_size(), out.data_ptr(), st]
        full = args + tail
        self._args = [t(v) if v is not None else None
                      for t, v in zip(self._fn.argtypes, full)]
        self._name = self._fn.__name__

    def __call__(self, k_pool=None, v_pool=None):
        a = self._args
        if k_pool is not None:
            self._check_pools(k_pool, v_pool)
            a = list(a)
            a[1] = k_pool.data_ptr()
            a[2] = v_pool.data_ptr()
        rc = self._fn(*a)
        if rc != PA_OK:
            raise PagedAttentionError(self._name, rc)
        return self.out

    def _check_pools(self, k_pool, v_pool):
        if (tuple(k_pool.shape), k_pool.dtype, k_pool.device) != self._kmeta or \
           (tuple(v_pool.shape), v_pool.dtype, v_pool.device) != self._kmeta:
            raise ValueError("replacement pools must match the planned pools")

    def bound(self, k_pool, v_pool):
        """A zero-argument callable that enqueues this decode on the given pools (another
        layer's cache of identical shape) with every argument already marshalled; it
        returns the library's status code. The pools must outlive the callable."""
        self._check_pools(k_pool, v_pool)
        a = list(self._args)
        a[1] = ctypes.c_void_p(k_pool.data_ptr())
        a[2] = ctypes.c_void_p(v_pool.data_ptr())
        return functools.partial(self._fn, *a)


def pa_append_kv(k_new, v_new, seq_ids, positions, block_tables, k_pool, v_pool,
                 k_scale: float = 1.0, v_scale: float = 1.0, stream=None):
    """Write new tokens' K/V rows ([T][Hkv][D], io dtype) into the paged pools in place."""
    torch = _torch()
    for n, t in (("k_new", k_new), ("v_new", v_new), ("seq_ids", seq_ids), ("positions", positions),
                 ("block_tables", block_tables), ("k_pool", k_pool), ("v_pool", v_pool)):
        _check_dev(n, t)
    if k_new.dim() != 3 or v_new.shape != k_new.shape or k_pool.dim() != 4 or v_pool.shape != k_pool.shape:
        raise ValueError("k_new/v_new must be [T][Hkv][D] and the pools [NB][Hkv][BS][D]")
    if seq_ids.dtype != torch.int32 or positions.dtype != torch.int32 or block_tables.dtype != torch.int32:
        raise ValueError("seq_ids, positions and block_tables must be int32")
    T, Hkv, D = k_new.shape
    NB, Hkv2, BS, D2 = k_pool.shape
    if Hkv2 != Hkv or D2 != D or seq_ids.shape != (T,) or positions.shape != (T,):
        raise ValueError("shapes of the new rows, ids and pools disagree")
    S, MB = block_tables.shape
    _raise("pa_append_kv",
           lib().pa_append_kv(k_new.data_ptr(), v_new.data_ptr(), seq_ids.data_ptr(),
                              positions.data_ptr(), T, block_tables.data_ptr(), S, MB,
                              k_pool.data_ptr(), v_pool.data_ptr(), NB, Hkv, D, BS,
                              dtype_code(k_new), dtype_code(k_pool), float(k_scale), float(v_scale),
                              _stream(stream)))
    return k_pool, v_pool


def pa_copy_blocks(k_pool, v_pool, block_pairs, stream=None):
    """Copy-on-write block copies: block_pairs is int32 [n][2] (src, dst) on the device."""
    torch = _torch()
    for n, t in (("k_pool", k_pool), ("v_pool", v_pool), ("block_pairs", block_pairs)):
        _check_dev(n, t)
    if k_pool.dim() != 4 or v_pool.shape != k_pool.shape or v_pool.dtype != k_pool.dtype:
        raise ValueError("pools must both be [NB][Hkv][BS][D] of one dtype")
    if block_pairs.dtype != torch.int32 or block_pairs.dim() != 2 or block_pairs.shape[1] != 2:
        raise ValueError("block_pairs must be int32 [n][2]")
    NB, Hkv, BS, D = k_pool.shape
    _raise("pa_copy_blocks",
           lib().pa_copy_blocks(k_pool.data_ptr(), v_pool.data_ptr(), block_pairs.data_ptr(),
                                block_pairs.shape[0], NB, Hkv, D, BS, dtype_code(k_pool), _stream(stream)))
    return k_pool, v_pool


def pa_check_tables(block_tables, context_lens, num_blocks: int, block_size: int,
                    max_context_len: int = 0, stream=None):
    """Per-sequence contract violation bits (see include/pa.h)."""
    torch = _torch()
    _check_dev("block_tables", block_tables)
    _check_dev("context_lens", context_lens)
    S, MB = block_tables.shape
    err = torch.empty(S, dtype=torch.int32, device=block_tables.device)
    _raise("pa_check_tables",
           lib().pa_check_tables(block_tables.data_ptr(), context_lens.data_ptr(), S, MB,
                                 int(num_blocks), int(block_size), int(max_context_len),
                                 err.data_ptr(), _stream(stream)))
    return err


def pa_debug_fp8_to_f32(codes, stream=None):
    torch = _torch()
    _check_dev("codes", codes)
    out = torch.empty(codes.numel(), dtype=torch.float32, device=codes.device)
    _raise("pa_debug_fp8_to_f32",
           lib().pa_debug_fp8_to_f32(codes.data_ptr(), out.data_ptr(), codes.numel(), _stream(stream)))
    return out


def pa_debug_fp8_to_16bit(codes, out_dtype, stream=None):
    """The matrix-core fp8 conversion: codes (uint8) -> out_dtype (torch.float16 or
    torch.bfloat16) on the device."""
    torch = _torch()
    _check_dev("codes", codes)
    out = torch.empty(codes.numel(), dtype=out_dtype, device=codes.device)
    _raise("pa_debug_fp8_to_16bit",
           lib().pa_debug_fp8_to_16bit(codes.data_ptr(), out.data_ptr(), codes.numel(), dtype_code(out),
                                       _stream(stream)))
    return out


class BlockManager:
    """Host block manager of the library (pa_bm_* in include/pa.h): the physical block pool
    of one paged cache, reference-counted sharing, optional prefix caching and copy on
    write. Methods raise PagedAttentionError on a failing status (PA_ERR_WORKSPACE when the
    pool has no block to give)."""

    def __init__(self, num_blocks: int, block_size: int, prefix_caching: bool = False, lru_k: int = 2):
        self._L = lib()
        self._h = self._L.pa_bm_create(int(num_blocks), int(block_size), int(bool(prefix_caching)), int(lru_k))
        if not self._h:
            raise ValueError("invalid block manager arguments")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)

    def close(self):
        if getattr(self, "_h", None):
            self._L.pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    @property
    def num_free(self) -> int:
        return int(self._L.pa_bm_num_free(self._h))

    def add_sequence(self, token_ids):
        """Returns (handle, number of prompt tokens found in the prefix cache)."""
        import numpy as np
        toks = np.ascontiguousarray(token_ids, dtype=np.int32)
        cached = ctypes.c_int(0)
        rc = self._L.pa_bm_add_sequence(self._h, toks.ctypes.data if toks.size else None, toks.size,
                                        ctypes.byref(cached))
        if rc < 0:
            raise PagedAttentionError("pa_bm_add_sequence", rc)
        return rc, cached.value

    def append_token(self, seq: int, token_id: int):
        """Returns (slot, copy_src, copy_dst); copy_* are -1 unless a shared block was copied."""
        slot, src, dst = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _raise("pa_bm_append_token", self._L.pa_bm_append_token(self._h, int(seq), int(token_id),
                                                                 ctypes.byref(slot), ctypes.byref(src),
                                                                 ctypes.byref(dst)))
        return slot.value, src.value, dst.value

    def fork(self, seq: int) -> int:
        rc = self._L.pa_bm_fork(self._h, int(seq))
        if rc < 0:
            raise PagedAttentionError("pa_bm_fork", rc)
        return rc

    def free_sequence(self, seq: int):
        _raise("pa_bm_free_sequence", self._L.pa_bm_free_sequence(self._h, int(seq)))

    def context_len(self, seq: int) -> int:
        rc = self._L.pa_bm_context_len(self._h, int(seq))
        if rc < 0:
            raise PagedAttentionError("pa_bm_context_len", rc)
        return rc

    def block_table(self, seq: int):
        n = self.context_len(seq)
        cap = max(1, (n + self.block_size - 1) // self.block_size)
        out = (ctypes.c_int32 * cap)()
        rc = self._L.pa_bm_block_table(self._h, int(seq), out, cap)
        if rc < 0:
            raise PagedAttentionError("pa_bm_block_table", rc)
        return list(out[:rc])

    def ref_count(self, block: int) -> int:
        rc = self._L.pa_bm_ref_count(self._h, int(block))
        if rc < 0:
            raise PagedAttentionError("pa_bm_ref_count", rc)
        return rc

    def export(self, seqs, max_blocks: int):
        """(block_tables int32 [n][max_blocks] padded with -1, context_lens int32 [n])."""
        import numpy as np
        ids = np.ascontiguousarray(seqs, dtype=np.int32)
        tables = np.empty((ids.size, max_blocks), dtype=np.int32)
        lens = np.empty(ids.size, dtype=np.int32)
        _raise("pa_bm_export", self._L.pa_bm_export(self._h, ids.ctypes.data, ids.size, int(max_blocks),
                                                     tables.ctypes.data, lens.ctypes.data))
        return tables, lens

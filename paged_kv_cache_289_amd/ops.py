"""Thin Python binding of libpagedattn.so (include/paged_attn.h).

Argument marshalling only: torch tensors become device pointers, shapes become
ints, and the current torch stream becomes the HIP stream.  Every step of the
computation runs in the library's HIP kernels; there is no fallback.  Importing
this module raises if the library has not been built
(``python -m paged_kv_cache_289_amd.build``).
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional

import torch

# PAGED_ATTN_LIB names another build of the same library (e.g. a host-side
# sanitizer build for the CPU tests); the in-tree build is the default.
_LIB_PATH = os.environ.get("PAGED_ATTN_LIB") or \
    os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedattn.so")

PA_OK, PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_HIP = \
    0, -1, -2, -3, -4, -5
PA_ERR_NO_BLOCKS, PA_ERR_INVALID, PA_ERR_SCRATCH = -6, -7, -8
PA_F32, PA_F16, PA_BF16, PA_FP8_E4M3 = 0, 1, 2, 3

_TORCH_DT = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16}

# symbol -> (restype, argtypes); must match include/paged_attn.h
_P, _I, _F, _Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "paged_attn_workspace_size": (_Z, [_I, _I, _I, _I, _I, _I, _I, _I, _I]),
    "paged_attn_decode": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _I,
                               _I, _I, _P, _Z, _P]),
    "paged_attn_decode_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I,
                                       _F, _I, _I, _I, _P]),
    "paged_attn_multiq": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I,
                               _I, _F, _I, _I, _I, _I, _P, _Z, _P]),
    "paged_kv_gather": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P]),
    "paged_attn_check_inputs": (_I, [_P, _P, _I, _I, _I, _I, _I, _P, _P]),
    "paged_attn_default_partition": (_I, [_I, _I, _I, _I, _I, _I]),
    "paged_attn_multiq_uses_split": (_I, [_I, _I, _I, _I, _I, _I, _I]),
    "paged_attn_set_kernel_events": (_I, [_P, _P]),
    "paged_attn_status_string": (ctypes.c_char_p, [_I]),
    "paged_attn_shared_prefix_workspace_size": (_Z, [_I, _I, _I, _I, _I, _I, _I]),
    "paged_attn_decode_shared_prefix": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I,
                                             _I, _I, _F, _I, _I, _P, _Z, _P]),
    "paged_attn_decode_fp8kv": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F,
                                     _F, _F, _I, _I, _P, _Z, _P]),
    "paged_kv_append": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _P]),
    "paged_kv_copy_blocks": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _P]),
    "paged_hbm_read": (_I, [_P, _Z, _P, _I, _I, _P]),
    "paged_pool_create": (_P, [_I, _I]),
    "paged_pool_destroy": (None, [_P]),
    "paged_pool_num_free": (_I, [_P]),
    "paged_pool_refcount": (_I, [_P, _I]),
    "paged_seq_create": (_I, [_P]),
    "paged_seq_fork": (_I, [_P, _I]),
    "paged_seq_release": (_I, [_P, _I]),
    "paged_seq_append": (_I, [_P, _I, _I, _P, _I, _P]),
    "paged_seq_length": (_I, [_P, _I]),
    "paged_seq_blocks": (_I, [_P, _I, _P, _I]),
    "paged_seq_commit": (_I, [_P, _I, _P, _I]),
    "paged_seq_match_prefix": (_I, [_P, _I, _P, _I]),
}


class PagedAttnError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} returned {status}: {msg}")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with "
                          f"`python -m paged_kv_cache_289_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(_LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


LIB = _load()
LIB_PATH = _LIB_PATH


def status_string(status: int) -> str:
    return LIB.paged_attn_status_string(status).decode()


def _check(fn: str, rc: int):
    if rc != PA_OK:
        raise PagedAttnError(fn, rc, status_string(rc))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else
                           int(stream))


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.uint8:            # 8-bit E4M3 cache codes
        return PA_FP8_E4M3
    try:
        return _TORCH_DT[t.dtype]
    except KeyError:
        raise PagedAttnError("dtype", PA_ERR_UNSUPPORTED, f"unsupported dtype {t.dtype}")


def _need_contig(**ts):
    for n, t in ts.items():
        if t is not None and not t.is_contiguous():
            raise PagedAttnError(n, PA_ERR_SHAPE, f"{n} must be contiguous")


def _same_dtype(q, k_cache, v_cache):
    """The attention entry points read K/V in the query's type (8-bit caches go through
    :func:`decode_fp8kv`); a mismatch would make the kernels mis-size every row."""
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise PagedAttnError("dtype", PA_ERR_UNSUPPORTED,
                             f"K/V caches ({k_cache.dtype}, {v_cache.dtype}) must have the "
                             f"query's dtype {q.dtype}")


def default_partition(num_seqs, num_heads, num_kv_heads, block_size, max_context_len,
                      max_q_len=1) -> int:
    return LIB.paged_attn_default_partition(num_seqs, num_heads, num_kv_heads, block_size,
                                            max_context_len, max_q_len)


def multiq_uses_split(num_seqs, max_q_len, num_heads, num_kv_heads, head_dim, dtype,
                      partition_tokens=0) -> bool:
    """Whether :func:`multiq` with these sizes takes the balanced split (else fixed
    partitions); ``dtype`` is a torch dtype or a pa_dtype code."""
    code = dtype if isinstance(dtype, int) else _TORCH_DT[dtype]
    return bool(LIB.paged_attn_multiq_uses_split(num_seqs, max_q_len, num_heads, num_kv_heads,
                                                 head_dim, code, partition_tokens))


def workspace_size(num_seqs, total_q, max_q_len, num_heads, num_kv_heads, head_dim, block_size,
                   max_context_len, partition_tokens=0) -> int:
    return int(LIB.paged_attn_workspace_size(num_seqs, total_q, max_q_len, num_heads,
                                             num_kv_heads, head_dim, block_size,
                                             max_context_len, partition_tokens))


def _alloc_stream(stream):
    """The torch stream the library will launch on, as a context for allocating the
    call's temporaries: the caching allocator then hands their memory to later
    allocations only in that stream's order, never while the kernels may still use it.
    A null context when the call runs on the current stream."""
    if stream is None:
        return contextlib.nullcontext()
    if not isinstance(stream, torch.cuda.Stream):
        stream = torch.cuda.ExternalStream(int(stream.cuda_stream) if hasattr(stream, "cuda_stream")
                                           else int(stream))
    if stream == torch.cuda.current_stream():
        return contextlib.nullcontext()
    return torch.cuda.stream(stream)


def _empty(shape, dtype, device, stream):
    with _alloc_stream(stream):
        return torch.empty(shape, dtype=dtype, device=device)


def _workspace(nbytes: int, device, workspace, stream=None):
    if nbytes == 0:
        return workspace, (workspace.numel() * workspace.element_size() if workspace is not None
                           else 0)
    if workspace is None:
        with _alloc_stream(stream):
            workspace = torch.zeros(nbytes, dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


def decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
           block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
           max_context_len: int, out: Optional[torch.Tensor] = None, out_dtype=None,
           partition_tokens: int = 0, workspace: Optional[torch.Tensor] = None,
           stream=None) -> torch.Tensor:
    """out[s, h] = paged attention of q[s, h] over sequence s's cached K/V.

    q ``[S, H, D]``; k_cache / v_cache ``[NB, Hk, B, D]``; block_tables int32
    ``[S, mbs]``; context_lens int32 ``[S]``; all on the same device."""
    _need_contig(q=q, k_cache=k_cache, v_cache=v_cache, block_tables=block_tables,
                 context_lens=context_lens, out=out)
    S, H, D = q.shape
    NB, Hk, B, D2 = k_cache.shape
    assert D2 == D and v_cache.shape == k_cache.shape and block_tables.shape[0] == S
    _same_dtype(q, k_cache, v_cache)
    assert block_tables.dtype == torch.int32 and context_lens.dtype == torch.int32
    if out is None:
        out = _empty((S, H, D), out_dtype or q.dtype, q.device, stream)
    need = workspace_size(S, S, 1, H, Hk, D, B, max_context_len, partition_tokens)
    workspace, wbytes = _workspace(need, q.device, workspace, stream)
    rc = LIB.paged_attn_decode(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                               _ptr(block_tables), _ptr(context_lens), S, H, Hk, D, B, NB,
                               block_tables.shape[1], int(max_context_len), float(scale),
                               _dtype(q), _dtype(out), int(partition_tokens), _ptr(workspace),
                               wbytes, _stream(stream))
    _check("paged_attn_decode", rc)
    return out


def decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                   max_context_len: int, out: torch.Tensor, partition_tokens: int = 0,
                   stream=None) -> torch.Tensor:
    """:func:`decode` through ``paged_attn_decode_noalloc``: no workspace, the library's
    per-GPU scratch instead; ``out`` must be given (nothing is allocated)."""
    _need_contig(q=q, k_cache=k_cache, v_cache=v_cache, block_tables=block_tables,
                 context_lens=context_lens, out=out)
    S, H, D = q.shape
    NB, Hk, B, _ = k_cache.shape
    _same_dtype(q, k_cache, v_cache)
    rc = LIB.paged_attn_decode_noalloc(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                       _ptr(block_tables), _ptr(context_lens), S, H, Hk, D, B,
                                       NB, block_tables.shape[1], int(max_context_len),
                                       float(scale), _dtype(q), _dtype(out),
                                       int(partition_tokens), _stream(stream))
    _check("paged_attn_decode_noalloc", rc)
    return out


def multiq(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
           block_tables: torch.Tensor, context_lens: torch.Tensor, q_offsets: torch.Tensor,
           scale: float, max_context_len: int, max_q_len: int, causal: bool = True,
           out: Optional[torch.Tensor] = None, out_dtype=None, partition_tokens: int = 0,
           workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Several query rows per sequence: q ``[total_q, H, D]``, rows of sequence s are
    ``q_offsets[s]:q_offsets[s+1]`` (int32 ``[S+1]`` on the device)."""
    _need_contig(q=q, k_cache=k_cache, v_cache=v_cache, block_tables=block_tables,
                 context_lens=context_lens, q_offsets=q_offsets, out=out)
    T, H, D = q.shape
    NB, Hk, B, _ = k_cache.shape
    S = context_lens.shape[0]
    assert q_offsets.shape[0] == S + 1 and q_offsets.dtype == torch.int32
    _same_dtype(q, k_cache, v_cache)
    if out is None:
        out = _empty((T, H, D), out_dtype or q.dtype, q.device, stream)
    need = workspace_size(S, T, max_q_len, H, Hk, D, B, max_context_len, partition_tokens)
    workspace, wbytes = _workspace(need, q.device, workspace, stream)
    rc = LIB.paged_attn_multiq(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                               _ptr(block_tables), _ptr(context_lens), _ptr(q_offsets), S, T,
                               int(max_q_len), H, Hk, D, B, NB, block_tables.shape[1],
                               int(max_context_len), float(scale), 1 if causal else 0, _dtype(q),
                               _dtype(out), int(partition_tokens), _ptr(workspace), wbytes,
                               _stream(stream))
    _check("paged_attn_multiq", rc)
    return out


def shared_prefix_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                 max_context_len, prefix_blocks) -> int:
    return int(LIB.paged_attn_shared_prefix_workspace_size(num_seqs, num_heads, num_kv_heads,
                                                           head_dim, block_size, max_context_len,
                                                           prefix_blocks))


def _shared_prefix_args(q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
                        prefix_blocks, out, workspace, stream):
    S, H, D = q.shape
    NB, Hk, B, _ = k_cache.shape
    _same_dtype(q, k_cache, v_cache)
    need = shared_prefix_workspace_size(S, H, Hk, D, B, max_context_len, prefix_blocks)
    workspace, wbytes = _workspace(need, q.device, workspace, stream)
    args = [_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
            _ptr(context_lens), S, H, Hk, D, B, NB, block_tables.shape[1], int(max_context_len),
            int(prefix_blocks), ctypes.c_float(scale), _dtype(q), _dtype(out), _ptr(workspace),
            ctypes.c_size_t(wbytes), _stream(stream)]
    return args, workspace


def decode_shared_prefix(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                         block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                         max_context_len: int, prefix_blocks: int,
                         out: Optional[torch.Tensor] = None, out_dtype=None,
                         workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """:func:`decode` for tables that all start with the same ``prefix_blocks`` blocks
    (and contexts that cover them): the prefix is attended once for all sequences."""
    _need_contig(q=q, k_cache=k_cache, v_cache=v_cache, block_tables=block_tables,
                 context_lens=context_lens, out=out)
    if out is None:
        out = _empty(q.shape, out_dtype or q.dtype, q.device, stream)
    args, workspace = _shared_prefix_args(q, k_cache, v_cache, block_tables, context_lens, scale,
                                          max_context_len, prefix_blocks, out, workspace, stream)
    _check("paged_attn_decode_shared_prefix", LIB.paged_attn_decode_shared_prefix(*args))
    return out


def prepare_decode_shared_prefix(q, k_cache, v_cache, block_tables, context_lens, scale,
                                 max_context_len, prefix_blocks, out, workspace=None,
                                 stream=None) -> "PreparedCall":
    """Check and marshal a :func:`decode_shared_prefix` call once."""
    _need_contig(q=q, k_cache=k_cache, v_cache=v_cache, block_tables=block_tables,
                 context_lens=context_lens, out=out)
    args, workspace = _shared_prefix_args(q, k_cache, v_cache, block_tables, context_lens, scale,
                                          max_context_len, prefix_blocks, out, workspace, stream)
    return PreparedCall("paged_attn_decode_shared_prefix", args, 2,
                        (q, k_cache, v_cache, block_tables, context_lens, out, workspace))


def _fp8kv_args(q, k_cache, v_cache, block_tables, context_lens, scale, k_scale, v_scale,
                max_context_len, out, workspace, stream, partition_tokens=0):
    assert k_cache.dtype == torch.uint8 and v_cache.dtype == torch.uint8 and q.dtype == torch.bfloat16
    S, H, D = q.shape
    NB, Hk, B, _ = k_cache.shape
    need = workspace_size(S, S, 1, H, Hk, D, B, max_context_len, partition_tokens)
    workspace, wbytes = _workspace(need, q.device, workspace, stream)
    args = [_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
            _ptr(context_lens), S, H, Hk, D, B, NB, block_tables.shape[1], int(max_context_len),
            ctypes.c_float(scale), ctypes.c_float(k_scale), ctypes.c_float(v_scale), _dtype(out),
            int(partition_tokens), _ptr(workspace), ctypes.c_size_t(wbytes), _stream(stream)]
    return args, workspace


def decode_fp8kv(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                 block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                 k_scale: float, v_scale: float, max_context_len: int,
                 out: Optional[torch.Tensor] = None, out_dtype=None, partition_tokens: int = 0,
                 workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """:func:`decode` over an 8-bit E4M3 cache (uint8 code tensors ``[NB, Hk, B, D]``)
    with per-tensor scales; ``q`` is bf16."""
    _need_contig(q=q, k_cache=k_cache, v_cache=v_cache, block_tables=block_tables,
                 context_lens=context_lens, out=out)
    if out is None:
        out = _empty(q.shape, out_dtype or q.dtype, q.device, stream)
    args, workspace = _fp8kv_args(q, k_cache, v_cache, block_tables, context_lens, scale,
                                  k_scale, v_scale, max_context_len, out, workspace, stream,
                                  partition_tokens)
    _check("paged_attn_decode_fp8kv", LIB.paged_attn_decode_fp8kv(*args))
    return out


def prepare_decode_fp8kv(q, k_cache, v_cache, block_tables, context_lens, scale, k_scale,
                         v_scale, max_context_len, out, workspace=None,
                         stream=None) -> "PreparedCall":
    """Check and marshal a :func:`decode_fp8kv` call once."""
    _need_contig(q=q, k_cache=k_cache, v_cache=v_cache, block_tables=block_tables,
                 context_lens=context_lens, out=out)
    args, workspace = _fp8kv_args(q, k_cache, v_cache, block_tables, context_lens, scale,
                                  k_scale, v_scale, max_context_len, out, workspace, stream)
    return PreparedCall("paged_attn_decode_fp8kv", args, 2,
                        (q, k_cache, v_cache, block_tables, context_lens, out, workspace))


def gather(k_cache: torch.Tensor, v_cache: torch.Tensor, block_tables: torch.Tensor,
           context_lens: torch.Tensor, token_offsets: torch.Tensor, total_tokens: int,
           stream=None):
    """Contiguous ``[total_tokens, Hk, D]`` copies of every sequence's K and V."""
    _need_contig(k_cache=k_cache, v_cache=v_cache, block_tables=block_tables,
                 context_lens=context_lens, token_offsets=token_offsets)
    NB, Hk, B, D = k_cache.shape
    S = context_lens.shape[0]
    k_out = _empty((total_tokens, Hk, D), k_cache.dtype, k_cache.device, stream)
    v_out = _empty((total_tokens, Hk, D), k_cache.dtype, k_cache.device, stream)
    rc = LIB.paged_kv_gather(_ptr(k_out), _ptr(v_out), _ptr(k_cache), _ptr(v_cache),
                             _ptr(block_tables), _ptr(context_lens), _ptr(token_offsets), S, Hk,
                             D, B, NB, block_tables.shape[1], _dtype(k_cache), _stream(stream))
    _check("paged_kv_gather", rc)
    return k_out, v_out


class PreparedCall:
    """A decode or multi-query call whose arguments were checked and marshalled once.

    ``run(k_cache, v_cache)`` re-issues it with another K/V pool of the same shape
    (one ctypes call, no Python-side checks), e.g. one layer's pool per call."""

    def __init__(self, fn_name: str, args: list, k_index: int, keep: tuple):
        self._fn = getattr(LIB, fn_name)
        self._name = fn_name
        self._args = args
        self._k = k_index
        self._keep = keep              # tensors whose pointers are baked into args

    def run(self, k_cache: Optional[torch.Tensor] = None, v_cache: Optional[torch.Tensor] = None):
        if k_cache is not None:
            self._args[self._k] = ctypes.c_void_p(k_cache.data_ptr())
            self._args[self._k + 1] = ctypes.c_void_p(v_cache.data_ptr())
        rc = self._fn(*self._args)
        if rc != PA_OK:
            _check(self._name, rc)


def prepare_decode(q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
                   out, partition_tokens=0, workspace=None, stream=None) -> PreparedCall:
    """Check and marshal a :func:`decode` call once (see :class:`PreparedCall`)."""
    _need_contig(q=q, k_cache=k_cache, v_cache=v_cache, block_tables=block_tables,
                 context_lens=context_lens, out=out)
    S, H, D = q.shape
    NB, Hk, B, _ = k_cache.shape
    _same_dtype(q, k_cache, v_cache)
    need = workspace_size(S, S, 1, H, Hk, D, B, max_context_len, partition_tokens)
    workspace, wbytes = _workspace(need, q.device, workspace, stream)
    args = [_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
            _ptr(context_lens), S, H, Hk, D, B, NB, block_tables.shape[1], int(max_context_len),
            ctypes.c_float(scale), _dtype(q), _dtype(out), int(partition_tokens),
            _ptr(workspace), ctypes.c_size_t(wbytes), _stream(stream)]
    return PreparedCall("paged_attn_decode", args, 2,
                        (q, k_cache, v_cache, block_tables, context_lens, out, workspace))


def prepare_multiq(q, k_cache, v_cache, block_tables, context_lens, q_offsets, scale,
                   max_context_len, max_q_len, out, causal=True, partition_tokens=0,
                   workspace=None, stream=None) -> PreparedCall:
    """Check and marshal a :func:`multiq` call once (see :class:`PreparedCall`)."""
    _need_contig(q=q, k_cache=k_cache, v_cache=v_cache, block_tables=block_tables,
                 context_lens=context_lens, q_offsets=q_offsets, out=out)
    T, H, D = q.shape
    NB, Hk, B, _ = k_cache.shape
    S = context_lens.shape[0]
    _same_dtype(q, k_cache, v_cache)
    need = workspace_size(S, T, max_q_len, H, Hk, D, B, max_context_len, partition_tokens)
    workspace, wbytes = _workspace(need, q.device, workspace, stream)
    args = [_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
            _ptr(context_lens), _ptr(q_offsets), S, T, int(max_q_len), H, Hk, D, B, NB,
            block_tables.shape[1], int(max_context_len), ctypes.c_float(scale),
            1 if causal else 0, _dtype(q), _dtype(out), int(partition_tokens), _ptr(workspace),
            ctypes.c_size_t(wbytes), _stream(stream)]
    return PreparedCall("paged_attn_multiq", args, 2,
                        (q, k_cache, v_cache, block_tables, context_lens, q_offsets, out,
                         workspace))


def set_kernel_events(start=None, stop=None):
    """Record torch.cuda.Event ``start``/``stop`` right around the main kernel of every
    later attention call on this thread (None, None turns it off)."""
    if start is None and stop is None:
        _check("paged_attn_set_kernel_events", LIB.paged_attn_set_kernel_events(None, None))
        return
    for e in (start, stop):
        if e.cuda_event == 0:             # torch creates the event lazily: force it
            e.record()
    rc = LIB.paged_attn_set_kernel_events(ctypes.c_void_p(start.cuda_event),
                                          ctypes.c_void_p(stop.cuda_event))
    _check("paged_attn_set_kernel_events", rc)


def check_inputs(block_tables: torch.Tensor, context_lens: torch.Tensor, block_size: int,
                 num_blocks: int, max_context_len: int, stream=None) -> torch.Tensor:
    """Device int32 scalar: count of bad context lengths and out-of-range block ids."""
    bad = _empty((1,), torch.int32, block_tables.device, stream)
    S, mbs = block_tables.shape
    rc = LIB.paged_attn_check_inputs(_ptr(block_tables), _ptr(context_lens), S, block_size,
                                     num_blocks, mbs, max_context_len, _ptr(bad), _stream(stream))
    _check("paged_attn_check_inputs", rc)
    return bad


# --------------------------------------------------------------------------
# filling and sharing the cache
# --------------------------------------------------------------------------

def append(k_cache: torch.Tensor, v_cache: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
           block_tables: torch.Tensor, context_lens: torch.Tensor, q_offsets: torch.Tensor,
           max_context_len: int, stream=None):
    """Write new tokens' K/V ``[total_new, Hk, D]`` into their pool slots (in place).
    New token i of sequence s takes position ``context_lens[s] - n_s + i``."""
    _need_contig(k_cache=k_cache, v_cache=v_cache, k_new=k_new, v_new=v_new,
                 block_tables=block_tables, context_lens=context_lens, q_offsets=q_offsets)
    NB, Hk, B, D = k_cache.shape
    T = k_new.shape[0]
    S = context_lens.shape[0]
    assert k_new.shape == (T, Hk, D) and v_new.shape == k_new.shape
    assert k_new.dtype == k_cache.dtype and q_offsets.shape[0] == S + 1
    rc = LIB.paged_kv_append(_ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new),
                             _ptr(block_tables), _ptr(context_lens), _ptr(q_offsets), S, T, Hk, D,
                             B, NB, block_tables.shape[1], int(max_context_len),
                             _dtype(k_cache), _stream(stream))
    _check("paged_kv_append", rc)


def copy_blocks(k_cache: torch.Tensor, v_cache: torch.Tensor, pairs: torch.Tensor, stream=None):
    """Block ``pairs[p, 1]`` of both pools receives block ``pairs[p, 0]`` (in place);
    ``pairs`` is int32 ``[n, 2]`` on the device."""
    _need_contig(k_cache=k_cache, v_cache=v_cache, pairs=pairs)
    NB, Hk, B, D = k_cache.shape
    assert pairs.dtype == torch.int32 and pairs.dim() == 2 and pairs.shape[1] == 2
    rc = LIB.paged_kv_copy_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(pairs), pairs.shape[0], Hk,
                                  D, B, NB, _dtype(k_cache), _stream(stream))
    _check("paged_kv_copy_blocks", rc)


class BlockPool:
    """The library's host block pool (``paged_pool_*`` / ``paged_seq_*``)."""

    def __init__(self, num_blocks: int, block_size: int):
        self._h = LIB.paged_pool_create(int(num_blocks), int(block_size))
        if not self._h:
            raise PagedAttnError("paged_pool_create", PA_ERR_SHAPE, "bad sizes or no memory")
        self.num_blocks, self.block_size = num_blocks, block_size

    def close(self):
        if self._h:
            LIB.paged_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    @staticmethod
    def _ok(fn: str, rc: int) -> int:
        if rc < 0:
            _check(fn, rc)
        return rc

    def num_free(self) -> int:
        return self._ok("paged_pool_num_free", LIB.paged_pool_num_free(self._h))

    def refcount(self, block: int) -> int:
        return self._ok("paged_pool_refcount", LIB.paged_pool_refcount(self._h, int(block)))

    def create(self) -> int:
        return self._ok("paged_seq_create", LIB.paged_seq_create(self._h))

    def fork(self, parent: int) -> int:
        return self._ok("paged_seq_fork", LIB.paged_seq_fork(self._h, int(parent)))

    def release(self, seq: int):
        self._ok("paged_seq_release", LIB.paged_seq_release(self._h, int(seq)))

    def append(self, seq: int, num_tokens: int):
        """Grow ``seq``; returns the (src, dst) block copies to run on the device first."""
        pairs = (ctypes.c_int32 * 2)()
        n = ctypes.c_int(0)
        self._ok("paged_seq_append", LIB.paged_seq_append(self._h, int(seq), int(num_tokens),
                                                          pairs, 1, ctypes.byref(n)))
        return [(pairs[0], pairs[1])] if n.value else []

    def length(self, seq: int) -> int:
        return self._ok("paged_seq_length", LIB.paged_seq_length(self._h, int(seq)))

    def blocks(self, seq: int):
        cap = -(-self.length(seq) // self.block_size)
        buf = (ctypes.c_int32 * max(cap, 1))()
        n = self._ok("paged_seq_blocks", LIB.paged_seq_blocks(self._h, int(seq), buf, cap))
        return list(buf[:n])

    def commit(self, seq: int, tokens) -> int:
        """Register the full blocks of ``seq``'s first ``len(tokens)`` tokens (K/V written)."""
        buf = (ctypes.c_int32 * max(len(tokens), 1))(*tokens)
        return self._ok("paged_seq_commit", LIB.paged_seq_commit(self._h, int(seq), buf,
                                                                 len(tokens)))

    def match_prefix(self, seq: int, tokens) -> int:
        """Give the empty ``seq`` the cached blocks of its leading tokens; returns how many
        tokens it now holds."""
        buf = (ctypes.c_int32 * max(len(tokens), 1))(*tokens)
        return self._ok("paged_seq_match_prefix",
                        LIB.paged_seq_match_prefix(self._h, int(seq), buf, len(tokens)))


def hbm_read(buf: torch.Tensor, sink: torch.Tensor, workgroups: int = 0, mode: int = 0,
             stream=None):
    """One streaming read of all of ``buf`` (a measurement aid: the device's HBM read rate).
    ``mode``: 0 grid-stride, 1 grid-stride non-temporal, 2 per-wave runs through LDS."""
    _need_contig(buf=buf)
    rc = LIB.paged_hbm_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                            int(workgroups), int(mode), _stream(stream))
    _check("paged_hbm_read", rc)


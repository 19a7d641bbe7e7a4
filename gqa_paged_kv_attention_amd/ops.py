"""ctypes binding over libgqa_paged.so (the C ABI in include/gqa_paged.h).

Argument marshalling only: shapes are read off torch tensors, device pointers
and the current HIP stream are handed to the library, and a nonzero status
raises.  Every step of the computation runs in the library's HIP kernels;
there is no fallback.  Torch provides device memory (outputs and workspaces)
and streams.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgqa_paged.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "gqa_paged.h")

GQA_F32, GQA_BF16 = 0, 1
STATUS = {0: "GQA_OK", 1: "GQA_ERR_INVALID_ARG", 2: "GQA_ERR_UNSUPPORTED", 3: "GQA_ERR_WORKSPACE",
          4: "GQA_ERR_LAUNCH", 5: "GQA_ERR_SCRATCH"}
NOALLOC_SCRATCH_BYTES = 64 << 20          # GQA_NOALLOC_SCRATCH_BYTES


class GqaError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({msg})")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("max_blocks_per_seq", ctypes.c_int32), ("q_dtype", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libgqa_paged.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m gqa_paged_kv_attention_amd.build` "
                           "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    lib.gqa_status_string.argtypes, lib.gqa_status_string.restype = [i32], ctypes.c_char_p
    lib.gqa_version.argtypes, lib.gqa_version.restype = [], i32
    lib.reshape_and_cache.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, Dims, vp]
    lib.reshape_and_cache.restype = i32
    lib.paged_gqa_decode_workspace_size.argtypes = [Dims, i32, i32]
    lib.paged_gqa_decode_workspace_size.restype = sz
    lib.paged_gqa_decode.argtypes = [vp, vp, vp, vp, vp, vp, i32, Dims, f32, i32, vp, sz, vp]
    lib.paged_gqa_decode.restype = i32
    lib.gqa_probe_mfma_bf16.argtypes = [vp, i32, i32, ctypes.POINTER(ctypes.c_longlong), vp]
    lib.gqa_probe_mfma_bf16.restype = i32
    lib.paged_gqa_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i32, Dims, f32, i32, vp]
    lib.paged_gqa_decode_noalloc.restype = i32
    lib.paged_gqa_decode_append.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, Dims, f32, i32, vp, sz, vp]
    lib.paged_gqa_decode_append.restype = i32
    lib.splitk_lse_reduce.argtypes = [vp, vp, vp, vp, vp, Dims, i32, i32, i32, vp]
    lib.splitk_lse_reduce.restype = i32
    lib.chunked_prefill_paged_decode_workspace_size.argtypes = [Dims, i32, i32, i32]
    lib.chunked_prefill_paged_decode_workspace_size.restype = sz
    lib.chunked_prefill_paged_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, Dims, f32, i32, vp, sz,
                                                 vp]
    lib.chunked_prefill_paged_decode.restype = i32
    lib.paged_cross_attention_workspace_size.argtypes = [Dims, i32, i32, i32]
    lib.paged_cross_attention_workspace_size.restype = sz
    lib.paged_cross_attention.argtypes = list(lib.chunked_prefill_paged_decode.argtypes)
    lib.paged_cross_attention.restype = i32
    lib.paged_gqa_decode_shared_prefix_workspace_size.argtypes = [Dims, i32, i32, i32, i32]
    lib.paged_gqa_decode_shared_prefix_workspace_size.restype = sz
    lib.paged_gqa_decode_shared_prefix.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, Dims, f32, i32,
                                                   vp, sz, vp]
    lib.paged_gqa_decode_shared_prefix.restype = i32
    _lib = lib
    return lib


def declared_functions(header: str = HEADER_PATH):
    """Names of the functions include/gqa_paged.h declares."""
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", text, flags=re.M)))


# --------------------------------------------------------------------------
# marshalling helpers
# --------------------------------------------------------------------------

def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return GQA_F32
    if t == torch.bfloat16:
        return GQA_BF16
    raise TypeError(f"unsupported dtype {t} (float32 or bfloat16)")


def _torch_dtype(code: int) -> torch.dtype:
    return torch.float32 if code == GQA_F32 else torch.bfloat16


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check_device(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")


def _check_int32(*ts):
    for t in ts:
        if t is not None and t.dtype != torch.int32:
            raise TypeError("block tables, lengths and index arrays must be int32")


def _shape_error(what: str, got, want):
    raise ValueError(f"{what} has shape {tuple(got)}, expected {tuple(want)}")


def _check_caches(key_cache, value_cache):
    """key_cache [num_blocks, Hkv, bs, d] (token-major pages), value_cache
    [num_blocks, Hkv, d, bs] (channel-major pages); returns (nb, Hkv, bs, d)."""
    if key_cache.dim() != 4:
        _shape_error("key_cache", key_cache.shape, ("num_blocks", "Hkv", "block_size", "head_dim"))
    nb, hkv, bs, d = key_cache.shape
    if tuple(value_cache.shape) != (nb, hkv, d, bs):
        _shape_error("value_cache", value_cache.shape, (nb, hkv, d, bs))
    if value_cache.dtype != key_cache.dtype:
        raise TypeError("key_cache and value_cache must share a dtype")
    return nb, hkv, bs, d


def _check_rows(name, t, rows, hq, d):
    if t is not None and tuple(t.shape) != (rows, hq, d):
        _shape_error(name, t.shape, (rows, hq, d))


def _check_tables(block_tables, num_seqs, seq_lens, query_start_loc=None, lens_name="seq_lens"):
    if block_tables.dim() != 2 or block_tables.shape[0] < num_seqs or block_tables.shape[1] < 1:
        _shape_error("block_tables", block_tables.shape, (f">={num_seqs}", "max_blocks_per_seq"))
    if seq_lens.dim() != 1 or seq_lens.shape[0] != num_seqs:
        _shape_error(lens_name, seq_lens.shape, (num_seqs,))
    if query_start_loc is not None and (query_start_loc.dim() != 1 or query_start_loc.shape[0] != num_seqs + 1):
        _shape_error("query_start_loc", query_start_loc.shape, (num_seqs + 1,))


def _check_query(query, hkv, d):
    if query.dim() != 3 or query.shape[2] != d or query.shape[1] % hkv != 0:
        _shape_error("query", query.shape, ("tokens", f"a multiple of {hkv}", d))


def make_dims(*, num_seqs, num_heads, key_cache, block_tables, q_dtype, out_dtype) -> Dims:
    nb, hkv, bs, d = key_cache.shape
    return Dims(num_seqs, num_heads, hkv, d, bs, nb, block_tables.shape[1], _dtype_code(q_dtype),
                _dtype_code(key_cache.dtype), _dtype_code(out_dtype))


def _call(fn: str, status: int):
    if status != 0:
        lib = load_library()
        raise GqaError(fn, status, lib.gqa_status_string(status).decode())


class BoundCall:
    """One library call with its arguments checked and marshalled once.

    Calling it re-issues the same C call (same tensors, workspace, output and
    stream) with no per-call Python work beyond the ctypes call itself, for
    loops that repeat a step on fixed buffers (the binding's checks cost about
    10 us of host time per call).  The tensors are kept alive by the object;
    `out` is the output tensor the call writes."""

    def __init__(self, name, fn, args, keep, out):
        self.name, self._fn, self._args, self._keep, self.out = name, fn, args, keep, out

    def __call__(self):
        status = self._fn(*self._args)
        if status != 0:
            _call(self.name, status)
        return self.out


def _issue(name, fn, args, bind, keep, out):
    if bind:
        return BoundCall(name, fn, args, keep, out)
    _call(name, fn(*args))
    return out


# --------------------------------------------------------------------------
# public API (same names as the C ABI)
# --------------------------------------------------------------------------

def reshape_and_cache(key, value, key_cache, value_cache, block_tables, seq_lens, query_start_loc, stream=None,
                      bind=False):
    """Write new keys/values ``[T, Hkv, d]`` into the paged caches (in place).  With ``bind`` a
    BoundCall is returned instead."""
    nb, hkv, bs, d = _check_caches(key_cache, value_cache)
    if key.dim() != 3 or tuple(key.shape[1:]) != (hkv, d):
        _shape_error("key", key.shape, ("tokens", hkv, d))
    if tuple(value.shape) != tuple(key.shape):
        _shape_error("value", value.shape, key.shape)
    _check_tables(block_tables, seq_lens.shape[0] if seq_lens.dim() == 1 else -1, seq_lens, query_start_loc)
    lib = load_library()
    _check_device(key, value, key_cache, value_cache, block_tables, seq_lens, query_start_loc)
    _check_int32(block_tables, seq_lens, query_start_loc)
    if key.dtype != key_cache.dtype or value.dtype != key_cache.dtype or value_cache.dtype != key_cache.dtype:
        raise TypeError("key/value and caches must share a dtype")
    dims = make_dims(num_seqs=seq_lens.shape[0], num_heads=key_cache.shape[1], key_cache=key_cache,
                     block_tables=block_tables, q_dtype=key.dtype, out_dtype=key.dtype)
    args = (_ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables), _ptr(seq_lens),
            _ptr(query_start_loc), key.shape[0], dims, _stream(stream))
    return _issue("reshape_and_cache", lib.reshape_and_cache, args, bind,
                  (key, value, key_cache, value_cache, block_tables, seq_lens, query_start_loc), None)


def decode_workspace_size(dims: Dims, max_seq_len: int, partition_size: int) -> int:
    return int(load_library().paged_gqa_decode_workspace_size(dims, int(max_seq_len), int(partition_size)))


def mixed_workspace_size(dims: Dims, num_tokens: int, max_seq_len: int, partition_size: int) -> int:
    return int(load_library().chunked_prefill_paged_decode_workspace_size(dims, int(num_tokens), int(max_seq_len),
                                                                          int(partition_size)))


def _workspace(nbytes: int, device, workspace):
    if nbytes == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    # a smaller workspace is passed through: the library either adapts (balanced
    # split: fewer waves) or returns GQA_ERR_WORKSPACE
    return workspace, workspace.numel() * workspace.element_size()


def paged_gqa_decode(query, key_cache, value_cache, block_tables, seq_lens, max_seq_len: int, scale: float,
                     partition_size: int = 0, out=None, out_dtype=None, workspace=None, stream=None, bind=False):
    """Decode attention: ``query [B, Hq, d]`` -> ``out [B, Hq, d]``.  With ``bind`` the
    call is not issued: a BoundCall that issues it is returned."""
    _, hkv, _, d = _check_caches(key_cache, value_cache)
    _check_query(query, hkv, d)
    B, Hq, d = query.shape
    _check_rows("out", out, B, Hq, d)
    _check_tables(block_tables, B, seq_lens)
    lib = load_library()
    _check_device(query, key_cache, value_cache, block_tables, seq_lens, out, workspace)
    _check_int32(block_tables, seq_lens)
    out_dtype = out.dtype if out is not None else (out_dtype or torch.float32)
    if out is None:
        out = torch.empty(B, Hq, d, dtype=out_dtype, device=query.device)
    dims = make_dims(num_seqs=B, num_heads=Hq, key_cache=key_cache, block_tables=block_tables, q_dtype=query.dtype,
                     out_dtype=out_dtype)
    nbytes = int(lib.paged_gqa_decode_workspace_size(dims, int(max_seq_len), int(partition_size)))
    ws, wsb = _workspace(nbytes, query.device, workspace)
    args = (_ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables), _ptr(seq_lens),
            int(max_seq_len), dims, float(scale), int(partition_size), _ptr(ws), wsb, _stream(stream))
    return _issue("paged_gqa_decode", lib.paged_gqa_decode, args, bind,
                  (query, key_cache, value_cache, block_tables, seq_lens, ws), out)


def paged_gqa_decode_noalloc(query, key_cache, value_cache, block_tables, seq_lens, max_seq_len: int, scale: float,
                             partition_size: int = 0, out=None, out_dtype=None, stream=None):
    """Decode attention as paged_gqa_decode, with the library's static per-device
    scratch in place of a workspace (the C call allocates nothing; pass ``out``
    to allocate nothing here either)."""
    _, hkv, _, d = _check_caches(key_cache, value_cache)
    _check_query(query, hkv, d)
    B, Hq, d = query.shape
    _check_rows("out", out, B, Hq, d)
    _check_tables(block_tables, B, seq_lens)
    lib = load_library()
    _check_device(query, key_cache, value_cache, block_tables, seq_lens, out)
    _check_int32(block_tables, seq_lens)
    out_dtype = out.dtype if out is not None else (out_dtype or torch.float32)
    if out is None:
        out = torch.empty(B, Hq, d, dtype=out_dtype, device=query.device)
    dims = make_dims(num_seqs=B, num_heads=Hq, key_cache=key_cache, block_tables=block_tables, q_dtype=query.dtype,
                     out_dtype=out_dtype)
    _call("paged_gqa_decode_noalloc",
          lib.paged_gqa_decode_noalloc(_ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache),
                                       _ptr(block_tables), _ptr(seq_lens), int(max_seq_len), dims, float(scale),
                                       int(partition_size), _stream(stream)))
    return out


def paged_gqa_decode_append(query, key, value, key_cache, value_cache, block_tables, seq_lens, max_seq_len: int,
                            scale: float, partition_size: int = 0, out=None, out_dtype=None, workspace=None,
                            stream=None, bind=False):
    """One decode step with the cache write fused: ``key``/``value [B, Hkv, d]`` (each sequence's new
    token, at position seq_lens[b] - 1) go into the caches, and ``query [B, Hq, d]`` -> ``out [B, Hq, d]``
    attends over all seq_lens[b] tokens.  With ``bind`` a BoundCall is returned instead."""
    _, hkv, _, d = _check_caches(key_cache, value_cache)
    _check_query(query, hkv, d)
    B, Hq, d = query.shape
    _check_rows("out", out, B, Hq, d)
    _check_rows("key", key, B, hkv, d)
    _check_rows("value", value, B, hkv, d)
    _check_tables(block_tables, B, seq_lens)
    lib = load_library()
    _check_device(query, key, value, key_cache, value_cache, block_tables, seq_lens, out, workspace)
    _check_int32(block_tables, seq_lens)
    out_dtype = out.dtype if out is not None else (out_dtype or torch.float32)
    if out is None:
        out = torch.empty(B, Hq, d, dtype=out_dtype, device=query.device)
    dims = make_dims(num_seqs=B, num_heads=Hq, key_cache=key_cache, block_tables=block_tables, q_dtype=query.dtype,
                     out_dtype=out_dtype)
    nbytes = int(lib.paged_gqa_decode_workspace_size(dims, int(max_seq_len), int(partition_size)))
    ws, wsb = _workspace(nbytes, query.device, workspace)
    args = (_ptr(out), _ptr(query), _ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache),
            _ptr(block_tables), _ptr(seq_lens), int(max_seq_len), dims, float(scale), int(partition_size), _ptr(ws),
            wsb, _stream(stream))
    return _issue("paged_gqa_decode_append", lib.paged_gqa_decode_append, args, bind,
                  (query, key, value, key_cache, value_cache, block_tables, seq_lens, ws), out)


def splitk_lse_reduce(partial_out, partial_lse, seq_lens, partition_size: int, *, num_kv_heads: int,
                      block_size: int = 16, max_blocks_per_seq: int, query_start_loc=None, out=None,
                      out_dtype=None, skip_single: bool = False, num_out_rows: Optional[int] = None, stream=None):
    """Merge split-K partials ``[B, Hq, P, d]`` / ``[B, Hq, P]`` into ``out``."""
    if partial_out.dim() != 4:
        _shape_error("partial_out", partial_out.shape, ("num_seqs", "Hq", "partitions", "head_dim"))
    B, Hq, P, d = partial_out.shape
    if tuple(partial_lse.shape) != (B, Hq, P):
        _shape_error("partial_lse", partial_lse.shape, (B, Hq, P))
    if seq_lens.dim() != 1 or seq_lens.shape[0] != B:
        _shape_error("seq_lens", seq_lens.shape, (B,))
    if query_start_loc is not None and (query_start_loc.dim() != 1 or query_start_loc.shape[0] != B + 1):
        _shape_error("query_start_loc", query_start_loc.shape, (B + 1,))
    if Hq % num_kv_heads != 0:
        raise ValueError(f"num_kv_heads {num_kv_heads} does not divide {Hq} heads")
    if out is not None:
        rows = query_start_loc is not None
        if out.dim() != 3 or tuple(out.shape[1:]) != (Hq, d) or (not rows and out.shape[0] != B):
            _shape_error("out", out.shape, ("rows" if rows else B, Hq, d))
    lib = load_library()
    _check_device(partial_out, partial_lse, seq_lens, query_start_loc, out)
    _check_int32(seq_lens, query_start_loc)
    if partial_out.dtype != torch.float32 or partial_lse.dtype != torch.float32:
        raise TypeError("partials are float32")
    out_dtype = out.dtype if out is not None else (out_dtype or torch.float32)
    if out is None:
        rows = num_out_rows if num_out_rows is not None else B
        out = torch.zeros(rows, Hq, d, dtype=out_dtype, device=partial_out.device)
    dims = Dims(B, Hq, num_kv_heads, d, block_size, 1, max_blocks_per_seq, _dtype_code(out_dtype),
                _dtype_code(out_dtype), _dtype_code(out_dtype))
    _call("splitk_lse_reduce", lib.splitk_lse_reduce(_ptr(out), _ptr(partial_out), _ptr(partial_lse), _ptr(seq_lens),
                                                     _ptr(query_start_loc), dims, P, int(partition_size),
                                                     int(bool(skip_single)), _stream(stream)))
    return out


def chunked_prefill_paged_decode(query, key_cache, value_cache, block_tables, seq_lens, query_start_loc,
                                 max_query_len: int, max_seq_len: int, scale: float, partition_size: int = 0,
                                 out=None, out_dtype=None, workspace=None, stream=None, bind=False):
    """Mixed prefill-chunk + decode attention: ``query [T, Hq, d]`` -> ``out [T, Hq, d]``.  With
    ``bind`` a BoundCall is returned instead."""
    _, hkv, _, d = _check_caches(key_cache, value_cache)
    _check_query(query, hkv, d)
    T, Hq, d = query.shape
    _check_rows("out", out, T, Hq, d)
    _check_tables(block_tables, seq_lens.shape[0] if seq_lens.dim() == 1 else -1, seq_lens, query_start_loc)
    lib = load_library()
    _check_device(query, key_cache, value_cache, block_tables, seq_lens, query_start_loc, out, workspace)
    _check_int32(block_tables, seq_lens, query_start_loc)
    out_dtype = out.dtype if out is not None else (out_dtype or torch.float32)
    if out is None:
        out = torch.empty(T, Hq, d, dtype=out_dtype, device=query.device)
    dims = make_dims(num_seqs=seq_lens.shape[0], num_heads=Hq, key_cache=key_cache, block_tables=block_tables,
                     q_dtype=query.dtype, out_dtype=out_dtype)
    nbytes = int(lib.chunked_prefill_paged_decode_workspace_size(dims, T, int(max_seq_len), int(partition_size)))
    ws, wsb = _workspace(nbytes, query.device, workspace)
    args = (_ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables), _ptr(seq_lens),
            _ptr(query_start_loc), T, int(max_query_len), int(max_seq_len), dims, float(scale), int(partition_size),
            _ptr(ws), wsb, _stream(stream))
    return _issue("chunked_prefill_paged_decode", lib.chunked_prefill_paged_decode, args, bind,
                  (query, key_cache, value_cache, block_tables, seq_lens, query_start_loc, ws), out)


def cross_workspace_size(dims: Dims, num_tokens: int, max_encoder_len: int, partition_size: int) -> int:
    return int(load_library().paged_cross_attention_workspace_size(dims, int(num_tokens), int(max_encoder_len),
                                                                    int(partition_size)))


def paged_cross_attention(query, key_cache, value_cache, block_tables, encoder_lens, query_start_loc,
                          max_query_len: int, max_encoder_len: int, scale: float, partition_size: int = 0,
                          out=None, out_dtype=None, workspace=None, stream=None):
    """Cross-attention of decoder rows ``query [T, Hq, d]`` over a static encoder cache -> ``out [T, Hq, d]``."""
    _, hkv, _, d = _check_caches(key_cache, value_cache)
    _check_query(query, hkv, d)
    T, Hq, d = query.shape
    _check_rows("out", out, T, Hq, d)
    _check_tables(block_tables, encoder_lens.shape[0] if encoder_lens.dim() == 1 else -1, encoder_lens,
                  query_start_loc, lens_name="encoder_lens")
    lib = load_library()
    _check_device(query, key_cache, value_cache, block_tables, encoder_lens, query_start_loc, out, workspace)
    _check_int32(block_tables, encoder_lens, query_start_loc)
    out_dtype = out.dtype if out is not None else (out_dtype or torch.float32)
    if out is None:
        out = torch.empty(T, Hq, d, dtype=out_dtype, device=query.device)
    dims = make_dims(num_seqs=encoder_lens.shape[0], num_heads=Hq, key_cache=key_cache, block_tables=block_tables,
                     q_dtype=query.dtype, out_dtype=out_dtype)
    nbytes = int(lib.paged_cross_attention_workspace_size(dims, T, int(max_encoder_len), int(partition_size)))
    ws, wsb = _workspace(nbytes, query.device, workspace)
    _call("paged_cross_attention",
          lib.paged_cross_attention(_ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
                                    _ptr(encoder_lens), _ptr(query_start_loc), T, int(max_query_len),
                                    int(max_encoder_len), dims, float(scale), int(partition_size), _ptr(ws), wsb,
                                    _stream(stream)))
    return out


def shared_prefix_workspace_size(dims: Dims, num_groups: int, max_group_size: int, max_seq_len: int,
                                 partition_size: int) -> int:
    return int(load_library().paged_gqa_decode_shared_prefix_workspace_size(
        dims, int(num_groups), int(max_group_size), int(max_seq_len), int(partition_size)))


def paged_gqa_decode_shared_prefix(query, key_cache, value_cache, block_tables, seq_lens, group_start, prefix_lens,
                                   max_group_size: int, max_seq_len: int, scale: float, partition_size: int = 0,
                                   out=None, out_dtype=None, workspace=None, stream=None):
    """Decode ``query [B, Hq, d]`` -> ``out [B, Hq, d]`` where the sequences of group g
    (``group_start[g] .. group_start[g+1]-1``) share their first ``prefix_lens[g]`` tokens."""
    _, hkv, _, d = _check_caches(key_cache, value_cache)
    _check_query(query, hkv, d)
    B, Hq, d = query.shape
    _check_rows("out", out, B, Hq, d)
    _check_tables(block_tables, B, seq_lens)
    if prefix_lens.dim() != 1 or group_start.dim() != 1 or group_start.shape[0] != prefix_lens.shape[0] + 1:
        _shape_error("group_start", group_start.shape, (prefix_lens.shape[0] + 1,))
    lib = load_library()
    _check_device(query, key_cache, value_cache, block_tables, seq_lens, group_start, prefix_lens, out, workspace)
    _check_int32(block_tables, seq_lens, group_start, prefix_lens)
    out_dtype = out.dtype if out is not None else (out_dtype or torch.float32)
    if out is None:
        out = torch.empty(B, Hq, d, dtype=out_dtype, device=query.device)
    dims = make_dims(num_seqs=B, num_heads=Hq, key_cache=key_cache, block_tables=block_tables, q_dtype=query.dtype,
                     out_dtype=out_dtype)
    num_groups = int(prefix_lens.shape[0])
    nbytes = int(lib.paged_gqa_decode_shared_prefix_workspace_size(dims, num_groups, int(max_group_size),
                                                                   int(max_seq_len), int(partition_size)))
    ws, wsb = _workspace(nbytes, query.device, workspace)
    _call("paged_gqa_decode_shared_prefix",
          lib.paged_gqa_decode_shared_prefix(_ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache),
                                             _ptr(block_tables), _ptr(seq_lens), _ptr(group_start),
                                             _ptr(prefix_lens), num_groups, int(max_group_size), int(max_seq_len),
                                             dims, float(scale), int(partition_size), _ptr(ws), wsb,
                                             _stream(stream)))
    return out


def probe_mfma_bf16(out: torch.Tensor, groups: int, iters: int, stream=None) -> int:
    """Enqueue the library's bf16 matrix-core rate probe (a measurement aid, not
    part of the attention path); returns the launch's flops."""
    lib = load_library()
    _check_device(out)
    if out.dtype != torch.float32 or out.numel() < 4 * groups:
        raise ValueError("out must be float32 with at least 4 * groups elements")
    flops = ctypes.c_longlong(0)
    _call("gqa_probe_mfma_bf16", lib.gqa_probe_mfma_bf16(_ptr(out), int(groups), int(iters), ctypes.byref(flops),
                                                         _stream(stream)))
    return int(flops.value)


def to_device(arr, device="cuda") -> torch.Tensor:
    """Host storage array -> device tensor (uint16 bit patterns become bfloat16)."""
    import numpy as np
    arr = np.ascontiguousarray(arr)
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(arr).to(device)


def to_host_storage(t: torch.Tensor):
    """Device tensor -> host storage array (bfloat16 becomes uint16 bit patterns)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()

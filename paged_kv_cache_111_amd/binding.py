"""Thin Python binding of libpa.so: argument marshalling only.

Each function takes torch tensors (device memory) and host integers, checks that the tensors have the layout the
C ABI expects, and passes raw pointers, sizes and the current HIP stream to the library. Every step of the
computation runs in the library's HIP kernels; nothing here computes on the host, and there is no fallback when
the library is missing: loading it raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")

PA_OK, PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_LAUNCH = range(6)
PA_F32, PA_BF16 = 0, 1

_c_i32 = ctypes.c_int32
_c_i64 = ctypes.c_int64
_c_ptr = ctypes.c_void_p
_c_size = ctypes.c_size_t
_c_f32 = ctypes.c_float

# name -> (restype, argtypes), in the order of include/pa.h
SIGNATURES = {
    "pa_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "pa_version": (ctypes.c_int, []),
    "pa_build_metadata": (ctypes.c_int, [_c_ptr, _c_ptr, _c_ptr, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_ptr,
                                         _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr]),
    "pa_store_kvcache": (ctypes.c_int, [_c_ptr, _c_i64, _c_ptr, _c_i64, _c_ptr, _c_ptr, _c_ptr, _c_i32, _c_i32,
                                        _c_i32, _c_i32, _c_i32, ctypes.c_int, _c_ptr]),
    "pa_build_metadata_store": (ctypes.c_int, [_c_ptr, _c_ptr, _c_ptr, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                               _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_i64, _c_ptr,
                                               _c_i64, _c_ptr, _c_ptr, _c_i32, _c_i32, ctypes.c_int, _c_ptr]),
    "pa_check_indices": (ctypes.c_int, [_c_ptr, _c_i32, _c_ptr, _c_i32, _c_i32, _c_ptr, _c_ptr, _c_ptr, _c_i32,
                                        _c_i32, _c_ptr, _c_ptr]),
    "pa_norm_rope_store_kvcache": (ctypes.c_int, [_c_ptr, _c_i64, _c_ptr, _c_i64, _c_ptr, _c_ptr, _c_i64, _c_ptr,
                                                  _c_ptr, _c_i32, _c_f32, _c_ptr, _c_ptr, _c_i32, _c_ptr, _c_ptr,
                                                  _c_ptr, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, ctypes.c_int,
                                                  _c_ptr]),
    "pa_sample": (ctypes.c_int, [_c_ptr, _c_i64, _c_ptr, _c_i32, _c_i32, ctypes.c_uint64, ctypes.c_uint64, _c_ptr,
                                 _c_ptr, _c_size, _c_ptr]),
    "pa_sample_workspace_bytes": (_c_size, [_c_i32, _c_i32]),
    "pa_prefill_varlen": (ctypes.c_int, [_c_ptr, _c_i64, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_i32, _c_i32,
                                         _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_f32,
                                         ctypes.c_int, _c_ptr, ctypes.c_int, _c_ptr, _c_size, _c_ptr]),
    "pa_prefill_workspace_bytes": (_c_size, [_c_i32, _c_i32, _c_i32, _c_i32, _c_i32]),
    "pa_decode": (ctypes.c_int, [_c_ptr, _c_i64, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_i32, _c_i32, _c_i32, _c_i32,
                                 _c_i32, _c_i32, _c_i32, _c_f32, ctypes.c_int, _c_ptr, ctypes.c_int, _c_i32, _c_ptr,
                                 _c_size, _c_ptr]),
    "pa_decode_append": (ctypes.c_int, [_c_ptr, _c_i64, _c_ptr, _c_i64, _c_ptr, _c_i64, _c_ptr, _c_ptr, _c_ptr,
                                        _c_ptr, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_f32,
                                        ctypes.c_int, _c_ptr, ctypes.c_int, _c_ptr, _c_size, _c_ptr]),
    "pa_decode_append_noalloc": (ctypes.c_int, [_c_ptr, _c_i64, _c_ptr, _c_i64, _c_ptr, _c_i64, _c_ptr, _c_ptr,
                                                _c_ptr, _c_ptr, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                                _c_i32, _c_f32, ctypes.c_int, _c_ptr, ctypes.c_int, _c_ptr]),
    "pa_decode_split_tokens": (_c_i32, [_c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32]),
    "pa_decode_workspace_bytes": (_c_size, [_c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32]),
}

_lib = None


class PAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status_str(status)}")


# pa_check_kind, in order
CHECK_KINDS = ("slot", "table", "len", "cu", "q_gt_k")


class PAIndexError(ValueError):
    """Index arrays that the path would follow out of bounds (raised in checked mode, before the launch)."""

    def __init__(self, fn: str, report: dict):
        self.report = report
        detail = ", ".join(f"{k}: {v['count']} (first at {v['first']})" for k, v in report.items())
        super().__init__(f"{fn}: invalid indices: {detail}")


def checked_mode() -> bool:
    """True when PA_CHECKED is set (and not 0): every call then validates its index arrays with
    pa_check_indices first, synchronising, and raises PAIndexError instead of launching on bad ones."""
    return os.environ.get("PA_CHECKED", "0") not in ("", "0")


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m paged_kv_cache_111_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_str(status: int) -> str:
    return lib().pa_status_str(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != PA_OK:
        raise PAError(fn, status)


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return PA_BF16
    if t == torch.float32:
        return PA_F32
    raise TypeError(f"unsupported dtype {t}")


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _require(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _cache_dims(k_cache: torch.Tensor, v_cache: torch.Tensor):
    _require(k_cache.dim() == 4 and k_cache.shape == v_cache.shape, "caches must be [num_blocks, bs, Hkv, D]")
    _require(k_cache.is_contiguous() and v_cache.is_contiguous(), "caches must be contiguous")
    _require(k_cache.dtype == v_cache.dtype, "K and V caches must share a dtype")
    return tuple(int(x) for x in k_cache.shape)


def _token_rows(x: torch.Tensor, heads: int, dim: int, what: str) -> int:
    """Token stride of a [T, heads, dim] tensor whose per-token heads*dim elements are contiguous."""
    _require(x.dim() == 3 and x.shape[1] == heads and x.shape[2] == dim, f"{what} must be [T, {heads}, {dim}]")
    _require(x.stride(2) == 1 and x.stride(1) == dim, f"{what}: each token's heads*dim elements must be contiguous")
    return int(x.stride(0))


def _i32(x: torch.Tensor, what: str) -> None:
    _require(x.dtype == torch.int32 and x.is_contiguous(), f"{what} must be a contiguous int32 tensor")


# ------------------------------------------------------------------------------------------------------ API


def build_metadata(num_cached, num_new, block_table, total_q: int, num_blocks: int, block_size: int,
                   stream=None) -> dict:
    """pa_build_metadata. Returns device int32 tensors cu_seqlens_q/k, context_lens, positions, slot_mapping."""
    for t, n in ((num_cached, "num_cached"), (num_new, "num_new"), (block_table, "block_table")):
        _i32(t, n)
    B = int(num_new.shape[0])
    dev = num_new.device
    out = {
        "cu_seqlens_q": torch.empty(B + 1, dtype=torch.int32, device=dev),
        "cu_seqlens_k": torch.empty(B + 1, dtype=torch.int32, device=dev),
        "context_lens": torch.empty(B, dtype=torch.int32, device=dev),
        "positions": torch.empty(max(total_q, 1), dtype=torch.int32, device=dev)[:total_q],
        "slot_mapping": torch.empty(max(total_q, 1), dtype=torch.int32, device=dev)[:total_q],
    }
    st = lib().pa_build_metadata(_ptr(num_cached), _ptr(num_new), _ptr(block_table), int(block_table.shape[1]), B,
                                 int(total_q), int(num_blocks), int(block_size), _ptr(out["cu_seqlens_q"]),
                                 _ptr(out["cu_seqlens_k"]), _ptr(out["context_lens"]), _ptr(out["positions"]),
                                 _ptr(out["slot_mapping"]), _stream(stream))
    _check("pa_build_metadata", st)
    if checked_mode() and B > 0:
        _validate("pa_build_metadata", num_blocks=num_blocks, block_size=block_size,
                  slot_mapping=out["slot_mapping"], block_table=block_table, context_lens=out["context_lens"],
                  stream=stream)
    return out


def check_indices(num_blocks: int, block_size: int, slot_mapping=None, num_tokens=None, block_table=None,
                  context_lens=None, cu_seqlens_q=None, cu_seqlens_k=None, stream=None) -> dict:
    """pa_check_indices on the given arrays (None skips their checks). Synchronises and returns
    {kind: {"count": n, "first": smallest offending index or None}} for the kinds in CHECK_KINDS."""
    for t, n in ((slot_mapping, "slot_mapping"), (block_table, "block_table"), (context_lens, "context_lens"),
                 (cu_seqlens_q, "cu_seqlens_q"), (cu_seqlens_k, "cu_seqlens_k")):
        if t is not None:
            _i32(t, n)
    if num_tokens is None:
        num_tokens = int(slot_mapping.shape[0]) if slot_mapping is not None else 0
    if block_table is not None:
        batch, mbps = int(block_table.shape[0]), int(block_table.shape[1])
    else:
        batch = int(cu_seqlens_q.shape[0]) - 1 if cu_seqlens_q is not None else 0
        mbps = 0
    dev = next(t.device for t in (slot_mapping, block_table, context_lens, cu_seqlens_q, cu_seqlens_k)
               if t is not None)
    report = torch.empty(2 * len(CHECK_KINDS), dtype=torch.int32, device=dev)
    st = lib().pa_check_indices(_ptr(slot_mapping), int(num_tokens), _ptr(block_table), batch, mbps,
                                _ptr(context_lens), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), int(num_blocks),
                                int(block_size), _ptr(report), _stream(stream))
    _check("pa_check_indices", st)
    torch.cuda.synchronize(dev)
    r = report.cpu().numpy().view("uint32")
    n = len(CHECK_KINDS)
    return {k: {"count": int(r[i]), "first": None if r[n + i] == 0xFFFFFFFF else int(r[n + i])}
            for i, k in enumerate(CHECK_KINDS)}


def _validate(fn: str, **kw) -> None:
    bad = {k: v for k, v in check_indices(**kw).items() if v["count"]}
    if bad:
        raise PAIndexError(fn, bad)


def store_kvcache(k, v, k_cache, v_cache, slot_mapping, stream=None) -> None:
    """pa_store_kvcache: k/v [T, Hkv, D] (token stride free), caches [num_blocks, bs, Hkv, D]."""
    nb, bs, hkv, d = _cache_dims(k_cache, v_cache)
    _require(k.dtype == k_cache.dtype and v.dtype == k_cache.dtype, "k/v must match the cache dtype")
    ks = _token_rows(k, hkv, d, "k")
    vs = _token_rows(v, hkv, d, "v")
    _i32(slot_mapping, "slot_mapping")
    T = int(k.shape[0])
    _require(v.shape[0] == T and slot_mapping.shape[0] == T, "k, v and slot_mapping must have one row per token")
    if checked_mode() and T > 0:
        _validate("pa_store_kvcache", num_blocks=nb, block_size=bs, slot_mapping=slot_mapping, stream=stream)
    st = lib().pa_store_kvcache(_ptr(k), ks, _ptr(v), vs, _ptr(k_cache), _ptr(v_cache), _ptr(slot_mapping), T, hkv,
                                d, nb, bs, _dtype_code(k_cache.dtype), _stream(stream))
    _check("pa_store_kvcache", st)


def build_metadata_store(num_cached, num_new, block_table, total_q: int, k, v, k_cache, v_cache,
                         stream=None) -> dict:
    """pa_build_metadata_store: build_metadata's outputs (returned as a dict), and k/v [total_q, Hkv, D] stored at
    the slots it computes."""
    for t, n in ((num_cached, "num_cached"), (num_new, "num_new"), (block_table, "block_table")):
        _i32(t, n)
    nb, bs, hkv, d = _cache_dims(k_cache, v_cache)
    _require(k.dtype == k_cache.dtype and v.dtype == k_cache.dtype, "k/v must match the cache dtype")
    ks = _token_rows(k, hkv, d, "k")
    vs = _token_rows(v, hkv, d, "v")
    _require(k.shape[0] == total_q and v.shape[0] == total_q, "k and v must have one row per new token")
    if checked_mode():
        meta = build_metadata(num_cached, num_new, block_table, total_q, nb, bs, stream=stream)
        store_kvcache(k, v, k_cache, v_cache, meta["slot_mapping"], stream=stream)
        return meta
    B = int(num_new.shape[0])
    dev = num_new.device
    out = {
        "cu_seqlens_q": torch.empty(B + 1, dtype=torch.int32, device=dev),
        "cu_seqlens_k": torch.empty(B + 1, dtype=torch.int32, device=dev),
        "context_lens": torch.empty(B, dtype=torch.int32, device=dev),
        "positions": torch.empty(max(total_q, 1), dtype=torch.int32, device=dev)[:total_q],
        "slot_mapping": torch.empty(max(total_q, 1), dtype=torch.int32, device=dev)[:total_q],
    }
    st = lib().pa_build_metadata_store(_ptr(num_cached), _ptr(num_new), _ptr(block_table),
                                       int(block_table.shape[1]), B, int(total_q), nb, bs, _ptr(out["cu_seqlens_q"]),
                                       _ptr(out["cu_seqlens_k"]), _ptr(out["context_lens"]), _ptr(out["positions"]),
                                       _ptr(out["slot_mapping"]), _ptr(k), ks, _ptr(v), vs, _ptr(k_cache),
                                       _ptr(v_cache), hkv, d, _dtype_code(k_cache.dtype), _stream(stream))
    _check("pa_build_metadata_store", st)
    return out


def norm_rope_store_kvcache(k, v, k_cache, v_cache, slot_mapping, k_norm_weight, positions, cos_sin,
                            rms_eps: float = 1e-6, q=None, q_norm_weight=None, q_out=None, stream=None):
    """pa_norm_rope_store_kvcache: k_norm + rotary embedding of k stored at its slot, v stored as is; with q,
    q_norm + rotary embedding into q_out ([T, Hq, D], allocated if None), which is returned."""
    nb, bs, hkv, d = _cache_dims(k_cache, v_cache)
    _require(k.dtype == k_cache.dtype and v.dtype == k_cache.dtype, "k/v must match the cache dtype")
    _require(k_norm_weight.dtype == k_cache.dtype and tuple(k_norm_weight.shape) == (d,),
             "k_norm_weight must be [head_dim] in the cache dtype")
    ks = _token_rows(k, hkv, d, "k")
    vs = _token_rows(v, hkv, d, "v")
    _i32(slot_mapping, "slot_mapping")
    _i32(positions, "positions")
    _require(cos_sin.dtype == torch.float32 and cos_sin.is_contiguous() and cos_sin.dim() == 2 and
             int(cos_sin.shape[1]) == d, "cos_sin must be contiguous float32 [max_position, head_dim]")
    T = int(k.shape[0])
    _require(v.shape[0] == T and slot_mapping.shape[0] == T and positions.shape[0] == T,
             "k, v, slot_mapping and positions must have one row per token")
    hq, qs = 0, 0
    if q is not None:
        _require(q.dtype == k_cache.dtype and q_norm_weight is not None and q_norm_weight.dtype == k_cache.dtype,
                 "q and q_norm_weight must be in the cache dtype")
        hq = int(q.shape[1])
        qs = _token_rows(q, hq, d, "q")
        if q_out is None:
            q_out = torch.empty((T, hq, d), dtype=q.dtype, device=q.device)
        _require(q_out.is_contiguous() and tuple(q_out.shape) == (T, hq, d), "q_out must be contiguous [T, Hq, D]")
    if checked_mode() and T > 0:
        _validate("pa_norm_rope_store_kvcache", num_blocks=nb, block_size=bs, slot_mapping=slot_mapping,
                  stream=stream)
    st = lib().pa_norm_rope_store_kvcache(_ptr(k), ks, _ptr(v), vs, _ptr(k_norm_weight), _ptr(q), qs,
                                          _ptr(q_norm_weight), _ptr(q_out), hq, float(rms_eps), _ptr(positions),
                                          _ptr(cos_sin), int(cos_sin.shape[0]), _ptr(k_cache), _ptr(v_cache),
                                          _ptr(slot_mapping), T, hkv, d, nb, bs, _dtype_code(k_cache.dtype),
                                          _stream(stream))
    _check("pa_norm_rope_store_kvcache", st)
    return q_out


def sample_workspace_bytes(batch: int, vocab: int) -> int:
    return int(lib().pa_sample_workspace_bytes(batch, vocab))


def sample(logits, temperatures, seed: int, offset: int, tokens=None, workspace=None, stream=None):
    """pa_sample: logits [B, V] float32 (row stride free), temperatures [B] float32 -> tokens [B] int32."""
    _require(logits.dtype == torch.float32 and logits.dim() == 2 and logits.stride(1) == 1,
             "logits must be float32 [B, V] with contiguous rows")
    _require(temperatures.dtype == torch.float32 and temperatures.is_contiguous(), "temperatures must be float32")
    B, V = int(logits.shape[0]), int(logits.shape[1])
    _require(temperatures.numel() == B, "one temperature per row")
    if tokens is None:
        tokens = torch.empty(B, dtype=torch.int32, device=logits.device)
    _i32(tokens, "tokens")
    need = sample_workspace_bytes(B, V)
    if workspace is None:
        workspace = torch.empty(max(need, 8), dtype=torch.uint8, device=logits.device)
    wbytes = workspace.numel() * workspace.element_size()
    st = lib().pa_sample(_ptr(logits), int(logits.stride(0)), _ptr(temperatures), B, V, int(seed) & (2 ** 64 - 1),
                         int(offset) & (2 ** 64 - 1), _ptr(tokens), _ptr(workspace), wbytes, _stream(stream))
    _check("pa_sample", st)
    return tokens


def prefill_workspace_bytes(batch, num_heads, head_dim, max_seqlen_q, max_seqlen_k) -> int:
    return int(lib().pa_prefill_workspace_bytes(batch, num_heads, head_dim, max_seqlen_q, max_seqlen_k))


def prefill_varlen(q, k_cache, v_cache, cu_seqlens_q, cu_seqlens_k, block_table, max_seqlen_q: int,
                   max_seqlen_k: int, softmax_scale: float, out=None, out_dtype=torch.float32, workspace=None,
                   stream=None):
    """pa_prefill_varlen. q [total_q, Hq, D]; returns out [total_q, Hq, D]."""
    nb, bs, hkv, d = _cache_dims(k_cache, v_cache)
    _require(q.dtype == k_cache.dtype, "q must match the cache dtype")
    hq = int(q.shape[1])
    qs = _token_rows(q, hq, d, "q")
    for t, n in ((cu_seqlens_q, "cu_seqlens_q"), (cu_seqlens_k, "cu_seqlens_k"), (block_table, "block_table")):
        _i32(t, n)
    B = int(cu_seqlens_q.shape[0]) - 1
    T = int(q.shape[0])
    if out is None:
        out = torch.empty((T, hq, d), dtype=out_dtype, device=q.device)
    _require(out.is_contiguous() and tuple(out.shape) == (T, hq, d), "out must be contiguous [total_q, Hq, D]")
    if checked_mode() and B > 0:
        _validate("pa_prefill_varlen", num_blocks=nb, block_size=bs, num_tokens=T, block_table=block_table,
                  cu_seqlens_q=cu_seqlens_q, cu_seqlens_k=cu_seqlens_k, stream=stream)
    need = prefill_workspace_bytes(B, hq, d, max_seqlen_q, max_seqlen_k)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().pa_prefill_varlen(_ptr(q), qs, _ptr(k_cache), _ptr(v_cache), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                                 _ptr(block_table), int(block_table.shape[1]), B, T, int(max_seqlen_q),
                                 int(max_seqlen_k), hq, hkv, d, nb, bs, float(softmax_scale),
                                 _dtype_code(q.dtype), _ptr(out), _dtype_code(out.dtype), _ptr(workspace), wbytes,
                                 _stream(stream))
    _check("pa_prefill_varlen", st)
    return out


def decode_append_noalloc(q, k_new, v_new, k_cache, v_cache, num_cached, block_table, softmax_scale: float, out,
                          stream=None):
    """pa_decode_append_noalloc: as decode_append, with the partials in the library's own device scratch (no
    workspace, nothing allocated here or in the library: out must be given). Raises on shapes the call does not
    take (no fallback, since the fallback would allocate)."""
    nb, bs, hkv, d = _cache_dims(k_cache, v_cache)
    _require(q.dtype == k_cache.dtype and k_new.dtype == k_cache.dtype and v_new.dtype == k_cache.dtype,
             "q, k_new and v_new must match the cache dtype")
    hq = int(q.shape[1])
    qs = _token_rows(q, hq, d, "q")
    ks = _token_rows(k_new, hkv, d, "k_new")
    vs = _token_rows(v_new, hkv, d, "v_new")
    _i32(num_cached, "num_cached")
    _i32(block_table, "block_table")
    B = int(q.shape[0])
    _require(k_new.shape[0] == B and v_new.shape[0] == B and num_cached.shape[0] == B,
             "q, k_new, v_new and num_cached must have one row per sequence")
    _require(out is not None and out.is_contiguous() and tuple(out.shape) == (B, hq, d),
             "out must be given, contiguous [B, Hq, D]")
    st = lib().pa_decode_append_noalloc(_ptr(q), qs, _ptr(k_new), ks, _ptr(v_new), vs, _ptr(k_cache), _ptr(v_cache),
                                        _ptr(num_cached), _ptr(block_table), int(block_table.shape[1]), B, hq, hkv, d,
                                        nb, bs, float(softmax_scale), _dtype_code(q.dtype), _ptr(out),
                                        _dtype_code(out.dtype), _stream(stream))
    _check("pa_decode_append_noalloc", st)
    return out


def decode_split_tokens(batch, num_heads, num_kv_heads, head_dim, max_blocks_per_seq, block_size) -> int:
    return int(lib().pa_decode_split_tokens(batch, num_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                                            block_size))


def decode_workspace_bytes(batch, num_heads, num_kv_heads, head_dim, max_blocks_per_seq, block_size,
                           split_tokens=0) -> int:
    return int(lib().pa_decode_workspace_bytes(batch, num_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                                               block_size, split_tokens))


def decode(q, k_cache, v_cache, context_lens, block_table, softmax_scale: float, out=None,
           out_dtype=torch.float32, split_tokens: int = 0, workspace=None, stream=None):
    """pa_decode. q [B, Hq, D]; returns out [B, Hq, D]."""
    nb, bs, hkv, d = _cache_dims(k_cache, v_cache)
    _require(q.dtype == k_cache.dtype, "q must match the cache dtype")
    hq = int(q.shape[1])
    qs = _token_rows(q, hq, d, "q")
    _i32(context_lens, "context_lens")
    _i32(block_table, "block_table")
    B = int(q.shape[0])
    mbps = int(block_table.shape[1])
    if out is None:
        out = torch.empty((B, hq, d), dtype=out_dtype, device=q.device)
    _require(out.is_contiguous() and tuple(out.shape) == (B, hq, d), "out must be contiguous [B, Hq, D]")
    if checked_mode() and B > 0:
        _validate("pa_decode", num_blocks=nb, block_size=bs, block_table=block_table, context_lens=context_lens,
                  stream=stream)
    need = decode_workspace_bytes(B, hq, hkv, d, mbps, bs, split_tokens)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().pa_decode(_ptr(q), qs, _ptr(k_cache), _ptr(v_cache), _ptr(context_lens), _ptr(block_table), mbps, B,
                         hq, hkv, d, nb, bs, float(softmax_scale), _dtype_code(q.dtype), _ptr(out),
                         _dtype_code(out.dtype), int(split_tokens), _ptr(workspace), wbytes, _stream(stream))
    _check("pa_decode", st)
    return out


def decode_append(q, k_new, v_new, k_cache, v_cache, num_cached, block_table, softmax_scale: float, out=None,
                  out_dtype=torch.float32, workspace=None, fallback=True, stream=None):
    """pa_decode_append: k_new/v_new [B, Hkv, D] stored at position num_cached[s] of each sequence, then decode
    over num_cached + 1 keys; returns out [B, Hq, D]. For shapes the fused call does not take, and in checked
    mode, the same result comes from build_metadata_store followed by decode (with fallback=False an unsupported
    shape raises instead)."""
    nb, bs, hkv, d = _cache_dims(k_cache, v_cache)
    _require(q.dtype == k_cache.dtype and k_new.dtype == k_cache.dtype and v_new.dtype == k_cache.dtype,
             "q, k_new and v_new must match the cache dtype")
    hq = int(q.shape[1])
    qs = _token_rows(q, hq, d, "q")
    ks = _token_rows(k_new, hkv, d, "k_new")
    vs = _token_rows(v_new, hkv, d, "v_new")
    _i32(num_cached, "num_cached")
    _i32(block_table, "block_table")
    B = int(q.shape[0])
    _require(k_new.shape[0] == B and v_new.shape[0] == B and num_cached.shape[0] == B,
             "q, k_new, v_new and num_cached must have one row per sequence")
    mbps = int(block_table.shape[1])
    if out is None:
        out = torch.empty((B, hq, d), dtype=out_dtype, device=q.device)
    _require(out.is_contiguous() and tuple(out.shape) == (B, hq, d), "out must be contiguous [B, Hq, D]")
    need = decode_workspace_bytes(B, hq, hkv, d, mbps, bs, 0)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = PA_ERR_UNSUPPORTED
    if not checked_mode():
        st = lib().pa_decode_append(_ptr(q), qs, _ptr(k_new), ks, _ptr(v_new), vs, _ptr(k_cache), _ptr(v_cache),
                                    _ptr(num_cached), _ptr(block_table), mbps, B, hq, hkv, d, nb, bs,
                                    float(softmax_scale), _dtype_code(q.dtype), _ptr(out), _dtype_code(out.dtype),
                                    _ptr(workspace), wbytes, _stream(stream))
    if st == PA_ERR_UNSUPPORTED and (fallback or checked_mode()):
        ones = torch.ones(B, dtype=torch.int32, device=q.device)
        meta = build_metadata_store(num_cached, ones, block_table, B, k_new, v_new, k_cache, v_cache, stream=stream)
        return decode(q, k_cache, v_cache, meta["context_lens"], block_table, softmax_scale, out=out,
                      workspace=workspace, stream=stream)
    _check("pa_decode_append", st)
    return out

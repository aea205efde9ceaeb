"""Thin ctypes binding of libattn (include/attn.h).

The functions named like the C entry points (``attn_prefill_fwd``,
``attn_decode_fwd``, ``attn_decode_combine``) take torch tensors on the GPU
and only marshal arguments: data pointers, element strides, sizes and the
current HIP stream. Every step of the computation runs in the HIP kernels.
``prefill`` and ``decode`` are conveniences that allocate outputs and the
decode workspace with torch, then call the entry points.

Loading fails loudly when the library is missing or a tensor is not on a
GPU: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libattn.so")

ATTN_F32, ATTN_F16, ATTN_BF16 = 0, 1, 2
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported configuration", 3: "kernel launch failed"}
SYMBOLS = ("attn_prefill_fwd", "attn_prefill_fwd_ex", "attn_prefill_fwd_fp8kv", "attn_prefill_varlen_fwd", "attn_decode_fwd", "attn_decode_fwd_fp8kv",
           "attn_decode_combine", "attn_decode_combine_ex", "attn_decode_validate_pages", "attn_decode_workspace_size",
           "attn_decode_fwd_noalloc", "attn_status_string", "attn_prefill_kernel_for", "attn_prefill_kernel_name",
           "attn_decode_heads_per_workgroup")
# Bytes of the library's device array for attn_decode_fwd_noalloc's partials (ATTN_DECODE_NOALLOC_MAX_BYTES).
DECODE_NOALLOC_MAX_BYTES = 32 << 20


class AttnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {STATUS.get(status, 'unknown')} (status {status})")
        self.status = status


class Strides(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seq", ctypes.c_int64), ("head", ctypes.c_int64)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libattn with argument types declared."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m flash_attention_forward_amd.build`")
    # torch first: its HIP runtime then satisfies the library's libamdhip64 dependency. Loaded the other
    # way round, the process holds two HIP runtimes, and a launch on a stream of torch's fails.
    import torch  # noqa: F401

    L = ctypes.CDLL(LIB_PATH)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    L.attn_prefill_fwd.argtypes = [vp, Strides, vp, Strides, vp, Strides, vp, Strides, i32, i32, i32, i32, i32,
                                   i32, i32, f32, i32, i32, vp]
    L.attn_prefill_fwd.restype = i32
    L.attn_prefill_fwd_ex.argtypes = [vp, Strides, vp, Strides, vp, Strides, vp, Strides, i32, i32, i32, i32, i32,
                                      i32, i32, f32, i32, i32, vp, vp, vp]
    L.attn_prefill_fwd_ex.restype = i32
    L.attn_prefill_fwd_fp8kv.argtypes = [vp, Strides, vp, Strides, vp, Strides, vp, Strides, i32, i32, i32, i32, i32,
                                         i32, i32, f32, f32, f32, i32, i32, vp, vp, vp]
    L.attn_prefill_fwd_fp8kv.restype = i32
    L.attn_prefill_varlen_fwd.argtypes = [vp, Strides, vp, Strides, vp, Strides, vp, Strides, i32, i32, i32, i32, vp,
                                          vp, i32, i32, i32, f32, i32, i32, vp, vp, vp, vp]
    L.attn_prefill_varlen_fwd.restype = i32
    L.attn_decode_fwd.argtypes = [vp, Strides, vp, vp, Strides, vp, i32, i32, vp, i32, i32, i32, i32, i32, i32,
                                  f32, i32, vp, vp, i32, i32, vp]
    L.attn_decode_fwd.restype = i32
    L.attn_decode_fwd_fp8kv.argtypes = [vp, Strides, vp, vp, Strides, vp, i32, i32, vp, i32, i32, i32, i32, i32, i32,
                                        f32, f32, f32, i32, vp, vp, i32, i32, vp]
    L.attn_decode_fwd_fp8kv.restype = i32
    L.attn_decode_combine.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, Strides, i32, vp]
    L.attn_decode_combine.restype = i32
    L.attn_decode_combine_ex.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, Strides, i32, vp, vp, vp]
    L.attn_decode_combine_ex.restype = i32
    L.attn_decode_validate_pages.argtypes = [vp, i32, i32, vp, i32, ctypes.c_int64, vp, vp]
    L.attn_decode_validate_pages.restype = i32
    L.attn_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(ctypes.c_size_t),
                                             ctypes.POINTER(ctypes.c_size_t)]
    L.attn_decode_workspace_size.restype = i32
    L.attn_decode_fwd_noalloc.argtypes = [vp, Strides, vp, vp, Strides, vp, i32, i32, vp, i32, i32, i32, i32, i32,
                                          i32, f32, i32, i32, i32, vp, Strides, vp]
    L.attn_decode_fwd_noalloc.restype = i32
    L.attn_status_string.argtypes = [i32]
    L.attn_status_string.restype = ctypes.c_char_p
    L.attn_prefill_kernel_for.argtypes = [i32] * 12
    L.attn_prefill_kernel_for.restype = i32
    L.attn_prefill_kernel_name.argtypes = [i32]
    L.attn_prefill_kernel_name.restype = ctypes.c_char_p
    L.attn_decode_heads_per_workgroup.argtypes = [i32] * 5
    L.attn_decode_heads_per_workgroup.restype = i32
    _lib = L
    return L


# ----------------------------------------------------------------------------- marshalling helpers
def _dtype_code(t) -> int:
    import torch

    codes = {torch.float32: ATTN_F32, torch.float16: ATTN_F16, torch.bfloat16: ATTN_BF16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _gpu(t, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (libattn has no CPU path)")
    return t


def _strides4(t, name: str) -> Strides:
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError(f"{name} must be 4-D [batch, seq, heads, head_dim] with a contiguous last dim")
    return Strides(t.stride(0), t.stride(1), t.stride(2))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream):
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn: str, rc: int):
    if rc != 0:
        raise AttnError(fn, rc)


# ----------------------------------------------------------------------------- entry points
def _f32_vec(t, name: str, n: int):
    """An optional contiguous float32 GPU tensor with n elements (None passes through)."""
    import torch

    if t is None:
        return None
    _gpu(t, name)
    if t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != n:
        raise ValueError(f"{name} must be a contiguous float32 tensor of {n} elements")
    return t


def attn_prefill_fwd(q, k, v, o, scale: float, causal: bool, window: int = 0, stream=None) -> None:
    """O <- attention(q, k, v). q, o: [B, Sq, Hq, D]; k, v: [B, Skv, Hkv, D]; same dtype."""
    attn_prefill_fwd_ex(q, k, v, o, scale, causal, window, None, None, stream, _name="attn_prefill_fwd")


def attn_prefill_fwd_ex(q, k, v, o, scale: float, causal: bool, window: int = 0, lse=None, sinks=None,
                        stream=None, _name: str = "attn_prefill_fwd_ex") -> None:
    """attn_prefill_fwd plus lse (float32 [B, Sq, Hq] out) and sinks (float32 [Hq] in), each optional."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _gpu(t, n)
    B, Sq, Hq, D = q.shape
    Bk, Skv, Hkv, Dk = k.shape
    if v.shape != k.shape or o.shape != q.shape or Bk != B or Dk != D:
        raise ValueError("shape mismatch between q, k, v, o")
    dt = _dtype_code(q)
    if not (k.dtype == v.dtype == o.dtype == q.dtype):
        raise TypeError("q, k, v, o must share one dtype")
    lse = _f32_vec(lse, "lse", B * Sq * Hq)
    sinks = _f32_vec(sinks, "sinks", Hq)
    L = lib()
    args = (_ptr(q), _strides4(q, "q"), _ptr(k), _strides4(k, "k"), _ptr(v), _strides4(v, "v"), _ptr(o),
            _strides4(o, "o"), dt, B, Hq, Hkv, Sq, Skv, D, float(scale), int(bool(causal)), int(window))
    if _name == "attn_prefill_fwd":
        rc = L.attn_prefill_fwd(*args, _stream(stream))
    else:
        rc = L.attn_prefill_fwd_ex(*args, _ptr(lse), _ptr(sinks), _stream(stream))
    _check(_name, rc)


def attn_prefill_fwd_fp8kv(q, k, v, o, scale: float, causal: bool, window: int = 0, k_scale: float = 1.0,
                           v_scale: float = 1.0, lse=None, sinks=None, stream=None) -> None:
    """attn_prefill_fwd_ex with K and V as FP8 E4M3 codes (torch.float8_e4m3fn or uint8, [B, Skv, Hkv, D]);
    a code stands for k_scale (v_scale) times its value. q and o are f16 or bf16."""
    import torch

    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _gpu(t, n)
    B, Sq, Hq, D = q.shape
    Bk, Skv, Hkv, Dk = k.shape
    if v.shape != k.shape or o.shape != q.shape or Bk != B or Dk != D:
        raise ValueError("shape mismatch between q, k, v, o")
    if k.dtype not in (torch.float8_e4m3fn, torch.uint8) or v.dtype != k.dtype:
        raise TypeError("k and v must be float8_e4m3fn (or uint8 codes)")
    if o.dtype != q.dtype:
        raise TypeError("q and o must share one dtype")
    dt = _dtype_code(q)
    lse = _f32_vec(lse, "lse", B * Sq * Hq)
    sinks = _f32_vec(sinks, "sinks", Hq)
    rc = lib().attn_prefill_fwd_fp8kv(_ptr(q), _strides4(q, "q"), _ptr(k), _strides4(k, "k"), _ptr(v),
                                      _strides4(v, "v"), _ptr(o), _strides4(o, "o"), dt, B, Hq, Hkv, Sq, Skv, D,
                                      float(scale), float(k_scale), float(v_scale), int(bool(causal)), int(window),
                                      _ptr(lse), _ptr(sinks), _stream(stream))
    _check("attn_prefill_fwd_fp8kv", rc)


def _strides3(t, name: str) -> Strides:
    """Strides of a packed [tokens, heads, head_dim] tensor (the batch stride is unused)."""
    if t.dim() != 3 or t.stride(2) != 1:
        raise ValueError(f"{name} must be 3-D [tokens, heads, head_dim] with a contiguous last dim")
    return Strides(0, t.stride(0), t.stride(1))


def attn_prefill_varlen_fwd(q, k, v, o, cu_seqlens_q, cu_seqlens_kv, max_seqlen_q: int, max_seqlen_kv: int,
                            scale: float, causal: bool, window: int = 0, lse=None, sinks=None, positions=None,
                            stream=None) -> None:
    """Packed sequences: q, o [total_q, Hq, D]; k, v [total_kv, Hkv, D]; cu_seqlens_* int32 [B + 1] on the GPU.
    lse: float32 [total_q, Hq] out; sinks: float32 [Hq] in; positions: int32 [total_q] in (each row's position
    within its sequence's keys, nondecreasing per sequence); all optional."""
    import torch

    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (cu_seqlens_q, "cu_seqlens_q"),
                 (cu_seqlens_kv, "cu_seqlens_kv")):
        _gpu(t, n)
    Tq, Hq, D = q.shape
    Tk, Hkv, Dk = k.shape
    if v.shape != k.shape or o.shape != q.shape or Dk != D:
        raise ValueError("shape mismatch between q, k, v, o")
    if not (k.dtype == v.dtype == o.dtype == q.dtype):
        raise TypeError("q, k, v, o must share one dtype")
    for c, n in ((cu_seqlens_q, "cu_seqlens_q"), (cu_seqlens_kv, "cu_seqlens_kv")):
        if c.dtype != torch.int32 or c.dim() != 1 or not c.is_contiguous():
            raise TypeError(f"{n} must be a contiguous int32 vector")
    if cu_seqlens_q.numel() != cu_seqlens_kv.numel() or cu_seqlens_q.numel() < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_kv must both hold batch + 1 offsets")
    B = cu_seqlens_q.numel() - 1
    lse = _f32_vec(lse, "lse", Tq * Hq)
    sinks = _f32_vec(sinks, "sinks", Hq)
    if positions is not None:
        _gpu(positions, "positions")
        if positions.dtype != torch.int32 or not positions.is_contiguous() or positions.numel() != Tq:
            raise ValueError(f"positions must be a contiguous int32 tensor of {Tq} elements")
    rc = lib().attn_prefill_varlen_fwd(_ptr(q), _strides3(q, "q"), _ptr(k), _strides3(k, "k"), _ptr(v),
                                       _strides3(v, "v"), _ptr(o), _strides3(o, "o"), _dtype_code(q), B, Hq, Hkv,
                                       _ptr(cu_seqlens_q), _ptr(cu_seqlens_kv), int(max_seqlen_q), int(max_seqlen_kv),
                                       D, float(scale), int(bool(causal)), int(window), _ptr(lse), _ptr(sinks),
                                       _ptr(positions), _stream(stream))
    _check("attn_prefill_varlen_fwd", rc)


def attn_decode_fwd(q, k_cache, v_cache, cache_len, part_o, part_lse, split_len: int, max_splits: int,
                    scale: float, block_table=None, window: int = 0, stream=None) -> None:
    """Split-KV partials. Paged if block_table is given ([B, max_pages] uint32 stored as int32)."""
    _decode_fwd(q, k_cache, v_cache, cache_len, part_o, part_lse, split_len, max_splits, scale, block_table, window,
                stream, None)


def attn_decode_fwd_fp8kv(q, k_cache, v_cache, cache_len, part_o, part_lse, split_len: int, max_splits: int,
                          scale: float, k_scale: float = 1.0, v_scale: float = 1.0, block_table=None, window: int = 0,
                          stream=None) -> None:
    """attn_decode_fwd for an FP8 E4M3 cache (torch.float8_e4m3fn or uint8 codes); q stays f16/bf16."""
    _decode_fwd(q, k_cache, v_cache, cache_len, part_o, part_lse, split_len, max_splits, scale, block_table, window,
                stream, (float(k_scale), float(v_scale)))


def _decode_fwd(q, k_cache, v_cache, cache_len, part_o, part_lse, split_len, max_splits, scale, block_table, window,
                stream, fp8_scales):
    import torch

    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (cache_len, "cache_len"),
                 (part_o, "part_o"), (part_lse, "part_lse")):
        _gpu(t, n)
    if cache_len.dtype != torch.int32 or part_o.dtype != torch.float32 or part_lse.dtype != torch.float32:
        raise TypeError("cache_len must be int32 and part_o / part_lse float32")
    B, sa, Hq, D = q.shape
    if k_cache.shape != v_cache.shape or k_cache.stride() != v_cache.stride():
        raise ValueError("k_cache and v_cache must have the same shape and strides")
    Hkv = k_cache.shape[2]
    if block_table is not None:
        _gpu(block_table, "block_table")
        if block_table.dtype not in (torch.int32, torch.uint32) or not block_table.is_contiguous():
            raise TypeError("block_table must be a contiguous 32-bit tensor")
        maxp, ps = block_table.shape[1], k_cache.shape[1]
    else:
        maxp, ps = 0, 0
    head = (_ptr(q), _strides4(q, "q"), _ptr(k_cache), _ptr(v_cache), _strides4(k_cache, "k_cache"),
            _ptr(block_table), maxp, ps, _ptr(cache_len), _dtype_code(q), B, sa, Hq, Hkv, D, float(scale))
    tail = (int(window), _ptr(part_o), _ptr(part_lse), int(split_len), int(max_splits), _stream(stream))
    if fp8_scales is None:
        if k_cache.dtype != q.dtype:
            raise TypeError("k_cache and v_cache must have q's dtype (use attn_decode_fwd_fp8kv for FP8 caches)")
        _check("attn_decode_fwd", lib().attn_decode_fwd(*head, *tail))
    else:
        if k_cache.dtype not in (torch.float8_e4m3fn, torch.uint8) or v_cache.dtype != k_cache.dtype:
            raise TypeError("FP8 caches must be torch.float8_e4m3fn (or uint8 codes)")
        _check("attn_decode_fwd_fp8kv", lib().attn_decode_fwd_fp8kv(*head, *fp8_scales, *tail))


def attn_decode_fwd_noalloc(q, k_cache, v_cache, cache_len, split_len: int, max_splits: int, scale: float, o,
                            block_table=None, window: int = 0, stream=None) -> None:
    """attn_decode_fwd + attn_decode_combine in one call, o [B, s_active, Hq, D] written, with the partials in
    the library's own device array: nothing is allocated (16-bit cache; see DECODE_NOALLOC_MAX_BYTES)."""
    import torch

    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (cache_len, "cache_len"), (o, "o")):
        _gpu(t, n)
    if cache_len.dtype != torch.int32:
        raise TypeError("cache_len must be int32")
    if k_cache.shape != v_cache.shape or k_cache.stride() != v_cache.stride():
        raise ValueError("k_cache and v_cache must have the same shape and strides")
    if k_cache.dtype != q.dtype or o.dtype != q.dtype or o.shape != q.shape:
        raise TypeError("k_cache, v_cache and o must have q's dtype, o q's shape")
    B, sa, Hq, D = q.shape
    if block_table is not None:
        _gpu(block_table, "block_table")
        if block_table.dtype not in (torch.int32, torch.uint32) or not block_table.is_contiguous():
            raise TypeError("block_table must be a contiguous 32-bit tensor")
        maxp, ps = block_table.shape[1], k_cache.shape[1]
    else:
        maxp, ps = 0, 0
    rc = lib().attn_decode_fwd_noalloc(_ptr(q), _strides4(q, "q"), _ptr(k_cache), _ptr(v_cache),
                                       _strides4(k_cache, "k_cache"), _ptr(block_table), maxp, ps, _ptr(cache_len),
                                       _dtype_code(q), B, sa, Hq, k_cache.shape[2], D, float(scale), int(window),
                                       int(split_len), int(max_splits), _ptr(o), _strides4(o, "o"), _stream(stream))
    _check("attn_decode_fwd_noalloc", rc)


def attn_decode_combine(part_o, part_lse, cache_len, split_len: int, max_splits: int, o, stream=None) -> None:
    """o [B, s_active, Hq, D] <- LSE merge of the partials."""
    attn_decode_combine_ex(part_o, part_lse, cache_len, split_len, max_splits, o, None, None, stream,
                           _name="attn_decode_combine")


def attn_decode_combine_ex(part_o, part_lse, cache_len, split_len: int, max_splits: int, o, lse=None, sinks=None,
                           stream=None, _name: str = "attn_decode_combine_ex") -> None:
    """attn_decode_combine plus lse (float32 [B, s_active, Hq] out) and sinks (float32 [Hq] in), each optional."""
    for t, n in ((part_o, "part_o"), (part_lse, "part_lse"), (cache_len, "cache_len"), (o, "o")):
        _gpu(t, n)
    B, sa, Hq, D = o.shape
    lse = _f32_vec(lse, "lse", B * sa * Hq)
    sinks = _f32_vec(sinks, "sinks", Hq)
    L = lib()
    args = (_ptr(part_o), _ptr(part_lse), _ptr(cache_len), int(split_len), int(max_splits), B, sa, Hq, D, _ptr(o),
            _strides4(o, "o"), _dtype_code(o))
    if _name == "attn_decode_combine":
        rc = L.attn_decode_combine(*args, _stream(stream))
    else:
        rc = L.attn_decode_combine_ex(*args, _ptr(lse), _ptr(sinks), _stream(stream))
    _check(_name, rc)


def attn_decode_validate_pages(block_table, cache_len, page_size: int, num_pages: int, result=None,
                               stream=None):
    """Device check of a page table ([B, max_pages] 32-bit) against cache_len and the pool's page count.
    Returns the int32 [2] GPU tensor (problem count, lowest bad flat index or INT32_MAX), written on the stream."""
    import torch

    for t, n in ((block_table, "block_table"), (cache_len, "cache_len")):
        _gpu(t, n)
    if block_table.dtype not in (torch.int32, torch.uint32) or block_table.dim() != 2 or not block_table.is_contiguous():
        raise TypeError("block_table must be a contiguous 2-D 32-bit tensor")
    if cache_len.dtype != torch.int32 or cache_len.numel() != block_table.shape[0]:
        raise TypeError("cache_len must be int32 with one entry per sequence")
    if result is None:
        result = torch.empty(2, dtype=torch.int32, device=block_table.device)
    _check("attn_decode_validate_pages",
           lib().attn_decode_validate_pages(_ptr(block_table), block_table.shape[1], int(page_size), _ptr(cache_len),
                                            block_table.shape[0], int(num_pages), _ptr(result), _stream(stream)))
    return result


# ----------------------------------------------------------------------------- conveniences
def prefill_kernel(dtype: str, batch: int, n_q_heads: int, n_kv_heads: int, seqlen_q: int, seqlen_kv: int,
                   head_dim: int, causal: bool, window: int = 0, fp8_kv: bool = False, packed: bool = False,
                   positions: bool = False) -> str:
    """Name of the kernel the prefill entry points launch for these sizes (attn_prefill_kernel_for:
    host arithmetic only, the same choice the launch makes). dtype is "f32", "f16" or "bf16"."""
    code = {"f32": ATTN_F32, "f16": ATTN_F16, "bf16": ATTN_BF16}[dtype]
    k = lib().attn_prefill_kernel_for(code, int(fp8_kv), int(packed), int(positions), batch, n_q_heads, n_kv_heads,
                                      seqlen_q, seqlen_kv, head_dim, int(bool(causal)), int(window))
    if k < 0:
        raise AttnError("attn_prefill_kernel_for", -k)
    return lib().attn_prefill_kernel_name(k).decode() if k > 0 else ""


def decode_heads_per_workgroup(batch: int, n_kv_heads: int, head_dim: int, max_splits: int,
                               fp8_kv: bool = False) -> int:
    """Kv-heads per workgroup of the decode split kernel for these sizes (attn_decode_heads_per_workgroup)."""
    return lib().attn_decode_heads_per_workgroup(int(fp8_kv), batch, n_kv_heads, head_dim, max_splits)


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)


def prefill(q, k, v, scale: float | None = None, causal: bool = False, window: int = 0, out=None, stream=None,
            sinks=None, return_lse: bool = False, k_scale: float = 1.0, v_scale: float = 1.0):
    """Output (and, with return_lse, the float32 [B, Sq, Hq] log-sum-exp); sinks: float32 [Hq] or None.
    K and V may be FP8 E4M3 (float8_e4m3fn or uint8 codes, scaled by k_scale and v_scale)."""
    import torch

    o = torch.empty_like(q) if out is None else out
    sc = default_scale(q.shape[-1]) if scale is None else scale
    if k.dtype in (torch.float8_e4m3fn, torch.uint8):
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if return_lse else None
        attn_prefill_fwd_fp8kv(q, k, v, o, sc, causal, window, k_scale, v_scale, lse, sinks, stream)
        return (o, lse) if return_lse else o
    if sinks is None and not return_lse:
        attn_prefill_fwd(q, k, v, o, sc, causal, window, stream)
        return o
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if return_lse else None
    attn_prefill_fwd_ex(q, k, v, o, sc, causal, window, lse, sinks, stream)
    return (o, lse) if return_lse else o


def prefill_varlen(q, k, v, seqlens_q, seqlens_kv=None, scale: float | None = None, causal: bool = False,
                   window: int = 0, out=None, stream=None, sinks=None, return_lse: bool = False, positions=None):
    """Packed-sequence prefill from per-sequence lengths (host ints); the offsets go to the GPU as int32."""
    import torch

    seqlens_kv = seqlens_q if seqlens_kv is None else seqlens_kv
    if len(seqlens_q) != len(seqlens_kv):
        raise ValueError("one q length and one k/v length per sequence")
    cu_q = torch.tensor([0] + list(_cumsum(seqlens_q)), dtype=torch.int32, device=q.device)
    cu_k = torch.tensor([0] + list(_cumsum(seqlens_kv)), dtype=torch.int32, device=q.device)
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device) if return_lse else None
    sc = default_scale(q.shape[-1]) if scale is None else scale
    attn_prefill_varlen_fwd(q, k, v, o, cu_q, cu_k, max(seqlens_q, default=0), max(seqlens_kv, default=0), sc, causal,
                            window, lse, sinks, positions, stream)
    return (o, lse) if return_lse else o


def _cumsum(xs):
    t = 0
    for x in xs:
        t += int(x)
        yield t


class DecodeWorkspace:
    """part_o / part_lse buffers for attn_decode_fwd, reusable across calls of the same shape."""

    def __init__(self, batch: int, s_active: int, n_q_heads: int, head_dim: int, max_splits: int, device):
        import torch

        self.max_splits = max_splits
        self.part_o = torch.empty((batch, s_active, n_q_heads, max_splits, head_dim), dtype=torch.float32, device=device)
        self.part_lse = torch.empty((batch, s_active, n_q_heads, max_splits), dtype=torch.float32, device=device)


def max_splits_for(max_len: int, split_len: int) -> int:
    return max(1, -(-max_len // split_len))


def auto_split_len(batch: int, n_kv_heads: int, max_len: int, page_size: int = 0, min_waves: int = 1024,
                   max_split: int = 4096) -> int:
    """The longest split (fewest partials to write and merge) that still gives the split kernel
    about min_waves waves (one per kv-head, split and sequence), down to 64 tokens. Measured on
    32 query heads over 8 kv-heads: 4096 for 32 sequences of up to 32K tokens, 1024 for 16 of 8K,
    512 for 8 of 8K, 256 for one of 32K, 128 for 4 of 4K and 64 for one of 4K (11 us there,
    against 28 us at 512-token splits). With pages (page_size > 0) it is a multiple of 16 and of
    the page size and spans at most 256 pages."""
    cands = [c for c in (4096, 2048, 1024, 512, 256, 128, 64) if c <= max_split] or [64]
    sl = cands[-1]
    for cand in cands:
        if batch * n_kv_heads * max_splits_for(max_len, cand) >= min_waves:
            sl = cand
            break
    if page_size > 0:
        unit = 16 * page_size // math.gcd(16, page_size)
        sl = max(unit, min(sl // unit * unit, 256 * page_size // unit * unit))
    return sl


def decode(q, k_cache, v_cache, cache_len, block_table=None, scale: float | None = None, window: int = 0,
           split_len: int | None = None, max_len: int | None = None, workspace: DecodeWorkspace | None = None, out=None,
           stream=None, sinks=None, return_lse: bool = False, k_scale: float = 1.0, v_scale: float = 1.0):
    """Split-KV decode followed by the combine, both on the current stream (optionally with
    attention sinks, float32 [Hq], and returning the float32 [B, s_active, Hq] log-sum-exp)."""
    import torch

    B, sa, Hq, D = q.shape
    if max_len is None:
        max_len = block_table.shape[1] * k_cache.shape[1] if block_table is not None else k_cache.shape[1]
    fp8 = k_cache.dtype in (torch.float8_e4m3fn, torch.uint8)
    if split_len is None:
        # FP8 splits stream half the bytes; on the paged workload (32 sequences of up to 32K) they
        # measured best at 2048 tokens (218 us, eight kv-heads per workgroup; 1024: 233 us, 4096: 250 us)
        split_len = auto_split_len(B, k_cache.shape[2], max_len, k_cache.shape[1] if block_table is not None else 0,
                                   max_split=2048 if fp8 else 4096)
    ms = max_splits_for(max_len, split_len)
    ws = workspace or DecodeWorkspace(B, sa, Hq, D, ms, q.device)
    if ws.max_splits < ms:
        raise ValueError("workspace has too few splits")
    o = torch.empty_like(q) if out is None else out
    sc = default_scale(D) if scale is None else scale
    if fp8:
        attn_decode_fwd_fp8kv(q, k_cache, v_cache, cache_len, ws.part_o, ws.part_lse, split_len, ws.max_splits, sc,
                              k_scale, v_scale, block_table, window, stream)
    else:
        attn_decode_fwd(q, k_cache, v_cache, cache_len, ws.part_o, ws.part_lse, split_len, ws.max_splits, sc,
                        block_table, window, stream)
    if sinks is None and not return_lse:
        attn_decode_combine(ws.part_o, ws.part_lse, cache_len, split_len, ws.max_splits, o, stream)
        return o
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if return_lse else None
    attn_decode_combine_ex(ws.part_o, ws.part_lse, cache_len, split_len, ws.max_splits, o, lse, sinks, stream)
    return (o, lse) if return_lse else o

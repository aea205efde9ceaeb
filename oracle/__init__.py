"""fp64 CPU oracle for softmax attention — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product path (the HIP library and
its binding) never imports it, and this package imports nothing from the
product path: the only thing the two sides share is the seeded input
generator module, which holds no attention arithmetic.

``attention`` / ``attention_rows`` call the C library ``attn_oracle.c`` (the
plain definition: materialised score row, mask by exclusion, two-pass
softmax in fp64). ``decode`` first gathers each sequence's logical KV
through the page table with numpy fancy indexing — the torch reference's
``block_cache[active_blocks_table[b]]`` gather on the decode page
("Flash-Attention: Decode (TKG)", section "Paged / block cache") — and then
applies the same definition with the query at the end of the cache
(bottom-right causal alignment), which for one query token is the validity
cut ``index < cache_len`` of that page's section "gen_mask_tkg".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_BUILD = os.path.join(_HERE, "_build")
_LIB = os.path.join(_BUILD, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (fp64, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB):
        os.makedirs(_BUILD, exist_ok=True)
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall", "-o", tmp, _SRC, "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.oracle_attention_rows.argtypes = [p, p, p, p, p, p, i64, i64, i64, i64, i64,
                                              ctypes.c_double, ctypes.c_int, i64, p, p, p, i64, p, p]
        lib.oracle_attention_rows.restype = ctypes.c_int
        lib.oracle_visible_mask.argtypes = [i64, i64, ctypes.c_int, i64, p]
        lib.oracle_visible_mask.restype = None
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _strides3(a: np.ndarray):
    """Element strides of a [B, S, H, D] float64 array (D must be contiguous)."""
    assert a.dtype == np.float64 and a.ndim == 4
    if a.size == 0:  # numpy leaves strides of empty arrays arbitrary; nothing is read
        return np.zeros(3, dtype=np.int64)
    assert a.strides[3] == 8 or a.shape[3] == 1
    return np.array([a.strides[0] // 8, a.strides[1] // 8, a.strides[2] // 8], dtype=np.int64)


def visible_mask(Sq: int, Skv: int, causal: bool, window: int = 0) -> np.ndarray:
    """bool [Sq, Skv]: which keys each query row sees (the oracle's own predicate)."""
    m = np.zeros((Sq, Skv), dtype=np.uint8)
    _load().oracle_visible_mask(Sq, Skv, int(bool(causal)), int(window), _ptr(m))
    return m.astype(bool)


def attention_rows(q, k, v, scale: float, causal: bool, window: int, rows, sinks=None, positions=None):
    """Oracle output for selected rows.

    q: float64 [B, Sq, Hq, D]; k, v: float64 [B, Skv, Hkv, D] (views allowed,
    head_dim contiguous). rows: int array [n, 3] of (b, i, h). sinks: None or
    [Hq] sink logits (scaled-score units; see attn_oracle.c). positions: None or
    [Sq] integer position of each query row (default i + Skv - Sq).
    Returns (o [n, D] float64, lse [n] float64, natural log).
    """
    lib = _load()
    B, Sq, Hq, D = q.shape
    Bk, Skv, Hkv, Dk = k.shape
    assert v.shape == k.shape and Dk == D and Bk == B
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
    n = rows.shape[0]
    if n and ((rows < 0).any() or (rows[:, 0] >= B).any() or (rows[:, 1] >= Sq).any() or (rows[:, 2] >= Hq).any()):
        raise ValueError("oracle_attention_rows: a row index lies outside [B, Sq, Hq]")
    o = np.zeros((n, D), dtype=np.float64)
    lse = np.zeros(n, dtype=np.float64)
    qs, ks, vs = _strides3(q), _strides3(k), _strides3(v)
    sk = None
    if sinks is not None:
        sk = np.ascontiguousarray(sinks, dtype=np.float64).reshape(-1)
        assert sk.shape[0] == Hq
    qp = None
    if positions is not None:
        qp = np.ascontiguousarray(positions, dtype=np.int64).reshape(-1)
        assert qp.shape[0] == Sq
    rc = lib.oracle_attention_rows(_ptr(q), _ptr(qs), _ptr(k), _ptr(ks), _ptr(v), _ptr(vs),
                                   Hq, Hkv, Sq, Skv, D, float(scale), int(bool(causal)), int(window),
                                   _ptr(sk) if sk is not None else None, _ptr(qp) if qp is not None else None,
                                   _ptr(rows), n, _ptr(o), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle_attention_rows rejected its arguments")
    return o, lse


def all_rows(B: int, Sq: int, Hq: int) -> np.ndarray:
    b, i, h = np.meshgrid(np.arange(B), np.arange(Sq), np.arange(Hq), indexing="ij")
    return np.stack([b.ravel(), i.ravel(), h.ravel()], axis=1)


def attention(q, k, v, scale: float, causal: bool = False, window: int = 0, return_lse: bool = False,
              sinks=None, positions=None):
    """Full oracle output [B, Sq, Hq, D] (and lse [B, Sq, Hq]); positions as for attention_rows."""
    B, Sq, Hq, D = q.shape
    o, lse = attention_rows(q, k, v, scale, causal, window, all_rows(B, Sq, Hq), sinks, positions)
    o = o.reshape(B, Sq, Hq, D)
    lse = lse.reshape(B, Sq, Hq)
    return (o, lse) if return_lse else o


def attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_kv, scale: float, causal: bool = False, window: int = 0,
                     sinks=None, return_lse: bool = False, positions=None):
    """Oracle for packed sequences: each sequence is attended on its own.

    q: float64 [total_q, Hq, D]; k, v: float64 [total_kv, Hkv, D]; cu_seqlens_*:
    [B + 1] cumulative offsets (sequence b owns q rows cu_q[b]..cu_q[b+1] and
    k/v rows cu_kv[b]..cu_kv[b+1]). Each sequence is the plain definition on its
    own slice, with its query rows bottom-right aligned to its own keys — the
    per-sequence bounds of the CTE page's dynamic range_select family
    ("Algorithm — the dynamic range_select family": sequence-packing bounds and
    a dynamic prefix length). positions: None, or [total_q] integer position of
    every packed query row within its sequence's keys (the minfer page's
    positions input), replacing that alignment. Returns o [total_q, Hq, D] (and
    lse [total_q, Hq]).
    """
    cq = np.asarray(cu_seqlens_q, dtype=np.int64)
    ck = np.asarray(cu_seqlens_kv, dtype=np.int64)
    assert cq.shape == ck.shape and cq.ndim == 1
    o = np.zeros(q.shape, dtype=np.float64)
    lse = np.full(q.shape[:2], -np.inf, dtype=np.float64)
    for b in range(cq.shape[0] - 1):
        q0, q1, k0, k1 = cq[b], cq[b + 1], ck[b], ck[b + 1]
        if q1 <= q0:
            continue
        pos = None if positions is None else np.asarray(positions)[q0:q1]
        ob, lb = attention(np.ascontiguousarray(q[None, q0:q1]), np.ascontiguousarray(k[None, k0:k1]),
                           np.ascontiguousarray(v[None, k0:k1]), scale, causal, window, return_lse=True, sinks=sinks,
                           positions=pos)
        o[q0:q1] = ob[0]
        lse[q0:q1] = lb[0]
    return (o, lse) if return_lse else o


def gather_paged(pool: np.ndarray, block_table_row: np.ndarray, length: int) -> np.ndarray:
    """Logical KV [length, Hkv, D] of one sequence from a [pages, page_size, Hkv, D] pool."""
    ps = pool.shape[1]
    npages = -(-length // ps)
    pages = pool[block_table_row[:npages].astype(np.int64)]  # [npages, ps, Hkv, D]
    return pages.reshape(npages * ps, *pool.shape[2:])[:length]


def decode(q, k_pool, v_pool, block_table, cache_len, scale: float, window: int = 0,
           batches=None, to_f64=None, return_lse: bool = False, sinks=None):
    """Oracle paged decode.

    q: float64 [B, s_active, Hq, D]; pools: [num_pages, page_size, Hkv, D]
    (float64, or any storage array with ``to_f64`` converting a gathered
    slice exactly); block_table: uint32 [B, max_pages]; cache_len: int [B]
    (counts the s_active current tokens); sinks: None or [Hq] sink logits.
    Returns o [len(batches), s_active, Hq, D] (and lse [len(batches), s_active, Hq]).
    """
    B, sa, Hq, D = q.shape
    batches = range(B) if batches is None else batches
    conv = to_f64 if to_f64 is not None else (lambda a: np.asarray(a, dtype=np.float64))
    outs, lses = [], []
    for b in batches:
        L = int(cache_len[b])
        kb = conv(gather_paged(k_pool, block_table[b], L))[None]
        vb = conv(gather_paged(v_pool, block_table[b], L))[None]
        o, lse = attention(np.ascontiguousarray(q[b : b + 1]), np.ascontiguousarray(kb),
                           np.ascontiguousarray(vb), scale, causal=True, window=window, return_lse=True,
                           sinks=sinks)
        outs.append(o[0])
        lses.append(lse[0])
    o = np.stack(outs) if outs else np.zeros((0, sa, Hq, D))
    lse = np.stack(lses) if lses else np.zeros((0, sa, Hq))
    return (o, lse) if return_lse else o

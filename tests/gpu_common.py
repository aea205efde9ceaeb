"""Helpers for the GPU parity tests: run the HIP path through the C ABI on
seeded inputs and compare with the fp64 oracle on the same rounded inputs.

Tolerances (written here once, used by every parity test):
  * f16 / bf16 outputs: max-abs error <= 2e-2 and mean-abs error <= 2e-3 over
    all compared elements, against the oracle in fp64;
  * f32 output: normwise relative error max|o - r| / max|r| <= 1e-5;
  * f16 / bf16 outputs, where a test passes the oracle's bound (see
    derived_bound): every element within the error bound that the kernels'
    arithmetic allows for that element.

Every comparison appends its achieved errors (max-abs, mean-abs, the largest
per-row normwise relative error and the largest error / bound ratio) to a
JSON-lines log, gpurun_out/parity_margins.jsonl by default (ATTN_PARITY_LOG
names another file; an empty value turns it off).
"""
from __future__ import annotations

import json
import math
import os
import sys

import numpy as np
import pytest

import oracle
from flash_attention_forward_amd import workloads as W

LOWP_MAX_ABS = 2e-2
LOWP_MEAN_ABS = 2e-3
F32_NORMWISE = 1e-5


def torch_cuda():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch


def say(*a):
    """Name the case before each GPU step, so a lost run still says what ran."""
    print(*a, flush=True, file=sys.stderr)


def errors(got: np.ndarray, ref: np.ndarray):
    e = np.abs(got - ref)
    return float(e.max(initial=0.0)), float(e.mean()) if e.size else 0.0


def row_normwise(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per output row (last axis): max|o - r| / max|r| (the absolute error where the row is all zeros)."""
    err = np.abs(got - ref).max(axis=-1, initial=0.0)
    scale = np.abs(ref).max(axis=-1, initial=0.0)
    return np.where(scale > 0, err / np.where(scale > 0, scale, 1.0), err)


_REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def log_margins(record: dict) -> None:
    """Append one comparison's achieved errors to the margins log (JSON lines)."""
    path = os.environ.get("ATTN_PARITY_LOG", os.path.join(_REPO, "gpurun_out", "parity_margins.jsonl"))
    if not path:
        return
    record = dict(record, test=os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0])
    try:
        os.makedirs(os.path.dirname(path) or ".", exist_ok=True)
        with open(path, "a") as f:
            f.write(json.dumps(record) + "\n")
    except OSError:
        pass


def check(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "", bound: np.ndarray | None = None):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    rows = row_normwise(got, ref) if got.size else np.zeros(0)
    rec = {"what": what, "dtype": dtype, "elements": int(got.size),
           "row_normwise_max": float(rows.max(initial=0.0))}
    if dtype == "f32":
        scale = np.abs(ref).max(initial=0.0)
        err = np.abs(got - ref).max(initial=0.0)
        rel = err / scale if scale > 0 else err
        log_margins(dict(rec, normwise=float(rel), gate=F32_NORMWISE))
        assert rel <= F32_NORMWISE, f"{what}: normwise rel err {rel:.3e}"
        return rel
    mx, mean = errors(got, ref)
    rec.update(max_abs=mx, mean_abs=mean)
    ratio = None
    if bound is not None:
        assert bound.shape == got.shape, (bound.shape, got.shape)
        err = np.abs(got - ref)
        # where the bound is 0 (no visible key: zeros exactly) the error must be 0 too
        ratio = float(np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), np.where(err > 0, np.inf, 0.0))
                      .max(initial=0.0))
        rec.update(bound_ratio_max=ratio)
    log_margins(rec)
    assert mx <= LOWP_MAX_ABS and mean <= LOWP_MEAN_ABS, f"{what}: max-abs {mx:.3e} mean-abs {mean:.3e}"
    if ratio is not None:
        assert ratio <= 1.0, f"{what}: error {ratio:.3f} x the derived per-element bound"
    return mx, mean


# ----------------------------------------------------------------------------- derived error bound
# Unit roundoff of the 16-bit types (round to nearest even, 8 and 11 significand bits).
UNIT_ROUNDOFF = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}
LOG2E = 1.4426950408889634


def derived_bound(ref, ref_absv, n_keys, qk_norms, c, dtype, vmax):
    """Per-element bound on |kernel - oracle| for a f16/bf16 output, from the kernels' arithmetic.

    The kernels compute O = sum_j P~_j v_j / sum_j P~_j, with P~_j = p_j (1 + d_j)
    the probability rounded to the 16-bit type once (the same P~ feeds both
    sums), f32 accumulation, and one final rounding of O. With w_j the exact
    softmax weights and A = sum_j w_j |v_j| (the oracle applied to |V|):
      * output rounding: u |r|;
      * the rounded weights: |sum_j w_j v_j (d_j - mean_w d)| / (1 + mean_w d)
        <= 2 delta (1 + delta) A, where |d_j| <= delta = u + 2^-21 (exp2 and
        fma in f32) + the f32 error of the score itself, ln 2 * c * (D + 2) *
        2^-23 * |q| |k|_max (its exponent error, c = |scale| log2 e);
      * f32 sums of up to n_keys products and probabilities: (n_keys + 64) *
        2^-23 * A (each add may round by 2^-23 relative; the extra 64 covers
        the rescales, the 1/l product and the split merge of decode);
      * f16 only: probabilities below 2^-14 are subnormal, with an absolute
        error up to 2^-25 each while the sum of P~ is at least 1: n_keys *
        2^-24 * max|v|.
    The sum of the terms, times 1.1 for second-order products, is the bound.
    Arrays: ref, ref_absv [..., D]; n_keys, qk_norms, vmax [...] (broadcast)."""
    u = UNIT_ROUNDOFF[dtype]
    d = ref.shape[-1]
    n_keys = np.asarray(n_keys, dtype=np.float64)
    delta = u + 2.0 ** -21 + math.log(2.0) * c * (d + 2) * 2.0 ** -23 * np.asarray(qk_norms, np.float64)
    coef = 2.0 * delta * (1.0 + delta) + (n_keys + 64.0) * 2.0 ** -23
    bound = u * np.abs(ref) + coef[..., None] * ref_absv
    if dtype == "f16":
        bound = bound + (n_keys * 2.0 ** -24 * np.asarray(vmax, np.float64))[..., None]
    return 1.1 * bound


def attention_with_bound(q64, k64, v64, scale: float, causal: bool, window: int, dtype: str, rows=None, sinks=None,
                         positions=None):
    """Oracle rows (all rows by default) and their derived_bound for a kernel output of `dtype`.
    q64 [B, Sq, Hq, D], k64 / v64 [B, Skv, Hkv, D] float64; rows [n, 3] of (b, i, h).
    Returns (ref, bound), shaped [n, D] with rows given, else [B, Sq, Hq, D]."""
    B, Sq, Hq, D = q64.shape
    Skv, Hkv = k64.shape[1], k64.shape[2]
    full = rows is None
    if full:
        rows = oracle.all_rows(B, Sq, Hq)
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    ref, _ = oracle.attention_rows(q64, k64, v64, scale, causal, window, rows, sinks, positions)
    ref_abs, _ = oracle.attention_rows(q64, k64, np.abs(v64), scale, causal, window, rows, sinks, positions)
    b, i, h = rows[:, 0], rows[:, 1], rows[:, 2]
    hk = h // (Hq // Hkv)
    pos = np.asarray(positions, dtype=np.int64)[i] if positions is not None else i + (Skv - Sq)
    hi = np.minimum(Skv - 1, pos) if causal else np.full_like(pos, Skv - 1)
    lo = np.maximum(0, pos - window + 1) if window > 0 else np.zeros_like(pos)
    n_keys = np.maximum(0, hi - lo + 1)
    if Skv > 0:
        kn = np.sqrt((k64 * k64).sum(axis=-1)).max(axis=1)  # [B, Hkv]
        vmax = np.abs(v64).max(axis=(1, 3))               # [B, Hkv]
        qk = np.linalg.norm(q64[b, i, h], axis=-1) * kn[b, hk]
        vm = vmax[b, hk]
    else:
        qk = vm = np.zeros(len(rows))
    bound = derived_bound(ref, ref_abs, n_keys, qk, abs(scale) * LOG2E, dtype, vm)
    if full:
        return ref.reshape(B, Sq, Hq, D), bound.reshape(B, Sq, Hq, D)
    return ref, bound


def dev(a: np.ndarray, dtype: str):
    return W.to_torch(a, dtype, "cuda")


def host64(t, dtype: str) -> np.ndarray:
    return W.as_f64(W.from_torch(t, dtype), dtype)


# ----------------------------------------------------------------------------- prefill
def gpu_prefill(inp: W.PrefillInputs, **over):
    """Run attn_prefill_fwd on inp; returns the output as float64 [B, Sq, Hq, D]."""
    import flash_attention_forward_amd as F

    torch = torch_cuda()
    s = inp.spec
    q, k, v = dev(inp.q, s.dtype), dev(inp.k, s.dtype), dev(inp.v, s.dtype)
    o = torch.empty_like(q)
    F.attn_prefill_fwd(q, k, v, o, over.get("scale", s.scale_f32), over.get("causal", s.causal),
                       over.get("window", s.window))
    torch.cuda.synchronize()
    return host64(o, s.dtype)


def prefill_with_bound(inp: W.PrefillInputs, rows=None, **over):
    """oracle_prefill and its derived_bound (16-bit outputs)."""
    s = inp.spec
    q, k, v = W.as_f64(inp.q, s.dtype), W.as_f64(inp.k, s.dtype), W.as_f64(inp.v, s.dtype)
    return attention_with_bound(q, k, v, over.get("scale", s.scale_f32), over.get("causal", s.causal),
                                over.get("window", s.window), s.dtype, rows=rows)


def oracle_prefill(inp: W.PrefillInputs, rows=None, **over):
    s = inp.spec
    q, k, v = W.as_f64(inp.q, s.dtype), W.as_f64(inp.k, s.dtype), W.as_f64(inp.v, s.dtype)
    args = (over.get("scale", s.scale_f32), over.get("causal", s.causal), over.get("window", s.window))
    if rows is None:
        return oracle.attention(q, k, v, *args)
    return oracle.attention_rows(q, k, v, *args, rows)[0]


def sample_rows(spec, n_random: int, seed: int = 0) -> np.ndarray:
    """(b, i, h) rows: tile boundaries, first/last rows, every head, plus random rows."""
    B, Sq, Hq = spec.batch, spec.seqlen_q, spec.n_q_heads
    edge = {0, 1, 31, 32, 63, 64, 127, 128, 129, Sq // 2, Sq - 129, Sq - 128, Sq - 65, Sq - 64, Sq - 33, Sq - 1}
    edge = sorted(i for i in edge if 0 <= i < Sq)
    rows = [(b, i, h) for b in range(B) for i in edge for h in range(Hq)]
    rng = np.random.default_rng(seed)
    rows += [(int(rng.integers(B)), int(rng.integers(Sq)), int(rng.integers(Hq))) for _ in range(n_random)]
    return np.array(rows, dtype=np.int64)


# ----------------------------------------------------------------------------- decode
def decode_tensors(inp: W.DecodeInputs):
    torch = torch_cuda()
    s = inp.spec
    return dict(
        q=dev(inp.q, s.dtype),
        k=dev(inp.k_pool, s.dtype),
        v=dev(inp.v_pool, s.dtype),
        cache_len=torch.from_numpy(inp.cache_len.astype(np.int32)).cuda(),
        block_table=torch.from_numpy(inp.block_table.view(np.int32)).cuda(),
    )


def gpu_decode(inp: W.DecodeInputs, split_len: int = 512, paged: bool = True, window: int = 0, tensors=None):
    import flash_attention_forward_amd as F

    torch = torch_cuda()
    s = inp.spec
    t = tensors or decode_tensors(inp)
    o = F.decode(t["q"], t["k"], t["v"], t["cache_len"], block_table=t["block_table"] if paged else None,
                 scale=s.scale_f32, window=window, split_len=split_len,
                 max_len=s.max_pages_per_seq * s.page_size)
    torch.cuda.synchronize()
    return host64(o, s.dtype)


def oracle_decode(inp: W.DecodeInputs, batches=None, window: int = 0):
    s = inp.spec
    f64 = lambda a: W.as_f64(a, s.dtype)
    return oracle.decode(f64(inp.q), inp.k_pool, inp.v_pool, inp.block_table, inp.cache_len, s.scale_f32,
                         window=window, batches=batches, to_f64=f64)


def decode_with_bound(inp: W.DecodeInputs, batches=None, window: int = 0, sinks=None):
    """Oracle decode output [len(batches), s_active, Hq, D] and its derived_bound: each sequence's
    logical K/V gathered through the page table (oracle.gather_paged), then attention_with_bound
    with the queries at the end of the cache. FP8 pools are widened and scaled as the cache defines."""
    s = inp.spec
    if s.cache_dtype == "fp8":
        kv64 = lambda a, sc: np.float64(np.float32(sc)) * W.as_f64(a, "fp8")
    else:
        kv64 = lambda a, sc: W.as_f64(a, s.cache_dtype)
    batches = range(s.batch) if batches is None else batches
    refs, bounds = [], []
    for b in batches:
        L = int(inp.cache_len[b])
        kb = kv64(oracle.gather_paged(inp.k_pool, inp.block_table[b], L), s.k_scale)[None]
        vb = kv64(oracle.gather_paged(inp.v_pool, inp.block_table[b], L), s.v_scale)[None]
        r, bd = attention_with_bound(W.as_f64(inp.q[b:b + 1], s.dtype), kb, vb, s.scale_f32, True, window, s.dtype,
                                     sinks=sinks)
        refs.append(r[0])
        bounds.append(bd[0])
    return np.stack(refs), np.stack(bounds)

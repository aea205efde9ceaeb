"""Helpers for the GPU parity tests: run the HIP path through the C ABI on
seeded inputs and compare with the fp64 oracle on the same rounded inputs.

Tolerances (written here once, used by every parity test):
  * f16 / bf16 outputs: max-abs error <= 2e-2 and mean-abs error <= 2e-3 over
    all compared elements, against the oracle in fp64;
  * f32 output: normwise relative error max|o - r| / max|r| <= 1e-5.
"""
from __future__ import annotations

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


def check(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    if dtype == "f32":
        scale = np.abs(ref).max(initial=0.0)
        err = np.abs(got - ref).max(initial=0.0)
        rel = err / scale if scale > 0 else err
        assert rel <= F32_NORMWISE, f"{what}: normwise rel err {rel:.3e}"
        return rel
    mx, mean = errors(got, ref)
    assert mx <= LOWP_MAX_ABS and mean <= LOWP_MEAN_ABS, f"{what}: max-abs {mx:.3e} mean-abs {mean:.3e}"
    return mx, mean


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

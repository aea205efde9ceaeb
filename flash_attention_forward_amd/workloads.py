"""Seeded synthetic inputs for the attention workloads.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the attention arithmetic, so both the fp64 oracle (tests)
and the HIP path (tests, bench) can take their inputs from it.

Distributions follow the workloads described on the pages: i.i.d. N(0,1)
queries/keys/values, rounded to the storage dtype with round-to-nearest-even.
The random generator is numpy's PCG64 ``default_rng(seed)`` drawing float32
normals; the draw order is fixed per workload kind:

* prefill: q, k, v (each ``[B, S, H, D]``), then the key "spike" positions;
* decode:  cache_len, the page permutation, the K pool, the V pool, then q.

Storage arrays are numpy: ``uint16`` bit patterns for bf16/f16, ``uint8``
bit patterns for fp8 (OCP FP8 E4M3, "e4m3fn": 1 sign, 4 exponent bits with
bias 7, 3 mantissa bits, subnormals, no infinities, NaN = S.1111.111, largest
finite value 448) and ``float32`` for fp32. ``as_f64`` widens a storage array
exactly to float64.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np

DTYPES = ("f32", "f16", "bf16", "fp8")
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}


# --------------------------------------------------------------------------- fp8 (E4M3, OCP "fn" variant)
def _e4m3_values() -> np.ndarray:
    """float64 value of each of the 256 codes (NaN for the two NaN codes), from the format definition."""
    c = np.arange(256)
    e, m = (c >> 3) & 15, (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e.astype(np.float64) - 7.0))
    val = np.where(c & 0x80, -mag, mag)
    val[(c & 0x7F) == 0x7F] = np.nan
    return val


E4M3_VALUES = _e4m3_values()
E4M3_MAX = 448.0


def f32_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to E4M3 (round-to-nearest-even), saturating at +-448; NaN -> 0x7F.
    Large arrays go through torch's CPU conversion after clamping to +-448 (the same rounding:
    the two are compared value by value in the tests); the rest follow the definition below."""
    if np.size(x) >= 1 << 20:
        import torch

        xc = np.clip(np.ascontiguousarray(x, dtype=np.float32), -E4M3_MAX, E4M3_MAX)
        code = torch.from_numpy(xc).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        nan = np.isnan(xc)
        if nan.any():
            code[nan] = 0x7F
        return code
    return f32_to_e4m3_bits_by_definition(x)


def f32_to_e4m3_bits_by_definition(x: np.ndarray) -> np.ndarray:
    """Round float32 to E4M3 (round-to-nearest-even), saturating at +-448; NaN -> 0x7F.
    Returns the 8-bit patterns. Normal results (|x| >= 2^-6) keep 3 of the 23 float32 mantissa
    bits with the usual add-and-shift RNE (a carry moves into the exponent), rebiased from 127 to
    7; smaller magnitudes are multiples of 2^-9, rounded with np.rint (ties to even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    a = np.minimum(bits & np.uint32(0x7FFFFFFF), np.uint32(0x43E00000))  # |x|, saturated at 448
    r = (a >> np.uint32(20)) & np.uint32(1)
    r += np.uint32(0x7FFFF)
    r += a
    r >>= np.uint32(20)
    r -= np.uint32(120 << 3)  # exponent bias 127 -> 7: now the [exp:mant] code (wraps below 2^-6; unused there)
    sub = a < np.uint32(0x3C800000)
    if sub.any():  # multiples of 2^-9
        r[sub] = np.rint(a[sub].view(np.float32) * np.float32(512.0)).astype(np.uint32)
    code = r.astype(np.uint8)
    code |= (bits >> np.uint32(24)).astype(np.uint8) & np.uint8(0x80)
    nan = np.isnan(x)
    if nan.any():
        code[nan] = 0x7F
    return code


# --------------------------------------------------------------------------- rounding
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round-to-nearest-even); return the 16-bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    b = b + (np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1)))
    return (b >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to IEEE half (numpy's conversion is round-to-nearest-even)."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 array -> storage array of ``dtype``."""
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f16":
        return f32_to_f16_bits(x)
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "fp8":
        return f32_to_e4m3_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def as_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array -> float32 (exact)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a)
    if dtype == "f16":
        return np.ascontiguousarray(a, dtype=np.uint16).view(np.float16).astype(np.float32)
    if dtype == "fp8":
        return E4M3_VALUES[np.asarray(a, dtype=np.uint8)].astype(np.float32)
    return np.asarray(a, dtype=np.float32)


def as_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array -> float64 (exact)."""
    return as_f32(a, dtype).astype(np.float64)


def to_torch(a: np.ndarray, dtype: str, device=None):
    """Storage array -> torch tensor of the matching dtype (same bits)."""
    import torch

    if dtype == "f32":
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    elif dtype == "fp8":
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).view(torch.float8_e4m3fn)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16))
        t = t.view(torch.bfloat16 if dtype == "bf16" else torch.float16)
    return t.to(device) if device is not None else t


def from_torch(t, dtype: str) -> np.ndarray:
    """torch tensor (on any device) -> storage array (same bits)."""
    import torch

    t = t.detach().to("cpu").contiguous()
    if dtype == "f32":
        return t.numpy().astype(np.float32, copy=False)
    if dtype == "fp8":
        return t.view(torch.uint8).numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


def normal_f32(rng: np.random.Generator, shape, chunk: int = 1 << 26) -> np.ndarray:
    """float32 N(0,1) draws, generated in chunks (same stream as one draw)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = rng.standard_normal(e - s, dtype=np.float32)
    return out.reshape(shape)


def normal_rounded(rng: np.random.Generator, shape, dtype: str, chunk: int = 1 << 24,
                   divide_by: float = 1.0) -> np.ndarray:
    """N(0,1) draws (divided by ``divide_by``) rounded to ``dtype``, chunked so no full float32 copy
    is held."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype={"f32": np.float32, "fp8": np.uint8}.get(dtype, np.uint16))
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        x = rng.standard_normal(e - s, dtype=np.float32)
        if divide_by != 1.0:
            x /= np.float32(divide_by)
        out[s:e] = round_to(x, dtype)
    return out.reshape(shape)


# --------------------------------------------------------------------------- prefill
@dataclass(frozen=True)
class PrefillSpec:
    batch: int
    n_q_heads: int
    n_kv_heads: int
    seqlen_q: int
    seqlen_kv: int
    head_dim: int
    dtype: str
    causal: bool
    window: int = 0
    scale: float | None = None  # None -> 1/sqrt(head_dim), rounded to float32
    spike_frac: float = 0.0  # fraction of key positions whose K row is doubled
    spike_factor: float = 2.0

    @property
    def scale_f32(self) -> float:
        s = 1.0 / math.sqrt(self.head_dim) if self.scale is None else self.scale
        return float(np.float32(s))


@dataclass
class PrefillInputs:
    spec: PrefillSpec
    q: np.ndarray  # [B, Sq, Hq, D] storage
    k: np.ndarray  # [B, Skv, Hkv, D]
    v: np.ndarray
    spike_positions: np.ndarray = field(default_factory=lambda: np.zeros((0, 0), np.int64))


def make_prefill(spec: PrefillSpec, seed: int) -> PrefillInputs:
    rng = np.random.default_rng(seed)
    B, Sq, Skv, D = spec.batch, spec.seqlen_q, spec.seqlen_kv, spec.head_dim
    q = normal_rounded(rng, (B, Sq, spec.n_q_heads, D), spec.dtype)
    if spec.spike_frac > 0:
        kf = normal_f32(rng, (B, Skv, spec.n_kv_heads, D))
    else:
        k = normal_rounded(rng, (B, Skv, spec.n_kv_heads, D), spec.dtype)
    v = normal_rounded(rng, (B, Skv, spec.n_kv_heads, D), spec.dtype)
    spikes = np.zeros((B, 0), np.int64)
    if spec.spike_frac > 0:
        n = int(math.floor(spec.spike_frac * Skv))
        spikes = np.stack([np.sort(rng.choice(Skv, size=n, replace=False)) for _ in range(B)])
        for b in range(B):
            kf[b, spikes[b]] *= np.float32(spec.spike_factor)
        k = round_to(kf, spec.dtype)
        del kf
    return PrefillInputs(spec, q, k, v, spikes)


# --------------------------------------------------------------------------- packed sequences
@dataclass(frozen=True)
class VarlenSpec:
    """Packed sequences: lengths drawn per sequence; each sequence's keys are a
    prefix of prefix_lo..prefix_hi cached tokens followed by its query tokens."""
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str
    causal: bool
    len_lo: int
    len_hi: int
    window: int = 0
    prefix_lo: int = 0
    prefix_hi: int = 0
    scale: float | None = None

    @property
    def scale_f32(self) -> float:
        s = 1.0 / math.sqrt(self.head_dim) if self.scale is None else self.scale
        return float(np.float32(s))


@dataclass
class VarlenInputs:
    spec: VarlenSpec
    lens_q: np.ndarray    # [B] int64
    lens_kv: np.ndarray   # [B] int64
    cu_q: np.ndarray      # [B + 1] int64 cumulative offsets
    cu_kv: np.ndarray
    q: np.ndarray         # [total_q, Hq, D] storage
    k: np.ndarray         # [total_kv, Hkv, D]
    v: np.ndarray


def make_varlen(spec: VarlenSpec, seed: int, lens_q=None, prefixes=None) -> VarlenInputs:
    """Draw order: q lengths U{len_lo..len_hi}, prefix lengths U{prefix_lo..prefix_hi}, q, k, v
    (explicit lens_q / prefixes replace the draws)."""
    rng = np.random.default_rng(seed)
    B = spec.batch
    lq = rng.integers(spec.len_lo, spec.len_hi + 1, size=B) if lens_q is None else np.asarray(lens_q)
    pre = rng.integers(spec.prefix_lo, spec.prefix_hi + 1, size=B) if prefixes is None else np.asarray(prefixes)
    lq = lq.astype(np.int64)
    lk = lq + pre.astype(np.int64)
    cq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int64)
    ck = np.concatenate([[0], np.cumsum(lk)]).astype(np.int64)
    q = normal_rounded(rng, (int(cq[-1]), spec.n_q_heads, spec.head_dim), spec.dtype)
    k = normal_rounded(rng, (int(ck[-1]), spec.n_kv_heads, spec.head_dim), spec.dtype)
    v = normal_rounded(rng, (int(ck[-1]), spec.n_kv_heads, spec.head_dim), spec.dtype)
    return VarlenInputs(spec, lq, lk, cq, ck, q, k, v)


def varlen_visible_pairs(inp: VarlenInputs) -> int:
    """Visible (query, key) pairs per q-head, summed over the sequences (bottom-right alignment)."""
    s = inp.spec
    tot = 0
    for Lq, Lk in zip(inp.lens_q.tolist(), inp.lens_kv.tolist()):
        for i in range(Lq):
            pos = i + Lk - Lq
            hi = min(Lk, pos + 1) if s.causal else Lk
            lo = max(0, pos - s.window + 1) if s.window > 0 else 0
            tot += max(0, hi - lo)
    return tot


# --------------------------------------------------------------------------- decode
@dataclass(frozen=True)
class DecodeSpec:
    batch: int
    s_active: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str
    page_size: int
    len_lo: int
    len_hi: int
    scale: float | None = None
    extra_pages: int = 0  # physical pages no sequence references
    kv_dtype: str = ""  # storage of the K/V pools; "" = dtype (q and the output are always dtype)
    k_scale: float = 1.0  # fp8 caches: the K row a code stands for is k_scale * its value
    v_scale: float = 1.0

    @property
    def cache_dtype(self) -> str:
        return self.kv_dtype or self.dtype

    @property
    def scale_f32(self) -> float:
        s = 1.0 / math.sqrt(self.head_dim) if self.scale is None else self.scale
        return float(np.float32(s))

    @property
    def max_pages_per_seq(self) -> int:
        return -(-self.len_hi // self.page_size)


@dataclass
class DecodeInputs:
    spec: DecodeSpec
    cache_len: np.ndarray  # int32 [B]
    block_table: np.ndarray  # uint32 [B, max_pages_per_seq]
    k_pool: np.ndarray  # [num_pages, page_size, Hkv, D] storage
    v_pool: np.ndarray
    q: np.ndarray  # [B, s_active, Hq, D]


def make_decode(spec: DecodeSpec, seed: int, unused_entry: int = 0) -> DecodeInputs:
    rng = np.random.default_rng(seed)
    B, ps = spec.batch, spec.page_size
    cache_len = rng.integers(spec.len_lo, spec.len_hi, B, endpoint=True).astype(np.int32)
    npages = -(-cache_len.astype(np.int64) // ps)
    total = int(npages.sum()) + spec.extra_pages
    perm = rng.permutation(total).astype(np.uint32)
    maxp = spec.max_pages_per_seq
    table = np.full((B, maxp), unused_entry, dtype=np.uint32)
    off = 0
    for b in range(B):
        table[b, : npages[b]] = perm[off : off + npages[b]]
        off += int(npages[b])
    shape = (total, ps, spec.n_kv_heads, spec.head_dim)
    if spec.cache_dtype == "fp8":  # N(0,1) in the units the cache represents, stored as x / scale
        k_pool = normal_rounded(rng, shape, "fp8", divide_by=spec.k_scale)
        v_pool = normal_rounded(rng, shape, "fp8", divide_by=spec.v_scale)
    else:
        k_pool = normal_rounded(rng, shape, spec.cache_dtype)
        v_pool = normal_rounded(rng, shape, spec.cache_dtype)
    q = normal_rounded(rng, (B, spec.s_active, spec.n_q_heads, spec.head_dim), spec.dtype)
    return DecodeInputs(spec, cache_len, table, k_pool, v_pool, q)


# --------------------------------------------------------------------------- the five workloads
WORKLOADS = {
    # 1 head, 256 x 256, D=64, fp32, full (non-causal) softmax
    "fp32_d64_s256": PrefillSpec(1, 1, 1, 256, 256, 64, "f32", causal=False, scale=1.0 / 8.0),
    # 7B-shaped causal GQA prefill: 28 q-heads over 4 kv-heads, 2048 tokens, D=128, f16
    "f16_gqa7_causal_2k": PrefillSpec(1, 28, 4, 2048, 2048, 128, "f16", causal=True),
    # long-context causal prefill: 8 q-heads over 1 kv-head, 32768 tokens, bf16, 1% K spikes x2
    "bf16_causal_32k": PrefillSpec(1, 8, 1, 32768, 32768, 128, "bf16", causal=True, spike_frac=0.01),
    # head_dim 256 with a 1024-token sliding window on top of causal, B=2, 16 q over 8 kv heads
    "bf16_swa1024_d256_8k": PrefillSpec(2, 16, 8, 8192, 8192, 256, "bf16", causal=True, window=1024),
    # paged decode: 32 sequences, 1 query token, 32 q over 8 kv heads, 16-token pages
    "paged_decode_b32_d128": DecodeSpec(32, 1, 32, 8, 128, "bf16", page_size=16, len_lo=1024, len_hi=32768),
}

# The paged-decode workload with its K/V cache in FP8 E4M3 (q and the output stay bf16).
FP8_DECODE = replace(WORKLOADS["paged_decode_b32_d128"], kv_dtype="fp8")

WORKLOAD_SEEDS = {name: 1001 + i for i, name in enumerate(WORKLOADS)}

# Packed-sequence prefill (per-row dynamic bounds): the 7B-shaped heads of the
# 2K context workload over 16 packed prompts of 256..4096 tokens.
VARLEN = "bf16_varlen_gqa7_b16"
VARLEN_SPEC = VarlenSpec(16, 28, 4, 128, "bf16", causal=True, len_lo=256, len_hi=4096)
VARLEN_SEED = 1006


def shrink(spec, **kw):
    """Same workload structure at other sizes (for tests)."""
    return replace(spec, **kw)

# Per-tensor scales (K, V) when the 32K causal workload's K and V are stored as FP8 E4M3: each
# value is divided by its scale and rounded, so E4M3's largest code (448) stands for 14 (K, whose
# spiked rows reach about 11) and 7 (V, N(0,1) draws).
FP8_PREFILL_SCALES = (1.0 / 32.0, 1.0 / 64.0)

"""Whole-tile schedule of the prefill at full size, and run-to-run determinism.

Tile census. With Q = 0 every score is 0, so each row's softmax is uniform over
its visible keys and o_i = the mean of V over them (the oracle's closed form
for a zero query: pinned on the CPU in tests/test_oracle_pins.py). V is a
one-hot code of each key's 64-key tile, v[j, d] = 1 iff d = (j // 64) mod D,
so o_i[d] counts the visible keys of the tiles of class d, divided by the
row's number of visible keys. A tile that the schedule drops, repeats or
misplaces changes that count by up to 64 in a class of at most a few hundred
keys, far beyond rounding. With all probabilities exactly 1 the kernels' sums
are exact integers; only 1/l and the final rounding remain, so every element
must lie within (u + 2^-22) relative of the oracle (u: the unit roundoff of
the output type) and be exactly 0 where the oracle gives 0. Compared on every
row of the launches the full-size workloads take (CTE page, "Algorithm —
compute-skip": whole tiles that no row sees are skipped, the rest run once).

Determinism. The hot launches repeated 50 times give bit-identical outputs:
the minfer "03 · 8n" page (sections "4. Verification" and "6. Lessons")
records a shared-memory race that only a repeated-run harness caught.
"""
import numpy as np
import pytest

import oracle
from flash_attention_forward_amd import workloads as W

from gpu_common import UNIT_ROUNDOFF, decode_tensors, log_margins, say, torch_cuda

pytestmark = pytest.mark.gpu

WL = W.WORKLOADS


def census_v(n_keys: int, d: int) -> np.ndarray:
    """[n_keys, d] one-hot tile code: 1 at d = (j // 64) % D."""
    v = np.zeros((n_keys, d), np.float32)
    v[np.arange(n_keys), (np.arange(n_keys) // 64) % d] = 1.0
    return v


def census_expected(sq: int, skv: int, d: int, causal: bool, window: int) -> np.ndarray:
    """[sq, d]: the mean of census_v over each row's visible keys (bottom-right alignment), from
    prefix counts per class: count of keys j in [lo, hi] with (j // 64) % D == c, over the count."""
    cls = (np.arange(skv) // 64) % d
    pref = np.zeros((d, skv + 1), np.int64)
    for c in range(d):
        pref[c, 1:] = np.cumsum(cls == c)
    pos = np.arange(sq) + (skv - sq)
    hi = np.minimum(skv - 1, pos) if causal else np.full(sq, skv - 1)
    lo = np.maximum(0, pos - window + 1) if window > 0 else np.zeros(sq, np.int64)
    n = np.maximum(0, hi - lo + 1)
    cnt = (pref[:, np.clip(hi + 1, 0, skv)] - pref[:, np.clip(lo, 0, skv)]).T  # [sq, d]
    cnt = np.where((n > 0)[:, None], cnt, 0)
    return cnt / np.maximum(n, 1)[:, None]


def check_census(got, exp, dtype, what):
    """got [B, Sq, H, D] vs exp [Sq, D] (the same for every batch and head)."""
    u = UNIT_ROUNDOFF[dtype]
    err = np.abs(got - exp[None, :, None, :])
    lim = (u + 2.0 ** -22) * np.abs(exp)[None, :, None, :]
    bad = err > lim
    log_margins({"what": what, "dtype": dtype, "elements": int(got.size), "census_max_abs": float(err.max()),
                 "census_ratio_max": float(np.where(lim > 0, err / np.where(lim > 0, lim, 1),
                                                    np.where(err > 0, np.inf, 0.0)).max())})
    assert not bad.any(), (what, np.argwhere(bad)[:5], err[bad][:5])


CENSUS = {
    "f16_gqa7_causal_2k": WL["f16_gqa7_causal_2k"],
    "bf16_causal_32k": WL["bf16_causal_32k"],
    "bf16_swa1024_d256_8k": WL["bf16_swa1024_d256_8k"],
    "wave8_d64_f16_window_4k": W.PrefillSpec(2, 16, 2, 4096, 4096, 64, "f16", causal=True, window=300),
    "wave8_d128_sq_lt_skv": W.PrefillSpec(8, 16, 4, 1024, 3000, 128, "bf16", causal=True),
}


@pytest.mark.parametrize("name", list(CENSUS))
def test_tile_census_full_size(name):
    torch = torch_cuda()
    import flash_attention_forward_amd as F

    spec = CENSUS[name]
    B, Sq, Skv, Hq, Hkv, D, dt = (spec.batch, spec.seqlen_q, spec.seqlen_kv, spec.n_q_heads, spec.n_kv_heads,
                                   spec.head_dim, spec.dtype)
    rng = np.random.default_rng(31)
    q = torch.zeros((B, Sq, Hq, D), dtype=torch.bfloat16 if dt == "bf16" else torch.float16, device="cuda")
    k = W.to_torch(W.normal_rounded(rng, (B, Skv, Hkv, D), dt), dt, "cuda")
    vc = census_v(Skv, D)
    v = W.to_torch(W.round_to(np.broadcast_to(vc[None, :, None, :], (B, Skv, Hkv, D)).copy(), dt), dt, "cuda")
    say("tile census", name)
    o = F.prefill(q, k, v, scale=spec.scale_f32, causal=spec.causal, window=spec.window)
    torch.cuda.synchronize()
    got = W.as_f64(W.from_torch(o, dt), dt)
    exp = census_expected(Sq, Skv, D, spec.causal, spec.window)
    # the closed form is the oracle's value: checked on rows spread over the sequence
    rows = np.array([(0, i, 0) for i in np.unique(np.linspace(0, Sq - 1, 40).astype(np.int64))])
    ref, _ = oracle.attention_rows(np.zeros((1, Sq, 1, D)), np.zeros((1, Skv, 1, D)),
                                   vc.astype(np.float64)[None, :, None, :], spec.scale_f32, spec.causal,
                                   spec.window, rows)
    np.testing.assert_allclose(ref, exp[rows[:, 1]], rtol=1e-13, atol=0)
    check_census(got, exp, dt, name)


def test_tile_census_packed_sequences():
    """The census on the packed-prompt workload's launch (16 causal prompts of 256..4096 tokens)."""
    torch = torch_cuda()
    import flash_attention_forward_amd as F

    spec = W.VARLEN_SPEC
    inp = W.make_varlen(spec, W.VARLEN_SEED)
    D = spec.head_dim
    q = torch.zeros((int(inp.cu_q[-1]), spec.n_q_heads, D), dtype=torch.bfloat16, device="cuda")
    k = W.to_torch(inp.k, "bf16", "cuda")
    vals = np.concatenate([census_v(int(n), D) for n in inp.lens_kv])
    v = W.to_torch(W.round_to(np.broadcast_to(vals[:, None, :], inp.v.shape).copy(), "bf16"), "bf16", "cuda")
    o = torch.empty_like(q)
    cq = torch.from_numpy(inp.cu_q.astype(np.int32)).cuda()
    ck = torch.from_numpy(inp.cu_kv.astype(np.int32)).cuda()
    say("tile census, packed")
    F.attn_prefill_varlen_fwd(q, k, v, o, cq, ck, int(inp.lens_q.max()), int(inp.lens_kv.max()), spec.scale_f32,
                              True)
    torch.cuda.synchronize()
    got = W.as_f64(W.from_torch(o, "bf16"), "bf16")
    for b in range(spec.batch):
        q0, q1 = int(inp.cu_q[b]), int(inp.cu_q[b + 1])
        exp = census_expected(q1 - q0, int(inp.lens_kv[b]), D, True, 0)
        check_census(got[None, q0:q1], exp, "bf16", f"packed sequence {b}")


def test_tile_census_fp8_kv_32k():
    """The census on the 32K workload's launch with K and V stored as FP8 E4M3 (1.0 is exact)."""
    torch = torch_cuda()
    import flash_attention_forward_amd as F

    spec = WL["bf16_causal_32k"]
    B, Sq, Skv, Hq, Hkv, D = spec.batch, spec.seqlen_q, spec.seqlen_kv, spec.n_q_heads, spec.n_kv_heads, spec.head_dim
    rng = np.random.default_rng(32)
    q = torch.zeros((B, Sq, Hq, D), dtype=torch.bfloat16, device="cuda")
    k8 = W.to_torch(W.normal_rounded(rng, (B, Skv, Hkv, D), "fp8", divide_by=0.25), "fp8", "cuda")
    vc = census_v(Skv, D)
    v8 = W.to_torch(W.f32_to_e4m3_bits(np.broadcast_to(vc[None, :, None, :], (B, Skv, Hkv, D)).copy()), "fp8", "cuda")
    say("tile census, fp8 k/v 32K")
    o = F.prefill(q, k8, v8, scale=spec.scale_f32, causal=True, k_scale=0.25, v_scale=1.0)
    torch.cuda.synchronize()
    check_census(W.as_f64(W.from_torch(o, "bf16"), "bf16"), census_expected(Sq, Skv, D, True, 0), "bf16",
                 "fp8 k/v 32K")


# ----------------------------------------------------------------------------- determinism
REPEATS = 50


@pytest.mark.parametrize("name", ["bf16_causal_32k", "bf16_swa1024_d256_8k", "f16_gqa7_causal_2k",
                                  "wave8_d128_gqa_xcd_4k"])
def test_prefill_50_runs_bit_identical(name):
    torch = torch_cuda()
    import flash_attention_forward_amd as F

    spec = WL.get(name) or W.PrefillSpec(4, 8, 2, 4096, 4096, 128, "bf16", causal=True)
    inp = W.make_prefill(spec, seed=W.WORKLOAD_SEEDS.get(name, 11))
    q, k, v = (W.to_torch(a, spec.dtype, "cuda") for a in (inp.q, inp.k, inp.v))
    args = dict(scale=spec.scale_f32, causal=spec.causal, window=spec.window)
    say("prefill 50 runs", name)
    ref = F.prefill(q, k, v, **args)
    o = torch.empty_like(ref)
    for r in range(REPEATS):
        F.attn_prefill_fwd(q, k, v, o, spec.scale_f32, spec.causal, spec.window)
        assert torch.equal(o.view(torch.int16), ref.view(torch.int16)), r


def test_decode_50_runs_bit_identical_full_size():
    """The paged-decode workload (split + combine, the benchmark's split length), 50 times."""
    torch = torch_cuda()
    import bench
    import flash_attention_forward_amd as F

    spec = WL["paged_decode_b32_d128"]
    inp = W.make_decode(spec, W.WORKLOAD_SEEDS["paged_decode_b32_d128"])
    t = decode_tensors(inp)
    args = dict(block_table=t["block_table"], scale=spec.scale_f32, split_len=bench.DEFAULT_SPLIT_LEN,
                max_len=spec.max_pages_per_seq * spec.page_size)
    say("decode 50 runs")
    ref = F.decode(t["q"], t["k"], t["v"], t["cache_len"], **args)
    for r in range(REPEATS):
        o = F.decode(t["q"], t["k"], t["v"], t["cache_len"], **args)
        assert torch.equal(o.view(torch.int16), ref.view(torch.int16)), r

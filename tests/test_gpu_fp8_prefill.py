"""GPU parity of attn_prefill_fwd_fp8kv (K and V as FP8 E4M3 codes with per-tensor scales,
f16/bf16 queries) against the fp64 oracle applied to scale * value(code), with the
tolerances of gpu_common; plus a bitwise comparison with attn_prefill_fwd fed the same
codes widened to the 16-bit type (the widening is exact, and both take the same launch
shape: 128-row tiles at the small sizes, the pipelined 256-row kernel on the wide grids)."""
import numpy as np
import pytest

import oracle
from flash_attention_forward_amd import workloads as W

from gpu_common import attention_with_bound, check, dev, host64, say, torch_cuda

pytestmark = pytest.mark.gpu

LSE_TOL = {"bf16": 3e-3, "f16": 5e-4}

# name: (B, Hq, Hkv, Sq, Skv, D, dtype, causal, window, k_scale, v_scale)
CASES = {
    "bf16_causal_gqa": (2, 8, 2, 300, 300, 128, "bf16", True, 0, 0.75, 1.25),
    "f16_nomask_ragged": (1, 4, 4, 200, 333, 64, "f16", False, 0, 1.0, 1.0),
    "bf16_d256_window": (1, 4, 2, 257, 257, 256, "bf16", True, 100, 0.5, 2.0),
    "bf16_prefix": (2, 4, 1, 100, 500, 128, "bf16", True, 0, 1.5, 0.625),
    "bf16_more_queries_than_keys": (1, 2, 1, 300, 100, 128, "bf16", True, 0, 1.0, 1.0),
    "f16_window_1": (1, 4, 2, 130, 130, 128, "f16", True, 1, 0.9, 1.1),
    "bf16_d64_window": (2, 6, 3, 190, 190, 64, "bf16", True, 33, 1.0, 0.8),
}


# Grids of at least 512 workgroups of 256 rows (D = 128): the pipelined eight-wave kernel
# with FP8 staging. Ragged key tails, a cached prefix (Sq < Skv), and more queries than
# keys (the first Sq - Skv rows see no key).
WAVE8 = {
    "bf16_wave8_gqa": (4, 8, 2, 4096, 4096, 128, "bf16", True, 0, 0.75, 1.25),
    "f16_wave8_window": (2, 16, 4, 4096, 4096, 128, "f16", True, 1000, 0.5, 2.0),
    "bf16_wave8_prefix_ragged": (8, 16, 4, 1024, 3000, 128, "bf16", True, 0, 1.5, 0.625),
    "bf16_wave8_more_queries": (2, 16, 2, 4000, 1500, 128, "bf16", True, 0, 1.0, 1.0),
    "f16_wave8_nomask_ragged": (4, 8, 8, 4096, 1000, 128, "f16", False, 0, 1.0, 0.5),
}


def make(case, seed):
    B, Hq, Hkv, Sq, Skv, D, dtype, causal, window, ks, vs = case
    rng = np.random.default_rng(seed)
    q = W.normal_rounded(rng, (B, Sq, Hq, D), dtype)
    k = W.normal_rounded(rng, (B, Skv, Hkv, D), "fp8", divide_by=ks)
    v = W.normal_rounded(rng, (B, Skv, Hkv, D), "fp8", divide_by=vs)
    return q, k, v


def run(case, q, k, v, sinks=None, lse=False):
    import flash_attention_forward_amd as F

    torch = torch_cuda()
    B, Hq, Hkv, Sq, Skv, D, dtype, causal, window, ks, vs = case
    scale = np.float32(1.0 / np.sqrt(D))
    out = F.prefill(dev(q, dtype), W.to_torch(k, "fp8", "cuda"), W.to_torch(v, "fp8", "cuda"), scale=float(scale),
                    causal=causal, window=window, k_scale=ks, v_scale=vs, return_lse=lse,
                    sinks=None if sinks is None else torch.from_numpy(sinks).cuda())
    torch.cuda.synchronize()
    o, l = out if lse else (out, None)
    return host64(o, dtype), (l.cpu().numpy().astype(np.float64) if lse else None)


def reference(case, q, k, v, sinks=None):
    B, Hq, Hkv, Sq, Skv, D, dtype, causal, window, ks, vs = case
    scale = float(np.float32(1.0 / np.sqrt(D)))
    k64 = np.float64(np.float32(ks)) * W.as_f64(k, "fp8")
    v64 = np.float64(np.float32(vs)) * W.as_f64(v, "fp8")
    return oracle.attention(W.as_f64(q, dtype), k64, v64, scale, causal, window, return_lse=True,
                            sinks=None if sinks is None else sinks.astype(np.float64))


@pytest.mark.parametrize("name", list(CASES))
def test_fp8_prefill_parity(name):
    case = CASES[name]
    q, k, v = make(case, 70 + len(name))
    say("fp8 prefill", name)
    got, _ = run(case, q, k, v)
    B, Hq, Hkv, Sq, Skv, D, dtype, causal, window, ks, vs = case
    k64 = np.float64(np.float32(ks)) * W.as_f64(k, "fp8")
    v64 = np.float64(np.float32(vs)) * W.as_f64(v, "fp8")
    ref, bound = attention_with_bound(W.as_f64(q, dtype), k64, v64, float(np.float32(1.0 / np.sqrt(D))), causal,
                                      window, dtype)
    check(got, ref, dtype, name, bound=bound)


@pytest.mark.parametrize("name", ["bf16_causal_gqa", "bf16_d256_window", "bf16_more_queries_than_keys"])
def test_fp8_prefill_lse_and_sinks(name):
    case = CASES[name]
    q, k, v = make(case, 90 + len(name))
    sinks = np.random.default_rng(4).uniform(-3.0, 4.0, case[1]).astype(np.float32)
    for sk in (None, sinks):
        say("fp8 prefill lse/sinks", name, sk is not None)
        got, lse = run(case, q, k, v, sinks=sk, lse=True)
        ref, ref_lse = reference(case, q, k, v, sinks=sk)
        check(got, ref, case[6], name)
        fin = np.isfinite(ref_lse)
        assert (np.isneginf(lse) == ~fin).all()
        assert np.abs(lse[fin] - ref_lse[fin]).max(initial=0.0) <= LSE_TOL[case[6]]


@pytest.mark.parametrize("name", ["bf16_causal_gqa", "f16_nomask_ragged", "bf16_d256_window", "bf16_prefix"])
def test_fp8_prefill_equals_the_16bit_kernel_on_widened_codes(name):
    """Unit scales: the FP8 kernel and attn_prefill_fwd on the codes widened to the 16-bit type agree bitwise."""
    import flash_attention_forward_amd as F

    torch = torch_cuda()
    case = CASES[name][:9] + (1.0, 1.0)
    q, k, v = make(case, 110 + len(name))
    dtype = case[6]
    say("fp8 prefill vs widened", name)
    got, _ = run(case, q, k, v)
    kw = W.to_torch(W.round_to(W.as_f32(k, "fp8"), dtype), dtype, "cuda")
    vw = W.to_torch(W.round_to(W.as_f32(v, "fp8"), dtype), dtype, "cuda")
    o = F.prefill(dev(q, dtype), kw, vw, scale=float(np.float32(1.0 / np.sqrt(case[5]))), causal=case[7],
                  window=case[8])
    torch.cuda.synchronize()
    assert np.array_equal(got, host64(o, dtype))


@pytest.mark.parametrize("name", list(WAVE8))
def test_fp8_prefill_eight_wave_equals_the_16bit_kernel_on_widened_codes(name):
    """Unit scales, eight-wave launches: bitwise equal to attn_prefill_fwd on the widened codes."""
    import flash_attention_forward_amd as F

    torch = torch_cuda()
    case = WAVE8[name][:9] + (1.0, 1.0)
    q, k, v = make(case, 150 + len(name))
    dtype = case[6]
    say("fp8 prefill vs widened, eight waves", name)
    got, _ = run(case, q, k, v)
    kw = W.to_torch(W.round_to(W.as_f32(k, "fp8"), dtype), dtype, "cuda")
    vw = W.to_torch(W.round_to(W.as_f32(v, "fp8"), dtype), dtype, "cuda")
    o = F.prefill(dev(q, dtype), kw, vw, scale=float(np.float32(1.0 / np.sqrt(case[5]))), causal=case[7],
                  window=case[8])
    torch.cuda.synchronize()
    assert np.array_equal(got, host64(o, dtype))


@pytest.mark.parametrize("name", list(WAVE8))
def test_fp8_prefill_eight_wave_parity_sampled(name):
    """Eight-wave launches with per-tensor scales against the oracle on rows spread over every
    batch, head and query tile (first, last and ragged rows included)."""
    case = WAVE8[name]
    B, Hq, Hkv, Sq, Skv, D, dtype, causal, window, ks, vs = case
    q, k, v = make(case, 170 + len(name))
    say("fp8 prefill eight waves", name)
    got, _ = run(case, q, k, v)
    rng = np.random.default_rng(9)
    edge = [0, 1, 255, 256, Sq // 2, Sq - 257, Sq - 1, Sq - Skv - 1, Sq - Skv, Sq - Skv + 1]  # last rows with no key
    ii = np.concatenate([np.array([e for e in edge if 0 <= e < Sq]), rng.integers(0, Sq, 120)])
    rows = np.stack([rng.integers(0, B, len(ii)), ii, rng.integers(0, Hq, len(ii))], axis=1).astype(np.int64)
    k64 = np.float64(np.float32(ks)) * W.as_f64(k, "fp8")
    v64 = np.float64(np.float32(vs)) * W.as_f64(v, "fp8")
    ref, bound = attention_with_bound(W.as_f64(q, dtype), k64, v64, float(np.float32(1.0 / np.sqrt(D))), causal,
                                      window, dtype, rows=rows)
    check(got[rows[:, 0], rows[:, 1], rows[:, 2]], ref, dtype, name, bound=bound)


def test_fp8_prefill_full_size_sampled():
    """The 32K causal workload (8 q-heads over one kv-head, spiked keys) with K and V stored as FP8
    (each value divided by its tensor's scale, then rounded to E4M3), on sampled rows, in the launch
    the benchmark times."""
    import flash_attention_forward_amd as F

    torch = torch_cuda()
    name = "bf16_causal_32k"
    spec = W.WORKLOADS[name]
    inp = W.make_prefill(spec, W.WORKLOAD_SEEDS[name])
    ks, vs = W.FP8_PREFILL_SCALES
    k8 = W.f32_to_e4m3_bits(W.as_f32(inp.k, spec.dtype) / np.float32(ks))
    v8 = W.f32_to_e4m3_bits(W.as_f32(inp.v, spec.dtype) / np.float32(vs))
    say("fp8 prefill full size", name)
    o = F.prefill(dev(inp.q, spec.dtype), W.to_torch(k8, "fp8", "cuda"), W.to_torch(v8, "fp8", "cuda"),
                  scale=spec.scale_f32, causal=True, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    got = host64(o, spec.dtype)
    rng = np.random.default_rng(8)
    S = spec.seqlen_q
    rows_i = sorted({0, 1, 127, 128, 4095, 16384, S - 1} | set(rng.integers(0, S, 24).tolist()))
    rows = np.array([(0, i, h) for i in rows_i for h in rng.choice(spec.n_q_heads, 2, replace=False)], dtype=np.int64)
    k64 = np.float64(np.float32(ks)) * W.as_f64(k8, "fp8")
    v64 = np.float64(np.float32(vs)) * W.as_f64(v8, "fp8")
    ref, _ = oracle.attention_rows(W.as_f64(inp.q, spec.dtype), k64, v64, spec.scale_f32, True, 0, rows)
    check(got[rows[:, 0], rows[:, 1], rows[:, 2]], ref, spec.dtype, "32K with an FP8 cache")


def test_fp8_prefill_nan_codes_outside_the_visible_keys_never_leak():
    """NaN codes (0x7F) past seqlen_kv, and in keys before the first query's window, change no bit."""
    import flash_attention_forward_amd as F

    torch = torch_cuda()
    case = (1, 2, 1, 130, 300, 128, "bf16", True, 90, 0.5, 0.25)
    q, k, v = make(case, 12)
    Sq, Skv, w = 130, 300, 90
    scale = float(np.float32(1.0 / np.sqrt(128)))
    qt = dev(q, "bf16")
    say("fp8 prefill nan codes outside the visible keys")
    ref = F.prefill(qt, W.to_torch(k, "fp8", "cuda"), W.to_torch(v, "fp8", "cuda"), scale=scale, causal=True, window=w,
                    k_scale=0.5, v_scale=0.25)
    kbig = np.full((1, Skv + 70, 1, 128), 0x7F, np.uint8)
    vbig = kbig.copy()
    first_visible = (Skv - Sq) - w + 1  # no query sees keys below this
    kbig[:, first_visible:Skv] = k[:, first_visible:]
    vbig[:, first_visible:Skv] = v[:, first_visible:]
    kt, vt = W.to_torch(kbig, "fp8", "cuda"), W.to_torch(vbig, "fp8", "cuda")
    o = F.prefill(qt, kt[:, :Skv], vt[:, :Skv], scale=scale, causal=True, window=w, k_scale=0.5, v_scale=0.25)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), ref.view(torch.int16))


def test_fp8_prefill_repeated_runs_bit_identical():
    """The same launch repeated gives bit-identical outputs (eight-wave launch, window masks)."""
    import flash_attention_forward_amd as F

    torch = torch_cuda()
    case = (2, 16, 2, 4096, 4096, 128, "bf16", True, 700, 0.5, 0.25)  # 16 tiles x 2 x 16 heads: the eight-wave launch
    q, k, v = make(case, 13)
    qt, kt, vt = dev(q, "bf16"), W.to_torch(k, "fp8", "cuda"), W.to_torch(v, "fp8", "cuda")
    say("fp8 prefill repeated runs")
    first = F.prefill(qt, kt, vt, causal=True, window=700, k_scale=0.5, v_scale=0.25)
    for _ in range(20):
        again = F.prefill(qt, kt, vt, causal=True, window=700, k_scale=0.5, v_scale=0.25)
        torch.cuda.synchronize()
        assert torch.equal(again.view(torch.int16), first.view(torch.int16))

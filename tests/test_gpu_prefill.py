"""GPU parity of attn_prefill_fwd against the fp64 oracle (tolerances in gpu_common)."""
import numpy as np
import pytest

from flash_attention_forward_amd import workloads as W

from gpu_common import check, gpu_prefill, oracle_prefill, prefill_with_bound, say, torch_cuda

pytestmark = pytest.mark.gpu

WL = W.WORKLOADS

# Same structure as the five workloads, at sizes the oracle finishes in seconds,
# spanning several tiles with a ragged tail.
SMALL = {
    "fp32_full": WL["fp32_d64_s256"],
    "fp32_ragged_causal": W.shrink(WL["fp32_d64_s256"], seqlen_q=200, seqlen_kv=200, causal=True),
    "fp32_d128_gqa_window": W.PrefillSpec(1, 4, 2, 150, 150, 128, "f32", causal=True, window=40),
    "fp32_d256": W.PrefillSpec(2, 2, 1, 97, 97, 256, "f32", causal=False),
    "f16_gqa7_ragged": W.shrink(WL["f16_gqa7_causal_2k"], seqlen_q=333, seqlen_kv=333),
    "bf16_ragged_spikes": W.shrink(WL["bf16_causal_32k"], seqlen_q=700, seqlen_kv=700),
    "bf16_swa_d256_ragged": W.shrink(WL["bf16_swa1024_d256_8k"], n_q_heads=4, n_kv_heads=2, seqlen_q=600, seqlen_kv=600,
                          window=150),
    "bf16_d64_nocausal": W.PrefillSpec(2, 3, 3, 190, 190, 64, "bf16", causal=False),
    "f16_d256_nocausal": W.PrefillSpec(1, 2, 1, 130, 130, 256, "f16", causal=False),
    "bf16_sq_lt_skv": W.PrefillSpec(1, 4, 1, 77, 300, 128, "bf16", causal=True),
    "bf16_sq_lt_skv_window": W.PrefillSpec(1, 4, 2, 150, 390, 128, "bf16", causal=True, window=70),
    "bf16_sq_gt_skv": W.PrefillSpec(1, 2, 1, 260, 100, 128, "bf16", causal=True),  # early rows see nothing
    "bf16_window1": W.PrefillSpec(1, 2, 1, 140, 140, 64, "bf16", causal=True, window=1),
    "bf16_single_row": W.PrefillSpec(1, 8, 1, 1, 1, 128, "bf16", causal=True),
    "f16_mqa_long_window": W.PrefillSpec(1, 8, 1, 520, 520, 128, "f16", causal=True, window=512),
    # enough 256-row query tiles (>= 512 workgroups) for the eight-wave launch
    "wide_bf16_causal_ragged": W.PrefillSpec(32, 8, 2, 300, 300, 128, "bf16", causal=True),
    "wide_f16_d64_window": W.PrefillSpec(32, 8, 4, 290, 290, 64, "f16", causal=True, window=100),
    "wide_bf16_nocausal_sq_lt_skv": W.PrefillSpec(128, 4, 1, 200, 330, 128, "bf16", causal=False),
    "wide_bf16_sq_lt_skv_window": W.PrefillSpec(64, 8, 8, 130, 400, 128, "bf16", causal=True, window=90),
    # longer rows (9 to 12 row tiles, up to 24 key tiles per row tile)
    "long_f16_gqa_causal_ragged": W.PrefillSpec(1, 8, 2, 1100, 1100, 128, "f16", causal=True),
    "long_bf16_d64_window": W.PrefillSpec(2, 4, 1, 1500, 1500, 64, "bf16", causal=True, window=700),
    "long_bf16_sq_lt_skv": W.PrefillSpec(1, 4, 2, 1030, 1300, 128, "bf16", causal=True),
    "long_bf16_sq_gt_skv": W.PrefillSpec(1, 2, 1, 1100, 700, 128, "bf16", causal=True),  # first rows see nothing
}


@pytest.mark.parametrize("name", list(SMALL))
def test_prefill_parity_small(name):
    spec = SMALL[name]
    inp = W.make_prefill(spec, seed=100 + len(name))
    say("prefill parity", name, spec)
    got = gpu_prefill(inp)
    if spec.dtype == "f32":
        check(got, oracle_prefill(inp), spec.dtype, name)
    else:
        ref, bound = prefill_with_bound(inp)
        check(got, ref, spec.dtype, name, bound=bound)


@pytest.mark.parametrize("name", ["f16_gqa7_causal_2k", "bf16_swa1024_d256_8k"])
def test_prefill_parity_full_size_every_row(name):
    """Full-size workloads, launched as the benchmark launches them, against the oracle on every
    output element (the fixed tolerances and the derived per-element bound)."""
    spec = WL[name]
    inp = W.make_prefill(spec, seed=W.WORKLOAD_SEEDS[name])
    say("prefill full-size, every row", name)
    got = gpu_prefill(inp)
    ref, bound = prefill_with_bound(inp)
    check(got, ref, spec.dtype, name, bound=bound)


def test_prefill_parity_32k_dense_stride():
    """The 32K causal workload as launched by the benchmark, against the oracle on every 16th
    query row of every head (plus the last one), offset per head so all residues mod 16 occur."""
    name = "bf16_causal_32k"
    spec = WL[name]
    inp = W.make_prefill(spec, seed=W.WORKLOAD_SEEDS[name])
    say("prefill 32K, every 16th row")
    got = gpu_prefill(inp)
    rows = np.array([(0, i, h) for h in range(spec.n_q_heads)
                     for i in list(range((5 * h) % 16, spec.seqlen_q, 16)) + [spec.seqlen_q - 1]], dtype=np.int64)
    ref, bound = prefill_with_bound(inp, rows=rows)
    check(got[rows[:, 0], rows[:, 1], rows[:, 2]], ref, spec.dtype, name, bound=bound)
    assert np.isfinite(got).all()


def test_prefill_fp32_full():
    spec = WL["fp32_d64_s256"]
    inp = W.make_prefill(spec, seed=W.WORKLOAD_SEEDS["fp32_d64_s256"])
    say("prefill fp32 d64 full")
    rel = check(gpu_prefill(inp), oracle_prefill(inp), "f32", "fp32_full")
    say("fp32 full normwise rel err", rel)


def test_empty_kv_gives_zeros():
    spec = W.PrefillSpec(1, 2, 1, 70, 0, 128, "bf16", causal=False)
    inp = W.make_prefill(spec, seed=3)
    say("prefill empty kv")
    assert (gpu_prefill(inp) == 0).all()


@pytest.mark.parametrize("scale", [0.0, -0.09, 0.5])
def test_scale_sign_and_zero(scale):
    spec = W.PrefillSpec(1, 2, 1, 150, 150, 128, "bf16", causal=True, window=60)
    inp = W.make_prefill(spec, seed=4)
    say("prefill scale", scale)
    ref, bound = prefill_with_bound(inp, scale=scale)
    check(gpu_prefill(inp, scale=scale), ref, "bf16", f"scale={scale}", bound=bound)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 64), ("bf16", 256), ("f32", 128)])
@pytest.mark.parametrize("scale", [0.0, 1e-12, 0.1])
def test_rows_without_keys_and_tiny_scales(dtype, d, scale):
    """seqlen_q > seqlen_kv with the causal mask: the first rows see no key and must be zeros,
    also when |scale| is zero or far below any normal softmax scale."""
    spec = W.PrefillSpec(1, 2, 1, 300, 120, d, dtype, causal=True)
    inp = W.make_prefill(spec, seed=41)
    say("prefill rows without keys", dtype, d, scale)
    out = gpu_prefill(inp, scale=scale)
    assert (out[:, :180] == 0).all()
    if dtype == "f32":
        check(out, oracle_prefill(inp, scale=scale), dtype, f"{dtype} d={d} scale={scale}")
    else:
        ref, bound = prefill_with_bound(inp, scale=scale)
        check(out, ref, dtype, f"{dtype} d={d} scale={scale}", bound=bound)


def test_gqa_equals_replicated_kv_bitwise():
    torch = torch_cuda()
    import flash_attention_forward_amd as F

    spec = W.PrefillSpec(2, 8, 2, 300, 300, 128, "bf16", causal=True, window=100)
    inp = W.make_prefill(spec, seed=5)
    say("gqa vs replicated")
    q, k, v = (W.to_torch(a, "bf16", "cuda") for a in (inp.q, inp.k, inp.v))
    o1 = F.prefill(q, k, v, scale=spec.scale_f32, causal=True, window=100)
    kr = k.repeat_interleave(4, dim=2).contiguous()
    vr = v.repeat_interleave(4, dim=2).contiguous()
    o2 = F.prefill(q, kr, vr, scale=spec.scale_f32, causal=True, window=100)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_strided_views_match_contiguous():
    """q/k/v as slices of one packed [B, S, Hq + 2Hkv, D] tensor, o as a slice too."""
    torch = torch_cuda()
    import flash_attention_forward_amd as F

    spec = W.PrefillSpec(1, 4, 2, 200, 200, 128, "f16", causal=True)
    inp = W.make_prefill(spec, seed=6)
    say("strided views")
    q, k, v = (W.to_torch(a, "f16", "cuda") for a in (inp.q, inp.k, inp.v))
    packed = torch.cat([q, k, v], dim=2)
    qs, ks, vs = packed[:, :, :4], packed[:, :, 4:6], packed[:, :, 6:8]
    obuf = torch.zeros(1, 200, 6, 128, dtype=torch.float16, device="cuda")
    F.attn_prefill_fwd(qs, ks, vs, obuf[:, :, 1:5], spec.scale_f32, True)
    o = F.prefill(q, k, v, scale=spec.scale_f32, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(obuf[:, :, 1:5], o)
    assert (obuf[:, :, 0] == 0).all() and (obuf[:, :, 5] == 0).all()


@pytest.mark.parametrize("causal,window", [(True, 0), (True, 37), (False, 0)])
def test_needles_bit_exact(causal, window):
    """Key j* aligned with query i (score gap >> 150 in log2 units): o_i == v[j*] bit-exactly
    when j* is visible; when it is masked, o_i is bit-identical to the run without the needle.
    j* sweeps tile (64), wave (32) and window edges."""
    torch = torch_cuda()
    import flash_attention_forward_amd as F

    S, D = 260, 128
    spec = W.PrefillSpec(1, 1, 1, S, S, D, "bf16", causal=causal, window=window)
    inp = W.make_prefill(spec, seed=7)
    q64 = W.as_f64(inp.q, "bf16")
    q, k, v = (W.to_torch(a, "bf16", "cuda") for a in (inp.q, inp.k, inp.v))
    base = F.prefill(q, k, v, scale=spec.scale_f32, causal=causal, window=window)
    say("needles", causal, window)
    for i in (0, 31, 32, 63, 64, 100, 127, 128, 200, 259):
        qpos = i
        cand = {0, 1, 31, 32, 63, 64, 65, 127, 128, qpos - 1, qpos, qpos + 1, qpos - window + 1, qpos - window,
                S - 1}
        for j in sorted(c for c in cand if 0 <= c < S):
            kk = inp.k.copy()
            needle = 300.0 * q64[0, i, 0] / (q64[0, i, 0] @ q64[0, i, 0]) / spec.scale_f32
            kk[0, j, 0] = W.round_to(needle.astype(np.float32), "bf16")
            o = F.prefill(q, W.to_torch(kk, "bf16", "cuda"), v, scale=spec.scale_f32, causal=causal, window=window)
            visible = (not causal or j <= qpos) and (window <= 0 or j >= qpos - window + 1)
            if visible:
                assert torch.equal(o[0, i, 0].view(torch.int16), v[0, j, 0].view(torch.int16)), (i, j)
            else:
                assert torch.equal(o[0, i, 0].view(torch.int16), base[0, i, 0].view(torch.int16)), (i, j)


def test_garbage_outside_kv_never_leaks():
    """NaN in memory past seqlen_kv, and in keys before the first query's window, changes nothing."""
    torch = torch_cuda()
    import flash_attention_forward_amd as F

    Sq, Skv, w = 130, 300, 90
    spec = W.PrefillSpec(1, 2, 1, Sq, Skv, 128, "bf16", causal=True, window=w)
    inp = W.make_prefill(spec, seed=8)
    q, k, v = (W.to_torch(a, "bf16", "cuda") for a in (inp.q, inp.k, inp.v))
    say("garbage outside kv")
    ref = F.prefill(q, k, v, scale=spec.scale_f32, causal=True, window=w)
    kbig = torch.full((1, Skv + 70, 1, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    vbig = kbig.clone()
    kbig[:, :Skv] = k
    vbig[:, :Skv] = v
    first_visible = (Skv - Sq) - w + 1  # no query sees keys below this
    kbig[:, :first_visible] = float("nan")
    vbig[:, :first_visible] = float("nan")
    o = F.prefill(q, kbig[:, :Skv], vbig[:, :Skv], scale=spec.scale_f32, causal=True, window=w)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), ref.view(torch.int16))


def test_constant_v_is_exact():
    """V = c (bf16-representable) gives O = c exactly: P is summed as rounded."""
    torch = torch_cuda()
    import flash_attention_forward_amd as F

    spec = W.PrefillSpec(1, 4, 2, 333, 333, 128, "bf16", causal=True, window=200)
    inp = W.make_prefill(spec, seed=9)
    q, k = (W.to_torch(a, "bf16", "cuda") for a in (inp.q, inp.k))
    v = torch.full_like(k, -1.375)
    say("constant v")
    o = F.prefill(q, k, v, scale=spec.scale_f32, causal=True, window=200)
    torch.cuda.synchronize()
    assert (o == -1.375).all()


def test_repeated_runs_bit_identical():
    """The same launch repeated gives bit-identical outputs (no scheduling-dependent races)."""
    torch = torch_cuda()
    import flash_attention_forward_amd as F

    spec = W.shrink(WL["bf16_causal_32k"], seqlen_q=4096, seqlen_kv=4096)
    inp = W.make_prefill(spec, seed=10)
    q, k, v = (W.to_torch(a, "bf16", "cuda") for a in (inp.q, inp.k, inp.v))
    say("repeated runs")
    ref = F.prefill(q, k, v, scale=spec.scale_f32, causal=True)
    for _ in range(30):
        o = F.prefill(q, k, v, scale=spec.scale_f32, causal=True)
        assert torch.equal(o.view(torch.int16), ref.view(torch.int16))

"""GPU parity of the softmax statistics (log-sum-exp per row) and the attention sinks:
attn_prefill_fwd_ex and attn_decode_combine_ex against the fp64 oracle.

Tolerances: outputs as in gpu_common. The LSE is log(sum of the rounded P) + m: every
term of the sum carries a relative rounding error of at most 2^-9 (bf16 P) or 2^-12
(f16 P), so the sum is off by at most that relative amount and the log by about as
much in absolute terms; f32 P is not rounded. The bounds below add the f32 arithmetic
of the kernels on top: 3e-3 (bf16), 5e-4 (f16), 1e-5 (f32), absolute.
"""
import numpy as np
import pytest

import oracle
from flash_attention_forward_amd import workloads as W

from gpu_common import check, decode_tensors, dev, host64, say, torch_cuda

pytestmark = pytest.mark.gpu

LSE_TOL = {"bf16": 3e-3, "f16": 5e-4, "f32": 1e-5}


def check_lse(got, ref, dtype, what):
    assert got.shape == ref.shape
    fin = np.isfinite(ref)
    assert (np.isneginf(got) == ~fin).all(), f"{what}: -inf rows differ"
    err = np.abs(got[fin] - ref[fin]).max(initial=0.0)
    assert err <= LSE_TOL[dtype], f"{what}: lse max-abs {err:.3e}"
    return err


def sinks_for(hq, seed):
    return np.random.default_rng(seed).uniform(-3.0, 4.0, hq).astype(np.float32)


PREFILL = {
    "bf16_causal_ragged": W.PrefillSpec(1, 4, 2, 333, 333, 128, "bf16", causal=True),
    "f16_window_sq_lt_skv": W.PrefillSpec(2, 4, 1, 150, 390, 128, "f16", causal=True, window=70),
    "bf16_d256_nocausal": W.PrefillSpec(1, 2, 1, 130, 130, 256, "bf16", causal=False),
    "bf16_d64_rows_without_keys": W.PrefillSpec(1, 2, 1, 300, 120, 64, "bf16", causal=True),
    "f32_d64_causal": W.PrefillSpec(1, 2, 1, 200, 200, 64, "f32", causal=True),
    "wide_bf16_causal": W.PrefillSpec(32, 8, 2, 300, 300, 128, "bf16", causal=True),  # eight-wave launch
}


@pytest.mark.parametrize("with_sinks", [False, True])
@pytest.mark.parametrize("name", list(PREFILL))
def test_prefill_lse_and_sinks(name, with_sinks):
    import flash_attention_forward_amd as F

    torch = torch_cuda()
    s = PREFILL[name]
    inp = W.make_prefill(s, seed=300 + len(name))
    sinks = sinks_for(s.n_q_heads, 7) if with_sinks else None
    say("prefill lse/sinks", name, with_sinks)
    q, k, v = dev(inp.q, s.dtype), dev(inp.k, s.dtype), dev(inp.v, s.dtype)
    o, lse = F.prefill(q, k, v, scale=s.scale_f32, causal=s.causal, window=s.window,
                       sinks=None if sinks is None else torch.from_numpy(sinks).cuda(), return_lse=True)
    torch.cuda.synchronize()
    f64 = lambda a: W.as_f64(a, s.dtype)
    ro, rl = oracle.attention(f64(inp.q), f64(inp.k), f64(inp.v), s.scale_f32, s.causal, s.window,
                              return_lse=True, sinks=None if sinks is None else sinks.astype(np.float64))
    check(host64(o, s.dtype), ro, s.dtype, name)
    say("lse max-abs", check_lse(lse.cpu().numpy().astype(np.float64), rl, s.dtype, name))


def test_prefill_full_size_with_sinks_and_lse():
    """The 32K causal workload, launched as the benchmark launches it, with sinks and lse."""
    import flash_attention_forward_amd as F
    from gpu_common import sample_rows

    torch = torch_cuda()
    name = "bf16_causal_32k"
    s = W.WORKLOADS[name]
    inp = W.make_prefill(s, seed=W.WORKLOAD_SEEDS[name])
    sinks = sinks_for(s.n_q_heads, 8)
    say("prefill full size sinks/lse")
    q, k, v = dev(inp.q, s.dtype), dev(inp.k, s.dtype), dev(inp.v, s.dtype)
    o, lse = F.prefill(q, k, v, scale=s.scale_f32, causal=True, sinks=torch.from_numpy(sinks).cuda(),
                       return_lse=True)
    torch.cuda.synchronize()
    rows = sample_rows(s, n_random=100, seed=2)
    f64 = lambda a: W.as_f64(a, s.dtype)
    ro, rl = oracle.attention_rows(f64(inp.q), f64(inp.k), f64(inp.v), s.scale_f32, True, 0, rows,
                                   sinks=sinks.astype(np.float64))
    got = host64(o, s.dtype)[rows[:, 0], rows[:, 1], rows[:, 2]]
    check(got, ro, "bf16", name)
    check_lse(lse.cpu().numpy().astype(np.float64)[rows[:, 0], rows[:, 1], rows[:, 2]], rl, "bf16", name)


def test_prefill_neg_inf_sinks_change_nothing():
    import flash_attention_forward_amd as F

    torch = torch_cuda()
    s = W.PrefillSpec(2, 4, 2, 260, 260, 128, "bf16", causal=True, window=90)
    inp = W.make_prefill(s, seed=5)
    q, k, v = dev(inp.q, s.dtype), dev(inp.k, s.dtype), dev(inp.v, s.dtype)
    say("prefill -inf sinks")
    o0 = F.prefill(q, k, v, scale=s.scale_f32, causal=True, window=90)
    o1, l1 = F.prefill(q, k, v, scale=s.scale_f32, causal=True, window=90,
                       sinks=torch.full((4,), float("-inf"), device="cuda"), return_lse=True)
    o2, l2 = F.prefill(q, k, v, scale=s.scale_f32, causal=True, window=90, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))
    assert torch.equal(o0.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


@pytest.mark.parametrize("split_len", [16, 256, 1024])
@pytest.mark.parametrize("kw", [dict(), dict(s_active=4, len_lo=4), dict(dtype="f16", head_dim=64)])
def test_decode_lse_and_sinks(kw, split_len):
    import flash_attention_forward_amd as F

    torch = torch_cuda()
    spec = W.shrink(W.WORKLOADS["paged_decode_b32_d128"], batch=6, len_lo=kw.get("len_lo", 1), len_hi=2500,
                    **{k: v for k, v in kw.items() if k != "len_lo"})
    inp = W.make_decode(spec, seed=11)
    sinks = sinks_for(spec.n_q_heads, 9)
    t = decode_tensors(inp)
    say("decode lse/sinks", kw, split_len)
    o, lse = F.decode(t["q"], t["k"], t["v"], t["cache_len"], block_table=t["block_table"], scale=spec.scale_f32,
                      split_len=split_len, max_len=spec.max_pages_per_seq * spec.page_size,
                      sinks=torch.from_numpy(sinks).cuda(), return_lse=True)
    torch.cuda.synchronize()
    f64 = lambda a: W.as_f64(a, spec.dtype)
    ro, rl = oracle.decode(f64(inp.q), inp.k_pool, inp.v_pool, inp.block_table, inp.cache_len, spec.scale_f32,
                           to_f64=f64, return_lse=True, sinks=sinks.astype(np.float64))
    check(host64(o, spec.dtype), ro, spec.dtype, f"decode {kw}")
    check_lse(lse.cpu().numpy().astype(np.float64), rl, spec.dtype, f"decode {kw}")


def test_decode_without_sinks_lse_matches_oracle_and_neg_inf_is_none():
    import flash_attention_forward_amd as F

    torch = torch_cuda()
    spec = W.shrink(W.WORKLOADS["paged_decode_b32_d128"], batch=5, len_lo=1, len_hi=3000)
    inp = W.make_decode(spec, seed=12)
    t = decode_tensors(inp)
    say("decode lse without sinks")
    kw = dict(block_table=t["block_table"], scale=spec.scale_f32, split_len=512,
              max_len=spec.max_pages_per_seq * spec.page_size)
    o0 = F.decode(t["q"], t["k"], t["v"], t["cache_len"], **kw)
    o1, l1 = F.decode(t["q"], t["k"], t["v"], t["cache_len"], return_lse=True, **kw)
    o2 = F.decode(t["q"], t["k"], t["v"], t["cache_len"], sinks=torch.full((spec.n_q_heads,), float("-inf"),
                                                                                device="cuda"), **kw)
    torch.cuda.synchronize()
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))
    assert torch.equal(o0.view(torch.int16), o2.view(torch.int16))
    f64 = lambda a: W.as_f64(a, spec.dtype)
    _, rl = oracle.decode(f64(inp.q), inp.k_pool, inp.v_pool, inp.block_table, inp.cache_len, spec.scale_f32,
                          to_f64=f64, return_lse=True)
    check_lse(l1.cpu().numpy().astype(np.float64), rl, "bf16", "decode lse")


def mixed_sinks(hq):
    """A finite sink, no sink (-inf), NaN and +inf, repeated over the q-heads."""
    return np.resize(np.array([1.5, -np.inf, np.nan, np.inf], np.float32), hq)


@pytest.mark.parametrize("name", ["bf16_causal_ragged", "f32_d64_causal", "wide_bf16_causal",
                                  "bf16_d64_rows_without_keys"])
def test_prefill_nan_and_inf_sinks_give_nan_rows(name):
    """A NaN or +inf sink gives NaN output rows and NaN lse for its head (every row, also those
    that see no key), as the oracle does; finite and -inf sinks are unaffected."""
    import flash_attention_forward_amd as F

    torch = torch_cuda()
    s = PREFILL[name]
    inp = W.make_prefill(s, seed=310 + len(name))
    sinks = mixed_sinks(s.n_q_heads)
    q, k, v = dev(inp.q, s.dtype), dev(inp.k, s.dtype), dev(inp.v, s.dtype)
    say("prefill NaN/inf sinks", name)
    o, lse = F.prefill(q, k, v, scale=s.scale_f32, causal=s.causal, window=s.window,
                       sinks=torch.from_numpy(sinks).cuda(), return_lse=True)
    torch.cuda.synchronize()
    f64 = lambda a: W.as_f64(a, s.dtype)
    ro, rl = oracle.attention(f64(inp.q), f64(inp.k), f64(inp.v), s.scale_f32, s.causal, s.window,
                              return_lse=True, sinks=sinks.astype(np.float64))
    got, gl = host64(o, s.dtype), lse.cpu().numpy().astype(np.float64)
    bad = ~np.isfinite(sinks) & ~np.isneginf(sinks)
    assert np.isnan(ro[:, :, bad]).all() and np.isnan(rl[:, :, bad]).all()  # the oracle's reading
    assert np.isnan(got[:, :, bad]).all() and np.isnan(gl[:, :, bad]).all()
    check(got[:, :, ~bad], ro[:, :, ~bad], s.dtype, name)
    check_lse(gl[:, :, ~bad], rl[:, :, ~bad], s.dtype, name)


def test_fp8_prefill_and_decode_combine_nan_and_inf_sinks():
    """The same for attn_prefill_fwd_fp8kv and for the decode merge (attn_decode_combine_ex)."""
    import flash_attention_forward_amd as F

    torch = torch_cuda()
    rng = np.random.default_rng(3)
    B, Sq, Hq, Hkv, D = 1, 200, 4, 2, 128
    q = W.normal_rounded(rng, (B, Sq, Hq, D), "bf16")
    k8 = W.normal_rounded(rng, (B, Sq, Hkv, D), "fp8")
    v8 = W.normal_rounded(rng, (B, Sq, Hkv, D), "fp8")
    sinks = mixed_sinks(Hq)
    bad = ~np.isfinite(sinks) & ~np.isneginf(sinks)
    say("fp8 prefill NaN/inf sinks")
    o, lse = F.prefill(dev(q, "bf16"), W.to_torch(k8, "fp8", "cuda"), W.to_torch(v8, "fp8", "cuda"),
                       scale=float(np.float32(D ** -0.5)), causal=True, sinks=torch.from_numpy(sinks).cuda(),
                       return_lse=True)
    torch.cuda.synchronize()
    got, gl = host64(o, "bf16"), lse.cpu().numpy()
    assert np.isnan(got[:, :, bad]).all() and np.isnan(gl[:, :, bad]).all()
    assert np.isfinite(got[:, :, ~bad]).all() and not np.isnan(gl[:, :, ~bad]).any()

    spec = W.shrink(W.WORKLOADS["paged_decode_b32_d128"], batch=4, n_q_heads=8, n_kv_heads=2, len_lo=1, len_hi=900)
    inp = W.make_decode(spec, seed=13)
    dsinks = mixed_sinks(spec.n_q_heads)
    dbad = ~np.isfinite(dsinks) & ~np.isneginf(dsinks)
    t = decode_tensors(inp)
    say("decode combine NaN/inf sinks")
    o, lse = F.decode(t["q"], t["k"], t["v"], t["cache_len"], block_table=t["block_table"], scale=spec.scale_f32,
                      split_len=128, max_len=spec.max_pages_per_seq * spec.page_size,
                      sinks=torch.from_numpy(dsinks).cuda(), return_lse=True)
    torch.cuda.synchronize()
    f64 = lambda a: W.as_f64(a, spec.dtype)
    ro, rl = oracle.decode(f64(inp.q), inp.k_pool, inp.v_pool, inp.block_table, inp.cache_len, spec.scale_f32,
                           to_f64=f64, return_lse=True, sinks=dsinks.astype(np.float64))
    got, gl = host64(o, spec.dtype), lse.cpu().numpy().astype(np.float64)
    assert np.isnan(ro[:, :, dbad]).all() and np.isnan(got[:, :, dbad]).all() and np.isnan(gl[:, :, dbad]).all()
    check(got[:, :, ~dbad], ro[:, :, ~dbad], spec.dtype, "decode finite sinks")
    check_lse(gl[:, :, ~dbad], rl[:, :, ~dbad], spec.dtype, "decode finite sinks")

"""GPU parity of the packed-sequence prefill (attn_prefill_varlen_fwd): per-sequence
bounds read from cumulative offsets on the device, against the fp64 oracle
(oracle.attention_varlen), with the tolerances of gpu_common; the LSE bound is
the one of test_gpu_sinks_lse."""
import numpy as np
import pytest

import oracle
from flash_attention_forward_amd import workloads as W

from gpu_common import attention_with_bound, check, dev, host64, say, torch_cuda

pytestmark = pytest.mark.gpu

LSE_TOL = {"bf16": 3e-3, "f16": 5e-4, "f32": 1e-5}

# name: (spec, explicit q lengths or None, explicit prefixes or None)
CASES = {
    "bf16_causal_ragged": (W.VarlenSpec(6, 4, 2, 128, "bf16", True, 1, 300), None, None),
    "bf16_causal_empty_and_prefix": (W.VarlenSpec(5, 4, 1, 128, "bf16", True, 0, 0),
                                     [130, 0, 1, 257, 64], [0, 40, 0, 300, 0]),
    "f16_window_prefix": (W.VarlenSpec(4, 8, 2, 128, "f16", True, 50, 400, window=70, prefix_lo=0, prefix_hi=200),
                          None, None),
    "bf16_d64_nocausal_no_keys": (W.VarlenSpec(4, 2, 1, 64, "bf16", False, 0, 0), [33, 70, 0, 129], [0, 0, 5, 0]),
    "bf16_d256_causal": (W.VarlenSpec(3, 2, 1, 256, "bf16", True, 20, 200), None, None),
    "f32_d64_causal_prefix": (W.VarlenSpec(4, 2, 1, 64, "f32", True, 1, 150, prefix_lo=0, prefix_hi=60), None, None),
    "f32_d128_window": (W.VarlenSpec(3, 4, 2, 128, "f32", True, 10, 130, window=33), None, None),
}


def run(inp, sinks=None, lse=False):
    import flash_attention_forward_amd as F

    torch = torch_cuda()
    s = inp.spec
    q, k, v = dev(inp.q, s.dtype), dev(inp.k, s.dtype), dev(inp.v, s.dtype)
    o = torch.empty_like(q)
    cq = torch.from_numpy(inp.cu_q.astype(np.int32)).cuda()
    ck = torch.from_numpy(inp.cu_kv.astype(np.int32)).cuda()
    lse_t = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda") if lse else None
    sk = None if sinks is None else torch.from_numpy(sinks).cuda()
    F.attn_prefill_varlen_fwd(q, k, v, o, cq, ck, int(inp.lens_q.max(initial=0)), int(inp.lens_kv.max(initial=0)),
                              s.scale_f32, s.causal, s.window, lse_t, sk)
    torch.cuda.synchronize()
    return host64(o, s.dtype), (lse_t.cpu().numpy().astype(np.float64) if lse else None)


def reference(inp, sinks=None):
    s = inp.spec
    f64 = lambda a: W.as_f64(a, s.dtype)
    return oracle.attention_varlen(f64(inp.q), f64(inp.k), f64(inp.v), inp.cu_q, inp.cu_kv, s.scale_f32, s.causal,
                                   s.window, sinks=None if sinks is None else sinks.astype(np.float64),
                                   return_lse=True)


@pytest.mark.parametrize("name", list(CASES))
def test_varlen_parity(name):
    spec, lq, pre = CASES[name]
    inp = W.make_varlen(spec, seed=500 + len(name), lens_q=lq, prefixes=pre)
    say("varlen", name, "lens_q", inp.lens_q.tolist(), "lens_kv", inp.lens_kv.tolist())
    got, _ = run(inp)
    ref, _ = reference(inp)
    if spec.dtype == "f32":
        check(got, ref, spec.dtype, name)
        return
    # the derived bound, sequence by sequence (each is the plain definition on its own slice)
    f64 = lambda a: W.as_f64(a, spec.dtype)
    bound = np.zeros_like(ref)
    for b in range(spec.batch):
        q0, q1, k0, k1 = inp.cu_q[b], inp.cu_q[b + 1], inp.cu_kv[b], inp.cu_kv[b + 1]
        if q1 > q0:
            _, bd = attention_with_bound(f64(inp.q[None, q0:q1]), f64(inp.k[None, k0:k1]), f64(inp.v[None, k0:k1]),
                                         spec.scale_f32, spec.causal, spec.window, spec.dtype)
            bound[q0:q1] = bd[0]
    check(got, ref, spec.dtype, name, bound=bound)


@pytest.mark.parametrize("name", ["bf16_causal_empty_and_prefix", "f16_window_prefix", "f32_d64_causal_prefix"])
def test_varlen_lse_and_sinks(name):
    spec, lq, pre = CASES[name]
    inp = W.make_varlen(spec, seed=600 + len(name), lens_q=lq, prefixes=pre)
    sinks = np.random.default_rng(9).uniform(-3.0, 4.0, spec.n_q_heads).astype(np.float32)
    for sk in (None, sinks):
        say("varlen lse/sinks", name, sk is not None)
        got, lse = run(inp, sinks=sk, lse=True)
        ref, ref_lse = reference(inp, sinks=sk)
        check(got, ref, spec.dtype, name)
        fin = np.isfinite(ref_lse)
        assert (np.isneginf(lse) == ~fin).all()
        assert np.abs(lse[fin] - ref_lse[fin]).max(initial=0.0) <= LSE_TOL[spec.dtype]


@pytest.mark.parametrize("B,Hq,Hkv,S,dtype,window", [
    (3, 4, 2, 200, "bf16", 0),
    (32, 8, 2, 300, "bf16", 0),     # the batched call takes the eight-wave launch, the packed one four waves
    (2, 4, 4, 150, "f16", 40),
    (2, 2, 1, 90, "f32", 0),
])
def test_varlen_equal_lengths_match_the_batched_kernel_bitwise(B, Hq, Hkv, S, dtype, window):
    import flash_attention_forward_amd as F

    torch = torch_cuda()
    spec = W.VarlenSpec(B, Hq, Hkv, 128, dtype, True, S, S, window=window)
    inp = W.make_varlen(spec, seed=700 + B)
    say("varlen vs batched", B, Hq, Hkv, S, dtype, window)
    got, _ = run(inp)
    q = dev(inp.q, dtype).view(B, S, Hq, 128)
    k = dev(inp.k, dtype).view(B, S, Hkv, 128)
    v = dev(inp.v, dtype).view(B, S, Hkv, 128)
    o = torch.empty_like(q)
    F.attn_prefill_fwd(q, k, v, o, spec.scale_f32, True, window)
    torch.cuda.synchronize()
    assert np.array_equal(got, host64(o, dtype).reshape(B * S, Hq, 128))


def test_varlen_full_size_sampled():
    """The packed workload at full size (16 prompts of 256..4096 tokens, 28/4 heads), on sampled rows of
    every sequence, in the launch the benchmark times."""
    spec = W.VARLEN_SPEC
    inp = W.make_varlen(spec, W.VARLEN_SEED)
    say("varlen full size", W.VARLEN, "total", int(inp.cu_q[-1]))
    got, _ = run(inp)
    rng = np.random.default_rng(3)
    f64 = lambda a: W.as_f64(a, spec.dtype)
    qa, ka, va = f64(inp.q), f64(inp.k), f64(inp.v)
    for b in range(spec.batch):
        q0, q1, k0, k1 = (int(x) for x in (inp.cu_q[b], inp.cu_q[b + 1], inp.cu_kv[b], inp.cu_kv[b + 1]))
        L = q1 - q0
        rows_i = sorted({0, 1, 63, 64, 255, 256, L - 1} | set(rng.integers(0, L, 12).tolist()))
        rows = np.array([(0, i, h) for i in rows_i if 0 <= i < L for h in rng.choice(spec.n_q_heads, 3, replace=False)],
                        dtype=np.int64)
        ref, _ = oracle.attention_rows(qa[None, q0:q1], ka[None, k0:k1], va[None, k0:k1], spec.scale_f32, True, 0,
                                       rows)
        check(got[q0 + rows[:, 1], rows[:, 2]], ref, spec.dtype, f"sequence {b}")


def monotone_positions(inp, seed, gap=True):
    """Nondecreasing positions per sequence inside [0, len_kv) (sorted draws, so repeats and gaps occur)."""
    rng = np.random.default_rng(seed)
    out = []
    for Lq, Lk in zip(inp.lens_q.tolist(), inp.lens_kv.tolist()):
        if Lq == 0:
            continue
        out.append(np.sort(rng.integers(0, max(Lk, 1), Lq)) if gap else np.arange(Lq) + Lk - Lq)
    return np.concatenate(out).astype(np.int32) if out else np.zeros(0, np.int32)


def run_pos(inp, pos, lse=False):
    import flash_attention_forward_amd as F

    torch = torch_cuda()
    s = inp.spec
    q, k, v = dev(inp.q, s.dtype), dev(inp.k, s.dtype), dev(inp.v, s.dtype)
    o = torch.empty_like(q)
    cq = torch.from_numpy(inp.cu_q.astype(np.int32)).cuda()
    ck = torch.from_numpy(inp.cu_kv.astype(np.int32)).cuda()
    lse_t = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda") if lse else None
    F.attn_prefill_varlen_fwd(q, k, v, o, cq, ck, int(inp.lens_q.max(initial=0)), int(inp.lens_kv.max(initial=0)),
                              s.scale_f32, s.causal, s.window, lse_t, None, torch.from_numpy(pos).cuda())
    torch.cuda.synchronize()
    return host64(o, s.dtype), (lse_t.cpu().numpy().astype(np.float64) if lse else None)


@pytest.mark.parametrize("name", ["bf16_causal_ragged", "f16_window_prefix", "bf16_d256_causal", "f32_d64_causal_prefix",
                                  "f32_d128_window"])
def test_varlen_positions_parity(name):
    spec, lq, pre = CASES[name]
    inp = W.make_varlen(spec, seed=800 + len(name), lens_q=lq, prefixes=pre)
    pos = monotone_positions(inp, 9)
    say("varlen positions", name)
    got, lse = run_pos(inp, pos, lse=True)
    s = spec
    f64 = lambda a: W.as_f64(a, s.dtype)
    ref, ref_lse = oracle.attention_varlen(f64(inp.q), f64(inp.k), f64(inp.v), inp.cu_q, inp.cu_kv, s.scale_f32,
                                           s.causal, s.window, return_lse=True, positions=pos)
    check(got, ref, s.dtype, name)
    fin = np.isfinite(ref_lse)
    assert (np.isneginf(lse) == ~fin).all()
    assert np.abs(lse[fin] - ref_lse[fin]).max(initial=0.0) <= LSE_TOL[s.dtype]


@pytest.mark.parametrize("name", ["bf16_causal_empty_and_prefix", "f16_window_prefix", "f32_d128_window"])
def test_varlen_positions_of_the_default_alignment_are_bitwise_the_default(name):
    spec, lq, pre = CASES[name]
    inp = W.make_varlen(spec, seed=900 + len(name), lens_q=lq, prefixes=pre)
    say("varlen default positions", name)
    got, _ = run_pos(inp, monotone_positions(inp, 0, gap=False))
    plain, _ = run(inp)
    assert np.array_equal(got, plain)


@pytest.mark.parametrize("name", ["bf16_causal_ragged", "f16_window_prefix", "f32_d64_causal_prefix"])
def test_varlen_positions_outside_the_keys(name):
    """Positions below 0 see no key (zeros, lse -inf); positions at or past len_kv see all keys."""
    spec, lq, pre = CASES[name]
    inp = W.make_varlen(spec, seed=950 + len(name), lens_q=lq, prefixes=pre)
    rng = np.random.default_rng(11)
    pos = np.concatenate([np.sort(rng.integers(-40, Lk + 40, Lq)) for Lq, Lk in
                          zip(inp.lens_q.tolist(), inp.lens_kv.tolist()) if Lq > 0]).astype(np.int32)
    say("varlen positions outside the keys", name)
    got, lse = run_pos(inp, pos, lse=True)
    f64 = lambda a: W.as_f64(a, spec.dtype)
    ref, ref_lse = oracle.attention_varlen(f64(inp.q), f64(inp.k), f64(inp.v), inp.cu_q, inp.cu_kv, spec.scale_f32,
                                           spec.causal, spec.window, return_lse=True, positions=pos)
    check(got, ref, spec.dtype, name)
    fin = np.isfinite(ref_lse)
    assert (~fin).any() and (np.isneginf(lse) == ~fin).all()
    assert np.all(got[~fin.any(axis=1)] == 0.0)
    assert np.abs(lse[fin] - ref_lse[fin]).max(initial=0.0) <= LSE_TOL[spec.dtype]

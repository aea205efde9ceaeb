"""The hot path captured in a HIP graph: decode (split + combine), prefill and the packed
prefill are recorded once with torch.cuda.graph and replayed on new inputs written in
place. Every replay must equal the eager call on the same inputs bit for bit (same
kernels, same launch shapes), and one replay per graph is also checked against the fp64
oracle. Eager work and synchronisations run between the replays."""
import dataclasses

import numpy as np
import pytest

import oracle
from flash_attention_forward_amd import workloads as W

from gpu_common import check, decode_tensors, dev, host64, oracle_decode, say, torch_cuda

pytestmark = pytest.mark.gpu

REPLAYS = 3


def capture(fn):
    """Warm fn up on a side stream, then record it into a graph."""
    torch = torch_cuda()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("kw", [dict(), dict(s_active=4, len_lo=4), dict(head_dim=256)])
def test_decode_graph_replays_match_eager(kw):
    import flash_attention_forward_amd as F

    torch = torch_cuda()
    base = dict(batch=6, len_lo=1, len_hi=1500)
    base.update(kw)
    inp = W.make_decode(W.shrink(W.WORKLOADS["paged_decode_b32_d128"], **base), 41)
    s = inp.spec
    t = decode_tensors(inp)
    max_len = s.max_pages_per_seq * s.page_size
    split = 256
    ms = F.max_splits_for(max_len, split)
    ws = F.DecodeWorkspace(s.batch, s.s_active, s.n_q_heads, s.head_dim, ms, "cuda")
    out = torch.empty_like(t["q"])

    def call(o, workspace):
        F.decode(t["q"], t["k"], t["v"], t["cache_len"], block_table=t["block_table"], scale=s.scale_f32,
                 split_len=split, max_len=max_len, workspace=workspace, out=o)

    say("decode graph", kw)
    g = capture(lambda: call(out, ws))
    ws_eager = F.DecodeWorkspace(s.batch, s.s_active, s.n_q_heads, s.head_dim, ms, "cuda")
    rng = np.random.default_rng(5)
    for it in range(REPLAYS):
        # new queries and shorter caches (the pages of the shorter caches are already in the table)
        q_new = W.normal_rounded(rng, inp.q.shape, s.dtype)
        len_new = np.minimum(inp.cache_len, rng.integers(1, inp.cache_len.max() + 1, s.batch)).astype(np.int32)
        t["q"].copy_(dev(q_new, s.dtype))
        t["cache_len"].copy_(torch.from_numpy(len_new))
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        ref = torch.empty_like(out)
        call(ref, ws_eager)
        torch.cuda.synchronize()
        say("replay", it, "cache_len", len_new.tolist())
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"replay {it}"
        if it == REPLAYS - 1:
            inp2 = dataclasses.replace(inp, q=q_new, cache_len=len_new)
            check(host64(got, s.dtype), oracle_decode(inp2), s.dtype, "graph replay vs oracle")


@pytest.mark.parametrize("dtype,D,window", [("bf16", 128, 0), ("f16", 64, 100), ("bf16", 256, 0)])
def test_prefill_graph_replays_match_eager(dtype, D, window):
    import flash_attention_forward_amd as F

    torch = torch_cuda()
    spec = W.PrefillSpec(2, 4, 2, 300, 300, D, dtype, causal=True, window=window)
    inp = W.make_prefill(spec, 42)
    q, k, v = dev(inp.q, dtype), dev(inp.k, dtype), dev(inp.v, dtype)
    out = torch.empty_like(q)

    def call(o):
        F.prefill(q, k, v, scale=spec.scale_f32, causal=True, window=window, out=o)

    say("prefill graph", dtype, D, window)
    g = capture(lambda: call(out))
    rng = np.random.default_rng(6)
    for it in range(REPLAYS):
        new = {n: W.normal_rounded(rng, getattr(inp, n).shape, dtype) for n in ("q", "k", "v")}
        for n, tt in (("q", q), ("k", k), ("v", v)):
            tt.copy_(dev(new[n], dtype))
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        ref = torch.empty_like(out)
        call(ref)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"replay {it}"
        if it == REPLAYS - 1:
            f64 = lambda a: W.as_f64(a, dtype)
            ref64 = oracle.attention(f64(new["q"]), f64(new["k"]), f64(new["v"]), spec.scale_f32, True, window)
            check(host64(got, dtype), ref64, dtype, "graph replay vs oracle")


def test_varlen_graph_serves_new_length_mixes():
    """The packed prefill reads the sequence bounds from the device, so one recorded graph
    serves any mix of lengths within its row count and maximum length."""
    import flash_attention_forward_amd as F

    torch = torch_cuda()
    B, Hq, Hkv, D, total, max_len = 5, 4, 2, 128, 1200, 512
    rng = np.random.default_rng(7)
    q = dev(W.normal_rounded(rng, (total, Hq, D), "bf16"), "bf16")
    k = dev(W.normal_rounded(rng, (total, Hkv, D), "bf16"), "bf16")
    v = dev(W.normal_rounded(rng, (total, Hkv, D), "bf16"), "bf16")
    cu = torch.zeros(B + 1, dtype=torch.int32, device="cuda")
    out = torch.zeros_like(q)
    scale = 1.0 / np.sqrt(D)

    def call(o):
        F.attn_prefill_varlen_fwd(q, k, v, o, cu, cu, max_len, max_len, scale, True, 0)

    def lengths():
        while True:
            ls = rng.integers(0, max_len + 1, B)
            if ls.sum() <= total:
                return ls

    cu.copy_(torch.from_numpy(np.concatenate([[0], np.cumsum(lengths())]).astype(np.int32)))
    say("varlen graph")
    g = capture(lambda: call(out))
    for it in range(REPLAYS):
        ls = lengths()
        cu_h = np.concatenate([[0], np.cumsum(ls)]).astype(np.int64)
        cu.copy_(torch.from_numpy(cu_h.astype(np.int32)))
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        ref = torch.zeros_like(out)
        call(ref)
        torch.cuda.synchronize()
        say("replay", it, "lengths", ls.tolist())
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"replay {it}"
        if it == REPLAYS - 1:
            n = int(cu_h[-1])
            f64 = lambda t: W.as_f64(W.from_torch(t[:n], "bf16"), "bf16")
            ref64 = oracle.attention_varlen(f64(q), f64(k), f64(v), cu_h, cu_h, scale, True, 0)
            check(host64(got, "bf16")[:n], ref64, "bf16", "graph replay vs oracle")


def test_fp8_prefill_graph_replays_match_eager():
    """attn_prefill_fwd_fp8kv in a graph: new FP8 codes written in place between replays."""
    import flash_attention_forward_amd as F

    torch = torch_cuda()
    B, Hq, Hkv, S, D, ks, vs = 2, 4, 2, 300, 128, 0.5, 0.25
    rng = np.random.default_rng(9)
    q = dev(W.normal_rounded(rng, (B, S, Hq, D), "bf16"), "bf16")
    k = W.to_torch(W.normal_rounded(rng, (B, S, Hkv, D), "fp8", divide_by=ks), "fp8", "cuda")
    v = W.to_torch(W.normal_rounded(rng, (B, S, Hkv, D), "fp8", divide_by=vs), "fp8", "cuda")
    out = torch.empty_like(q)
    scale = float(np.float32(1.0 / np.sqrt(D)))

    def call(o):
        F.prefill(q, k, v, scale=scale, causal=True, window=90, out=o, k_scale=ks, v_scale=vs)

    say("fp8 prefill graph")
    g = capture(lambda: call(out))
    for it in range(REPLAYS):
        k8 = W.normal_rounded(rng, (B, S, Hkv, D), "fp8", divide_by=ks)
        v8 = W.normal_rounded(rng, (B, S, Hkv, D), "fp8", divide_by=vs)
        k.copy_(W.to_torch(k8, "fp8", "cuda"))
        v.copy_(W.to_torch(v8, "fp8", "cuda"))
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        ref = torch.empty_like(out)
        call(ref)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"replay {it}"
        if it == REPLAYS - 1:
            q64 = W.as_f64(W.from_torch(q, "bf16"), "bf16")
            ref64 = oracle.attention(q64, np.float64(ks) * W.as_f64(k8, "fp8"), np.float64(vs) * W.as_f64(v8, "fp8"),
                                     scale, True, 90)
            check(host64(got, "bf16"), ref64, "bf16", "graph replay vs oracle")

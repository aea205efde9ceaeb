"""attn_decode_fwd_noalloc (partials in the library's device array, nothing allocated) against
the workspace entry points attn_decode_fwd + attn_decode_combine on the same inputs: bit-identical
outputs (the same kernels), and both within the parity bounds of the oracle; two calls in a row,
the second with a smaller input, so the second reuses the array the first filled."""
import numpy as np
import pytest

from flash_attention_forward_amd import workloads as W

from gpu_common import check, decode_tensors, decode_with_bound, host64, say, torch_cuda

pytestmark = pytest.mark.gpu


def run_both(inp, split_len, window=0):
    torch = torch_cuda()
    import flash_attention_forward_amd as F

    s = inp.spec
    t = decode_tensors(inp)
    max_len = s.max_pages_per_seq * s.page_size
    ms = F.max_splits_for(max_len, split_len)
    ws = F.DecodeWorkspace(s.batch, s.s_active, s.n_q_heads, s.head_dim, ms, "cuda")
    ref = torch.empty_like(t["q"])
    F.attn_decode_fwd(t["q"], t["k"], t["v"], t["cache_len"], ws.part_o, ws.part_lse, split_len, ms, s.scale_f32,
                      t["block_table"], window)
    F.attn_decode_combine(ws.part_o, ws.part_lse, t["cache_len"], split_len, ms, ref)
    o = torch.full_like(t["q"], float("nan"))
    F.attn_decode_fwd_noalloc(t["q"], t["k"], t["v"], t["cache_len"], split_len, ms, s.scale_f32, o,
                              block_table=t["block_table"], window=window)
    torch.cuda.synchronize()
    return o, ref


def test_noalloc_matches_the_workspace_entry_points_twice():
    torch = torch_cuda()
    import bench

    # first call: the paged-decode workload at its full size (4 MiB of partials at 4096-token splits)
    big = W.make_decode(W.WORKLOADS["paged_decode_b32_d128"], W.WORKLOAD_SEEDS["paged_decode_b32_d128"])
    say("noalloc decode, full size", int(big.cache_len.sum()))
    o, ref = run_both(big, bench.DEFAULT_SPLIT_LEN)
    assert torch.equal(o.view(torch.int16), ref.view(torch.int16))
    r, bound = decode_with_bound(big)
    check(host64(o, "bf16"), r, "bf16", "noalloc full size", bound=bound)

    # second call: smaller (6 sequences, 4 draft tokens, a window, 64-token splits): the array keeps
    # the first call's partials, and only the splits this call writes may be read
    small = W.make_decode(W.shrink(W.WORKLOADS["paged_decode_b32_d128"], batch=6, s_active=4, len_lo=4, len_hi=1500),
                          5)
    say("noalloc decode, smaller", small.cache_len.tolist())
    o, ref = run_both(small, 64, window=300)
    assert torch.equal(o.view(torch.int16), ref.view(torch.int16))
    r, bound = decode_with_bound(small, window=300)
    check(host64(o, "bf16"), r, "bf16", "noalloc smaller", bound=bound)


def test_noalloc_rejects_partials_beyond_the_array():
    torch = torch_cuda()
    import flash_attention_forward_amd as F

    inp = W.make_decode(W.WORKLOADS["paged_decode_b32_d128"], W.WORKLOAD_SEEDS["paged_decode_b32_d128"])
    s = inp.spec
    t = decode_tensors(inp)
    o = torch.zeros_like(t["q"])
    ms = F.max_splits_for(s.max_pages_per_seq * s.page_size, 512)  # 32 x 32 x 64 x 129 floats > 32 MiB
    with pytest.raises(F.AttnError, match="unsupported"):
        F.attn_decode_fwd_noalloc(t["q"], t["k"], t["v"], t["cache_len"], 512, ms, s.scale_f32, o,
                                  block_table=t["block_table"])
    torch.cuda.synchronize()
    assert (o == 0).all()

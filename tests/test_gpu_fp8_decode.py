"""GPU parity of attn_decode_fwd_fp8kv (FP8 E4M3 K/V cache, f16/bf16 queries) + attn_decode_combine
against the fp64 oracle on the same FP8-rounded cache (the codes widened exactly, times the scales).
Tolerances as for the 16-bit decode (gpu_common): the oracle sees exactly the values the kernel reads."""
import numpy as np
import pytest

import oracle
from flash_attention_forward_amd import workloads as W

from gpu_common import check, decode_with_bound, dev, host64, say, torch_cuda

pytestmark = pytest.mark.gpu


def fp8_tensors(inp):
    torch = torch_cuda()
    s = inp.spec
    return dict(q=dev(inp.q, s.dtype), k=W.to_torch(inp.k_pool, "fp8", "cuda"), v=W.to_torch(inp.v_pool, "fp8", "cuda"),
                cache_len=torch.from_numpy(inp.cache_len.astype(np.int32)).cuda(),
                block_table=torch.from_numpy(inp.block_table.view(np.int32)).cuda())


def gpu_fp8(inp, split_len, window=0, t=None, paged=True):
    import flash_attention_forward_amd as F

    torch = torch_cuda()
    s = inp.spec
    t = t or fp8_tensors(inp)
    o = F.decode(t["q"], t["k"], t["v"], t["cache_len"], block_table=t["block_table"] if paged else None,
                 scale=s.scale_f32, window=window, split_len=split_len, max_len=s.max_pages_per_seq * s.page_size,
                 k_scale=s.k_scale, v_scale=s.v_scale)
    torch.cuda.synchronize()
    return host64(o, s.dtype)


def oracle_fp8(inp, batches=None, window=0):
    s = inp.spec
    kp = np.float64(np.float32(s.k_scale)) * W.as_f64(inp.k_pool, "fp8")
    vp = np.float64(np.float32(s.v_scale)) * W.as_f64(inp.v_pool, "fp8")
    return oracle.decode(W.as_f64(inp.q, s.dtype), kp, vp, inp.block_table, inp.cache_len, s.scale_f32,
                         window=window, batches=batches)


def small(seed, **kw):
    base = dict(batch=6, len_lo=1, len_hi=1500)
    base.update(kw)
    return W.make_decode(W.shrink(W.FP8_DECODE, **base), seed)


@pytest.mark.parametrize("split_len", [16, 64, 512, 1024])
def test_fp8_decode_parity_split_lens(split_len):
    inp = small(1)
    say("fp8 decode split_len", split_len)
    ref, bound = decode_with_bound(inp)
    check(gpu_fp8(inp, split_len), ref, "bf16", f"fp8 split {split_len}", bound=bound)


@pytest.mark.parametrize("kw", [
    dict(head_dim=64), dict(head_dim=256), dict(dtype="f16"), dict(n_q_heads=8, n_kv_heads=8),
    dict(n_q_heads=16, n_kv_heads=1), dict(page_size=32), dict(page_size=8), dict(page_size=1, len_hi=300),
    dict(s_active=4, len_lo=4), dict(k_scale=0.03125, v_scale=3.0), dict(k_scale=0.37, v_scale=0.011),
    dict(s_active=8, len_lo=8), dict(s_active=3, n_q_heads=32, n_kv_heads=4, len_lo=3),  # > 16 rows per kv-head
])
def test_fp8_decode_parity_variants(kw):
    inp = small(2, **kw)
    say("fp8 decode variant", kw)
    split = 64 if inp.spec.page_size <= 64 else inp.spec.page_size
    ref, bound = decode_with_bound(inp)
    check(gpu_fp8(inp, split), ref, inp.spec.dtype, str(kw), bound=bound)


@pytest.mark.parametrize("window", [1, 100, 700])
def test_fp8_decode_window(window):
    inp = small(3, s_active=2, len_lo=2)
    say("fp8 decode window", window)
    ref, bound = decode_with_bound(inp, window=window)
    check(gpu_fp8(inp, 128, window=window), ref, "bf16", f"fp8 w={window}", bound=bound)


def test_fp8_decode_flat_matches_paged_bitwise():
    torch = torch_cuda()
    inp = small(4)
    s = inp.spec
    say("fp8 decode flat")
    maxlen = s.max_pages_per_seq * s.page_size
    t = fp8_tensors(inp)
    kf = t["k"].view(torch.uint8)[t["block_table"].long()].reshape(s.batch, maxlen, s.n_kv_heads, s.head_dim)
    vf = t["v"].view(torch.uint8)[t["block_table"].long()].reshape(s.batch, maxlen, s.n_kv_heads, s.head_dim)
    flat = dict(t, k=kf.view(torch.float8_e4m3fn), v=vf.view(torch.float8_e4m3fn))
    a = gpu_fp8(inp, 256, t=flat, paged=False)
    b = gpu_fp8(inp, 256, t=t)
    np.testing.assert_array_equal(a, b)
    check(a, oracle_fp8(inp), "bf16", "fp8 flat")


def test_fp8_decode_eight_and_four_head_workgroups_bitwise():
    """The launch takes eight kv-heads per workgroup on grids of at least 512 workgroups and four
    below; a workspace with more splits than needed widens the grid (the extra splits are empty), so
    the same call runs both shapes, which must give the same bits (each wave's arithmetic is the same)."""
    import flash_attention_forward_amd as F

    torch = torch_cuda()
    inp = small(7, batch=8, len_lo=1, len_hi=4000)
    s = inp.spec
    say("fp8 decode eight vs four heads per workgroup")
    t = fp8_tensors(inp)
    maxlen = s.max_pages_per_seq * s.page_size
    ms = F.attn.max_splits_for(maxlen, 256)
    assert F.decode_heads_per_workgroup(s.batch, s.n_kv_heads, s.head_dim, ms, fp8_kv=True) == 4
    assert F.decode_heads_per_workgroup(s.batch, s.n_kv_heads, s.head_dim, 64, fp8_kv=True) == 8
    outs = []
    for splits in (ms, 64):
        ws = F.DecodeWorkspace(s.batch, s.s_active, s.n_q_heads, s.head_dim, splits, "cuda")
        o = F.decode(t["q"], t["k"], t["v"], t["cache_len"], block_table=t["block_table"], scale=s.scale_f32,
                     split_len=256, max_len=maxlen, workspace=ws, k_scale=s.k_scale, v_scale=s.v_scale)
        torch.cuda.synchronize()
        outs.append(host64(o, s.dtype))
    np.testing.assert_array_equal(outs[0], outs[1])
    ref, bound = decode_with_bound(inp)
    check(outs[1], ref, s.dtype, "fp8 eight heads per workgroup", bound=bound)


def test_fp8_decode_full_size_every_sequence():
    """The paged-decode workload with an FP8 cache, launched as the benchmark launches it, against
    the oracle on all 32 sequences."""
    import bench

    say("fp8 decode full size: generating the cache")
    inp = W.make_decode(W.FP8_DECODE, W.WORKLOAD_SEEDS["paged_decode_b32_d128"])
    say("fp8 decode full size", int(inp.cache_len.sum()))
    got = gpu_fp8(inp, bench.FP8_SPLIT_LEN)
    ref, bound = decode_with_bound(inp)
    check(got, ref, "bf16", "fp8 full size", bound=bound)


def test_fp8_decode_page_permutation_bitwise_and_nan_codes_never_read():
    """Permuting the physical pages (with the table) changes no bit; NaN codes in every slot at or past
    cache_len and in unreferenced pages change no bit either."""
    torch = torch_cuda()
    spec = W.shrink(W.FP8_DECODE, batch=5, len_lo=1, len_hi=900, extra_pages=7)
    inp = W.make_decode(spec, 5)
    say("fp8 permutation / poison")
    base = gpu_fp8(inp, 64)
    rng = np.random.default_rng(6)
    npg = inp.k_pool.shape[0]
    perm = rng.permutation(npg)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(npg)
    moved = W.DecodeInputs(spec, inp.cache_len, inv[inp.block_table].astype(np.uint32), inp.k_pool[perm],
                           inp.v_pool[perm], inp.q)
    # moved.k_pool[inv[p]] == inp.k_pool[p]: page p now lives at inv[p]
    np.testing.assert_array_equal(gpu_fp8(moved, 64), base)
    kp, vp = inp.k_pool.copy(), inp.v_pool.copy()
    used = np.zeros(npg, bool)
    for b in range(spec.batch):
        L = int(inp.cache_len[b])
        pages = inp.block_table[b, : -(-L // spec.page_size)]
        used[pages] = True
        last = int(pages[-1])
        tail = L - (len(pages) - 1) * spec.page_size
        kp[last, tail:], vp[last, tail:] = 0x7F, 0x7F  # NaN codes past cache_len
    kp[~used], vp[~used] = 0xFF, 0xFF
    poisoned = W.DecodeInputs(spec, inp.cache_len, inp.block_table, kp, vp, inp.q)
    np.testing.assert_array_equal(gpu_fp8(poisoned, 64), base)

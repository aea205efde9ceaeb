"""GPU parity of attn_decode_fwd + attn_decode_combine against the fp64 oracle,
plus the bit-exact page-table gather and mask-index checks."""
import numpy as np
import pytest

from flash_attention_forward_amd import workloads as W

from gpu_common import check, decode_tensors, decode_with_bound, gpu_decode, oracle_decode, say, torch_cuda

pytestmark = pytest.mark.gpu

C5 = W.WORKLOADS["paged_decode_b32_d128"]


def small(seed=0, **kw):
    base = dict(batch=6, len_lo=1, len_hi=1500)
    base.update(kw)
    return W.make_decode(W.shrink(C5, **base), seed)


@pytest.mark.parametrize("split_len", [16, 64, 512, 4096])
def test_decode_parity_small(split_len):
    inp = small(1)
    say("decode parity split_len", split_len, inp.cache_len)
    ref, bound = decode_with_bound(inp)
    check(gpu_decode(inp, split_len=split_len), ref, "bf16", f"split {split_len}", bound=bound)


@pytest.mark.parametrize("kw", [
    dict(head_dim=64), dict(head_dim=256), dict(dtype="f16"), dict(n_q_heads=8, n_kv_heads=8),
    dict(n_q_heads=16, n_kv_heads=1), dict(page_size=32), dict(page_size=8), dict(page_size=1, len_hi=300),
    dict(s_active=4, len_lo=4), dict(s_active=2, n_q_heads=16, n_kv_heads=2, len_lo=2),
    # more than 16 query rows per kv-head: a second 16-column MFMA block
    dict(s_active=8, len_lo=8), dict(s_active=3, n_q_heads=32, n_kv_heads=4, len_lo=3),
    dict(s_active=6, head_dim=64, len_lo=6), dict(s_active=5, dtype="f16", len_lo=5, page_size=8),
])
def test_decode_parity_variants(kw):
    inp = small(2, **kw)
    say("decode variant", kw)
    split = 64 if inp.spec.page_size <= 64 else inp.spec.page_size
    ref, bound = decode_with_bound(inp)
    check(gpu_decode(inp, split_len=split), ref, inp.spec.dtype, str(kw), bound=bound)


@pytest.mark.parametrize("window", [1, 100, 700])
def test_decode_window(window):
    inp = small(3, s_active=2, len_lo=2)
    say("decode window", window)
    ref, bound = decode_with_bound(inp, window=window)
    check(gpu_decode(inp, split_len=128, window=window), ref, "bf16", f"w={window}", bound=bound)


def test_decode_flat_cache():
    """block_table = NULL: k/v are [batch, max_len, Hkv, D]."""
    torch = torch_cuda()
    import flash_attention_forward_amd as F

    inp = small(4)
    s = inp.spec
    say("decode flat")
    maxlen = s.max_pages_per_seq * s.page_size
    kf = np.zeros((s.batch, maxlen, s.n_kv_heads, s.head_dim), np.uint16)
    vf = np.zeros_like(kf)
    for b in range(s.batch):
        for p in range(s.max_pages_per_seq):
            kf[b, p * s.page_size:(p + 1) * s.page_size] = inp.k_pool[inp.block_table[b, p]]
            vf[b, p * s.page_size:(p + 1) * s.page_size] = inp.v_pool[inp.block_table[b, p]]
    t = decode_tensors(inp)
    o = F.decode(t["q"], W.to_torch(kf, "bf16", "cuda"), W.to_torch(vf, "bf16", "cuda"), t["cache_len"],
                 scale=s.scale_f32, split_len=256)
    o_paged = F.decode(t["q"], t["k"], t["v"], t["cache_len"], block_table=t["block_table"], scale=s.scale_f32,
                       split_len=256)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_paged.view(torch.int16))
    check(W.as_f64(W.from_torch(o, "bf16"), "bf16"), oracle_decode(inp), "bf16", "flat")


def test_decode_full_size_every_sequence():
    """The full paged-decode workload, launched as the benchmark does, against the oracle on all
    32 sequences (the fixed tolerances and the derived per-element bound)."""
    name = "paged_decode_b32_d128"
    inp = W.make_decode(C5, W.WORKLOAD_SEEDS[name])
    say("decode full size", int(inp.cache_len.sum()))
    import bench

    got = gpu_decode(inp, split_len=bench.DEFAULT_SPLIT_LEN)
    ref, bound = decode_with_bound(inp)
    check(got, ref, "bf16", name, bound=bound)


def test_page_permutation_bitwise():
    """Random-permutation page table == identity table with the pages moved accordingly."""
    torch = torch_cuda()
    import flash_attention_forward_amd as F

    inp = small(5)
    s = inp.spec
    say("page permutation")
    t = decode_tensors(inp)
    o1 = F.decode(t["q"], t["k"], t["v"], t["cache_len"], block_table=t["block_table"], scale=s.scale_f32,
                  split_len=128)
    B, maxp = inp.block_table.shape
    ident = np.arange(B * maxp, dtype=np.uint32).reshape(B, maxp)
    kp = inp.k_pool[inp.block_table.reshape(-1)]
    vp = inp.v_pool[inp.block_table.reshape(-1)]
    o2 = F.decode(t["q"], W.to_torch(kp, "bf16", "cuda"), W.to_torch(vp, "bf16", "cuda"), t["cache_len"],
                  block_table=torch.from_numpy(ident.view(np.int32)).cuda(), scale=s.scale_f32, split_len=128)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_tail_slots_and_unreferenced_pages_never_leak():
    """NaN in page slots at or beyond cache_len, in pages no sequence references, and in
    block-table entries past the last used page changes nothing (bit-exact)."""
    torch = torch_cuda()
    import flash_attention_forward_amd as F

    spec = W.shrink(C5, batch=5, len_lo=1, len_hi=700, extra_pages=4)
    inp = W.make_decode(spec, 6)
    s = inp.spec
    say("tail poison")
    t = decode_tensors(inp)
    o1 = F.decode(t["q"], t["k"], t["v"], t["cache_len"], block_table=t["block_table"], scale=s.scale_f32,
                  split_len=64)
    used = np.zeros(inp.k_pool.shape[:2], bool)
    for b in range(s.batch):
        for tok in range(inp.cache_len[b]):
            used[inp.block_table[b, tok // s.page_size], tok % s.page_size] = True
    nan16 = W.round_to(np.array([np.nan], np.float32), "bf16")[0]
    kp, vp = inp.k_pool.copy(), inp.v_pool.copy()
    kp[~used] = nan16
    vp[~used] = nan16
    bt = inp.block_table.copy()
    for b in range(s.batch):  # entries past the last page point at a NaN-filled unreferenced page
        bt[b, -(-int(inp.cache_len[b]) // s.page_size):] = int(np.nonzero(~used.any(axis=1))[0][0])
    o2 = F.decode(t["q"], W.to_torch(kp, "bf16", "cuda"), W.to_torch(vp, "bf16", "cuda"), t["cache_len"],
                  block_table=torch.from_numpy(bt.view(np.int32)).cuda(), scale=s.scale_f32, split_len=64)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_needles_name_the_gathered_slot():
    """A needle key at logical token t of sequence b returns that slot's V bit-exactly; V rows
    encode (page, slot) as exact bf16 integers, so the output names the slot the gather read."""
    torch = torch_cuda()
    import flash_attention_forward_amd as F

    spec = W.shrink(C5, batch=4, n_q_heads=4, n_kv_heads=1, len_lo=40, len_hi=300)
    inp = W.make_decode(spec, 7)
    s = inp.spec
    npg = inp.k_pool.shape[0]
    vcode = np.zeros(inp.v_pool.shape, np.float32)
    vcode[..., 0] = np.arange(npg)[:, None, None] + 1
    vcode[..., 1] = np.arange(s.page_size)[None, :, None] + 1
    v = W.to_torch(W.round_to(vcode, "bf16"), "bf16", "cuda")
    q64 = W.as_f64(inp.q, "bf16")
    t = decode_tensors(inp)
    say("decode needles")
    for b in range(s.batch):
        L = int(inp.cache_len[b])
        for tok in sorted({0, 15, 16, L // 2, L - 17, L - 16, L - 1}):
            if tok < 0:
                continue
            kp = np.zeros(inp.k_pool.shape, np.float32)
            pg, sl = inp.block_table[b, tok // s.page_size], tok % s.page_size
            qv = q64[b, 0, 0]
            kp[pg, sl, 0] = 300.0 * qv / (qv @ qv) / s.scale_f32
            o = F.decode(t["q"], W.to_torch(W.round_to(kp, "bf16"), "bf16", "cuda"), v, t["cache_len"],
                         block_table=t["block_table"], scale=s.scale_f32, split_len=64)
            torch.cuda.synchronize()
            got = o[b, 0, 0, :2].float().cpu().numpy()
            assert got[0] == pg + 1 and got[1] == sl + 1, (b, tok, got, pg, sl)


def test_split_len_invariance():
    inp = small(8, len_lo=500, len_hi=3000)
    say("split_len invariance")
    outs = [gpu_decode(inp, split_len=sl) for sl in (16, 256, 512, 4096)]
    for o in outs[1:]:
        assert np.abs(o - outs[0]).max() <= 2 ** -7 * np.abs(outs[0]).max()


def test_decode_partials_match_oracle_lse():
    """attn_decode_fwd alone: each split's output and natural-log LSE equal the oracle's
    attention over that split's keys."""
    torch = torch_cuda()
    import oracle
    import flash_attention_forward_amd as F

    inp = small(9, batch=3, len_lo=100, len_hi=700)
    s = inp.spec
    split = 128
    ms = -(-s.max_pages_per_seq * s.page_size // split)
    t = decode_tensors(inp)
    ws = F.DecodeWorkspace(s.batch, 1, s.n_q_heads, s.head_dim, ms, "cuda")
    say("decode partials")
    F.attn_decode_fwd(t["q"], t["k"], t["v"], t["cache_len"], ws.part_o, ws.part_lse, split, ms, s.scale_f32,
                      t["block_table"])
    torch.cuda.synchronize()
    po, pl = ws.part_o.cpu().numpy(), ws.part_lse.cpu().numpy()
    f64 = lambda a: W.as_f64(a, "bf16")
    for b in range(s.batch):
        L = int(inp.cache_len[b])
        kb = f64(oracle.gather_paged(inp.k_pool, inp.block_table[b], L))[None]
        vb = f64(oracle.gather_paged(inp.v_pool, inp.block_table[b], L))[None]
        for sp in range(-(-L // split)):
            a, e = sp * split, min(L, (sp + 1) * split)
            o, lse = oracle.attention(f64(inp.q[b:b + 1]), np.ascontiguousarray(kb[:, a:e]),
                                      np.ascontiguousarray(vb[:, a:e]), s.scale_f32, False, return_lse=True)
            check(po[b, 0, :, sp], o[0, 0], "bf16", f"partial b{b} s{sp}")
            assert np.abs(pl[b, 0, :, sp] - lse[0, 0]).max() <= 1e-3 * max(1.0, np.abs(lse).max())


def test_decode_repeated_runs_bit_identical():
    torch = torch_cuda()
    import flash_attention_forward_amd as F

    inp = small(10, batch=8, len_lo=1000, len_hi=5000)
    t = decode_tensors(inp)
    say("decode repeated runs")
    ref = F.decode(t["q"], t["k"], t["v"], t["cache_len"], block_table=t["block_table"], scale=inp.spec.scale_f32)
    for _ in range(30):
        o = F.decode(t["q"], t["k"], t["v"], t["cache_len"], block_table=t["block_table"], scale=inp.spec.scale_f32)
        assert torch.equal(o.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("window", [3, 200])
def test_decode_many_rows_window_and_flat(window):
    """32 rows per kv-head (8 tokens x 4 q-heads) with a window, paged and through a flat copy (bitwise equal)."""
    torch = torch_cuda()
    import flash_attention_forward_amd as F

    inp = small(3, s_active=8, len_lo=8)
    s = inp.spec
    say("decode 32 rows window", window)
    maxlen = s.max_pages_per_seq * s.page_size
    kf = np.zeros((s.batch, maxlen, s.n_kv_heads, s.head_dim), np.uint16)
    vf = np.zeros_like(kf)
    for b in range(s.batch):
        for p in range(s.max_pages_per_seq):
            kf[b, p * s.page_size:(p + 1) * s.page_size] = inp.k_pool[inp.block_table[b, p]]
            vf[b, p * s.page_size:(p + 1) * s.page_size] = inp.v_pool[inp.block_table[b, p]]
    t = decode_tensors(inp)
    o_paged = F.decode(t["q"], t["k"], t["v"], t["cache_len"], block_table=t["block_table"], scale=s.scale_f32,
                       window=window, split_len=64)
    o_flat = F.decode(t["q"], W.to_torch(kf, "bf16", "cuda"), W.to_torch(vf, "bf16", "cuda"), t["cache_len"],
                      scale=s.scale_f32, window=window, split_len=64)
    torch.cuda.synchronize()
    assert torch.equal(o_flat.view(torch.int16), o_paged.view(torch.int16))
    check(W.as_f64(W.from_torch(o_paged, "bf16"), "bf16"), oracle_decode(inp, window=window), "bf16",
          f"32 rows window {window}")


def expected_problems(table, cache_len, page_size, num_pages):
    """Count and lowest flat index of the problems attn_decode_validate_pages reports (plain numpy)."""
    B, maxp = table.shape
    bad = []
    for b in range(B):
        L = int(cache_len[b])
        if L < 0 or L > maxp * page_size:
            bad.append(b * maxp)
            continue
        n = -(-L // page_size)
        bad += [b * maxp + i for i in range(n) if int(table[b, i]) >= num_pages]
    return len(bad), (min(bad) if bad else 2**31 - 1)


def test_validate_pages_accepts_the_workload_and_finds_planted_errors():
    torch = torch_cuda()
    import flash_attention_forward_amd as F

    inp = W.make_decode(C5, W.WORKLOAD_SEEDS["paged_decode_b32_d128"])
    s = inp.spec
    num_pages = inp.k_pool.shape[0]
    t = decode_tensors(inp)
    say("validate pages: workload table")
    r = F.attn_decode_validate_pages(t["block_table"], t["cache_len"], s.page_size, num_pages).cpu().tolist()
    assert r == [0, 2**31 - 1]
    # planted: out-of-range entries inside used pages, others past the used pages (not checked),
    # and two sequences whose cache_len does not fit their row
    table = inp.block_table.copy()
    cl = inp.cache_len.astype(np.int32).copy()
    rng = np.random.default_rng(5)
    for b in rng.choice(s.batch, 6, replace=False):
        used = -(-int(cl[b]) // s.page_size)
        table[b, rng.integers(0, used)] = num_pages + int(rng.integers(0, 1000))
        if used < table.shape[1]:
            table[b, used] = 0xFFFFFFFF  # past the used pages: ignored
    cl[3] = -5
    cl[7] = table.shape[1] * s.page_size + 1
    want = expected_problems(table, cl, s.page_size, num_pages)
    say("validate pages: planted", want)
    r = F.attn_decode_validate_pages(torch.from_numpy(table.view(np.int32)).cuda(), torch.from_numpy(cl).cuda(),
                                     s.page_size, num_pages).cpu().tolist()
    assert tuple(r) == want and want[0] >= 6

"""Mask index logic of the prefill, bit-exact, on the launch shapes the full-size
workloads take: the eight-wave 256-row launch (D = 64 and 128, with and without
the kv-head chunking across XCDs), the four-wave launch at D = 64 and 128, the
paired-wave D = 256 launch and its persistent form,
causal and sliding-window masks, Sq < Skv, packed sequences and FP8 K/V.

* Masked-key poison inside loaded tiles. Keys above a cut (causal) and below a
  cut (window) are overwritten with random finite values, and so are the keys
  of the same tiles: the rows whose visible keys all lie between the cuts load
  those tiles (diagonal and window-edge tiles) but must stay bit-identical to
  the unpoisoned run. Masked columns contribute nothing to the numerator or to
  the running sum ("Flash-Attention: Context (CTE)", section "The masking").
* Needles. Key j* set to a multiple of query row i's direction (score about
  300 above every other key of that row, so every other probability underflows
  to exactly 0): o_i must equal v[j*] bit for bit when j* is visible to row i,
  and be bit-identical to the run without the needle when it is masked. j*
  sweeps key-tile (64), wave (32), query-tile (128 / 256), diagonal and window
  edges (CTE page, "Algorithm — compute-skip" and "the diagonal affine_select
  mask").
* Decode: finite poison in keys before the window of the earliest query and
  in the later speculative tokens changes no bit of the rows that cannot see
  them.
"""
import numpy as np
import pytest

from flash_attention_forward_amd import workloads as W

from gpu_common import decode_tensors, say, torch_cuda

pytestmark = pytest.mark.gpu

# Launch shapes: the dispatch takes eight 32-row waves per workgroup for D <= 128
# when the grid has >= 512 256-row workgroups, else four.
LAUNCHES = {
    # the long-context workload's heads (8 over 1, D128, bf16, causal) at 16K: 512 workgroups of 8 waves
    "wave8_d128_heads8over1_16k": W.PrefillSpec(1, 8, 1, 16384, 16384, 128, "bf16", causal=True),
    # 8 waves with the kv-head chunks dealt to XCDs (batch * n_kv_heads = 8)
    "wave8_d128_gqa_xcd_4k": W.PrefillSpec(4, 8, 2, 4096, 4096, 128, "bf16", causal=True),
    "wave8_d128_f16_window_4k": W.PrefillSpec(2, 16, 4, 4096, 4096, 128, "f16", causal=True, window=1000),
    "wave8_d64_f16_window_4k": W.PrefillSpec(2, 16, 2, 4096, 4096, 64, "f16", causal=True, window=300),
    # the D = 256 sliding-window launch (paired waves, one workgroup per CU)
    "wave4_d256_window": W.PrefillSpec(2, 4, 2, 1500, 1500, 256, "bf16", causal=True, window=333),
    "wave4_d256_f16_causal": W.PrefillSpec(1, 2, 1, 900, 900, 256, "f16", causal=True),
    "wave4_d64_f16_causal": W.PrefillSpec(1, 4, 1, 700, 700, 64, "f16", causal=True),
    "wave4_d128_window_sq_lt_skv": W.PrefillSpec(2, 4, 2, 400, 900, 128, "bf16", causal=True, window=200),
    # the four-wave launch of the 2K f16 prefill (one round of causal row tiles), and D64 with a window
    "wave4_f16_gqa_causal_2k": W.PrefillSpec(1, 8, 2, 2048, 2048, 128, "f16", causal=True),
    "wave4_bf16_d64_window_1k": W.PrefillSpec(2, 4, 2, 1200, 1200, 64, "bf16", causal=True, window=400),
    # the persistent D = 256 launch (512 q tiles, one workgroup per CU walking its tiles): a window
    # that is not a multiple of 64, and a cached prefix whose first visible key is past 0
    "persistent_d256_window1000_4k": W.PrefillSpec(2, 8, 4, 4096, 4096, 256, "bf16", causal=True, window=1000),
    "persistent_d256_prefix_window385": W.PrefillSpec(2, 8, 4, 4096, 4608, 256, "bf16", causal=True, window=385),
}
PERSISTENT = [n for n in LAUNCHES if n.startswith("persistent")]


@pytest.mark.parametrize("name", PERSISTENT)
def test_persistent_shapes_take_the_persistent_launch(name):
    import flash_attention_forward_amd as F

    s = LAUNCHES[name]
    assert F.prefill_kernel(s.dtype, s.batch, s.n_q_heads, s.n_kv_heads, s.seqlen_q, s.seqlen_kv, s.head_dim, s.causal,
                            s.window) == "prefill_pair_items"


def random_finite(rng, shape, dtype):
    """Finite poison of mixed magnitudes (up to about 1e4), rounded to dtype."""
    mag = rng.choice(np.array([1e-3, 1.0, 30.0, 1e4], np.float32), size=shape[:-1] + (1,))
    return W.round_to((rng.standard_normal(shape, dtype=np.float32) * mag).astype(np.float32), dtype)


def poison_plan(spec, rng):
    """Per (b, kv-head): key cuts (c_lo, c_hi) not aligned to tiles; keys < c_lo or > c_hi are poisoned.
    Returns [(b, hk, c_lo, c_hi, row_lo, row_hi)], rows [row_lo, row_hi] seeing only keys in [c_lo, c_hi]."""
    Sq, off, w = spec.seqlen_q, spec.seqlen_kv - spec.seqlen_q, spec.window
    plan = []
    for b in range(spec.batch):
        for hk in range(spec.n_kv_heads):
            row_hi = int(rng.integers(max(100, Sq // 3), Sq - 40))
            c_hi = row_hi + off                                # rows up to row_hi see no key above c_hi
            if w > 0:
                lo_min = max(0, w - off)                       # the first row whose window starts above key 0
                row_lo = int(rng.integers(min(lo_min, row_hi - 70), row_hi - 70 + 1))
                c_lo = max(0, row_lo + off - w + 1)            # rows from row_lo on see no key below c_lo
            else:
                row_lo, c_lo = 0, 0
            plan.append((b, hk, c_lo, c_hi, row_lo, row_hi))
    return plan


@pytest.mark.parametrize("name", list(LAUNCHES))
def test_masked_poison_inside_tiles_bit_exact(name):
    torch = torch_cuda()
    import flash_attention_forward_amd as F

    spec = LAUNCHES[name]
    inp = W.make_prefill(spec, seed=300 + len(name))
    dt = spec.dtype
    q, k, v = (W.to_torch(a, dt, "cuda") for a in (inp.q, inp.k, inp.v))
    base = F.prefill(q, k, v, scale=spec.scale_f32, causal=spec.causal, window=spec.window)
    rng = np.random.default_rng(len(name))
    plan = poison_plan(spec, rng)
    kp, vp = inp.k.copy(), inp.v.copy()
    for b, hk, c_lo, c_hi, _, _ in plan:
        for sl in (slice(c_hi + 1, spec.seqlen_kv), slice(0, c_lo)):
            n = len(range(spec.seqlen_kv)[sl])
            if n:
                kp[b, sl, hk] = random_finite(rng, (n, spec.head_dim), dt)
                vp[b, sl, hk] = random_finite(rng, (n, spec.head_dim), dt)
    say("masked poison", name, [(p[2], p[3]) for p in plan[:4]])
    o = F.prefill(q, W.to_torch(kp, dt, "cuda"), W.to_torch(vp, dt, "cuda"), scale=spec.scale_f32,
                  causal=spec.causal, window=spec.window)
    torch.cuda.synchronize()
    G = spec.n_q_heads // spec.n_kv_heads
    for b, hk, c_lo, c_hi, r0, r1 in plan:
        assert r1 >= r0 + 70, (r0, r1)  # the protected rows span whole tiles and their edges
        heads = slice(hk * G, (hk + 1) * G)
        assert torch.equal(o[b, r0:r1 + 1, heads].view(torch.int16), base[b, r0:r1 + 1, heads].view(torch.int16)), \
            (b, hk, c_lo, c_hi)


def test_masked_poison_packed_sequences_bit_exact():
    """The same on the packed-sequence launch (per-sequence bounds read on the device)."""
    torch = torch_cuda()
    import flash_attention_forward_amd as F

    spec = W.VarlenSpec(6, 8, 2, 128, "bf16", True, 150, 900, window=0, prefix_lo=0, prefix_hi=300)
    inp = W.make_varlen(spec, seed=77)
    q, k, v = (W.to_torch(a, "bf16", "cuda") for a in (inp.q, inp.k, inp.v))
    cq = torch.from_numpy(inp.cu_q.astype(np.int32)).cuda()
    ck = torch.from_numpy(inp.cu_kv.astype(np.int32)).cuda()
    mq, mk = int(inp.lens_q.max()), int(inp.lens_kv.max())

    def run(kk, vv):
        o = torch.empty_like(q)
        F.attn_prefill_varlen_fwd(q, kk, vv, o, cq, ck, mq, mk, spec.scale_f32, True)
        torch.cuda.synchronize()
        return o

    base = run(k, v)
    rng = np.random.default_rng(8)
    kp, vp = inp.k.copy(), inp.v.copy()
    keep = []
    for b in range(spec.batch):
        lq, lk = int(inp.lens_q[b]), int(inp.lens_kv[b])
        c_hi = int(rng.integers(lk - lq + 40, lk - 20))  # keys past c_hi of this sequence are poisoned
        k0 = int(inp.cu_kv[b])
        n = lk - 1 - c_hi
        kp[k0 + c_hi + 1:k0 + lk] = random_finite(rng, (n, spec.n_kv_heads, spec.head_dim), "bf16")
        vp[k0 + c_hi + 1:k0 + lk] = random_finite(rng, (n, spec.n_kv_heads, spec.head_dim), "bf16")
        keep.append((int(inp.cu_q[b]), int(inp.cu_q[b]) + c_hi - (lk - lq)))  # rows at positions <= c_hi
    say("masked poison, packed", inp.lens_q.tolist())
    o = run(W.to_torch(kp, "bf16", "cuda"), W.to_torch(vp, "bf16", "cuda"))
    for r0, r1 in keep:
        assert torch.equal(o[r0:r1 + 1].view(torch.int16), base[r0:r1 + 1].view(torch.int16)), (r0, r1)


@pytest.mark.parametrize("shape", ["wave8", "wave4_d256_window"])
def test_masked_poison_fp8_kv_bit_exact(shape):
    """The same for attn_prefill_fwd_fp8kv: finite E4M3 codes (never 0x7F / 0xFF) as poison."""
    torch = torch_cuda()
    import flash_attention_forward_amd as F

    spec = LAUNCHES["wave8_d128_gqa_xcd_4k" if shape == "wave8" else "wave4_d256_window"]
    rng = np.random.default_rng(12)
    B, Sq, Hq, Hkv, D = spec.batch, spec.seqlen_q, spec.n_q_heads, spec.n_kv_heads, spec.head_dim
    q = W.to_torch(W.normal_rounded(rng, (B, Sq, Hq, D), spec.dtype), spec.dtype, "cuda")
    k8 = W.normal_rounded(rng, (B, spec.seqlen_kv, Hkv, D), "fp8", divide_by=0.5)
    v8 = W.normal_rounded(rng, (B, spec.seqlen_kv, Hkv, D), "fp8", divide_by=0.25)

    def run(kk, vv):
        o = F.prefill(q, W.to_torch(kk, "fp8", "cuda"), W.to_torch(vv, "fp8", "cuda"), scale=spec.scale_f32,
                      causal=True, window=spec.window, k_scale=0.5, v_scale=0.25)
        torch.cuda.synchronize()
        return o

    base = run(k8, v8)
    plan = poison_plan(spec, rng)
    kp, vp = k8.copy(), v8.copy()
    for b, hk, c_lo, c_hi, _, _ in plan:
        for sl in (slice(c_hi + 1, spec.seqlen_kv), slice(0, c_lo)):
            n = len(range(spec.seqlen_kv)[sl])
            codes = rng.integers(0, 256, size=(2, n, D)).astype(np.uint8)
            codes[(codes & 0x7F) == 0x7F] = 0x3C  # no NaN codes: finite poison only
            kp[b, sl, hk], vp[b, sl, hk] = codes[0], codes[1]
    say("masked poison, fp8 k/v", shape)
    o = run(kp, vp)
    G = Hq // Hkv
    for b, hk, _, _, r0, r1 in plan:
        heads = slice(hk * G, (hk + 1) * G)
        assert torch.equal(o[b, r0:r1 + 1, heads].view(torch.int16), base[b, r0:r1 + 1, heads].view(torch.int16))


def needle_cases(spec):
    """(query row, key) pairs around key-tile, wave, query-tile, diagonal and window edges."""
    Sq, Skv, w = spec.seqlen_q, spec.seqlen_kv, spec.window
    off = Skv - Sq
    rows = {0, 1, 31, 32, 63, 64, 127, 128, 129, 255, 256, 257, 511, 512, Sq // 2 + 17, Sq - 257, Sq - 256,
            Sq - 129, Sq - 128, Sq - 33, Sq - 32, Sq - 1}
    cases = []
    for i in sorted(r for r in rows if 0 <= r < Sq):
        pos = i + off
        t0 = 64 * (pos // 64)
        keys = {0, 63, 64, t0 - 1, t0, t0 + 63, pos - 1, pos, pos + 1, pos + 33, Skv - 1,
                64 * ((pos - 300) // 64), 64 * ((pos - 300) // 64) - 1}
        if w > 0:
            keys |= {pos - w, pos - w + 1, pos - w + 2, 64 * ((pos - w + 1) // 64), 64 * ((pos - w + 1) // 64) - 1,
                     64 * ((pos - w + 1) // 64) + 63}
        cases += [(i, j) for j in sorted(keys) if 0 <= j < Skv]
    return cases


@pytest.mark.parametrize("name", list(LAUNCHES))
def test_needles_on_launch_bit_exact(name):
    torch = torch_cuda()
    import flash_attention_forward_amd as F

    spec = LAUNCHES[name]
    dt = spec.dtype
    inp = W.make_prefill(spec, seed=400 + len(name))
    q64 = W.as_f64(inp.q, dt)
    q, k, v = (W.to_torch(a, dt, "cuda") for a in (inp.q, inp.k, inp.v))
    args = dict(scale=spec.scale_f32, causal=spec.causal, window=spec.window)
    base = F.prefill(q, k, v, **args)
    G = spec.n_q_heads // spec.n_kv_heads
    streams = [(b, hk) for b in range(spec.batch) for hk in range(spec.n_kv_heads)]
    cases = needle_cases(spec)
    off = spec.seqlen_kv - spec.seqlen_q
    say("needles", name, len(cases), "cases")
    for start in range(0, len(cases), len(streams)):
        chunk = cases[start:start + len(streams)]
        kk = k.clone()
        placed = []
        for n, (i, j) in enumerate(chunk):  # one needle per (batch, kv-head) stream and launch
            b, hk = streams[n]
            h = hk * G + (start + n) % G
            qi = q64[b, i, h]
            needle = 300.0 * qi / (qi @ qi) / spec.scale_f32
            kk[b, j, hk] = W.to_torch(W.round_to(needle.astype(np.float32), dt), dt, "cuda")
            placed.append((b, i, h, hk, j))
        o = F.prefill(q, kk, v, **args)
        torch.cuda.synchronize()
        for b, i, h, hk, j in placed:
            pos = i + off
            visible = (not spec.causal or j <= pos) and (spec.window <= 0 or j >= pos - spec.window + 1)
            want = v[b, j, hk] if visible else base[b, i, h]
            assert torch.equal(o[b, i, h].view(torch.int16), want.view(torch.int16)), (b, i, h, j, visible)


@pytest.mark.parametrize("window", [0, 100])
def test_decode_poison_before_window_and_in_later_tokens_bit_exact(window):
    """Decode with four speculative tokens: finite poison in every key before the earliest query's
    window, and in the last active token's K/V (masked for the three earlier queries), changes no
    bit of the rows that cannot see it."""
    torch = torch_cuda()
    import flash_attention_forward_amd as F

    spec = W.shrink(W.WORKLOADS["paged_decode_b32_d128"], batch=6, s_active=4, len_lo=300, len_hi=2500)
    inp = W.make_decode(spec, 21)
    s = inp.spec
    t = decode_tensors(inp)
    args = dict(block_table=t["block_table"], scale=s.scale_f32, window=window, split_len=128)
    base = F.decode(t["q"], t["k"], t["v"], t["cache_len"], **args)
    rng = np.random.default_rng(5)
    kp, vp = inp.k_pool.copy(), inp.v_pool.copy()
    for b in range(s.batch):
        L = int(inp.cache_len[b])
        toks = [L - 1] + (list(range(0, L - s.s_active - window + 1)) if window > 0 else [])
        for tok in toks:
            pg, sl = inp.block_table[b, tok // s.page_size], tok % s.page_size
            kp[pg, sl] = random_finite(rng, (s.n_kv_heads, s.head_dim), "bf16")
            vp[pg, sl] = random_finite(rng, (s.n_kv_heads, s.head_dim), "bf16")
    say("decode poison", window)
    o = F.decode(t["q"], W.to_torch(kp, "bf16", "cuda"), W.to_torch(vp, "bf16", "cuda"), t["cache_len"], **args)
    torch.cuda.synchronize()
    assert torch.equal(o[:, :3].view(torch.int16), base[:, :3].view(torch.int16))


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_decode_never_reads_keys_before_the_window(cache):
    """NaN in every cache slot before the earliest query's window changes no bit: the decode
    kernels clamp the rows of the first block below the window start to visible rows, as they
    clamp rows at or past cache_len."""
    torch = torch_cuda()
    import flash_attention_forward_amd as F

    base_spec = W.WORKLOADS["paged_decode_b32_d128"] if cache == "bf16" else W.FP8_DECODE
    spec = W.shrink(base_spec, batch=6, s_active=2, len_lo=200, len_hi=3000)
    inp = W.make_decode(spec, 23)
    s = inp.spec
    window = 77  # a window start that is not a multiple of the 32-key blocks
    store = "fp8" if cache == "fp8" else "bf16"
    t = dict(decode_tensors(inp)) if cache == "bf16" else None
    if t is None:
        t = dict(q=W.to_torch(inp.q, s.dtype, "cuda"), cache_len=torch.from_numpy(inp.cache_len.astype(np.int32)).cuda(),
                 block_table=torch.from_numpy(inp.block_table.view(np.int32)).cuda())
    args = dict(block_table=t["block_table"], scale=s.scale_f32, window=window, split_len=64, k_scale=s.k_scale,
                v_scale=s.v_scale)
    base = F.decode(t["q"], W.to_torch(inp.k_pool, store, "cuda"), W.to_torch(inp.v_pool, store, "cuda"),
                    t["cache_len"], **args)
    nan = np.uint8(0x7F) if cache == "fp8" else W.round_to(np.array([np.nan], np.float32), "bf16")[0]
    kp, vp = inp.k_pool.copy(), inp.v_pool.copy()
    for b in range(s.batch):
        L = int(inp.cache_len[b])
        for tok in range(0, L - s.s_active - window + 1):
            pg, sl = inp.block_table[b, tok // s.page_size], tok % s.page_size
            kp[pg, sl] = nan
            vp[pg, sl] = nan
    say("decode NaN before the window", cache)
    o = F.decode(t["q"], W.to_torch(kp, store, "cuda"), W.to_torch(vp, store, "cuda"), t["cache_len"], **args)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), base.view(torch.int16))

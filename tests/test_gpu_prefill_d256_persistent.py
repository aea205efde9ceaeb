"""The persistent D = 256 prefill: one workgroup per CU walks its q tiles with the K/V tile
stream running on from one tile into the next (taken for dense window or unmasked launches
whose q tiles each cover an even number of 64-key tiles, with seqlen_kv and the first
visible key on tile boundaries, and at least two tiles per CU).

- Bitwise equality with the per-tile kernel: the same rows sent through the packed-sequence
  entry point (which never takes the persistent path) must give the same bits, since the
  arithmetic per row is the same.
- Oracle parity on sampled rows of four eligible shapes (window, no mask, f16 with as many
  kv-heads as q-heads, a cached prefix whose first visible key is past 0), and with sinks
  and the log-sum-exp.
- NaN in every key before the call's first window changes no bit (those rows are never read).
"""
import numpy as np
import pytest

import oracle
from flash_attention_forward_amd import workloads as W

from gpu_common import attention_with_bound, check, host64, say, torch_cuda

pytestmark = pytest.mark.gpu

# name: (B, Hq, Hkv, Sq, Skv, dtype, window)  (window 0 with mask none: causal=False)
SHAPES = {
    "bf16_window1024_8k": (2, 16, 8, 8192, 8192, "bf16", 1024),
    "bf16_nomask_16k_1k": (1, 4, 2, 16384, 1024, "bf16", 0),
    "f16_window1024_mha_4k": (1, 16, 16, 4096, 4096, "f16", 1024),
    "bf16_prefix_window385": (2, 8, 4, 4096, 4608, "bf16", 385),
    # a ragged last q tile (rows 3968..3999): three of its four wave pairs hold no rows
    "bf16_nomask_ragged_4000": (1, 16, 8, 4000, 1024, "bf16", 0),
}


def eligible(B, Hq, Sq, Skv, window):
    """The host's rule for the persistent launch (D = 256, dense, no positions)."""
    if Skv % 64 or Skv <= 0:
        return False
    n_tiles = -(-Sq // 128)
    if n_tiles * B * Hq < 512:
        return False
    off = Skv - Sq
    if window > 0 and max(0, off - window + 1) % 64:
        return False
    for t in range(n_tiles):
        q0, qlast = 128 * t, min(128 * t + 128, Sq) - 1
        lo, hi = (max(0, q0 + off - window + 1), min(Skv, qlast + off + 1)) if window > 0 else (0, Skv)
        if hi <= lo:
            return False
        nt = -(-hi // 64) - lo // 64
        if nt < 2 or nt % 2:
            return False
    return True


def make(name, seed):
    B, Hq, Hkv, Sq, Skv, dt, w = SHAPES[name]
    spec = W.PrefillSpec(B, Hq, Hkv, Sq, Skv, 256, dt, causal=w > 0, window=w)
    return spec, W.make_prefill(spec, seed)


@pytest.mark.parametrize("name", list(SHAPES))
def test_shapes_take_the_persistent_launch(name):
    import flash_attention_forward_amd as F

    B, Hq, Hkv, Sq, Skv, dt, w = SHAPES[name]
    assert eligible(B, Hq, Sq, Skv, w)
    assert F.prefill_kernel(dt, B, Hq, Hkv, Sq, Skv, 256, w > 0, w) == "prefill_pair_items"


@pytest.mark.parametrize("name", ["bf16_window1024_8k", "bf16_nomask_16k_1k", "bf16_prefix_window385",
                                  "bf16_nomask_ragged_4000"])
def test_persistent_equals_the_per_tile_kernel(name):
    torch = torch_cuda()
    import flash_attention_forward_amd as F

    spec, inp = make(name, 61)
    dt = spec.dtype
    q, k, v = (W.to_torch(a, dt, "cuda") for a in (inp.q, inp.k, inp.v))
    say("persistent vs per-tile", name)
    dense = F.prefill(q, k, v, scale=spec.scale_f32, causal=spec.causal, window=spec.window)
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    packed = F.prefill_varlen(q.reshape(B * Sq, Hq, D), k.reshape(B * Skv, Hkv, D), v.reshape(B * Skv, Hkv, D),
                              [Sq] * B, [Skv] * B, scale=spec.scale_f32, causal=spec.causal, window=spec.window)
    torch.cuda.synchronize()
    assert torch.equal(dense.view(torch.int16), packed.view(B, Sq, Hq, D).view(torch.int16))


@pytest.mark.parametrize("name", list(SHAPES))
def test_persistent_parity_sampled(name):
    torch = torch_cuda()
    import flash_attention_forward_amd as F

    spec, inp = make(name, 62)
    dt = spec.dtype
    say("persistent parity", name)
    o = F.prefill(*(W.to_torch(a, dt, "cuda") for a in (inp.q, inp.k, inp.v)), scale=spec.scale_f32,
                  causal=spec.causal, window=spec.window)
    torch.cuda.synchronize()
    got = host64(o, dt)
    rng = np.random.default_rng(7)
    B, Sq, Hq = spec.batch, spec.seqlen_q, spec.n_q_heads
    edge = [0, 1, 127, 128, 255, 1023, 1024, 1151, Sq // 2, Sq - 129, Sq - 128, Sq - 1]
    ii = np.concatenate([np.array([e for e in edge if 0 <= e < Sq]), rng.integers(0, Sq, 150)])
    rows = np.stack([rng.integers(0, B, len(ii)), ii, rng.integers(0, Hq, len(ii))], axis=1).astype(np.int64)
    ref, bound = attention_with_bound(W.as_f64(inp.q, dt), W.as_f64(inp.k, dt), W.as_f64(inp.v, dt), spec.scale_f32,
                                      spec.causal, spec.window, dt, rows=rows)
    check(got[rows[:, 0], rows[:, 1], rows[:, 2]], ref, dt, name, bound=bound)


def test_persistent_sinks_and_lse():
    torch = torch_cuda()
    import flash_attention_forward_amd as F

    spec, inp = make("bf16_window1024_8k", 63)
    dt = spec.dtype
    sinks = np.random.default_rng(5).uniform(-2.0, 3.0, spec.n_q_heads).astype(np.float32)
    say("persistent sinks and lse")
    o, lse = F.prefill(*(W.to_torch(a, dt, "cuda") for a in (inp.q, inp.k, inp.v)), scale=spec.scale_f32,
                       causal=True, window=spec.window, sinks=torch.from_numpy(sinks).cuda(), return_lse=True)
    torch.cuda.synchronize()
    got, lse = host64(o, dt), lse.cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(8)
    ii = np.concatenate([np.array([0, 127, 128, 1024, spec.seqlen_q - 1]), rng.integers(0, spec.seqlen_q, 100)])
    rows = np.stack([rng.integers(0, spec.batch, len(ii)), ii, rng.integers(0, spec.n_q_heads, len(ii))],
                    axis=1).astype(np.int64)
    q64, k64, v64 = W.as_f64(inp.q, dt), W.as_f64(inp.k, dt), W.as_f64(inp.v, dt)
    ref, bound = attention_with_bound(q64, k64, v64, spec.scale_f32, True, spec.window, dt, rows=rows,
                                      sinks=sinks.astype(np.float64))
    check(got[rows[:, 0], rows[:, 1], rows[:, 2]], ref, dt, "persistent with sinks", bound=bound)
    _, ref_lse = oracle.attention_rows(q64, k64, v64, spec.scale_f32, True, spec.window, rows,
                                       sinks.astype(np.float64))
    assert np.abs(lse[rows[:, 0], rows[:, 1], rows[:, 2]] - ref_lse).max() <= 3e-3


def test_persistent_never_reads_keys_before_the_first_window():
    """Cached prefix of 512 keys with a window of 385: no row sees keys 0..127, which hold NaN."""
    torch = torch_cuda()
    import flash_attention_forward_amd as F

    spec, inp = make("bf16_prefix_window385", 64)
    dt = spec.dtype
    q, k, v = (W.to_torch(a, dt, "cuda") for a in (inp.q, inp.k, inp.v))
    say("persistent, NaN before the first window")
    base = F.prefill(q, k, v, scale=spec.scale_f32, causal=True, window=spec.window)
    first_visible = spec.seqlen_kv - spec.seqlen_q - spec.window + 1
    assert first_visible == 128
    kp, vp = k.clone(), v.clone()
    kp[:, :first_visible] = float("nan")
    vp[:, :first_visible] = float("nan")
    o = F.prefill(q, kp, vp, scale=spec.scale_f32, causal=True, window=spec.window)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), base.view(torch.int16))

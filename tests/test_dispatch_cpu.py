"""Which kernel each call shape launches, from the library's own choice (attn_prefill_kernel_for,
attn_decode_heads_per_workgroup: host arithmetic, the same functions the launches dispatch on), so
that the GPU tests that claim to exercise a launch shape can be checked without a GPU:

* the benchmark workloads take the kernels they are measured as;
* the shapes of the masking, needle and persistent-launch tests take the launch their names say;
* the tests' own replica of the persistent launch's rule agrees with the library's on a sweep;
* the FP8 decode takes eight kv-heads per workgroup on wide grids only;
* arguments the entry points reject are rejected here with the same status.
"""
import numpy as np
import pytest

import flash_attention_forward_amd as F
from flash_attention_forward_amd import attn as A
from flash_attention_forward_amd import workloads as W

from test_gpu_masking_launches import LAUNCHES
from test_gpu_prefill_d256_persistent import SHAPES as PERSISTENT_SHAPES
from test_gpu_prefill_d256_persistent import eligible

MFMA4, MFMA8, PAIR, ITEMS = "prefill_mfma (4 waves)", "prefill_mfma (8 waves)", "prefill_pair", "prefill_pair_items"


def kernel_of(spec, **kw):
    return F.prefill_kernel(spec.dtype, spec.batch, spec.n_q_heads, spec.n_kv_heads, spec.seqlen_q, spec.seqlen_kv,
                            spec.head_dim, spec.causal, spec.window, **kw)


@pytest.mark.parametrize("name,want", [
    ("fp32_d64_s256", "prefill_f32"),
    ("f16_gqa7_causal_2k", MFMA4),
    ("bf16_causal_32k", MFMA8),
    ("bf16_swa1024_d256_8k", ITEMS),
])
def test_benchmark_workloads_take_their_kernels(name, want):
    assert kernel_of(W.WORKLOADS[name]) == want


def test_fp8_and_packed_workloads():
    assert kernel_of(W.WORKLOADS["bf16_causal_32k"], fp8_kv=True) == "prefill_mfma (8 waves, FP8 K/V)"
    assert kernel_of(W.WORKLOADS["bf16_swa1024_d256_8k"], fp8_kv=True) == "prefill_f8kv"
    vs = W.VARLEN_SPEC
    got = F.prefill_kernel(vs.dtype, vs.batch, vs.n_q_heads, vs.n_kv_heads, vs.len_hi, vs.len_hi, vs.head_dim,
                           vs.causal, packed=True)
    assert got == MFMA4  # packed sequences keep four waves


@pytest.mark.parametrize("name", list(LAUNCHES))
def test_masking_launch_shapes_take_the_named_launch(name):
    spec = LAUNCHES[name]
    got = kernel_of(spec)
    if name.startswith("persistent"):
        assert got == ITEMS
    elif name.startswith("wave8"):
        assert got == MFMA8
    elif spec.head_dim == 256:
        assert got == PAIR
    else:
        assert got == MFMA4


@pytest.mark.parametrize("name", list(PERSISTENT_SHAPES))
def test_persistent_test_shapes_take_the_persistent_launch(name):
    B, Hq, Hkv, Sq, Skv, dt, w = PERSISTENT_SHAPES[name]
    assert F.prefill_kernel(dt, B, Hq, Hkv, Sq, Skv, 256, w > 0, w) == ITEMS


def test_persistent_rule_replica_agrees_with_the_library():
    rng = np.random.default_rng(11)
    agree = 0
    for _ in range(400):
        B = int(rng.choice([1, 2, 4]))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        Hq = Hkv * int(rng.choice([1, 2, 4]))
        Sq = int(rng.choice([128, 1000, 2048, 4000, 4096, 8192, 16384]))
        Skv = Sq + int(rng.choice([0, 64, 128, 512, 96]))
        w = int(rng.choice([0, 0, 64, 385, 1000, 1024, 4096]))
        causal = bool(w > 0 or rng.integers(0, 2))
        lib = F.prefill_kernel("bf16", B, Hq, Hkv, Sq, Skv, 256, causal, w)
        assert lib in (PAIR, ITEMS)
        # the replica covers window and unmasked launches (causal-only launches never take it)
        want = ITEMS if ((w > 0 or not causal) and eligible(B, Hq, Sq, Skv, w if causal else 0)) else PAIR
        assert lib == want, (B, Hq, Hkv, Sq, Skv, causal, w)
        agree += lib == ITEMS
    assert agree > 0  # the sweep reached the persistent launch


def test_fp8_decode_heads_per_workgroup():
    import bench

    s = W.WORKLOADS["paged_decode_b32_d128"]
    ms = A.max_splits_for(s.max_pages_per_seq * s.page_size, bench.FP8_SPLIT_LEN)
    assert F.decode_heads_per_workgroup(s.batch, s.n_kv_heads, s.head_dim, ms, fp8_kv=True) == 8  # the benchmark's FP8 launch
    assert F.decode_heads_per_workgroup(8, 8, 128, 16, fp8_kv=True) == 4       # 128 workgroups: not wide
    assert F.decode_heads_per_workgroup(8, 8, 128, 64, fp8_kv=True) == 8       # the same call with 64 splits
    assert F.decode_heads_per_workgroup(32, 8, 128, 8, fp8_kv=False) == 4      # the 16-bit cache
    assert F.decode_heads_per_workgroup(32, 8, 256, 8, fp8_kv=False) == 1
    assert F.decode_heads_per_workgroup(32, 8, 256, 64, fp8_kv=True) == 2
    assert F.decode_heads_per_workgroup(32, 6, 128, 64, fp8_kv=True) == 2      # 6 kv-heads: pairs
    assert F.decode_heads_per_workgroup(0, 8, 128, 8) == 0


def test_rejections_match_the_entry_points():
    L = A.lib()
    args = lambda **kw: [kw.get(k, d) for k, d in (("dtype", A.ATTN_BF16), ("fp8", 0), ("packed", 0), ("pos", 0),
                                                    ("B", 1), ("Hq", 8), ("Hkv", 2), ("Sq", 256), ("Skv", 256),
                                                    ("D", 128), ("causal", 1), ("w", 0))]
    assert L.attn_prefill_kernel_for(*args()) > 0
    assert L.attn_prefill_kernel_for(*args(Hkv=3)) == -1          # n_q_heads % n_kv_heads
    assert L.attn_prefill_kernel_for(*args(D=96)) == -2           # head_dim
    assert L.attn_prefill_kernel_for(*args(causal=0, w=64)) == -2  # window without causal
    assert L.attn_prefill_kernel_for(*args(dtype=A.ATTN_F32, fp8=1)) == -2
    assert L.attn_prefill_kernel_for(*args(dtype=7)) == -1
    assert L.attn_prefill_kernel_for(*args(Sq=0)) == 0            # empty: nothing launched
    assert L.attn_prefill_kernel_name(99) == b"?"

"""bench.py helpers that need no GPU: the committed profile summaries parse, and the
algorithmic work figures match their definitions."""
import bench
from flash_attention_forward_amd import workloads as W


def test_profile_summaries_parse():
    u = bench.utilisation_from_profiles()
    assert isinstance(u, dict)
    for key, row in u.items():
        assert 0.0 <= row["mfma_busy"] <= 1.0 and row["clock_ghz"] > 0
        assert row["frac_of_peak_at_clock"] is None or 0.0 < row["frac_of_peak_at_clock"] <= 1.0
    for key in ("prefill_causal_32k", "decode_paged_b32", "decode_paged_b32_fp8", "prefill_varlen_b16",
                "prefill_swa_d256"):
        t = bench.traffic_from_profiles(key)
        assert t is None or t > 0


def test_prefill_flops_count_visible_pairs():
    # causal S x S: S(S+1)/2 pairs per head, 4 D FLOPs each
    s = W.PrefillSpec(1, 3, 1, 100, 100, 64, "bf16", causal=True)
    assert bench.prefill_flops(s) == 4 * 64 * 3 * 100 * 101 // 2
    # window w: row i sees min(i + 1, w) keys
    s = W.PrefillSpec(2, 1, 1, 50, 50, 128, "bf16", causal=True, window=7)
    assert bench.prefill_flops(s) == 4 * 128 * 2 * sum(min(i + 1, 7) for i in range(50))


def test_bench_refuses_more_than_one_gpu():
    """One GPU only: --gpus 2 exits non-zero with a message, before touching any device."""
    import os
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr

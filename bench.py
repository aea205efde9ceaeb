"""Benchmark of the flash-attention forward hot path on one MI355X.

One step = one long-context causal prefill (8 q-heads over 1 kv-head, 32768
tokens, head_dim 128, bf16, 1% of keys doubled) followed by one paged decode
(32 sequences, 32 q-heads over 8 kv-heads, head_dim 128, bf16, 16-token pages,
cache_len uniform in [1024, 32768]): attn_prefill_fwd, then attn_decode_fwd and
attn_decode_combine, all on one stream with every input resident in HBM.

Prints ONE JSON line. `value` is the prefill's effective TFLOP/s (only visible
(q, k) pairs count, 4*head_dim FLOPs each); the decode's achieved HBM GB/s over
the K/V bytes of tokens below cache_len is reported beside it. Kernel times
come from HIP events recorded on the launch stream around each kernel.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--small-batch-decode]
    python bench.py --calibrate-copy     # plain 1 GiB device copy, for counter scaling
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E, published
PREFILL = "bf16_causal_32k"
DECODE = "paged_decode_b32_d128"
SWA = "bf16_swa1024_d256_8k"
CONTEXT = "f16_gqa7_causal_2k"  # the 7B-shaped 2K prefill the minfer page times
PAGES_CONTEXT_MS_PER_LAYER = 8.5   # minfer 8n page, results: 7B @2K prefill attention, on its own (NVIDIA) GPU
DEFAULT_SPLIT_LEN = 4096  # decode keys per split (timed sweep on the paged workload: 416 us against 420 at 2048
                          # and 448 at 1024 with four kv-heads per workgroup)
FP8_SPLIT_LEN = 2048      # FP8 split sweep (eight kv-heads per workgroup): 1536: 234 us, 1792: 214, 2048: 218,
                          # 2304: 247, 4096: 250; four kv-heads per workgroup: 230 us at 512, 233 at 1024


def visible_pairs(spec) -> int:
    """Visible (query, key) pairs of one (batch, q-head) under the spec's mask."""
    off = spec.seqlen_kv - spec.seqlen_q
    i = np.arange(spec.seqlen_q, dtype=np.int64)
    pos = i + off
    hi = np.minimum(spec.seqlen_kv - 1, pos) if spec.causal else np.full_like(i, spec.seqlen_kv - 1)
    lo = np.maximum(0, pos - spec.window + 1) if spec.window > 0 else np.zeros_like(i)
    return int(np.maximum(0, hi - lo + 1).sum())


def prefill_flops(spec) -> float:
    return 4.0 * spec.head_dim * visible_pairs(spec) * spec.batch * spec.n_q_heads


def decode_kv_bytes(inp) -> int:
    s = inp.spec
    return int(inp.cache_len.astype(np.int64).sum()) * s.n_kv_heads * s.head_dim * 2 * 2


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "flash_attention_forward_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp", ".cpp")):
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def utilisation_from_profiles():
    """MFMA-busy fraction and average shader clock per kernel from the committed counter
    summary (profiles/utilisation.md), while the kernel sources match the ones it was taken with."""
    path = os.path.join(ROOT, "profiles", "utilisation.md")
    out = {}
    if not os.path.exists(path):
        return out
    for line in open(path):
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) == 5 and cells[1] == kernel_source_digest():
            try:
                busy, ghz = float(cells[2]), float(cells[3])
            except ValueError:
                continue
            frac = None if cells[4] == "-" else float(cells[4])
            out[cells[0]] = {"mfma_busy": busy, "clock_ghz": ghz, "frac_of_peak_at_clock": frac}
    return out


def traffic_from_profiles(kernel_key: str):
    """HBM bytes per launch from the committed counter summary (profiles/hbm_traffic.md),
    or None if the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.md")
    if not os.path.exists(path):
        return None
    for line in open(path):
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) == 3 and cells[0] == kernel_key:
            return int(cells[2]) if cells[1] == kernel_source_digest() else None
    return None


def practical_hbm_gbps(stream, ev) -> float:
    """Read + write rate of a plain 1 GiB device copy: the practical HBM line."""
    import torch

    n = 1 << 30
    x = torch.empty(n, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    x.fill_(1)
    for _ in range(3):
        y.copy_(x)
    e = [ev(), ev()]
    e[0].record(stream)
    for _ in range(10):
        y.copy_(x)
    e[1].record(stream)
    torch.cuda.synchronize()
    ms = e[0].elapsed_time(e[1]) / 10
    del x, y
    return 2.0 * n / (ms * 1e-3) / 1e9


def small_batch_decode(ev, batch: int, context: int, steps: int = 50) -> dict:
    """Decode steps of `batch` sequences of `context` tokens each (the paged workload's heads
    and pages) with the split length decode() picks. The steps are recorded into one graph,
    so the events time the GPU and not the host's launch cost."""
    import torch

    import flash_attention_forward_amd as F
    from flash_attention_forward_amd import workloads as W

    spec = W.shrink(W.WORKLOADS[DECODE], batch=batch, len_lo=context, len_hi=context)
    inp = W.make_decode(spec, W.WORKLOAD_SEEDS[DECODE])
    s = inp.spec
    q = W.to_torch(inp.q, s.dtype, "cuda")
    k, v = W.to_torch(inp.k_pool, s.dtype, "cuda"), W.to_torch(inp.v_pool, s.dtype, "cuda")
    cl = torch.from_numpy(inp.cache_len.astype(np.int32)).cuda()
    bt = torch.from_numpy(inp.block_table.view(np.int32)).cuda()
    max_len = s.max_pages_per_seq * s.page_size
    sl = F.auto_split_len(batch, s.n_kv_heads, max_len, s.page_size)
    ws = F.DecodeWorkspace(batch, s.s_active, s.n_q_heads, s.head_dim, F.max_splits_for(max_len, sl), "cuda")
    out = torch.empty_like(q)

    def step():
        F.decode(q, k, v, cl, block_table=bt, scale=s.scale_f32, split_len=sl, max_len=max_len, workspace=ws, out=out)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(steps):
            step()
    g.replay()
    torch.cuda.synchronize()
    e = [ev(), ev()]
    e[0].record()
    g.replay()
    g.replay()
    e[1].record()
    torch.cuda.synchronize()
    us = e[0].elapsed_time(e[1]) * 1e3 / (2 * steps)
    kv = decode_kv_bytes(inp)
    return {"us": round(us, 2), "gbps": round(kv / (us * 1e-6) / 1e9, 1), "split_len": sl}


def calibrate_copy():
    import torch

    n = 1 << 30
    x = torch.empty(n, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    x.fill_(1)
    for _ in range(5):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read": n, "bytes_written": n, "launches": 5}))


def cpu_threads() -> int:
    return int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo) and its logical CPU count."""
    name = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                name = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return f"{name}, {os.cpu_count()} logical CPUs"


def row_pairs(spec, rows) -> float:
    """Visible (query, key) pairs of the given rows (b, i, h) under the spec's mask."""
    pos = rows[:, 1] + (spec.seqlen_kv - spec.seqlen_q)
    hi = np.minimum(spec.seqlen_kv - 1, pos) if spec.causal else np.full_like(pos, spec.seqlen_kv - 1)
    lo = np.maximum(0, pos - spec.window + 1) if spec.window > 0 else np.zeros_like(pos)
    return float(np.maximum(0, hi - lo + 1).sum())


def cpu_baseline(inp, seconds_target: float = 15.0, what: str = "the 32768-token causal prefill"):
    """The fp64 oracle, timed on a bounded random sample of a prefill workload's query rows
    (the whole workload when it takes less than the target)."""
    import oracle
    from flash_attention_forward_amd import workloads as W

    s = inp.spec
    q, k, v = W.as_f64(inp.q, s.dtype), W.as_f64(inp.k, s.dtype), W.as_f64(inp.v, s.dtype)
    rng = np.random.default_rng(0)
    total = s.batch * s.seqlen_q * s.n_q_heads

    def run(n):
        if n >= total:
            rows = oracle.all_rows(s.batch, s.seqlen_q, s.n_q_heads)
        else:
            rows = np.stack([rng.integers(0, s.batch, n), rng.integers(0, s.seqlen_q, n),
                             rng.integers(0, s.n_q_heads, n)], 1)
        t = time.perf_counter()
        oracle.attention_rows(q, k, v, s.scale_f32, s.causal, s.window, rows)
        dt = time.perf_counter() - t
        return len(rows), dt, 4.0 * s.head_dim * row_pairs(s, rows)

    n, dt, fl = run(min(4096, total))  # a pilot large enough that the per-row time is not its start-up cost
    if n < total:
        n, dt, fl = run(int(min(total, 200000, max(256, n * seconds_target / max(dt, 1e-3)))))
    sample = "all" if n >= total else f"{n} random"
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": cpu_threads(), "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"{sample} query rows of {what} (all keys each row sees), {dt:.1f} s wall, fp64, OpenMP over rows"}


def parity_prefill(spec, inp, got_t, n_random: int = 240) -> dict:
    """The timed prefill output against the fp64 oracle on sampled rows (tile and sequence edges of
    every head plus random rows; every row for the fp32 workload): the fixed tolerances, the
    per-row normwise relative error and the ratio to the per-element error bound of the kernels'
    arithmetic (tests/gpu_common.derived_bound)."""
    import oracle
    from flash_attention_forward_amd import workloads as W

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import gpu_common as G

    got = W.as_f64(W.from_torch(got_t, spec.dtype), spec.dtype)
    q, k, v = W.as_f64(inp.q, spec.dtype), W.as_f64(inp.k, spec.dtype), W.as_f64(inp.v, spec.dtype)
    if spec.dtype == "f32":
        ref = oracle.attention(q, k, v, spec.scale_f32, spec.causal, spec.window)
        err = np.abs(got - ref).max() / np.abs(ref).max()
        return {"rows": int(np.prod(got.shape[:3])), "normwise_rel": float(err), "gate": G.F32_NORMWISE,
                "pass": bool(err <= G.F32_NORMWISE)}
    rows = G.sample_rows(spec, n_random=n_random, seed=3)
    ref, bound = G.attention_with_bound(q, k, v, spec.scale_f32, spec.causal, spec.window, spec.dtype, rows=rows)
    sel = got[rows[:, 0], rows[:, 1], rows[:, 2]]
    return parity_record(sel, ref, bound, len(rows))


def parity_record(sel, ref, bound, nrows) -> dict:
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import gpu_common as G

    err = np.abs(sel - ref)
    ratio = float(np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), np.where(err > 0, np.inf, 0.0)).max())
    mx, mean = float(err.max()), float(err.mean())
    ok = bool(np.isfinite(sel).all() and mx <= G.LOWP_MAX_ABS and mean <= G.LOWP_MEAN_ABS and ratio <= 1.0)
    return {"rows": int(nrows), "max_abs": mx, "mean_abs": mean,
            "row_normwise_max": float(G.row_normwise(sel, ref).max()), "bound_ratio_max": ratio, "pass": ok}


def parity_decode(inp, got_t, batches) -> dict:
    """The timed decode output against the fp64 oracle on the given sequences (as parity_prefill)."""
    from flash_attention_forward_amd import workloads as W

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import gpu_common as G

    got = W.as_f64(W.from_torch(got_t, inp.spec.dtype), inp.spec.dtype)[batches]
    ref, bound = G.decode_with_bound(inp, batches=batches)
    return dict(parity_record(got, ref, bound, got.shape[0] * got.shape[1] * got.shape[2]), sequences=list(batches))


def cpu_baseline_decode(inp):
    import oracle
    from flash_attention_forward_amd import workloads as W

    s = inp.spec
    f64 = lambda a: W.as_f64(a, s.dtype)
    order = np.argsort(inp.cache_len)
    batches = [int(order[len(order) // 2]), int(order[-1])]
    t = time.perf_counter()
    oracle.decode(f64(inp.q), inp.k_pool, inp.v_pool, inp.block_table, inp.cache_len, s.scale_f32,
                  batches=batches, to_f64=f64)
    dt = time.perf_counter() - t
    nbytes = int(inp.cache_len[batches].astype(np.int64).sum()) * s.n_kv_heads * s.head_dim * 2 * 2
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": cpu_threads(), "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"sequences {batches} of the paged decode (gather + fp64 attention), {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--split-len", type=int, default=DEFAULT_SPLIT_LEN)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--small-batch-decode", action="store_true",
                    help="also time decode steps of 1 and 4 sequences (graph-recorded)")
    ap.add_argument("--calibrate-copy", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return

    import torch

    import flash_attention_forward_amd as F
    from flash_attention_forward_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = "cuda"

    def log(*a):
        print(*a, file=sys.stderr, flush=True)

    # ---------------------------------------------------------------- inputs (resident in HBM)
    pspec = W.WORKLOADS[PREFILL]
    log("generating", PREFILL)
    pin = W.make_prefill(pspec, W.WORKLOAD_SEEDS[PREFILL])
    q, k, v = (W.to_torch(a, pspec.dtype, dev) for a in (pin.q, pin.k, pin.v))
    o = torch.empty_like(q)

    dspec = W.WORKLOADS[DECODE]
    log("generating", DECODE)
    din = W.make_decode(dspec, W.WORKLOAD_SEEDS[DECODE])
    dq = W.to_torch(din.q, dspec.dtype, dev)
    kc = W.to_torch(din.k_pool, dspec.dtype, dev)
    vc = W.to_torch(din.v_pool, dspec.dtype, dev)
    cl = torch.from_numpy(din.cache_len.astype(np.int32)).to(dev)
    bt = torch.from_numpy(din.block_table.view(np.int32)).to(dev)
    max_len = dspec.max_pages_per_seq * dspec.page_size
    ms = F.attn.max_splits_for(max_len, args.split_len)
    ws = F.DecodeWorkspace(dspec.batch, dspec.s_active, dspec.n_q_heads, dspec.head_dim, ms, dev)
    do = torch.empty_like(dq)

    # the same caches read by four query tokens per sequence (speculative decode),
    # and through a flat [batch, max_len, Hkv, D] copy instead of the page table
    rng = np.random.default_rng(W.WORKLOAD_SEEDS[DECODE] + 100)
    dq4 = W.to_torch(W.round_to(rng.standard_normal((dspec.batch, 4, dspec.n_q_heads, dspec.head_dim),
                                                    dtype=np.float32), dspec.dtype), dspec.dtype, dev)
    # four tokens make the partials four times larger, so fewer, longer splits pay
    # (measured: 483 us at split_len 1024, 456 us at 4096)
    spec_split = 4096
    ms4 = F.attn.max_splits_for(max_len, spec_split)
    ws4 = F.DecodeWorkspace(dspec.batch, 4, dspec.n_q_heads, dspec.head_dim, ms4, dev)
    do4 = torch.empty_like(dq4)
    btl = bt.long()
    kflat = kc[btl].reshape(dspec.batch, max_len, dspec.n_kv_heads, dspec.head_dim)
    vflat = vc[btl].reshape(dspec.batch, max_len, dspec.n_kv_heads, dspec.head_dim)

    cspec = W.WORKLOADS[CONTEXT]
    cin = W.make_prefill(cspec, W.WORKLOAD_SEEDS[CONTEXT])
    cq, ck, cv = (W.to_torch(a, cspec.dtype, dev) for a in (cin.q, cin.k, cin.v))
    co = torch.empty_like(cq)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def step(events=None):
        if events is not None:
            events[0].record(stream)
        F.attn_prefill_fwd(q, k, v, o, pspec.scale_f32, True, 0)
        if events is not None:
            events[1].record(stream)
        F.attn_decode_fwd(dq, kc, vc, cl, ws.part_o, ws.part_lse, args.split_len, ms, dspec.scale_f32, bt)
        if events is not None:
            events[2].record(stream)
        F.attn_decode_combine(ws.part_o, ws.part_lse, cl, args.split_len, ms, do)
        if events is not None:
            events[3].record(stream)

    log("warmup", args.warmup)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[ev() for _ in range(4)] for _ in range(args.steps)]
    log("timing", args.steps, "steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # the outputs of the last timed step, checked against the oracle in the CPU leg below
    o_timed, do_timed = o.cpu(), do.cpu()
    pre_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    split_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    comb_ms = np.array([e[2].elapsed_time(e[3]) for e in evs])
    dec_ms = split_ms + comb_ms

    # 7B-shaped 2K context prefill: 20 back-to-back launches between one event pair, as a model
    # runs its layers (an event pair around each 45 us launch adds the events' own few microseconds).
    # A burst of 20 (about 1 ms) runs at the boost clock; the same 20 after about 4 ms more of
    # back-to-back launches run at the sustained, power-limited clock. Both are reported.
    def ctx_block(n):
        e = [ev(), ev()]
        e[0].record(stream)
        for _ in range(n):
            F.attn_prefill_fwd(cq, ck, cv, co, cspec.scale_f32, True, 0)
        e[1].record(stream)
        return e
    for _ in range(3):
        F.attn_prefill_fwd(cq, ck, cv, co, cspec.scale_f32, True, 0)
    cev = ctx_block(20)
    ctx_block(80)
    cev_s = ctx_block(20)
    torch.cuda.synchronize()
    ctx_ms = cev[0].elapsed_time(cev[1]) / 20
    ctx_sustained_ms = cev_s[0].elapsed_time(cev_s[1]) / 20
    co_timed = co.cpu()

    # sliding window over D = 256 (bf16, B2, 16/8 heads, 8192 tokens, window 1024): 20 back-to-back launches
    wspec = W.WORKLOADS[SWA]
    win = W.make_prefill(wspec, W.WORKLOAD_SEEDS[SWA])
    wq, wk, wv = (W.to_torch(a, wspec.dtype, dev) for a in (win.q, win.k, win.v))
    wo = torch.empty_like(wq)
    for _ in range(30):  # about 12 ms of warm-up: the clock ramps over the first few milliseconds
        F.attn_prefill_fwd(wq, wk, wv, wo, wspec.scale_f32, True, wspec.window)
    wev = [ev(), ev()]
    wev[0].record(stream)
    for _ in range(20):
        F.attn_prefill_fwd(wq, wk, wv, wo, wspec.scale_f32, True, wspec.window)
    wev[1].record(stream)
    torch.cuda.synchronize()
    swa_ms = wev[0].elapsed_time(wev[1]) / 20
    swa_flops = prefill_flops(wspec)
    wo_timed = wo.cpu()
    del wq, wk, wv, wo

    # the 32K causal workload with K and V stored as FP8 E4M3 (attn_prefill_fwd_fp8kv), timed as the
    # main loop times the 16-bit prefill: each launch followed by the paged decode (split + combine),
    # events around the prefill only, 10 steps. Then 10 back-to-back launches of each prefill, which
    # draw more power and run at a lower clock than the alternating steps.
    fks, fvs = W.FP8_PREFILL_SCALES
    k8 = W.to_torch(W.f32_to_e4m3_bits(W.as_f32(pin.k, pspec.dtype) / np.float32(fks)), "fp8", dev)
    v8 = W.to_torch(W.f32_to_e4m3_bits(W.as_f32(pin.v, pspec.dtype) / np.float32(fvs)), "fp8", dev)

    def decode_step():
        F.attn_decode_fwd(dq, kc, vc, cl, ws.part_o, ws.part_lse, args.split_len, ms, dspec.scale_f32, bt)
        F.attn_decode_combine(ws.part_o, ws.part_lse, cl, args.split_len, ms, do)

    for _ in range(5):
        F.attn_prefill_fwd_fp8kv(q, k8, v8, o, pspec.scale_f32, True, 0, fks, fvs)
        decode_step()
    f8ev = [[ev(), ev()] for _ in range(10)]
    for e in f8ev:
        e[0].record(stream)
        F.attn_prefill_fwd_fp8kv(q, k8, v8, o, pspec.scale_f32, True, 0, fks, fvs)
        e[1].record(stream)
        decode_step()
    torch.cuda.synchronize()
    pf8_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in f8ev]))

    def back_to_back(launch, n=10):
        launch()
        e = [ev(), ev()]
        e[0].record(stream)
        for _ in range(n):
            launch()
        e[1].record(stream)
        torch.cuda.synchronize()
        return e[0].elapsed_time(e[1]) / n

    pf8_b2b_ms = back_to_back(lambda: F.attn_prefill_fwd_fp8kv(q, k8, v8, o, pspec.scale_f32, True, 0, fks, fvs))
    pre_b2b_ms = back_to_back(lambda: F.attn_prefill_fwd(q, k, v, o, pspec.scale_f32, True, 0))
    del k8, v8

    # packed prompts of different lengths (attn_prefill_varlen_fwd): 20 back-to-back launches after
    # about 25 ms of warm-up (the power-bound clock is still settling 10 ms after the window launches)
    vspec = W.VARLEN_SPEC
    vin = W.make_varlen(vspec, W.VARLEN_SEED)
    vq, vk, vv = (W.to_torch(a, vspec.dtype, dev) for a in (vin.q, vin.k, vin.v))
    vo = torch.empty_like(vq)
    vcq = torch.from_numpy(vin.cu_q.astype(np.int32)).to(dev)
    vck = torch.from_numpy(vin.cu_kv.astype(np.int32)).to(dev)
    vmq, vmk = int(vin.lens_q.max()), int(vin.lens_kv.max())
    for _ in range(45):
        F.attn_prefill_varlen_fwd(vq, vk, vv, vo, vcq, vck, vmq, vmk, vspec.scale_f32, True)
    vev = [ev(), ev()]
    vev[0].record(stream)
    for _ in range(20):
        F.attn_prefill_varlen_fwd(vq, vk, vv, vo, vcq, vck, vmq, vmk, vspec.scale_f32, True)
    vev[1].record(stream)
    torch.cuda.synchronize()
    varlen_ms = vev[0].elapsed_time(vev[1]) / 20
    # the same launch with every row's position passed explicitly (the default alignment)
    vpos = torch.from_numpy(np.concatenate([np.arange(lq) + lk - lq for lq, lk in zip(vin.lens_q, vin.lens_kv)])
                            .astype(np.int32)).to(dev)
    for _ in range(5):
        F.attn_prefill_varlen_fwd(vq, vk, vv, vo, vcq, vck, vmq, vmk, vspec.scale_f32, True, 0, None, None, vpos)
    vev = [ev(), ev()]
    vev[0].record(stream)
    for _ in range(20):
        F.attn_prefill_varlen_fwd(vq, vk, vv, vo, vcq, vck, vmq, vmk, vspec.scale_f32, True, 0, None, None, vpos)
    vev[1].record(stream)
    torch.cuda.synchronize()
    varlen_pos_ms = vev[0].elapsed_time(vev[1]) / 20
    varlen_flops = 4.0 * vspec.head_dim * vspec.n_q_heads * W.varlen_visible_pairs(vin)
    del vq, vk, vv, vo

    def time_decode(qq, kk, vv, table, w, out, reps=20, split_len=None):
        sl = args.split_len if split_len is None else split_len
        for _ in range(3):
            F.attn_decode_fwd(qq, kk, vv, cl, w.part_o, w.part_lse, sl, w.max_splits, dspec.scale_f32, table)
            F.attn_decode_combine(w.part_o, w.part_lse, cl, sl, w.max_splits, out)
        evv = [[ev(), ev()] for _ in range(reps)]
        for e in evv:
            e[0].record(stream)
            F.attn_decode_fwd(qq, kk, vv, cl, w.part_o, w.part_lse, sl, w.max_splits, dspec.scale_f32, table)
            F.attn_decode_combine(w.part_o, w.part_lse, cl, sl, w.max_splits, out)
            e[1].record(stream)
        torch.cuda.synchronize()
        return float(np.mean([e[0].elapsed_time(e[1]) for e in evv]))

    spec_us = time_decode(dq4, kc, vc, bt, ws4, do4, split_len=spec_split) * 1e3
    # eight draft tokens: 32 query rows per kv-head (two 16-column MFMA blocks per wave)
    dq8 = W.to_torch(W.round_to(rng.standard_normal((dspec.batch, 8, dspec.n_q_heads, dspec.head_dim),
                                                    dtype=np.float32), dspec.dtype), dspec.dtype, dev)
    ws8 = F.DecodeWorkspace(dspec.batch, 8, dspec.n_q_heads, dspec.head_dim, ms4, dev)
    spec8_us = time_decode(dq8, kc, vc, bt, ws8, torch.empty_like(dq8), split_len=spec_split) * 1e3
    del dq8, ws8
    flat_us = time_decode(dq, kflat, vflat, None, ws, torch.empty_like(dq)) * 1e3
    del kflat, vflat

    # the same caches stored as FP8 E4M3 (attn_decode_fwd_fp8kv + combine): the values rounded on the GPU
    kc8, vc8 = kc.to(torch.float8_e4m3fn), vc.to(torch.float8_e4m3fn)
    ms8 = F.attn.max_splits_for(max_len, FP8_SPLIT_LEN)
    wsf = F.DecodeWorkspace(dspec.batch, dspec.s_active, dspec.n_q_heads, dspec.head_dim, ms8, dev)
    for _ in range(3):
        F.attn_decode_fwd_fp8kv(dq, kc8, vc8, cl, wsf.part_o, wsf.part_lse, FP8_SPLIT_LEN, ms8, dspec.scale_f32,
                                block_table=bt)
    fev = [[ev(), ev(), ev()] for _ in range(20)]
    for e in fev:
        e[0].record(stream)
        F.attn_decode_fwd_fp8kv(dq, kc8, vc8, cl, wsf.part_o, wsf.part_lse, FP8_SPLIT_LEN, ms8, dspec.scale_f32,
                                block_table=bt)
        e[1].record(stream)
        F.attn_decode_combine(wsf.part_o, wsf.part_lse, cl, FP8_SPLIT_LEN, ms8, do)
        e[2].record(stream)
    torch.cuda.synchronize()
    fp8_split_us = float(np.mean([e[0].elapsed_time(e[1]) for e in fev])) * 1e3
    fp8_us = float(np.mean([e[0].elapsed_time(e[2]) for e in fev])) * 1e3
    del kc8, vc8, wsf

    # opt-in: these launches share the paged decode's kernel and would dilute its profiled average
    small = ({f"batch{b}_context{c // 1024}k": small_batch_decode(ev, b, c) for b, c in ((1, 4096), (4, 4096), (1, 32768))}
             if args.small_batch_decode else None)

    # the same prefill and decode with an attention sink per q-head and the
    # per-row log-sum-exp written out (attn_prefill_fwd_ex, attn_decode_combine_ex)
    psinks = torch.linspace(-1.0, 2.0, pspec.n_q_heads, device=dev)
    plse = torch.empty((pspec.batch, pspec.seqlen_q, pspec.n_q_heads), dtype=torch.float32, device=dev)
    dsinks = torch.linspace(-1.0, 2.0, dspec.n_q_heads, device=dev)
    dlse = torch.empty((dspec.batch, dspec.s_active, dspec.n_q_heads), dtype=torch.float32, device=dev)
    for _ in range(2):
        F.attn_prefill_fwd_ex(q, k, v, o, pspec.scale_f32, True, 0, plse, psinks)
    # groups of back-to-back launches between two events (the host stays ahead of the GPU),
    # alternating with the same number of plain launches, so that both run at the same clock
    # (back-to-back prefills draw more power than the main loop's, and the clock drifts over
    # the run): medians of three groups each
    n_ex = 8
    ex_groups, plain_groups = [], []
    for _ in range(3):
        plain_groups.append(back_to_back(lambda: F.attn_prefill_fwd(q, k, v, o, pspec.scale_f32, True, 0), n=n_ex))
        ex_groups.append(back_to_back(lambda: F.attn_prefill_fwd_ex(q, k, v, o, pspec.scale_f32, True, 0, plse, psinks),
                                      n=n_ex))
    pre_ex_ms = float(np.median(ex_groups))
    pre_plain_alt_ms = float(np.median(plain_groups))
    # the combine takes a few microseconds, less than one host call: each timed
    # group of combines is queued behind a split, so the GPU never waits for the host
    comb_ex = []
    for _ in range(5):
        cev = [ev(), ev()]
        F.attn_decode_fwd(dq, kc, vc, cl, ws.part_o, ws.part_lse, args.split_len, ms, dspec.scale_f32, bt)
        cev[0].record(stream)
        for _ in range(n_ex):
            F.attn_decode_combine_ex(ws.part_o, ws.part_lse, cl, args.split_len, ms, do, dlse, dsinks)
        cev[1].record(stream)
        torch.cuda.synchronize()
        comb_ex.append(cev[0].elapsed_time(cev[1]) / n_ex)
    comb_ex_us = float(np.median(comb_ex)) * 1e3

    copy_gbps = practical_hbm_gbps(stream, ev)
    flops = prefill_flops(pspec)
    kv_bytes = decode_kv_bytes(din)
    pre_tflops = flops / (pre_ms.mean() * 1e-3) / 1e12
    dec_gbps = kv_bytes / (dec_ms.mean() * 1e-3) / 1e9
    split_gbps = kv_bytes / (split_ms.mean() * 1e-3) / 1e9

    line = {
        "metric": "prefill causal TFLOP/s + decode KV GB/s, % of MI355X peak",
        "value": round(pre_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{PREFILL} + {DECODE}",
            "prefill": "B1 Sq=Skv=32768 Hq8 Hkv1 D128 bf16 causal, 327 K rows x2, scale 1/sqrt(128)",
            "decode": f"B32 s_active1 Hq32 Hkv8 D128 bf16 page16, sum(cache_len)={int(din.cache_len.sum())}, "
                      f"split_len {args.split_len}",
            "prefill_flops": flops,
            "decode_kv_bytes": kv_bytes,
        },
        "prefill_ms": round(float(pre_ms.mean()), 4),
        "decode_us": round(float(dec_ms.mean()) * 1e3, 2),
        "decode_split_us": round(float(split_ms.mean()) * 1e3, 2),
        "decode_combine_us": round(float(comb_ms.mean()) * 1e3, 2),
        "decode": {"value": round(dec_gbps, 1), "unit": "GB/s", "frac_of_peak": round(dec_gbps / PEAK_HBM_GBPS, 4)},
        "roofline": {
            "kernel": "prefill_mfma<bf16, D128, causal>",
            "bound": "mfma",
            "achieved": round(pre_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(pre_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic_from_profiles("prefill_causal_32k"),
        },
        "practical_hbm": {"what": "1 GiB device copy, bytes read + written per second", "gbps": round(copy_gbps, 1),
                          "frac_of_peak": round(copy_gbps / PEAK_HBM_GBPS, 4)},
        "utilisation": utilisation_from_profiles(),
        "roofline_decode": {
            "kernel": "decode_split<bf16, D128>",
            "bound": "hbm",
            "achieved": round(split_gbps, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(split_gbps / PEAK_HBM_GBPS, 4),
            "traffic": traffic_from_profiles("decode_paged_b32"),
        },
        "roofline_decode_fp8": {
            "kernel": "decode_split_f8<bf16 q, D128>",
            "bound": "hbm",
            "achieved": round(kv_bytes / 2 / (fp8_split_us * 1e-6) / 1e9, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(kv_bytes / 2 / (fp8_split_us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
            "traffic": traffic_from_profiles("decode_paged_b32_fp8"),
        },
        "context": {
            "workload": CONTEXT,
            "ms_per_layer": round(ctx_ms, 4),
            "ms_per_layer_sustained": round(ctx_sustained_ms, 4),
            "note": "20 back-to-back launches after 3 warm-up launches (a burst of about 1 ms, at the boost clock); "
                    "sustained: the same 20 after about 4 ms more of back-to-back launches (power-limited clock)",
            "tflops": round(prefill_flops(cspec) / (ctx_ms * 1e-3) / 1e12, 2),
            "roofline": {"bound": "mfma", "achieved": round(prefill_flops(cspec) / (ctx_ms * 1e-3) / 1e12, 2),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(prefill_flops(cspec) / (ctx_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                         "traffic": traffic_from_profiles("prefill_ctx_2k")},
            "pages_ms_per_layer": PAGES_CONTEXT_MS_PER_LAYER,
            "pages_hardware": "unnamed NVIDIA GPU (minfer 8n page); context only",
        },
        "swa_d256": {
            "workload": SWA,
            "flops": swa_flops,
            "ms": round(swa_ms, 4),
            "tflops": round(swa_flops / (swa_ms * 1e-3) / 1e12, 2),
            "note": "B2 Sq=Skv=8192 Hq16 Hkv8 D256 bf16 causal + window 1024; FLOPs over visible pairs only",
            "roofline": {"bound": "mfma", "achieved": round(swa_flops / (swa_ms * 1e-3) / 1e12, 2),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(swa_flops / (swa_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                         "traffic": traffic_from_profiles("prefill_swa_d256")},
        },
        "prefill_fp8kv": {
            "workload": PREFILL,
            "ms": round(pf8_ms, 4),
            "tflops": round(prefill_flops(pspec) / (pf8_ms * 1e-3) / 1e12, 2),
            "ms_back_to_back": round(pf8_b2b_ms, 4),
            "bf16_ms_back_to_back": round(pre_b2b_ms, 4),
            "k_scale": fks,
            "v_scale": fvs,
            "note": "the 32K causal prefill with K and V stored as FP8 E4M3 (per-tensor scales), q and o bf16; "
                    "ms is timed as prefill_ms (each launch followed by the paged decode), the back-to-back "
                    "pair times 10 launches of each kernel in a row",
            "roofline": {"bound": "mfma", "achieved": round(prefill_flops(pspec) / (pf8_ms * 1e-3) / 1e12, 2),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(prefill_flops(pspec) / (pf8_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                         "traffic": traffic_from_profiles("prefill_fp8kv_32k")},
        },
        "varlen": {
            "workload": W.VARLEN,
            "sequences": vspec.batch,
            "total_tokens": int(vin.cu_q[-1]),
            "flops": varlen_flops,
            "ms": round(varlen_ms, 4),
            "tflops": round(varlen_flops / (varlen_ms * 1e-3) / 1e12, 2),
            "ms_with_positions": round(varlen_pos_ms, 4),
            "note": "packed causal prompts, 28/4 heads, D128, bf16, lengths uniform in [256, 4096]",
            "roofline": {"bound": "mfma", "achieved": round(varlen_flops / (varlen_ms * 1e-3) / 1e12, 2),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(varlen_flops / (varlen_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                         "traffic": traffic_from_profiles("prefill_varlen_b16")},
        },
        "sinks_and_lse": {
            "prefill_ex_ms": round(pre_ex_ms, 4),
            "prefill_plain_ms_alternating": round(pre_plain_alt_ms, 4),
            "prefill_ex_tflops": round(prefill_flops(pspec) / (pre_ex_ms * 1e-3) / 1e12, 2),
            "decode_combine_ex_us": round(comb_ex_us, 2),
            "note": "attn_prefill_fwd_ex / attn_decode_combine_ex with one sink per q-head and the lse output; "
                    "the prefill timed in groups of back-to-back launches alternating with groups of the plain "
                    "prefill (prefill_plain_ms_alternating), medians of three groups each",
        },
        "decode_variants": {
            "speculative_s_active4_us": round(spec_us, 2),
            "speculative_s_active4_gbps": round(kv_bytes / (spec_us * 1e-6) / 1e9, 1),
            "speculative_split_len": spec_split,
            "speculative_s_active8_us": round(spec8_us, 2),
            "speculative_s_active8_gbps": round(kv_bytes / (spec8_us * 1e-6) / 1e9, 1),
            "flat_cache_us": round(flat_us, 2),
            "flat_cache_gbps": round(kv_bytes / (flat_us * 1e-6) / 1e9, 1),
            "fp8_kv_split_us": round(fp8_split_us, 2),
            "fp8_kv_us": round(fp8_us, 2),
            "fp8_kv_split_gbps": round(kv_bytes / 2 / (fp8_split_us * 1e-6) / 1e9, 1),
            "fp8_kv_split_frac_of_peak": round(kv_bytes / 2 / (fp8_split_us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
            "fp8_kv_speedup_vs_bf16": round(float(dec_ms.mean()) * 1e3 / fp8_us, 3),
            "note": "split + combine over the same caches: 4 query tokens per sequence, a flat cache copy, and the "
                    "cache stored as FP8 E4M3 (half the bytes)",
        },
        "decode_small_batch": None if small is None else dict(
            small, note="split + combine with decode()'s split length, GPU time per step of 50 steps recorded in "
                        "one graph"),
        "kernel_source_digest": kernel_source_digest(),
    }
    if not args.no_cpu_baseline:
        # the fp32 workload (correctness only: 1.7e7 FLOP), run once for its parity line
        fspec = W.WORKLOADS["fp32_d64_s256"]
        fin = W.make_prefill(fspec, W.WORKLOAD_SEEDS["fp32_d64_s256"])
        fo = F.prefill(*(W.to_torch(a, "f32", dev) for a in (fin.q, fin.k, fin.v)), scale=fspec.scale_f32,
                       causal=fspec.causal)
        fo_timed = fo.cpu()
        log("cpu baseline (oracle)")
        line["cpu_model"] = cpu_model()
        line["cpu_baseline"] = cpu_baseline(pin, seconds_target=12.0)
        line["cpu_baseline_decode"] = cpu_baseline_decode(din)
        line["cpu_baselines"] = {
            "fp32_d64_s256": cpu_baseline(fin, 3.0, "the fp32 256-token workload"),
            CONTEXT: cpu_baseline(cin, 3.0, "the 7B-shaped 2K f16 causal prefill"),
            PREFILL: line["cpu_baseline"],
            SWA: cpu_baseline(win, 3.0, "the D = 256 window-1024 prefill"),
            DECODE: line["cpu_baseline_decode"],
            "note": "the fp64 oracle on the box's host cores; value in each workload's unit (TFLOP/s over the "
                    "sampled rows' visible pairs, GB/s over the sampled sequences' K/V bytes)",
        }
        log("parity of the timed outputs (oracle)")
        order = np.argsort(din.cache_len)
        dec_rows = sorted({int(order[0]), int(order[1]), int(order[-1]), int(order[-2]), int(order[len(order) // 2]),
                           3, 17, 29})
        line["parity"] = {
            "fp32_d64_s256": parity_prefill(fspec, fin, fo_timed),
            CONTEXT: parity_prefill(cspec, cin, co_timed),
            PREFILL: parity_prefill(pspec, pin, o_timed),
            SWA: parity_prefill(wspec, win, wo_timed),
            DECODE: parity_decode(din, do_timed, dec_rows),
            "note": "outputs of the timed launches against the fp64 oracle on sampled rows (tile and sequence "
                    "edges of every head plus random rows; every row of the fp32 workload; 8 whole sequences of "
                    "the decode): the fixed tolerances (max-abs 2e-2, mean-abs 2e-3; fp32 normwise 1e-5) and "
                    "the per-element bound of the kernels' arithmetic (bound_ratio_max <= 1)",
        }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

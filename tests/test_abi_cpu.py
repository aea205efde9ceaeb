"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects malformed arguments with a status code before
making any HIP call (the pointers passed here are never dereferenced)."""
import ctypes
import os
import re
import subprocess

import pytest

from flash_attention_forward_amd import attn as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

INVALID, UNSUPPORTED = 1, 2
FAKE = 0x100000  # 16-byte aligned, never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(attn_\w+)\s*\(", text, flags=re.M)))


def test_header_functions_are_exported():
    names = declared_functions()
    assert names == sorted(A.SYMBOLS)
    L = A.lib()
    for n in names:
        assert getattr(L, n) is not None
    out = subprocess.run(["nm", "-D", "--defined-only", A.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r" T (\w+)$", out, flags=re.M))
    assert set(names) <= exported


def test_status_strings():
    L = A.lib()
    assert L.attn_status_string(0) == b"ok"
    assert L.attn_status_string(1) == b"invalid argument"
    assert L.attn_status_string(2) == b"unsupported configuration"
    assert L.attn_status_string(3) == b"kernel launch failed"
    assert L.attn_status_string(99) == b"unknown status"


def st(b, s, h):
    return A.Strides(b, s, h)


def prefill(**kw):
    a = dict(q=FAKE, qs=st(2048 * 8 * 128, 8 * 128, 128), k=FAKE, ks=st(2048 * 128, 128, 128), v=FAKE,
             vs=st(2048 * 128, 128, 128), o=FAKE, os=st(2048 * 8 * 128, 8 * 128, 128), dtype=A.ATTN_BF16, batch=1,
             hq=8, hkv=1, sq=2048, skv=2048, d=128, scale=0.088, causal=1, window=0)
    a.update(kw)
    return A.lib().attn_prefill_fwd(a["q"], a["qs"], a["k"], a["ks"], a["v"], a["vs"], a["o"], a["os"], a["dtype"],
                                    a["batch"], a["hq"], a["hkv"], a["sq"], a["skv"], a["d"], a["scale"], a["causal"],
                                    a["window"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), INVALID),
    (dict(d=96), UNSUPPORTED),
    (dict(d=512), UNSUPPORTED),
    (dict(hq=6, hkv=4), INVALID),
    (dict(hkv=0), INVALID),
    (dict(window=64, causal=0), UNSUPPORTED),
    (dict(q=FAKE + 2), INVALID),
    (dict(o=0), INVALID),
    (dict(k=0), INVALID),
    (dict(qs=st(2048 * 8 * 128, 8 * 128 + 1, 128)), INVALID),
    (dict(vs=st(-1, 128, 128)), INVALID),
    (dict(batch=-1), INVALID),
    (dict(sq=-5), INVALID),
    (dict(scale=float("nan")), INVALID),
    (dict(scale=float("inf")), INVALID),
    (dict(ks=st(0, 1 << 25, 128)), UNSUPPORTED),               # a 64-row tile would span more than 2^31 elements
    (dict(ks=st(0, 3 << 23, 128)), UNSUPPORTED),               # ... or more than 2^31 bytes of 16-bit values
    (dict(vs=st(0, 3 << 23, 128)), UNSUPPORTED),
    (dict(batch=1 << 20, hq=1 << 12, hkv=1 << 12), UNSUPPORTED),  # more than 2^31 workgroups
])
def test_prefill_rejects(kw, status):
    assert prefill(**kw) == status


@pytest.mark.parametrize("kw", [dict(batch=0), dict(sq=0), dict(hq=0), dict(batch=0, q=0, k=0, v=0, o=0)])
def test_prefill_empty_is_noop(kw):
    assert prefill(**kw) == 0


def decode(**kw):
    a = dict(q=FAKE, qs=st(32 * 128, 32 * 128, 128), k=FAKE, v=FAKE, kvs=st(16 * 8 * 128, 8 * 128, 128), bt=FAKE,
             maxp=2048, ps=16, cl=FAKE, dtype=A.ATTN_BF16, batch=32, sa=1, hq=32, hkv=8, d=128, scale=0.088, window=0,
             po=FAKE, pl=FAKE, split=512, ms=64)
    a.update(kw)
    return A.lib().attn_decode_fwd(a["q"], a["qs"], a["k"], a["v"], a["kvs"], a["bt"], a["maxp"], a["ps"], a["cl"],
                                   a["dtype"], a["batch"], a["sa"], a["hq"], a["hkv"], a["d"], a["scale"],
                                   a["window"], a["po"], a["pl"], a["split"], a["ms"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(split=500), INVALID),          # not a multiple of 16
    (dict(split=0), INVALID),
    (dict(ps=32, split=48), INVALID),    # not a multiple of the page size
    (dict(ms=63), INVALID),              # splits do not cover max_pages * page_size
    (dict(ps=0), INVALID),
    (dict(dtype=A.ATTN_F32), UNSUPPORTED),
    (dict(d=80), UNSUPPORTED),
    (dict(sa=9), UNSUPPORTED),           # 4 q-heads per kv-head x 9 tokens > 32 rows
    (dict(sa=5, d=256), UNSUPPORTED),    # more than 16 rows at head_dim 256
    (dict(hq=30), INVALID),
    (dict(cl=0), INVALID),
    (dict(po=0), INVALID),
    (dict(k=FAKE + 8), INVALID),
    (dict(scale=float("nan")), INVALID),
    (dict(split=16, ms=70000), UNSUPPORTED),   # more splits than a grid dimension holds
    (dict(batch=70000), UNSUPPORTED),          # more sequences than a grid dimension holds
])
def test_decode_rejects(kw, status):
    assert decode(**kw) == status


def test_decode_flat_ignores_page_args():
    # flat cache: page_size/max_pages are not checked, but split_len still is
    assert decode(bt=0, ps=0, maxp=0, split=24) == INVALID


@pytest.mark.parametrize("kw", [dict(batch=0), dict(sa=0), dict(hq=0)])
def test_decode_empty_is_noop(kw):
    assert decode(**kw) == 0


def decode_noalloc(**kw):
    a = dict(q=FAKE, qs=st(32 * 128, 32 * 128, 128), k=FAKE, v=FAKE, kvs=st(16 * 8 * 128, 8 * 128, 128), bt=FAKE,
             maxp=2048, ps=16, cl=FAKE, dtype=A.ATTN_BF16, batch=32, sa=1, hq=32, hkv=8, d=128, scale=0.088, window=0,
             split=4096, ms=8, o=FAKE, os=st(32 * 128, 32 * 128, 128))
    a.update(kw)
    return A.lib().attn_decode_fwd_noalloc(a["q"], a["qs"], a["k"], a["v"], a["kvs"], a["bt"], a["maxp"], a["ps"],
                                           a["cl"], a["dtype"], a["batch"], a["sa"], a["hq"], a["hkv"], a["d"],
                                           a["scale"], a["window"], a["split"], a["ms"], a["o"], a["os"], None)


@pytest.mark.parametrize("kw,status", [
    # the partials of 32 x 32 rows x 64 splits x 129 floats exceed the 32 MiB device array
    (dict(split=512, ms=64), UNSUPPORTED),
    (dict(split=4096, ms=8, batch=256), UNSUPPORTED),
    (dict(split=500), INVALID),
    (dict(ms=7), INVALID),               # splits do not cover max_pages * page_size
    (dict(dtype=A.ATTN_F32), UNSUPPORTED),
    (dict(sa=9), UNSUPPORTED),
    (dict(o=0), INVALID),
    (dict(o=FAKE + 4), INVALID),
    (dict(os=st(3, 128, 128)), INVALID),
    (dict(cl=0), INVALID),
    (dict(scale=float("inf")), INVALID),
])
def test_decode_noalloc_rejects_before_any_hip_call(kw, status):
    assert decode_noalloc(**kw) == status


@pytest.mark.parametrize("kw", [dict(batch=0), dict(sa=0), dict(hq=0)])
def test_decode_noalloc_empty_is_noop(kw):
    assert decode_noalloc(**kw) == 0


def test_decode_noalloc_limit_matches_the_header():
    hdr = open(os.path.join(ROOT, "include", "attn.h")).read()
    assert "#define ATTN_DECODE_NOALLOC_MAX_BYTES ((size_t)32 << 20)" in hdr
    assert A.DECODE_NOALLOC_MAX_BYTES == 32 << 20


def combine(**kw):
    a = dict(po=FAKE, pl=FAKE, cl=FAKE, split=512, ms=64, batch=32, sa=1, hq=32, d=128, o=FAKE,
             os=st(32 * 128, 32 * 128, 128), dtype=A.ATTN_BF16)
    a.update(kw)
    return A.lib().attn_decode_combine(a["po"], a["pl"], a["cl"], a["split"], a["ms"], a["batch"], a["sa"], a["hq"],
                                       a["d"], a["o"], a["os"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(split=0), INVALID), (dict(ms=0), INVALID), (dict(dtype=A.ATTN_F32), UNSUPPORTED), (dict(d=32), UNSUPPORTED),
    (dict(o=FAKE + 4), INVALID), (dict(pl=0), INVALID), (dict(os=st(3, 128, 128)), INVALID), (dict(dtype=9), INVALID),
])
def test_combine_rejects(kw, status):
    assert combine(**kw) == status


def test_workspace_size():
    o, l = ctypes.c_size_t(), ctypes.c_size_t()
    assert A.lib().attn_decode_workspace_size(32, 1, 32, 128, 64, ctypes.byref(o), ctypes.byref(l)) == 0
    assert o.value == 32 * 32 * 64 * 128 * 4 and l.value == 32 * 32 * 64 * 4
    assert A.lib().attn_decode_workspace_size(-1, 1, 32, 128, 64, ctypes.byref(o), ctypes.byref(l)) == INVALID


def test_binding_refuses_cpu_tensors():
    import torch

    x = torch.zeros(1, 4, 1, 64)
    with pytest.raises(ValueError, match="GPU"):
        A.attn_prefill_fwd(x, x, x, x, 1.0, False)


def prefill_ex(lse=None, sinks=None, **kw):
    a = dict(q=FAKE, qs=st(2048 * 8 * 128, 8 * 128, 128), k=FAKE, ks=st(2048 * 128, 128, 128), v=FAKE,
             vs=st(2048 * 128, 128, 128), o=FAKE, os=st(2048 * 8 * 128, 8 * 128, 128), dtype=A.ATTN_BF16, batch=1,
             hq=8, hkv=1, sq=2048, skv=2048, d=128, scale=0.088, causal=1, window=0)
    a.update(kw)
    return A.lib().attn_prefill_fwd_ex(a["q"], a["qs"], a["k"], a["ks"], a["v"], a["vs"], a["o"], a["os"],
                                       a["dtype"], a["batch"], a["hq"], a["hkv"], a["sq"], a["skv"], a["d"],
                                       a["scale"], a["causal"], a["window"], lse, sinks, None)


def combine_ex(lse=None, sinks=None, **kw):
    a = dict(po=FAKE, pl=FAKE, cl=FAKE, split=512, ms=64, batch=32, sa=1, hq=32, d=128, o=FAKE,
             os=st(32 * 128, 32 * 128, 128), dtype=A.ATTN_BF16)
    a.update(kw)
    return A.lib().attn_decode_combine_ex(a["po"], a["pl"], a["cl"], a["split"], a["ms"], a["batch"], a["sa"],
                                          a["hq"], a["d"], a["o"], a["os"], a["dtype"], lse, sinks, None)


@pytest.mark.parametrize("lse,sinks", [(FAKE + 2, None), (None, FAKE + 1), (FAKE + 6, FAKE)])
def test_ex_entry_points_reject_misaligned_extras(lse, sinks):
    assert prefill_ex(lse=lse, sinks=sinks) == INVALID
    assert combine_ex(lse=lse, sinks=sinks) == INVALID


def test_ex_entry_points_check_like_the_plain_ones():
    assert prefill_ex(d=96, lse=FAKE) == UNSUPPORTED
    assert prefill_ex(batch=0, lse=FAKE + 2) == 0  # empty: nothing is checked or enqueued
    assert combine_ex(ms=0, sinks=FAKE) == INVALID


def decode_fp8(**kw):
    a = dict(q=FAKE, qs=st(32 * 128, 32 * 128, 128), k=FAKE, v=FAKE, kvs=st(16 * 8 * 128, 8 * 128, 128), bt=FAKE,
             maxp=2048, ps=16, cl=FAKE, dtype=A.ATTN_BF16, batch=32, sa=1, hq=32, hkv=8, d=128, scale=0.088,
             ks=1.0, vs=1.0, window=0, po=FAKE, pl=FAKE, split=512, ms=64)
    a.update(kw)
    return A.lib().attn_decode_fwd_fp8kv(a["q"], a["qs"], a["k"], a["v"], a["kvs"], a["bt"], a["maxp"], a["ps"],
                                         a["cl"], a["dtype"], a["batch"], a["sa"], a["hq"], a["hkv"], a["d"],
                                         a["scale"], a["ks"], a["vs"], a["window"], a["po"], a["pl"], a["split"],
                                         a["ms"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(ks=float("inf")), INVALID), (dict(vs=float("nan")), INVALID), (dict(ks=1e30, scale=1e30), INVALID),
    (dict(kvs=st(16 * 8 * 128, 8 * 128, 8)), INVALID),  # 8-byte head stride: rows not 16-byte aligned
    (dict(dtype=A.ATTN_F32), UNSUPPORTED), (dict(d=96), UNSUPPORTED), (dict(split=500), INVALID),
    (dict(k=FAKE + 8), INVALID),
])
def test_decode_fp8_rejects(kw, status):
    assert decode_fp8(**kw) == status


def test_decode_fp8_accepts_byte_strides():
    # 16-byte-aligned byte strides are fine for one-byte codes; an empty batch enqueues nothing
    assert decode_fp8(batch=0) == 0


def prefill_fp8(**kw):
    a = dict(q=FAKE, qs=st(2048 * 8 * 128, 8 * 128, 128), k=FAKE, ks=st(2048 * 128, 128, 128), v=FAKE,
             vs=st(2048 * 128, 128, 128), o=FAKE, os=st(2048 * 8 * 128, 8 * 128, 128), dtype=A.ATTN_BF16, batch=1,
             hq=8, hkv=1, sq=2048, skv=2048, d=128, scale=0.088, kscale=1.0, vscale=1.0, causal=1, window=0,
             lse=None, sinks=None)
    a.update(kw)
    return A.lib().attn_prefill_fwd_fp8kv(a["q"], a["qs"], a["k"], a["ks"], a["v"], a["vs"], a["o"], a["os"],
                                          a["dtype"], a["batch"], a["hq"], a["hkv"], a["sq"], a["skv"], a["d"],
                                          a["scale"], a["kscale"], a["vscale"], a["causal"], a["window"], a["lse"],
                                          a["sinks"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=A.ATTN_F32), UNSUPPORTED), (dict(dtype=7), INVALID), (dict(d=96), UNSUPPORTED),
    (dict(kscale=float("inf")), INVALID), (dict(vscale=float("nan")), INVALID), (dict(kscale=1e30, scale=1e30), INVALID),
    (dict(ks=st(2048 * 128, 128, 8)), INVALID),  # 8-byte head stride: rows not 16-byte aligned
    (dict(k=FAKE + 8), INVALID), (dict(hq=6, hkv=4), INVALID), (dict(window=64, causal=0), UNSUPPORTED),
    (dict(qs=st(2048 * 8 * 128, 8 * 128 + 1, 128)), INVALID), (dict(lse=FAKE + 2), INVALID),
])
def test_prefill_fp8_rejects(kw, status):
    assert prefill_fp8(**kw) == status


def test_prefill_fp8_accepts_byte_strides_and_empty_shapes():
    # 16-byte-aligned byte strides are fine for one-byte codes; empty shapes enqueue nothing
    assert prefill_fp8(batch=0, ks=st(2048 * 16, 16, 16), vs=st(2048 * 16, 16, 16)) == 0
    assert prefill_fp8(sq=0) == 0


def prefill_varlen(**kw):
    a = dict(q=FAKE, qs=st(0, 8 * 128, 128), k=FAKE, ks=st(0, 128, 128), v=FAKE, vs=st(0, 128, 128), o=FAKE,
             os=st(0, 8 * 128, 128), dtype=A.ATTN_BF16, batch=4, hq=8, hkv=1, cuq=FAKE, cuk=FAKE, mq=2048, mk=2048,
             d=128, scale=0.088, causal=1, window=0, lse=None, sinks=None, pos=None)
    a.update(kw)
    return A.lib().attn_prefill_varlen_fwd(a["q"], a["qs"], a["k"], a["ks"], a["v"], a["vs"], a["o"], a["os"],
                                           a["dtype"], a["batch"], a["hq"], a["hkv"], a["cuq"], a["cuk"], a["mq"],
                                           a["mk"], a["d"], a["scale"], a["causal"], a["window"], a["lse"],
                                           a["sinks"], a["pos"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(cuq=None), INVALID), (dict(cuk=None), INVALID), (dict(cuq=FAKE + 2), INVALID), (dict(cuk=FAKE + 1), INVALID),
    (dict(hq=6, hkv=4), INVALID), (dict(d=96), UNSUPPORTED), (dict(window=16, causal=0), UNSUPPORTED),
    (dict(mq=-1), INVALID), (dict(mk=-5), INVALID), (dict(lse=FAKE + 2), INVALID), (dict(scale=float("nan")), INVALID),
    (dict(pos=FAKE + 2), INVALID),
    (dict(qs=st(0, 8 * 128 + 4, 128)), INVALID),  # 8-byte token stride: rows not 16-byte aligned
    (dict(ks=st(0, 1 << 25, 128)), UNSUPPORTED),  # a 64-row tile would span more than 2^31 elements
    (dict(batch=0, cuq=None, cuk=None), 0), (dict(mq=0), 0),  # empty: nothing is enqueued
])
def test_prefill_varlen_rejects_before_any_hip_call(kw, status):
    assert prefill_varlen(**kw) == status


@pytest.mark.parametrize("batch,hkv,max_len,ps", [(32, 8, 32768, 16), (1, 8, 32768, 16), (4, 8, 2048, 0), (128, 8, 4096, 16),
                                                  (32, 8, 32768, 1), (32, 8, 32768, 24), (2, 1, 100, 100), (64, 4, 8192, 8)])
def test_auto_split_len_is_accepted_by_the_library_rules(batch, hkv, max_len, ps):
    sl = A.auto_split_len(batch, hkv, max_len, ps)
    assert sl > 0 and sl % 16 == 0
    if ps:
        assert sl % ps == 0 and sl // ps <= 256
    assert A.max_splits_for(max_len, sl) * sl >= max_len
    if (batch, hkv, max_len, ps) == (32, 8, 32768, 16):
        assert sl == 4096  # the paged-decode workload's measured best


@pytest.mark.parametrize("batch,max_len,best", [(32, 32768, 4096), (16, 8192, 1024), (8, 8192, 512), (4, 16384, 512),
                                                (1, 32768, 256), (4, 4096, 128), (1, 4096, 64)])
def test_auto_split_len_picks_the_measured_best(batch, max_len, best):
    """32 q-heads over 8 kv-heads, page size 16: the split lengths that timed fastest for each shape."""
    assert A.auto_split_len(batch, 8, max_len, 16) == best


def test_auto_split_len_respects_max_split():
    assert A.auto_split_len(32, 8, 32768, 16, max_split=1024) == 1024
    assert A.auto_split_len(1, 8, 4096, 16, max_split=32) == 64


def validate(**kw):
    a = dict(bt=FAKE, maxp=2048, ps=16, cl=FAKE, batch=32, num=100000, res=FAKE)
    a.update(kw)
    return A.lib().attn_decode_validate_pages(a["bt"], a["maxp"], a["ps"], a["cl"], a["batch"], a["num"], a["res"],
                                              None)


@pytest.mark.parametrize("kw,status", [
    (dict(res=None), INVALID), (dict(res=FAKE + 2), INVALID), (dict(bt=None), INVALID), (dict(cl=None), INVALID),
    (dict(ps=0), INVALID), (dict(batch=-1), INVALID), (dict(num=-1), INVALID), (dict(maxp=0), INVALID),
    (dict(bt=FAKE + 2), INVALID), (dict(batch=1 << 20, maxp=1 << 12), UNSUPPORTED),
])
def test_validate_pages_rejects_before_any_hip_call(kw, status):
    assert validate(**kw) == status


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """No fallback path: without the built library every entry point raises before doing anything."""
    import torch

    monkeypatch.setattr(A, "LIB_PATH", str(tmp_path / "libattn.so"))
    monkeypatch.setattr(A, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        A.lib()
    t = torch.zeros(1, 1, 1, 64)
    with pytest.raises((RuntimeError, ValueError)):
        A.prefill(t, t, t)


def test_one_hip_runtime_whatever_the_import_order():
    """The library and torch share one HIP runtime, also when the library is loaded before torch is
    imported (two runtimes in one process make every launch on a torch stream fail)."""
    code = ("from flash_attention_forward_amd import attn as A\n"
            "A.lib()\n"
            "import torch\n"
            "maps = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}\n"
            "print(len(maps))\n")
    out = subprocess.run(["python3", "-c", code], cwd=ROOT, capture_output=True, text=True, check=True).stdout
    assert out.split()[-1] == "1"

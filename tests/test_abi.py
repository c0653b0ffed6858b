"""The C ABI library loads, exports every function include/nvfp4kv.h
declares, and rejects bad arguments on the host (no kernel is launched on
these paths, so they run without a GPU)."""
import ctypes
import os
import re

import pytest

import bit_quantized_paged_amd as nvk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4kv.h")

pytestmark = pytest.mark.skipif(not os.path.exists(nvk.LIB_PATH), reason="libnvfp4kv.so not built")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(nvfp4[a-z_0-9]*)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = _declared()
    assert names == sorted(nvk.EXPORTS), names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(nvk.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name


def test_full_dim_and_status_strings():
    lib = nvk.library()
    assert [lib.nvfp4_kv_full_dim(d) for d in (64, 128, 256)] == [36, 72, 144]
    assert lib.nvfp4_kv_full_dim(0) == -1 and lib.nvfp4_kv_full_dim(100) == -1
    assert lib.nvfp4kv_status_string(0) == b"ok"
    assert lib.nvfp4kv_status_string(3) == b"workspace too small"


def _desc(**kw):
    base = dict(data=16 * 1024, num_blocks=4, block_size=16, num_kv_heads=2, head_size=128, kv_dtype=0,
                stride_block=2 * 2 * 16 * 72, stride_kv=2 * 16 * 72, stride_token=72, stride_head=16 * 72)
    base.update(kw)
    return nvk.CacheDesc(**base)


def _append(desc, **kw):
    lib = nvk.library()
    a = dict(key=4096, kst=256, ksh=128, value=8192, vst=256, vsh=128, slots=64, n=3, ks=32, vs=48)
    a.update(kw)
    return lib.nvfp4_kv_append(ctypes.byref(desc), a["key"], a["kst"], a["ksh"], a["value"], a["vst"], a["vsh"],
                               a["slots"], a["n"], a["ks"], a["vs"], None)


def test_append_validation():
    lib = nvk.library()
    assert _append(_desc(data=None)) == 1
    assert _append(_desc(head_size=96)) == 2
    assert _append(_desc(block_size=8)) == 2
    assert _append(_desc(kv_dtype=3)) == 1 and _append(_desc(kv_dtype=-1)) == 1
    # FP8 rows need 16-byte strides (72 is a packed NVFP4 width)
    assert _append(_desc(kv_dtype=1)) == 1
    assert _append(_desc(stride_token=70)) == 1
    assert _append(_desc(stride_token=(1 << 26) + 4)) == 2
    assert _append(_desc(stride_kv=(1 << 30) + 4)) == 2
    assert _append(_desc(data=16 * 1024 + 4)) == 1
    assert _append(_desc(), key=None) == 1
    assert b"key" in lib.nvfp4kv_last_error()
    assert _append(_desc(), kst=100) == 1
    assert _append(_desc(), slots=None) == 1
    assert _append(_desc(), n=-1) == 1
    assert _append(_desc(), n=0) == 0            # no-op, nothing launched
    assert lib.nvfp4kv_last_error() == b""


def test_decode_validation():
    lib = nvk.library()
    d = _desc()
    need = lib.nvfp4_paged_attention_decode_workspace_size(3, 8, 2, 128)
    assert need > 0

    def call(**kw):
        a = dict(q=4096, qst=1024, qsh=128, hq=8, bt=64, mb=4, sl=96, B=3, ml=64, ks=32, vs=48, out=8192,
                 ws=1 << 20, wsb=need)
        a.update(kw)
        return lib.nvfp4_paged_attention_decode(ctypes.byref(d), a["q"], a["qst"], a["qsh"], a["hq"], a["bt"],
                                                a["mb"], a["sl"], a["B"], a["ml"], a["ks"], a["vs"], 0.1,
                                                a["out"], a["ws"], a["wsb"], None)
    assert call(hq=7) == 1          # not a multiple of the kv heads
    assert call(hq=34) == 2         # group of 17 > 16
    assert call(wsb=need - 1) == 3
    assert call(ws=None) == 3
    assert call(q=None) == 1
    assert call(out=8194) == 1
    assert call(B=5000) == 2
    assert call(B=4097) == 2        # one past the largest batch a decode call takes
    assert call(B=0) == 0


def test_prefill_and_dequant_validation():
    lib = nvk.library()
    d = _desc()
    r = lib.nvfp4_paged_attention_prefill(ctypes.byref(d), 4096, 1024, 128, 8, None, 16, 16, 64, 4, 96, 1, 64,
                                          32, 48, 0.1, 1, 8192, None, 0, None)
    assert r == 1  # cu_seqlens_q is NULL
    r = lib.nvfp4_paged_attention_prefill(ctypes.byref(d), 4096, 1024, 128, 8, 128, 0, 0, 64, 4, 96, 1, 64,
                                          32, 48, 0.1, 1, 8192, None, 0, None)
    assert r == 0  # nothing to do
    r = lib.nvfp4_kv_dequant_paged(ctypes.byref(d), 64, 4, 96, 128, 2, 64, 32, 48, None, 8192, 10, None)
    assert r == 1
    r = lib.nvfp4_kv_dequant_paged(ctypes.byref(d), 64, 4, 96, 128, 70000, 64, 32, 48, 4096, 8192, 10, None)
    assert r == 1


def test_prefill_workspace_validation():
    """The key split's workspace is checked on the host before any launch: a
    size without a pointer, a pointer not 256-byte aligned, one below the size
    query, or more than 4096 sequences with a workspace are argument errors;
    the size query answers 0 for a head size the library does not build."""
    lib = nvk.library()
    d = _desc()
    need = lib.nvfp4_paged_attention_prefill_workspace_size(128)
    assert need > 0 and lib.nvfp4_paged_attention_prefill_workspace_size(96) == 0

    def call(ws, nbytes, B=1):
        return lib.nvfp4_paged_attention_prefill(ctypes.byref(d), 4096, 1024, 128, 8, 128, 16, 16, 64, 4, 96, B, 64,
                                                 32, 48, 0.1, 1, 8192, ws, nbytes, None)
    assert call(None, 5) == 1
    assert call(4096 + 16, need) == 1
    assert call(4096, need - 1) == 1
    assert call(4096, need, B=4097) == 1


def test_decode_plan_rejects_bad_sizes():
    """The plan query validates its sizes on the host (no device needed for
    these paths)."""
    assert nvk.decode_plan(4, 2, 96, 16, 8, 100) == -1   # head size not built
    assert nvk.decode_plan(4, 0, 128, 16, 8, 100) == -1  # no kv heads
    assert nvk.decode_plan(-1, 2, 128, 16, 8, 100) == -1
    assert nvk.decode_plan(4, 2, 128, 0, 8, 100) == -1
    assert nvk.decode_plan(4, 2, 128, 16, 0, 100) == -1
    assert nvk.library().nvfp4_paged_attention_decode_plan(4, 2, 128, 16, 8, 100, 3) == -1  # unknown format


def test_quant_activations_sizes_and_rejects():
    lib = nvk.library()
    assert nvk.quant_activations_scale_bytes(200, 80, True) == 256 * 8
    assert nvk.quant_activations_scale_bytes(200, 80, False) == 200 * 5
    assert nvk.quant_activations_scale_bytes(1, 16, True) == 128 * 4
    assert nvk.quant_activations_scale_bytes(8192, 4096, True) == 8192 * 256
    assert nvk.quant_activations_scale_bytes(0, 64, True) == 0
    assert nvk.quant_activations_scale_bytes(4, 40, True) == -1
    assert nvk.quant_activations_scale_bytes(-1, 64, False) == -1
    null = ctypes.c_void_p(0)
    # bad k, negative m, misaligned x: rejected before any device work
    assert lib.nvfp4_quant_activations(null, 64, 4, 40, null, 1, null, null, null) != 0
    assert lib.nvfp4_quant_activations(null, 64, -1, 64, null, 1, null, null, null) != 0
    assert lib.nvfp4_quant_activations(ctypes.c_void_p(8), 64, 4, 64, ctypes.c_void_p(16), 1, ctypes.c_void_p(16),
                                       ctypes.c_void_p(16), null) != 0
    assert lib.nvfp4_quant_activations(ctypes.c_void_p(16), 60, 4, 64, ctypes.c_void_p(16), 1, ctypes.c_void_p(16),
                                       ctypes.c_void_p(16), null) != 0
    # m = 0 is a no-op that touches nothing
    assert lib.nvfp4_quant_activations(null, 64, 0, 64, null, 1, null, null, null) == 0


def test_probe_library_exports_and_rejects():
    """The benchmark's read-stream measurement library: its header's one
    function is exported and bad arguments are refused before any launch."""
    from bit_quantized_paged_amd import probe
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "nvfp4kv_probe.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"^\s*[a-z_0-9]+\s*\*?\s*(nvfp4[a-z_0-9]*)\s*\(", text, flags=re.M)))
    assert names == probe.EXPORTS
    lib = probe.library()
    f = lib.nvfp4kv_probe_read_stream
    assert f(None, 1024, 4, 64, 64, None) == 1          # NULL data
    assert f(16, 1000, 4, 64, 64, None) == 1            # bytes not a multiple of 16
    assert f(16, 1024, 0, 64, 64, None) == 1            # no workgroups
    assert f(8, 1024, 4, 64, 64, None) == 1             # misaligned data
    assert f(16, 1024, 8, 64, 64, None) == 1            # sink smaller than grid * 16 bytes
    g = lib.nvfp4kv_probe_read_pages
    ok = dict(pool=64, nb=4, sb=2304, skv=1152, sh=1152 * 2, slab=1152, bs=16, hkv=1, bt=64, mb=2, sl=64, B=1,
              splits=4, sink=64, sink_bytes=64)
    call = lambda **k: g(*({**ok, **k}.values()), None)
    assert call(pool=0) == 1                            # NULL pool
    assert call(slab=1000) == 1                         # slab not a multiple of 16
    assert call(slab=4112) == 1                         # slab above 4096 bytes
    assert call(sb=2300) == 1                           # strides must be multiples of 16
    assert call(splits=8) == 1                          # sink smaller than 16 bytes per workgroup

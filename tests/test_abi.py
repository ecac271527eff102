"""The C-ABI library: it loads, exports what the header declares, and rejects bad arguments
from the host side (CPU only: every case here returns before any HIP call)."""
import ctypes
import os
import re

import pytest

import attention_nvfp4_quantized_amd as A
from attention_nvfp4_quantized_amd.binding import CacheDesc, load_library

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4kv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\*?([a-z_0-9]+)\s*\(", text, re.M)))


def test_header_declares_the_path():
    names = declared_functions()
    for n in ("nvfp4_kv_append", "nvfp4_kv_dequant", "nvfp4_kv_repack", "paged_prefill_nvfp4", "paged_decode_nvfp4",
              "paged_prefill_nvfp4_workspace_size", "paged_decode_nvfp4_workspace_size",
              "nvfp4kv_last_error", "nvfp4kv_version"):
        assert n in names, names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(A.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert load_library().nvfp4kv_version() == 100


def _desc(**over):
    d = dict(k_data=16, k_scale=16, v_data=16, v_scale=16, k_global=1.0, v_global=1.0,
             num_pages=4, page_size=16, num_kv_heads=8, head_dim=128, kv_format=0)
    d.update(over)
    return CacheDesc(**d)


def _err():
    return load_library().nvfp4kv_last_error().decode()


@pytest.mark.parametrize("over,code,needle", [
    (dict(head_dim=64), -2, "head_dim"),
    (dict(page_size=32), -2, "page_size"),
    (dict(k_data=None), -1, "NULL"),
    (dict(num_kv_heads=0), -1, "num_kv_heads"),
    (dict(k_global=0.0), -1, "global"),
    (dict(v_global=float("inf")), -1, "global"),
    (dict(kv_format=3), -1, "kv_format"),
    (dict(k_scale=None), -1, "NULL"),
])
def test_append_rejects_bad_cache(over, code, needle):
    lib = load_library()
    d = _desc(**over)
    rc = lib.nvfp4_kv_append(ctypes.byref(d), 16, 16, 1024, 1024, 0, 16, 4, None)
    assert rc == code and needle in _err()


def test_append_rejects_short_stride_and_null_inputs():
    lib = load_library()
    d = _desc()
    assert lib.nvfp4_kv_append(ctypes.byref(d), 16, 16, 512, 1024, 0, 16, 4, None) == -1
    assert lib.nvfp4_kv_append(ctypes.byref(d), None, 16, 1024, 1024, 0, 16, 4, None) == -1
    assert lib.nvfp4_kv_append(None, 16, 16, 1024, 1024, 0, 16, 4, None) == -1
    assert lib.nvfp4_kv_append(ctypes.byref(d), 16, 16, 1024, 1024, 0, 16, 0, None) == 0
    assert lib.nvfp4_kv_append(ctypes.byref(d), 16, 16, 1024, 1024, 1, 16, 0, None) == 0
    assert _err() == ""
    assert lib.nvfp4_kv_append(ctypes.byref(d), 16, 16, 1024, 1024, 2, 16, 4, None) == -1
    assert b"input_dtype" in lib.nvfp4kv_last_error()


def test_dequant_argument_checks():
    lib = A.load_library()
    d = _desc()
    assert lib.nvfp4_kv_dequant(ctypes.byref(d), 16, 4, 16, 16, 3, None) == -1
    assert b"out_dtype" in lib.nvfp4kv_last_error()
    assert lib.nvfp4_kv_dequant(ctypes.byref(d), None, 4, 16, 16, 0, None) == -1
    assert lib.nvfp4_kv_dequant(ctypes.byref(d), 16, 4, 8, 16, 0, None) == -1
    assert b"aligned" in lib.nvfp4kv_last_error()
    assert lib.nvfp4_kv_dequant(ctypes.byref(d), 16, -1, 16, 16, 0, None) == -1
    assert lib.nvfp4_kv_dequant(None, 16, 4, 16, 16, 0, None) == -1
    assert lib.nvfp4_kv_dequant(ctypes.byref(d), 16, 0, 16, 16, 2, None) == 0
    assert _err() == ""


def _prefill(lib, d, **kw):
    a = dict(q=16, cu=16, kv=16, bt=16, bts=8, batch=1, total_q=16, max_q=16, max_kv=128,
             hq=32, sm=0.088, causal=1, out=16, odt=0, lse=None, splits=0, ws=None, wsb=0)
    a.update(kw)
    return lib.paged_prefill_nvfp4(ctypes.byref(d), a["q"], a["cu"], a["kv"], a["bt"], a["bts"],
                                   a["batch"], a["total_q"], a["max_q"], a["max_kv"], a["hq"],
                                   a["sm"], a["causal"], a["out"], a["odt"], a["lse"], a["splits"],
                                   a["ws"], a["wsb"], None)


def test_prefill_argument_checks():
    lib = load_library()
    d = _desc()
    assert _prefill(lib, d, hq=30) == -1 and "multiple" in _err()
    assert _prefill(lib, d, hq=8 * 3) == -2  # group 3 does not divide 256
    assert _prefill(lib, d, bts=2) == -1 and "block_table_stride" in _err()
    assert _prefill(lib, d, sm=0.0) == -1
    assert _prefill(lib, d, odt=7) == -1
    assert _prefill(lib, d, q=None) == -1
    assert _prefill(lib, d, q=8) == -1 and "aligned" in _err()
    assert _prefill(lib, _desc(head_dim=96)) == -2
    assert _prefill(lib, d, total_q=1 << 26) == -1 and "too large" in _err()  # 2^31 output rows
    assert _prefill(lib, d, total_q=0) == 0  # empty problem: no launch
    assert _prefill(lib, d, batch=0) == 0


def test_prefill_split_needs_workspace():
    lib = load_library()
    d = _desc()
    need = A.prefill_workspace_size(1, 16, 16, 128, 32, 8, num_splits=4)
    assert need == 4 * 16 * 32 * (128 * 2 + 4)  # fp16 partial + float32 log-sum-exp per row
    assert _prefill(lib, d, splits=4) == -3 and str(need) in _err()
    assert _prefill(lib, d, splits=4, ws=16, wsb=need - 1) == -3


def test_decode_argument_checks():
    lib = load_library()
    d = _desc()

    def dec(**kw):
        a = dict(q=16, kv=16, bt=16, bts=2048, batch=64, max_kv=32768, hq=32, sm=0.088, out=16,
                 odt=0, lse=None, splits=0, ws=16, wsb=1 << 40)
        a.update(kw)
        return lib.paged_decode_nvfp4(ctypes.byref(d), a["q"], a["kv"], a["bt"], a["bts"], a["batch"],
                                      a["max_kv"], a["hq"], a["sm"], a["out"], a["odt"], a["lse"],
                                      a["splits"], a["ws"], a["wsb"], None)
    assert dec(hq=8 * 32) == -2 and "16" in _err()
    assert dec(bts=100) == -1
    assert dec(ws=None) == -3
    assert dec(wsb=100) == -3
    assert dec(max_kv=0) == -1
    assert dec(batch=1 << 26) == -1 and "too large" in _err()  # 2^31 output rows
    assert dec(batch=0) == 0
    need = A.decode_workspace_size(64, 32768, 32, 8, num_splits=8)
    assert need == 8 * 64 * 32 * (128 * 2 + 4)


def test_workspace_sizes_follow_split_policy():
    # long single-sequence prefill: enough workgroups without splitting
    assert A.prefill_workspace_size(1, 16384, 16384, 16384, 32, 8) == 0
    # short tails over long caches split the key range
    assert A.prefill_workspace_size(8, 128, 16, 16384, 32, 8) > 0
    assert A.decode_workspace_size(64, 32768, 32, 8) > 0


def test_binding_refuses_missing_library(tmp_path):
    import attention_nvfp4_quantized_amd.binding as B
    saved = B._lib
    try:
        B._lib = None
        with pytest.raises(RuntimeError, match="not built"):
            B.load_library(str(tmp_path / "missing.so"))
    finally:
        B._lib = saved


def test_fp8_format_needs_no_scale_plane():
    """The FP8 control cache has no block scales: NULL scale pointers pass the checks (the
    zero-token calls return before any launch)."""
    lib = load_library()
    d = _desc(kv_format=1, k_scale=None, v_scale=None)
    assert lib.nvfp4_kv_append(ctypes.byref(d), 16, 16, 1024, 1024, 0, 16, 0, None) == 0
    assert lib.nvfp4_kv_dequant(ctypes.byref(d), 16, 0, 16, 16, 0, None) == 0
    assert _prefill(lib, d, total_q=0) == 0
    assert _err() == ""
    assert lib.nvfp4_kv_append(ctypes.byref(d), 16, 16, 512, 1024, 0, 16, 4, None) == -1


def test_descriptor_layout_matches_header():
    """The ctypes descriptor has the header's fields in the header's order."""
    text = open(HEADER).read()
    body = text[text.index("typedef struct nvfp4kv_cache"):text.index("} nvfp4kv_cache_t;")]
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    names = re.findall(r"\b([a-z_0-9]+);", body)
    assert names == [f[0] for f in CacheDesc._fields_]


def _repack(lib, src, dst, bt=16, bts=4, lens=16, batch=2, max_kv=64):
    return lib.nvfp4_kv_repack(ctypes.byref(src), ctypes.byref(dst), bt, bts, lens, batch, max_kv, None)


def test_repack_argument_checks():
    lib = load_library()
    src = _desc()
    dst = _desc(kv_format=2, k_scale=None, v_scale=None)
    assert _repack(lib, src, dst, batch=0) == 0 and _err() == ""
    assert _repack(lib, src, dst, max_kv=0) == 0
    assert _repack(lib, src, src) == -1 and "NVFP4KV_FORMAT_F16" in _err()
    assert _repack(lib, dst, dst) == -2 and "source" in _err()
    assert _repack(lib, _desc(kv_format=1, k_scale=None, v_scale=None), dst) == -2
    assert _repack(lib, src, _desc(kv_format=2, num_pages=5)) == -1 and "match" in _err()
    assert _repack(lib, src, _desc(kv_format=2, k_global=2.0)) == -1
    assert _repack(lib, src, dst, bts=3) == -1 and "block_table_stride" in _err()
    assert _repack(lib, src, dst, bt=None) == -1
    assert _repack(lib, src, dst, batch=70000) == -1
    assert _repack(lib, src, _desc(kv_format=2, k_data=24)) == -1 and "aligned" in _err()


def test_f16_format_is_prefill_only():
    lib = load_library()
    d = _desc(kv_format=2, k_scale=None, v_scale=None)
    assert lib.nvfp4_kv_append(ctypes.byref(d), 16, 16, 1024, 1024, 0, 16, 4, None) == -2
    assert "fp16" in _err()
    assert lib.nvfp4_kv_dequant(ctypes.byref(d), 16, 4, 16, 16, 0, None) == -2
    assert lib.paged_decode_nvfp4(ctypes.byref(d), 16, 16, 16, 2048, 64, 32768, 32, 0.088, 16, 0,
                                  None, 0, 16, 1 << 40, None) == -2
    assert _prefill(lib, d, total_q=0) == 0


def test_binding_rejects_fp16_attention_output():
    """Attention outputs are bf16 or float32: an fp16 out_dtype, or a caller's fp16 `out`, is
    refused before any device call (the C ABI would otherwise be told bf16 and write bf16 bit
    patterns into a float16 tensor)."""
    import torch
    for fn, args in ((A.prefill, (None, None, None, None, None, 16, 16, 0.088)),
                     (A.decode, (None, None, None, None, 16, 0.088))):
        with pytest.raises(TypeError, match="bfloat16 or float32"):
            fn(*args, out_dtype=torch.float16)
        with pytest.raises(TypeError, match="bfloat16 or float32"):
            fn(*args, out=torch.empty((1, 1, 128), dtype=torch.float16))
        with pytest.raises(TypeError, match="bfloat16 or float32"):
            fn(*args, out_dtype=torch.int32)


def test_noalloc_decode_rejects_more_than_its_scratch():
    """The allocation-free decode refuses, before any device call, a problem whose partials pass
    its static scratch (here 16 splits x 4096 sequences x 32 heads x 260 B), and names both sizes;
    argument errors come first, as in paged_decode_nvfp4."""
    lib = load_library()
    d = _desc()

    def dec(**kw):
        a = dict(q=16, kv=16, bt=16, bts=8192, batch=4096, max_kv=131072, hq=32, sm=0.088, out=16,
                 odt=0, lse=None, splits=0)
        a.update(kw)
        return lib.paged_decode_nvfp4_noalloc(ctypes.byref(d), a["q"], a["kv"], a["bt"], a["bts"],
                                              a["batch"], a["max_kv"], a["hq"], a["sm"], a["out"],
                                              a["odt"], a["lse"], a["splits"], None)
    need = A.decode_workspace_size(4096, 131072, 32, 8)
    assert need > A.DECODE_SCRATCH_BYTES
    assert dec() == -3
    msg = _err()
    assert str(need) in msg and str(A.DECODE_SCRATCH_BYTES) in msg
    assert dec(q=None) == -1
    assert dec(hq=8 * 32) == -2
    assert dec(batch=0) == 0 and _err() == ""


def test_a4q_prefill_argument_checks():
    """The A4Q-style prefill: unknown query formats and non-NVFP4 caches are refused, the other
    checks are the stock prefill's, and its workspace follows the 8-wave kernel's split rule."""
    lib = load_library()

    def call(d, **kw):
        a = dict(q=16, cu=16, kv=16, bt=16, bts=8, batch=1, total_q=16, max_q=16, max_kv=128,
                 hq=32, sm=0.088, causal=1, out=16, odt=0, lse=None, qf=0, splits=0, ws=None, wsb=0)
        a.update(kw)
        return lib.paged_prefill_nvfp4_a4q(ctypes.byref(d), a["q"], a["cu"], a["kv"], a["bt"],
                                           a["bts"], a["batch"], a["total_q"], a["max_q"],
                                           a["max_kv"], a["hq"], a["sm"], a["causal"], a["out"],
                                           a["odt"], a["lse"], a["qf"], a["splits"], a["ws"],
                                           a["wsb"], None)
    d = _desc()
    assert call(d, qf=2) == -1 and "q_format" in _err()
    assert call(d, qf=0x12) == -1 and "q_format" in _err()  # the one-term flag on no format
    assert call(d, qf=0x20) == -1 and "q_format" in _err()
    assert call(d, qf=0x11, total_q=0) == 0 and _err() == ""  # MXFP4 queries, one-term K
    with pytest.raises(ValueError, match="k_terms"):
        A.prefill_a4q(None, None, None, None, None, 1, 1, 1.0, k_terms=3)
    assert call(_desc(kv_format=1, k_scale=None, v_scale=None)) == -2 and "NVFP4" in _err()
    assert call(d, hq=30) == -1 and "multiple" in _err()
    assert call(d, bts=2) == -1 and "block_table_stride" in _err()
    assert call(d, total_q=0) == 0 and _err() == ""
    need = A.prefill_a4q_workspace_size(1, 16, 16, 128, 32, 8, num_splits=4)
    assert need == 4 * 16 * 32 * (128 * 2 + 4)
    assert call(d, splits=4) == -3 and str(need) in _err()
    # short tails run the 8-wave kernel (256 columns per tile), so the split count differs
    assert A.prefill_a4q_workspace_size(8, 128, 16, 16384, 32, 8) > 0

"""The allocation-free decode entry point (paged_decode_nvfp4_noalloc), called through the C ABI,
against paged_decode_nvfp4 with a caller workspace.  Both run the same kernels with the same
split count, so outputs and log-sum-exps must agree bit for bit (stricter than the max-abs 1e-2 /
mean-abs 1e-3 bar, which the larger call also meets against the oracle).  Calls come in a row,
each smaller than the one before: the static scratch keeps the previous call's partials."""
import ctypes

import numpy as np
import pytest
import torch

import attention_nvfp4_quantized_amd as A
import workload as W
from oracle import attention as oattn
from gpu_cases import GpuPrefillCase, assert_attention_close, oracle_cache, say

pytestmark = pytest.mark.gpu

_ODT = {torch.bfloat16: 0, torch.float32: 1}


def _decode_case(lens, hq, hkv, seed, kv_format):
    w = W.custom("noalloc", [1] * len(lens), lens, hq, hkv, seed, k_outlier_channels=2)
    pc = W.prefill_case(w)  # one query per sequence: its last position
    g = GpuPrefillCase(pc, kv_format=kv_format)
    g.append()
    return pc, g


def _noalloc(g, pc, out_dtype, splits):
    """paged_decode_nvfp4_noalloc through ctypes on the current stream."""
    lib = A.load_library()
    batch, hq = g.q.shape[0], g.q.shape[1]
    out = torch.full((batch, hq, 128), float("nan"), dtype=out_dtype, device="cuda")
    lse = torch.full((batch, hq), float("nan"), dtype=torch.float32, device="cuda")
    d = g.cache.desc()
    rc = lib.paged_decode_nvfp4_noalloc(
        ctypes.byref(d), g.q.data_ptr(), g.kv.data_ptr(), g.bt.data_ptr(), g.bt.shape[1], batch,
        pc.max_kv_len, hq, pc.w.sm_scale, out.data_ptr(), _ODT[out_dtype], lse.data_ptr(), splits,
        torch.cuda.current_stream().cuda_stream)
    assert rc == 0, lib.nvfp4kv_last_error().decode()
    return out, lse


def _check_pair(pc, g, out_dtype, splits):
    ref, ref_lse = A.decode(g.cache, g.q, g.kv, g.bt, pc.max_kv_len, pc.w.sm_scale,
                            out_dtype=out_dtype, return_lse=True, num_splits=splits)
    out, lse = _noalloc(g, pc, out_dtype, splits)
    torch.cuda.synchronize()
    iview = torch.int16 if out_dtype == torch.bfloat16 else torch.int32
    assert torch.equal(out.view(iview), ref.view(iview)), "outputs differ"
    assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32)), "log-sum-exps differ"
    return out


@pytest.mark.parametrize("kv_format", ["nvfp4", "fp8"])
def test_noalloc_decode_matches_workspace_decode_in_a_row(kv_format):
    # largest first: 64 sequences x 32 heads in 16 key splits (8.5 MB of the 16 MiB scratch)
    lens = [int(x) for x in np.random.default_rng(3301).integers(1, 6000, 64)]
    say(f"[noalloc] {kv_format}: 64 x 32 heads over up to {max(lens)} keys, 16 splits, fp32")
    pc, g = _decode_case(lens, 32, 8, 3301, kv_format)
    out = _check_pair(pc, g, torch.float32, 16)
    oc = oracle_cache(pc, kv_format=kv_format)
    ref, _ = oattn.decode(oc, pc.q_bits, pc.kv_lens, pc.layout.block_table, pc.w.sm_scale)
    assert_attention_close(out.cpu().numpy(), ref, f"noalloc {kv_format} vs oracle")
    # then smaller calls on the same GPU, automatic and explicit splits, both output types
    say(f"[noalloc] {kv_format}: 8 x 32 heads, automatic splits, bf16")
    pc2, g2 = _decode_case([1, 15, 16, 17, 100, 1023, 4999, 2048], 32, 8, 3302, kv_format)
    _check_pair(pc2, g2, torch.bfloat16, 0)
    say(f"[noalloc] {kv_format}: 3 x 8 heads, 3 splits, fp32")
    pc3, g3 = _decode_case([700, 1, 33], 8, 2, 3303, kv_format)
    _check_pair(pc3, g3, torch.float32, 3)


def test_noalloc_decode_binding_and_rejection():
    """The Python binding of the entry point gives the same bits, and a problem past the static
    scratch is rejected with EWORKSPACE (nothing launched: the output keeps its contents)."""
    say("[noalloc] binding, and a request past the scratch")
    pc, g = _decode_case([300, 5000, 77], 32, 8, 3304, "nvfp4")
    ref = A.decode(g.cache, g.q, g.kv, g.bt, pc.max_kv_len, pc.w.sm_scale, out_dtype=torch.float32)
    got = A.decode_noalloc(g.cache, g.q, g.kv, g.bt, pc.max_kv_len, pc.w.sm_scale,
                           out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int32), ref.view(torch.int32))
    sentinel = torch.full_like(got, 7.0)
    with pytest.raises(A.Nvfp4KVError, match="EWORKSPACE"):
        A.decode_noalloc(g.cache, g.q, g.kv, g.bt, pc.max_kv_len, pc.w.sm_scale, out=sentinel,
                         num_splits=3000)  # 3000 x 3 x 32 x 260 B > 16 MiB
    torch.cuda.synchronize()
    assert bool((sentinel == 7.0).all())

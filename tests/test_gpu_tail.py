"""GPU parity of the short-query prefill kernel: up to 64 query columns (query rows x heads of a
group) per sequence and KV head, the chunked-prefill tails and speculative chunks of "NVFP4 KV
cache A4Q prefill explained" (sections "Compare A4Q with dequantize-ahead repacking" and "Build
the benchmark matrix").  Every output row and its log-sum-exp is compared with the oracle, for
both cache formats the kernel reads, with and without the causal mask, and across key-slice
counts; the shapes cover one and two 16-column blocks, the wavefront-pair kernel (33 to 64
columns, with half-empty pairs), group sizes 1 to 64,
a sequence without queries, a single key, keys ending inside a page, and wavefront ranges long
enough to use both page-id registers."""
import numpy as np
import pytest
import torch

import workload as W
from gpu_cases import (LSE_ATOL, GpuPrefillCase, assert_attention_close, assert_attention_close_bf16,
                       oracle_cache, oracle_prefill, say)

pytestmark = pytest.mark.gpu

# (q_lens, kv_lens, num_qo_heads, num_kv_heads): the longest q_len x group is at most 64
CASES = [
    ([1], [1], 8, 8),                       # one key, one column
    ([1, 3, 16], [700, 35, 16], 8, 8),      # group 1: 1-16 columns, one block
    ([17, 5], [2000, 17], 8, 8),            # group 1: 17 columns, two blocks
    ([8, 1, 2], [9000, 4097, 2], 32, 8),    # group 4: 32 columns; 9000 keys in few slices
    ([16, 13, 0, 9], [16384, 300, 50, 9], 32, 8),  # 64 columns (wavefront pairs); no queries in one
    ([4, 2], [1000, 2500], 64, 4),          # group 16
    ([9, 3], [5000, 40], 32, 8),            # 36 columns: wavefront pairs, second pair half-empty
    ([6, 6, 1], [3333, 6, 129], 64, 8),     # group 8: 48 columns; q_len = kv_len
    ([1, 1], [5000, 77], 64, 1),            # group 64, one row
]
SPLITS = [0, 1, 3, 7]


@pytest.mark.parametrize("kv_format", ["nvfp4", "fp8"])
@pytest.mark.parametrize("ci", range(len(CASES)))
def test_tail_parity(ci, kv_format):
    q_lens, kv_lens, hq, hkv = CASES[ci]
    assert max(q_lens) * (hq // hkv) <= 64
    say(f"[tail] case {ci}: q_lens {q_lens} kv_lens {kv_lens} Hq {hq} Hkv {hkv} {kv_format}")
    pc = W.prefill_case(W.custom("tail", q_lens, kv_lens, hq, hkv, 3600 + ci, k_outlier_channels=4))
    g = GpuPrefillCase(pc, kv_format=kv_format)
    g.append()
    oc = oracle_cache(pc, kv_format=kv_format)
    for causal in (True, False):
        ref, ref_lse = oracle_prefill(pc, oc, causal=causal)
        for splits in SPLITS:
            say(f"  causal {causal} splits {splits}")
            o, lse = g.prefill(torch.float32, causal=causal, num_splits=splits, return_lse=True)
            name = f"tail case {ci} {kv_format} causal={causal} splits={splits}"
            assert_attention_close(o.cpu().numpy(), ref, name)
            np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, rtol=0, atol=LSE_ATOL, err_msg=name)
        o16 = g.prefill(torch.bfloat16, causal=causal)
        assert_attention_close_bf16(o16.float().cpu().numpy(), ref, f"tail case {ci} {kv_format} bf16")


def test_tail_rows_do_not_depend_on_the_slicing():
    """The slices only regroup the same keys: outputs over 1..7 slices agree within the fp16
    rounding of the partials (and every one matches the oracle above)."""
    say("[tail] slicing invariance")
    pc = W.prefill_case(W.custom("tail", [16, 11], [6000, 3001], 32, 8, 3650))
    g = GpuPrefillCase(pc)
    g.append()
    outs = [g.prefill(torch.float32, num_splits=s).cpu().numpy() for s in (1, 2, 5, 7)]
    for o in outs[1:]:
        assert np.abs(o - outs[0]).max() < 2e-3

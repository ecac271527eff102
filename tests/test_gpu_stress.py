"""GPU value-range stress cases against the oracle: query outlier channels, extreme query
scales (the per-column power-of-two conversion to fp16), and K/V spanning the E4M3 block-scale
range from subnormal to saturated.  Inputs are the seeded workloads under the transforms of
``workload.scale_channels`` / ``workload.scale_tokens_pow2``."""
import numpy as np
import pytest
import torch

import workload as W
from gpu_cases import (GpuPrefillCase, assert_attention_close, assert_cache_equal, oracle_cache,
                       oracle_prefill, say)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("factor", [8.0, 64.0])
def test_prefill_query_outlier_channels(factor):
    say(f"[stress] tail128, 4 query channels per head x{factor}")
    pc = W.prefill_case(W.get("tail128"))
    pc.q_bits = W.scale_channels(pc.q_bits, 77, 4, factor)
    g = GpuPrefillCase(pc)
    g.append()
    o = g.prefill(torch.float32).cpu().numpy()
    ref, _ = oracle_prefill(pc, oracle_cache(pc))
    assert_attention_close(o, ref, f"q outliers x{factor}")


@pytest.mark.parametrize("e", [-20, 12])
def test_prefill_query_scale_extremes(e):
    """q x 2^-20 (a near-uniform softmax) and q x 2^12 (a near one-hot softmax; base-2 logits
    ~1e4, where float32 still resolves them to ~1e-3 -- far larger logits exceed what any
    float32-accumulating kernel can resolve against a float64 reference)."""
    say(f"[stress] q lens [70, 41], kv lens [70, 300], q x 2^{e}")
    pc = W.prefill_case(W.custom("case", [70, 41], [70, 300], 32, 8, 3301, k_outlier_channels=4))
    pc.q_bits = W.scale_tokens_pow2(pc.q_bits, 0, e, e)
    g = GpuPrefillCase(pc)
    g.append()
    o = g.prefill(torch.float32).cpu().numpy()
    ref, _ = oracle_prefill(pc, oracle_cache(pc))
    assert_attention_close(o, ref, f"q x 2^{e}")


def test_kv_across_the_block_scale_range():
    """Every K token scaled by its own 2^e, e in [-14, 12] (block scales from E4M3 subnormals to
    saturation at 448, where values clip to 2688), V by 2^e, e in [-14, 0]: the cache bytes stay
    bit-exact and the prefill meets the output bar."""
    say("[stress] K x 2^[-14, 12], V x 2^[-14, 0] per token")
    pc = W.prefill_case(W.custom("case", [70, 41], [70, 300], 32, 8, 3302, k_outlier_channels=4))
    pc.k_bits = W.scale_tokens_pow2(pc.k_bits, 1, -14, 12)
    pc.v_bits = W.scale_tokens_pow2(pc.v_bits, 2, -14, 0)
    g = GpuPrefillCase(pc)
    g.append()
    torch.cuda.synchronize()
    oc = oracle_cache(pc)
    assert_cache_equal(g.cache_host(), oc)
    sc = oc.k_scale
    assert (sc == 0x7E).any() and ((sc > 0) & (sc < 8)).any()  # saturated and subnormal scales
    o = g.prefill(torch.float32).cpu().numpy()
    ref, _ = oracle_prefill(pc, oc)
    assert_attention_close(o, ref, "K/V wide range")

"""NVFP4 paged KV-cache attention for AMD MI355X (gfx950).

The path: ``append`` (quantize bf16 or fp16 K/V into the packed NVFP4
cache), ``prefill`` (causal paged prefill over the cache) and ``decode``
(split-KV single-token decode); ``dequant`` reads cache rows back as
bf16 / fp16 / fp32; ``repack`` writes an fp16 copy of the pages a batch
reads (dequantize-ahead), which ``prefill`` can read instead of the packed
cache; ``decode_noalloc`` is ``decode`` without a workspace (a static
per-GPU scratch array in the library); ``prefill_a4q`` is the A4Q-style
prefill (query quantized to MX blocks in the kernel, QK on the block-scaled
MFMA).  All compute runs in the HIP library ``libnvfp4kv.so`` (C ABI
declared in ``include/nvfp4kv.h``); this package is a thin binding.
"""
from .binding import (DECODE_SCRATCH_BYTES, NVFP4KVCache, Nvfp4KVError, append,  # noqa: F401
                      decode, decode_noalloc, decode_workspace_size, dequant, load_library,
                      prefill, prefill_a4q, prefill_a4q_workspace_size, prefill_workspace_size,
                      repack)
from .build import LIB_PATH  # noqa: F401

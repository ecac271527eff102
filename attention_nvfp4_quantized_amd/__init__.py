"""NVFP4 paged KV-cache attention for AMD MI355X (gfx950).

The path: ``append`` (quantize bf16 or fp16 K/V into the packed NVFP4
cache), ``prefill`` (causal paged prefill over the cache) and ``decode``
(split-KV single-token decode); ``dequant`` reads cache rows back as
bf16 / fp16 / fp32; ``repack`` writes an fp16 copy of the pages a batch
reads (dequantize-ahead), which ``prefill`` can read instead of the packed
cache.  All compute runs in the HIP library ``libnvfp4kv.so`` (C ABI
declared in ``include/nvfp4kv.h``); this package is a thin binding.
"""
from .binding import (NVFP4KVCache, Nvfp4KVError, append, decode, decode_workspace_size,  # noqa: F401
                      dequant, load_library, prefill, prefill_workspace_size, repack)
from .build import LIB_PATH  # noqa: F401

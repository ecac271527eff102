"""CPU oracle for NVFP4 paged-KV attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the C-ABI library
and its Python binding) never imports, links or calls it, and it shares no
code with that path: no kernels, headers, tables or helpers.  Its inputs come
from the seeded generators in ``workload`` and nowhere else.

What it computes, in plain NumPy with float64 arithmetic wherever the pages
leave the precision open:

* ``codec``      -- the NVFP4 element and scale formats: E2M1 values packed
                    two per byte with one E4M3 scale per 16-value block
                    ("NVFP4 KV cache prefill vs decode performance", section
                    "NVFP4 stores 4.5 bits per value before padding"; "NVFP4
                    KV cache vs NVFP4 weights", section "NVFP4 KV cache vs
                    NVFP4 weights").
* ``cache``      -- the cache writer: quantize, choose block scales, pack,
                    and place the result in paged slots ("NVFP4 KV cache vs
                    NVFP4 weights", section "The cache quantizes values during
                    serving"), and the read-side dequantization.
* ``attention``  -- causal paged prefill and single-token decode with bf16
                    queries over the dequantized cache ("NVFP4 KV cache A4Q
                    prefill explained", section "Why NVFP4 KV cache A4Q
                    prefill exists"; "NVFP4 KV cache prefill vs decode
                    performance", section "NVFP4 KV cache prefill vs decode
                    performance").

Every function is the plain definition of its result.  No tiling, online
softmax, splitting or reordering of the fast kernels is mirrored here.
"""
from . import codec, cache, attention  # noqa: F401

"""Thin ctypes binding over ``libnvfp4kv.so`` (argument marshalling only).

Every step of the path runs in the HIP library; this module only checks tensor
dtypes/devices, passes device pointers and the current HIP stream, and allocates
the workspace tensors the C ABI asks for.  If the library is missing it raises:
there is no CPU or PyTorch fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

from .build import LIB_PATH

HEAD_DIM = 128
PAGE_SIZE = 16

_ERRORS = {-1: "EINVAL", -2: "EUNSUPPORTED", -3: "EWORKSPACE", -4: "EHIP"}


class Nvfp4KVError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_ERRORS.get(code, code)}: {msg}")
        self.code = code


class CacheDesc(ctypes.Structure):
    _fields_ = [("k_data", ctypes.c_void_p), ("k_scale", ctypes.c_void_p),
                ("v_data", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("k_global", ctypes.c_float), ("v_global", ctypes.c_float),
                ("num_pages", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("kv_format", ctypes.c_int32)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library {path} is not built; run __graft_entry__.build() "
                           "(there is no fallback path)")
    lib = ctypes.CDLL(path)
    P, I32, I64, F, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    C = ctypes.POINTER(CacheDesc)
    lib.nvfp4_kv_append.argtypes = [C, P, P, I64, I64, I32, P, I32, P]
    lib.nvfp4_kv_append.restype = ctypes.c_int
    lib.nvfp4_kv_dequant.argtypes = [C, P, I32, P, P, I32, P]
    lib.nvfp4_kv_dequant.restype = ctypes.c_int
    lib.nvfp4_kv_repack.argtypes = [C, C, P, I32, P, I32, I32, P]
    lib.nvfp4_kv_repack.restype = ctypes.c_int
    lib.paged_prefill_nvfp4_workspace_size.argtypes = [I32, I32, I32, I32, I32, I32, I32, I32]
    lib.paged_prefill_nvfp4_workspace_size.restype = SZ
    lib.paged_prefill_nvfp4.argtypes = [C, P, P, P, P, I32, I32, I32, I32, I32, I32, F, I32, P, I32,
                                        P, I32, P, SZ, P]
    lib.paged_prefill_nvfp4.restype = ctypes.c_int
    lib.paged_decode_nvfp4_workspace_size.argtypes = [I32, I32, I32, I32, I32, I32]
    lib.paged_decode_nvfp4_workspace_size.restype = SZ
    lib.paged_decode_nvfp4.argtypes = [C, P, P, P, I32, I32, I32, I32, F, P, I32, P, I32, P, SZ, P]
    lib.paged_decode_nvfp4.restype = ctypes.c_int
    lib.paged_prefill_nvfp4_a4q_workspace_size.argtypes = [I32, I32, I32, I32, I32, I32, I32, I32]
    lib.paged_prefill_nvfp4_a4q_workspace_size.restype = SZ
    lib.paged_prefill_nvfp4_a4q.argtypes = [C, P, P, P, P, I32, I32, I32, I32, I32, I32, F, I32, P,
                                            I32, P, I32, I32, P, SZ, P]
    lib.paged_prefill_nvfp4_a4q.restype = ctypes.c_int
    lib.paged_decode_nvfp4_noalloc.argtypes = [C, P, P, P, I32, I32, I32, I32, F, P, I32, P, I32, P]
    lib.paged_decode_nvfp4_noalloc.restype = ctypes.c_int
    lib.nvfp4kv_last_error.argtypes = []
    lib.nvfp4kv_last_error.restype = ctypes.c_char_p
    lib.nvfp4kv_version.argtypes = []
    lib.nvfp4kv_version.restype = ctypes.c_int32
    _lib = lib
    return lib


def _check(rc: int):
    if rc != 0:
        raise Nvfp4KVError(rc, load_library().nvfp4kv_last_error().decode())


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


_FORMATS = {"nvfp4": 0, "fp8": 1, "f16": 2}


class NVFP4KVCache:
    """Device memory of one layer's paged KV cache (allocated with torch, zero-filled).

    kv_format "nvfp4": packed E2M1 codes [pages][Hkv][16][64] plus E4M3 block scales
    [pages][Hkv][16][8] per K and V.  kv_format "fp8": the FP8 (E4M3FN) control cache, one byte
    per value [pages][Hkv][16][128] and no scale plane.  kv_format "f16": the fp16 copy that
    ``repack`` writes ([pages][Hkv][16][128] float16), read by ``prefill`` only."""

    def __init__(self, num_pages: int, num_kv_heads: int, device="cuda", k_global: float = 1.0,
                 v_global: float = 1.0, kv_format: str = "nvfp4"):
        if kv_format not in _FORMATS:
            raise ValueError(f"kv_format must be one of {sorted(_FORMATS)}, got {kv_format!r}")
        z = lambda s: torch.zeros(s, dtype=torch.uint8, device=device)  # noqa: E731
        if kv_format in ("fp8", "f16"):
            shape_d = (num_pages, num_kv_heads, PAGE_SIZE, HEAD_DIM * (1 if kv_format == "fp8" else 2))
            self.k_data, self.v_data = z(shape_d), z(shape_d)
            self.k_scale = self.v_scale = None
        else:
            shape_d = (num_pages, num_kv_heads, PAGE_SIZE, HEAD_DIM // 2)
            shape_s = (num_pages, num_kv_heads, PAGE_SIZE, HEAD_DIM // 16)
            self.k_data, self.k_scale = z(shape_d), z(shape_s)
            self.v_data, self.v_scale = z(shape_d), z(shape_s)
        self.kv_format = kv_format
        self.num_pages, self.num_kv_heads = num_pages, num_kv_heads
        self.k_global, self.v_global = float(k_global), float(v_global)

    def desc(self) -> CacheDesc:
        return CacheDesc(self.k_data.data_ptr(), _ptr(self.k_scale), self.v_data.data_ptr(),
                         _ptr(self.v_scale), self.k_global, self.v_global, self.num_pages,
                         PAGE_SIZE, self.num_kv_heads, HEAD_DIM, _FORMATS[self.kv_format])

    def nbytes(self) -> int:
        return sum(t.numel() for t in (self.k_data, self.k_scale, self.v_data, self.v_scale)
                   if t is not None)


def _need(t, dtype, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != dtype:
        raise TypeError(f"{name} must be a {dtype} CUDA tensor")


_IN_DTYPES = {torch.bfloat16: 0, torch.float16: 1}
_OUT_DTYPES = {torch.bfloat16: 0, torch.float32: 1, torch.float16: 2}
# attention outputs (prefill, decode): bf16 or float32 only
_ATTN_OUT_DTYPES = {torch.bfloat16: 0, torch.float32: 1}


def _attn_out_code(dtype) -> int:
    if dtype not in _ATTN_OUT_DTYPES:
        raise TypeError(f"attention output must be bfloat16 or float32, got {dtype}")
    return _ATTN_OUT_DTYPES[dtype]


def _check_out(out, rows: int, hq: int, device):
    if not isinstance(out, torch.Tensor) or not out.is_cuda or out.device != device:
        raise TypeError(f"out must be a CUDA tensor on {device}")
    if tuple(out.shape) != (rows, hq, HEAD_DIM) or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous [{rows}][{hq}][{HEAD_DIM}] tensor, "
                         f"got {tuple(out.shape)}")


def append(cache: NVFP4KVCache, k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor):
    """nvfp4_kv_append: k, v bf16 or fp16 [T][Hkv][128] (head/dim contiguous, same dtype);
    slot_mapping int64 [T]."""
    if k.dtype not in _IN_DTYPES or v.dtype != k.dtype:
        raise TypeError(f"k and v must both be bfloat16 or both float16, got {k.dtype}, {v.dtype}")
    _need(k, k.dtype, "k"); _need(v, k.dtype, "v")
    _need(slot_mapping, torch.int64, "slot_mapping")
    if k.shape != v.shape or k.dim() != 3 or k.shape[1:] != (cache.num_kv_heads, HEAD_DIM):
        raise ValueError(f"k/v must be [T][{cache.num_kv_heads}][{HEAD_DIM}]")
    if k.stride(2) != 1 or k.stride(1) != HEAD_DIM or v.stride(2) != 1 or v.stride(1) != HEAD_DIM:
        raise ValueError("k/v heads and head dims must be contiguous")
    if not slot_mapping.is_contiguous() or slot_mapping.numel() != k.shape[0]:
        raise ValueError("slot_mapping must be contiguous with one slot per token")
    d = cache.desc()
    _check(load_library().nvfp4_kv_append(ctypes.byref(d), k.data_ptr(), v.data_ptr(), k.stride(0),
                                          v.stride(0), _IN_DTYPES[k.dtype], slot_mapping.data_ptr(),
                                          k.shape[0], _stream()))


def dequant(cache: NVFP4KVCache, slot_mapping: torch.Tensor, out_dtype=torch.bfloat16):
    """nvfp4_kv_dequant: the cache rows of the given slots (int64 [T]; slot < 0 -> zero row) as
    (k, v), each [T][Hkv][128] of out_dtype (bfloat16, float16 or float32)."""
    _need(slot_mapping, torch.int64, "slot_mapping")
    if out_dtype not in _OUT_DTYPES:
        raise TypeError(f"out_dtype must be bfloat16, float16 or float32, got {out_dtype}")
    if not slot_mapping.is_contiguous() or slot_mapping.dim() != 1:
        raise ValueError("slot_mapping must be a contiguous 1-D tensor")
    t = slot_mapping.shape[0]
    k = torch.empty((t, cache.num_kv_heads, HEAD_DIM), dtype=out_dtype, device=slot_mapping.device)
    v = torch.empty_like(k)
    d = cache.desc()
    _check(load_library().nvfp4_kv_dequant(ctypes.byref(d), slot_mapping.data_ptr(), t,
                                           k.data_ptr(), v.data_ptr(), _OUT_DTYPES[out_dtype],
                                           _stream()))
    return k, v


def repack(src: NVFP4KVCache, dst: NVFP4KVCache, block_table: torch.Tensor,
           kv_lens: torch.Tensor, max_kv_len: int):
    """nvfp4_kv_repack: convert every page that holds keys of the given sequences from the NVFP4
    cache ``src`` into the fp16 copy ``dst`` (kv_format "f16", same pages, heads and global
    scales); ``prefill(dst, ...)`` then reads the copy with the same block table."""
    _need(block_table, torch.int32, "block_table"); _need(kv_lens, torch.int32, "kv_lens")
    if not block_table.is_contiguous() or block_table.dim() != 2:
        raise ValueError("block_table must be a contiguous [batch][stride] tensor")
    if kv_lens.numel() != block_table.shape[0]:
        raise ValueError("kv_lens must hold one length per block-table row")
    s, d = src.desc(), dst.desc()
    _check(load_library().nvfp4_kv_repack(ctypes.byref(s), ctypes.byref(d), block_table.data_ptr(),
                                          block_table.shape[1], kv_lens.data_ptr(),
                                          kv_lens.numel(), max_kv_len, _stream()))


def prefill_workspace_size(batch, total_q, max_q_len, max_kv_len, num_qo_heads, num_kv_heads,
                           num_splits=0) -> int:
    return load_library().paged_prefill_nvfp4_workspace_size(batch, total_q, max_q_len, max_kv_len,
                                                            num_qo_heads, num_kv_heads, HEAD_DIM,
                                                            num_splits)


def prefill(cache: NVFP4KVCache, q: torch.Tensor, cu_seqlens_q: torch.Tensor,
            kv_lens: torch.Tensor, block_table: torch.Tensor, max_q_len: int, max_kv_len: int,
            sm_scale: float, causal: bool = True, out: torch.Tensor | None = None,
            out_dtype=torch.bfloat16, return_lse: bool = False, num_splits: int = 0,
            workspace: torch.Tensor | None = None):
    """paged_prefill_nvfp4: q bf16 [total_q][Hq][128]; returns out (and lse if asked).
    out_dtype (or the dtype of a caller-supplied ``out``) must be bfloat16 or float32."""
    odt = _attn_out_code(out_dtype if out is None else out.dtype)
    _need(q, torch.bfloat16, "q"); _need(cu_seqlens_q, torch.int32, "cu_seqlens_q")
    _need(kv_lens, torch.int32, "kv_lens"); _need(block_table, torch.int32, "block_table")
    if not q.is_contiguous() or not block_table.is_contiguous() or block_table.dim() != 2:
        raise ValueError("q and block_table must be contiguous (block_table [batch][stride])")
    if q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise ValueError(f"q must be [total_q][Hq][{HEAD_DIM}], got {tuple(q.shape)}")
    total_q, hq = q.shape[0], q.shape[1]
    batch = kv_lens.numel()
    if cu_seqlens_q.numel() != batch + 1 or block_table.shape[0] != batch:
        raise ValueError(f"cu_seqlens_q must hold batch + 1 = {batch + 1} offsets and "
                         f"block_table {batch} rows (one per kv_lens entry)")
    if out is None:
        out = torch.empty((total_q, hq, HEAD_DIM), dtype=out_dtype, device=q.device)
    _check_out(out, total_q, hq, q.device)
    lse = torch.empty((total_q, hq), dtype=torch.float32, device=q.device) if return_lse else None
    ws_bytes = prefill_workspace_size(batch, total_q, max_q_len, max_kv_len, hq, cache.num_kv_heads,
                                      num_splits)
    if ws_bytes and (workspace is None or workspace.numel() < ws_bytes):
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    d = cache.desc()
    _check(load_library().paged_prefill_nvfp4(
        ctypes.byref(d), q.data_ptr(), cu_seqlens_q.data_ptr(), kv_lens.data_ptr(),
        block_table.data_ptr(), block_table.shape[1], batch, total_q, max_q_len, max_kv_len, hq,
        sm_scale, 1 if causal else 0, out.data_ptr(), odt,
        _ptr(lse), num_splits, _ptr(workspace) if ws_bytes else None, ws_bytes, _stream()))
    return (out, lse) if return_lse else out


_A4Q_FORMATS = {"mxfp8": 0, "mxfp4": 1}
_A4Q_K_ONE_TERM = 0x10


def prefill_a4q_workspace_size(batch, total_q, max_q_len, max_kv_len, num_qo_heads, num_kv_heads,
                               num_splits=0) -> int:
    return load_library().paged_prefill_nvfp4_a4q_workspace_size(
        batch, total_q, max_q_len, max_kv_len, num_qo_heads, num_kv_heads, HEAD_DIM, num_splits)


def prefill_a4q(cache: NVFP4KVCache, q: torch.Tensor, cu_seqlens_q: torch.Tensor,
                kv_lens: torch.Tensor, block_table: torch.Tensor, max_q_len: int, max_kv_len: int,
                sm_scale: float, q_format: str = "mxfp8", causal: bool = True,
                out: torch.Tensor | None = None, out_dtype=torch.bfloat16, return_lse: bool = False,
                num_splits: int = 0, workspace: torch.Tensor | None = None, k_terms: int = 2):
    """paged_prefill_nvfp4_a4q: ``prefill`` with the query quantized in the kernel to MX blocks
    (q_format "mxfp8" or "mxfp4") and QK on gfx950's block-scaled MFMA; NVFP4 caches only.
    k_terms 2 feeds K exactly (two E4M3 terms), 1 its one-term form (K rounded to one E4M3 term
    per value: half the QK matrix-core work)."""
    if q_format not in _A4Q_FORMATS:
        raise ValueError(f"q_format must be one of {sorted(_A4Q_FORMATS)}, got {q_format!r}")
    if k_terms not in (1, 2):
        raise ValueError(f"k_terms must be 1 or 2, got {k_terms!r}")
    odt = _attn_out_code(out_dtype if out is None else out.dtype)
    _need(q, torch.bfloat16, "q"); _need(cu_seqlens_q, torch.int32, "cu_seqlens_q")
    _need(kv_lens, torch.int32, "kv_lens"); _need(block_table, torch.int32, "block_table")
    if not q.is_contiguous() or not block_table.is_contiguous() or block_table.dim() != 2:
        raise ValueError("q and block_table must be contiguous (block_table [batch][stride])")
    if q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise ValueError(f"q must be [total_q][Hq][{HEAD_DIM}], got {tuple(q.shape)}")
    total_q, hq = q.shape[0], q.shape[1]
    batch = kv_lens.numel()
    if cu_seqlens_q.numel() != batch + 1 or block_table.shape[0] != batch:
        raise ValueError(f"cu_seqlens_q must hold batch + 1 = {batch + 1} offsets and "
                         f"block_table {batch} rows (one per kv_lens entry)")
    if out is None:
        out = torch.empty((total_q, hq, HEAD_DIM), dtype=out_dtype, device=q.device)
    _check_out(out, total_q, hq, q.device)
    lse = torch.empty((total_q, hq), dtype=torch.float32, device=q.device) if return_lse else None
    ws_bytes = prefill_a4q_workspace_size(batch, total_q, max_q_len, max_kv_len, hq,
                                          cache.num_kv_heads, num_splits)
    if ws_bytes and (workspace is None or workspace.numel() < ws_bytes):
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    d = cache.desc()
    _check(load_library().paged_prefill_nvfp4_a4q(
        ctypes.byref(d), q.data_ptr(), cu_seqlens_q.data_ptr(), kv_lens.data_ptr(),
        block_table.data_ptr(), block_table.shape[1], batch, total_q, max_q_len, max_kv_len, hq,
        sm_scale, 1 if causal else 0, out.data_ptr(), odt, _ptr(lse),
        _A4Q_FORMATS[q_format] | (_A4Q_K_ONE_TERM if k_terms == 1 else 0),
        num_splits, _ptr(workspace) if ws_bytes else None, ws_bytes, _stream()))
    return (out, lse) if return_lse else out


def decode_workspace_size(batch, max_kv_len, num_qo_heads, num_kv_heads, num_splits=0) -> int:
    return load_library().paged_decode_nvfp4_workspace_size(batch, max_kv_len, num_qo_heads,
                                                           num_kv_heads, HEAD_DIM, num_splits)


def decode(cache: NVFP4KVCache, q: torch.Tensor, kv_lens: torch.Tensor, block_table: torch.Tensor,
           max_kv_len: int, sm_scale: float, out: torch.Tensor | None = None,
           out_dtype=torch.bfloat16, return_lse: bool = False, num_splits: int = 0,
           workspace: torch.Tensor | None = None):
    """paged_decode_nvfp4: q bf16 [B][Hq][128]; returns out (and lse if asked).
    out_dtype (or the dtype of a caller-supplied ``out``) must be bfloat16 or float32."""
    odt = _attn_out_code(out_dtype if out is None else out.dtype)
    _need(q, torch.bfloat16, "q"); _need(kv_lens, torch.int32, "kv_lens")
    _need(block_table, torch.int32, "block_table")
    if not q.is_contiguous() or not block_table.is_contiguous() or block_table.dim() != 2:
        raise ValueError("q and block_table must be contiguous (block_table [batch][stride])")
    if q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise ValueError(f"q must be [batch][Hq][{HEAD_DIM}], got {tuple(q.shape)}")
    batch, hq = q.shape[0], q.shape[1]
    if kv_lens.numel() != batch or block_table.shape[0] != batch:
        raise ValueError(f"kv_lens and block_table must have one entry / row per sequence ({batch})")
    if out is None:
        out = torch.empty((batch, hq, HEAD_DIM), dtype=out_dtype, device=q.device)
    _check_out(out, batch, hq, q.device)
    lse = torch.empty((batch, hq), dtype=torch.float32, device=q.device) if return_lse else None
    ws_bytes = decode_workspace_size(batch, max_kv_len, hq, cache.num_kv_heads, num_splits)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=q.device)
    d = cache.desc()
    _check(load_library().paged_decode_nvfp4(
        ctypes.byref(d), q.data_ptr(), kv_lens.data_ptr(), block_table.data_ptr(),
        block_table.shape[1], batch, max_kv_len, hq, sm_scale, out.data_ptr(),
        odt, _ptr(lse), num_splits, workspace.data_ptr(),
        workspace.numel(), _stream()))
    return (out, lse) if return_lse else out


DECODE_SCRATCH_BYTES = 16 << 20  # the library's static decode scratch per GPU


def decode_noalloc(cache: NVFP4KVCache, q: torch.Tensor, kv_lens: torch.Tensor,
                   block_table: torch.Tensor, max_kv_len: int, sm_scale: float,
                   out: torch.Tensor | None = None, out_dtype=torch.bfloat16,
                   return_lse: bool = False, num_splits: int = 0):
    """paged_decode_nvfp4_noalloc: ``decode`` without a workspace (the library's static
    per-GPU scratch holds the partials; calls on one GPU must not overlap).  ``out`` and ``lse``
    are allocated here only when the caller passes none."""
    odt = _attn_out_code(out_dtype if out is None else out.dtype)
    _need(q, torch.bfloat16, "q"); _need(kv_lens, torch.int32, "kv_lens")
    _need(block_table, torch.int32, "block_table")
    if not q.is_contiguous() or not block_table.is_contiguous() or block_table.dim() != 2:
        raise ValueError("q and block_table must be contiguous (block_table [batch][stride])")
    if q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise ValueError(f"q must be [batch][Hq][{HEAD_DIM}], got {tuple(q.shape)}")
    batch, hq = q.shape[0], q.shape[1]
    if kv_lens.numel() != batch or block_table.shape[0] != batch:
        raise ValueError(f"kv_lens and block_table must have one entry / row per sequence ({batch})")
    if out is None:
        out = torch.empty((batch, hq, HEAD_DIM), dtype=out_dtype, device=q.device)
    _check_out(out, batch, hq, q.device)
    lse = torch.empty((batch, hq), dtype=torch.float32, device=q.device) if return_lse else None
    d = cache.desc()
    _check(load_library().paged_decode_nvfp4_noalloc(
        ctypes.byref(d), q.data_ptr(), kv_lens.data_ptr(), block_table.data_ptr(),
        block_table.shape[1], batch, max_kv_len, hq, sm_scale, out.data_ptr(), odt, _ptr(lse),
        num_splits, _stream()))
    return (out, lse) if return_lse else out

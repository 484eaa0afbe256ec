"""Decode attention over a KV cache (multiquery / grouped-query) for MI355X.

Thin ctypes binding of ``libkvdecode.so`` (C ABI in ``include/kvdecode.h``).
The functions carry the C names and only marshal arguments: torch tensors
become device pointers, the current torch stream becomes the HIP stream.
Every step of the computation runs in the library's HIP kernels; there is no
CPU fallback, and every entry point raises ``KvdLibraryMissing`` when the
built library cannot be loaded.

    cache = KVCache(k_cache, v_cache, lengths, num_q_heads)
    cache.append(k_new, v_new)      # write slot lengths[b], then lengths[b] += 1
    out = cache.attend(q)           # softmax(q K^T * scale) V over each valid prefix
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "KVD_OK", "KVD_EINVAL", "KVD_EUNSUPPORTED", "KVD_EALIGN", "KVD_ECAPACITY", "KVD_EHIP",
    "KVD_ENOMEM", "KVD_ELENGTH", "KVD_EPAGE", "KVD_ESCRATCH", "KVD_NOALLOC_SCRATCH_MIB", "KVD_F32", "KVD_FP8_E4M3", "KVD_BF16", "KVD_VARIANT_AUTO", "KVD_VARIANT_VALU",
    "KVD_VARIANT_MFMA", "KVD_VARIANT_LDS", "KVD_VARIANT_WAVE", "KVD_VARIANT_XCHG", "KvdError", "KvdLibraryMissing", "kvdecode_desc_t", "kvdecode_paged_desc_t", "kvdecode_fp8_desc_t", "kvdecode_create", "kvdecode_create_paged",
    "kvdecode_create_fp8", "kvdecode_create_fp8_paged", "kvdecode_fp8_paged_desc_t",
    "kvdecode_append", "kvdecode_attend", "kvdecode_append_attend", "kvdecode_append_attend_multi",
    "kvdecode_append_attend_noalloc", "kvdecode_status", "KVD_MAX_NEW_TOKENS", "KVD_TIME_PARTIAL", "KVD_TIME_COMBINE",
    "KVD_TIME_APPEND", "KVD_TIME_ALL",
    "kvdecode_reserve", "kvdecode_set_num_splits",
    "kvdecode_set_variant", "kvdecode_set_unified_max", "kvdecode_get_plan", "kvdecode_get_plan_multi",
    "kvdecode_timing_enable", "kvdecode_timing_read", "kvdecode_destroy", "kvdecode_strerror", "KVCache", "library",
    "LIB_PATH",
]

KVD_OK, KVD_EINVAL, KVD_EUNSUPPORTED, KVD_EALIGN = 0, -1, -2, -3
KVD_ECAPACITY, KVD_EHIP, KVD_ENOMEM, KVD_ELENGTH, KVD_EPAGE, KVD_ESCRATCH = -4, -5, -6, -7, -8, -9
KVD_NOALLOC_SCRATCH_MIB = 32
KVD_F32, KVD_BF16, KVD_FP8_E4M3 = 0, 1, 2
KVD_VARIANT_AUTO, KVD_VARIANT_VALU, KVD_VARIANT_MFMA, KVD_VARIANT_LDS, KVD_VARIANT_WAVE, KVD_VARIANT_XCHG = 0, 1, 2, 3, 4, 5
KVD_TIME_PARTIAL, KVD_TIME_COMBINE, KVD_TIME_APPEND, KVD_TIME_ALL = 1, 2, 4, 7

# KVD_LIBRARY may name another build of the same library (e.g. one compiled
# with different tuning constants); by default the in-tree build is used.
LIB_PATH = os.environ.get("KVD_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                         "libkvdecode.so")

EXPORTS = (
    "kvdecode_create", "kvdecode_create_paged", "kvdecode_create_fp8", "kvdecode_create_fp8_paged",
    "kvdecode_append", "kvdecode_attend",
    "kvdecode_append_attend", "kvdecode_append_attend_multi", "kvdecode_append_attend_noalloc",
    "kvdecode_status", "kvdecode_reserve",
    "kvdecode_set_num_splits", "kvdecode_set_variant", "kvdecode_set_unified_max", "kvdecode_get_plan",
    "kvdecode_get_plan_multi", "kvdecode_timing_enable", "kvdecode_timing_read", "kvdecode_destroy",
    "kvdecode_strerror",
)


class KvdLibraryMissing(RuntimeError):
    """The HIP library is not built (run ``__graft_entry__.build()``)."""


class KvdError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {kvdecode_strerror(code)} (code {code})")


class kvdecode_desc_t(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("capacity", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("lengths", ctypes.c_void_p),
    ]


class kvdecode_paged_desc_t(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32),
        ("max_pages", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("k_pages", ctypes.c_void_p), ("v_pages", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p), ("lengths", ctypes.c_void_p),
    ]


class kvdecode_fp8_desc_t(ctypes.Structure):
    _fields_ = [("cache", kvdecode_desc_t), ("k_exp", ctypes.c_void_p), ("v_exp", ctypes.c_void_p)]


class kvdecode_fp8_paged_desc_t(ctypes.Structure):
    _fields_ = [("pages", kvdecode_paged_desc_t), ("k_exp", ctypes.c_void_p), ("v_exp", ctypes.c_void_p)]


_lib = None


def library():
    """Load libkvdecode.so once; raise KvdLibraryMissing if it is absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise KvdLibraryMissing(f"{LIB_PATH} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, F, D = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.POINTER(ctypes.c_double)
    IP = ctypes.POINTER(ctypes.c_int32)
    sig = {
        "kvdecode_create": (I, [ctypes.POINTER(kvdecode_desc_t), ctypes.POINTER(P)]),
        "kvdecode_create_paged": (I, [ctypes.POINTER(kvdecode_paged_desc_t), ctypes.POINTER(P)]),
        "kvdecode_create_fp8": (I, [ctypes.POINTER(kvdecode_fp8_desc_t), ctypes.POINTER(P)]),
        "kvdecode_create_fp8_paged": (I, [ctypes.POINTER(kvdecode_fp8_paged_desc_t), ctypes.POINTER(P)]),
        "kvdecode_append": (I, [P, P, P, P]),
        "kvdecode_attend": (I, [P, P, P, F, P]),
        "kvdecode_append_attend": (I, [P, P, P, P, P, F, P]),
        "kvdecode_append_attend_multi": (I, [P, I, P, P, P, P, F, P]),
        "kvdecode_append_attend_noalloc": (I, [P, P, P, P, P, F, P]),
        "kvdecode_status": (I, [P, P]),
        "kvdecode_reserve": (I, [P, I]),
        "kvdecode_set_num_splits": (I, [P, I]),
        "kvdecode_set_variant": (I, [P, I]),
        "kvdecode_set_unified_max": (I, [P, I, F]),
        "kvdecode_get_plan": (I, [P, IP, IP, IP]),
        "kvdecode_get_plan_multi": (I, [P, I, IP, IP, IP]),
        "kvdecode_timing_enable": (I, [P, I, I]),
        "kvdecode_timing_read": (I, [P, D, D, D, IP, IP]),
        "kvdecode_destroy": (I, [P]),
        "kvdecode_strerror": (ctypes.c_char_p, [I]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(rc: int, where: str) -> int:
    if rc != KVD_OK:
        raise KvdError(rc, where)
    return rc


def _stream_ptr(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


_DT = {torch.float32: KVD_F32, torch.bfloat16: KVD_BF16}


# --- C-ABI mirrors -----------------------------------------------------------

def kvdecode_strerror(code: int) -> str:
    return library().kvdecode_strerror(code).decode()


def kvdecode_create(k_cache: torch.Tensor, v_cache: torch.Tensor, lengths: torch.Tensor,
                    num_q_heads: int) -> int:
    """Handle over caller-owned caches [B, Hkv, T_cap, d] and lengths [B] int32."""
    for t in (k_cache, v_cache):
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError("caches must be contiguous [B, Hkv, T_cap, d] tensors")
    if k_cache.shape != v_cache.shape or k_cache.dtype != v_cache.dtype:
        raise ValueError("k_cache and v_cache must match in shape and dtype")
    if k_cache.dtype not in _DT:
        raise ValueError(f"unsupported cache dtype {k_cache.dtype}")
    if lengths.dtype != torch.int32 or lengths.dim() != 1 or lengths.shape[0] != k_cache.shape[0]:
        raise ValueError("lengths must be an int32 [B] tensor")
    if not (k_cache.is_cuda and v_cache.is_cuda and lengths.is_cuda):
        raise ValueError("caches and lengths must be device tensors")
    B, Hkv, T_cap, D = k_cache.shape
    desc = kvdecode_desc_t(B, num_q_heads, Hkv, D, T_cap, _DT[k_cache.dtype],
                           k_cache.data_ptr(), v_cache.data_ptr(), lengths.data_ptr())
    h = ctypes.c_void_p()
    _check(library().kvdecode_create(ctypes.byref(desc), ctypes.byref(h)), "kvdecode_create")
    return h.value


def kvdecode_create_fp8(k_codes: torch.Tensor, v_codes: torch.Tensor, k_exp: torch.Tensor,
                        v_exp: torch.Tensor, lengths: torch.Tensor, num_q_heads: int) -> int:
    """Handle over an fp8 cache: E4M3 codes [B, Hkv, T_cap, d] uint8 and
    per-row power-of-two exponents [B, Hkv, T_cap] int8 for K and for V."""
    for t in (k_codes, v_codes):
        if t.dim() != 4 or not t.is_contiguous() or t.dtype != torch.uint8:
            raise ValueError("fp8 caches must be contiguous uint8 [B, Hkv, T_cap, d] tensors of codes")
    if k_codes.shape != v_codes.shape:
        raise ValueError("k and v codes must match in shape")
    for t in (k_exp, v_exp):
        if t.dtype != torch.int8 or tuple(t.shape) != tuple(k_codes.shape[:3]) or not t.is_contiguous():
            raise ValueError("exponents must be contiguous int8 [B, Hkv, T_cap] tensors")
    if lengths.dtype != torch.int32 or lengths.dim() != 1 or lengths.shape[0] != k_codes.shape[0]:
        raise ValueError("lengths must be an int32 [B] tensor")
    if not all(t.is_cuda for t in (k_codes, v_codes, k_exp, v_exp, lengths)):
        raise ValueError("caches, exponents and lengths must be device tensors")
    B, Hkv, T_cap, D = k_codes.shape
    desc = kvdecode_fp8_desc_t(kvdecode_desc_t(B, num_q_heads, Hkv, D, T_cap, KVD_FP8_E4M3,
                                               k_codes.data_ptr(), v_codes.data_ptr(), lengths.data_ptr()),
                               k_exp.data_ptr(), v_exp.data_ptr())
    h = ctypes.c_void_p()
    _check(library().kvdecode_create_fp8(ctypes.byref(desc), ctypes.byref(h)), "kvdecode_create_fp8")
    return h.value


def kvdecode_create_paged(k_pages: torch.Tensor, v_pages: torch.Tensor, block_table: torch.Tensor,
                          lengths: torch.Tensor, num_q_heads: int) -> int:
    """Handle over a caller-owned paged cache: pools [num_pages, Hkv, page_size, d],
    block table [B, max_pages] int32 and lengths [B] int32."""
    for t in (k_pages, v_pages):
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError("page pools must be contiguous [num_pages, Hkv, page_size, d] tensors")
    if k_pages.shape != v_pages.shape or k_pages.dtype != v_pages.dtype:
        raise ValueError("k_pages and v_pages must match in shape and dtype")
    if k_pages.dtype not in _DT:
        raise ValueError(f"unsupported cache dtype {k_pages.dtype}")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or not block_table.is_contiguous():
        raise ValueError("block_table must be a contiguous int32 [B, max_pages] tensor")
    B = block_table.shape[0]
    if lengths.dtype != torch.int32 or lengths.dim() != 1 or lengths.shape[0] != B:
        raise ValueError("lengths must be an int32 [B] tensor")
    if not (k_pages.is_cuda and v_pages.is_cuda and block_table.is_cuda and lengths.is_cuda):
        raise ValueError("pools, block table and lengths must be device tensors")
    num_pages, Hkv, page_size, D = k_pages.shape
    desc = kvdecode_paged_desc_t(B, num_q_heads, Hkv, D, page_size, num_pages, block_table.shape[1],
                                 _DT[k_pages.dtype], k_pages.data_ptr(), v_pages.data_ptr(),
                                 block_table.data_ptr(), lengths.data_ptr())
    h = ctypes.c_void_p()
    _check(library().kvdecode_create_paged(ctypes.byref(desc), ctypes.byref(h)), "kvdecode_create_paged")
    return h.value


def kvdecode_create_fp8_paged(k_pages: torch.Tensor, v_pages: torch.Tensor, k_exp: torch.Tensor,
                              v_exp: torch.Tensor, block_table: torch.Tensor, lengths: torch.Tensor,
                              num_q_heads: int) -> int:
    """Handle over an fp8 cache in page pools: E4M3 code pools
    [num_pages, Hkv, page_size, d] uint8, exponent pools [num_pages, Hkv,
    page_size] int8, block table [B, max_pages] int32, lengths [B] int32."""
    for t in (k_pages, v_pages):
        if t.dim() != 4 or not t.is_contiguous() or t.dtype != torch.uint8:
            raise ValueError("fp8 page pools must be contiguous uint8 [num_pages, Hkv, page_size, d] tensors")
    if k_pages.shape != v_pages.shape:
        raise ValueError("k and v pools must match in shape")
    for t in (k_exp, v_exp):
        if t.dtype != torch.int8 or tuple(t.shape) != tuple(k_pages.shape[:3]) or not t.is_contiguous():
            raise ValueError("exponent pools must be contiguous int8 [num_pages, Hkv, page_size] tensors")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or not block_table.is_contiguous():
        raise ValueError("block_table must be a contiguous int32 [B, max_pages] tensor")
    B = block_table.shape[0]
    if lengths.dtype != torch.int32 or lengths.dim() != 1 or lengths.shape[0] != B:
        raise ValueError("lengths must be an int32 [B] tensor")
    if not all(t.is_cuda for t in (k_pages, v_pages, k_exp, v_exp, block_table, lengths)):
        raise ValueError("pools, exponents, block table and lengths must be device tensors")
    num_pages, Hkv, page_size, D = k_pages.shape
    desc = kvdecode_fp8_paged_desc_t(
        kvdecode_paged_desc_t(B, num_q_heads, Hkv, D, page_size, num_pages, block_table.shape[1], KVD_FP8_E4M3,
                              k_pages.data_ptr(), v_pages.data_ptr(), block_table.data_ptr(), lengths.data_ptr()),
        k_exp.data_ptr(), v_exp.data_ptr())
    h = ctypes.c_void_p()
    _check(library().kvdecode_create_fp8_paged(ctypes.byref(desc), ctypes.byref(h)), "kvdecode_create_fp8_paged")
    return h.value


def kvdecode_append(h: int, k_new: torch.Tensor, v_new: torch.Tensor, stream=None) -> None:
    _check(library().kvdecode_append(h, _ptr(k_new), _ptr(v_new), _stream_ptr(stream)),
           "kvdecode_append")


def kvdecode_attend(h: int, q: torch.Tensor, out: torch.Tensor, scale: float, stream=None) -> None:
    _check(library().kvdecode_attend(h, _ptr(q), _ptr(out), float(scale), _stream_ptr(stream)),
           "kvdecode_attend")


def kvdecode_append_attend(h: int, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                           out: torch.Tensor, scale: float, stream=None) -> None:
    _check(library().kvdecode_append_attend(h, _ptr(k_new), _ptr(v_new), _ptr(q), _ptr(out),
                                            float(scale), _stream_ptr(stream)),
           "kvdecode_append_attend")


def kvdecode_append_attend_noalloc(h: int, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                                   out: torch.Tensor, scale: float, stream=None) -> None:
    """kvdecode_append_attend with its workspace in the library's static
    per-GPU buffer: no device allocation (calls on one GPU must not overlap)."""
    _check(library().kvdecode_append_attend_noalloc(h, _ptr(k_new), _ptr(v_new), _ptr(q), _ptr(out),
                                                    float(scale), _stream_ptr(stream)),
           "kvdecode_append_attend_noalloc")


KVD_MAX_NEW_TOKENS = 16


def kvdecode_append_attend_multi(h: int, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                                 out: torch.Tensor, scale: float, stream=None) -> None:
    """Several new tokens per sequence: k_new/v_new [B, Hkv, T, d], q/out [B, Hq, T, d]."""
    n = k_new.shape[2]
    _check(library().kvdecode_append_attend_multi(h, n, _ptr(k_new), _ptr(v_new), _ptr(q), _ptr(out),
                                                  float(scale), _stream_ptr(stream)),
           "kvdecode_append_attend_multi")


def kvdecode_status(h: int, stream=None) -> int:
    """Sync the stream and return (and clear) the sticky device status code."""
    return library().kvdecode_status(h, _stream_ptr(stream))


def kvdecode_reserve(h: int, max_new_tokens: int = 1) -> None:
    _check(library().kvdecode_reserve(h, max_new_tokens), "kvdecode_reserve")


def kvdecode_set_num_splits(h: int, n: int) -> None:
    _check(library().kvdecode_set_num_splits(h, n), "kvdecode_set_num_splits")


def kvdecode_set_unified_max(h: int, phi) -> None:
    """Unified softmax maximum phi (a bound on scale*q.k), or None to turn it off."""
    _check(library().kvdecode_set_unified_max(h, 0 if phi is None else 1, 0.0 if phi is None else float(phi)),
           "kvdecode_set_unified_max")


def kvdecode_set_variant(h: int, variant: int) -> None:
    _check(library().kvdecode_set_variant(h, variant), "kvdecode_set_variant")


def _plan_dict(v, s, c) -> dict:
    return {"variant": {1: "valu", 2: "mfma", 3: "lds", 4: "wave", 5: "xchg"}.get(v.value, str(v.value)),
            "num_splits": s.value, "split_tokens": c.value}


def kvdecode_get_plan(h: int) -> dict:
    v, s, c = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(library().kvdecode_get_plan(h, ctypes.byref(v), ctypes.byref(s), ctypes.byref(c)),
           "kvdecode_get_plan")
    return _plan_dict(v, s, c)


def kvdecode_get_plan_multi(h: int, n_tokens: int) -> dict:
    v, s, c = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(library().kvdecode_get_plan_multi(h, n_tokens, ctypes.byref(v), ctypes.byref(s), ctypes.byref(c)),
           "kvdecode_get_plan_multi")
    return _plan_dict(v, s, c)


def kvdecode_timing_enable(h: int, max_calls: int, what: int = None) -> None:
    """Time up to max_calls attends (and appends) with HIP events; `what` is
    a mask of KVD_TIME_PARTIAL / KVD_TIME_COMBINE / KVD_TIME_APPEND
    (default all three)."""
    what = KVD_TIME_ALL if what is None else what
    _check(library().kvdecode_timing_enable(h, max_calls, what), "kvdecode_timing_enable")


def kvdecode_timing_read(h: int) -> dict:
    p, c, a = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    na, nb = ctypes.c_int32(), ctypes.c_int32()
    _check(library().kvdecode_timing_read(h, ctypes.byref(p), ctypes.byref(c), ctypes.byref(a),
                                          ctypes.byref(na), ctypes.byref(nb)),
           "kvdecode_timing_read")
    return {"partial_ms": p.value, "combine_ms": c.value, "append_ms": a.value,
            "n_attend": na.value, "n_append": nb.value}


def kvdecode_destroy(h: int) -> None:
    _check(library().kvdecode_destroy(h), "kvdecode_destroy")


# --- convenience object --------------------------------------------------------

class KVCache:
    """A decode-time KV cache: caller-owned tensors plus a library handle.

    k_cache, v_cache: [B, Hkv, T_cap, d] (fp32 or bf16, on the GPU);
    lengths: [B] int32 on the GPU (valid tokens per sequence).
    The tensors must outlive the object; ``close()`` frees the handle.
    """

    def __init__(self, k_cache, v_cache, lengths, num_q_heads: int, block_table=None,
                 k_exp=None, v_exp=None):
        """Contiguous caches [B, Hkv, T_cap, d]; or -- with ``block_table``
        [B, max_pages] -- page pools [num_pages, Hkv, page_size, d]; or --
        with ``k_exp``/``v_exp`` [B, Hkv, T_cap] int8 -- an fp8 cache of
        uint8 E4M3 codes, whose queries and outputs are bf16 (with both, fp8
        page pools and exponent pools [num_pages, Hkv, page_size])."""
        self.k_cache, self.v_cache, self.lengths = k_cache, v_cache, lengths
        self.block_table = block_table
        self.k_exp, self.v_exp = k_exp, v_exp
        self.Hq = num_q_heads
        self.dtype = torch.bfloat16 if k_exp is not None else k_cache.dtype
        if k_exp is not None and block_table is not None:
            _, self.Hkv, page_size, self.D = k_cache.shape
            self.B = block_table.shape[0]
            self.T_cap = block_table.shape[1] * page_size
            self.handle = kvdecode_create_fp8_paged(k_cache, v_cache, k_exp, v_exp, block_table, lengths,
                                                    num_q_heads)
        elif k_exp is not None:
            self.B, self.Hkv, self.T_cap, self.D = k_cache.shape
            self.handle = kvdecode_create_fp8(k_cache, v_cache, k_exp, v_exp, lengths, num_q_heads)
        elif block_table is None:
            self.B, self.Hkv, self.T_cap, self.D = k_cache.shape
            self.handle = kvdecode_create(k_cache, v_cache, lengths, num_q_heads)
        else:
            _, self.Hkv, page_size, self.D = k_cache.shape
            self.B = block_table.shape[0]
            self.T_cap = block_table.shape[1] * page_size
            self.handle = kvdecode_create_paged(k_cache, v_cache, block_table, lengths, num_q_heads)

    def _check_token(self, t, heads, name):
        if t.shape != (self.B, heads, self.D) or t.dtype != self.dtype or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [{self.B}, {heads}, {self.D}] "
                             f"{self.dtype} tensor, got {tuple(t.shape)} {t.dtype}")
        if t.device != self.k_cache.device:
            raise ValueError(f"{name} is on {t.device}, the cache on {self.k_cache.device}")

    def append(self, k_new, v_new, stream=None):
        self._check_token(k_new, self.Hkv, "k_new")
        self._check_token(v_new, self.Hkv, "v_new")
        kvdecode_append(self.handle, k_new, v_new, stream)

    def attend(self, q, out=None, scale=None, stream=None):
        self._check_token(q, self.Hq, "q")
        if out is None:
            out = torch.empty_like(q)
        else:
            self._check_token(out, self.Hq, "out")
        kvdecode_attend(self.handle, q, out, self.D ** -0.5 if scale is None else scale, stream)
        return out

    def step(self, k_new, v_new, q, out=None, scale=None, stream=None):
        """append(k_new, v_new) then attend(q), in one call."""
        self._check_token(k_new, self.Hkv, "k_new")
        self._check_token(v_new, self.Hkv, "v_new")
        self._check_token(q, self.Hq, "q")
        if out is None:
            out = torch.empty_like(q)
        else:
            self._check_token(out, self.Hq, "out")
        kvdecode_append_attend(self.handle, k_new, v_new, q, out,
                               self.D ** -0.5 if scale is None else scale, stream)
        return out

    def step_multi(self, k_new, v_new, q, out=None, scale=None, stream=None):
        """Append T new tokens per sequence (k_new/v_new [B, Hkv, T, d]) and
        attend their queries (q [B, Hq, T, d]) causally, in one call."""
        T = k_new.shape[2] if k_new.dim() == 4 else -1
        for t, heads, name in ((k_new, self.Hkv, "k_new"), (v_new, self.Hkv, "v_new"), (q, self.Hq, "q")):
            if t.shape != (self.B, heads, T, self.D) or t.dtype != self.dtype or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous [{self.B}, {heads}, T, {self.D}] {self.dtype} "
                                 f"tensor with the same T, got {tuple(t.shape)} {t.dtype}")
            if t.device != self.k_cache.device:
                raise ValueError(f"{name} is on {t.device}, the cache on {self.k_cache.device}")
        if out is None:
            out = torch.empty_like(q)
        elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
            raise ValueError("out must match q")
        kvdecode_append_attend_multi(self.handle, k_new, v_new, q, out,
                                     self.D ** -0.5 if scale is None else scale, stream)
        return out

    def status(self, stream=None) -> int:
        return kvdecode_status(self.handle, stream)

    def reserve(self, max_new_tokens: int = 1):
        """Bind to the current device and allocate now the workspace of
        steps with up to max_new_tokens new tokens per sequence."""
        kvdecode_reserve(self.handle, max_new_tokens)

    def set_num_splits(self, n: int):
        kvdecode_set_num_splits(self.handle, n)

    def set_unified_max(self, phi):
        kvdecode_set_unified_max(self.handle, phi)

    def set_variant(self, variant: int):
        kvdecode_set_variant(self.handle, variant)

    def plan(self, n_tokens: int = 1) -> dict:
        """The plan of a step with n_tokens new tokens per sequence."""
        return kvdecode_get_plan(self.handle) if n_tokens == 1 else kvdecode_get_plan_multi(self.handle, n_tokens)

    def close(self):
        if self.handle is not None:
            kvdecode_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

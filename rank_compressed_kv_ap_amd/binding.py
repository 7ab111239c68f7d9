"""Python binding of libap.so: argument marshalling only.

Every call passes torch device tensors' data pointers and the current HIP
stream straight to the C ABI declared in include/ap.h; all arithmetic runs in
the library's kernels.  Importing this module fails loudly if the library has
not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libap.so")

AP_OK, AP_ERR_NULL_ARG, AP_ERR_BAD_SHAPE, AP_ERR_BAD_DTYPE, AP_ERR_UNSUPPORTED, \
    AP_ERR_OUT_OF_MEMORY, AP_ERR_HIP = range(7)
AP_F32, AP_BF16, AP_INT4 = 0, 1, 2
KERNEL_NAMES = ("select", "attn", "combine", "decode", "ema", "text")

EXPORTED = (
    "ap_compress", "ap_recompress", "ap_recompress_noalloc", "ap_cache_set_factors", "ap_cache_get_factors",
    "ap_cache_get_sigma", "ap_cache_info", "ap_decode_attn", "ap_free", "ap_timing_enable",
    "ap_timing_read", "ap_status_string", "ap_last_error", "ap_read_bandwidth",
)


class CompressParams(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_tokens", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("rank", ctypes.c_int32),
        ("oversample", ctypes.c_int32), ("power_iters", ctypes.c_int32), ("storage", ctypes.c_int32),
        ("reserved", ctypes.c_int32), ("seed", ctypes.c_uint64), ("omega", ctypes.c_void_p),
    ]


class DecodeParams(ctypes.Structure):
    _fields_ = [
        ("r_lo", ctypes.c_int32), ("top_k", ctypes.c_int32), ("scale", ctypes.c_float),
        ("n_text", ctypes.c_int32), ("text_k", ctypes.c_void_p), ("text_v", ctypes.c_void_p),
        ("sel_out", ctypes.c_void_p), ("splits", ctypes.c_int32),
        ("select_mode", ctypes.c_int32), ("ema_alpha", ctypes.c_float), ("ema_first", ctypes.c_int32),
        ("importance", ctypes.c_void_p), ("ema_scratch", ctypes.c_void_p),
        ("text_cache", ctypes.c_void_p), ("text_r_lo", ctypes.c_int32), ("text_top_k", ctypes.c_int32),
        ("text_sel_out", ctypes.c_void_p),
    ]


SELECT_MODES = {"logit": 0, "ema_token": 1, "ema_head": 2}


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m rank_compressed_kv_ap_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    lib.ap_compress.argtypes = [vp, vp, ctypes.POINTER(CompressParams), vp, ctypes.POINTER(vp)]
    lib.ap_recompress.argtypes = [vp, vp, vp, vp, ctypes.c_uint64, vp]
    lib.ap_recompress_noalloc.argtypes = [vp, vp, vp, vp, ctypes.c_uint64, vp]
    lib.ap_cache_set_factors.argtypes = [vp, vp, vp, vp, vp, vp]
    lib.ap_cache_get_factors.argtypes = [vp, vp, vp, vp, vp, vp]
    lib.ap_cache_get_sigma.argtypes = [vp, vp, vp, vp]
    lib.ap_cache_info.argtypes = [vp, ctypes.POINTER(CompressParams), ctypes.POINTER(ctypes.c_size_t),
                                  ctypes.POINTER(ctypes.c_size_t)]
    lib.ap_decode_attn.argtypes = [vp, vp, vp, ctypes.POINTER(DecodeParams), vp]
    lib.ap_free.argtypes = [vp]
    lib.ap_free.restype = None
    lib.ap_timing_enable.argtypes = [vp, i32]
    lib.ap_timing_read.argtypes = [vp, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(i32)]
    lib.ap_status_string.argtypes = [i32]
    lib.ap_status_string.restype = ctypes.c_char_p
    lib.ap_last_error.argtypes = []
    lib.ap_last_error.restype = ctypes.c_char_p
    lib.ap_read_bandwidth.argtypes = [vp, ctypes.c_size_t, i32, vp, ctypes.POINTER(ctypes.c_float)]
    for name in ("ap_compress", "ap_recompress", "ap_recompress_noalloc", "ap_cache_set_factors", "ap_cache_get_factors", "ap_cache_get_sigma",
                 "ap_cache_info", "ap_decode_attn", "ap_timing_enable", "ap_timing_read", "ap_read_bandwidth"):
        getattr(lib, name).restype = i32
    return lib


lib = load_library()


class APError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib.ap_status_string(status).decode()
        detail = lib.ap_last_error().decode()
        super().__init__(f"{where}: {msg} ({detail})")


def _check(status: int, where: str) -> None:
    if status != AP_OK:
        raise APError(status, where)


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def storage_code(dtype) -> int:
    """torch.float32, torch.bfloat16, or "int4" (4-bit U, bf16 B)."""
    if dtype == "int4":
        return AP_INT4
    if dtype == torch.float32:
        return AP_F32
    if dtype == torch.bfloat16:
        return AP_BF16
    raise ValueError(f"unsupported storage {dtype}")


def torch_dtype(storage: int) -> torch.dtype:
    """dtype of K, V, text tokens and B for a storage code."""
    return torch.float32 if storage == AP_F32 else torch.bfloat16


class Cache:
    """A factored visual cache (owned by the library) for a batch of sequences."""

    def __init__(self, handle: int, params: CompressParams):
        self._h = ctypes.c_void_p(handle)
        self.params = params

    @property
    def handle(self) -> ctypes.c_void_p:
        if not self._h:
            raise RuntimeError("cache already freed")
        return self._h

    @property
    def batch(self): return self.params.batch
    @property
    def n_tokens(self): return self.params.n_tokens
    @property
    def rank(self): return self.params.rank
    @property
    def width(self): return self.params.n_kv_heads * self.params.head_dim
    @property
    def dtype(self): return torch_dtype(self.params.storage)
    @property
    def u_dtype(self):
        """dtype of U in set_factors / get_factors (float32 values for 4-bit caches)."""
        return torch.float32 if self.params.storage == AP_INT4 else self.dtype

    def recompress(self, k: torch.Tensor, v: torch.Tensor, *, seed: int = 0,
                   omega: Optional[torch.Tensor] = None) -> None:
        """ap_recompress: factor new k, v [B, N, W] into this cache."""
        _check(lib.ap_recompress(self.handle, _ptr(k), _ptr(v), _ptr(omega), seed, _stream()),
               "ap_recompress")

    def recompress_noalloc(self, k: torch.Tensor, v: torch.Tensor, *, seed: int = 0,
                           omega: Optional[torch.Tensor] = None) -> None:
        """ap_recompress_noalloc: as recompress, with the library's fixed workspace."""
        _check(lib.ap_recompress_noalloc(self.handle, _ptr(k), _ptr(v), _ptr(omega), seed, _stream()),
               "ap_recompress_noalloc")

    def set_factors(self, U_k, B_k, U_v, B_v) -> None:
        _check(lib.ap_cache_set_factors(self.handle, _ptr(U_k), _ptr(B_k), _ptr(U_v), _ptr(B_v),
                                        _stream()), "ap_cache_set_factors")

    def get_factors(self):
        p = self.params
        dev = torch.device("cuda")
        U_k = torch.empty(p.batch, p.n_tokens, p.rank, dtype=self.u_dtype, device=dev)
        U_v = torch.empty_like(U_k)
        B_k = torch.empty(p.batch, p.rank, self.width, dtype=self.dtype, device=dev)
        B_v = torch.empty_like(B_k)
        _check(lib.ap_cache_get_factors(self.handle, _ptr(U_k), _ptr(B_k), _ptr(U_v), _ptr(B_v),
                                        _stream()), "ap_cache_get_factors")
        return U_k, B_k, U_v, B_v

    def get_sigma(self):
        p = self.params
        sk = torch.empty(p.batch, p.rank, dtype=torch.float32, device="cuda")
        sv = torch.empty_like(sk)
        _check(lib.ap_cache_get_sigma(self.handle, _ptr(sk), _ptr(sv), _stream()), "ap_cache_get_sigma")
        return sk, sv

    def info(self):
        p = CompressParams()
        fb, db = ctypes.c_size_t(), ctypes.c_size_t()
        _check(lib.ap_cache_info(self.handle, ctypes.byref(p), ctypes.byref(fb), ctypes.byref(db)),
               "ap_cache_info")
        return p, fb.value, db.value

    def timing_enable(self, max_calls: int) -> None:
        _check(lib.ap_timing_enable(self.handle, max_calls), "ap_timing_enable")

    def timing_read(self):
        ms = (ctypes.c_float * len(KERNEL_NAMES))()
        calls = ctypes.c_int32()
        _check(lib.ap_timing_read(self.handle, ms, ctypes.byref(calls)), "ap_timing_read")
        return dict(zip(KERNEL_NAMES, list(ms))), calls.value

    def free(self) -> None:
        if self._h:
            lib.ap_free(self._h)
            self._h = ctypes.c_void_p(None)

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def compress(k: Optional[torch.Tensor], v: Optional[torch.Tensor], *, batch: int, n_tokens: int,
             n_kv_heads: int, n_q_heads: int, head_dim: int, rank: int, storage: torch.dtype,
             oversample: int = 16, power_iters: int = 2, seed: int = 0,
             omega: Optional[torch.Tensor] = None) -> Cache:
    """ap_compress: factor k, v [B, N, W] (or allocate only when both are None)."""
    p = CompressParams(batch, n_tokens, n_kv_heads, n_q_heads, head_dim, rank, oversample,
                       power_iters, storage_code(storage), 0, seed, _ptr(omega))
    out = ctypes.c_void_p()
    _check(lib.ap_compress(_ptr(k), _ptr(v), ctypes.byref(p), _stream(), ctypes.byref(out)),
           "ap_compress")
    p.omega = None
    return Cache(out.value, p)


def decode(cache: Cache, q: torch.Tensor, *, r_lo: int, top_k: int, scale: float,
           text_k: Optional[torch.Tensor] = None, text_v: Optional[torch.Tensor] = None,
           out: Optional[torch.Tensor] = None, sel_out: Optional[torch.Tensor] = None,
           splits: int = 0, select: str = "logit", ema_alpha: float = 0.0,
           ema_first: bool = False, importance: Optional[torch.Tensor] = None,
           ema_scratch: Optional[torch.Tensor] = None, text_cache: Optional["Cache"] = None,
           text_r_lo: int = 0, text_top_k: int = 0,
           text_sel_out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """ap_decode_attn: q [B, Hq*d] float32 -> out [B, Hq*d] float32.

    select: "logit" (current-step low-rank logit), "ema_token" or "ema_head" (moving
    average of the attention weights; importance float32 [B, N] or [B, Hq, N] is read
    and updated in place; ema_scratch float32 [B, Hq, N] is the step's workspace).
    text_cache: the text tokens factored apart (a second segment, its own text_r_lo and
    text_top_k); text_k / text_v then hold the dense tokens appended since;
    text_sel_out int32 [B, Hq, text_top_k] receives that segment's selected ids."""
    if out is None:
        out = torch.empty_like(q)
    n_text = 0 if text_k is None else text_k.shape[1]
    p = DecodeParams(r_lo, top_k, scale, n_text, _ptr(text_k) if n_text else None,
                     _ptr(text_v) if n_text else None, _ptr(sel_out), splits,
                     SELECT_MODES[select], ema_alpha, 1 if ema_first else 0, _ptr(importance),
                     _ptr(ema_scratch), text_cache.handle.value if text_cache is not None else None,
                     text_r_lo, text_top_k, _ptr(text_sel_out))
    _check(lib.ap_decode_attn(cache.handle, _ptr(q), _ptr(out), ctypes.byref(p), _stream()),
           "ap_decode_attn")
    return out


def read_bandwidth(buf: torch.Tensor, passes: int = 10) -> float:
    """ap_read_bandwidth: the device's streaming-read rate over buf (GB/s)."""
    ms = ctypes.c_float()
    nbytes = buf.numel() * buf.element_size()
    _check(lib.ap_read_bandwidth(_ptr(buf), nbytes, passes, _stream(), ctypes.byref(ms)),
           "ap_read_bandwidth")
    return nbytes / (ms.value * 1e-3) / 1e9

"""ctypes binding of libtabit.so: argument marshalling only.

Every computation runs in the HIP library; this module checks tensor dtype,
device and contiguity, allocates outputs with torch when the caller passes
none, and forwards raw device pointers and the current HIP stream.  It fails
loudly if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtabit.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "tabit.h")

OK, EINVAL, ESHAPE, EALIGN, ERANGE, ENOSCHED, EHIP, ENOMEM = 0, -1, -2, -3, -4, -5, -6, -7
FMT_INT8, FMT_MXFP4 = 0, 1
PATH_MASKED, PATH_BITSERIAL, PATH_PLANES, PATH_HQDM = 0, 1, 3, 4
OPT_GEMM_CONFIG, OPT_MXFP4_CONFIG, OPT_PLANE_CONFIG, OPT_HQDM_CONFIG = 0, 1, 2, 3
PATH_MXFP4_GEMM = 2
ACT_NONE, ACT_GELU = 0, 1

_c_int, _c_void_p, _c_size_t, _c_float = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_float
_PINT = ctypes.POINTER(ctypes.c_int)

# name -> (restype, argtypes)
_SIGNATURES = {
    "tabit_create": (_c_int, [ctypes.POINTER(_c_void_p)]),
    "tabit_destroy": (None, [_c_void_p]),
    "tabit_last_error": (ctypes.c_char_p, [_c_void_p]),
    "tabit_version": (ctypes.c_char_p, []),
    "tabit_quantize_weights": (_c_int, [_c_void_p, _c_void_p, _c_int, _c_int, _c_int, _c_void_p,
                                        _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "tabit_set_step_schedule": (_c_int, [_c_void_p, _c_int, _c_int, _c_void_p, _c_void_p]),
    "tabit_schedule_lookup": (_c_int, [_c_void_p, _c_int, _c_int, _PINT, _PINT]),
    "tabit_hadamard_quant_act": (_c_int, [_c_void_p, _c_void_p, _c_int, _c_int, _c_int, _c_int,
                                          _c_void_p, _c_void_p, _c_void_p]),
    "tabit_masked_qgemm": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int,
                                    _c_int, _c_int, _c_int, _c_void_p, _c_void_p, _c_void_p]),
    "tabit_qgemm_bitserial": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                       _c_int, _c_int, _c_int, _c_int, _c_void_p, _c_void_p,
                                       _c_void_p]),
    "tabit_mxfp4_qgemm": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int,
                                   _c_int, _c_int, _c_float, _c_void_p, _c_void_p, _c_void_p]),
    "tabit_act_workspace_bytes": (_c_size_t, [_c_int, _c_int]),
    "tabit_scheduled_linear": (_c_int, [_c_void_p, _c_int, _c_int, _c_int, _c_void_p, _c_int,
                                        _c_int, _c_int, _c_int, _c_void_p, _c_void_p, _c_void_p,
                                        _c_void_p, _c_void_p, _c_size_t, _c_void_p, _c_void_p]),
    "tabit_noalloc_scratch_bytes": (_c_size_t, []),
    "tabit_scheduled_linear_noalloc": (_c_int, [_c_void_p, _c_int, _c_int, _c_int, _c_void_p,
                                                _c_int, _c_int, _c_int, _c_int, _c_void_p,
                                                _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                                _c_void_p]),
    "tabit_run_schedule": (_c_int, [_c_void_p, _c_int, _c_int, _c_void_p, _c_int, _c_void_p,
                                    _c_int, _c_int, _c_void_p, _c_size_t, _c_void_p, _c_void_p]),
    "tabit_autotune_gemm": (_c_int, [_c_void_p, _c_int, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                     _c_int, _c_int, _c_int, _c_int, _c_void_p, _c_int, _PINT,
                                     _c_void_p]),
    "tabit_set_option": (_c_int, [_c_void_p, _c_int, _c_int]),
    "tabit_gemm_config_info": (_c_int, [_c_int, _PINT, _PINT, _PINT]),
    "tabit_gemm_config_choose": (_c_int, [_c_int, _c_int, _c_int, _c_int]),
    "tabit_mxfp4_config_info": (_c_int, [_c_int, _PINT, _PINT]),
    "tabit_pack_weight_planes": (_c_int, [_c_void_p, _c_void_p, _c_int, _c_int, _c_void_p,
                                          _c_void_p]),
    "tabit_plane_qgemm": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int,
                                   _c_int, _c_int, _c_int, _c_void_p, _c_void_p, _c_void_p]),
    "tabit_plane_config_info": (_c_int, [_c_int, _PINT, _PINT, _PINT]),
    "tabit_plane_config_choose": (_c_int, [_c_int, _c_int, _c_int, _c_int]),
    "tabit_mxfp4_config_choose": (_c_int, [_c_int, _c_int, _c_int, _c_int]),
    "tabit_mfma_peak_probe": (_c_int, [_c_void_p, _c_int, _c_int, _c_void_p, _c_size_t,
                                       ctypes.POINTER(ctypes.c_double), _c_void_p]),
    "tabit_mfma_probe_sink_ints": (_c_size_t, [_c_int]),
    "tabit_weight_planes_bytes": (_c_size_t, [_c_int, _c_int]),
    "tabit_dmpq_workspace_bytes": (_c_size_t, [_c_int]),
    "tabit_gelu_quant_act": (_c_int, [_c_void_p, _c_void_p, _c_int, _c_int, _c_int, _c_int,
                                      _c_void_p, _c_void_p, _c_void_p]),
    "tabit_hqdm_quant_act": (_c_int, [_c_void_p, _c_void_p, _c_int, _c_int, _c_int, _c_void_p,
                                      _c_void_p, _c_void_p, _c_void_p]),
    "tabit_hqdm_qgemm": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                  _c_int, _c_int, _c_int, _c_int, _c_void_p, _c_void_p, _c_void_p]),
    "tabit_hqdm_config_info": (_c_int, [_c_int, _PINT, _PINT]),
    "tabit_dmpq_select": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_int, _c_int, _c_void_p,
                                   _c_int, _c_void_p, _c_void_p, _c_void_p, _c_size_t, _c_void_p]),
    "tabit_gated_linear": (_c_int, [_c_void_p, _c_void_p, _c_int, _c_int, _c_void_p, _c_int, _c_int,
                                    _c_int, _c_int, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                    _c_void_p, _c_size_t, _c_void_p, _c_void_p]),
}



class Layer(ctypes.Structure):
    """tabit_layer: one linear of a stack (device pointers as integers)."""
    _fields_ = [("M", ctypes.c_int), ("N", ctypes.c_int), ("K", ctypes.c_int),
                ("w_q", ctypes.c_void_p), ("w_scale", ctypes.c_void_p),
                ("w_fp4", ctypes.c_void_p), ("w_e8m0", ctypes.c_void_p),
                ("y_bf16", ctypes.c_void_p), ("input_from", ctypes.c_int),
                ("input_act", ctypes.c_int)]


_lib = None


def header_functions() -> list:
    """Names of the functions include/tabit.h declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(tabit_[a-z0-9_]+)\s*\(", text)))


def load() -> ctypes.CDLL:
    """Load libtabit.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m timestep_adaptive_bit_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class TabitError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"tabit status {status}: {message}")
        self.status = status


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _dev(t: torch.Tensor, dtype, name: str, shape=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def version() -> str:
    return load().tabit_version().decode()


def noalloc_scratch_bytes() -> int:
    return int(load().tabit_noalloc_scratch_bytes())


def act_workspace_bytes(M: int, K: int) -> int:
    return int(load().tabit_act_workspace_bytes(M, K))


def gemm_config_info(index: int = -1):
    """Number of INT8 GEMM configs (index < 0) or (bm, bn, k_groups) of one."""
    lib = load()
    if index < 0:
        return int(lib.tabit_gemm_config_info(-1, None, None, None))
    bm, bn, sk = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    st = lib.tabit_gemm_config_info(index, ctypes.byref(bm), ctypes.byref(bn), ctypes.byref(sk))
    if st != OK:
        raise TabitError(st, "bad config index")
    return bm.value, bn.value, sk.value


def mxfp4_config_info(index: int = -1):
    """Number of MXFP4 GEMM configs (index < 0) or (bm, bn) of one."""
    lib = load()
    if index < 0:
        return int(lib.tabit_mxfp4_config_info(-1, None, None))
    bm, bn = ctypes.c_int(), ctypes.c_int()
    st = lib.tabit_mxfp4_config_info(index, ctypes.byref(bm), ctypes.byref(bn))
    if st != OK:
        raise TabitError(st, "bad config index")
    return bm.value, bn.value


def hqdm_config_info(index: int = -1):
    """Number of HQ-DM GEMM configs (index < 0) or (bm, bn) of one."""
    lib = load()
    if index < 0:
        return int(lib.tabit_hqdm_config_info(-1, None, None))
    bm, bn = ctypes.c_int(), ctypes.c_int()
    st = lib.tabit_hqdm_config_info(index, ctypes.byref(bm), ctypes.byref(bn))
    if st != OK:
        raise TabitError(st, "bad config index")
    return bm.value, bn.value


def dmpq_workspace_bytes(M: int) -> int:
    return int(load().tabit_dmpq_workspace_bytes(M))


def weight_planes_bytes(N: int, K: int) -> int:
    return int(load().tabit_weight_planes_bytes(N, K))


def plane_config_info(index: int = -1):
    """Number of plane-major GEMM configs (index < 0) or (bm, bn, k_groups) of one."""
    lib = load()
    if index < 0:
        return int(lib.tabit_plane_config_info(-1, None, None, None))
    bm, bn, kg = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    st = lib.tabit_plane_config_info(index, ctypes.byref(bm), ctypes.byref(bn), ctypes.byref(kg))
    if st != OK:
        raise TabitError(st, "bad config index")
    return bm.value, bn.value, kg.value


def plane_config_choose(M: int, N: int, K: int, num_cus: int = 0) -> int:
    """Index of the plane-major GEMM configuration the library picks for M x N x K."""
    st = int(load().tabit_plane_config_choose(M, N, K, num_cus))
    if st < 0:
        raise TabitError(st, "bad shape")
    return st


def mxfp4_config_choose(M: int, N: int, K: int, num_cus: int = 0) -> int:
    """Index of the MXFP4 GEMM configuration the library picks for M x N x K."""
    st = int(load().tabit_mxfp4_config_choose(M, N, K, num_cus))
    if st < 0:
        raise TabitError(st, "bad shape")
    return st


def gemm_config_choose(M: int, N: int, K: int, num_cus: int = 0) -> int:
    return int(load().tabit_gemm_config_choose(M, N, K, num_cus))


class Context:
    """A tabit_ctx: schedule table, options and last error (host state only)."""

    def __init__(self):
        self._lib = load()
        h = ctypes.c_void_p()
        st = self._lib.tabit_create(ctypes.byref(h))
        if st != OK:
            raise TabitError(st, "tabit_create failed")
        self._h = h

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            self._lib.tabit_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def handle(self):
        return self._h

    def last_error(self) -> str:
        return self._lib.tabit_last_error(self._h).decode()

    def _check(self, st: int) -> None:
        if st != OK:
            raise TabitError(st, self.last_error())

    # ------------------------------------------------------------ options
    def set_option(self, option: int, value: int) -> None:
        self._check(self._lib.tabit_set_option(self._h, option, value))

    # ------------------------------------------------------------ schedule
    def set_step_schedule(self, k_bits, fmt=None) -> None:
        import numpy as np
        k = np.ascontiguousarray(k_bits, dtype=np.uint8)
        if k.ndim != 2:
            raise ValueError("k_bits must be [steps, layers]")
        f = None if fmt is None else np.ascontiguousarray(fmt, dtype=np.uint8)
        if f is not None and f.shape != k.shape:
            raise ValueError("fmt must match k_bits' shape")
        st = self._lib.tabit_set_step_schedule(self._h, k.shape[0], k.shape[1],
                                               k.ctypes.data, None if f is None else f.ctypes.data)
        self._check(st)

    def schedule_lookup(self, step: int, layer: int) -> Tuple[int, int]:
        k, f = ctypes.c_int(), ctypes.c_int()
        self._check(self._lib.tabit_schedule_lookup(self._h, step, layer, ctypes.byref(k), ctypes.byref(f)))
        return k.value, f.value

    # ------------------------------------------------------------ kernels
    def quantize_weights(self, w: torch.Tensor, had_block: int, int8: bool = True, mx: bool = False,
                         out=None):
        """bf16 [N, K] -> dict with w_q/w_scale (int8) and/or w_fp4/w_e8m0 (mx)."""
        N, K = w.shape
        _dev(w, torch.bfloat16, "w")
        out = dict(out or {})
        dev = w.device
        if int8:
            out.setdefault("w_q", torch.empty((N, K), dtype=torch.int8, device=dev))
            out.setdefault("w_scale", torch.empty((N,), dtype=torch.float32, device=dev))
            _dev(out["w_q"], torch.int8, "w_q", (N, K))
            _dev(out["w_scale"], torch.float32, "w_scale", (N,))
        if mx:
            out.setdefault("w_fp4", torch.empty((N, K // 2), dtype=torch.uint8, device=dev))
            out.setdefault("w_e8m0", torch.empty((N, K // 32), dtype=torch.uint8, device=dev))
            _dev(out["w_fp4"], torch.uint8, "w_fp4", (N, K // 2))
            _dev(out["w_e8m0"], torch.uint8, "w_e8m0", (N, K // 32))
        st = self._lib.tabit_quantize_weights(
            self._h, w.data_ptr(), N, K, had_block,
            _ptr(out.get("w_q")) if int8 else None, _ptr(out.get("w_scale")) if int8 else None,
            _ptr(out.get("w_fp4")) if mx else None, _ptr(out.get("w_e8m0")) if mx else None,
            _stream(dev))
        self._check(st)
        return out

    def hadamard_quant_act(self, x: torch.Tensor, had_block: int, fmt: int = FMT_INT8,
                           x_q: Optional[torch.Tensor] = None, x_scale: Optional[torch.Tensor] = None):
        """bf16 [M, K] -> (codes, scales): int8 [M, K] + fp32 [M], or fp4 [M, K/2] + e8m0 [M, K/32]."""
        _dev(x, torch.bfloat16, "x")
        M, K = x.shape
        dev = x.device
        if fmt == FMT_INT8:
            x_q = torch.empty((M, K), dtype=torch.int8, device=dev) if x_q is None else x_q
            x_scale = torch.empty((M,), dtype=torch.float32, device=dev) if x_scale is None else x_scale
            _dev(x_q, torch.int8, "x_q", (M, K))
            _dev(x_scale, torch.float32, "x_scale", (M,))
        else:
            x_q = torch.empty((M, K // 2), dtype=torch.uint8, device=dev) if x_q is None else x_q
            x_scale = torch.empty((M, K // 32), dtype=torch.uint8, device=dev) if x_scale is None else x_scale
            _dev(x_q, torch.uint8, "x_q", (M, K // 2))
            _dev(x_scale, torch.uint8, "x_scale", (M, K // 32))
        st = self._lib.tabit_hadamard_quant_act(self._h, x.data_ptr(), M, K, had_block, fmt,
                                                x_q.data_ptr(), x_scale.data_ptr(), _stream(dev))
        self._check(st)
        return x_q, x_scale

    def _gemm_i8(self, fn, x_q, x_scale, w_q, w_scale, k_bits, y=None, acc=None, want_y=True,
                 want_acc=False, planes=False):
        _dev(x_q, torch.int8, "x_q")
        M, K = x_q.shape
        if planes:
            _dev(w_q, torch.int32, "w_planes")
            if w_q.dim() != 4 or w_q.shape[0] != 8 or w_q.shape[1] != (K + 127) // 128 or w_q.shape[3] != 4:
                raise ValueError("w_planes must be [8][ceil(K/128)][N][4] words")
            N = w_q.shape[2]
        else:
            _dev(w_q, torch.int8, "w_q")
            N = w_q.shape[0]
            if w_q.shape[1] != K:
                raise ValueError("x_q and w_q disagree on K")
        _dev(x_scale, torch.float32, "x_scale", (M,))
        _dev(w_scale, torch.float32, "w_scale", (N,))
        dev = x_q.device
        if want_y and y is None:
            y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        if want_acc and acc is None:
            acc = torch.empty((M, N), dtype=torch.int32, device=dev)
        if y is not None:
            _dev(y, torch.bfloat16, "y", (M, N))
        if acc is not None:
            _dev(acc, torch.int32, "acc", (M, N))
        st = fn(self._h, x_q.data_ptr(), x_scale.data_ptr(), w_q.data_ptr(), w_scale.data_ptr(),
                M, N, K, k_bits, _ptr(y), _ptr(acc), _stream(dev))
        self._check(st)
        return y, acc

    def masked_qgemm(self, x_q, x_scale, w_q, w_scale, k_bits, y=None, acc=None, want_y=True,
                     want_acc=False):
        return self._gemm_i8(self._lib.tabit_masked_qgemm, x_q, x_scale, w_q, w_scale, k_bits, y,
                             acc, want_y, want_acc)

    def qgemm_bitserial(self, x_q, x_scale, w_q, w_scale, k_bits, y=None, acc=None, want_y=True,
                        want_acc=False):
        return self._gemm_i8(self._lib.tabit_qgemm_bitserial, x_q, x_scale, w_q, w_scale, k_bits, y,
                             acc, want_y, want_acc)

    def gelu_quant_act(self, x: torch.Tensor, had_block: int, x_q=None, x_scale=None,
                       fmt: int = FMT_INT8):
        """Down projection's input codes with the GELU folded in: int8 [M, K] + fp32 [M], or
        (fmt = FMT_MXFP4) fp4 [M, K/2] + e8m0 [M, K/32]."""
        _dev(x, torch.bfloat16, "x")
        M, K = x.shape
        dev = x.device
        if fmt == FMT_INT8:
            x_q = torch.empty((M, K), dtype=torch.int8, device=dev) if x_q is None else x_q
            x_scale = torch.empty((M,), dtype=torch.float32, device=dev) if x_scale is None else x_scale
            _dev(x_q, torch.int8, "x_q", (M, K))
            _dev(x_scale, torch.float32, "x_scale", (M,))
        else:
            x_q = torch.empty((M, K // 2), dtype=torch.uint8, device=dev) if x_q is None else x_q
            x_scale = torch.empty((M, K // 32), dtype=torch.uint8, device=dev) if x_scale is None else x_scale
            _dev(x_q, torch.uint8, "x_q", (M, K // 2))
            _dev(x_scale, torch.uint8, "x_scale", (M, K // 32))
        st = self._lib.tabit_gelu_quant_act(self._h, x.data_ptr(), M, K, had_block, fmt,
                                            x_q.data_ptr(), x_scale.data_ptr(), _stream(dev))
        self._check(st)
        return x_q, x_scale

    def hqdm_quant_act(self, x: torch.Tensor, had_block: int):
        """HQ-DM single-Hadamard codes: (x_hi int8 [M,K], x_lo int8 [M,K], x_scale fp32 [M])."""
        _dev(x, torch.bfloat16, "x")
        M, K = x.shape
        hi = torch.empty((M, K), dtype=torch.int8, device=x.device)
        lo = torch.empty((M, K), dtype=torch.int8, device=x.device)
        sc = torch.empty((M,), dtype=torch.float32, device=x.device)
        st = self._lib.tabit_hqdm_quant_act(self._h, x.data_ptr(), M, K, had_block, hi.data_ptr(),
                                            lo.data_ptr(), sc.data_ptr(), _stream(x.device))
        self._check(st)
        return hi, lo, sc

    def hqdm_qgemm(self, x_hi, x_lo, x_scale, w_q, w_scale, k_bits, y=None, want_y=True,
                   want_acc=False):
        """y bf16 [M,N] and/or the exact int64 accumulator of Z . W_k^T."""
        _dev(x_hi, torch.int8, "x_hi")
        M, K = x_hi.shape
        _dev(x_lo, torch.int8, "x_lo", (M, K))
        _dev(w_q, torch.int8, "w_q")
        N = w_q.shape[0]
        if w_q.shape[1] != K:
            raise ValueError("x and w_q disagree on K")
        _dev(x_scale, torch.float32, "x_scale", (M,))
        _dev(w_scale, torch.float32, "w_scale", (N,))
        if want_y and y is None:
            y = torch.empty((M, N), dtype=torch.bfloat16, device=x_hi.device)
        acc = torch.empty((M, N), dtype=torch.int64, device=x_hi.device) if want_acc else None
        st = self._lib.tabit_hqdm_qgemm(self._h, x_hi.data_ptr(), x_lo.data_ptr(), x_scale.data_ptr(),
                                        w_q.data_ptr(), w_scale.data_ptr(), M, N, K, k_bits, _ptr(y),
                                        _ptr(acc), _stream(x_hi.device))
        self._check(st)
        return y, acc

    def pack_weight_planes(self, w_q: torch.Tensor, out: Optional[torch.Tensor] = None):
        """Plane-major copy of int8 codes [N][K]: int32 tensor [8][ceil(K/128)][N][4] (uint32 words)."""
        _dev(w_q, torch.int8, "w_q")
        N, K = w_q.shape
        shape = (8, (K + 127) // 128, N, 4)
        if out is None:
            out = torch.empty(shape, dtype=torch.int32, device=w_q.device)
        _dev(out, torch.int32, "w_planes", shape)
        st = self._lib.tabit_pack_weight_planes(self._h, w_q.data_ptr(), N, K, out.data_ptr(),
                                                _stream(w_q.device))
        self._check(st)
        return out

    def plane_qgemm(self, x_q, x_scale, w_planes, w_scale, k_bits, y=None, acc=None, want_y=True,
                    want_acc=False):
        return self._gemm_i8(self._lib.tabit_plane_qgemm, x_q, x_scale, w_planes, w_scale, k_bits,
                             y, acc, want_y, want_acc, planes=True)

    def mxfp4_qgemm(self, x_fp4, x_e8m0, w_fp4, w_e8m0, out_scale: float, y=None, acc=None,
                    want_y=True, want_acc=False):
        for t, n in ((x_fp4, "x_fp4"), (x_e8m0, "x_e8m0"), (w_fp4, "w_fp4"), (w_e8m0, "w_e8m0")):
            _dev(t, torch.uint8, n)
        M, KB = x_fp4.shape
        N = w_fp4.shape[0]
        K = 2 * KB
        if w_fp4.shape[1] != KB or x_e8m0.shape != (M, K // 32) or w_e8m0.shape != (N, K // 32):
            raise ValueError("inconsistent MXFP4 operand shapes")
        dev = x_fp4.device
        if want_y and y is None:
            y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        if want_acc and acc is None:
            acc = torch.empty((M, N), dtype=torch.float32, device=dev)
        if y is not None:
            _dev(y, torch.bfloat16, "y", (M, N))
        if acc is not None:
            _dev(acc, torch.float32, "acc", (M, N))
        st = self._lib.tabit_mxfp4_qgemm(self._h, x_fp4.data_ptr(), x_e8m0.data_ptr(),
                                         w_fp4.data_ptr(), w_e8m0.data_ptr(), M, N, K,
                                         float(out_scale), _ptr(y), _ptr(acc), _stream(dev))
        self._check(st)
        return y, acc

    def scheduled_linear(self, step: int, layer: int, x: torch.Tensor, weights: dict,
                         had_block: int, act_ws: torch.Tensor, y: Optional[torch.Tensor] = None,
                         path: int = PATH_MASKED):
        """One linear at (step, layer): schedule lookup, quantize, GEMM -- all in the library."""
        _dev(x, torch.bfloat16, "x")
        M, K = x.shape
        wq = weights.get("w_planes") if path == PATH_PLANES else weights.get("w_q")
        wf = weights.get("w_fp4")
        if wq is not None:
            N = wq.shape[2] if path == PATH_PLANES else wq.shape[0]   # planes: [8][S][N][4]
        else:
            N = wf.shape[0]
        if y is None:
            y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
        _dev(y, torch.bfloat16, "y", (M, N))
        st = self._lib.tabit_scheduled_linear(
            self._h, step, layer, path, x.data_ptr(), M, N, K, had_block,
            _ptr(wq), _ptr(weights.get("w_scale")), _ptr(wf), _ptr(weights.get("w_e8m0")),
            act_ws.data_ptr(), act_ws.numel() * act_ws.element_size(), y.data_ptr(),
            _stream(x.device))
        self._check(st)
        return y

    def scheduled_linear_noalloc(self, step: int, layer: int, x: torch.Tensor, weights: dict,
                                 had_block: int, y: torch.Tensor, path: int = PATH_MASKED):
        """As scheduled_linear, with the library's static device scratch instead of a
        workspace; `y` [M, N] bf16 must be given (nothing is allocated here)."""
        _dev(x, torch.bfloat16, "x")
        M, K = x.shape
        N = y.shape[1]
        _dev(y, torch.bfloat16, "y", (M, N))
        wq = weights.get("w_planes") if path == PATH_PLANES else weights.get("w_q")
        st = self._lib.tabit_scheduled_linear_noalloc(
            self._h, step, layer, path, x.data_ptr(), M, N, K, had_block,
            _ptr(wq), _ptr(weights.get("w_scale")), _ptr(weights.get("w_fp4")),
            _ptr(weights.get("w_e8m0")), y.data_ptr(), _stream(x.device))
        self._check(st)
        return y

    def dmpq_select(self, x_in: torch.Tensor, x_out: torch.Tensor, theta: Optional[torch.Tensor],
                    fmt: Optional[torch.Tensor], gamma: Optional[torch.Tensor],
                    ws: Optional[torch.Tensor] = None):
        """Gamma of a block (device fp64) and fmt[l] = Gamma > theta[l] ? INT8 : MXFP4 (device)."""
        _dev(x_in, torch.bfloat16, "x_in")
        M, H = x_in.shape
        _dev(x_out, torch.bfloat16, "x_out", (M, H))
        n = 0
        if theta is not None:
            n = theta.numel()
            _dev(theta, torch.float32, "theta", (n,))
            _dev(fmt, torch.uint8, "fmt", (n,))
        if gamma is not None:
            _dev(gamma, torch.float64, "gamma", (1,))
        if ws is None:
            ws = torch.empty(dmpq_workspace_bytes(M), dtype=torch.uint8, device=x_in.device)
        st = self._lib.tabit_dmpq_select(self._h, x_in.data_ptr(), x_out.data_ptr(), M, H,
                                         _ptr(theta), n, _ptr(fmt), _ptr(gamma), ws.data_ptr(),
                                         ws.numel() * ws.element_size(), _stream(x_in.device))
        self._check(st)

    def gated_linear(self, fmt_dev: torch.Tensor, k_bits: int, x: torch.Tensor, weights: dict,
                     had_block: int, act_ws: torch.Tensor, y: Optional[torch.Tensor] = None,
                     path: int = PATH_MASKED):
        """One linear whose format is the device byte fmt_dev (both weight formats needed)."""
        _dev(x, torch.bfloat16, "x")
        M, K = x.shape
        wq = weights["w_planes"] if path == PATH_PLANES else weights["w_q"]
        N = wq.shape[2] if path == PATH_PLANES else wq.shape[0]
        if y is None:
            y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
        _dev(y, torch.bfloat16, "y", (M, N))
        st = self._lib.tabit_gated_linear(
            self._h, fmt_dev.data_ptr(), k_bits, path, x.data_ptr(), M, N, K, had_block,
            wq.data_ptr(), weights["w_scale"].data_ptr(), weights["w_fp4"].data_ptr(),
            weights["w_e8m0"].data_ptr(), act_ws.data_ptr(), act_ws.numel() * act_ws.element_size(),
            y.data_ptr(), _stream(x.device))
        self._check(st)
        return y

    def run_schedule(self, first_step: int, num_steps: int, layers, x_ptrs, had_block: int,
                     act_ws: torch.Tensor, path: int = PATH_MASKED, gemm_events=None,
                     stream: Optional[int] = None):
        """Native driver over steps [first_step, first_step+num_steps) x all layers.

        layers: a ctypes array of Layer; x_ptrs: a ctypes array of c_void_p of
        length num_steps * len(layers); gemm_events: None or a ctypes array of
        2 * num_steps * len(layers) hipEvent_t handles (c_void_p).
        """
        if stream is None:
            stream = _stream(act_ws.device)
        st = self._lib.tabit_run_schedule(
            self._h, first_step, num_steps, ctypes.cast(layers, ctypes.c_void_p), len(layers),
            ctypes.cast(x_ptrs, ctypes.c_void_p), had_block, path, act_ws.data_ptr(),
            act_ws.numel() * act_ws.element_size(),
            None if gemm_events is None else ctypes.cast(gemm_events, ctypes.c_void_p), stream)
        self._check(st)

    def mfma_peak_probe(self, kind: int = 0, iters: int = 20000, device="cuda:0") -> float:
        """Sustained matrix-core rate (ops or flops per second) of the device at its
        running clock: kind 0 INT8 MFMA, 1 FP4 scaled MFMA.  Synchronizes."""
        dev = torch.device(device)
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        n = int(self._lib.tabit_mfma_probe_sink_ints(cus))
        sink = torch.empty(n, dtype=torch.int32, device=dev)
        out = ctypes.c_double()
        st = self._lib.tabit_mfma_peak_probe(self._h, kind, iters, sink.data_ptr(), n,
                                             ctypes.byref(out), _stream(dev))
        self._check(st)
        return out.value

    def autotune_gemm(self, path: int, x_q, x_scale, w_q, w_scale, M: int, N: int, K: int,
                      k_bits: int, y: torch.Tensor, reps: int = 3) -> int:
        """Time every tile configuration for (path, M, N, K); the ctx keeps the fastest."""
        best = ctypes.c_int(-1)
        st = self._lib.tabit_autotune_gemm(self._h, path, x_q.data_ptr(), x_scale.data_ptr(),
                                           w_q.data_ptr(), w_scale.data_ptr(), M, N, K, k_bits,
                                           y.data_ptr(), reps, ctypes.byref(best), _stream(y.device))
        self._check(st)
        return best.value

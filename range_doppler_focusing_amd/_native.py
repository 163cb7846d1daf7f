"""ctypes declarations of the C ABI in include/rdfocus.h (argument marshalling only).

Every function here has the name of the C entry point it calls.  Device buffers are passed as
torch tensors (complex64, contiguous, on the plan's device) or raw integer addresses; the stream
defaults to torch's current stream on the tensor's device.  There is no CPU fallback: if the
library is missing, loading fails with an error.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("RDFOCUS_LIB", os.path.join(HERE, "librdfocus.so"))

RD_OK = 0
RD_ERR_INVALID_ARG = -1
RD_ERR_UNSUPPORTED_LENGTH = -2
RD_ERR_OUT_OF_MEMORY = -3
RD_ERR_DEVICE = -4
RD_ERR_LAUNCH = -5
RD_ERR_NOT_CONFIGURED = -6
RD_WINDOW_RECT = 0
RD_WINDOW_HAMMING = 1

# every symbol the header declares
EXPORTS = ("rd_length_supported", "rd_plan_create", "rd_plan_destroy", "rd_range_compress",
           "rd_range_compress_f16",
           "rd_azimuth_focus", "rd_focus", "rd_focus_f16", "rd_azimuth_focus_f16", "rd_debug_azimuth_stages", "rd_debug_line_fft",
           "rd_backproject", "rd_corner_turn", "rd_omega_k", "rd_omega_k_f16", "rd_status_string", "rd_last_error")


class rd_params(ctypes.Structure):
    _fields_ = [
        ("Na", ctypes.c_int32),
        ("Nr", ctypes.c_int32),
        ("pulse_s", ctypes.c_double),
        ("bandwidth_hz", ctypes.c_double),
        ("fs_hz", ctypes.c_double),
        ("range_window", ctypes.c_int32),
        ("carrier_hz", ctypes.c_double),
        ("prf_hz", ctypes.c_double),
        ("velocity_mps", ctypes.c_double),
        ("range_bin0_m", ctypes.c_double),
        ("rcmc_taps", ctypes.c_int32),
        ("kaiser_beta", ctypes.c_double),
        ("flags", ctypes.c_uint32),
    ]


class rd_bp_grid(ctypes.Structure):
    _fields_ = [
        ("nx", ctypes.c_int32),
        ("ny", ctypes.c_int32),
        ("x0_m", ctypes.c_double),
        ("dx_m", ctypes.c_double),
        ("r0_m", ctypes.c_double),
        ("dr_m", ctypes.c_double),
    ]


class RdError(RuntimeError):
    def __init__(self, status: int, func: str, message: str):
        super().__init__(f"{func} failed with status {status}: {message}")
        self.status = status


_lib = None


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load librdfocus.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"{p} not found: build it first (python -m range_doppler_focusing_amd.build)")
    lib = ctypes.CDLL(p)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.rd_length_supported.argtypes = [i32]
    lib.rd_length_supported.restype = ctypes.c_int
    lib.rd_plan_create.argtypes = [ctypes.POINTER(rd_params), ctypes.POINTER(vp)]
    lib.rd_plan_create.restype = ctypes.c_int
    lib.rd_plan_destroy.argtypes = [vp]
    lib.rd_plan_destroy.restype = ctypes.c_int
    for name in ("rd_range_compress", "rd_azimuth_focus", "rd_focus"):
        f = getattr(lib, name)
        f.argtypes = [vp, vp, vp, vp]
        f.restype = ctypes.c_int
    lib.rd_range_compress_f16.argtypes = [vp, vp, vp, vp]
    lib.rd_range_compress_f16.restype = ctypes.c_int
    lib.rd_focus_f16.argtypes = [vp, vp, vp, vp]
    lib.rd_focus_f16.restype = ctypes.c_int
    lib.rd_azimuth_focus_f16.argtypes = [vp, vp, vp, vp]
    lib.rd_azimuth_focus_f16.restype = ctypes.c_int
    lib.rd_omega_k_f16.argtypes = [vp, vp, vp, ctypes.c_int32, vp]
    lib.rd_omega_k_f16.restype = ctypes.c_int
    lib.rd_debug_azimuth_stages.argtypes = [vp, vp, vp, vp, vp, vp]
    lib.rd_debug_azimuth_stages.restype = ctypes.c_int
    lib.rd_debug_line_fft.argtypes = [vp, i32, i32, vp, vp, i64, vp]
    lib.rd_debug_line_fft.restype = ctypes.c_int
    lib.rd_backproject.argtypes = [vp, vp, vp, ctypes.POINTER(rd_bp_grid), vp]
    lib.rd_backproject.restype = ctypes.c_int
    lib.rd_omega_k.argtypes = [vp, vp, vp, i32, vp]
    lib.rd_omega_k.restype = ctypes.c_int
    lib.rd_corner_turn.argtypes = [vp, vp, i64, i64, vp]
    lib.rd_corner_turn.restype = ctypes.c_int
    lib.rd_status_string.argtypes = [ctypes.c_int]
    lib.rd_status_string.restype = ctypes.c_char_p
    lib.rd_last_error.argtypes = []
    lib.rd_last_error.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def _check(status: int, func: str) -> int:
    if status != RD_OK:
        msg = load_library().rd_last_error().decode(errors="replace")
        raise RdError(status, func, msg)
    return status


def _addr(x) -> int:
    """Device address of a tensor (complex64, contiguous) or an integer address."""
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    if not x.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return x.data_ptr()


def _addr_half(x) -> int:
    """Device address of a binary16 tensor [..., 2] (real, imaginary last) or an integer address."""
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    import torch
    if x.dtype != torch.float16 or x.shape[-1] != 2 or not x.is_contiguous():
        raise ValueError("binary16 data must be a contiguous float16 tensor with a last dimension of 2")
    return x.data_ptr()


def _stream(stream, *tensors) -> int:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    for t in tensors:
        if hasattr(t, "device") and t.device.type == "cuda":
            return torch.cuda.current_stream(t.device).cuda_stream
    return torch.cuda.current_stream().cuda_stream


def make_params(**kw) -> rd_params:
    p = rd_params()
    p.rcmc_taps = 8
    p.kaiser_beta = 2.5
    for k, v in kw.items():
        if not hasattr(p, k):
            raise TypeError(f"unknown rd_params field {k!r}")
        setattr(p, k, v)
    return p


# ------------------------------------------------------------------ entry points, same names
def rd_length_supported(n: int) -> bool:
    return bool(load_library().rd_length_supported(int(n)))


def rd_plan_create(params: rd_params | dict) -> int:
    if isinstance(params, dict):
        params = make_params(**params)
    h = ctypes.c_void_p()
    _check(load_library().rd_plan_create(ctypes.byref(params), ctypes.byref(h)), "rd_plan_create")
    return h.value


def rd_plan_destroy(plan: int) -> None:
    _check(load_library().rd_plan_destroy(plan), "rd_plan_destroy")


def rd_range_compress(plan: int, echo, rc, stream=None) -> None:
    _check(load_library().rd_range_compress(plan, _addr(echo), _addr(rc), _stream(stream, echo, rc)),
           "rd_range_compress")


def rd_range_compress_f16(plan: int, echo, rc, stream=None) -> None:
    _check(load_library().rd_range_compress_f16(plan, _addr_half(echo), _addr_half(rc), _stream(stream, echo, rc)),
           "rd_range_compress_f16")


def rd_azimuth_focus(plan: int, rc, img, stream=None) -> None:
    _check(load_library().rd_azimuth_focus(plan, _addr(rc), _addr(img), _stream(stream, rc, img)),
           "rd_azimuth_focus")


def rd_focus(plan: int, echo, img, stream=None) -> None:
    _check(load_library().rd_focus(plan, _addr(echo), _addr(img), _stream(stream, echo, img)),
           "rd_focus")


def rd_focus_f16(plan: int, echo, img, stream=None) -> None:
    _check(load_library().rd_focus_f16(plan, _addr_half(echo), _addr_half(img), _stream(stream, echo, img)),
           "rd_focus_f16")


def rd_azimuth_focus_f16(plan: int, rc, img, stream=None) -> None:
    _check(load_library().rd_azimuth_focus_f16(plan, _addr_half(rc), _addr_half(img), _stream(stream, rc, img)),
           "rd_azimuth_focus_f16")


def rd_omega_k_f16(plan: int, echo, img, ref_bin: int, stream=None) -> None:
    _check(load_library().rd_omega_k_f16(plan, _addr_half(echo), _addr_half(img), int(ref_bin),
                                         _stream(stream, echo, img)), "rd_omega_k_f16")


def rd_debug_azimuth_stages(plan: int, rc, azfft, rcmc, img, stream=None) -> None:
    _check(load_library().rd_debug_azimuth_stages(plan, _addr(rc), _addr(azfft), _addr(rcmc),
                                                  _addr(img), _stream(stream, rc, img)),
           "rd_debug_azimuth_stages")


def rd_debug_line_fft(plan: int, axis: int, inverse: int, x, y, lines: int, stream=None) -> None:
    _check(load_library().rd_debug_line_fft(plan, int(axis), int(inverse), _addr(x), _addr(y),
                                            int(lines), _stream(stream, x, y)),
           "rd_debug_line_fft")


def make_bp_grid(**kw) -> rd_bp_grid:
    g = rd_bp_grid()
    for k, v in kw.items():
        if not hasattr(g, k):
            raise TypeError(f"unknown rd_bp_grid field {k!r}")
        setattr(g, k, v)
    return g


def rd_backproject(plan: int, rc, img, grid, stream=None) -> None:
    if isinstance(grid, dict):
        grid = make_bp_grid(**grid)
    _check(load_library().rd_backproject(plan, _addr(rc), _addr(img), ctypes.byref(grid) if grid is not None else None,
                                         _stream(stream, rc, img)),
           "rd_backproject")


def rd_omega_k(plan: int, echo, img, ref_bin: int, stream=None) -> None:
    _check(load_library().rd_omega_k(plan, _addr(echo), _addr(img), int(ref_bin), _stream(stream, echo, img)),
           "rd_omega_k")


def rd_corner_turn(x, y, rows: int, cols: int, stream=None) -> None:
    _check(load_library().rd_corner_turn(_addr(x), _addr(y), int(rows), int(cols), _stream(stream, x, y)),
           "rd_corner_turn")


def rd_status_string(status: int) -> str:
    return load_library().rd_status_string(int(status)).decode()


def rd_last_error() -> str:
    return load_library().rd_last_error().decode(errors="replace")

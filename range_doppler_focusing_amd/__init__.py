"""Range-Doppler SAR focusing on AMD MI355X (gfx950): Python binding of librdfocus.so.

The compute path is the HIP library; this package only marshals arguments.  ``Plan`` wraps a
plan handle and allocates outputs with torch (device memory and the current stream).  Functions
with the C names (``rd_plan_create``, ``rd_range_compress``, ...) are re-exported from
``_native``.
"""
from __future__ import annotations

from ._native import (EXPORTS, RD_WINDOW_HAMMING, RD_WINDOW_RECT, RdError, load_library,  # noqa: F401
                      make_bp_grid, make_params, rd_azimuth_focus, rd_azimuth_focus_f16,
                      rd_backproject, rd_bp_grid, rd_corner_turn, rd_debug_azimuth_stages,
                      rd_debug_line_fft, rd_debug_rcmc, rd_focus, rd_focus_f16, rd_focus_noalloc, rd_last_error, rd_length_supported,
                      rd_omega_k, rd_omega_k_f16, rd_params, rd_plan_create, rd_plan_destroy,
                      rd_range_compress, rd_range_compress_f16, rd_status_string)


class Plan:
    """A focusing plan on the current HIP device (see include/rdfocus.h)."""

    def __init__(self, **params):
        import torch
        if not torch.cuda.is_available():
            raise RuntimeError("a HIP device is required (torch.cuda.is_available() is False)")
        self.params = dict(params)
        self.Na = int(params["Na"])
        self.Nr = int(params["Nr"])
        self.device = torch.device("cuda", torch.cuda.current_device())
        self.handle = rd_plan_create(make_params(**params))

    def close(self):
        if getattr(self, "handle", None):
            rd_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def _check(self, x, shape=None):
        import torch
        if x.dtype != torch.complex64 or x.device != self.device or not x.is_contiguous():
            raise ValueError(f"expected a contiguous complex64 tensor on {self.device}")
        if shape is not None and tuple(x.shape) != tuple(shape):
            raise ValueError(f"expected shape {shape}, got {tuple(x.shape)}")
        return x

    def _empty(self, shape):
        import torch
        return torch.empty(shape, dtype=torch.complex64, device=self.device)

    def range_compress(self, echo, out=None):
        self._check(echo, (self.Na, self.Nr))
        out = self._empty((self.Na, self.Nr)) if out is None else self._check(out, (self.Na, self.Nr))
        rd_range_compress(self.handle, echo, out)
        return out

    def azimuth_focus(self, rc, out=None):
        self._check(rc, (self.Na, self.Nr))
        out = self._empty((self.Na, self.Nr)) if out is None else self._check(out, (self.Na, self.Nr))
        rd_azimuth_focus(self.handle, rc, out)
        return out

    def focus(self, echo, out=None):
        self._check(echo, (self.Na, self.Nr))
        out = self._empty((self.Na, self.Nr)) if out is None else self._check(out, (self.Na, self.Nr))
        rd_focus(self.handle, echo, out)
        return out

    def azimuth_stages(self, rc):
        """(azfft, rcmc, img), each [Na][Nr]: azimuth spectrum and RCMC output with row k the
        Doppler bin in FFT order, and the focused image."""
        self._check(rc, (self.Na, self.Nr))
        az = self._empty((self.Na, self.Nr))
        rcmc = self._empty((self.Na, self.Nr))
        img = self._empty((self.Na, self.Nr))
        rd_debug_azimuth_stages(self.handle, rc, az, rcmc, img)
        return az, rcmc, img

    def rcmc_stage(self, x, filter: bool = True, out=None):
        """The chain's row stage alone on x [Na][Nr] with row k = Doppler bin k (FFT order): RCMC,
        and the azimuth filter with 1/Na if `filter` (rd_debug_rcmc); out may be x (in place)."""
        self._check(x, (self.Na, self.Nr))
        out = self._empty((self.Na, self.Nr)) if out is None else self._check(out, (self.Na, self.Nr))
        rd_debug_rcmc(self.handle, x, out, int(filter))
        return out

    def _half_pair(self, x, out):
        import torch
        shape = (self.Na, self.Nr, 2)
        if tuple(x.shape) != shape:
            raise ValueError(f"input must have shape {shape}")
        if out is None:
            out = torch.empty(shape, dtype=torch.float16, device=x.device)
        elif tuple(out.shape) != shape:
            raise ValueError(f"out must have shape {shape}")
        return out

    def range_compress_f16(self, echo, out=None):
        """Range compression with binary16 storage: echo and the result are float16 tensors
        [Na][Nr][2] (real, imaginary), float32 arithmetic inside (rd_range_compress_f16)."""
        out = self._half_pair(echo, out)
        rd_range_compress_f16(self.handle, echo, out)
        return out

    def azimuth_focus_f16(self, rc, out=None):
        """Azimuth half of focus_f16 on binary16 range-compressed data (rd_azimuth_focus_f16)."""
        out = self._half_pair(rc, out)
        rd_azimuth_focus_f16(self.handle, rc, out)
        return out

    def focus_f16(self, echo, out=None):
        """Focusing with binary16 storage of echo, intermediates and image (float16 tensors
        [Na][Nr][2]); the image is rd_focus's image divided by Na (rd_focus_f16)."""
        out = self._half_pair(echo, out)
        rd_focus_f16(self.handle, echo, out)
        return out

    def omega_k(self, echo, ref_bin: int, out=None):
        """omega-k image [Na][Nr] of the raw echo with reference range R(ref_bin) (rd_omega_k)."""
        self._check(echo, (self.Na, self.Nr))
        out = self._empty((self.Na, self.Nr)) if out is None else self._check(out, (self.Na, self.Nr))
        rd_omega_k(self.handle, echo, out, ref_bin)
        return out

    def omega_k_f16(self, echo, ref_bin: int, out=None):
        """omega-k with binary16 storage (float16 tensors [Na][Nr][2]); the image is rd_omega_k's
        divided by Na (rd_omega_k_f16)."""
        out = self._half_pair(echo, out)
        rd_omega_k_f16(self.handle, echo, out, ref_bin)
        return out

    def backproject(self, rc, grid: dict, out=None):
        """Back-projection image [nx][ny] of range-compressed data rc [Na][Nr] (rd_backproject)."""
        self._check(rc, (self.Na, self.Nr))
        shape = (int(grid["nx"]), int(grid["ny"]))
        out = self._empty(shape) if out is None else self._check(out, shape)
        rd_backproject(self.handle, rc, out, grid)
        return out

    def line_fft(self, x, axis: int, inverse: bool = False, out=None):
        n = self.Na if axis == 0 else self.Nr
        self._check(x)
        if x.shape[-1] != n:
            raise ValueError(f"last dimension must be {n}")
        lines = x.numel() // n
        out = self._empty(tuple(x.shape)) if out is None else self._check(out, tuple(x.shape))
        rd_debug_line_fft(self.handle, axis, int(inverse), x, out, lines)
        return out


def corner_turn(x, out=None):
    """out[c][r] = x[r][c] for a contiguous complex64 [rows][cols] tensor on the GPU (rd_corner_turn);
    returns the [cols][rows] result."""
    import torch
    if x.dtype != torch.complex64 or x.dim() != 2 or not x.is_contiguous() or x.device.type != "cuda":
        raise ValueError("expected a contiguous 2-D complex64 tensor on the GPU")
    rows, cols = x.shape
    if out is None:
        out = torch.empty((cols, rows), dtype=torch.complex64, device=x.device)
    elif out.dtype != torch.complex64 or tuple(out.shape) != (cols, rows) or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous complex64 tensor of shape {(cols, rows)}")
    rd_corner_turn(x, out, rows, cols)
    return out

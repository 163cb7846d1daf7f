"""Plain fp64 CPU oracle of the Range-Doppler (RD) focusing chain.

TEST INFRASTRUCTURE ONLY.  This module is the parity reference for the HIP library.  Only the
test suite, the package's smoke check and the benchmark's CPU-baseline leg may import it; the
library itself never calls it and shares no code, table or constant generator with it.

Every function is the textbook definition of its step, written for a reader to check by eye:
no blocking, fusion or reordering beyond what the definition states.  SciPy's FFT is used as a
library primitive, with as many worker threads as the process may use (``workers()``); a
transform's value does not depend on the thread count beyond rounding.  All arithmetic is
float64 / complex128; the raw echo is upcast on entry.

Page references (the source pages, by site and section):
  [SAR-GPU]  nxmr.cn/news/101525 -- "ultra-high-resolution airborne SAR imaging on GPU"
  [M1-RD]    cf-1.com/news/2323550 -- "SAR imaging acceleration on Apple Silicon"
  [BP-GPU]   framerc.cn/news/4459478 -- "GPU back-projection SAR imaging"

Readings of points the pages leave open (sign conventions, replica placement, window, RCMC
model, azimuth filter form) are stated at each function.
"""
from __future__ import annotations

import math
import os

import numpy as np
import scipy.fft
from scipy.special import i0 as bessel_i0

C_LIGHT = 299_792_458.0


def workers() -> int:
    """Threads the FFTs may use: the CPUs this process may run on, capped by OMP_NUM_THREADS
    where that is set (a machine's share of cores can be smaller than its CPU count)."""
    n = len(os.sched_getaffinity(0))
    try:
        cap = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        cap = 0
    return max(1, min(n, cap) if cap > 0 else n)


def fft(x, axis=-1):
    """Forward DFT X[k] = sum_n x[n] e^{-j 2 pi k n / N} along `axis` (unnormalised)."""
    return scipy.fft.fft(x, axis=axis, workers=workers())


def ifft(x, axis=-1):
    """Inverse DFT x[n] = (1/N) sum_k X[k] e^{+j 2 pi k n / N} along `axis`."""
    return scipy.fft.ifft(x, axis=axis, workers=workers())


# ----------------------------------------------------------------------------------------------
# Parameters: the same fields as the library's parameter block.
# ----------------------------------------------------------------------------------------------
def _p(params, name):
    return params[name] if isinstance(params, dict) else getattr(params, name)


def range_spacing(params) -> float:
    """Slant-range spacing of one range sample, dr = c / (2 Fs)."""
    return C_LIGHT / (2.0 * _p(params, "fs_hz"))


def replica_length(params) -> int:
    """L = ceil(Tp * Fs) samples in the transmitted pulse (tolerant to binary rounding)."""
    return int(math.ceil(_p(params, "pulse_s") * _p(params, "fs_hz") - 1e-6))


def wavelength(params) -> float:
    return C_LIGHT / _p(params, "carrier_hz")


# ----------------------------------------------------------------------------------------------
# Range compression.  [SAR-GPU] §2.1 states the CPU form y = ifft(fft(x) * fft(h)) per line with a
# precomputed chirp spectrum; [M1-RD] §2.1 / §3.1: FFT per line, multiply by the precomputed
# matched filter, IFFT.  Reading: the matched filter is the conjugate spectrum of the replica
# (correlation with the transmitted pulse), replica at indices [0, L) of the Nr buffer, forward
# transform e^{-j...} unnormalised, inverse with 1/N (NumPy convention).
# ----------------------------------------------------------------------------------------------
def replica_window(L: int, kind: int) -> np.ndarray:
    """0 = rectangular, 1 = symmetric Hamming 0.54 - 0.46 cos(2 pi n / (L-1)); a one-sample
    Hamming window (where the formula is 0/0) is [1], the usual convention.

    [BP-GPU] §3.1: an unweighted matched filter has about -13 dB sidelobes; Hamming lowers them
    at the cost of a 1.3-1.5x wider mainlobe.  The window is applied to the replica."""
    n = np.arange(L, dtype=np.float64)
    if kind == 0 or (kind == 1 and L == 1):
        return np.ones(L)
    if kind == 1:
        return 0.54 - 0.46 * np.cos(2.0 * np.pi * n / (L - 1))
    raise ValueError(f"unknown window {kind}")


def chirp_replica(params) -> np.ndarray:
    """h[n] = w[n] * exp(j pi Kr (n/Fs - Tp/2)^2), n < L; up-chirp Kr = B / Tp."""
    Tp, B, Fs = _p(params, "pulse_s"), _p(params, "bandwidth_hz"), _p(params, "fs_hz")
    L = replica_length(params)
    t = np.arange(L, dtype=np.float64) / Fs
    return replica_window(L, _p(params, "range_window")) * np.exp(1j * np.pi * (B / Tp) * (t - Tp / 2) ** 2)


def matched_filter(params) -> np.ndarray:
    """H[k] = conj(FFT_Nr(h zero-padded to Nr))."""
    Nr = _p(params, "Nr")
    h = np.zeros(Nr, np.complex128)
    rep = chirp_replica(params)
    if rep.size > Nr:
        raise ValueError("replica longer than the range line")
    h[:rep.size] = rep
    return np.conj(fft(h))


def range_compress(echo: np.ndarray, params) -> np.ndarray:
    """rc[m] = IFFT(FFT(echo[m]) * H) for every line m (circular correlation with the replica)."""
    H = matched_filter(params)
    x = np.asarray(echo, dtype=np.complex128)
    return ifft(fft(x, axis=1) * H[None, :], axis=1)


# ----------------------------------------------------------------------------------------------
# Azimuth processing.  [M1-RD] §2.1 / §5.1: azimuth FFT, range cell migration correction (RCMC)
# by sinc interpolation, multiply by the azimuth matched filter, azimuth IFFT.  [SAR-GPU] §2.2:
# RCMC looks up each output at the migrated slant range of a hyperbolic history and interpolates.
# ----------------------------------------------------------------------------------------------
def corner_turn(x: np.ndarray) -> np.ndarray:
    """[M1-RD] §5.1-§5.2 and [SAR-GPU] §2.2.1: the corner turn between range lines and azimuth
    lines, out[c][r] = x[r][c] for a [rows][cols] array (a plain transpose, returned
    contiguous).  A data move: exact, no arithmetic."""
    return np.ascontiguousarray(np.asarray(x).T)


def azimuth_fft(rc: np.ndarray) -> np.ndarray:
    """S[k][n] = sum_m rc[m][n] e^{-j 2 pi k m / Na}: forward DFT down every range bin."""
    return fft(rc, axis=0)


def doppler_freqs(params) -> np.ndarray:
    """Doppler of azimuth bin k: NumPy fftfreq order (zero squint, centroid 0)."""
    return np.fft.fftfreq(_p(params, "Na"), 1.0 / _p(params, "prf_hz"))


def migration_factor(params) -> np.ndarray:
    """D_k = sqrt(1 - (lambda f_k / (2 V))^2), the cosine of the squint angle seen at Doppler f_k."""
    u = (wavelength(params) * doppler_freqs(params) / (2.0 * _p(params, "velocity_mps"))) ** 2
    if np.any(u >= 1.0):
        raise ValueError("Doppler band exceeds the velocity-limited maximum")
    return np.sqrt(1.0 - u)


def bin_range(params, n) -> np.ndarray:
    """R(n) = range_bin0 + n dr: slant range of range bin n (leading-edge convention)."""
    return _p(params, "range_bin0_m") + np.asarray(n, dtype=np.float64) * range_spacing(params)


def rcmc_shift(params, n, k=None) -> np.ndarray:
    """Delta[k][i] = R(n_i) (1/D_k - 1) / dr  (samples), for range bins n and Doppler bins k
    (all of them by default).

    A target at closest range R0 appears at range R0 / D_k in Doppler bin k, so output bin n
    reads the input at x = n + Delta.  Evaluated as R u / (D (1 + D)) / dr, which equals
    R (1/D - 1) / dr without the cancellation of 1/D - 1 near D = 1."""
    D = migration_factor(params)
    D = D if k is None else D[np.asarray(k)]
    u = 1.0 - D * D
    q = u / (D * (1.0 + D))
    return bin_range(params, n)[None, :] * q[:, None] / range_spacing(params)


def kaiser_sinc(t: np.ndarray, taps: int, beta: float) -> np.ndarray:
    """Kaiser-windowed sinc kernel value at offset t (|t| <= taps/2), before normalisation:
    sinc(t) * I0(beta sqrt(1 - (t / (taps/2))^2)) / I0(beta)."""
    half = taps / 2.0
    arg = np.clip(1.0 - (t / half) ** 2, 0.0, None)
    return np.sinc(t) * bessel_i0(beta * np.sqrt(arg)) / bessel_i0(beta)


def rcmc(S: np.ndarray, shift: np.ndarray, taps: int = 8, beta: float = 2.5,
         out_bins=None, in_bins=None, Nr: int | None = None) -> np.ndarray:
    """RCMC by interpolation along range in the range-Doppler domain.

    out[k][i] = sum_{j=-(taps/2-1)}^{taps/2} w_j S[k][floor(x) + j],  x = n_i + shift[k][i],
    w_j = kaiser_sinc(x - floor(x) - j) / (sum of the taps weights); samples outside [0, Nr)
    are zero.

    By default S holds every range bin and every bin is an output.  For sampled evaluation,
    column c of S holds global range bin in_bins[c] (sorted) and out_bins lists the global
    range bins to produce; a needed bin missing from in_bins is an error."""
    Na, W = S.shape
    Nr = W if Nr is None else Nr
    out_bins = np.arange(Nr) if out_bins is None else np.asarray(out_bins)
    column_of = np.full(Nr, -1, np.int64)          # global range bin -> column of S
    column_of[np.arange(W) if in_bins is None else np.asarray(in_bins)] = np.arange(W)
    x = out_bins[None, :].astype(np.float64) + shift
    i0 = np.floor(x).astype(np.int64)
    frac = x - i0
    half = taps // 2
    acc = np.zeros(x.shape, np.complex128)
    wsum = np.zeros(x.shape, np.float64)
    for j in range(-(half - 1), half + 1):
        idx = i0 + j
        w = kaiser_sinc(frac - j, taps, beta)
        wsum += w
        inside = (idx >= 0) & (idx < Nr)
        col = column_of[np.clip(idx, 0, Nr - 1)]
        if np.any(inside & (col < 0)):
            raise ValueError("RCMC input columns do not cover a needed range bin")
        vals = np.take_along_axis(S, np.maximum(col, 0), axis=1)
        acc += np.where(inside, w, 0.0) * vals
    return acc / wsum


def azimuth_matched_filter(params, n, k=None) -> np.ndarray:
    """Haz[k][i] = exp(+j 4 pi R(n_i) D_k / lambda) for range bins n and Doppler bins k (all of
    them by default).

    After RCMC a target at R0 carries the range-Doppler phase exp(-j 4 pi R0 D_k / lambda)
    (stationary phase of the hyperbolic history); the filter removes it.  Phase-only,
    range-dependent, unwindowed."""
    D = migration_factor(params)
    D = D if k is None else D[np.asarray(k)]
    phase = 4.0 * np.pi * bin_range(params, n)[None, :] * D[:, None] / wavelength(params)
    return np.exp(1j * phase)


def azimuth_ifft(Z: np.ndarray) -> np.ndarray:
    """img[m][n] = (1/Na) sum_k Z[k][n] e^{+j 2 pi k m / Na}."""
    return ifft(Z, axis=0)


# ----------------------------------------------------------------------------------------------
# Whole chain.
# ----------------------------------------------------------------------------------------------
def focus_stages(echo: np.ndarray, params) -> dict:
    """Every intermediate of the chain, [Na][Nr] layout (rows = pulses or Doppler bins)."""
    Nr = _p(params, "Nr")
    n = np.arange(Nr)
    rc = range_compress(echo, params)
    S = azimuth_fft(rc)
    R = rcmc(S, rcmc_shift(params, n), _p(params, "rcmc_taps"), _p(params, "kaiser_beta"))
    Z = R * azimuth_matched_filter(params, n)
    img = azimuth_ifft(Z)
    return {"rc": rc, "azfft": S, "rcmc": R, "img": img}


def focus(echo: np.ndarray, params) -> np.ndarray:
    """Focused complex image [Na][Nr]."""
    return focus_stages(echo, params)["img"]


def azimuth_focus(rc: np.ndarray, params) -> np.ndarray:
    """The chain's azimuth half on range-compressed data rc [Na][Nr]: the same steps as
    focus_stages after its range compression."""
    n = np.arange(_p(params, "Nr"))
    S = azimuth_fft(rc)
    R = rcmc(S, rcmc_shift(params, n), _p(params, "rcmc_taps"), _p(params, "kaiser_beta"))
    return azimuth_ifft(R * azimuth_matched_filter(params, n))


def focus_columns(echo: np.ndarray, params, out_bins, block_rows: int = 1024, stages: bool = False):
    """Image columns img[:, out_bins] from the same definitions, for scenes too large to focus
    whole.  Range compression runs line by line and keeps only the range bins that the RCMC of
    the requested outputs reads; azimuth FFT, RCMC, filter and IFFT then run on those columns.
    Returns (columns [Na][len(bins)], bins) with bins = sorted unique out_bins; with stages,
    (dict of the rc, azfft, rcmc and img columns at those bins, bins) instead."""
    Na, Nr = _p(params, "Na"), _p(params, "Nr")
    taps = _p(params, "rcmc_taps")
    out_bins = np.asarray(sorted(set(int(b) for b in out_bins)))
    shift = rcmc_shift(params, out_bins)
    reach = int(np.ceil(shift.max())) + 1
    need = set()
    for n in out_bins:
        need.update(range(max(0, n - taps // 2), min(Nr, n + taps // 2 + reach + 1)))
    in_bins = np.asarray(sorted(need))
    rc_cols = np.empty((Na, in_bins.size), np.complex128)
    for m0 in range(0, Na, block_rows):
        blk = range_compress(echo[m0:m0 + block_rows], params)
        rc_cols[m0:m0 + block_rows] = blk[:, in_bins]
    S = azimuth_fft(rc_cols)
    R = rcmc(S, shift, taps, _p(params, "kaiser_beta"), out_bins=out_bins, in_bins=in_bins, Nr=Nr)
    img = azimuth_ifft(R * azimuth_matched_filter(params, out_bins))
    if not stages:
        return img, out_bins
    at = np.searchsorted(in_bins, out_bins)     # every output bin is among the input bins
    return {"rc": rc_cols[:, at], "azfft": S[:, at], "rcmc": R, "img": img}, out_bins


# ----------------------------------------------------------------------------------------------
# Back-projection: [BP-GPU] §1.1 (principle), §1.2 (cost), §2.2 (per-pixel range history, linear
# interpolation on the range axis, phase compensation, coherent accumulation), §4.2 (carrier
# wavelength in the phase).
# Readings (the page works with 3-D platform positions and leaves the grid to the user): the
# geometry is the slant plane of the focusing scenes -- a straight track along x with the
# platform at x_m = V m / PRF at pulse m, a pixel at along-track position x and closest-approach
# slant range r, so its range at pulse m is d = sqrt(r^2 + (x - x_m)^2); every pulse is summed
# (the page visits all pulses); samples outside the range line count as zero; no normalisation.
# ----------------------------------------------------------------------------------------------
def bp_grid_axes(grid):
    """Pixel coordinates of a back-projection grid: along-track positions x[i] = x0 + i dx
    (i < nx) and closest-approach slant ranges r[j] = r0 + j dr (j < ny)."""
    nx, ny = int(_p(grid, "nx")), int(_p(grid, "ny"))
    x = _p(grid, "x0_m") + _p(grid, "dx_m") * np.arange(nx, dtype=np.float64)
    r = _p(grid, "r0_m") + _p(grid, "dr_m") * np.arange(ny, dtype=np.float64)
    return x, r


def range_line_sample(line: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Linear interpolation of one range-compressed line at fractional bins b ([BP-GPU] §2.2);
    bins outside [0, Nr) contribute zero."""
    Nr = line.shape[0]
    i0 = np.floor(b).astype(np.int64)
    w = b - i0
    def at(i):
        ok = (i >= 0) & (i < Nr)
        out = np.zeros(i.shape, np.complex128)
        out[ok] = line[i[ok]]
        return out
    return (1.0 - w) * at(i0) + w * at(i0 + 1)


def backproject(rc: np.ndarray, params, grid) -> np.ndarray:
    """Back-projection image img[i][j] = sum_m s_m(d_m) exp(+j 4 pi d_m / lambda) with
    d_m = sqrt(r_j^2 + (x_i - V m / PRF)^2) and s_m the linear interpolation of range line m at
    bin (d_m - range_bin0) / dr ([BP-GPU] §1.1, §2.2, §4.2).  rc is [Na][Nr]; img is [nx][ny]."""
    rc = np.asarray(rc, dtype=np.complex128)
    Na = rc.shape[0]
    V, prf = _p(params, "velocity_mps"), _p(params, "prf_hz")
    lam, rb0, dr = wavelength(params), _p(params, "range_bin0_m"), range_spacing(params)
    x, r = bp_grid_axes(grid)
    img = np.zeros((x.size, r.size), np.complex128)
    for m in range(Na):
        d = np.sqrt(r[None, :] ** 2 + (x[:, None] - V * m / prf) ** 2)
        img += range_line_sample(rc[m], (d - rb0) / dr) * np.exp(4j * math.pi * d / lam)
    return img


def backproject_pixels(rc: np.ndarray, params, grid, pix) -> np.ndarray:
    """backproject() at selected pixels only: pix is a list of (i, j); returns their values."""
    x, r = bp_grid_axes(grid)
    sub = {"nx": 1, "ny": 1, "dx_m": 0.0, "dr_m": 0.0}
    out = np.empty(len(pix), np.complex128)
    for k, (i, j) in enumerate(pix):
        out[k] = backproject(rc, params, dict(sub, x0_m=x[i], r0_m=r[j]))[0, 0]
    return out


# ----------------------------------------------------------------------------------------------
# omega-k (wavenumber-domain) focusing: [SAR-GPU] §3 (Stolt interpolation makes the migration
# correction a frequency-domain operation; forward range and azimuth transforms, the inverse
# transforms, and two large complex multiplies), §3.2 (a phase compensation built from the range
# and Doppler frequencies), §3.3 (the Doppler band sets the extent of the mapping).
# Readings (the page gives the steps without their formulas; these are the zero-squint
# textbook forms in the notation of this module):
#   * the input is the raw echo; the range matched filter H is one of the two multiplies, the
#     reference function the other, both on the 2-D spectrum;
#   * reference range Rref = R(ref_bin) for an integer range bin, so that the two linear phase
#     terms below are exact roots of unity;
#   * the Stolt interpolator is the RCMC one (8-tap Kaiser-windowed sinc, normalised weights),
#     run along range frequency in natural (centred) order, zero outside the sampled band;
#   * after the mapping, exp(-j 2 pi f' 2 (Rref - range_bin0) / c) puts the image on the RD grid
#     (bin n at R(n), row m at pulse m), so the two methods can be compared pixel by pixel.
# ----------------------------------------------------------------------------------------------
def range_freqs(params) -> np.ndarray:
    """Baseband range frequency of range-FFT bin j (NumPy fftfreq order), Hz."""
    return np.fft.fftfreq(_p(params, "Nr"), 1.0 / _p(params, "fs_hz"))


def doppler_wavenumber_sq(params) -> np.ndarray:
    """b_k^2 = (c f_k / (2 V))^2 per Doppler bin k (Hz^2): the azimuth part of the 2-D
    wavenumber, written as a frequency."""
    return (C_LIGHT * doppler_freqs(params) / (2.0 * _p(params, "velocity_mps"))) ** 2


def reference_function(params, ref_bin: int) -> np.ndarray:
    """RFM[k][j] = exp(+j 2 pi [ (2 Rref / c) Q(f_j, f_k) - f_j tau0 ]),
    Q = sqrt((f0 + f_j)^2 - b_k^2), tau0 = 2 range_bin0 / c (the fast time of range sample 0).

    A target at closest range R0 and pulse time eta0 carries, after range compression and the
    2-D transform, the phase -2 pi [ (2 R0 / c) Q - f tau0 + f_k eta0 ] (stationary phase of
    the hyperbolic history); the RFM removes it exactly at R0 = Rref."""
    f0 = _p(params, "carrier_hz")
    f = range_freqs(params)[None, :]
    Q = np.sqrt((f0 + f) ** 2 - doppler_wavenumber_sq(params)[:, None])
    r_ref = float(bin_range(params, ref_bin))
    tau0 = 2.0 * _p(params, "range_bin0_m") / C_LIGHT
    return np.exp(2j * np.pi * ((2.0 * r_ref / C_LIGHT) * Q - f * tau0))


def stolt_shift(params) -> np.ndarray:
    """delta[k][u] (range-frequency bins) for output bin u in natural order
    (f'_u = (u - Nr/2) Fs / Nr): the Stolt mapping reads the input at the frequency f with
    Q(f, f_k) = f0 + f', i.e. f = sqrt((f0 + f')^2 + b_k^2) - f0, so the source lies
    delta = (sqrt((f0 + f')^2 + b_k^2) - (f0 + f')) Nr / Fs bins above the output."""
    Nr, fs, f0 = _p(params, "Nr"), _p(params, "fs_hz"), _p(params, "carrier_hz")
    fp = (np.arange(Nr) - Nr // 2) * (fs / Nr)
    a = f0 + fp[None, :]
    return (np.sqrt(a * a + doppler_wavenumber_sq(params)[:, None]) - a) * (Nr / fs)


def omega_k_stages(echo: np.ndarray, params, ref_bin: int) -> dict:
    """Every intermediate of omega-k focusing, [Na][Nr] (rows = pulses or Doppler bins).

    spec  : S[k][j] = 2-D DFT of the echo (range then azimuth), range bins in FFT order
    rfm   : S H[j] RFM[k][j]                       (the two multiplies)
    stolt : interpolated at f' in natural order, times exp(-j 2 pi f' 2 (Rref - range_bin0)/c),
            returned in FFT order
    img   : inverse 2-D DFT (1/(Na Nr))"""
    Nr = _p(params, "Nr")
    x = np.asarray(echo, dtype=np.complex128)
    spec = fft(fft(x, axis=1), axis=0)
    rfm = spec * matched_filter(params)[None, :] * reference_function(params, ref_bin)
    centred = np.fft.fftshift(rfm, axes=1)
    T = rcmc(centred, stolt_shift(params), _p(params, "rcmc_taps"), _p(params, "kaiser_beta"))
    fp = (np.arange(Nr) - Nr // 2) * (_p(params, "fs_hz") / Nr)
    shift_m = float(bin_range(params, ref_bin)) - _p(params, "range_bin0_m")
    T = T * np.exp(-2j * np.pi * fp * (2.0 * shift_m / C_LIGHT))[None, :]
    stolt = np.fft.ifftshift(T, axes=1)
    img = ifft(ifft(stolt, axis=1), axis=0)
    return {"spec": spec, "rfm": rfm, "stolt": stolt, "img": img}


def omega_k(echo: np.ndarray, params, ref_bin: int) -> np.ndarray:
    """Focused complex image [Na][Nr] by omega-k with Stolt interpolation."""
    return omega_k_stages(echo, params, ref_bin)["img"]

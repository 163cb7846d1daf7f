"""Image-quality and parity metrics (TEST INFRASTRUCTURE ONLY, like the rest of ``oracle``).

The same routines run on the HIP path's images and on the oracle's, so a difference in a
metric is a difference in the images.

Point-target analysis: a 1-D cut through the peak (along range or along azimuth), a window of
``half`` samples either side taken circularly, FFT-upsampled by ``up``; the mainlobe spans the
first nulls (first local minima of the power either side of the peak).  The cut is first
shifted to baseband (see ``demodulate``).
  PSLR = highest sidelobe power / peak power, in dB;
  ISLR = sidelobe energy / mainlobe energy inside the window, in dB;
  IRW  = width of the mainlobe at half power (-3 dB), in original samples, with the crossings
         interpolated linearly on the upsampled grid.
[BP-GPU] (framerc.cn/news/4459478) §4.2 checks a focus by comparing the point response with
the theoretical impulse response; §3.1 gives about -13 dB sidelobes for an unweighted filter.
"""
from __future__ import annotations

import numpy as np


def rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    """||a - b||_2 / ||b||_2, accumulated in float64 (b is the reference)."""
    a = np.asarray(a, dtype=np.complex128)
    b = np.asarray(b, dtype=np.complex128)
    den = np.sqrt(np.sum(np.abs(b) ** 2))
    return float(np.sqrt(np.sum(np.abs(a - b) ** 2)) / den) if den > 0 else float(np.sqrt(np.sum(np.abs(a) ** 2)))


def line_errors(a: np.ndarray, b: np.ndarray, axis: int) -> np.ndarray:
    """Relative L2 error of every line of a 2-D array against the reference b: line i along
    `axis` (axis=1: rows, axis=0: columns) gives ||a_i - b_i|| / max(||b_i||, RMS(b) sqrt(len_i)),
    i.e. the line's own relative error, or its error relative to an average line where the
    line holds less than average energy.  A defect confined to a few rows or columns, which a
    whole-array norm dilutes by the square root of the line count, shows at full size here."""
    a = np.asarray(a, dtype=np.complex128)
    b = np.asarray(b, dtype=np.complex128)
    num = np.sqrt(np.sum(np.abs(a - b) ** 2, axis=axis))
    own = np.sqrt(np.sum(np.abs(b) ** 2, axis=axis))
    avg = np.sqrt(np.mean(np.abs(b) ** 2) * b.shape[axis])
    return num / np.maximum(own, avg) if avg > 0 else num


def worst_line_errors(a: np.ndarray, b: np.ndarray) -> tuple:
    """(worst row error, worst column error) of line_errors."""
    return float(line_errors(a, b, 1).max()), float(line_errors(a, b, 0).max())


def peak_near(img: np.ndarray, m: int, n: int, radius: int = 16) -> tuple:
    """(row, col) of the largest |img| within +-radius of (m, n), circular in both axes;
    ties resolve to the first in row-major order of the scanned window."""
    Na, Nr = img.shape
    rows = (m + np.arange(-radius, radius + 1)) % Na
    cols = (n + np.arange(-radius, radius + 1)) % Nr
    win = np.abs(img[np.ix_(rows, cols)])
    r, c = np.unravel_index(int(np.argmax(win)), win.shape)
    return int(rows[r]), int(cols[c])


def upsample(x: np.ndarray, up: int) -> np.ndarray:
    """Band-limited (FFT zero-padding) interpolation of a 1-D sequence by an integer factor."""
    N = x.size
    X = np.fft.fft(x)
    Y = np.zeros(N * up, np.complex128)
    h = N // 2
    if N % 2 == 0:
        Y[:h] = X[:h]
        Y[h] = X[h] / 2
        Y[-h] = X[h] / 2
        Y[-h + 1:] = X[h + 1:]
    else:
        Y[:h + 1] = X[:h + 1]
        Y[-h:] = X[h + 1:]
    return np.fft.ifft(Y) * up


def demodulate(cut: np.ndarray) -> np.ndarray:
    """Remove the cut's mean frequency (phase of its lag-1 autocorrelation) so its spectrum sits
    at baseband before band-limited upsampling.  A focused image carries a linear phase ramp
    across range bins (the azimuth filter's 4 pi R(n) / lambda term); without this step the
    spectrum of a range cut wraps and the interpolation between samples is wrong.  Magnitudes at
    the samples are unchanged."""
    cut = np.asarray(cut, np.complex128)
    step = np.angle(np.sum(cut[1:] * np.conj(cut[:-1])))
    return cut * np.exp(-1j * step * np.arange(cut.size))


def cut_metrics(cut: np.ndarray, up: int = 32) -> dict:
    """PSLR / ISLR / IRW of a 1-D point-response cut whose peak is near the middle."""
    p = np.abs(upsample(demodulate(cut), up)) ** 2
    k = int(np.argmax(p))
    left = k
    while left > 0 and p[left - 1] < p[left]:
        left -= 1
    right = k
    while right < p.size - 1 and p[right + 1] < p[right]:
        right += 1
    main = p[left:right + 1].sum()
    side = p.sum() - main
    sidelobes = np.concatenate([p[:left], p[right + 1:]])
    pslr = 10 * np.log10(sidelobes.max() / p[k]) if sidelobes.size else -np.inf
    islr = 10 * np.log10(side / main) if side > 0 else -np.inf
    half = p[k] / 2

    def cross(i_from, step):
        i = i_from
        while p[i + step] > half:
            i += step
        a, b = p[i], p[i + step]
        return i + step * (a - half) / (a - b)

    irw = (cross(k, 1) - cross(k, -1)) / up
    return {"pslr_db": float(pslr), "islr_db": float(islr), "irw": float(irw),
            "peak_pos": k / up, "peak_power": float(p[k])}


def point_target(img: np.ndarray, m: int, n: int, half: int = 32, up: int = 32,
                 axes=("range", "azimuth")) -> dict:
    """Metrics of the point response at (m, n): cuts along range (a row) and azimuth (a column)."""
    Na, Nr = img.shape
    out = {}
    if "range" in axes:
        cols = (n + np.arange(-half, half)) % Nr
        out["range"] = cut_metrics(img[m, cols], up)
    if "azimuth" in axes:
        rows = (m + np.arange(-half, half)) % Na
        out["azimuth"] = cut_metrics(img[rows, n], up)
    return out

"""Seeded synthetic raw-echo generator (point targets + circular complex Gaussian noise).

The echo model is the forward physics of a stripmap pulse radar at zero squint, not any
part of the focusing method:

* transmitted pulse g(t) = exp(j*pi*Kr*(t - Tp/2)^2) for 0 <= t < Tp, Kr = B/Tp (up-chirp);
* slant range of target t at slow time eta: R_t(eta) = sqrt(R_t0^2 + V^2 (eta - eta_t)^2),
  the hyperbolic range history of a straight, constant-velocity track;
* sample i of pulse m is taken at fast time tau_i = 2*range_bin0/c + i/Fs, so the echo of
  a target at range R starts at fractional sample (R - range_bin0)/dr;
* carrier phase exp(-j*4*pi*R_t(eta)/lambda) (two-way path at the carrier wavelength);
* the target is illuminated for |eta - eta_t| < Ta/2 with Ta = Na/(2*PRF).

Targets sit on the sample grid (R_t0 = range_bin0 + n_t*dr, eta_t = m_t/PRF), so a correct
focusing places target t at pixel (m_t, n_t).  Range-only scenes carry, in every line, a
copy of the pulse at an integer delay n_t with a seeded phase per line.

Randomness: ``numpy.random.SeedSequence(seed)`` is split into three children (target
placement, per-line phases, noise); the noise child is split again into one stream per
block of BLOCK_ROWS lines, so the echo does not depend on the number of worker threads.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

from .configs import C_LIGHT, SceneConfig

BLOCK_ROWS = 256
_TWO_PI = 2.0 * math.pi


@dataclass
class Scene:
    cfg: SceneConfig
    echo: np.ndarray            # complex64 [Na][Nr], C-contiguous
    targets: list               # [(m_t, n_t)] predicted focus pixels (range-only: m_t = -1)


def _place_targets(cfg: SceneConfig, rng: np.random.Generator) -> list:
    if cfg.full_chain:
        n_lo, n_hi = 4, 4 + cfg.usable_bins
        m_lo, m_hi = cfg.Na // 4 + 8, 3 * cfg.Na // 4 - 8
    else:
        n_lo, n_hi = 0, cfg.Nr - cfg.replica_len
        m_lo = m_hi = -1
    out = []
    for _ in range(100000):
        if len(out) == cfg.n_targets:
            break
        n = int(rng.integers(n_lo, n_hi + 1))
        m = int(rng.integers(m_lo, m_hi + 1)) if cfg.full_chain else -1
        ok = True
        for (mm, nn) in out:
            far_r = abs(nn - n) >= cfg.sep_range
            far_a = cfg.full_chain and cfg.sep_az > 0 and abs(mm - m) >= cfg.sep_az
            if not (far_r or far_a):
                ok = False
                break
        if ok:
            out.append((m, n))
    if len(out) != cfg.n_targets:
        raise RuntimeError(f"{cfg.name}: could not place {cfg.n_targets} separated targets")
    return out


def _pulse(cfg: SceneConfig, t_s: np.ndarray, extra_phase: np.ndarray) -> np.ndarray:
    """exp(j*(pi*Kr*(t - Tp/2)^2 + extra_phase)) inside 0 <= t < Tp, else 0 (complex64).

    The phase is formed in float64, reduced modulo 2*pi, then evaluated in float32."""
    Tp = cfg.pulse_s
    kr = cfg.bandwidth_hz / Tp
    tfs = t_s * cfg.fs_hz
    inside = (tfs >= -1e-6) & (tfs < Tp * cfg.fs_hz - 1e-6)
    ph = math.pi * kr * (t_s - Tp / 2.0) ** 2 + extra_phase
    ph = (ph - _TWO_PI * np.round(ph / _TWO_PI)).astype(np.float32)
    out = np.empty(ph.shape, np.complex64)
    out.real = np.cos(ph)
    out.imag = np.sin(ph)
    out[~inside] = 0
    return out


def _block_full_chain(cfg: SceneConfig, targets, m0: int, m1: int, out: np.ndarray) -> None:
    lam = cfg.wavelength
    dr = cfg.dr
    rb0 = cfg.range_bin0_m
    half = cfg.aperture_pulses // 2
    L = cfg.replica_len
    for (mt, nt) in targets:
        lo, hi = max(m0, mt - half), min(m1, mt + half)
        if lo >= hi:
            continue
        m = np.arange(lo, hi, dtype=np.float64)
        eta = (m - mt) / cfg.prf_hz
        r0 = rb0 + nt * dr
        R = np.sqrt(r0 * r0 + (cfg.velocity_mps * eta) ** 2)
        x = (R - rb0) / dr                          # fractional sample where the echo starts
        i_lo = max(0, int(math.floor(x.min())) - 1)
        i_hi = min(cfg.Nr, int(math.ceil(x.max())) + L + 2)
        i = np.arange(i_lo, i_hi, dtype=np.float64)
        t = (i[None, :] - x[:, None]) / cfg.fs_hz   # fast time relative to the echo start
        carrier = (-4.0 * math.pi / lam) * R
        carrier = carrier - _TWO_PI * np.round(carrier / _TWO_PI)
        out[lo - m0:hi - m0, i_lo:i_hi] += _pulse(cfg, t, carrier[:, None])


def _block_range_only(cfg: SceneConfig, targets, phases: np.ndarray, m0: int, m1: int,
                      out: np.ndarray) -> None:
    L = cfg.replica_len
    t = np.arange(L, dtype=np.float64) / cfg.fs_hz
    g = _pulse(cfg, t, np.zeros(L))
    for ti, (_, nt) in enumerate(targets):
        ph = phases[ti, m0:m1].astype(np.float32)
        rot = (np.cos(ph) + 1j * np.sin(ph)).astype(np.complex64)
        out[:, nt:nt + L] += rot[:, None] * g[None, :]


def _block_noise(cfg: SceneConfig, ss: np.random.SeedSequence, out: np.ndarray) -> None:
    if cfg.noise_power <= 0:
        return
    rng = np.random.default_rng(ss)
    rows = out.shape[0]
    z = rng.standard_normal((rows, cfg.Nr, 2), dtype=np.float32)
    z *= np.float32(math.sqrt(cfg.noise_power / 2.0))
    out += z.view(np.complex64)[..., 0]


def make_scene(cfg: SceneConfig, noise: bool = True, workers: int | None = None) -> Scene:
    """Generate the seeded raw echo of ``cfg`` as complex64 [Na][Nr]."""
    ss_targets, ss_phase, ss_noise = np.random.SeedSequence(cfg.seed).spawn(3)
    targets = _place_targets(cfg, np.random.default_rng(ss_targets))
    phases = None
    if not cfg.full_chain:
        phases = np.random.default_rng(ss_phase).uniform(0.0, _TWO_PI, (cfg.n_targets, cfg.Na))
    echo = np.zeros((cfg.Na, cfg.Nr), np.complex64)
    nblk = (cfg.Na + BLOCK_ROWS - 1) // BLOCK_ROWS
    noise_ss = ss_noise.spawn(nblk)

    def run(b: int) -> None:
        m0, m1 = b * BLOCK_ROWS, min(cfg.Na, (b + 1) * BLOCK_ROWS)
        view = echo[m0:m1]
        if cfg.full_chain:
            _block_full_chain(cfg, targets, m0, m1, view)
        else:
            _block_range_only(cfg, targets, phases, m0, m1, view)
        if noise:
            _block_noise(cfg, noise_ss[b], view)

    if workers is None:
        workers = min(16, len(os.sched_getaffinity(0)))
    if workers <= 1 or nblk == 1:
        for b in range(nblk):
            run(b)
    else:
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(run, range(nblk)))
    return Scene(cfg=cfg, echo=echo, targets=targets)


def cached_scene(cfg: SceneConfig, noise: bool = True, cache_dir: str | None = None) -> Scene:
    """make_scene with an on-disk cache keyed by the full configuration (regenerable)."""
    import hashlib
    import json
    cache_dir = cache_dir or os.environ.get(
        "RD_SCENE_CACHE", os.path.join(os.path.dirname(os.path.dirname(__file__)), ".scene_cache"))
    key = hashlib.sha1(repr((cfg, noise, BLOCK_ROWS, 2)).encode()).hexdigest()[:16]
    path = os.path.join(cache_dir, f"{cfg.name}_{key}")
    try:
        echo = np.load(path + ".npy", mmap_mode=None, allow_pickle=False)
        with open(path + ".json") as f:
            targets = [tuple(t) for t in json.load(f)]
        return Scene(cfg=cfg, echo=echo, targets=targets)
    except (OSError, ValueError):
        pass
    sc = make_scene(cfg, noise=noise)
    try:
        os.makedirs(cache_dir, exist_ok=True)
        np.save(path + ".npy", sc.echo, allow_pickle=False)
        with open(path + ".json", "w") as f:
            json.dump(sc.targets, f)
    except OSError:
        pass
    return sc

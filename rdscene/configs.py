"""Scene configurations: the five synthetic workloads the focusing path is tested and measured on.

This module holds acquisition geometry only (radar, platform, receive window, target and
noise recipe).  It contains none of the focusing arithmetic: no transform, no matched filter,
no interpolation.  Both the HIP path (through the library's parameter block) and the CPU
oracle read their inputs from here and from ``rdscene.simulate``.

Where the source pages leave a quantity open, the value chosen here is the plainest reading
that the rest of the pages support; every such reading is listed in the design notes.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

C_LIGHT = 299_792_458.0


@dataclass(frozen=True)
class SceneConfig:
    name: str
    Na: int                 # pulses (azimuth lines)
    Nr: int                 # range samples per line
    pulse_s: float          # Tp
    bandwidth_hz: float     # B (up-chirp, Kr = B / Tp)
    fs_hz: float            # range sampling rate
    window: str             # "rect" or "hamming" (on the replica)
    n_targets: int
    noise_power: float      # sigma^2 of the circular complex Gaussian noise per sample
    seed: int
    carrier_hz: float = 0.0     # 0 => range-only scene
    prf_hz: float = 0.0
    velocity_mps: float = 0.0
    r_ref_m: float = 0.0        # closest-approach slant range of the scene centre
    rcmc_taps: int = 8
    kaiser_beta: float = 2.5
    # minimum separation of two targets: they must differ by >= sep_range bins OR >= sep_az pulses
    sep_range: int = 64
    sep_az: int = 0

    # ---- derived acquisition quantities (geometry, not method) ----
    @property
    def full_chain(self) -> bool:
        return self.carrier_hz > 0.0

    @property
    def dr(self) -> float:
        """Slant-range spacing of one range sample."""
        return C_LIGHT / (2.0 * self.fs_hz)

    @property
    def replica_len(self) -> int:
        """Samples in the transmitted pulse: ceil(Tp * Fs), robust to binary rounding."""
        return int(math.ceil(self.pulse_s * self.fs_hz - 1e-6))

    @property
    def wavelength(self) -> float:
        return C_LIGHT / self.carrier_hz

    @property
    def aperture_pulses(self) -> int:
        """Pulses for which a target is illuminated: Ta = Na / (2 PRF)."""
        return self.Na // 2

    @property
    def rcm_max_samples(self) -> float:
        if not self.full_chain:
            return 0.0
        half = self.velocity_mps * (self.aperture_pulses / self.prf_hz) / 2.0
        return (math.hypot(self.r_ref_m, half) - self.r_ref_m) / self.dr

    @property
    def usable_bins(self) -> int:
        """Leading-edge range bins that hold a target's whole echo (plus migration)."""
        if not self.full_chain:
            return self.Nr - self.replica_len
        return self.Nr - self.replica_len - int(math.ceil(self.rcm_max_samples)) - 8

    @property
    def range_bin0_m(self) -> float:
        """Slant range of range sample 0 (the receive window opens at 2*range_bin0/c)."""
        if not self.full_chain:
            return 0.0
        return self.r_ref_m - self.dr * (4 + self.usable_bins / 2.0)

    def plan_params(self) -> dict:
        """The library's parameter block for this scene (field names follow the C header)."""
        return dict(
            Na=self.Na, Nr=self.Nr, pulse_s=self.pulse_s, bandwidth_hz=self.bandwidth_hz,
            fs_hz=self.fs_hz, range_window=1 if self.window == "hamming" else 0,
            carrier_hz=self.carrier_hz, prf_hz=self.prf_hz, velocity_mps=self.velocity_mps,
            range_bin0_m=self.range_bin0_m, rcmc_taps=self.rcmc_taps,
            kaiser_beta=self.kaiser_beta, flags=0)

    def with_(self, **kw) -> "SceneConfig":
        return replace(self, **kw)


# Tiny full-chain scene: 256 x 256, 2 us / 100 MHz / 120 MHz, X band 9.6 GHz, PRF 1 kHz,
# 100 m/s, 5 km.  Only ~8 leading-edge bins hold a whole echo, so separation is relaxed.
C1 = SceneConfig(
    name="tiny_rd_256x256", Na=256, Nr=256, pulse_s=2e-6, bandwidth_hz=100e6, fs_hz=120e6,
    window="rect", n_targets=3, noise_power=0.01, seed=1, carrier_hz=9.6e9, prf_hz=1000.0,
    velocity_mps=100.0, r_ref_m=5000.0, sep_range=4, sep_az=64)

# Range compression only, 4096 lines x 4096 samples, TBP 1000 (10 us, 100 MHz, 120 MHz),
# Hamming-windowed replica, 5 targets present in every line, unit-variance clutter.
C2 = SceneConfig(
    name="rc_4096x4096", Na=4096, Nr=4096, pulse_s=10e-6, bandwidth_hz=100e6, fs_hz=120e6,
    window="hamming", n_targets=5, noise_power=1.0, seed=2, sep_range=64)

# Full airborne RD focusing 4096 x 4096: 300 MHz / 360 MHz / 5 us, PRF 1.5 kHz, 150 m/s,
# 10 km, 16 targets, clutter -20 dB.
C3 = SceneConfig(
    name="rd_4096x4096", Na=4096, Nr=4096, pulse_s=5e-6, bandwidth_hz=300e6, fs_hz=360e6,
    window="rect", n_targets=16, noise_power=0.01, seed=3, carrier_hz=9.6e9, prf_hz=1500.0,
    velocity_mps=150.0, r_ref_m=10000.0, sep_range=9, sep_az=54)

# Non-power-of-two range length 6000 = 2^4 * 3 * 5^3, 8192 lines, chirp family of C2 with the
# sampling rate scaled to 6000 samples per line (same receive-window duration).
C4 = SceneConfig(
    name="rc_8192x6000", Na=8192, Nr=6000, pulse_s=10e-6, bandwidth_hz=100e6,
    fs_hz=120e6 * 6000.0 / 4096.0, window="hamming", n_targets=32, noise_power=1.0, seed=4,
    sep_range=64)

# Large scene 16384 x 16384 (2 GiB raw echo), 600 MHz / 720 MHz, PRF 2 kHz, 200 m/s, 15 km.
C5 = SceneConfig(
    name="rd_16384x16384", Na=16384, Nr=16384, pulse_s=5e-6, bandwidth_hz=600e6, fs_hz=720e6,
    window="rect", n_targets=64, noise_power=0.01, seed=5, carrier_hz=9.6e9, prf_hz=2000.0,
    velocity_mps=200.0, r_ref_m=15000.0, sep_range=9, sep_az=21)

CONFIGS = {"c1": C1, "c2": C2, "c3": C3, "c4": C4, "c5": C5}

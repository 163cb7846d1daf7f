"""Pins of the CPU oracle to what the pages and the mathematics fix (CPU only, no GPU).

Each test ties an oracle function to something other than itself: hand-worked DFT pairs, a
naive O(N^2) DFT, the time-domain correlation that range compression must equal, closed-form
point-response figures, exact special cases of the interpolator, the range-Doppler migration
that the scene simulator's independent forward model produces, and invariants of the chain.
A plausible mistake (dropped conjugate, wrong sign of a shift or of a phase, transposed axis,
off-by-one tap window, missing normalisation) fails at least one of them.
"""
import cmath
import json
import math
import os

import numpy as np
import pytest

from oracle import metrics as M
from oracle import rd_oracle as O
from rdscene import C1, C2, C3, C4, SceneConfig, make_scene

GOLD = os.path.join(os.path.dirname(__file__), "golden")
THEORY = json.load(open(os.path.join(GOLD, "point_response_theory.json")))

# C3's azimuth geometry (9.6 GHz, PRF 1.5 kHz, 150 m/s, 10 km, 4096 pulses) with a shorter pulse
# (1 us -> 360 samples) so the range axis is small enough for CPU tests; range resolution as C3.
C3_AZ = C3.with_(name="c3_azimuth_geometry", Nr=512, pulse_s=1e-6, n_targets=1, noise_power=0.0)
# A geometry with large migration (L band, 200 m/s, 3 km, 3.4 s aperture: ~15 samples RCM).
BIG = SceneConfig(name="large_migration", Na=4096, Nr=1024, pulse_s=2e-6, bandwidth_hz=100e6,
                  fs_hz=120e6, window="rect", n_targets=2, noise_power=0.0, seed=11,
                  carrier_hz=1.0e9, prf_hz=600.0, velocity_mps=200.0, r_ref_m=3000.0,
                  sep_range=9, sep_az=100)


def naive_dft(x, sign=-1.0):
    N = x.shape[0]
    n = np.arange(N)
    return np.exp(sign * 2j * np.pi * np.outer(n, n) / N) @ x


def single_chirp(cfg, window, n0):
    """One noiseless line holding the unweighted pulse at integer delay n0."""
    p = cfg.plan_params()
    p["range_window"] = window
    L = cfg.replica_len
    t = np.arange(L) / cfg.fs_hz
    x = np.zeros((1, cfg.Nr), np.complex128)
    x[0, n0:n0 + L] = np.exp(1j * np.pi * (cfg.bandwidth_hz / cfg.pulse_s) * (t - cfg.pulse_s / 2) ** 2)
    return p, x


@pytest.fixture(scope="module")
def c3az():
    sc = make_scene(C3_AZ, noise=False)
    return sc, O.focus_stages(sc.echo, C3_AZ.plan_params())


@pytest.fixture(scope="module")
def big():
    sc = make_scene(BIG, noise=False)
    return sc, O.focus_stages(sc.echo, BIG.plan_params())


# ---------------------------------------------------------------- transforms
def test_dft_hand_worked_pairs():
    for case in json.load(open(os.path.join(GOLD, "dft_small.json")))["cases"]:
        x = np.array([complex(*v) for v in case["x"]])
        X = np.array([complex(*v) for v in case["X"]])
        np.testing.assert_allclose(O.azimuth_fft(x[:, None])[:, 0], X, atol=1e-12)
        np.testing.assert_allclose(O.azimuth_ifft(X[:, None])[:, 0], x, atol=1e-12)


@pytest.mark.parametrize("N", list(range(1, 65)) + [240, 256, 375, 400])
def test_azimuth_transforms_match_naive_dft(N):
    rng = np.random.default_rng(N)
    x = rng.standard_normal((N, 3)) + 1j * rng.standard_normal((N, 3))
    X = naive_dft(x)
    np.testing.assert_allclose(O.azimuth_fft(x), X, rtol=0, atol=1e-11 * max(1, np.abs(X).max()))
    np.testing.assert_allclose(O.azimuth_ifft(X), naive_dft(X, +1.0) / N, atol=1e-11 * max(1, np.abs(x).max()))


def test_inverse_identity_and_parseval():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((4096, 2)) + 1j * rng.standard_normal((4096, 2))
    X = O.azimuth_fft(x)
    np.testing.assert_allclose(O.azimuth_ifft(X), x, atol=1e-14 * 64)
    # cf-1.com/news/2323550 §3.2: IFFT(x) = (1/N) conj(FFT(conj(x)))
    np.testing.assert_allclose(np.conj(O.azimuth_fft(np.conj(X))) / 4096, O.azimuth_ifft(X), atol=1e-13)
    assert abs(np.sum(np.abs(X) ** 2) / 4096 / np.sum(np.abs(x) ** 2) - 1) < 1e-13


# ---------------------------------------------------------------- range compression
@pytest.mark.parametrize("Nr", [40, 37, 12])     # composite, prime, replica as long as the line
def test_range_compression_is_circular_correlation_with_replica(Nr):
    p = dict(Na=3, Nr=Nr, pulse_s=1e-7, bandwidth_hz=80e6, fs_hz=120e6, range_window=1)
    h = O.chirp_replica(p)
    assert h.size == 12
    rng = np.random.default_rng(3)
    echo = rng.standard_normal((3, Nr)) + 1j * rng.standard_normal((3, Nr))
    brute = np.zeros_like(echo)
    for m in range(3):
        for i in range(Nr):
            brute[m, i] = sum(echo[m, (i + n) % Nr] * np.conj(h[n]) for n in range(h.size))
    np.testing.assert_allclose(O.range_compress(echo, p), brute, atol=1e-12)


def test_replica_is_windowed_up_chirp():
    p = C2.plan_params()
    h = O.chirp_replica(p)
    L = C2.replica_len
    assert h.size == L == 1200
    n = np.arange(L)
    np.testing.assert_allclose(np.abs(h), 0.54 - 0.46 * np.cos(2 * np.pi * n / (L - 1)), atol=1e-14)
    # instantaneous frequency rises linearly from -B/2 to +B/2 (up-chirp, Kr = B/Tp)
    f_inst = np.angle(h[1:] * np.conj(h[:-1])) * C2.fs_hz / (2 * np.pi)
    mid = (n[1:] + n[:-1]) / 2 / C2.fs_hz - C2.pulse_s / 2
    np.testing.assert_allclose(f_inst, C2.bandwidth_hz / C2.pulse_s * mid, atol=1e-3)
    assert C4.replica_len == 1758 and C3.replica_len == 1800 and C1.replica_len == 240


@pytest.mark.parametrize("L", [1, 2, 3, 12, 1200, 1758])
def test_hamming_window_is_the_symmetric_library_window(L):
    np.testing.assert_allclose(O.replica_window(L, 1), np.hamming(L), rtol=0, atol=1e-15)
    assert np.array_equal(O.replica_window(L, 0), np.ones(L))


@pytest.mark.parametrize("cfg", [C1, C2, C3, C4], ids=lambda c: c.name)
def test_compressed_chirp_matches_closed_forms(cfg):
    n0 = min(17, cfg.Nr - cfg.replica_len)
    L = cfg.replica_len
    irw = {}
    for window in (0, 1):
        p, x = single_chirp(cfg, window, n0)
        rc = O.range_compress(x, p)[0]
        k = int(np.argmax(np.abs(rc)))
        assert k == n0
        peak = L if window == 0 else 0.54 * L - 0.46
        assert abs(abs(rc[k]) / peak - 1) < 1e-9
        met = M.cut_metrics(rc[(k + np.arange(-32, 32)) % cfg.Nr])
        irw[window] = met["irw"]
        if window == 0:
            assert abs(met["pslr_db"] - THEORY["sinc_pslr_db"]) < THEORY["sinc_pslr_tol_db"]
            assert abs(met["islr_db"] - THEORY["sinc_islr_window64_db"]) < THEORY["sinc_islr_tol_db"]
            want = THEORY["sinc_irw_factor"] * cfg.fs_hz / cfg.bandwidth_hz
            assert abs(met["irw"] / want - 1) < THEORY["sinc_irw_rel_tol"]
        else:
            lo, hi = THEORY["hamming_pslr_db_range"]
            assert lo < met["pslr_db"] < hi
    lo, hi = THEORY["hamming_irw_ratio_range"]
    assert lo < irw[1] / irw[0] < hi


# ---------------------------------------------------------------- RCMC interpolator
def _rd_field(rows=6, cols=64, seed=0):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((rows, cols)) + 1j * rng.standard_normal((rows, cols))


def test_rcmc_zero_shift_is_identity():
    S = _rd_field()
    np.testing.assert_allclose(O.rcmc(S, np.zeros(S.shape)), S, rtol=0, atol=1e-14)


def test_rcmc_integer_shift_is_exact_shift_with_zero_fill():
    S = _rd_field()
    for s in (1, 3, -2):
        out = O.rcmc(S, np.full(S.shape, float(s)))
        want = np.zeros_like(S)
        if s > 0:
            want[:, :-s] = S[:, s:]
        else:
            want[:, -s:] = S[:, :s]
        np.testing.assert_allclose(out, want, atol=1e-15)


def test_rcmc_keeps_a_constant_field_constant_away_from_edges():
    S = np.full((4, 64), 2.0 - 1.0j)
    rng = np.random.default_rng(1)
    out = O.rcmc(S, rng.uniform(0, 3, S.shape))
    np.testing.assert_allclose(out[:, 4:-8], 2.0 - 1.0j, atol=1e-14)


def test_rcmc_interpolates_a_bandlimited_signal_at_the_shifted_position():
    # Output bin n must read the input at n + shift (not n - shift), from taps floor(x)-3..+4.
    n = np.arange(128)
    for nu, tol in ((0.01, 2e-3), (0.03, 1e-2)):        # a reversed shift errs by >= 0.026 / 0.078
        S = np.exp(2j * np.pi * nu * n)[None, :].repeat(3, 0)
        for frac in (0.2, 0.5, 0.77, 2.4):
            out = O.rcmc(S, np.full(S.shape, frac))
            want = np.exp(2j * np.pi * nu * (n + frac))
            assert np.max(np.abs(out[:, 8:-12] - want[8:-12])) < tol


def test_rcmc_weights_symmetric_at_half_sample():
    j = np.arange(-3, 5)
    w = O.kaiser_sinc(0.5 - j, 8, 2.5)
    np.testing.assert_allclose(w, w[::-1], atol=1e-15)
    # beta = 0 is the plain truncated sinc
    np.testing.assert_allclose(O.kaiser_sinc(0.3 - j, 8, 0.0), np.sinc(0.3 - j), atol=1e-15)


def _kaiser_window_error(kernel, beta):
    """Largest deviation of kernel(t, 8, beta) / sinc(t) from NumPy's M-point Kaiser window
    (an independent implementation of I0(beta sqrt(1 - (2n/(M-1) - 1)^2)) / I0(beta)) on the
    grid t = 4 (2n/(M-1) - 1), M = 81, integer t (where sinc vanishes) left out."""
    M = 81
    n = np.arange(M)
    t = 4.0 * (2.0 * n / (M - 1) - 1.0)
    keep = np.abs(t - np.round(t)) > 1e-9
    return np.max(np.abs(kernel(t[keep], 8, beta) / np.sinc(t[keep]) - np.kaiser(M, beta)[keep]))


@pytest.mark.parametrize("beta", [0.0, 2.5, 8.0])
def test_rcmc_window_is_the_library_kaiser_window(beta):
    """The interpolator's window over its 8-tap span is the Kaiser window (the 4096 x 4096
    airborne scene interpolates its RCMC with an 8-tap Kaiser-windowed sinc), pinned to
    numpy.kaiser rather than to its own formula."""
    assert _kaiser_window_error(O.kaiser_sinc, beta) < 1e-12


def test_rcmc_window_pin_rejects_plausible_misreadings():
    """Planted mistakes in the window formula -- the square root dropped, or a half-width of 3.5
    taps instead of 4 -- fail the pin above (each by far more than its tolerance)."""
    from scipy.special import i0

    def no_sqrt(t, taps, beta):
        return np.sinc(t) * i0(beta * np.clip(1.0 - (t / (taps / 2.0)) ** 2, 0.0, None)) / i0(beta)

    def half_width_35(t, taps, beta):
        arg = np.clip(1.0 - (t / 3.5) ** 2, 0.0, None)
        return np.sinc(t) * i0(beta * np.sqrt(arg)) / i0(beta)

    for beta in (2.5, 8.0):
        assert _kaiser_window_error(no_sqrt, beta) > 1e-2
        assert _kaiser_window_error(half_width_35, beta) > 1e-2


def test_rcmc_shift_matches_simulated_range_doppler_migration(big):
    """In Doppler bin k the compressed echo of a target at bin n_t peaks at n_t + Delta(n_t, k);
    the simulator's independent hyperbolic forward model puts it there."""
    sc, st = big
    p = BIG.plan_params()
    m, n = sc.targets[0]
    S = st["azfft"]
    shift = O.rcmc_shift(p, [n])[:, 0]
    f = O.doppler_freqs(p)
    half_band = BIG.velocity_mps ** 2 * 2 * (BIG.aperture_pulses / BIG.prf_hz / 2) / (BIG.wavelength * BIG.r_ref_m)
    energy = np.abs(S[:, n - 8:n + 40]).max(1)
    checked = 0
    for k in range(0, BIG.Na, 7):
        if abs(f[k]) > 0.8 * half_band or energy[k] < 0.3 * energy.max():
            continue
        u = M.upsample(S[k, n - 8:n + 40], 32)
        pos = np.argmax(np.abs(u)) / 32 + n - 8
        assert abs(pos - (n + shift[k])) < 0.1, (k, pos, n + shift[k])
        checked += 1
    assert checked > 100 and shift[np.abs(f) <= 0.8 * half_band].max() > 8


# ---------------------------------------------------------------- whole chain
def test_lone_targets_focus_at_predicted_pixels(c3az, big):
    for sc, st in (c3az, big):
        img = st["img"]
        for (m, n) in sc.targets:
            assert M.peak_near(img, m, n) == (m, n)
    sc = make_scene(C1.with_(n_targets=1, noise_power=0.0), noise=False)
    img = O.focus(sc.echo, C1.plan_params())
    (m, n), = sc.targets
    assert M.peak_near(img, m, n) == (m, n)


def test_focused_point_response_matches_theory(c3az):
    sc, st = c3az
    (m, n), = sc.targets
    pt = M.point_target(st["img"], m, n)
    ta = C3_AZ.aperture_pulses / C3_AZ.prf_hz
    ba = 2 * C3_AZ.velocity_mps ** 2 * ta / (C3_AZ.wavelength * (C3_AZ.range_bin0_m + n * C3_AZ.dr))
    assert abs(pt["azimuth"]["pslr_db"] - THEORY["sinc_pslr_db"]) < 0.3
    assert abs(pt["azimuth"]["irw"] / (0.886 * C3_AZ.prf_hz / ba) - 1) < 0.03
    assert abs(pt["range"]["pslr_db"] - THEORY["sinc_pslr_db"]) < 0.3
    assert abs(pt["range"]["irw"] / (0.886 * C3_AZ.fs_hz / C3_AZ.bandwidth_hz) - 1) < 0.03


def test_missing_or_reversed_rcmc_or_mf_is_detected(big):
    """Planted mistakes (on the CPU, in the oracle's own steps) degrade the focus visibly."""
    sc, st = big
    p = BIG.plan_params()
    nn = np.arange(BIG.Nr)
    m, n = sc.targets[0]
    good = abs(st["img"][m, n])
    S = st["azfft"]
    H = O.azimuth_matched_filter(p, nn)
    for R, Hf in ((O.rcmc(S, -O.rcmc_shift(p, nn)), H), (S, H), (st["rcmc"], np.conj(H))):
        bad = O.azimuth_ifft(R * Hf)
        assert np.abs(bad[m - 16:m + 17, n - 4:n + 5]).max() < 0.6 * good


def test_chain_is_linear():
    cfg = C1
    a = make_scene(cfg).echo.astype(np.complex128)
    b = make_scene(cfg.with_(seed=9)).echo.astype(np.complex128)
    p = cfg.plan_params()
    lhs = O.focus(0.7 * a - 1.3j * b, p)
    rhs = 0.7 * O.focus(a, p) - 1.3j * O.focus(b, p)
    assert M.rel_l2(lhs, rhs) < 1e-13


def test_azimuth_processing_is_circularly_shift_equivariant():
    cfg = C1
    x = make_scene(cfg).echo
    p = cfg.plan_params()
    img = O.focus(x, p)
    for s in (1, 37, -5):
        np.testing.assert_allclose(O.focus(np.roll(x, s, axis=0), p), np.roll(img, s, axis=0),
                                   atol=1e-12 * np.abs(img).max())


def test_sampled_columns_equal_whole_image(c3az):
    sc, st = c3az
    bins = [0, 3, 100, 101, 250, 511]
    cols, got_bins = O.focus_columns(sc.echo, C3_AZ.plan_params(), bins, block_rows=700)
    assert list(got_bins) == sorted(bins)
    np.testing.assert_allclose(cols, st["img"][:, got_bins], atol=1e-12 * np.abs(st["img"]).max())


def test_sampled_column_stages_equal_whole_chain_stages(c3az):
    """focus_columns(stages=True) returns the whole chain's rc, azimuth spectrum, RCMC output and
    image at the sampled range bins (the sampled C5 parity test compares each stage there)."""
    sc, st = c3az
    bins = [0, 1, 2, 255, 256, 300, 508, 509, 510, 511]
    got, got_bins = O.focus_columns(sc.echo, C3_AZ.plan_params(), bins, block_rows=1000, stages=True)
    assert list(got_bins) == bins
    for name in ("rc", "azfft", "rcmc", "img"):
        ref = st[name][:, bins]
        np.testing.assert_allclose(got[name], ref, atol=1e-12 * np.abs(ref).max(), err_msg=name)


def test_shift_and_filter_at_selected_doppler_bins_are_the_rows_of_the_whole():
    p = C3_AZ.plan_params()
    n = np.arange(0, C3_AZ.Nr, 7)
    k = [0, 5, C3_AZ.Na // 2, C3_AZ.Na - 1]
    np.testing.assert_array_equal(O.rcmc_shift(p, n, k), O.rcmc_shift(p, n)[k])
    np.testing.assert_array_equal(O.azimuth_matched_filter(p, n, k), O.azimuth_matched_filter(p, n)[k])


def test_line_errors_find_a_defect_that_the_whole_array_norm_dilutes():
    """A 5e-4 relative error confined to one column of a 4096 x 4096-like array passes a 1e-5
    bar on the whole-array norm but shows at full size in the column error; uniform rounding
    noise gives line errors of the order of the global error."""
    rng = np.random.default_rng(9)
    ref = rng.standard_normal((1024, 1024)) + 1j * rng.standard_normal((1024, 1024))
    bad = ref.copy()
    bad[:, 77] *= 1 + 5e-4
    assert M.rel_l2(bad, ref) < 1e-5 * 2
    worst_row, worst_col = M.worst_line_errors(bad, ref)
    assert abs(worst_col - 5e-4) < 2e-5 and worst_row < 1e-4   # a row holds one bad sample of 1024
    noisy = ref * (1 + 1e-7 * rng.standard_normal(ref.shape))
    g = M.rel_l2(noisy, ref)
    assert max(M.worst_line_errors(noisy, ref)) < 2 * g
    # a line with almost no energy is measured against an average line, not its own norm
    quiet = ref.copy()
    quiet[5] *= 1e-9
    q2 = quiet.copy()
    q2[5] += 1e-9
    assert M.worst_line_errors(q2, quiet)[0] < 1e-8


def test_azimuth_half_composes_with_range_compression_to_the_chain(c3az):
    """azimuth_focus(range_compress(echo)) is the whole chain's image, and the azimuth half is
    linear in its input (a scaled and a summed input give the scaled and summed images)."""
    sc, st = c3az
    p = C3_AZ.plan_params()
    img = O.azimuth_focus(st["rc"], p)
    np.testing.assert_allclose(img, st["img"], atol=1e-12 * np.abs(st["img"]).max())
    rng = np.random.default_rng(5)
    x = rng.standard_normal(st["rc"].shape) + 1j * rng.standard_normal(st["rc"].shape)
    lin = O.azimuth_focus((2 - 1j) * st["rc"] + x, p)
    np.testing.assert_allclose(lin, (2 - 1j) * img + O.azimuth_focus(x, p), atol=1e-10 * np.abs(lin).max())


def test_metrics_ignore_a_linear_phase_ramp():
    p, x = single_chirp(C3, 0, 17)
    rc = O.range_compress(x, p)[0]
    cut = rc[np.arange(-15, 49)]
    ramp = cut * np.exp(1j * 2.3 * np.arange(64))
    a, b = M.cut_metrics(cut), M.cut_metrics(ramp)
    for key in ("pslr_db", "islr_db", "irw"):
        assert abs(a[key] - b[key]) < 1e-6
    assert M.rel_l2(cut * 1.001, cut) == pytest.approx(1e-3, rel=1e-9)


def test_corner_turn_is_the_element_by_element_transpose():
    """out[c][r] = x[r][c] by a brute-force double loop on ragged shapes; two turns restore x."""
    rng = np.random.default_rng(7)
    for rows, cols in ((1, 1), (1, 5), (3, 2), (7, 13), (64, 65)):
        x = (rng.standard_normal((rows, cols)) + 1j * rng.standard_normal((rows, cols))).astype(np.complex64)
        y = O.corner_turn(x)
        assert y.shape == (cols, rows) and y.flags["C_CONTIGUOUS"]
        for r in range(rows):
            for c in range(cols):
                assert y[c, r] == x[r, c]
        assert np.array_equal(O.corner_turn(y), x)


# ------------------------------------------------------------------------------ back-projection
def _bp_brute(rc, params, grid):
    """Pure-Python triple loop of the back-projection definition (tiny sizes only)."""
    Na, Nr = rc.shape
    V, prf, lam = params["velocity_mps"], params["prf_hz"], 299_792_458.0 / params["carrier_hz"]
    dr = 299_792_458.0 / (2 * params["fs_hz"])
    out = np.zeros((grid["nx"], grid["ny"]), complex)
    for i in range(grid["nx"]):
        x = grid["x0_m"] + i * grid["dx_m"]
        for j in range(grid["ny"]):
            r = grid["r0_m"] + j * grid["dr_m"]
            acc = 0j
            for m in range(Na):
                d = math.hypot(r, x - V * m / prf)
                b = (d - params["range_bin0_m"]) / dr
                i0 = math.floor(b)
                w = b - i0
                s0 = complex(rc[m, i0]) if 0 <= i0 < Nr else 0j
                s1 = complex(rc[m, i0 + 1]) if 0 <= i0 + 1 < Nr else 0j
                acc += ((1 - w) * s0 + w * s1) * cmath.exp(4j * math.pi * d / lam)
            out[i, j] = acc
    return out


def test_backprojection_matches_brute_force_loops():
    """The vectorised oracle equals a pure-Python loop over pixels and pulses, including pixels
    whose range history leaves the line (zero samples)."""
    rng = np.random.default_rng(11)
    params = C1.plan_params()
    Na, Nr = 9, 40
    params.update(Na=Na, Nr=Nr)
    rc = rng.standard_normal((Na, Nr)) + 1j * rng.standard_normal((Na, Nr))
    dr = O.range_spacing(params)
    grid = dict(nx=3, ny=5, x0_m=-0.7, dx_m=0.9, r0_m=params["range_bin0_m"] - 2.3 * dr, dr_m=9.7 * dr)
    got = O.backproject(rc, params, grid)
    want = _bp_brute(rc, params, grid)
    # the phases 4 pi d / lambda reach ~2e6 rad, whose float64 rounding is ~5e-10 rad per term
    assert np.max(np.abs(got - want)) < 1e-8 * np.max(np.abs(want))
    assert np.allclose(O.backproject_pixels(rc, params, grid, [(0, 0), (2, 4)]), want[[0, 2], [0, 4]], rtol=1e-8)


def test_backprojection_outside_the_swath_is_zero():
    rc = np.ones((8, 64), complex)
    params = C1.plan_params()
    params.update(Na=8, Nr=64)
    grid = dict(nx=2, ny=2, x0_m=0.0, dx_m=1.0, r0_m=params["range_bin0_m"] + 1e4, dr_m=1.0)
    assert np.all(O.backproject(rc, params, grid) == 0)


def test_backprojection_of_a_lone_target_is_the_coherent_sum_of_its_peaks():
    """Closed form: with negligible range migration, a unit target's range-compressed peak is L
    (rect window) in every illuminated pulse and the carrier phase is compensated exactly, so
    the target pixel sums to L * (illuminated pulses), real and positive."""
    cfg = SceneConfig(name="bp_far", Na=128, Nr=256, pulse_s=1e-6, bandwidth_hz=100e6, fs_hz=120e6,
                      window="rect", n_targets=1, noise_power=0.0, seed=21, carrier_hz=9.6e9,
                      prf_hz=1000.0, velocity_mps=10.0, r_ref_m=2.0e5, sep_range=4, sep_az=0)
    sc = make_scene(cfg, noise=False)
    p = cfg.plan_params()
    (mt, nt), = sc.targets
    rc = O.range_compress(sc.echo, p)
    assert cfg.rcm_max_samples < 1e-4
    grid = dict(nx=1, ny=1, x0_m=cfg.velocity_mps * mt / cfg.prf_hz, dx_m=0.0,
                r0_m=p["range_bin0_m"] + nt * O.range_spacing(p), dr_m=0.0)
    v = O.backproject(rc, p, grid)[0, 0]
    want = cfg.replica_len * cfg.aperture_pulses
    assert abs(v - want) < 1e-3 * want          # float32 echo; migration < 1e-4 sample


def test_backprojection_and_range_doppler_focus_targets_at_the_same_pixels(big):
    """Two independent focusing methods of the oracle agree on where every noiseless target of a
    large-migration scene (~15 samples of migration) focuses: back-projection on the focusing
    grid (one pixel per pulse and per range bin) peaks at the pixel where the range-Doppler
    image peaks, the predicted (m_t, n_t)."""
    cfg = BIG
    sc, ref = big
    p = cfg.plan_params()
    rc = ref["rc"]
    dr = O.range_spacing(p)
    for (mt, nt) in sc.targets:
        assert M.peak_near(ref["img"], mt, nt) == (mt, nt)
        grid = dict(nx=9, ny=9, x0_m=cfg.velocity_mps * (mt - 4) / cfg.prf_hz, dx_m=cfg.velocity_mps / cfg.prf_hz,
                    r0_m=p["range_bin0_m"] + (nt - 4) * dr, dr_m=dr)
        img = O.backproject(rc, p, grid)
        assert np.unravel_index(np.argmax(np.abs(img)), img.shape) == (4, 4), (mt, nt)


def test_backprojection_misfocuses_with_a_wrong_wavelength_or_velocity(big):
    """Planted mistakes ([BP-GPU] §3.2 and §4.2's defocus causes: wrong platform speed, wrong
    wavelength) collapse the target's coherent sum on the large-migration geometry."""
    sc, ref = big
    p = BIG.plan_params()
    (mt, nt) = sc.targets[0]
    grid = dict(nx=1, ny=1, x0_m=BIG.velocity_mps * mt / BIG.prf_hz, dx_m=0.0,
                r0_m=p["range_bin0_m"] + nt * O.range_spacing(p), dr_m=0.0)
    good = abs(O.backproject(ref["rc"], p, grid)[0, 0])
    # most of L x (illuminated pulses) survives the interpolation across ~15 samples of migration
    assert good > 0.75 * BIG.replica_len * BIG.aperture_pulses
    for wrong in (dict(carrier_hz=0.95e9), dict(carrier_hz=1.05e9), dict(velocity_mps=190.0),
                  dict(velocity_mps=210.0)):
        assert abs(O.backproject(ref["rc"], dict(p, **wrong), grid)[0, 0]) < 0.2 * good, wrong


# ---------------------------------------------------------------- omega-k
def ref_bin_of(cfg) -> int:
    """Range bin of the scene's reference (closest-approach) range."""
    return int(round((cfg.r_ref_m - cfg.range_bin0_m) / cfg.dr))


# a tiny geometry with Stolt shifts of ~1.6 bins on a 16-bin line
TINY_WK = dict(Na=8, Nr=16, pulse_s=1e-7, bandwidth_hz=80e6, fs_hz=120e6, range_window=0,
               carrier_hz=1.0e9, prf_hz=200.0, velocity_mps=100.0, range_bin0_m=1000.0,
               rcmc_taps=8, kaiser_beta=2.5)


def _brute_omega_k(x, p, ref):
    """omega-k with explicit loops: 2-D DFT by sums, the filter and reference phase per element,
    the Stolt mapping as an absolute source position on the centred frequency axis, Kaiser
    weights from their formula, inverse 2-D DFT by sums."""
    Na, Nr = x.shape
    fs, f0, prf, V = p["fs_hz"], p["carrier_hz"], p["prf_hz"], p["velocity_mps"]
    c = 299_792_458.0
    dr = c / (2 * fs)
    rb0 = p["range_bin0_m"]
    r_ref = rb0 + ref * dr
    h = O.chirp_replica(p)
    H = [sum(h[n] * cmath.exp(-2j * math.pi * j * n / Nr) for n in range(h.size)).conjugate() for j in range(Nr)]
    S = np.zeros((Na, Nr), complex)
    for k in range(Na):
        for j in range(Nr):
            S[k, j] = sum(x[m, n] * cmath.exp(-2j * math.pi * (k * m / Na + j * n / Nr))
                          for m in range(Na) for n in range(Nr))
    sfreq = lambda i, N, rate: (i if i < N // 2 else i - N) * rate / N
    G = np.zeros_like(S)
    for k in range(Na):
        b2 = (c * sfreq(k, Na, prf) / (2 * V)) ** 2
        for j in range(Nr):
            f = sfreq(j, Nr, fs)
            Q = math.sqrt((f0 + f) ** 2 - b2)
            G[k, j] = S[k, j] * H[j] * cmath.exp(2j * math.pi * ((2 * r_ref / c) * Q - f * 2 * rb0 / c))
    T = np.zeros_like(S)
    beta = p["kaiser_beta"]
    for k in range(Na):
        b2 = (c * sfreq(k, Na, prf) / (2 * V)) ** 2
        for u in range(Nr):
            fp = (u - Nr // 2) * fs / Nr
            src = math.sqrt((f0 + fp) ** 2 + b2) - f0
            pos = src / (fs / Nr) + Nr // 2          # natural-order position of the source
            i0 = math.floor(pos)
            acc, wsum = 0j, 0.0
            for jt in range(-3, 5):
                idx = i0 + jt
                t = pos - idx
                w = (math.sin(math.pi * t) / (math.pi * t) if t != 0 else 1.0) * \
                    float(np.i0(beta * math.sqrt(max(0.0, 1 - (t / 4) ** 2)))) / float(np.i0(beta))
                wsum += w
                if 0 <= idx < Nr:
                    acc += w * G[k, (idx + Nr // 2) % Nr]
            T[k, (u + Nr // 2) % Nr] = acc / wsum * cmath.exp(-2j * math.pi * fp * 2 * (r_ref - rb0) / c)
    img = np.zeros_like(S)
    for m in range(Na):
        for n in range(Nr):
            img[m, n] = sum(T[k, j] * cmath.exp(2j * math.pi * (k * m / Na + j * n / Nr))
                            for k in range(Na) for j in range(Nr)) / (Na * Nr)
    return img


def test_omega_k_matches_brute_force_loops():
    rng = np.random.default_rng(21)
    x = rng.standard_normal((8, 16)) + 1j * rng.standard_normal((8, 16))
    assert 1.0 < O.stolt_shift(TINY_WK).max() < 3.0
    for ref in (0, 5):
        got = O.omega_k(x, TINY_WK, ref)
        want = _brute_omega_k(x, TINY_WK, ref)
        assert M.rel_l2(got, want) < 1e-11


def test_omega_k_of_an_azimuth_constant_echo_is_range_compression():
    """Only the zero-Doppler row is non-zero: no Stolt shift, the reference phase reduces to a
    constant and a linear ramp that the final phase cancels, so the image is every line's range
    compression times exp(+j 4 pi Rref / lambda)."""
    p = dict(C3_AZ.plan_params(), Na=16)
    rng = np.random.default_rng(4)
    line = rng.standard_normal(p["Nr"]) + 1j * rng.standard_normal(p["Nr"])
    echo = np.tile(line, (16, 1))
    ref = 37
    r_ref = p["range_bin0_m"] + ref * C3_AZ.dr
    want = O.range_compress(echo, p) * np.exp(4j * np.pi * r_ref / O.wavelength(p))
    np.testing.assert_allclose(O.omega_k(echo, p, ref), want, rtol=0, atol=1e-9 * np.abs(want).max())


def test_stolt_mapping_lands_on_the_wavenumber_circle():
    p = dict(BIG.plan_params(), Na=512)
    Nr, fs, f0 = BIG.Nr, BIG.fs_hz, BIG.carrier_hz
    d = O.stolt_shift(p)
    b2 = O.doppler_wavenumber_sq(p)
    fp = (np.arange(Nr) - Nr // 2) * fs / Nr
    src = fp[None, :] + d * fs / Nr
    # the source frequency has Q(f_src, f_k) = f0 + f'
    np.testing.assert_allclose(np.sqrt((f0 + src) ** 2 - b2[:, None]), f0 + fp[None, :] + 0 * d, rtol=1e-13)
    assert np.all(d >= 0) and np.all(d[0] == 0.0)
    k = np.argsort(b2)
    assert np.all(np.diff(d[k, 0]) >= 0)              # larger Doppler, larger shift


@pytest.fixture(scope="module")
def big_wk(big):
    sc, _ = big
    return O.omega_k(sc.echo, BIG.plan_params(), ref_bin_of(BIG))


def test_omega_k_focuses_lone_targets_at_predicted_pixels(c3az, big, big_wk):
    sc, st = c3az
    img = O.omega_k(sc.echo, C3_AZ.plan_params(), ref_bin_of(C3_AZ))
    (m, n), = sc.targets
    assert M.peak_near(img, m, n) == (m, n)
    # same pixel and nearly the same peak as range-Doppler focusing
    assert abs(abs(img[m, n]) / abs(st["img"][m, n]) - 1) < 0.02
    pt = M.point_target(img, m, n)
    assert abs(pt["azimuth"]["pslr_db"] - THEORY["sinc_pslr_db"]) < 0.3
    assert abs(pt["range"]["pslr_db"] - THEORY["sinc_pslr_db"]) < 0.3
    sc, st = big
    for (m, n) in sc.targets:
        assert M.peak_near(big_wk, m, n) == (m, n)


def test_omega_k_keeps_the_range_response_where_range_doppler_loses_it(big, big_wk):
    """Large migration (L band, 3 km): the wavenumber-domain mapping is exact in range frequency,
    so the range cut keeps the textbook sinc, while range-Doppler focusing (no secondary range
    compression) loses ~0.7 dB of range PSLR and ~5% of the peak."""
    sc, st = big
    for (m, n) in sc.targets:
        wk = M.point_target(big_wk, m, n)
        rd = M.point_target(st["img"], m, n)
        assert abs(wk["range"]["pslr_db"] - THEORY["sinc_pslr_db"]) < 0.15
        assert abs(wk["azimuth"]["pslr_db"] - THEORY["sinc_pslr_db"]) < 0.15
        assert rd["range"]["pslr_db"] > wk["range"]["pslr_db"] + 0.4
        assert abs(big_wk[m, n]) > 1.03 * abs(st["img"][m, n])


@pytest.mark.parametrize("mistake", ["reversed_stolt", "no_stolt", "conjugate_reference", "velocity_10pct"])
def test_omega_k_planted_mistakes_are_detected(big, big_wk, monkeypatch, mistake):
    """Planted mistakes (on the CPU, in the oracle's own steps) collapse the focus."""
    sc, _ = big
    m, n = sc.targets[0]
    good = abs(big_wk[m, n])
    s, r, b = O.stolt_shift, O.reference_function, O.doppler_wavenumber_sq
    if mistake == "reversed_stolt":
        monkeypatch.setattr(O, "stolt_shift", lambda q: -s(q))
    elif mistake == "no_stolt":
        monkeypatch.setattr(O, "stolt_shift", lambda q: 0.0 * s(q))
    elif mistake == "conjugate_reference":
        monkeypatch.setattr(O, "reference_function", lambda q, k: np.conj(r(q, k)))
    else:
        monkeypatch.setattr(O, "doppler_wavenumber_sq", lambda q: b(q) / 1.1 ** 2)
    bad = O.omega_k(sc.echo, BIG.plan_params(), ref_bin_of(BIG))
    assert np.abs(bad[m - 16:m + 17, n - 4:n + 5]).max() < 0.3 * good

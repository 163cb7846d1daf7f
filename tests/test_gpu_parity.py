"""Parity of the HIP path (through the C ABI) with the CPU fp64 oracle, on the GPU.

Bars: relative L2 <= 1e-5 per stage and <= 1e-4 for the focused image, over the whole array and
over every row and every column on its own (check_stage); target peak indices identical to the
oracle's; PSLR / ISLR of every target within 0.1 dB of the oracle's.
Binary16 storage has its own tier against the oracle on the same binary16 input: range
compression within half a binary16 ulp (+1e-5 of the RMS) per stored component and rel-L2 <=
4e-4; the focusing chains rel-L2 <= 3e-3 (six stored roundings of at most 2^-11 each), peaks a
valid argmax within that error, PSLR within 0.1 dB.
Sizes: the five workloads at their full sizes (the 16384 x 16384 scene on sampled lines and
range bins, which the oracle computes one by one), plus ragged line counts and every built
transform length for the line FFT.
"""
import sys

import numpy as np
import pytest

from oracle import metrics as M
from oracle import rd_oracle as O
from rdscene import C1, C2, C3, C4, C5, SceneConfig, cached_scene, make_scene

pytestmark = pytest.mark.gpu

# L band, slow platform, long rows: ~540 samples of range migration at the Doppler band edge,
# so the chunked RCMC kernel stages a halo longer than one pass of its threads.
LONG_MIGRATION = SceneConfig(
    name="long_migration_512x8192", Na=512, Nr=8192, pulse_s=2e-6, bandwidth_hz=100e6,
    fs_hz=120e6, window="rect", n_targets=4, noise_power=0.01, seed=12, carrier_hz=1.3e9,
    prf_hz=800.0, velocity_mps=150.0, r_ref_m=8000.0, sep_range=9, sep_az=64)

# full-chain scenes at line lengths with no built transform (padded range compression, RCMC on
# rows of run-time length in 1024-sample chunks with a ragged last chunk)
RD_1200 = C3.with_(name="rd_1024x1200", Na=1024, Nr=1200, pulse_s=1e-6, n_targets=4)
RD_3001 = SceneConfig(
    name="rd_2048x3001_large_migration", Na=2048, Nr=3001, pulse_s=2e-6, bandwidth_hz=100e6,
    fs_hz=120e6, window="rect", n_targets=3, noise_power=0.01, seed=13, carrier_hz=1.0e9,
    prf_hz=600.0, velocity_mps=200.0, r_ref_m=3000.0, sep_range=9, sep_az=100)

# azimuth lengths that are not powers of two (Na = 32 x 25): the image size of the airborne
# test in nxmr.cn/news/101525 §5.3 (1200 range samples x 800 pulses), and an omega-k case
RD_800 = C3.with_(name="rd_800x1200", Na=800, Nr=1200, pulse_s=1e-6, n_targets=4)
WK_800 = C3.with_(name="wk_800x1024", Na=800, Nr=1024, pulse_s=1e-6, n_targets=3)
# azimuth lengths through the Bluestein form: 1000 = 2^3 5^3, and the prime 997
RD_1000 = C3.with_(name="rd_1000x1024", Na=1000, Nr=1024, pulse_s=1e-6, n_targets=3)
WK_997 = C3.with_(name="wk_997x1024", Na=997, Nr=1024, pulse_s=1e-6, n_targets=3)

STAGE_TOL = 1e-5
IMAGE_TOL = 1e-4
LENGTHS = (256, 512, 1024, 2048, 4096, 8192, 16384, 6000)


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    torch.cuda.set_device(0)
    return torch


@pytest.fixture(scope="module")
def rdf(torch_dev):
    import range_doppler_focusing_amd as rdf
    rdf.load_library()
    return rdf


def dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.complex64)).to("cuda")


_oracle_cache = {}


def scene_and_stages(cfg):
    if cfg.name not in _oracle_cache:
        sc = make_scene(cfg)
        log(f"[oracle] {cfg.name}: focusing on the CPU")
        _oracle_cache[cfg.name] = (sc, O.focus_stages(sc.echo, cfg.plan_params()))
    return _oracle_cache[cfg.name]


def check_stage(label, got, ref, bar):
    """The parity bar of one stage: the whole-array relative L2 error within `bar`, and so is the
    error of every row and of every column on its own (metrics.line_errors).  A defect confined
    to a few lines -- a chunk seam, a ragged tail, an edge -- is diluted by the square root of
    the line count in the whole-array norm, but not in its line's error."""
    err = M.rel_l2(got, ref)
    worst_row, worst_col = M.worst_line_errors(got, ref)
    log(f"{label}: rel-L2 {err:.2e}, worst row {worst_row:.2e}, worst column {worst_col:.2e}")
    assert err <= bar and worst_row <= bar and worst_col <= bar, (label, err, worst_row, worst_col)
    return err


# ------------------------------------------------------------------------------ line transform
@pytest.mark.parametrize("n", LENGTHS)
def test_line_fft_matches_dft(torch_dev, rdf, n):
    torch = torch_dev
    lines = 37                       # not a multiple of any lines-per-workgroup count
    rng = np.random.default_rng(n)
    x = (rng.standard_normal((lines, n)) + 1j * rng.standard_normal((lines, n))).astype(np.complex64)
    log(f"[line fft] n={n} lines={lines}")
    with rdf.Plan(Na=64, Nr=n, pulse_s=1e-6, bandwidth_hz=100e6, fs_hz=120e6) as plan:
        xd = dev(torch, x)
        X = plan.line_fft(xd, axis=1).cpu().numpy()
        xi = plan.line_fft(dev(torch, X), axis=1, inverse=True).cpu().numpy()
        # in place gives the same bits
        y = xd.clone()
        rdf.rd_debug_line_fft(plan.handle, 1, 0, y, y, lines)
        torch.cuda.synchronize()
        assert torch.equal(y.cpu(), torch.from_numpy(X))
    ref = np.fft.fft(x.astype(np.complex128), axis=1)
    assert M.rel_l2(X, ref) < 2e-7 * np.log2(n)
    assert M.rel_l2(xi, x) < 4e-7 * np.log2(n)


def test_line_fft_zero_lines_is_a_no_op(torch_dev, rdf):
    with rdf.Plan(Na=64, Nr=256, pulse_s=1e-6, bandwidth_hz=100e6, fs_hz=120e6) as plan:
        x = torch_dev.zeros((1, 256), dtype=torch_dev.complex64, device="cuda")
        rdf.rd_debug_line_fft(plan.handle, 1, 0, x, x, 0)


# ------------------------------------------------------------------------------ range compression
@pytest.mark.parametrize("cfg", [C1, C2, C3, C4], ids=lambda c: c.name)
def test_range_compression_full(torch_dev, rdf, cfg):
    torch = torch_dev
    sc = make_scene(cfg)
    log(f"[range] {cfg.name} {cfg.Na}x{cfg.Nr}")
    with rdf.Plan(**cfg.plan_params()) as plan:
        echo = dev(torch, sc.echo)
        rc = plan.range_compress(echo).cpu().numpy()
        # in place gives the same bits
        plan.range_compress(echo, out=echo)
        torch.cuda.synchronize()
        assert np.array_equal(echo.cpu().numpy(), rc)
    ref = O.range_compress(sc.echo, cfg.plan_params())
    check_stage(f"[range] {cfg.name}", rc, ref, STAGE_TOL)
    if not cfg.full_chain:
        # every target's compressed peak sits at its delay in every sampled line
        for m in (0, cfg.Na // 2, cfg.Na - 1):
            for (_, n) in sc.targets:
                win = np.abs(rc[m, n - 4:n + 5])
                assert int(np.argmax(win)) == 4 == int(np.argmax(np.abs(ref[m, n - 4:n + 5])))


@pytest.mark.parametrize("n", LENGTHS)
@pytest.mark.parametrize("lines", [1, 37])
def test_range_compression_every_length(torch_dev, rdf, n, lines):
    """Every built line length, a ragged line count and a single line: the register-cached
    kernel against the oracle, in place bit-identical to out of place."""
    torch = torch_dev
    rng = np.random.default_rng(1000 + n + lines)
    fs = 120e6
    params = dict(Na=lines, Nr=n, pulse_s=(n // 3) / fs, bandwidth_hz=90e6, fs_hz=fs,
                  range_window=int(n % 3 == 0))
    echo = (rng.standard_normal((lines, n)) + 1j * rng.standard_normal((lines, n))).astype(np.complex64)
    log(f"[range] every length: n={n} lines={lines}")
    with rdf.Plan(**params) as plan:
        x = dev(torch, echo)
        rc = plan.range_compress(x).cpu().numpy()
        plan.range_compress(x, out=x)
        torch.cuda.synchronize()
        assert np.array_equal(x.cpu().numpy(), rc)
    check_stage(f"[range] n={n} lines={lines}", rc, O.range_compress(echo, params), STAGE_TOL)


# Line counts above one round of the persistent grid and not a multiple of it (4096: 1024
# workgroups; 6000: 512; 16384: 256 on 256 CUs): some workgroups take one line more than others,
# and every line crosses the loop's prefetch, exchange and table paths at least twice.
@pytest.mark.parametrize("n,lines", [(4096, 1531), (6000, 777), (16384, 301)], ids=lambda v: str(v))
def test_range_compression_persistent_ragged(torch_dev, rdf, n, lines):
    """The persistent range kernels over more lines than one grid round (float32 and binary16):
    every line against the oracle, element by element per line; in place equals out of place."""
    torch = torch_dev
    rng = np.random.default_rng(5000 + n + lines)
    fs = 120e6
    params = dict(Na=lines, Nr=n, pulse_s=(n // 3) / fs, bandwidth_hz=90e6, fs_hz=fs, range_window=1)
    echo = (rng.standard_normal((lines, n)) + 1j * rng.standard_normal((lines, n))).astype(np.complex64)
    log(f"[range] persistent ragged: n={n} lines={lines}")
    ref = O.range_compress(echo, params)
    with rdf.Plan(**params) as plan:
        x = dev(torch, echo)
        rc = plan.range_compress(x).cpu().numpy()
        plan.range_compress(x, out=x)
        torch.cuda.synchronize()
        assert np.array_equal(x.cpu().numpy(), rc)
        check_stage(f"[range] persistent n={n} lines={lines}", rc, ref, STAGE_TOL)
        eh = to_half(echo)
        xh = torch.from_numpy(eh).to("cuda")
        rch = plan.range_compress_f16(xh).cpu().numpy()
    err = check_half(rch, O.range_compress(from_half(eh), params))
    log(f"[range f16] persistent n={n} lines={lines} rel-L2 {err:.2e}")


# (line length, replica length): padded transform lengths M = nextpow2(max(256, n + L - 1))
# 256, 512, 1024, 2048, 4096, 8192, 16384, and replicas of one sample up to the whole line
ANY_LENGTHS = [(1, 1), (7, 7), (127, 42), (129, 43), (300, 100), (700, 233), (1000, 333),
               (1200, 400), (1201, 1201), (2049, 683), (3001, 1000), (4097, 1365), (5000, 1666),
               (8191, 2730), (8191, 8191)]


@pytest.mark.parametrize("n,L", ANY_LENGTHS, ids=lambda v: str(v))
@pytest.mark.parametrize("lines", [1, 37])
def test_range_compression_any_length(torch_dev, rdf, n, L, lines):
    """Line lengths with no built transform (range-only plans): the zero-padded convolution
    against the oracle's length-n circular correlation, in place bit-identical to out of place."""
    torch = torch_dev
    rng = np.random.default_rng(2000 + n + L + lines)
    fs = 120e6
    params = dict(Na=lines, Nr=n, pulse_s=L / fs, bandwidth_hz=90e6, fs_hz=fs,
                  range_window=int(n % 2 == 0))
    assert O.replica_length(params) == L
    echo = (rng.standard_normal((lines, n)) + 1j * rng.standard_normal((lines, n))).astype(np.complex64)
    log(f"[range] any length: n={n} L={L} lines={lines}")
    with rdf.Plan(**params) as plan:
        x = dev(torch, echo)
        rc = plan.range_compress(x).cpu().numpy()
        plan.range_compress(x, out=x)
        torch.cuda.synchronize()
        assert np.array_equal(x.cpu().numpy(), rc)
    check_stage(f"[range] n={n} L={L} lines={lines}", rc, O.range_compress(echo, params), STAGE_TOL)


def test_range_compression_any_length_large(torch_dev, rdf):
    """16384 lines of 1200 samples (the padded kernel at its bench size, persistent grid over
    many lines per workgroup) on sampled lines, and a lone chirp's peak at its delay."""
    torch = torch_dev
    Na, n, fs = 16384, 1200, 120e6
    params = dict(Na=Na, Nr=n, pulse_s=400 / fs, bandwidth_hz=100e6, fs_hz=fs, range_window=1)
    rows = np.array([0, 1, 2, 255, 4095, 8191, 12000, 16383])
    echo = torch.empty((Na, n), dtype=torch.complex64, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(5)
    echo.view(torch.float32).normal_(generator=gen)
    h = O.chirp_replica(params)
    lone = np.zeros(n, np.complex128)
    lone[333:333 + h.size] = np.exp(1j * np.pi * (100e6 / (400 / fs)) * (np.arange(h.size) / fs - 200 / fs) ** 2)
    echo[5] = torch.from_numpy(lone.astype(np.complex64)).to("cuda")
    rows = np.union1d(rows, [5])
    with rdf.Plan(**params) as plan:
        rc = plan.range_compress(echo)
        got = rc[torch.from_numpy(rows).to("cuda")].cpu().numpy()
        ech = echo[torch.from_numpy(rows).to("cuda")].cpu().numpy()
        del rc, echo
    ref = O.range_compress(ech, params)
    check_stage("[range] 16384x1200 sampled lines", got, ref, STAGE_TOL)
    k = int(np.argmax(np.abs(got[list(rows).index(5)])))
    assert k == 333 == int(np.argmax(np.abs(ref[list(rows).index(5)])))


# ------------------------------------------------------------------------------ binary16 storage
def to_half(x):
    """complex array -> float16 [..., 2] (real, imaginary), rounded to nearest even."""
    return np.stack([x.real, x.imag], axis=-1).astype(np.float16)


def from_half(h):
    return h[..., 0].astype(np.float64) + 1j * h[..., 1].astype(np.float64)


def check_half(got, ref):
    """The binary16-storage bar: every stored component lies within half a binary16 ulp of the
    float64 result (the rounding on store) plus the float32 arithmetic's error (1e-5 of the
    RMS); and the relative L2 error is at most 4e-4 (the RMS of a round-to-nearest error is
    about 2^-11 / sqrt(3) = 2.8e-4 of the magnitude)."""
    g = got.astype(np.float64)
    r = np.stack([ref.real, ref.imag], axis=-1)
    ulp = np.spacing(np.abs(r).astype(np.float16)).astype(np.float64)
    rms = np.sqrt(np.mean(np.abs(ref) ** 2))
    excess = np.abs(g - r) - (0.5 * ulp * (1 + 2.0 ** -10) + 1e-5 * rms)
    assert excess.max() <= 0, f"worst excess {excess.max():.3g} at {np.unravel_index(np.argmax(excess), excess.shape)}"
    err = M.rel_l2(from_half(got), ref)
    assert err <= 4e-4
    return err


@pytest.mark.parametrize("n", LENGTHS)
@pytest.mark.parametrize("lines", [1, 37])
def test_range_compression_f16_every_length(torch_dev, rdf, n, lines):
    """binary16 storage, every built length: each output is the float64 result rounded to
    binary16; in place bit-identical to out of place."""
    torch = torch_dev
    rng = np.random.default_rng(3000 + n + lines)
    fs = 120e6
    params = dict(Na=lines, Nr=n, pulse_s=(n // 3) / fs, bandwidth_hz=90e6, fs_hz=fs,
                  range_window=int(n % 3 == 0))
    echo = to_half(rng.standard_normal((lines, n)) + 1j * rng.standard_normal((lines, n)))
    log(f"[range f16] n={n} lines={lines}")
    with rdf.Plan(**params) as plan:
        x = torch.from_numpy(echo).to("cuda")
        rc = plan.range_compress_f16(x).cpu().numpy()
        plan.range_compress_f16(x, out=x)
        torch.cuda.synchronize()
        assert np.array_equal(x.cpu().numpy().view(np.uint16), rc.view(np.uint16))
    err = check_half(rc, O.range_compress(from_half(echo), params))
    log(f"[range f16] n={n} lines={lines} rel-L2 {err:.2e}")


def test_range_compression_f16_workload(torch_dev, rdf):
    """The 4096 x 4096 range-compression scene stored in binary16, against the oracle on the
    same binary16 input; target peaks where the float64 result has them."""
    torch = torch_dev
    cfg = C2
    sc = make_scene(cfg)
    echo = to_half(sc.echo)
    with rdf.Plan(**cfg.plan_params()) as plan:
        rc = plan.range_compress_f16(torch.from_numpy(echo).to("cuda")).cpu().numpy()
    ref = O.range_compress(from_half(echo), cfg.plan_params())
    err = check_half(rc, ref)
    log(f"[range f16] 4096 x 4096 rel-L2 {err:.2e}")
    got = from_half(rc)
    for m in (0, cfg.Na // 2, cfg.Na - 1):
        for (_, n) in sc.targets:
            assert int(np.argmax(np.abs(got[m, n - 4:n + 5]))) == 4 == int(np.argmax(np.abs(ref[m, n - 4:n + 5])))


@pytest.mark.parametrize("n,L", [(1, 1), (1200, 400), (1201, 1201), (5000, 1666), (8191, 2730)],
                         ids=lambda v: str(v))
def test_range_compression_f16_any_length(torch_dev, rdf, n, L):
    """binary16 storage at line lengths with no built transform (the padded form)."""
    torch = torch_dev
    rng = np.random.default_rng(5000 + n)
    fs = 120e6
    params = dict(Na=37, Nr=n, pulse_s=L / fs, bandwidth_hz=90e6, fs_hz=fs, range_window=1)
    echo = to_half(rng.standard_normal((37, n)) + 1j * rng.standard_normal((37, n)))
    with rdf.Plan(**params) as plan:
        x = torch.from_numpy(echo).to("cuda")
        rc = plan.range_compress_f16(x).cpu().numpy()
        plan.range_compress_f16(x, out=x)
        torch.cuda.synchronize()
        assert np.array_equal(x.cpu().numpy().view(np.uint16), rc.view(np.uint16))
    err = check_half(rc, O.range_compress(from_half(echo), params))
    log(f"[range f16] any length n={n} L={L} rel-L2 {err:.2e}")


def test_range_compression_f16_error_paths(torch_dev, rdf):
    torch = torch_dev
    with rdf.Plan(Na=4, Nr=256, pulse_s=100 / 120e6, bandwidth_hz=100e6, fs_hz=120e6) as plan:
        x = torch.zeros((4, 256, 2), dtype=torch.float16, device="cuda")
        with pytest.raises(rdf.RdError) as ei:
            rdf.rd_range_compress_f16(plan.handle, x.data_ptr() + 2, x)
        assert ei.value.status == -1
        with pytest.raises(rdf.RdError) as ei:      # partial overlap
            rdf.rd_range_compress_f16(plan.handle, x, x.data_ptr() + 4)
        assert ei.value.status == -1


def test_range_compression_random_sweep(torch_dev, rdf):
    """40 seeded random cases: line length 1..8192 (built or not), replica length 1..n, 1..40
    lines, either window, float32 or binary16 storage; each against the oracle on the same
    input."""
    torch = torch_dev
    rng = np.random.default_rng(4242)
    fs = 120e6
    for case in range(40):
        n = int(rng.choice([int(rng.integers(1, 8193)), int(rng.choice(LENGTHS[:-2] + (6000,)))]))
        L = int(rng.integers(1, n + 1))
        lines = int(rng.integers(1, 41))
        params = dict(Na=lines, Nr=n, pulse_s=L / fs, bandwidth_hz=float(rng.uniform(20e6, 110e6)), fs_hz=fs,
                      range_window=int(rng.integers(0, 2)))
        assert O.replica_length(params) == L
        half = rng.random() < 0.3
        x = rng.standard_normal((lines, n)) + 1j * rng.standard_normal((lines, n))
        log(f"[sweep] case {case}: n={n} L={L} lines={lines} window={params['range_window']} half={half}")
        with rdf.Plan(**params) as plan:
            if half:
                e16 = to_half(x)
                got = plan.range_compress_f16(torch.from_numpy(e16).to("cuda")).cpu().numpy()
                check_half(got, O.range_compress(from_half(e16), params))
            else:
                x64 = x.astype(np.complex64)
                got = plan.range_compress(dev(torch, x64)).cpu().numpy()
                check_stage(f"[sweep] case {case}", got, O.range_compress(x64, params), STAGE_TOL)


def test_range_compression_table_variant(torch_dev, rdf, monkeypatch):
    """The table-twiddle kernel (selected by RD_RC_VARIANT=table) meets the same bar."""
    torch = torch_dev
    cfg = C2.with_(Na=300)
    sc = make_scene(cfg)
    monkeypatch.setenv("RD_RC_VARIANT", "table")
    with rdf.Plan(**cfg.plan_params()) as plan:
        rc = plan.range_compress(dev(torch, sc.echo)).cpu().numpy()
    check_stage("[range] table variant", rc, O.range_compress(sc.echo, cfg.plan_params()), STAGE_TOL)


def test_range_compression_large_sampled_lines(torch_dev, rdf):
    torch = torch_dev
    cfg = C5
    log("[range] 16384 x 16384 scene: generating echo")
    sc = cached_scene(cfg)
    rows = np.array([0, 1, 777, 8191, 8192, 12345, 16382, 16383])
    with rdf.Plan(**cfg.plan_params()) as plan:
        echo = dev(torch, sc.echo)
        rc = plan.range_compress(echo)
        got = rc[torch.from_numpy(rows).to("cuda")].cpu().numpy()
        del rc, echo
    ref = O.range_compress(sc.echo[rows], cfg.plan_params())
    check_stage("[range] 16384 sampled lines", got, ref, STAGE_TOL)
    torch.cuda.empty_cache()


# ------------------------------------------------------------------------------ full chain
def check_targets(img, ref_img, targets, axes=("range", "azimuth")):
    for (m, n) in targets:
        pk = M.peak_near(img, m, n)
        assert pk == M.peak_near(ref_img, m, n), (m, n)
        got, want = M.point_target(img, *pk, axes=axes), M.point_target(ref_img, *pk, axes=axes)
        for axis in axes:
            for key in ("pslr_db", "islr_db"):
                a, b = got[axis][key], want[axis][key]
                if np.isinf(a) and a == b:        # no sidelobe in the window on either side
                    continue
                assert abs(a - b) <= 0.1, (m, n, axis, key)


# 6000-sample rows (the mixed-radix range length) through the float32 chain
RD_6000 = C3.with_(name="rd_512x6000", Na=512, Nr=6000, n_targets=4)


@pytest.mark.parametrize("cfg", [C1, C3, LONG_MIGRATION, RD_1200, RD_3001, RD_800, RD_1000, WK_997, RD_6000],
                         ids=lambda c: c.name)
def test_focus_every_stage(torch_dev, rdf, cfg):
    torch = torch_dev
    sc, ref = scene_and_stages(cfg)
    log(f"[focus] {cfg.name}")
    with rdf.Plan(**cfg.plan_params()) as plan:
        echo = dev(torch, sc.echo)
        rc = plan.range_compress(echo)
        az, rcmc, img_dbg = plan.azimuth_stages(rc)
        img = plan.focus(echo)
        img_az = plan.azimuth_focus(rc)
        torch.cuda.synchronize()
        stages = {"rc": rc.cpu().numpy(), "azfft": az.cpu().numpy(), "rcmc": rcmc.cpu().numpy(),
                  "img": img.cpu().numpy()}
        assert torch.equal(img, img_dbg) and torch.equal(img, img_az)
    for name in ("rc", "azfft", "rcmc"):
        check_stage(f"[focus] {cfg.name} {name}", stages[name], ref[name], STAGE_TOL)
    check_stage(f"[focus] {cfg.name} img", stages["img"], ref["img"], IMAGE_TOL)
    if cfg is not LONG_MIGRATION:  # its azimuth TBP is ~3: peaks are broad, compared via L2 only
        check_targets(stages["img"], ref["img"], sc.targets)


def test_focus_in_place_and_noiseless_targets(torch_dev, rdf):
    torch = torch_dev
    cfg = C3
    sc = make_scene(cfg, noise=False)
    with rdf.Plan(**cfg.plan_params()) as plan:
        echo = dev(torch, sc.echo)
        img = plan.focus(echo)
        plan.focus(echo, out=echo)            # echo == img
        torch.cuda.synchronize()
        assert torch.equal(echo, img)
        gi = img.cpu().numpy()
    for (m, n) in sc.targets:
        assert M.peak_near(gi, m, n) == (m, n)


# Binary16 storage through the whole chain: six stored stages (range compression, two forward
# and two inverse azimuth steps, the row stage; the Bluestein form's workspace stays float32),
# each rounding to nearest with a relative error of at most 2^-11 per component in the normal
# range.  Every later stage is a scaled unitary map (column DFT / L, twiddles, phase-only
# filter) or the normalised interpolator, so the errors add at most linearly:
# rel-L2 <= 6 * 2^-11 = 2.9e-3.  The oracle takes the same binary16 echo.
F16_CHAIN_TOL = 3e-3


def check_targets_near(img, ref_img, targets, rel):
    """Target peaks of an image whose stored values carry a relative error up to `rel`: where
    the oracle's peak is flat (neighbours within `rel` of its maximum), any of those pixels is a
    correct argmax, so the image's peak must be a pixel whose oracle magnitude is within `rel` of
    the oracle's maximum.  PSLR is compared at the oracle's peak.  ISLR is not: its mainlobe ends
    at the first nulls, which are shallow on weakly focused (short-aperture) targets, and an
    error of a few 1e-4 can move the null the measurement picks and with it a large share of
    energy between mainlobe and sidelobes."""
    for (m, n) in targets:
        pk, pr = M.peak_near(img, m, n), M.peak_near(ref_img, m, n)
        assert abs(ref_img[pk]) >= (1 - rel) * abs(ref_img[pr]), (m, n, pk, pr)
        got, want = M.point_target(img, *pr), M.point_target(ref_img, *pr)
        for axis in ("range", "azimuth"):
            a, b = got[axis]["pslr_db"], want[axis]["pslr_db"]
            if not (np.isinf(a) and a == b):
                assert abs(a - b) <= 0.1, (m, n, axis)


@pytest.mark.parametrize("cfg", [C1, C3, LONG_MIGRATION, RD_1200, RD_800, WK_997, RD_6000], ids=lambda c: c.name)
def test_focus_f16(torch_dev, rdf, cfg):
    """rd_focus_f16: the image divided by Na, against the oracle on the binary16 echo; target
    peaks and sidelobe ratios as the oracle's; in place bit-identical to out of place."""
    torch = torch_dev
    sc = make_scene(cfg)
    echo = to_half(sc.echo)
    log(f"[focus f16] {cfg.name}")
    with rdf.Plan(**cfg.plan_params()) as plan:
        x = torch.from_numpy(echo).to("cuda")
        img = plan.focus_f16(x).cpu().numpy()
        plan.focus_f16(x, out=x)
        torch.cuda.synchronize()
        assert np.array_equal(x.cpu().numpy().view(np.uint16), img.view(np.uint16))
    assert np.isfinite(img.astype(np.float32)).all()
    log(f"[oracle] {cfg.name}: focusing the binary16 echo on the CPU")
    ref = O.focus(from_half(echo), cfg.plan_params()) / cfg.Na
    got = from_half(img)
    check_stage(f"[focus f16] {cfg.name} img", got, ref, F16_CHAIN_TOL)
    if cfg is not LONG_MIGRATION:
        check_targets_near(got, ref, sc.targets, F16_CHAIN_TOL)


def test_focus_f16_error_paths(torch_dev, rdf):
    torch = torch_dev
    x = torch.zeros((4, 256, 2), dtype=torch.float16, device="cuda")
    with rdf.Plan(Na=4, Nr=256, pulse_s=100 / 120e6, bandwidth_hz=100e6, fs_hz=120e6) as plan:
        with pytest.raises(rdf.RdError) as ei:      # range-only plan
            plan.focus_f16(x)
        assert ei.value.status == -6
    with rdf.Plan(**C1.plan_params()) as plan:
        y = torch.zeros((C1.Na, C1.Nr, 2), dtype=torch.float16, device="cuda")
        for a, b in ((y.data_ptr() + 2, y), (y, y.data_ptr() + 4)):   # misaligned; partial overlap
            with pytest.raises(rdf.RdError) as ei:
                rdf.rd_focus_f16(plan.handle, a, b)
            assert ei.value.status == -1
    # 512-sample rows: the migration (~77 samples) exceeds the RCMC margin built for that length
    with rdf.Plan(**C3.with_(Nr=512, pulse_s=1e-6).plan_params()) as plan:
        z = torch.zeros((C3.Na, 512, 2), dtype=torch.float16, device="cuda")
        with pytest.raises(rdf.RdError) as ei:
            plan.focus_f16(z)
        assert ei.value.status == -2
    torch.cuda.synchronize()


@pytest.mark.parametrize("cfg", [C1, C3, RD_1200, WK_997], ids=lambda c: c.name)
def test_azimuth_focus_f16(torch_dev, rdf, cfg):
    """rd_azimuth_focus_f16 on binary16 range-compressed data (the oracle's, rounded) against the
    oracle's azimuth half of the same data, divided by Na (five stored stages, within the
    six-stage bound); rd_focus_f16 equals rd_range_compress_f16 followed by it, bit for bit."""
    torch = torch_dev
    sc = make_scene(cfg)
    p = cfg.plan_params()
    rc16 = to_half(O.range_compress(sc.echo, p))
    with rdf.Plan(**p) as plan:
        img = plan.azimuth_focus_f16(torch.from_numpy(rc16).to("cuda")).cpu().numpy()
        x = torch.from_numpy(to_half(sc.echo)).to("cuda")
        a = plan.focus_f16(x)
        b = plan.azimuth_focus_f16(plan.range_compress_f16(x))
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    ref = O.azimuth_focus(from_half(rc16), p) / cfg.Na
    check_stage(f"[azimuth f16] {cfg.name}", from_half(img), ref, F16_CHAIN_TOL)


def test_focus_random_sweep(torch_dev, rdf):
    """12 seeded random scenes on the 4096 x 4096 scene's platform (1 us pulse): azimuth lengths
    that are powers of two, 25 * 2^k, or anything else in [200, 1100] (the Bluestein form), and
    range lengths in [700, 2048] (built or padded); each through rd_focus and rd_focus_f16
    against the oracle on the same input, with every target's peak a valid argmax."""
    torch = torch_dev
    rng = np.random.default_rng(777)
    for i in range(12):
        kind = i % 3
        na = int(rng.choice([256, 512, 1024])) if kind == 0 else (
            int(rng.choice([400, 800])) if kind == 1 else int(rng.integers(200, 1101)))
        nr = int(rng.choice([1024, 2048])) if i % 4 == 0 else int(rng.integers(700, 2049))
        cfg = C3.with_(name=f"sweep_{i}_{na}x{nr}", Na=na, Nr=nr, pulse_s=1e-6, n_targets=2, seed=300 + i)
        sc = make_scene(cfg)
        e16 = to_half(sc.echo)
        log(f"[focus sweep] {cfg.name}")
        with rdf.Plan(**cfg.plan_params()) as plan:
            img = plan.focus(dev(torch, sc.echo)).cpu().numpy()
            h = from_half(plan.focus_f16(torch.from_numpy(e16).to("cuda")).cpu().numpy())
        ref = O.focus(sc.echo, cfg.plan_params())
        ref16 = O.focus(from_half(e16), cfg.plan_params()) / na
        check_stage(f"[focus sweep] {cfg.name} float32", img, ref, IMAGE_TOL)
        check_stage(f"[focus sweep] {cfg.name} binary16", h, ref16, F16_CHAIN_TOL)
        for got, want, rel in ((img, ref, IMAGE_TOL), (h, ref16, F16_CHAIN_TOL)):
            for (m, n) in sc.targets:
                pk, pr = M.peak_near(got, m, n), M.peak_near(want, m, n)
                assert abs(want[pk]) >= (1 - rel) * abs(want[pr]), (cfg.name, m, n, pk, pr)


def test_focus_large_every_stage_sampled(torch_dev, rdf):
    """The 16384 x 16384 scene through the stage hook (range compression, azimuth spectrum, RCMC,
    image) against the oracle at sampled range bins over all 16384 pulses / Doppler bins: both
    sides of every RCMC chunk seam (4096-sample chunks: every bin within 8 of a seam, every
    second bin over the reach of the halo before it), the row edges, and two targets'
    neighbourhoods wide enough for range and azimuth cuts.  Each stage meets its bar per row and
    per column; the targets' peaks, PSLR and ISLR along both axes are the oracle's."""
    torch = torch_dev
    cfg = C5
    log("[focus 16384] echo")
    sc = cached_scene(cfg)
    p = cfg.plan_params()
    halo = int(np.floor(O.rcmc_shift(p, [cfg.Nr - 1]).max())) + 5
    tg = sorted(sc.targets, key=lambda t: t[1])
    picks = (tg[0], tg[len(tg) // 2])
    bins = set(range(4)) | set(range(cfg.Nr - 4, cfg.Nr))
    for c in range(4096, cfg.Nr, 4096):
        bins.update(range(c - halo - 4, c - 8, 2))
        bins.update(range(c - 8, c + 8))
    for (_, n) in picks:
        bins.update(range(n - 40, n + 41))
    bins = sorted(bins)
    log(f"[focus 16384] {len(bins)} range bins, halo {halo}")
    idx = torch.tensor(bins, device="cuda")
    with rdf.Plan(**p) as plan:
        echo = dev(torch, sc.echo)
        rc = plan.range_compress(echo)
        del echo
        az, rcmc, img = plan.azimuth_stages(rc)
        torch.cuda.synchronize()
        got = {name: t[:, idx].cpu().numpy() for name, t in (("rc", rc), ("azfft", az), ("rcmc", rcmc), ("img", img))}
        del rc, az, rcmc, img
    torch.cuda.empty_cache()
    log("[focus 16384] oracle on the sampled range bins")
    ref, ref_bins = O.focus_columns(sc.echo, p, bins, stages=True)
    assert list(ref_bins) == bins
    for name in ("rc", "azfft", "rcmc"):
        check_stage(f"[focus 16384] {name}", got[name], ref[name], STAGE_TOL)
    check_stage("[focus 16384] img", got["img"], ref["img"], IMAGE_TOL)
    col = {b: i for i, b in enumerate(bins)}
    for (m, n) in picks:
        sel = [col[b] for b in range(n - 40, n + 41)]
        sub_g, sub_r = got["img"][:, sel], ref["img"][:, sel]
        assert M.peak_near(sub_g, m, 40) == M.peak_near(sub_r, m, 40) == (m, 40)
        a, b = M.point_target(sub_g, m, 40), M.point_target(sub_r, m, 40)
        for axis in ("range", "azimuth"):
            for key in ("pslr_db", "islr_db"):
                log(f"[focus 16384] target ({m}, {n}) {axis} {key}: {a[axis][key]:.3f} vs {b[axis][key]:.3f}")
                assert abs(a[axis][key] - b[axis][key]) <= 0.1, (m, n, axis, key)


# Row-stage geometries whose rows are processed in chunks: 8192-sample rows with ~540 samples of
# migration (2 chunks of 4096, a halo longer than one pass of the threads), 16384-sample rows of
# the 16384 x 16384 geometry (4 chunks), and rows of run-time length (512-sample chunks, ragged
# last chunk).  More rows than one residency wave of the GPU, so chunks of one row would run in
# different waves if they were independent work items.
RCMC_CHUNKED = [
    LONG_MIGRATION.with_(name="rcmc_16384x8192_long_migration", Na=16384),
    C5.with_(name="rcmc_4096x16384", Na=4096),
    RD_1200.with_(name="rcmc_16384x1200", Na=16384),
    RD_3001.with_(name="rcmc_4096x3001_large_migration", Na=4096),
]


@pytest.mark.parametrize("cfg", RCMC_CHUNKED, ids=lambda c: c.name)
def test_rcmc_stage_in_place_equals_out_of_place(torch_dev, rdf, cfg):
    """The row stage (RCMC + azimuth filter) runs in place in the chain.  On chunked rows it must
    give the same bits in place as out of place (and on a repeat), and match the oracle's RCMC
    and filter on sampled Doppler rows, including every chunk seam: the error of each window
    around a seam (the outputs whose taps reach across it) is held to the stage bar on its own."""
    torch = torch_dev
    p = cfg.plan_params()
    gen = torch.Generator(device="cuda").manual_seed(cfg.seed)
    x = torch.randn((cfg.Na, cfg.Nr), dtype=torch.complex64, device="cuda", generator=gen)
    log(f"[rcmc] {cfg.name}")
    with rdf.Plan(**p) as plan:
        y = plan.rcmc_stage(x)
        y2 = plan.rcmc_stage(x)
        z = x.clone()
        plan.rcmc_stage(z, out=z)
        torch.cuda.synchronize()
        assert torch.equal(y, y2), "row stage is not deterministic"
        assert torch.equal(y, z), "in place differs from out of place"
        rows = np.unique(np.r_[0, 1, cfg.Na // 4, cfg.Na // 2 - 1, cfg.Na // 2, cfg.Na // 2 + 1, cfg.Na - 1])
        ri = torch.from_numpy(rows).to("cuda")
        got, xin = y[ri].cpu().numpy(), x[ri].cpu().numpy()
    n = np.arange(cfg.Nr)
    shift = O.rcmc_shift(p, n, rows)
    want = O.rcmc(xin.astype(np.complex128), shift, p["rcmc_taps"], p["kaiser_beta"])
    want = want * O.azimuth_matched_filter(p, n, rows) / cfg.Na
    check_stage(f"[rcmc] {cfg.name} sampled rows", got, want, STAGE_TOL)
    chunk = 4096 if cfg.Nr in (8192, 16384) else 512
    reach = int(np.ceil(shift.max())) + 8
    rms = np.sqrt(np.mean(np.abs(want) ** 2, axis=1))
    for c in range(chunk, cfg.Nr, chunk):
        lo, hi = max(0, c - reach), min(cfg.Nr, c + 8)
        e = np.sqrt(np.mean(np.abs(got[:, lo:hi] - want[:, lo:hi]) ** 2, axis=1)) / rms
        assert e.max() <= STAGE_TOL, (cfg.name, c, e.max())
    log(f"[rcmc] {cfg.name}: in place == out of place, seams within the stage bar")


def test_focus_f16_large_sampled_range_bins(torch_dev, rdf):
    """rd_focus_f16 on the 16384 x 16384 scene (128-point column steps, chunked rows), against
    the oracle on the binary16 echo at sampled range bins."""
    torch = torch_dev
    cfg = C5
    log("[focus f16] 16384 x 16384: echo")
    sc = cached_scene(cfg)
    tg = sorted(sc.targets, key=lambda t: t[1])
    bins = sorted(set(range(tg[1][1] - 16, tg[1][1] + 17)) | {0, cfg.Nr // 3, cfg.Nr - 1})
    echo = to_half(sc.echo)
    with rdf.Plan(**cfg.plan_params()) as plan:
        x = torch.from_numpy(echo).to("cuda")
        plan.focus_f16(x, out=x)
        torch.cuda.synchronize()
        got = from_half(x[:, torch.tensor(bins, device="cuda")].cpu().numpy())
        del x
    torch.cuda.empty_cache()
    log("[focus f16] 16384 x 16384: oracle on sampled range bins")
    ref, ref_bins = O.focus_columns(from_half(echo), cfg.plan_params(), bins)
    del echo
    assert list(ref_bins) == bins
    ref = ref / cfg.Na
    err = M.rel_l2(got, ref)
    log(f"[focus f16] 16384 sampled rel-L2 {err:.2e}")
    assert err <= F16_CHAIN_TOL
    m, n = tg[1]
    col = {b: i for i, b in enumerate(bins)}
    sub_g = got[:, [col[b] for b in range(n - 16, n + 17)]]
    sub_r = ref[:, [col[b] for b in range(n - 16, n + 17)]]
    pk, pr = M.peak_near(sub_g, m, 16), M.peak_near(sub_r, m, 16)
    assert pr == (m, 16) and abs(sub_r[pk]) >= (1 - F16_CHAIN_TOL) * abs(sub_r[pr])


# ------------------------------------------------------------------------------ omega-k
# the large-migration L-band geometry (Stolt shifts up to 226 bins of 1024), a short-pulse
# version of the 4096-pulse airborne geometry, and 6000-sample rows (mixed radix)
WK_BIG = SceneConfig(name="wk_large_migration_4096x1024", Na=4096, Nr=1024, pulse_s=2e-6,
                     bandwidth_hz=100e6, fs_hz=120e6, window="rect", n_targets=2, noise_power=0.0,
                     seed=11, carrier_hz=1.0e9, prf_hz=600.0, velocity_mps=200.0, r_ref_m=3000.0,
                     sep_range=9, sep_az=100)
WK_C3AZ = C3.with_(name="wk_4096x512", Nr=512, pulse_s=1e-6, n_targets=3, noise_power=0.01)
WK_6000 = C3.with_(name="wk_512x6000", Na=512, Nr=6000, n_targets=4)
# 16384-sample rows on the 16384 x 16384 scene's platform, few enough pulses for the oracle
WK_16K = C5.with_(name="wk_256x16384", Na=256, n_targets=3)
# 2048- and 8192-sample rows on the 4096 x 4096 scene's platform
WK_2K = C3.with_(name="wk_256x2048", Na=256, Nr=2048, n_targets=3)
WK_8K = C3.with_(name="wk_256x8192", Na=256, Nr=8192, n_targets=3)
# 256 pulses of platforms whose apertures span thousands: the azimuth response is wider than the
# metric window, so only the peak and the range cut are compared there
SHORT_APERTURE = (WK_16K, WK_2K, WK_8K)


def wk_ref_bin(cfg) -> int:
    return int(round((cfg.r_ref_m - cfg.range_bin0_m) / cfg.dr))


@pytest.mark.parametrize("cfg", [C1, WK_BIG, WK_C3AZ, WK_6000, WK_800, WK_997, WK_2K, WK_8K, WK_16K],
                         ids=lambda c: c.name)
def test_omega_k_matches_oracle(torch_dev, rdf, cfg):
    """rd_omega_k against the oracle at the scene's reference bin and at bin 0; in place gives
    the same bits; targets at the oracle's pixels with the same PSLR / ISLR."""
    torch = torch_dev
    sc = make_scene(cfg)
    p = cfg.plan_params()
    with rdf.Plan(**p) as plan:
        for ref in (wk_ref_bin(cfg), 0):
            log(f"[omega-k] {cfg.name} ref_bin={ref}")
            echo = dev(torch, sc.echo)
            img = plan.omega_k(echo, ref)
            plan.omega_k(echo, ref, out=echo)
            torch.cuda.synchronize()
            assert torch.equal(img, echo)
            got = img.cpu().numpy()
            want = O.omega_k(sc.echo, p, ref)
            check_stage(f"[omega-k] {cfg.name} ref_bin={ref}", got, want, IMAGE_TOL)
            if ref == wk_ref_bin(cfg):
                check_targets(got, want, sc.targets,
                              axes=("range",) if cfg in SHORT_APERTURE else ("range", "azimuth"))


def test_omega_k_full_airborne_scene(torch_dev, rdf):
    """The 4096 x 4096 airborne scene (16 targets) against the oracle."""
    torch = torch_dev
    cfg = C3
    sc = cached_scene(cfg)
    ref = wk_ref_bin(cfg)
    with rdf.Plan(**cfg.plan_params()) as plan:
        got = plan.omega_k(dev(torch, sc.echo), ref).cpu().numpy()
    log("[omega-k] 4096 x 4096: oracle")
    want = O.omega_k(sc.echo, cfg.plan_params(), ref)
    check_stage("[omega-k] 4096 x 4096", got, want, IMAGE_TOL)
    check_targets(got, want, sc.targets)


def test_omega_k_16384_properties(torch_dev, rdf):
    """16384 x 16384 (no whole-image oracle: the mapping is global in range frequency):
    every target peaks at its predicted pixel, and delaying the echo by s pulses delays the
    image by s rows (the azimuth processing is circular and shift-invariant)."""
    torch = torch_dev
    cfg = C5
    log("[omega-k] 16384 x 16384: echo")
    sc = cached_scene(cfg)
    ref = wk_ref_bin(cfg)
    s = 777
    with rdf.Plan(**cfg.plan_params()) as plan:
        echo = dev(torch, sc.echo)
        img = plan.omega_k(echo, ref)
        echo = torch.roll(echo, s, dims=0)
        img2 = plan.omega_k(echo, ref)
        del echo
        d = torch.roll(img, s, dims=0) - img2
        err = float(torch.linalg.vector_norm(d) / torch.linalg.vector_norm(img2))
        del d, img2
        for (m, n) in sc.targets:
            win = img[m - 16:m + 17, n - 16:n + 17].abs().cpu().numpy()
            k = np.unravel_index(int(np.argmax(win)), win.shape)
            assert (k[0] - 16, k[1] - 16) == (0, 0), (m, n, k)
        del img
    torch.cuda.empty_cache()
    log(f"[omega-k] 16384 shift equivariance rel-L2 {err:.2e}")
    assert err <= 1e-5


def test_omega_k_error_paths(torch_dev, rdf):
    torch = torch_dev
    with rdf.Plan(**C2.with_(Na=256).plan_params()) as plan:   # range only
        x = torch.zeros((256, C2.Nr), dtype=torch.complex64, device="cuda")
        with pytest.raises(rdf.RdError) as ei:
            plan.omega_k(x, 0)
        assert ei.value.status == -6
    with rdf.Plan(**C1.plan_params()) as plan:
        x = torch.zeros((C1.Na, C1.Nr), dtype=torch.complex64, device="cuda")
        for ref in (-1, C1.Nr):
            with pytest.raises(rdf.RdError) as ei:
                plan.omega_k(x, ref)
            assert ei.value.status == -1
        with pytest.raises(rdf.RdError) as ei:   # partial overlap
            rdf.rd_omega_k(plan.handle, x, x.data_ptr() + 8, 0)
        assert ei.value.status == -1
    with rdf.Plan(**WK_C3AZ.plan_params()) as plan:   # RD migration beyond the RCMC margin
        x = torch.zeros((WK_C3AZ.Na, WK_C3AZ.Nr), dtype=torch.complex64, device="cuda")
        for call in (plan.focus, plan.azimuth_focus):
            with pytest.raises(rdf.RdError) as ei:
                call(x)
            assert ei.value.status == -2
        plan.omega_k(x, 0)                              # the same plan still serves omega-k
    with rdf.Plan(**RD_1200.plan_params()) as plan:   # no built range transform
        x = torch.zeros((RD_1200.Na, RD_1200.Nr), dtype=torch.complex64, device="cuda")
        with pytest.raises(rdf.RdError) as ei:
            plan.omega_k(x, 0)
        assert ei.value.status == -2
    with rdf.Plan(**LONG_MIGRATION.plan_params()) as plan:   # Stolt shift beyond the staged margin
        x = torch.zeros((LONG_MIGRATION.Na, LONG_MIGRATION.Nr), dtype=torch.complex64, device="cuda")
        with pytest.raises(rdf.RdError) as ei:
            plan.omega_k(x, 0)
        assert ei.value.status == -2


@pytest.mark.parametrize("cfg", [C1, C3, WK_C3AZ, WK_6000, WK_800, WK_997, WK_2K, WK_8K, WK_16K],
                         ids=lambda c: c.name)
def test_omega_k_f16(torch_dev, rdf, cfg):
    """rd_omega_k_f16: the image divided by Na against the oracle on the same binary16 echo
    (five stored stages: two forward azimuth steps, the row stage, two inverse steps; within the
    six-stage bound), target peaks valid; in place bit-identical to out of place."""
    torch = torch_dev
    sc = make_scene(cfg)
    rb = wk_ref_bin(cfg)
    e16 = to_half(sc.echo)
    log(f"[omega-k f16] {cfg.name}")
    with rdf.Plan(**cfg.plan_params()) as plan:
        x = torch.from_numpy(e16).to("cuda")
        img = plan.omega_k_f16(x, rb).cpu().numpy()
        plan.omega_k_f16(x, rb, out=x)
        torch.cuda.synchronize()
        assert np.array_equal(x.cpu().numpy().view(np.uint16), img.view(np.uint16))
        with pytest.raises(rdf.RdError) as ei:      # misaligned
            rdf.rd_omega_k_f16(plan.handle, x.data_ptr() + 2, x, rb)
        assert ei.value.status == -1
    ref = O.omega_k(from_half(e16), cfg.plan_params(), rb) / cfg.Na
    got = from_half(img)
    check_stage(f"[omega-k f16] {cfg.name}", got, ref, F16_CHAIN_TOL)
    for (m, n) in sc.targets:
        pk, pr = M.peak_near(got, m, n), M.peak_near(ref, m, n)
        assert abs(ref[pk]) >= (1 - F16_CHAIN_TOL) * abs(ref[pr]), (m, n, pk, pr)


# ------------------------------------------------------------------------------ corner turn
@pytest.mark.parametrize("rows,cols", [(256, 256), (4096, 4096), (37, 1000), (1, 5), (5, 1),
                                       (65, 63), (8192, 6000), (64, 16384)])
def test_corner_turn_bit_exact(torch_dev, rdf, rows, cols):
    """rd_corner_turn equals the oracle's transpose bit for bit (full tiles, ragged edges, a
    single row or column, and an array above the non-temporal threshold); two turns restore."""
    torch = torch_dev
    rng = np.random.default_rng(rows * 7919 + cols)
    x = (rng.standard_normal((rows, cols)) + 1j * rng.standard_normal((rows, cols))).astype(np.complex64)
    log(f"[corner turn] {rows} x {cols}")
    xd = dev(torch, x)
    y = rdf.corner_turn(xd)
    z = rdf.corner_turn(y)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy(), O.corner_turn(x))
    assert torch.equal(z, xd)


def test_corner_turn_of_range_compressed_scene(torch_dev, rdf):
    """The azimuth-major layout of the 256 x 256 scene's range-compressed data: turned on the
    GPU equals the oracle's range compression turned on the CPU, to the stage tolerance."""
    torch = torch_dev
    sc, ref = scene_and_stages(C1)
    with rdf.Plan(**C1.plan_params()) as plan:
        rc = plan.range_compress(dev(torch, sc.echo))
        t = rdf.corner_turn(rc).cpu().numpy()
    assert M.rel_l2(t, O.corner_turn(ref["rc"])) <= STAGE_TOL


# ------------------------------------------------------------------------------ back-projection
BP_TOL = 1e-5


def focus_grid(cfg, m_lo, n_lo, nx, ny):
    """The focusing image's own grid: one row per pulse position, one column per range bin."""
    p = cfg.plan_params()
    return dict(nx=nx, ny=ny, x0_m=cfg.velocity_mps * m_lo / cfg.prf_hz, dx_m=cfg.velocity_mps / cfg.prf_hz,
                r0_m=p["range_bin0_m"] + n_lo * O.range_spacing(p), dr_m=O.range_spacing(p))


@pytest.mark.parametrize("variant", ["native", "accurate"])
def test_backproject_small_grids(torch_dev, rdf, monkeypatch, variant):
    """Whole 256 x 256 scene on its focusing grid, and a ragged grid partly outside the swath:
    the same complex64 range-compressed input on both sides, the kernel against the oracle."""
    torch = torch_dev
    if variant == "accurate":
        monkeypatch.setenv("RD_BP_SINCOS", "accurate")
    sc, ref = scene_and_stages(C1)
    rc = ref["rc"].astype(np.complex64)
    p = C1.plan_params()
    dr = O.range_spacing(p)
    grids = [focus_grid(C1, 0, 0, 256, 256),
             dict(nx=37, ny=50, x0_m=-3.1, dx_m=0.37, r0_m=p["range_bin0_m"] - 20.3 * dr, dr_m=5.9 * dr)]
    with rdf.Plan(**p) as plan:
        rcd = dev(torch, rc)
        for g in grids:
            log(f"[bp] {variant} grid {g['nx']}x{g['ny']}")
            got = plan.backproject(rcd, g).cpu().numpy()
            want = O.backproject(rc, p, g)
            err = M.rel_l2(got, want)
            log(f"[bp] {variant} {g['nx']}x{g['ny']} rel-L2 {err:.2e}")
            assert err <= BP_TOL
    img = O.backproject(rc, p, grids[0])
    gimg = None
    with rdf.Plan(**p) as plan:
        gimg = plan.backproject(dev(torch, rc), grids[0]).cpu().numpy()
    for (m, n) in sc.targets:
        assert M.peak_near(gimg, m, n) == M.peak_near(img, m, n)


def test_backproject_any_line_length(torch_dev, rdf):
    """Back-projection on a plan whose line length (1200) has no built transform, on 64 x 64
    grids around two targets: the same complex64 range-compressed input on both sides."""
    torch = torch_dev
    cfg = RD_1200
    sc, ref = scene_and_stages(cfg)
    rc = ref["rc"].astype(np.complex64)
    p = cfg.plan_params()
    with rdf.Plan(**p) as plan:
        rcd = dev(torch, rc)
        for (m, n) in sc.targets[:2]:
            g = focus_grid(cfg, m - 32, n - 32, 64, 64)
            got = plan.backproject(rcd, g).cpu().numpy()
            want = O.backproject(rc, p, g)
            err = M.rel_l2(got, want)
            log(f"[bp] {cfg.name} around ({m}, {n}) rel-L2 {err:.2e}")
            assert err <= BP_TOL
            assert M.peak_near(got, 32, 32) == M.peak_near(want, 32, 32)


def test_backproject_large_grid_sampled(torch_dev, rdf):
    """4096 pulses onto a 1024 x 1024 grid of the 4096 x 4096 airborne scene (the workload the
    bench times): sampled pixels against the oracle computed pixel by pixel, and every target in
    the grid peaks where the oracle's 9 x 9 neighbourhood image peaks."""
    torch = torch_dev
    cfg = C3
    sc, ref = scene_and_stages(cfg)
    rc = ref["rc"].astype(np.complex64)
    p = cfg.plan_params()
    m_lo, n_lo = cfg.Na // 2 - 512, cfg.Nr // 2 - 512
    g = focus_grid(cfg, m_lo, n_lo, 1024, 1024)
    with rdf.Plan(**p) as plan:
        log("[bp] 4096 pulses -> 1024 x 1024")
        img = plan.backproject(dev(torch, rc), g).cpu().numpy()
    rng = np.random.default_rng(5)
    pix = [(int(a), int(b)) for a, b in zip(rng.integers(0, 1024, 48), rng.integers(0, 1024, 48))]
    inside = [(m - m_lo, n - n_lo) for (m, n) in sc.targets if 4 <= m - m_lo < 1020 and 4 <= n - n_lo < 1020]
    pix += inside
    want = O.backproject_pixels(rc, p, g, pix)
    got = np.array([img[i, j] for (i, j) in pix])
    err = M.rel_l2(got, want)
    log(f"[bp] sampled {len(pix)} pixels rel-L2 {err:.2e} ({len(inside)} targets inside)")
    assert err <= BP_TOL
    for (i, j) in inside:
        sub = dict(g, nx=9, ny=9, x0_m=g["x0_m"] + (i - 4) * g["dx_m"], r0_m=g["r0_m"] + (j - 4) * g["dr_m"])
        w = O.backproject(rc, p, sub)
        assert np.unravel_index(np.argmax(np.abs(w)), w.shape) == (4, 4)
        assert M.peak_near(img, i, j) == (i, j)


def test_backproject_error_paths(torch_dev, rdf):
    torch = torch_dev
    g = dict(nx=8, ny=8, x0_m=0.0, dx_m=0.1, r0_m=5000.0, dr_m=1.0)
    with rdf.Plan(**C2.with_(Na=256, Nr=4096).plan_params()) as plan:
        x = torch.zeros((256, 4096), dtype=torch.complex64, device="cuda")
        with pytest.raises(rdf.RdError) as ei:
            plan.backproject(x, g)
        assert ei.value.status == -6
    with rdf.Plan(**C1.plan_params()) as plan:
        x = torch.zeros((256, 256), dtype=torch.complex64, device="cuda")
        with pytest.raises(rdf.RdError) as ei:      # image overlapping the input
            rdf.rd_backproject(plan.handle, x, x.data_ptr() + 8 * 64, g)
        assert ei.value.status == -1
        with pytest.raises(rdf.RdError) as ei:
            rdf.rd_backproject(plan.handle, x, torch.empty((8, 8), dtype=torch.complex64, device="cuda"),
                               dict(g, r0_m=-1.0))
        assert ei.value.status == -1
        rdf.rd_backproject(plan.handle, x, torch.empty((1,), dtype=torch.complex64, device="cuda"), dict(g, nx=0))


# ------------------------------------------------------------------------------ error paths
def test_error_paths_on_device(torch_dev, rdf):
    torch = torch_dev
    with rdf.Plan(**C2.with_(Na=256, Nr=4096).plan_params()) as plan:
        x = torch.zeros((256, 4096), dtype=torch.complex64, device="cuda")
        with pytest.raises(rdf.RdError) as ei:
            plan.focus(x)
        assert ei.value.status == -6
        with pytest.raises(rdf.RdError) as ei:
            rdf.rd_range_compress(plan.handle, x.data_ptr() + 4, x)
        assert ei.value.status == -1
        with pytest.raises(rdf.RdError) as ei:   # partial overlap
            rdf.rd_range_compress(plan.handle, x, x.data_ptr() + 8)
        assert ei.value.status == -1
        # the binding checks tensors before their addresses reach the library
        small = torch.zeros((255, 4096), dtype=torch.complex64, device="cuda")
        for bad, what in ((small, "samples"), (x.to(torch.complex128), "complex64"),
                          (x.t(), "contiguous"), (x.cpu(), "GPU tensor")):
            with pytest.raises(ValueError, match=what):
                rdf.rd_range_compress(plan.handle, x, bad)
            with pytest.raises(ValueError, match=what):
                rdf.rd_range_compress(plan.handle, bad, x)
        h16 = torch.zeros((256, 4096, 2), dtype=torch.float16, device="cuda")
        with pytest.raises(ValueError, match="samples"):
            rdf.rd_range_compress_f16(plan.handle, h16, h16[:255])
        with pytest.raises(ValueError, match="float16"):
            rdf.rd_range_compress_f16(plan.handle, h16, x)
        h = plan.handle
    with pytest.raises(rdf.RdError) as ei:        # destroyed plan
        rdf.rd_range_compress(h, x, x)
    assert ei.value.status == -1


# ------------------------------------------------------------------------------ graph capture
def test_entry_points_replay_from_a_captured_graph(torch_dev, rdf):
    """rd_range_compress, rd_focus, rd_focus_f16, rd_omega_k and rd_omega_k_f16 allocate nothing
    and issue no memsets per call, so they can be captured into a HIP graph: each of several replays, with
    eager work and synchronisation between them, gives the eager result bit for bit."""
    torch = torch_dev
    cfg = C1
    sc = make_scene(cfg)
    ref_bin = int(round((cfg.r_ref_m - cfg.range_bin0_m) / cfg.dr))
    with rdf.Plan(**cfg.plan_params()) as plan:
        echo = dev(torch, sc.echo)
        e16 = torch.from_numpy(to_half(sc.echo)).to("cuda")
        rc_e, img_e, wk_e = plan.range_compress(echo), plan.focus(echo), plan.omega_k(echo, ref_bin)
        h_e, hw_e = plan.focus_f16(e16), plan.omega_k_f16(e16, ref_bin)
        rc, img, wk = torch.empty_like(echo), torch.empty_like(echo), torch.empty_like(echo)
        h, hw = torch.empty_like(e16), torch.empty_like(e16)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):                 # warm the capture stream
            plan.range_compress(echo, out=rc)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            plan.range_compress(echo, out=rc)
            plan.focus(echo, out=img)
            plan.focus_f16(e16, out=h)
            plan.omega_k(echo, ref_bin, out=wk)
            plan.omega_k_f16(e16, ref_bin, out=hw)
        for i in range(4):
            rc.zero_(), img.zero_(), wk.zero_(), h.zero_(), hw.zero_()
            _ = (echo * (i + 1)).sum()                # eager work between replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(rc, rc_e) and torch.equal(img, img_e) and torch.equal(wk, wk_e), i
            assert torch.equal(h.view(torch.int16), h_e.view(torch.int16)), i
            assert torch.equal(hw.view(torch.int16), hw_e.view(torch.int16)), i
        log("[graph] 4 replays bit-identical to eager")
        del g


@pytest.mark.parametrize("n", [4096, 6000, 16384], ids=lambda v: str(v))
def test_range_compression_plans_alternating_on_one_stream(torch_dev, rdf, n):
    """The persistent range kernels load their plan's filter and twiddles once per launch and hold
    them across lines: launches of two plans with different replicas (Hamming and rectangular
    windows, different pulse lengths), alternating back to back on one stream, each give exactly
    the result of their own plan computed alone."""
    torch = torch_dev
    lines = 300 if n < 16384 else 96
    base = C2.with_(Na=lines, Nr=n, fs_hz=C2.fs_hz * n / 4096)
    pa_params = base.plan_params()
    pb_params = dict(base.with_(pulse_s=base.pulse_s / 2).plan_params(), range_window=0)
    g = torch.Generator(device="cuda").manual_seed(11)
    x = torch.randn((lines, n), dtype=torch.complex64, device="cuda", generator=g)
    with rdf.Plan(**pa_params) as pa, rdf.Plan(**pb_params) as pb:
        ya, yb = pa.range_compress(x), pb.range_compress(x)
        torch.cuda.synchronize()
        assert not torch.equal(ya, yb)
        s = torch.cuda.current_stream()
        outs = []
        for _ in range(4):
            oa, ob = torch.empty_like(x), torch.empty_like(x)
            rdf.rd_range_compress(pa.handle, x, oa, s)
            rdf.rd_range_compress(pb.handle, x, ob, s)
            outs.append((oa, ob))
        torch.cuda.synchronize()
        for oa, ob in outs:
            assert torch.equal(oa, ya) and torch.equal(ob, yb)
    log(f"[alternating] {n}: alternating plans give each plan's own result")


def test_two_plans_on_two_streams_concurrently(torch_dev, rdf):
    """Two plans driven from two streams at once (range compression of one scene while another is
    focused, then omega-k): plans share no mutable device state, so each result equals the one
    computed alone."""
    torch = torch_dev
    sa, sb = make_scene(C2.with_(Na=512)), make_scene(C1)
    ref_bin = int(round((C1.r_ref_m - C1.range_bin0_m) / C1.dr))
    with rdf.Plan(**C2.with_(Na=512).plan_params()) as pa, rdf.Plan(**C1.plan_params()) as pb:
        ea, eb = dev(torch, sa.echo), dev(torch, sb.echo)
        rc_alone, img_alone, wk_alone = pa.range_compress(ea), pb.focus(eb), pb.omega_k(eb, ref_bin)
        torch.cuda.synchronize()
        s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
        outs = []
        for _ in range(3):
            rc, img, wk = torch.empty_like(ea), torch.empty_like(eb), torch.empty_like(eb)
            s1.wait_stream(torch.cuda.current_stream())
            s2.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s1):
                for _ in range(4):
                    rdf.rd_range_compress(pa.handle, ea, rc, s1)
            with torch.cuda.stream(s2):
                rdf.rd_focus(pb.handle, eb, img, s2)
                rdf.rd_omega_k(pb.handle, eb, wk, ref_bin, s2)
            outs.append((rc, img, wk))
        torch.cuda.synchronize()
        for rc, img, wk in outs:
            assert torch.equal(rc, rc_alone) and torch.equal(img, img_alone) and torch.equal(wk, wk_alone)
    log("[streams] concurrent results equal the ones computed alone")

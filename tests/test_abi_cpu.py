"""The C-ABI library on the CPU side: it loads, exports every symbol the header declares, its
parameter block matches the C layout, and argument validation fails before any device work.
No kernel is launched here (there may be no GPU)."""
import ctypes
import os
import re
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rdfocus.h")
LIB = os.path.join(ROOT, "range_doppler_focusing_amd", "librdfocus.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="librdfocus.so not built")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rd_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    import range_doppler_focusing_amd as rdf
    lib = rdf.load_library()
    declared = header_functions()
    assert len(declared) == 19
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(rdf.EXPORTS) == declared
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (rd_[a-z0-9_]+)$", out, flags=re.M))
    assert set(declared) <= exported


def test_param_block_layout_matches_c():
    """Offsets of every rd_params field as gcc lays out the header, vs the ctypes mirror."""
    from range_doppler_focusing_amd import rd_params
    fields = [f for f, _ in rd_params._fields_]
    src = "#include <stdio.h>\n#include <stddef.h>\n#include \"rdfocus.h\"\nint main(void){\n"
    src += 'printf("%zu\\n", sizeof(rd_params));\n'
    for f in fields:
        src += f'printf("%zu\\n", offsetof(rd_params, {f}));\n'
    src += "return 0;}\n"
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "layout.c")
        exe = os.path.join(d, "layout")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), c, "-o", exe], check=True)
        got = [int(x) for x in subprocess.run([exe], capture_output=True, text=True).stdout.split()]
    assert got[0] == ctypes.sizeof(rd_params)
    assert got[1:] == [getattr(rd_params, f).offset for f in fields]


def test_status_strings_and_lengths():
    import range_doppler_focusing_amd as rdf
    assert rdf.rd_status_string(0) == "ok"
    assert "unsupported" in rdf.rd_status_string(-2)
    for n in (256, 512, 1024, 2048, 4096, 8192, 16384, 6000):
        assert rdf.rd_length_supported(n)
    for n in (0, -1, 100, 1000, 4095, 6001, 32768):
        assert not rdf.rd_length_supported(n)


def good_params(**kw):
    from rdscene import C3
    p = C3.plan_params()
    p.update(kw)
    return p


@pytest.mark.parametrize("bad,status", [
    (dict(Na=0), -1), (dict(Nr=-4), -1), (dict(pulse_s=0.0), -1), (dict(fs_hz=float("nan")), -1),
    (dict(range_window=7), -1), (dict(flags=1), -1),
    (dict(pulse_s=1e-3), -1),                       # replica longer than the line
    (dict(prf_hz=0.0), -1),                         # half-configured azimuth
    (dict(Nr=9000), -2), (dict(Na=9000), -2),       # no transform of that length, none padded
    (dict(Na=12), -2),                              # azimuth below the Bluestein form's range
    (dict(Nr=9000, carrier_hz=0.0, prf_hz=0.0, velocity_mps=0.0), -2),  # range-only, beyond 8192
    (dict(rcmc_taps=6), -1), (dict(kaiser_beta=-1.0), -1),
    (dict(velocity_mps=1.0), -1),                   # Doppler band beyond 2V/lambda
    (dict(range_bin0_m=0.0), -1),
])
def test_invalid_parameters_rejected_before_device_work(bad, status):
    import range_doppler_focusing_amd as rdf
    with pytest.raises(rdf.RdError) as ei:
        rdf.rd_plan_create(good_params(**bad))
    assert ei.value.status == status
    assert rdf.rd_last_error() != ""


def test_null_arguments():
    import range_doppler_focusing_amd as rdf
    lib = rdf.load_library()
    assert lib.rd_plan_create(None, None) == -1
    h = ctypes.c_void_p()
    assert lib.rd_plan_create(None, ctypes.byref(h)) == -1 and h.value is None
    assert lib.rd_plan_destroy(None) == 0
    assert lib.rd_range_compress(None, None, None, None) == -1
    assert lib.rd_focus(None, None, None, None) == -1
    assert "plan" in rdf.rd_last_error()


def test_corner_turn_argument_errors_return_before_any_launch():
    """Invalid sizes and pointers are rejected on the host; an empty turn is a no-op."""
    import range_doppler_focusing_amd as rdf
    lib = rdf.load_library()
    a, b = 1 << 20, 1 << 30          # host-side stand-in addresses (never dereferenced)
    assert lib.rd_corner_turn(a, b, 0, 7, None) == 0
    assert lib.rd_corner_turn(a, b, 7, 0, None) == 0
    assert lib.rd_corner_turn(a, b, -1, 7, None) == -1
    assert lib.rd_corner_turn(a, b, 7, -1, None) == -1
    assert lib.rd_corner_turn(0, b, 7, 7, None) == -1
    assert lib.rd_corner_turn(a + 4, b, 7, 7, None) == -1
    assert lib.rd_corner_turn(a, a + 8, 7, 7, None) == -1          # overlapping buffers
    assert lib.rd_corner_turn(a, b, 1, 1 << 37, None) == -1         # 2^31 tiles of 64 x 64
    assert "tiles" in lib.rd_last_error().decode()
    assert lib.rd_corner_turn(a, b, 1 << 21, 1 << 20, None) == -1    # beyond 2^40 elements
    assert "2^40" in lib.rd_last_error().decode()


def test_bp_grid_layout_matches_c():
    from range_doppler_focusing_amd import rd_bp_grid
    fields = [f for f, _ in rd_bp_grid._fields_]
    src = "#include <stdio.h>\n#include <stddef.h>\n#include \"rdfocus.h\"\nint main(void){\n"
    src += 'printf("%zu\\n", sizeof(rd_bp_grid));\n'
    for f in fields:
        src += f'printf("%zu\\n", offsetof(rd_bp_grid, {f}));\n'
    src += "return 0;}\n"
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "layout.c")
        exe = os.path.join(d, "layout")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), c, "-o", exe], check=True)
        got = [int(x) for x in subprocess.run([exe], capture_output=True, text=True).stdout.split()]
    assert got[0] == ctypes.sizeof(rd_bp_grid)
    assert got[1:] == [getattr(rd_bp_grid, f).offset for f in fields]


def test_binding_checks_tensors_before_the_call():
    """The Python entry points check a tensor argument before taking its address: a host tensor
    raises ValueError and anything else that is neither a tensor nor an integer address raises
    TypeError, so nothing reaches the library (the plan handle here is not even a plan).  The
    dtype, contiguity and size checks are exercised on the GPU."""
    import torch

    import range_doppler_focusing_amd as rdf
    x = torch.zeros((4, 256), dtype=torch.complex64)
    h = torch.zeros((4, 256, 2), dtype=torch.float16)
    for call in (lambda: rdf.rd_range_compress(1, x, x), lambda: rdf.rd_focus(1, x, x),
                 lambda: rdf.rd_azimuth_focus(1, x, x), lambda: rdf.rd_omega_k(1, x, x, 0),
                 lambda: rdf.rd_debug_rcmc(1, x, x, 1), lambda: rdf.rd_debug_line_fft(1, 1, 0, x, x, 4),
                 lambda: rdf.rd_debug_azimuth_stages(1, x, x, x, x),
                 lambda: rdf.rd_backproject(1, x, x, dict(nx=2, ny=2, x0_m=0.0, dx_m=1.0, r0_m=1e3, dr_m=1.0)),
                 lambda: rdf.rd_range_compress_f16(1, h, h), lambda: rdf.rd_focus_f16(1, h, h),
                 lambda: rdf.rd_azimuth_focus_f16(1, h, h), lambda: rdf.rd_omega_k_f16(1, h, h, 0)):
        with pytest.raises(ValueError, match="GPU tensor"):
            call()
    with pytest.raises(TypeError):
        rdf.rd_range_compress(1, [0.0], 1 << 20)


def test_backproject_rejects_a_null_plan_before_any_launch():
    import range_doppler_focusing_amd as rdf
    lib = rdf.load_library()
    g = rdf.make_bp_grid(nx=4, ny=4, x0_m=0.0, dx_m=1.0, r0_m=1000.0, dr_m=1.0)
    assert lib.rd_backproject(None, 1 << 20, 1 << 30, ctypes.byref(g), None) == -1
    assert lib.rd_omega_k(None, 1 << 20, 1 << 30, 0, None) == -1
    assert lib.rd_range_compress_f16(None, 1 << 20, 1 << 30, None) == -1
    assert lib.rd_focus_f16(None, 1 << 20, 1 << 30, None) == -1
    assert lib.rd_azimuth_focus_f16(None, 1 << 20, 1 << 30, None) == -1
    assert lib.rd_omega_k_f16(None, 1 << 20, 1 << 30, 0, None) == -1


def test_bench_refuses_more_than_one_gpu():
    """The path runs on one GPU: bench.py --gpus N with N > 1 exits with a message, before any
    device work."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)

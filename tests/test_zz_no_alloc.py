"""rd_focus_noalloc: rd_focus with the Bluestein workspace in the library's static device scratch
instead of the plan's, for callers that cannot allocate.  Checked against rd_focus through the C
ABI on two calls in a row, the second with a smaller input, plus a plan that needs no scratch and
a plan whose workspace exceeds the scratch."""
import sys

import numpy as np
import pytest

from rdscene import C3

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _scene(torch, cfg, seed):
    gen = torch.Generator(device="cuda").manual_seed(seed)
    return torch.randn((cfg.Na, cfg.Nr), dtype=torch.complex64, device="cuda", generator=gen)


def test_focus_noalloc_equals_focus():
    import torch

    import range_doppler_focusing_amd as rdf
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    torch.cuda.set_device(0)
    rdf.load_library()
    # Bluestein azimuth lengths (997 is prime, 300 = 12 * 25): workspaces of M * Nr * 8 bytes,
    # 2048 * 1024 * 8 = 16 MiB, then a smaller 1024 * 700 * 8 = 5.5 MiB; then a power-of-two
    # azimuth length, which uses no scratch
    cases = [C3.with_(name="noalloc_997x1024", Na=997, Nr=1024, pulse_s=1e-6, n_targets=2),
             C3.with_(name="noalloc_300x700", Na=300, Nr=700, pulse_s=1e-6, n_targets=2),
             C3.with_(name="noalloc_512x1024", Na=512, Nr=1024, pulse_s=1e-6, n_targets=2)]
    for i, cfg in enumerate(cases):
        log(f"[noalloc] {cfg.name}")
        x = _scene(torch, cfg, 40 + i)
        with rdf.Plan(**cfg.plan_params()) as plan:
            want = plan.focus(x)
            got = torch.empty_like(x)
            rdf.rd_focus_noalloc(plan.handle, x, got)
            y = x.clone()
            rdf.rd_focus_noalloc(plan.handle, y, y)          # in place, like rd_focus
            torch.cuda.synchronize()
            assert torch.equal(got, want), cfg.name
            assert torch.equal(y, want), cfg.name
            err = float(torch.linalg.vector_norm(got - want) / torch.linalg.vector_norm(want))
        log(f"[noalloc] {cfg.name}: equal to rd_focus (rel-L2 {err:.1e})")


def test_focus_noalloc_rejects_a_workspace_beyond_the_scratch():
    import torch

    import range_doppler_focusing_amd as rdf
    torch.cuda.set_device(0)
    # Na = 1000 needs M = 2048 rows of 8192 samples: 128 MiB > 64 MiB
    cfg = C3.with_(name="noalloc_1000x8192", Na=1000, Nr=8192, pulse_s=1e-6, n_targets=1)
    x = torch.zeros((cfg.Na, cfg.Nr), dtype=torch.complex64, device="cuda")
    with rdf.Plan(**cfg.plan_params()) as plan:
        with pytest.raises(rdf.RdError) as ei:
            rdf.rd_focus_noalloc(plan.handle, x, x)
        assert ei.value.status == -1 and "static scratch" in str(ei.value)
        with pytest.raises(rdf.RdError) as ei:              # the same argument checks as rd_focus
            rdf.rd_focus_noalloc(plan.handle, x, x.data_ptr() + 8)
        assert ei.value.status == -1
    with rdf.Plan(**C3.with_(Na=256, Nr=4096, carrier_hz=0.0, prf_hz=0.0, velocity_mps=0.0).plan_params()) as plan:
        y = torch.zeros((256, 4096), dtype=torch.complex64, device="cuda")
        with pytest.raises(rdf.RdError) as ei:
            rdf.rd_focus_noalloc(plan.handle, y, y)
        assert ei.value.status == -6
    torch.cuda.synchronize()

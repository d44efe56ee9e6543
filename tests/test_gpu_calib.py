"""GPU parity of pace_calibrate_heads (e_h, a_h of the head ranking) against the oracle's
calibration, and of the resulting 8-bit head map (pace_head_alloc on the GPU figures vs
the oracle's ranking).

The calibration runs the exact recurrence without feeding any rounding back, so the GPU
(fp32 state) and the oracle (fp64 state) follow the same trajectory up to rounding
order; the rounding error energies then agree to ~1e-5 relative (a code can flip only at
a near-tie, which changes one element's error by at most a step)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import pace_oracle as po  # noqa: E402
from pace_synth import make_tokens  # noqa: E402
from test_gpu_decode import dev, io_dev  # noqa: E402

pytestmark = pytest.mark.gpu

E_TOL = 1e-3      # relative, per head
A_TOL = 1e-12     # relative, per head (fp64 sums of the same fp32 values)

CASES = {
    # name: (B, Hv, Hk, d, group, asym, bf16, dP, T)
    "d64_asym_g32_f32": (2, 8, 4, 64, 32, True, False, 8, 96),
    "d128_asym_g32_bf16": (2, 8, 4, 128, 32, True, True, 8, 64),
    "d128_sym_g64_bf16_dP4": (1, 4, 2, 128, 64, False, True, 4, 40),
}


@pytest.mark.parametrize("name", list(CASES))
def test_calibration_matches_oracle(name):
    import bit_recurrent_state_amd as pace
    print(f"[calibration parity] case={name}", flush=True)
    B, Hv, Hk, d, g, asym, bf16, dP, T = CASES[name]
    toks = make_tokens(300 + len(name), B, T, Hv, Hk, d, d, bf16=bf16)
    e_ref, a_ref = po.calibrate_heads(toks, dP, bits=4, group=g, asym=asym)
    cfg = pace.LayerConfig(B=B, Hv=Hv, Hk=Hk, dk=d, dv=d, group=g, asym=asym, buf="int8",
                           bf16_io=bf16, dP=dP)
    e_gpu, a_gpu = pace.calibrate_heads(cfg, io_dev(toks.k, bf16), io_dev(toks.v, bf16),
                                        dev(toks.a, torch.float32), dev(toks.beta, torch.float32))
    torch.cuda.synchronize()
    e_gpu, a_gpu = e_gpu.cpu().numpy(), a_gpu.cpu().numpy()
    assert np.all(e_ref > 0)
    np.testing.assert_allclose(a_gpu, a_ref, rtol=A_TOL)
    np.testing.assert_allclose(e_gpu, e_ref, rtol=E_TOL)

    # the 8-bit head map from the GPU figures equals the oracle's, unless two heads sit
    # within the tolerance of each other at the quarter's boundary
    n8 = po.quarter(Hv)
    bits_ref, E_ref = po.head_alloc(e_ref, a_ref, dP, n8)
    bits_gpu, _ = pace.head_alloc(e_gpu, a_gpu, dP, n8)
    order = np.sort(E_ref)[::-1]
    boundary_tie = n8 < Hv and abs(order[n8 - 1] - order[n8]) <= 4 * E_TOL * order[n8 - 1]
    if not boundary_tie:
        assert list(bits_gpu) == list(bits_ref)


def test_calibration_without_rounding_points_reports_zero():
    """T < dP: no rounding point, e_h = 0; a_h is still the mean decay."""
    import bit_recurrent_state_amd as pace
    B, Hv, Hk, d = 1, 4, 4, 64
    toks = make_tokens(9, B, 5, Hv, Hk, d, d)
    cfg = pace.LayerConfig(B=B, Hv=Hv, Hk=Hk, dk=d, dv=d, group=32, asym=True, buf="int8",
                           bf16_io=False, dP=8)
    e_gpu, a_gpu = pace.calibrate_heads(cfg, io_dev(toks.k, False), io_dev(toks.v, False),
                                        dev(toks.a, torch.float32), dev(toks.beta, torch.float32))
    torch.cuda.synchronize()
    assert np.all(e_gpu.cpu().numpy() == 0.0)
    np.testing.assert_allclose(a_gpu.cpu().numpy(), toks.a.astype(np.float64).mean(axis=(0, 1)), rtol=1e-12)

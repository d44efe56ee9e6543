"""GPU-vs-oracle comparison protocol shared by the GPU tests.

Rules (tolerances from the method's accuracy budget for this path):
  * outputs o and dequantised states: max |x - y| / max |y| <= 2e-3 per (sequence, head)
    slice (fp32 accumulation); outputs delivered in bf16 also carry their own rounding,
    at most half a bf16 ulp, i.e. 2^-8 |y| per element, which is added to the bound;
  * buffer codes and scales: bit-exact (both sides take the same fp32 decisions);
  * state scales: bit-exact, except a one-ulp bf16 difference when the exact
    range / levels lies within 1e-5 (relative) of the bf16 rounding boundary;
  * state codes: each GPU code is round-half-even(x / s) (+ z) of the oracle's fp32
    pre-rounding value x under the GPU's own scale, or one away from it where x / s is
    within 1e-4 of a half-integer; such flips are counted and must stay <= 1e-4 of the
    entries (plus one for small tests);
  * every GPU-dequantised element lies within s/2 (+ tolerance) of the oracle's
    pre-rounding value.
"""
from __future__ import annotations

import numpy as np

from oracle import pace_oracle as po

TOL_REL = 2e-3
TIE_WINDOW = 1e-4
SCALE_BOUNDARY_REL = 1e-5


def rel_err(x, y):
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    den = np.max(np.abs(y))
    return float(np.max(np.abs(x - y)) / den) if den > 0 else float(np.max(np.abs(x)))


def rel_err_io(x, y, out_bf16: bool):
    """rel_err after removing the output dtype's own rounding (half a bf16 ulp)."""
    if not out_bf16:
        return rel_err(x, y)
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    den = np.max(np.abs(y))
    excess = np.maximum(np.abs(x - y) - np.abs(y) * 2.0 ** -8, 0.0)
    return float(np.max(excess) / den) if den > 0 else float(np.max(np.abs(x)))


def check_outputs(o_gpu, o_ref, tiles, label="", out_bf16=False):
    worst = 0.0
    for b, h in tiles:
        e = rel_err_io(o_gpu[b, h], o_ref[b, h], out_bf16)
        worst = max(worst, e)
        assert e <= TOL_REL, f"{label} o mismatch at (b={b}, h={h}): rel err {e:.3g}"
    return worst


def _bf16_next_up(s):
    return po.bf16_ceil(s * (1 + 2.0 ** -20)) if s > 0 else float(2.0 ** -133)


def check_requant(S_pre, q_gpu: po.QState, label=""):
    """Check one flushed tile.  Returns (flips, entries, exempt_groups)."""
    x = po.to_f32(S_pre)
    dk, dv = x.shape
    g, bits = q_gpu.group, q_gpu.bits
    levels = (1 << bits) - 1
    zsym = 1 << (bits - 1)
    qmax = zsym - 1
    flips = 0
    exempt = 0
    for j in range(dv):
        for G in range(dk // g):
            xs = x[G * g:(G + 1) * g, j]
            s_g = float(q_gpu.scales[G, j])
            if q_gpu.asym:
                lo, hi = min(0.0, xs.min()), max(0.0, xs.max())
                exact = (hi - lo) / levels
            else:
                exact = float(np.abs(xs).max()) / qmax
            s_o = float(po.bf16_ceil(exact))
            if s_g != s_o:
                lo_s, hi_s = min(s_g, s_o), max(s_g, s_o)
                adjacent = _bf16_next_up(lo_s) == hi_s
                near = abs(exact - lo_s) <= SCALE_BOUNDARY_REL * max(exact, 1e-300)
                assert adjacent and near, (f"{label} scale mismatch col {j} group {G}: "
                                           f"gpu {s_g!r} oracle {s_o!r} exact {exact!r}")
                exempt += 1
            codes = q_gpu.codes[G * g:(G + 1) * g, j]
            if s_g == 0.0:
                assert s_o == 0.0
                want = 0 if q_gpu.asym else zsym
                assert np.all(codes == want), f"{label} zero group codes"
                continue
            if q_gpu.asym:
                zq = -lo / s_g
                z_ref = int(np.clip(np.rint(zq), 0, levels))
                z = int(q_gpu.zeros[G, j])
                if z != z_ref:
                    assert abs(z - z_ref) == 1 and abs(abs(zq - np.floor(zq)) - 0.5) < TIE_WINDOW, \
                        f"{label} zero point col {j} group {G}: {z} vs {z_ref}"
                    flips += 1
                t = xs / s_g
                ref = np.clip(np.rint(t) + z, 0, levels)
            else:
                z = zsym
                t = xs / s_g
                ref = np.clip(np.rint(t), -qmax, qmax) + zsym
            diff = codes.astype(np.int64) - ref.astype(np.int64)
            bad = np.nonzero(diff)[0]
            for r in bad:
                frac = abs(t[r] - np.floor(t[r]))
                assert abs(diff[r]) == 1 and abs(frac - 0.5) < TIE_WINDOW, (
                    f"{label} code col {j} key {G * g + r}: gpu {codes[r]} ref {ref[r]} x/s {t[r]!r}")
            flips += len(bad)
            # dequantised value within half a step of the pre-rounding value
            deq = s_g * (codes.astype(np.float64) - z)
            assert np.all(np.abs(deq - xs) <= s_g * 0.5 * (1 + 1e-3) + 1e-6 * np.abs(xs).max()), \
                f"{label} dequantised value outside s/2 at col {j} group {G}"
    return flips, dk * dv, exempt


def check_flushed_tiles(pre: dict, q_gpu_tiles, label=""):
    total_flips = total = 0
    for (b, h), S in pre.items():
        f, n, _ = check_requant(S, q_gpu_tiles[b][h], f"{label}(b={b},h={h})")
        total_flips += f
        total += n
    assert total_flips <= 1e-4 * total + 1, f"{label} {total_flips} code flips in {total} entries"
    return total_flips, total


def _bf16_neighbour(w: float, up: bool) -> float:
    """The bf16 value next to w (a bf16 value) toward +inf (up) or -inf."""
    nudge = max(abs(w) * 2.0 ** -20, 2.0 ** -140)
    return float(po.bf16_ceil(w + nudge)) if up else -float(po.bf16_ceil(-w + nudge))


def check_bf16_rounding(stored, x, tol, label=""):
    """bf16 values a kernel stored after rounding its fp32 value of x (fp64 oracle values).

    Each stored value must be bf16_rne of fp32(x), unless x lies within `tol` (the fp32
    evaluation error bound of the element, same shape) of the edge of the stored value's
    rounding interval: then the stored value must be the bf16 rounding of some value
    within tol of x.  Returns the number of such deviations."""
    stored = np.asarray(stored, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    tol = np.broadcast_to(np.asarray(tol, dtype=np.float64), x.shape)
    want = po.bf16_rne(po.to_f32(x))
    bad = np.nonzero(stored != want)
    for idx in zip(*bad):
        g, w, xv, t = float(stored[idx]), float(want[idx]), float(x[idx]), float(tol[idx])
        assert float(po.bf16_rne(g)) == g, f"{label} stored {g!r} is not a bf16 value"
        lo, hi = 0.5 * (g + _bf16_neighbour(g, False)), 0.5 * (g + _bf16_neighbour(g, True))
        assert xv + t >= lo and xv - t <= hi, (
            f"{label} at {idx}: stored {g!r} vs rne {w!r}; x = {xv!r} lies "
            f"{min(abs(xv - lo), abs(xv - hi)):.3g} outside its rounding interval (error bound {t:.3g})")
    return int(bad[0].size)

"""Pins of the oracle's bit accounting and retained-error head allocation: the numbers
the pages print (tests/golden/accounting.txt), the geometric-series origin of
E_h = e_h / (1 - a_h^(2 dP)) by Monte Carlo, brute force over head subsets, and the
ranking of measured retained error on tiny gated-delta heads."""
import itertools
import os

import numpy as np
import pytest

from oracle import pace_oracle as po
from oracle import packing as pk
from pace_synth import make_tokens

GOLD = os.path.join(os.path.dirname(__file__), "golden", "accounting.txt")


def _golden():
    out = {}
    for line in open(GOLD):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, val, tol, kind, cite = line.split()
        out[name] = (float(val), float(tol), kind, cite)
    return out


def _pace48_bits(H=32):
    bits = np.full(H, 4)
    bits[:po.quarter(H)] = 8
    return bits


def test_payload_of_pace48_is_the_printed_5_66():
    val, tol, _, _ = _golden()["payload_pace48"]
    p = po.payload_bits(_pace48_bits(), 32, asym=True)
    assert p == 5.65625                    # 3/4 (4 + 20/32) + 1/4 (8 + 24/32)
    assert abs(p - val) <= tol
    assert po.payload_bits(np.full(32, 4), 64, asym=False) == 4.25     # PACE-4
    assert po.payload_bits(np.full(4, 4), 32, asym=False) == 4.5       # tiny reference


def test_resident_bits_soft_pins_and_closed_forms():
    g = _golden()
    c_int8 = po.buffer_cost_per_token(128, 128, 2, 8, 8)
    assert c_int8 == (8 * 64 + 8 * 128 + 32) / 16384
    r4 = po.resident_bits(np.full(32, 4), 64, False, 128, 128, 2, 8, "int8")
    r48 = po.resident_bits(_pace48_bits(), 32, True, 128, 128, 2, 8, "int8")
    r48m = po.resident_bits(_pace48_bits(), 32, True, 128, 128, 2, 8, "mixed")
    assert (r4, r48, r48m) == (5.015625, 6.421875, 6.796875)
    v, tol, _, _ = g["resident_pace4_int8"]
    assert abs(r4 - v) <= tol
    v, tol, _, _ = g["resident_pace48_mixed"]
    assert abs(r48m - v) <= tol
    # the buffer cost is linear in dP: a longer period costs proportionally more memory
    assert po.buffer_bits_model(128, 128, 2, 32, "int8") == 4 * po.buffer_bits_model(128, 128, 2, 8, "int8")
    assert g["default_dP"][0] == 8 and g["prefill_period"][0] == 256


def test_retained_error_is_the_stationary_sum_of_decayed_roundings():
    """Inject an independent rounding error of energy e at every flush of a head that
    only decays by a per token; the mean retained energy converges to
    e * sum_k a^(2 dP k) = e / (1 - a^(2 dP))."""
    rng = np.random.default_rng(0)
    for a, dP in [(0.9, 1), (0.9, 8), (0.97, 4), (0.99, 8)]:
        e = 2.5
        n_chains, n_periods = 4000, 400
        X = np.zeros((n_chains, 4))
        acc, cnt = 0.0, 0
        for p in range(n_periods):
            X *= a ** dP
            X += rng.standard_normal(X.shape) * np.sqrt(e / 4)
            if p > n_periods // 2:
                acc += np.mean(np.sum(X * X, axis=1))
                cnt += 1
        mc = acc / cnt
        E = po.retained_error([e], [a], dP)[0]
        assert abs(mc - E) / E < 0.03, (a, dP, mc, E)
    assert po.retained_error([1.0], [1.0], 8)[0] == np.inf


def test_head_alloc_maximises_total_retained_error_brute_force():
    rng = np.random.default_rng(1)
    for trial in range(40):
        H = 8
        e = rng.uniform(0, 1, H)
        a = rng.uniform(0.5, 0.999, H)
        if trial % 4 == 0:
            e[3] = e[5]
            a[3] = a[5]                   # an exact tie
        bits, E = po.head_alloc(e, a, 8, 2)
        chosen = set(np.nonzero(bits == 8)[0].tolist())
        best = max(itertools.combinations(range(H), 2),
                   key=lambda s: (sum(E[list(s)]), [-x for x in s]))
        assert chosen == set(best)
        assert np.all(bits[list(set(range(H)) - chosen)] == 4)
    # ties go to the lower head index
    bits, _ = po.head_alloc([1.0] * 4, [0.9] * 4, 8, 1)
    assert bits.tolist() == [8, 4, 4, 4]


def test_e_h_ranking_matches_measured_retained_error_on_tiny_heads():
    """Heads with well separated decays: ranking by E_h (from calibrated e_h, a_h)
    equals the ranking of the retained error actually measured between a periodically
    rounded decode and the exact recurrence."""
    dk = dv = 32
    dP = 8
    decays = [0.5, 0.9, 0.99, 0.999]
    H = len(decays)
    T = 160
    rng = np.random.default_rng(4)
    toks = make_tokens(21, 2, T, H, H, dk, dv)
    toks.a[:] = np.array(decays, dtype=np.float32)[None, None, :]
    e_h, a_h = po.calibrate_heads(toks, dP, bits=4, group=32, asym=True, n_tokens=T)
    assert np.allclose(a_h, np.array(decays, dtype=np.float32))
    E = po.retained_error(e_h, a_h, dP)
    measured = np.zeros(H)
    rq = lambda S: po.quantize_state(S, 4, 32, True)
    for b in range(2):
        for h in range(H):
            tile = po.TileState(po.zero_qstate(dk, dv, 4, 32, True))
            S = np.zeros((dk, dv))
            errs = []
            for t in range(T):
                args = (toks.q[b, t, h], toks.k[b, t, h], toks.v[b, t, h], toks.a[b, t, h], toks.beta[b, t, h])
                _, flushed = po.decode_tile_step(tile, *args, dP, "exact", rq)
                S, _ = po.exact_step(S, *args[1:])
                if flushed and t > T // 2:
                    d = po.dequantize_state(tile.q) - S
                    errs.append(np.sum(d * d))
            measured[h] += np.mean(errs)
    assert np.argsort(E).tolist() == np.argsort(measured).tolist()


def test_calibration_zero_inputs_and_mean_decay():
    toks = make_tokens(5, 1, 32, 2, 2, 32, 32)
    toks.v[:] = 0
    e_h, a_h = po.calibrate_heads(toks, 8, n_tokens=32)
    assert np.all(e_h == 0)
    assert np.allclose(a_h, toks.a[0].astype(np.float64).mean(axis=0))


def test_layout_sizes_of_named_configurations():
    cfg = pk.LayerCfg(B=64, Hv=32, Hk=16, dk=128, dv=128, group=64, asym=False, buf="int8", dP=8)
    _, stride, total = pk.state_layout(cfg)
    assert stride == 32 * 8704 and total == 64 * 32 * 8704
    _, btotal = pk.buffer_layout(cfg)
    # count + k codes/scales per key head + v codes/scales + a + beta per value head
    assert btotal == 64 * 32 * 4 + 64 * 16 * 8 * (128 + 4) + 64 * 32 * 8 * (128 + 4 + 4 + 4)

"""Pins of the oracle's periodic decode on a bf16 state (the decode buffer alone, with the
state kept in bf16: [p1] "Assumptions and limits", throughput paragraph).

What fixes it, independently of the periodic machinery:
  * with an identity buffer quantiser and dP = 1 it is the per-token bf16 recurrence the
    pages compare against (round the state to bf16 after every token, read o from the
    unrounded state), written here as a plain loop;
  * the stored state is always bf16-representable and within half a bf16 ulp (at most
    2^-8 of the magnitude) of the unrounded state it came from, and it changes only at
    flushes;
  * its byte layout is the bf16 [column][key] record of the per-token comparator;
  * with the rounding switched off it is the exact recurrence (P1, shared with the packed
    states), so every difference from the exact run comes from the once-per-period
    rounding: it is much smaller than the 4-bit state's on the same tokens."""
import numpy as np

from oracle import pace_oracle as po
from oracle import packing as pk
from pace_synth import make_tokens, random_bf16_state


def _toks(seed, T, d=32, outliers=0):
    return make_tokens(seed, 1, T, 1, 1, d, d, n_outlier=outliers)


def test_dP1_identity_buffer_is_per_token_bf16_recurrence():
    d, T = 32, 40
    t = _toks(3, T, d)
    S0 = po.bf16_rne(np.random.default_rng(0).standard_normal((d, d)) * 0.2)
    tile = po.TileState(S0.copy(), [])
    S = S0.copy()
    for i in range(T):
        q, k, v, a, b = t.q[0, i, 0], t.k[0, i, 0], t.v[0, i, 0], float(t.a[0, i, 0]), float(t.beta[0, i, 0])
        o, flushed = po.decode_tile_step(tile, q, k, v, a, b, 1, "exact", po.round_state_bf16)
        assert flushed
        # per-token bf16 reference: exact update, output from the unrounded state, then
        # every element rounded to the nearest bf16 of its fp32 value
        u = b * (v.astype(np.float64) - a * (S.T @ k.astype(np.float64)))
        S_new = a * S + np.outer(k.astype(np.float64), u)
        o_ref = S_new.T @ q.astype(np.float64)
        S = po.bf16_rne(S_new.astype(np.float32).astype(np.float64))
        assert np.allclose(o, o_ref, rtol=0, atol=1e-12)
        assert np.array_equal(tile.q, S)


def test_flush_rounds_to_half_ulp_once_per_period():
    d, T, dP = 32, 41, 8
    t = _toks(5, T, d, outliers=2)
    S0 = random_bf16_state(9, 1, 1, d, d)[0, 0].astype(np.float64)
    tile = po.TileState(S0.copy(), [])
    captured = {}

    def rq(S):
        captured["S"] = S
        return po.round_state_bf16(S)

    stored = S0.copy()
    flush_steps = []
    for i in range(T):
        _, flushed = po.decode_tile_step(tile, t.q[0, i, 0], t.k[0, i, 0], t.v[0, i, 0], float(t.a[0, i, 0]),
                                         float(t.beta[0, i, 0]), dP, "int8", rq)
        if flushed:
            flush_steps.append(i)
            pre = captured["S"]
            got = tile.q
            assert np.array_equal(po.bf16_rne(got), got)                      # bf16 values
            # half a bf16 ulp: at most 2^-8 of the magnitude (the bottom of a binade), plus
            # the fp32 step of the pre-rounding value the decision is taken on
            assert np.all(np.abs(got - pre) <= 2.0 ** -8 * (1 + 2.0 ** -15) * np.abs(pre))
            stored = got.copy()
        else:
            assert np.array_equal(tile.q, stored)                              # untouched
    assert flush_steps == [7, 15, 23, 31, 39]


def test_bf16_state_record_is_column_major_bf16():
    cfg = pk.LayerCfg(B=2, Hv=3, Hk=3, dk=64, dv=64, group=32, asym=False, buf="int8", dP=8, bf16_state=True)
    S = random_bf16_state(2, 2, 3, 64, 64).astype(np.float64)
    raw = pk.pack_state(cfg, [[S[b, h] for h in range(3)] for b in range(2)])
    offs, stride, total = pk.state_layout(cfg)
    assert stride == 3 * 64 * 64 * 2 and total == 2 * stride and offs == [0, 8192, 16384]
    # element (key r, column j) of (b, h) is the bf16 at index ((b * Hv + h) * dv + j) * dk + r
    bits = raw.view(np.uint16).reshape(2, 3, 64, 64)
    want = (np.asarray(S, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(bits, np.transpose(want, (0, 1, 3, 2)))
    back = pk.unpack_state(cfg, raw)
    assert all(np.array_equal(back[b][h], S[b, h]) for b in range(2) for h in range(3))


def test_rounding_error_far_below_the_4bit_state():
    """Same tokens, same buffer: the bf16 state's drift from the exact recurrence after 256
    decode tokens is a small fraction of the 4-bit state's (the 4-bit rounding moves each
    value by up to a fourteenth of its group's largest magnitude, bf16 by 2^-8 of itself)."""
    d, T, dP = 32, 256, 8
    t = _toks(7, T, d, outliers=2)
    S0 = np.zeros((d, d))
    exact = S0.copy()
    bf = po.TileState(S0.copy(), [])
    q4 = po.TileState(po.zero_qstate(d, d, 4, 32, False), [])
    rq4 = lambda S: po.quantize_state(S, 4, 32, False)
    for i in range(T):
        q, k, v, a, b = t.q[0, i, 0], t.k[0, i, 0], t.v[0, i, 0], float(t.a[0, i, 0]), float(t.beta[0, i, 0])
        entry = po.buffer_entry(k, v, a, b, "int8")
        exact, _ = po.exact_step(exact, entry.k, entry.v, a, b)
        po.decode_tile_step(bf, q, k, v, a, b, dP, "int8", po.round_state_bf16)
        po.decode_tile_step(q4, q, k, v, a, b, dP, "int8", rq4)
    e_bf = np.linalg.norm(po._replay(bf.q, bf.buf) - exact)
    e_4 = np.linalg.norm(po._replay(q4.q, q4.buf) - exact)
    assert e_bf < e_4 / 20, (e_bf, e_4)

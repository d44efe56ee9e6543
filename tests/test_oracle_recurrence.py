"""Pins of the oracle's recurrence, buffer replay, flush schedule and prefill schedule:
closed forms, the delta rule's write property, special cases, and the identities the
pages state (periodic rounding with no quantiser is the plain recurrence; dP = 1 is
per-token rounding; prefill rounds once per chunk)."""
import numpy as np
import pytest

from oracle import pace_oracle as po
from oracle import packing as pk
from pace_synth import make_tokens, random_buffer_parts, random_packed_state_parts


def _unit(rng, n):
    x = rng.standard_normal(n)
    return x / np.linalg.norm(x)


def test_delta_rule_writes_value_at_key():
    """With beta = 1 and |k| = 1 the updated state returns exactly v for key k
    (S_t^T k = a S^T k + (k.k) u = v); for general beta it returns the convex mix
    (1 - beta) a S^T k + beta v.  A sign, index or transpose slip breaks this."""
    rng = np.random.default_rng(0)
    for _ in range(50):
        S = rng.standard_normal((16, 12))
        k, v = _unit(rng, 16), rng.standard_normal(12)
        a, beta = rng.uniform(0.5, 1.0), rng.uniform(0, 1)
        S1, u = po.exact_step(S, k, v, a, 1.0)
        assert np.allclose(S1.T @ k, v, atol=1e-12)
        S2, u = po.exact_step(S, k, v, a, beta)
        assert np.allclose(S2.T @ k, (1 - beta) * a * (S.T @ k) + beta * v, atol=1e-12)
        assert np.allclose(po.readout(S1, k), v, atol=1e-12)
        # directions orthogonal to k only decay
        w = rng.standard_normal(16)
        w -= (w @ k) * k
        assert np.allclose(S2.T @ w, a * (S.T @ w), atol=1e-12)


def test_special_cases_closed_forms():
    rng = np.random.default_rng(1)
    S0 = rng.standard_normal((8, 6))
    T = 20
    ks = [_unit(rng, 8) for _ in range(T)]
    vs = [rng.standard_normal(6) for _ in range(T)]
    as_ = rng.uniform(0.8, 1.0, T)
    qs = [rng.standard_normal(8) for _ in range(T)]
    # beta = 0: pure decay S_t = (prod a) S_0
    _, S = po.exact_run(S0, ks, vs, as_, np.zeros(T), qs)
    assert np.allclose(S, np.prod(as_) * S0, atol=1e-13)
    # k = 0: no write
    _, S = po.exact_run(S0, [np.zeros(8)] * T, vs, as_, np.ones(T), qs)
    assert np.allclose(S, np.prod(as_) * S0, atol=1e-13)
    # zero state and zero values: zero outputs
    o, S = po.exact_run(np.zeros((8, 6)), ks, [np.zeros(6)] * T, as_, np.ones(T), qs)
    assert np.all(o == 0) and np.all(S == 0)


def test_equivalent_householder_like_form():
    """S_t = a (I - beta k k^T) S_{t-1} + beta k v^T (the same update, regrouped)."""
    rng = np.random.default_rng(2)
    for _ in range(20):
        S = rng.standard_normal((10, 7))
        k, v = rng.standard_normal(10), rng.standard_normal(7)
        a, beta = rng.uniform(0.5, 1), rng.uniform(0, 1)
        S1, _ = po.exact_step(S, k, v, a, beta)
        S2 = a * (np.eye(10) - beta * np.outer(k, k)) @ S + beta * np.outer(k, v)
        assert np.allclose(S1, S2, atol=1e-12)


def _stream(rng, T, dk=12, dv=9):
    return ([_unit(rng, dk) for _ in range(T)], [rng.standard_normal(dv) for _ in range(T)],
            rng.uniform(0.7, 0.999, T), rng.uniform(0, 1, T), [rng.standard_normal(dk) for _ in range(T)])


@pytest.mark.parametrize("dP", [1, 3, 8, 10 ** 9])
def test_buffered_decode_without_rounding_is_the_plain_recurrence(dP):
    """Quantiser = identity and exact buffer: periodic decode equals the sequential
    recurrence for any dP (including never flushing)."""
    rng = np.random.default_rng(dP % 97)
    ks, vs, as_, bs, qs = _stream(rng, 40)
    S0 = rng.standard_normal((12, 9))
    ref, Sref = po.exact_run(S0, ks, vs, as_, bs, qs)
    tile = po.TileState(S0.copy())
    outs = []
    for t in range(40):
        o, _ = po.decode_tile_step(tile, qs[t], ks[t], vs[t], as_[t], bs[t], dP, "exact", lambda S: S)
        outs.append(o)
    assert np.allclose(np.array(outs), ref, atol=1e-12)
    po.flush_tile(tile, lambda S: S)
    assert np.allclose(tile.q, Sref, atol=1e-12)


@pytest.mark.parametrize("buf", ["int8", "mixed"])
def test_dP1_is_per_token_rounding(buf):
    """dP = 1: the state is rounded after every token, outputs come from the
    pre-rounding state (same buffered k^, v^ on both sides)."""
    rng = np.random.default_rng(7)
    dk = dv = 64
    ks, vs, as_, bs, qs = _stream(rng, 24, dk, dv)
    rq = lambda S: po.quantize_state(S, 4, 32, False)
    tile = po.TileState(po.zero_qstate(dk, dv, 4, 32, False))
    S = np.zeros((dk, dv))
    for t in range(24):
        o, flushed = po.decode_tile_step(tile, qs[t], ks[t], vs[t], as_[t], bs[t], 1, buf, rq)
        assert flushed
        e = po.buffer_entry(ks[t], vs[t], as_[t], bs[t], buf)
        S, _ = po.exact_step(S, e.k, e.v, e.a, e.beta)
        assert np.allclose(o, S.T @ qs[t], atol=1e-12)
        qref = rq(S)
        assert np.array_equal(qref.codes, tile.q.codes) and np.array_equal(qref.scales, tile.q.scales)
        S = po.dequantize_state(qref)


def test_periodic_decode_rounds_once_per_period():
    rng = np.random.default_rng(8)
    ks, vs, as_, bs, qs = _stream(rng, 30, 32, 32)
    calls = []

    def rq(S):
        calls.append(1)
        return po.quantize_state(S, 4, 32, False)

    tile = po.TileState(po.zero_qstate(32, 32, 4, 32, False))
    flushes = [po.decode_tile_step(tile, qs[t], ks[t], vs[t], as_[t], bs[t], 8, "int8", rq)[1]
               for t in range(30)]
    assert [t for t, f in enumerate(flushes) if f] == [7, 15, 23]
    assert len(calls) == 3 and len(tile.buf) == 6
    po.flush_tile(tile, rq)
    assert len(calls) == 4 and tile.buf == []
    assert po.flush_tile(tile, rq) is False          # empty buffer: no-op


def test_prefill_without_rounding_is_the_plain_recurrence_and_rounds_per_chunk():
    rng = np.random.default_rng(9)
    T, chunk = 21, 8
    ks, vs, as_, bs, qs = _stream(rng, T, 16, 16)
    o, S = po.prefill_tile(np.zeros((16, 16)), qs, ks, vs, as_, bs, chunk, lambda S: S)
    ref, Sref = po.exact_run(np.zeros((16, 16)), ks, vs, as_, bs, qs)
    assert np.allclose(o, ref, atol=1e-12) and np.allclose(S, Sref, atol=1e-12)
    # rounding points: after tokens 8, 16 and the last (21)
    seen = []

    def rq(S):
        seen.append(S.copy())
        return po.quantize_state(S, 4, 16, False)

    o2, q = po.prefill_tile(po.zero_qstate(16, 16, 4, 16, False), qs, ks, vs, as_, bs, chunk, rq)
    assert len(seen) == 3
    # chunk 1 is exact from zero
    _, S8 = po.exact_run(np.zeros((16, 16)), ks[:8], vs[:8], as_[:8], bs[:8], qs[:8])
    assert np.allclose(seen[0], S8, atol=1e-12)
    assert np.allclose(o2[:8], ref[:8], atol=1e-12)
    # chunk 2 starts from the rounded state
    S0b = po.dequantize_state(rq(S8))
    seen.pop()
    _, S16 = po.exact_run(S0b, ks[8:16], vs[8:16], as_[8:16], bs[8:16], qs[8:16])
    assert np.allclose(seen[1], S16, atol=1e-12)


def test_wy_chunk_algebra_equals_token_loop():
    """The chunked (WY) form the prefill kernel evaluates equals the token loop before
    rounding (checks the derivation, independent of the oracle's code)."""
    rng = np.random.default_rng(10)
    C, dk, dv = 40, 16, 12
    K = np.array([_unit(rng, dk) for _ in range(C)])
    Q = rng.standard_normal((C, dk))
    V = rng.standard_normal((C, dv))
    a = rng.uniform(0.7, 0.999, C)
    beta = rng.uniform(0, 1, C)
    S0 = rng.standard_normal((dk, dv))
    g = np.cumsum(np.log(a))                        # log Gamma_t
    ratio = np.exp(g[:, None] - g[None, :])         # Gamma_i / Gamma_j
    A = np.tril(ratio * (K @ K.T), -1)
    Tm = np.linalg.inv(np.eye(C) + beta[:, None] * A)
    Wv = Tm @ (beta[:, None] * V)
    Wk = Tm @ ((beta * np.exp(g))[:, None] * K)
    U = Wv - Wk @ S0
    M = np.tril(ratio)
    O = np.exp(g)[:, None] * (Q @ S0) + (M * (Q @ K.T)) @ U
    SC = np.exp(g[-1]) * S0 + K.T @ (np.exp(g[-1] - g)[:, None] * U)
    ref, Sref = po.exact_run(S0, K, V, a, beta, Q)
    assert np.allclose(O, ref, atol=1e-12) and np.allclose(SC, Sref, atol=1e-12)


def test_buffer_projection_recurrence_equals_replay():
    """The decode kernel's projection form: with p_i = S_0^T k_i and r = S_0^T q,
    iterate u_i = beta_i (v_i - a_i y_i), y_m <- a_i y_m + (k_i.k_m) u_i,
    y_q <- a_i y_q + (k_i.q) u_i -- equals replaying the buffer on S_0; the fold is
    S_n = Gamma_n S_0 + sum_i (prod_{l>i} a_l) k_i u_i^T."""
    rng = np.random.default_rng(11)
    dk, dv, n = 16, 10, 8
    S0 = rng.standard_normal((dk, dv))
    ks, vs, as_, bs, qs = _stream(rng, n, dk, dv)
    q = qs[-1]
    y = [S0.T @ k for k in ks]
    yq = S0.T @ q
    us = []
    for i in range(n):
        u = bs[i] * (vs[i] - as_[i] * y[i])
        us.append(u)
        for m in range(i + 1, n):
            y[m] = as_[i] * y[m] + (ks[i] @ ks[m]) * u
        yq = as_[i] * yq + (ks[i] @ q) * u
    ref, Sref = po.exact_run(S0, ks, vs, as_, bs, [q] * n)
    assert np.allclose(yq, ref[-1], atol=1e-12)
    fold = np.prod(as_) * S0 + sum(np.prod(as_[i + 1:]) * np.outer(ks[i], us[i]) for i in range(n))
    assert np.allclose(fold, Sref, atol=1e-12)


def test_layer_oracle_key_sharing_and_staggered_counts():
    """gamma = 2: value heads of one key head see identical key codes; per-sequence
    counts advance independently; a sequence whose count reaches dP flushes."""
    cfg = pk.LayerCfg(B=3, Hv=4, Hk=2, dk=64, dv=64, group=32, asym=False, buf="int8", dP=4)
    parts = random_packed_state_parts(1, 3, 4, 64, 64, 32, [4] * 4, False)
    st = pk.pack_state(cfg, pk.state_from_parts(cfg, parts))
    bp = random_buffer_parts(2, 3, 4, 2, 64, 64, 4, False, counts=[0, 2, 3])
    buf = pk.pack_buffer(cfg, bp)
    toks = make_tokens(3, 3, 1, 4, 2, 64, 64)
    o, st2, buf2, pre = pk.decode_step_layer(cfg, st, buf, *toks.token(0))
    d = pk.unpack_buffer(cfg, buf2)
    assert d["count"][:, 0].tolist() == [1, 3, 0]
    assert set(pre) == {(2, h) for h in range(4)}
    # the new key codes (slot 0 of sequence 0 / slot 2 of sequence 1) equal the buffer
    # quantiser of the key; written once per key head
    for b, slot in [(0, 0), (1, 2)]:
        for kh in range(2):
            kc, ks = po.quant_buffer_vec(toks.k[b, 0, kh], 127)
            assert np.array_equal(d["kc"][b, kh, slot], kc) and d["ks"][b, kh, slot] == np.float32(ks)
    # untouched state for non-flushing sequences; touched for the flushing one
    offs, stride, _ = pk.state_layout(cfg)
    assert np.array_equal(st2[:2 * stride], st[:2 * stride])
    assert not np.array_equal(st2[2 * stride:], st[2 * stride:])
    # inactive sequences are untouched
    o3, st3, buf3, _ = pk.decode_step_layer(cfg, st, buf, *toks.token(0), active=[0, 0, 0])
    assert np.array_equal(st3, st) and np.array_equal(buf3, buf) and np.isnan(o3).all()


def test_flush_layer_equals_decode_replay():
    cfg = pk.LayerCfg(B=2, Hv=2, Hk=2, dk=64, dv=64, group=32, asym=True, buf="mixed", dP=8,
                      head_bits=[4, 8])
    parts = random_packed_state_parts(4, 2, 2, 64, 64, 32, [4, 8], True)
    qst = pk.state_from_parts(cfg, parts)
    st = pk.pack_state(cfg, qst)
    bp = random_buffer_parts(5, 2, 2, 2, 64, 64, 8, True, counts=[5, 0])
    buf = pk.pack_buffer(cfg, bp)
    st2, buf2, pre = pk.flush_layer(cfg, st, buf)
    assert set(pre) == {(0, 0), (0, 1)}
    d = pk.unpack_buffer(cfg, buf2)
    assert d["count"].tolist() == [[0, 0], [0, 0]]
    # sequence 0 head 1: replay by hand
    S = po.dequantize_state(qst[0][1])
    for i in range(5):
        k = bp["kc"][0, 1, i] * float(bp["ks"][0, 1, i])
        S, _ = po.exact_step(S, k, bp["v"][0, 1, i].astype(np.float64), float(bp["a"][0, 1, i]),
                             float(bp["beta"][0, 1, i]))
    assert np.allclose(pre[(0, 1)], S, atol=1e-12)
    q = pk.unpack_state(cfg, st2)[0][1]
    ref = po.quantize_state(S, 8, 32, True)
    assert np.array_equal(q.codes, ref.codes) and np.array_equal(q.zeros, ref.zeros)

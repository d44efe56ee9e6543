"""Pins of the oracle's quantisers against things other than the oracle itself:
an enumerated bf16 value table, the nearest-grid-point property, the s/2 error bound,
idempotence, column locality of channel-aligned groups, and the byte layout derived
key-by-key in the inverse direction of the packer."""
import numpy as np
import pytest

from oracle import pace_oracle as po
from oracle import packing as pk

# Every finite positive bf16 value, enumerated from the 16-bit patterns (sign 0,
# exponent 1..254 normal, exponent 0 subnormal): an independent table.
_PATTERNS = np.arange(1, 0x7F80, dtype=np.uint32)
BF16_TABLE = np.sort((_PATTERNS << np.uint32(16)).view(np.float32).astype(np.float64))


def _table_ceil(x):
    i = np.searchsorted(BF16_TABLE, x, side="left")
    return BF16_TABLE[i]


def _table_nearest_even(x):
    i = np.searchsorted(BF16_TABLE, x, side="left")
    hi = BF16_TABLE[i]
    lo = BF16_TABLE[i - 1] if i > 0 else 0.0
    if x - lo < hi - x:
        return lo
    if hi - x < x - lo:
        return hi
    # tie: the one whose 16-bit pattern is even
    pat_hi = int(np.float32(hi).view(np.uint32) >> 16)
    return hi if pat_hi % 2 == 0 else lo


def test_bf16_ceil_matches_enumerated_table():
    rng = np.random.default_rng(11)
    xs = np.concatenate([np.exp(rng.uniform(-80, 80, 4000)), BF16_TABLE[::997],
                         BF16_TABLE[::991] * (1 + 2.0 ** -30), [2.0 ** -130, 3e-39]])
    for x in xs:
        assert po.bf16_ceil(x) == _table_ceil(x), x


def test_bf16_rne_matches_enumerated_table():
    rng = np.random.default_rng(12)
    mids = (BF16_TABLE[1000:1200] + BF16_TABLE[1001:1201]) / 2   # exact ties
    xs = np.concatenate([np.exp(rng.uniform(-60, 60, 3000)), mids])
    for x in xs:
        assert po.bf16_rne(x) == _table_nearest_even(x), x
        assert po.bf16_rne(-x) == -_table_nearest_even(x)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("asym", [False, True])
def test_quantiser_nearest_grid_point_and_half_step_bound(bits, asym):
    rng = np.random.default_rng(bits * 10 + asym)
    for trial in range(300):
        g = 32
        scale = np.exp(rng.uniform(-8, 4))
        x = rng.standard_normal(g) * scale
        if trial % 5 == 0:
            x = np.abs(x)                  # single-sign groups (asym range must include 0)
        if trial % 7 == 0:
            x[rng.integers(0, g)] *= 20    # an outlier
        if asym:
            c, s, z = po.quant_group_asym(x, bits)
            levels = np.arange(0, 1 << bits)
            grid = s * (levels - z)
        else:
            c, s = po.quant_group_sym(x, bits)
            z = 1 << (bits - 1)
            qmax = z - 1
            levels = np.arange(-qmax, qmax + 1) + z
            grid = s * (levels - z)
        x32 = po.to_f32(x)
        xh = s * (c - z)
        # |x - x^| <= s/2 with the stored bf16 scale (the reason scales round up)
        assert np.all(np.abs(x32 - xh) <= s / 2 * (1 + 1e-12)), (trial, np.max(np.abs(x32 - xh)) / s)
        # no other representable level is strictly closer
        for xi, ci in zip(x32, c):
            d = np.abs(grid - xi)
            assert abs(s * (ci - z) - xi) <= d.min() * (1 + 1e-12)
        # scale is the smallest bf16 >= range / levels
        if asym:
            lo, hi = min(0, x32.min()), max(0, x32.max())
            assert s == _table_ceil((hi - lo) / ((1 << bits) - 1))
            assert 0 <= z <= (1 << bits) - 1
        else:
            assert s == _table_ceil(np.abs(x32).max() / ((1 << (bits - 1)) - 1))
        assert c.min() >= 0 and c.max() <= (1 << bits) - 1


def test_symmetric_requantisation_is_idempotent():
    """4-bit: the bf16 scale is at most 2^-7 above M/7, so the largest code is always 7
    and requantising the dequantised state reproduces codes and scales.  (At 8 bits the
    largest code can be 126, so the property does not hold there.)"""
    rng = np.random.default_rng(5)
    S = rng.standard_normal((64, 48)) * np.exp(rng.uniform(-3, 3, 48))[None, :]
    for bits, g in [(4, 32), (4, 64)]:
        q1 = po.quantize_state(S, bits, g, asym=False)
        q2 = po.quantize_state(po.dequantize_state(q1), bits, g, asym=False)
        assert np.array_equal(q1.codes, q2.codes)
        assert np.array_equal(q1.scales, q2.scales)


def test_zero_group_gives_zero_scale_and_zero_value():
    S = np.zeros((64, 4))
    S[:, 1] = 1.0
    for asym in (False, True):
        q = po.quantize_state(S, 4, 32, asym)
        assert q.scales[0, 0] == 0 and q.scales[1, 0] == 0
        d = po.dequantize_state(q)
        assert np.all(d[:, 0] == 0)
        assert np.allclose(d[:, 1], 1.0, atol=q.scales[0, 1] / 2)


def test_channel_aligned_groups_are_column_local():
    """Permuting value columns permutes codes and scales identically (key-axis groups
    live inside one column); a value-axis grouping would not have this property."""
    rng = np.random.default_rng(9)
    S = rng.standard_normal((64, 32))
    S[:, 5] *= 30                      # an outlier column
    perm = rng.permutation(32)
    for asym in (False, True):
        q = po.quantize_state(S, 4, 32, asym)
        qp = po.quantize_state(S[:, perm], 4, 32, asym)
        assert np.array_equal(q.codes[:, perm], qp.codes)
        assert np.array_equal(q.scales[:, perm], qp.scales)
    # the outlier column does not widen the step of any other column
    q = po.quantize_state(S, 4, 32, False)
    assert q.scales[:, 5].min() > 5 * np.delete(q.scales, 5, axis=1).max()


def test_buffer_quantiser_half_step_bound_and_fp32_scale():
    rng = np.random.default_rng(3)
    for qmax in (127, 7):
        for _ in range(200):
            x = (rng.standard_normal(128) * np.exp(rng.uniform(-5, 3))).astype(np.float32)
            c, s = po.quant_buffer_vec(x, qmax)
            assert s == float(np.float32(np.abs(x).max()) / np.float32(qmax))
            assert np.all(np.abs(c) <= qmax)
            # the fp32 scale may round down by half an fp32 ulp, so the largest element
            # can sit at qmax (1 + 2^-24) steps: bound s/2 + qmax * 2^-24 * s
            assert np.all(np.abs(x.astype(np.float64) - c * s) <= s * (0.5 + qmax * 2.0 ** -23))


def _inverse_position(r, dk, bits):
    """Byte index and nibble of key r inside a column, derived key-first from the
    layout rule: unit u = (r%32)//8 * (dk/32) + r//32 holds keys 32*(u mod dk/32) +
    8*(u div dk/32) + 0..7."""
    kb, qq, e = r // 32, (r % 32) // 8, r % 8
    u = qq * (dk // 32) + kb
    if bits == 8:
        return u * 8 + e, None
    return u * 4 + (e % 4), e // 4


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("dk", [64, 128])
def test_state_packing_matches_layout_rule(bits, dk):
    dv, g = 16, 32
    cfg = pk.LayerCfg(B=1, Hv=1, Hk=1, dk=dk, dv=dv, group=g, asym=True, buf="int8", dP=8,
                      head_bits=[bits])
    rng = np.random.default_rng(dk + bits)
    codes = rng.integers(0, 1 << bits, size=(dk, dv))
    scales = po.bf16_rne(np.abs(rng.standard_normal((dk // g, dv))) + 0.01)
    zeros = rng.integers(0, 1 << bits, size=(dk // g, dv))
    raw = pk.pack_state(cfg, [[po.QState(codes, scales, zeros, bits, g, True)]])
    colb = dk * bits // 8
    for j in range(dv):
        for r in range(dk):
            byte, nib = _inverse_position(r, dk, bits)
            val = int(raw[j * colb + byte])
            if nib is not None:
                val = (val >> (4 * nib)) & 15
            assert val == codes[r, j]
    sc_off = dv * colb
    ng = dk // g
    sc = (raw[sc_off:sc_off + dv * ng * 2].view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(sc.reshape(dv, ng).T, scales.astype(np.float32))
    z_off = sc_off + ((dv * ng * 2 + 15) // 16) * 16
    for j in range(dv):
        for G in range(ng):
            e = j * ng + G
            if bits == 8:
                assert raw[z_off + e] == zeros[G, j]
            else:
                assert (raw[z_off + e // 2] >> (4 * (e % 2))) & 15 == zeros[G, j]
    # record sizes of the configurations the kernels run (no padding needed there)
    assert pk.record_parts(cfg, bits)[3] % 256 == 0


def test_record_sizes_of_named_configurations():
    p4 = pk.LayerCfg(B=1, Hv=1, Hk=1, dk=128, dv=128, group=64, asym=False, buf="int8", dP=8)
    assert pk.record_parts(p4, 4)[3] == 8704            # 8192 codes + 512 scale bytes
    p48 = pk.LayerCfg(B=1, Hv=1, Hk=1, dk=128, dv=128, group=32, asym=True, buf="int8", dP=8)
    assert pk.record_parts(p48, 4)[3] == 9472           # + 1024 scales + 256 zero bytes
    assert pk.record_parts(p48, 8)[3] == 17920
    tiny = pk.LayerCfg(B=1, Hv=1, Hk=1, dk=64, dv=64, group=32, asym=False, buf="int8", dP=8)
    assert pk.record_parts(tiny, 4)[3] == 2304

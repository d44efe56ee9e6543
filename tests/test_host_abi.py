"""CPU tests of the C ABI library: it loads, exports every symbol include/pace.h
declares, and its host-only entry points (layout, bit accounting, head allocation,
argument validation) agree with the oracle.  No kernel is launched here."""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import pace_oracle as po
from oracle import packing as pk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pace.h")


def _pace():
    import bit_recurrent_state_amd as pace
    return pace


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pace_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    pace = _pace()
    names = declared_functions()
    assert "pace_decode_step" in names and "pace_prefill_chunk" in names
    lib = ctypes.CDLL(pace.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in pace.h but not exported"
    assert set(pace.EXPORTS) == set(names)


CFGS = [
    dict(B=64, Hv=32, Hk=16, d=128, g=64, asym=False, buf="int8", dP=8, hb=None),
    dict(B=64, Hv=32, Hk=16, d=128, g=32, asym=True, buf="int8", dP=8, hb="quarter"),
    dict(B=64, Hv=32, Hk=16, d=128, g=32, asym=True, buf="mixed", dP=8, hb="quarter"),
    dict(B=2, Hv=4, Hk=4, d=64, g=32, asym=False, buf="int8", dP=8, hb=None),
    dict(B=3, Hv=8, Hk=2, d=64, g=32, asym=True, buf="mixed", dP=32, hb=[8, 4, 4, 8, 4, 4, 4, 4]),
]


def _cfgs(c):
    hb = c["hb"]
    if hb == "quarter":
        hb = [8 if h < c["Hv"] // 4 else 4 for h in range(c["Hv"])]
    pace = _pace()
    g = pace.LayerConfig(B=c["B"], Hv=c["Hv"], Hk=c["Hk"], dk=c["d"], dv=c["d"], group=c["g"],
                         asym=c["asym"], buf=c["buf"], dP=c["dP"], head_bits=hb)
    o = pk.LayerCfg(B=c["B"], Hv=c["Hv"], Hk=c["Hk"], dk=c["d"], dv=c["d"], group=c["g"],
                    asym=c["asym"], buf=c["buf"], dP=c["dP"], head_bits=hb)
    return g, o, hb


@pytest.mark.parametrize("c", CFGS)
def test_layout_and_accounting_agree_with_oracle(c):
    pace = _pace()
    g, o, hb = _cfgs(c)
    L = pace.layout(g)
    _, stride, total = pk.state_layout(o)
    _, btotal = pk.buffer_layout(o)
    assert L["state_bytes"] == total and L["seq_stride"] == stride
    assert L["buffer_bytes"] == btotal
    bits = hb if hb is not None else [4] * c["Hv"]
    assert L["payload_bits"] == pytest.approx(po.payload_bits(bits, c["g"], c["asym"]), abs=1e-12)
    assert L["buffer_bits_model"] == pytest.approx(
        po.buffer_bits_model(c["d"], c["d"], c["Hv"] // c["Hk"], c["dP"], c["buf"]), abs=1e-12)
    assert L["buffer_bits_actual"] == pytest.approx(btotal * 8 / (c["B"] * c["Hv"] * c["d"] ** 2))


def test_pace48_payload_is_the_printed_value():
    pace = _pace()
    g, _, _ = _cfgs(CFGS[1])
    assert abs(pace.layout(g)["payload_bits"] - 5.66) < 0.005


def test_head_alloc_matches_oracle():
    pace = _pace()
    rng = np.random.default_rng(0)
    for trial in range(50):
        H = int(rng.integers(1, 64))
        e = rng.uniform(0, 2, H)
        a = rng.uniform(0.3, 1.0, H)
        if trial % 5 == 0:
            a[0] = 1.0                     # no decay: infinite retained error
        if trial % 3 == 0 and H > 2:
            e[1], a[1] = e[2], a[2]        # tie
        n8 = po.quarter(H)
        bits, E = pace.head_alloc(e, a, 8, n8)
        rb, rE = po.head_alloc(e, a, 8, n8)
        assert bits.tolist() == rb.tolist()
        assert np.allclose(E[np.isfinite(rE)], rE[np.isfinite(rE)], rtol=1e-14)
        assert np.all(np.isinf(E) == np.isinf(rE))


def test_validation_errors():
    pace = _pace()
    bad = [
        dict(B=0), dict(Hk=3), dict(group=48), dict(dP=0),
    ]
    for kw in bad:
        c = pace.LayerConfig(B=2, Hv=4, Hk=4, dk=64, dv=64, group=32)
        for k, v in kw.items():
            setattr(c, k, v)
        with pytest.raises(pace.PaceError) as ei:
            pace.layout(c)
        assert ei.value.status == pace.PACE_EINVAL, kw
    unsupported = [dict(dk=96, dv=96, group=32), dict(dP=33), dict(Hv=128, Hk=128), dict(chunk=100),
                   dict(dk=128, dv=64),
                   # asymmetric 4-bit zero points are packed two a byte within a column, so
                   # the number of groups per column must be even
                   dict(group=64, asym=True)]
    for kw in unsupported:
        c = pace.LayerConfig(B=2, Hv=4, Hk=4, dk=64, dv=64, group=32)
        for k, v in kw.items():
            setattr(c, k, v)
        with pytest.raises(pace.PaceError) as ei:
            pace.layout(c)
        assert ei.value.status == pace.PACE_EUNSUPPORTED, kw
    for chunk in (64, 128, 512):                 # prefill rounding periods: multiples of 64
        pace.layout(pace.LayerConfig(B=2, Hv=4, Hk=4, dk=64, dv=64, group=32, chunk=chunk))
    c = pace.LayerConfig(B=2, Hv=4, Hk=4, dk=64, dv=64, group=32, head_bits=[4, 5, 4, 4])
    with pytest.raises(pace.PaceError):
        pace.layout(c)
    with pytest.raises(pace.PaceError):
        pace.head_alloc([1.0, -1.0], [0.9, 0.9], 8, 1)
    with pytest.raises(pace.PaceError):
        pace.head_alloc([1.0, 1.0], [0.9, 0.0], 8, 1)


def test_null_pointers_rejected_before_any_launch():
    pace = _pace()
    c = pace.LayerConfig(B=2, Hv=4, Hk=4, dk=64, dv=64, group=32)._c()
    L = pace._lib
    st = L.LIB.pace_decode_step(ctypes.byref(c), None, None, None, None, None, None, None, None, None, None)
    assert st == pace.PACE_EINVAL
    st = L.LIB.pace_flush_requant(ctypes.byref(c), None, None, None, None)
    assert st == pace.PACE_EINVAL
    st = L.LIB.pace_prefill_chunk(ctypes.byref(c), None, None, None, None, None, None, 4, None, None, 0, None)
    assert st == pace.PACE_EINVAL
    st = L.LIB.pace_bf16_decode_step(ctypes.byref(c), None, None, None, None, None, None, None, None)
    assert st == pace.PACE_EINVAL
    # misaligned (fake, never dereferenced) pointers
    fake = ctypes.c_void_p(0x1001)
    st = L.LIB.pace_decode_step(ctypes.byref(c), fake, fake, fake, fake, fake, fake, fake, None, fake, None)
    assert st == pace.PACE_EINVAL
    assert L.LIB.pace_status_str(-2).decode().startswith("PACE_EUNSUPPORTED")


def test_sequence_order_validated_before_any_launch():
    """pace_decode_step_ordered takes a host permutation of the B sequences; anything else
    is refused on the host (aligned stand-in device pointers, never dereferenced)."""
    pace = _pace()
    L = pace._lib
    fake = ctypes.c_void_p(0x10000)

    def call(B, order, d=128, bf16_io=True, dP=8):
        c = pace.LayerConfig(B=B, Hv=4, Hk=4, dk=d, dv=d, group=32, bf16_io=bf16_io, dP=dP)._c()
        ptr = None if order is None else np.asarray(order, dtype=np.int32).ctypes.data_as(
            ctypes.POINTER(ctypes.c_int32))
        return L.LIB.pace_decode_step_ordered(ctypes.byref(c), fake, fake, fake, fake, fake, fake, fake,
                                              None, ptr, fake, None)

    assert call(4, None) == pace.PACE_EINVAL
    assert call(4, [0, 1, 1, 3]) == pace.PACE_EINVAL       # repeated sequence
    assert call(4, [0, 1, 2, 4]) == pace.PACE_EINVAL       # index past B
    assert call(4, [-1, 0, 1, 2]) == pace.PACE_EINVAL
    assert call(300, list(range(300))) == pace.PACE_EUNSUPPORTED
    # layouts whose kernels do not apply an order are refused, never run in launch order
    assert call(4, [3, 2, 1, 0], d=64) == pace.PACE_EUNSUPPORTED
    assert call(4, [3, 2, 1, 0], bf16_io=False) == pace.PACE_EUNSUPPORTED
    assert call(4, [3, 2, 1, 0], dP=12) == pace.PACE_EUNSUPPORTED
    with pytest.raises(ValueError):
        pace._lib._order(pace.LayerConfig(B=4, Hv=4, Hk=4, dk=64, dv=64, group=32), [0, 1, 2])


def test_prefill_workspace_query_distinguishes_errors_from_zero():
    """pace_prefill_workspace_bytes returns a status: an invalid or unsupported
    configuration is an error (and writes nothing), a valid one writes its size."""
    pace = _pace()
    L = pace._lib
    out = ctypes.c_size_t(12345)
    good = pace.LayerConfig(B=2, Hv=4, Hk=4, dk=64, dv=64, group=32)._c()
    assert L.LIB.pace_prefill_workspace_bytes(ctypes.byref(good), 256, ctypes.byref(out)) == pace.PACE_OK
    assert out.value == 0                     # the kernels keep every intermediate on chip
    out.value = 12345
    bad = pace.LayerConfig(B=2, Hv=4, Hk=3, dk=64, dv=64, group=32)._c()        # Hv % Hk != 0
    assert L.LIB.pace_prefill_workspace_bytes(ctypes.byref(bad), 256, ctypes.byref(out)) == pace.PACE_EINVAL
    uns = pace.LayerConfig(B=2, Hv=4, Hk=4, dk=96, dv=96, group=32)._c()        # no kernel for d = 96
    assert L.LIB.pace_prefill_workspace_bytes(ctypes.byref(uns), 256, ctypes.byref(out)) == pace.PACE_EUNSUPPORTED
    assert L.LIB.pace_prefill_workspace_bytes(ctypes.byref(good), 0, ctypes.byref(out)) == pace.PACE_EINVAL
    assert L.LIB.pace_prefill_workspace_bytes(ctypes.byref(good), 256, None) == pace.PACE_EINVAL
    assert out.value == 12345
    with pytest.raises(pace.PaceError):
        pace.prefill_workspace_bytes(pace.LayerConfig(B=2, Hv=4, Hk=3, dk=64, dv=64, group=32), 256)


def test_bf16_state_layout_matches_the_oracles():
    """PACE_STATE_BF16: one dv x dk bf16 record per (sequence, head), 16 payload bits, no
    head map, int8 buffer only; the sizes agree with the oracle's byte layout."""
    pace = _pace()
    for d, B, Hv, Hk in [(128, 64, 32, 16), (64, 3, 4, 2)]:
        g = pace.LayerConfig(B=B, Hv=Hv, Hk=Hk, dk=d, dv=d, group=64, buf="int8", bf16_state=True)
        o = pk.LayerCfg(B=B, Hv=Hv, Hk=Hk, dk=d, dv=d, group=64, asym=False, buf="int8", dP=8, bf16_state=True)
        L = pace.layout(g)
        offs, stride, total = pk.state_layout(o)
        assert L["state_bytes"] == total and L["seq_stride"] == stride == Hv * d * d * 2
        assert L["buffer_bytes"] == pk.buffer_layout(o)[1]
        assert L["payload_bits"] == 16.0
    with pytest.raises(pace.PaceError) as e:
        pace.layout(pace.LayerConfig(B=2, Hv=4, Hk=2, dk=128, dv=128, group=64, buf="mixed", bf16_state=True))
    assert e.value.status == pace.PACE_EUNSUPPORTED
    with pytest.raises(pace.PaceError) as e:
        pace.layout(pace.LayerConfig(B=2, Hv=4, Hk=2, dk=128, dv=128, group=64, bf16_state=True, head_bits=[4] * 4))
    assert e.value.status == pace.PACE_EINVAL
    with pytest.raises(pace.PaceError) as e:
        pace.prefill_workspace_bytes(pace.bf16_periodic(B=2, Hv=4, Hk=2), 256)
    assert e.value.status == pace.PACE_EUNSUPPORTED


def test_measurement_library_exports_its_header():
    """libpace_measure.so (the launch-floor and streaming-ceiling kernels bench.py times)
    exports every function include/pace_measure.h declares, and refuses bad shapes on the
    host (no launch happens for an invalid call)."""
    path = os.path.join(ROOT, "bit_recurrent_state_amd", "libpace_measure.so")
    _pace()                                   # torch's HIP runtime first (see the binding)
    lib = ctypes.CDLL(path)
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "pace_measure.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(pace_[a-z0-9_]+)\s*\(", text)))
    assert names == ["pace_measure_empty", "pace_measure_stream"]
    for n in names:
        assert hasattr(lib, n)
    lib.pace_measure_empty.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    assert lib.pace_measure_empty(0, 1, 128, None) == -1
    assert lib.pace_measure_empty(1, 1, 100, None) == -1
    lib.pace_measure_stream.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    assert lib.pace_measure_stream(None, 4096, 32, 64, 128, ctypes.c_void_p(0x1000), None) == -1
    assert lib.pace_measure_stream(ctypes.c_void_p(0x1008), 4096, 32, 64, 128, ctypes.c_void_p(0x1000), None) == -1
    assert lib.pace_measure_stream(ctypes.c_void_p(0x1000), 4100, 32, 64, 128, ctypes.c_void_p(0x1000), None) == -1

"""GPU parity of pace_decode_step / pace_flush_requant / pace_bf16_decode_step against the
fp64 oracle, called through the C ABI on identical seeded inputs.

Every case starts both sides from the same packed state and decode buffer (seeded random
fields: any stored code is a legal state) and runs ONE call; the oracle never sees a
GPU result.  Counts are random per sequence so both the append-only and the flushing
paths run in every launch."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import pace_oracle as po  # noqa: E402
from oracle import packing as pk  # noqa: E402
from pace_synth import make_tokens, random_buffer_parts, random_packed_state_parts  # noqa: E402
import parity  # noqa: E402

pytestmark = pytest.mark.gpu


def _lib():
    import bit_recurrent_state_amd as pace
    return pace


def dev(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def io_dev(x, bf16):
    return dev(np.asarray(x, dtype=np.float32), torch.bfloat16 if bf16 else torch.float32)


def host(t):
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy()


CASES = {
    # name: (B, Hv, Hk, d, group, asym, buf, bf16_io, dP, head_bits)
    "tiny_sym4_g32_int8": (2, 4, 4, 64, 32, False, "int8", False, 8, None),
    "pace4_g64_int8": (6, 32, 16, 128, 64, False, "int8", True, 8, None),
    "pace48_g32_int8": (4, 32, 16, 128, 32, True, "int8", True, 8, "quarter"),
    "pace48_g32_mixed": (4, 32, 16, 128, 32, True, "mixed", True, 8, "quarter"),
    "d64_asym_mixed_f32": (3, 8, 4, 64, 32, True, "mixed", False, 5, [8, 4, 4, 8, 4, 4, 4, 8]),
    "dP1_sym_int8": (2, 4, 2, 128, 32, False, "int8", True, 1, None),
    "dP16_sym_int8": (2, 4, 2, 64, 32, False, "int8", True, 16, None),
    "dP32_asym_int8": (2, 4, 2, 64, 32, True, "int8", False, 32, [4, 8, 4, 4]),
    "sym8_heads": (2, 4, 2, 128, 64, False, "int8", True, 8, [8, 8, 4, 8]),
    # asymmetric 64-key groups (two 32-key MFMA blocks per group); symmetric state with the
    # mixed buffer
    "asym_g64_int8": (2, 8, 4, 128, 64, True, "int8", True, 8, [4, 8, 4, 4, 8, 4, 4, 4]),
    "sym4_g64_mixed": (2, 8, 4, 128, 64, False, "mixed", True, 8, None),
    # asymmetric 32-key groups with every head at 4 bits (no 8-bit heads)
    "asym_g32_4bit_int8": (2, 8, 4, 128, 32, True, "int8", True, 8, None),
    # general kernels: fp32 I/O at d = 128 (both buffers), a 32-slot buffer at d = 128, the
    # mixed buffer with bf16 I/O at d = 64
    "d128_f32_sym_g64_mixed": (2, 4, 2, 128, 64, False, "mixed", False, 8, None),
    "d128_f32_asym_g32_int8": (2, 4, 2, 128, 32, True, "int8", False, 8, None),
    "d128_dP12_asym_int8": (2, 4, 2, 128, 32, True, "int8", True, 12, [4, 8, 4, 4]),
    "d64_bf16_asym_mixed": (2, 4, 2, 64, 32, True, "mixed", True, 8, [8, 4, 4, 4]),
}


def make_case(name, seed, counts=None):
    B, Hv, Hk, d, g, asym, buf, bf16, dP, hb = CASES[name]
    if hb == "quarter":
        hb = [8 if h % 4 == 1 else 4 for h in range(Hv)]
    ocfg = pk.LayerCfg(B=B, Hv=Hv, Hk=Hk, dk=d, dv=d, group=g, asym=asym, buf=buf, dP=dP,
                       bf16_io=bf16, head_bits=hb)
    pace = _lib()
    gcfg = pace.LayerConfig(B=B, Hv=Hv, Hk=Hk, dk=d, dv=d, group=g, asym=asym, buf=buf,
                            bf16_io=bf16, dP=dP, head_bits=hb)
    bits = [ocfg.bits(h) for h in range(Hv)]
    parts = random_packed_state_parts(seed, B, Hv, d, d, g, bits, asym)
    state = pk.pack_state(ocfg, pk.state_from_parts(ocfg, parts))
    if counts is None:
        rng = np.random.default_rng(seed + 7)
        counts = rng.integers(0, dP, size=B)
        counts[0] = dP - 1                    # at least one flushing sequence
    bufp = random_buffer_parts(seed + 1, B, Hv, Hk, d, d, dP, buf == "mixed", counts=counts)
    buffer = pk.pack_buffer(ocfg, bufp)
    toks = make_tokens(seed + 2, B, 1, Hv, Hk, d, d, bf16=bf16)
    return ocfg, gcfg, state, buffer, toks


def run_gpu_decode(gcfg, state, buffer, toks, active=None, order=None):
    pace = _lib()
    q, k, v, a, beta = toks.token(0)
    bf16 = gcfg.bf16_io
    st = dev(state)
    bu = dev(buffer)
    o = torch.full((gcfg.B, gcfg.Hv, gcfg.dv), float("nan"),
                   dtype=torch.bfloat16 if bf16 else torch.float32, device="cuda")
    act = dev(np.asarray(active, dtype=np.uint8)) if active is not None else None
    pace.decode_step(gcfg, st, bu, io_dev(q, bf16), io_dev(k, bf16), io_dev(v, bf16), dev(a), dev(beta), o,
                     active=act, order=order)
    torch.cuda.synchronize()
    return host(o), st.cpu().numpy(), bu.cpu().numpy()


def compare_buffers(ocfg, b_gpu, b_ref, tiles):
    dg, dr = pk.unpack_buffer(ocfg, b_gpu), pk.unpack_buffer(ocfg, b_ref)
    assert np.array_equal(dg["count"], dr["count"]), "buffer counts differ"
    for b, h in tiles:
        n = int(dr["count"][b, h])
        kh = h // ocfg.gamma
        for key in ("a", "beta"):
            assert np.array_equal(dg[key][b, h, :n], dr[key][b, h, :n]), key
        assert np.array_equal(dg["kc"][b, kh, :n], dr["kc"][b, kh, :n]), f"k codes (b={b},kh={kh})"
        assert np.array_equal(dg["ks"][b, kh, :n], dr["ks"][b, kh, :n]), "k scales"
        if ocfg.buf == "int8":
            assert np.array_equal(dg["vc"][b, h, :n], dr["vc"][b, h, :n]), "v codes"
            assert np.array_equal(dg["vs"][b, h, :n], dr["vs"][b, h, :n]), "v scales"
        else:
            assert np.array_equal(dg["v"][b, h, :n], dr["v"][b, h, :n]), "bf16 v"


def check_states(ocfg, s_gpu, s_in, pre, tiles, label):
    offs, stride, _ = pk.state_layout(ocfg)
    qg = pk.unpack_state(ocfg, s_gpu, list(pre.keys()))
    parity.check_flushed_tiles(pre, qg, label)
    for b, h in tiles:
        if (b, h) in pre:
            continue
        o = b * stride + offs[h]
        n = pk.record_parts(ocfg, ocfg.bits(h))[3]
        assert np.array_equal(s_gpu[o:o + n], s_in[o:o + n]), f"{label} untouched state changed (b={b},h={h})"


@pytest.mark.parametrize("name", list(CASES))
def test_decode_step_matches_oracle(name):
    print(f"[decode parity] case={name}", flush=True)
    ocfg, gcfg, state, buffer, toks = make_case(name, seed=100 + len(name))
    o_ref, s_ref, b_ref, pre = pk.decode_step_layer(ocfg, state, buffer, *toks.token(0))
    o_gpu, s_gpu, b_gpu = run_gpu_decode(gcfg, state, buffer, toks)
    tiles = [(b, h) for b in range(ocfg.B) for h in range(ocfg.Hv)]
    parity.check_outputs(o_gpu, o_ref, tiles, name, out_bf16=ocfg.bf16_io)
    compare_buffers(ocfg, b_gpu, b_ref, tiles)
    assert len(pre) > 0
    check_states(ocfg, s_gpu, state, pre, tiles, name)


FULL = {
    # name: (B, Hv, Hk, d, group, asym, buf, head_bits) -- the benchmark's layer shapes
    "pace4_b64": (64, 32, 16, 128, 64, False, "int8", None),
    "pace4_b128": (128, 32, 16, 128, 64, False, "int8", None),
    # more tiles than one round of resident workgroups (eight per CU): a ragged second round
    "pace4_b65_asym_g32": (65, 32, 16, 128, 32, True, "int8", None),
    "pace48_int8_b64": (64, 32, 16, 128, 32, True, "int8", "quarter"),
    "pace48_mixed_b64": (64, 32, 16, 128, 32, True, "mixed", "quarter"),
}


@pytest.mark.parametrize("name", list(FULL))
def test_decode_full_size_sampled(name):
    """One pace_decode_step at the benchmark's full layer size (grid of 32 value heads x B
    sequences, bf16, dP = 8) with random per-sequence counts.  Sampled tiles (both value
    heads of a key head, flushing and appending sequences) are compared with the oracle;
    every tile's count is checked against the rule count' = count + 1, or 0 on a flush."""
    full_size_case(name, ordered=False)


@pytest.mark.parametrize("name", ["pace4_b64", "pace48_int8_b64"])
def test_ordered_decode_full_size_sampled(name):
    """The same at full size through pace_decode_step_ordered, in the launch configuration
    of the benchmark's continuous-batching leg: the sequences that flush at this step
    placed first, the others after them."""
    full_size_case(name, ordered=True)


def test_decode_full_size_two_rounds_with_inactive_sequences():
    """B = 128 (4096 tiles: two rounds of resident workgroups) with an active mask that idles
    sequences in both rounds."""
    active = np.ones(128, dtype=np.uint8)
    active[[0, 3, 64 + 1, 64 + 3, 10, 74]] = 0
    full_size_case("pace4_b128", ordered=False, active=active)


def full_size_case(name, ordered, active=None):
    print(f"[decode full size] case={name} ordered={ordered} active_mask={active is not None}", flush=True)
    B, Hv, Hk, d, g, asym, buf, hb = FULL[name]
    if hb == "quarter":
        hb = [8 if h % 4 == 1 else 4 for h in range(Hv)]
    dP = 8
    ocfg = pk.LayerCfg(B=B, Hv=Hv, Hk=Hk, dk=d, dv=d, group=g, asym=asym, buf=buf, dP=dP,
                       bf16_io=True, head_bits=hb)
    gcfg = _lib().LayerConfig(B=B, Hv=Hv, Hk=Hk, dk=d, dv=d, group=g, asym=asym, buf=buf,
                              bf16_io=True, dP=dP, head_bits=hb)
    seed = 500 + len(name)
    bits = [ocfg.bits(h) for h in range(Hv)]
    state = pk.pack_state(ocfg, pk.state_from_parts(ocfg, random_packed_state_parts(seed, B, Hv, d, d, g, bits, asym)))
    counts = np.random.default_rng(seed + 7).integers(0, dP, size=B)
    counts[::5] = dP - 1                               # a fifth of the sequences flush
    buffer = pk.pack_buffer(ocfg, random_buffer_parts(seed + 1, B, Hv, Hk, d, d, dP, buf == "mixed", counts=counts))
    toks = make_tokens(seed + 2, B, 1, Hv, Hk, d, d, bf16=True)
    seqs = [0, 1, 2, B // 2, B // 2 + 1, B // 2 + 3, B - 1]
    if active is not None:
        # (every fifth sequence flushes: 5, 70 and 75 flush in active tiles)
        seqs = sorted(set(seqs) | {1, 2, 3, 4, 5, 64, 65, 66, 67, 68, 69, 70, 75})
    tiles = [(b, h) for b in seqs for h in (0, 1, 14, 15, Hv - 2, Hv - 1)]
    o_ref, s_ref, b_ref, pre = pk.decode_step_layer(ocfg, state, buffer, *toks.token(0), tiles=tiles,
                                                    active=active)
    order = None
    if ordered:
        flushing = np.asarray(counts) == dP - 1
        order = np.concatenate([np.flatnonzero(flushing), np.flatnonzero(~flushing)])
    o_gpu, s_gpu, b_gpu = run_gpu_decode(gcfg, state, buffer, toks, order=order, active=active)
    live = [(b, h) for b, h in tiles if active is None or active[b]]
    parity.check_outputs(o_gpu, o_ref, live, name, out_bf16=True)
    if active is not None:
        for b in np.flatnonzero(np.asarray(active) == 0):
            assert np.isnan(o_gpu[b]).all(), f"inactive output written (b={b})"
    assert len(pre) > 0
    qg = pk.unpack_state(ocfg, s_gpu, list(pre.keys()))
    parity.check_flushed_tiles(pre, qg, name)
    dg, dr = pk.unpack_buffer(ocfg, b_gpu), pk.unpack_buffer(ocfg, b_ref)
    for b, h in tiles:
        n = int(dr["count"][b, h])
        assert dg["count"][b, h] == n
        kh = h // ocfg.gamma
        for key in ("a", "beta"):
            assert np.array_equal(dg[key][b, h, :n], dr[key][b, h, :n]), key
        assert np.array_equal(dg["kc"][b, kh, :n], dr["kc"][b, kh, :n]), f"k codes (b={b},kh={kh})"
        assert np.array_equal(dg["ks"][b, kh, :n], dr["ks"][b, kh, :n]), "k scales"
        if buf == "int8":
            assert np.array_equal(dg["vc"][b, h, :n], dr["vc"][b, h, :n]), "v codes"
            assert np.array_equal(dg["vs"][b, h, :n], dr["vs"][b, h, :n]), "v scales"
        else:
            assert np.array_equal(dg["v"][b, h, :n], dr["v"][b, h, :n]), "bf16 v"
    old = np.repeat(np.asarray(counts)[:, None], Hv, axis=1)
    want = np.where(old + 1 >= dP, 0, old + 1)
    if active is not None:
        want = np.where(np.asarray(active)[:, None] != 0, want, old)
        offs, stride, _ = pk.state_layout(ocfg)
        n = pk.record_parts(ocfg, 4)[3]
        for b in np.flatnonzero(np.asarray(active) == 0):
            for h in range(Hv):
                o = b * stride + offs[h]
                assert np.array_equal(s_gpu[o:o + n], state[o:o + n]), f"inactive state changed (b={b},h={h})"
    assert np.array_equal(dg["count"], want), "count rule violated"


def test_flush_full_size_b128():
    """pace_flush_requant at B = 128 (two rounds of resident workgroups) under a sequence
    mask, with sequences holding nothing to flush: every flushed tile matches the oracle,
    every other state byte is untouched, the counts follow the mask."""
    print("[flush full size] B=128 pace4", flush=True)
    B, Hv, Hk, d, g, asym, buf, _ = FULL["pace4_b128"]
    dP = 8
    ocfg = pk.LayerCfg(B=B, Hv=Hv, Hk=Hk, dk=d, dv=d, group=g, asym=asym, buf=buf, dP=dP, bf16_io=True)
    gcfg = _lib().LayerConfig(B=B, Hv=Hv, Hk=Hk, dk=d, dv=d, group=g, asym=asym, buf=buf, bf16_io=True, dP=dP)
    seed = 911
    state = pk.pack_state(ocfg, pk.state_from_parts(ocfg, random_packed_state_parts(seed, B, Hv, d, d, g,
                                                                                     [4] * Hv, asym)))
    counts = np.random.default_rng(seed + 7).integers(1, dP, size=B)
    counts[[0, 64, 5, 70, 71]] = 0                    # nothing buffered
    buffer = pk.pack_buffer(ocfg, random_buffer_parts(seed + 1, B, Hv, Hk, d, d, dP, False, counts=counts))
    mask = np.array([0 if b % 7 == 3 else 1 for b in range(B)], dtype=np.uint8)
    seqs = [0, 1, 2, 3, 4, 5, 6, 64, 65, 66, 67, 69, 70, 127]
    tiles = [(b, h) for b in seqs for h in (0, 1, 14, 15, Hv - 1)]
    s_ref, b_ref, pre = pk.flush_layer(ocfg, state, buffer, seq_mask=mask, tiles=tiles)
    pace = _lib()
    st, bu = dev(state), dev(buffer)
    pace.flush_requant(gcfg, st, bu, seq_mask=dev(mask))
    torch.cuda.synchronize()
    s_gpu, b_gpu = st.cpu().numpy(), bu.cpu().numpy()
    assert len(pre) > 0
    check_states(ocfg, s_gpu, state, pre, tiles, "flush b128")
    want = np.where((mask[:, None] != 0), 0, np.repeat(counts[:, None], Hv, axis=1))
    assert np.array_equal(pk.unpack_buffer(ocfg, b_gpu)["count"], want), "flush count rule violated"
    _, stride, _ = pk.state_layout(ocfg)
    for b in range(B):
        if mask[b] and counts[b] > 0:
            continue
        assert np.array_equal(s_gpu[b * stride:(b + 1) * stride], state[b * stride:(b + 1) * stride]), \
            f"state of a sequence with nothing to flush changed (b={b})"


def test_decode_inactive_sequences_untouched():
    print("[decode parity] active mask", flush=True)
    ocfg, gcfg, state, buffer, toks = make_case("pace4_g64_int8", seed=7)
    active = [1, 0, 1, 0, 0, 1]
    o_ref, s_ref, b_ref, pre = pk.decode_step_layer(ocfg, state, buffer, *toks.token(0), active=active)
    o_gpu, s_gpu, b_gpu = run_gpu_decode(gcfg, state, buffer, toks, active=active)
    tiles = [(b, h) for b in range(ocfg.B) if active[b] for h in range(ocfg.Hv)]
    parity.check_outputs(o_gpu, o_ref, tiles, "active", out_bf16=ocfg.bf16_io)
    for b in range(ocfg.B):
        if not active[b]:
            assert np.isnan(o_gpu[b]).all(), "inactive output written"
    compare_buffers(ocfg, b_gpu, b_ref, [(b, h) for b in range(ocfg.B) for h in range(ocfg.Hv)])
    check_states(ocfg, s_gpu, state, pre, [(b, h) for b in range(ocfg.B) for h in range(ocfg.Hv)], "active")


@pytest.mark.parametrize("name", ["pace4_g64_int8", "pace48_g32_mixed", "pace48_g32_int8", "sym4_g64_mixed"])
def test_ordered_decode_equals_unordered(name):
    """pace_decode_step_ordered (continuous batching: the sequences that flush at this step
    placed first) gives the results of pace_decode_step bit for bit -- outputs, packed
    state and buffer -- for a random order, with and without an active mask; the outputs
    also match the oracle."""
    print(f"[ordered decode] case={name}", flush=True)
    ocfg, gcfg, state, buffer, toks = make_case(name, seed=300 + len(name))
    B = gcfg.B
    order = np.random.default_rng(5 + B).permutation(B)
    o_ref, _, _, _ = pk.decode_step_layer(ocfg, state, buffer, *toks.token(0))
    for active in (None, [1 if b % 3 else 0 for b in range(B)]):
        o1, s1, b1 = run_gpu_decode(gcfg, state, buffer, toks, active=active)
        o2, s2, b2 = run_gpu_decode(gcfg, state, buffer, toks, active=active, order=order)
        both_nan = np.isnan(o1) & np.isnan(o2)          # rows of inactive sequences stay unwritten
        assert np.array_equal(np.where(both_nan, 0, o1), np.where(both_nan, 0, o2)), "outputs differ"
        assert np.array_equal(s1, s2), "packed state differs"
        assert np.array_equal(b1, b2), "buffer differs"
    tiles = [(b, h) for b in range(B) for h in range(gcfg.Hv)]
    o2, _, _ = run_gpu_decode(gcfg, state, buffer, toks, order=order)
    parity.check_outputs(o2, o_ref, tiles, name + "/ordered", out_bf16=ocfg.bf16_io)


def test_ordered_decode_refused_where_no_kernel_orders():
    """Layouts served by the general kernels (here d = 64 with fp32 I/O) cannot place the
    sequences in a given order, so pace_decode_step_ordered refuses them before any launch
    instead of running them in launch order."""
    ocfg, gcfg, state, buffer, toks = make_case("d64_asym_mixed_f32", seed=31)
    pace = _lib()
    with pytest.raises(pace.PaceError) as e:
        run_gpu_decode(gcfg, state, buffer, toks, order=list(range(gcfg.B))[::-1])
    assert e.value.status == pace.PACE_EUNSUPPORTED


@pytest.mark.parametrize("name", ["pace4_g64_int8", "pace48_g32_mixed", "d64_asym_mixed_f32", "asym_g64_int8",
                                  "d128_f32_asym_g32_int8"])
def test_flush_requant_matches_oracle(name):
    print(f"[flush parity] case={name}", flush=True)
    ocfg, gcfg, state, buffer, _ = make_case(name, seed=300 + len(name))
    d = pk.unpack_buffer(ocfg, buffer)
    mask = np.array([1 if b % 3 != 1 else 0 for b in range(ocfg.B)], dtype=np.uint8)
    s_ref, b_ref, pre = pk.flush_layer(ocfg, state, buffer, seq_mask=mask)
    pace = _lib()
    st, bu = dev(state), dev(buffer)
    pace.flush_requant(gcfg, st, bu, seq_mask=dev(mask))
    torch.cuda.synchronize()
    s_gpu, b_gpu = st.cpu().numpy(), bu.cpu().numpy()
    dg = pk.unpack_buffer(ocfg, b_gpu)
    assert np.array_equal(dg["count"], pk.unpack_buffer(ocfg, b_ref)["count"])
    tiles = [(b, h) for b in range(ocfg.B) for h in range(ocfg.Hv)]
    check_states(ocfg, s_gpu, state, pre, tiles, name)
    assert any(d["count"][b, 0] > 0 and mask[b] for b in range(ocfg.B))


def test_decode_zero_state_zero_inputs_gives_zero():
    """Special case of the recurrence: S = 0 and v = 0 keep everything at zero."""
    print("[decode parity] zero state", flush=True)
    ocfg, gcfg, _, _, toks = make_case("pace4_g64_int8", seed=9)
    pace = _lib()
    L = pace.layout(gcfg)
    st = torch.zeros(L["state_bytes"], dtype=torch.uint8, device="cuda")
    bu = torch.zeros(L["buffer_bytes"], dtype=torch.uint8, device="cuda")
    q, k, v, a, beta = toks.token(0)
    o = torch.empty((gcfg.B, gcfg.Hv, gcfg.dv), dtype=torch.bfloat16, device="cuda")
    for step in range(gcfg.dP):
        pace.decode_step(gcfg, st, bu, io_dev(q, True), io_dev(k, True), io_dev(0 * v, True), dev(a),
                         dev(beta), o)
        torch.cuda.synchronize()
        assert torch.count_nonzero(o.float()).item() == 0
    d = pk.unpack_buffer(ocfg, bu.cpu().numpy())
    assert np.all(d["count"] == 0)
    qs = pk.unpack_state(ocfg, st.cpu().numpy(), [(0, 0), (5, 31)])
    for b, h in [(0, 0), (5, 31)]:
        assert np.all(qs[b][h].scales == 0)


def _bf16_ref_step(S, q, k, v, a, beta):
    """Per-token bf16 baseline, fp64: u = beta (v - a S^T k); S' = a S + k u^T; o = S'^T q."""
    S2, _ = po.exact_step(S, k, v, a, beta)
    return S2, po.readout(S2, q)


def bf16_state_bits_check(S_gpu, S_new, S_old, k, v, a, beta):
    """Stored bf16 state against round-to-nearest-even of the oracle's fp64 update.

    The kernel forms S' in fp32 and rounds that to bf16.  The fp32 evaluation error bound
    of an element is 2^-18 of the magnitudes that enter it, a_t |S_ij| + |k_i| beta (|v_j| +
    a_t sum_k |S_kj k_k|) (64 fp32 ulps of the largest term): for an ordinary element a
    small fraction of a bf16 ulp, so only a value close to a rounding midpoint may land on
    the other neighbour, while truncation or rounding away from zero fail."""
    Sabs = np.abs(S_old)
    U = beta * (np.abs(v) + a * (Sabs.T @ np.abs(k)))                 # [dv]
    tol = 2.0 ** -18 * (a * Sabs + np.outer(np.abs(k), U))
    return parity.check_bf16_rounding(S_gpu, S_new, tol, "bf16 baseline")


# (the 8 x 32-head case holds 8 MiB of bf16 state, where the kernel streams the state with
# non-temporal accesses; the others use ordinary accesses)
@pytest.mark.parametrize("bf16_io,d,B,Hv,Hk", [(True, 128, 3, 8, 4), (False, 64, 3, 8, 4), (True, 128, 8, 32, 16)])
def test_bf16_baseline_matches_oracle(bf16_io, d, B, Hv, Hk):
    print(f"[bf16 baseline parity] d={d} B={B} Hv={Hv}", flush=True)
    rng = np.random.default_rng(d)
    S = po.bf16_rne(rng.standard_normal((B, Hv, d, d)) * 0.3)        # [b, h, col, key]
    toks = make_tokens(d + 1, B, 1, Hv, Hk, d, d, bf16=bf16_io)
    q, k, v, a, beta = toks.token(0)
    pace = _lib()
    cfg = pace.LayerConfig(B=B, Hv=Hv, Hk=Hk, dk=d, dv=d, group=32, bf16_io=bf16_io)
    st = dev(S.astype(np.float32), torch.bfloat16)
    o = torch.empty((B, Hv, d), dtype=torch.bfloat16 if bf16_io else torch.float32, device="cuda")
    pace.bf16_decode_step(cfg, st, io_dev(q, bf16_io), io_dev(k, bf16_io), io_dev(v, bf16_io), dev(a), dev(beta), o)
    torch.cuda.synchronize()
    S_gpu = host(st).astype(np.float64)
    o_gpu = host(o)
    flips = 0
    for b in range(B):
        for h in range(Hv):
            kh = h // (Hv // Hk)
            S_old = S[b, h].T                                           # [key, col]
            S2, oo = _bf16_ref_step(S_old, q[b, kh], k[b, kh], v[b, h], float(a[b, h]), float(beta[b, h]))
            assert parity.rel_err_io(o_gpu[b, h], oo, bf16_io) <= parity.TOL_REL
            flips += bf16_state_bits_check(S_gpu[b, h].T, S2, S_old, np.asarray(k[b, kh], np.float64),
                                           np.asarray(v[b, h], np.float64), float(a[b, h]), float(beta[b, h]))
    n = B * Hv * d * d
    print(f"[bf16 baseline parity] {flips} rounding-window flips in {n} stored values", flush=True)
    assert flips <= 1e-4 * n + 1


def test_library_imported_before_torch_launches_on_torch_memory():
    """The binding loads torch's HIP runtime before libpace.so, so that a program that
    imports this package first still launches the kernels on the runtime that owns its
    tensors (two HIP runtimes in one process would reject the launch)."""
    import subprocess
    import sys
    import os
    code = (
        "import bit_recurrent_state_amd as pace\n"
        "import torch\n"
        "cfg = pace.pace4(B=2, Hv=4, Hk=2)\n"
        "L = pace.layout(cfg)\n"
        "st = torch.zeros(L['state_bytes'], dtype=torch.uint8, device='cuda')\n"
        "bu = torch.zeros(L['buffer_bytes'], dtype=torch.uint8, device='cuda')\n"
        "g = torch.Generator(device='cuda'); g.manual_seed(0)\n"
        "q = torch.randn((2, 2, 128), device='cuda', generator=g).to(torch.bfloat16)\n"
        "k = torch.randn((2, 2, 128), device='cuda', generator=g).to(torch.bfloat16)\n"
        "v = torch.randn((2, 4, 128), device='cuda', generator=g).to(torch.bfloat16)\n"
        "a = torch.full((2, 4), 0.9, device='cuda'); b = torch.full((2, 4), 0.5, device='cuda')\n"
        "o = torch.zeros((2, 4, 128), dtype=torch.bfloat16, device='cuda')\n"
        "pace.decode_step(cfg, st, bu, q, k, v, a, b, o)\n"
        "torch.cuda.synchronize()\n"
        "assert torch.isfinite(o.float()).all() and o.float().abs().sum() > 0\n"
        "print('import order OK')\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300, cwd=root)
    assert r.returncode == 0 and "import order OK" in r.stdout, (r.stdout + r.stderr)[-3000:]

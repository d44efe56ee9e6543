"""GPU parity of periodic decode on a bf16 state (PACE_STATE_BF16: the int8 decode buffer and
once-per-dP fold with the state kept as bf16 values; [p1] "Assumptions and limits") against
the fp64 oracle, through the C ABI on identical seeded inputs.

Checked: every output o_t (2e-3 of the slice), the appended buffer slot bit for bit, the
count rule, untouched states of tiles that did not flush, and every flushed state: each
stored bf16 value is round-to-nearest-even of the oracle's fp32 pre-rounding value, except
where that value lies within the fp32 accumulation error of a rounding boundary (counted,
and bounded by deviation_budget).
The multi-step case runs the benchmark's layer size (B = 64, 32 value heads over 16 key
heads, d = 128, bf16 I/O) for 64 steps on the column-outlier stream, teacher-forced after
every flush."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import pace_oracle as po  # noqa: E402
from oracle import packing as pk  # noqa: E402
from pace_synth import make_tokens, random_bf16_state, random_buffer_parts  # noqa: E402
import parity  # noqa: E402

pytestmark = pytest.mark.gpu

CASES = {
    # name: (B, Hv, Hk, d, bf16_io, dP)
    "bench_heads_d128": (6, 32, 16, 128, True, 8),
    "d64_f32": (3, 4, 2, 64, False, 8),
    "d128_f32": (2, 4, 2, 128, False, 8),
    "dP1": (2, 4, 2, 128, True, 1),
    "dP12": (2, 4, 2, 128, True, 12),
    "dP32_d64": (2, 4, 4, 64, True, 32),
}


def dev(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def io_dev(x, bf16):
    return dev(np.asarray(x, dtype=np.float32), torch.bfloat16 if bf16 else torch.float32)


def host(t):
    return (t.float() if t.dtype == torch.bfloat16 else t).cpu().numpy()


def cfgs(B, Hv, Hk, d, bf16, dP):
    import bit_recurrent_state_amd as pace
    o = pk.LayerCfg(B=B, Hv=Hv, Hk=Hk, dk=d, dv=d, group=64, asym=False, buf="int8", dP=dP, bf16_io=bf16,
                    bf16_state=True)
    g = pace.LayerConfig(B=B, Hv=Hv, Hk=Hk, dk=d, dv=d, group=64, buf="int8", bf16_io=bf16, dP=dP,
                         bf16_state=True)
    return o, g


def state_bytes(ocfg, S):
    return pk.pack_state(ocfg, [[S[b, h] for h in range(ocfg.Hv)] for b in range(ocfg.B)])


def flush_tolerance(S0, entries):
    """fp32 accumulation error bound of the pre-rounding state after replaying `entries` on
    S0: 2^-18 of the elementwise magnitudes that enter it (decayed |S0| plus the rank-one
    terms |k| |u|^T)."""
    S, M = np.array(S0, dtype=np.float64), np.abs(S0)
    for e in entries:
        S, u = po.exact_step(S, e.k, e.v, e.a, e.beta)
        M = e.a * M + np.outer(np.abs(e.k), np.abs(u))
    return 2.0 ** -18 * M


def deviation_budget(n_values, dP):
    """Bound on the count of rounding-window deviations among n_values stored bf16 values.

    Each deviation is checked on its own (the stored value is the bf16 rounding of a value
    within the fp32 error bound of the oracle's); this bounds how many there may be.  The
    fold accumulates up to dP + 1 terms in fp32, so the GPU's pre-rounding value carries a
    relative error of about (dP + 2) 2^-24, and it straddles a bf16 rounding midpoint (bf16
    ulps are 2^-8 relative) for a fraction of about 2 (dP + 2) 2^-16 of the values; the
    budget is twice that.  (Integer codes have a far sparser grid relative to the error,
    hence their 1e-4 budget.)"""
    return 4 * (dP + 2) * 2.0 ** -16 * n_values + 1


def run_step(pace, gcfg, st, bu, tok, bf16):
    q, k, v, a, beta = tok
    o = torch.full((gcfg.B, gcfg.Hv, gcfg.dv), float("nan"), dtype=torch.bfloat16 if bf16 else torch.float32,
                   device="cuda")
    pace.decode_step(gcfg, st, bu, io_dev(q, bf16), io_dev(k, bf16), io_dev(v, bf16), dev(a), dev(beta), o)
    torch.cuda.synchronize()
    return host(o)


@pytest.mark.parametrize("name", list(CASES))
def test_bf16_state_decode_step_matches_oracle(name):
    import bit_recurrent_state_amd as pace
    B, Hv, Hk, d, bf16, dP = CASES[name]
    print(f"[bf16 state parity] case={name}", flush=True)
    ocfg, gcfg = cfgs(B, Hv, Hk, d, bf16, dP)
    seed = 900 + len(name)
    S = random_bf16_state(seed, B, Hv, d, d).astype(np.float64)
    state = state_bytes(ocfg, S)
    counts = np.random.default_rng(seed + 7).integers(0, dP, size=B)
    counts[0] = dP - 1
    buffer = pk.pack_buffer(ocfg, random_buffer_parts(seed + 1, B, Hv, Hk, d, d, dP, False, counts=counts))
    toks = make_tokens(seed + 2, B, 1, Hv, Hk, d, d, bf16=bf16)
    o_ref, s_ref, b_ref, pre = pk.decode_step_layer(ocfg, state, buffer, *toks.token(0))
    st, bu = dev(state), dev(buffer)
    o_gpu = run_step(pace, gcfg, st, bu, toks.token(0), bf16)
    tiles = [(b, h) for b in range(B) for h in range(Hv)]
    parity.check_outputs(o_gpu, o_ref, tiles, name, out_bf16=bf16)
    s_gpu, b_gpu = st.cpu().numpy(), bu.cpu().numpy()
    assert np.array_equal(b_gpu, b_ref), "decode buffer differs from the oracle's"
    got = pk.unpack_state(ocfg, s_gpu)
    d_in = pk.unpack_buffer(ocfg, buffer)
    dev_count = 0
    for b, h in tiles:
        if (b, h) not in pre:
            assert np.array_equal(got[b][h], S[b, h]), f"untouched state changed (b={b}, h={h})"
            continue
        n0 = int(d_in["count"][b, h])
        kh = h // ocfg.gamma
        q, k, v, a, beta = toks.token(0)
        entries = [pk._entry(ocfg, d_in, b, h, i) for i in range(n0)]
        entries.append(po.buffer_entry(k[b, kh], v[b, h], a[b, h], beta[b, h], "int8"))
        tol = flush_tolerance(S[b, h], entries)
        dev_count += parity.check_bf16_rounding(got[b][h], pre[(b, h)], tol, f"{name} (b={b}, h={h})")
    n = len(pre) * d * d
    print(f"[bf16 state parity] {name}: {len(pre)} flushed tiles, {dev_count} rounding-window deviations "
          f"in {n} values", flush=True)
    assert len(pre) > 0 and dev_count <= deviation_budget(n, dP)


def test_bf16_state_explicit_flush():
    import bit_recurrent_state_amd as pace
    B, Hv, Hk, d, bf16, dP = 4, 8, 4, 128, True, 8
    ocfg, gcfg = cfgs(B, Hv, Hk, d, bf16, dP)
    S = random_bf16_state(31, B, Hv, d, d).astype(np.float64)
    state = state_bytes(ocfg, S)
    counts = [3, 0, 7, 1]
    buffer = pk.pack_buffer(ocfg, random_buffer_parts(32, B, Hv, Hk, d, d, dP, False, counts=counts))
    mask = np.array([1, 1, 1, 0], dtype=np.uint8)
    s_ref, b_ref, pre = pk.flush_layer(ocfg, state, buffer, seq_mask=mask)
    st, bu = dev(state), dev(buffer)
    pace.flush_requant(gcfg, st, bu, seq_mask=dev(mask))
    torch.cuda.synchronize()
    assert np.array_equal(bu.cpu().numpy(), b_ref)
    got = pk.unpack_state(ocfg, st.cpu().numpy())
    d_in = pk.unpack_buffer(ocfg, buffer)
    for b in range(B):
        for h in range(Hv):
            if (b, h) in pre:
                entries = [pk._entry(ocfg, d_in, b, h, i) for i in range(counts[b])]
                parity.check_bf16_rounding(got[b][h], pre[(b, h)], flush_tolerance(S[b, h], entries), "flush")
            else:
                assert np.array_equal(got[b][h], S[b, h])
    assert {b for b, _ in pre} == {0, 2}


def test_bf16_state_64_steps_full_size_teacher_forced():
    """B = 64, 32 value / 16 key heads, d = 128, bf16 I/O, dP = 8, column-outlier tokens:
    64 decode steps from a seeded bf16 state; sampled tiles against the oracle every step,
    the GPU's stored state adopted after every flush."""
    import bit_recurrent_state_amd as pace
    B, Hv, Hk, d, dP, T = 64, 32, 16, 128, 8, 64
    print("[bf16 state multistep] B=64 steps=64", flush=True)
    ocfg, gcfg = cfgs(B, Hv, Hk, d, True, dP)
    S = random_bf16_state(77, B, Hv, d, d).astype(np.float64)
    st = dev(state_bytes(ocfg, S))
    bu = torch.zeros(pace.layout(gcfg)["buffer_bytes"], dtype=torch.uint8, device="cuda")
    toks = make_tokens(78, B, T, Hv, Hk, d, d, bf16=True, n_outlier=4)
    sample = [(b, h) for b in (0, 9, 40, 63) for h in (0, 1, 17, 31)]
    tiles = {(b, h): po.TileState(S[b, h].copy(), []) for b, h in sample}
    deviations = 0
    for t in range(T):
        tok = toks.token(t)
        o_gpu = run_step(pace, gcfg, st, bu, tok, True)
        flush = (t + 1) % dP == 0
        got = pk.unpack_state(ocfg, st.cpu().numpy(), sample) if flush else None
        q, k, v, a, beta = tok
        for (b, h), tile in tiles.items():
            kh = h // ocfg.gamma
            cap = {}

            def rq(X, _cap=cap):
                _cap["S"] = X
                return po.round_state_bf16(X)

            S0, entries = tile.q.copy(), list(tile.buf)
            o_ref, flushed = po.decode_tile_step(tile, q[b, kh], k[b, kh], v[b, h], float(a[b, h]),
                                                 float(beta[b, h]), dP, "int8", rq)
            assert flushed == flush
            assert parity.rel_err_io(o_gpu[b, h], o_ref, True) <= parity.TOL_REL, f"step {t} o (b={b}, h={h})"
            if flushed:
                entries.append(po.buffer_entry(k[b, kh], v[b, h], a[b, h], beta[b, h], "int8"))
                deviations += parity.check_bf16_rounding(got[b][h], cap["S"], flush_tolerance(S0, entries),
                                                         f"step {t} (b={b}, h={h})")
                tile.q = got[b][h].copy()                 # adopt the GPU's stored state
    n = (T // dP) * len(sample) * d * d
    print(f"[bf16 state multistep] {deviations} rounding-window deviations in {n} stored values", flush=True)
    assert deviations <= deviation_budget(n, dP)


def test_bf16_state_outside_the_decode_calls_is_refused():
    import bit_recurrent_state_amd as pace
    cfg = pace.bf16_periodic(B=2, Hv=4, Hk=2)
    L = pace.layout(cfg)
    assert L["state_bytes"] == 2 * 4 * 128 * 128 * 2 and L["payload_bits"] == 16.0
    T = 64
    st = torch.zeros(L["state_bytes"], dtype=torch.uint8, device="cuda")
    x = torch.zeros((2, T, 2, 128), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros((2, T, 4, 128), dtype=torch.bfloat16, device="cuda")
    g = torch.full((2, T, 4), 0.9, device="cuda")
    with pytest.raises(pace.PaceError) as e:
        pace.prefill_chunk(cfg, st, x, x, v, g, g, torch.zeros_like(v))
    assert e.value.status == pace.PACE_EUNSUPPORTED
    mixed = pace.LayerConfig(B=2, Hv=4, Hk=2, dk=128, dv=128, group=64, buf="mixed", bf16_state=True)
    with pytest.raises(pace.PaceError) as e:
        pace.layout(mixed)
    assert e.value.status == pace.PACE_EUNSUPPORTED

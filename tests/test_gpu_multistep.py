"""Multi-step GPU parity on the benchmark's own workload: the PACE-4 and PACE-4/8 layers at
full size (B = 64 sequences, 32 value heads over 16 key heads, d = 128, bf16 q/k/v/o,
dP = 8) on the column-outlier token stream (4 of 128 value channels per head scaled x8 on
runs of 50-200 tokens), through the C ABI:

  * a 512-token context written by pace_prefill_chunk (two 256-token calls, so that the
    oracle can adopt the GPU's packed bytes after each rounding);
  * then 256 decode steps (32 flushes of every tile) with pace_decode_step.

On sampled tiles (both value heads of a key head, 8-bit heads of the PACE-4/8 map, first
and last sequences) the fp64 oracle runs the same tokens alongside: every output o_t,
every appended buffer slot (codes, scales, gates: bit-exact) and every rounding (scales
bit-exact, codes valid roundings of the oracle's pre-rounding state) is checked.  After
each rounding the oracle adopts the GPU's packed state (teacher forcing), so that one
legal tie flip cannot cascade.  The count rule is checked on every tile at every step.
The number of tie flips is printed."""
import functools

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import pace_oracle as po  # noqa: E402
from oracle import packing as pk  # noqa: E402
from pace_synth import make_tokens  # noqa: E402
import parity  # noqa: E402

pytestmark = pytest.mark.gpu

B, HV, HK, D, DP = 64, 32, 16, 128, 8
CONTEXT, STEPS = 512, 256
QUARTER = [8 if h % 4 == 1 else 4 for h in range(HV)]

CONFIGS = {
    # name: (group, asym, buffer, head bits)
    "pace4_int8": (64, False, "int8", None),
    "pace48_int8": (32, True, "int8", QUARTER),
    "pace48_mixed": (32, True, "mixed", QUARTER),
}
SEQS = (0, 5, 37, B - 1)
HEADS = (0, 1, 13, HV - 2)
TILES = [(b, h) for b in SEQS for h in HEADS]


@functools.lru_cache(maxsize=1)
def tokens():
    # drawn once for every configuration of this module
    return make_tokens(4242, B, CONTEXT + STEPS, HV, HK, D, D, bf16=True, n_outlier=4)


def dev(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def bf(x):
    return dev(np.asarray(x, dtype=np.float32), torch.bfloat16)


def host_f(t):
    return t.float().cpu().numpy()


def check_buffer_slot(ocfg, dg, b, h, slot, k, v, a, beta):
    """GPU buffer slot `slot` of tile (b, h) against the oracle's buffer quantiser."""
    kh = h // ocfg.gamma
    qmax_k = 127 if ocfg.buf == "int8" else 7
    kc, ks = po.quant_buffer_vec(k, qmax_k)
    assert np.array_equal(dg["kc"][b, kh, slot], kc), f"key codes (b={b}, kh={kh}, slot={slot})"
    assert dg["ks"][b, kh, slot] == np.float32(ks), "key scale"
    if ocfg.buf == "int8":
        vc, vs = po.quant_buffer_vec(v, 127)
        assert np.array_equal(dg["vc"][b, h, slot], vc), f"value codes (b={b}, h={h}, slot={slot})"
        assert dg["vs"][b, h, slot] == np.float32(vs), "value scale"
    else:
        assert np.array_equal(dg["v"][b, h, slot], po.bf16_rne(np.asarray(v, dtype=np.float64)).astype(np.float32))
    assert dg["a"][b, h, slot] == np.float32(a) and dg["beta"][b, h, slot] == np.float32(beta)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", list(CONFIGS))
def test_prefill_then_256_decode_steps_teacher_forced(name):
    import bit_recurrent_state_amd as pace
    g, asym, buf, hb = CONFIGS[name]
    print(f"[multistep] case={name} B={B} context={CONTEXT} steps={STEPS}", flush=True)
    ocfg = pk.LayerCfg(B=B, Hv=HV, Hk=HK, dk=D, dv=D, group=g, asym=asym, buf=buf, dP=DP,
                       bf16_io=True, head_bits=hb)
    gcfg = pace.LayerConfig(B=B, Hv=HV, Hk=HK, dk=D, dv=D, group=g, asym=asym, buf=buf, bf16_io=True,
                            dP=DP, head_bits=hb)
    L = pace.layout(gcfg)
    toks = tokens()
    st = torch.zeros(L["state_bytes"], dtype=torch.uint8, device="cuda")
    bu = torch.zeros(L["buffer_bytes"], dtype=torch.uint8, device="cuda")
    requant = {h: (lambda S, _b=ocfg.bits(h): po.quantize_state(S, _b, g, asym)) for h in range(HV)}
    qstate = {(b, h): po.zero_qstate(D, D, ocfg.bits(h), g, asym) for b, h in TILES}
    flips = entries = 0

    # ---- context: two 256-token prefill calls, teacher-forced at the rounding after each
    for c in range(CONTEXT // 256):
        t0, t1 = 256 * c, 256 * (c + 1)
        q, k, v, a, beta = toks.span(t0, t1)
        o = torch.empty((B, t1 - t0, HV, D), dtype=torch.bfloat16, device="cuda")
        pace.prefill_chunk(gcfg, st, bf(q), bf(k), bf(v), dev(a), dev(beta), o)
        torch.cuda.synchronize()
        og = host_f(o)
        s_gpu = pk.unpack_state(ocfg, st.cpu().numpy(), TILES)
        pre = {}
        for b, h in TILES:
            kh = h // ocfg.gamma
            cap = {}

            def rq(S, _h=h, _cap=cap):
                _cap["S"] = S
                return requant[_h](S)

            o_ref, _ = po.prefill_tile(qstate[(b, h)], q[b, :, kh], k[b, :, kh], v[b, :, h], a[b, :, h],
                                       beta[b, :, h], 256, rq)
            e = parity.rel_err_io(og[b, :, h], o_ref, True)
            assert e <= parity.TOL_REL, f"{name} prefill chunk {c} o (b={b}, h={h}): {e:.3g}"
            pre[(b, h)] = cap["S"]
        f, n = parity.check_flushed_tiles(pre, s_gpu, f"{name} prefill {c}")
        flips, entries = flips + f, entries + n
        for b, h in TILES:
            qstate[(b, h)] = s_gpu[b][h]                   # adopt the GPU's packed bytes

    # ---- decode: 256 steps; the oracle keeps each sampled tile's buffer and state
    tiles = {(b, h): po.TileState(qstate[(b, h)], []) for b, h in TILES}
    o = torch.empty((B, HV, D), dtype=torch.bfloat16, device="cuda")
    worst = 0.0
    for step in range(STEPS):
        t = CONTEXT + step
        q, k, v, a, beta = toks.token(t)
        pace.decode_step(gcfg, st, bu, bf(q), bf(k), bf(v), dev(a), dev(beta), o)
        torch.cuda.synchronize()
        og = host_f(o)
        dg = pk.unpack_buffer(ocfg, bu.cpu().numpy())
        flush = (step + 1) % DP == 0
        assert np.all(dg["count"] == (0 if flush else (step + 1) % DP)), f"{name} count rule at step {step}"
        pre = {}
        for (b, h), tile in tiles.items():
            kh = h // ocfg.gamma
            n0 = len(tile.buf)
            cap = {}

            def rq(S, _h=h, _cap=cap):
                _cap["S"] = S
                return requant[_h](S)

            o_ref, flushed = po.decode_tile_step(tile, q[b, kh], k[b, kh], v[b, h], float(a[b, h]),
                                                 float(beta[b, h]), DP, buf, rq)
            assert flushed == flush
            e = parity.rel_err_io(og[b, h], o_ref, True)
            worst = max(worst, e)
            assert e <= parity.TOL_REL, f"{name} step {step} o (b={b}, h={h}): {e:.3g}"
            if flushed:
                pre[(b, h)] = cap["S"]
            else:
                check_buffer_slot(ocfg, dg, b, h, n0, k[b, kh], v[b, h], a[b, h], beta[b, h])
        if flush:
            s_gpu = pk.unpack_state(ocfg, st.cpu().numpy(), TILES)
            f, n = parity.check_flushed_tiles(pre, s_gpu, f"{name} step {step}")
            flips, entries = flips + f, entries + n
            for b, h in TILES:
                tiles[(b, h)].q = s_gpu[b][h]                # adopt the GPU's packed bytes
        if step % 64 == 63:
            print(f"[multistep] {name}: {step + 1} steps, worst o rel err {worst:.3g}, "
                  f"tie flips {flips} / {entries} entries", flush=True)
    assert flips <= 1e-4 * entries + 1
    print(f"[multistep] {name}: done; {flips} tie flips in {entries} rounded entries "
          f"({CONTEXT // 256 + STEPS // DP} roundings x {len(TILES)} tiles)", flush=True)

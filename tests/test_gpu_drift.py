"""Free-running drift on the GPU against the oracle (the non-gating statistic of the parity
protocol, and the GPU leg of the quantiser studies: [p1] "Assumptions and limits" reports
that state drift falls as dP grows).

From S = 0, 256 seeded column-outlier tokens are decoded at dP in {1, 8, 32}, by the HIP
path (pace_decode_step) and by the oracle, each on its own (no teacher forcing: a legal
tie flip on either side is free to propagate).  Drift of a tile is the squared distance of
its dequantised final state from the exact recurrence on the same buffered tokens,
relative to that state's energy.  The GPU's mean drift over the tiles must agree with the
oracle's within 5% at every period, and fall as the period grows.  Layouts: symmetric
4-bit heads with 32-key groups, and asymmetric 32-key groups with 8-bit heads in the map."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import pace_oracle as po  # noqa: E402
from oracle import packing as pk  # noqa: E402
from pace_synth import make_tokens  # noqa: E402

pytestmark = pytest.mark.gpu

B, HV, HK, D, T = 2, 4, 2, 64, 256
LAYOUTS = {
    # name: (asym, head bits)
    "sym4_g32": (False, None),
    "asym_g32_with_8bit_heads": (True, [4, 8, 4, 8]),
}


def dev(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    return (t.to(dtype) if dtype is not None else t).cuda()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", list(LAYOUTS))
def test_free_running_drift_agrees_with_the_oracle(name):
    import bit_recurrent_state_amd as pace
    asym, hb = LAYOUTS[name]
    toks = make_tokens(606, B, T, HV, HK, D, D, bf16=True, n_outlier=4)
    tiles = [(b, h) for b in range(B) for h in range(HV)]
    # exact recurrence on the buffered (int8) tokens, per tile
    exact = {}
    for b, h in tiles:
        kh = h // (HV // HK)
        S = np.zeros((D, D))
        for t in range(T):
            e = po.buffer_entry(toks.k[b, t, kh], toks.v[b, t, h], toks.a[b, t, h], toks.beta[b, t, h], "int8")
            S, _ = po.exact_step(S, e.k, e.v, e.a, e.beta)
        exact[(b, h)] = S
    report = {}
    for dP in (1, 8, 32):
        print(f"[drift] layout={name} dP={dP}", flush=True)
        ocfg = pk.LayerCfg(B=B, Hv=HV, Hk=HK, dk=D, dv=D, group=32, asym=asym, buf="int8", dP=dP,
                           bf16_io=True, head_bits=hb)
        gcfg = pace.LayerConfig(B=B, Hv=HV, Hk=HK, dk=D, dv=D, group=32, asym=asym, buf="int8", bf16_io=True,
                                dP=dP, head_bits=hb)
        L = pace.layout(gcfg)
        st = torch.zeros(L["state_bytes"], dtype=torch.uint8, device="cuda")
        bu = torch.zeros(L["buffer_bytes"], dtype=torch.uint8, device="cuda")
        o = torch.empty((B, HV, D), dtype=torch.bfloat16, device="cuda")
        for t in range(T):
            q, k, v, a, beta = toks.token(t)
            pace.decode_step(gcfg, st, bu, dev(q, torch.bfloat16), dev(k, torch.bfloat16),
                             dev(v, torch.bfloat16), dev(a), dev(beta), o)
        torch.cuda.synchronize()
        got = pk.unpack_state(ocfg, st.cpu().numpy())
        gpu, ora = [], []
        for b, h in tiles:
            kh = h // (HV // HK)
            bits = ocfg.bits(h)
            tile = po.TileState(po.zero_qstate(D, D, bits, 32, asym), [])
            rq = lambda S, _b=bits: po.quantize_state(S, _b, 32, asym)
            for t in range(T):
                po.decode_tile_step(tile, toks.q[b, t, kh], toks.k[b, t, kh], toks.v[b, t, h],
                                    float(toks.a[b, t, h]), float(toks.beta[b, t, h]), dP, "int8", rq)
            assert not tile.buf                      # T is a multiple of every period
            Sx = exact[(b, h)]
            energy = float(np.sum(Sx ** 2))
            ora.append(float(np.sum((po.dequantize_state(tile.q) - Sx) ** 2)) / energy)
            gpu.append(float(np.sum((po.dequantize_state(got[b][h]) - Sx) ** 2)) / energy)
        report[dP] = (float(np.mean(gpu)), float(np.mean(ora)))
        print(f"[drift] {name} dP={dP}: mean drift GPU {report[dP][0]:.4e} oracle {report[dP][1]:.4e} "
              f"(ratio {report[dP][0] / report[dP][1]:.4f})", flush=True)
        assert abs(report[dP][0] / report[dP][1] - 1.0) <= 0.05, (dP, report[dP])
    assert report[1][0] > report[8][0] > report[32][0], report

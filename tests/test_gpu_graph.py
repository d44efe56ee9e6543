"""The decode as bench.py times it: one decode period of launches prepared once
(prepare_decode_step) and captured in a HIP graph, replayed several times with eager work
and synchronisations between the replays.  Every replay must leave the packed state, the
buffer (counts included) and the last outputs bit for bit where the same launches issued
eagerly leave them.  Cases: PACE-4 aligned (every tile flushes on the period's last
step) and PACE-4/8 with the mixed buffer at staggered counts through
pace_decode_step_ordered (the flushing sequences first, as the continuous-batching leg
issues them)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import packing as pk  # noqa: E402
from pace_synth import make_tokens, random_buffer_parts, random_packed_state_parts  # noqa: E402

pytestmark = pytest.mark.gpu

B, HV, HK, D, DP = 8, 32, 16, 128, 8
QUARTER = [8 if h % 4 == 1 else 4 for h in range(HV)]
CASES = {
    # name: (group, asym, buffer, head bits, staggered counts + ordered launches)
    "pace4_aligned": (64, False, "int8", None, False),
    "pace48_mixed_staggered_ordered": (32, True, "mixed", QUARTER, True),
}


def dev(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    return (t.to(dtype) if dtype is not None else t).cuda()


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_equal_eager_launches(name):
    import bit_recurrent_state_amd as pace
    print(f"[graph] case={name}", flush=True)
    g, asym, buf, hb, staggered = CASES[name]
    ocfg = pk.LayerCfg(B=B, Hv=HV, Hk=HK, dk=D, dv=D, group=g, asym=asym, buf=buf, dP=DP, bf16_io=True,
                       head_bits=hb)
    cfg = pace.LayerConfig(B=B, Hv=HV, Hk=HK, dk=D, dv=D, group=g, asym=asym, buf=buf, bf16_io=True, dP=DP,
                           head_bits=hb)
    seed = 4000 + len(name)
    bits = [ocfg.bits(h) for h in range(HV)]
    state0 = pk.pack_state(ocfg, pk.state_from_parts(ocfg, random_packed_state_parts(seed, B, HV, D, D, g, bits,
                                                                                      asym)))
    counts = (np.random.default_rng(seed + 7).integers(0, DP, size=B) if staggered
              else np.zeros(B, dtype=np.int64))
    buffer0 = pk.pack_buffer(ocfg, random_buffer_parts(seed + 1, B, HV, HK, D, D, DP, buf == "mixed", counts=counts))
    toks = make_tokens(seed + 2, B, DP, HV, HK, D, D, bf16=True, n_outlier=4)
    tok = [tuple(dev(x, torch.bfloat16) if i < 3 else dev(x) for i, x in enumerate(toks.token(t)))
           for t in range(DP)]
    orders = []
    for t in range(DP):
        flushing = (counts + t) % DP == DP - 1
        orders.append(np.concatenate([np.flatnonzero(flushing), np.flatnonzero(~flushing)]) if staggered else None)

    def run_period(st, bu, o, stream):
        for t in range(DP):
            pace.decode_step(cfg, st, bu, *tok[t], o, stream=stream, order=orders[t])

    # eager reference after one, two and three periods
    stream = torch.cuda.Stream()
    st, bu = dev(state0), dev(buffer0)
    o = torch.empty((B, HV, D), dtype=torch.bfloat16, device="cuda")
    ref = []
    for _ in range(3):
        run_period(st, bu, o, stream)
        stream.synchronize()
        ref.append((st.clone(), bu.clone(), o.clone()))

    # the prepared calls: one eager pass (period 1), then captured and replayed twice
    st, bu = dev(state0), dev(buffer0)
    o = torch.full((B, HV, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    calls = [pace.prepare_decode_step(cfg, st, bu, *tok[t], o, stream=stream, order=orders[t]) for t in range(DP)]
    with torch.cuda.stream(stream):
        for c in calls:
            c()
    stream.synchronize()

    def same(i):
        return (torch.equal(st, ref[i][0]) and torch.equal(bu, ref[i][1])
                and torch.equal(o.view(torch.int16), ref[i][2].view(torch.int16)))

    assert same(0), "prepared eager period differs"
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for c in calls:
            c()
    for i in (1, 2):
        graph.replay()
        torch.cuda.synchronize()
        assert same(i), f"graph replay {i} differs from the eager launches"
        # eager work of the program's own between the replays
        scratch = torch.randn(1 << 20, device="cuda")
        scratch.mul_(2.0).sum().item()
        torch.cuda.synchronize()
    del graph

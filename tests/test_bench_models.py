"""The work models behind bench.py's rooflines (CPU):
- the decode's algorithmic bytes per launch, rebuilt here from the sizes the library's
  own pace_layout reports (state, buffer) and the I/O tensor shapes, at every buffer count
  of the period, for each layout the bench times (bf16 I/O);
- the prefill's algorithmic flops, rebuilt from the WY form's products one by one;
- the prefill's executed matrix-core work, against the hardware MFMA counters committed in
  profiles/prefill_long_b4_mfma_counters.txt (both workloads recorded there)."""
import os
import re
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

QUARTER = [8 if h % 4 == 1 else 4 for h in range(32)]


def _configs():
    import bit_recurrent_state_amd as pace
    return {
        "pace4_b64": pace.pace4(B=64),
        "pace4_b128": pace.pace4(B=128),
        "pace4_b1": pace.pace4(B=1),
        "pace4_b16_dP4": pace.pace4(B=16, dP=4),
        "pace48_int8_b64": pace.pace48(QUARTER, B=64),
        "pace48_mixed_b64": pace.pace48(QUARTER, B=64, buf="mixed"),
        "bf16_periodic_b64": pace.bf16_periodic(B=64),
    }


@pytest.mark.parametrize("name", ["pace4_b64", "pace4_b128", "pace4_b1", "pace4_b16_dP4", "pace48_int8_b64",
                                  "pace48_mixed_b64", "bf16_periodic_b64"])
def test_decode_bytes_rebuilt_from_layout_sizes(name):
    import bit_recurrent_state_amd as pace
    cfg = _configs()[name]
    L = pace.layout(cfg)
    B, Hv, Hk, d, dP = cfg.B, cfg.Hv, cfg.Hk, cfg.dk, cfg.dP
    # the buffer is an int32 count per (sequence, head), padded to 256 B, then dP token slots
    # per sequence: everything after the count region is slot payload
    count_region = -(-4 * B * Hv // 256) * 256
    slots = L["buffer_bytes"] - count_region               # all B x dP slots of all heads
    assert slots > 0 and slots % (B * dP) == 0
    io_in = 2 * (B * Hk * d * 2) + B * Hv * d * 2 + 2 * (B * Hv * 4)   # q, k (bf16, per key head), v, a, beta
    o_out = B * Hv * d * 2
    for n0 in range(dP):
        flush = n0 + 1 == dP
        want = (L["state_bytes"]                        # the state is read every step
                + n0 * slots / dP                       # the n0 buffered tokens
                + io_in + o_out
                + (L["state_bytes"] if flush else slots / dP))   # rewritten state, or the appended slot
        got = bench.algorithmic_bytes_per_launch(cfg, n0, L)
        assert got == pytest.approx(want, rel=1e-12), (name, n0)


def test_decode_bytes_headline_figure():
    """PACE-4 at B = 64: 23,489,024 bytes per launch over the period (11,469.25 per tile)."""
    import bit_recurrent_state_amd as pace
    cfg = _configs()["pace4_b64"]
    L = pace.layout(cfg)
    mean = sum(bench.algorithmic_bytes_per_launch(cfg, n0, L) for n0 in range(cfg.dP)) / cfg.dP
    assert mean == 23489024
    assert L["state_bytes"] == 64 * 32 * 8704


@pytest.mark.parametrize("d", [64, 128])
def test_prefill_algorithmic_flops_term_by_term(d):
    """One 256-token chunk of one head in WY form, each product counted once (triangular
    products at half the flops of the full product):
    K K^T and Q K^T (strictly lower / lower, C^2 d each), T = (I + diag(beta) A)^-1 by
    substitution (C^3 / 3), W_v = T diag(beta) V and W_k = T diag(beta Gamma) K (C^2 d each),
    U = W_v - W_k S_0 (2 C d^2), Q S_0 (2 C d^2), the masked (Q K^T) U (C^2 d), and the end
    state K^T diag(.) U (2 C d^2)."""
    C = 256
    terms = {"KKt": C * C * d, "QKt": C * C * d, "T": C ** 3 / 3, "Wv": C * C * d, "Wk": C * C * d,
             "U": 2 * C * d * d, "QS0": 2 * C * d * d, "PU": C * C * d, "SC": 2 * C * d * d}
    per_chunk = sum(terms.values())
    if d == 128:
        assert per_chunk == pytest.approx(72.7e6, rel=1e-3)
    for T, B, Hv in ((256, 1, 1), (512, 2, 3), (300, 1, 2), (32768, 4, 32)):
        alg, _ = bench.prefill_flops(T, Hv, B, d)
        assert alg == pytest.approx(per_chunk * (-(-T // C)) * B * Hv, rel=1e-12), (T, B, Hv)
    if d == 128:
        assert bench.prefill_flops(32768, 32, 4, 128)[0] == pytest.approx(1.1911e12, rel=1e-4)


def _counter_sections():
    path = os.path.join(ROOT, "profiles", "prefill_long_b4_mfma_counters.txt")
    text = open(path).read()
    out = []
    for head, body in re.findall(r"\n\[([^\]]+)\]\n(.*?)(?=\n\[|\Z)", text, re.S):
        vals = dict(re.findall(r"^(SQ_INSTS_VALU_MFMA_MOPS_\w+): (\d+)", body, re.M))
        m = re.search(r"B=(\d+) x (\d+) tokens", head)
        out.append((int(m.group(1)), int(m.group(2)), {k: int(v) for k, v in vals.items()}))
    return out


def test_prefill_executed_mfma_model_matches_the_hardware_counters():
    """The counters count matrix-core work in units of 512 flops per dispatch; the model in
    bench.py (prefill_flops) must give the same bf16 and fp32 totals for both recorded
    workloads (32/16 heads, d = 128, bf16 I/O)."""
    sections = _counter_sections()
    assert {(B, T) for B, T, _ in sections} == {(4, 32768), (64, 512)}
    for B, T, c in sections:
        _, ex = bench.prefill_flops(T, 32, B, 128, bf16_io=True)
        assert c["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 == ex["bf16"], (B, T)
        assert c["SQ_INSTS_VALU_MFMA_MOPS_F32"] * 512 == ex["f32"], (B, T)

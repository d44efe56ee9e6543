"""GPU parity of pace_prefill_chunk, and the tiny reference configuration end to end
(512-token prefill in two 256-token chunks, then 64 decode tokens at dP = 8).

Protocol: the oracle runs its own trajectory; every GPU call starts from the oracle's
packed state (and buffer), so one legal near-tie code flip cannot cascade.  Multi-chunk
calls are additionally checked for self-consistency (one call over several chunks equals
the same chunks issued as separate calls, bit for bit)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import pace_oracle as po  # noqa: E402
from oracle import packing as pk  # noqa: E402
from pace_synth import make_tokens  # noqa: E402
import parity  # noqa: E402
from test_gpu_decode import dev, io_dev, host  # noqa: E402

pytestmark = pytest.mark.gpu


def _lib():
    import bit_recurrent_state_amd as pace
    return pace


PCASES = {
    # name: (B, Hv, Hk, d, group, asym, bf16, head_bits)
    # d = 64 (fp32 / bf16 I/O): one four-wave workgroup per (sequence, head)
    "tiny_sym4_g32_f32": (2, 4, 4, 64, 32, False, False, None),
    "d64_asym_g32_bf16": (2, 4, 2, 64, 32, True, True, [4, 8, 4, 4]),
    # d = 128, bf16 I/O: the warp-specialised kernel, two column blocks per pair
    "pace4_g64_bf16": (2, 32, 16, 128, 64, False, True, None),
    "pace48_g32_bf16": (2, 8, 4, 128, 32, True, True, [8, 4, 4, 4, 4, 8, 4, 4]),
    # d = 128, fp32 I/O, few pairs: the four-wave kernel with the columns split in two
    "d128_sym_g64_f32": (2, 8, 4, 128, 64, False, False, None),
}


def cfgs(name, dP=8):
    B, Hv, Hk, d, g, asym, bf16, hb = PCASES[name]
    o = pk.LayerCfg(B=B, Hv=Hv, Hk=Hk, dk=d, dv=d, group=g, asym=asym, buf="int8", dP=dP,
                    bf16_io=bf16, head_bits=hb)
    gc = _lib().LayerConfig(B=B, Hv=Hv, Hk=Hk, dk=d, dv=d, group=g, asym=asym, buf="int8",
                            bf16_io=bf16, dP=dP, head_bits=hb)
    return o, gc


def gpu_prefill(gcfg, state_bytes, span):
    pace = _lib()
    q, k, v, a, beta = span
    bf16 = gcfg.bf16_io
    T = a.shape[1]
    st = dev(state_bytes)
    o = torch.empty((gcfg.B, T, gcfg.Hv, gcfg.dv), dtype=torch.bfloat16 if bf16 else torch.float32, device="cuda")
    ws_n = pace.prefill_workspace_bytes(gcfg, T)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda") if ws_n else None
    pace.prefill_chunk(gcfg, st, io_dev(q, bf16), io_dev(k, bf16), io_dev(v, bf16), dev(a), dev(beta), o,
                       workspace=ws)
    torch.cuda.synchronize()
    return host(o), st.cpu().numpy()


def check_prefill_call(ocfg, gcfg, state_in, span, tiles, label):
    o_ref, s_ref, pre = pk.prefill_layer(ocfg, state_in, *span, tiles=tiles)
    o_gpu, s_gpu = gpu_prefill(gcfg, state_in, span)
    T = span[3].shape[1]
    for b, h in tiles:
        for t in range(T):
            e = parity.rel_err_io(o_gpu[b, t, h], o_ref[b, t, h], ocfg.bf16_io)
            assert e <= parity.TOL_REL, f"{label} o (b={b}, t={t}, h={h}) rel err {e:.3g}"
    qg = pk.unpack_state(ocfg, s_gpu, tiles)
    parity.check_flushed_tiles(pre, qg, label)
    return s_ref


@pytest.mark.parametrize("name", list(PCASES))
def test_prefill_chunks_match_oracle(name):
    print(f"[prefill parity] case={name}", flush=True)
    ocfg, gcfg = cfgs(name)
    toks = make_tokens(40 + len(name), ocfg.B, 356, ocfg.Hv, ocfg.Hk, ocfg.dk, ocfg.dv, bf16=ocfg.bf16_io)
    tiles = [(b, h) for b in range(ocfg.B) for h in range(ocfg.Hv)]
    zero = np.zeros(pk.state_layout(ocfg)[2], dtype=np.uint8)
    s1 = check_prefill_call(ocfg, gcfg, zero, toks.span(0, 256), tiles, name + "/chunk1")
    # a partial chunk continuing from the oracle's rounded state
    check_prefill_call(ocfg, gcfg, s1, toks.span(256, 356), tiles, name + "/partial")


@pytest.mark.parametrize("name,chunk", [("pace48_g32_bf16", 64), ("pace48_g32_bf16", 512),
                                        ("tiny_sym4_g32_f32", 128)])
def test_prefill_rounding_period(name, chunk):
    """Prefill rounding periods other than 256 (multiples of 64), on the warp-specialised
    kernel (bf16, d = 128) and the four-wave kernel (fp32, d = 64):
      * one call of `chunk` tokens from the oracle's rounded state (one rounding, at its
        end) matches the oracle -- the parity protocol, which starts every rounding from
        the oracle's state;
      * one call over 600 tokens equals `chunk`-token calls issued one after another, bit
        for bit (outputs and packed state), so it rounds exactly after every `chunk` tokens
        and after the last."""
    print(f"[prefill parity] case={name} chunk={chunk}", flush=True)
    B, Hv, Hk, d, g, asym, bf16, hb = PCASES[name]
    ocfg = pk.LayerCfg(B=B, Hv=Hv, Hk=Hk, dk=d, dv=d, group=g, asym=asym, buf="int8", dP=8,
                       bf16_io=bf16, head_bits=hb, chunk=chunk)
    gcfg = _lib().LayerConfig(B=B, Hv=Hv, Hk=Hk, dk=d, dv=d, group=g, asym=asym, buf="int8",
                              bf16_io=bf16, dP=8, head_bits=hb, chunk=chunk)
    toks = make_tokens(500 + chunk, B, 856, Hv, Hk, d, d, bf16=bf16)
    tiles = [(b, h) for b in range(B) for h in range(Hv)]
    zero = np.zeros(pk.state_layout(ocfg)[2], dtype=np.uint8)
    _, s1, _ = pk.prefill_layer(ocfg, zero, *toks.span(0, 256), tiles=tiles)
    check_prefill_call(ocfg, gcfg, s1, toks.span(256, 256 + chunk), tiles, f"{name}/chunk{chunk}")
    o_all, s_all = gpu_prefill(gcfg, s1, toks.span(256, 856))
    st, outs = s1, []
    for t0 in range(256, 856, chunk):
        o, st = gpu_prefill(gcfg, st, toks.span(t0, min(t0 + chunk, 856)))
        outs.append(o)
    assert np.array_equal(s_all, st), "packed state after one call differs from per-period calls"
    assert np.array_equal(o_all, np.concatenate(outs, axis=1)), "outputs differ"


@pytest.mark.parametrize("T", [1, 5, 64, 65])
def test_prefill_short_prompts(T):
    """Prompts of at most one 64-token sub-block and just past it (one sub-block, so the
    producer waves of the bf16 kernel prepare nothing after the first; a second holding a
    single token), starting from a non-zero rounded state: outputs and the state rounded
    after the last token match the oracle."""
    print(f"[prefill parity] short prompt T={T}", flush=True)
    ocfg, gcfg = cfgs("pace48_g32_bf16")
    toks = make_tokens(900 + T, ocfg.B, 256 + T, ocfg.Hv, ocfg.Hk, ocfg.dk, ocfg.dv, bf16=True)
    tiles = [(b, h) for b in range(ocfg.B) for h in range(ocfg.Hv)]
    zero = np.zeros(pk.state_layout(ocfg)[2], dtype=np.uint8)
    _, s1, _ = pk.prefill_layer(ocfg, zero, *toks.span(0, 256), tiles=tiles)
    check_prefill_call(ocfg, gcfg, s1, toks.span(256, 256 + T), tiles, f"short T={T}")


def test_prefill_multi_chunk_call_equals_separate_calls():
    print("[prefill] multi-chunk self-consistency", flush=True)
    ocfg, gcfg = cfgs("pace48_g32_bf16")
    toks = make_tokens(77, ocfg.B, 600, ocfg.Hv, ocfg.Hk, ocfg.dk, ocfg.dv, bf16=True)
    zero = np.zeros(pk.state_layout(ocfg)[2], dtype=np.uint8)
    o_all, s_all = gpu_prefill(gcfg, zero, toks.span(0, 600))
    st = zero
    outs = []
    for t0, t1 in [(0, 256), (256, 512), (512, 600)]:
        o, st = gpu_prefill(gcfg, st, toks.span(t0, t1))
        outs.append(o)
    assert np.array_equal(s_all, st)
    assert np.array_equal(o_all, np.concatenate(outs, axis=1))


def test_prefill_long_shape_first_chunk_sampled():
    """Launch configuration of the long-prefill workload (4 sequences, 32 value / 16 key
    heads, d = 128, bf16), one 256-token chunk; sampled tiles against the oracle."""
    print("[prefill parity] long shape, sampled tiles", flush=True)
    B, Hv, Hk, d = 4, 32, 16, 128
    ocfg = pk.LayerCfg(B=B, Hv=Hv, Hk=Hk, dk=d, dv=d, group=64, asym=False, buf="int8", dP=8, bf16_io=True)
    gcfg = _lib().LayerConfig(B=B, Hv=Hv, Hk=Hk, dk=d, dv=d, group=64, bf16_io=True)
    toks = make_tokens(4, B, 256, Hv, Hk, d, d, bf16=True)
    zero = np.zeros(pk.state_layout(ocfg)[2], dtype=np.uint8)
    tiles = [(0, 0), (1, 7), (2, 16), (3, 31)]
    check_prefill_call(ocfg, gcfg, zero, toks.span(0, 256), tiles, "long/first-chunk")


@pytest.mark.parametrize("bf16", [True, False], ids=["bf16", "f32"])
def test_prefill_many_pairs(bf16):
    """512 (sequence, head) pairs at d = 128, a partial chunk, sampled tiles against the
    oracle.  bf16: the warp-specialised kernel's 1,024 workgroups take more than one round
    of the CUs; fp32: twice the pairs no longer fit the CUs, so one workgroup per pair owns
    all value columns."""
    print(f"[prefill parity] 512 pairs, bf16={bf16}", flush=True)
    B, Hv, Hk, d = 16, 32, 16, 128
    ocfg = pk.LayerCfg(B=B, Hv=Hv, Hk=Hk, dk=d, dv=d, group=64, asym=False, buf="int8", dP=8, bf16_io=bf16)
    gcfg = _lib().LayerConfig(B=B, Hv=Hv, Hk=Hk, dk=d, dv=d, group=64, bf16_io=bf16)
    toks = make_tokens(16, B, 96, Hv, Hk, d, d, bf16=bf16)
    zero = np.zeros(pk.state_layout(ocfg)[2], dtype=np.uint8)
    tiles = [(0, 0), (3, 9), (7, 16), (15, 31)]
    check_prefill_call(ocfg, gcfg, zero, toks.span(0, 96), tiles, f"512pairs/partial/bf16={bf16}")


def test_long_prefill_full_size():
    """The long-prefill workload at its full size (4 sequences x 32,768 tokens, 32 value /
    16 key heads, d = 128, bf16, int4 g = 64, 128 chunks) in the launch configuration the
    benchmark times (one call over all tokens).  Properties that hold at any size:
      * the one call equals 128 successive one-chunk calls, bit for bit (outputs and the
        packed state), so it rounds exactly once per chunk from its own rounded state;
      * sampled tiles, at sampled chunks (first, second, middle, last), match the oracle
        running its own trajectory chunk by chunk (GPU started from the oracle's packed
        state of that chunk, compared by the parity protocol)."""
    from pace_synth import make_tokens_chunk
    B, Hv, Hk, d, C, NC = 4, 32, 16, 128, 256, 128
    T = C * NC
    ocfg = pk.LayerCfg(B=B, Hv=Hv, Hk=Hk, dk=d, dv=d, group=64, asym=False, buf="int8", dP=8, bf16_io=True)
    gcfg = _lib().LayerConfig(B=B, Hv=Hv, Hk=Hk, dk=d, dv=d, group=64, bf16_io=True)
    pace = _lib()
    print("[long prefill full size] generating inputs", flush=True)
    chunks = []
    for c in range(NC):
        chunks.append(make_tokens_chunk(44, c, B, C, Hv, Hk, d, d, bf16=True))
        if c % 32 == 31:
            print(f"[long prefill full size] {c + 1} chunks generated", flush=True)
    dev_chunks = [tuple(io_dev(x, True) if i < 3 else dev(x) for i, x in enumerate(ch.span(0, C)))
                  for ch in chunks]
    full = [torch.cat([dc[i] for dc in dev_chunks], dim=1) for i in range(5)]
    L = pace.layout(gcfg)
    zero = torch.zeros(L["state_bytes"], dtype=torch.uint8, device="cuda")
    o_all = torch.empty((B, T, Hv, d), dtype=torch.bfloat16, device="cuda")
    st_all = zero.clone()
    print("[long prefill full size] one call over all tokens", flush=True)
    pace.prefill_chunk(gcfg, st_all, *full, o_all)
    st = zero.clone()
    o_c = torch.empty((B, C, Hv, d), dtype=torch.bfloat16, device="cuda")
    print("[long prefill full size] chunk-by-chunk calls", flush=True)
    for c in range(NC):
        pace.prefill_chunk(gcfg, st, *dev_chunks[c], o_c)
        assert torch.equal(o_c, o_all[:, C * c:C * (c + 1)]), f"outputs of chunk {c} differ"
    torch.cuda.synchronize()
    assert torch.equal(st, st_all), "packed state after the one call differs from chunk-by-chunk"
    del full, o_all, dev_chunks
    print("[long prefill full size] oracle trajectory on sampled tiles", flush=True)
    tiles = [(0, 0), (1, 7), (2, 16), (3, 31)]
    state = np.zeros(pk.state_layout(ocfg)[2], dtype=np.uint8)
    for c in range(NC):
        span = chunks[c].span(0, C)
        if c % 32 == 0:
            print(f"[long prefill full size] oracle at chunk {c}", flush=True)
        if c in (0, 1, NC // 2, NC - 1):
            state = check_prefill_call(ocfg, gcfg, state, span, tiles, f"long/chunk{c}")
        else:
            _, state, _ = pk.prefill_layer(ocfg, state, *span, tiles=tiles)


def test_tiny_reference_end_to_end():
    """Tiny reference: B = 2, 4 heads, d = 64, fp32, sym int4 g = 32, int8 buffer,
    512-token prompt (2 chunks) then 64 decode tokens (8 flushes).  Every GPU call
    starts from the oracle's packed state / buffer of that point."""
    print("[tiny reference] prefill + decode", flush=True)
    ocfg, gcfg = cfgs("tiny_sym4_g32_f32")
    T = 512 + 64
    toks = make_tokens(0, ocfg.B, T, ocfg.Hv, ocfg.Hk, ocfg.dk, ocfg.dv)
    tiles = [(b, h) for b in range(ocfg.B) for h in range(ocfg.Hv)]
    state = np.zeros(pk.state_layout(ocfg)[2], dtype=np.uint8)
    for c in range(2):
        state = check_prefill_call(ocfg, gcfg, state, toks.span(256 * c, 256 * (c + 1)), tiles, f"tiny/chunk{c}")
    buffer = np.zeros(pk.buffer_layout(ocfg)[1], dtype=np.uint8)
    from test_gpu_decode import run_gpu_decode, compare_buffers, check_states

    class One:
        def __init__(self, t):
            self.t = t

        def token(self, _):
            return toks.token(self.t)

    flushes = 0
    for t in range(512, T):
        o_ref, s_ref, b_ref, pre = pk.decode_step_layer(ocfg, state, buffer, *toks.token(t))
        o_gpu, s_gpu, b_gpu = run_gpu_decode(gcfg, state, buffer, One(t))
        parity.check_outputs(o_gpu, o_ref, tiles, f"tiny/decode{t}")
        compare_buffers(ocfg, b_gpu, b_ref, tiles)
        check_states(ocfg, s_gpu, state, pre, tiles, f"tiny/decode{t}")
        flushes += bool(pre)
        state, buffer = s_ref, b_ref
    assert flushes == 8

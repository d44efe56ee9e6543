"""fp64 CPU oracle of the PACE gated-delta state path.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
leg may import or run anything under oracle/.  The library's product path never calls
it, and this module imports nothing from the library: it shares no code, table or
helper with the HIP path.  Only the seeded input generators (pace_synth) feed both.

Plain, slow, one (sequence, head) tile at a time, float64 throughout.  Each function
names the passage of the PACE pages it follows:
  [p1] onedev.kr/papers/1282 (editorial summary): "How it works", "How it differs",
       "Assumptions and limits";
  [p2] blog.secrett2633.cloud review of the paper: "1. Key Terms & Definitions",
       "3. Method & Key Results";
  [p3] news.hamidun.com news item: "Two observations".

Readings taken where the pages are silent (each is also listed in the design notes):
  * readout o_t = S_t^T q_t from the post-update state, before rounding, no 1/sqrt(dk);
  * scales are bf16 rounded toward +inf; codes are round-half-to-even; symmetric codes
    use +-(2^(b-1)-1); asymmetric ranges include 0 and zero points have the head's b bits;
  * codes and scales are decided on the fp32 value of the pre-rounding state (the
    precision the kernels hold it in); the decision itself is exact;
  * an all-zero group gets scale 0, codes 0, zero point 0;
  * the decode buffer also stores beta_t; int8 buffer: one symmetric fp32 scale
    max|x|/127 per token vector (keys per key head, values per value head); mixed buffer:
    4-bit symmetric keys (scale max|k|/7), bf16 values; buffer codes rne(x/scale) in fp32;
  * the token being decoded passes through the buffer quantiser before its own output;
  * the flush happens after o_t is emitted, on the step where the count reaches dP;
  * prefill rounds after every `chunk` tokens and after the last token of the prompt;
  * value head h uses key head h // gamma; initial state is zero.

Parity pins for every function live in tests/ (see test_oracle_*.py).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

# ----------------------------------------------------------------------------------
# bf16 rounding written from the format's definition: 8 significant bits (1 implicit +
# 7 stored), exponent range of fp32.  Values below 2^-126 use the subnormal spacing
# 2^-133.
# ----------------------------------------------------------------------------------
_BF16_SUBNORMAL_STEP = 2.0 ** -133
_BF16_MIN_NORMAL = 2.0 ** -126


def _bf16_round(x, mode: str):
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = x != 0
    xs = x[nz]
    mant, expo = np.frexp(xs)            # xs = mant * 2**expo, 0.5 <= |mant| < 1
    scaled = mant * 256.0                # 8 significant bits -> integer part
    step_exp = expo - 8
    small = np.abs(xs) < _BF16_MIN_NORMAL
    if mode == "rne":
        r = np.rint(scaled)              # numpy rint: round half to even
    elif mode == "up":
        r = np.ceil(scaled)
    else:
        raise ValueError(mode)
    res = np.ldexp(r, step_exp)
    if np.any(small):
        sub = xs[small] / _BF16_SUBNORMAL_STEP
        sub = np.rint(sub) if mode == "rne" else np.ceil(sub)
        res[small] = sub * _BF16_SUBNORMAL_STEP
    out[nz] = res
    return out


def bf16_rne(x):
    """Round to the nearest bf16 value, ties to even."""
    return _bf16_round(x, "rne")


def bf16_ceil(x):
    """Smallest bf16 value >= x (x >= 0): the scale rounding of the quantiser."""
    return _bf16_round(x, "up")


def to_f32(x):
    """Value of x rounded to fp32 (round to nearest even), returned as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------------
# State quantiser with channel-aligned groups ([p1] "How it differs": g contiguous
# key-axis elements of one column share a scale; PACE-4 symmetric g = 64, PACE-4/8
# integer zero points g = 32; [p2] "Method": scale groups formed along the key axis
# within a column).  Stored code fields are unsigned: sym code c is stored as
# c + 2^(b-1); dequantised value = s * (stored - z), z = 2^(b-1) for sym.
# ----------------------------------------------------------------------------------

def quant_group_sym(x, bits: int):
    """Symmetric b-bit quantisation of one group. Returns (stored codes, scale)."""
    x32 = to_f32(x)
    qmax = (1 << (bits - 1)) - 1
    m = float(np.max(np.abs(x32))) if x32.size else 0.0
    if m == 0.0:
        return np.full(x32.shape, 1 << (bits - 1), dtype=np.int64), 0.0
    s = float(bf16_ceil(m / qmax))
    c = np.clip(np.rint(x32 / s), -qmax, qmax).astype(np.int64)
    return c + (1 << (bits - 1)), s


def quant_group_asym(x, bits: int):
    """Asymmetric b-bit quantisation of one group, range forced to include 0.
    Returns (stored codes, scale, zero point)."""
    x32 = to_f32(x)
    levels = (1 << bits) - 1
    lo = min(0.0, float(np.min(x32)))
    hi = max(0.0, float(np.max(x32)))
    s = float(bf16_ceil((hi - lo) / levels))
    if s == 0.0:
        return np.zeros(x32.shape, dtype=np.int64), 0.0, 0
    z = int(np.clip(np.rint(-lo / s), 0, levels))
    c = np.clip(np.rint(x32 / s) + z, 0, levels).astype(np.int64)
    return c, s, z


@dataclass
class QState:
    """Quantised state of one (sequence, value head): stored codes [dk, dv],
    scales [dk/g, dv], zero points [dk/g, dv] (asym) or None."""
    codes: np.ndarray
    scales: np.ndarray
    zeros: Optional[np.ndarray]
    bits: int
    group: int
    asym: bool

    def copy(self):
        return QState(self.codes.copy(), self.scales.copy(),
                      None if self.zeros is None else self.zeros.copy(),
                      self.bits, self.group, self.asym)


def zero_qstate(dk, dv, bits, group, asym) -> QState:
    """The all-zero state S = 0 (scales 0)."""
    ng = dk // group
    codes = np.full((dk, dv), 0 if asym else (1 << (bits - 1)), dtype=np.int64)
    return QState(codes, np.zeros((ng, dv)), np.zeros((ng, dv), dtype=np.int64) if asym else None,
                  bits, group, asym)


def quantize_state(S, bits: int, group: int, asym: bool) -> QState:
    """Quantise S [dk, dv] group by group: for each value column j and key group G,
    rows [G g, (G+1) g) share one scale."""
    S = np.asarray(S, dtype=np.float64)
    dk, dv = S.shape
    ng = dk // group
    codes = np.zeros((dk, dv), dtype=np.int64)
    scales = np.zeros((ng, dv))
    zeros = np.zeros((ng, dv), dtype=np.int64) if asym else None
    for j in range(dv):
        for G in range(ng):
            rows = slice(G * group, (G + 1) * group)
            if asym:
                c, s, z = quant_group_asym(S[rows, j], bits)
                zeros[G, j] = z
            else:
                c, s = quant_group_sym(S[rows, j], bits)
            codes[rows, j] = c
            scales[G, j] = s
    return QState(codes, scales, zeros, bits, group, asym)


def dequantize_state(qs: QState) -> np.ndarray:
    """S^ [dk, dv] = s * (stored - z), z = 2^(b-1) for symmetric heads."""
    dk, dv = qs.codes.shape
    S = np.zeros((dk, dv))
    for j in range(dv):
        for G in range(dk // qs.group):
            rows = slice(G * qs.group, (G + 1) * qs.group)
            z = qs.zeros[G, j] if qs.asym else (1 << (qs.bits - 1))
            S[rows, j] = qs.scales[G, j] * (qs.codes[rows, j].astype(np.float64) - z)
    return S


# ----------------------------------------------------------------------------------
# Decode-buffer quantisers ([p1] "How it works": the buffer keeps (a_t, k_t, v_t) of
# each token; int8 keys and values in the uniform configuration, 4-bit keys and bf16
# values in the mixed one).  Codes decided in fp32: scale = fp32(max|x| / qmax),
# code = rne(fp32(x / scale)).
# ----------------------------------------------------------------------------------

def quant_buffer_vec(x, qmax: int):
    """Symmetric per-vector quantisation with an fp32 scale. Returns (codes int, scale)."""
    x32 = np.asarray(x, dtype=np.float32)
    m = np.float32(np.max(np.abs(x32)))
    if m == 0:
        return np.zeros(x32.shape, dtype=np.int64), 0.0
    s = np.float32(m / np.float32(qmax))              # fp32 IEEE division
    c = np.rint(x32 / s).astype(np.int64)             # fp32 IEEE division, then rne
    return np.clip(c, -qmax, qmax), float(s)


@dataclass
class BufEntry:
    """One buffered token of one (sequence, value head): the values the replay uses."""
    k: np.ndarray      # k^ (dequantised key, fp64)
    v: np.ndarray      # v^ (dequantised value, fp64)
    a: float
    beta: float


def buffer_entry(k, v, a, beta, buf_kind: str) -> BufEntry:
    """Pass one token through the buffer quantiser of `buf_kind` ('int8', 'mixed',
    or 'exact' -- identity, used by the oracle's own pins)."""
    if buf_kind == "int8":
        kc, ks = quant_buffer_vec(k, 127)
        vc, vs = quant_buffer_vec(v, 127)
        kh, vh = kc * ks, vc * vs
    elif buf_kind == "mixed":
        kc, ks = quant_buffer_vec(k, 7)
        kh, vh = kc * ks, bf16_rne(np.asarray(v, dtype=np.float64))
    elif buf_kind == "exact":
        kh, vh = np.asarray(k, dtype=np.float64), np.asarray(v, dtype=np.float64)
    else:
        raise ValueError(buf_kind)
    return BufEntry(np.asarray(kh, dtype=np.float64), np.asarray(vh, dtype=np.float64),
                    float(a), float(beta))


# ----------------------------------------------------------------------------------
# Exact gated-delta step ([p2] "Key Terms", delta value):
#   u_t = beta_t (v_t - a_t S_{t-1}^T k_t);  S_t = a_t S_{t-1} + k_t u_t^T.
# ----------------------------------------------------------------------------------

def exact_step(S, k, v, a, beta):
    S = np.asarray(S, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    u = beta * (v - a * (S.T @ k))
    return a * S + np.outer(k, u), u


def readout(S, q):
    """o_t = S_t^T q_t."""
    return np.asarray(S, dtype=np.float64).T @ np.asarray(q, dtype=np.float64)


def exact_run(S0, ks, vs, as_, betas, qs):
    """Sequential exact recurrence over tokens; returns (outputs [T, dv], final S)."""
    S = np.array(S0, dtype=np.float64)
    outs = []
    for k, v, a, b, q in zip(ks, vs, as_, betas, qs):
        S, _ = exact_step(S, k, v, a, b)
        outs.append(readout(S, q))
    return np.array(outs), S


# ----------------------------------------------------------------------------------
# Periodic decode with a decode buffer ([p1] "How it works": round once per dP decode
# tokens, buffer the tokens in between and apply them at the flush; [p2] "Key Terms",
# decode buffer and periodic rounding).  The rounding is a pluggable function so that
# the oracle's pins can switch it off.
# ----------------------------------------------------------------------------------

@dataclass
class TileState:
    """Per-(sequence, value head) decode state: the last-rounded state (held as a QState,
    or as a float array when rounding is switched off) and the buffered tokens."""
    q: object
    buf: List[BufEntry] = field(default_factory=list)


def _deq(qstate):
    return dequantize_state(qstate) if isinstance(qstate, QState) else np.array(qstate, dtype=np.float64)


def _replay(qstate, buf):
    S = _deq(qstate)
    for e in buf:
        S, _ = exact_step(S, e.k, e.v, e.a, e.beta)
    return S


def decode_tile_step(tile: TileState, q, k, v, a, beta, dP: int, buf_kind: str, requant):
    """One decode token for one tile.  Returns (o_t, flushed?).
    1. append the token through the buffer quantiser; 2. S <- deq(last rounded state);
    3. replay every buffered token with the exact step; 4. o_t = S^T q_t;
    5. if the buffer holds dP tokens: round S once (requant), empty the buffer."""
    tile.buf.append(buffer_entry(k, v, a, beta, buf_kind))
    S = _replay(tile.q, tile.buf)
    o = readout(S, q)
    flushed = False
    if len(tile.buf) >= dP:
        tile.q = requant(S)
        tile.buf = []
        flushed = True
    return o, flushed


def flush_tile(tile: TileState, requant):
    """Explicit flush: fold the (fewer than dP) buffered tokens in and round once."""
    if not tile.buf:
        return False
    tile.q = requant(_replay(tile.q, tile.buf))
    tile.buf = []
    return True


# ----------------------------------------------------------------------------------
# Periodic decode on a bf16 state ([p1] "Assumptions and limits": in the throughput
# study most of the decode-time reduction comes from the decode buffer with the state
# still in bf16, and the 4-bit state reduces it further).  The buffer, the replay and the
# once-per-dP fold are those of decode_tile_step; only the state's storage differs: it is
# kept as bf16 values, so a flush rounds every element to the nearest bf16 (ties to
# even), decided on the fp32 value of the pre-rounding state.  Use round_state_bf16 as
# the `requant` of decode_tile_step / flush_tile; the tile's state is then a float array.
# ----------------------------------------------------------------------------------

def round_state_bf16(S):
    """The bf16 state after a flush: bf16_rne of the fp32 pre-rounding state."""
    return bf16_rne(to_f32(S))


# ----------------------------------------------------------------------------------
# Prefill ([p1] "How it works": the prefill rounding period is fixed to the chunk
# kernel's chunk length, 256 tokens; [p3] "Two observations": chunked prefill kernels
# write the state once per chunk).  Exact recurrence inside a chunk, rounding after
# every `chunk` tokens and after the last token.
# ----------------------------------------------------------------------------------

def prefill_tile(qstate, qs, ks, vs, as_, betas, chunk: int, requant):
    """Returns (outputs [T, dv], rounded state after the last token)."""
    S = _deq(qstate)
    T = len(ks)
    outs = np.zeros((T, S.shape[1]))
    cur = qstate
    for t in range(T):
        S, _ = exact_step(S, ks[t], vs[t], as_[t], betas[t])
        outs[t] = readout(S, qs[t])
        if (t + 1) % chunk == 0 or t == T - 1:
            cur = requant(S)
            S = _deq(cur)
    return outs, cur


# ----------------------------------------------------------------------------------
# Retained error and head-level precision allocation ([p1] "How it differs": the 8-bit
# heads are the ones with the largest E_h = e_h / (1 - a_h^(2 dP)); [p2] "Method": a
# quarter of the heads per layer at 8 bits).
# ----------------------------------------------------------------------------------

def retained_error(e_h, a_h, dP: int):
    """E_h = e_h / (1 - a_h^(2 dP)); +inf when a_h >= 1 (no decay retains forever)."""
    e_h = np.asarray(e_h, dtype=np.float64)
    a_h = np.asarray(a_h, dtype=np.float64)
    E = np.full(e_h.shape, np.inf)
    ok = a_h < 1.0
    E[ok] = e_h[ok] / (1.0 - a_h[ok] ** (2 * dP))
    return E


def head_alloc(e_h, a_h, dP: int, n_8bit: int):
    """Head bit widths: the n_8bit heads of largest E_h get 8 bits (ties -> lower head
    index first), the rest 4.  Returns (bits [H] int, E [H])."""
    E = retained_error(e_h, a_h, dP)
    H = len(E)
    order = sorted(range(H), key=lambda h: (-E[h], h))
    bits = np.full(H, 4, dtype=np.int64)
    for h in order[:n_8bit]:
        bits[h] = 8
    return bits, E


def quarter(H: int) -> int:
    """Number of 8-bit heads: a quarter of the heads, rounded to nearest."""
    return int(math.floor(H / 4 + 0.5))


def calibrate_heads(tokens, dP: int, bits: int = 4, group: int = 32, asym: bool = True,
                    n_tokens: Optional[int] = None):
    """Offline calibration of e_h and a_h ([p1] "How it differs": e_h is the error energy
    one rounding leaves, a_h the head's decay).  Runs the exact recurrence from S = 0;
    at every dP-th token adds ||deq(quant(S)) - S||_F^2 of the 4-bit quantiser;
    e_h = mean over those points and sequences; a_h = mean a_t over tokens and sequences.
    tokens: pace_synth.TokenInputs ([B, T, ...])."""
    q, k, v, a, beta = tokens.q, tokens.k, tokens.v, tokens.a, tokens.beta
    B, T, Hv = a.shape
    Hk, dk = k.shape[2], k.shape[3]
    dv = v.shape[3]
    gamma = Hv // Hk
    T = T if n_tokens is None else min(T, n_tokens)
    e = np.zeros(Hv)
    cnt = np.zeros(Hv)
    for b in range(B):
        for h in range(Hv):
            kh = h // gamma
            S = np.zeros((dk, dv))
            for t in range(T):
                S, _ = exact_step(S, k[b, t, kh], v[b, t, h], float(a[b, t, h]), float(beta[b, t, h]))
                if (t + 1) % dP == 0:
                    err = dequantize_state(quantize_state(S, bits, group, asym)) - S
                    e[h] += float(np.sum(err * err))
                    cnt[h] += 1
    e_h = e / np.maximum(cnt, 1)
    a_h = np.mean(a[:, :T, :].astype(np.float64), axis=(0, 1))
    return e_h, a_h


# ----------------------------------------------------------------------------------
# Bit accounting ([p1] "How it works": the buffer is resident memory, cost per state
# value c dP with c = (b_k dk / gamma + b_v dv + 32) / (dk dv); [p1] "How it differs":
# PACE-4/8 payload 5.66 bits per value).
# ----------------------------------------------------------------------------------

def payload_bits(head_bits, group: int, asym: bool) -> float:
    """Mean over heads of b_h + (16 + z_h) / g: b-bit codes, one bf16 scale per g values,
    and (asym) one b-bit zero point per g values."""
    hb = np.asarray(head_bits, dtype=np.float64)
    z = hb if asym else np.zeros_like(hb)
    return float(np.mean(hb + (16.0 + z) / group))


def buffer_cost_per_token(dk, dv, gamma, b_k, b_v) -> float:
    """c = (b_k dk / gamma + b_v dv + 32) / (dk dv)."""
    return (b_k * dk / gamma + b_v * dv + 32.0) / (dk * dv)


def buffer_bits_model(dk, dv, gamma, dP, buf_kind: str) -> float:
    b_k, b_v = {"int8": (8, 8), "mixed": (4, 16)}[buf_kind]
    return buffer_cost_per_token(dk, dv, gamma, b_k, b_v) * dP


def resident_bits(head_bits, group, asym, dk, dv, gamma, dP, buf_kind) -> float:
    return payload_bits(head_bits, group, asym) + buffer_bits_model(dk, dv, gamma, dP, buf_kind)

"""Seeded synthetic inputs for the PACE decode / prefill path.

This module only draws random numbers and shapes them.  It holds none of the method's
arithmetic (no recurrence, no quantiser, no packing rule), so the fp64 oracle and the
HIP path can both take their inputs from it without sharing any computation.

Distributions follow the workload description of the gated-delta token mixer used to
study PACE on Qwen3.5-shaped layers:
  q, k ~ N(0, 1), then L2-normalised per (token, key head);
  v ~ N(0, 1);
  a = exp(-softplus(x)), x ~ N(-4, 1)  (per sequence, token, value head);
  beta = sigmoid(N(0, 1));
  optional column outliers: per head, `n_outlier` of the dv value channels are chosen
  without replacement; for each (sequence, head, channel) the token timeline alternates
  off/on runs with lengths uniform in [run_lo, run_hi] and a random initial phase, and
  v is multiplied by `outlier_gain` on "on" runs.  This produces the column structure of
  the state that channel-aligned scale groups target (PACE paper review, "3. Method &
  Key Results", Figure 3 discussion).
Draw order is fixed: q, k, v, gate logits, beta logits, outlier channels, outlier runs.

bf16 inputs are produced as float32 arrays whose values are exactly representable in
bf16 (round to nearest even on the float32 bit pattern), so both sides see the same
numbers.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "round_to_bf16", "bf16_bits", "from_bf16_bits",
    "TokenInputs", "make_tokens", "random_packed_state_parts", "random_buffer_parts", "random_bf16_state",
]


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bf16 value (ties to even), as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # finite patterns stay below 2^32 after the increment (at most 0xFF807FFF)
    u = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) & np.uint32(0xFFFF0000)
    return u.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are already bf16-representable."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def from_bf16_bits(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


class TokenInputs:
    """q, k: [B, T, Hk, dk]; v: [B, T, Hv, dv]; a, beta: [B, T, Hv] (float32)."""

    def __init__(self, q, k, v, a, beta, outlier_channels=None):
        self.q, self.k, self.v, self.a, self.beta = q, k, v, a, beta
        self.outlier_channels = outlier_channels

    @property
    def T(self):
        return self.q.shape[1]

    def token(self, t):
        """Inputs of token t for every sequence: q, k [B, Hk, dk]; v [B, Hv, dv]; a, beta [B, Hv]."""
        return (self.q[:, t], self.k[:, t], self.v[:, t], self.a[:, t], self.beta[:, t])

    def span(self, t0, t1):
        return (self.q[:, t0:t1], self.k[:, t0:t1], self.v[:, t0:t1],
                self.a[:, t0:t1], self.beta[:, t0:t1])


def _softplus(x):
    return np.logaddexp(0.0, x)


def make_tokens(seed: int, B: int, T: int, Hv: int, Hk: int, dk: int, dv: int,
                bf16: bool = False, n_outlier: int = 0, outlier_gain: float = 8.0,
                run_lo: int = 50, run_hi: int = 200) -> TokenInputs:
    """Seeded token stream of T tokens for B sequences (see module docstring)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((B, T, Hk, dk))
    k = rng.standard_normal((B, T, Hk, dk))
    v = rng.standard_normal((B, T, Hv, dv))
    gate_logit = rng.normal(-4.0, 1.0, size=(B, T, Hv))
    beta_logit = rng.standard_normal((B, T, Hv))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    a = np.exp(-_softplus(gate_logit))
    beta = 1.0 / (1.0 + np.exp(-beta_logit))
    chans = None
    if n_outlier > 0:
        chans = np.stack([rng.choice(dv, size=n_outlier, replace=False) for _ in range(Hv)])
        gain = np.ones((B, T, Hv, dv))
        for b in range(B):
            for h in range(Hv):
                for c in chans[h]:
                    on = bool(rng.integers(0, 2))
                    t = 0
                    while t < T:
                        run = int(rng.integers(run_lo, run_hi + 1))
                        if on:
                            gain[b, t:t + run, h, c] = outlier_gain
                        on = not on
                        t += run
        v = v * gain
    f32 = np.float32
    q, k, v = q.astype(f32), k.astype(f32), v.astype(f32)
    if bf16:
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    return TokenInputs(q, k, v, a.astype(f32), beta.astype(f32), chans)


def make_tokens_chunk(seed: int, chunk: int, B: int, T: int, Hv: int, Hk: int, dk: int, dv: int,
                      bf16: bool = False) -> TokenInputs:
    """Chunk `chunk` (T tokens) of a long seeded token stream, generated on its own
    (seed sequence [seed, chunk]) so that streams of any length fit in memory; same
    distributions and draw order as make_tokens without outlier channels."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, chunk])))
    q = rng.standard_normal((B, T, Hk, dk))
    k = rng.standard_normal((B, T, Hk, dk))
    v = rng.standard_normal((B, T, Hv, dv))
    gate_logit = rng.normal(-4.0, 1.0, size=(B, T, Hv))
    beta_logit = rng.standard_normal((B, T, Hv))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    a = np.exp(-_softplus(gate_logit))
    beta = 1.0 / (1.0 + np.exp(-beta_logit))
    f32 = np.float32
    q, k, v = q.astype(f32), k.astype(f32), v.astype(f32)
    if bf16:
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    return TokenInputs(q, k, v, a.astype(f32), beta.astype(f32), None)


def random_packed_state_parts(seed: int, B: int, Hv: int, dk: int, dv: int, group: int,
                              head_bits, asym: bool, scale_mag: float = 0.05):
    """Random per-(sequence, head) quantised-state fields, for one-step parity tests.

    Returns a list over b of lists over h of (stored_codes uint8 [dk, dv] in [0, 2^b - 1],
    scales float32 [dk/group, dv] (bf16-representable, positive), zeros uint8
    [dk/group, dv] or None).  Any stored code value is a legal state, so these need no
    quantiser to produce.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for b in range(B):
        row = []
        for h in range(Hv):
            bits = int(head_bits[h])
            hi = (1 << bits) - 1
            codes = rng.integers(0, hi + 1, size=(dk, dv)).astype(np.uint8)
            scales = round_to_bf16((np.abs(rng.standard_normal((dk // group, dv))) * scale_mag
                                    + 1e-3).astype(np.float32))
            zeros = rng.integers(0, hi + 1, size=(dk // group, dv)).astype(np.uint8) if asym else None
            row.append((codes, scales, zeros))
        out.append(row)
    return out


def random_bf16_state(seed: int, B: int, Hv: int, dk: int, dv: int, scale: float = 0.3):
    """Seeded random bf16-representable state values [B, Hv, dk, dv] (float32), drawn
    N(0, scale^2) and rounded to bf16: any such array is a legal bf16 state."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return round_to_bf16((rng.standard_normal((B, Hv, dk, dv)) * scale).astype(np.float32))


def random_buffer_parts(seed: int, B: int, Hv: int, Hk: int, dk: int, dv: int, dP: int,
                        mixed: bool, counts=None):
    """Random decode-buffer fields (codes, scales, gates) and per-sequence counts.

    counts: None = uniform random in [0, dP-1] per sequence.  Returns a dict of arrays:
      count [B] int32; kc [B, Hk, dP, dk] int8 codes (|c| <= 127, or <= 7 when mixed);
      ks [B, Hk, dP] float32; vc [B, Hv, dP, dv] int8 (int8 buffer) or
      v [B, Hv, dP, dv] bf16-representable float32 (mixed); vs [B, Hv, dP] float32;
      a, beta [B, Hv, dP] float32 drawn like the token gates.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    if counts is None:
        counts = rng.integers(0, dP, size=B)
    counts = np.asarray(counts, dtype=np.int32)
    kmax = 7 if mixed else 127
    kc = rng.integers(-kmax, kmax + 1, size=(B, Hk, dP, dk)).astype(np.int8)
    ks = (np.abs(rng.standard_normal((B, Hk, dP))) * 1e-3 + 1.5e-3).astype(np.float32)
    d = {"count": counts, "kc": kc, "ks": ks}
    if mixed:
        d["v"] = round_to_bf16(rng.standard_normal((B, Hv, dP, dv)).astype(np.float32))
    else:
        d["vc"] = rng.integers(-127, 128, size=(B, Hv, dP, dv)).astype(np.int8)
        d["vs"] = (np.abs(rng.standard_normal((B, Hv, dP))) * 0.02 + 1e-3).astype(np.float32)
    gate_logit = rng.normal(-4.0, 1.0, size=(B, Hv, dP))
    d["a"] = np.exp(-_softplus(gate_logit)).astype(np.float32)
    d["beta"] = (1.0 / (1.0 + np.exp(-rng.standard_normal((B, Hv, dP))))).astype(np.float32)
    return d

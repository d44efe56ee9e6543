"""Byte layout of the packed state and the decode buffer, written by the oracle from
the layout specification (the comment block of include/pace.h) -- TEST INFRASTRUCTURE.

This is the oracle's own reading of the specification; it shares no code with the
library's host or device side.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may use it.

Also holds the layer-level oracle routines (decode step, flush, prefill) that work on
packed bytes, built from the per-tile functions of pace_oracle.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

from . import pace_oracle as po


def _pad(n: int, a: int) -> int:
    return (n + a - 1) // a * a


@dataclass
class LayerCfg:
    """Mirror of the C struct pace_layer_cfg (oracle side)."""
    B: int
    Hv: int
    Hk: int
    dk: int
    dv: int
    group: int
    asym: bool
    buf: str            # 'int8' | 'mixed'
    dP: int
    chunk: int = 256
    bf16_io: bool = False
    head_bits: Optional[Sequence[int]] = None
    bf16_state: bool = False   # state kept as bf16 values (periodic decode on a bf16 state)

    @property
    def gamma(self) -> int:
        return self.Hv // self.Hk

    def bits(self, h: int) -> int:
        return 4 if self.head_bits is None else int(self.head_bits[h])


# ------------------------------------------------------------------------- state ----

def record_parts(cfg: LayerCfg, bits: int):
    if cfg.bf16_state:                   # dv columns of dk bf16 values, nothing else
        return cfg.dv * cfg.dk * 2, 0, 0, cfg.dv * cfg.dk * 2
    codes = cfg.dv * cfg.dk * bits // 8
    scales = cfg.dv * (cfg.dk // cfg.group) * 2
    zeros = cfg.dv * (cfg.dk // cfg.group) * bits // 8 if cfg.asym else 0
    c, s, z = _pad(codes, 16), _pad(scales, 16), _pad(zeros, 16)
    return c, s, z, _pad(c + s + z, 256)


def state_layout(cfg: LayerCfg):
    """(head offsets [Hv], sequence stride, total bytes)."""
    offs, o = [], 0
    for h in range(cfg.Hv):
        offs.append(o)
        o += record_parts(cfg, cfg.bits(h))[3]
    return offs, o, o * cfg.B


def unit_base(u: int, dk: int) -> int:
    """First key of 8-key unit u inside a column."""
    kb = dk // 32
    return 32 * (u % kb) + 8 * (u // kb)


def _pack_column(stored: np.ndarray, bits: int, dk: int) -> np.ndarray:
    out = np.zeros(dk * bits // 8, dtype=np.uint8)
    for u in range(dk // 8):
        base = unit_base(u, dk)
        if bits == 4:
            for w in range(4):
                lo, hi = int(stored[base + w]), int(stored[base + 4 + w])
                out[u * 4 + w] = (lo & 15) | ((hi & 15) << 4)
        else:
            for e in range(8):
                out[u * 8 + e] = int(stored[base + e]) & 255
    return out


def _unpack_column(raw: np.ndarray, bits: int, dk: int) -> np.ndarray:
    stored = np.zeros(dk, dtype=np.int64)
    for u in range(dk // 8):
        base = unit_base(u, dk)
        if bits == 4:
            for w in range(4):
                byte = int(raw[u * 4 + w])
                stored[base + w] = byte & 15
                stored[base + 4 + w] = byte >> 4
        else:
            for e in range(8):
                stored[base + e] = int(raw[u * 8 + e])
    return stored


def _bf16_to_bytes(vals: np.ndarray) -> np.ndarray:
    v32 = np.asarray(vals, dtype=np.float64).astype(np.float32)
    bits = (v32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    if not np.array_equal(bits.astype(np.uint32) << np.uint32(16), v32.view(np.uint32)):
        raise ValueError("value not representable in bf16")
    return bits.view(np.uint8)


def _bytes_to_bf16(raw: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(raw).view(np.uint16).astype(np.uint32) << np.uint32(16)
    return bits.view(np.float32).astype(np.float64)


def pack_record(cfg: LayerCfg, qs) -> np.ndarray:
    if cfg.bf16_state:
        # value-column-major: element (key r, column j) at bf16 index j * dk + r
        S = np.asarray(qs, dtype=np.float64)
        return _bf16_to_bytes(np.ascontiguousarray(S.T).reshape(-1))
    bits = qs.bits
    c, s, z, rec = record_parts(cfg, bits)
    out = np.zeros(rec, dtype=np.uint8)
    colb = cfg.dk * bits // 8
    for j in range(cfg.dv):
        out[j * colb:(j + 1) * colb] = _pack_column(qs.codes[:, j], bits, cfg.dk)
    ng = cfg.dk // cfg.group
    sc = np.zeros(cfg.dv * ng)
    for j in range(cfg.dv):
        for G in range(ng):
            sc[j * ng + G] = qs.scales[G, j]
    out[c:c + cfg.dv * ng * 2] = _bf16_to_bytes(sc)
    if cfg.asym:
        zz = np.zeros(cfg.dv * ng, dtype=np.int64)
        for j in range(cfg.dv):
            for G in range(ng):
                zz[j * ng + G] = qs.zeros[G, j]
        if bits == 8:
            out[c + s:c + s + cfg.dv * ng] = zz.astype(np.uint8)
        else:
            for e in range(0, cfg.dv * ng, 2):
                out[c + s + e // 2] = (zz[e] & 15) | ((zz[e + 1] & 15) << 4)
    return out


def unpack_record(cfg: LayerCfg, raw: np.ndarray, bits: int):
    if cfg.bf16_state:
        vals = _bytes_to_bf16(raw[:cfg.dv * cfg.dk * 2])
        return vals.reshape(cfg.dv, cfg.dk).T.copy()
    c, s, z, rec = record_parts(cfg, bits)
    colb = cfg.dk * bits // 8
    codes = np.zeros((cfg.dk, cfg.dv), dtype=np.int64)
    for j in range(cfg.dv):
        codes[:, j] = _unpack_column(raw[j * colb:(j + 1) * colb], bits, cfg.dk)
    ng = cfg.dk // cfg.group
    sc = _bytes_to_bf16(raw[c:c + cfg.dv * ng * 2])
    scales = np.zeros((ng, cfg.dv))
    for j in range(cfg.dv):
        for G in range(ng):
            scales[G, j] = sc[j * ng + G]
    zeros = None
    if cfg.asym:
        zz = np.zeros(cfg.dv * ng, dtype=np.int64)
        if bits == 8:
            zz[:] = raw[c + s:c + s + cfg.dv * ng]
        else:
            for e in range(cfg.dv * ng):
                byte = int(raw[c + s + e // 2])
                zz[e] = (byte & 15) if e % 2 == 0 else (byte >> 4)
        zeros = np.zeros((ng, cfg.dv), dtype=np.int64)
        for j in range(cfg.dv):
            for G in range(ng):
                zeros[G, j] = zz[j * ng + G]
    return po.QState(codes, scales, zeros, bits, cfg.group, cfg.asym)


def pack_state(cfg: LayerCfg, qstates) -> np.ndarray:
    """qstates[b][h] -> state bytes of the layer."""
    offs, stride, total = state_layout(cfg)
    out = np.zeros(total, dtype=np.uint8)
    for b in range(cfg.B):
        for h in range(cfg.Hv):
            rec = pack_record(cfg, qstates[b][h])
            o = b * stride + offs[h]
            out[o:o + len(rec)] = rec
    return out


def unpack_state(cfg: LayerCfg, raw: np.ndarray, tiles=None):
    """State bytes -> qstates[b][h] (None for tiles not requested)."""
    offs, stride, _ = state_layout(cfg)
    raw = np.asarray(raw, dtype=np.uint8)
    out = [[None] * cfg.Hv for _ in range(cfg.B)]
    want = tiles if tiles is not None else [(b, h) for b in range(cfg.B) for h in range(cfg.Hv)]
    for b, h in want:
        bits = cfg.bits(h)
        o = b * stride + offs[h]
        out[b][h] = unpack_record(cfg, raw[o:o + record_parts(cfg, bits)[3]], bits)
    return out


def state_from_parts(cfg: LayerCfg, parts) -> list:
    """pace_synth.random_packed_state_parts output -> qstates[b][h]."""
    out = []
    for b in range(cfg.B):
        row = []
        for h in range(cfg.Hv):
            codes, scales, zeros = parts[b][h]
            row.append(po.QState(codes.astype(np.int64), scales.astype(np.float64),
                                 None if zeros is None else zeros.astype(np.int64),
                                 cfg.bits(h), cfg.group, cfg.asym))
        out.append(row)
    return out


# ------------------------------------------------------------------------ buffer ----

def buffer_regions(cfg: LayerCfg):
    """Ordered (name, dtype, shape) of the buffer regions; each padded to 256 bytes."""
    B, Hv, Hk, dP, dk, dv = cfg.B, cfg.Hv, cfg.Hk, cfg.dP, cfg.dk, cfg.dv
    regs = [("count", np.int32, (B, Hv))]
    if cfg.buf == "int8":
        regs += [("kc", np.int8, (B, Hk, dP, dk)), ("ks", np.float32, (B, Hk, dP)),
                 ("vc", np.int8, (B, Hv, dP, dv)), ("vs", np.float32, (B, Hv, dP))]
    elif cfg.buf == "mixed":
        regs += [("kc", np.uint8, (B, Hk, dP, dk // 2)), ("ks", np.float32, (B, Hk, dP)),
                 ("v", np.uint16, (B, Hv, dP, dv))]
    else:
        raise ValueError(cfg.buf)
    regs += [("a", np.float32, (B, Hv, dP)), ("beta", np.float32, (B, Hv, dP))]
    return regs


def buffer_layout(cfg: LayerCfg):
    offs, o = {}, 0
    for name, dt, shape in buffer_regions(cfg):
        offs[name] = o
        o += _pad(int(np.prod(shape)) * np.dtype(dt).itemsize, 256)
    return offs, o


def _pack_k4(codes: np.ndarray) -> np.ndarray:
    """[..., dk] symmetric 4-bit codes -> [..., dk/2] bytes (stored c + 8, 8-key units)."""
    st = (codes.astype(np.int64) + 8) & 15
    dk = st.shape[-1]
    out = np.zeros(st.shape[:-1] + (dk // 2,), dtype=np.uint8)
    for m in range(dk // 8):
        for w in range(4):
            out[..., m * 4 + w] = (st[..., 8 * m + w] | (st[..., 8 * m + 4 + w] << 4)).astype(np.uint8)
    return out


def _unpack_k4(raw: np.ndarray) -> np.ndarray:
    dk = raw.shape[-1] * 2
    out = np.zeros(raw.shape[:-1] + (dk,), dtype=np.int64)
    for m in range(dk // 8):
        for w in range(4):
            byte = raw[..., m * 4 + w].astype(np.int64)
            out[..., 8 * m + w] = (byte & 15) - 8
            out[..., 8 * m + 4 + w] = (byte >> 4) - 8
    return out


def pack_buffer(cfg: LayerCfg, d: dict) -> np.ndarray:
    """Buffer fields (as from pace_synth.random_buffer_parts or unpack_buffer) -> bytes.
    count may be [B] (per sequence) or [B, Hv]."""
    offs, total = buffer_layout(cfg)
    out = np.zeros(total, dtype=np.uint8)
    cnt = np.asarray(d["count"], dtype=np.int32)
    if cnt.ndim == 1:
        cnt = np.repeat(cnt[:, None], cfg.Hv, axis=1)
    fields = {"count": cnt, "ks": d["ks"], "a": d["a"], "beta": d["beta"]}
    if cfg.buf == "int8":
        fields.update(kc=d["kc"], vc=d["vc"], vs=d["vs"])
    else:
        fields.update(kc=_pack_k4(np.asarray(d["kc"])),
                      v=(np.asarray(d["v"], dtype=np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16))
    for name, dt, shape in buffer_regions(cfg):
        arr = np.ascontiguousarray(np.asarray(fields[name]).astype(dt).reshape(shape))
        raw = arr.view(np.uint8).reshape(-1)
        out[offs[name]:offs[name] + raw.size] = raw
    return out


def unpack_buffer(cfg: LayerCfg, raw: np.ndarray) -> dict:
    offs, _ = buffer_layout(cfg)
    raw = np.asarray(raw, dtype=np.uint8)
    d = {}
    for name, dt, shape in buffer_regions(cfg):
        n = int(np.prod(shape)) * np.dtype(dt).itemsize
        d[name] = raw[offs[name]:offs[name] + n].copy().view(dt).reshape(shape)
    if cfg.buf == "mixed":
        d["kc"] = _unpack_k4(d["kc"])
        d["v"] = (d["v"].astype(np.uint32) << np.uint32(16)).view(np.float32)
    return d


def _entry(cfg: LayerCfg, d: dict, b: int, h: int, i: int) -> po.BufEntry:
    kh = h // cfg.gamma
    k = d["kc"][b, kh, i].astype(np.float64) * float(d["ks"][b, kh, i])
    if cfg.buf == "int8":
        v = d["vc"][b, h, i].astype(np.float64) * float(d["vs"][b, h, i])
    else:
        v = np.asarray(d["v"][b, h, i], dtype=np.float64)
    return po.BufEntry(k, v, float(d["a"][b, h, i]), float(d["beta"][b, h, i]))


def _store_token(cfg: LayerCfg, d: dict, b: int, h: int, slot: int, k, v, a, beta, write_key: bool):
    """Write one token's buffer codes (the oracle's buffer quantiser) into slot."""
    kh = h // cfg.gamma
    if cfg.buf == "int8":
        kc, ks = po.quant_buffer_vec(k, 127)
        vc, vs = po.quant_buffer_vec(v, 127)
        d["vc"][b, h, slot] = vc
        d["vs"][b, h, slot] = vs
    else:
        kc, ks = po.quant_buffer_vec(k, 7)
        d["v"][b, h, slot] = po.bf16_rne(np.asarray(v, dtype=np.float64)).astype(np.float32)
    if write_key:
        d["kc"][b, kh, slot] = kc
        d["ks"][b, kh, slot] = ks
    d["a"][b, h, slot] = a
    d["beta"][b, h, slot] = beta


def _requant_fn(cfg: LayerCfg, bits: int):
    if cfg.bf16_state:
        return po.round_state_bf16
    return lambda S: po.quantize_state(S, bits, cfg.group, cfg.asym)


def decode_step_layer(cfg: LayerCfg, state: np.ndarray, buf: np.ndarray, q, k, v, a, beta,
                      active=None, tiles=None):
    """Oracle of pace_decode_step on packed bytes.

    q, k [B, Hk, dk]; v [B, Hv, dv]; a, beta [B, Hv].  tiles: optional list of (b, h)
    to compute (others are left untouched and their o rows NaN).  Returns
    (o [B, Hv, dv] float64, new state bytes, new buffer bytes, pre-rounding states
    {(b, h): S} of the tiles that flushed)."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    a, beta = np.asarray(a, dtype=np.float64), np.asarray(beta, dtype=np.float64)
    want = tiles if tiles is not None else [(b, h) for b in range(cfg.B) for h in range(cfg.Hv)]
    if active is not None:
        want = [(b, h) for b, h in want if active[b]]
    qstates = unpack_state(cfg, state, want)
    d = unpack_buffer(cfg, buf)
    d_out = {key: val.copy() for key, val in d.items()}
    o = np.full((cfg.B, cfg.Hv, cfg.dv), np.nan)
    pre = {}
    offs, stride, _ = state_layout(cfg)
    new_state = np.array(state, dtype=np.uint8, copy=True)
    for b, h in want:
        n0 = int(d["count"][b, h])
        kh = h // cfg.gamma
        entries = [_entry(cfg, d, b, h, i) for i in range(n0)]
        tile = po.TileState(qstates[b][h], entries)
        captured = {}

        def requant(S, _b=b, _h=h, _cap=captured):
            _cap["S"] = S
            return _requant_fn(cfg, cfg.bits(_h))(S)

        ob, flushed = po.decode_tile_step(tile, q[b, kh], k[b, kh], v[b, h], a[b, h], beta[b, h],
                                          cfg.dP, cfg.buf, requant)
        o[b, h] = ob
        if flushed:
            pre[(b, h)] = captured["S"]
            rec = pack_record(cfg, tile.q)
            off = b * stride + offs[h]
            new_state[off:off + len(rec)] = rec
            d_out["count"][b, h] = 0
        else:
            _store_token(cfg, d_out, b, h, n0, k[b, kh], v[b, h], a[b, h], beta[b, h],
                         write_key=(h % cfg.gamma == 0))
            d_out["count"][b, h] = n0 + 1
    new_buf = _repack_buffer(cfg, d_out)
    return o, new_state, new_buf, pre


def _repack_buffer(cfg: LayerCfg, d: dict) -> np.ndarray:
    return pack_buffer(cfg, d)


def flush_layer(cfg: LayerCfg, state: np.ndarray, buf: np.ndarray, seq_mask=None, tiles=None):
    """Oracle of pace_flush_requant.  Returns (new state bytes, new buffer bytes, pre)."""
    want = tiles if tiles is not None else [(b, h) for b in range(cfg.B) for h in range(cfg.Hv)]
    if seq_mask is not None:
        want = [(b, h) for b, h in want if seq_mask[b]]
    d = unpack_buffer(cfg, buf)
    qstates = unpack_state(cfg, state, want)
    offs, stride, _ = state_layout(cfg)
    new_state = np.array(state, dtype=np.uint8, copy=True)
    pre = {}
    for b, h in want:
        n0 = int(d["count"][b, h])
        if n0 == 0:
            continue
        tile = po.TileState(qstates[b][h], [_entry(cfg, d, b, h, i) for i in range(n0)])
        cap = {}

        def requant(S, _h=h, _cap=cap):
            _cap["S"] = S
            return _requant_fn(cfg, cfg.bits(_h))(S)

        po.flush_tile(tile, requant)
        pre[(b, h)] = cap["S"]
        rec = pack_record(cfg, tile.q)
        off = b * stride + offs[h]
        new_state[off:off + len(rec)] = rec
        d["count"][b, h] = 0
    return new_state, pack_buffer(cfg, d), pre


def prefill_layer(cfg: LayerCfg, state: np.ndarray, q, k, v, a, beta, tiles=None):
    """Oracle of pace_prefill_chunk.  q, k [B, T, Hk, dk]; v [B, T, Hv, dv]; a, beta
    [B, T, Hv].  Returns (o [B, T, Hv, dv], new state bytes, pre-rounding state of the
    last chunk {(b, h): S})."""
    if cfg.bf16_state:
        raise ValueError("prefill is defined for the packed states only")
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    a, beta = np.asarray(a, dtype=np.float64), np.asarray(beta, dtype=np.float64)
    B, T = a.shape[0], a.shape[1]
    want = tiles if tiles is not None else [(b, h) for b in range(cfg.B) for h in range(cfg.Hv)]
    qstates = unpack_state(cfg, state, want)
    offs, stride, _ = state_layout(cfg)
    new_state = np.array(state, dtype=np.uint8, copy=True)
    o = np.full((B, T, cfg.Hv, cfg.dv), np.nan)
    pre = {}
    for b, h in want:
        kh = h // cfg.gamma
        cap = {}

        def requant(S, _h=h, _cap=cap):
            _cap["S"] = S
            return _requant_fn(cfg, cfg.bits(_h))(S)

        ob, qs = po.prefill_tile(qstates[b][h], q[b, :, kh], k[b, :, kh], v[b, :, h],
                                 a[b, :, h], beta[b, :, h], cfg.chunk, requant)
        o[b, :, h] = ob
        pre[(b, h)] = cap["S"]
        rec = pack_record(cfg, qs)
        off = b * stride + offs[h]
        new_state[off:off + len(rec)] = rec
    return o, new_state, pre

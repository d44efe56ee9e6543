"""ctypes binding of libpace.so (the C ABI declared in include/pace.h).

Argument marshalling only: every step of the decode / prefill path runs in the HIP
kernels behind the C ABI.  There is no fallback: if the library is missing, importing
this module raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpace.so")

PACE_OK, PACE_EINVAL, PACE_EUNSUPPORTED, PACE_EHIP = 0, -1, -2, -3
STATE_SYM, STATE_ASYM, STATE_BF16 = 0, 1, 2
BUF_INT8, BUF_K4_VBF16 = 0, 1
IO_F32, IO_BF16 = 0, 1


class PaceError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {_status_str(status)} ({status})")
        self.status = status


class _Cfg(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hv", ctypes.c_int32), ("Hk", ctypes.c_int32),
                ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("group", ctypes.c_int32),
                ("state_kind", ctypes.c_int32), ("buf_kind", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("dP", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("head_bits", ctypes.POINTER(ctypes.c_int8))]


class _Info(ctypes.Structure):
    _fields_ = [("state_bytes", ctypes.c_size_t), ("buffer_bytes", ctypes.c_size_t),
                ("workspace_bytes", ctypes.c_size_t), ("seq_stride", ctypes.c_size_t),
                ("payload_bits", ctypes.c_double), ("buffer_bits_model", ctypes.c_double),
                ("buffer_bits_actual", ctypes.c_double)]


EXPORTS = ["pace_layout", "pace_head_alloc", "pace_calibrate_heads", "pace_prefill_chunk",
           "pace_prefill_workspace_bytes", "pace_decode_step", "pace_decode_step_ordered",
           "pace_flush_requant", "pace_bf16_decode_step", "pace_status_str"]


def _load():
    # torch ships its own HIP runtime, under the same soname as ROCm's.  Load torch first
    # so that libpace.so binds to that runtime: loaded the other way round, the process
    # can hold two HIP runtimes, and kernels launched through one on memory allocated
    # through the other fail.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m bit_recurrent_state_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    P, C = ctypes.c_void_p, ctypes.POINTER(_Cfg)
    lib.pace_layout.argtypes = [C, ctypes.POINTER(_Info)]
    lib.pace_head_alloc.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_double),
                                    ctypes.POINTER(ctypes.c_double), ctypes.c_int32,
                                    ctypes.POINTER(ctypes.c_int8), ctypes.POINTER(ctypes.c_double)]
    lib.pace_prefill_chunk.argtypes = [C, P, P, P, P, P, P, ctypes.c_int32, P, P, ctypes.c_size_t, P]
    lib.pace_prefill_workspace_bytes.argtypes = [C, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
    lib.pace_decode_step.argtypes = [C, P, P, P, P, P, P, P, P, P, P]
    lib.pace_decode_step_ordered.argtypes = [C, P, P, P, P, P, P, P, P, ctypes.POINTER(ctypes.c_int32), P, P]
    lib.pace_flush_requant.argtypes = [C, P, P, P, P]
    lib.pace_bf16_decode_step.argtypes = [C, P, P, P, P, P, P, P, P]
    lib.pace_calibrate_heads.argtypes = [C, P, P, P, P, ctypes.c_int32, P, P, P]
    lib.pace_status_str.argtypes = [ctypes.c_int]
    lib.pace_status_str.restype = ctypes.c_char_p
    for name in ["pace_layout", "pace_head_alloc", "pace_prefill_chunk", "pace_prefill_workspace_bytes",
                 "pace_decode_step",
                 "pace_decode_step_ordered", "pace_flush_requant", "pace_bf16_decode_step", "pace_calibrate_heads"]:
        getattr(lib, name).restype = ctypes.c_int
    return lib


LIB = _load()


def _status_str(s: int) -> str:
    return LIB.pace_status_str(s).decode()


def _check(status: int, what: str):
    if status != PACE_OK:
        raise PaceError(status, what)


@dataclass
class LayerConfig:
    """Python mirror of pace_layer_cfg."""
    B: int
    Hv: int
    Hk: int
    dk: int
    dv: int
    group: int
    asym: bool = False
    buf: str = "int8"            # 'int8' | 'mixed'
    bf16_io: bool = True
    dP: int = 8
    chunk: int = 256
    head_bits: Optional[Sequence[int]] = None
    bf16_state: bool = False     # state kept as bf16 values (PACE_STATE_BF16)

    def _c(self):
        hb = None
        if self.head_bits is not None:
            hb = (ctypes.c_int8 * self.Hv)(*[int(x) for x in self.head_bits])
        cfg = _Cfg(self.B, self.Hv, self.Hk, self.dk, self.dv, self.group,
                   STATE_BF16 if self.bf16_state else (STATE_ASYM if self.asym else STATE_SYM),
                   BUF_INT8 if self.buf == "int8" else BUF_K4_VBF16,
                   IO_BF16 if self.bf16_io else IO_F32, self.dP, self.chunk,
                   ctypes.cast(hb, ctypes.POINTER(ctypes.c_int8)) if hb is not None else None)
        cfg._keep = hb
        return cfg


def layout(cfg: LayerConfig) -> dict:
    info = _Info()
    c = cfg._c()
    _check(LIB.pace_layout(ctypes.byref(c), ctypes.byref(info)), "pace_layout")
    return {f: getattr(info, f) for f, _ in _Info._fields_}


def head_alloc(e_h, a_h, dP: int, n_8bit: int):
    import numpy as np
    e = np.ascontiguousarray(e_h, dtype=np.float64)
    a = np.ascontiguousarray(a_h, dtype=np.float64)
    H = len(e)
    bits = np.zeros(H, dtype=np.int8)
    E = np.zeros(H, dtype=np.float64)
    dp = ctypes.POINTER(ctypes.c_double)
    _check(LIB.pace_head_alloc(H, dP, e.ctypes.data_as(dp), a.ctypes.data_as(dp), n_8bit,
                               bits.ctypes.data_as(ctypes.POINTER(ctypes.c_int8)), E.ctypes.data_as(dp)),
           "pace_head_alloc")
    return bits, E


# ----------------------------------------------------------------- device calls ----

def _ptr(t, name, dtype=None, numel=None, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _io(cfg):
    import torch
    return torch.bfloat16 if cfg.bf16_io else torch.float32


def _order(cfg: LayerConfig, order):
    """Host int32 copy of a sequence order (pace_decode_step_ordered checks it)."""
    arr = np.ascontiguousarray(np.asarray(order, dtype=np.int32))
    if arr.shape != (cfg.B,):
        raise ValueError(f"order: expected {cfg.B} sequence indices, got shape {arr.shape}")
    return arr, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _decode_args(cfg: LayerConfig, state, buffer, q, k, v, a, beta, o, active, stream, order):
    """(function, name, marshalled arguments, objects to keep alive) of one decode step."""
    import torch
    L = layout(cfg)
    io = _io(cfg)
    c = cfg._c()
    head = (ctypes.byref(c), _ptr(state, "state", torch.uint8, L["state_bytes"]),
            _ptr(buffer, "buffer", torch.uint8, L["buffer_bytes"]),
            _ptr(q, "q", io, cfg.B * cfg.Hk * cfg.dk), _ptr(k, "k", io, cfg.B * cfg.Hk * cfg.dk),
            _ptr(v, "v", io, cfg.B * cfg.Hv * cfg.dv), _ptr(a, "a", torch.float32, cfg.B * cfg.Hv),
            _ptr(beta, "beta", torch.float32, cfg.B * cfg.Hv),
            _ptr(active, "active", torch.uint8, cfg.B, optional=True))
    tail = (_ptr(o, "o", io, cfg.B * cfg.Hv * cfg.dv), _stream(stream))
    if order is None:
        return LIB.pace_decode_step, "pace_decode_step", head + tail, (c,)
    arr, ptr = _order(cfg, order)
    return LIB.pace_decode_step_ordered, "pace_decode_step_ordered", head + (ptr,) + tail, (c, arr)


def decode_step(cfg: LayerConfig, state, buffer, q, k, v, a, beta, o, active=None, stream=None,
                order=None):
    """pace_decode_step (pace_decode_step_ordered when `order` is given: a host sequence
    of the B sequence indices, the sequences to start first listed first).  q, k
    [B, Hk, dk]; v, o [B, Hv, dv]; a, beta fp32 [B, Hv]; state / buffer uint8 tensors of
    pace_layout sizes; active optional uint8 [B]."""
    fn, name, args, _keep = _decode_args(cfg, state, buffer, q, k, v, a, beta, o, active, stream, order)
    _check(fn(*args), name)


def flush_requant(cfg: LayerConfig, state, buffer, seq_mask=None, stream=None):
    import torch
    L = layout(cfg)
    c = cfg._c()
    st = LIB.pace_flush_requant(ctypes.byref(c), _ptr(state, "state", torch.uint8, L["state_bytes"]),
                                _ptr(buffer, "buffer", torch.uint8, L["buffer_bytes"]),
                                _ptr(seq_mask, "seq_mask", torch.uint8, cfg.B, optional=True),
                                _stream(stream))
    _check(st, "pace_flush_requant")


def prefill_workspace_bytes(cfg: LayerConfig, T: int) -> int:
    c = cfg._c()
    out = ctypes.c_size_t(0)
    _check(LIB.pace_prefill_workspace_bytes(ctypes.byref(c), T, ctypes.byref(out)), "pace_prefill_workspace_bytes")
    return int(out.value)


def prefill_chunk(cfg: LayerConfig, state, q, k, v, a, beta, o, workspace=None, stream=None):
    """pace_prefill_chunk.  q, k [B, T, Hk, dk]; v, o [B, T, Hv, dv]; a, beta [B, T, Hv]."""
    import torch
    T = a.shape[1]
    L = layout(cfg)
    io = _io(cfg)
    c = cfg._c()
    need = prefill_workspace_bytes(cfg, T)
    ws = _ptr(workspace, "workspace", torch.uint8, optional=need == 0)
    wsb = workspace.numel() if workspace is not None else 0
    st = LIB.pace_prefill_chunk(
        ctypes.byref(c), _ptr(state, "state", torch.uint8, L["state_bytes"]),
        _ptr(q, "q", io, cfg.B * T * cfg.Hk * cfg.dk), _ptr(k, "k", io, cfg.B * T * cfg.Hk * cfg.dk),
        _ptr(v, "v", io, cfg.B * T * cfg.Hv * cfg.dv), _ptr(a, "a", torch.float32, cfg.B * T * cfg.Hv),
        _ptr(beta, "beta", torch.float32, cfg.B * T * cfg.Hv), T,
        _ptr(o, "o", io, cfg.B * T * cfg.Hv * cfg.dv), ws, wsb, _stream(stream))
    _check(st, "pace_prefill_chunk")


def calibrate_heads(cfg: LayerConfig, k, v, a, beta, stream=None):
    """pace_calibrate_heads.  k [B, T, Hk, dk], v [B, T, Hv, dv] (io dtype), a, beta
    [B, T, Hv] fp32, all on the device.  Returns (e_h, a_h): fp64 device tensors [Hv]."""
    import torch
    T = a.shape[1]
    io = _io(cfg)
    c = cfg._c()
    e_h = torch.empty(cfg.Hv, dtype=torch.float64, device=a.device)
    a_h = torch.empty(cfg.Hv, dtype=torch.float64, device=a.device)
    st = LIB.pace_calibrate_heads(
        ctypes.byref(c), _ptr(k, "k", io, cfg.B * T * cfg.Hk * cfg.dk), _ptr(v, "v", io, cfg.B * T * cfg.Hv * cfg.dv),
        _ptr(a, "a", torch.float32, cfg.B * T * cfg.Hv), _ptr(beta, "beta", torch.float32, cfg.B * T * cfg.Hv), T,
        _ptr(e_h, "e_h", torch.float64, cfg.Hv), _ptr(a_h, "a_h", torch.float64, cfg.Hv), _stream(stream))
    _check(st, "pace_calibrate_heads")
    return e_h, a_h


def prepare_prefill_chunk(cfg: LayerConfig, state, q, k, v, a, beta, o, workspace=None, stream=None):
    """Pre-marshalled pace_prefill_chunk (see prepare_decode_step)."""
    import torch
    T = a.shape[1]
    L = layout(cfg)
    io = _io(cfg)
    c = cfg._c()
    need = prefill_workspace_bytes(cfg, T)
    ws = _ptr(workspace, "workspace", torch.uint8, optional=need == 0)
    wsb = workspace.numel() if workspace is not None else 0
    args = (ctypes.byref(c), _ptr(state, "state", torch.uint8, L["state_bytes"]),
            _ptr(q, "q", io, cfg.B * T * cfg.Hk * cfg.dk), _ptr(k, "k", io, cfg.B * T * cfg.Hk * cfg.dk),
            _ptr(v, "v", io, cfg.B * T * cfg.Hv * cfg.dv), _ptr(a, "a", torch.float32, cfg.B * T * cfg.Hv),
            _ptr(beta, "beta", torch.float32, cfg.B * T * cfg.Hv), T,
            _ptr(o, "o", io, cfg.B * T * cfg.Hv * cfg.dv), ws, wsb, _stream(stream))
    fn = LIB.pace_prefill_chunk

    def call():
        st = fn(*args)
        if st != PACE_OK:
            raise PaceError(st, "pace_prefill_chunk")
    call._keep = (c, args)
    return call


def bf16_decode_step(cfg: LayerConfig, state, q, k, v, a, beta, o, stream=None):
    """pace_bf16_decode_step; state bf16 [B, Hv, dv, dk]."""
    import torch
    io = _io(cfg)
    c = cfg._c()
    st = LIB.pace_bf16_decode_step(
        ctypes.byref(c), _ptr(state, "state", torch.bfloat16, cfg.B * cfg.Hv * cfg.dv * cfg.dk),
        _ptr(q, "q", io, cfg.B * cfg.Hk * cfg.dk), _ptr(k, "k", io, cfg.B * cfg.Hk * cfg.dk),
        _ptr(v, "v", io, cfg.B * cfg.Hv * cfg.dv), _ptr(a, "a", torch.float32, cfg.B * cfg.Hv),
        _ptr(beta, "beta", torch.float32, cfg.B * cfg.Hv), _ptr(o, "o", io, cfg.B * cfg.Hv * cfg.dv),
        _stream(stream))
    _check(st, "pace_bf16_decode_step")


def prepare_decode_step(cfg: LayerConfig, state, buffer, q, k, v, a, beta, o, active=None, stream=None,
                        order=None):
    """Validate and marshal the arguments of pace_decode_step (or, with `order`,
    pace_decode_step_ordered) once; returns a callable that issues the same call again
    with no Python-side checks (for graph capture and timing loops).  The tensors must
    stay alive while the callable is used."""
    fn, name, args, keep = _decode_args(cfg, state, buffer, q, k, v, a, beta, o, active, stream, order)

    def call():
        st = fn(*args)
        if st != PACE_OK:
            raise PaceError(st, name)
    call._keep = (keep, args)
    return call


def prepare_bf16_decode_step(cfg: LayerConfig, state, q, k, v, a, beta, o, stream=None):
    """Pre-marshalled pace_bf16_decode_step (see prepare_decode_step)."""
    import torch
    io = _io(cfg)
    c = cfg._c()
    args = (ctypes.byref(c), _ptr(state, "state", torch.bfloat16, cfg.B * cfg.Hv * cfg.dv * cfg.dk),
            _ptr(q, "q", io, cfg.B * cfg.Hk * cfg.dk), _ptr(k, "k", io, cfg.B * cfg.Hk * cfg.dk),
            _ptr(v, "v", io, cfg.B * cfg.Hv * cfg.dv), _ptr(a, "a", torch.float32, cfg.B * cfg.Hv),
            _ptr(beta, "beta", torch.float32, cfg.B * cfg.Hv), _ptr(o, "o", io, cfg.B * cfg.Hv * cfg.dv),
            _stream(stream))
    fn = LIB.pace_bf16_decode_step

    def call():
        st = fn(*args)
        if st != PACE_OK:
            raise PaceError(st, "pace_bf16_decode_step")
    call._keep = (c, args)
    return call

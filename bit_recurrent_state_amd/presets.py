"""Layer configurations named on the PACE pages (onedev.kr summary, "How it works" and
"How it differs"): PACE-4 = symmetric int4, 64-key groups, int8 decode buffer;
PACE-4/8 = asymmetric, 32-key groups with integer zero points, a quarter of the heads
at 8 bits, int8 or mixed (4-bit key / bf16 value) buffer; decode period 8, prefill
rounding period 256.  Also the decode buffer on a bf16 state ("Assumptions and limits":
the share of the decode gain that comes from the buffer alone).  Shapes are the Qwen3.5-like gated-delta layer (32 value heads
over 16 key heads, head dimension 128)."""
from ._lib import LayerConfig


def pace4(B: int = 64, Hv: int = 32, Hk: int = 16, d: int = 128, dP: int = 8) -> LayerConfig:
    return LayerConfig(B=B, Hv=Hv, Hk=Hk, dk=d, dv=d, group=64, asym=False, buf="int8",
                       bf16_io=True, dP=dP)


def pace48(head_bits, B: int = 64, Hv: int = 32, Hk: int = 16, d: int = 128, dP: int = 8,
           buf: str = "int8") -> LayerConfig:
    return LayerConfig(B=B, Hv=Hv, Hk=Hk, dk=d, dv=d, group=32, asym=True, buf=buf,
                       bf16_io=True, dP=dP, head_bits=list(head_bits))


def tiny_ref() -> LayerConfig:
    """One layer, 2 sequences, 4 heads, d = 64, fp32 I/O, sym int4 g = 32, int8 buffer."""
    return LayerConfig(B=2, Hv=4, Hk=4, dk=64, dv=64, group=32, asym=False, buf="int8",
                       bf16_io=False, dP=8)


def bf16_periodic(B: int = 64, Hv: int = 32, Hk: int = 16, d: int = 128, dP: int = 8) -> LayerConfig:
    """Periodic decode on a bf16 state: the int8 decode buffer and once-per-dP fold of
    PACE-4 with the state kept as bf16 values."""
    return LayerConfig(B=B, Hv=Hv, Hk=Hk, dk=d, dv=d, group=64, asym=False, buf="int8",
                       bf16_io=True, dP=dP, bf16_state=True)

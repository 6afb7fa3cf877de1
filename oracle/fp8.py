"""fp8 inputs for the oracle: decoding and per-tensor dequantisation.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle/``).

The aclnnBlockSparseAttentionGrad page names two 8-bit float types
(FLOAT8_E5M2, FLOAT8_E4M3FN) only to say that the Atlas A2/A3 training
products do not take them; it fixes neither their encoding nor a scaling rule.
The readings used here:

* the two types are the OCP 8-bit floating-point formats of those names:
  E4M3FN has 1 sign, 4 exponent (bias 7) and 3 mantissa bits, no infinities,
  and NaN only where exponent and mantissa bits are all ones; E5M2 has 1 sign,
  5 exponent (bias 15) and 2 mantissa bits, with IEEE infinities and NaNs;
  both have subnormals at exponent field 0;
* each fp8 input tensor comes with one dequantisation factor: the value an
  element stands for is its decoded code times that factor (per-tensor
  scaling), and the backward is the ordinary one on those values;
* softmaxLse stays fp32, of the dequantised attention.

The oracle decodes in fp64 from the bit fields, so every code maps to its
exact value.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

from . import ref

__all__ = ["E4M3", "E5M2", "decode", "decode_e4m3fn", "decode_e5m2", "dequantize",
           "backward_fp8", "forward_fp8"]

E4M3 = "e4m3fn"
E5M2 = "e5m2"


def _fields(codes: np.ndarray, exp_bits: int, man_bits: int):
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7 == 1, -1.0, 1.0)
    e = (c >> man_bits) & ((1 << exp_bits) - 1)
    m = c & ((1 << man_bits) - 1)
    return sign, e, m


def _value(sign, e, m, bias: int, man_bits: int) -> np.ndarray:
    """Normal: (1 + m / 2^man) * 2^(e - bias); subnormal (e = 0): (m / 2^man) * 2^(1 - bias)."""
    frac = m.astype(np.float64) / float(1 << man_bits)
    normal = (1.0 + frac) * np.exp2((e - bias).astype(np.float64))
    sub = frac * np.exp2(float(1 - bias))
    return sign * np.where(e == 0, sub, normal)


def decode_e4m3fn(codes) -> np.ndarray:
    """OCP E4M3FN codes -> float64 values (exponent field 15 with mantissa 7 is NaN; no infinities)."""
    sign, e, m = _fields(codes, 4, 3)
    v = _value(sign, e, m, 7, 3)
    return np.where((e == 15) & (m == 7), np.nan, v)


def decode_e5m2(codes) -> np.ndarray:
    """OCP E5M2 codes -> float64 values (exponent field 31: infinity if mantissa 0, else NaN)."""
    sign, e, m = _fields(codes, 5, 2)
    v = _value(sign, e, m, 15, 2)
    v = np.where((e == 31) & (m == 0), sign * np.inf, v)
    return np.where((e == 31) & (m != 0), np.nan, v)


def decode(codes, fmt: str) -> np.ndarray:
    if fmt == E4M3:
        return decode_e4m3fn(codes)
    if fmt == E5M2:
        return decode_e5m2(codes)
    raise ValueError(f"unknown fp8 format {fmt!r}")


def dequantize(codes, fmt: str, factor: float) -> np.ndarray:
    """The values an fp8 tensor stands for: decoded code times its dequantisation factor."""
    return decode(codes, fmt) * float(factor)


_BWD_TENSORS = ("dout", "query", "key", "value", "attention_out")


def backward_fp8(q, k, v, o, do, lse, mask, *, formats: Dict[str, str], descale: Optional[Sequence[float]] = None,
                 **kw):
    """The backward on fp8 inputs: dequantise dout, query, key, value, attentionOut
    (``descale`` in that order, default all 1; ``formats`` maps each name to
    E4M3 or E5M2) and take ``ref.backward`` of the values."""
    f = [1.0] * 5 if descale is None else [float(x) for x in descale]
    vals = {name: dequantize(codes, formats[name], f[i])
            for i, (name, codes) in enumerate(zip(_BWD_TENSORS, (do, q, k, v, o)))}
    return ref.backward(vals["query"], vals["key"], vals["value"], vals["attention_out"], vals["dout"], lse, mask,
                        **kw)


def forward_fp8(q, k, v, mask, *, formats: Dict[str, str], descale: Optional[Sequence[float]] = None, **kw):
    """The forward on fp8 query, key, value (``descale`` in that order, default all 1)."""
    f = [1.0] * 3 if descale is None else [float(x) for x in descale]
    qv = dequantize(q, formats["query"], f[0])
    kv = dequantize(k, formats["key"], f[1])
    vv = dequantize(v, formats["value"], f[2])
    return ref.forward(qv, kv, vv, mask, **kw)

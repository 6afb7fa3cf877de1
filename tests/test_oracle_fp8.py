"""Pins for the oracle's fp8 decoding and dequantisation (``oracle/fp8.py``),
against things other than its own bit-field code: values worked out by hand
from the OCP format definitions (tests/golden/fp8_values.json), torch's
float8 dtypes over all 256 codes, IEEE half precision (E5M2 is the top byte
of a binary16), monotonicity of the positive codes, and the per-tensor factors
entering the backward exactly where the definition puts them."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import oracle.fp8 as fp8
import synth

from test_oracle import _kw

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fp8_values.json")
ALL = np.arange(256, dtype=np.uint8)


@pytest.mark.parametrize("fmt", [fp8.E4M3, fp8.E5M2])
def test_hand_worked_values(fmt):
    table = json.load(open(GOLDEN))[fmt]
    codes = np.array([int(k, 16) for k in table], dtype=np.uint8)
    want = np.array([float(v) for v in table.values()])
    got = fp8.decode(codes, fmt)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))  # -0.0 stays negative


@pytest.mark.parametrize("fmt,tdt", [(fp8.E4M3, torch.float8_e4m3fn), (fp8.E5M2, torch.float8_e5m2)])
def test_all_codes_match_torch_float8(fmt, tdt):
    ref = torch.from_numpy(ALL.copy()).view(tdt).to(torch.float64).numpy()
    got = fp8.decode(ALL, fmt)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_e5m2_is_the_top_byte_of_binary16():
    half = (ALL.astype(np.uint16) << 8).view(np.float16).astype(np.float64)
    got = fp8.decode(ALL, fp8.E5M2)
    nan = np.isnan(half)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], half[~nan])


@pytest.mark.parametrize("fmt,last", [(fp8.E4M3, 0x7E), (fp8.E5M2, 0x7C)])
def test_positive_codes_increase(fmt, last):
    v = fp8.decode(np.arange(last + 1, dtype=np.uint8), fmt)
    assert np.all(np.diff(v) > 0)
    # negative codes mirror the positive ones
    assert np.array_equal(fp8.decode(np.arange(last + 1, dtype=np.uint8) | 0x80, fmt)[1:], -v[1:])


def _fp8_case(seed=141):
    c = synth.make_case(layout="BNSD", dtype="bf16", B=1, N=2, Nkv=1, D=4, Sq=9, Skv=11, bx=4, by=4,
                        p=0.7, mask_rule="bernoulli_diag", scale=0.6, seed=seed)
    rng = np.random.default_rng(seed)
    codes = {n: rng.integers(0, 0x70, size=x.shape, dtype=np.uint8) | (rng.integers(0, 2, size=x.shape,
                                                                                    dtype=np.uint8) << 7)
             for n, x in (("dout", c.do), ("query", c.q), ("key", c.k), ("value", c.v), ("attention_out", c.q))}
    return c, codes


def test_backward_uses_each_factor_on_its_tensor():
    """Per-tensor factors enter as value = code * factor: scaling the codes' values by hand
    and running the plain oracle gives the same gradients, and the factors scale the
    outputs the way the definition says (dV linear in dO's factor; S unchanged when
    query's factor is doubled and key's halved)."""
    c, codes = _fp8_case()
    fmts = {"dout": fp8.E5M2, "query": fp8.E4M3, "key": fp8.E4M3, "value": fp8.E4M3, "attention_out": fp8.E4M3}
    f = [0.5, 0.25, 2.0, 0.125, 0.75]
    kw = _kw(c)
    # O/LSE: any fixed arrays work for this identity; take the forward of the dequantised values
    dec = {n: fp8.decode(codes[n], fmts[n]) for n in codes}
    o_val = dec["attention_out"] * f[4]
    _, lse = oracle.forward(dec["query"] * f[1], dec["key"] * f[2], dec["value"] * f[3], c.mask, **kw)
    got = fp8.backward_fp8(codes["query"], codes["key"], codes["value"], codes["attention_out"], codes["dout"],
                           lse, c.mask, formats=fmts, descale=f, **kw)
    want = oracle.backward(dec["query"] * f[1], dec["key"] * f[2], dec["value"] * f[3], o_val,
                           dec["dout"] * f[0], lse, c.mask, **kw)
    for g, w in zip(got, want):
        assert np.array_equal(g, w)
    # dV is linear in dout's factor
    f2 = list(f)
    f2[0] *= 3.0
    got2 = fp8.backward_fp8(codes["query"], codes["key"], codes["value"], codes["attention_out"], codes["dout"],
                            lse, c.mask, formats=fmts, descale=f2, **kw)
    assert np.allclose(got2[2], 3.0 * got[2], rtol=1e-12, atol=0)
    # query x2, key /2: same scores, so dQ halves... and dK doubles (dQ = scale dS K, dK = scale dS^T Q)
    f3 = list(f)
    f3[1] *= 2.0
    f3[2] /= 2.0
    got3 = fp8.backward_fp8(codes["query"], codes["key"], codes["value"], codes["attention_out"], codes["dout"],
                            lse, c.mask, formats=fmts, descale=f3, **kw)
    assert np.allclose(got3[0], 0.5 * got[0], rtol=1e-12, atol=1e-300)
    assert np.allclose(got3[1], 2.0 * got[1], rtol=1e-12, atol=1e-300)
    assert np.allclose(got3[2], got[2], rtol=1e-12, atol=1e-300)


def test_forward_fp8_is_the_forward_of_the_values():
    c, codes = _fp8_case(142)
    fmts = {"query": fp8.E4M3, "key": fp8.E5M2, "value": fp8.E4M3}
    f = [0.5, 0.25, 4.0]
    kw = _kw(c)
    o, lse = fp8.forward_fp8(codes["query"], codes["key"], codes["value"], c.mask, formats=fmts, descale=f, **kw)
    # value's factor scales O and leaves LSE alone; query's and key's only enter through their product
    o2, lse2 = fp8.forward_fp8(codes["query"], codes["key"], codes["value"], c.mask, formats=fmts,
                               descale=[1.0, 0.125, 8.0], **kw)
    assert np.allclose(o2, 2.0 * o, rtol=1e-12, atol=1e-300)
    assert np.allclose(lse2[np.isfinite(lse)], lse[np.isfinite(lse)], rtol=1e-12)
    # torch fp64 on the decoded values, dense mask rows, as an independent forward
    q = torch.from_numpy(fp8.decode(codes["query"], fp8.E4M3) * 0.5)
    k = torch.from_numpy(fp8.decode(codes["key"], fp8.E5M2) * 0.25)
    v = torch.from_numpy(fp8.decode(codes["value"], fp8.E4M3) * 4.0)
    em = np.stack([oracle.element_mask(c.mask[0, n], c.bx, c.by, c.Sq, c.Skv) for n in range(c.N)])
    s = c.scale * (q[0] @ k[0, 0].T)
    s = s.masked_fill(~torch.from_numpy(em), float("-inf"))
    ref_lse = torch.logsumexp(s, dim=-1)
    ok = torch.isfinite(ref_lse)
    p = torch.exp(s - ref_lse[..., None])
    ref_o = torch.where(ok[..., None], p.nan_to_num(0.0) @ v[0, 0], torch.zeros(()))
    assert np.allclose(lse[0][ok.numpy()], ref_lse[ok].numpy(), rtol=1e-12)
    assert np.allclose(o[0], ref_o.numpy(), rtol=1e-10, atol=1e-12)

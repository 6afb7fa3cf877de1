"""Host-side checks of the fp8 entry points and of the input alignment rule
(no GPU needed): accepted and rejected dtypes, factors, the staging region."""
import pytest
import torch

import block_sparse_attention_bwd_amd as bsa

from test_api import INVALID, _bnsd, _code, _fwd, _tnd

E4, E5 = torch.float8_e4m3fn, torch.float8_e5m2


def _fp8(base=_bnsd, dout=E5, rest=E4, **kw):
    """A base case with fp8 inputs (dout in `dout`, the others in `rest`) and bf16 outputs."""
    a = base(**kw)
    for k in ("query", "key", "value", "attention_out"):
        a[k] = torch.zeros(a[k].shape, dtype=rest)
    a["dout"] = torch.zeros(a["dout"].shape, dtype=dout)
    for k in ("dq", "dk", "dv"):
        a[k] = torch.zeros(a[k].shape, dtype=torch.bfloat16)
    return a


def _code8(args, descale=None):
    try:
        bsa.bsa_bwd_fp8_workspace_size(**args, descale=descale)
    except bsa.BsaError as e:
        return e.code
    return bsa.BSA_OK


def test_fp8_inputs_accepted_by_fp8_entry_only():
    assert _code8(_fp8()) == bsa.BSA_OK
    assert _code8(_fp8(_tnd, dout=E4, rest=E5)) == bsa.BSA_OK
    assert _code8(_fp8(), descale=[0.5, 2.0, 1e-3, 3.0, 0.25]) == bsa.BSA_OK
    assert _code(_fp8()) == INVALID           # the fp16/bf16 entry point refuses fp8
    assert _code8(_bnsd()) == INVALID          # and the fp8 one refuses bf16 inputs


@pytest.mark.parametrize("field", ["dq", "dk", "dv"])
def test_fp8_outputs_must_be_bf16(field):
    a = _fp8()
    a[field] = torch.zeros(a[field].shape, dtype=torch.float16)
    assert _code8(a) == INVALID
    a[field] = torch.zeros(a[field].shape, dtype=E4)
    assert _code8(a) == INVALID


@pytest.mark.parametrize("bad", [[0.0, 1, 1, 1, 1], [1, -1.0, 1, 1, 1], [1, 1, float("nan"), 1, 1],
                                 [1, 1, 1, float("inf"), 1]])
def test_fp8_factors_must_be_finite_positive(bad):
    assert _code8(_fp8(), descale=bad) == INVALID


def test_fp8_factor_products_must_stay_normal():
    # scale * f_query * f_key underflows fp32
    assert _code8(_fp8(), descale=[1, 1e-25, 1e-25, 1, 1]) == INVALID


def test_fp8_staging_region():
    """The fp8 workspace is the bf16 one plus a 256-byte aligned bf16 copy of each input."""
    al = lambda x: -(-x // 256) * 256
    a = _fp8()
    base = bsa.bsa_bwd_workspace_size(**_bnsd())
    got = bsa.bsa_bwd_fp8_workspace_size(**a)
    staged = sum(al(2 * a[k].numel()) for k in ("dout", "query", "key", "value", "attention_out"))
    assert got == base + staged
    offs, _ = bsa.bsa_bwd_workspace_layout(**_bnsd())
    assert offs["stage"] == offs["total"]  # empty without fp8 inputs


def test_fp8_forward_phase1():
    a = _fwd(_fp8)
    a["attention_out"] = torch.zeros(a["query"].shape, dtype=torch.bfloat16)
    assert bsa.bsa_fwd_fp8_workspace_size(**a, descale=[1.0, 2.0, 0.5]) > bsa.bsa_fwd_workspace_size(
        **_fwd(_bnsd))
    a["attention_out"] = torch.zeros(a["query"].shape, dtype=E4)
    with pytest.raises(bsa.BsaError) as e:
        bsa.bsa_fwd_fp8_workspace_size(**a)
    assert e.value.code == INVALID
    with pytest.raises(ValueError):
        bsa.bsa_fwd_fp8_workspace_size(**a, descale=[1.0, 2.0])  # three factors


@pytest.mark.parametrize("field", ["dout", "query", "key", "value", "attention_out"])
def test_inputs_must_be_16_byte_aligned(field):
    a = _bnsd()
    t = a[field]
    flat = torch.zeros(t.numel() + 8, dtype=t.dtype)
    a[field] = flat[1:1 + t.numel()].view(t.shape)  # contiguous, 2 bytes off
    assert _code(a) == INVALID
    b = _fp8()
    t = b[field]
    flat = torch.zeros(t.numel() + 16, dtype=torch.uint8)
    b[field] = flat[4:4 + t.numel()].view(t.dtype).view(t.shape)
    assert _code8(b) == INVALID

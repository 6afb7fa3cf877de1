"""GPU parity of the fp8 entry points (bsa_bwd_fp8, bsa_fwd_fp8) through the
C ABI against the fp64 oracle on the dequantised values (oracle/fp8.py).

Bar: per tensor max|gpu - ref| <= 2e-2 * max|ref| (the bf16 bound).  The
decode to bf16 is exact, so the kernels see exactly the codes' values and run
the bf16 arithmetic the bf16 bound was set for; the factors enter as fp32
multiplications (relative error 2^-24 each).  The decode itself is compared
exactly, over all 256 codes of each format.
"""
import numpy as np
import pytest

import oracle
import oracle.fp8 as fp8
import synth
from cases import case as _case
from gpu_common import assert_close, oracle_kw, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TDT = {fp8.E4M3: torch.float8_e4m3fn, fp8.E5M2: torch.float8_e5m2}
ORDER = ("dout", "query", "key", "value", "attention_out")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_bwd_amd as bsa
    bsa.load_library()
    yield


def _fp8_inputs(c, fmts):
    """Quantised Q, K, V, dO (per-tensor factors); O and LSE from the oracle forward
    of the dequantised values, O then quantised too."""
    qz = {n: synth.quantize_fp8(x, fmts[n]) for n, x in (("query", c.q), ("key", c.k), ("value", c.v),
                                                        ("dout", c.do))}
    deq = {n: fp8.dequantize(codes, fmts[n], f) for n, (codes, f) in qz.items()}
    o, lse = oracle.forward(deq["query"], deq["key"], deq["value"], c.mask, **oracle_kw(c))
    qz["attention_out"] = synth.quantize_fp8(o, fmts["attention_out"])
    return qz, lse.astype(np.float32)


def _dev(codes, fmt):
    return torch.from_numpy(np.ascontiguousarray(codes)).cuda().view(TDT[fmt])


def _runner(c, qz, lse, fmts):
    from bench import Runner, to_device
    dev = to_device(c)
    for key, name in (("q", "query"), ("k", "key"), ("v", "value"), ("do", "dout")):
        dev[key] = _dev(qz[name][0], fmts[name])
    o = _dev(qz["attention_out"][0], fmts["attention_out"])
    lse_d = torch.from_numpy(np.ascontiguousarray(lse)).cuda()
    return Runner(c, dev, o, lse_d, descale=[qz[n][1] for n in ORDER])


BWD_CASES = [
    ("bnsd_bf16_d128_b128x128_ragged", fp8.E5M2, fp8.E4M3),
    ("tnd_fp16_d128_b64x128_gqa", fp8.E5M2, fp8.E5M2),
    ("bnsd_bf16_d128_window", fp8.E4M3, fp8.E4M3),
    ("bnsd_bf16_d128_local_sink_split", fp8.E5M2, fp8.E4M3),
    ("bnsd_fp16_d64_b64x128_padded", fp8.E4M3, fp8.E5M2),
    ("bnsd_bf16_d256_b128x128_ragged", fp8.E5M2, fp8.E4M3),
]


@pytest.mark.parametrize("name,f_do,f_rest", BWD_CASES, ids=[b[0] for b in BWD_CASES])
def test_fp8_backward_parity(name, f_do, f_rest):
    c = _case(name)
    fmts = {n: f_rest for n in ORDER}
    fmts["dout"] = f_do
    qz, lse = _fp8_inputs(c, fmts)
    r = _runner(c, qz, lse, fmts)
    dq, dk, dv = r()
    torch.cuda.synchronize()
    assert dq.dtype == torch.bfloat16
    ref = fp8.backward_fp8(*(qz[n][0] for n in ("query", "key", "value", "attention_out", "dout")), lse,
                           c.mask, formats=fmts, descale=[qz[n][1] for n in ORDER], **oracle_kw(c))
    floor = float(np.abs(ref[2]).max())
    for nm, got, want in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        assert_close(f"{name}/{nm}", to_np(got), want, "bf16", floor_ref=floor)


def test_fp8_backward_deterministic():
    c = _case("bnsd_bf16_d128_local_sink_split")
    fmts = {n: fp8.E4M3 for n in ORDER}
    qz, lse = _fp8_inputs(c, fmts)
    r = _runner(c, qz, lse, fmts)
    first = [t.clone() for t in r()]
    for _ in range(2):
        r()
    torch.cuda.synchronize()
    for a, b in zip(first, (r.dq, r.dk, r.dv)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_fp8_decode_is_exact_for_every_code():
    """dout holds every E5M2 code and query every E4M3FN code, cyclically; the bf16
    copies in the workspace's staging region equal the decoded values exactly."""
    c = _case("bnsd_bf16_d128_b128x128_ragged")
    fmts = {n: fp8.E4M3 for n in ORDER}
    fmts["dout"] = fp8.E5M2
    qz, lse = _fp8_inputs(c, fmts)
    all_codes = np.arange(256, dtype=np.uint8)
    qz["dout"] = (np.resize(all_codes, qz["dout"][0].shape), 1.0)
    qz["query"] = (np.resize(all_codes[::-1].copy(), qz["query"][0].shape), 1.0)
    r = _runner(c, qz, lse, fmts)
    r()
    torch.cuda.synchronize()
    # the staging region is the workspace's last: dout's copy, then query's, ... (each 256-byte aligned)
    al = lambda x: -(-x // 256) * 256
    sizes = [al(2 * qz[n][0].size) for n in ORDER]
    start = r.ws_size - sum(sizes)
    ws = r.ws.cpu()
    n_do, n_q = qz["dout"][0].size, qz["query"][0].size
    got_do = ws[start:start + 2 * n_do].view(torch.bfloat16).double().numpy()
    q0 = start + sizes[0]
    got_q = ws[q0:q0 + 2 * n_q].view(torch.bfloat16).double().numpy()
    for got, codes, fmt in ((got_do, qz["dout"][0], fp8.E5M2), (got_q, qz["query"][0], fp8.E4M3)):
        want = fp8.decode(codes.reshape(-1), fmt)
        nan = np.isnan(want)
        assert np.array_equal(np.isnan(got), nan), fmt
        assert np.array_equal(got[~nan], want[~nan]), fmt
        assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan])), fmt


FWD_CASES = [("bnsd_bf16_d128_b128x128_ragged", fp8.E4M3), ("tnd_fp16_d128_b64x128_gqa", fp8.E5M2),
             ("bnsd_bf16_d128_window", fp8.E4M3)]


@pytest.mark.parametrize("name,fmt", FWD_CASES, ids=[f[0] for f in FWD_CASES])
def test_fp8_forward_parity(name, fmt):
    from bench import FwdRunner, to_device
    c = _case(name)
    fmts = {n: fmt for n in ("query", "key", "value")}
    qz = {n: synth.quantize_fp8(x, fmt) for n, x in (("query", c.q), ("key", c.k), ("value", c.v))}
    dev = to_device(c)
    for key, n in (("q", "query"), ("k", "key"), ("v", "value")):
        dev[key] = _dev(qz[n][0], fmt)
    r = FwdRunner(c, dev, descale=[qz[n][1] for n in ("query", "key", "value")])
    o, lse = r()
    torch.cuda.synchronize()
    assert o.dtype == torch.bfloat16
    ref_o, ref_l = fp8.forward_fp8(qz["query"][0], qz["key"][0], qz["value"][0], c.mask, formats=fmts,
                                   descale=[qz[n][1] for n in ("query", "key", "value")], **oracle_kw(c))
    assert_close(f"{name}/O", to_np(o), ref_o, "bf16")
    got_l = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(ref_l)
    assert np.array_equal(np.isneginf(got_l), ~fin)
    assert np.all(np.abs(got_l[fin] - ref_l[fin]) <= 1e-3 * np.maximum(1.0, np.abs(ref_l[fin])))

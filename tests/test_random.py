"""Seeded random GPU parity cases: layout, dtype, head dim, heads and GQA
ratio, batch, ragged (sometimes empty) lengths, block shapes from 1 to 256,
mask density with and without the diagonal, a sliding window and an
attenMask, each drawn independently; backward and forward through the C ABI
against the fp64 oracle, with the bars of the other parity tests."""
import numpy as np
import pytest

import oracle
import synth
from gpu_common import assert_close, oracle_fwd_inputs, oracle_kw, to_np, upload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

N_CASES = 64
HEADS = [(1, 1), (2, 1), (4, 2), (4, 4), (6, 3), (8, 1)]
BLOCKS = [1, 16, 32, 48, 64, 80, 128, 200, 256]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_bwd_amd as bsa
    bsa.load_library()
    yield


def draw(seed):
    """One random case (pure function of the seed)."""
    rng = np.random.default_rng(7000 + seed)
    layout = ["BNSD", "TND"][int(rng.integers(2))]
    dtype = ["fp16", "bf16"][int(rng.integers(2))]
    D = [64, 128, 256][int(rng.integers(3))]
    N, Nkv = HEADS[int(rng.integers(len(HEADS)))]
    B = int(rng.integers(1, 4))
    bx, by = (BLOCKS[int(rng.integers(len(BLOCKS)))] for _ in range(2))
    cap = 120 if min(bx, by) == 1 else 300  # element masks stay small
    lq = [int(x) for x in rng.integers(0, cap + 1, size=B)]
    lk = [int(x) for x in rng.integers(0, cap + 1, size=B)]
    lq[0], lk[0] = max(lq[0], 1), max(lk[0], 1)  # at least one query and key somewhere
    kw = dict(layout=layout, dtype=dtype, B=B, N=N, Nkv=Nkv, D=D, bx=bx, by=by,
              mask_rule=["bernoulli", "bernoulli_diag"][int(rng.integers(2))], p=float(rng.uniform(0.1, 0.9)),
              seed=8000 + seed, name=f"random{seed}")
    if layout == "TND":
        kw.update(lengths_q=lq, lengths_kv=lk)
    else:
        Sq, Skv = max(lq), max(lk)
        kw.update(Sq=Sq, Skv=Skv)
        if rng.random() < 0.5:  # padded tails
            kw.update(lengths_q=lq, lengths_kv=lk)
    if rng.random() < 0.3:
        kw["window"] = (int(rng.integers(-20, 200)), int(rng.integers(-20, 200)))
    c = synth.make_case(**kw)
    if rng.random() < 0.25:
        sq, sk = (c.Sq, c.Skv) if c.layout == "BNSD" else (int(c.len_q.max()), int(c.len_kv.max()))
        c.atten_mask = (rng.random((sq, sk)) < rng.uniform(0.05, 0.5)).astype(np.uint8)
    return c


def _describe(c):
    return (f"{c.name}: {c.layout} {c.dtype} B={c.B} N={c.N} Nkv={c.Nkv} D={c.D} block={c.bx}x{c.by} "
            f"len_q={list(map(int, c.len_q))} len_kv={list(map(int, c.len_kv))} window={c.window} "
            f"attenmask={c.atten_mask is not None}")


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_case_backward(seed):
    from bench import Runner
    c = draw(seed)
    print("[random bwd]", _describe(c), flush=True)
    o, lse = oracle_fwd_inputs(c)
    dev = upload(c, o, lse)
    dq, dk, dv = Runner(c, dev, dev["o"], dev["lse"])()
    torch.cuda.synchronize()
    ref = oracle.backward(c.q, c.k, c.v, o.astype(np.float64), c.do, lse, c.mask, **oracle_kw(c))
    floor = float(np.abs(ref[2]).max()) if ref[2].size else 1.0
    for nm, got, want in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        assert_close(f"random{seed}/{nm}", to_np(got), want, c.dtype, floor_ref=floor)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_case_forward(seed):
    from bench import FwdRunner, to_device
    c = draw(seed)
    print("[random fwd]", _describe(c), flush=True)
    o, lse = FwdRunner(c, to_device(c))()
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.forward(c.q, c.k, c.v, c.mask, **oracle_kw(c))
    assert_close(f"random{seed}/O", to_np(o), ref_o, c.dtype)
    got_l = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(ref_l)
    assert np.array_equal(np.isneginf(got_l), ~fin), f"random{seed}/LSE: -inf pattern differs"
    assert np.all(np.abs(got_l[fin] - ref_l[fin]) <= 1e-3 * np.maximum(1.0, np.abs(ref_l[fin])))


@pytest.mark.parametrize("seed", range(16))
def test_random_case_fp8_backward(seed):
    """The same draws with fp8 inputs (each tensor E4M3FN or E5M2 at random, per-tensor factors)
    through bsa_bwd_fp8, against the oracle on the dequantised values (the bf16 bar)."""
    import oracle.fp8 as fp8
    from bench import Runner, to_device
    c = draw(seed)
    rng = np.random.default_rng(9000 + seed)
    fmts = {n: [fp8.E4M3, fp8.E5M2][int(rng.integers(2))] for n in ("dout", "query", "key", "value", "attention_out")}
    print("[random fp8 bwd]", _describe(c), fmts, flush=True)
    qz = {n: synth.quantize_fp8(x, fmts[n]) for n, x in (("query", c.q), ("key", c.k), ("value", c.v),
                                                        ("dout", c.do))}
    deq = {n: fp8.dequantize(codes, fmts[n], f) for n, (codes, f) in qz.items()}
    o, lse = oracle.forward(deq["query"], deq["key"], deq["value"], c.mask, **oracle_kw(c))
    qz["attention_out"] = synth.quantize_fp8(o, fmts["attention_out"])
    lse = lse.astype(np.float32)
    tdt = {fp8.E4M3: torch.float8_e4m3fn, fp8.E5M2: torch.float8_e5m2}
    dev = to_device(c)
    for key, n in (("q", "query"), ("k", "key"), ("v", "value"), ("do", "dout")):
        dev[key] = torch.from_numpy(np.ascontiguousarray(qz[n][0])).cuda().view(tdt[fmts[n]])
    o_dev = torch.from_numpy(np.ascontiguousarray(qz["attention_out"][0])).cuda().view(tdt[fmts["attention_out"]])
    order = ("dout", "query", "key", "value", "attention_out")
    r = Runner(c, dev, o_dev, torch.from_numpy(lse).cuda(), descale=[qz[n][1] for n in order])
    dq, dk, dv = r()
    torch.cuda.synchronize()
    ref = fp8.backward_fp8(*(qz[n][0] for n in ("query", "key", "value", "attention_out", "dout")), lse, c.mask,
                           formats=fmts, descale=[qz[n][1] for n in order], **oracle_kw(c))
    floor = float(np.abs(ref[2]).max()) if ref[2].size else 1.0
    for nm, got, want in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        assert_close(f"random{seed}/fp8/{nm}", to_np(got), want, "bf16", floor_ref=floor)

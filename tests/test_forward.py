"""GPU parity of the forward (O, LSE) through the C ABI against the fp64 oracle forward.

Bars: O per tensor within max|gpu - ref| <= tol * max|ref| (tol 5e-3 fp16,
2e-2 bf16, as for the gradients); LSE (fp32 output) within
1e-3 * max(1, |ref|) where the oracle's is finite, and -inf exactly where the
oracle's is -inf (rows that select nothing, BNSD padding).  The LSE bound: the
scores are fp32 sums of exact fp16/bf16 products (relative error about
D * 2^-24 of |S|, below 1e-4 for |S| < 10^1.5), and the fp32 running sum and
the exp2/log2 instructions add a few ulp, so 1e-3 leaves an order of
magnitude of margin while still catching a wrong scale, base or mask.
"""
import numpy as np
import pytest

import oracle
import synth
from cases import SMALL, case as _case
from gpu_common import TOL, assert_close, oracle_kw, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

LSE_TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_bwd_amd as bsa
    bsa.load_library()
    yield


def _run_fwd(c, out=None):
    import block_sparse_attention_bwd_amd as bsa
    from bench import to_device
    dev = to_device(c)
    lengths = c.explicit_lengths or c.layout == "TND"
    o = torch.empty_like(dev["q"]) if out is None else out(dev["q"])
    lse = torch.empty(dev["q"].shape[:-1], dtype=torch.float32, device="cuda")
    kw = dict(block_sparse_mask=dev["mask"], atten_mask=dev.get("amask"), block_shape=[c.bx, c.by],
              actual_seq_lengths=list(map(int, c.len_q)) if lengths else None,
              actual_seq_lengths_kv=list(map(int, c.len_kv)) if lengths else None,
              q_input_layout=c.layout, kv_input_layout=c.layout, num_key_value_heads=c.Nkv,
              mask_type=0, scale_value=c.scale,
              pre_tokens=bsa.NO_WINDOW if c.window is None else c.window[0],
              next_tokens=bsa.NO_WINDOW if c.window is None else c.window[1],
              attention_out=o, softmax_lse=lse)
    ws = bsa.bsa_fwd_workspace_size(dev["q"], dev["k"], dev["v"], **kw)
    wbuf = torch.empty(max(ws, 1), dtype=torch.uint8, device="cuda")
    bsa.bsa_fwd(dev["q"], dev["k"], dev["v"], **kw, workspace=wbuf, workspace_size=ws)
    torch.cuda.synchronize()
    return o, lse


def _check(name, c, o, lse):
    ref_o, ref_l = oracle.forward(c.q, c.k, c.v, c.mask, **oracle_kw(c))
    assert_close(f"{name}/O", to_np(o), ref_o, c.dtype)
    got_l = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(ref_l)
    assert np.array_equal(np.isneginf(got_l), ~fin), f"{name}/LSE: -inf pattern differs"
    if fin.any():
        err = np.abs(got_l[fin] - ref_l[fin])
        bound = LSE_TOL * np.maximum(1.0, np.abs(ref_l[fin]))
        worst = int(np.argmax(err - bound))
        assert np.all(err <= bound), f"{name}/LSE: err {err[worst]:.3e} > {bound[worst]:.3e}"


@pytest.mark.parametrize("name", SMALL)
def test_forward_small_case_parity(name):
    print(f"[forward] {name}", flush=True)
    c = _case(name)
    o, lse = _run_fwd(c)
    _check(name, c, o, lse)


@pytest.mark.parametrize("k", [2, 3, 4, 5])
def test_forward_full_config_parity(k):
    """The whole output of the full workloads (the oracle forward takes seconds)."""
    print(f"[forward] config {k}", flush=True)
    c = synth.config(k)
    o, lse = _run_fwd(c)
    _check(f"config{k}", c, o, lse)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_forward_rising_scores_rescale(dtype):
    """Scores that climb along the keys (head 0: S_ij = q_i . k_j grows by about 6 log2 units
    per 32-key slice, 50 in all) make each row's maximum pass the kernel's running reference
    many times in the middle of the walk, so the output is rescaled there; in head 1 the
    scores fall instead (the maximum is the first key's and never moves).  Random inputs
    almost never exercise the first path after the first slice."""
    print(f"[forward] rising scores {dtype}", flush=True)
    c = synth.make_case(layout="BNSD", dtype=dtype, B=1, N=2, Nkv=1, D=64, Sq=160, Skv=300,
                        bx=64, by=64, mask_rule="dense", seed=131)
    rng = np.random.default_rng(131)
    sign = np.array([1.0, -1.0], np.float32)[None, :, None, None]
    q = sign * (0.25 + 0.05 * rng.standard_normal(c.q.shape).astype(np.float32))
    k = np.broadcast_to((np.arange(c.k.shape[2], dtype=np.float32) / 16.0)[None, None, :, None], c.k.shape)
    c.q = synth.round_to_dtype(np.ascontiguousarray(q, np.float32), dtype)
    c.k = synth.round_to_dtype(np.ascontiguousarray(k, np.float32), dtype)
    o, lse = _run_fwd(c)
    _check(f"rising_{dtype}", c, o, lse)
    ref_l = oracle.forward(c.q, c.k, c.v, c.mask, **oracle_kw(c))[1]
    assert ref_l[0, 0].min() > 25.0 and ref_l[0, 1].max() < 10.0  # the two regimes are the intended ones


def test_forward_noncontiguous_output():
    c = _case("bnsd_bf16_d128_b128x128_ragged")
    o_ref, l_ref = _run_fwd(c)
    o2, l2 = _run_fwd(c, out=lambda q: torch.zeros(q.shape[0], q.shape[2], q.shape[1], q.shape[3],
                                                    dtype=q.dtype, device=q.device).transpose(1, 2))
    assert torch.equal(o_ref, o2) and torch.equal(l_ref, l2)


@pytest.mark.parametrize("name", ["bnsd_fp16_d64_b64x128_padded", "tnd_fp16_d128_b64x128_gqa",
                                  "bnsd_bf16_d256_window_attenmask"])
def test_forward_guard_bytes(name):
    """Nothing is written outside attention_out, softmax_lse and the workspace."""
    import block_sparse_attention_bwd_amd as bsa
    from bench import FwdRunner, to_device
    from gpu_common import _guarded, _guards_intact
    c = _case(name)
    r = FwdRunner(c, to_device(c))
    o_want, l_want = (t.clone() for t in r())
    torch.cuda.synchronize()
    go, gl = _guarded(r.o.shape, r.o.dtype), _guarded(r.lse.shape, r.lse.dtype)
    ws = _guarded((r.ws_size,), torch.uint8)
    kw = dict(r.kw, attention_out=go[0], softmax_lse=gl[0])
    bsa.bsa_fwd(*r.args, **kw, workspace=ws[0], workspace_size=r.ws_size)
    torch.cuda.synchronize()
    for (t, buf, pat), w in ((go, o_want), (gl, l_want)):
        assert _guards_intact(buf, pat)
        assert torch.equal(t, w)
    assert _guards_intact(ws[1], ws[2])


def test_forward_bitwise_deterministic():
    c = _case("tnd_fp16_d128_b64x128_gqa")
    a = _run_fwd(c)
    b = _run_fwd(c)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_forward_page_sample():
    """The page's sample program (constant fp16 Q = K = V = 0.1, every block
    selected): every score equals scale * D * q^2, so each row's softmax is
    uniform over its keys, O equals V's constant exactly, and
    LSE = scale * D * q^2 + ln(Skv) (= 4.96511..., not the 5.0 the sample feeds
    the backward)."""
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_sample.json")))
    B, N, S, D = g["batch"], g["numHeads"], g["qSeqlen"], g["headDim"]
    bx, by = g["blockShape"]
    q16 = float(np.float16(g["query"]))
    dev = lambda x: torch.full((B, N, S, D), x, dtype=torch.float16, device="cuda")
    q, k, v = dev(g["query"]), dev(g["key"]), dev(g["value"])
    mask = torch.ones(g["maskShape"], dtype=torch.bool, device="cuda")
    import block_sparse_attention_bwd_amd as bsa
    o, lse = bsa.block_sparse_attention(q, k, v, mask, block_shape=[bx, by], layout="BNSD",
                                        num_key_value_heads=g["numKvHeads"], scale_value=D ** -0.5)
    torch.cuda.synchronize()
    assert torch.all(o == torch.tensor(q16, dtype=torch.float16, device="cuda"))
    want = D ** -0.5 * D * q16 * q16 + np.log(g["kvSeqlen"])
    assert abs(want - 4.96511) < 1e-5
    assert float((lse.double() - want).abs().max()) < 1e-5

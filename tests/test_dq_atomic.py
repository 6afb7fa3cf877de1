"""GPU parity of the opt-in dQ mode of bsa_bwd_ex, BSA_DQ_ATOMIC (the dK/dV
kernel adds dS K into an fp32 accumulator with atomic adds), against the fp64
oracle: dQ within the per-tensor bound of the default mode (5e-3 fp16, 2e-2
bf16 of max|ref|), and dK, dV bitwise those of the default mode, whose dK/dV
arithmetic is the same.  The mode's argument rules are checked on the CPU in
test_api.py."""
import numpy as np
import pytest

import oracle
import synth
from gpu_common import assert_close, oracle_backward_threaded, oracle_fwd_inputs, oracle_kw, to_np, upload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from cases import ATTEN, SMALL, case as _case  # noqa: E402

# the mode takes head dims 64 and 128 without an attenMask
ELIGIBLE = [n for n in SMALL if "_d256_" not in n and n not in ATTEN]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_bwd_amd as bsa
    bsa.load_library()
    yield


def _both_modes(c, dev, o, lse):
    from bench import Runner
    plain = [t.clone() for t in Runner(c, dev, o, lse)()]
    atomic = Runner(c, dev, o, lse, dq_mode=1)()
    torch.cuda.synchronize()
    return plain, atomic


@pytest.mark.parametrize("name", ELIGIBLE)
def test_atomic_dq_small_cases(name):
    c = _case(name)
    print(f"[dq-atomic] {name}", flush=True)
    o, lse = oracle_fwd_inputs(c)
    ref = oracle.backward(c.q, c.k, c.v, o, c.do, lse, c.mask, **oracle_kw(c))
    dev = upload(c, o, lse)
    (dq0, dk0, dv0), (dq, dk, dv) = _both_modes(c, dev, dev["o"], dev["lse"])
    floor = float(np.abs(ref[2]).max())
    for nm, got, want in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
        assert_close(f"{name}/{nm}", to_np(got), want, c.dtype, floor_ref=floor)
    assert torch.equal(dk, dk0) and torch.equal(dv, dv0), f"{name}: dK/dV differ from the default mode"


@pytest.mark.parametrize("k", [2, 4])
def test_atomic_dq_full_workload_whole_tensors(k):
    """Workloads 2 (BNSD bf16, 128x128 blocks) and 4 (ragged TND fp16, 64x128
    blocks, GQA 32:4) at full size: dQ against the oracle element by element."""
    from bench import gpu_forward, to_device
    c = synth.config(k)
    print(f"[dq-atomic] config {k}: {c.name}", flush=True)
    dev = to_device(c)
    o, lse = gpu_forward(c, dev)
    torch.cuda.synchronize()
    (dq0, dk0, dv0), (dq, dk, dv) = _both_modes(c, dev, o, lse)
    assert torch.equal(dk, dk0) and torch.equal(dv, dv0), f"config{k}: dK/dV differ from the default mode"
    o_h, lse_h = o.float().cpu().numpy(), lse.cpu().numpy()
    ref = oracle_backward_threaded(c, c.q, c.k, c.v, o_h, c.do, lse_h)
    err, ref_max = assert_close(f"config{k}/dq", to_np(dq), ref[0], c.dtype)
    print(f"[dq-atomic] config {k}: dq err / max|ref| = {err / ref_max:.2e}", flush=True)


@pytest.mark.parametrize("k", [3, 5])
def test_atomic_dq_full_workload_sampled_rows(k):
    """Workloads 3 (sink columns: split dK/dV units) and 5 (64-row KV blocks,
    two-wave dK/dV workgroups) at full size: 64 dQ rows of every kind against
    the oracle row by row, the rest against the default mode's dQ within the bar."""
    from bench import gpu_forward, to_device
    c = synth.config(k)
    print(f"[dq-atomic] config {k}: {c.name}", flush=True)
    dev = to_device(c)
    o, lse = gpu_forward(c, dev)
    torch.cuda.synchronize()
    (dq0, dk0, dv0), (dq, dk, dv) = _both_modes(c, dev, o, lse)
    assert torch.equal(dk, dk0) and torch.equal(dv, dv0), f"config{k}: dK/dV differ from the default mode"
    o_h, lse_h = o.float().cpu().numpy(), lse.cpu().numpy()
    rng = np.random.default_rng(7 + k)
    got = to_np(dq)
    rows = [(int(rng.integers(c.B)), int(rng.integers(c.N)), int(rng.integers(c.Sq))) for _ in range(64)]
    want = oracle.backward_dq_rows(c.q, c.k, c.v, o_h, c.do, lse_h, c.mask, rows=rows, **oracle_kw(c))
    g = np.stack([got[b, n, i] for b, n, i in rows])
    assert_close(f"config{k}/dq rows", g, np.stack([want[r] for r in rows]), c.dtype)
    # every element: within the bar of the default mode's dQ (itself checked whole in test_parity.py)
    assert_close(f"config{k}/dq vs default", got, to_np(dq0), c.dtype)

"""bsa_bwd_noalloc (the backward on the library's own scratch array, for callers
that cannot allocate) through the C ABI, against bsa_bwd with a caller
workspace on the same inputs: two calls in a row, the second on a smaller
problem, each bitwise equal to bsa_bwd (the same kernels and plan) and within
the oracle's per-tensor bound; a problem larger than the scratch array is
rejected before anything is enqueued."""
import numpy as np
import pytest

import oracle
from cases import case as _case
from gpu_common import assert_close, oracle_fwd_inputs, oracle_kw, run_bsa, to_np, upload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_bwd_amd as bsa
    bsa.load_library()
    yield


def _noalloc_vs_workspace(name):
    import block_sparse_attention_bwd_amd as bsa
    c = _case(name)
    o, lse = oracle_fwd_inputs(c)
    dev = upload(c, o, lse)
    (dq, dk, dv), r = run_bsa(c, dev)
    torch.cuda.synchronize()
    # outputs pre-filled with NaN bit patterns: every element must be written
    outs = [torch.full_like(t, float("nan")) for t in (dq, dk, dv)]
    kw = dict(r.kw, dq=outs[0], dk=outs[1], dv=outs[2])
    bsa.bsa_bwd_noalloc(*r.args, **kw)
    torch.cuda.synchronize()
    for got, want, nm in zip(outs, (dq, dk, dv), ("dq", "dk", "dv")):
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"{name}/{nm}"
    ref = oracle.backward(c.q, c.k, c.v, o, c.do, lse, c.mask, **oracle_kw(c))
    floor = float(np.abs(ref[2]).max())
    for got, want, nm in zip(outs, ref, ("dq", "dk", "dv")):
        assert_close(f"{name}/{nm} (no-alloc)", to_np(got), want, c.dtype, floor_ref=floor)


def test_noalloc_two_calls_second_smaller():
    # a split-unit case (partial slots in the scratch), then a smaller TND case
    _noalloc_vs_workspace("bnsd_bf16_d128_local_sink_split")
    _noalloc_vs_workspace("tnd_fp16_d64_window_ahead")


def test_noalloc_rejects_a_problem_beyond_the_scratch():
    """BNSD 1 x 8 x 65536 x 64 with 16 x 16 blocks: the lists alone need 1 GiB.
    Rejected on the host (161002) with both sizes named; nothing runs."""
    import block_sparse_attention_bwd_amd as bsa
    buf = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")

    def desc(shape, dtype):
        t = bsa.bsa_tensor()
        t.data = buf.data_ptr()
        t.dtype = dtype
        t.ndim = len(shape)
        st = 1
        for i in reversed(range(len(shape))):
            t.shape[i] = shape[i]
            t.stride[i] = st
            st *= shape[i]
        return t

    x = desc((1, 8, 65536, 64), bsa.BSA_DTYPE_BF16)
    args = [desc((1, 8, 65536, 64), bsa.BSA_DTYPE_BF16) for _ in range(5)]
    lse = desc((1, 8, 65536), bsa.BSA_DTYPE_F32)
    mask = desc((1, 8, 4096, 4096), bsa.BSA_DTYPE_BOOL)
    with pytest.raises(bsa.BsaError) as e:
        bsa.bsa_bwd_noalloc(*args, lse, block_sparse_mask=mask, block_shape=[16, 16], num_key_value_heads=8,
                            scale_value=0.125, dq=x, dk=desc((1, 8, 65536, 64), bsa.BSA_DTYPE_BF16),
                            dv=desc((1, 8, 65536, 64), bsa.BSA_DTYPE_BF16))
    assert e.value.code == bsa.BSA_ERR_PARAM_INVALID
    assert "scratch" in e.value.message and str(64 << 20) in e.value.message
    torch.cuda.synchronize()
    assert int(buf.count_nonzero()) == 0

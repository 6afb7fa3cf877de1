"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function the header declares, and phase 1 returns the documented status
for every invalid argument (aclnnBlockSparseAttentionGrad page, 返回值 table:
161001 for null inputs and TND without lengths, 161002 for invalid dtypes,
layouts and other parameters)."""
import ctypes
import os

import pytest
import torch

import block_sparse_attention_bwd_amd as bsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not os.path.exists(bsa.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    bsa.load_library()


def test_exports_every_header_function():
    lib = bsa.load_library()
    names = bsa.header_functions()
    assert {"bsa_bwd_workspace_size", "bsa_bwd", "bsa_last_error"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def _bnsd(B=2, N=4, Nkv=2, Sq=300, Skv=270, D=128, dt=torch.bfloat16, bx=128, by=128):
    q = torch.zeros(B, N, Sq, D, dtype=dt)
    k = torch.zeros(B, Nkv, Skv, D, dtype=dt)
    lse = torch.zeros(B, N, Sq, dtype=torch.float32)
    mask = torch.ones(B, N, -(-Sq // bx), -(-Skv // by), dtype=torch.bool)
    return dict(dout=q, query=q, key=k, value=k, attention_out=q, softmax_lse=lse, block_sparse_mask=mask,
                atten_mask=None, block_shape=[bx, by], actual_seq_lengths=None, actual_seq_lengths_kv=None,
                q_input_layout="BNSD", kv_input_layout="BNSD", num_key_value_heads=Nkv, mask_type=0,
                scale_value=D ** -0.5, pre_tokens=bsa.NO_WINDOW, next_tokens=bsa.NO_WINDOW,
                dq=q.clone(), dk=k.clone(), dv=k.clone())


def _tnd(lq=(100, 37, 250), lk=(80, 90, 5), N=4, Nkv=1, D=64, dt=torch.float16, bx=64, by=128):
    q = torch.zeros(sum(lq), N, D, dtype=dt)
    k = torch.zeros(sum(lk), Nkv, D, dtype=dt)
    lse = torch.zeros(sum(lq), N, 1, dtype=torch.float32)
    mask = torch.ones(len(lq), N, -(-max(lq) // bx), -(-max(lk) // by), dtype=torch.uint8)
    return dict(dout=q, query=q, key=k, value=k, attention_out=q, softmax_lse=lse, block_sparse_mask=mask,
                atten_mask=None, block_shape=[bx, by], actual_seq_lengths=list(lq),
                actual_seq_lengths_kv=list(lk), q_input_layout="TND", kv_input_layout="TND",
                num_key_value_heads=Nkv, mask_type=0, scale_value=D ** -0.5, pre_tokens=bsa.NO_WINDOW,
                next_tokens=bsa.NO_WINDOW, dq=q.clone(), dk=k.clone(), dv=k.clone())


def _code(args):
    try:
        bsa.bsa_bwd_workspace_size(**args)
    except bsa.BsaError as e:
        assert bsa.bsa_last_error() == e.message
        return e.code
    return bsa.BSA_OK


def test_valid_arguments_are_accepted():
    assert bsa.bsa_bwd_workspace_size(**_bnsd()) > 0
    assert bsa.bsa_bwd_workspace_size(**_tnd()) > 0
    a = _bnsd()
    a["softmax_lse"] = a["softmax_lse"][..., None]  # trailing 1 accepted
    assert _code(a) == bsa.BSA_OK
    a = _bnsd()
    a["block_sparse_mask"] = None  # no mask = dense; block shape ignored
    a["block_shape"] = [0, 0]
    assert _code(a) == bsa.BSA_OK
    a = _bnsd(bx=64, by=128)
    a["block_shape"] = [64, 128, 999]  # at least two elements; the first two are used
    assert _code(a) == bsa.BSA_OK
    a = _bnsd(bx=128, by=128)
    a["block_shape"] = None  # default [128, 128]
    assert _code(a) == bsa.BSA_OK
    a = _bnsd()
    a["actual_seq_lengths"] = [300, 17]
    a["actual_seq_lengths_kv"] = [0, 270]
    assert _code(a) == bsa.BSA_OK


def test_workspace_size_depends_on_shapes_only():
    a = _bnsd()
    s1 = bsa.bsa_bwd_workspace_size(**a)
    a["block_sparse_mask"] = torch.zeros_like(a["block_sparse_mask"])
    assert bsa.bsa_bwd_workspace_size(**a) == s1
    a["block_sparse_mask"] = torch.rand(a["block_sparse_mask"].shape) < 0.3
    assert bsa.bsa_bwd_workspace_size(**a) == s1
    b = _bnsd(Sq=600)
    assert bsa.bsa_bwd_workspace_size(**b) > s1


def test_layout_regions_are_ordered_and_aligned():
    offs, dims = bsa.bsa_bwd_workspace_layout(**_tnd())
    vals = [offs[k] for k in bsa.WS_REGIONS]
    assert vals == sorted(vals)
    assert all(v % 256 == 0 for v in vals)
    assert offs["total"] == bsa.bsa_bwd_workspace_size(**_tnd())
    assert dims == (64, 128, 4, 1)


def test_layout_region_sizes():
    """Every region holds what the header says it holds (BNSD, B=2, N=4, Nkv=2,
    Sq=300, Skv=270, 128 x 128 blocks: nQB = nKB = 3, 12 dK/dV units of one
    128-row part, 72 possible pieces)."""
    offs, dims = bsa.bsa_bwd_workspace_layout(**_bnsd())
    B, N, Nkv, Sq, D, nqb, nkb = 2, 4, 2, 300, 128, 3, 3
    n_units, slots = B * Nkv * nkb, min(B * Nkv * nkb * (N // Nkv) * nqb, 768)
    size = {k: offs[b] - offs[a] for k, a, b in zip(bsa.WS_REGIONS, bsa.WS_REGIONS, bsa.WS_REGIONS[1:])}
    assert size["seq"] >= B * 32 + 128 * 4
    assert size["delta"] >= B * N * Sq * 4 and size["lse2"] >= B * N * Sq * 4
    assert size["row_cnt"] >= B * N * nqb * 4 and size["row_list"] >= B * N * nqb * nkb * 4
    assert size["col_cnt"] >= B * N * nkb * 4 and size["col_list"] >= B * N * nkb * nqb * 4
    assert size["plan"] >= 4 * (4 + 4 * (n_units + slots))
    assert size["partial"] >= slots * 2 * 128 * D * 4


def test_row_stride_beyond_32bit_tile_offsets_is_rejected():
    """The kernels address a tile's rows (at most 128) from its first row by 32-bit byte
    offsets, so a TND row of N * D elements may not exceed (2**32 / 2 - D) / 128 elements."""
    ok = _tnd(lq=(1,), lk=(1,), N=128, Nkv=1, D=128)  # row stride 16384 elements
    assert bsa.bsa_bwd_workspace_size(**ok) > 0
    bad = _tnd(lq=(1,), lk=(1,), N=131072, Nkv=1, D=128)  # 16 Mi elements per token row
    assert _code(bad) == INVALID
    assert "row stride" in bsa.bsa_last_error()


def test_layout_partial_region_scales_with_head_dim():
    """The fp32 partials hold [slots][dK, dV][128 rows][D]: twice as large at D = 256."""
    sizes = {}
    for D in (64, 128, 256):
        offs, _ = bsa.bsa_bwd_workspace_layout(**_bnsd(D=D))
        i = bsa.WS_REGIONS.index("partial")
        sizes[D] = offs[bsa.WS_REGIONS[i + 1]] - offs["partial"]
    slots = min(2 * 2 * 3 * 2 * 3, 768)
    for D in (64, 128, 256):
        assert sizes[D] >= slots * 2 * 128 * D * 4
    assert sizes[256] > sizes[128] > sizes[64]


NULLPTR = bsa.BSA_ERR_PARAM_NULLPTR
INVALID = bsa.BSA_ERR_PARAM_INVALID


def _mut(base, **kv):
    a = base()
    a.update(kv)
    return a


def _tr(x):
    return x.transpose(-1, -2).contiguous().transpose(-1, -2)


CASES = [
    # null inputs (161001)
    ("dout null", lambda: _mut(_bnsd, dout=None), NULLPTR),
    ("query null", lambda: _mut(_bnsd, query=None), NULLPTR),
    ("key null", lambda: _mut(_bnsd, key=None), NULLPTR),
    ("value null", lambda: _mut(_bnsd, value=None), NULLPTR),
    ("attentionOut null", lambda: _mut(_bnsd, attention_out=None), NULLPTR),
    ("softmaxLse null", lambda: _mut(_bnsd, softmax_lse=None), NULLPTR),
    ("dq null", lambda: _mut(_bnsd, dq=None), NULLPTR),
    ("dk null", lambda: _mut(_bnsd, dk=None), NULLPTR),
    ("dv null", lambda: _mut(_bnsd, dv=None), NULLPTR),
    ("TND without q lengths", lambda: _mut(_tnd, actual_seq_lengths=None), NULLPTR),
    ("TND without kv lengths", lambda: _mut(_tnd, actual_seq_lengths_kv=None), NULLPTR),
    ("layout string null", lambda: _mut(_bnsd, q_input_layout=None), NULLPTR),
    # invalid dtypes (161002)
    ("fp32 data", lambda: _mut(_bnsd, query=torch.zeros(2, 4, 300, 128)), INVALID),
    ("mixed dtypes", lambda: _mut(_bnsd, key=torch.zeros(2, 2, 270, 128, dtype=torch.float16),
                                  value=torch.zeros(2, 2, 270, 128, dtype=torch.float16)), INVALID),
    ("fp16 lse", lambda: _mut(_bnsd, softmax_lse=torch.zeros(2, 4, 300, dtype=torch.float16)), INVALID),
    ("float mask", lambda: _mut(_bnsd, block_sparse_mask=torch.ones(2, 4, 3, 3)), INVALID),
    ("fp16 dq with bf16 inputs", lambda: _mut(_bnsd, dq=torch.zeros(2, 4, 300, 128, dtype=torch.float16)), INVALID),
    # invalid layouts
    ("layout BSND", lambda: _mut(_bnsd, q_input_layout="BSND", kv_input_layout="BSND"), INVALID),
    ("layouts differ", lambda: _mut(_bnsd, kv_input_layout="TND"), INVALID),
    ("ndim mismatch", lambda: _mut(_bnsd, q_input_layout="TND", kv_input_layout="TND",
                                   actual_seq_lengths=[300, 300], actual_seq_lengths_kv=[270, 270]), INVALID),
    # heads and dims
    ("N % Nkv != 0", lambda: _mut(lambda: _bnsd(N=3, Nkv=2)), INVALID),
    ("N < Nkv", lambda: _mut(lambda: _bnsd(N=2, Nkv=4)), INVALID),
    ("numKeyValueHeads mismatch", lambda: _mut(_bnsd, num_key_value_heads=1), INVALID),
    ("head dim 96", lambda: _mut(lambda: _bnsd(D=96)), INVALID),
    ("head dim 512", lambda: _mut(lambda: _bnsd(D=512)), INVALID),
    ("head dim 256", lambda: _mut(lambda: _bnsd(D=256)), bsa.BSA_OK),
    ("head dim 64", lambda: _mut(lambda: _bnsd(D=64)), bsa.BSA_OK),
    ("query/key batch differ", lambda: _mut(_bnsd, key=torch.zeros(1, 2, 270, 128, dtype=torch.bfloat16)), INVALID),
    ("dout shape differs", lambda: _mut(_bnsd, dout=torch.zeros(2, 4, 299, 128, dtype=torch.bfloat16)), INVALID),
    ("dk shape differs", lambda: _mut(_bnsd, dk=torch.zeros(2, 2, 271, 128, dtype=torch.bfloat16)), INVALID),
    ("lse shape", lambda: _mut(_bnsd, softmax_lse=torch.zeros(2, 4, 299)), INVALID),
    ("lse trailing 2", lambda: _mut(_bnsd, softmax_lse=torch.zeros(2, 4, 300, 2)), INVALID),
    ("empty dim", lambda: _mut(_bnsd, query=torch.zeros(2, 4, 0, 128, dtype=torch.bfloat16)), NULLPTR),
    # mask and block shape
    ("mask shape", lambda: _mut(_bnsd, block_sparse_mask=torch.ones(2, 4, 3, 2, dtype=torch.bool)), INVALID),
    ("mask on KV heads", lambda: _mut(_bnsd, block_sparse_mask=torch.ones(2, 2, 3, 3, dtype=torch.bool)), INVALID),
    ("blockShape one element", lambda: _mut(_bnsd, block_shape=[128]), INVALID),
    ("blockShape zero", lambda: _mut(_bnsd, block_shape=[0, 128]), INVALID),
    ("blockShape negative", lambda: _mut(_bnsd, block_shape=[128, -1]), INVALID),
    ("blockShape mismatches mask", lambda: _mut(_bnsd, block_shape=[64, 128]), INVALID),
    # reserved attributes
    ("attenMask [Sq, Skv]", lambda: _mut(_bnsd, atten_mask=torch.zeros(300, 270, dtype=torch.bool)), bsa.BSA_OK),
    ("attenMask shape", lambda: _mut(_bnsd, atten_mask=torch.zeros(300, 271, dtype=torch.bool)), INVALID),
    ("attenMask 4-D", lambda: _mut(_bnsd, atten_mask=torch.zeros(1, 1, 300, 270, dtype=torch.bool)), INVALID),
    ("attenMask float", lambda: _mut(_bnsd, atten_mask=torch.zeros(300, 270)), INVALID),
    ("attenMask non-contiguous", lambda: _mut(_bnsd, atten_mask=torch.zeros(270, 300, dtype=torch.bool).t()), INVALID),
    ("maskType 1", lambda: _mut(_bnsd, mask_type=1), INVALID),
    # a sliding window (preTokens / nextTokens other than 2147483647) is accepted
    ("preTokens window", lambda: _mut(_bnsd, pre_tokens=1024), bsa.BSA_OK),
    ("nextTokens window", lambda: _mut(_bnsd, next_tokens=0), bsa.BSA_OK),
    ("negative window", lambda: _mut(_bnsd, pre_tokens=-5, next_tokens=2**40), bsa.BSA_OK),
    ("scale NaN", lambda: _mut(_bnsd, scale_value=float("nan")), INVALID),
    # strides
    ("non-contiguous query", lambda: _mut(_bnsd, query=_tr(torch.zeros(2, 4, 300, 128, dtype=torch.bfloat16))), INVALID),
    ("non-contiguous key", lambda: _mut(_bnsd, key=torch.zeros(2, 270, 2, 128, dtype=torch.bfloat16).transpose(1, 2)), INVALID),
    ("dq inner stride", lambda: _mut(_bnsd, dq=_tr(torch.zeros(2, 4, 300, 128, dtype=torch.bfloat16))), INVALID),
    ("dq zero head stride", lambda: _mut(_bnsd, dq=torch.zeros(2, 1, 300, 128, dtype=torch.bfloat16).expand(2, 4, 300, 128)),
     INVALID),
    ("dk overlapping rows", lambda: _mut(_bnsd, dk=torch.zeros(2 * 2 * 270 * 64 + 64, dtype=torch.bfloat16).as_strided(
        (2, 2, 270, 128), (2 * 270 * 64, 270 * 64, 64, 1))), INVALID),
    ("dv with padded rows", lambda: _mut(_bnsd, dv=torch.zeros(2, 2, 270, 200, dtype=torch.bfloat16)[..., :128]),
     bsa.BSA_OK),
    ("dq heads interleaved (transposed outer dims)", lambda: _mut(
        _bnsd, dq=torch.zeros(2, 300, 4, 128, dtype=torch.bfloat16).transpose(1, 2)), bsa.BSA_OK),
    # sequence lengths
    ("BNSD length > S", lambda: _mut(_bnsd, actual_seq_lengths=[301, 3]), INVALID),
    ("BNSD length count", lambda: _mut(_bnsd, actual_seq_lengths=[300]), INVALID),
    ("BNSD negative length", lambda: _mut(_bnsd, actual_seq_lengths_kv=[-1, 3]), INVALID),
    ("TND q sum", lambda: _mut(_tnd, actual_seq_lengths=[100, 37, 249]), INVALID),
    ("TND kv sum", lambda: _mut(_tnd, actual_seq_lengths_kv=[80, 90, 6]), INVALID),
    ("TND count mismatch", lambda: _mut(_tnd, actual_seq_lengths_kv=[170, 5]), INVALID),
    ("TND prefix sums", lambda: _mut(_tnd, actual_seq_lengths=[100, 137, 387]), INVALID),
]


@pytest.mark.parametrize("name,make,code", CASES, ids=[c[0] for c in CASES])
def test_phase1_status(name, make, code):
    assert _code(make()) == code


def test_null_workspace_size_pointer():
    lib = bsa.load_library()
    from block_sparse_attention_bwd_amd._binding import _marshal
    a = _bnsd()
    args = _marshal(**a)
    assert lib.bsa_bwd_workspace_size(*args, None) == NULLPTR


def test_phase2_rejects_before_touching_the_device():
    """bsa_bwd re-validates; a short or null workspace fails before any HIP call."""
    lib = bsa.load_library()
    from block_sparse_attention_bwd_amd._binding import _marshal
    a = _bnsd()
    need = bsa.bsa_bwd_workspace_size(**a)
    args = _marshal(**a)
    assert lib.bsa_bwd(*args, ctypes.c_void_p(4096), need - 1, None) == INVALID
    assert lib.bsa_bwd(*args, None, need, None) == NULLPTR
    assert lib.bsa_bwd(*args, ctypes.c_void_p(4096 + 8), need, None) == INVALID  # misaligned
    bad = _marshal(**_mut(_bnsd, mask_type=3))
    assert lib.bsa_bwd(*bad, ctypes.c_void_p(4096), need, None) == INVALID


def test_binding_refuses_cpu_tensors_for_phase2():
    with pytest.raises(ValueError):
        bsa.bsa_bwd(**_bnsd(), workspace=None, workspace_size=0)


def test_stage_names():
    assert [bsa.bsa_stage_name(i) for i in range(5)] == ["prologue", "dkdv", "dq", "fwd", None]


def _fake(t):
    """Descriptor of a meta tensor with a non-null address: phase 1 never reads data."""
    d = bsa.bsa_tensor()
    d.data = 0x1000
    d.dtype = bsa._binding._dtype_code(t)
    d.ndim = t.dim()
    for i in range(t.dim()):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return d


def _huge(B, N, Sq, Skv, bx, by, D=64):
    meta = dict(device="meta")
    q = torch.empty(B, N, Sq, D, dtype=torch.bfloat16, **meta)
    k = torch.empty(B, 1, Skv, D, dtype=torch.bfloat16, **meta)
    lse = torch.empty(B, N, Sq, dtype=torch.float32, **meta)
    mask = torch.empty(B, N, -(-Sq // bx), -(-Skv // by), dtype=torch.bool, **meta)
    return dict(dout=_fake(q), query=_fake(q), key=_fake(k), value=_fake(k), attention_out=_fake(q),
                softmax_lse=_fake(lse), block_sparse_mask=_fake(mask), atten_mask=None, block_shape=[bx, by],
                actual_seq_lengths=None, actual_seq_lengths_kv=None, q_input_layout="BNSD",
                kv_input_layout="BNSD", num_key_value_heads=1, mask_type=0, scale_value=D ** -0.5,
                pre_tokens=bsa.NO_WINDOW, next_tokens=bsa.NO_WINDOW, dq=_fake(q), dk=_fake(k), dv=_fake(k))


# Prologue workgroups with one query row, Skv = 16384 and 1 x 1 blocks: N
# (softmax_grad, one 64-row run per head) + ceil(N / 4) (row lists) + 256 N
# (column lists, 64 KV blocks each), i.e. 16,777,074 for N = 65217 and
# 16,777,331 for N = 65218, against a limit of (2^32 - 1) / 256 = 16,777,215.
@pytest.mark.parametrize("what,shape", [
    ("prologue", (1, 65218, 1, 16384, 1, 1)),
    # 2^24 dQ workgroups of 128 query rows
    ("dq", (1, 16384, 131072, 128, 128, 128)),
    # 2^24 dK/dV units of 128 key rows (a 1 x 2^24 block grid per head)
    ("dkdv", (1, 1, 128, (1 << 31) - 1, 128, 128)),
])
def test_launch_grid_limit(what, shape):
    args = _huge(*shape)
    assert _code(args) == INVALID, what
    assert "launch grid too large" in bsa.bsa_last_error()


def test_attenmask_packing_launch_limit():
    """The attenMask is packed by one wave per 64 x 64 tile, 4 per workgroup: with
    Sq = Skv = 2^19 that is 2^26 / 4 = 2^24 workgroups, above (2^32 - 1) / 256."""
    S = 1 << 19
    args = _huge(1, 1, S, S, S, S)  # one block: the lists stay tiny
    args["atten_mask"] = _fake(torch.empty(S, S, dtype=torch.bool, device="meta"))
    assert _code(args) == INVALID
    assert "attenMask too large" in bsa.bsa_last_error()
    args = _huge(1, 1, 1 << 16, 1 << 16, 1 << 16, 1 << 16)
    args["atten_mask"] = _fake(torch.empty(1 << 16, 1 << 16, dtype=torch.bool, device="meta"))
    assert _code(args) == bsa.BSA_OK


def test_launch_grid_just_below_limit():
    args = _huge(1, 65217, 1, 16384, 1, 1)
    assert _code(args) == bsa.BSA_OK, bsa.bsa_last_error()


# ---- forward (bsa_fwd_workspace_size): same validation, O and LSE are outputs ----
def _fwd(base=_bnsd, **kv):
    a = base()
    for k in ("dout", "dq", "dk", "dv"):
        a.pop(k)
    a.update(kv)
    return a


def _fcode(args):
    try:
        bsa.bsa_fwd_workspace_size(**args)
    except bsa.BsaError as e:
        assert bsa.bsa_last_error() == e.message
        return e.code
    return bsa.BSA_OK


FWD_CASES = [
    ("valid BNSD", lambda: _fwd(), bsa.BSA_OK),
    ("valid TND", lambda: _fwd(_tnd), bsa.BSA_OK),
    ("valid LSE [B,N,S,1]", lambda: _fwd(softmax_lse=torch.zeros(2, 4, 300, 1)), bsa.BSA_OK),
    ("O with outer strides", lambda: _fwd(attention_out=torch.zeros(2, 300, 4, 128, dtype=torch.bfloat16).transpose(1, 2)),
     bsa.BSA_OK),
    ("O null", lambda: _fwd(attention_out=None), NULLPTR),
    ("LSE null", lambda: _fwd(softmax_lse=None), NULLPTR),
    ("query null", lambda: _fwd(query=None), NULLPTR),
    ("O dtype", lambda: _fwd(attention_out=torch.zeros(2, 4, 300, 128, dtype=torch.float16)), INVALID),
    ("O shape", lambda: _fwd(attention_out=torch.zeros(2, 4, 299, 128, dtype=torch.bfloat16)), INVALID),
    ("O inner stride", lambda: _fwd(attention_out=_tr(torch.zeros(2, 4, 300, 128, dtype=torch.bfloat16))), INVALID),
    ("O row stride not a multiple of 4", lambda: _fwd(
        attention_out=torch.zeros(2, 4, 300, 130, dtype=torch.bfloat16)[..., :128]), INVALID),
    ("O row stride a multiple of 4", lambda: _fwd(
        attention_out=torch.zeros(2, 4, 300, 132, dtype=torch.bfloat16)[..., :128]), bsa.BSA_OK),
    ("O data pointer not 8-byte aligned", lambda: _fwd(
        attention_out=torch.zeros(2 * 4 * 300 * 128 + 1, dtype=torch.bfloat16)[1:].view(2, 4, 300, 128)), INVALID),
    ("O overlapping heads", lambda: _fwd(attention_out=torch.zeros(2, 1, 300, 128, dtype=torch.bfloat16).expand(
        2, 4, 300, 128)), INVALID),
    ("LSE fp16", lambda: _fwd(softmax_lse=torch.zeros(2, 4, 300, dtype=torch.float16)), INVALID),
    ("LSE non-contiguous", lambda: _fwd(softmax_lse=torch.zeros(2, 300, 4).transpose(1, 2)), INVALID),
    ("LSE shape", lambda: _fwd(softmax_lse=torch.zeros(2, 4, 299)), INVALID),
    ("sliding window", lambda: _fwd(pre_tokens=64, next_tokens=0), bsa.BSA_OK),
    ("TND without lengths", lambda: _fwd(_tnd, actual_seq_lengths=None), NULLPTR),
]


@pytest.mark.parametrize("name,make,code", FWD_CASES, ids=[c[0] for c in FWD_CASES])
def test_forward_phase1_status(name, make, code):
    assert _fcode(make()) == code


def test_forward_workspace_is_sequence_table_and_row_lists():
    """The forward needs the sequence table, 128 constants and the row lists only."""
    fwd = bsa.bsa_fwd_workspace_size(**_fwd())
    B, N, nqb, nkb = 2, 4, 3, 3
    al = lambda x: -(-x // 256) * 256
    assert fwd == al(B * 32 + 128 * 4) + al(B * N * nqb * 4) + al(B * N * nqb * nkb * 4)
    assert fwd < bsa.bsa_bwd_workspace_size(**_bnsd())


def test_forward_binding_refuses_cpu_tensors():
    a = _fwd()
    with pytest.raises(ValueError):
        bsa.bsa_fwd(**a, workspace=None)


def test_plan_dump_with_bsa_log():
    """BSA_LOG=1 makes a validated call print its plan to stderr (read per call)."""
    import subprocess
    import sys
    code = ("import sys; sys.path[:0] = [%r, %r]; import test_api as t, block_sparse_attention_bwd_amd as bsa; "
            "bsa.bsa_bwd_workspace_size(**t._tnd())" % (ROOT, os.path.join(ROOT, "tests")))
    env = dict(os.environ, BSA_LOG="1")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "[bsa] bsa_bwd_workspace_size: TND B=3 N=4 Nkv=1 G=4 D=64" in r.stderr
    assert "ws row_list" in r.stderr and "workspace total" in r.stderr
    r = subprocess.run([sys.executable, "-c", code], env=dict(os.environ, BSA_LOG="0"), capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0 and "[bsa]" not in r.stderr


# ---- dq_mode of bsa_bwd_ex ----------------------------------------------------

def _ex_code(args, mode):
    try:
        bsa.bsa_bwd_ex_workspace_size(**args, dq_mode=mode)
    except bsa.BsaError as e:
        return e.code
    return bsa.BSA_OK


def test_dq_mode_recompute_is_the_plain_call():
    for make in (_bnsd, _tnd):
        a = make()
        assert bsa.bsa_bwd_ex_workspace_size(**a, dq_mode=bsa.BSA_DQ_RECOMPUTE) == bsa.bsa_bwd_workspace_size(**a)


def test_dq_mode_atomic_adds_the_accumulator():
    """The accumulator is fp32 [B, N, maxSq, D]; nothing else changes."""
    for make, (B, N, Sq, D) in ((_bnsd, (2, 4, 300, 128)), (_tnd, (3, 4, 250, 64))):
        a = make()
        plain = bsa.bsa_bwd_workspace_size(**a)
        atomic = bsa.bsa_bwd_ex_workspace_size(**a, dq_mode=bsa.BSA_DQ_ATOMIC)
        acc = 4 * B * N * Sq * D
        assert atomic - plain == -(-acc // 256) * 256


def test_dq_mode_rejections():
    ok = _bnsd()
    assert _ex_code(ok, bsa.BSA_DQ_ATOMIC) == bsa.BSA_OK
    assert _ex_code(ok, 2) == bsa.BSA_ERR_PARAM_INVALID
    assert _ex_code(ok, -1) == bsa.BSA_ERR_PARAM_INVALID
    # head dim 256: the generic dK/dV build, which has no dQ product
    assert _ex_code(_bnsd(D=256), bsa.BSA_DQ_ATOMIC) == bsa.BSA_ERR_PARAM_INVALID
    assert _ex_code(_bnsd(D=256), bsa.BSA_DQ_RECOMPUTE) == bsa.BSA_OK
    # an attenMask: likewise
    am = _bnsd()
    am["atten_mask"] = torch.zeros(300, 270, dtype=torch.bool)
    assert _ex_code(am, bsa.BSA_DQ_ATOMIC) == bsa.BSA_ERR_PARAM_INVALID
    assert _ex_code(am, bsa.BSA_DQ_RECOMPUTE) == bsa.BSA_OK
    msg = bsa.bsa_last_error()
    assert msg == ""

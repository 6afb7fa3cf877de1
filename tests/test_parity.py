"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Bars: block lists bit-exact; dQ, dK, dV per tensor within
max|gpu - ref| <= tol * max|ref| (tol 5e-3 fp16, 2e-2 bf16); bitwise
run-to-run determinism.
"""
import math
import time

import numpy as np
import pytest

import oracle
import synth
from gpu_common import (TOL, _guarded, _guards_intact, assert_close, oracle_backward_threaded, oracle_fwd_inputs,
                        oracle_kw, run_bsa, to_np, upload)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_bwd_amd as bsa
    bsa.load_library()
    torch.backends.cuda.matmul.allow_tf32 = False
    yield


from cases import SMALL, case as _case  # noqa: E402

_cache = {}


def _prepared(name):
    if name not in _cache:
        c = _case(name)
        o, lse = oracle_fwd_inputs(c)
        ref = oracle.backward(c.q, c.k, c.v, o, c.do, lse, c.mask, **oracle_kw(c))
        _cache[name] = (c, o, lse, ref)
    return _cache[name]


@pytest.mark.parametrize("name", SMALL)
def test_small_case_parity(name):
    c, o, lse, ref = _prepared(name)
    print(f"[parity] {name}", flush=True)
    dev = upload(c, o, lse)
    (dq, dk, dv), _ = run_bsa(c, dev)
    torch.cuda.synchronize()
    floor = float(np.abs(ref[2]).max())
    for nm, got, want in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
        assert_close(f"{name}/{nm}", to_np(got), want, c.dtype, floor_ref=floor)


@pytest.mark.parametrize("scale", [0.0, 1e-32, 1e-20, -0.09])
def test_scale_edges(scale):
    """The scheduled dK/dV kernel starts its score accumulator at -lse2 / c
    (c = scale * log2 e): a scale of 0, one below 2^-100 (scores taken as 0),
    a tiny one (-lse2 / c near 1e20) and a negative one against the oracle."""
    c = synth.make_case(layout="BNSD", dtype="bf16", B=1, N=2, Nkv=1, D=128, Sq=256, Skv=288, bx=128, by=128,
                        p=0.6, scale=scale, seed=131)
    o, lse = oracle_fwd_inputs(c)
    ref = oracle.backward(c.q, c.k, c.v, o, c.do, lse, c.mask, **oracle_kw(c))
    dev = upload(c, o, lse)
    (dq, dk, dv), _ = run_bsa(c, dev)
    torch.cuda.synchronize()
    floor = float(np.abs(ref[2]).max())
    for nm, got, want in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
        assert_close(f"scale {scale}/{nm}", to_np(got), want, c.dtype, floor_ref=floor)


def _read_ws(runner, offs, name, count, dtype=np.int32):
    import block_sparse_attention_bwd_amd  # noqa: F401
    start = offs[name]
    nbytes = count * np.dtype(dtype).itemsize
    return runner.ws[start:start + nbytes].cpu().numpy().view(dtype)


@pytest.mark.parametrize("name", SMALL)
def test_block_lists_bit_exact(name):
    import block_sparse_attention_bwd_amd as bsa
    c, o, lse, _ = _prepared(name)
    dev = upload(c, o, lse)
    _, r = run_bsa(c, dev)
    torch.cuda.synchronize()
    offs, (bx, by, nqb, nkb) = bsa.bsa_bwd_workspace_layout(*r.args, **r.kw)
    rows, cols = oracle.block_lists(c.mask, c.B, c.N, nqb, nkb, bx, by, c.len_q, c.len_kv, window=c.window)
    rc = _read_ws(r, offs, "row_cnt", c.B * c.N * nqb).reshape(c.B, c.N, nqb)
    rl = _read_ws(r, offs, "row_list", c.B * c.N * nqb * nkb).reshape(c.B, c.N, nqb, nkb)
    cc = _read_ws(r, offs, "col_cnt", c.B * c.N * nkb).reshape(c.B, c.N, nkb)
    cl = _read_ws(r, offs, "col_list", c.B * c.N * nkb * nqb).reshape(c.B, c.N, nkb, nqb)
    for b in range(c.B):
        for n in range(c.N):
            for i in range(nqb):
                assert rc[b, n, i] == len(rows[b][n][i]), (b, n, i)
                assert list(rl[b, n, i, :rc[b, n, i]]) == rows[b][n][i], (b, n, i)
            for j in range(nkb):
                assert cc[b, n, j] == len(cols[b][n][j]), (b, n, j)
                assert list(cl[b, n, j, :cc[b, n, j]]) == cols[b][n][j], (b, n, j)


@pytest.mark.parametrize("name", ["config1", "tnd_fp16_d128_b64x128_gqa", "bnsd_fp16_d64_b64x128_padded",
                                  "tnd_fp16_d256_b64x64_gqa", "tnd_bf16_d64_empty_seqs", "bnsd_fp16_d128_b256x256"])
def test_delta_and_lse2(name):
    """softmax_grad (stored negated) and lse2 as the dQ kernel writes them for
    the dK/dV kernel: every row of [B, N, maxSq], zeros past a sequence's end
    (a sequence with no queries; Q blocks of two 128-row parts)."""
    import block_sparse_attention_bwd_amd as bsa
    c, o, lse, _ = _prepared(name)
    dev = upload(c, o, lse)
    _, r = run_bsa(c, dev)
    torch.cuda.synchronize()
    offs, _ = bsa.bsa_bwd_workspace_layout(*r.args, **r.kw)
    sq = c.Sq
    delta = -_read_ws(r, offs, "delta", c.B * c.N * sq, np.float32).reshape(c.B, c.N, sq)  # stored negated
    lse2 = _read_ws(r, offs, "lse2", c.B * c.N * sq, np.float32).reshape(c.B, c.N, sq)
    offq = oracle.sequence_offsets(c.len_q)
    for b in range(c.B):
        L = int(c.len_q[b])
        if c.layout == "BNSD":
            dob, ob, lb = c.do[b, :, :L], o[b, :, :L], lse[b, :, :L]
        else:
            dob = c.do[offq[b]:offq[b] + L].transpose(1, 0, 2)
            ob = o[offq[b]:offq[b] + L].transpose(1, 0, 2)
            lb = lse[offq[b]:offq[b] + L].T
        want = oracle.softmax_grad(dob, ob)
        mag = np.sum(np.abs(dob.astype(np.float64) * ob), axis=-1)
        assert np.all(np.abs(delta[b, :, :L] - want) <= 1e-5 * mag + 1e-30)
        assert np.all(delta[b, :, L:] == 0)
        fin = np.isfinite(lb)
        np.testing.assert_allclose(lse2[b, :, :L][fin], lb[fin].astype(np.float64) * math.log2(math.e), rtol=1e-6)


@pytest.mark.parametrize("name", ["bnsd_bf16_d128_b128x128_ragged", "tnd_fp16_d128_b64x128_gqa",
                                  "bnsd_bf16_d128_local_sink_split", "bnsd_fp16_d256_sink_split"])
def test_bitwise_deterministic(name):
    c, o, lse, _ = _prepared(name)
    dev = upload(c, o, lse)
    (dq, dk, dv), r = run_bsa(c, dev)
    a = [t.clone() for t in (dq, dk, dv)]
    for _ in range(3):
        r()
    torch.cuda.synchronize()
    for x, y in zip(a, (r.dq, r.dk, r.dv)):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_split_units_are_planned():
    """The sink-column case really takes the split path: read the plan back.

    Checks the chunk rule, the piece count of every unit, and that the launch
    order lists every (unit, piece) once, longest first by cost class."""
    import block_sparse_attention_bwd_amd as bsa
    c, o, lse, _ = _prepared("bnsd_bf16_d128_local_sink_split")
    dev = upload(c, o, lse)
    _, r = run_bsa(c, dev)
    torch.cuda.synchronize()
    offs, (bx, by, nqb, nkb) = bsa.bsa_bwd_workspace_layout(*r.args, **r.kw)
    n_units = c.B * c.Nkv * nkb
    G = c.N // c.Nkv
    slots = min(n_units * G * nqb, 768)
    assert offs["partial"] - offs["plan"] >= 4 * (4 + 4 * (n_units + slots))
    plan = _read_ws(r, offs, "plan", 4 + 4 * (n_units + slots))
    pc, n_items = int(plan[0]), int(plan[1])
    pieces = [int(k) for k in plan[4:4 + n_units]]
    _, cols = oracle.block_lists(c.mask, c.B, c.N, nqb, nkb, bx, by, c.len_q, c.len_kv)
    totals = [sum(len(cols[0][n][j]) for n in range(c.N)) for j in range(nkb)]
    chunk = max(4, -(-sum(totals) // 256))  # a unit with more entries is split
    assert pc == (chunk + 1) // 2  # entries per piece
    assert pieces == [(-(-t // pc) if t > chunk else 1) for t in totals]
    assert max(pieces) > 1
    assert n_items == sum(pieces)
    ou = plan[4 + 2 * (n_units + slots):][:n_items]
    op = plan[4 + 3 * (n_units + slots):][:n_items]
    assert sorted(zip(ou.tolist(), op.tolist())) == [(u, k) for u in range(n_units) for k in range(pieces[u])]

    def cls(u, k):
        cost = min(pc, totals[u] - k * pc) if pieces[u] > 1 else totals[u]
        return 0 if cost <= 0 else min(63, 1 + (cost - 1) * 63 // chunk)
    classes = [cls(u, k) for u, k in zip(ou.tolist(), op.tolist())]
    assert classes == sorted(classes, reverse=True)


@pytest.mark.parametrize("name", ["config1", "tnd_fp16_d128_b64x128_gqa", "bnsd_bf16_d128_local_sink_split",
                                  "bnsd_fp16_d128_b256x256"])
def test_dq_order_choice(name):
    """plan[2]: XCD-range order for dQ iff the eight contiguous ranges of dQ
    units carry work within 1/32 of each other (unit cost = selected KV blocks + 1);
    the dQ launch order is longest first within each range (or overall)."""
    import block_sparse_attention_bwd_amd as bsa
    c, o, lse, _ = _prepared(name)
    dev = upload(c, o, lse)
    _, r = run_bsa(c, dev)
    torch.cuda.synchronize()
    offs, (bx, by, nqb, nkb) = bsa.bsa_bwd_workspace_layout(*r.args, **r.kw)
    rows, _ = oracle.block_lists(c.mask, c.B, c.N, nqb, nkb, bx, by, c.len_q, c.len_kv)
    nsub = -(-bx // 128)
    cost = [1 + len(rows[b][n][i]) for b in range(c.B) for n in range(c.N) for i in range(nqb) for _ in range(nsub)]
    nd = len(cost)
    per, rem = nd // 8, nd % 8
    bounds = [x * per + min(x, rem) for x in range(9)]
    work = [sum(cost[bounds[x]:bounds[x + 1]]) for x in range(8)]
    want = 1 if 8 * max(work) * 32 <= sum(work) * 33 else 0
    assert int(_read_ws(r, offs, "plan", 4)[2]) == want
    # the dQ launch order (the plan's last nd words): a permutation of the units;
    # with ranges, workgroup 8k + x runs range x's units, else all units, longest
    # first by cost class (selected KV blocks, 64 classes scaled to the largest)
    n_units = c.B * c.Nkv * nkb * -(-by // 128)
    slots = min(n_units * (c.N // c.Nkv) * nqb, 768)
    words = 4 + 4 * (n_units + slots) + nd
    order = _read_ws(r, offs, "plan", words)[4 + 4 * (n_units + slots):].tolist()
    assert sorted(order) == list(range(nd))
    sel = [x - 1 for x in cost]
    mx = max(1, max(sel))
    klass = [0 if v <= 0 else min(63, 1 + (v - 1) * 63 // mx) for v in sel]
    groups = [[order[k] for k in range(x, nd, 8)] for x in range(8)] if want else [order]
    for x, grp in enumerate(groups):
        if want:
            assert sorted(grp) == list(range(bounds[x], bounds[x + 1]))
        cl = [klass[u] for u in grp]
        assert cl == sorted(cl, reverse=True)


# dQ units are sorted longest first only up to this many (the plan kernel's threshold)
DQ_SORT_MAX_UNITS = 8192


@pytest.mark.parametrize("k", [2, 4])
def test_full_config_dq_order(k):
    """The dQ launch order at full size: workload 2 (1024 dQ units) longest first
    by cost class; workload 4 (32768 units, above the sort threshold) in unit
    order, dealt to the XCD ranges when the plan chose them."""
    import block_sparse_attention_bwd_amd as bsa
    c, r, _, _, _ = _full_run(k)
    offs, (bx, by, nqb, nkb) = bsa.bsa_bwd_workspace_layout(*r.args, **r.kw)
    rc = _read_ws(r, offs, "row_cnt", c.B * c.N * nqb).astype(np.int64)
    nsub = -(-bx // 128)
    cost = np.repeat(rc, nsub)
    nd = cost.size
    n_units = c.B * c.Nkv * nkb * -(-by // 128)
    slots = min(n_units * (c.N // c.Nkv) * nqb, 768)
    head = _read_ws(r, offs, "plan", 4)
    words = 4 + 4 * (n_units + slots) + nd
    order = _read_ws(r, offs, "plan", words)[4 + 4 * (n_units + slots):]
    assert np.array_equal(np.sort(order), np.arange(nd))
    ranges = int(head[2]) == 1
    per, rem = nd // 8, nd % 8
    bounds = [x * per + min(x, rem) for x in range(9)]
    groups = [order[x::8] for x in range(8)] if ranges else [order]
    if ranges:
        for x in range(8):
            assert np.array_equal(np.sort(groups[x]), np.arange(bounds[x], bounds[x + 1]))
    if nd <= DQ_SORT_MAX_UNITS:
        mx = max(1, int(cost.max()))
        klass = np.where(cost <= 0, 0, np.minimum(63, 1 + (cost - 1) * 63 // mx))
        for grp in groups:
            cl = klass[grp]
            assert np.all(cl[:-1] >= cl[1:]), "not longest first"
    else:
        for grp in groups:
            assert np.all(np.diff(grp) == 1), "not in unit order"


def test_noncontiguous_outputs_match():
    c, o, lse, ref = _prepared("bnsd_bf16_d128_b128x128_ragged")
    dev = upload(c, o, lse)
    (dq, dk, dv), r = run_bsa(c, dev)
    torch.cuda.synchronize()
    base = [t.clone() for t in (dq, dk, dv)]
    bigq = torch.full((c.B, c.N, c.Sq, 2 * c.D), 7.0, dtype=dq.dtype, device="cuda")
    bigk = torch.full((c.B, c.Nkv, c.Skv, 2 * c.D), 7.0, dtype=dq.dtype, device="cuda")
    bigv = torch.full((c.B, c.Nkv, c.Skv, 2 * c.D), 7.0, dtype=dq.dtype, device="cuda")
    r.kw.update(dq=bigq[..., c.D:], dk=bigk[..., :c.D], dv=bigv[..., c.D:])
    r()
    torch.cuda.synchronize()
    assert torch.equal(bigq[..., c.D:], base[0])
    assert torch.equal(bigk[..., :c.D], base[1])
    assert torch.equal(bigv[..., c.D:], base[2])
    assert torch.all(bigq[..., :c.D] == 7.0) and torch.all(bigk[..., c.D:] == 7.0)


def test_page_worked_sample():
    """The page's sample: constant fp16 inputs; dQ = dK = 0 and dV = 128 exp(S - 5) dout."""
    import block_sparse_attention_bwd_amd as bsa
    B, N, S, D = 1, 1, 128, 128
    full = lambda val: torch.full((B, N, S, D), val, dtype=torch.float16, device="cuda")
    q, k, v, o, do = full(0.1), full(0.1), full(0.1), full(0.1), full(0.01)
    lse = torch.full((B, N, S), 5.0, dtype=torch.float32, device="cuda")
    mask = torch.ones((B, N, 2, 2), dtype=torch.uint8, device="cuda")
    dq, dk, dv = bsa.block_sparse_attention_grad(do, q, k, v, o, lse, mask, block_shape=[64, 64],
                                                 actual_seq_lengths=[S], actual_seq_lengths_kv=[S],
                                                 scale_value=1 / math.sqrt(D))
    torch.cuda.synchronize()
    q16, d16 = 0.0999755859375, 0.01000213623046875
    want_dv = S * math.exp(D * q16 * q16 / math.sqrt(D) - 5.0) * d16
    assert_close("page/dq", to_np(dq), np.zeros((B, N, S, D)), "fp16", floor_ref=want_dv)
    assert_close("page/dk", to_np(dk), np.zeros((B, N, S, D)), "fp16", floor_ref=want_dv)
    assert_close("page/dv", to_np(dv), np.full((B, N, S, D), want_dv), "fp16")


def test_convenience_call_on_a_raw_stream_handle():
    """block_sparse_attention_grad on another stream given as a raw handle: the
    workspace it allocates stays reserved for that stream's work (allocations
    made meanwhile on the current stream do not reuse it), and the result equals
    the current-stream call's bitwise."""
    import block_sparse_attention_bwd_amd as bsa
    c, o, lse, _ = _prepared("bnsd_bf16_d128_b128x128_ragged")
    dev = upload(c, o, lse)
    kw = dict(block_shape=[c.bx, c.by], actual_seq_lengths=list(map(int, c.len_q)),
              actual_seq_lengths_kv=list(map(int, c.len_kv)), layout=c.layout, num_key_value_heads=c.Nkv,
              scale_value=c.scale)
    args = (dev["do"], dev["q"], dev["k"], dev["v"], dev["o"], dev["lse"], dev["mask"])
    want = bsa.block_sparse_attention_grad(*args, **kw)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    got = bsa.block_sparse_attention_grad(*args, **kw, stream=side.cuda_stream)
    junk = [torch.full((1 << 20,), 7, dtype=torch.uint8, device="cuda") for _ in range(8)]
    torch.cuda.synchronize()
    del junk
    for x, y in zip(want, got):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("name", ["bnsd_fp16_d64_b64x128_padded", "tnd_fp16_d128_b64x128_gqa",
                                  "bnsd_bf16_d128_local_sink_split", "bnsd_bf16_d128_attenmask",
                                  "bnsd_fp16_d256_sink_split", "tnd_bf16_d64_empty_seqs"])
def test_guard_bytes_around_outputs_and_workspace(name):
    """Nothing is written outside dq, dk, dv and the workspace: guard bytes on both
    sides of each are unchanged after a call, and the results equal an unguarded call."""
    import block_sparse_attention_bwd_amd as bsa
    c, o, lse, _ = _prepared(name)
    dev = upload(c, o, lse)
    (dq, dk, dv), r = run_bsa(c, dev)
    torch.cuda.synchronize()
    want = [t.clone() for t in (dq, dk, dv)]
    outs = [_guarded(t.shape, t.dtype) for t in (dq, dk, dv)]
    ws = _guarded((r.ws_size,), torch.uint8)
    kw = dict(r.kw, dq=outs[0][0], dk=outs[1][0], dv=outs[2][0])
    bsa.bsa_bwd(*r.args, **kw, workspace=ws[0], workspace_size=r.ws_size)
    torch.cuda.synchronize()
    for (t, buf, pat), w, nm in zip(outs, want, ("dq", "dk", "dv")):
        assert _guards_intact(buf, pat), f"{name}: bytes written next to {nm}"
        assert torch.equal(t.view(torch.int16), w.view(torch.int16)), nm
    assert _guards_intact(ws[1], ws[2]), f"{name}: bytes written next to the workspace"


def _at_high_low_word(tensors):
    """Copies of `tensors` inside one 4.1 GiB buffer, each at an address whose low
    32 bits have bit 31 set (256-byte aligned, packed one after another)."""
    big = torch.empty((1 << 32) + (1 << 26), dtype=torch.uint8, device="cuda")
    base = big.data_ptr()
    off = (((1 << 31) - base % (1 << 32)) % (1 << 32) + 255) // 256 * 256
    out = []
    for t in tensors:
        n = t.numel() * t.element_size()
        assert (base + off) % (1 << 32) >= 1 << 31 and (base + off + n) % (1 << 32) > (base + off) % (1 << 32)
        v = big[off:off + n].view(t.dtype).view(t.shape)
        v.copy_(t)
        out.append(v)
        off += (n + 255) // 256 * 256
    return big, out


@pytest.mark.parametrize("name", ["bnsd_bf16_d128_local_sink_split", "tnd_fp16_d64_window_ahead"])
def test_inputs_at_addresses_with_bit31_of_the_low_word_set(name):
    """The tile copies take their wave-uniform source address from scalar
    registers, put together from two 32-bit halves; a sign-extended low half
    once turned such addresses into invalid ones.  Every input and output here
    sits at an address whose low word has bit 31 set; the results equal those
    at ordinary addresses bitwise (backward and forward)."""
    import block_sparse_attention_bwd_amd as bsa
    from bench import FwdRunner
    c, o, lse, _ = _prepared(name)
    dev = upload(c, o, lse)
    (dq, dk, dv), r = run_bsa(c, dev)
    torch.cuda.synchronize()
    want = [t.clone() for t in (dq, dk, dv)]
    keys = ["do", "q", "k", "v", "o", "lse"]
    big, moved = _at_high_low_word([dev[k] for k in keys] + [dq, dk, dv])
    d2 = dict(dev, **dict(zip(keys, moved[:6])))
    kw = dict(r.kw, dq=moved[6], dk=moved[7], dv=moved[8])
    bsa.bsa_bwd(d2["do"], d2["q"], d2["k"], d2["v"], d2["o"], d2["lse"], **kw, workspace=r.ws,
                workspace_size=r.ws_size)
    torch.cuda.synchronize()
    for got, w in zip(moved[6:], want):
        assert torch.equal(got.view(torch.int16), w.view(torch.int16))
    f = FwdRunner(c, dev)
    o_want, l_want = (t.clone() for t in f())
    torch.cuda.synchronize()
    _, (q2, k2, v2, o2, l2) = _at_high_low_word([dev["q"], dev["k"], dev["v"], f.o, f.lse])
    bsa.bsa_fwd(q2, k2, v2, **dict(f.kw, attention_out=o2, softmax_lse=l2), workspace=f.ws, workspace_size=f.ws_size)
    torch.cuda.synchronize()
    assert torch.equal(o2, o_want) and torch.equal(l2, l_want)
    del big


def test_too_small_workspace_launches_nothing():
    import block_sparse_attention_bwd_amd as bsa
    c, o, lse, _ = _prepared("config1")
    dev = upload(c, o, lse)
    (dq, dk, dv), r = run_bsa(c, dev)
    torch.cuda.synchronize()
    for t in (r.dq, r.dk, r.dv):
        t.fill_(3.0)
    with pytest.raises(bsa.BsaError) as e:
        bsa.bsa_bwd(*r.args, **r.kw, workspace=r.ws, workspace_size=r.ws_size - 1)
    assert e.value.code == bsa.BSA_ERR_PARAM_INVALID
    with pytest.raises(ValueError):
        bsa.bsa_bwd(*r.args, **r.kw, workspace=r.ws.cpu(), workspace_size=r.ws_size)
    torch.cuda.synchronize()
    for t in (r.dq, r.dk, r.dv):
        assert torch.all(t == 3.0)


# ---------------------------------------------------------------------------
# full-size workloads: whole tensors and whole block lists against the oracle
# ---------------------------------------------------------------------------
_full = {}


def _full_run(k):
    """Workload k at full size, run once in the benchmark's launch configuration:
    (case, runner, O and LSE on the host, dq/dk/dv on the host).  O and LSE come
    from a plain torch fp32 forward; the oracle and the library both take them
    as given."""
    if k not in _full:
        from bench import gpu_forward, to_device, Runner
        c = synth.config(k)
        print(f"[full] config {k}: {c.name}", flush=True)
        dev = to_device(c)
        o, lse = gpu_forward(c, dev)
        torch.cuda.synchronize()
        r = Runner(c, dev, o, lse)
        dq, dk, dv = r()
        torch.cuda.synchronize()
        _full[k] = (c, r, o.float().cpu().numpy(), lse.cpu().numpy(), (to_np(dq), to_np(dk), to_np(dv)))
    return _full[k]


@pytest.mark.parametrize("k", [2, 3, 4, 5])
def test_full_config_lists_bit_exact(k):
    """The per-Q-block and per-KV-block lists of the full workloads, every entry
    (workload 5 walks rows of 1024 KV blocks, past the 512 one sweep covers)."""
    import block_sparse_attention_bwd_amd as bsa
    c, r, _, _, _ = _full_run(k)
    offs, (bx, by, nqb, nkb) = bsa.bsa_bwd_workspace_layout(*r.args, **r.kw)
    want_rc, want_ri, want_cc, want_ci = oracle.block_list_arrays(c.mask, c.B, c.N, nqb, nkb, bx, by,
                                                                  c.len_q, c.len_kv, window=c.window)
    for cnt_name, list_name, wc, wi, n_in in (("row_cnt", "row_list", want_rc, want_ri, nqb),
                                               ("col_cnt", "col_list", want_cc, want_ci, nkb)):
        width = nkb if list_name == "row_list" else nqb
        cnt = _read_ws(r, offs, cnt_name, c.B * c.N * n_in).reshape(c.B, c.N, n_in)
        lst = _read_ws(r, offs, list_name, c.B * c.N * n_in * width).reshape(c.B, c.N, n_in, width)
        assert np.array_equal(cnt, wc), f"config{k}/{cnt_name}"
        used = np.arange(width)[None, None, None, :] < wc[..., None]
        assert np.array_equal(lst[used], wi[used]), f"config{k}/{list_name}"


@pytest.mark.parametrize("k", [2, 3, 4, 5])
def test_full_config_whole_tensors(k):
    """dQ, dK, dV of the full workloads, every element, against the oracle's
    backward on the same inputs; the bound uses max|ref| over the whole tensor."""
    c, _, o_h, lse_h, got = _full_run(k)
    t0 = time.perf_counter()
    ref = oracle_backward_threaded(c, c.q, c.k, c.v, o_h, c.do, lse_h)
    print(f"[full] config {k}: oracle backward {time.perf_counter() - t0:.1f} s", flush=True)
    for nm, g, want in zip(("dq", "dk", "dv"), got, ref):
        err, ref_max = assert_close(f"config{k}/{nm}", g, want, c.dtype)
        print(f"[full] config {k} {nm}: max err {err:.3e} = {err / ref_max:.2e} x max|ref|", flush=True)


# The measured variants of the full workloads (head dim 256, a sliding window,
# an attenMask, fp8 inputs), in the launch configuration the benchmark times,
# compared with the oracle on whole tensors like the plain workloads.
VARIANTS = ["config2_d256", "config3_window1024_0", "config2_attenmask0.1", "config2_fp8"]


def _variant(name):
    import oracle.fp8 as fp8
    from bench import gpu_forward, to_device, Runner
    k = int(name[6])
    c = synth.config(k, head_dim=256 if name.endswith("_d256") else None)
    if "window" in name:
        c.window = (1024, 0)
    if "attenmask" in name:  # drawn as bench.py --atten-mask draws it
        rng = np.random.default_rng(c.seed + 2)
        c.atten_mask = (rng.random((c.Sq, c.Skv), dtype=np.float32) < 0.1).astype(np.uint8)
    dev = to_device(c)
    o, lse = gpu_forward(c, dev)
    torch.cuda.synchronize()
    o_h = o.float().cpu().numpy()
    lse_h = lse.cpu().numpy()
    vals = dict(q=c.q, k=c.k, v=c.v, do=c.do, o=o_h)
    if not name.endswith("_fp8"):
        return c, Runner(c, dev, o, lse), vals, lse_h, c.dtype
    # fp8: E4M3FN query/key/value/attentionOut, E5M2 dout, per-tensor factors; the oracle
    # takes the dequantised values of the same codes
    fmts = dict(q=fp8.E4M3, k=fp8.E4M3, v=fp8.E4M3, o=fp8.E4M3, do=fp8.E5M2)
    tdt = {fp8.E4M3: torch.float8_e4m3fn, fp8.E5M2: torch.float8_e5m2}
    dev8, fac = dict(dev), {}
    for key in ("do", "q", "k", "v", "o"):
        codes, fac[key] = synth.quantize_fp8(vals[key], fmts[key])
        dev8[key] = torch.from_numpy(codes).cuda().view(tdt[fmts[key]])
        vals[key] = fp8.dequantize(codes, fmts[key], fac[key])
    r = Runner(c, dev8, dev8["o"], lse, descale=[fac[key] for key in ("do", "q", "k", "v", "o")])
    return c, r, vals, lse_h, "bf16"


@pytest.mark.parametrize("name", VARIANTS)
def test_full_variant_whole_tensors(name):
    print(f"[full variant] {name}", flush=True)
    _full.clear()
    c, r, vals, lse_h, tol_dtype = _variant(name)
    dq, dk, dv = r()
    torch.cuda.synchronize()
    got = (to_np(dq), to_np(dk), to_np(dv))
    del dq, dk, dv, r
    t0 = time.perf_counter()
    ref = oracle_backward_threaded(c, vals["q"], vals["k"], vals["v"], vals["o"], vals["do"], lse_h)
    print(f"[full variant] {name}: oracle backward {time.perf_counter() - t0:.1f} s", flush=True)
    for nm, g, want in zip(("dq", "dk", "dv"), got, ref):
        err, ref_max = assert_close(f"{name}/{nm}", g, want, tol_dtype)
        print(f"[full variant] {name} {nm}: max err {err:.3e} = {err / ref_max:.2e} x max|ref|", flush=True)

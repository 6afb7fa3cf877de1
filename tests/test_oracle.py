"""Pins for the fp64 oracle, checked against things other than the oracle itself.

Each test names what fixes the expected value: finite differences of the
masked forward, torch fp64 autograd (dense and element-mask special cases), a
closed form, an invariant, an identity between layouts, or a hand-worked
fixture under ``tests/golden``.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _kw(c):
    kw = dict(layout=c.layout, bx=c.bx, by=c.by, scale=c.scale)
    if c.explicit_lengths:
        kw.update(len_q=c.len_q, len_kv=c.len_kv)
    return kw


def _exact_fwd(c):
    """Unrounded fp64 forward (O, LSE) of a case."""
    return oracle.forward(c.q, c.k, c.v, c.mask, **_kw(c))


# ---------------------------------------------------------------------------
# finite differences of L(Q, K, V) = sum(dO * O(Q, K, V))
# ---------------------------------------------------------------------------
FD_CASES = [
    # GQA (2 query heads on 1 KV head), partial last blocks on both axes
    dict(layout="BNSD", dtype="bf16", B=1, N=2, Nkv=1, D=3, Sq=7, Skv=9, bx=2, by=4, p=0.6, seed=11),
    # two varlen sequences in TND, GQA
    dict(layout="TND", dtype="fp16", B=2, N=2, Nkv=1, D=3, bx=2, by=3, p=0.6,
         lengths_q=[5, 3], lengths_kv=[6, 4], seed=12),
    # padded BNSD (actual lengths shorter than S)
    dict(layout="BNSD", dtype="bf16", B=2, N=1, Nkv=1, D=2, Sq=6, Skv=7, bx=3, by=2, p=0.7,
         lengths_q=[6, 4], lengths_kv=[7, 3], seed=13),
]


@pytest.mark.parametrize("spec", FD_CASES)
def test_backward_matches_finite_differences(spec):
    c = synth.make_case(mask_rule="bernoulli_diag", scale=0.7, **spec)
    kw = _kw(c)
    o, lse = oracle.forward(c.q, c.k, c.v, c.mask, **kw)
    dq, dk, dv = oracle.backward(c.q, c.k, c.v, o, c.do, lse, c.mask, **kw)
    dof = c.do.astype(np.float64)

    def loss(q, k, v):
        oo, _ = oracle.forward(q, k, v, c.mask, **kw)
        return float(np.sum(dof * oo))

    h = 1e-6
    base = [c.q.astype(np.float64), c.k.astype(np.float64), c.v.astype(np.float64)]
    for which, grad in enumerate((dq, dk, dv)):
        x = base[which]
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            args_p = [a.copy() for a in base]
            args_m = [a.copy() for a in base]
            args_p[which][idx] += h
            args_m[which][idx] -= h
            fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        scale = max(1.0, np.abs(fd).max())
        assert np.abs(fd - grad).max() <= 1e-7 * scale, (which, np.abs(fd - grad).max())


# ---------------------------------------------------------------------------
# torch fp64 autograd: dense (all-ones / null mask) and element masks (bx=by=1)
# ---------------------------------------------------------------------------
def _torch_reference(q, k, v, do, scale, G, elem_mask=None):
    """Plain attention in torch fp64 for BNSD tensors; K/V repeated per group."""
    Q = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    K = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    V = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    Kr = K.repeat_interleave(G, dim=1)
    Vr = V.repeat_interleave(G, dim=1)
    s = scale * torch.matmul(Q, Kr.transpose(-1, -2).contiguous())
    if elem_mask is not None:
        s = s.masked_fill(~torch.tensor(elem_mask), float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    o = torch.matmul(torch.softmax(s, dim=-1), Vr)
    o.backward(torch.tensor(do, dtype=torch.float64))
    return o.detach().numpy(), lse.detach().numpy(), Q.grad.numpy(), K.grad.numpy(), V.grad.numpy()


@pytest.mark.parametrize("mask_rule", ["dense", "ones"])
def test_dense_mask_equals_torch_autograd(mask_rule):
    c = synth.make_case(layout="BNSD", dtype="bf16", B=2, N=4, Nkv=2, D=16, Sq=37, Skv=29,
                        bx=8, by=16, mask_rule=mask_rule, seed=21)
    o, lse = _exact_fwd(c)
    t_o, t_lse, t_dq, t_dk, t_dv = _torch_reference(c.q, c.k, c.v, c.do, c.scale, c.G)
    np.testing.assert_allclose(o, t_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, t_lse, rtol=0, atol=1e-12)
    dq, dk, dv = oracle.backward(c.q, c.k, c.v, o, c.do, lse, c.mask, **_kw(c))
    for a, b in ((dq, t_dq), (dk, t_dk), (dv, t_dv)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-11 * max(1.0, np.abs(b).max()))


def test_element_mask_equals_torch_masked_autograd():
    """bx = by = 1 turns the block mask into an element mask, different per query head."""
    rng = np.random.default_rng(5)
    B, N, Nkv, Sq, Skv, D = 1, 4, 2, 13, 11, 8
    m = rng.random((B, N, Sq, Skv)) < 0.4
    m[..., np.arange(Sq), np.arange(Sq) % Skv] = True  # every row keeps at least one key
    c = synth.make_case(layout="BNSD", dtype="fp16", B=B, N=N, Nkv=Nkv, D=D, Sq=Sq, Skv=Skv,
                        bx=1, by=1, mask_rule="ones", seed=22)
    c.mask = m.astype(np.uint8)
    o, lse = _exact_fwd(c)
    t_o, t_lse, t_dq, t_dk, t_dv = _torch_reference(c.q, c.k, c.v, c.do, c.scale, c.G, elem_mask=m)
    np.testing.assert_allclose(o, t_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, t_lse, rtol=0, atol=1e-12)
    dq, dk, dv = oracle.backward(c.q, c.k, c.v, o, c.do, lse, c.mask, **_kw(c))
    for a, b in ((dq, t_dq), (dk, t_dk), (dv, t_dv)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-11 * max(1.0, np.abs(b).max()))


def test_block_mask_expansion_equals_torch_with_kron_mask():
    """Block mask -> element mask by i // bx, j // by, checked via an independently expanded mask."""
    c = synth.make_case(layout="BNSD", dtype="bf16", B=1, N=2, Nkv=1, D=8, Sq=11, Skv=10,
                        bx=3, by=4, mask_rule="bernoulli_diag", p=0.5, seed=23)
    big = np.kron(c.mask, np.ones((c.bx, c.by), np.uint8))[..., :c.Sq, :c.Skv].astype(bool)
    assert big.any(axis=-1).all()
    o, lse = _exact_fwd(c)
    t_o, t_lse, t_dq, t_dk, t_dv = _torch_reference(c.q, c.k, c.v, c.do, c.scale, c.G, elem_mask=big)
    np.testing.assert_allclose(o, t_o, rtol=0, atol=1e-12)
    dq, dk, dv = oracle.backward(c.q, c.k, c.v, o, c.do, lse, c.mask, **_kw(c))
    for a, b in ((dq, t_dq), (dk, t_dk), (dv, t_dv)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-11 * max(1.0, np.abs(b).max()))


# ---------------------------------------------------------------------------
# slab evaluation == literal dense evaluation; sampled rows == full result
# ---------------------------------------------------------------------------
SLAB_CASES = [
    dict(layout="BNSD", dtype="bf16", B=2, N=4, Nkv=2, D=8, Sq=45, Skv=38, bx=8, by=16, p=0.4, seed=31),
    dict(layout="TND", dtype="fp16", B=3, N=2, Nkv=1, D=8, bx=16, by=8, p=0.3,
         lengths_q=[20, 33, 9], lengths_kv=[17, 40, 12], seed=32),
    dict(layout="BNSD", dtype="fp16", B=2, N=2, Nkv=2, D=4, Sq=30, Skv=26, bx=7, by=5, p=0.5,
         lengths_q=[30, 12], lengths_kv=[26, 9], seed=33),
]


@pytest.mark.parametrize("spec", SLAB_CASES)
def test_slab_path_equals_dense_path(spec):
    c = synth.make_case(mask_rule="bernoulli_diag", **spec)
    kw = _kw(c)
    o, lse = oracle.forward(c.q, c.k, c.v, c.mask, **kw)
    od, lsed = oracle.forward_dense(c.q, c.k, c.v, c.mask, **kw)
    np.testing.assert_allclose(o, od, rtol=0, atol=1e-13)
    np.testing.assert_array_equal(np.isinf(lse), np.isinf(lsed))
    fin = np.isfinite(lse)
    np.testing.assert_allclose(lse[fin], lsed[fin], rtol=0, atol=1e-12)
    o32 = synth.round_to_dtype(o.astype(np.float32), c.dtype)
    l32 = lse.astype(np.float32)
    a = oracle.backward(c.q, c.k, c.v, o32, c.do, l32, c.mask, **kw)
    b = oracle.backward_dense(c.q, c.k, c.v, o32, c.do, l32, c.mask, **kw)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=0, atol=1e-12 * max(1.0, np.abs(y).max()))


@pytest.mark.parametrize("spec", SLAB_CASES)
def test_sampled_rows_equal_full_backward(spec):
    c = synth.make_case(mask_rule="bernoulli_diag", **spec)
    kw = _kw(c)
    o, lse = oracle.forward(c.q, c.k, c.v, c.mask, **kw)
    o32 = synth.round_to_dtype(o.astype(np.float32), c.dtype)
    l32 = lse.astype(np.float32)
    dq, dk, dv = oracle.backward(c.q, c.k, c.v, o32, c.do, l32, c.mask, **kw)
    offq = oracle.sequence_offsets(c.len_q)
    offk = oracle.sequence_offsets(c.len_kv)
    qrows = [(b, n, i) for b in range(c.B) for n in range(c.N) for i in range(int(c.len_q[b]))]
    krows = [(b, h, j) for b in range(c.B) for h in range(c.Nkv) for j in range(int(c.len_kv[b]))]
    rq = oracle.backward_dq_rows(c.q, c.k, c.v, o32, c.do, l32, c.mask, rows=qrows, **kw)
    rk, rv = oracle.backward_dkdv_rows(c.q, c.k, c.v, o32, c.do, l32, c.mask, rows=krows, **kw)

    def at(x, b, n, r, off):
        return x[b, n, r] if c.layout == "BNSD" else x[off[b] + r, n]

    for (b, n, i), val in rq.items():
        np.testing.assert_allclose(val, at(dq, b, n, i, offq), rtol=0, atol=1e-12)
    for key in rk:
        b, h, j = key
        np.testing.assert_allclose(rk[key], at(dk, b, h, j, offk), rtol=0, atol=1e-12)
        np.testing.assert_allclose(rv[key], at(dv, b, h, j, offk), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------
def test_column_sum_invariants():
    """sum_j dK_j = 0 (rows of dS sum to zero when O and LSE are exact);
    sum_j dV_j = sum of dO over rows that select a key (rows of P sum to one)."""
    c = synth.make_case(layout="BNSD", dtype="bf16", B=2, N=4, Nkv=2, D=16, Sq=70, Skv=52,
                        bx=16, by=8, mask_rule="bernoulli_diag", p=0.3,
                        lengths_q=[70, 41], lengths_kv=[52, 30], seed=41)
    o, lse = _exact_fwd(c)
    dq, dk, dv = oracle.backward(c.q, c.k, c.v, o, c.do, lse, c.mask, **_kw(c))
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-11)
    nonempty = np.isfinite(lse)  # [B, N, Sq]
    expect = np.zeros((c.B, c.Nkv, c.D))
    for n in range(c.N):
        expect[:, n // c.G] += np.einsum("bs,bsd->bd", nonempty[:, n].astype(np.float64),
                                         c.do[:, n].astype(np.float64))
    np.testing.assert_allclose(dv.sum(axis=2), expect, atol=1e-10)
    # padded positions are zero
    assert np.all(dq[1, :, 41:] == 0) and np.all(dk[1, :, 30:] == 0) and np.all(dv[1, :, 30:] == 0)


def test_dv_invariant_holds_with_rounded_out():
    """The dV column sum needs only consistent LSE, so it survives rounding O to bf16."""
    c = synth.make_case(layout="TND", dtype="bf16", B=2, N=2, Nkv=1, D=8, bx=8, by=8,
                        mask_rule="bernoulli_diag", p=0.4, lengths_q=[30, 19], lengths_kv=[25, 33], seed=42)
    o, lse = _exact_fwd(c)
    o16 = synth.round_to_dtype(o.astype(np.float32), "bf16")
    _, _, dv = oracle.backward(c.q, c.k, c.v, o16, c.do, lse, c.mask, **_kw(c))
    offq = oracle.sequence_offsets(c.len_q)
    offk = oracle.sequence_offsets(c.len_kv)
    for b in range(c.B):
        sl = slice(offq[b], offq[b] + c.len_q[b])
        want = (np.isfinite(lse[sl])[..., None] * c.do[sl].astype(np.float64)).sum(axis=(0, 1))
        got = dv[offk[b]:offk[b] + c.len_kv[b]].sum(axis=(0, 1))
        np.testing.assert_allclose(got, want, atol=1e-10)


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------
def test_closed_form_zero_query():
    """Q = 0: P_ij = 1/n_i over row i's selected keys; dK = 0;
    dV_j = sum_i M_ij dO_i / n_i; dQ_i = (scale/n_i) sum_j M_ij (dO_i . (v_j - vbar_i)) k_j."""
    c = synth.make_case(layout="BNSD", dtype="fp16", B=1, N=2, Nkv=1, D=4, Sq=9, Skv=10,
                        bx=3, by=4, mask_rule="bernoulli_diag", p=0.5, seed=51)
    c.q[:] = 0.0
    o, lse = _exact_fwd(c)
    dq, dk, dv = oracle.backward(c.q, c.k, c.v, o, c.do, lse, c.mask, **_kw(c))
    k = c.k.astype(np.float64)[0, 0]
    v = c.v.astype(np.float64)[0, 0]
    exp_dv = np.zeros_like(v)
    for n in range(c.N):
        dO = c.do.astype(np.float64)[0, n]
        for i in range(c.Sq):
            sel = [j for j in range(c.Skv) if c.mask[0, n, i // c.bx, j // c.by]]
            ni = len(sel)
            vbar = sum(v[j] for j in sel) / ni
            want = np.zeros(c.D)
            for j in sel:
                want += (c.scale / ni) * float(dO[i] @ (v[j] - vbar)) * k[j]
                exp_dv[j] += dO[i] / ni
            np.testing.assert_allclose(dq[0, n, i], want, atol=1e-13)
    np.testing.assert_allclose(dk, 0.0, atol=1e-13)
    np.testing.assert_allclose(dv[0, 0], exp_dv, atol=1e-13)


def test_closed_form_one_key_per_row():
    """Each row keeps exactly one key (by = 1, one selected KV block per Q-block):
    P = 1 and O = v_j, so dS = 0, dQ = dK = 0 and dV_j = sum of dO over rows choosing j."""
    rng = np.random.default_rng(7)
    c = synth.make_case(layout="BNSD", dtype="bf16", B=1, N=2, Nkv=1, D=6, Sq=8, Skv=5,
                        bx=2, by=1, mask_rule="ones", seed=52)
    choice = rng.integers(0, c.Skv, size=(c.N, c.Sq // c.bx))
    m = np.zeros_like(c.mask)
    for n in range(c.N):
        for i in range(c.Sq // c.bx):
            m[0, n, i, choice[n, i]] = 1
    c.mask = m
    o, lse = _exact_fwd(c)
    dq, dk, dv = oracle.backward(c.q, c.k, c.v, o, c.do, lse, c.mask, **_kw(c))
    want = np.zeros((c.Skv, c.D))
    for n in range(c.N):
        for i in range(c.Sq):
            want[choice[n, i // c.bx]] += c.do[0, n, i]
    np.testing.assert_allclose(dq, 0.0, atol=1e-12)
    np.testing.assert_allclose(dk, 0.0, atol=1e-12)
    np.testing.assert_allclose(dv[0, 0], want, atol=1e-12)


def test_page_worked_sample_closed_form():
    """The aclnnBlockSparseAttentionGrad page's sample (调用示例): constant fp16 inputs.

    O = V and every dO row is constant, so dP_ij = dO_i . v_j equals
    softmax_grad_i = dO_i . O_i exactly: dS = 0, hence dQ = dK = 0 exactly, and
    dV_j = sum_i exp(S - 5) * 0.01 = 128 * exp(S - 5) * dout, with
    S = scale * 128 * q^2 (q, dout the fp16 roundings of 0.1 and 0.01).
    The sample's LSE (5.0) is not the true log-sum-exp, so rows of P do not sum
    to one here and no normalisation is assumed.
    """
    with open(os.path.join(GOLDEN, "page_sample.json")) as f:
        g = json.load(f)
    B, N, S, D = g["batch"], g["numHeads"], g["qSeqlen"], g["headDim"]
    bx, by = g["blockShape"]
    q16 = float(np.float16(g["query"]))
    d16 = float(np.float16(g["dout"]))
    assert q16 == 0.0999755859375 and d16 == 0.01000213623046875
    full = lambda val: np.full((B, N, S, D), np.float16(val), np.float32)
    q, k, v, o, do = full(g["query"]), full(g["key"]), full(g["value"]), full(g["attentionOut"]), full(g["dout"])
    lse = np.full(g["softmaxLseShape"], g["softmaxLse"], np.float32)
    mask = np.full(g["maskShape"], g["blockSparseMask"], np.uint8)
    scale = 1.0 / math.sqrt(D)
    dq, dk, dv = oracle.backward(q, k, v, o, do, lse, mask, layout="BNSD", bx=bx, by=by, scale=scale)
    s = scale * D * q16 * q16
    want_dv = g["kvSeqlen"] * math.exp(s - g["softmaxLse"]) * d16
    assert abs(s - 0.11308184901606315) < 1e-15
    assert np.all(dq == 0.0) and np.all(dk == 0.0)
    np.testing.assert_allclose(dv, want_dv, rtol=1e-14)


# ---------------------------------------------------------------------------
# identities between layouts and head groupings
# ---------------------------------------------------------------------------
def test_gqa_equals_mha_with_repeated_kv():
    c = synth.make_case(layout="BNSD", dtype="bf16", B=1, N=4, Nkv=2, D=8, Sq=24, Skv=20,
                        bx=8, by=4, mask_rule="bernoulli_diag", p=0.5, seed=61)
    o, lse = _exact_fwd(c)
    dq, dk, dv = oracle.backward(c.q, c.k, c.v, o, c.do, lse, c.mask, **_kw(c))
    kr = np.repeat(c.k, c.G, axis=1)
    vr = np.repeat(c.v, c.G, axis=1)
    dq2, dk2, dv2 = oracle.backward(c.q, kr, vr, o, c.do, lse, c.mask, **_kw(c))
    np.testing.assert_allclose(dq, dq2, atol=1e-13)
    np.testing.assert_allclose(dk, dk2.reshape(c.B, c.Nkv, c.G, c.Skv, c.D).sum(axis=2), atol=1e-13)
    np.testing.assert_allclose(dv, dv2.reshape(c.B, c.Nkv, c.G, c.Skv, c.D).sum(axis=2), atol=1e-13)


def test_tnd_equals_per_sequence_bnsd():
    c = synth.make_case(layout="TND", dtype="fp16", B=3, N=2, Nkv=1, D=8, bx=4, by=8,
                        mask_rule="bernoulli_diag", p=0.5, lengths_q=[9, 20, 5],
                        lengths_kv=[16, 11, 8], seed=62)
    o, lse = _exact_fwd(c)
    dq, dk, dv = oracle.backward(c.q, c.k, c.v, o, c.do, lse, c.mask, **_kw(c))
    offq, offk = oracle.sequence_offsets(c.len_q), oracle.sequence_offsets(c.len_kv)
    for b in range(c.B):
        lq, lk = int(c.len_q[b]), int(c.len_kv[b])
        sq = lambda x: x[offq[b]:offq[b] + lq].transpose(1, 0, 2)[None]
        sk = lambda x: x[offk[b]:offk[b] + lk].transpose(1, 0, 2)[None]
        mb = c.mask[b:b + 1, :, :-(-lq // c.bx), :-(-lk // c.by)]
        ob, lb = oracle.forward(sq(c.q), sk(c.k), sk(c.v), mb, layout="BNSD", bx=c.bx, by=c.by, scale=c.scale)
        np.testing.assert_allclose(ob, sq(o), atol=1e-13)
        g = oracle.backward(sq(c.q), sk(c.k), sk(c.v), ob, sq(c.do), lb, mb, layout="BNSD",
                            bx=c.bx, by=c.by, scale=c.scale)
        np.testing.assert_allclose(g[0], sq(dq), atol=1e-13)
        np.testing.assert_allclose(g[1], sk(dk), atol=1e-13)
        np.testing.assert_allclose(g[2], sk(dv), atol=1e-13)


def test_padded_bnsd_equals_truncated_bnsd():
    c = synth.make_case(layout="BNSD", dtype="bf16", B=2, N=2, Nkv=2, D=8, Sq=24, Skv=21,
                        bx=8, by=4, mask_rule="bernoulli_diag", p=0.5, lengths_q=[24, 13],
                        lengths_kv=[21, 10], seed=63)
    c.q[1, :, 13:] = 1e3  # garbage in the padding must not leak
    c.k[1, :, 10:] = -1e3
    o, lse = _exact_fwd(c)
    dq, dk, dv = oracle.backward(c.q, c.k, c.v, o, c.do, lse, c.mask, **_kw(c))
    b = 1
    mb = c.mask[b:b + 1, :, :2, :3]
    sl = lambda x, L: x[b:b + 1, :, :L]
    ob, lb = oracle.forward(sl(c.q, 13), sl(c.k, 10), sl(c.v, 10), mb, layout="BNSD", bx=8, by=4, scale=c.scale)
    g = oracle.backward(sl(c.q, 13), sl(c.k, 10), sl(c.v, 10), ob, sl(c.do, 13), lb, mb,
                        layout="BNSD", bx=8, by=4, scale=c.scale)
    np.testing.assert_allclose(g[0], sl(dq, 13), atol=1e-13)
    np.testing.assert_allclose(g[1], sl(dk, 10), atol=1e-13)
    np.testing.assert_allclose(g[2], sl(dv, 10), atol=1e-13)
    assert np.all(dq[1, :, 13:] == 0) and np.all(dk[1, :, 10:] == 0) and np.all(dv[1, :, 10:] == 0)


# ---------------------------------------------------------------------------
# block lists
# ---------------------------------------------------------------------------
def test_block_lists_hand_worked_example():
    with open(os.path.join(GOLDEN, "block_lists_tiny.json")) as f:
        g = json.load(f)
    mask = np.array(g["mask"], np.uint8)
    nqb, nkb = mask.shape[2], mask.shape[3]
    rows, cols = oracle.block_lists(mask, g["B"], g["N"], nqb, nkb, g["bx"], g["by"], g["len_q"], g["len_kv"])
    assert rows == g["rows"]
    assert cols == g["cols"]
    em = oracle.element_mask(mask[1, 0], g["bx"], g["by"], g["len_q"][1], g["len_kv"][1])
    np.testing.assert_array_equal(em, np.array(g["element_mask_b1_n0"], bool))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_block_lists_properties(seed):
    rng = np.random.default_rng(seed)
    B, N, bx, by = 3, 2, 5, 3
    lq = rng.integers(1, 40, size=B)
    lk = rng.integers(1, 40, size=B)
    nqb, nkb = -(-int(lq.max()) // bx), -(-int(lk.max()) // by)
    mask = (rng.random((B, N, nqb, nkb)) < 0.4).astype(np.uint8)
    rows, cols = oracle.block_lists(mask, B, N, nqb, nkb, bx, by, lq, lk)
    pairs_r = set()
    pairs_c = set()
    for b in range(B):
        for n in range(N):
            for i in range(nqb):
                assert rows[b][n][i] == sorted(set(rows[b][n][i]))
                pairs_r |= {(b, n, i, j) for j in rows[b][n][i]}
            for j in range(nkb):
                assert cols[b][n][j] == sorted(set(cols[b][n][j]))
                pairs_c |= {(b, n, i, j) for i in cols[b][n][j]}
    assert pairs_r == pairs_c
    # the listed pairs are exactly the nonzero, in-range mask entries
    want = set()
    for (b, n, i, j) in zip(*np.nonzero(mask)):
        if i * bx < lq[b] and j * by < lk[b]:
            want.add((int(b), int(n), int(i), int(j)))
    assert pairs_r == want


def test_null_mask_is_dense():
    c = synth.make_case(layout="BNSD", dtype="bf16", B=1, N=2, Nkv=1, D=8, Sq=20, Skv=17,
                        bx=8, by=4, mask_rule="dense", seed=71)
    assert c.mask is None
    o, lse = _exact_fwd(c)
    ones = np.ones((1, 2, 3, 5), np.uint8)
    o2, lse2 = oracle.forward(c.q, c.k, c.v, ones, **_kw(c))
    np.testing.assert_array_equal(o, o2)
    g1 = oracle.backward(c.q, c.k, c.v, o, c.do, lse, None, **_kw(c))
    g2 = oracle.backward(c.q, c.k, c.v, o, c.do, lse, ones, **_kw(c))
    for a, b in zip(g1, g2):
        np.testing.assert_array_equal(a, b)


# ---------------------------------------------------------------------------
# rows of P sum to one and rows of dS to zero (the P and dS the backward contracts)
# ---------------------------------------------------------------------------
ROW_CASES = [
    dict(layout="BNSD", dtype="bf16", B=2, N=4, Nkv=2, D=16, Sq=70, Skv=90, bx=16, by=32, p=0.5, seed=21),
    dict(layout="TND", dtype="fp16", B=2, N=2, Nkv=1, D=8, bx=8, by=16, p=0.6, lengths_q=[40, 23],
         lengths_kv=[50, 31], seed=22),
    dict(layout="BNSD", dtype="bf16", B=1, N=2, Nkv=1, D=8, Sq=60, Skv=60, bx=16, by=16, p=0.8,
         window=(10, 3), seed=23),
]


def _heads(c, o, lse):
    """Per (b, n): the head's q, o, do, lse rows and its KV head's k, v (sequence-local)."""
    offq, offk = oracle.sequence_offsets(c.len_q), oracle.sequence_offsets(c.len_kv)
    G = c.N // c.Nkv
    for b in range(c.B):
        lq, lk = int(c.len_q[b]), int(c.len_kv[b])
        for n in range(c.N):
            h = n // G
            if c.layout == "BNSD":
                qs, os_, dos, ls = c.q[b, n, :lq], o[b, n, :lq], c.do[b, n, :lq], lse[b, n, :lq]
                ks, vs = c.k[b, h, :lk], c.v[b, h, :lk]
            else:
                sl = slice(offq[b], offq[b] + lq)
                qs, os_, dos, ls = c.q[sl, n], o[sl, n], c.do[sl, n], lse[sl, n]
                ks, vs = c.k[offk[b]:offk[b] + lk, h], c.v[offk[b]:offk[b] + lk, h]
            yield b, n, qs, ks, vs, os_, dos, ls


@pytest.mark.parametrize("spec", ROW_CASES, ids=["bnsd_gqa", "tnd", "window"])
@pytest.mark.parametrize("with_amask", [False, True])
def test_ds_rows_sum_to_zero(spec, with_amask):
    """sum_j dS_ij = delta_i - delta_i * sum_j P_ij = 0 when O and LSE are the exact forward
    (sum_j P_ij dP_ij = dO_i . O_i = delta_i): a wrong delta, P or dS fails it."""
    c = synth.make_case(**spec)
    amask = None
    if with_amask:
        rng = np.random.default_rng(spec["seed"])
        sq, sk = int(c.len_q.max()), int(c.len_kv.max())
        amask = (rng.random((sq, sk)) < 0.3).astype(np.uint8)
    kw = dict(_kw(c), window=c.window, atten_mask=amask)
    if c.layout == "TND":
        kw.update(len_q=c.len_q, len_kv=c.len_kv)
    o, lse = oracle.forward(c.q, c.k, c.v, c.mask, **kw)
    n_rows = 0
    for b, n, qs, ks, vs, os_, dos, ls in _heads(c, o, lse):
        P, dS = oracle.head_probs_and_ds(qs, ks, vs, os_, dos, ls, c.mask[b, n], bx=c.bx, by=c.by, scale=c.scale,
                                         window=c.window, atten_mask=amask)
        mag = np.abs(dS).sum(axis=1)
        assert np.all(np.abs(dS.sum(axis=1)) <= 1e-12 * mag + 1e-300), (b, n)
        n_rows += int((mag > 0).sum())
    assert n_rows > 0


@pytest.mark.parametrize("spec", ROW_CASES, ids=["bnsd_gqa", "tnd", "window"])
def test_p_rows_sum_to_one_with_fp32_lse(spec):
    """With the LSE of the oracle forward rounded to fp32 (as the kernels receive it),
    every row that selects a key has sum_j P_ij = exp(LSE_exact - LSE_fp32) = 1 within
    4 * 2^-24 * max(1, |LSE_i|); rows that select none (LSE = -inf) have P = 0."""
    c = synth.make_case(**spec)
    kw = dict(_kw(c), window=c.window)
    if c.layout == "TND":
        kw.update(len_q=c.len_q, len_kv=c.len_kv)
    o, lse = oracle.forward(c.q, c.k, c.v, c.mask, **kw)
    lse32 = lse.astype(np.float32).astype(np.float64)
    for b, n, qs, ks, vs, os_, dos, ls in _heads(c, o, lse32):
        P, _ = oracle.head_probs_and_ds(qs, ks, vs, os_, dos, ls, c.mask[b, n], bx=c.bx, by=c.by, scale=c.scale,
                                        window=c.window)
        fin = np.isfinite(ls)
        rs = P.sum(axis=1)
        assert np.all(np.abs(rs[fin] - 1.0) <= 4 * 2.0 ** -24 * np.maximum(1.0, np.abs(ls[fin]))), (b, n)
        assert np.all(rs[~fin] == 0.0)


@pytest.mark.parametrize("seed,window", [(0, None), (1, None), (2, (5, 0)), (3, (-2, 7)), (4, (0, -3))])
def test_block_list_arrays_match_brute_force(seed, window):
    """The whole-array form of the list rule (used on full-size problems) gives
    exactly the brute-force lists: counts, and the first `count` entries of each row."""
    rng = np.random.default_rng(100 + seed)
    B, N, bx, by = 3, 2, int(rng.integers(1, 6)), int(rng.integers(1, 6))
    lq = rng.integers(0, 40, size=B)
    lk = rng.integers(0, 40, size=B)
    lq[0], lk[0] = 37, 39  # at least one long sequence
    nqb, nkb = -(-int(lq.max()) // bx), -(-int(lk.max()) // by)
    mask = (rng.random((B, N, nqb, nkb)) < 0.45).astype(np.uint8)
    rows, cols = oracle.block_lists(mask, B, N, nqb, nkb, bx, by, lq, lk, window=window)
    rc, ri, cc, ci = oracle.block_list_arrays(mask, B, N, nqb, nkb, bx, by, lq, lk, window=window)
    for b in range(B):
        for n in range(N):
            for i in range(nqb):
                assert rc[b, n, i] == len(rows[b][n][i])
                assert ri[b, n, i, :rc[b, n, i]].tolist() == rows[b][n][i]
            for j in range(nkb):
                assert cc[b, n, j] == len(cols[b][n][j])
                assert ci[b, n, j, :cc[b, n, j]].tolist() == cols[b][n][j]


def test_block_list_arrays_null_mask_and_long_rows():
    """No mask selects every in-range block; rows longer than 512 blocks (by = 1)."""
    B, N, bx, by = 2, 1, 64, 1
    lq, lk = np.array([130, 64]), np.array([600, 517])
    nqb, nkb = 3, 600
    rows, cols = oracle.block_lists(None, B, N, nqb, nkb, bx, by, lq, lk)
    rc, ri, cc, ci = oracle.block_list_arrays(None, B, N, nqb, nkb, bx, by, lq, lk)
    assert rc[0, 0].tolist() == [600, 600, 600] and rc[1, 0].tolist() == [517, 0, 0]
    assert ri[0, 0, 2, :600].tolist() == list(range(600)) == rows[0][0][2]
    assert cc[1, 0, :517].tolist() == [1] * 517 and cc[1, 0, 517:].tolist() == [0] * 83
    assert all(ci[1, 0, j, :1].tolist() == cols[1][0][j] for j in range(517))


@pytest.mark.parametrize("layout", ["BNSD", "TND"])
def test_piecewise_threaded_backward_equals_whole(layout):
    """The full-size parity tests and the CPU baseline run the oracle on
    (sequence, KV head) pieces in threads; put back together the pieces are
    bitwise the whole-problem result (same arithmetic, same order per head)."""
    from gpu_common import oracle_backward_threaded
    kw = dict(layout=layout, dtype="bf16", B=3, N=4, Nkv=2, D=16, bx=8, by=16, p=0.5, seed=77)
    if layout == "TND":
        kw.update(lengths_q=[40, 0, 23], lengths_kv=[30, 17, 50])
    else:
        kw.update(Sq=40, Skv=50, lengths_q=[40, 11, 30], lengths_kv=[50, 20, 1])
    c = synth.make_case(**kw)
    c.window = (20, 3)
    okw = dict(layout=c.layout, bx=c.bx, by=c.by, scale=c.scale, window=c.window, len_q=c.len_q, len_kv=c.len_kv)
    o, lse = oracle.forward(c.q, c.k, c.v, c.mask, **okw)
    whole = oracle.backward(c.q, c.k, c.v, o, c.do, lse, c.mask, **okw)
    parts = oracle_backward_threaded(c, c.q, c.k, c.v, o, c.do, lse, workers=4)
    for a, b in zip(whole, parts):
        assert np.array_equal(a, b)

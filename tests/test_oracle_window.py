"""Pins for the oracle's sliding window (preTokens / nextTokens), checked
against things other than the oracle's own window code: finite differences
of the windowed forward, torch fp64 autograd on an explicitly built element
mask, a closed form (a zero-width window), the dense twin, an interval
formula for the block lists, and the row-sampled helpers."""
import numpy as np
import pytest
import torch

import oracle
import synth

from test_oracle import _kw, _torch_reference


def _band(lq, lk, pre, nxt):
    """The window as an explicit [lq, lk] matrix, written out independently."""
    m = np.zeros((lq, lk), dtype=bool)
    for i in range(lq):
        for j in range(lk):
            m[i, j] = (i - pre) <= j <= (i + nxt)
    return m


@pytest.mark.parametrize("window", [(2, 1), (0, 3), (-1, 3)])
def test_window_backward_matches_finite_differences(window):
    c = synth.make_case(layout="BNSD", dtype="bf16", B=1, N=2, Nkv=1, D=3, Sq=7, Skv=9, bx=2, by=4,
                        p=0.7, mask_rule="bernoulli_diag", scale=0.7, seed=111)
    kw = dict(_kw(c), window=window)
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
            ap = [a.copy() for a in base]
            am = [a.copy() for a in base]
            ap[which][idx] += h
            am[which][idx] -= h
            fd[idx] = (loss(*ap) - loss(*am)) / (2 * h)
        assert np.abs(fd - grad).max() <= 1e-7 * max(1.0, np.abs(fd).max()), (window, which)


def test_window_equals_torch_autograd_with_explicit_mask():
    """Block mask (expanded by hand) and the window (written out) as one element mask in torch."""
    B, N, Nkv, Sq, Skv, D, bx, by, pre, nxt = 1, 4, 2, 19, 23, 8, 4, 8, 5, 2
    c = synth.make_case(layout="BNSD", dtype="fp16", B=B, N=N, Nkv=Nkv, D=D, Sq=Sq, Skv=Skv, bx=bx,
                        by=by, mask_rule="ones", seed=112)
    rng = np.random.default_rng(3)
    c.mask = (rng.random(c.mask.shape) < 0.7).astype(np.uint8)
    c.mask[..., np.arange(c.mask.shape[2]), (np.arange(c.mask.shape[2]) * bx) // by] = 1  # diagonal blocks on
    em = np.zeros((B, N, Sq, Skv), dtype=bool)
    for n in range(N):
        em[0, n] = np.kron(c.mask[0, n], np.ones((bx, by), dtype=np.uint8))[:Sq, :Skv].astype(bool)
    em &= _band(Sq, Skv, pre, nxt)[None, None]
    assert em.any(axis=-1).all()  # every row keeps a key (its own position), so torch is defined
    kw = dict(_kw(c), window=(pre, nxt))
    o, lse = oracle.forward(c.q, c.k, c.v, c.mask, **kw)
    t_o, t_lse, t_dq, t_dk, t_dv = _torch_reference(c.q, c.k, c.v, c.do, c.scale, c.G, elem_mask=em)
    np.testing.assert_allclose(o, t_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, t_lse, rtol=0, atol=1e-12)
    dq, dk, dv = oracle.backward(c.q, c.k, c.v, o, c.do, lse, c.mask, **kw)
    for a, b in ((dq, t_dq), (dk, t_dk), (dv, t_dv)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-11 * max(1.0, np.abs(b).max()))


def test_zero_width_window_closed_form():
    """preTokens = nextTokens = 0: each query sees only its own position, so P = 1
    there: O_i = v_i, LSE_i = scale * q_i . k_i, dS = 0 (dQ = dK = 0) and dV_j = dO_j."""
    c = synth.make_case(layout="BNSD", dtype="bf16", B=2, N=2, Nkv=2, D=8, Sq=12, Skv=12, bx=4, by=4,
                        mask_rule="ones", seed=113)
    kw = dict(_kw(c), window=(0, 0))
    o, lse = oracle.forward(c.q, c.k, c.v, c.mask, **kw)
    q, k, v, do = (x.astype(np.float64) for x in (c.q, c.k, c.v, c.do))
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, c.scale * np.sum(q * k, axis=-1), rtol=0, atol=1e-13)
    dq, dk, dv = oracle.backward(c.q, c.k, c.v, o, c.do, lse, c.mask, **kw)
    assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13
    np.testing.assert_allclose(dv, do, rtol=0, atol=1e-14)


WINDOWS = [(0, 0), (2, 1), (-2, 4), (5, -3), (40, 40), (3, 0), (2, -4)]


@pytest.mark.parametrize("window", WINDOWS)
def test_window_slab_path_equals_dense_path(window):
    """Including windows that leave rows with no key (LSE = -inf, O = dQ = 0)."""
    c = synth.make_case(layout="TND", dtype="fp16", B=2, N=2, Nkv=1, D=6, bx=3, by=4, p=0.6,
                        lengths_q=[11, 7], lengths_kv=[9, 13], mask_rule="bernoulli", seed=114)
    kw = dict(_kw(c), len_q=c.len_q, len_kv=c.len_kv, window=window)
    o, lse = oracle.forward(c.q, c.k, c.v, c.mask, **kw)
    od, lsed = oracle.forward_dense(c.q, c.k, c.v, c.mask, **kw)
    np.testing.assert_allclose(o, od, rtol=0, atol=1e-13)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lsed))
    fin = np.isfinite(lse)
    np.testing.assert_allclose(lse[fin], lsed[fin], rtol=0, atol=1e-13)
    g = oracle.backward(c.q, c.k, c.v, o, c.do, lse, c.mask, **kw)
    gd = oracle.backward_dense(c.q, c.k, c.v, o, c.do, lse, c.mask, **kw)
    for a, b in zip(g, gd):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12 * max(1.0, np.abs(b).max()))
    # rows left no key have zero output and dQ
    empty = np.isneginf(lse)
    assert np.all(o[empty] == 0) and np.all(g[0][empty] == 0)


@pytest.mark.parametrize("window", WINDOWS)
def test_window_block_lists_follow_the_interval_rule(window):
    """A selected in-range block is listed iff the differences j - i over its clipped
    rectangle, the integer range [c0 - (r1 - 1), (c1 - 1) - r0], meet [-pre, nxt]
    (which is empty when pre + nxt < 0: then nothing is listed)."""
    rng = np.random.default_rng(7)
    B, N, bx, by = 2, 2, 3, 4
    lq, lk = np.array([17, 9]), np.array([13, 21])
    nqb, nkb = -(-int(lq.max()) // bx), -(-int(lk.max()) // by)
    mask = (rng.random((B, N, nqb, nkb)) < 0.6).astype(np.uint8)
    rows, cols = oracle.block_lists(mask, B, N, nqb, nkb, bx, by, lq, lk, window=window)
    pre, nxt = window
    for b in range(B):
        for n in range(N):
            for i in range(nqb):
                want = []
                for j in range(nkb):
                    if not mask[b, n, i, j] or i * bx >= lq[b] or j * by >= lk[b]:
                        continue
                    r0, r1 = i * bx, min(i * bx + bx, int(lq[b]))
                    c0, c1 = j * by, min(j * by + by, int(lk[b]))
                    if c0 - (r1 - 1) <= nxt and (c1 - 1) - r0 >= -pre and -pre <= nxt:
                        want.append(j)
                assert rows[b][n][i] == want, (b, n, i)
            for j in range(nkb):
                assert cols[b][n][j] == [i for i in range(nqb) if j in rows[b][n][i]]


@pytest.mark.parametrize("window", [(2, 1), (5, -3)])
def test_window_sampled_rows_equal_full_backward(window):
    c = synth.make_case(layout="BNSD", dtype="bf16", B=1, N=4, Nkv=2, D=8, Sq=20, Skv=18, bx=4, by=6,
                        p=0.6, seed=115)
    kw = dict(_kw(c), window=window)
    o, lse = oracle.forward(c.q, c.k, c.v, c.mask, **kw)
    dq, dk, dv = oracle.backward(c.q, c.k, c.v, o, c.do, lse, c.mask, **kw)
    rq = [(0, n, i) for n in range(4) for i in range(20)]
    got = oracle.backward_dq_rows(c.q, c.k, c.v, o, c.do, lse, c.mask, rows=rq, **kw)
    for (b, n, i), r in got.items():
        np.testing.assert_allclose(r, dq[b, n, i], rtol=0, atol=1e-13)
    rk = [(0, h, j) for h in range(2) for j in range(18)]
    gk, gv = oracle.backward_dkdv_rows(c.q, c.k, c.v, o, c.do, lse, c.mask, rows=rk, **kw)
    for (b, h, j) in rk:
        np.testing.assert_allclose(gk[(b, h, j)], dk[b, h, j], rtol=0, atol=1e-13)
        np.testing.assert_allclose(gv[(b, h, j)], dv[b, h, j], rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------
# attenMask (1 = the pair does not take part), alone and with a window
# ---------------------------------------------------------------------------
def _atten(rng, sq, sk, p=0.3):
    return (rng.random((sq, sk)) < p).astype(np.uint8)


@pytest.mark.parametrize("window", [None, (4, 3)])
def test_atten_mask_equals_torch_autograd_with_explicit_mask(window):
    B, N, Nkv, Sq, Skv, D, bx, by = 1, 2, 1, 17, 21, 8, 4, 8
    c = synth.make_case(layout="BNSD", dtype="bf16", B=B, N=N, Nkv=Nkv, D=D, Sq=Sq, Skv=Skv, bx=bx, by=by,
                        mask_rule="ones", seed=121)
    rng = np.random.default_rng(9)
    am = _atten(rng, Sq, Skv)
    am[np.arange(Sq), np.arange(Sq)] = 0  # keep each row's own position, so torch's softmax is defined
    em = np.ones((B, N, Sq, Skv), dtype=bool) & (am == 0)[None, None]
    if window is not None:
        em &= _band(Sq, Skv, *window)[None, None]
    assert em.any(axis=-1).all()
    kw = dict(_kw(c), window=window, atten_mask=am)
    o, lse = oracle.forward(c.q, c.k, c.v, c.mask, **kw)
    t_o, t_lse, t_dq, t_dk, t_dv = _torch_reference(c.q, c.k, c.v, c.do, c.scale, c.G, elem_mask=em)
    np.testing.assert_allclose(o, t_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, t_lse, rtol=0, atol=1e-12)
    dq, dk, dv = oracle.backward(c.q, c.k, c.v, o, c.do, lse, c.mask, **kw)
    for a, b in ((dq, t_dq), (dk, t_dk), (dv, t_dv)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-11 * max(1.0, np.abs(b).max()))


def test_atten_mask_finite_differences():
    c = synth.make_case(layout="TND", dtype="fp16", B=2, N=2, Nkv=1, D=3, bx=2, by=3, p=0.7,
                        lengths_q=[5, 4], lengths_kv=[6, 5], scale=0.7, seed=122)
    am = _atten(np.random.default_rng(4), 5, 6, 0.4)
    kw = dict(layout=c.layout, bx=c.bx, by=c.by, scale=c.scale, len_q=c.len_q, len_kv=c.len_kv,
              atten_mask=am, window=(3, 2))
    o, lse = oracle.forward(c.q, c.k, c.v, c.mask, **kw)
    dq, dk, dv = oracle.backward(c.q, c.k, c.v, o, c.do, lse, c.mask, **kw)
    dof = c.do.astype(np.float64)
    h = 1e-6
    base = [c.q.astype(np.float64), c.k.astype(np.float64), c.v.astype(np.float64)]
    for which, grad in enumerate((dq, dk, dv)):
        x = base[which]
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            ap = [a.copy() for a in base]
            am_ = [a.copy() for a in base]
            ap[which][idx] += h
            am_[which][idx] -= h
            fd[idx] = (float(np.sum(dof * oracle.forward(*ap, c.mask, **kw)[0]))
                       - float(np.sum(dof * oracle.forward(*am_, c.mask, **kw)[0]))) / (2 * h)
        assert np.abs(fd - grad).max() <= 1e-7 * max(1.0, np.abs(fd).max()), which


def test_atten_mask_slab_equals_dense_and_rows():
    """Including rows the attenMask empties (LSE = -inf, zero O and dQ)."""
    c = synth.make_case(layout="BNSD", dtype="bf16", B=1, N=4, Nkv=2, D=8, Sq=20, Skv=18, bx=4, by=6,
                        p=0.6, seed=123)
    am = _atten(np.random.default_rng(5), 20, 18, 0.5)
    am[3, :] = 1  # row 3 loses every key
    kw = dict(_kw(c), atten_mask=am)
    o, lse = oracle.forward(c.q, c.k, c.v, c.mask, **kw)
    od, lsed = oracle.forward_dense(c.q, c.k, c.v, c.mask, **kw)
    np.testing.assert_allclose(o, od, rtol=0, atol=1e-13)
    assert np.all(np.isneginf(lse[:, :, 3])) and np.all(o[:, :, 3] == 0)
    g = oracle.backward(c.q, c.k, c.v, o, c.do, lse, c.mask, **kw)
    gd = oracle.backward_dense(c.q, c.k, c.v, o, c.do, lse, c.mask, **kw)
    for a, b in zip(g, gd):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12 * max(1.0, np.abs(b).max()))
    rq = [(0, n, i) for n in range(4) for i in range(20)]
    got = oracle.backward_dq_rows(c.q, c.k, c.v, o, c.do, lse, c.mask, rows=rq, **kw)
    for (b, n, i), r in got.items():
        np.testing.assert_allclose(r, g[0][b, n, i], rtol=0, atol=1e-13)
    rk = [(0, h, j) for h in range(2) for j in range(18)]
    gk, gv = oracle.backward_dkdv_rows(c.q, c.k, c.v, o, c.do, lse, c.mask, rows=rk, **kw)
    for (b, h, j) in rk:
        np.testing.assert_allclose(gk[(b, h, j)], g[1][b, h, j], rtol=0, atol=1e-13)
        np.testing.assert_allclose(gv[(b, h, j)], g[2][b, h, j], rtol=0, atol=1e-13)

"""CPU fp64 oracle for the block-sparse attention backward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
executes this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` do.  It shares no code with the HIP path
(no kernels, headers, helpers or tables); the only thing both sides share is
the seeded input generator, which holds none of the method's arithmetic.

Source of the definition: the aclnnBlockSparseAttentionGrad page
("CANN/ops-transformer块稀疏注意力梯度算子"):

* 功能说明, 计算公式 -- forward:  S = Mask(scale*Q*K_sparse^T),  P = Softmax(S),
  Out = P*V_sparse;  backward: softmax_grad = softmaxGrad(dOut, attentionOut),
  dP = dOut*V^T,  dS = P*(dP - softmax_grad),  dV = P^T*dOut,
  dQ = (dS*K)*scale,  dK = (dS^T*Q)*scale.
* 参数说明 (blockSparseMaskOptional) -- mask [B, N, ceil(maxSq/bx),
  ceil(maxSkv/by)]; 1 = the block takes part, 0 = it is skipped; a null mask
  means every token pair is computed.
* 参数说明 (blockShapeOptional) -- block [bx, by] along Q and KV, default
  [128, 128].
* 参数说明 (actualSeqLengths[Kv]Optional) -- per-batch valid token counts;
  required for TND; for BNSD the padding past them is ignored.
* 约束说明 -- N1 >= N2, N1 % N2 == 0 (GQA).

Readings taken where the page is silent or garbled (each also listed in the
design notes):

* ``*`` is a matrix product except in dS, where it is element-wise (shapes
  decide).
* softmax_grad(dOut, attentionOut) is the row sum ``delta_i = sum_d dO_id*O_id``
  of the given O (the softmax-Jacobian identity).
* softmaxLse is the natural-log log-sum-exp of the scaled scores over the
  selected valid keys, so ``P_ij = exp(S_ij - LSE_i)`` on selected entries.
* query head n uses KV head ``n // (N // Nkv)`` (contiguous groups); the mask's
  head index is the query head.
* block (i, j) covers sequence-local rows [i*bx, (i+1)*bx) and columns
  [j*by, (j+1)*by), clipped to the sequence's lengths; TND tokens of sequence
  b start at the sum of the previous sequences' lengths.
* outputs at padded BNSD positions, rows with no selected key (dQ) and keys
  no row selects (dK, dV) are zero.
* sliding window (参数说明 preTokens / nextTokens: how many earlier and later
  tokens the current token may attend to): with ``window = (pre, nxt)`` key j
  takes part for query i only if ``i - pre <= j <= i + nxt``, both positions
  sequence-local and counted from 0; ``None`` (2147483647 for both) means no
  window.  A block stays in the lists only if the block mask selects it and at
  least one of its in-range elements lies in the window.  A query row that
  the window leaves no key has LSE = -inf and zero O and dQ.
* attenMask (参数说明 attenMaskOptional, BOOL, 2 dims; the FlashAttentionScore
  page's polarity, 1 = the pair does not take part): ``atten_mask`` is
  ``[maxSq, maxSkv]``, shared by every batch and head and indexed by
  sequence-local positions; it removes pairs without changing the block lists.

Everything is computed in float64 from the exact input values (fp16/bf16
values upcast, the given fp32 LSE upcast).  The work is organised per
(batch, query head) and per Q-block slab: inside one slab every row selects the
same column set, so the slab's element mask restricted to those columns is all
true and the definition is evaluated on that dense sub-matrix.  ``*_dense``
functions evaluate the same definition literally on the full ``[Sq, Skv]``
element mask, for tiny shapes.
"""
from __future__ import annotations

from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "sequence_offsets",
    "in_window",
    "allowed_pairs",
    "element_mask",
    "block_lists",
    "block_list_arrays",
    "softmax_grad",
    "head_probs_and_ds",
    "forward",
    "backward",
    "forward_dense",
    "backward_dense",
    "backward_dq_rows",
    "backward_dkdv_rows",
]


# ---------------------------------------------------------------------------
# layout helpers
# ---------------------------------------------------------------------------
def sequence_offsets(lengths: Sequence[int]) -> np.ndarray:
    """TND token offset of each sequence: the sum of the earlier lengths."""
    lengths = np.asarray(lengths, np.int64)
    out = np.zeros(len(lengths), np.int64)
    if len(lengths) > 1:
        out[1:] = np.cumsum(lengths)[:-1]
    return out


def _seq(x: np.ndarray, layout: str, b: int, length: int, off: int) -> np.ndarray:
    """Per-sequence view [heads, length, D] of a BNSD or TND tensor, as float64."""
    if layout == "BNSD":
        return np.asarray(x[b, :, :length, :], dtype=np.float64)
    return np.asarray(x[off:off + length], dtype=np.float64).transpose(1, 0, 2)


def _seq_lse(lse: np.ndarray, layout: str, b: int, length: int, off: int) -> np.ndarray:
    """Per-sequence LSE [N, length] (a trailing size-1 axis is accepted)."""
    lse = np.asarray(lse, dtype=np.float64)
    if layout == "BNSD":
        if lse.ndim == 4:
            lse = lse[..., 0]
        return lse[b, :, :length]
    if lse.ndim == 3:
        lse = lse[..., 0]
    return lse[off:off + length].T


def _put(out: np.ndarray, val: np.ndarray, layout: str, b: int, length: int, off: int):
    if layout == "BNSD":
        out[b, :, :length, :] = val
    else:
        out[off:off + length] = val.transpose(1, 0, 2)


def _put_lse(out: np.ndarray, val: np.ndarray, layout: str, b: int, length: int, off: int):
    if layout == "BNSD":
        out[b, :, :length] = val
    else:
        out[off:off + length] = val.T


# ---------------------------------------------------------------------------
# mask: block mask -> element mask, and the per-block lists
# ---------------------------------------------------------------------------
def in_window(rows: np.ndarray, cols: np.ndarray, window) -> np.ndarray:
    """[len(rows), len(cols)] bool: query position i may see key position j,
    i.e. ``i - pre <= j <= i + nxt`` for ``window = (pre, nxt)``; all true for None."""
    rows = np.asarray(rows, np.int64)
    cols = np.asarray(cols, np.int64)
    if window is None:
        return np.ones((rows.size, cols.size), dtype=bool)
    pre, nxt = window
    d = cols[None, :] - rows[:, None]
    return (d >= -pre) & (d <= nxt)


def allowed_pairs(rows, cols, window=None, atten_mask=None) -> np.ndarray:
    """[len(rows), len(cols)] bool: pairs the window and the attenMask leave in."""
    ok = in_window(rows, cols, window)
    if atten_mask is not None:
        ok &= np.asarray(atten_mask)[np.ix_(np.asarray(rows, np.int64), np.asarray(cols, np.int64))] == 0
    return ok


def element_mask(block_mask_bn: Optional[np.ndarray], bx: int, by: int, lq: int, lkv: int,
                 window=None, atten_mask=None) -> np.ndarray:
    """Element mask [lq, lkv] of one (batch, head): M[i, j] = mask[i // bx, j // by] != 0,
    (i, j) in the window, and atten_mask[i, j] == 0.

    ``None`` (no block mask) selects every pair.  Rows and columns past the
    sequence's lengths do not exist in the result.
    """
    if block_mask_bn is None:
        m = np.ones((lq, lkv), dtype=bool)
    else:
        m = np.zeros((lq, lkv), dtype=bool)
        for i in range(lq):
            for j in range(lkv):
                m[i, j] = block_mask_bn[i // bx, j // by] != 0
    return m & allowed_pairs(np.arange(lq), np.arange(lkv), window, atten_mask)


def _selected_blocks(block_mask_bn: Optional[np.ndarray], ib: int, nkb_b: int) -> List[int]:
    """In-range KV blocks selected by Q-block ``ib`` (ascending)."""
    if block_mask_bn is None:
        return list(range(nkb_b))
    return [jb for jb in range(nkb_b) if block_mask_bn[ib, jb] != 0]


def block_lists(mask: Optional[np.ndarray], B: int, N: int, nqb: int, nkb: int, bx: int, by: int,
                len_q: Sequence[int], len_kv: Sequence[int], window=None):
    """Per-Q-block and per-KV-block lists of selected in-range blocks.

    Returns ``(row_lists, col_lists)``: ``row_lists[b][n][i]`` is the ascending
    list of KV blocks ``j`` with ``mask[b, n, i, j] != 0``, ``i < ceil(Lq_b/bx)``
    and ``j < ceil(Lkv_b/by)`` (and, with a window, at least one in-range element
    of the block inside it); ``col_lists[b][n][j]`` is the ascending list of
    such ``i`` for KV block ``j``.  Lists of out-of-range blocks are empty.
    Brute force over every mask entry (and every element of a block for the window).
    """
    row_lists = [[[[] for _ in range(nqb)] for _ in range(N)] for _ in range(B)]
    col_lists = [[[[] for _ in range(nkb)] for _ in range(N)] for _ in range(B)]
    for b in range(B):
        nq_b = -(-int(len_q[b]) // bx)
        nk_b = -(-int(len_kv[b]) // by)
        for n in range(N):
            for i in range(nqb):
                for j in range(nkb):
                    on = True if mask is None else bool(mask[b, n, i, j] != 0)
                    if on and i < nq_b and j < nk_b and window is not None:
                        rr = np.arange(i * bx, min(i * bx + bx, int(len_q[b])))
                        cc = np.arange(j * by, min(j * by + by, int(len_kv[b])))
                        on = bool(in_window(rr, cc, window).any())
                    if on and i < nq_b and j < nk_b:
                        row_lists[b][n][i].append(j)
                        col_lists[b][n][j].append(i)
    return row_lists, col_lists


def block_list_arrays(mask: Optional[np.ndarray], B: int, N: int, nqb: int, nkb: int, bx: int, by: int,
                      len_q: Sequence[int], len_kv: Sequence[int], window=None):
    """``block_lists``' rule evaluated on whole arrays, for full-size problems.

    Returns ``(row_cnt [B,N,nqb], row_idx [B,N,nqb,nkb], col_cnt [B,N,nkb],
    col_idx [B,N,nkb,nqb])`` (int64): row (b, n, i) lists its ``row_cnt``
    selected KV blocks ascending in ``row_idx[b, n, i, :row_cnt]``; the entries
    after them are not part of the result.  A block (i, j) is listed when the
    mask selects it, ``i < ceil(Lq_b/bx)``, ``j < ceil(Lkv_b/by)`` and, with a
    window ``(pre, nxt)``, some in-range pair of it has ``-pre <= j' - i' <= nxt``:
    over the block's in-range rows [r0, r1) and keys [c0, c1) the differences
    j' - i' fill the interval [c0 - (r1 - 1), (c1 - 1) - r0], which must meet
    [-pre, nxt] (an empty window, ``pre + nxt < 0``, meets no block).
    """
    sel = np.ones((B, N, nqb, nkb), bool) if mask is None else np.asarray(mask).reshape(B, N, nqb, nkb) != 0
    sel = sel.copy()
    i = np.arange(nqb, dtype=np.int64)[:, None]
    j = np.arange(nkb, dtype=np.int64)[None, :]
    for b in range(B):
        lq, lk = int(len_q[b]), int(len_kv[b])
        ok = (i < -(-lq // bx)) & (j < -(-lk // by))
        if window is not None:
            pre, nxt = window
            r0, r1 = i * bx, np.minimum(i * bx + bx, lq)
            c0, c1 = j * by, np.minimum(j * by + by, lk)
            ok &= (c0 - (r1 - 1) <= nxt) & ((c1 - 1) - r0 >= -pre) & (-pre <= nxt)
        sel[b] &= ok[None]
    # a stable sort of "not selected" puts the selected indices first, ascending
    row_idx = np.argsort(~sel, axis=3, kind="stable")
    col_sel = np.ascontiguousarray(sel.transpose(0, 1, 3, 2))
    col_idx = np.argsort(~col_sel, axis=3, kind="stable")
    return sel.sum(axis=3), row_idx, col_sel.sum(axis=3), col_idx


# ---------------------------------------------------------------------------
# the method's steps
# ---------------------------------------------------------------------------
def softmax_grad(do: np.ndarray, o: np.ndarray) -> np.ndarray:
    """softmax_grad(dOut, attentionOut): delta_i = sum_d dO[i, d] * O[i, d]."""
    return np.sum(np.asarray(do, np.float64) * np.asarray(o, np.float64), axis=-1)


def _slab_columns(block_mask_bn, ib, by, lkv):
    """Column indices of every KV block selected by Q-block ``ib`` (clipped to lkv)."""
    nkb_b = -(-lkv // by)
    cols = [np.arange(jb * by, min(jb * by + by, lkv)) for jb in _selected_blocks(block_mask_bn, ib, nkb_b)]
    if not cols:
        return np.zeros(0, np.int64)
    return np.concatenate(cols)


def _head_forward(q, k, v, bm, bx, by, scale, window=None, atten_mask=None):
    """Forward of one (batch, query head): O [lq, D], LSE [lq] (fp64)."""
    lq, lkv = q.shape[0], k.shape[0]
    o = np.zeros_like(q)
    lse = np.full(lq, -np.inf)
    for ib in range(-(-lq // bx)):
        r = np.arange(ib * bx, min(ib * bx + bx, lq))
        cols = _slab_columns(bm, ib, by, lkv)
        if cols.size == 0:
            continue
        allowed = allowed_pairs(r, cols, window, atten_mask)
        live = allowed.any(axis=1)          # rows the window / attenMask leave some key
        if not live.any():
            continue
        rl, al = r[live], allowed[live]
        s = np.where(al, scale * (q[rl] @ k[cols].T), -np.inf)
        m = s.max(axis=1, keepdims=True)
        l = m[:, 0] + np.log(np.sum(np.exp(s - m), axis=1))
        lse[rl] = l
        o[rl] = np.exp(s - l[:, None]) @ v[cols]
    return o, lse


def _head_slabs(q, k, v, o, do, lse, bm, bx, by, scale, window=None, atten_mask=None):
    """P and dS of one (batch, query head), one Q-block slab at a time:
    yields (rows, cols, P, dS) over the slab's rows and its selected columns."""
    lq, lkv = q.shape[0], k.shape[0]
    delta = softmax_grad(do, o)
    for ib in range(-(-lq // bx)):
        rows = slice(ib * bx, min(ib * bx + bx, lq))
        cols = _slab_columns(bm, ib, by, lkv)
        if cols.size == 0:
            continue
        allowed = allowed_pairs(np.arange(rows.start, rows.stop), cols, window, atten_mask)
        s = scale * (q[rows] @ k[cols].T)          # S
        with np.errstate(over="ignore", invalid="ignore"):  # P, recomputed from the LSE, 0 off the window
            p = np.where(allowed, np.exp(np.where(allowed, s - lse[rows, None], 0.0)), 0.0)
        dp = do[rows] @ v[cols].T                  # dP = dOut * V^T
        ds = p * (dp - delta[rows, None])          # dS = P o (dP - softmax_grad)
        yield rows, cols, p, ds


def _head_backward(q, k, v, o, do, lse, bm, bx, by, scale, window=None, atten_mask=None):
    """Backward of one (batch, query head): dQ, and this head's dK, dV terms."""
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for rows, cols, p, ds in _head_slabs(q, k, v, o, do, lse, bm, bx, by, scale, window, atten_mask):
        dv[cols] += p.T @ do[rows]                 # dV = P^T * dOut
        dq[rows] = scale * (ds @ k[cols])          # dQ = (dS * K) * scale
        dk[cols] += scale * (ds.T @ q[rows])       # dK = (dS^T * Q) * scale
    return dq, dk, dv


def head_probs_and_ds(q, k, v, o, do, lse, block_mask_bn, *, bx, by, scale, window=None, atten_mask=None):
    """P and dS of one (batch, query head) as dense [lq, lkv] fp64 arrays, 0
    outside the selected pairs (the values the backward contracts; for the
    pins that every row of P sums to one and every row of dS to zero).
    q, o, do: [lq, D] of the head; k, v: [lkv, D] of its KV head; lse [lq]."""
    q, k, v, o, do = (np.asarray(x, np.float64) for x in (q, k, v, o, do))
    lse = np.asarray(lse, np.float64)
    P = np.zeros((q.shape[0], k.shape[0]))
    dS = np.zeros_like(P)
    for rows, cols, p, ds in _head_slabs(q, k, v, o, do, lse, block_mask_bn, bx, by, scale, window, atten_mask):
        P[rows, cols] = p
        dS[rows, cols] = ds
    return P, dS


def _check_heads(N, Nkv):
    if N < Nkv or N % Nkv != 0:
        raise ValueError("need N >= Nkv and N % Nkv == 0")
    return N // Nkv


def _dims(q, k, layout):
    if layout == "BNSD":
        B, N, _, D = q.shape
        Nkv = k.shape[1]
    elif layout == "TND":
        _, N, D = q.shape
        Nkv = k.shape[1]
        B = None
    else:
        raise ValueError(layout)
    return B, N, Nkv, D


def _lengths(layout, q, k, len_q, len_kv):
    if layout == "BNSD":
        B = q.shape[0]
        lq = np.full(B, q.shape[2], np.int64) if len_q is None else np.asarray(len_q, np.int64)
        lk = np.full(B, k.shape[2], np.int64) if len_kv is None else np.asarray(len_kv, np.int64)
    else:
        if len_q is None or len_kv is None:
            raise ValueError("TND needs per-sequence lengths")
        lq = np.asarray(len_q, np.int64)
        lk = np.asarray(len_kv, np.int64)
    return lq, lk


def forward(q, k, v, mask, *, layout, bx, by, scale, len_q=None, len_kv=None, window=None, atten_mask=None):
    """Masked attention forward: O (q's layout) and LSE ([B,N,S] or [T,N]), fp64."""
    _, N, Nkv, _ = _dims(q, k, layout)
    G = _check_heads(N, Nkv)
    lq, lk = _lengths(layout, q, k, len_q, len_kv)
    offq, offk = sequence_offsets(lq), sequence_offsets(lk)
    o = np.zeros(q.shape, np.float64)
    lse = np.full(q.shape[:-1], -np.inf)
    for b in range(len(lq)):
        Lq, Lk = int(lq[b]), int(lk[b])
        qs = _seq(q, layout, b, Lq, offq[b])
        ks = _seq(k, layout, b, Lk, offk[b])
        vs = _seq(v, layout, b, Lk, offk[b])
        ob = np.zeros_like(qs)
        lb = np.full((N, Lq), -np.inf)
        for n in range(N):
            bm = None if mask is None else mask[b, n]
            ob[n], lb[n] = _head_forward(qs[n], ks[n // G], vs[n // G], bm, bx, by, scale, window, atten_mask)
        _put(o, ob, layout, b, Lq, offq[b])
        _put_lse(lse, lb, layout, b, Lq, offq[b])
    return o, lse


def backward(q, k, v, o, do, lse, mask, *, layout, bx, by, scale, len_q=None, len_kv=None, window=None,
             atten_mask=None):
    """dQ, dK, dV (fp64, in the inputs' layouts) of block-sparse attention."""
    _, N, Nkv, _ = _dims(q, k, layout)
    G = _check_heads(N, Nkv)
    lq, lk = _lengths(layout, q, k, len_q, len_kv)
    offq, offk = sequence_offsets(lq), sequence_offsets(lk)
    dq = np.zeros(q.shape, np.float64)
    dk = np.zeros(k.shape, np.float64)
    dv = np.zeros(v.shape, np.float64)
    for b in range(len(lq)):
        Lq, Lk = int(lq[b]), int(lk[b])
        qs = _seq(q, layout, b, Lq, offq[b])
        os_ = _seq(o, layout, b, Lq, offq[b])
        dos = _seq(do, layout, b, Lq, offq[b])
        ls = _seq_lse(lse, layout, b, Lq, offq[b])
        ks = _seq(k, layout, b, Lk, offk[b])
        vs = _seq(v, layout, b, Lk, offk[b])
        dqb = np.zeros_like(qs)
        dkb = np.zeros_like(ks)
        dvb = np.zeros_like(vs)
        for n in range(N):
            h = n // G
            bm = None if mask is None else mask[b, n]
            dqn, dkn, dvn = _head_backward(qs[n], ks[h], vs[h], os_[n], dos[n], ls[n], bm, bx, by, scale, window,
                                           atten_mask)
            dqb[n] = dqn
            dkb[h] += dkn
            dvb[h] += dvn
        _put(dq, dqb, layout, b, Lq, offq[b])
        _put(dk, dkb, layout, b, Lk, offk[b])
        _put(dv, dvb, layout, b, Lk, offk[b])
    return dq, dk, dv


# ---------------------------------------------------------------------------
# literal dense versions (tiny shapes): full element mask, full matrices
# ---------------------------------------------------------------------------
def forward_dense(q, k, v, mask, *, layout, bx, by, scale, len_q=None, len_kv=None, window=None,
                  atten_mask=None):
    """Same as ``forward`` but on the full [Lq, Lkv] element mask."""
    _, N, Nkv, _ = _dims(q, k, layout)
    G = _check_heads(N, Nkv)
    lq, lk = _lengths(layout, q, k, len_q, len_kv)
    offq, offk = sequence_offsets(lq), sequence_offsets(lk)
    o = np.zeros(q.shape, np.float64)
    lse = np.full(q.shape[:-1], -np.inf)
    for b in range(len(lq)):
        Lq, Lk = int(lq[b]), int(lk[b])
        qs = _seq(q, layout, b, Lq, offq[b])
        ks = _seq(k, layout, b, Lk, offk[b])
        vs = _seq(v, layout, b, Lk, offk[b])
        ob = np.zeros_like(qs)
        lb = np.full((N, Lq), -np.inf)
        for n in range(N):
            h = n // G
            m = element_mask(None if mask is None else mask[b, n], bx, by, Lq, Lk, window, atten_mask)
            s = np.where(m, scale * (qs[n] @ ks[h].T), -np.inf)
            for i in range(Lq):
                if m[i].any():
                    mx = s[i][m[i]].max()
                    lb[n, i] = mx + np.log(np.sum(np.exp(s[i][m[i]] - mx)))
                    p = np.where(m[i], np.exp(s[i] - lb[n, i]), 0.0)
                    ob[n, i] = p @ vs[h]
        _put(o, ob, layout, b, Lq, offq[b])
        _put_lse(lse, lb, layout, b, Lq, offq[b])
    return o, lse


def backward_dense(q, k, v, o, do, lse, mask, *, layout, bx, by, scale, len_q=None, len_kv=None,
                   window=None, atten_mask=None):
    """Same as ``backward`` but on the full [Lq, Lkv] element mask."""
    _, N, Nkv, _ = _dims(q, k, layout)
    G = _check_heads(N, Nkv)
    lq, lk = _lengths(layout, q, k, len_q, len_kv)
    offq, offk = sequence_offsets(lq), sequence_offsets(lk)
    dq = np.zeros(q.shape, np.float64)
    dk = np.zeros(k.shape, np.float64)
    dv = np.zeros(v.shape, np.float64)
    for b in range(len(lq)):
        Lq, Lk = int(lq[b]), int(lk[b])
        qs = _seq(q, layout, b, Lq, offq[b])
        os_ = _seq(o, layout, b, Lq, offq[b])
        dos = _seq(do, layout, b, Lq, offq[b])
        ls = _seq_lse(lse, layout, b, Lq, offq[b])
        ks = _seq(k, layout, b, Lk, offk[b])
        vs = _seq(v, layout, b, Lk, offk[b])
        dqb = np.zeros_like(qs)
        dkb = np.zeros_like(ks)
        dvb = np.zeros_like(vs)
        for n in range(N):
            h = n // G
            m = element_mask(None if mask is None else mask[b, n], bx, by, Lq, Lk, window, atten_mask)
            delta = softmax_grad(dos[n], os_[n])
            s = scale * (qs[n] @ ks[h].T)
            with np.errstate(over="ignore", invalid="ignore"):
                p = np.where(m, np.exp(np.where(m, s - ls[n][:, None], 0.0)), 0.0)
            dp = dos[n] @ vs[h].T
            ds = p * (dp - delta[:, None])
            dqb[n] = scale * (ds @ ks[h])
            dkb[h] += scale * (ds.T @ qs[n])
            dvb[h] += p.T @ dos[n]
        _put(dq, dqb, layout, b, Lq, offq[b])
        _put(dk, dkb, layout, b, Lk, offk[b])
        _put(dv, dvb, layout, b, Lk, offk[b])
    return dq, dk, dv


# ---------------------------------------------------------------------------
# single output rows (for checking large problems on a sample)
# ---------------------------------------------------------------------------
def _row_of(x, layout, b, n, r, off):
    if layout == "BNSD":
        return np.asarray(x[b, n, r], np.float64)
    return np.asarray(x[off + r, n], np.float64)


def _rows_of(x, layout, b, n, rows, off):
    if layout == "BNSD":
        return np.asarray(x[b, n, rows], np.float64)
    return np.asarray(x[off + rows, n], np.float64)


def _lse_rows(lse, layout, b, n, rows, off):
    lse = np.asarray(lse)
    if layout == "BNSD":
        if lse.ndim == 4:
            lse = lse[..., 0]
        return np.asarray(lse[b, n, rows], np.float64)
    if lse.ndim == 3:
        lse = lse[..., 0]
    return np.asarray(lse[off + rows, n], np.float64)


def backward_dq_rows(q, k, v, o, do, lse, mask, *, layout, bx, by, scale, len_q=None, len_kv=None,
                     rows: Iterable[Tuple[int, int, int]] = (), window=None,
                     atten_mask=None) -> Dict[Tuple[int, int, int], np.ndarray]:
    """dQ rows for ``(b, n, i)`` triples (sequence-local i), fp64 [D] each.

    Row i of head n sums over the columns of the KV blocks its Q-block selects.
    """
    _, N, Nkv, _ = _dims(q, k, layout)
    G = _check_heads(N, Nkv)
    lq, lk = _lengths(layout, q, k, len_q, len_kv)
    offq, offk = sequence_offsets(lq), sequence_offsets(lk)
    out = {}
    for (b, n, i) in rows:
        Lq, Lk = int(lq[b]), int(lk[b])
        D = q.shape[-1]
        if i >= Lq:
            out[(b, n, i)] = np.zeros(D)
            continue
        h = n // G
        bm = None if mask is None else mask[b, n]
        cols = _slab_columns(bm, i // bx, by, Lk)
        cols = cols[allowed_pairs([i], cols, window, atten_mask)[0]]
        if cols.size == 0:
            out[(b, n, i)] = np.zeros(D)
            continue
        qi = _row_of(q, layout, b, n, i, offq[b])
        oi = _row_of(o, layout, b, n, i, offq[b])
        doi = _row_of(do, layout, b, n, i, offq[b])
        li = float(_lse_rows(lse, layout, b, n, np.array([i]), offq[b])[0])
        kc = _rows_of(k, layout, b, h, cols, offk[b])
        vc = _rows_of(v, layout, b, h, cols, offk[b])
        s = scale * (kc @ qi)
        p = np.exp(s - li)
        dp = vc @ doi
        ds = p * (dp - softmax_grad(doi, oi))
        out[(b, n, i)] = scale * (ds @ kc)
    return out


def backward_dkdv_rows(q, k, v, o, do, lse, mask, *, layout, bx, by, scale, len_q=None, len_kv=None,
                       rows: Iterable[Tuple[int, int, int]] = (), window=None, atten_mask=None):
    """dK and dV rows for ``(b, h, j)`` triples (sequence-local j), fp64 [D] each.

    Key j of KV head h sums over every query head n of its group and every row
    of each Q-block that selects j's KV block.
    """
    _, N, Nkv, _ = _dims(q, k, layout)
    G = _check_heads(N, Nkv)
    lq, lk = _lengths(layout, q, k, len_q, len_kv)
    offq, offk = sequence_offsets(lq), sequence_offsets(lk)
    dk_out, dv_out = {}, {}
    D = q.shape[-1]
    for (b, h, j) in rows:
        Lq, Lk = int(lq[b]), int(lk[b])
        dkj = np.zeros(D)
        dvj = np.zeros(D)
        if j < Lk:
            kj = _row_of(k, layout, b, h, j, offk[b])
            vj = _row_of(v, layout, b, h, j, offk[b])
            nqb_b = -(-Lq // bx)
            for n in range(h * G, (h + 1) * G):
                bm = None if mask is None else mask[b, n]
                for ib in range(nqb_b):
                    if bm is not None and bm[ib, j // by] == 0:
                        continue
                    rr = np.arange(ib * bx, min(ib * bx + bx, Lq))
                    rr = rr[allowed_pairs(rr, [j], window, atten_mask)[:, 0]]
                    if rr.size == 0:
                        continue
                    qr = _rows_of(q, layout, b, n, rr, offq[b])
                    orr = _rows_of(o, layout, b, n, rr, offq[b])
                    dor = _rows_of(do, layout, b, n, rr, offq[b])
                    lr = _lse_rows(lse, layout, b, n, rr, offq[b])
                    s = scale * (qr @ kj)
                    p = np.exp(s - lr)
                    dp = dor @ vj
                    ds = p * (dp - softmax_grad(dor, orr))
                    dvj += p @ dor
                    dkj += scale * (ds @ qr)
        dk_out[(b, h, j)] = dkj
        dv_out[(b, h, j)] = dvj
    return dk_out, dv_out

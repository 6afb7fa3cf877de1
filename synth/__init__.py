"""Seeded synthetic inputs for the block-sparse attention backward.

This module only draws random data and lays it out; it holds none of the
method's arithmetic (no scores, softmax, log-sum-exp or gradients).  Both the
CPU oracle's tests and the GPU path's tests and benchmark take their inputs
from here, so the two sides always see bit-identical values.

What is drawn, in this order, from ``numpy.random.Generator(PCG64(seed))``:

1. per-sequence lengths (only for cases that draw them),
2. the block mask ``[B, N, ceil(maxSq/bx), ceil(maxSkv/by)]`` (uint8, 1 = the
   block takes part, as the aclnnBlockSparseAttentionGrad page's parameter
   table defines blockSparseMaskOptional),
3. Q, K, V, dO as float32 standard normals, rounded to the case's dtype with
   round-to-nearest-even.

The forward output O and the log-sum-exp are not drawn here: they are a
function of Q, K, V and the mask, and whoever needs them computes them.

The named workloads (``config(k)``) follow the five configurations the
benchmark plan uses (shapes, dtypes, block shapes, mask rules); the mask rules
are read as follows:

* "Bernoulli(p) per block, diagonal forced on": i.i.d. ``U[0,1) < p`` per
  (b, n, i, j), then block ``(i, floor(i*bx/by))`` set for every in-range
  Q-block ``i`` of the sequence.
* "block-causal local window of 8 blocks plus first 2 KV blocks always on":
  ``j in [max(0, i-7), i]`` or ``j in {0, 1}``, for every (b, n); row 0 thus
  also selects block 1.
* "each Q-block row guaranteed >= 1 active block": after the draw, every
  in-range row with no in-range selected block gets one block drawn uniformly
  from the in-range ones with the same generator.
* varlen lengths ``Uniform[512, 8192]``: inclusive integers, one per sequence,
  drawn first; ``Sq_b == Skv_b``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "Case",
    "config",
    "make_case",
    "round_to_dtype",
    "dtype_bits",
    "CONFIG_NAMES",
    "FP8_MAX",
    "quantize_fp8",
]

CONFIG_NAMES = {
    1: "bnsd_b1_n2_s256_d64_fp16_blk64x64_p0.5",
    2: "bnsd_b2_n16_s4096_d128_bf16_blk128x128_p0.25",
    3: "bnsd_gqa32to8_s8192_d128_bf16_blk128x128_local8_sink2",
    4: "tnd_b8_len512to8192_gqa32to4_d128_fp16_blk64x128_p0.1",
    5: "bnsd_gqa32to8_sq16384_skv65536_d128_bf16_blk128x64_p0.05",
}


# ---------------------------------------------------------------------------
# rounding helpers (data preparation: float32 -> storage dtype, RNE)
# ---------------------------------------------------------------------------
def _bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    # NaN stays NaN (quiet); the generators never produce one
    nan = np.isnan(x)
    if nan.any():
        r = np.where(nan, np.uint32(0x7FC0), r)
    return r.astype(np.uint16)


def dtype_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Storage bit patterns (uint16) of float32 values in ``dtype``."""
    if dtype == "bf16":
        return _bf16_bits(x)
    if dtype == "fp16":
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)
    raise ValueError(f"unknown dtype {dtype!r}")


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to ``dtype`` (RNE) and return them as float32."""
    if dtype == "bf16":
        b = _bf16_bits(x).astype(np.uint32) << np.uint32(16)
        return b.view(np.float32)
    if dtype == "fp16":
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).astype(np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------------------
# the case description
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class Case:
    """One synthetic problem.

    Tensors are float32 arrays holding values exactly representable in
    ``dtype``; ``layout`` decides their shape:

    * ``"BNSD"``: q/do ``[B, N, Sq, D]``, k/v ``[B, Nkv, Skv, D]``;
    * ``"TND"``:  q/do ``[Tq, N, D]``,  k/v ``[Tkv, Nkv, D]``.

    ``mask`` is uint8 ``[B, N, ceil(maxSq/bx), ceil(maxSkv/by)]`` (or None for
    the dense case).  ``len_q``/``len_kv`` hold per-sequence token counts
    (always filled in; for BNSD without explicit lengths they equal S and
    ``explicit_lengths`` is False).
    """

    name: str
    layout: str
    dtype: str
    B: int
    N: int
    Nkv: int
    D: int
    Sq: int  # BNSD: tensor S dim; TND: max sequence length
    Skv: int
    bx: int
    by: int
    scale: float
    len_q: np.ndarray
    len_kv: np.ndarray
    explicit_lengths: bool
    mask: Optional[np.ndarray]
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    do: np.ndarray
    seed: int
    # (preTokens, nextTokens) of a sliding window, or None for none; a
    # parameter handed to both sides unchanged
    window: Optional[tuple] = None
    # attenMask [maxSq, maxSkv] uint8 (1 = the pair does not take part), or None
    atten_mask: Optional[np.ndarray] = None

    @property
    def G(self) -> int:
        return self.N // self.Nkv

    @property
    def nqb(self) -> int:
        return -(-self.Sq // self.bx)

    @property
    def nkb(self) -> int:
        return -(-self.Skv // self.by)


def _draw_mask(rng, B, N, nqb, nkb, bx, by, len_q, len_kv, rule, p):
    shape = (B, N, nqb, nkb)
    if rule == "dense":
        return None
    if rule == "ones":
        return np.ones(shape, np.uint8)
    if rule == "bernoulli":
        m = (rng.random(shape) < p).astype(np.uint8)
        return m
    if rule == "bernoulli_diag":
        m = (rng.random(shape) < p).astype(np.uint8)
        for b in range(B):
            nq_b = -(-int(len_q[b]) // bx)
            nk_b = -(-int(len_kv[b]) // by)
            for i in range(nq_b):
                j = (i * bx) // by
                if j < nk_b:
                    m[b, :, i, j] = 1
        return m
    if rule == "local8_sink2":
        i = np.arange(nqb)[:, None]
        j = np.arange(nkb)[None, :]
        pat = ((j <= i) & (j >= i - 7)) | (j < 2)
        return np.broadcast_to(pat.astype(np.uint8), shape).copy()
    if rule == "bernoulli_rowguard":
        m = (rng.random(shape) < p).astype(np.uint8)
        for b in range(B):
            nq_b = -(-int(len_q[b]) // bx)
            nk_b = -(-int(len_kv[b]) // by)
            for n in range(N):
                for i in range(nq_b):
                    if not m[b, n, i, :nk_b].any():
                        m[b, n, i, int(rng.integers(0, nk_b))] = 1
        return m
    raise ValueError(f"unknown mask rule {rule!r}")


def make_case(
    *,
    layout: str = "BNSD",
    dtype: str = "bf16",
    B: int = 1,
    N: int = 1,
    Nkv: int = 1,
    D: int = 64,
    Sq: int = 128,
    Skv: int = 128,
    bx: int = 64,
    by: int = 64,
    mask_rule: str = "bernoulli_diag",
    p: float = 0.5,
    lengths_q: Optional[Sequence[int]] = None,
    lengths_kv: Optional[Sequence[int]] = None,
    draw_lengths: Optional[tuple] = None,
    scale: Optional[float] = None,
    seed: int = 0,
    name: str = "custom",
    window: Optional[tuple] = None,
) -> Case:
    """Draw one case.

    ``draw_lengths=(lo, hi)`` draws ``B`` inclusive integer lengths first and
    uses them for both Q and KV (``Sq``/``Skv`` then become the maxima).
    ``lengths_q``/``lengths_kv`` give explicit lengths (TND requires them one
    way or the other; for BNSD they mark padded tails).
    """
    if layout not in ("BNSD", "TND"):
        raise ValueError(layout)
    rng = np.random.Generator(np.random.PCG64(seed))
    explicit = False
    if draw_lengths is not None:
        lo, hi = draw_lengths
        lq = rng.integers(lo, hi + 1, size=B).astype(np.int64)
        lk = lq.copy()
        explicit = True
    elif lengths_q is not None:
        lq = np.asarray(lengths_q, np.int64)
        lk = np.asarray(lengths_kv if lengths_kv is not None else lengths_q, np.int64)
        explicit = True
    else:
        if layout == "TND":
            raise ValueError("TND needs lengths")
        lq = np.full(B, Sq, np.int64)
        lk = np.full(B, Skv, np.int64)
    if layout == "TND" or draw_lengths is not None:
        Sq = int(lq.max())
        Skv = int(lk.max())
    nqb = -(-Sq // bx)
    nkb = -(-Skv // by)
    mask = _draw_mask(rng, B, N, nqb, nkb, bx, by, lq, lk, mask_rule, p)

    if layout == "BNSD":
        qshape = (B, N, Sq, D)
        kshape = (B, Nkv, Skv, D)
    else:
        qshape = (int(lq.sum()), N, D)
        kshape = (int(lk.sum()), Nkv, D)

    def draw(shape):
        return round_to_dtype(rng.standard_normal(shape, dtype=np.float32), dtype)

    q = draw(qshape)
    k = draw(kshape)
    v = draw(kshape)
    do = draw(qshape)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return Case(
        name=name, layout=layout, dtype=dtype, B=B, N=N, Nkv=Nkv, D=D, Sq=Sq, Skv=Skv,
        bx=bx, by=by, scale=float(scale), len_q=lq, len_kv=lk, explicit_lengths=explicit,
        mask=mask, q=q, k=k, v=v, do=do, seed=seed, window=window,
    )


def config(k: int, seed: Optional[int] = None, head_dim: Optional[int] = None) -> Case:
    """The five named workloads (seed defaults to 1000 + k).

    ``head_dim`` replaces the workload's head dim (and its scale, D^-0.5)
    while keeping everything else; lengths and mask are drawn before the
    tensors, so they stay the same.  The name gets a ``_d<D>`` suffix.
    """
    if seed is None:
        seed = 1000 + k
    name = CONFIG_NAMES[k]
    if k == 1:
        kw = dict(layout="BNSD", dtype="fp16", B=1, N=2, Nkv=2, D=64, Sq=256, Skv=256,
                  bx=64, by=64, mask_rule="bernoulli_diag", p=0.5, scale=1.0 / 8)
    elif k == 2:
        kw = dict(layout="BNSD", dtype="bf16", B=2, N=16, Nkv=16, D=128, Sq=4096,
                  Skv=4096, bx=128, by=128, mask_rule="bernoulli_diag", p=0.25)
    elif k == 3:
        kw = dict(layout="BNSD", dtype="bf16", B=1, N=32, Nkv=8, D=128, Sq=8192,
                  Skv=8192, bx=128, by=128, mask_rule="local8_sink2")
    elif k == 4:
        kw = dict(layout="TND", dtype="fp16", B=8, N=32, Nkv=4, D=128, bx=64, by=128,
                  mask_rule="bernoulli_diag", p=0.1, draw_lengths=(512, 8192))
    elif k == 5:
        kw = dict(layout="BNSD", dtype="bf16", B=1, N=32, Nkv=8, D=128, Sq=16384,
                  Skv=65536, bx=128, by=64, mask_rule="bernoulli_rowguard", p=0.05)
    else:
        raise KeyError(k)
    if head_dim is not None:
        kw["D"] = int(head_dim)
        kw["scale"] = 1.0 / math.sqrt(kw["D"])
        name = f"{name}_d{kw['D']}"
    return make_case(seed=seed, name=name, **kw)


FP8_MAX = {"e4m3fn": 448.0, "e5m2": 57344.0}


def quantize_fp8(x: np.ndarray, fmt: str, factor: Optional[float] = None):
    """Input synthesis for fp8 runs: per-tensor factor (default max|x| / the
    format's largest finite value, so nothing saturates) and the codes of
    x / factor rounded to nearest-even by torch's float8 conversion.
    Returns (uint8 codes, factor)."""
    import torch
    tdt = {"e4m3fn": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}[fmt]
    x = np.asarray(x, dtype=np.float64)
    if factor is None:
        amax = float(np.abs(x).max()) if x.size else 0.0
        factor = amax / FP8_MAX[fmt] if amax > 0 else 1.0
    codes = torch.from_numpy(np.ascontiguousarray(x / factor, dtype=np.float32)).to(tdt).view(torch.uint8)
    return codes.numpy(), float(factor)


def active_blocks(case: Case) -> int:
    """Number of selected in-range (b, q-head, Q-block, KV-block) tuples.

    This is bookkeeping over the drawn mask (how much work the case holds),
    used to count the benchmark's nominal FLOPs.
    """
    total = 0
    for b in range(case.B):
        nq_b = -(-int(case.len_q[b]) // case.bx)
        nk_b = -(-int(case.len_kv[b]) // case.by)
        if case.mask is None:
            total += case.N * nq_b * nk_b
        else:
            total += int(np.count_nonzero(case.mask[b, :, :nq_b, :nk_b]))
    return total

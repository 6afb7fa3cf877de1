"""Helpers for the GPU tests: upload a case, run the library, compare with the oracle."""
from __future__ import annotations

import numpy as np

import oracle
import synth

# per-tensor bound: max|gpu - ref| <= TOL * max|ref|
TOL = {"fp16": 5e-3, "bf16": 2e-2}


def oracle_fwd_inputs(case):
    """O rounded to the case dtype and LSE rounded to fp32, from the oracle forward."""
    kw = dict(layout=case.layout, bx=case.bx, by=case.by, scale=case.scale, window=case.window,
              atten_mask=case.atten_mask)
    if case.explicit_lengths:
        kw.update(len_q=case.len_q, len_kv=case.len_kv)
    o, lse = oracle.forward(case.q, case.k, case.v, case.mask, **kw)
    return synth.round_to_dtype(o.astype(np.float32), case.dtype), lse.astype(np.float32)


def oracle_kw(case):
    kw = dict(layout=case.layout, bx=case.bx, by=case.by, scale=case.scale, window=case.window,
              atten_mask=case.atten_mask)
    if case.explicit_lengths or case.layout == "TND":
        kw.update(len_q=case.len_q, len_kv=case.len_kv)
    return kw


def upload(case, o=None, lse=None):
    import torch
    from bench import to_device
    dev = to_device(case)
    dt = dev["q"].dtype
    if o is not None:
        dev["o"] = torch.from_numpy(np.ascontiguousarray(o, np.float32)).cuda().to(dt)
        dev["lse"] = torch.from_numpy(np.ascontiguousarray(lse, np.float32)).cuda()
    return dev


def run_bsa(case, dev, *, mask="auto", lengths="auto", out_strides=None):
    """Run the library on uploaded tensors; returns (dq, dk, dv) torch tensors and the runner."""
    from bench import Runner
    r = Runner(case, dev, dev["o"], dev["lse"])
    if out_strides is not None:
        r.kw.update(out_strides)
    return r(), r


def to_np(t):
    return t.float().cpu().numpy().astype(np.float64)


def assert_close(name, got, ref, dtype, floor_ref=None):
    """The per-tensor bound; when max|ref| is 0 an absolute floor applies."""
    ref_max = float(np.abs(ref).max()) if ref.size else 0.0
    err = float(np.abs(got - ref).max()) if ref.size else 0.0
    if ref_max > 0:
        bound = TOL[dtype] * ref_max
    else:
        bound = 1e-6 * max(1.0, floor_ref if floor_ref is not None else 1.0)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    if err > bound:
        idx = np.unravel_index(int(np.argmax(np.abs(got - ref))), ref.shape)
        raise AssertionError(
            f"{name}: max abs err {err:.3e} > {bound:.3e} (max|ref| {ref_max:.3e}); worst at {idx}: "
            f"gpu {got[idx]:.6e} ref {ref[idx]:.6e}")
    return err, ref_max


def oracle_backward_threaded(case, q, k, v, o, do, lse, workers=16):
    """oracle.backward on the whole problem, run as independent (sequence, KV head)
    pieces on a pool of threads (one BLAS thread each) and put back together.
    Each piece is an unchanged oracle call; the pieces' outputs are disjoint."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    from bench import _sub_problems
    dq = np.zeros(q.shape, np.float64)
    dk = np.zeros(k.shape, np.float64)
    dv = np.zeros(v.shape, np.float64)
    pieces = list(_sub_problems(case, q, k, v, o, do, lse))

    def one(piece):
        iq, ik, args, kw = piece
        pq, pk, pv = oracle.backward(*args, **kw)
        dq[iq], dk[ik], dv[ik] = pq, pk, pv

    n = max(1, min(workers, len(os.sched_getaffinity(0)), len(pieces)))
    with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(max_workers=n) as pool:
        list(pool.map(one, pieces))
    return dq, dk, dv


GUARD = 4096  # guard bytes on each side of every output and of the workspace


def _guarded(shape, dtype):
    """A tensor of `shape` in the middle of a larger buffer whose GUARD bytes on
    each side hold a fixed pattern; returns (tensor, buffer, pattern)."""
    import torch
    n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
    buf = torch.randint(0, 256, (n + 2 * GUARD,), dtype=torch.uint8, device="cuda",
                        generator=torch.Generator(device="cuda").manual_seed(n))
    return buf[GUARD:GUARD + n].view(dtype).view(shape), buf, buf.clone()


def _guards_intact(buf, pattern):
    import torch
    return torch.equal(buf[:GUARD], pattern[:GUARD]) and torch.equal(buf[-GUARD:], pattern[-GUARD:])

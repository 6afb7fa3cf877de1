#!/usr/bin/env python3
"""Benchmark: block-sparse attention backward on one MI355X.

One step = one full ``bsa_bwd`` call (sequence table, delta pre-pass, mask
compaction, dK/dV kernel, dQ kernel) over the workload's inputs, which are
resident in HBM before timing starts.  Prints one JSON line:

  value    backward TFLOP/s counted over active blocks: 10*bx*by*D FLOPs per
           selected in-range (batch, query head, Q block, KV block)
  roofline the dominant kernel (dK/dV) against the dense bf16 MFMA peak,
           timed with HIP events recorded between the library's stages on
           the launch stream, over a second run of the same K steps
  cpu_baseline  the fp64 CPU oracle's backward on a bounded sample of the
           same workload, on this host's cores

Inputs are synthetic: Q, K, V, dO ~ N(0, 1) rounded to the dtype; O and LSE
come from a plain torch fp32 masked-attention forward on the GPU
(``gpu_forward``), outside the timed region.

With ``--op fwd`` a step is one ``bsa_fwd`` call (sequence table, row lists,
forward kernel) producing O and LSE, counted at 4*bx*by*D FLOPs per active
block (the S and PV products), with the forward kernel as the roofline and the
oracle's forward as the CPU baseline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2] [--op bwd|fwd]
                      [--head-dim 64|128|256] [--window PRE,NEXT] [--atten-mask FRACTION]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

MFMA_PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16/fp16 MFMA (published figure)
HBM_PEAK_GBS = 8000.0


def _torch():
    import torch
    return torch


# ---------------------------------------------------------------------------
# input synthesis on the GPU
# ---------------------------------------------------------------------------
def to_device(case, device="cuda"):
    """Upload a synth.Case: returns dict of torch tensors (dtype-exact values)."""
    torch = _torch()
    dt = torch.bfloat16 if case.dtype == "bf16" else torch.float16
    d = {
        "q": torch.from_numpy(case.q).to(device=device).to(dt),
        "k": torch.from_numpy(case.k).to(device=device).to(dt),
        "v": torch.from_numpy(case.v).to(device=device).to(dt),
        "do": torch.from_numpy(case.do).to(device=device).to(dt),
        "mask": None if case.mask is None else torch.from_numpy(case.mask).to(device),
        "amask": (None if case.atten_mask is None
                  else torch.from_numpy(np.ascontiguousarray(case.atten_mask, np.uint8)).to(device)),
    }
    return d


def _seq_views(x, layout, b, length, off):
    """[heads, length, D] view of sequence b."""
    if layout == "BNSD":
        return x[b, :, :length]
    return x[off:off + length].transpose(0, 1)


def gpu_forward(case, dev, rows_per_chunk=2048):
    """O (case dtype) and LSE (fp32) of masked attention, computed with plain torch fp32 ops.

    Input synthesis for large workloads: the block mask is expanded to an
    element mask per chunk of query rows (block i//bx, j//by; only the
    sequence's valid rows/columns), scores outside it are -inf, and
    LSE = logsumexp, O = softmax * V.  Rows with no selected key get O = 0,
    LSE = -inf.
    """
    torch = _torch()
    q, k, v, mask = dev["q"], dev["k"], dev["v"], dev["mask"]
    o = torch.zeros_like(q)
    lse = torch.full(q.shape[:-1], float("-inf"), dtype=torch.float32, device=q.device)
    offq = np.concatenate([[0], np.cumsum(case.len_q)[:-1]]).astype(np.int64)
    offk = np.concatenate([[0], np.cumsum(case.len_kv)[:-1]]).astype(np.int64)
    G = case.N // case.Nkv
    bx, by = case.bx, case.by
    chunk_blocks = max(1, rows_per_chunk // bx)
    for b in range(case.B):
        lq, lk = int(case.len_q[b]), int(case.len_kv[b])
        if lq == 0:
            continue
        qs = _seq_views(q, case.layout, b, lq, offq[b])
        ks = _seq_views(k, case.layout, b, lk, offk[b])
        vs = _seq_views(v, case.layout, b, lk, offk[b])
        os_ = _seq_views(o, case.layout, b, lq, offq[b])
        ls = lse[b, :, :lq] if case.layout == "BNSD" else lse[offq[b]:offq[b] + lq].transpose(0, 1)
        nqb_b, nkb_b = -(-lq // bx), -(-lk // by)
        for n in range(case.N):
            h = n // G
            kf = ks[h].float()
            vf = vs[h].float()
            for ib0 in range(0, nqb_b, chunk_blocks):
                ib1 = min(nqb_b, ib0 + chunk_blocks)
                r0, r1 = ib0 * bx, min(ib1 * bx, lq)
                s = case.scale * (qs[n, r0:r1].float() @ kf.t().contiguous())
                if mask is not None and lk > 0:
                    mb = mask[b, n, ib0:ib1, :nkb_b].bool()
                    em = mb.repeat_interleave(bx, dim=0)[: r1 - r0].repeat_interleave(by, dim=1)[:, :lk]
                    s.masked_fill_(~em, float("-inf"))
                if dev.get("amask") is not None and lk > 0:  # attenMask: 1 = the pair is left out
                    s.masked_fill_(dev["amask"][r0:r1, :lk].bool(), float("-inf"))
                if case.window is not None and lk > 0:  # sliding window: i - pre <= j <= i + next
                    d = (torch.arange(lk, device=s.device)[None, :]
                         - torch.arange(r0, r1, device=s.device)[:, None])
                    s.masked_fill_((d < -case.window[0]) | (d > case.window[1]), float("-inf"))
                l = torch.logsumexp(s, dim=1)
                p = torch.exp(s - l[:, None])
                p = torch.nan_to_num(p, nan=0.0)
                os_[n, r0:r1] = (p @ vf).to(q.dtype)
                ls[n, r0:r1] = l
                del s, p
    return o, lse


def quantize_inputs(dev, keys):
    """fp8 copies of dev[k] for k in keys (dout E5M2, the others E4M3FN), each with the
    per-tensor factor max|x| / the format's largest finite value; returns (dict, factors)."""
    torch = _torch()
    out, fac = dict(dev), {}
    for k in keys:
        tdt, top = (torch.float8_e5m2, 57344.0) if k == "do" else (torch.float8_e4m3fn, 448.0)
        x = dev[k].float()
        amax = float(x.abs().max())
        f = amax / top if amax > 0 else 1.0
        out[k] = (x / f).to(tdt)
        fac[k] = f
        del x
    return out, fac


# ---------------------------------------------------------------------------
# running the library
# ---------------------------------------------------------------------------
class Runner:
    """Pre-allocated outputs and workspace for repeated bsa_bwd calls.

    With ``descale`` (a list of the five dequantisation factors of dout,
    query, key, value, attention_out) the tensors are fp8 and the calls go to
    bsa_bwd_fp8, with bf16 gradients.
    """

    def __init__(self, case, dev, o, lse, descale=None, dq_mode=0):
        torch = _torch()
        import block_sparse_attention_bwd_amd as bsa
        self.bsa = bsa
        self.dev = dev
        self.fp8 = descale is not None
        self.descale = descale
        self.dq_mode = dq_mode
        odt = torch.bfloat16 if self.fp8 else dev["q"].dtype
        self.dq = torch.empty(dev["q"].shape, dtype=odt, device=dev["q"].device)
        self.dk = torch.empty(dev["k"].shape, dtype=odt, device=dev["k"].device)
        self.dv = torch.empty(dev["v"].shape, dtype=odt, device=dev["v"].device)
        lengths = case.explicit_lengths or case.layout == "TND"
        self.kw = dict(
            block_sparse_mask=dev["mask"], atten_mask=dev.get("amask"), block_shape=[case.bx, case.by],
            actual_seq_lengths=list(map(int, case.len_q)) if lengths else None,
            actual_seq_lengths_kv=list(map(int, case.len_kv)) if lengths else None,
            q_input_layout=case.layout, kv_input_layout=case.layout, num_key_value_heads=case.Nkv,
            mask_type=0, scale_value=case.scale,
            pre_tokens=bsa.NO_WINDOW if case.window is None else int(case.window[0]),
            next_tokens=bsa.NO_WINDOW if case.window is None else int(case.window[1]),
            dq=self.dq, dk=self.dk, dv=self.dv)
        self.args = (dev["do"], dev["q"], dev["k"], dev["v"], o, lse)
        if self.fp8:
            self.ws_size = bsa.bsa_bwd_fp8_workspace_size(*self.args, **self.kw, descale=descale)
        elif dq_mode:
            self.ws_size = bsa.bsa_bwd_ex_workspace_size(*self.args, **self.kw, dq_mode=dq_mode)
        else:
            self.ws_size = bsa.bsa_bwd_workspace_size(*self.args, **self.kw)
        self.ws = torch.empty(max(1, self.ws_size), dtype=torch.uint8, device=dev["q"].device)

    def __call__(self, stream=None):
        if self.fp8:
            self.bsa.bsa_bwd_fp8(*self.args, **self.kw, descale=self.descale, workspace=self.ws,
                                 workspace_size=self.ws_size, stream=stream)
        elif self.dq_mode:
            self.bsa.bsa_bwd_ex(*self.args, **self.kw, dq_mode=self.dq_mode, workspace=self.ws,
                                workspace_size=self.ws_size, stream=stream)
        else:
            self.bsa.bsa_bwd(*self.args, **self.kw, workspace=self.ws, workspace_size=self.ws_size,
                             stream=stream)
        return self.dq, self.dk, self.dv


class FwdRunner:
    """Pre-allocated O, LSE and workspace for repeated bsa_fwd calls (fp8
    query/key/value through bsa_fwd_fp8, with a bf16 O, when ``descale`` gives
    their three factors)."""

    def __init__(self, case, dev, descale=None):
        torch = _torch()
        import block_sparse_attention_bwd_amd as bsa
        self.bsa = bsa
        self.descale = descale
        odt = torch.bfloat16 if descale is not None else dev["q"].dtype
        self.o = torch.empty(dev["q"].shape, dtype=odt, device=dev["q"].device)
        self.lse = torch.empty(dev["q"].shape[:-1], dtype=torch.float32, device=dev["q"].device)
        lengths = case.explicit_lengths or case.layout == "TND"
        self.kw = dict(
            block_sparse_mask=dev["mask"], atten_mask=dev.get("amask"), block_shape=[case.bx, case.by],
            actual_seq_lengths=list(map(int, case.len_q)) if lengths else None,
            actual_seq_lengths_kv=list(map(int, case.len_kv)) if lengths else None,
            q_input_layout=case.layout, kv_input_layout=case.layout, num_key_value_heads=case.Nkv,
            mask_type=0, scale_value=case.scale,
            pre_tokens=bsa.NO_WINDOW if case.window is None else int(case.window[0]),
            next_tokens=bsa.NO_WINDOW if case.window is None else int(case.window[1]),
            attention_out=self.o, softmax_lse=self.lse)
        self.args = (dev["q"], dev["k"], dev["v"])
        if descale is not None:
            self.ws_size = bsa.bsa_fwd_fp8_workspace_size(*self.args, **self.kw, descale=descale)
        else:
            self.ws_size = bsa.bsa_fwd_workspace_size(*self.args, **self.kw)
        self.ws = torch.empty(max(1, self.ws_size), dtype=torch.uint8, device=dev["q"].device)

    def __call__(self, stream=None):
        if self.descale is not None:
            self.bsa.bsa_fwd_fp8(*self.args, **self.kw, descale=self.descale, workspace=self.ws,
                                 workspace_size=self.ws_size, stream=stream)
        else:
            self.bsa.bsa_fwd(*self.args, **self.kw, workspace=self.ws, workspace_size=self.ws_size,
                             stream=stream)
        return self.o, self.lse


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample
# ---------------------------------------------------------------------------
def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _sub_problems(case, q, k, v, o, do, lse):
    """The workload cut into independent (sequence, KV head) pieces: each holds one
    sequence and the query heads of one KV head's group, with their mask rows, so
    the oracle's results on the pieces are disjoint slices of the whole result.
    Yields (query-side index, key-side index, oracle arguments, oracle keywords);
    the indices place a piece's dq (resp. dk, dv) in the whole tensor."""
    G = case.N // case.Nkv
    offq = np.concatenate([[0], np.cumsum(case.len_q)[:-1]]).astype(np.int64)
    offk = np.concatenate([[0], np.cumsum(case.len_kv)[:-1]]).astype(np.int64)
    lengths = case.explicit_lengths or case.layout == "TND"
    for b in range(case.B):
        for h in range(case.Nkv):
            hs = slice(h * G, (h + 1) * G)
            if case.layout == "BNSD":
                iq, ik = (slice(b, b + 1), hs), (slice(b, b + 1), slice(h, h + 1))
            else:
                iq = (slice(int(offq[b]), int(offq[b] + case.len_q[b])), hs)
                ik = (slice(int(offk[b]), int(offk[b] + case.len_kv[b])), slice(h, h + 1))
            kw = dict(layout=case.layout, bx=case.bx, by=case.by, scale=case.scale, window=case.window,
                      atten_mask=case.atten_mask)
            if lengths:
                kw.update(len_q=case.len_q[b:b + 1], len_kv=case.len_kv[b:b + 1])
            mask = None if case.mask is None else case.mask[b:b + 1, hs]
            sub = lambda x, i: None if x is None else x[i]
            yield iq, ik, (q[iq], k[ik], v[ik], sub(o, iq), do[iq], sub(lse, iq), mask), kw


def cpu_baseline(case, o_host, lse_host, min_seconds=10.0, max_runs=5, op="bwd", max_workers=16):
    """Time the fp64 oracle backward (or forward) on the whole workload.

    The oracle runs unchanged on independent (sequence, KV head) pieces of the
    workload, spread over a pool of threads (NumPy's BLAS calls and large array
    operations release the interpreter lock), with BLAS held to one thread per
    worker so that ``cores`` is the number of threads actually used.  The
    median of repeated runs (at least one, until ``min_seconds`` have passed)."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits
    pieces = [(a, kw) for _, _, a, kw in _sub_problems(case, case.q, case.k, case.v, o_host, case.do, lse_host)]
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        avail = os.cpu_count() or 1
    workers = max(1, min(avail, max_workers, len(pieces)))
    blas = [f"{i.get('internal_api')} {i.get('version')}" for i in threadpool_info() if i.get("user_api") == "blas"]

    def one(piece):
        (q, k, v, o, do, lse, mask), kw = piece
        if op == "fwd":
            oracle.forward(q, k, v, mask, **kw)
        else:
            oracle.backward(q, k, v, o, do, lse, mask, **kw)

    times = []
    with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(max_workers=workers) as pool:
        t_start = time.perf_counter()
        while not times or (time.perf_counter() - t_start < min_seconds and len(times) < max_runs):
            t0 = time.perf_counter()
            list(pool.map(one, pieces))
            times.append(time.perf_counter() - t0)
    dt = float(np.median(times))
    flops = (4.0 if op == "fwd" else 10.0) * case.bx * case.by * case.D * synth_blocks(case)
    return {
        "value": round(flops / dt / 1e12, 5),
        "unit": "TFLOP/s",
        "cores": int(workers),
        "kind": "oracle",
        "sample": f"the whole workload (all batches and heads), fp64 NumPy {'forward' if op == 'fwd' else 'backward'} only, "
                  f"as {len(pieces)} (sequence, KV head) pieces on {workers} threads with 1 BLAS thread each; "
                  f"median of {len(times)} runs: {dt:.2f} s",
        "cpu_model": _cpu_model(),
        "cpus_available": int(avail),
        "blas": ", ".join(blas) or "unknown",
    }


def active_blocks(case):
    """Blocks that take part (the FLOP count's unit): selected, in range and, with a
    sliding window, meeting it (some element with -pre <= j - i <= next)."""
    import synth
    if case.window is None:
        return synth.active_blocks(case)
    pre, nxt = case.window
    total = 0
    for b in range(case.B):
        lq, lk = int(case.len_q[b]), int(case.len_kv[b])
        nq_b, nk_b = -(-lq // case.bx), -(-lk // case.by)
        i = np.arange(nq_b)[:, None]
        j = np.arange(nk_b)[None, :]
        r0, r1 = i * case.bx, np.minimum(i * case.bx + case.bx, lq)
        c0, c1 = j * case.by, np.minimum(j * case.by + case.by, lk)
        meets = (c0 - (r1 - 1) <= nxt) & ((c1 - 1) - r0 >= -pre) & (-pre <= nxt)
        sel = np.ones((case.N, nq_b, nk_b), bool) if case.mask is None else case.mask[b, :, :nq_b, :nk_b] != 0
        total += int(np.count_nonzero(sel & meets[None]))
    return total


def synth_blocks(case):
    return active_blocks(case)


PEAK_CLOCK_MHZ = 2400.0  # the clock the published MFMA peak is quoted at


def _driver_gfxclk(torch):
    """(activity %, shader clock MHz) from the driver's metrics table: the clock
    is the median over the XCDs of its per-XCD readings where it gives them,
    else its single reading; None if there is no reading."""
    try:
        import amdsmi
        h = torch.cuda._get_amdsmi_handler(torch.cuda.current_device())
        m = amdsmi.amdsmi_get_gpu_metrics_info(h)
        vals = [float(x) for x in (m.get("current_gfxclks") or []) if isinstance(x, (int, float)) and 0 < x < 10000]
        if not vals and isinstance(m.get("current_gfxclk"), (int, float)) and 0 < m["current_gfxclk"] < 10000:
            vals = [float(m["current_gfxclk"])]
        act = m.get("average_gfx_activity")
        if not vals or not isinstance(act, (int, float)):
            return None
        return float(act), float(np.median(vals))
    except Exception:  # no reading on this machine
        return None


def sustained_clock_mhz(run, torch, seconds=2.5, chunk=20):
    """Median shader clock (MHz) the driver reports while the calls run back to
    back: the driver refreshes its table about once a second, so the run lasts
    a few refreshes and only readings taken with the GPU at least 90% busy
    count (the first ones after the start still show the idle clock); None
    where it gives no such reading."""
    import threading
    samples, done = [], threading.Event()

    def poll():
        while not done.is_set():
            r = _driver_gfxclk(torch)
            if r is None:
                return
            if r[0] >= 90:
                samples.append(r[1])
            done.wait(0.005)

    for _ in range(chunk):  # the GPU is busy before the first sample
        run()
    t = threading.Thread(target=poll, daemon=True)
    t.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(chunk):
            run()
        torch.cuda.synchronize()
    done.set()
    t.join()
    return float(np.median(samples)) if samples else None


def counter_clock_mhz(workload, kernel):
    """Shader clock (MHz) over the dominant kernel from a committed rocprofv3 counter
    summary: GRBM_GUI_ACTIVE (busy cycles, summed over the 8 XCDs) / 8 / the
    kernel's duration in the same run; None if absent or taken on other source."""
    vals = _profile_values(workload, kernel)
    if not vals or "GRBM_GUI_ACTIVE" not in vals or "kernel_duration_ns" not in vals:
        return None
    return float(vals["GRBM_GUI_ACTIVE"]) / 8.0 / float(vals["kernel_duration_ns"]) * 1e3


def clock_report(driver_mhz, counter_mhz, tflops):
    """The value as a fraction of the MFMA peak scaled to the sustained clock (the
    counter-derived clock where a current profile gives it, else the driver's)."""
    mhz = counter_mhz if counter_mhz is not None else driver_mhz
    out = {"driver_mhz": None if driver_mhz is None else round(driver_mhz, 1),
           "counter_mhz": None if counter_mhz is None else round(counter_mhz, 1),
           "sustained_mhz": None if mhz is None else round(mhz, 1),
           "source": "counters" if counter_mhz is not None else ("driver" if driver_mhz is not None else None)}
    if mhz is None:
        out["frac_of_peak_at_sustained_clock"] = None
        return out
    peak = MFMA_PEAK_BF16_TFLOPS * mhz / PEAK_CLOCK_MHZ
    out.update(peak_at_sustained_clock=round(peak, 1), frac_of_peak_at_sustained_clock=round(tflops / peak, 4))
    return out


def kernel_source_hash():
    """sha256 over the device sources (csrc/*.hip and csrc/*.h, by name, each
    name followed by its bytes)."""
    import hashlib
    csrc = os.path.join(ROOT, "block_sparse_attention_bwd_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(n for n in os.listdir(csrc) if n.endswith((".hip", ".h"))):
        h.update(name.encode() + b"\0")
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _profile_values(workload, kernel):
    """The `key: value` lines of a committed counter summary, or None if it is
    missing or was taken on another version of the kernel source."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_counters.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return vals


def traffic_from_profile(workload, kernel, launches_per_step=1):
    """HBM bytes per launch of `kernel` from a committed rocprofv3 counter summary.

    The summary records FETCH_SIZE and WRITE_SIZE (KiB per dispatch), the scale
    factors measured on a plain copy kernel, and the sha256 of the kernel source
    it was taken on; if the source has changed since, the figure is stale and
    None is returned.
    """
    vals = _profile_values(workload, kernel)
    if not vals:
        return None
    fetch = float(vals["FETCH_SIZE_KiB_per_dispatch"]) * float(vals["fetch_scale"])
    write = float(vals["WRITE_SIZE_KiB_per_dispatch"]) * float(vals["write_scale"])
    return round((fetch + write) * 1024.0 * launches_per_step)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed calls first: the GPU reaches its steady clock after ~100 calls (~35 ms)")
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--window", default=None,
                    help="PRE,NEXT: a sliding window (preTokens, nextTokens) on top of the workload's mask")
    ap.add_argument("--atten-mask", type=float, default=None, metavar="FRACTION",
                    help="add an attenMask removing this fraction of (query, key) pairs (seeded, uniform)")
    ap.add_argument("--head-dim", type=int, default=None, choices=[64, 128, 256],
                    help="replace the workload's head dim (same lengths and mask, scale D^-0.5)")
    ap.add_argument("--fp8", action="store_true",
                    help="fp8 inputs (E4M3FN query/key/value/attentionOut, E5M2 dout, per-tensor factors) "
                         "through the fp8 entry points; bf16 compute and outputs")
    ap.add_argument("--op", choices=["bwd", "fwd"], default="bwd",
                    help="bwd: the backward (default); fwd: the forward that produces O and LSE")
    ap.add_argument("--clock-seconds", type=float, default=2.5,
                    help="how long to sample the driver's shader clock while calls run (0: skip)")
    ap.add_argument("--dq-mode", choices=["recompute", "atomic"], default="recompute",
                    help="backward dQ mode (bsa_bwd_ex): recompute (the default, deterministic) or atomic "
                         "(dS K added into an fp32 accumulator by the dK/dV kernel)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on exactly one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        return 2

    torch = _torch()
    import synth
    import block_sparse_attention_bwd_amd as bsa

    torch.backends.cuda.matmul.allow_tf32 = False
    case = synth.config(args.config, head_dim=args.head_dim)
    if args.window:
        pre, nxt = (int(x) for x in args.window.split(","))
        case.window = (pre, nxt)
        case.name += f"_window{pre}_{nxt}"
    if args.atten_mask is not None:
        rng = np.random.default_rng(case.seed + 2)
        sq, sk = (case.Sq, case.Skv) if case.layout == "BNSD" else (int(case.len_q.max()), int(case.len_kv.max()))
        case.atten_mask = (rng.random((sq, sk), dtype=np.float32) < args.atten_mask).astype(np.uint8)
        case.name += f"_attenmask{args.atten_mask:g}"
    blocks = active_blocks(case)
    fwd = args.op == "fwd"
    flops = (4.0 if fwd else 10.0) * case.bx * case.by * case.D * blocks
    print(f"# workload {case.name}: {blocks} active blocks, {flops / 1e9:.1f} GFLOP counted", file=sys.stderr, flush=True)

    dev = to_device(case)
    if args.fp8:
        case.name += "_fp8"
    dq_mode = {"recompute": 0, "atomic": 1}[args.dq_mode]
    if dq_mode and (fwd or args.fp8):
        print(json.dumps({"error": "--dq-mode atomic applies to the bf16/fp16 backward only"}))
        return 2
    if dq_mode:
        case.name += "_dqatomic"
    if fwd:
        o = lse = None
        if args.fp8:
            dev8, fac = quantize_inputs(dev, ("q", "k", "v"))
            run = FwdRunner(case, dev8, descale=[fac["q"], fac["k"], fac["v"]])
        else:
            run = FwdRunner(case, dev)
    else:
        o, lse = gpu_forward(case, dev)
        torch.cuda.synchronize()
        if args.fp8:
            dev["o"] = o
            dev8, fac = quantize_inputs(dev, ("do", "q", "k", "v", "o"))
            run = Runner(case, dev8, dev8["o"], lse, descale=[fac[k] for k in ("do", "q", "k", "v", "o")])
        else:
            run = Runner(case, dev, o, lse, dq_mode=dq_mode)
    stream = torch.cuda.current_stream()

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()

    # timed region: K whole calls with nothing else on the stream
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        run()
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    # per-call durations: K more calls, each between its own pair of events
    # (outside the timed region: events between calls add to the stream's time)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in evs:
        a.record(stream)
        run()
        b.record(stream)
    torch.cuda.synchronize()
    per_call = np.array([a.elapsed_time(b) for a, b in evs])
    p10, p50, p90 = (float(x) for x in np.percentile(per_call, [10, 50, 90]))
    clock_mhz = sustained_clock_mhz(run, torch, seconds=args.clock_seconds) if args.clock_seconds > 0 else None
    # per-kernel durations: K more calls with the library's HIP events between
    # its stages, on the launch stream (kept out of the timed region above,
    # since each event adds a few microseconds to the stream)
    bsa.bsa_profile_start(args.steps)
    for _ in range(args.steps):
        run()
    torch.cuda.synchronize()
    stage_ms, ncalls = bsa.bsa_profile_stop()
    ms = total_ms / args.steps
    tflops = flops / (ms * 1e-3) / 1e12
    print(f"# per call: median {p50:.4f} ms (p10 {p10:.4f}, p90 {p90:.4f}); clock {clock_mhz} MHz", file=sys.stderr,
          flush=True)
    print(f"# {ms:.4f} ms/step; stages (avg ms): " +
          ", ".join(f"{k}={v / max(1, ncalls):.4f}" for k, v in stage_ms.items()), file=sys.stderr, flush=True)

    # dominant kernel: dK/dV, credited with 4 of the 5 counted block GEMMs (S, dP, dV, dK);
    # the forward kernel for --op fwd, credited with both of its GEMMs (S, PV)
    # (with --dq-mode atomic the dK/dV kernel also forms dS K: all five); the
    # scheduled dK/dV build runs head dims up to 128 without an attenMask
    scheduled = case.D <= 128 and case.atten_mask is None and case.N // case.Nkv <= 256
    dk_name = "dkdv_pipe_kernel" if scheduled else "dkdv_kernel"
    kname, kstage, kflop = ("fwd_kernel", "fwd", 4.0) if fwd else (dk_name, "dkdv", 10.0 if dq_mode else 8.0)
    dkdv_ms = stage_ms[kstage] / max(1, ncalls)
    dkdv_flops = kflop * case.bx * case.by * case.D * blocks
    achieved = dkdv_flops / (dkdv_ms * 1e-3) / 1e12
    roofline = {
        "bound": "mfma",
        "achieved": round(achieved, 2),
        "peak": MFMA_PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / MFMA_PEAK_BF16_TFLOPS, 4),
        "traffic": traffic_from_profile(case.name, kname),
        "kernel": kname,
        "kernel_ms": round(dkdv_ms, 5),
        "stage_ms": {k: round(v / max(1, ncalls), 5) for k, v in stage_ms.items()},
    }

    cpu = None
    if not args.no_cpu:
        if fwd:
            cpu = cpu_baseline(case, None, None, op="fwd")
        else:
            o_h = o.float().cpu().numpy()
            l_h = lse.cpu().numpy()
            cpu = cpu_baseline(case, o_h, l_h)

    out = {
        "metric": ("fwd TFLOP/s over active blocks (4*bx*by*D per block) + % of MFMA peak, 1xMI355X" if fwd
                   else "bwd TFLOP/s over active blocks (bf16) + % of MFMA peak, 1xMI355X"),
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if args.fp8 else case.dtype,
        "data": "synthetic",
        "config": {
            "workload": case.name,
            "layout": case.layout, "B": case.B, "N": case.N, "Nkv": case.Nkv,
            "Sq": case.Sq, "Skv": case.Skv, "D": case.D, "block": [case.bx, case.by],
            "active_blocks": blocks, "gflop_counted": round(flops / 1e9, 3),
            "frac_of_mfma_peak": round(tflops / MFMA_PEAK_BF16_TFLOPS, 4),
            "parallelism": "single-gpu",
            "inputs": ("fp8: e4m3fn query/key/value/attentionOut, e5m2 dout, per-tensor factors"
                       if args.fp8 else case.dtype),
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "call_ms": {"median": round(p50, 5), "p10": round(p10, 5), "p90": round(p90, 5), "calls": args.steps,
                    "tflops_at_median": round(flops / (p50 * 1e-3) / 1e12, 3)},
        "clock": clock_report(clock_mhz, counter_clock_mhz(case.name, kname), tflops),
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

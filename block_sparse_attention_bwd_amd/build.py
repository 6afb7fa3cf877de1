"""Build the HIP shared library ``libbsa_bwd.so`` in-tree for gfx950.

Usage: ``python -m block_sparse_attention_bwd_amd.build`` (or ``build()``).
Always recompiles; writes the library next to this file atomically.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libbsa_bwd.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = os.environ.get("BSA_OFFLOAD_ARCH", "gfx950")

# (source, extra defines): translation units compiled in parallel.  The
# scheduled dK/dV source is compiled once per element type and head dim.
SOURCES = [
    ("bsa_api.cpp", ()),
    ("bsa_prologue.hip", ()),
    ("bsa_dkdv.hip", ()),
    ("bsa_dkdv_am.hip", ()),
    *[("bsa_dkdv_pipe.hip", (f"BSA_PIPE_BF16={e}", f"BSA_PIPE_D={d}")) for e in (1, 0) for d in (128, 64)],
    ("bsa_dq.hip", ()),
    ("bsa_fwd.hip", ()),
]


def _jobs() -> int:
    n = os.environ.get("MAX_JOBS")
    if n and n.isdigit() and int(n) > 0:
        return int(n)
    return max(1, min(len(SOURCES), os.cpu_count() or 1))


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def compile_flags() -> list:
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-Wall",
        # packed fp32 VALU ops stay off: the compiler would otherwise form them
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE,
        "-I", CSRC,
    ]


def build(verbose: bool = False, out: str = LIB_PATH, csrc: str = CSRC, defines=()) -> str:
    hipcc = _hipcc()
    with tempfile.TemporaryDirectory(prefix="bsa_build_") as tmp:
        def compile_one(i):
            src, extra = SOURCES[i]
            obj = os.path.join(tmp, f"{i:02d}_" + os.path.splitext(src)[0] + ".o")
            cmd = [hipcc, *compile_flags(), *[f"-D{d}" for d in (*defines, *extra)], "-I", csrc, "-c",
                   os.path.join(csrc, src), "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
            return src, cmd, r.returncode, err, obj

        with ThreadPoolExecutor(max_workers=_jobs()) as pool:
            results = list(pool.map(compile_one, range(len(SOURCES))))
        objs = []
        for src, cmd, rc, err, obj in results:
            if verbose:
                print(" ".join(cmd), flush=True)
            if rc != 0:
                raise RuntimeError(f"compiling {src} failed:\n{err}")
            if verbose and err.strip():
                print(err, file=sys.stderr)
            objs.append(obj)
        out_tmp = os.path.join(tmp, LIB_NAME)
        cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out_tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"linking {LIB_NAME} failed:\n{r.stderr}")
        shutil.copyfile(out_tmp, out + ".tmp")
        os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

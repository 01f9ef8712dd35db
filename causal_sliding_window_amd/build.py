"""Build libswattn.so in-tree with hipcc for gfx950.

Usage: ``python -m causal_sliding_window_amd.build`` (or ``build()`` from Python).
Every call recompiles; the result is ``causal_sliding_window_amd/libswattn.so``.
"""

from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libswattn.so")
SOURCES = ["api.hip", "fwd_bf16.hip", "bwd_bf16.hip", "dkdv_bf16.hip", "decode.hip", "f32.hip",
           "prologue.hip", "noalloc.hip", "probe.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # no packed-fp32 instructions anywhere (they are avoided on this hardware)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    # per-kernel register / scratch report, checked below
    "-Rpass-analysis=kernel-resource-usage",
]
# Per-source extra flags.  The kernels keep MFMA results in arch VGPRs, where they
# feed ALU work (avoids accumulator <-> VGPR copies).
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
EXTRA_FLAGS = {s: VGPR_FORM for s in SOURCES}
# The forward's row maxima and the dK/dV pass's largest P are taken over MFMA results
# and exponentials, which are never NaN.  Without this flag every fmaxf operand is
# first quieted (one extra v_max per element) and the three-input v_max3 is not formed.
EXTRA_FLAGS["fwd_bf16.hip"] = VGPR_FORM + ["-fno-honor-nans"]
EXTRA_FLAGS["dkdv_bf16.hip"] = VGPR_FORM + ["-fno-honor-nans"]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; ROCm is required to build libswattn")
    return exe


def resource_report(remarks: str) -> dict:
    """Per-kernel resource figures from the compiler's kernel-resource-usage remarks."""
    kernels, cur = {}, None
    for line in remarks.splitlines():
        if "remark:" not in line:
            continue
        body = line.split("remark:", 1)[1].split("[-Rpass", 1)[0].strip()
        if body.startswith("Function Name:"):
            cur = kernels.setdefault(body.split(":", 1)[1].strip(), {})
        elif cur is not None and ":" in body:
            key, val = body.rsplit(":", 1)
            cur[key.strip()] = val.strip()
    return kernels


def check_resources(source: str, kernels: dict) -> list:
    """Kernels that spill vector registers or use per-lane scratch memory: every kernel
    must run without either (that traffic goes to HBM on every launch).  Scalar
    spills into vector-register lanes (scratch 0) stay on chip and are allowed."""
    bad = []
    for name, r in kernels.items():
        scratch = int(r.get("ScratchSize [bytes/lane]", "0") or 0)
        spills = int(r.get("VGPRs Spill", "0") or 0)
        if scratch or spills:
            bad.append(f"{source}: {name}: scratch {scratch} B/lane, {spills} spilled VGPRs")
    return bad


def build(verbose: bool = False, csrc: str = CSRC, out: str = LIB) -> str:
    """Compile every source to an object (in parallel), then link the library.  Fails
    when a kernel spills registers or uses scratch memory."""
    noise = "not a recognized feature for this target"
    with tempfile.TemporaryDirectory(prefix="swattn_build_") as tmpdir:
        procs, objs = [], []
        for s in [s for s in SOURCES if os.path.exists(os.path.join(csrc, s))]:
            obj = os.path.join(tmpdir, s + ".o")
            cmd = [hipcc(), *HIPCC_FLAGS, *EXTRA_FLAGS.get(s, []), "-I", INCLUDE, "-I", csrc, "-c",
                   os.path.join(csrc, s), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((s, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                              text=True)))
            objs.append(obj)
        errors = []
        for s, p in procs:
            _, err = p.communicate()
            err = "\n".join(l for l in err.splitlines() if noise not in l)
            if p.returncode != 0:
                errors.append(f"{s}: hipcc failed ({p.returncode}):\n{err}")
                continue
            kernels = resource_report(err)
            errors.extend(check_resources(s, kernels))
            if verbose:
                for name, r in kernels.items():
                    print(f"{s}: {name[:60]}: VGPRs {r.get('VGPRs')} AGPRs {r.get('AGPRs')} "
                          f"LDS {r.get('LDS Size [bytes/block]')} occupancy "
                          f"{r.get('Occupancy [waves/SIMD]')}", file=sys.stderr)
                rest = "\n".join(l for l in err.splitlines()
                                 if "remark:" not in l and not re.match(r"\s*(\d+ )?\|", l))
                if rest.strip():
                    print(rest, file=sys.stderr)
        if errors:
            raise RuntimeError("\n".join(errors))
        tmp = out + ".tmp"
        cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed ({res.returncode}):\n{res.stderr}")
        os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))

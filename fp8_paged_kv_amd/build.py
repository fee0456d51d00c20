"""Compile the HIP library for gfx950 (hipcc, in-tree)."""
from __future__ import annotations

import os
import re
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libpa_fp8.so")
SOURCES = ["pa_fp8_decode.hip", "pa_fp8_decode_rows.hip", "pa_fp8_prefill.hip", "pa_fp8_mla.hip", "pa_fp8_cache.hip", "pa_fp8_epilog.hip",
           "pa_fp8_api.hip"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


# Per-source extra flags.  The whole-row kernels unroll a whole tile so that its
# scores stay in statically indexed registers; LLVM's default size cap for
# "#pragma unroll" would stop that.  Their MFMA accumulators are kept in
# architectural VGPRs: left to its heuristics the compiler keeps O in VGPRs
# between steps and copies it to AGPRs and back around every P.V step
# (64 extra moves per step).
EXTRA = {"pa_fp8_decode_rows.hip": ["-mllvm", "-pragma-unroll-threshold=1000000", "-mllvm", "-amdgpu-mfma-vgpr-form"]}


PHASES_LIB = os.path.join(PKG, "libpa_fp8_phases.so")


def build_phases() -> str:
    """The phase-stamp variant of the library (the same results; the decode and MLA
    kernels also record per-workgroup phase times for bench.py --op phases);
    writes fp8_paged_kv_amd/libpa_fp8_phases.so."""
    return build(lib_path=PHASES_LIB, defines=["-DPA_FP8_PHASES"], objsub="_build_phases")


def build(verbose: bool = False, lib_path: str = LIB, defines=(), objsub: str = "_build") -> str:
    """Always recompiles; writes fp8_paged_kv_amd/libpa_fp8.so."""
    objdir = os.path.join(PKG, objsub)
    os.makedirs(objdir, exist_ok=True)
    base = [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
            # packed FP32 instructions stay off (ordinary scalar float code only)
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Rpass-analysis=kernel-resource-usage",
            "-I", os.path.join(ROOT, "include")]
    procs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = base + list(defines) + EXTRA.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    remarks = []
    for src, pr in procs:
        out, err = pr.communicate()
        if pr.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n" + out + err)
        remarks.append(err)
    spills = scratch_kernels("\n".join(remarks))
    if spills:
        print("warning: kernels using scratch (register spills): " + ", ".join(spills))
    if verbose:
        print("\n".join(remarks))
    tmp = lib_path + ".tmp"
    r = subprocess.run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs,
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib_path)
    return lib_path


PROBE_SRC = os.path.join(CSRC, "probe", "pa_probe_stream.hip")
PROBE_LIB = os.path.join(PKG, "libpa_probe.so")


def build_probe() -> str:
    """Always recompiles the bandwidth probes (a measurement tool beside the decode
    library, not part of its ABI); writes fp8_paged_kv_amd/libpa_probe.so."""
    tmp = PROBE_LIB + ".tmp"
    r = subprocess.run([hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", PROBE_SRC, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on the probes:\n" + r.stdout + r.stderr)
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def scratch_kernels(remarks: str) -> list:
    """Names of kernels whose resource-usage remark reports a nonzero ScratchSize."""
    out, name = [], None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name and int(m.group(1)) > 0:
            out.append(f"{name} ({m.group(1)} B/lane)")
    return out


if __name__ == "__main__":
    print(build())
    print(build_probe())
    print(build_phases())

"""Build the HIP library libkvp.so for gfx950, in-tree (next to this file).

hipcc cross-compiles for gfx950 without a GPU.  Every HIP translation unit is compiled
with packed-FP32 instruction selection turned off.
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libkvp.so")
SOURCES = ["kvp_manager.cpp", "kvp_plan.cpp", "kvp_sched.cpp", "kvp_cache_ops.hip", "kvp_decode.hip", "kvp_decode_f16.hip",
           "kvp_decode_f32.hip", "kvp_prefill.hip", "kvp_probe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# per-source flags: the decode kernels take the plan-record pointer as their first argument
# and have the dispatcher preload it (two SGPRs), so a wave's first instruction is its record
# load rather than a kernel-argument fetch
EXTRA_FLAGS = {"kvp_decode_f16.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=2"]}
ARCH = "gfx950"


def hip_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # MFMA accumulators in ordinary VGPRs: no copies between accumulation registers
            # and VGPRs around the VALU work on scores and outputs
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            # fp32 division and square root correctly rounded (the int8 codes are decided by
            # an fp32 division and must match the definition bit for bit)
            "-fhip-fp32-correctly-rounded-divide-sqrt",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def build(verbose=False, jobs=4):
    objs = []
    procs = []
    for src in SOURCES:
        obj = os.path.join(CSRC, "_build", src + ".o")
        os.makedirs(os.path.dirname(obj), exist_ok=True)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [HIPCC] + hip_flags() + EXTRA_FLAGS.get(src, []) + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
        if len([p for _, p in procs if p.poll() is None]) >= jobs:
            procs[0][1].wait()
    failed = False
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # the host pass does not know the packed-fp32 feature; that note is harmless
        text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
        if text.strip() and (verbose or p.returncode):
            print(f"[{src}]\n{text}", flush=True)
        failed |= p.returncode != 0
    if failed:
        raise RuntimeError("HIP build failed")
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", LIB + ".tmp"] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print("built", LIB)

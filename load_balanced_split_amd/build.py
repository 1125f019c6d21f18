"""Build libhpa.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc."""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
SOURCES = ["plan.hip", "attn.hip", "prologue.hip", "probe.hip", "router.hip", "noalloc.hip", "pack.hip", "moe.hip", "host.cpp",
           "router_host.cpp"]
# Packed-fp32 VALU ops are kept out of every kernel (the compiler would otherwise
# form v_pk_* from scalar float code). The atomic optimizer is off: it turns a
# one-lane counter update into a wave reduction that waits for the returned value
# at once (s_waitcnt vmcnt(0)), which would drain the K/V stream in flight at
# every work claim; without it the wait lands where the value is used.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
         # leading scalar kernel arguments arrive in SGPRs at dispatch
         "-mllvm", "-amdgpu-kernarg-preload-count=16",
         "-I", INCLUDE, "-I", CSRC]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


# Library variants: the product build, the instrumented build (per-wave realtime
# stamps and CU ids of the attention kernels) and the comparison build whose
# attention kernels compute Q.K^T and P.V with VALU dot products instead of MFMA.
VARIANTS = {
    "product": ("libhpa.so", "_build", []),
    "trace": ("libhpa_trace.so", "_build_trace", ["-DHPA_TRACE=1"]),
    "valu": ("libhpa_valu.so", "_build_valu", ["-DHPA_VALU_PRODUCTS=1"]),
}
TRACE_LIB = os.path.join(PKG, VARIANTS["trace"][0])


def build(verbose: bool = False, trace: bool = False, variant: str = "product") -> str:
    """Compile one variant of the library (trace=True is variant "trace")."""
    cc = hipcc()
    name, objdir, extra = VARIANTS["trace" if trace else variant]
    objdir = os.path.join(PKG, objdir)
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [cc, *FLAGS, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{out}")
        if verbose and out.strip():
            print(out, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    target = os.path.join(PKG, name)
    tmp = target + ".tmp"
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, target)
    return target


if __name__ == "__main__":
    for v in VARIANTS:
        print(build(verbose=True, variant=v))

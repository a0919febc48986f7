"""Build the HIP library in place: mla_latent_kv_26_amd/libmla_latent_kv.so.

Compiles every source under csrc/ for gfx950 with hipcc (one process per
source, in parallel), then links them.  Packed-fp32 VALU instructions are
disabled for all device code; kernel arguments are preloaded into scalar
registers where the hardware supports it.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmla_latent_kv.so")
ARCH = os.environ.get("MLA_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # leading kernel arguments arrive in scalar registers at wave
         # launch instead of through a scalar load each kernel starts with
         "-mllvm", "-amdgpu-kernarg-preload-count=16",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines()
            if "packed-fp32-ops" not in ln and ln.strip()]
    return r.returncode, msgs


def build(verbose: bool = False, out: str = LIB, jobs: int = 0) -> str:
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 1)))
    with tempfile.TemporaryDirectory(prefix="mla_build_") as tmp:
        objs = [os.path.join(tmp, os.path.basename(s) + ".o") for s in srcs]
        cmds = [[HIPCC, *FLAGS, "-x", "hip", "-c", s, "-o", o] for s, o in zip(srcs, objs)]
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        with ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(_run, cmds))
        for (rc, msgs), s in zip(results, srcs):
            if rc != 0:
                raise RuntimeError(f"hipcc failed on {s}:\n" + "\n".join(msgs))
            if verbose and msgs:
                print("\n".join(msgs), file=sys.stderr)
        tmp_lib = out + ".tmp"
        link = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        if verbose:
            print(" ".join(link), flush=True)
        rc, msgs = _run(link)
        if rc != 0:
            raise RuntimeError("link failed:\n" + "\n".join(msgs))
    os.replace(tmp_lib, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))

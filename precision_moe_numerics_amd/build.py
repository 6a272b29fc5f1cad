"""Build libnvq.so (the gfx950 HIP kernels and their C ABI) in-tree with hipcc.

    python -m precision_moe_numerics_amd.build

Flags that the numerics depend on:
  -ffp-contract=off     no silent fused multiply-adds: codes and scales are
                        decided by fp32 operation sequences that must round
                        exactly as written;
  -packed-fp32-ops off  no v_pk_*_f32 generated for fp32 code.
Denormals stay enabled (the HIP default) and fp32 division stays correctly
rounded (the HIP default).
"""
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libnvq.so")
ARCH = os.environ.get("NVQ_OFFLOAD_ARCH", "gfx950")

FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include")]


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile each .hip to an object in parallel, then link libnvq.so."""
    objdir = os.path.join(ROOT, "_build", "nvq")
    os.makedirs(objdir, exist_ok=True)
    procs, objs = [], []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = ["hipcc", *[f for f in FLAGS if f != "-shared"], "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        if len(procs) >= jobs:
            _drain(procs)
    _drain(procs)
    tmp = LIB + ".tmp"
    link = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(tmp, LIB)
    return LIB


def _drain(procs):
    errors = []
    while procs:
        src, p = procs.pop(0)
        out, _ = p.communicate()
        if p.returncode != 0:
            errors.append(f"{src}:\n{out}")
        elif out.strip():
            filtered = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
            if filtered:
                print("\n".join(filtered), file=sys.stderr)
    if errors:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errors))


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

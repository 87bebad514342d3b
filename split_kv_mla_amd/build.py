"""Build the HIP library in-tree: split_kv_mla_amd/libmla_split_kv.so for gfx950."""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmla_split_kv.so")
SOURCES = [os.path.join(HERE, "csrc", "mla_split_kv.hip"), os.path.join(HERE, "csrc", "mla_merge.hip"),
           os.path.join(HERE, "csrc", "mla_gather.hip")]
HEADERS = [os.path.join(HERE, "csrc", "mla_kernels.h"), os.path.join(HERE, "csrc", "mla_plan.h"),
           os.path.join(HERE, "csrc", "mla_merge.h"), os.path.join(HERE, "csrc", "mla_gather.h"),
           os.path.join(ROOT, "include", "mla_split_kv.h")]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def command(out=LIB, extra=()):
    return [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
            # keep packed-fp32 instructions out of the generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
            # assembly output (-S) is one file: the decode kernels' translation unit
            *extra, *(SOURCES[:1] if "-S" in extra else SOURCES), "-o", out]


def build(verbose=False):
    cmd = command()
    tmp = LIB + ".tmp"
    cmd[-1] = tmp
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libmla_split_kv.so")
    if verbose:
        sys.stderr.write(res.stderr)
    os.replace(tmp, LIB)
    return LIB


def assembly(out_path):
    """Device assembly of the library for inspection."""
    cmd = command(out=out_path, extra=("--cuda-device-only", "-S"))
    cmd.remove("-shared")
    subprocess.run(cmd, check=True, capture_output=True)
    return out_path


if __name__ == "__main__":
    print(build(verbose=True))

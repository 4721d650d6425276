"""Build libq8kv.so for gfx950 in-tree with hipcc (no GPU needed)."""
from __future__ import annotations

import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
OUT = os.path.join(HERE, "libq8kv.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed-fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I" + INCLUDE,
]


# Per-file additions.  The prefill kernel keeps its matrix-core accumulators
# in VGPRs (the MFMAs read and write them there), so the rare rescale of the
# accumulators does not make the compiler copy them between register files
# on every key tile.
FILE_FLAGS = {
    "q8kv_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; drop that noise
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err)


def build(verbose: bool = False, extra=(), out: str = OUT, link_extra=()) -> str:
    """Compile every source to an object (in parallel, with its own flags),
    then link the shared library (at `out`; `extra` and `link_extra` are added
    to every compile and to the link)."""
    import tempfile
    from concurrent.futures import ThreadPoolExecutor

    srcs = sources()
    with tempfile.TemporaryDirectory(prefix="q8kv_build_") as tmp:
        objs = [os.path.join(tmp, os.path.basename(f) + ".o") for f in srcs]
        compile_flags = [f for f in FLAGS if f != "-shared"]
        cmds = [[HIPCC, *compile_flags, *FILE_FLAGS.get(os.path.basename(f), []), *extra, "-c", "-o", o, f]
                for f, o in zip(srcs, objs)]
        with ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
            for fut in [ex.submit(_run, c, verbose) for c in cmds]:
                fut.result()
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *link_extra, "-o", out + ".tmp", *objs], verbose)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))

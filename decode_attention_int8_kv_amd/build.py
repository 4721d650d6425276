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


# Every compile reports each kernel's registers, spills, scratch, LDS and
# occupancy; build() gathers them into RESOURCES (a function that stops being
# inlined shows up there as a scratch frame and a jump in VGPRs).
REMARKS = "-Rpass-analysis=kernel-resource-usage"
RESOURCES = os.path.join(HERE, "libq8kv.resources.json")
_FIELDS = {
    "VGPRs": "vgprs", "AGPRs": "agprs", "TotalSGPRs": "sgprs", "ScratchSize [bytes/lane]": "scratch",
    "Occupancy [waves/SIMD]": "occupancy", "SGPRs Spill": "sgpr_spill", "VGPRs Spill": "vgpr_spill",
    "LDS Size [bytes/block]": "lds",
}


def parse_resource_remarks(text: str) -> dict:
    """{kernel symbol: {field: int}} from hipcc's kernel-resource-usage remarks."""
    out, cur = {}, None
    for line in text.splitlines():
        if "remark:" not in line or "kernel-resource-usage" not in line:
            continue
        body = line.split("remark:", 1)[1].rsplit("[-Rpass", 1)[0].strip()
        key, _, val = body.partition(":")
        key, val = key.strip(), val.strip()
        if key == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None and key in _FIELDS:
            try:
                cur[_FIELDS[key]] = int(val)
            except ValueError:
                pass
    return out


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; drop that
    # noise, and the resource remarks (returned, not printed)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l and "kernel-resource-usage" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err)
    return r.stderr


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
        cmds = [[HIPCC, *compile_flags, *FILE_FLAGS.get(os.path.basename(f), []), *extra, REMARKS,
                 "-c", "-o", o, f] for f, o in zip(srcs, objs)]
        resources = {}
        with ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
            for src, fut in zip(srcs, [ex.submit(_run, c, verbose) for c in cmds]):
                for k, v in parse_resource_remarks(fut.result()).items():
                    resources[k] = dict(v, source=os.path.basename(src))
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *link_extra, "-o", out + ".tmp", *objs], verbose)
    os.replace(out + ".tmp", out)
    if out == OUT:
        import json
        with open(RESOURCES + ".tmp", "w") as f:
            json.dump(resources, f, indent=1, sort_keys=True)
        os.replace(RESOURCES + ".tmp", RESOURCES)
    return out


if __name__ == "__main__":
    print(build(verbose=True))

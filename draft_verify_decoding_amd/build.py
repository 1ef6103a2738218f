"""Build libisd.so (all HIP sources, gfx950) in place next to this file."""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = ["isd_runtime.hip", "isd_attention.hip", "isd_accept.hip", "isd_linear.hip", "isd_forward.hip"]
LIB = os.path.join(HERE, "libisd.so")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function",
    # no packed-FP32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build(verbose=False):
    """Compile every source to an object (in parallel, one hipcc each), then
    link them into libisd.so."""
    from concurrent.futures import ThreadPoolExecutor
    import tempfile

    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    incs = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]
    compile_flags = [f for f in FLAGS if f != "-shared"]
    noise = "is not a recognized feature for this target"
    tmp = LIB + ".tmp"
    with tempfile.TemporaryDirectory(dir=HERE, prefix="_build") as obj_dir:
        def run(cmd):
            if verbose:
                print(" ".join(cmd), flush=True)
            res = subprocess.run(cmd, capture_output=True, text=True)
            err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
            if res.returncode != 0:
                raise RuntimeError("hipcc failed:\n" + err)
            if err.strip() and verbose:
                print(err, file=sys.stderr)

        objs = [os.path.join(obj_dir, s.replace(".hip", ".o")) for s in SOURCES]
        cmds = [[hipcc, *compile_flags, *incs, "-c", os.path.join(HERE, "csrc", s), "-o", o]
                for s, o in zip(SOURCES, objs)]
        with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1)) as ex:
            list(ex.map(run, cmds))
        run([hipcc, "--offload-arch=gfx950", "-fPIC", "-shared", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

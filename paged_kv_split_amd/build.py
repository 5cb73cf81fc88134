"""Compile the HIP library libpdattn.so for gfx950, in-tree.

    python paged_kv_split_amd/build.py
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIBRARY = os.path.join(HERE, "libpdattn.so")
SOURCES = [os.path.join(CSRC, "pdattn.hip"), os.path.join(CSRC, "decode_kernels.hip"),
           os.path.join(CSRC, "decode_stream.hip"),
           os.path.join(CSRC, "decode_dynamic.hip"), os.path.join(CSRC, "stream_read.hip"),
           os.path.join(CSRC, "kv_append.hip"), os.path.join(CSRC, "merge.hip"),
           os.path.join(CSRC, "prefill.hip"), os.path.join(CSRC, "tq4.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Per-source flags. The decode kernels keep their MFMA accumulators in VGPRs:
# the tile loop rescales them on the VALU, and with AGPR accumulators the
# compiler copies all of them between register files on every tile.
SOURCE_FLAGS = {
    "decode_kernels.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "decode_stream.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "decode_dynamic.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-fvisibility=hidden",
    # packed fp32 VALU forms stay off: ordinary scalar fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Werror=array-bounds",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 target feature; that
    # warning is expected and harmless
    lines = [ln for ln in res.stdout.splitlines() if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines))


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile each source to an object in parallel, then link the library."""
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.basename(src) + ".o") for src in SOURCES]
    cflags = [f for f in FLAGS if f != "-shared"] + list(extra_flags)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        futs = [ex.submit(_run, [HIPCC] + cflags + SOURCE_FLAGS.get(os.path.basename(src), []) + ["-c", src, "-o", obj],
                          verbose)
                for src, obj in zip(SOURCES, objs)]
        for f in futs:
            f.result()
    tmp = LIBRARY + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp], verbose)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True, extra_flags=sys.argv[1:]))

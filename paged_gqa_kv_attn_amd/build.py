"""Build ``libdecode_attn.so`` (the C-ABI library with the gfx950 HIP kernels) in-tree.

    python -m paged_gqa_kv_attn_amd.build

Every call recompiles. Objects go to ``paged_gqa_kv_attn_amd/_build/``; the library is written
next to this file, where ``binding.load_library`` finds it.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdecode_attn.so")
SOURCES = ["decode_attn.cpp", "stage1.hip", "prefill.hip", "stage2.hip", "append.hip",
           "append_rope.hip", "noalloc.hip", "stage1_ks.hip"]
ARCH = "gfx950"

# Packed-FP32 VALU instructions are kept out of the generated code.
COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH, "-Wall", "-Wextra",
                "-Wno-unused-parameter", "-Xclang", "-target-feature", "-Xclang",
                "-packed-fp32-ops", "-I" + os.path.join(os.path.dirname(HERE), "include")]


def _hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


# Per-source flags. The prefill and stage-1 kernels keep their MFMA accumulators in ordinary VGPRs:
# with the default heuristics the output accumulators live in AGPRs for the MFMAs and in VGPRs for
# the softmax rescale, and the compiler copies the output block between the two register files on
# every loop step (stage 1: 32 copies per step at head_dim 512, 208 with two row groups).
SOURCE_FLAGS = {"prefill.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"],
                "stage1.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"]}


def _compile(src: str, extra=()) -> str:
    obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
    cmd = ([_hipcc()] + COMMON_FLAGS + SOURCE_FLAGS.get(src, []) + list(extra) +
           ["-c", os.path.join(CSRC, src), "-o", obj])
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s\n%s" % (src, " ".join(cmd), res.stderr))
    # The host pass does not know the GPU-only feature flag; drop that one harmless warning.
    noise = "'-packed-fp32-ops' is not a recognized feature"
    warn = "\n".join(l for l in res.stderr.splitlines() if noise not in l).strip()
    if warn:
        sys.stderr.write(warn + "\n")
    return obj


def build(extra_flags=(), out=None, obj_dir=None) -> str:
    """Compile all sources and link the shared library; returns its path. ``extra_flags`` (e.g.
    "-DDECODE_ATTN_STAGE1_SUB=2") and ``out``/``obj_dir`` serve A/B builds of variants."""
    global OBJ_DIR
    lib = out or LIB
    saved = OBJ_DIR
    OBJ_DIR = obj_dir or OBJ_DIR
    os.makedirs(OBJ_DIR, exist_ok=True)
    try:
        with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
            objs = list(ex.map(lambda s: _compile(s, extra_flags), SOURCES))
    finally:
        OBJ_DIR = saved
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH] + objs + ["-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), res.stderr))
    os.replace(tmp, lib)
    if out is None:
        _write_build_info()
        build_copy_rate()
    return lib


COPY_RATE = os.path.join(HERE, "copy_rate")


def build_copy_rate() -> str:
    """Compile the standalone copy-rate program (``csrc/copy_rate.hip``, not part of the library):
    the copy and read-only bandwidth the part reaches, which ``bench.py --copy-rate`` reports."""
    tmp = COPY_RATE + ".tmp%d" % os.getpid()
    cmd = ([_hipcc(), "-x", "hip"] + [f for f in COMMON_FLAGS if f != "-fPIC"] +
           [os.path.join(CSRC, "copy_rate.hip"), "-o", tmp])
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed on copy_rate.hip:\n%s\n%s" % (" ".join(cmd), res.stderr))
    os.replace(tmp, COPY_RATE)
    return COPY_RATE


def _write_build_info() -> None:
    """Record the source revision next to the library (``_build_info.json``), so that a copy of
    the tree without its repository still tells which revision the library was built from."""
    import json
    root = os.path.dirname(HERE)
    info = {"git_sha": None, "git_dirty": None}
    try:
        sha = subprocess.run(["git", "-C", root, "rev-parse", "HEAD"], capture_output=True,
                             text=True, timeout=10)
        if sha.returncode == 0:
            dirty = subprocess.run(["git", "-C", root, "status", "--porcelain",
                                    "--untracked-files=no"], capture_output=True, text=True,
                                   timeout=10)
            info = {"git_sha": sha.stdout.strip(), "git_dirty": bool(dirty.stdout.strip())}
    except (OSError, subprocess.SubprocessError):
        pass
    with open(os.path.join(HERE, "_build_info.json"), "w") as f:
        json.dump(info, f)


if __name__ == "__main__":
    print(build())

"""Build libmoe_decode.so in-tree with hipcc for gfx950.

    python -m moe_decode_amd.build              # the library
    python -m moe_decode_amd.build --sanitize   # libmoe_decode_san.so: host code
                                                # with ASan + UBSan (CPU tests only)
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
OUT = os.path.join(HERE, "libmoe_decode.so")
OUT_SAN = os.path.join(HERE, "libmoe_decode_san.so")
BUILD = os.path.join(HERE, "_build")
BUILD_SAN = os.path.join(HERE, "_build_san")

SOURCES = ["gemv.hip", "decode.hip", "route.hip", "prefill.hip", "abi.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions (v_pk_fma_f32 and friends) anywhere
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-pass-failed",
    "-I", os.path.join(ROOT, "include"),
]
# host-side sanitizers only (the device code is built as usual)
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
SAN_LINK = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libsan"]


def _compile(src, build_dir=BUILD, defines=(), extra=()):
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC] + FLAGS + list(extra) + [f"-D{d}" for d in defines] + lang + ["-c", os.path.join(CSRC, src), "-o",
                                                                               obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    warn = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    return obj, warn


def build(verbose=False, out=None, build_dir=None, defines=(), sanitize=False):
    """Compile every source and link the shared library (out); `defines` are
    extra -D settings of the kernels' compile-time parameters; sanitize: host
    code with AddressSanitizer + UndefinedBehaviorSanitizer (a process that
    loads it must preload the clang ASan runtime)."""
    out = out or (OUT_SAN if sanitize else OUT)
    build_dir = build_dir or (BUILD_SAN if sanitize else BUILD)
    extra = SAN_FLAGS if sanitize else []
    os.makedirs(build_dir, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(lambda s: _compile(s, build_dir, defines, extra), srcs))
    objs = [o for o, _ in results]
    if verbose:
        for (_, w), s in zip(results, srcs):
            if w:
                print(f"--- {s}\n{w}")
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + (SAN_LINK if sanitize else []) + ["-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    if not sanitize and out == OUT:
        _write_build_info(srcs)
    return out


BUILD_INFO = os.path.join(HERE, "build_info.json")


def _write_build_info(srcs):
    """The commit and source hash the library was built from, beside it (the
    library travels without the repository's history)."""
    import hashlib
    import json
    sha = None
    try:
        r = subprocess.run(["git", "rev-parse", "HEAD"], cwd=os.path.dirname(HERE), capture_output=True, text=True,
                           timeout=10)
        sha = r.stdout.strip() or None
        d = subprocess.run(["git", "status", "--porcelain", "--", "moe_decode_amd/csrc", "include"],
                           cwd=os.path.dirname(HERE), capture_output=True, text=True, timeout=10)
        dirty = bool(d.stdout.strip())
    except (OSError, subprocess.SubprocessError):
        dirty = None
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        h.update(name.encode())
        h.update(open(os.path.join(CSRC, name), "rb").read())
    with open(BUILD_INFO, "w") as f:
        json.dump({"git_sha": sha, "sources_differ_from_commit": dirty, "csrc_sha256": h.hexdigest()}, f)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))

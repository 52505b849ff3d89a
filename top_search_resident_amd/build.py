"""Build libresident_topk.so for gfx950 with hipcc, in-tree.

Each HIP source is compiled to an object in parallel, then linked into
``top_search_resident_amd/libresident_topk.so``.  Packed-fp32 instructions are
disabled on every device compile.
"""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIBRARY = os.path.join(HERE, "libresident_topk.so")
SOURCES = ["engine.hip", "stream_topk.hip", "mfma_scores.hip", "batch_select.hip", "filter_topk.hip", "mfma_filter.hip", "filter8.hip", "read_probe.hip", "select_static.hip", "batcher.hip", "validate.cpp"] + \
    [f"stream_r{r}{m}.hip" for r in (16, 8, 4, 2, 1) for m in ("", "c")] + \
    [f"filter_r{r}.hip" for r in (16, 8, 4, 2, 1)]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include")]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    return res


def _newest_dependency(path, seen=None):
    """Latest modification time of `path` and of the local headers it includes
    (#include "..."), recursively."""
    seen = set() if seen is None else seen
    if path in seen or not os.path.exists(path):
        return 0.0
    seen.add(path)
    newest = os.path.getmtime(path)
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line.startswith("#include \""):
                inc = os.path.normpath(os.path.join(os.path.dirname(path), line.split('"')[1]))
                newest = max(newest, _newest_dependency(inc, seen))
    return newest


def build(verbose=False, force=True):
    """Compile every source (force=True, what the build check runs) or only the
    objects older than their source or any header (force=False), then link."""
    os.makedirs(BUILD_DIR, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        path = os.path.join(CSRC, src)
        if not force and os.path.exists(obj) and os.path.getmtime(obj) > _newest_dependency(path):
            return obj
        _run([HIPCC, *FLAGS, "-c", path, "-o", obj])
        return obj

    with ThreadPoolExecutor(max(1, min(len(SOURCES), os.cpu_count() or 1))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIBRARY + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIBRARY)
    if verbose:
        print("built", LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    import sys
    build(verbose=True, force="--changed" not in sys.argv)

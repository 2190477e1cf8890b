"""Build libmoe.so in-tree from csrc/*.hip with hipcc for gfx950."""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe.so")
ARCH = "gfx950"

FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    # no packed fp32 arithmetic anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src, extra=()):
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = ["hipcc", *FLAGS, *extra, "-c", src, "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    return src, obj, p.returncode, p.stdout + p.stderr


def build(verbose: bool = False, defines=(), out=LIB) -> str:
    """Compile every csrc/*.hip and link `out`.  defines: extra -D flags
    (tuning experiments)."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    extra = tuple("-D" + d for d in defines)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(lambda s: _compile(s, extra), srcs))
    errs = []
    for src, obj, rc, log in results:
        # the host pass does not know the gfx950 feature flag; that note is noise
        noise = "is not a recognized feature for this target"
        lines = [l for l in log.splitlines() if noise not in l]
        if rc != 0:
            errs.append(f"--- {os.path.basename(src)} ---\n" + "\n".join(lines))
        elif verbose and lines:
            print("\n".join(lines), file=sys.stderr)
    if errs:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errs))
    tmp = out + ".tmp%d" % os.getpid()
    p = subprocess.run(["hipcc", "--offload-arch=" + ARCH, "-shared", "-fPIC",
                        *[o for _, o, _, _ in results], "-o", tmp],
                       capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError("link failed:\n" + p.stdout + p.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))

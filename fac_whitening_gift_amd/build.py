"""Build libgift.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: python -m fac_whitening_gift_amd.build   (or build() from Python).
Every source is compiled on every call; objects go to _build/ next to this
file and the library to fac_whitening_gift_amd/libgift.so.
"""

import hashlib
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgift.so")
# HBM streaming probes (include/gift_probe.h), a separate library used by
# bench.py --study stream; not part of libgift.so or its source hash
PROBE_SRC = os.path.join(CSRC, "probe", "stream.hip")
PROBE_LIB = os.path.join(HERE, "libgift_probe.so")
PROBE_HEADER = os.path.join(ROOT, "include", "gift_probe.h")
ARCH = "gfx950"

SOURCES = ["api.cpp", "roundtrip.hip", "roundtrip_rt2.hip", "refresh.hip"]

# -packed-fp32-ops: keep hipcc from forming packed fp32 VALU ops (the host
# pass does not know the feature and warns; that is expected).
HIPFLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
    "-I" + os.path.join(ROOT, "include"),
]


def source_hash():
    """First 16 hex digits of the SHA-256 of every source the library is
    built from (csrc/ and include/, in name order); compiled into the
    library and returned by gift_build_hash()."""
    h = hashlib.sha256()
    files = [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC))]
    files += [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))
              if f != os.path.basename(PROBE_HEADER)]
    for path in files:
        if os.path.isfile(path):
            h.update(os.path.basename(path).encode())
            with open(path, "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src, defines=()):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [hipcc()] + HIPFLAGS + list(defines) + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s" % (src, msgs))
    return obj, msgs


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    defines = ['-DGIFT_BUILD_HASH="%s"' % source_hash()]
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        results = list(ex.map(lambda src: _compile(src, defines), SOURCES))
    for _, msgs in results:
        if msgs.strip() and verbose:
            print(msgs, file=sys.stderr)
    objs = [o for o, _ in results]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    build_probe()
    return LIB


def build_probe():
    tmp = PROBE_LIB + ".tmp"
    cmd = [hipcc()] + HIPFLAGS + ["-shared", PROBE_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s" % (PROBE_SRC, r.stdout + r.stderr))
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


if __name__ == "__main__":
    print(build(verbose=True))

"""Compile the gfx950 HIP library libllmint8.so in-tree with hipcc.

Every .hip source under csrc/ is one translation unit of the shared library;
only the extern "C" entry points declared in include/llmint8.h are exported.
"""
from __future__ import annotations

import glob
import hashlib
import json
import os
import re
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libllmint8.so")
# per-kernel register use, scratch and occupancy reported by the compiler
RESOURCES = os.path.join(HERE, "libllmint8.kernels.json")
# what the library was built from: a digest of its sources, the compiler and flags
RECORD = os.path.join(HERE, "libllmint8.build.json")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fvisibility=hidden", "-Wall",
    # packed fp32 instructions stay off for every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Rpass-analysis=kernel-resource-usage",
]

_REMARK = re.compile(r"remark:\s+(Function Name|[A-Za-z ]+?)(?: \[[^\]]*\])?:\s+(\S+)\s+\[-Rpass")


def kernel_resources(stderr: str) -> dict:
    """{kernel symbol: {field: value}} from the kernel-resource-usage remarks."""
    out, cur = {}, None
    for line in stderr.splitlines():
        m = _REMARK.search(line)
        if not m:
            continue
        key, val = m.group(1).strip(), m.group(2)
        if key == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None:
            cur[key] = int(val) if val.isdigit() else val
    return out


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def source_digest() -> str:
    """sha256 over the library's sources: every file of csrc/ and the header."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.hpp")))
    files.append(os.path.join(INCLUDE, "llmint8.h"))
    for p in files:
        h.update(os.path.basename(p).encode() + b"\0")
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def file_digest(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def compiler_version() -> str:
    out = subprocess.run([HIPCC, "--version"], capture_output=True, text=True)
    lines = [l for l in out.stdout.splitlines() if "clang version" in l or "HIP version" in l]
    return "; ".join(lines)


def build(verbose: bool = False) -> str:
    cmd = [HIPCC, *FLAGS, "-I", INCLUDE, "-I", CSRC, *sources(), "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    noise = ("is not a recognized feature for this target", "-Rpass-analysis=kernel-resource",
             "remark:", "| ^", " | ")
    err = "\n".join(l for l in proc.stderr.splitlines() if not any(n in l for n in noise))
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(LIB + ".tmp", LIB)
    with open(RESOURCES, "w") as f:
        json.dump(kernel_resources(proc.stderr), f, indent=1, sort_keys=True)
    record = {"source_digest": source_digest(), "library_digest": file_digest(LIB),
              "compiler": compiler_version(), "flags": FLAGS,
              "built_at": time.strftime("%Y-%m-%dT%H:%M:%SZ", time.gmtime())}
    with open(RECORD, "w") as f:
        json.dump(record, f, indent=1)
    return LIB


def check_record() -> dict:
    """The build record of the library in the package, after checking that the
    library is the one recorded and that it was built from the sources as they
    are now. Raises ImportError otherwise (a stale or foreign library)."""
    if not os.path.exists(RECORD):
        raise ImportError(f"{RECORD} is missing: rebuild the HIP library")
    with open(RECORD) as f:
        record = json.load(f)
    if record.get("library_digest") != file_digest(LIB):
        raise ImportError(f"{LIB} is not the library its build record describes: rebuild it")
    if record.get("source_digest") != source_digest():
        raise ImportError(f"{LIB} was built from different sources than csrc/ holds: rebuild it")
    return record


if __name__ == "__main__":
    build(verbose=True)

"""Build libgemm.so (HIP kernels for gfx950 plus the C ABI) in-tree.

``python -m tiled_gemm_f32_amd.build`` compiles every source under csrc/
with hipcc for gfx950 and links them into tiled_gemm_f32_amd/libgemm.so.
Objects go to _build/ at the repository root.

Every kernel source is compiled with the compiler's kernel-resource remarks
on, and the per-kernel figures (registers, scratch, LDS, occupancy) are kept
in _build/kernel_resources.json together with a hash of the sources they
came from.  ``resource_usage()`` returns that table (recompiling the device
code of any source whose hash no longer matches), and
``python -m tiled_gemm_f32_amd.build --resources FILE`` writes it as a
Markdown summary.  A kernel whose accumulator tile or fragment registers do
not fit spills them to scratch memory, which costs a memory round trip per
access on the hot path ("Tiled matrix multiplication", "Implementation
notes" and "Pitfalls"); the table is how that is caught.
"""
from __future__ import annotations

import hashlib
import json
import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(HERE, "libgemm.so")

SOURCES = ["gemm_api.cpp", "gemm_f32_tiled.hip", "gemm_bf16_tiled.hip", "gemm_f32_skinny.hip", "gemm_fp8_tiled.hip",
           "gemm_general.hip", "gemm_bf16_skinny.hip", "gemm_skinny_nt.hip", "gemm_scratch.hip",
           "gemm_bf16_lines.hip", "gemm_fp8_lines.hip", "gemm_fp8_skinny.hip"]
HEADERS = ["gemm_device.hpp", "gemm_kernels.hpp", "gemm_lines.hpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU
# instructions; the host pass warns that it does not know the feature, which
# is harmless.
COMPILE_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-I", INCLUDE, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


RESOURCE_FILE = os.path.join(BUILD_DIR, "kernel_resources.json")
REMARK_FLAG = "-Rpass-analysis=kernel-resource-usage"


def source_hash(src: str) -> str:
    """sha256 over a kernel source and the headers every source includes."""
    h = hashlib.sha256()
    for path in [os.path.join(CSRC, src)] + [os.path.join(CSRC, x) for x in HEADERS] + \
            [os.path.join(INCLUDE, "gemm.h")]:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


_FIELDS = {"TotalSGPRs": "sgprs", "VGPRs": "vgprs", "AGPRs": "agprs", "ScratchSize [bytes/lane]": "scratch",
           "Occupancy [waves/SIMD]": "occupancy", "SGPRs Spill": "sgpr_spill", "VGPRs Spill": "vgpr_spill",
           "LDS Size [bytes/block]": "lds"}


def parse_remarks(text: str) -> dict:
    """{mangled kernel name: {field: int}} from hipcc's kernel-resource remarks."""
    out, cur = {}, None
    for line in text.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z][A-Za-z /\[\]]*?): (\d+) \[", line)
        if m and cur is not None and m.group(1) in _FIELDS:
            cur[_FIELDS[m.group(1)]] = int(m.group(2))
    return out


def _demangle(names):
    try:
        proc = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True)
        lines = proc.stdout.splitlines()
        if proc.returncode == 0 and len(lines) == len(names):
            return lines
    except OSError:
        pass
    return list(names)


def _check(proc, src):
    if proc.returncode != 0:
        noise = "is not a recognized feature for this target"
        err = "\n".join(l for l in proc.stderr.splitlines() if noise not in l and "remark" not in l)
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")


def _compile(src: str):
    """Compile one source to its object; for kernel sources also return the
    parsed resource remarks."""
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMPILE_FLAGS]
    if src.endswith(".hip"):
        cmd += ["-x", "hip", REMARK_FLAG]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    _check(proc, src)
    return obj, (parse_remarks(proc.stderr) if src.endswith(".hip") else None)


def _device_remarks(src: str) -> dict:
    """Device-only compile of one kernel source, for its resource remarks."""
    out = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".resources.o")
    cmd = [HIPCC, *COMPILE_FLAGS, "--cuda-device-only", "-x", "hip", REMARK_FLAG, "-c", os.path.join(CSRC, src),
           "-o", out]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    _check(proc, src)
    return parse_remarks(proc.stderr)


def _store_resources(per_src: dict) -> None:
    table = {}
    for src, kernels in per_src.items():
        names = sorted(kernels)
        for mangled, pretty in zip(names, _demangle(names)):
            table[mangled] = dict(kernels[mangled], source=src, name=pretty)
    rec = {"sources": {src: source_hash(src) for src in per_src}, "kernels": table}
    with open(RESOURCE_FILE, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)


def resource_usage(jobs: int | None = None) -> dict:
    """{mangled name: {name, source, vgprs, agprs, sgprs, scratch, vgpr_spill,
    sgpr_spill, lds, occupancy}} for every kernel, from the last build's
    remarks, recompiling (device code only) the sources changed since."""
    kernel_srcs = [s for s in SOURCES if s.endswith(".hip")]
    rec = {"sources": {}, "kernels": {}}
    if os.path.exists(RESOURCE_FILE):
        with open(RESOURCE_FILE) as f:
            rec = json.load(f)
    stale = [s for s in kernel_srcs if rec["sources"].get(s) != source_hash(s)]
    if stale:
        os.makedirs(BUILD_DIR, exist_ok=True)
        with ThreadPoolExecutor(max_workers=jobs or min(len(stale), os.cpu_count() or 1)) as ex:
            fresh = dict(zip(stale, ex.map(_device_remarks, stale)))
        per_src = {s: {} for s in kernel_srcs}
        for m, k in rec["kernels"].items():
            if k["source"] in per_src and k["source"] not in fresh:
                per_src[k["source"]][m] = {f: v for f, v in k.items() if f not in ("source", "name")}
        per_src.update(fresh)
        _store_resources(per_src)
        with open(RESOURCE_FILE) as f:
            rec = json.load(f)
    return rec["kernels"]


def resource_markdown(table: dict) -> str:
    rows = sorted(table.values(), key=lambda k: (k["source"], k["name"]))
    out = ["# Kernel resources (gfx950)", "",
           "Per-kernel figures from hipcc's kernel-resource remarks, written by",
           "`python -m tiled_gemm_f32_amd.build --resources profiles/kernel_resources.md`",
           f"({len(rows)} kernels; scratch is bytes per lane, LDS bytes per workgroup).", "",
           "| source | kernel | VGPR | AGPR | SGPR | scratch | VGPR spill | SGPR spill (to lanes) | LDS | waves/SIMD |",
           "|---|---|---|---|---|---|---|---|---|---|"]
    for k in rows:
        name = re.sub(r"^void gemm::\(anonymous namespace\)::", "", k["name"])
        name = re.sub(r"\(gemm::GemmParams.*$", "", name)
        out.append(f"| {k['source']} | `{name}` | {k.get('vgprs')} | {k.get('agprs')} | {k.get('sgprs')} | "
                   f"{k.get('scratch')} | {k.get('vgpr_spill')} | {k.get('sgpr_spill')} | {k.get('lds')} | {k.get('occupancy')} |")
    return "\n".join(out) + "\n"


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile all kernels and the ABI; returns the path of libgemm.so."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = [obj for obj, _ in results]
    _store_resources({src: rem for src, (_, rem) in zip(SOURCES, results) if rem is not None})
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"link failed:\n{proc.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    if len(sys.argv) == 3 and sys.argv[1] == "--resources":
        with open(sys.argv[2], "w") as f:
            f.write(resource_markdown(resource_usage()))
    else:
        build(verbose=True)
    sys.exit(0)

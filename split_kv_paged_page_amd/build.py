"""Build libsplitkv.so (the decode library) and libsplitkv_probe.so (a plain
device-memory read the benchmark times beside it) in-tree with hipcc for gfx950.

    python -m split_kv_paged_page_amd.build
    python -m split_kv_paged_page_amd.build --resource-usage   # also print the decode kernels' registers / LDS
    python -m split_kv_paged_page_amd.build --host-check       # host code under ASan + UBSan, for CPU tests

Every HIP source is compiled with packed-FP32 instructions disabled: the
compiler then never forms v_pk_{add,mul,fma}_f32 from scalar float code.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libsplitkv.so")
BUILD = os.path.join(ROOT, "_build")

SOURCES = ["host.cpp", "stage1_valu.hip", "stage1_mfma.hip", "stage1_mfma_mla.hip", "stage2.hip"]
# Per-file options.  The matrix-core shapes at head dims 64-256 take MFMA
# results in VGPRs instead of AGPRs (stage1_mfma.hip says why and what it
# measured); the MLA shapes do not.
FILE_FLAGS = {"stage1_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
PROBE_SRC = os.path.join(HERE, "probe", "read_probe.hip")
PROBE_LIB = os.path.join(HERE, "libsplitkv_probe.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++20", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str, usage: list | None = None) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"]
    extra = ["-Rpass-analysis=kernel-resource-usage"] if usage is not None else []
    extra += FILE_FLAGS.get(os.path.basename(src), [])
    cmd = [HIPCC, *FLAGS, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]   # src may be absolute
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    lines = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if usage is not None:
        import re
        usage.extend(ln for ln in lines if "kernel-resource-usage" in ln)
        # drop the remarks and the source excerpts the compiler prints under them
        lines = [ln for ln in lines if "kernel-resource-usage" not in ln and not re.match(r"^\s*\d*\s*\|", ln)
                 and not ln.startswith("In file included from")]
    if lines:
        sys.stderr.write("\n".join(lines) + "\n")
    return obj


def resource_table(remarks: list) -> list:
    """(kernel, VGPRs, AGPRs, spilled VGPRs, LDS bytes, waves per SIMD) from the
    compiler's kernel-resource-usage remarks."""
    import re
    rows, cur = [], None
    for ln in remarks:
        m = re.search(r"Function Name: (\S+)", ln)
        if m:
            cur = {"kernel": _demangle(m.group(1))}
            rows.append(cur)
            continue
        for key, pat in (("vgpr", r" VGPRs: (\d+)"), ("agpr", r"AGPRs: (\d+)"), ("spill", r"VGPRs Spill: (\d+)"),
                         ("lds", r"LDS Size \[bytes/block\]: (\d+)"), ("occ", r"Occupancy \[waves/SIMD\]: (\d+)")):
            m = re.search(pat, ln)
            if m and cur is not None and key not in cur:
                cur[key] = int(m.group(1))
    return rows


def _demangle(name: str) -> str:
    try:
        r = subprocess.run(["c++filt", name], capture_output=True, text=True)
        out = r.stdout.strip() or name
    except OSError:
        out = name
    return out.replace("splitkv::(anonymous namespace)::", "").replace("(splitkv::Stage1Params)", "").replace(
        "(splitkv::Stage2Params)", "")


def _link(objs: list, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    shutil.move(tmp, out)


# Host-side sanitizers for the CPU test tier: the same sources with the host
# code built under AddressSanitizer and UndefinedBehaviorSanitizer (device
# code unchanged: each flag applies to the host compilation only).  The
# library leaves the sanitizer runtime symbols undefined; the test process
# preloads the runtime.
HOSTCHECK_LIB = os.path.join(BUILD, "libsplitkv_hostcheck.so")
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def build_hostcheck() -> str:
    """Build _build/libsplitkv_hostcheck.so (host code sanitized) for the
    CPU tests that run the planner and argument checks under the
    sanitizers."""
    out = os.path.join(BUILD, "hostcheck")
    os.makedirs(out, exist_ok=True)

    def one(src):
        obj = os.path.join(out, "hc_" + os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, *FLAGS, *HOST_SANITIZE, *FILE_FLAGS.get(src, []), "-x", "hip", "-c",
               os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(one, SOURCES))
    _link(objs, HOSTCHECK_LIB)
    return HOSTCHECK_LIB


def build(verbose: bool = False, usage: list | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + 1)) as ex:
        jobs = [ex.submit(_compile, src, usage) for src in SOURCES]
        probe = ex.submit(_compile, PROBE_SRC)
        objs = [j.result() for j in jobs]
        _link([probe.result()], PROBE_LIB)
    _link(objs, LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    if "--resource-usage" in sys.argv:
        remarks: list = []
        build(verbose=True, usage=remarks)
        print("| kernel | VGPRs | AGPRs | spilled VGPRs | LDS bytes | waves / SIMD |")
        print("|---|---|---|---|---|---|")
        for r in resource_table(remarks):
            print(f"| `{r['kernel']}` | {r.get('vgpr', '')} | {r.get('agpr', '')} | {r.get('spill', '')} | "
                  f"{r.get('lds', '')} | {r.get('occ', '')} |")
    elif "--host-check" in sys.argv:
        print(build_hostcheck())
    else:
        build(verbose=True)

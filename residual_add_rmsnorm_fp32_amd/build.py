"""Build the HIP library ``libfar.so`` for gfx950 in this package's directory.

    python -m residual_add_rmsnorm_fp32_amd.build        (or build() from Python)

``csrc/far_inst.hip`` is compiled once per (storage dtype, quant mode) pair, in
parallel, together with ``csrc/far_api.hip``; the objects are linked into one shared
library with a plain C ABI (``include/far.h``). ``csrc/far_ceiling.hip`` (the
benchmark's pure-stream kernels, ``include/far_ceiling.h``) becomes
``libfar_ceiling.so``. Object files go to ``_build/`` at the repository root, with
``kernel_resources.tsv``: each kernel's registers, occupancy and LDS as the compiler
reports them.
"""

from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libfar.so")
CEILING_LIB_PATH = os.path.join(PKG_DIR, "libfar_ceiling.so")
# registers, occupancy and LDS of every kernel, as the compiler reports them
RESOURCES_PATH = os.path.join(BUILD_DIR, "kernel_resources.tsv")
C_CONSUMER_SRC = os.path.join(PKG_DIR, "examples", "far_c_consumer.c")
C_CONSUMER_BIN = os.path.join(PKG_DIR, "examples", "far_c_consumer")

ARCH = "gfx950"
DTYPES = ("bf16", "fp16")
QUANTS = ("none", "static", "dynamic", "group", "tensor")

# Packed fp32 instructions are switched off (the compiler forms them from ordinary
# float code; the kernels here do not need them).
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfar.so)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return res


_REMARK_FN = re.compile(r"remark: Function Name: (\S+)")
_REMARK_SCRATCH = re.compile(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)")


def _check_no_scratch(stderr: str, what: str):
    """The kernels keep rows in registers by design: a kernel that needs scratch
    (a register spill) is a build error, not a silent slowdown."""
    fn = None
    bad = []
    for line in stderr.splitlines():
        m = _REMARK_FN.search(line)
        if m:
            fn = m.group(1)
            continue
        m = _REMARK_SCRATCH.search(line)
        if m and int(m.group(1)) != 0:
            bad.append((fn, int(m.group(1))))
    if bad:
        raise RuntimeError(f"{what}: kernels use scratch memory (register spills): {bad[:5]}")


_REMARK_FIELDS = {
    "TotalSGPRs": "sgprs", "VGPRs": "vgprs", "AGPRs": "agprs",
    "ScratchSize [bytes/lane]": "scratch", "Occupancy [waves/SIMD]": "waves_per_simd",
    "LDS Size [bytes/block]": "lds_bytes",
}
_REMARK_FIELD = re.compile(r"remark:\s+(" + "|".join(re.escape(k) for k in _REMARK_FIELDS)
                           + r"): (\d+)")


def _resources(stderr: str) -> list[tuple[str, dict]]:
    """(mangled kernel name, {field: value}) for each kernel's resource-usage remarks."""
    out = []
    for line in stderr.splitlines():
        m = _REMARK_FN.search(line)
        if m:
            out.append((m.group(1), {}))
            continue
        m = _REMARK_FIELD.search(line)
        if m and out:
            out[-1][1][_REMARK_FIELDS[m.group(1)]] = int(m.group(2))
    return out


def _write_resources(stderrs: list[str]):
    rows = {}
    for err in stderrs:
        for name, fields in _resources(err):
            rows[name] = fields
    names = sorted(rows)
    demangled = names
    filt = shutil.which("c++filt")
    if filt and names:
        res = subprocess.run([filt], input="\n".join(names), capture_output=True, text=True)
        if res.returncode == 0 and len(res.stdout.splitlines()) == len(names):
            demangled = res.stdout.splitlines()
    cols = list(_REMARK_FIELDS.values())
    with open(RESOURCES_PATH, "w") as f:
        f.write("kernel\t" + "\t".join(cols) + "\n")
        for name, pretty in zip(names, demangled):
            f.write(pretty + "\t" + "\t".join(str(rows[name].get(c, "")) for c in cols) + "\n")


def build(verbose: bool = False, jobs: int | None = None) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    common = [hipcc] + HIPCC_FLAGS + ["-I", INCLUDE, "-I", CSRC]
    jobs_list = []
    for d in DTYPES:
        for q in QUANTS:
            obj = os.path.join(BUILD_DIR, f"far_inst_{d}_{q}.o")
            jobs_list.append(common + [f"-DFAR_INST_DTYPE={d}", f"-DFAR_INST_QUANT={q}",
                                       "-Rpass-analysis=kernel-resource-usage", "-c",
                                       os.path.join(CSRC, "far_inst.hip"), "-o", obj])
    api_obj = os.path.join(BUILD_DIR, "far_api.o")
    jobs_list.append(common + ["-c", os.path.join(CSRC, "far_api.hip"), "-o", api_obj])
    ceiling_obj = os.path.join(BUILD_DIR, "far_ceiling.o")
    jobs_list.append(common + ["-Rpass-analysis=kernel-resource-usage", "-c",
                               os.path.join(CSRC, "far_ceiling.hip"), "-o", ceiling_obj])
    n = jobs or min(len(jobs_list), max(1, (os.cpu_count() or 2)))
    with ThreadPoolExecutor(max_workers=n) as ex:
        results = list(ex.map(lambda c: _run(c, verbose), jobs_list))
    for cmd, res in zip(jobs_list, results):
        _check_no_scratch(res.stderr, os.path.basename(cmd[cmd.index("-o") + 1]))
    _write_resources([res.stderr for res in results])
    objs = [c[c.index("-o") + 1] for c in jobs_list if c[c.index("-o") + 1] != ceiling_obj]
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB_PATH)
    # the benchmark's measurement aids (pure streams of the same bytes) in a library of
    # their own, so the epilogue's library holds only the epilogue
    tmp = CEILING_LIB_PATH + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, ceiling_obj], verbose)
    os.replace(tmp, CEILING_LIB_PATH)
    # the plain C example links the library through the C ABI only (no HIP device code)
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc)))
    _run(["gcc", "-std=c11", "-O2", "-Wall", "-I", INCLUDE, "-I", os.path.join(rocm, "include"),
          C_CONSUMER_SRC, "-o", C_CONSUMER_BIN, "-L", PKG_DIR, "-lfar",
          "-L", os.path.join(rocm, "lib"), "-lamdhip64",
          "-Wl,-rpath,$ORIGIN/..", "-Wl,-rpath," + os.path.join(rocm, "lib")], verbose)
    return LIB_PATH


SANITIZED_DIR = os.path.join(BUILD_DIR, "sanitized")


def build_sanitized(verbose: bool = False) -> tuple[str, str]:
    """A copy of libfar.so whose host code (validation, planning, dispatch) is built with
    AddressSanitizer and UndefinedBehaviorSanitizer, for checking the C ABI's host
    paths on the CPU. Device code is unchanged (the sanitizers are host-only flags). Needs
    the objects of build(). Returns (library path, ASan runtime to preload)."""
    hipcc = _hipcc()
    os.makedirs(SANITIZED_DIR, exist_ok=True)
    inst = [os.path.join(BUILD_DIR, f"far_inst_{d}_{q}.o") for d in DTYPES for q in QUANTS]
    missing = [o for o in inst if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"build() first: missing {missing[:2]}")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer"]
    api_obj = os.path.join(SANITIZED_DIR, "far_api.o")
    _run([hipcc] + HIPCC_FLAGS + san + ["-g", "-I", INCLUDE, "-I", CSRC, "-c",
                                         os.path.join(CSRC, "far_api.hip"), "-o", api_obj], verbose)
    lib = os.path.join(SANITIZED_DIR, "libfar.so")
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-shared-libsan"] + san[:4] +
         ["-o", lib, api_obj] + inst, verbose)
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc)))
    clang = os.path.join(rocm, "llvm", "bin", "clang")
    runtime = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                             capture_output=True, text=True, check=True).stdout.strip()
    return lib, runtime


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)

"""Build libattn_prefill.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

The kernel source is compiled once per kernel configuration (ATTN_CONFIG =
0 .. N_CONFIGS - 1) and once for the configuration table and the merge kernel
(ATTN_CONFIG = -1), in parallel, then linked with the C ABI into one shared
library.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libattn_prefill.so")
KERNEL = os.path.join(CSRC, "attn_kernel.hip")
API = os.path.join(CSRC, "attn_api.cpp")
N_CONFIGS = 7

# Packed-fp32 VALU instructions are disabled for all device code.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-variable", "-Wno-unused-function",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]

# the host pass does not know the packed-fp32 target feature: drop that note
_NOISE = "not a recognized feature for this target"


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(ln for ln in res.stderr.splitlines() if _NOISE not in ln)
    return res.returncode, err


def build(verbose: bool = False, extra_flags=None, out=None, jobs=None) -> str:
    """Compile every translation unit (in parallel) and link the library to
    `out` (default: the in-tree libattn_prefill.so).  Returns its path."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    out = out or LIB
    os.makedirs(OBJ, exist_ok=True)
    tag = os.path.basename(out).replace(".so", "")
    flags = HIPCC_FLAGS + list(extra_flags or [])
    units = [(KERNEL, ["-DATTN_CONFIG=%d" % i], os.path.join(OBJ, f"{tag}_cfg{i}.o"))
             for i in range(N_CONFIGS)]
    units.append((KERNEL, ["-DATTN_CONFIG=-1"], os.path.join(OBJ, f"{tag}_table.o")))
    units.append((API, [], os.path.join(OBJ, f"{tag}_api.o")))
    cmds = [[hipcc] + flags + d + ["-c", src, "-o", o] for src, d, o in units]
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    jobs = jobs or min(len(cmds), max(1, os.cpu_count() or 1))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_run, cmds))
    for (src, d, o), (rc, err) in zip(units, results):
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {os.path.basename(src)} {' '.join(d)} "
                               f"({rc}):\n{err}")
        if verbose and err.strip():
            print(err, file=sys.stderr)
    link = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC"] + [o for _, _, o in units] + \
        ["-o", out + ".tmp"]
    rc, err = _run(link)
    if rc != 0:
        raise RuntimeError(f"link failed ({rc}):\n{err}")
    os.replace(out + ".tmp", out)
    return out


# AddressSanitizer + UBSan on the host side of the C ABI layer only (each
# -fsanitize after -Xarch_host: device code is never built with them), linked
# with the device objects of the last build() into a separate library that
# only the host-sanitizer test loads, under the clang ASan runtime.
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
LIB_HOST_SANITIZED = os.path.join(OBJ, "libattn_prefill_host_sanitized.so")


def build_host_sanitized() -> str:
    """Link LIB_HOST_SANITIZED from a host-sanitized compile of the C ABI
    layer and the kernel objects of the last build() (which must exist)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    kernels = [os.path.join(OBJ, f"libattn_prefill_cfg{i}.o") for i in range(N_CONFIGS)]
    kernels.append(os.path.join(OBJ, "libattn_prefill_table.o"))
    missing = [k for k in kernels if not os.path.exists(k)]
    if missing:
        raise RuntimeError(f"kernel objects missing ({missing[0]}): run build() first")
    api_o = os.path.join(OBJ, "host_sanitized_api.o")
    rc, err = _run([hipcc] + HIPCC_FLAGS + HOST_SANITIZE + ["-c", API, "-o", api_o])
    if rc != 0:
        raise RuntimeError(f"hipcc failed on the sanitized C ABI layer ({rc}):\n{err}")
    out = LIB_HOST_SANITIZED
    rc, err = _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC"] + HOST_SANITIZE +
                   kernels + [api_o, "-o", out + ".tmp"])
    if rc != 0:
        raise RuntimeError(f"link failed ({rc}):\n{err}")
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

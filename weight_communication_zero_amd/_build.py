"""Build libzq.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Flags that the bit-exact contract depends on:
  -ffp-contract=off                        no a*b+c fused into one rounding
  -fhip-fp32-correctly-rounded-divide-sqrt IEEE divide for the block scales
  -fno-gpu-flush-denormals-to-zero         subnormal values are kept
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                           no packed fp32 VALU instructions
"""
from __future__ import annotations

import glob
import os
import re
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libzq.so")
ARCH = os.environ.get("ZQ_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-mcode-object-version=5",
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


# Every kernel must run without private (scratch) memory: libzq promises
# that it never has the runtime back anything for it.  The compiler's
# resource-usage remarks name each kernel and its scratch bytes per lane.
RESOURCE_REMARKS = "-Rpass-analysis=kernel-resource-usage"


def scratch_users(stderr: str) -> list[tuple[str, int]]:
    """(kernel, bytes per lane) of every kernel the remarks show using scratch."""
    out, name = [], None
    for line in stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and int(m.group(1)) > 0:
            out.append((name, int(m.group(1))))
    return out


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(c for c in cmd if c != RESOURCE_REMARKS), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stderr[-8000:]}")
    users = scratch_users(r.stderr)
    if users:
        raise RuntimeError(f"kernels using scratch memory: {users}")


def build(verbose: bool = False, extra: list[str] | None = None, out: str | None = None) -> str:
    """Compile every source to an object in parallel, then link the shared
    library (each object carries its own gfx950 code object)."""
    out = out or LIB
    tmp = out + ".tmp"
    with tempfile.TemporaryDirectory(prefix="zq_build_") as d:
        objs = [os.path.join(d, os.path.basename(s) + ".o") for s in sources()]
        jobs = [[HIPCC, *FLAGS, *(extra or []), RESOURCE_REMARKS, "-c", "-o", o, s]
                for s, o in zip(sources(), objs)]
        with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1, 8)) as ex:
            for f in [ex.submit(_run, j, verbose) for j in jobs]:
                f.result()
        _run([HIPCC, *FLAGS, *(extra or []), "-o", tmp, *objs], verbose)
    os.replace(tmp, out)
    return out


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    deps = sources() + glob.glob(os.path.join(CSRC, "*.h")) + [os.path.join(ROOT, "include", "zq.h")]
    return any(os.path.getmtime(d) > t for d in deps)


if __name__ == "__main__":
    print(build(verbose=True))

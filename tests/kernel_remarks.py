"""Kernels of the HIP library as the compiler reports them (CPU only).

Compiles every csrc/*.hip with the library's own flags and
-Rpass-analysis=kernel-resource-usage, and returns {mangled kernel symbol:
{remark field: value}}: register and scratch use per kernel, and the set of
kernel instances the library actually ships.  Cached per process.
"""

import concurrent.futures
import functools
import glob
import os
import re
import runpy
import shutil
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "combine_moe_layout_03_amd", "csrc")


def build_settings():
    return runpy.run_path(os.path.join(ROOT, "combine_moe_layout_03_amd", "build.py"))


def hipcc_available() -> bool:
    hipcc = build_settings()["HIPCC"]
    return bool(os.path.exists(hipcc) or shutil.which(hipcc))


def _resource_remarks(src: str, hipcc: str, flags) -> str:
    cmd = [hipcc, *flags, "-c", src, "-o", os.devnull, "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"hipcc failed on {src}:\n{r.stderr[-2000:]}"
    return r.stderr


def _parse(text: str):
    out, cur = {}, None
    for line in text.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\S+) \[-Rpass-analysis", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = m.group(2)
    return out


@functools.lru_cache(maxsize=1)
def kernel_remarks():
    b = build_settings()
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(6, len(sources))) as ex:
        texts = list(ex.map(lambda s: _resource_remarks(s, b["HIPCC"], b["CXXFLAGS"]), sources))
    found = {}
    for t in texts:
        found.update(_parse(t))
    return found


def demangle(symbols):
    """Mangled -> demangled names through c++filt (one process for all)."""
    symbols = list(symbols)
    r = subprocess.run(["c++filt"], input="\n".join(symbols), capture_output=True, text=True, check=True)
    return dict(zip(symbols, r.stdout.splitlines()))

"""Register and scratch use of every HIP kernel, from hipcc's resource-usage
remarks (CPU only: hipcc cross-compiles for gfx950 here).

A kernel that keeps an array in scratch memory (per-lane private memory in
HBM) instead of registers runs far below its bandwidth bound: the fused
kernel's passthrough form once copied its row register array with 16-byte
struct copies, which the compiler lowered to memcpy and left in 240 bytes of
scratch per lane, and took twice as long.  This test compiles each source
with the library's own flags and requires no scratch at all, except for a
few spilled scalars in the one instantiation that needs more registers than
a 1024-thread workgroup allows (the fused int8 kernel for 7168 < h <= 8192).
"""

import concurrent.futures
import glob
import os
import re
import runpy
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "combine_moe_layout_03_amd", "csrc")

# fused_kernel<kFp16, kQuant = true, kVpl = 16>: up to 32 bytes of spilled scalars
SPILL_ALLOWED = re.compile(r"fused_kernelILb[01]ELb1ELi16E")


def _resource_remarks(src: str, hipcc: str, flags) -> str:
    cmd = [hipcc, *flags, "-c", src, "-o", os.devnull, "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"hipcc failed on {src}:\n{r.stderr[-2000:]}"
    return r.stderr


def _parse(text: str):
    """{kernel symbol: {field: value}} from the remark lines."""
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


@pytest.fixture(scope="module")
def kernels():
    b = runpy.run_path(os.path.join(ROOT, "combine_moe_layout_03_amd", "build.py"))
    hipcc = b["HIPCC"]
    if not (os.path.exists(hipcc) or shutil.which(hipcc)):
        pytest.skip("hipcc not available")
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(6, len(sources))) as ex:
        texts = list(ex.map(lambda s: _resource_remarks(s, hipcc, b["CXXFLAGS"]), sources))
    found = {}
    for t in texts:
        found.update(_parse(t))
    return found


def test_every_kernel_reports_resources(kernels):
    names = " ".join(kernels)
    for k in ("layout_count_kernel", "layout_rank_kernel", "notify_kernel", "notify_multi_kernel",
              "dispatch_kernel", "combine_kernel", "fused_kernel"):
        assert k in names, f"{k} missing from the resource-usage remarks"
    for name, f in kernels.items():
        assert "ScratchSize" in f and "VGPRs Spill" in f, (name, f)


def test_no_scratch_memory(kernels):
    bad = []
    for name, f in kernels.items():
        scratch = int(f["ScratchSize"])
        limit = 32 if SPILL_ALLOWED.search(name) else 0
        if scratch > limit or f.get("Dynamic Stack", "False") != "False":
            bad.append((name, f["ScratchSize"], f.get("VGPRs Spill"), f.get("Dynamic Stack")))
    assert not bad, f"kernels using scratch memory: {bad}"

"""Build-time resource check of every HIP kernel for gfx950 (CPU only: hipcc
cross-compiles without a GPU).

The streaming kernels keep each lane's elements in registers.  A loop that
indexes a lane's element array with a run-time bound makes the compiler move
that array to LDS (8 KiB per workgroup) or to scratch, which costs
bandwidth without any error.  This test compiles each source with the
library's flags and the compiler's per-kernel resource report and checks
that no kernel uses scratch or spills vector registers (scalar spills only
where listed, into vector-register lanes), and that static LDS stays
within the few small reduction buffers the kernels declare themselves.
"""
import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from ring_all_reduce_scatter_amd import build as rar_build  # noqa: E402

STATIC_LDS_MAX = 128  # bytes: the largest declared reduction buffer is 96
# Kernels allowed to spill scalar registers, provided the spills land in
# vector-register lanes (v_writelane / v_readlane, no scratch memory): the
# pipelined sparse ring keeps a unit's geometry, message pointers and the
# decision state of a whole hop chain uniform in one long loop; its partial
# sums live in LDS and its vector registers and scratch stay clean.
SGPR_LANE_SPILLS_OK = ("sparse_pipe_kernel",)


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


def _report(src, tmpdir):
    obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *rar_build.CFLAGS, "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    kernels, cur = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"remark:\s+Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            kernels[cur] = {}
            continue
        m = re.search(r"remark:\s+(ScratchSize \[bytes/lane\]|VGPRs Spill|SGPRs Spill|LDS Size \[bytes/block\]): (\d+)",
                      line)
        if m and cur:
            kernels[cur][m.group(1)] = int(m.group(2))
    return kernels


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not found")
def test_kernels_use_no_scratch_spills_or_promoted_lds(tmp_path):
    srcs = sorted(os.path.join(rar_build.CSRC, f) for f in os.listdir(rar_build.CSRC) if f.endswith(".hip"))
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        reports = list(ex.map(lambda s: (s, _report(s, str(tmp_path))), srcs))
    bad, nkernels = [], 0
    for src, kernels in reports:
        for name, res in kernels.items():
            nkernels += 1
            if res.get("ScratchSize [bytes/lane]", 0):
                bad.append(f"{name}: scratch {res['ScratchSize [bytes/lane]']} B per lane")
            if res.get("VGPRs Spill", 0):
                bad.append(f"{name}: vector register spills")
            if res.get("SGPRs Spill", 0) and not any(k in name for k in SGPR_LANE_SPILLS_OK):
                bad.append(f"{name}: scalar register spills")
            if res.get("LDS Size [bytes/block]", 0) > STATIC_LDS_MAX:
                bad.append(f"{name}: {res['LDS Size [bytes/block]']} B of static LDS")
    assert nkernels > 50, f"only {nkernels} kernels reported"
    assert not bad, "\n".join(bad)

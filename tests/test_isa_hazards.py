"""The prefill kernels' hand-written HBM -> LDS copies, checked in the gfx950 assembly the
compiler emits (CPU only: hipcc cross-compiles).  A copy reads its LDS address from M0, and an
LDS DMA must not issue in the instruction right after a scalar write of M0: every
global_load_lds_dwordx4 must follow its M0 write by at least one instruction (the copies put an
s_nop 0 there; the compiler pads its own such pairs the same way)."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_write_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.timeout(600)
def test_lds_dma_copies_wait_after_the_m0_write(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path / "prefill.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "--cuda-device-only", "-S", os.path.join(CSRC, "prefill.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln.strip() for ln in out.read_text().splitlines()]
    instrs = [ln for ln in lines if ln and not ln.startswith((";", ".", "//")) and not ln.endswith(":")]
    copies = 0
    for i, ins in enumerate(instrs):
        if ins.startswith("global_load_lds"):
            copies += 1
            prev = instrs[i - 1]
            assert not re.match(r"s_\w+\s+m0\b", prev), \
                f"LDS DMA right after a write of M0: {prev!r} / {ins!r}"
    assert copies > 0, "no LDS DMA copies found in the prefill kernels"

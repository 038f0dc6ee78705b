"""The prefill scan's memory pipeline, checked in the gfx950 assembly.

The scan keeps D steps of gathers in flight and waits, once per step, until
at most (D - 1) * NVM vector-memory instructions are outstanding (NVM = the
fixed count a step issues).  A tighter wait anywhere in the steady state
(for instance one the compiler adds when it has to move a loaded register
at the loop edge) drains the pipeline every step and costs a large part of
the kernel's time without changing any result, so it is checked here on the
code hipcc emits.  Runs on the CPU (hipcc cross-compiles for gfx950).
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_memory_linear_pkm_amd", "csrc")


def _hipcc():
    return shutil.which("hipcc") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else None)


def _device_asm(tmp_path_factory, src):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    import sys
    sys.path.insert(0, os.path.join(ROOT, "sparse_memory_linear_pkm_amd"))
    import build as B
    flags = [f for f in B.CFLAGS if f != "-fPIC"]
    out = str(tmp_path_factory.mktemp("asm") / (src + ".s"))
    r = subprocess.run([hipcc, *flags, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read()


@pytest.fixture(scope="module")
def lanes_asm(tmp_path_factory):
    return _device_asm(tmp_path_factory, "sdm_scan_lanes.hip")


@pytest.fixture(scope="module")
def bwd_lanes_asm(tmp_path_factory):
    return _device_asm(tmp_path_factory, "sdm_scan_bwd_lanes.hip")


def _kernels(asm):
    # sdm_scan_lanes_kernel<Q, D, G, BF16, SAVE>: mangled as ...ILi<Q>ELi<D>ELi<G>ELb<0|1>ELb<0|1>E...
    pat = re.compile(r"^(_ZN3sdm21sdm_scan_lanes_kernelILi(\d+)ELi(\d+)ELi(\d+)ELb([01])ELb([01])E\w*):", re.M)
    for m in pat.finditer(asm):
        end = asm.index(".Lfunc_end", m.start())
        yield int(m.group(3)), m.group(5) == "1", m.group(6) == "1", asm[m.start():end]


def test_scan_steady_state_waits(lanes_asm):
    found = 0
    for D, bf16, save, body in _kernels(lanes_asm):
        found += 1
        nvm = 6 + (1 if bf16 else 2) + (2 if save else 0)
        waits = [int(x) for x in re.findall(r"s_waitcnt vmcnt\((\d+)\)", body)]
        tight = [w for w in waits if 0 < w < (D - 1) * nvm]
        assert not tight, f"D={D} bf16={bf16} save={save}: waits below (D-1)*NVM = {(D - 1) * nvm}: {tight}"
        # vmcnt(0) only in the prologue (twice) and after the loop (once)
        assert waits.count(0) <= 3, f"D={D} bf16={bf16} save={save}: {waits.count(0)} full drains"
    assert found >= 16


def test_backward_scan_steady_state_waits(bwd_lanes_asm):
    """The same check on the backward's lane kernel
    (sdm_scan_bwd_lanes_kernel<Q, D, G, BF16>), whose steps issue NVM = 8 +
    NTR vector-memory instructions (NTR = 1 for bf16 v, 2 for fp32)."""
    pat = re.compile(r"^(_ZN3sdm25sdm_scan_bwd_lanes_kernelILi(\d+)ELi(\d+)ELi(\d+)ELb([01])E\w*):", re.M)
    found = 0
    for m in pat.finditer(bwd_lanes_asm):
        end = bwd_lanes_asm.index(".Lfunc_end", m.start())
        body = bwd_lanes_asm[m.start():end]
        D, bf16 = int(m.group(3)), m.group(5) == "1"
        nvm = 8 + (1 if bf16 else 2)
        waits = [int(x) for x in re.findall(r"s_waitcnt vmcnt\((\d+)\)", body)]
        tight = [w for w in waits if 0 < w < (D - 1) * nvm]
        assert not tight, f"{m.group(1)}: waits below (D-1)*NVM = {(D - 1) * nvm}: {tight}"
        assert waits.count(0) <= 3, f"{m.group(1)}: {waits.count(0)} full drains"
        found += 1
    assert found >= 16

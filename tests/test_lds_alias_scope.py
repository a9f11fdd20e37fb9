"""Compile-time check of the sparse dK/dV kernel's memory waits (no GPU needed).

The kernel's two ring stages are filled by direct global -> LDS loads while
the other stage is computed on.  The compiler tells the stages apart, and so
avoids draining those loads before an LDS access, only when the access keeps
its LDS array's alias scope; an access built through a long address chain
loses it, and the compiler then waits for every load in flight.  This test
compiles the kernel as the library build does and checks, before the wait
insertion pass, that every LDS access of the sparse D = 128, G = 4 instance
carries an alias scope, and, in the assembly, that the step wait leaves the
previous step's share stores in flight (vmcnt(4)).
"""
import os
import re
import shutil
import subprocess

import pytest

from trainable_block_sparse_sas_amd import build

KERNEL = "_ZN3sas12_GLOBAL__N_115bwd_dkdv_kernelILi128ELi4ELb1ELb0EEEvNS0_7BwdArgsENS_8SelListsE"
SRC = os.path.join(build.CSRC, "attn_bwd_mfma.hip")


@pytest.fixture(scope="module")
def compiled(tmp_path_factory):
    if not os.path.exists(build.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "bwd.s"
    cmd = [build.HIPCC, *build.COMMON, *build.DEVICE_FLAGS, "--cuda-device-only", "-S",
           "-mllvm", "-print-before=si-insert-waitcnts", "-mllvm", f"-filter-print-funcs={KERNEL}",
           SRC, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    return r.stderr, out.read_text()


def test_every_lds_access_keeps_its_alias_scope(compiled):
    mir, _ = compiled
    assert f"Machine code for function {KERNEL}" in mir
    ds = [l for l in mir.splitlines() if re.search(r"\bDS_(READ|WRITE)", l)]
    assert len(ds) > 50
    # a merged access (ds_write2, ds_read2) lists one memory operand per part
    lost = [l.strip() for l in ds
            if l.count("!alias.scope") < len(re.findall(r"\((?:load|store) \(", l))]
    assert not lost, "LDS accesses without alias scope:\n" + "\n".join(lost[:8])


def test_step_wait_leaves_the_share_stores_in_flight(compiled):
    _, asm = compiled
    start = asm.index(f"{KERNEL}:")
    body = asm[start:asm.index("s_endpgm", start)]
    assert body.count("s_waitcnt vmcnt(4)") >= 4  # one per unrolled step of the ring loops
    # A step: the wait, the ring barrier, compute, a barrier once the dS rows
    # are complete, the staged dQ rows, a barrier once they are complete.
    # Nothing between the ring barrier and the third barrier may drain the
    # next stage's loads (code after a loop's last step, which continues into
    # other control flow, is only checked up to its second barrier).
    clean = 0
    for step in re.split(r"s_waitcnt vmcnt\(4\)", body)[1:]:
        barriers = [m.start() for m in re.finditer(r"s_barrier", step)]
        if len(barriers) < 3:
            continue
        assert "vmcnt(0)" not in step[barriers[1]:barriers[2]], "a full drain before the staged dQ rows"
        clean += "vmcnt(0)" not in step[barriers[0]:barriers[2]]
    assert clean >= 4

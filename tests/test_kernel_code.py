"""Checks on the generated gfx950 code of the prefill MFMA kernels (no GPU needed).

Their K loops load both operands straight into LDS with inline-asm buffer loads and
wait for them with one hand-counted `s_waitcnt vmcnt(16)` per stage.  That count is
safe whatever else the compiler puts in the loop: vector-memory operations complete
in issue order, so any extra load or store it issues only adds to the operations
newer than the ones a stage waits for.  What would break it is an inline-asm load
whose destination is a register (the compiler could copy or spill the register
before the data lands), so the loop's asm loads must all write LDS.
"""
import os
import re
import subprocess

import pytest

from moe_expert_offload_amd import build

KERNELS = ("ffn_gateup_mfma_kernel", "ffn_down_mfma_kernel")


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    if not os.path.exists(build.HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "kernels.s"
    cmd = [build.HIPCC, f"--offload-arch={build.ARCH}", "--cuda-device-only", "-S", "-O3", "-std=c++17",
           f"-I{build.CSRC}", f"-I{os.path.join(build.PKG, '..', 'include')}", "-o", str(out),
           os.path.join(build.CSRC, "kernels.hip")] + build.DEVICE_FLAGS
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    return out.read_text()


def _body(src, name):
    m = re.search(r"^(_Z\w*" + name + r"\w*):[^\n]*\n(.*?); -- End function", src, re.S | re.M)
    assert m, name
    return m.group(2)


def _asm_blocks(body):
    return re.findall(r";;#ASMSTART\n(.*?);;#ASMEND", body, re.S)


@pytest.mark.parametrize("name", KERNELS)
def test_loop_loads_write_lds_only(device_asm, name):
    blocks = _asm_blocks(_body(device_asm, name))
    loads = [l.strip() for b in blocks for l in b.split("\n") if re.match(r"\s*(buffer|global|flat|scratch)_load", l)]
    assert loads, "no hand-issued loads found"
    assert all(l.endswith(" lds") for l in loads), [l for l in loads if not l.endswith(" lds")][:4]


@pytest.mark.parametrize("name", KERNELS)
def test_one_stage_wait_per_stage(device_asm, name):
    body = _body(device_asm, name)
    waits = [b for b in _asm_blocks(body) if "s_waitcnt vmcnt(16)" in b]
    barriers = body.count("s_barrier")
    # 8 row-subtile variants, each an unrolled group of 4 stages
    assert len(waits) == 32
    assert barriers >= len(waits)

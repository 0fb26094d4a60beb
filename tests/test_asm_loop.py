"""Host-side checks of the hand-scheduled attention loop (no GPU needed).

The loop of the head-size-128 kernel is one inline-asm statement that pins its accumulators and
scratch registers.  The compiler allocates the statement's other operands; an input placed in a
register the loop writes would be overwritten mid-loop.  These tests compile the kernel source to
gfx950 assembly and check the allocation, and check that the committed generated loop matches its
generator."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tensor_head_attention_amd", "csrc")
sys.path.insert(0, CSRC)
import gen_attn_loop as G  # noqa: E402

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def test_generated_loop_is_current(tmp_path):
    out = tmp_path / "loop.inc"
    G.main(str(out))
    with open(os.path.join(CSRC, "attn_loop_d128.inc")) as f:
        assert f.read() == out.read_text(), "attn_loop_d128.inc is stale: rerun gen_attn_loop.py"


def test_loop_structure():
    lines = G.gen_loop()
    # 16 score MFMAs + 16 value MFMAs per tile with a successor, 16 per last tile;
    # two halves x (unmasked, masked) + two last blocks
    n_mfma = sum(l.startswith("v_mfma") for l in lines)
    assert n_mfma == 2 * 2 * 32 + 2 * 16
    # every lgkmcnt wait fits the 4-bit counter field
    for l in lines:
        if "lgkmcnt(" in l:
            assert 0 <= int(l.split("lgkmcnt(")[1].rstrip(")")) <= 15
    # one barrier per tile (two per unrolled iteration)
    assert sum(l == "s_barrier" for l in lines) == 2


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None, reason="hipcc not available")
def test_operand_registers_do_not_overlap_loop_writes(tmp_path):
    asm = tmp_path / "d128.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--cuda-device-only", "-S",
           "-o", str(asm), os.path.join(CSRC, "attn_bf16_d128.hip")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    names = G.check_operand_allocation(asm.read_text())
    # every named operand of the template was found
    expected = {"ka%d" % i for i in range(8)} | {"va%d" % i for i in range(4)} | \
               {"koff%d" % i for i in range(4)} | {"voff%d" % i for i in range(4)} | \
               {"mrun", "lrun", "nmc", "base2", "c", "thr", "nkt", "tmask", "kvlim", "rowb", "kp_lo", "kp_hi",
                "vp_lo", "vp_hi", "tstride_lo", "tstride_hi", "kdst0", "vdst0"}
    assert expected <= set(names), expected - set(names)

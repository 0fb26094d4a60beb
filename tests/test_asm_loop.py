"""Host-side checks of the hand-scheduled attention loop (no GPU needed).

The loop of the head-size-128 kernel is one inline-asm statement that pins its accumulators and
scratch registers.  The compiler allocates the statement's other operands; an input placed in a
register the loop writes would be overwritten mid-loop.  These tests compile the kernel source to
gfx950 assembly and check the allocation, and check that the committed generated loop matches its
generator."""
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tensor_head_attention_amd", "csrc")
sys.path.insert(0, CSRC)
import gen_attn_loop as G  # noqa: E402
import gen_attn_loop_wide as GW  # noqa: E402

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def test_generated_loop_is_current(tmp_path):
    out = tmp_path / "loop.inc"
    G.main(str(out))
    with open(os.path.join(CSRC, "attn_loop_d128.inc")) as f:
        assert f.read() == out.read_text(), "attn_loop_d128.inc is stale: rerun gen_attn_loop.py"


@pytest.mark.parametrize("nloads", sorted(G.LOOP_VARIANTS))
def test_loop_structure(nloads):
    lines = G.gen_loop(nloads)
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
    # each block with a successor copies one K and one V tile: nloads copies of each, every
    # copy through its own offset operand, with M0 set (and a wait state) right before it
    loads = [i for i, l in enumerate(lines) if l.startswith("buffer_load_dwordx4")]
    assert len(loads) == 4 * 2 * nloads
    used = {l.split()[1].rstrip(",") for l in lines if l.startswith("buffer_load_dwordx4")}
    assert used == {f"%[{w}off{u}]" for w in "kv" for u in range(nloads)}
    for i in loads:
        assert lines[i - 1] == "s_nop 0" and lines[i - 2].startswith("s_mov_b32 m0, ")
    # the copies' LDS destinations advance 1 KiB per copy: nloads KiB per wavefront per tile
    steps = sum(l == "s_add_u32 s84, s84, 1024" for l in lines)
    assert steps == 4 * 2 * (nloads - 1)


def test_l8_loop_differs_from_l4_in_copies_and_prefetch_only():
    """The 8-copy loop makes twice the tile copies and reads fragments five ahead (through its own
    buffers) instead of three; the arithmetic instructions are the same, in the same order."""
    a, b = G.gen_loop(4), G.gen_loop(8)
    keep = ("v_mfma", "v_exp", "v_fma", "v_add", "v_max", "v_cvt", "v_cmp", "v_cndmask", "v_mul", "v_sub",
            "v_permlane", "v_accvgpr", "s_barrier", "s_cbranch", "s_branch")
    arith = lambda ls: [re.sub(r"v\[\d+:\d+\]", "F", l) for l in ls if l.startswith(keep)]  # noqa: E731
    assert arith(a) == arith(b)
    # every fragment register of the 8-copy loop is one of its six rotating buffers
    for l in b:
        if l.startswith("ds_read"):
            r = int(re.match(r"ds_read_\w+ v\[(\d+):", l).group(1))
            assert r in G.FRAGS[8].regs()


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None, reason="hipcc not available")
def test_operand_registers_do_not_overlap_loop_writes(tmp_path):
    asm = tmp_path / "d128.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--cuda-device-only", "-S",
           "-o", str(asm), os.path.join(CSRC, "attn_bf16_d128.hip")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    text = asm.read_text()
    names = G.check_operand_allocation(text)
    # both loop variants were compiled (and so checked): the 4-copy loop of the narrow and split
    # forms and the 8-copy loop of the 64-row split form, whose extra copy offsets are operands
    found = {len([l for l in b.strip().splitlines() if l.strip()])
             for b in re.findall(r";;#ASMSTART\n(.*?);;#ASMEND", text, flags=re.S)}
    assert {len(G.gen_loop(n)) for n in G.LOOP_VARIANTS} <= found
    l8_names = set(re.findall(r"%\[(\w+)\]", "\n".join(G.gen_loop(8))))
    assert {"koff%d" % i for i in range(4, 8)} | {"voff%d" % i for i in range(4, 8)} <= l8_names
    # every named operand of the template was found
    expected = {"ka%d" % i for i in range(8)} | {"va%d" % i for i in range(4)} | \
               {"koff%d" % i for i in range(4)} | {"voff%d" % i for i in range(4)} | \
               {"mrun", "lrun", "nmc", "base2", "c", "thr", "nkt", "tmask", "kvlim", "rowb", "kp_lo", "kp_hi",
                "vp_lo", "vp_hi", "tstride_lo", "tstride_hi", "kdst0", "vdst0"}
    assert expected <= set(names), expected - set(names)


def test_wide_generated_loop_is_current(tmp_path):
    out = tmp_path / "loop.inc"
    GW.main(str(out))
    with open(os.path.join(CSRC, "attn_loop_d128_wide.inc")) as f:
        assert f.read() == out.read_text(), "attn_loop_d128_wide.inc is stale: rerun gen_attn_loop_wide.py"


def test_wide_loop_structure():
    lines = GW.gen_loop()
    # 64 MFMAs per tile with a successor (four unrolled tiles x unmasked/masked), 32 per last tile
    assert sum(l.startswith("v_mfma") for l in lines) == 4 * 2 * 64 + 4 * 32
    for l in lines:
        if "lgkmcnt(" in l:
            assert 0 <= int(l.split("lgkmcnt(")[1].rstrip(")")) <= 15
    assert sum(l == "s_barrier" for l in lines) == 4
    # every LDS read addresses a fixed buffer: an instruction offset inside the 4 K / 2 V buffers
    for l in lines:
        if l.startswith("ds_read"):
            off = int(l.split("offset:")[1])
            limit = 4 * 16384 if "%[ka" in l else 2 * 16384
            assert 0 <= off < limit, l
    # no per-tile address arithmetic on the read addresses
    assert not any(l.startswith("v_add_u32") and "%[ka" in l or "%[va" in l and l.startswith("v_add") for l in lines)
    # tile copies are only ever waited for as a whole, before a barrier
    assert not any(l.startswith("s_waitcnt vmcnt(") and l != "s_waitcnt vmcnt(0)" for l in lines)


def _regset(tok):
    m = re.fullmatch(r"([va])\[(\d+):(\d+)\]", tok) or re.fullmatch(r"([va])(\d+)", tok)
    lo = int(m.group(2))
    hi = int(m.group(3)) if m.lastindex == 3 else lo
    return {(m.group(1), r) for r in range(lo, hi + 1)}


def _simulate_lds_waits(lines, in_flight):
    """In-order LDS completion model: lgkmcnt(n) leaves at most the n most recent reads pending.
    Fails if an MFMA or VALU instruction reads, or an LDS read overwrites, a register that a
    pending LDS read still writes."""
    pending = list(in_flight)  # register sets of reads not yet known complete, oldest first
    for l in lines:
        op = l.split()[0] if l.split() else ""
        if op.startswith("ds_read"):
            dst = _regset(l.split()[1].rstrip(","))
            assert not any(dst & p for p in pending), f"LDS read overwrites a pending destination: {l}"
            pending.append(dst)
        elif op == "s_waitcnt" and "lgkmcnt(" in l:
            n = int(l.split("lgkmcnt(")[1].rstrip(")"))
            pending = pending[len(pending) - n:] if n < len(pending) else pending
            if n == 0:
                pending = []
        elif op.startswith("v_"):
            toks = [t.rstrip(",") for t in l.split()[1:]]
            srcs = toks[1:] if op.startswith("v_mfma") else toks
            for t in srcs:
                if re.fullmatch(r"[va](\[\d+:\d+\]|\d+)", t):
                    regs = _regset(t)
                    assert not any(regs & p for p in pending), f"reads a register still being loaded: {l}"
    return pending


@pytest.mark.parametrize("gen", ["narrow", "narrow_l8", "wide"])
def test_lds_waits_cover_every_fragment_use(gen):
    mod = GW if gen == "wide" else G
    saved = G.FR
    G.FR = G.FRAGS[8] if gen == "narrow_l8" else G.FRAGS[4]  # the 8-copy loop's deeper prefetch
    try:
        _check_lds_waits(gen, mod)
    finally:
        G.FR = saved


def _check_lds_waits(gen, mod):
    for has_next, masked in ((True, False), (True, True), (False, False)):
        for parity in (0, 1):
            A = mod.Asm()
            if gen == "wide":
                cur, nxt = (GW.V_SA, GW.V_SB) if parity == 0 else (GW.V_SB, GW.V_SA)
                GW.block(A, cur, nxt, has_next, masked, (parity + 1) % GW.NKBUF, parity % GW.NVBUF)
                # entry state: K fragments 0..2 of the next tile in flight (issued before the barrier)
                entry = [_regset(f"v[{GW.V_KF + 4 * i}:{GW.V_KF + 4 * i + 3}]") for i in range(3)] if has_next else []
            else:
                cur, nxt = (G.SA_BASE, G.SB_BASE) if parity == 0 else (G.SB_BASE, G.SA_BASE)
                G.block(A, cur, nxt, 1 - parity, parity, has_next, masked)
                entry = []
            left = _simulate_lds_waits(A.lines, entry)
            assert not left or gen == "wide", "narrow blocks leave no LDS read pending"


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None, reason="hipcc not available")
def test_wide_operand_registers_do_not_overlap_loop_writes(tmp_path):
    asm = tmp_path / "wide.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--cuda-device-only", "-S",
           "-o", str(asm), os.path.join(CSRC, "attn_bf16_d128_wide.hip")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    names = GW.check_operand_allocation(asm.read_text())
    expected = {"ka%d" % i for i in range(8)} | {"va%d" % i for i in range(4)} | \
               {"koff%d" % i for i in range(4)} | {"voff%d" % i for i in range(4)} | \
               {"mrun0", "mrun1", "lrun0", "lrun1", "nmc0", "nmc1", "base2_0", "base2_1", "c", "thr", "nkt",
                "tmask", "kvlim", "rowb", "kp_lo", "kp_hi", "vp_lo", "vp_hi", "tstride_lo", "tstride_hi",
                "kdst0", "vdst0"}
    assert expected <= set(names), expected - set(names)

#!/usr/bin/env python3
"""Writes attn_loop_d128.inc: the main loop of the pipelined bf16 attention kernel (D = 128) as the
text of one inline-asm statement, scheduled by hand for CDNA4 (gfx950).  The build runs this script
before compiling attn_bf16_d128.hip, which defines the operands and the C++ around the loop.

Per 64-key tile t, for a wavefront of 32 query rows (the kernel source explains the layout):
  phase A: S(t+1) = K(t+1) Q^T, 16 v_mfma_f32_32x32x16_bf16, each followed by a slice of the
           softmax of tile t (p = 2^(s*c + neg_mc) and the bf16 packing of P into its own
           registers) and by one group of scalar work for the copies of K(t+2) and V(t+1);
  phase B: O^T += V(t)^T P(t)^T, 16 MFMAs, each followed by a slice of the mask and row max of
           tile t+1; in unmasked tiles the row max is complete by slot 7, and the exchange across
           the half-waves and the rescale test (into SCC) follow in slots 8..13.
  Unmasked tiles split the softmax between the phases with the list scheduler of the wide loop:
  the exponentials of the first 12 pairs and the packing of the first 16-key step in phase A;
  the other exponentials and packings (each two MFMAs before the value product that reads it)
  and the fp32 row sums, in pair order, in phase B.  Masked tiles keep the whole softmax and the
  row sums in phase A (the mask adds VALU work to phase B).
  then the lazy running-max update (a branch taken only when some row needs it) and the barrier.
Fragments are read from LDS three MFMAs ahead (five in the 8-copy variant, whose single wavefront
per SIMD has no partner to cover the latency; the first V fragments during the last slots of
phase A); each wait covers exactly the fragment needed.
The loop runs over nkt tiles starting at key tile tbase (0, or the second half of the key range
when two wavefront groups of one workgroup split the keys); tmask counts from tbase.

Register map (physical VGPRs, pinned by the operand constraints):
  O^T[db]   a[16db : 16db+15]           (fp32 accumulators in AGPRs, 4 blocks of 32 dims)
  S set A   v[128:159], S set B v[96:127] (scores of the current / next tile, alternating)
  Q^T[t]    v[64+4t : 67+4t]            (bf16 fragments, loaded once)
  P(ks)     v[160+4ks : 163+4ks]        (bf16 probabilities of the current tile, 16 keys per step)
  K frags   v[48:63], V frags v[32:47]   (rotating prefetch buffers; 8-copy variant: six each,
                                          v[176:199] and v[200:223])
  v31 row sum, v30 row max, v29 -inf, v28/v27 temporaries (the rescale also uses v[48:55]); s[80:99] scalar
  temporaries.
Wait states: every VALU read of an MFMA result, and every MFMA read of a VALU result, is separated
from the writer by at least two MFMAs or three s_nop 7, so no hazard needs hardware interlocks.
"""
import sys

from gen_attn_loop_wide import pack  # the list scheduler that fills MFMA slots with VALU groups

SA_BASE, SB_BASE, Q_BASE, K_BASE, V_BASE = 128, 96, 64, 48, 32
P_BASE = 160                 # bf16 probabilities of the current tile: P(ks) in v[160 + 4ks : +3]
O_AGPR = 0                   # O^T accumulators in a[0:63]
TMP_BASE, N_TMP = 48, 8      # rescale temporaries: the K fragment buffers, idle at that point


class Frag:
    """Fragment prefetch of a loop variant: reads run `pf` fragments ahead of the MFMA that uses
    them, through pf + 1 rotating 4-register buffers for K at `kbase` and for V at `vbase`."""
    def __init__(self, pf, kbase, vbase):
        self.pf, self.kbase, self.vbase = pf, kbase, vbase

    def regs(self):
        n = 4 * (self.pf + 1)
        return set(range(self.kbase, self.kbase + n)) | set(range(self.vbase, self.vbase + n))


# Two wavefronts per SIMD cover each other's LDS latency: three fragments ahead.  The 64-row split
# form runs one wavefront per SIMD and has registers to spare (one workgroup per CU): five ahead,
# its buffers above the pinned sets (v[176:223]).
FRAG_L4 = Frag(3, K_BASE, V_BASE)
FRAG_L8 = Frag(5, 176, 200)
FRAGS = {4: FRAG_L4, 8: FRAG_L8}  # per loop variant (copies per lane)
FR = FRAG_L4  # the variant being generated
RS, MX, NEGINF, T0, ALPHA = 31, 30, 29, 28, 27
# scalar temporaries (clobbered)
S_T, S_T1, S_KEY, S_ROWS, S_TMP = 80, 81, 82, 83, 84
S_KP, S_VP = 86, 88          # running 64-bit K/V tile pointers (pairs)
S_KR, S_VR = 92, 96          # buffer resource quads (aligned)
S_C = 82                     # rescale-test lane mask (pair; S_KEY/S_ROWS are free in phase B)
TILE_BYTES = 16384
SLOT_BUDGET = 13             # VALU issue units per MFMA slot (v_exp 5, other VALU 2; see the wide loop)
N_A = 12                     # softmax pairs of an unmasked tile whose FMA/exp run in phase A


def vr(a, n=1):
    return f"v{a}" if n == 1 else f"v[{a}:{a + n - 1}]"


def ar(a, n=1):
    return f"a{a}" if n == 1 else f"a[{a}:{a + n - 1}]"


def sr(a, n=1):
    return f"s{a}" if n == 1 else f"s[{a}:{a + n - 1}]"


class Asm:
    def __init__(self):
        self.lines = []
        self.lds_ops = 0

    def e(self, s):
        self.lines.append(s)

    def lds(self, s):
        self.e(s)
        self.lds_ops += 1
        return self.lds_ops - 1

    def wait_for(self, op):
        n = max(0, min(self.lds_ops - 1 - op, 15))
        self.e(f"s_waitcnt lgkmcnt({n})")


def block(A, cur_base, nxt_base, kbuf, vbuf, has_next, mask_next, extra_a=()):
    """One tile: phase A (QK of tile t+1 || probabilities of tile t), phase B (PV of t || mask+max of t+1).
    extra_a: groups of scalar work (the tile copies) placed after the MFMAs of phase A."""
    A.lds_ops = 0
    A.e("s_waitcnt lgkmcnt(0)")
    A.e(f"v_mov_b32 {vr(RS)}, 0")
    if mask_next:
        A.e(f"v_mov_b32 {vr(NEGINF)}, 0xff800000")
        # per-lane bound for tile t+1: hide key c (in-tile, minus 4hi) iff c >= base2 - key0
        A.e(f"v_subrev_u32_e32 {vr(T0)}, {sr(S_KEY)}, %[base2]")

    def cur(kb, r):
        return cur_base + 16 * kb + r

    def nxt(kb, r):
        return nxt_base + 16 * kb + r

    k_ops, v_ops = {}, {}

    def issue_k(i):
        kb, tt = divmod(i, 8)
        off = kbuf * TILE_BYTES + kb * 8192
        k_ops[i] = A.lds(f"ds_read_b128 {vr(FR.kbase + 4 * (i % (FR.pf + 1)), 4)}, %[ka{tt}] offset:{off}")

    def issue_v(i):
        ks, db = divmod(i, 4)
        base = FR.vbase + 4 * (i % (FR.pf + 1))
        off = vbuf * TILE_BYTES + ks * 4096
        A.lds(f"ds_read_b64_tr_b16 {vr(base, 2)}, %[va{db}] offset:{off}")
        v_ops[i] = A.lds(f"ds_read_b64_tr_b16 {vr(base + 2, 2)}, %[va{db}] offset:{off + 2048}")

    # pair p = 4ks + m: elements r = 8h + 2m, r + 1 of score block kb (ks = 2kb + h); the pairs
    # in this order are also the row-sum order
    pairs = []
    for p in range(16):
        ks, m = divmod(p, 4)
        kb, h = divmod(ks, 2)
        a = cur(kb, 8 * h + 2 * m)
        pairs.append((ks, m, a, a + 1))

    def cvt(p):
        ks, m, a, b = pairs[p]
        return f"v_cvt_pk_bf16_f32 {vr(P_BASE + 4 * ks + m)}, {vr(a)}, {vr(b)}"

    def rowsum(p):
        ks, m, a, b = pairs[p]
        return [f"v_add_f32_e32 {vr(RS)}, {vr(RS)}, {vr(a)}", f"v_add_f32_e32 {vr(RS)}, {vr(RS)}, {vr(b)}"]

    def softmax(p):
        ks, m, a, b = pairs[p]
        return ([f"v_fma_f32 {vr(a)}, {vr(a)}, %[c], %[nmc]"], [f"v_exp_f32_e32 {vr(a)}, {vr(a)}"],
                [f"v_fma_f32 {vr(b)}, {vr(b)}, %[c], %[nmc]"], [f"v_exp_f32_e32 {vr(b)}, {vr(b)}"])

    balanced = has_next and not mask_next
    if balanced:
        stream = []
        for p in range(N_A):
            stream += [(g, 15, None, False) for g in softmax(p)]
            if p < 4:  # the first 16-key step of P: read by the first value-product MFMA
                stream.append(([cvt(p)], 13, len(stream) - 1, False))
        slots, _ = pack(stream, [[] for _ in range(16)], SLOT_BUDGET, nslots=16)
    else:
        slots = []
        for p in range(16):
            f, ea, fb, eb = softmax(p)
            slots.append(f + fb + ea + eb + rowsum(p))
        for p in range(16):  # packing one slot after its exponentials (transcendental -> VALU)
            slots[min(p + 1, 15)].append(cvt(p))

    if has_next:
        for i in range(FR.pf):
            issue_k(i)
        for i in range(16):
            if i + FR.pf < 16:
                issue_k(i + FR.pf)
            else:
                issue_v(i + FR.pf - 16)  # the first V fragments of phase B: V(t) is visible since the last barrier
            kb, tt = divmod(i, 8)
            A.wait_for(k_ops[i])
            src2 = "0" if tt == 0 else vr(nxt(kb, 0), 16)
            A.e(f"v_mfma_f32_32x32x16_bf16 {vr(nxt(kb, 0), 16)}, {vr(FR.kbase + 4 * (i % (FR.pf + 1)), 4)}, "
                f"{vr(Q_BASE + 4 * tt, 4)}, {src2}")
            for op in slots[i]:
                A.e(op)
            for op in (extra_a[i] if i < len(extra_a) else []):
                A.e(op)
    else:
        for i in range(16):
            for op in slots[i]:
                A.e(op)
        for i in range(FR.pf):
            issue_v(i)

    bsl = [[] for _ in range(16)]
    if has_next:
        mpairs = [(nxt(kb, r), nxt(kb, r + 1)) for kb in range(2) for r in range(0, 16, 2)]
        if mask_next:
            for kb in range(2):
                for r in range(16):
                    slot = kb * 8 + r // 2
                    e_ = nxt(kb, r)
                    cconst = kb * 32 + (r >> 2) * 8 + (r & 3)
                    bsl[slot].append(f"v_cmp_ge_i32_e32 vcc, {cconst}, {vr(T0)}")
                    bsl[slot].append(f"v_cndmask_b32_e32 {vr(e_)}, {vr(e_)}, {vr(NEGINF)}, vcc")
            for pi, (ea, eb) in enumerate(mpairs):
                if pi == 0:
                    bsl[pi].append(f"v_max_f32_e32 {vr(MX)}, {vr(ea)}, {vr(eb)}")
                else:
                    bsl[pi].append(f"v_max3_f32 {vr(MX)}, {vr(MX)}, {vr(ea)}, {vr(eb)}")
        else:
            # the row max of S(t+1) in slots 0..7 (block kb = 1, written by the last MFMA of phase A,
            # from slot 4 on); then the exchange across the half-waves and the rescale test, each step
            # one slot after the one it reads (VALU -> permlane, permlane -> VALU, VALU-written SGPR ->
            # SALU); T0 ends as m_run + thr, which the rescale path reads.
            for pi, (ea, eb) in enumerate(mpairs):
                if pi == 0:
                    bsl[0].append(f"v_max_f32_e32 {vr(MX)}, {vr(ea)}, {vr(eb)}")
                else:
                    bsl[pi // 2].append(f"v_max3_f32 {vr(MX)}, {vr(MX)}, {vr(ea)}, {vr(eb)}")
            bsl[8].append(f"v_mov_b32 {vr(T0)}, {vr(MX)}")
            bsl[9].append(f"v_permlane32_swap_b32_e32 {vr(T0)}, {vr(MX)}")
            bsl[10].append(f"v_max_f32_e32 {vr(MX)}, {vr(T0)}, {vr(MX)}")
            bsl[11].append(f"v_add_f32_e32 {vr(T0)}, %[thr], %[mrun]")
            bsl[12].append(f"v_cmp_gt_f32_e64 {sr(S_C, 2)}, {vr(MX)}, {vr(T0)}")
            bsl[13].append(f"s_cmp_lg_u64 {sr(S_C, 2)}, 0")                  # SCC: some row rescales
            # the rest of the softmax of tile t: exponentials of pairs N_A.. and packings (each
            # two MFMAs before the value product that reads it), then the row sums in pair order
            stream, exp_b, cvt_dep = [], {}, {}
            for ks in range(1, 4):
                dl = 4 * ks - 2
                for p in range(4 * ks, 4 * ks + 4):
                    if p >= N_A:
                        stream += [(g, dl - 1, None, False) for g in softmax(p)]
                        exp_b[p] = len(stream) - 1
                for p in range(4 * ks, 4 * ks + 4):
                    stream.append(([cvt(p)], dl, exp_b.get(p), False))
            for p in range(16):
                stream.append((rowsum(p), 15, exp_b.get(p), True))
            bsl, _ = pack(stream, bsl, SLOT_BUDGET, nslots=16)

    for i in range(16):
        if i + FR.pf < 16:
            issue_v(i + FR.pf)
        ks, db = divmod(i, 4)
        kb, h = divmod(ks, 2)
        A.wait_for(v_ops[i])
        A.e(f"v_mfma_f32_32x32x16_bf16 {ar(O_AGPR + 16 * db, 16)}, {vr(FR.vbase + 4 * (i % (FR.pf + 1)), 4)}, "
            f"{vr(P_BASE + 4 * ks, 4)}, {ar(O_AGPR + 16 * db, 16)}")
        for op in bsl[i]:
            A.e(op)

    if has_next and mask_next:
        A.e("s_nop 1")
        A.e(f"v_mov_b32 {vr(T0)}, {vr(MX)}")
        A.e("s_nop 1")
        A.e(f"v_permlane32_swap_b32_e32 {vr(T0)}, {vr(MX)}")
        A.e("s_nop 1")
        A.e(f"v_max_f32_e32 {vr(MX)}, {vr(T0)}, {vr(MX)}")
        A.e(f"v_add_f32_e32 {vr(T0)}, %[thr], %[mrun]")
        A.e(f"v_cmp_gt_f32_e64 {sr(S_C, 2)}, {vr(MX)}, {vr(T0)}")
        A.e("s_nop 4")
        A.e(f"s_cmp_lg_u64 {sr(S_C, 2)}, 0")
    A.e(f"v_add_f32_e32 %[lrun], %[lrun], {vr(RS)}")


def rescale(A):
    """Out-of-line path, taken after phase B when the test found a row whose tile max exceeds
    m_run + thr (SCC set; rare): raise the running max of those rows, rescale O^T and l_run, and
    follow with neg_mc.  T0 holds m_run + thr and MX the row max of tile t+1."""
    # O^T, written by the value product just before, is read by VALU below: >= 24 wait states
    A.e("s_nop 7")
    A.e("s_nop 7")
    A.e("s_nop 7")
    A.e(f"v_cmp_gt_f32_e32 vcc, {vr(MX)}, {vr(T0)}")
    A.e(f"v_cndmask_b32_e32 {vr(T0)}, %[mrun], {vr(MX)}, vcc")        # m_new
    A.e(f"v_sub_f32_e32 {vr(ALPHA)}, %[mrun], {vr(T0)}")
    A.e(f"v_mul_f32_e32 {vr(ALPHA)}, %[c], {vr(ALPHA)}")
    A.e(f"v_exp_f32_e32 {vr(ALPHA)}, {vr(ALPHA)}")
    A.e("s_nop 0")                                                       # transcendental result -> VALU
    A.e(f"v_cndmask_b32_e64 {vr(ALPHA)}, 1.0, {vr(ALPHA)}, vcc")      # lanes that keep their max: 1
    A.e(f"v_mov_b32 %[mrun], {vr(T0)}")
    A.e(f"v_mul_f32_e32 %[lrun], %[lrun], {vr(ALPHA)}")
    # O^T lives in AGPRs: read 8 at a time into temporaries, scale, write back
    for g in range(0, 64, N_TMP):
        for j in range(N_TMP):
            A.e(f"v_accvgpr_read_b32 {vr(TMP_BASE + j)}, {ar(O_AGPR + g + j)}")
        for j in range(N_TMP):
            A.e(f"v_mul_f32_e32 {vr(TMP_BASE + j)}, {vr(TMP_BASE + j)}, {vr(ALPHA)}")
        for j in range(N_TMP):
            A.e(f"v_accvgpr_write_b32 {ar(O_AGPR + g + j)}, {vr(TMP_BASE + j)}")
    A.e(f"v_mul_f32_e64 %[nmc], -%[mrun], %[c]")                      # neg_mc follows m_run
    A.e(f"v_cmp_eq_f32_e32 vcc, 0xff800000, %[mrun]")
    A.e(f"v_cndmask_b32_e64 %[nmc], %[nmc], 0, vcc")
    A.e("s_nop 1")


def dma_groups(which, ahead, buf, nloads=4):
    """Copy of tile t + ahead of K or V into LDS buffer `buf`, without branches: past this group's
    last tile the copy has 0 valid rows (no memory is read; the buffer it fills is not read
    again).  Returned as groups of scalar instructions, each placed after one MFMA of phase A;
    every SCC producer sits next to its consumer inside a group.  nloads: 16-byte copies per lane
    (4 rows of the tile each) -- 4 when four wavefronts share a tile, 8 when two do (then two
    copies per group, so the groups of a K and a V copy still fit the 16 phase-A slots)."""
    ptr, rsrc, offs, dst = (S_KP, S_KR, "koff", "kdst") if which == "k" else (S_VP, S_VR, "voff", "vdst")
    g = []
    g.append([f"s_add_u32 {sr(S_TMP)}, {sr(S_T)}, {ahead}",
              f"s_add_u32 {sr(S_ROWS)}, {sr(S_TMP)}, %[tbase]",     # tile index in the key tensor
              f"s_lshl_b32 {sr(S_ROWS)}, {sr(S_ROWS)}, 6",           # rows = min(64, kv_lim - 64 tile)
              f"s_sub_i32 {sr(S_ROWS)}, %[kvlim], {sr(S_ROWS)}",
              f"s_min_i32 {sr(S_ROWS)}, {sr(S_ROWS)}, 64",
              f"s_max_i32 {sr(S_ROWS)}, {sr(S_ROWS)}, 0",
              f"s_cmp_lt_u32 {sr(S_TMP)}, %[nkt]",                   # no such tile: 0 rows
              f"s_cselect_b32 {sr(S_ROWS)}, {sr(S_ROWS)}, 0"])
    g.append([f"s_mul_i32 {sr(rsrc + 2)}, {sr(S_ROWS)}, %[rowb]",
              f"s_mov_b32 {sr(rsrc)}, {sr(ptr)}",
              f"s_and_b32 {sr(rsrc + 1)}, {sr(ptr + 1)}, 0xffff",
              f"s_mov_b32 {sr(rsrc + 3)}, 0x20000",
              f"s_add_u32 {sr(S_TMP)}, %[{dst}0], {buf * TILE_BYTES}"])
    per_group = nloads // 4
    for u0 in range(0, nloads, per_group):
        c = []
        for u in range(u0, u0 + per_group):
            c += [f"s_mov_b32 m0, {sr(S_TMP)}", "s_nop 0", f"buffer_load_dwordx4 %[{offs}{u}], {sr(rsrc, 4)}, 0 offen lds"]
            if u < nloads - 1:
                c.append(f"s_add_u32 {sr(S_TMP)}, {sr(S_TMP)}, 1024")
        g.append(c)
    g.append([f"s_add_u32 {sr(ptr)}, {sr(ptr)}, %[tstride_lo]",     # advance the running pointer
              f"s_addc_u32 {sr(ptr + 1)}, {sr(ptr + 1)}, %[tstride_hi]"])
    return g


def half(A, parity, uid, cold, nloads=4):
    """Process tile t (= S_T) whose S lives in set A (parity 0) or B (parity 1).  The common path
    (an unmasked tile that moves no running max) runs straight through; the masked block and the
    rescale go to `cold`, emitted after the loop, and branch back."""
    cur_base, nxt_base = (SA_BASE, SB_BASE) if parity == 0 else (SB_BASE, SA_BASE)
    kb_read = 1 - parity       # K buffer holding tile t+1
    vb_read = parity           # V buffer holding tile t
    p = f"{parity}_{uid}"
    # K(t+2) -> K buffer t&1 (held K(t)), V(t+1) -> V buffer (t+1)&1 (held V(t-1)), both consumed
    # before the last barrier; 7 + 7 groups over the 16 phase-A slots
    extra_a = dma_groups("k", 2, parity, nloads) + [[]] + dma_groups("v", 1, 1 - parity, nloads)
    A.e(f"s_add_u32 {sr(S_T1)}, {sr(S_T)}, 1")
    A.e(f"s_cmp_lt_u32 {sr(S_T1)}, %[nkt]")
    A.e(f"s_cbranch_scc0 Llast{p}")
    A.e(f"s_add_u32 {sr(S_KEY)}, {sr(S_T1)}, %[tbase]")
    A.e(f"s_lshl_b32 {sr(S_KEY)}, {sr(S_KEY)}, 6")
    A.e(f"s_cmp_ge_u32 {sr(S_T1)}, %[tmask]")
    A.e(f"s_cbranch_scc1 Lmask{p}")
    block(A, cur_base, nxt_base, kb_read, vb_read, True, False, extra_a)
    A.e(f"Lpost{p}:")
    A.e(f"s_cbranch_scc1 Lresc{p}")       # SCC from the rescale test: some row's max moved
    A.e(f"Lback{p}:")
    cold.e(f"Lmask{p}:")
    block(cold, cur_base, nxt_base, kb_read, vb_read, True, True, extra_a)
    cold.e(f"s_branch Lpost{p}")
    cold.e(f"Lresc{p}:")
    rescale(cold)
    cold.e(f"s_branch Lback{p}")
    A.e("s_waitcnt vmcnt(0)")
    A.e("s_barrier")
    A.e(f"s_add_u32 {sr(S_T)}, {sr(S_T)}, 1")


def last(A, parity, uid):
    cur_base, nxt_base = (SA_BASE, SB_BASE) if parity == 0 else (SB_BASE, SA_BASE)
    A.e(f"Llast{parity}_{uid}:")
    block(A, cur_base, nxt_base, 1 - parity, parity, False, False)
    A.e(f"s_branch Lend_{uid}")


def gen_loop(nloads=4):
    """The loop for tile copies of `nloads` 16-byte copies per lane (see dma_groups), with that
    variant's fragment prefetch (FRAGS)."""
    global FR
    saved, FR = FR, FRAGS[nloads]
    try:
        return _gen_loop(nloads)
    finally:
        FR = saved


def _gen_loop(nloads):
    A = Asm()
    uid = "%="
    # running tile pointers: K starts at tile 2 (tiles 0, 1 are loaded before the loop), V at tile 1
    A.e(f"s_mov_b32 {sr(S_T)}, 0")
    A.e(f"s_mov_b32 {sr(S_KP)}, %[kp_lo]")
    A.e(f"s_mov_b32 {sr(S_KP + 1)}, %[kp_hi]")
    A.e(f"s_mov_b32 {sr(S_VP)}, %[vp_lo]")
    A.e(f"s_mov_b32 {sr(S_VP + 1)}, %[vp_hi]")
    A.e(f"s_cmp_lt_u32 {sr(S_T)}, %[nkt]")
    A.e(f"s_cbranch_scc0 Lend_{uid}")
    A.e(f"Ltop_{uid}:")
    cold = Asm()
    half(A, 0, uid, cold, nloads)
    half(A, 1, uid, cold, nloads)
    A.e(f"s_cmp_lt_u32 {sr(S_T)}, %[nkt]")
    A.e(f"s_cbranch_scc1 Ltop_{uid}")
    A.e(f"s_branch Lend_{uid}")
    A.lines += cold.lines
    last(A, 0, uid)
    last(A, 1, uid)
    A.e(f"Lend_{uid}:")
    # the code after the statement reads O^T, written by the last value-product MFMAs: >= 24 wait
    # states (the compiler does not see the MFMAs inside the statement)
    A.e("s_nop 7")
    A.e("s_nop 7")
    A.e("s_nop 7")
    return A.lines


# Registers the loop writes besides its own "+v" operands: pinned accumulator / score sets and
# the clobber list.  No input operand may be allocated inside these.
WRITTEN_VGPRS = set(range(27, 64)) | set(range(96, 176)) | set(range(TMP_BASE, TMP_BASE + N_TMP))
WRITTEN_SGPRS = set(range(80, 100))
WRITTEN_AGPRS = set(range(O_AGPR, O_AGPR + 64))
READ_WRITE_OPERANDS = ("mrun", "lrun", "nmc")


def _regs(tok):
    """'v5' -> ('v', {5}); 's[4:7]' -> ('s', {4..7}); 'a3' -> ('a', {3}); anything else -> None."""
    import re
    m = re.fullmatch(r"-?([vsa])(\d+)", tok) or re.fullmatch(r"-?([vsa])\[(\d+):(\d+)\]", tok)
    if not m:
        return None
    lo = int(m.group(2))
    hi = int(m.group(3)) if m.lastindex == 3 else lo
    return m.group(1), set(range(lo, hi + 1))


def check_operand_allocation(compiled_asm: str) -> dict:
    """Matches every instance of the loop in compiler output (the text between ASMSTART and
    ASMEND that starts like the loop) against the template, and checks that each named operand
    got one register, that no two operands share one (read-write operands with anything) and that
    no operand lies in a register the loop writes.  Returns {operand: register} of the last
    instance; raises AssertionError on a violation."""
    import re
    tpls = {len(gen_loop(n)): (gen_loop(n), n) for n in LOOP_VARIANTS}
    first = next(iter(tpls.values()))[0][0]
    blocks = re.findall(r";;#ASMSTART\n(.*?);;#ASMEND", compiled_asm, flags=re.S)
    loops = [b for b in blocks if b.lstrip().startswith(first.split()[0] + " s80, 0")]
    assert loops, "loop statement not found in the compiled assembly"
    result = {}
    for body in loops:
        got = [l.strip() for l in body.strip().splitlines() if l.strip()]
        assert len(got) in tpls, (len(got), sorted(tpls))
        tpl, nloads = tpls[len(got)]
        names = {}
        for t, g in zip(tpl, got):
            pat, keys = "", []
            for part in re.split(r"(%\[\w+\]|%=)", t):
                if part == "%=":
                    pat += r"\d+"
                elif part.startswith("%["):
                    keys.append(part[2:-1])
                    pat += r"(\S+?)"
                else:
                    pat += re.escape(part)
            m = re.fullmatch(pat, g.split(" ;")[0].rstrip(","))
            assert m, f"compiled line does not match template: {g!r} vs {t!r}"
            for k, v in zip(keys, m.groups()):
                v = v.lstrip("-")
                assert names.setdefault(k, v) == v, f"operand {k} in two registers: {names[k]}, {v}"
        owner = {}
        for k, v in names.items():
            r = _regs(v)
            if r is None:
                continue  # literal or special operand
            kind, regs = r
            written = {"v": WRITTEN_VGPRS | clobbered_vgprs(nloads), "s": WRITTEN_SGPRS, "a": WRITTEN_AGPRS}[kind]
            assert not (regs & written), f"operand {k} = {v} lies in a register the loop writes"
            for x in regs:
                other = owner.setdefault((kind, x), k)
                if other != k and (k in READ_WRITE_OPERANDS or other in READ_WRITE_OPERANDS):
                    raise AssertionError(f"read-write operand shares {kind}{x}: {k}, {other}")
        result = names
    return result


# Loop variants written to the .inc: copies per lane and tile -> macro name (the first is the one
# the four-wavefront groups use; the L8 loop serves groups of two wavefronts).
LOOP_VARIANTS = {4: "THA_ATTN_LOOP_ASM", 8: "THA_ATTN_LOOP_ASM_L8"}


def clobbered_vgprs(nloads):
    """VGPRs the loop variant writes outside its operands (its clobber list)."""
    v = set(range(V_BASE, V_BASE + 32)) | {RS, MX, NEGINF, T0, ALPHA}
    v |= set(range(TMP_BASE, TMP_BASE + N_TMP)) | set(range(P_BASE, P_BASE + 16))
    return v | FRAGS[nloads].regs()


def main(out):
    sclob = [f"s{i}" for i in range(80, 100)]
    txt = "// Generated by gen_attn_loop.py (do not edit): main loop of the pipelined bf16 attention kernel.\n"
    for nloads, name in LOOP_VARIANTS.items():
        body = "".join('      "%s\\n\\t" \\\n' % l for l in gen_loop(nloads))
        txt += f"#define {name} \\\n" + body + "\n"
    base = [f"v{i}" for i in range(V_BASE, V_BASE + 32)] + [f"v{i}" for i in (RS, MX, NEGINF, T0, ALPHA)]
    base += [f"v{i}" for i in range(TMP_BASE, TMP_BASE + N_TMP)] + [f"v{i}" for i in range(P_BASE, P_BASE + 16)]
    for nloads, suffix in ((4, ""), (8, "_L8")):
        extra = sorted(clobbered_vgprs(nloads) - clobbered_vgprs(4))
        assert {int(c[1:]) for c in base} | set(extra) == clobbered_vgprs(nloads)
        clob = ", ".join('"%s"' % c for c in base + [f"v{i}" for i in extra] + sclob + ["vcc", "scc", "m0", "memory"])
        txt += f"#define THA_ATTN_LOOP_CLOBBERS{suffix} " + clob + "\n"
    open(out, "w").write(txt)


if __name__ == "__main__":
    import os
    main(sys.argv[1] if len(sys.argv) > 1 else os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                            "attn_loop_d128.inc"))

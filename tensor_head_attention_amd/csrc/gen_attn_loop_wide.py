#!/usr/bin/env python3
"""Writes attn_loop_d128_wide.inc: the main loop of the wide bf16 attention kernel (head size 128,
64 query rows per wavefront) as the text of one inline-asm statement, scheduled by hand for CDNA4
(gfx950).  The build runs this script before compiling attn_bf16_d128_wide.hip, which defines the
operands and the C++ around the loop.

Per 64-key tile t, for a wavefront of 64 query rows (two 32-row blocks qb = 0, 1):
  phase A: S(t+1) = K(t+1) Q^T, 32 v_mfma_f32_32x32x16_bf16 (each K fragment read from LDS feeds
           the MFMAs of both row blocks), each followed by a slice of the softmax of tile t:
           p = 2^(s*c + neg_mc) and the bf16 packing of P into its own registers;
  phase B: O^T += V(t)^T P(t)^T, 32 MFMAs (each V fragment feeds both row blocks), each followed
           by a slice of the row sums of tile t (fp32) and of the mask and row max of tile t+1;
  then the lazy running-max update and the barrier.
K tiles live in four LDS buffers (tile t in buffer t mod 4) and V tiles in two (t mod 2), and the
loop is unrolled four times, so every LDS read and copy destination is a fixed offset (no address
arithmetic per tile).  Block t copies K(t+3) and V(t+1); the first K fragments of the next block
are read before the barrier that ends this one (K(t+2) is visible since the previous barrier), so
no LDS read waits behind a barrier.  Fragment reads run three fragments (six MFMAs) ahead; each
wait covers exactly the fragment needed.

Register map (pinned by the operand constraints):
  O^T[qb][db]  a[64qb + 16db : +15]       fp32 accumulators (AGPRs)
  Q^T[qb][tt]  a[128 + 32qb + 4tt : +3]   bf16 B operands of the score product (AGPRs)
  S sets       v[128:191] (A), v[192:255] (B); S[qb][kb] at base + 32qb + 16kb
  K frags      v[96:111], V frags v[112:127] (4 rotating fragments each)
  P[qb][ks]    v[64 + 16qb + 4ks : +3]    bf16 probabilities of the current tile
  v[54:63]     row max / mask bound / alpha / row sum per row block, -inf, a temporary
  s[80:99]     scalar temporaries
LDS: K buffers 0..3 at 16 KiB steps from %[ka*]'s base, V buffers 0..1 from %[va*]'s base.
Wait states: VALU reads of MFMA results and MFMA reads of VALU results are separated by at least
two MFMAs; before O^T is read by VALU the loop issues three s_nop 7.
"""
import os
import re
import sys

# ---- registers ----
A_O, A_Q = 0, 128
V_SA, V_SB = 128, 192
V_KF, V_VF, V_P = 96, 112, 64
V_MX = (62, 63)
V_T0 = (60, 61)
V_AL = (58, 59)
V_RS = (56, 57)
V_NEGINF = 55
V_TMP = 54
TMP_BASE, N_TMP = V_VF, 8   # rescale temporaries: the V fragment buffers, idle at that point

S_T, S_T1, S_KEY, S_ROWS, S_TMP, S_X = 80, 81, 82, 83, 84, 85
S_KP, S_VP = 86, 88          # running 64-bit K / V tile pointers
S_Y = 91
S_KR, S_VR = 92, 96          # buffer resource quads
S_C = (82, 84)               # rescale-test lane masks of the row blocks (S_KEY/S_ROWS, S_TMP/S_X: free then)
TILE_BYTES = 16384
NKBUF, NVBUF = 4, 2          # K and V LDS buffers; the loop is unrolled NKBUF times


def vr(a, n=1):
    return f"v{a}" if n == 1 else f"v[{a}:{a + n - 1}]"


def ar(a, n=1):
    return f"a{a}" if n == 1 else f"a[{a}:{a + n - 1}]"


def sr(a, n=1):
    return f"s{a}" if n == 1 else f"s[{a}:{a + n - 1}]"


class Asm:
    def __init__(self):
        self.lines = []
        self.n_ops = 0  # LDS ops issued in the current block (including those in flight at entry)

    def e(self, s):
        self.lines.append(s)

    def lds(self, s):
        self.e(s)
        self.n_ops += 1
        return self.n_ops - 1

    def wait_for(self, op):
        n = max(0, min(self.n_ops - 1 - op, 15))
        self.e(f"s_waitcnt lgkmcnt({n})")


def s_reg(base, qb, kb, r=0):
    return base + 32 * qb + 16 * kb + r


def issue_k(A, i, kbuf):
    """K fragment i (kb = i // 8, dims 16tt..: tt = i % 8) of the tile in K buffer kbuf."""
    kb, tt = divmod(i, 8)
    return A.lds(f"ds_read_b128 {vr(V_KF + 4 * (i % 4), 4)}, %[ka{tt}] offset:{kbuf * TILE_BYTES + kb * 8192}")


def issue_v(A, j, vbuf):
    """V fragment j (16-key step ks = j // 4, 32-dim block db = j % 4) of the tile in V buffer vbuf."""
    ks, db = divmod(j, 4)
    base = V_VF + 4 * (j % 4)
    off = vbuf * TILE_BYTES + ks * 4096
    A.lds(f"ds_read_b64_tr_b16 {vr(base, 2)}, %[va{db}] offset:{off}")
    return A.lds(f"ds_read_b64_tr_b16 {vr(base + 2, 2)}, %[va{db}] offset:{off + 2048}")


# VALU issue cost in units of ~2.4 cycles: a wave64 v_exp_f32 ~12 cycles (5 units), other VALU
# ~4.6 cycles (2 units), measured on the device with MFMA chains; one 32x32x16 MFMA lasts ~32
# cycles (~13 units), the VALU budget of a slot.
SLOT_BUDGET_A, SLOT_BUDGET_B = 13, 13


def units(op):
    if op.startswith("s_"):
        return 0
    return 5 if op.startswith("v_exp") else 2


def pack(stream, fixed, budget, nslots=32):
    """List-schedules a stream of VALU groups into the MFMA slots, after each slot's fixed ops.
    Slot by slot, the ready group with the earliest deadline (then the earliest in the stream)
    that fits in `budget` is placed; a group at its deadline is placed even over budget.  A group
    is ready when the group it depends on sits at least one slot earlier (a transcendental result
    read by VALU; a VALU result read by MFMA is covered by deadlines two slots early), and, for
    groups marked ordered, when the previous ordered group is placed (the row sums keep their
    accumulation order).
    stream: list of (ops, deadline, dep, ordered) with dep the index of an earlier group, a 1-tuple
    holding a slot fixed earlier, or None.  Returns the slots and the slot of each group."""
    out = [list(f) for f in fixed]
    load = [sum(units(o) for o in f) for f in fixed]
    n = len(stream)
    slot_of = [None] * n
    ordered = [i for i in range(n) if stream[i][3]]
    prev_ord = {ordered[k]: ordered[k - 1] for k in range(1, len(ordered))}
    for sl in range(nslots):
        while True:
            best = None
            for i, (ops, deadline, dep, _) in enumerate(stream):
                if slot_of[i] is not None:
                    continue
                if isinstance(dep, int) and (slot_of[dep] is None or slot_of[dep] + 1 > sl):
                    continue
                if isinstance(dep, tuple) and dep[0] + 1 > sl:
                    continue
                if i in prev_ord and slot_of[prev_ord[i]] is None:
                    continue
                cost = sum(units(o) for o in ops)
                if load[sl] + cost > budget and deadline > sl:
                    continue
                if best is None or (deadline, i) < (stream[best][1], best):
                    best = i
            if best is None:
                break
            slot_of[best] = sl
            out[sl] += stream[best][0]
            load[sl] += sum(units(o) for o in stream[best][0])
    for i, (ops, deadline, dep, _) in enumerate(stream):
        assert slot_of[i] is not None and slot_of[i] <= deadline, (ops, slot_of[i], deadline)
    # emit each slot's groups in stream order (a group never precedes one it depends on)
    for sl in range(nslots):
        mine = sorted((i for i in range(n) if slot_of[i] == sl))
        out[sl] = list(fixed[sl]) + [o for i in mine for o in stream[i][0]]
    return out, slot_of


def block(A, cur, nxt, has_next, masked, kbuf, vbuf, extra_a=(), extra_b=()):
    """One tile t.  kbuf: K buffer of tile t+1; vbuf: V buffer of tile t.  With has_next, K
    fragments 0..2 of tile t+1 are in flight at entry.
    extra_a / extra_b: groups of scalar-unit work (tile copies, buffer rotation) issued after the
    MFMA of slot i of phase A / B, so they run in the shadow of the matrix core."""
    A.n_ops = 0
    k_ops, v_ops = {}, {}
    if has_next:
        for i in range(3):
            k_ops[i] = i
        A.n_ops = 3
    else:
        A.e("s_waitcnt lgkmcnt(0)")
    if masked:
        A.e(f"v_mov_b32 {vr(V_NEGINF)}, 0xff800000")
        for qb in range(2):  # hide in-tile key c (without its 4hi part) when c >= base2 - key0
            A.e(f"v_subrev_u32_e32 {vr(V_T0[qb])}, {sr(S_KEY)}, %[base2_{qb}]")

    # softmax pairs of S(t), in the order the value product consumes P: pair s -> (ks, qb, m)
    pairs = []
    for ks in range(4):
        kb, h = divmod(ks, 2)
        for qb in range(2):
            for m in range(4):
                a = s_reg(cur, qb, kb, 8 * h + 2 * m)
                pairs.append((qb, ks, m, a, a + 1))

    def cvt(p):
        qb, ks, m, a, b = pairs[p]
        return f"v_cvt_pk_bf16_f32 {vr(V_P + 16 * qb + 4 * ks + m)}, {vr(a)}, {vr(b)}"

    def softmax(p):
        qb, ks, m, a, b = pairs[p]
        return ([f"v_fma_f32 {vr(a)}, {vr(a)}, %[c], %[nmc{qb}]",
                 f"v_fma_f32 {vr(b)}, {vr(b)}, %[c], %[nmc{qb}]"],
                [f"v_exp_f32_e32 {vr(a)}, {vr(a)}"], [f"v_exp_f32_e32 {vr(b)}, {vr(b)}"])

    def deadline_p(p):
        """Last slot of phase B for the packing of pair p: two MFMAs before the value-product
        slot 8ks + qb that reads it."""
        qb, ks = pairs[p][0], pairs[p][1]
        return 8 * ks + qb - 2

    # Unmasked tiles split the softmax of S(t) between the phases so that both carry about the
    # same VALU load: p = 2^(s*c + neg_mc) for pairs 0..N_A-1 and the bf16 packing of step
    # ks = 0 in phase A; the remaining pairs, the other packings and the row sums in phase B.
    # Masked tiles (the mask adds VALU work to phase B) keep the whole softmax in phase A.
    balanced = has_next and not masked
    N_A = 24 if balanced else 32
    slots_a = []
    if balanced:
        stream, exp_b = [], {}
        for p in range(N_A):
            f, ea, eb = softmax(p)
            stream += [(f[:1], 31, None, False), (ea, 31, None, False), (f[1:], 31, None, False),
                       (eb, 31, None, False)]
            exp_b[p] = len(stream) - 1
            if 1 <= p <= 8:       # the packing of the previous pair (read from phase-B slot 0 on)
                stream.append(([cvt(p - 1)], 29, exp_b[p - 1], False))
        slots_a, _ = pack(stream, [[] for _ in range(32)], SLOT_BUDGET_A)
    else:
        for p, (qb, ks, m, a, b) in enumerate(pairs):
            ops = [f"v_fma_f32 {vr(a)}, {vr(a)}, %[c], %[nmc{qb}]",
                   f"v_fma_f32 {vr(b)}, {vr(b)}, %[c], %[nmc{qb}]",
                   f"v_exp_f32_e32 {vr(a)}, {vr(a)}",
                   f"v_exp_f32_e32 {vr(b)}, {vr(b)}"]
            if p > 0:
                ops.append(cvt(p - 1))  # the previous pair: its exp results are a slot old
            slots_a.append(ops)

    # ---- phase A ----
    if has_next:
        for s in range(32):
            i, qb = divmod(s, 2)
            kb, tt = divmod(i, 8)
            if qb == 0:
                if i + 3 < 16:
                    k_ops[i + 3] = issue_k(A, i + 3, kbuf)
                else:
                    jv = i + 3 - 16
                    v_ops[jv] = issue_v(A, jv, vbuf)
                A.wait_for(k_ops[i])
            dst = s_reg(nxt, qb, kb)
            src2 = "0" if tt == 0 else vr(dst, 16)
            A.e(f"v_mfma_f32_32x32x16_bf16 {vr(dst, 16)}, {vr(V_KF + 4 * (i % 4), 4)}, "
                f"{ar(A_Q + 32 * qb + 4 * tt, 4)}, {src2}")
            for op in slots_a[s]:
                A.e(op)
            for op in (extra_a[s] if s < len(extra_a) else []):
                A.e(op)
    else:
        for jv in range(3):
            v_ops[jv] = issue_v(A, jv, vbuf)
        for s in range(32):
            for op in slots_a[s]:
                A.e(op)

    # ---- phase B ----
    slots_b = [[] for _ in range(32)]
    if not balanced:
        for p, (qb, ks, m, a, b) in enumerate(pairs):  # row sums of S(t) (fp32 probabilities)
            slots_b[p] += [f"v_add_f32_e32 {vr(V_RS[qb])}, {vr(V_RS[qb])}, {vr(a)}",
                           f"v_add_f32_e32 {vr(V_RS[qb])}, {vr(V_RS[qb])}, {vr(b)}"]
    if has_next:  # mask and row max of S(t+1): (qb, kb) blocks in the order their MFMAs finished,
        # in slots 0..23, so that the row-max exchange and the rescale test fit in slots 24..29
        order = [(0, 0), (1, 0), (0, 1), (1, 1)]
        first = {0: True, 1: True}
        for bi, (qb, kb) in enumerate(order):
            for r2 in range(8):
                s = bi * 6 + (r2 * 6) // 8
                ea = s_reg(nxt, qb, kb, 2 * r2)
                eb = ea + 1
                if masked:
                    for r, e_ in ((2 * r2, ea), (2 * r2 + 1, eb)):
                        cconst = kb * 32 + (r >> 2) * 8 + (r & 3)
                        slots_b[s].append(f"v_cmp_ge_i32_e32 vcc, {cconst}, {vr(V_T0[qb])}")
                        slots_b[s].append(f"v_cndmask_b32_e32 {vr(e_)}, {vr(e_)}, {vr(V_NEGINF)}, vcc")
                if first[qb]:
                    slots_b[s].append(f"v_max_f32_e32 {vr(V_MX[qb])}, {vr(ea)}, {vr(eb)}")
                    first[qb] = False
                else:
                    slots_b[s].append(f"v_max3_f32 {vr(V_MX[qb])}, {vr(V_MX[qb])}, {vr(ea)}, {vr(eb)}")
        # Row max across the half-waves, then the rescale test (tile max above m_run + thr for any
        # row of either block) into SCC; each step one slot after the one it reads, which covers
        # the VALU -> permlane, permlane -> VALU and VALU-written SGPR -> SALU wait states.
        # V_T0 (the mask bounds) is free after slot 23.
        for qb in range(2):
            slots_b[24].append(f"v_mov_b32 {vr(V_AL[qb])}, {vr(V_MX[qb])}")
            slots_b[25].append(f"v_permlane32_swap_b32_e32 {vr(V_AL[qb])}, {vr(V_MX[qb])}")
            slots_b[26].append(f"v_max_f32_e32 {vr(V_MX[qb])}, {vr(V_AL[qb])}, {vr(V_MX[qb])}")
            slots_b[27].append(f"v_add_f32_e32 {vr(V_T0[qb])}, %[thr], %[mrun{qb}]")
            slots_b[28].append(f"v_cmp_gt_f32_e64 {sr(S_C[qb], 2)}, {vr(V_MX[qb])}, {vr(V_T0[qb])}")
        slots_b[29].append(f"s_or_b64 {sr(S_C[0], 2)}, {sr(S_C[0], 2)}, {sr(S_C[1], 2)}")  # SCC: any row

    if balanced:
        # Flexible phase-B work, packed in order: the packings of P still missing (each at least
        # two MFMAs before the value-product slot that reads it), the remaining softmax pairs and
        # their packings, and the fp32 row sums in pair order (so the sums of each row block are
        # those of the narrow kernel bit for bit).
        stream, exp_b = [], {}
        for dl in sorted({deadline_p(p) for p in range(8, 32)}):
            group = [p for p in range(8, 32) if deadline_p(p) == dl]
            for p in group:
                if p >= N_A:
                    f, ea, eb = softmax(p)
                    stream += [(f[:1], dl - 1, None, False), (ea, dl - 1, None, False),
                               (f[1:], dl - 1, None, False), (eb, dl - 1, None, False)]
                    exp_b[p] = len(stream) - 1
            for p in group:
                stream.append(([cvt(p)], dl, exp_b.get(p), False))
        # and the row sums, in pair order per row block (after the exps they read)
        for p, (qb, ks, m, a, b) in enumerate(pairs):
            stream.append(([f"v_add_f32_e32 {vr(V_RS[qb])}, {vr(V_RS[qb])}, {vr(a)}",
                            f"v_add_f32_e32 {vr(V_RS[qb])}, {vr(V_RS[qb])}, {vr(b)}"], 31, exp_b.get(p), True))
        slots_b, _ = pack(stream, slots_b, SLOT_BUDGET_B)

    A.e(f"v_mov_b32 {vr(V_RS[0])}, 0")
    A.e(f"v_mov_b32 {vr(V_RS[1])}, 0")
    for s in range(32):
        j, qb = divmod(s, 2)
        ks, db = divmod(j, 4)
        if qb == 0:
            if j + 3 < 16:
                v_ops[j + 3] = issue_v(A, j + 3, vbuf)
            A.wait_for(v_ops[j])
        A.e(f"v_mfma_f32_32x32x16_bf16 {ar(A_O + 64 * qb + 16 * db, 16)}, {vr(V_VF + 4 * (j % 4), 4)}, "
            f"{vr(V_P + 16 * qb + 4 * ks, 4)}, {ar(A_O + 64 * qb + 16 * db, 16)}")
        if s == 0 and not balanced:
            A.e(cvt(31))  # last pair of P (read by the MFMAs of step ks = 3)
        for op in slots_b[s]:
            A.e(op)
        for op in (extra_b[s] if s < len(extra_b) else []):
            A.e(op)

    for qb in range(2):
        A.e(f"v_add_f32_e32 %[lrun{qb}], %[lrun{qb}], {vr(V_RS[qb])}")


def rescale_rows(A, p):
    """Out-of-line path, taken after phase B when the test of slot 29 found a row whose tile max
    exceeds its running max by more than thr (rare): rescale the affected row blocks."""
    # O^T, written by the value product just before, is read by VALU below: >= 24 wait states
    A.e("s_nop 7")
    A.e("s_nop 7")
    A.e("s_nop 7")
    rescale(A, 0, f"Lnor0_{p}")
    rescale(A, 1, f"Lnor1_{p}")


def rescale(A, qb, lbl):
    """Lazy running-max update of row block qb (V_T0 holds m_run + thr), with its neg_mc."""
    t0, al, mx = V_T0[qb], V_AL[qb], V_MX[qb]
    A.e(f"v_cmp_gt_f32_e32 vcc, {vr(mx)}, {vr(t0)}")
    A.e("s_nop 4")                                                        # VALU vcc -> vccz branch
    A.e(f"s_cbranch_vccz {lbl}")
    A.e(f"v_cndmask_b32_e32 {vr(t0)}, %[mrun{qb}], {vr(mx)}, vcc")     # m_new
    A.e(f"v_sub_f32_e32 {vr(al)}, %[mrun{qb}], {vr(t0)}")
    A.e(f"v_mul_f32_e32 {vr(al)}, %[c], {vr(al)}")
    A.e(f"v_exp_f32_e32 {vr(al)}, {vr(al)}")
    A.e("s_nop 0")                                                        # transcendental -> VALU
    A.e(f"v_cndmask_b32_e64 {vr(al)}, 1.0, {vr(al)}, vcc")             # rows that keep their max: 1
    A.e(f"v_mov_b32 %[mrun{qb}], {vr(t0)}")
    A.e(f"v_mul_f32_e32 %[lrun{qb}], %[lrun{qb}], {vr(al)}")
    base = A_O + 64 * qb
    for g in range(0, 64, N_TMP):
        for j in range(N_TMP):
            A.e(f"v_accvgpr_read_b32 {vr(TMP_BASE + j)}, {ar(base + g + j)}")
        for j in range(N_TMP):
            A.e(f"v_mul_f32_e32 {vr(TMP_BASE + j)}, {vr(TMP_BASE + j)}, {vr(al)}")
        for j in range(N_TMP):
            A.e(f"v_accvgpr_write_b32 {ar(base + g + j)}, {vr(TMP_BASE + j)}")
    A.e(f"v_mul_f32_e64 %[nmc{qb}], -%[mrun{qb}], %[c]")              # neg_mc follows m_run
    A.e(f"v_cmp_eq_f32_e32 vcc, 0xff800000, %[mrun{qb}]")
    A.e(f"v_cndmask_b32_e64 %[nmc{qb}], %[nmc{qb}], 0, vcc")
    A.e("s_nop 1")
    A.e(f"{lbl}:")


class Lines:
    """Collects instruction lines (to be placed into MFMA slots later)."""
    def __init__(self):
        self.lines = []

    def e(self, s):
        self.lines.append(s)


def dma_groups(which, ahead, buf):
    """Copy of tile t + ahead of K or V into LDS buffer `buf`, without branches:
    past the last tile the copy has 0 valid rows (no memory is read; the buffer it fills is not
    read again).  Returned as groups of instructions, each group placed after one MFMA; every
    SCC producer sits next to its consumer inside a group."""
    ptr, rsrc, offs, dst = (S_KP, S_KR, "koff", "kdst") if which == "k" else (S_VP, S_VR, "voff", "vdst")
    g = []
    g.append([f"s_add_u32 {sr(S_TMP)}, {sr(S_T)}, {ahead}",
              f"s_lshl_b32 {sr(S_ROWS)}, {sr(S_TMP)}, 6",          # rows = min(64, kv_lim - 64 (t + ahead))
              f"s_sub_i32 {sr(S_ROWS)}, %[kvlim], {sr(S_ROWS)}",
              f"s_min_i32 {sr(S_ROWS)}, {sr(S_ROWS)}, 64",
              f"s_max_i32 {sr(S_ROWS)}, {sr(S_ROWS)}, 0",
              f"s_cmp_lt_u32 {sr(S_TMP)}, %[nkt]",                  # no such tile: 0 rows
              f"s_cselect_b32 {sr(S_ROWS)}, {sr(S_ROWS)}, 0"])
    g.append([f"s_mul_i32 {sr(rsrc + 2)}, {sr(S_ROWS)}, %[rowb]",
              f"s_mov_b32 {sr(rsrc)}, {sr(ptr)}",
              f"s_and_b32 {sr(rsrc + 1)}, {sr(ptr + 1)}, 0xffff",
              f"s_mov_b32 {sr(rsrc + 3)}, 0x20000"])
    g[-1].append(f"s_add_u32 {sr(S_TMP)}, %[{dst}0], {buf * TILE_BYTES}")
    for u in range(4):
        c = [f"s_mov_b32 m0, {sr(S_TMP)}", "s_nop 0", f"buffer_load_dwordx4 %[{offs}{u}], {sr(rsrc, 4)}, 0 offen lds"]
        if u < 3:
            c.append(f"s_add_u32 {sr(S_TMP)}, {sr(S_TMP)}, 1024")
        g.append(c)
    g.append([f"s_add_u32 {sr(ptr)}, {sr(ptr)}, %[tstride_lo]",
              f"s_addc_u32 {sr(ptr + 1)}, {sr(ptr + 1)}, %[tstride_hi]"])
    return g


KA = [f"ka{t}" for t in range(8)]
VA = [f"va{d}" for d in range(4)]


def half(A, u, uid, cold):
    """Tile t with t mod 4 == u (when t + 1 < nkt; else the last block).  The common path (an
    unmasked tile that moves no running max) runs straight through; the masked block and the
    rescale go to `cold`, emitted after the loop, and branch back."""
    cur, nxt = (V_SA, V_SB) if u % 2 == 0 else (V_SB, V_SA)
    p = f"{u}_{uid}"
    # Scalar work of the tile, spread over the MFMA slots of phase A: K(t+3) -> K buffer (t+3) mod 4
    # (held K(t-1), consumed two barriers ago), V(t+1) -> V buffer (t+1) mod 2 (held V(t-1),
    # consumed before the last barrier)
    extra_a = dma_groups("k", 3, (u + 3) % NKBUF) + dma_groups("v", 1, (u + 1) % NVBUF)
    A.e(f"s_add_u32 {sr(S_T1)}, {sr(S_T)}, 1")
    A.e(f"s_cmp_lt_u32 {sr(S_T1)}, %[nkt]")
    A.e(f"s_cbranch_scc0 Llast{p}")
    A.e(f"s_lshl_b32 {sr(S_KEY)}, {sr(S_T1)}, 6")
    A.e(f"s_cmp_ge_u32 {sr(S_T1)}, %[tmask]")
    A.e(f"s_cbranch_scc1 Lmask{p}")
    block(A, cur, nxt, True, False, (u + 1) % NKBUF, u % NVBUF, extra_a)
    A.e(f"Lpost{p}:")
    A.e(f"s_cbranch_scc1 Lresc{p}")       # SCC from the rescale test: some row's max moved
    A.e(f"Lback{p}:")
    cold.e(f"Lmask{p}:")
    block(cold, cur, nxt, True, True, (u + 1) % NKBUF, u % NVBUF, extra_a)
    cold.e(f"s_branch Lpost{p}")
    cold.e(f"Lresc{p}:")
    rescale_rows(cold, p)
    cold.e(f"s_branch Lback{p}")
    A.e(f"s_add_u32 {sr(S_TMP)}, {sr(S_T)}, 2")
    A.e(f"s_cmp_lt_u32 {sr(S_TMP)}, %[nkt]")
    A.e(f"s_cbranch_scc0 Lnopre{p}")
    for i in range(3):                    # first K fragments of the next block (K(t+2) is visible)
        issue_k(A, i, (u + 2) % NKBUF)
    A.e(f"Lnopre{p}:")
    A.e("s_waitcnt vmcnt(0)")
    A.e("s_barrier")
    A.e(f"s_add_u32 {sr(S_T)}, {sr(S_T)}, 1")


def last(A, u, uid):
    cur, nxt = (V_SA, V_SB) if u % 2 == 0 else (V_SB, V_SA)
    A.e(f"Llast{u}_{uid}:")
    block(A, cur, nxt, False, False, (u + 1) % NKBUF, u % NVBUF)
    A.e(f"s_branch Lend_{uid}")


def gen_loop():
    A = Asm()
    uid = "%="
    A.e(f"s_mov_b32 {sr(S_T)}, 0")
    A.e(f"s_mov_b32 {sr(S_KP)}, %[kp_lo]")
    A.e(f"s_mov_b32 {sr(S_KP + 1)}, %[kp_hi]")
    A.e(f"s_mov_b32 {sr(S_VP)}, %[vp_lo]")
    A.e(f"s_mov_b32 {sr(S_VP + 1)}, %[vp_hi]")
    A.e(f"s_cmp_lt_u32 {sr(S_T)}, %[nkt]")
    A.e(f"s_cbranch_scc0 Lend_{uid}")
    A.e("s_cmp_lt_u32 1, %[nkt]")
    A.e(f"s_cbranch_scc0 Ltop_{uid}")
    for i in range(3):                    # first K fragments of tile 1 (K buffer 1)
        issue_k(A, i, 1)
    A.e(f"Ltop_{uid}:")
    cold = Asm()
    for u in range(NKBUF):
        half(A, u, uid, cold)
    A.e(f"s_branch Ltop_{uid}")
    A.lines += cold.lines
    for u in range(NKBUF):
        last(A, u, uid)
    A.e(f"Lend_{uid}:")
    # the code after the statement reads O^T, written by the last value-product MFMAs: >= 24 wait
    # states (the compiler does not see the MFMAs inside the statement)
    A.e("s_nop 7")
    A.e("s_nop 7")
    A.e("s_nop 7")
    return A.lines


VCLOB = list(range(V_P, 128)) + list(range(V_TMP, 64))
SCLOB = list(range(80, 100))


def main(out):
    lines = gen_loop()
    clob = ", ".join('"%s"' % c for c in [f"v{i}" for i in VCLOB] + [f"s{i}" for i in SCLOB]
                     + ["vcc", "scc", "m0", "memory"])
    body = "".join('      "%s\\n\\t" \\\n' % l for l in lines)
    txt = ("// Generated by gen_attn_loop_wide.py (do not edit): main loop of the wide bf16 attention kernel.\n"
           "#define THA_ATTN_WIDE_LOOP_ASM \\\n" + body + "\n"
           "#define THA_ATTN_WIDE_LOOP_CLOBBERS " + clob + "\n")
    open(out, "w").write(txt)


# Registers the loop writes besides its own read-write operands (pinned sets and clobbers).
WRITTEN = {"v": set(VCLOB) | set(range(V_SA, 256)), "s": set(SCLOB), "a": set(range(A_O, A_O + 128))}
READ_WRITE_OPERANDS = tuple([f"mrun{q}" for q in range(2)] + [f"lrun{q}" for q in range(2)]
                            + [f"nmc{q}" for q in range(2)])


def _regs(tok):
    m = re.fullmatch(r"-?([vsa])(\d+)", tok) or re.fullmatch(r"-?([vsa])\[(\d+):(\d+)\]", tok)
    if not m:
        return None
    lo = int(m.group(2))
    hi = int(m.group(3)) if m.lastindex == 3 else lo
    return m.group(1), set(range(lo, hi + 1))


def check_operand_allocation(compiled_asm: str) -> dict:
    """Matches each instance of the loop in compiler output against the template and checks that
    every named operand got one register, that no read-write operand shares a register with
    another operand, and that no operand lies in a register the loop writes.  Returns
    {operand: register} of the last instance; raises AssertionError on a violation."""
    tpl = gen_loop()
    blocks = re.findall(r";;#ASMSTART\n(.*?);;#ASMEND", compiled_asm, flags=re.S)
    loops = [b for b in blocks if b.strip().splitlines()[0].strip() == tpl[0]
             and sum(1 for l in b.strip().splitlines() if l.strip()) == len(tpl)]
    assert loops, "loop statement not found in the compiled assembly"
    result = {}
    for body in loops:
        got = [l.strip() for l in body.strip().splitlines() if l.strip()]
        assert len(got) == len(tpl), (len(got), len(tpl))
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
                continue
            kind, regs = r
            assert not (regs & WRITTEN[kind]), f"operand {k} = {v} lies in a register the loop writes"
            for x in regs:
                other = owner.setdefault((kind, x), k)
                if other != k and (k in READ_WRITE_OPERANDS or other in READ_WRITE_OPERANDS):
                    raise AssertionError(f"read-write operand shares {kind}{x}: {k}, {other}")
        result = names
    return result


if __name__ == "__main__":
    main(sys.argv[1] if len(sys.argv) > 1 else os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                            "attn_loop_d128_wide.inc"))

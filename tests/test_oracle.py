"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test names what fixes the expected result: a hand-derived example, a
closed form, an invariant the pages state, a brute-force route, or a library
routine (torch's fp64 matmul/softmax and scaled_dot_product_attention).
"""
import json
import math
import os

import pytest
import torch
import torch.nn.functional as F

import oracle
import tha_workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f(x):
    return float("-inf") if x == "-inf" else float(x)


def _t(vals, shape, dtype=torch.float32):
    return torch.tensor([_f(v) for v in vals], dtype=torch.float64).to(dtype).reshape(shape)


# ---------------------------------------------------------------- golden ---

@pytest.mark.parametrize("case", json.load(open(os.path.join(GOLDEN, "hand_examples.json")))["attention"],
                         ids=lambda c: c["name"])
def test_hand_examples_attention(case):
    B, Sq, Sk, H, D = case["B"], case["Sq"], case["Sk"], case["H"], case["D"]
    q = _t(case["q"], (B, Sq, H, D))
    k = _t(case["k"], (B, Sk, H, D))
    v = _t(case["v"], (B, Sk, H, D))
    kv = torch.tensor(case["kv_len"], dtype=torch.int32) if case["kv_len"] is not None else None
    out, lse = oracle.attention(q, k, v, causal=case["causal"], q_pos0=case["q_pos0"], k_pos0=case["k_pos0"],
                                kv_len=kv, scale=case["scale"])
    exp_out = _t(case["out"], (B, Sq, H, D), torch.float64)
    exp_lse = _t(case["lse_bhs"], (B, H, Sq), torch.float64)
    assert torch.allclose(out, exp_out, atol=1e-12, rtol=0)
    assert torch.equal(torch.isinf(lse), torch.isinf(exp_lse))
    fin = torch.isfinite(exp_lse)
    assert torch.allclose(lse[fin], exp_lse[fin], atol=1e-12, rtol=0)


def test_hand_example_merge():
    c = json.load(open(os.path.join(GOLDEN, "hand_examples.json")))["merge"]
    shp = (c["B"], c["S"], c["H"], c["D"])
    o_parts = [_t(p, shp, torch.float64) for p in c["o_parts"]]
    l_parts = [_t(p, (c["B"], c["H"], c["S"]), torch.float64) for p in c["lse_parts"]]
    out, lse = oracle.merge_lse(o_parts, l_parts)
    assert torch.allclose(out, _t(c["out"], shp, torch.float64), atol=1e-12, rtol=0)
    exp_lse = _t(c["lse"], (c["B"], c["H"], c["S"]), torch.float64)
    assert torch.equal(torch.isinf(lse), torch.isinf(exp_lse))
    fin = torch.isfinite(exp_lse)
    assert torch.allclose(lse[fin], exp_lse[fin], atol=1e-12, rtol=0)


def test_hand_example_permute():
    c = json.load(open(os.path.join(GOLDEN, "hand_examples.json")))["permute"]
    P, B, S, H, D = c["P"], c["B"], c["S"], c["H"], c["D"]
    shards = [torch.tensor(s, dtype=torch.int16).reshape(B, S // P, H, D) for s in c["shards"]]
    for g in range(P):
        out = oracle.shard_permute(shards, g)
        assert out.tolist() == torch.tensor(c["groups"][g], dtype=torch.int16).reshape(B, S, H // P, D).tolist()


def test_page_check_q_split_fp32():
    """'adv07: Sequence Parallel' section 6, check 1: [16, 32], 2 splits, fp32, max-abs < 1e-5.

    The pages print no values, so the pin is the shape, the split rule and the tolerance:
    chunks of ceil(16/2) query rows attend to the full K/V and are concatenated.
    """
    c = json.load(open(os.path.join(GOLDEN, "page_checks.json")))["q_split_equivalence"]
    S, D = c["shape"]
    g = W.generator(11)
    q, k, v = (W.randn((1, S, 1, D), g, torch.float32) for _ in range(3))
    full, _ = oracle.attention(q, k, v)
    chunk = (S + c["seq_splits"] - 1) // c["seq_splits"]
    parts = []
    for s in range(c["seq_splits"]):
        lo, hi = s * chunk, min((s + 1) * chunk, S)
        o, _ = oracle.attention(q[:, lo:hi], k, v)
        parts.append(o)
    split = torch.cat(parts, dim=1)
    assert (split - full).abs().max().item() < c["max_abs_tolerance"]
    # rows depend on their own query only: the fp64 results agree bit for bit
    assert torch.equal(split, full)
    # the same check through torch's fp32 library attention on the page's shape
    ref = F.scaled_dot_product_attention(q.permute(0, 2, 1, 3), k.permute(0, 2, 1, 3), v.permute(0, 2, 1, 3))
    assert (ref.permute(0, 2, 1, 3).double() - full).abs().max().item() < c["max_abs_tolerance"]


def test_page_check_q_split_bug_differs():
    """The plan's bug (each Q chunk sees only its own K/V) must NOT equal attention."""
    g = W.generator(12)
    q, k, v = (W.randn((1, 16, 1, 32), g, torch.float32) for _ in range(3))
    full, _ = oracle.attention(q, k, v)
    bug = torch.cat([oracle.attention(q[:, lo:lo + 8], k[:, lo:lo + 8], v[:, lo:lo + 8])[0] for lo in (0, 8)], 1)
    assert (bug - full).abs().max().item() > 1e-3


# ------------------------------------------------- independent routes ---

SHAPES = [
    # B, Sq, Sk, H, D, causal, q_pos0, k_pos0, with_len
    (1, 7, 7, 1, 3, False, 0, 0, False),
    (2, 9, 9, 3, 4, True, 0, 0, False),
    (1, 5, 11, 2, 8, True, 6, 0, False),
    (2, 6, 10, 2, 5, False, 0, 0, True),
    (3, 8, 8, 2, 4, True, 0, 0, True),
    (1, 4, 6, 1, 2, True, 0, 3, False),   # early rows see nothing
]


def _inputs(B, Sq, Sk, H, D, with_len, seed, dtype=torch.float32):
    g = W.generator(seed)
    kv = torch.randint(0, Sk + 1, (B,), generator=g).to(torch.int32) if with_len else None
    q = W.randn((B, Sq, H, D), g, dtype)
    k = W.randn((B, Sk, H, D), g, dtype)
    v = W.randn((B, Sk, H, D), g, dtype)
    return q, k, v, kv


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_two_pass_matches_bruteforce(shape, dtype):
    B, Sq, Sk, H, D, causal, qp, kp, wl = shape
    q, k, v, kv = _inputs(B, Sq, Sk, H, D, wl, 3, dtype)
    o1, l1 = oracle.attention(q, k, v, causal=causal, q_pos0=qp, k_pos0=kp, kv_len=kv)
    o2, l2, P = oracle.attention_bruteforce(q, k, v, causal=causal, q_pos0=qp, k_pos0=kp, kv_len=kv)
    assert (o1 - o2).abs().max().item() <= 1e-12
    assert torch.equal(torch.isinf(l1), torch.isinf(l2))
    fin = torch.isfinite(l1)
    assert (l1[fin] - l2[fin]).abs().max().item() <= 1e-12 if fin.any() else True
    # softmax rows sum to 1 (rows with no visible key are all zero)
    rs = P.sum(-1)
    nonempty = torch.isfinite(l2)
    assert torch.allclose(rs[nonempty], torch.ones_like(rs[nonempty]), atol=1e-12, rtol=0)
    assert torch.all(rs[~nonempty] == 0)


def _vis_mask(B, Sq, Sk, causal, qp, kp, kv):
    i = torch.arange(Sq).view(Sq, 1) + qp
    j = torch.arange(Sk).view(1, Sk) + kp
    m = torch.ones(B, 1, Sq, Sk, dtype=torch.bool)
    if causal:
        m = m & (j <= i)
    if kv is not None:
        m = m & (torch.arange(Sk).view(1, 1, 1, Sk) < kv.view(B, 1, 1, 1).clamp(0, Sk))
    return m


@pytest.mark.parametrize("shape", [s for s in SHAPES if s != SHAPES[-1]] + [(2, 33, 47, 4, 16, True, 14, 0, True)])
def test_matches_torch_fp64_library_routes(shape):
    """Library routes: the forward of 'parallel multi-head attention' section 3.2
    (matmul, additive mask, softmax over keys, matmul) in torch fp64, and torch's
    scaled_dot_product_attention in fp64.  Rows with no visible key are excluded
    (torch gives NaN there; the oracle's reading gives 0)."""
    B, Sq, Sk, H, D, causal, qp, kp, wl = shape
    q, k, v, kv = _inputs(B, Sq, Sk, H, D, wl, 5)
    out, lse = oracle.attention(q, k, v, causal=causal, q_pos0=qp, k_pos0=kp, kv_len=kv)
    vis = _vis_mask(B, Sq, Sk, causal, qp, kp, kv)
    qt, kt, vt = (x.double().permute(0, 2, 1, 3) for x in (q, k, v))
    add = torch.zeros(vis.shape, dtype=torch.float64).masked_fill(~vis, float("-inf"))
    scores = torch.matmul(qt, kt.transpose(2, 3)) / math.sqrt(D) + add
    ref = torch.matmul(F.softmax(scores, dim=-1), vt).permute(0, 2, 1, 3)
    ref_lse = torch.logsumexp(scores, dim=-1)
    sdpa = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=vis).permute(0, 2, 1, 3)
    rows_ok = vis.any(-1).permute(0, 2, 1).expand(B, Sq, H)  # [B, Sq, H]
    assert (out[rows_ok] - ref[rows_ok]).abs().max().item() <= 1e-12
    assert (out[rows_ok] - sdpa[rows_ok]).abs().max().item() <= 1e-12
    lse_ok = rows_ok.permute(0, 2, 1)
    assert (lse[lse_ok] - ref_lse.expand(B, H, Sq)[lse_ok]).abs().max().item() <= 1e-12


# ------------------------------------------------------- closed forms ---

def test_causal_row0_is_v0():
    q, k, v, _ = _inputs(2, 12, 12, 3, 16, False, 7)
    out, lse = oracle.attention(q, k, v, causal=True)
    assert torch.equal(out[:, 0], v[:, 0].double())
    s00 = (q[:, 0].double() * k[:, 0].double()).sum(-1) / 4.0  # [B, H]; scale 1/sqrt(16)
    assert torch.allclose(lse[:, :, 0], s00, atol=1e-12, rtol=0)


def test_single_visible_key():
    q, k, v, _ = _inputs(3, 10, 10, 2, 8, False, 8)
    kv = torch.ones(3, dtype=torch.int32)
    out, lse = oracle.attention(q, k, v, kv_len=kv)
    assert torch.equal(out, v[:, :1].double().expand_as(out))
    s = torch.einsum("bihd,bhd->bhi", q.double(), k[:, 0].double()) / math.sqrt(8)
    assert torch.allclose(lse, s, atol=1e-12, rtol=0)


def test_zero_query_gives_prefix_mean_and_log_count():
    _, k, v, _ = _inputs(1, 20, 20, 2, 6, False, 9)
    q = torch.zeros(1, 20, 2, 6)
    out, lse = oracle.attention(q, k, v, causal=True)
    cm = v.double().cumsum(1) / torch.arange(1, 21, dtype=torch.float64).view(1, 20, 1, 1)
    assert torch.allclose(out, cm, atol=1e-12, rtol=0)
    assert torch.allclose(lse, torch.log(torch.arange(1, 21, dtype=torch.float64)).view(1, 1, 20).expand(1, 2, 20),
                          atol=1e-12, rtol=0)


def test_constant_values_give_constant_output():
    q, k, _, _ = _inputs(2, 9, 13, 2, 4, False, 10)
    v = torch.full((2, 13, 2, 4), 0.75)
    out, _ = oracle.attention(q, k, v, causal=True, q_pos0=4)
    assert torch.allclose(out, torch.full_like(out, 0.75), atol=1e-14, rtol=0)


def test_key_shift_invariance():
    """Adding u to every key adds q.u*scale to every score of a row: out unchanged, lse shifted."""
    q, k, v, _ = _inputs(1, 10, 10, 2, 8, False, 11, torch.bfloat16)
    q, k, v = q.float(), k.float(), v.float()
    u = torch.tensor([0.5, -0.25, 1.0, 0.0, -0.5, 0.125, 2.0, -1.0]).view(1, 1, 1, 8).expand(1, 1, 2, 8)
    k2 = k + u
    assert torch.equal(k2.double() - u.double(), k.double())  # the shift is exact in fp32
    out1, lse1 = oracle.attention(q, k, v, causal=True)
    out2, lse2 = oracle.attention(q, k2, v, causal=True)
    assert torch.allclose(out1, out2, atol=1e-12, rtol=0)
    shift = (q.double() * u.double()).sum(-1).permute(0, 2, 1) / math.sqrt(8)
    assert torch.allclose(lse2 - lse1, shift, atol=1e-12, rtol=0)


# ------------------------------------------------ page invariants ---

def test_head_split_concat_equals_full():
    """Workload 1 (fp32, B1 S64 H2 D8, causal): per-head runs concatenated == all heads,
    bit-identical; heads are never split ('parallel multi-head attention' 2.2, 3.1)."""
    inp, p = W.workload_inputs(1)
    q, k, v = inp["q"], inp["k"], inp["v"]
    full, lfull = oracle.attention(q, k, v, causal=True)
    per = [oracle.attention(q[:, :, h:h + 1].contiguous(), k[:, :, h:h + 1].contiguous(),
                            v[:, :, h:h + 1].contiguous(), causal=True) for h in range(p["H"])]
    assert torch.equal(torch.cat([o for o, _ in per], dim=2), full)
    assert torch.equal(torch.cat([l for _, l in per], dim=1), lfull)


def test_row_subset_equals_full_rows():
    q, k, v, kv = _inputs(2, 16, 16, 2, 8, True, 12)
    full, lfull = oracle.attention(q, k, v, causal=True, kv_len=kv)
    rows = torch.tensor([0, 5, 15, 16, 31])
    o, l = oracle.attention(q, k, v, causal=True, kv_len=kv, rows=rows)
    fo = full.reshape(32, 2, 8)
    fl = lfull.permute(0, 2, 1).reshape(32, 2)
    assert torch.equal(o, fo[rows])
    assert torch.equal(l, fl[rows])


@pytest.mark.parametrize("causal", [True, False])
def test_kv_chunks_merged_equal_unchunked(causal):
    """Ring share in miniature: a late Q chunk against P KV chunks at their global
    positions, merged by log-sum-exp, equals the unchunked result ('adv07: Sequence
    Parallel', Q5 and section 5, Ring Attention).  Chunks wholly in the future give
    -inf and weight 0."""
    P, Sc, H, D = 4, 6, 2, 8
    g = W.generator(13)
    q = W.randn((1, Sc, H, D), g, torch.float32)
    k = W.randn((1, P * Sc, H, D), g, torch.float32)
    v = W.randn((1, P * Sc, H, D), g, torch.float32)
    qp = 2 * Sc  # third chunk: chunk 3 is entirely in the future
    ref, lref = oracle.attention(q, k, v, causal=causal, q_pos0=qp, k_pos0=0)
    parts = [oracle.attention(q, k[:, t * Sc:(t + 1) * Sc], v[:, t * Sc:(t + 1) * Sc], causal=causal,
                              q_pos0=qp, k_pos0=t * Sc) for t in range(P)]
    if causal:
        assert torch.all(torch.isinf(parts[3][1]))
    out, lse = oracle.merge_lse([o for o, _ in parts], [l for _, l in parts])
    assert (out - ref).abs().max().item() <= 1e-12
    assert (lse - lref).abs().max().item() <= 1e-12
    # pairwise streaming merge gives the same
    o_run, l_run = parts[0]
    for o, l in parts[1:]:
        o_run, l_run = oracle.merge_lse([o_run, o], [l_run, l])
    assert (o_run - ref).abs().max().item() <= 1e-12


def test_merge_extremes():
    g = W.generator(14)
    B, S, H, D = 1, 5, 2, 4
    os_ = [torch.randn(B, S, H, D, generator=g, dtype=torch.float64) for _ in range(3)]
    ls_ = [torch.randn(B, H, S, generator=g, dtype=torch.float64) * 80 for _ in range(3)]
    ls_[0][0, 0, 0] = float("-inf")
    for l in ls_:
        l[0, 1, 1] = float("-inf")
    out, lse = oracle.merge_lse(os_, ls_)
    assert torch.all(torch.isfinite(out))
    assert lse[0, 1, 1] == float("-inf") and torch.all(out[0, 1, 1] == 0)
    # a single part is returned unchanged
    o1, l1 = oracle.merge_lse(os_[:1], ls_[:1])
    assert torch.allclose(o1[torch.isfinite(ls_[0]).permute(0, 2, 1)],
                          os_[0][torch.isfinite(ls_[0]).permute(0, 2, 1)], atol=1e-15, rtol=0)
    # weights: exact by hand for one row
    w = torch.tensor([ls_[k][0, 0, 2].item() for k in range(3)], dtype=torch.float64)
    ww = torch.exp(w - w.max())
    exp = sum((ww[k] / ww.sum()) * os_[k][0, 2, 0] for k in range(3))
    assert torch.allclose(out[0, 2, 0], exp, atol=1e-12, rtol=0)


def test_permute_matches_concat_then_slice():
    """shard_permute == 'concatenate shards along the sequence, keep head group g'
    (data collator slices of 'Support deepspeed sequence parallel'; contiguous head
    groups of 'parallel multi-head attention' 2.2); and concatenating all groups along
    heads restores the concatenated shards (bit-exact)."""
    P, B, S, H, D = 4, 2, 12, 8, 3
    g = W.generator(15)
    shards = [W.randn((B, S // P, H, D), g, torch.bfloat16) for _ in range(P)]
    full = torch.cat(shards, dim=1)
    outs = []
    for grp in range(P):
        o = oracle.shard_permute(shards, grp)
        ref = full[:, :, grp * (H // P):(grp + 1) * (H // P)]
        assert torch.equal(o.view(torch.int16), ref.contiguous().view(torch.int16))
        outs.append(o)
    assert torch.equal(torch.cat(outs, dim=2).view(torch.int16), full.view(torch.int16))
    back = oracle.shard_unpermute(outs)
    for a, b in zip(back, shards):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("case", json.load(open(os.path.join(GOLDEN, "hand_examples.json")))["all_to_all"],
                         ids=["ulysses_forward", "ulysses_return", "seq_first_with_middle_dim"])
def test_hand_example_all_to_all(case):
    """Hand-derived all-to-all layouts (values worked out by hand in the derivation strings)."""
    ins = [torch.tensor(x, dtype=torch.int32) for x in case["inputs"]]
    for r in range(case["P"]):
        out = oracle.all_to_all(ins, r, case["scatter_dim"], case["gather_dim"])
        assert out.tolist() == case["outputs"][r]


# (shape per rank, P, scatter dim, gather dim): Ulysses forward/return on [B,S,H,D], the
# sequence-first [S,B,H,D] layout, packed QKV [B,S,3,H,D], 1-byte and 8-byte elements, and dims at
# both ends of the shape
A2A_CASES = [((2, 3, 8, 4), 4, 2, 1, torch.bfloat16), ((2, 12, 2, 4), 4, 1, 2, torch.bfloat16),
             ((3, 2, 6, 5), 3, 2, 0, torch.float32), ((2, 3, 3, 4, 2), 2, 3, 1, torch.bfloat16),
             ((4, 6), 2, 0, 1, torch.int8), ((5, 2, 4), 4, 2, 0, torch.float64),
             ((2, 2, 2, 2, 2, 2, 2, 4), 2, 7, 0, torch.int16)]


def _a2a_inputs(shape, P, dtype, seed):
    g = W.generator(seed)
    if dtype in (torch.int8, torch.int16):
        return [torch.randint(-100, 100, shape, generator=g, dtype=dtype) for _ in range(P)]
    return [W.randn(shape, g, torch.float32).to(dtype) for _ in range(P)]


@pytest.mark.parametrize("shape,P,sd,gd,dtype", A2A_CASES)
def test_all_to_all_matches_split_and_cat(shape, P, sd, gd, dtype):
    """The definition with library routines: rank r's result = concatenation along the gather dim,
    in rank order, of chunk r of every rank's tensor split into P parts along the scatter dim
    (torch.tensor_split / torch.cat, the all_to_all of "Support deepspeed sequence parallel")."""
    ins = _a2a_inputs(shape, P, dtype, seed=len(shape) * 10 + sd)
    for r in range(P):
        ref = torch.cat([torch.tensor_split(x, P, dim=sd)[r] for x in ins], dim=gd)
        got = oracle.all_to_all(ins, r, sd, gd)
        assert got.shape == ref.shape and torch.equal(got.view(torch.uint8), ref.contiguous().view(torch.uint8))


@pytest.mark.parametrize("shape,P,sd,gd,dtype", A2A_CASES)
def test_all_to_all_round_trip(shape, P, sd, gd, dtype):
    """The all-to-all with the dims swapped undoes it: every rank gets its own tensor back."""
    ins = _a2a_inputs(shape, P, dtype, seed=len(shape) * 10 + gd + 1)
    mid = [oracle.all_to_all(ins, r, sd, gd) for r in range(P)]
    for r in range(P):
        back = oracle.all_to_all(mid, r, gd, sd)
        assert torch.equal(back.view(torch.uint8), ins[r].view(torch.uint8))


def test_all_to_all_ulysses_case_is_shard_permute():
    """Scatter heads (dim 2), gather seq (dim 1) on [B, S/P, H, D] shards is shard_permute."""
    P, B, S, H, D = 4, 2, 12, 8, 3
    ins = _a2a_inputs((B, S // P, H, D), P, torch.bfloat16, seed=21)
    for r in range(P):
        assert torch.equal(oracle.all_to_all(ins, r, 2, 1).view(torch.int16),
                           oracle.shard_permute(ins, r).view(torch.int16))


def test_all_to_all_rejects_bad_dims():
    ins = _a2a_inputs((4, 6), 2, torch.float32, seed=1)
    with pytest.raises(ValueError):
        oracle.all_to_all(ins, 0, 1, 1)       # scatter dim == gather dim
    with pytest.raises(ValueError):
        oracle.all_to_all(_a2a_inputs((3, 6), 2, torch.float32, 1), 0, 0, 1)  # 3 rows over 2 ranks
    with pytest.raises(ValueError):
        oracle.all_to_all(ins, 2, 0, 1)       # rank out of range


def test_workload_one_full_check():
    """Workload 1 end to end on the oracle: two-pass == brute force == torch fp64 MHA."""
    inp, p = W.workload_inputs(1)
    q, k, v = inp["q"], inp["k"], inp["v"]
    o1, l1 = oracle.attention(q, k, v, causal=True)
    o2, l2, _ = oracle.attention_bruteforce(q, k, v, causal=True)
    assert (o1 - o2).abs().max().item() <= 1e-12
    qt, kt, vt = (x.double().permute(0, 2, 1, 3) for x in (q, k, v))
    ref = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True).permute(0, 2, 1, 3)
    assert (o1 - ref).abs().max().item() <= 1e-12


def test_inputs_are_seeded_and_rounded():
    a, _ = W.workload_inputs(2, B=1, S=64, H=2)
    b, _ = W.workload_inputs(2, B=1, S=64, H=2)
    assert a["q"].dtype == torch.bfloat16 and torch.equal(a["q"], b["q"])
    c, p = W.workload_inputs(5, B=8, S=64, len_lo=16, len_hi=64, H=1, D=8)
    assert c["kv_len"].dtype == torch.int32
    assert int(c["kv_len"].min()) >= 16 and int(c["kv_len"].max()) <= 64


def test_oracle_rejects_bad_arguments():
    q = torch.zeros(1, 4, 2, 8)
    with pytest.raises(ValueError):
        oracle.attention(q, q, q, rows=torch.tensor([8]))
    with pytest.raises(ValueError):
        oracle.shard_permute([torch.zeros(1, 2, 3, 4)] * 2, 0)  # H=3 not divisible by P=2
    with pytest.raises(ValueError):
        oracle.shard_permute([torch.zeros(1, 2, 4, 4)] * 2, 2)  # group out of range


# ---- attention backward ----------------------------------------------------------------------

def _dyadic(shape, g, lo=-24, hi=24):
    """fp32 values that are multiples of 2^-8 (so +-2^-10 perturbations are exact in fp32)."""
    return torch.randint(lo, hi + 1, shape, generator=g).to(torch.float32) / 256.0


def _loss(q, k, v, dout, **kw):
    out, _ = oracle.attention(q, k, v, **kw)
    return float((out * dout.double()).sum())


@pytest.mark.parametrize("kw", [dict(causal=True, q_pos0=1, k_pos0=0),
                                dict(causal=False, kv_len=torch.tensor([3, 5], dtype=torch.int32)),
                                dict(causal=True, q_pos0=0, k_pos0=2)])  # first rows see no key
def test_backward_matches_finite_differences(kw):
    """Central differences of the forward oracle's L = sum(dout * out) against every element of
    the analytic dq, dk, dv (the chain rule through softmax)."""
    g = torch.Generator().manual_seed(71)
    B = 2 if "kv_len" in kw else 1
    q, k, v = _dyadic((B, 4, 2, 3), g), _dyadic((B, 5, 2, 3), g), _dyadic((B, 5, 2, 3), g)
    dout = _dyadic((B, 4, 2, 3), g)
    dq, dk, dv = oracle.attention_backward(q, k, v, dout, **kw)
    h = 2.0 ** -10
    for name, t, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        flat = t.view(-1)
        num = torch.empty(flat.numel(), dtype=torch.float64)
        for e in range(flat.numel()):
            x0 = float(flat[e])
            flat[e] = x0 + h
            lp = _loss(q, k, v, dout, **kw)
            flat[e] = x0 - h
            lm = _loss(q, k, v, dout, **kw)
            flat[e] = x0
            num[e] = (lp - lm) / (2 * h)
        assert torch.allclose(grad.reshape(-1), num, rtol=1e-5, atol=1e-6), (name, (grad.reshape(-1) - num).abs().max())


def _torch_attention_grads(q, k, v, dout, causal, q_pos0, k_pos0, kv_len, scale):
    """fp64 autograd of attention written with plain torch ops (every row must see a key)."""
    q, k, v = (t.double().requires_grad_(True) for t in (q, k, v))
    B, Sq, H, D = q.shape
    Sk = k.shape[1]
    s = torch.einsum("bihd,bjhd->bhij", q, k) * scale
    i = torch.arange(Sq).view(Sq, 1)
    j = torch.arange(Sk).view(1, Sk)
    vis = torch.ones(B, 1, Sq, Sk, dtype=torch.bool)
    if causal:
        vis = vis & (k_pos0 + j <= q_pos0 + i)
    if kv_len is not None:
        vis = vis & (j < kv_len.view(B, 1, 1, 1).long())
    s = s.masked_fill(~vis, float("-inf"))
    out = torch.einsum("bhij,bjhd->bihd", torch.softmax(s, dim=-1), v)
    (out * dout.double()).sum().backward()
    return q.grad, k.grad, v.grad


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_backward_matches_fp64_autograd(dtype):
    """The oracle's gradients equal fp64 torch autograd through a plain attention (a library
    routine on the same fp64 values)."""
    g = W.generator(72)
    B, Sq, Sk, H, D = 2, 33, 40, 3, 16
    q, k, v, dout = (W.randn(s, g, dtype) for s in ((B, Sq, H, D), (B, Sk, H, D), (B, Sk, H, D), (B, Sq, H, D)))
    kv = torch.tensor([40, 29], dtype=torch.int32)
    for causal, qp, kp, kl in ((True, 7, 0, None), (False, 0, 0, kv), (True, 10, 3, kv)):
        dq, dk, dv = oracle.attention_backward(q, k, v, dout, causal=causal, q_pos0=qp, k_pos0=kp, kv_len=kl)
        tq, tk, tv = _torch_attention_grads(q, k, v, dout, causal, qp, kp, kl, 1.0 / math.sqrt(D))
        for a, b in ((dq, tq), (dk, tk), (dv, tv)):
            assert torch.allclose(a, b, rtol=1e-10, atol=1e-12)


def test_backward_invariants():
    """Closed forms: sum over keys of dK is 0 (each softmax row's dS sums to 0); sum over keys of
    dV equals the sum of dout over rows that see a key; V = 0 gives dQ = dK = 0; a row with no
    visible key gets dQ = 0."""
    g = W.generator(73)
    B, Sq, Sk, H, D = 1, 20, 24, 2, 8
    q, k, v, dout = (W.randn(s, g, torch.float32) for s in ((B, Sq, H, D), (B, Sk, H, D), (B, Sk, H, D), (B, Sq, H, D)))
    dq, dk, dv = oracle.attention_backward(q, k, v, dout, causal=True, q_pos0=0, k_pos0=5)
    # rows i < 5 see no key (k_pos0 + j <= i needs i >= 5)
    assert torch.all(dq[:, :5] == 0)
    assert dk.sum(dim=1).abs().max() < 1e-12
    assert torch.allclose(dv.sum(dim=1), dout[:, 5:].double().sum(dim=1), atol=1e-12)
    dq0, dk0, _ = oracle.attention_backward(q, k, torch.zeros_like(v), dout, causal=True)
    assert torch.all(dq0 == 0) and torch.all(dk0 == 0)

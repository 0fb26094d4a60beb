"""GPU parity of attn_fwd against the fp64 oracle on seeded inputs (through the C ABI).

Shapes span several 128-row query tiles and 64-key tiles with ragged tails,
both head dims of the matrix-core path, the fp32 path, every mask mode,
global position offsets that put the causal diagonal at odd places, rows
and whole calls with no visible key, and both output dtypes.
"""
import math

import pytest
import torch

import oracle
import tensor_head_attention_amd as T
import tha_workloads as W
from parity import DEV, check_lse, check_out, say, to_dev

pytestmark = pytest.mark.gpu


def _inputs(B, Sq, Sk, H, D, dtype, seed, lens=None):
    g = W.generator(seed)
    kv = None
    if lens is not None:
        kv = torch.tensor(lens, dtype=torch.int32)
    q = W.randn((B, Sq, H, D), g, dtype)
    k = W.randn((B, Sk, H, D), g, dtype)
    v = W.randn((B, Sk, H, D), g, dtype)
    return q, k, v, kv


CASES = [
    # B, Sq, Sk, H, D, dtype, causal, q_pos0, k_pos0, lens
    (1, 128, 128, 1, 128, torch.bfloat16, False, 0, 0, None),
    (1, 256, 256, 2, 128, torch.bfloat16, True, 0, 0, None),
    (2, 300, 300, 3, 128, torch.bfloat16, True, 0, 0, None),        # ragged tails
    (2, 200, 333, 2, 128, torch.bfloat16, False, 0, 0, None),       # Sq != Sk
    (1, 77, 500, 2, 128, torch.bfloat16, True, 423, 0, None),       # late query chunk (ring-like)
    (1, 190, 260, 2, 128, torch.bfloat16, True, 37, 5, None),       # diagonal at odd offsets
    (1, 64, 64, 2, 128, torch.bfloat16, True, 0, 40, None),         # early rows see nothing
    (3, 160, 160, 2, 128, torch.bfloat16, False, 0, 0, [1, 97, 160]),
    (2, 150, 200, 2, 128, torch.bfloat16, True, 50, 0, [0, 130]),   # an empty sequence
    (2, 330, 330, 3, 64, torch.bfloat16, True, 0, 0, None),
    (2, 129, 257, 2, 64, torch.bfloat16, False, 0, 0, [200, 257]),
    (1, 1, 1, 1, 128, torch.bfloat16, False, 0, 0, None),
    (1, 1, 700, 1, 128, torch.bfloat16, True, 699, 0, None),        # decode-like single row
    (48, 70, 70, 1, 128, torch.bfloat16, True, 0, 0, None),         # many sequences, one head
    (5, 90, 130, 40, 128, torch.bfloat16, False, 0, 0, [130, 1, 64, 0, 99]),  # 40 heads: 10 KiB tokens
    (1, 64, 64, 2, 8, torch.float32, True, 0, 0, None),
    (2, 70, 90, 3, 40, torch.float32, False, 0, 0, [90, 17]),
    (1, 33, 200, 2, 256, torch.float32, True, 167, 0, None),
    (1, 50, 50, 1, 1, torch.float32, True, 0, 0, None),
]


def _id(c):
    B, Sq, Sk, H, D, dt, causal, qp, kp, lens = c
    return f"B{B}_Sq{Sq}_Sk{Sk}_H{H}_D{D}_{'bf16' if dt == torch.bfloat16 else 'f32'}" \
           f"{'_causal' if causal else ''}_qp{qp}_kp{kp}{'_pad' if lens else ''}"


# every case on the automatic choice; the bf16 head-size-128 cases also on each kernel forced
KCASES = [(c, None) for c in CASES] + [(c, kn) for c in CASES if c[4] == 128 and c[5] == torch.bfloat16
                                       for kn in ("narrow", "wide", "split", "split64")]


@pytest.mark.parametrize("case,kernel", KCASES, ids=lambda x: _id(x) if isinstance(x, tuple) else str(x))
@pytest.mark.parametrize("out_f32", [False, True])
def test_attn_matches_oracle(case, kernel, out_f32):
    B, Sq, Sk, H, D, dt, causal, qp, kp, lens = case
    say(f"attn case {_id(case)} kernel={kernel} out_f32={out_f32}")
    q, k, v, kv = _inputs(B, Sq, Sk, H, D, dt, seed=Sq * 7 + Sk + D)
    ref, ref_lse = oracle.attention(q, k, v, causal=causal, q_pos0=qp, k_pos0=kp, kv_len=kv)
    qd, kd, vd = to_dev(q, k, v)
    kvd = kv.to(DEV) if kv is not None else None
    out, lse = T.attn_fwd(qd, kd, vd, causal=causal, q_pos0=qp, k_pos0=kp, kv_len=kvd,
                          out_dtype=torch.float32 if out_f32 else dt, kernel=kernel)
    torch.cuda.synchronize()
    check_out(out, ref, dt)
    check_lse(lse, ref_lse, dt)


@pytest.mark.parametrize("shape", [(1, 600, 600, 3, True, 0, 0, None), (2, 513, 700, 2, False, 0, 0, [700, 333]),
                                   (1, 300, 900, 2, True, 600, 0, None), (1, 1024, 1024, 8, True, 0, 0, None)])
def test_attn_d128_kernels_bitwise_equal(shape):
    """The narrow and wide head-size-128 kernels take the same arithmetic steps per row (same key
    tile order, product order, softmax and row-sum order, rescale decisions), so their results
    agree bit for bit; both also match the oracle."""
    B, Sq, Sk, H, causal, qp, kp, lens = shape
    say(f"narrow vs wide {shape}")
    q, k, v, kv = _inputs(B, Sq, Sk, H, 128, torch.bfloat16, seed=Sq + 3 * Sk + H)
    qd, kd, vd = to_dev(q, k, v)
    kvd = kv.to(DEV) if kv is not None else None
    res = {}
    for kn in ("narrow", "wide"):
        res[kn] = T.attn_fwd(qd, kd, vd, causal=causal, q_pos0=qp, k_pos0=kp, kv_len=kvd,
                             out_dtype=torch.float32, kernel=kn)
        torch.cuda.synchronize()
    assert torch.equal(res["narrow"][0], res["wide"][0])
    assert torch.equal(res["narrow"][1], res["wide"][1])
    ref, ref_lse = oracle.attention(q, k, v, causal=causal, q_pos0=qp, k_pos0=kp, kv_len=kv)
    check_out(res["wide"][0], ref, torch.bfloat16)
    check_lse(res["wide"][1], ref_lse, torch.bfloat16)


def test_attn_custom_scale_and_no_lse():
    q, k, v, _ = _inputs(1, 200, 200, 2, 128, torch.bfloat16, seed=3)
    ref, _ = oracle.attention(q, k, v, causal=True, scale=0.3)
    qd, kd, vd = to_dev(q, k, v)
    out = T.attn_fwd(qd, kd, vd, causal=True, scale=0.3, return_lse=False)
    torch.cuda.synchronize()
    check_out(out, ref, torch.bfloat16)


def test_attn_kv_len_clamped():
    """kv_len outside [0, Sk] is clamped on the device."""
    q, k, v, _ = _inputs(3, 70, 90, 1, 128, torch.bfloat16, seed=4)
    kv = torch.tensor([-5, 1000, 45], dtype=torch.int32)
    ref, ref_lse = oracle.attention(q, k, v, kv_len=kv)
    qd, kd, vd, kvd = to_dev(q, k, v, kv)
    out, lse = T.attn_fwd(qd, kd, vd, kv_len=kvd)
    torch.cuda.synchronize()
    check_out(out, ref, torch.bfloat16)
    check_lse(lse, ref_lse, torch.bfloat16)
    assert torch.all(out[0] == 0)


@pytest.mark.parametrize("kernel", ["narrow", "wide", "split", "split64", None])
def test_attn_deterministic_and_q_split(kernel):
    """Repeated calls are bit-identical, and splitting the query rows into chunks
    (each chunk against the full K/V, 'adv07: Sequence Parallel' section 4) gives
    the same bits as the whole call when both take the same kernel form, since each
    row depends on its own query only.  With the automatic choice the chunks may take
    another form than the whole call (it depends on the grid size), so there the split
    result is compared with the oracle at the bf16 tolerance."""
    q, k, v, _ = _inputs(1, 1000, 1000, 4, 128, torch.bfloat16, seed=5)
    qd, kd, vd = to_dev(q, k, v)
    o1, l1 = T.attn_fwd(qd, kd, vd, causal=True, kernel=kernel)
    o2, l2 = T.attn_fwd(qd, kd, vd, causal=True, kernel=kernel)
    parts = []
    for lo in range(0, 1000, 384):
        hi = min(lo + 384, 1000)
        parts.append(T.attn_fwd(qd[:, lo:hi].contiguous(), kd, vd, causal=True, q_pos0=lo, kernel=kernel))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o_split = torch.cat([o for o, _ in parts], dim=1)
    l_split = torch.cat([l for _, l in parts], dim=2)
    if kernel is not None:
        assert torch.equal(o_split, o1) and torch.equal(l_split, l1)
    ref, ref_lse = oracle.attention(q, k, v, causal=True)
    check_out(o_split, ref, torch.bfloat16)
    check_lse(l_split, ref_lse, torch.bfloat16)


def test_attn_head_split_concat_equals_full():
    """Per-head calls concatenated equal the all-heads call ('parallel multi-head
    attention' sections 2.2 and 3.1: whole heads per device), on the fp32 tiny
    workload and a bf16 shape."""
    inp, p = W.workload_inputs(1)
    for q, k, v, dt in [(inp["q"], inp["k"], inp["v"], torch.float32),
                        (*_inputs(1, 300, 300, 4, 128, torch.bfloat16, seed=6)[:3], torch.bfloat16)]:
        qd, kd, vd = to_dev(q, k, v)
        # one kernel form for both calls (the automatic choice depends on the grid size)
        kn = "split" if dt == torch.bfloat16 else None
        full, lfull = T.attn_fwd(qd, kd, vd, causal=True, kernel=kn)
        per = [T.attn_fwd(qd[:, :, h:h + 1].contiguous(), kd[:, :, h:h + 1].contiguous(),
                          vd[:, :, h:h + 1].contiguous(), causal=True, kernel=kn) for h in range(q.shape[2])]
        torch.cuda.synchronize()
        assert torch.equal(torch.cat([o for o, _ in per], dim=2), full)
        assert torch.equal(torch.cat([l for _, l in per], dim=1), lfull)
        ref, ref_lse = oracle.attention(q, k, v, causal=True)
        check_out(full, ref, dt)
        check_lse(lfull, ref_lse, dt)


def test_attn_kv_chunks_merged_equal_unchunked():
    """Ring share in miniature on the device: a late Q chunk against 5 KV chunks at
    their global positions (one wholly in the future), fp32 partials merged by
    attn_merge_lse, equals the oracle's unchunked attention."""
    P, Sc, H, D = 5, 200, 2, 128
    g = W.generator(21)
    q = W.randn((1, Sc, H, D), g, torch.bfloat16)
    k = W.randn((1, P * Sc, H, D), g, torch.bfloat16)
    v = W.randn((1, P * Sc, H, D), g, torch.bfloat16)
    qp = 3 * Sc
    ref, ref_lse = oracle.attention(q, k, v, causal=True, q_pos0=qp, k_pos0=0)
    qd, kd, vd = to_dev(q, k, v)
    parts = [T.attn_fwd(qd, kd[:, t * Sc:(t + 1) * Sc].contiguous(), vd[:, t * Sc:(t + 1) * Sc].contiguous(),
                        causal=True, q_pos0=qp, k_pos0=t * Sc, out_dtype=torch.float32) for t in range(P)]
    out, lse = T.attn_merge_lse([o for o, _ in parts], [l for _, l in parts], out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.all(torch.isinf(parts[4][1]))
    check_out(out, ref, torch.bfloat16)
    check_lse(lse, ref_lse, torch.bfloat16)


def _expected_form(B, Sq, Sk, H, causal, qp, kp, cus):
    """The automatic choice for bf16, head size 128 (tha.h attn_fwd), restated."""
    if B * H * -(-Sq // 256) >= 2 * cus:
        return "wide"
    blocks = B * H * -(-Sq // 128)
    if blocks >= 2 * cus:
        return "narrow"
    if 2 * blocks <= cus:
        return "split64"

    def keys(rows):
        return min(max(qp - kp + rows, 0), Sk)
    if causal and blocks <= cus and 2 * keys(min(Sq, 128)) <= keys(Sq):
        return "split64"
    return "split"


@pytest.mark.parametrize("shape", [
    (1, 4096, 4096, 8, True, 0, 0),         # causal, as many 128-row tiles as CUs: 64-row split
    (1, 4096, 4096, 8, True, 28672, 0),     # a Ring chunk wholly in the past: balanced, 128-row split
    (1, 4096, 4096, 8, False, 0, 0),        # non-causal: 128-row split
    (1, 1024, 3000, 8, False, 0, 0),        # a quarter of the CUs as 128-row tiles: 64-row split
    (1, 6144, 6144, 8, True, 0, 0),         # causal, more 128-row tiles than CUs: 128-row split
    (2, 4096, 4096, 8, True, 0, 0),         # two 128-row tiles per CU: narrow
    (1, 8192, 8192, 8, True, 0, 0)])        # wide
def test_attn_automatic_form(shape):
    """The automatic choice takes the form the rule in tha.h names for the device's CU count: its
    result equals that form's, forced, bit for bit."""
    B, Sq, Sk, H, causal, qp, kp = shape
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    form = _expected_form(B, Sq, Sk, H, causal, qp, kp, cus)
    say(f"automatic form {shape} on {cus} CUs -> {form}")
    q, k, v, _ = _inputs(B, Sq, Sk, H, 128, torch.bfloat16, seed=Sq + H + B)
    qd, kd, vd = to_dev(q, k, v)
    auto = T.attn_fwd(qd, kd, vd, causal=causal, q_pos0=qp, k_pos0=kp)
    forced = T.attn_fwd(qd, kd, vd, causal=causal, q_pos0=qp, k_pos0=kp, kernel=form)
    torch.cuda.synchronize()
    assert torch.equal(auto[0], forced[0]) and torch.equal(auto[1], forced[1])
    others = [kn for kn in ("narrow", "split", "split64") if kn != form and not (form == "wide" and kn == "narrow")]
    # the forms differ in the last bits somewhere (so the equality above identifies the form)
    assert any(not torch.equal(auto[0], T.attn_fwd(qd, kd, vd, causal=causal, q_pos0=qp, k_pos0=kp, kernel=kn)[0])
               for kn in others)

"""GPU checks of attn_fwd_ex: strided views (packed QKV, head subsets, strided outputs) and the
fused Ring step (THA_ACCUMULATE), through the C ABI.

Strided calls run the same kernels as attn_fwd with different addressing only, so they must give
the same bits as attn_fwd on contiguous copies; they are also checked against the oracle.  The
fused Ring step merges each chunk's result into a running fp32 (o, lse) by the rule of
attn_merge_lse; it is checked against the oracle's unchunked attention (bf16 tolerances) and
against the separate partials + merge route (fp32 rounding of the two association orders)."""
import pytest
import torch

import oracle
import tensor_head_attention_amd as T
import tha_workloads as W
from parity import DEV, check_lse, check_out, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,S,H,D,dt,causal,kernel", [
    (2, 300, 3, 128, torch.bfloat16, True, "narrow"),
    (2, 300, 3, 128, torch.bfloat16, True, "wide"),
    (2, 300, 3, 128, torch.bfloat16, True, "split"),
    (2, 300, 3, 128, torch.bfloat16, True, "split64"),
    (1, 520, 2, 128, torch.bfloat16, False, None),
    (2, 200, 2, 64, torch.bfloat16, True, None),
    (2, 70, 3, 40, torch.float32, True, None),
])
def test_packed_qkv_views(B, S, H, D, dt, causal, kernel):
    say(f"packed qkv B{B} S{S} H{H} D{D} {dt} causal={causal} kernel={kernel}")
    g = W.generator(B * 1000 + S + D)
    qkv = W.randn((B, S, 3, H, D), g, dt)
    q, k, v = (qkv[:, :, i].contiguous() for i in range(3))
    ref, ref_lse = oracle.attention(q, k, v, causal=causal)
    dev = qkv.to(DEV)
    qv, kv_, vv = dev[:, :, 0], dev[:, :, 1], dev[:, :, 2]   # views, token stride 3*H*D
    out, lse = T.attn_fwd_ex(qv, kv_, vv, causal=causal, kernel=kernel)
    base, base_lse = T.attn_fwd(*to_dev(q, k, v), causal=causal, kernel=kernel)
    torch.cuda.synchronize()
    assert torch.equal(out, base) and torch.equal(lse, base_lse)
    check_out(out, ref, dt)
    check_lse(lse, ref_lse, dt)


@pytest.mark.parametrize("kernel", ["narrow", "wide", "split", "split64"])
def test_head_subset_views_and_strided_output(kernel):
    """q, k, v are heads 2..4 of wider [B, S, 8, D] tensors (token stride 8*D), and the output is
    written into heads 1..3 of a [B, S, 6, D] fp32 buffer: the rest of that buffer is untouched."""
    B, S, D = 2, 300, 128
    g = W.generator(7)
    big = [W.randn((B, S, 8, D), g, torch.bfloat16).to(DEV) for _ in range(3)]
    qv, kv_, vv = (t[:, :, 2:5] for t in big)
    o_big = torch.full((B, S, 6, D), 7.0, dtype=torch.float32, device=DEV)
    lse = torch.empty((B, 3, S), dtype=torch.float32, device=DEV)
    T.attn_fwd_ex(qv, kv_, vv, causal=True, out=o_big[:, :, 1:4], lse=lse, kernel=kernel)
    base, base_lse = T.attn_fwd(qv.contiguous(), kv_.contiguous(), vv.contiguous(), causal=True,
                                out_dtype=torch.float32, kernel=kernel)
    torch.cuda.synchronize()
    assert torch.equal(o_big[:, :, 1:4], base) and torch.equal(lse, base_lse)
    assert torch.all(o_big[:, :, 0] == 7.0) and torch.all(o_big[:, :, 4:] == 7.0)
    ref, ref_lse = oracle.attention(*(t.cpu() for t in (qv.contiguous(), kv_.contiguous(), vv.contiguous())),
                                    causal=True)
    check_out(o_big[:, :, 1:4], ref, torch.bfloat16)


@pytest.mark.parametrize("D,dt,kernel", [(128, torch.bfloat16, "narrow"), (128, torch.bfloat16, "wide"),
                                         (128, torch.bfloat16, "split"), (128, torch.bfloat16, "split64"),
                                         (64, torch.bfloat16, None), (32, torch.float32, None)])
def test_fused_ring_step(D, dt, kernel):
    """A late Q chunk against P KV chunks at their global positions (one wholly in the future),
    each call merging into the running fp32 (o, lse) that starts as (NaN, -inf): the result equals
    the oracle's unchunked attention and the partials + attn_merge_lse route."""
    P, Sc, H = 5, 200, 2
    say(f"fused ring step D{D} {dt} kernel={kernel}")
    g = W.generator(31 + D)
    q = W.randn((1, Sc, H, D), g, dt)
    k = W.randn((1, P * Sc, H, D), g, dt)
    v = W.randn((1, P * Sc, H, D), g, dt)
    qp = 3 * Sc
    ref, ref_lse = oracle.attention(q, k, v, causal=True, q_pos0=qp, k_pos0=0)
    qd, kd, vd = to_dev(q, k, v)
    o = torch.full((1, Sc, H, D), float("nan"), dtype=torch.float32, device=DEV)  # never read while lse = -inf
    lse = torch.full((1, H, Sc), float("-inf"), dtype=torch.float32, device=DEV)
    parts = []
    for t in range(P):
        kc, vc = kd[:, t * Sc:(t + 1) * Sc], vd[:, t * Sc:(t + 1) * Sc]   # views into the full K/V
        if t == 4:
            before = (o.clone(), lse.clone())
        T.attn_fwd_ex(qd, kc, vc, causal=True, q_pos0=qp, k_pos0=t * Sc, out=o, lse=lse, accumulate=True, kernel=kernel)
        if t == 4:  # the chunk lies wholly in the queries' future: the running result is unchanged
            torch.cuda.synchronize()
            assert torch.equal(o, before[0]) and torch.equal(lse, before[1])
        parts.append(T.attn_fwd(qd, kc.contiguous(), vc.contiguous(), causal=True, q_pos0=qp, k_pos0=t * Sc,
                                out_dtype=torch.float32, kernel=kernel))
    merged, merged_lse = T.attn_merge_lse([p[0] for p in parts], [p[1] for p in parts],
                                          out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()
    check_out(o, ref, dt)
    check_lse(lse, ref_lse, dt)
    assert (o - merged).abs().max().item() <= 1e-5
    assert (lse - merged_lse).abs().max().item() <= 1e-5


def test_fused_ring_step_padding_and_batches():
    """B = 3 with key padding (one sequence empty) and the fused step over 3 chunks."""
    B, Sq, Sc, P, H, D = 3, 130, 96, 3, 2, 128
    g = W.generator(44)
    q = W.randn((B, Sq, H, D), g, torch.bfloat16)
    k = W.randn((B, P * Sc, H, D), g, torch.bfloat16)
    v = W.randn((B, P * Sc, H, D), g, torch.bfloat16)
    kv = torch.tensor([0, 150, 288], dtype=torch.int32)
    ref, ref_lse = oracle.attention(q, k, v, kv_len=kv)
    qd, kd, vd = to_dev(q, k, v)
    o = torch.zeros((B, Sq, H, D), dtype=torch.float32, device=DEV)
    lse = torch.full((B, H, Sq), float("-inf"), dtype=torch.float32, device=DEV)
    for t in range(P):
        # the padding length of chunk t, relative to its first key
        kvc = (kv - t * Sc).clamp(0, Sc).to(torch.int32).to(DEV)
        T.attn_fwd_ex(qd, kd[:, t * Sc:(t + 1) * Sc], vd[:, t * Sc:(t + 1) * Sc], kv_len=kvc, out=o, lse=lse,
                      accumulate=True)
    torch.cuda.synchronize()
    check_out(o, ref, torch.bfloat16)
    check_lse(lse, ref_lse, torch.bfloat16)
    assert torch.all(o[0] == 0) and torch.all(torch.isinf(lse[0]))

"""Global positions: causal visibility depends on q_pos0 - k_pos0 only (key j is visible to query
row i iff k_pos0 + j <= q_pos0 + i), for any positions the ABI accepts (|pos| < 2^62), negative and
very large ones included.  Every forward kernel and the backward must give bit-identical results
when both positions move by the same amount, every key to a query chunk far after the keys, and
none to one far before them."""
import pytest
import torch

import oracle
import tensor_head_attention_amd as T
import tha_workloads as W
from parity import DEV, check_lse, check_out, say, to_dev

pytestmark = pytest.mark.gpu

BIG = (1 << 62) - 1
SHIFTS = [-5000, 1 << 40, -(1 << 40), (1 << 61) + 12345, -(1 << 61)]
# (head dim, dtype, forced head-size-128 kernel)
KERNELS = [(128, torch.bfloat16, "narrow"), (128, torch.bfloat16, "wide"), (128, torch.bfloat16, "split"),
           (128, torch.bfloat16, "split64"),
           (64, torch.bfloat16, None), (40, torch.float32, None)]


def _kid(k):
    D, dt, kn = k
    return f"D{D}_{'bf16' if dt == torch.bfloat16 else 'f32'}_{kn or 'auto'}"


def _inputs(D, dt, seed, B=1, Sq=190, Sk=260, H=2):
    g = W.generator(seed)
    q, k, v = (W.randn((B, n, H, D), g, dt) for n in (Sq, Sk, Sk))
    return q, k, v


@pytest.mark.parametrize("kern", KERNELS, ids=_kid)
def test_fwd_position_shift(kern):
    D, dt, kn = kern
    say(f"positions fwd {_kid(kern)}")
    q, k, v = _inputs(D, dt, seed=901 + D)
    qd, kd, vd = to_dev(q, k, v)
    o0, l0 = T.attn_fwd(qd, kd, vd, causal=True, q_pos0=37, k_pos0=5, out_dtype=torch.float32, kernel=kn)
    for s in SHIFTS:
        o1, l1 = T.attn_fwd(qd, kd, vd, causal=True, q_pos0=37 + s, k_pos0=5 + s, out_dtype=torch.float32, kernel=kn)
        torch.cuda.synchronize()
        assert torch.equal(o0, o1) and torch.equal(l0, l1), f"shift {s}"
    # a query chunk far after every key sees them all: the non-causal result
    on, ln = T.attn_fwd(qd, kd, vd, out_dtype=torch.float32, kernel=kn)
    oa, la = T.attn_fwd(qd, kd, vd, causal=True, q_pos0=BIG, k_pos0=-BIG, out_dtype=torch.float32, kernel=kn)
    # and one far before every key sees none
    oz, lz = T.attn_fwd(qd, kd, vd, causal=True, q_pos0=-BIG, k_pos0=BIG, out_dtype=torch.float32, kernel=kn)
    torch.cuda.synchronize()
    assert torch.equal(oa, on) and torch.equal(la, ln)
    assert torch.count_nonzero(oz).item() == 0 and bool(torch.all(lz == float("-inf")))
    ref, ref_lse = oracle.attention(q, k, v, causal=True, q_pos0=37, k_pos0=5)
    check_out(o0, ref, dt)
    check_lse(l0, ref_lse, dt)


@pytest.mark.parametrize("D,dt", [(128, torch.bfloat16), (64, torch.bfloat16), (40, torch.float32)],
                         ids=["D128_bf16", "D64_bf16", "D40_f32"])
def test_bwd_position_shift(D, dt):
    say(f"positions bwd D{D} {dt}")
    q, k, v = _inputs(D, dt, seed=911 + D)
    g = W.generator(912 + D)
    dout = W.randn(tuple(q.shape), g, dt)
    qd, kd, vd, dd = to_dev(q, k, v, dout)
    res = []
    for qp, kp in [(37, 5)] + [(37 + s, 5 + s) for s in SHIFTS]:
        o, lse = T.attn_fwd(qd, kd, vd, causal=True, q_pos0=qp, k_pos0=kp)
        res.append(T.attn_bwd(qd, kd, vd, o, dd, lse, causal=True, q_pos0=qp, k_pos0=kp))
    torch.cuda.synchronize()
    for s, r in zip(SHIFTS, res[1:]):
        assert all(torch.equal(x, y) for x, y in zip(res[0], r)), f"shift {s}"

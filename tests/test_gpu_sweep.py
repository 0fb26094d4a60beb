"""Seeded sweep of random small shapes through the C ABI against the oracle: every bf16 forward
kernel (head size 128 narrow / wide / split, head size 64), the backward, and the fused Ring step.
Shapes, offsets, masks and key lengths are drawn from a fixed seed, so the sweep is the same on
every run; each case prints its parameters before it runs."""
import random

import pytest
import torch

import oracle
import tensor_head_attention_amd as T
import tha_workloads as W
from parity import DEV, check_lse, check_out, say, to_dev
from test_gpu_bwd import check_grad

pytestmark = pytest.mark.gpu


def _cases(seed, n):
    rnd = random.Random(seed)
    out = []
    for _ in range(n):
        B = rnd.choice([1, 1, 2, 3])
        Sq = rnd.choice([1, 7, 63, 64, 65, 129, 200, 257, 384, 511])
        Sk = rnd.choice([1, 5, 64, 100, 191, 256, 333, 520])
        H = rnd.choice([1, 2, 3])
        causal = rnd.random() < 0.6
        qp = rnd.choice([0, 0, Sk - 1, rnd.randrange(0, 2 * Sk)])
        kp = rnd.choice([0, 0, rnd.randrange(0, Sk + 1)])
        lens = [rnd.randrange(0, Sk + 1) for _ in range(B)] if rnd.random() < 0.4 else None
        out.append((B, Sq, Sk, H, causal, qp, kp, lens))
    return out


FWD = [(c, D, kn) for i, c in enumerate(_cases(2024, 24))
       for D, kn in ([(128, "narrow"), (128, "wide"), (128, "split"), (128, "split64")] if i % 2 == 0 else [(64, None), (128, None)])]


def _id(x):
    if isinstance(x, tuple):
        B, Sq, Sk, H, causal, qp, kp, lens = x
        return f"B{B}_Sq{Sq}_Sk{Sk}_H{H}{'_c' if causal else ''}_qp{qp}_kp{kp}{'_pad' if lens else ''}"
    return str(x)


@pytest.mark.parametrize("case,D,kernel", FWD, ids=_id)
def test_fwd_sweep(case, D, kernel):
    B, Sq, Sk, H, causal, qp, kp, lens = case
    say(f"sweep fwd {_id(case)} D{D} kernel={kernel}")
    g = W.generator(Sq * 31 + Sk * 7 + H + D)
    q = W.randn((B, Sq, H, D), g, torch.bfloat16)
    k = W.randn((B, Sk, H, D), g, torch.bfloat16)
    v = W.randn((B, Sk, H, D), g, torch.bfloat16)
    kv = torch.tensor(lens, dtype=torch.int32) if lens is not None else None
    ref, ref_lse = oracle.attention(q, k, v, causal=causal, q_pos0=qp, k_pos0=kp, kv_len=kv)
    qd, kd, vd = to_dev(q, k, v)
    kvd = kv.to(DEV) if kv is not None else None
    out, lse = T.attn_fwd(qd, kd, vd, causal=causal, q_pos0=qp, k_pos0=kp, kv_len=kvd, out_dtype=torch.float32,
                          kernel=kernel)
    torch.cuda.synchronize()
    check_out(out, ref, torch.bfloat16)
    check_lse(lse, ref_lse, torch.bfloat16)


@pytest.mark.parametrize("case", _cases(77, 12), ids=_id)
@pytest.mark.parametrize("D", [64, 128])
def test_bwd_sweep(case, D):
    B, Sq, Sk, H, causal, qp, kp, lens = case
    say(f"sweep bwd {_id(case)} D{D}")
    g = W.generator(Sq * 13 + Sk * 5 + H + D)
    q, dout = (W.randn((B, Sq, H, D), g, torch.bfloat16) for _ in range(2))
    k, v = (W.randn((B, Sk, H, D), g, torch.bfloat16) for _ in range(2))
    kv = torch.tensor(lens, dtype=torch.int32) if lens is not None else None
    rq, rk, rv = oracle.attention_backward(q, k, v, dout, causal=causal, q_pos0=qp, k_pos0=kp, kv_len=kv)
    qd, kd, vd, dd = to_dev(q, k, v, dout)
    kvd = kv.to(DEV) if kv is not None else None
    o, lse = T.attn_fwd(qd, kd, vd, causal=causal, q_pos0=qp, k_pos0=kp, kv_len=kvd)
    dq, dk, dv = T.attn_bwd(qd, kd, vd, o, dd, lse, causal=causal, q_pos0=qp, k_pos0=kp, kv_len=kvd)
    torch.cuda.synchronize()
    for got, ref, name in ((dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv")):
        check_grad(got, ref, torch.bfloat16, name)


@pytest.mark.parametrize("kernel", ["narrow", "wide", "split", "split64"])
@pytest.mark.parametrize("seed", [5, 6])
def test_fused_ring_sweep(kernel, seed):
    """Random chunk counts and sizes, a random query position, key padding on some sequences:
    the fused Ring pass (attn_fwd_ex with accumulate) equals the unchunked oracle."""
    rnd = random.Random(seed)
    B, H, D = rnd.choice([1, 2]), rnd.choice([1, 2]), 128
    P, Sc = rnd.choice([2, 3, 5]), rnd.choice([64, 100, 160])
    Sq = rnd.choice([50, 128, 200])
    qp = rnd.randrange(0, P * Sc)
    lens = [rnd.randrange(1, P * Sc + 1) for _ in range(B)]
    say(f"sweep fused ring B{B} H{H} P{P} Sc{Sc} Sq{Sq} qp{qp} lens{lens} kernel={kernel}")
    g = W.generator(seed * 101)
    q = W.randn((B, Sq, H, D), g, torch.bfloat16)
    k = W.randn((B, P * Sc, H, D), g, torch.bfloat16)
    v = W.randn((B, P * Sc, H, D), g, torch.bfloat16)
    kv = torch.tensor(lens, dtype=torch.int32)
    ref, ref_lse = oracle.attention(q, k, v, causal=True, q_pos0=qp, k_pos0=0, kv_len=kv)
    qd, kd, vd = to_dev(q, k, v)
    o = torch.zeros((B, Sq, H, D), dtype=torch.float32, device=DEV)
    lse = torch.full((B, H, Sq), float("-inf"), dtype=torch.float32, device=DEV)
    for t in range(P):
        kvc = (kv - t * Sc).clamp(0, Sc).to(torch.int32).to(DEV)
        T.attn_fwd_ex(qd, kd[:, t * Sc:(t + 1) * Sc], vd[:, t * Sc:(t + 1) * Sc], causal=True, q_pos0=qp,
                      k_pos0=t * Sc, kv_len=kvc, out=o, lse=lse, accumulate=True, kernel=kernel)
    torch.cuda.synchronize()
    check_out(o, ref, torch.bfloat16)
    check_lse(lse, ref_lse, torch.bfloat16)

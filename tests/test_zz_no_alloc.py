"""attn_bwd_noalloc (the backward with its Delta scratch in a fixed per-device array instead of a
caller workspace) against attn_bwd, through the C ABI: two calls in a row, the second with a
smaller input, each equal to attn_bwd's gradients bit for bit (same kernels, same Delta values),
and within the bf16 backward tolerance of the fp64 oracle."""
import pytest
import torch

import oracle
import tensor_head_attention_amd as T
import tha_workloads as W
from parity import DEV, say, to_dev

pytestmark = pytest.mark.gpu


def _case(B, Sq, Sk, H, D, dt, causal, lens, seed):
    g = W.generator(seed)
    q, dout = (W.randn((B, Sq, H, D), g, dt) for _ in range(2))
    k, v = (W.randn((B, Sk, H, D), g, dt) for _ in range(2))
    kv = torch.tensor(lens, dtype=torch.int32) if lens is not None else None
    return q, k, v, dout, kv


def _rel_l2(a, b):
    return ((a - b).norm() / b.norm()).item()


def test_noalloc_matches_attn_bwd_two_calls():
    cases = [(2, 700, 700, 3, 128, torch.bfloat16, True, None, 11),       # first call
             (1, 300, 500, 2, 128, torch.bfloat16, False, [333], 12)]     # second, smaller: stale scratch
    for B, Sq, Sk, H, D, dt, causal, lens, seed in cases:
        say(f"noalloc bwd B{B} Sq{Sq} Sk{Sk} H{H} D{D} causal={causal} lens={lens}")
        q, k, v, dout, kv = _case(B, Sq, Sk, H, D, dt, causal, lens, seed)
        qd, kd, vd, dd = to_dev(q, k, v, dout)
        kvd = kv.to(DEV) if kv is not None else None
        o, lse = T.attn_fwd(qd, kd, vd, causal=causal, kv_len=kvd)
        ref = T.attn_bwd(qd, kd, vd, o, dd, lse, causal=causal, kv_len=kvd)
        got = tuple(torch.zeros_like(t) for t in ref)
        T.attn_bwd_noalloc(qd, kd, vd, o, dd, lse, dq=got[0], dk=got[1], dv=got[2], causal=causal, kv_len=kvd)
        torch.cuda.synchronize()
        for a, b, n in zip(got, ref, ("dq", "dk", "dv")):
            assert torch.equal(a, b), n
        oq, ok_, ov = oracle.attention_backward(q, k, v, dout, causal=causal, kv_len=kv)
        for a, r, n in zip(got, (oq, ok_, ov), ("dq", "dk", "dv")):
            rel = _rel_l2(a.double().cpu(), r)
            say(f"  {n}: rel-L2 vs oracle {rel:.3e}")
            assert rel <= 1e-2


def test_noalloc_fp32_path_and_capacity():
    """The fp32 path through the same scratch, and a request beyond the scratch capacity rejected
    on the host before any launch."""
    q, k, v, dout, _ = _case(1, 90, 120, 2, 40, torch.float32, True, None, 13)
    qd, kd, vd, dd = to_dev(q, k, v, dout)
    o, lse = T.attn_fwd(qd, kd, vd, causal=True)
    ref = T.attn_bwd(qd, kd, vd, o, dd, lse, causal=True)
    got = tuple(torch.zeros_like(t) for t in ref)
    T.attn_bwd_noalloc(qd, kd, vd, o, dd, lse, dq=got[0], dk=got[1], dv=got[2], causal=True)
    torch.cuda.synchronize()
    for a, b in zip(got, ref):
        assert torch.equal(a, b)
    lib = T.load_library()
    p = qd.data_ptr()
    big_sq = T.THA_NOALLOC_MAX_DELTA + 1  # B*H*Sq over the capacity (pointers never used)
    rc = lib.attn_bwd_noalloc(p, p, p, p, p, p, p, p, p, 1, big_sq, 8, 1, 64, T.THA_BF16, 0, 0, 0, None, 0.125, None)
    assert rc == T.THA_ERR_TOO_LARGE

"""GPU check of the differentiable wrapper `attention` (attn_fwd forward, attn_bwd backward):
its output and the gradients autograd returns equal the direct calls, and match the oracle."""
import pytest
import torch

import oracle
import tensor_head_attention_amd as T
import tha_workloads as W
from parity import DEV, check_out, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_attention_autograd(dt):
    B, S, H, D = 2, 200, 2, (128 if dt == torch.bfloat16 else 40)
    say(f"autograd attention {dt} D{D}")
    g = W.generator(71)
    q, k, v, dout = (W.randn((B, S, H, D), g, dt) for _ in range(4))
    qd, kd, vd = (t.requires_grad_(True) for t in to_dev(q, k, v))
    dd = to_dev(dout)[0]
    out = T.attention(qd, kd, vd, causal=True, q_pos0=10)
    out.backward(dd)
    torch.cuda.synchronize()
    o_ref, _ = oracle.attention(q, k, v, causal=True, q_pos0=10)
    check_out(out.detach(), o_ref, dt)
    rq, rk, rv = oracle.attention_backward(q, k, v, dout, causal=True, q_pos0=10)
    direct_o, lse = T.attn_fwd(qd.detach(), kd.detach(), vd.detach(), causal=True, q_pos0=10)
    direct = T.attn_bwd(qd.detach(), kd.detach(), vd.detach(), direct_o, dd, lse, causal=True, q_pos0=10)
    torch.cuda.synchronize()
    assert torch.equal(out.detach(), direct_o)
    for grad, ref, dg, name in zip((qd.grad, kd.grad, vd.grad), (rq, rk, rv), direct, ("dq", "dk", "dv")):
        assert grad.dtype == dt
        assert torch.equal(grad, dg.to(dt)), name
        err = (grad.double().cpu() - ref).abs().max().item()
        scale = ref.abs().max().item()
        say(f"  {name}: max-abs {err:.3e} (max|ref| {scale:.3e})")
        assert err <= (3e-2 if dt == torch.bfloat16 else 1e-5) * max(1.0, scale), name

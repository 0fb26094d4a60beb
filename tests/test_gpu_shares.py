"""GPU checks of the share-level helpers of the binding, which only compose library calls:
ulysses_share (shard_permute x 3 + attn_fwd) and ring_share (chunk calls fused by accumulate, or
fp32 partials + attn_merge_lse), against the oracle on scaled-down versions of the Ulysses and
Ring workloads."""
import pytest
import torch

import oracle
import tensor_head_attention_amd as T
import tha_workloads as W
from parity import DEV, check_lse, check_out, say, to_dev

pytestmark = pytest.mark.gpu


def test_ulysses_share_helper():
    P, S, H, D, grp = 4, 1024, 16, 128, 2
    say(f"ulysses_share P{P} S{S} H{H} group {grp}")
    sh = W.shard_inputs(P, 1, S, H, D, torch.bfloat16, seed=91)
    dev = {n: [t.to(DEV) for t in sh[n]] for n in ("q", "k", "v")}
    out, lse = T.ulysses_share(dev["q"], dev["k"], dev["v"], grp, causal=True)
    torch.cuda.synchronize()
    q, k, v = (oracle.shard_permute(sh[n], grp) for n in ("q", "k", "v"))
    ref, ref_lse = oracle.attention(q, k, v, causal=True)
    check_out(out, ref, torch.bfloat16)
    check_lse(lse, ref_lse, torch.bfloat16)


@pytest.mark.parametrize("fused", [True, False])
def test_ring_share_helper(fused):
    P, Sc, H, D, qc = 4, 256, 4, 128, 3
    say(f"ring_share P{P} Sc{Sc} H{H} q chunk {qc} fused={fused}")
    g = W.generator(92)
    q = W.randn((1, Sc, H, D), g, torch.bfloat16)
    k = W.randn((1, P * Sc, H, D), g, torch.bfloat16)
    v = W.randn((1, P * Sc, H, D), g, torch.bfloat16)
    qd, kd, vd = to_dev(q, k, v)
    kc = [kd[:, t * Sc:(t + 1) * Sc].contiguous() for t in range(P)]
    vc = [vd[:, t * Sc:(t + 1) * Sc].contiguous() for t in range(P)]
    out, lse = T.ring_share(qd, kc, vc, q_pos0=qc * Sc, k_pos0s=[t * Sc for t in range(P)], causal=True,
                            fused=fused, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attention(q, k, v, causal=True, q_pos0=qc * Sc, k_pos0=0)
    check_out(out, ref, torch.bfloat16)
    check_lse(lse, ref_lse, torch.bfloat16)

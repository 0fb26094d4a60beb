"""The library allocates nothing and enqueues only kernels on the caller's stream, so its calls can
be captured in a HIP graph.  A whole fused Ring pass (lse reset, 8 accumulate calls, the final cast
by a one-part merge) and a Ulysses step (3 permutes + attention) are captured once and replayed
several times, with eager work and synchronisations between replays; every replay must equal
the eager result bit for bit."""
import pytest
import torch

import tensor_head_attention_amd as T
import tha_workloads as W
from parity import DEV, say, to_dev

pytestmark = pytest.mark.gpu


def test_ring_pass_graph_replays():
    P, Sc, H, D = 8, 256, 2, 128
    say(f"graph: fused Ring pass P{P} Sc{Sc} H{H}")
    g = W.generator(61)
    q = W.randn((1, Sc, H, D), g, torch.bfloat16)
    k = W.randn((1, P * Sc, H, D), g, torch.bfloat16)
    v = W.randn((1, P * Sc, H, D), g, torch.bfloat16)
    qd, kd, vd = to_dev(q, k, v)
    qp = (P - 1) * Sc
    o_run = torch.empty((1, Sc, H, D), dtype=torch.float32, device=DEV)
    l_run = torch.empty((1, H, Sc), dtype=torch.float32, device=DEV)
    out = torch.empty((1, Sc, H, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((1, H, Sc), dtype=torch.float32, device=DEV)

    def ring_pass():
        l_run.fill_(float("-inf"))
        for t in range(P):
            T.attn_fwd_ex(qd, kd[:, t * Sc:(t + 1) * Sc], vd[:, t * Sc:(t + 1) * Sc], causal=True, q_pos0=qp,
                          k_pos0=t * Sc, out=o_run, lse=l_run, accumulate=True)
        T.attn_merge_lse([o_run], [l_run], out=out, lse_out=lse)

    ring_pass()
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up on a side stream before capture
        ring_pass()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ring_pass()
    for rep in range(3):
        out.zero_()
        lse.zero_()
        o_run.normal_()  # eager work between replays: the replay must not depend on stale state
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"replay {rep}"


def test_ulysses_step_graph_replays():
    P, Sl, Hs, D = 4, 128, 8, 128
    say(f"graph: Ulysses step P{P} Sl{Sl} H{Hs}")
    inp = W.shard_inputs(P, 1, P * Sl, Hs, D, torch.bfloat16, seed=62)
    shards = {n: [t.to(DEV) for t in inp[n]] for n in ("q", "k", "v")}
    grouped = {n: torch.empty((1, P * Sl, Hs // P, D), dtype=torch.bfloat16, device=DEV) for n in shards}
    out = torch.empty((1, P * Sl, Hs // P, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((1, Hs // P, P * Sl), dtype=torch.float32, device=DEV)

    def step():
        for n in ("q", "k", "v"):
            T.shard_permute(shards[n], 1, out=grouped[n])
        T.attn_fwd(grouped["q"], grouped["k"], grouped["v"], causal=True, out=out, lse=lse)

    step()
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        for t in grouped.values():
            t.zero_()
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"replay {rep}"

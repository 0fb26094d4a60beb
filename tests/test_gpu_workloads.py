"""The five workloads at their full sizes, in the launch configuration bench.py
times, checked against the fp64 oracle: fully where the oracle finishes in
seconds, else on sampled rows (first/last rows, tile boundaries, padded rows,
seeded random rows), plus properties that hold at any size."""
import math

import pytest
import torch

import oracle
import tensor_head_attention_amd as T
import tha_workloads as W
from parity import DEV, check_lse, check_out, say, to_dev

pytestmark = pytest.mark.gpu


def _sample_rows(B, S, extra, seed, n_rand=24):
    g = W.generator(seed)
    base = [0, 1, 31, 32, 63, 64, 127, 128, 129, S // 2, S - 129, S - 128, S - 2, S - 1] + list(extra)
    rows = set()
    for b in range(B):
        for i in base:
            if 0 <= i < S:
                rows.add(b * S + i)
    rows.update(torch.randint(0, B * S, (n_rand,), generator=g).tolist())
    return torch.tensor(sorted(rows), dtype=torch.int64)


def _check_rows(out_dev, lse_dev, rows, ref, ref_lse, B, S, H, dtype):
    o = out_dev.reshape(B * S, H, -1)[rows.to(out_dev.device)]
    l = lse_dev.permute(0, 2, 1).reshape(B * S, H)[rows.to(lse_dev.device)]
    check_out(o, ref, dtype)
    check_lse(l, ref_lse, dtype)


def test_workload1_tiny_fp32_full():
    say("workload 1: tiny fp32 MHA")
    inp, p = W.workload_inputs(1)
    q, k, v = inp["q"], inp["k"], inp["v"]
    ref, ref_lse = oracle.attention(q, k, v, causal=True)
    qd, kd, vd = to_dev(q, k, v)
    out, lse = T.attn_fwd(qd, kd, vd, causal=True)
    per = [T.attn_fwd(qd[:, :, h:h + 1].contiguous(), kd[:, :, h:h + 1].contiguous(), vd[:, :, h:h + 1].contiguous(),
                      causal=True)[0] for h in range(p["H"])]
    torch.cuda.synchronize()
    check_out(out, ref, torch.float32)
    check_lse(lse, ref_lse, torch.float32)
    assert torch.equal(torch.cat(per, dim=2), out)


def test_workload2_causal_4k_full():
    say("workload 2: causal S4096 H8 D128 bf16, whole output")
    inp, p = W.workload_inputs(2)
    q, k, v = inp["q"], inp["k"], inp["v"]
    assert max(t.abs().max().item() for t in (q, k, v)) < 8  # bf16 output rounding stays < 2e-2
    ref, ref_lse = oracle.attention(q, k, v, causal=True)
    qd, kd, vd = to_dev(q, k, v)
    out, lse = T.attn_fwd(qd, kd, vd, causal=True)
    torch.cuda.synchronize()
    check_out(out, ref, torch.bfloat16)
    check_lse(lse, ref_lse, torch.bfloat16)


def test_workload3_ulysses_share():
    say("workload 3: 8 shards [4096,64,128] -> [32768,8,128]; causal attention S32768")
    inp, p = W.workload_inputs(3)
    P, S, H, D = p["P"], p["S"], p["H"], p["D"]
    dev = {n: to_dev(*inp[n]) for n in ("q", "k", "v")}
    grouped = {}
    for n in ("q", "k", "v"):
        got = T.shard_permute(dev[n], p["group"])
        torch.cuda.synchronize()
        ref = oracle.shard_permute(inp[n], p["group"])
        assert torch.equal(got.cpu().view(torch.int16), ref.view(torch.int16)), n
        grouped[n] = (got, ref)
    # another head group, bit-exact too
    g7 = T.shard_permute(dev["q"], 7)
    torch.cuda.synchronize()
    assert torch.equal(g7.cpu().view(torch.int16), oracle.shard_permute(inp["q"], 7).view(torch.int16))
    del g7, dev
    qd, kd, vd = (grouped[n][0] for n in ("q", "k", "v"))
    q, k, v = (grouped[n][1] for n in ("q", "k", "v"))
    out, lse = T.attn_fwd(qd, kd, vd, causal=True)  # the wide kernel, as timed
    torch.cuda.synchronize()
    # the other head-size-128 kernel gives the same bits
    out_n, lse_n = T.attn_fwd(qd, kd, vd, causal=True, kernel="narrow")
    torch.cuda.synchronize()
    assert torch.equal(out_n, out) and torch.equal(lse_n, lse)
    del out_n, lse_n
    Hl = H // P
    rows = _sample_rows(1, S, [4095, 4096, 8191, 8192, 16383, 16384, 28672], seed=33)
    ref, ref_lse = oracle.attention(q, k, v, causal=True, rows=rows)
    _check_rows(out, lse, rows, ref, ref_lse, 1, S, Hl, torch.bfloat16)
    # any-size properties: finite everywhere; causal row 0 equals V[0]; lse of row 0 = scale * q0.k0
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    assert torch.equal(out[0, 0], vd[0, 0])
    s00 = (q[0, 0].double() * k[0, 0].double()).sum(-1) / math.sqrt(D)
    assert torch.allclose(lse[0, :, 0].cpu().double(), s00, atol=1e-4, rtol=0)


def test_workload4_ring_share():
    say("workload 4: Q chunk 7 of 8 against 8 KV chunks of 4096, fp32 partials, 8-way merge")
    inp, p = W.workload_inputs(4)
    P, S, H, D = p["P"], p["S"], p["H"], p["D"]
    Sc = S // P
    qp = p["q_chunk"] * Sc
    q, k, v = inp["q"], inp["k"], inp["v"]
    qd, kd, vd = to_dev(q, k, v)
    kc = [kd[:, t * Sc:(t + 1) * Sc].contiguous() for t in range(P)]
    vc = [vd[:, t * Sc:(t + 1) * Sc].contiguous() for t in range(P)]
    parts = [T.attn_fwd(qd, kc[t], vc[t], causal=True, q_pos0=qp, k_pos0=t * Sc, out_dtype=torch.float32)
             for t in range(P)]
    out, lse = T.attn_merge_lse([o for o, _ in parts], [l for _, l in parts], out_dtype=torch.bfloat16)
    # pairwise streaming form
    o_run, l_run = parts[0][0].clone(), parts[0][1].clone()
    for t in range(1, P):
        T.attn_merge_lse([o_run, parts[t][0]], [l_run, parts[t][1]], out=o_run, lse_out=l_run)
    torch.cuda.synchronize()
    rows = _sample_rows(1, Sc, [], seed=44, n_rand=40)
    ref, ref_lse = oracle.attention(q, k, v, causal=True, q_pos0=qp, k_pos0=0, rows=rows)
    _check_rows(out, lse, rows, ref, ref_lse, 1, Sc, H, torch.bfloat16)
    _check_rows(o_run, l_run, rows, ref, ref_lse, 1, Sc, H, torch.bfloat16)
    assert torch.isfinite(out).all()


def test_workload5_padded_batch():
    say("workload 5: B4 S8192 H32 D128 bf16, key padding, non-causal")
    inp, p = W.workload_inputs(5)
    B, S, H, D = p["B"], p["S"], p["H"], p["D"]
    q, k, v, kv = inp["q"], inp["k"], inp["v"], inp["kv_len"]
    qd, kd, vd, kvd = to_dev(q, k, v, kv)
    out, lse = T.attn_fwd(qd, kd, vd, kv_len=kvd)
    torch.cuda.synchronize()
    out_n, lse_n = T.attn_fwd(qd, kd, vd, kv_len=kvd, kernel="narrow")
    torch.cuda.synchronize()
    assert torch.equal(out_n, out) and torch.equal(lse_n, lse)
    del out_n, lse_n
    lens = kv.tolist()
    extra = []
    for L in lens:
        extra += [L - 1, L, L + 1]  # last valid row and the first padded query rows
    rows = _sample_rows(B, S, extra, seed=55, n_rand=16)
    ref, ref_lse = oracle.attention(q, k, v, kv_len=kv, rows=rows)
    _check_rows(out, lse, rows, ref, ref_lse, B, S, H, torch.bfloat16)
    assert torch.isfinite(out).all()

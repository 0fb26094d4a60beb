"""The five workloads at their full sizes, in the launch configuration bench.py
times, checked against the fp64 oracle over the WHOLE output and lse tensors.
Where the oracle takes minutes for a workload it runs per head (Ulysses share)
or per sequence (padded batch), one test each, and a last test checks the
whole-tensor max-abs and rel-L2 from the per-slice sums.  Sampled rows (first/
last rows, tile boundaries, padded rows, seeded random rows) run first as a
quick pre-check, with properties that hold at any size."""
import math

import pytest
import torch

import oracle
import tensor_head_attention_amd as T
import tha_workloads as W
from parity import DEV, WholeTensor, check_lse, check_out, host_threads, say, to_dev

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


@pytest.mark.parametrize("kernel", [None, "split", "narrow"])
def test_workload2_causal_4k_full(kernel):
    """The automatic choice (the 64-row split form at this grid, as timed) and the two other forms
    the grid could take, over the whole output."""
    say(f"workload 2: causal S4096 H8 D128 bf16, whole output, kernel={kernel}")
    inp, p = W.workload_inputs(2)
    q, k, v = inp["q"], inp["k"], inp["v"]
    assert max(t.abs().max().item() for t in (q, k, v)) < 8  # bf16 output rounding stays < 2e-2
    ref, ref_lse = oracle.attention(q, k, v, causal=True, nthreads=host_threads())
    qd, kd, vd = to_dev(q, k, v)
    out, lse = T.attn_fwd(qd, kd, vd, causal=True, kernel=kernel)
    torch.cuda.synchronize()
    check_out(out, ref, torch.bfloat16)
    check_lse(lse, ref_lse, torch.bfloat16)


# ---- workload 3: Ulysses share ------------------------------------------------------------------

@pytest.fixture(scope="module")
def w3():
    """8 sequence shards of Q, K, V permuted to head group 0 on the device in one shard_permute_n
    launch (as bench.py does), head group 7 of Q by shard_permute, and
    the causal attention of that group; the host copies are the oracle's own permutes."""
    say("workload 3: 8 shards [4096,64,128] -> [32768,8,128]; causal attention S32768")
    inp, p = W.workload_inputs(3)
    dev = {n: to_dev(*inp[n]) for n in ("q", "k", "v")}
    grouped = dict(zip(("q", "k", "v"), T.shard_permute_n([dev[n] for n in ("q", "k", "v")], p["group"])))
    g7 = T.shard_permute(dev["q"], 7)
    out, lse = T.attn_fwd(grouped["q"], grouped["k"], grouped["v"], causal=True)  # the wide kernel, as timed
    torch.cuda.synchronize()
    host = {n: oracle.shard_permute(inp[n], p["group"]) for n in ("q", "k", "v")}
    st = dict(p=p, grouped=grouped, host=host, out=out, lse=lse,
              g7=(g7, oracle.shard_permute(inp["q"], 7)), whole=WholeTensor("workload 3", torch.bfloat16))
    del dev, inp  # the 3 x 512 MiB of shards, on both sides
    yield st


def test_workload3_permute_bit_exact(w3):
    for n in ("q", "k", "v"):
        assert torch.equal(w3["grouped"][n].cpu().view(torch.int16), w3["host"][n].view(torch.int16)), n
    got, ref = w3["g7"]  # another head group
    assert torch.equal(got.cpu().view(torch.int16), ref.view(torch.int16))


def test_workload3_sampled_rows_and_properties(w3):
    p = w3["p"]
    P, S, H, D = p["P"], p["S"], p["H"], p["D"]
    qd, kd, vd = (w3["grouped"][n] for n in ("q", "k", "v"))
    q, k, v = (w3["host"][n] for n in ("q", "k", "v"))
    out, lse = w3["out"], w3["lse"]
    # the other head-size-128 kernel gives the same bits
    out_n, lse_n = T.attn_fwd(qd, kd, vd, causal=True, kernel="narrow")
    torch.cuda.synchronize()
    assert torch.equal(out_n, out) and torch.equal(lse_n, lse)
    del out_n, lse_n
    rows = _sample_rows(1, S, [4095, 4096, 8191, 8192, 16383, 16384, 28672], seed=33)
    ref, ref_lse = oracle.attention(q, k, v, causal=True, rows=rows, nthreads=host_threads())
    _check_rows(out, lse, rows, ref, ref_lse, 1, S, H // P, torch.bfloat16)
    # any-size properties: finite everywhere; causal row 0 equals V[0]; lse of row 0 = scale * q0.k0
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    assert torch.equal(out[0, 0], vd[0, 0])
    s00 = (q[0, 0].double() * k[0, 0].double()).sum(-1) / math.sqrt(D)
    assert torch.allclose(lse[0, :, 0].cpu().double(), s00, atol=1e-4, rtol=0)


W3_HEADS = list(range(8))


def _w3_head(w3, h):
    q, k, v = (w3["host"][n][:, :, h:h + 1].contiguous() for n in ("q", "k", "v"))
    ref, ref_lse = oracle.attention(q, k, v, causal=True, nthreads=host_threads())
    w3["whole"].add(h, w3["out"][:, :, h:h + 1], ref, w3["lse"][:, h:h + 1], ref_lse)


@pytest.mark.parametrize("h", W3_HEADS)
def test_workload3_full_head(w3, h):
    say(f"workload 3: head {h}, all 32768 rows against the oracle")
    _w3_head(w3, h)


def test_workload3_whole_output(w3):
    for h in w3["whole"].missing(W3_HEADS):  # heads not compared above (a test run on its own)
        _w3_head(w3, h)
    w3["whole"].finish(W3_HEADS)


# ---- workload 4: Ring share ---------------------------------------------------------------------

@pytest.fixture(scope="module")
def w4():
    """Q chunk 7 of 8 against 8 KV chunks of 4096 keys: the oracle's unchunked result over all
    4096 x 8 rows, and the device inputs."""
    say("workload 4: Q chunk 7 of 8 against 8 KV chunks of 4096; unchunked oracle, all rows")
    inp, p = W.workload_inputs(4)
    P, S = p["P"], p["S"]
    Sc = S // P
    qp = p["q_chunk"] * Sc
    q, k, v = inp["q"], inp["k"], inp["v"]
    ref, ref_lse = oracle.attention(q, k, v, causal=True, q_pos0=qp, k_pos0=0, nthreads=host_threads())
    qd, kd, vd = to_dev(q, k, v)
    kc = [kd[:, t * Sc:(t + 1) * Sc].contiguous() for t in range(P)]
    vc = [vd[:, t * Sc:(t + 1) * Sc].contiguous() for t in range(P)]
    yield dict(p=p, Sc=Sc, qp=qp, qd=qd, kc=kc, vc=vc, ref=ref, ref_lse=ref_lse)


def test_workload4_partials_and_merge_full(w4):
    """fp32 partials of the 8 chunk calls, one 8-way attn_merge_lse to bf16 (the bench's Ring share),
    and the pairwise streaming form (running result merged in place with each new part)."""
    P, Sc, qp = w4["p"]["P"], w4["Sc"], w4["qp"]
    parts = [T.attn_fwd(w4["qd"], w4["kc"][t], w4["vc"][t], causal=True, q_pos0=qp, k_pos0=t * Sc,
                        out_dtype=torch.float32) for t in range(P)]
    out, lse = T.attn_merge_lse([o for o, _ in parts], [l for _, l in parts], out_dtype=torch.bfloat16)
    o_run, l_run = parts[0][0].clone(), parts[0][1].clone()
    for t in range(1, P):
        T.attn_merge_lse([o_run, parts[t][0]], [l_run, parts[t][1]], out=o_run, lse_out=l_run)
    torch.cuda.synchronize()
    say("  8-way merge:")
    check_out(out, w4["ref"], torch.bfloat16)
    check_lse(lse, w4["ref_lse"], torch.bfloat16)
    say("  pairwise streaming merge:")
    check_out(o_run, w4["ref"], torch.bfloat16)
    check_lse(l_run, w4["ref_lse"], torch.bfloat16)
    assert torch.isfinite(out).all()


def test_workload4_fused_ring_full(w4):
    """The fused Ring pass: each chunk call merges into the running fp32 (o, lse) in its epilogue
    (attn_fwd_ex with accumulate), then a one-part attn_merge_lse casts the result to bf16."""
    P, Sc, qp = w4["p"]["P"], w4["Sc"], w4["qp"]
    out, lse = T.ring_share(w4["qd"], w4["kc"], w4["vc"], q_pos0=qp, k_pos0s=[t * Sc for t in range(P)],
                            fused=True, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    check_out(out, w4["ref"], torch.bfloat16)
    check_lse(lse, w4["ref_lse"], torch.bfloat16)


# ---- workload 5: padded batch -------------------------------------------------------------------

@pytest.fixture(scope="module")
def w5():
    say("workload 5: B4 S8192 H32 D128 bf16, key padding, non-causal")
    inp, p = W.workload_inputs(5)
    q, k, v, kv = inp["q"], inp["k"], inp["v"], inp["kv_len"]
    qd, kd, vd, kvd = to_dev(q, k, v, kv)
    out, lse = T.attn_fwd(qd, kd, vd, kv_len=kvd)
    torch.cuda.synchronize()
    yield dict(p=p, inp=inp, dev=(qd, kd, vd, kvd), out=out, lse=lse,
               whole=WholeTensor("workload 5", torch.bfloat16))


def test_workload5_sampled_rows(w5):
    p, inp = w5["p"], w5["inp"]
    B, S, H = p["B"], p["S"], p["H"]
    out, lse = w5["out"], w5["lse"]
    qd, kd, vd, kvd = w5["dev"]
    out_n, lse_n = T.attn_fwd(qd, kd, vd, kv_len=kvd, kernel="narrow")
    torch.cuda.synchronize()
    assert torch.equal(out_n, out) and torch.equal(lse_n, lse)
    del out_n, lse_n
    extra = []
    for L in inp["kv_len"].tolist():
        extra += [L - 1, L, L + 1]  # last valid row and the first padded query rows
    rows = _sample_rows(B, S, extra, seed=55, n_rand=16)
    ref, ref_lse = oracle.attention(inp["q"], inp["k"], inp["v"], kv_len=inp["kv_len"], rows=rows,
                                    nthreads=host_threads())
    _check_rows(out, lse, rows, ref, ref_lse, B, S, H, torch.bfloat16)
    assert torch.isfinite(out).all()


W5_SEQS = list(range(4))


def _w5_seq(w5, b):
    inp = w5["inp"]
    q, k, v = (inp[n][b:b + 1].contiguous() for n in ("q", "k", "v"))
    ref, ref_lse = oracle.attention(q, k, v, kv_len=inp["kv_len"][b:b + 1], nthreads=host_threads())
    w5["whole"].add(b, w5["out"][b:b + 1], ref, w5["lse"][b:b + 1], ref_lse)


@pytest.mark.parametrize("b", W5_SEQS)
def test_workload5_full_sequence(w5, b):
    say(f"workload 5: sequence {b} (kv_len {int(w5['inp']['kv_len'][b])}), all 8192 rows x 32 heads")
    _w5_seq(w5, b)


def test_workload5_whole_output(w5):
    for b in w5["whole"].missing(W5_SEQS):
        _w5_seq(w5, b)
    w5["whole"].finish(W5_SEQS)

"""GPU parity of shard_permute / shard_unpermute (bit-exact) and attn_merge_lse
(against the fp64 oracle merge) through the C ABI."""
import pytest
import torch

import oracle
import tensor_head_attention_amd as T
import tha_workloads as W
from parity import DEV, check_lse, check_out, say, to_dev

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.contiguous().view(torch.uint8)


@pytest.mark.parametrize("P,B,S,H,D,dtype", [
    (8, 1, 256, 64, 128, torch.bfloat16),
    (4, 2, 40, 8, 64, torch.bfloat16),
    (2, 1, 6, 2, 3, torch.bfloat16),      # 6-byte runs: element path
    (3, 2, 9, 3, 5, torch.float32),       # odd sizes
    (4, 1, 16, 8, 7, torch.int8),         # 1-byte elements
    (2, 3, 8, 4, 2, torch.float64),       # 8-byte elements
    (1, 1, 5, 2, 16, torch.bfloat16),     # P = 1 is a plain copy
    (2, 2, 14, 4, 32, torch.bfloat16),    # odd shard length (7 tokens): plain visiting order
    (3, 2, 18, 6, 24, torch.bfloat16),    # 96-byte runs (6 vectors, not a power of two), even/odd order
    (16, 2, 64, 32, 16, torch.float32),   # 16 shards
    (64, 1, 128, 64, 8, torch.bfloat16),  # the most shards a call takes; 16-byte runs, 2 tokens a shard
])
def test_permute_and_unpermute_bit_exact(P, B, S, H, D, dtype):
    say(f"permute P{P} B{B} S{S} H{H} D{D} {dtype}")
    g = W.generator(P * 100 + S)
    if dtype in (torch.int8,):
        shards = [torch.randint(-128, 128, (B, S // P, H, D), generator=g, dtype=torch.int8) for _ in range(P)]
    else:
        shards = [W.randn((B, S // P, H, D), g, torch.float32).to(dtype) for _ in range(P)]
    sd = to_dev(*shards)
    outs = []
    for grp in range(P):
        ref = oracle.shard_permute(shards, grp)
        got = T.shard_permute(sd, grp)
        torch.cuda.synchronize()
        assert torch.equal(_bits(got.cpu()), _bits(ref)), f"group {grp}"
        outs.append(got)
    back = [torch.full_like(s, 0) for s in sd]
    for grp in range(P):
        T.shard_unpermute(outs[grp], grp, back)
    torch.cuda.synchronize()
    for a, b in zip(back, shards):
        assert torch.equal(_bits(a.cpu()), _bits(b))
    ref_back = oracle.shard_unpermute([o.cpu() for o in outs])
    for a, b in zip(back, ref_back):
        assert torch.equal(_bits(a.cpu()), _bits(b))


@pytest.mark.parametrize("n,P,B,S,H,D,dtype", [
    (3, 8, 1, 256, 64, 128, torch.bfloat16),   # Q, K, V of a Ulysses step
    (2, 4, 2, 40, 8, 64, torch.bfloat16),
    (4, 3, 2, 9, 3, 5, torch.float32),         # element path, the most tensors a call takes
    (1, 2, 1, 6, 2, 3, torch.bfloat16),
    (3, 64, 1, 128, 64, 8, torch.bfloat16),    # 64 shards of 2 tokens
    (2, 16, 2, 64, 32, 16, torch.float32),
])
def test_permute_n_equals_separate_calls(n, P, B, S, H, D, dtype):
    """shard_permute_n / shard_unpermute_n over n tensors in one launch give the bits of n single
    calls and of the oracle, every head group."""
    say(f"permute_n n{n} P{P} B{B} S{S} H{H} D{D} {dtype}")
    g = W.generator(n * 1000 + P * 10 + S)
    sets = [[W.randn((B, S // P, H, D), g, torch.float32).to(dtype) for _ in range(P)] for _ in range(n)]
    dsets = [to_dev(*ss) for ss in sets]
    for grp in sorted({0, P // 2, P - 1}):
        outs = T.shard_permute_n(dsets, grp)
        torch.cuda.synchronize()
        for t in range(n):
            assert torch.equal(_bits(outs[t].cpu()), _bits(oracle.shard_permute(sets[t], grp))), (grp, t)
        back = [[torch.zeros_like(x) for x in ss] for ss in dsets]
        T.shard_unpermute_n(outs, grp, back)
        ref_back = [[torch.zeros_like(x) for x in ss] for ss in dsets]
        for t in range(n):
            T.shard_unpermute(outs[t], grp, ref_back[t])
        torch.cuda.synchronize()
        for t in range(n):
            for a, b in zip(back[t], ref_back[t]):
                assert torch.equal(_bits(a), _bits(b))


def test_permute_unaligned_pointer_uses_element_path():
    P, B, S, H, D = 2, 1, 8, 4, 8
    g = W.generator(5)
    shards = [W.randn((B, S // P, H, D), g, torch.bfloat16) for _ in range(P)]
    big = [torch.empty(B * (S // P) * H * D + 1, dtype=torch.bfloat16, device=DEV) for _ in range(P)]
    views = []
    for bg, s in zip(big, shards):
        vw = bg[1:].view(B, S // P, H, D)  # 2-byte offset: not 16-byte aligned
        vw.copy_(s.to(DEV))
        views.append(vw)
    got = T.shard_permute(views, 1)
    torch.cuda.synchronize()
    assert torch.equal(_bits(got.cpu()), _bits(oracle.shard_permute(shards, 1)))


def _parts(n, B, S, H, D, seed, part_dtype=torch.float32, spread=80.0):
    g = W.generator(seed)
    os_ = [W.randn((B, S, H, D), g, torch.float32).to(part_dtype) for _ in range(n)]
    ls_ = [W.randn((B, H, S), g, torch.float32) * spread for _ in range(n)]
    # rows with some parts empty, and rows where every part is empty
    ls_[0][:, :, ::7] = float("-inf")
    for l in ls_:
        l[:, :, 3::11] = float("-inf")
    return os_, ls_


@pytest.mark.parametrize("n,B,S,H,D", [(1, 1, 50, 2, 128), (2, 2, 33, 3, 128), (8, 1, 100, 8, 128),
                                       (5, 1, 17, 2, 64), (3, 2, 9, 2, 6), (64, 1, 4, 1, 8), (9, 1, 5, 2, 12),
                                       (2, 1, 3, 2, 1024), (2, 1, 3, 1, 1028)])
@pytest.mark.parametrize("part_dt,out_dt", [(torch.float32, torch.bfloat16), (torch.float32, torch.float32),
                                            (torch.bfloat16, torch.bfloat16)])
def test_merge_matches_oracle(n, B, S, H, D, part_dt, out_dt):
    say(f"merge n{n} B{B} S{S} H{H} D{D} {part_dt}->{out_dt}")
    os_, ls_ = _parts(n, B, S, H, D, seed=n * 31 + S, part_dtype=part_dt)
    ref, ref_lse = oracle.merge_lse([o.double() for o in os_], [l.double() for l in ls_])
    od, ld = to_dev(*os_), to_dev(*ls_)
    out, lse = T.attn_merge_lse(od, ld, out_dtype=out_dt)
    torch.cuda.synchronize()
    tol_dt = torch.bfloat16 if torch.bfloat16 in (part_dt, out_dt) else torch.float32
    check_out(out, ref, tol_dt)
    check_lse(lse, ref_lse, torch.float32)


def test_merge_in_place_streaming():
    """Pairwise streaming form: o_run, lse_run updated in place with each new part
    (o_out aliases o_parts[0], lse_out aliases lse_parts[0])."""
    n, B, S, H, D = 6, 1, 300, 4, 128
    os_, ls_ = _parts(n, B, S, H, D, seed=77)
    ref, ref_lse = oracle.merge_lse([o.double() for o in os_], [l.double() for l in ls_])
    od, ld = to_dev(*os_), to_dev(*ls_)
    o_run, l_run = od[0].clone(), ld[0].clone()
    for k in range(1, n):
        T.attn_merge_lse([o_run, od[k]], [l_run, ld[k]], out=o_run, lse_out=l_run)
    torch.cuda.synchronize()
    check_out(o_run, ref, torch.float32)
    check_lse(l_run, ref_lse, torch.float32)


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("D", [128, 22])  # the vector and the scalar kernel
def test_merge_in_place_any_part(dt, D):
    """o_out and lse_out may be any part (here the last of three), not only the first."""
    n, B, S, H = 3, 2, 70, 4
    os_, ls_ = _parts(n, B, S, H, D, seed=78, part_dtype=dt)
    ref, ref_lse = oracle.merge_lse([o.double() for o in os_], [l.double() for l in ls_])
    od, ld = to_dev(*os_), to_dev(*ls_)
    expect, expect_lse = T.attn_merge_lse(od, ld, out_dtype=dt)
    T.attn_merge_lse(od, ld, out=od[-1], lse_out=ld[-1])
    torch.cuda.synchronize()
    assert torch.equal(od[-1], expect) and torch.equal(ld[-1], expect_lse)
    check_out(od[-1], ref, dt)
    check_lse(ld[-1], ref_lse, torch.float32)


@pytest.mark.parametrize("n", [9, 17, 64])
@pytest.mark.parametrize("D", [512, 1024])
def test_merge_in_place_rows_across_wavefronts(n, D):
    """Rows of 512 or 1024 elements span two or four wavefronts of the vector kernel, and parts
    beyond the eighth are weighted after the first barrier: with lse_out (and o_out) equal to the
    last part, every wavefront of a row must read that part's lse before the row's lse store."""
    B, S, H = 1, 40, 2
    say(f"merge in place n{n} D{D} (rows across wavefronts)")
    # lse values within a few units of each other: the merged lse exceeds every part's by about
    # log(n), so a weight read after the store (exp(lse_out - M) for the last part) would be off
    # by a factor of about n
    os_, ls_ = _parts(n, B, S, H, D, seed=n * 7 + D, spread=1.0)
    ref, ref_lse = oracle.merge_lse([o.double() for o in os_], [l.double() for l in ls_])
    od, ld = to_dev(*os_), to_dev(*ls_)
    expect, expect_lse = T.attn_merge_lse(od, ld, out_dtype=torch.float32)
    T.attn_merge_lse(od, ld, out=od[-1], lse_out=ld[-1])
    torch.cuda.synchronize()
    assert torch.equal(od[-1], expect) and torch.equal(ld[-1], expect_lse)
    check_out(od[-1], ref, torch.float32)
    check_lse(ld[-1], ref_lse, torch.float32)

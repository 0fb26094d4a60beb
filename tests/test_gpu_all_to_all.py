"""GPU parity of shard_all_to_all (the all-to-all local layout with general scatter and gather
dims) against the oracle, bit-exact, through the C ABI: the Ulysses forward and return cases,
the sequence-first layout, packed QKV, dims at both ends of an 8-dim shape, 1/2/4/8-byte
elements, 64 ranks, unaligned pointers (element path), and the Ulysses share at full size."""
import pytest
import torch

import oracle
import tensor_head_attention_amd as T
import tha_workloads as W
from parity import DEV, say, to_dev

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.contiguous().view(torch.uint8)


def _inputs(shape, P, dtype, seed):
    g = W.generator(seed)
    if dtype in (torch.int8, torch.int16):
        return [torch.randint(-100, 100, shape, generator=g, dtype=dtype) for _ in range(P)]
    return [W.randn(shape, g, torch.float32).to(dtype) for _ in range(P)]


# (shape per rank, P, scatter dim, gather dim, dtype)
CASES = [
    ((2, 12, 8, 16), 4, 2, 1, torch.bfloat16),        # Ulysses forward [B, S/P, H, D]
    ((2, 48, 2, 16), 4, 1, 2, torch.bfloat16),        # Ulysses return [B, S, H/P, D]
    ((12, 2, 6, 8), 3, 2, 0, torch.float32),          # sequence-first [S/P, B, H, D]
    ((2, 6, 3, 8, 8), 2, 3, 1, torch.bfloat16),       # packed QKV [B, S/P, 3, H, D]
    ((4, 6, 2), 2, 0, 1, torch.int8),                 # 1-byte elements, scatter before gather
    ((5, 2, 4), 4, 2, 0, torch.float64),              # 8-byte elements, element path
    ((2, 2, 2, 2, 2, 2, 2, 16), 2, 7, 0, torch.int16),  # 8 dims, the special dims at both ends
    ((1, 64, 64, 8), 64, 2, 1, torch.bfloat16),       # the most ranks a call takes
    ((1, 128, 1, 8), 64, 1, 2, torch.bfloat16),
    ((3, 10, 6, 5), 2, 2, 1, torch.float32),          # 12-byte runs: element path
    ((2, 8, 4, 3), 4, 1, 2, torch.bfloat16),          # 24-byte runs: element path
    ((8, 4), 8, 0, 1, torch.bfloat16),
    ((4, 8), 8, 1, 0, torch.bfloat16),
]


def _id(c):
    shape, P, sd, gd, dt = c
    return f"{'x'.join(map(str, shape))}_P{P}_s{sd}_g{gd}_{str(dt).split('.')[-1]}"


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_all_to_all_bit_exact(case):
    shape, P, sd, gd, dt = case
    say(f"all_to_all {_id(case)}")
    ins = _inputs(shape, P, dt, seed=P * 13 + len(shape) + sd)
    dev = to_dev(*ins)
    for r in sorted({0, P // 2, P - 1}):
        got = T.shard_all_to_all(dev, r, sd, gd)
        torch.cuda.synchronize()
        ref = oracle.all_to_all(ins, r, sd, gd)
        assert got.shape == ref.shape
        assert torch.equal(_bits(got.cpu()), _bits(ref)), f"rank {r}"


@pytest.mark.parametrize("case", [c for c in CASES if c[1] <= 8], ids=_id)
def test_all_to_all_round_trip_on_device(case):
    """The all-to-all with the dims swapped, applied to every rank's result, returns each rank's
    own tensor."""
    shape, P, sd, gd, dt = case
    ins = _inputs(shape, P, dt, seed=P * 17 + len(shape) + gd)
    dev = to_dev(*ins)
    mid = [T.shard_all_to_all(dev, r, sd, gd) for r in range(P)]
    for r in range(P):
        back = T.shard_all_to_all(mid, r, gd, sd)
        torch.cuda.synchronize()
        assert torch.equal(_bits(back.cpu()), _bits(ins[r])), f"rank {r}"


def test_all_to_all_ulysses_case_equals_shard_permute():
    """Scatter heads / gather sequence on [B, S/P, H, D] shards gives shard_permute's bits."""
    shape, P = (2, 12, 8, 16), 4
    ins = to_dev(*_inputs(shape, P, torch.bfloat16, seed=3))
    for r in range(P):
        a = T.shard_all_to_all(ins, r, 2, 1)
        b = T.shard_permute(ins, r)
        torch.cuda.synchronize()
        assert torch.equal(_bits(a), _bits(b))


def test_all_to_all_unaligned_pointers_use_element_path():
    shape, P = (2, 12, 8, 16), 4
    ins = _inputs(shape, P, torch.bfloat16, seed=9)
    n = 2 * 12 * 8 * 16
    big = [torch.empty(n + 1, dtype=torch.bfloat16, device=DEV) for _ in range(P)]
    views = []
    for bg, x in zip(big, ins):
        vw = bg[1:].view(shape)  # 2-byte offset: not 16-byte aligned
        vw.copy_(x.to(DEV))
        views.append(vw)
    got = T.shard_all_to_all(views, 1, 2, 1)
    torch.cuda.synchronize()
    assert torch.equal(_bits(got.cpu()), _bits(oracle.all_to_all(ins, 1, 2, 1)))


@pytest.mark.parametrize("r", [0, 7])
def test_all_to_all_ulysses_share_full_size(r):
    """The Ulysses share of the LLaMA-70B shape: 8 sequence shards [1, 4096, 64, 128] bf16 to head
    group r over the whole sequence, and back (the return all-to-all from all 8 ranks' head groups
    restores rank r's shard), bit-exact against the oracle."""
    say(f"all_to_all Ulysses share full size, rank {r}")
    inp, p = W.workload_inputs(3)
    shards = inp["q"]
    dev = to_dev(*shards)
    got = T.shard_all_to_all(dev, r, 2, 1)
    torch.cuda.synchronize()
    assert torch.equal(_bits(got.cpu()), _bits(oracle.all_to_all(shards, r, 2, 1)))
    groups = [T.shard_all_to_all(dev, g, 2, 1) for g in range(8)]
    back = T.shard_all_to_all(groups, r, 1, 2)
    torch.cuda.synchronize()
    assert torch.equal(_bits(back.cpu()), _bits(shards[r]))

"""Seeded synthetic inputs shaped like the pages' workloads.

This module is shared by the tests, the oracle-side checks and bench.py.  It
holds only the configuration table and seeded random draws (normal values
rounded to the input dtype, key lengths); none of the attention arithmetic.

Recipe: a torch CPU generator seeded with `seed`; draw order is key lengths
(only where the workload has key padding), then Q, then K, then V, each as
float32 N(0, 1) rounded to the input dtype with round-to-nearest-even (what
torch's `.to(torch.bfloat16)` does).  The same host bytes feed the oracle and
the device.

Shapes come from the pages: the LLaMA-70B activation example of
"adv07: Sequence Parallel" section 2 (hidden 8192 = 64 heads x 128, sequence
32768) split over 8 ranks, the per-rank contiguous sequence slices of the data
collator in "Support deepspeed sequence parallel", and the [batch, seq, heads,
head_dim] layout of "parallel multi-head attention" section 3.2.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import torch


@dataclass(frozen=True)
class Workload:
    key: int
    name: str
    desc: str
    dtype: torch.dtype
    params: Dict = field(default_factory=dict)


WORKLOADS: Dict[int, Workload] = {
    1: Workload(1, "tiny_mha_fp32", "MHA fwd, batch 1, seq 64, 2 heads, head_dim 8, fp32, causal",
                torch.float32, dict(B=1, S=64, H=2, D=8, causal=True)),
    2: Workload(2, "causal_4k", "causal attention, batch 1, seq 4096, 8 heads x 128, bf16, with LSE",
                torch.bfloat16, dict(B=1, S=4096, H=8, D=128, causal=True)),
    3: Workload(3, "ulysses_share_32k",
                "8 seq-shards [4096, 64 heads, 128] bf16 -> head group [32768, 8, 128]; causal attention",
                torch.bfloat16, dict(P=8, B=1, S=32768, H=64, D=128, group=0, causal=True)),
    4: Workload(4, "ring_share_32k",
                "Q chunk of 4096 at positions 28672..32767 vs 8 KV chunks of 4096, 8 heads x 128, bf16, causal",
                torch.bfloat16, dict(P=8, B=1, S=32768, H=8, D=128, q_chunk=7, causal=True)),
    5: Workload(5, "padded_batch",
                "batch 4, seq 8192, 32 heads x 128, bf16, key padding, lengths uniform in [4096, 8192]",
                torch.bfloat16, dict(B=4, S=8192, H=32, D=128, len_lo=4096, len_hi=8192, causal=False)),
}


def generator(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def randn(shape, g: torch.Generator, dtype: torch.dtype) -> torch.Tensor:
    """float32 N(0,1) from `g`, rounded to `dtype` (RNE)."""
    x = torch.randn(tuple(shape), generator=g, dtype=torch.float32)
    return x if dtype == torch.float32 else x.to(dtype)


def key_lengths(B: int, lo: int, hi: int, g: torch.Generator) -> torch.Tensor:
    """Per-sequence valid key lengths, uniform integers in [lo, hi] inclusive (int32)."""
    return torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64).to(torch.int32)


def attention_inputs(B: int, Sq: int, Sk: int, H: int, D: int, dtype: torch.dtype, seed: int,
                     len_range: Optional[tuple] = None) -> Dict[str, torch.Tensor]:
    """q [B,Sq,H,D], k/v [B,Sk,H,D] and optional kv_len [B] on the host."""
    g = generator(seed)
    out: Dict[str, torch.Tensor] = {}
    if len_range is not None:
        out["kv_len"] = key_lengths(B, len_range[0], len_range[1], g)
    out["q"] = randn((B, Sq, H, D), g, dtype)
    out["k"] = randn((B, Sk, H, D), g, dtype)
    out["v"] = randn((B, Sk, H, D), g, dtype)
    return out


def shard_inputs(P: int, B: int, S: int, H: int, D: int, dtype: torch.dtype, seed: int) -> Dict[str, List[torch.Tensor]]:
    """Per-rank sequence shards [B, S/P, H, D] of Q, K and V (shard i = tokens [i*S/P, (i+1)*S/P))."""
    g = generator(seed)
    Sl = S // P
    return {name: [randn((B, Sl, H, D), g, dtype) for _ in range(P)] for name in ("q", "k", "v")}


def workload_inputs(key: int, seed: Optional[int] = None, **override):
    """Inputs of workload `key` (seed defaults to the workload number).

    Keyword overrides replace shape parameters, for scaled-down parity cases
    that keep the workload's structure.
    """
    w = WORKLOADS[key]
    p = dict(w.params)
    p.update(override)
    seed = key if seed is None else seed
    if key in (1, 2):
        return attention_inputs(p["B"], p["S"], p["S"], p["H"], p["D"], w.dtype, seed), p
    if key == 3:
        return shard_inputs(p["P"], p["B"], p["S"], p["H"], p["D"], w.dtype, seed), p
    if key == 4:
        return attention_inputs(p["B"], p["S"] // p["P"], p["S"], p["H"], p["D"], w.dtype, seed), p
    if key == 5:
        return attention_inputs(p["B"], p["S"], p["S"], p["H"], p["D"], w.dtype, seed,
                                len_range=(p["len_lo"], p["len_hi"])), p
    raise KeyError(key)

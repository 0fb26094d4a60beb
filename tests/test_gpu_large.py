"""Tensors beyond 4 GiB: key and value tensors of 2^23 + 77 tokens x 2 heads x 128 (4.3 GB each in
bf16), key padding ending 1000 tokens before the end, so every kernel form walks keys whose byte
offsets need more than 32 bits.  Compared with the oracle over the whole output and lse."""
import pytest
import torch

import oracle
import tensor_head_attention_amd as T
import tha_workloads as W
from parity import DEV, check_lse, check_out, host_threads, say

pytestmark = pytest.mark.gpu

SK = (1 << 23) + 77
SQ, H, D = 64, 2, 128


@pytest.fixture(scope="module")
def big():
    say(f"large: K, V [1, {SK}, {H}, {D}] bf16 ({SK * H * D * 2 / 2**30:.2f} GiB each)")
    g = W.generator(4242)
    q = W.randn((1, SQ, H, D), g, torch.bfloat16)
    k = W.randn((1, SK, H, D), g, torch.bfloat16)
    v = W.randn((1, SK, H, D), g, torch.bfloat16)
    kv = torch.tensor([SK - 1000], dtype=torch.int32)
    ref, ref_lse = oracle.attention(q, k, v, kv_len=kv, nthreads=host_threads())
    dev = (q.to(DEV), k.to(DEV), v.to(DEV), kv.to(DEV))
    del k, v
    yield dev, ref, ref_lse


@pytest.mark.parametrize("kernel", [None, "narrow", "wide", "split", "split64"])
def test_keys_beyond_4GiB(big, kernel):
    (qd, kd, vd, kvd), ref, ref_lse = big
    say(f"large: kernel={kernel}")
    out, lse = T.attn_fwd(qd, kd, vd, kv_len=kvd, out_dtype=torch.float32, kernel=kernel)
    torch.cuda.synchronize()
    check_out(out, ref, torch.bfloat16)
    check_lse(lse, ref_lse, torch.bfloat16)

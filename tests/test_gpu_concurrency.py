"""The library keeps no state between calls, so calls on several streams at once, and from several
host threads at once, give the same bits as the same calls one after the other."""
import threading

import pytest
import torch

import tensor_head_attention_amd as T
import tha_workloads as W
from parity import DEV, say, to_dev

pytestmark = pytest.mark.gpu


def _case(seed, Sq=700, Sk=900, H=4, D=128, dt=torch.bfloat16):
    g = W.generator(seed)
    return to_dev(*(W.randn((1, n, H, D), g, dt) for n in (Sq, Sk, Sk)))


def _run(q, k, v):
    o, lse = T.attn_fwd(q, k, v, causal=True, q_pos0=200, out_dtype=torch.float32)
    parts = [T.attn_fwd(q, k[:, c:c + 300].contiguous(), v[:, c:c + 300].contiguous(), causal=True, q_pos0=200,
                        k_pos0=c, out_dtype=torch.float32) for c in (0, 300, 600)]
    mo, ml = T.attn_merge_lse([p[0] for p in parts], [p[1] for p in parts])
    return o, lse, mo, ml


def test_streams_concurrent_equal_serial():
    say("concurrency: two streams")
    cases = [_case(71), _case(72)]
    serial = [_run(*c) for c in cases]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in cases]
    out = [None, None]
    for rep in range(3):
        for s in streams:
            s.wait_stream(torch.cuda.current_stream())
        for i, (s, c) in enumerate(zip(streams, cases)):
            with torch.cuda.stream(s):
                out[i] = _run(*c)
        torch.cuda.synchronize()
        for a, b in zip(serial, out):
            assert all(torch.equal(x, y) for x, y in zip(a, b)), f"repetition {rep}"


def test_host_threads_concurrent_equal_serial():
    say("concurrency: four host threads, a stream each")
    cases = [_case(80 + i) for i in range(4)]
    serial = [_run(*c) for c in cases]
    torch.cuda.synchronize()
    out = [None] * len(cases)
    errors = []

    def work(i):
        try:
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.default_stream())
            with torch.cuda.stream(s):
                for _ in range(3):
                    out[i] = _run(*cases[i])
            s.synchronize()
        except Exception as e:  # reported below, in the test's thread
            errors.append(e)

    ts = [threading.Thread(target=work, args=(i,)) for i in range(len(cases))]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert not errors, errors
    for a, b in zip(serial, out):
        assert all(torch.equal(x, y) for x, y in zip(a, b))

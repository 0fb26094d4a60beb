"""GPU parity of attn_bwd against the fp64 oracle backward (through the C ABI).

The device pipeline runs as a user would: attn_fwd on the device gives o and lse, then attn_bwd.
The oracle computes the gradients from q, k, v and dout alone (its own softmax, its own Delta).

Tolerances (per output tensor, derived from the arithmetic of the bf16 path):
  bf16: P and dS are rounded to bf16 (relative error <= 2^-9 each) before the products that
        consume them, and Delta uses the bf16 forward output; over sums of many terms these give
        relative L2 errors of ~1e-3.  Bound: rel-L2 <= 1e-2, max |dev - ref| <= 2e-2 *
        max(max |ref|, 1e-3) (the floor covers gradients that are exactly 0 on paper, e.g. dq with a
        single visible key, where fp32 rounding of dP - Delta leaves ~1e-7).
  fp32: fp32 throughout: rel-L2 <= 1e-5, max |dev - ref| <= 1e-5 * max(1, max |ref|).
"""
import math

import pytest
import torch

import oracle
import tensor_head_attention_amd as T
import tha_workloads as W
from parity import DEV, say, to_dev

pytestmark = pytest.mark.gpu

TOL = {torch.bfloat16: (1e-2, 2e-2), torch.float32: (1e-5, 1e-5)}


def check_grad(dev, ref, dtype, what):
    d = dev.detach().double().cpu()
    assert d.shape == ref.shape, (what, d.shape, ref.shape)
    assert torch.isfinite(d).all(), f"{what}: non-finite values"
    rel_tol, abs_tol = TOL[dtype]
    scale = ref.abs().max().item()
    err = (d - ref).abs().max().item()
    rel = ((d - ref).norm() / ref.norm().clamp_min(1e-300)).item() if ref.norm() > 0 else err
    say(f"  {what}: max-abs {err:.3e} (max|ref| {scale:.3e}), rel-L2 {rel:.3e}")
    if dtype == torch.float32:
        assert err <= abs_tol * max(1.0, scale), f"{what}: max-abs {err:.3e}"
    else:
        assert err <= abs_tol * max(scale, 1e-3), f"{what}: max-abs {err:.3e} > {abs_tol} * {scale:.3e}"
    assert rel <= rel_tol, f"{what}: rel-L2 {rel:.3e} > {rel_tol}"


def _inputs(B, Sq, Sk, H, D, dtype, seed):
    g = W.generator(seed)
    q = W.randn((B, Sq, H, D), g, dtype)
    k = W.randn((B, Sk, H, D), g, dtype)
    v = W.randn((B, Sk, H, D), g, dtype)
    dout = W.randn((B, Sq, H, D), g, dtype)
    return q, k, v, dout


CASES = [
    # B, Sq, Sk, H, D, dtype, causal, q_pos0, k_pos0, lens
    (1, 128, 128, 1, 128, torch.bfloat16, False, 0, 0, None),
    (1, 256, 256, 2, 128, torch.bfloat16, True, 0, 0, None),
    (2, 300, 300, 3, 128, torch.bfloat16, True, 0, 0, None),        # ragged tails
    (2, 200, 333, 2, 128, torch.bfloat16, False, 0, 0, None),       # Sq != Sk
    (1, 77, 500, 2, 128, torch.bfloat16, True, 423, 0, None),       # late query chunk (ring-like)
    (1, 190, 260, 2, 128, torch.bfloat16, True, 37, 5, None),       # diagonal at odd offsets
    (1, 64, 64, 2, 128, torch.bfloat16, True, 0, 40, None),         # early rows see nothing
    (3, 160, 160, 2, 128, torch.bfloat16, False, 0, 0, [1, 97, 160]),
    (2, 150, 200, 2, 128, torch.bfloat16, True, 50, 0, [0, 130]),   # an empty sequence
    (2, 330, 330, 3, 64, torch.bfloat16, True, 0, 0, None),
    (2, 129, 257, 2, 64, torch.bfloat16, False, 0, 0, [200, 257]),
    (1, 1, 1, 1, 128, torch.bfloat16, False, 0, 0, None),
    (1, 1, 700, 1, 128, torch.bfloat16, True, 699, 0, None),        # decode-like single row
    (1, 64, 64, 2, 8, torch.float32, True, 0, 0, None),
    (2, 70, 90, 3, 40, torch.float32, False, 0, 0, [90, 17]),
    (1, 33, 200, 2, 256, torch.float32, True, 167, 0, None),
    (1, 50, 50, 1, 1, torch.float32, True, 0, 0, None),
]


def _id(c):
    B, Sq, Sk, H, D, dt, causal, qp, kp, lens = c
    return f"B{B}_Sq{Sq}_Sk{Sk}_H{H}_D{D}_{'bf16' if dt == torch.bfloat16 else 'f32'}" \
           f"{'_causal' if causal else ''}_qp{qp}_kp{kp}{'_pad' if lens else ''}"


def _device_bwd(q, k, v, dout, causal, qp, kp, kv, dq=None, dk=None, dv=None):
    qd, kd, vd, dd = to_dev(q, k, v, dout)
    kvd = kv.to(DEV) if kv is not None else None
    o, lse = T.attn_fwd(qd, kd, vd, causal=causal, q_pos0=qp, k_pos0=kp, kv_len=kvd)
    return T.attn_bwd(qd, kd, vd, o, dd, lse, causal=causal, q_pos0=qp, k_pos0=kp, kv_len=kvd, dq=dq, dk=dk, dv=dv)


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_bwd_matches_oracle(case):
    B, Sq, Sk, H, D, dt, causal, qp, kp, lens = case
    say(f"bwd case {_id(case)}")
    q, k, v, dout = _inputs(B, Sq, Sk, H, D, dt, seed=Sq * 5 + Sk + D)
    kv = torch.tensor(lens, dtype=torch.int32) if lens is not None else None
    rq, rk, rv = oracle.attention_backward(q, k, v, dout, causal=causal, q_pos0=qp, k_pos0=kp, kv_len=kv)
    dq, dk, dv = _device_bwd(q, k, v, dout, causal, qp, kp, kv)
    torch.cuda.synchronize()
    check_grad(dq, rq, dt, "dq")
    check_grad(dk, rk, dt, "dk")
    check_grad(dv, rv, dt, "dv")


def test_bwd_accumulates():
    """dq, dk, dv are accumulated into: a second call on the same buffers doubles them exactly."""
    q, k, v, dout = _inputs(1, 200, 200, 2, 128, torch.bfloat16, seed=81)
    dq1, dk1, dv1 = _device_bwd(q, k, v, dout, True, 0, 0, None)
    a = [t.clone() for t in (dq1, dk1, dv1)]
    _device_bwd(q, k, v, dout, True, 0, 0, None, dq=dq1, dk=dk1, dv=dv1)
    torch.cuda.synchronize()
    for x, y in zip((dq1, dk1, dv1), a):
        assert torch.equal(x, 2 * y)


def test_bwd_deterministic():
    q, k, v, dout = _inputs(2, 300, 300, 2, 128, torch.bfloat16, seed=82)
    r1 = _device_bwd(q, k, v, dout, True, 0, 0, None)
    r2 = _device_bwd(q, k, v, dout, True, 0, 0, None)
    torch.cuda.synchronize()
    for x, y in zip(r1, r2):
        assert torch.equal(x, y)


def test_bwd_ring_chunks_sum_to_full():
    """Ring share backward in miniature: a late Q chunk against 5 KV chunks at their global
    positions, each step using the FULL o and lse of the forward (merged over all chunks):
    dq accumulates over the steps, dk / dv of each chunk come from its step; together they equal
    the oracle's unchunked gradients."""
    P, Sc, H, D = 5, 200, 2, 128
    g = W.generator(83)
    q = W.randn((1, Sc, H, D), g, torch.bfloat16)
    k = W.randn((1, P * Sc, H, D), g, torch.bfloat16)
    v = W.randn((1, P * Sc, H, D), g, torch.bfloat16)
    dout = W.randn((1, Sc, H, D), g, torch.bfloat16)
    qp = 3 * Sc
    rq, rk, rv = oracle.attention_backward(q, k, v, dout, causal=True, q_pos0=qp, k_pos0=0)
    qd, kd, vd, dd = to_dev(q, k, v, dout)
    o, lse = T.attn_fwd(qd, kd, vd, causal=True, q_pos0=qp, k_pos0=0)  # the merged result of a Ring pass
    dq = torch.zeros((1, Sc, H, D), dtype=torch.float32, device=DEV)
    dks, dvs = [], []
    for t in range(P):
        kc, vc = kd[:, t * Sc:(t + 1) * Sc].contiguous(), vd[:, t * Sc:(t + 1) * Sc].contiguous()
        _, dk, dv = T.attn_bwd(qd, kc, vc, o, dd, lse, causal=True, q_pos0=qp, k_pos0=t * Sc, dq=dq)
        dks.append(dk)
        dvs.append(dv)
    torch.cuda.synchronize()
    assert torch.all(dks[4] == 0) and torch.all(dvs[4] == 0)  # chunk 4 lies wholly in the future
    check_grad(dq, rq, torch.bfloat16, "dq")
    check_grad(torch.cat(dks, dim=1), rk, torch.bfloat16, "dk")
    check_grad(torch.cat(dvs, dim=1), rv, torch.bfloat16, "dv")


def test_bwd_workload2_causal_4k_full():
    """The single-GPU causal workload (B1 S4096 H8 D128 bf16) at full size, every element."""
    say("bwd workload 2: causal S4096 H8 D128 bf16")
    inp, p = W.workload_inputs(2)
    q, k, v = inp["q"], inp["k"], inp["v"]
    dout = W.randn(q.shape, W.generator(92), torch.bfloat16)
    rq, rk, rv = oracle.attention_backward(q, k, v, dout, causal=True)
    dq, dk, dv = _device_bwd(q, k, v, dout, True, 0, 0, None)
    torch.cuda.synchronize()
    check_grad(dq, rq, torch.bfloat16, "dq")
    check_grad(dk, rk, torch.bfloat16, "dk")
    check_grad(dv, rv, torch.bfloat16, "dv")


@pytest.fixture(scope="module")
def bwd32k():
    """The Ulysses share's attention (causal S32768, 8 heads x 128, bf16) and its full-size backward
    on the device, as a user runs it (attn_fwd, then attn_bwd)."""
    say("bwd Ulysses share 32k: device forward and backward")
    g = W.generator(93)
    S, H, D = 32768, 8, 128
    q, k, v, dout = (W.randn((1, S, H, D), g, torch.bfloat16) for _ in range(4))
    dq, dk, dv = _device_bwd(q, k, v, dout, True, 0, 0, None)
    torch.cuda.synchronize()
    yield dict(S=S, H=H, D=D, g=g, host=(q, k, v, dout), dev=(dq, dk, dv))


def test_bwd_ulysses_share_32k_sampled(bwd32k):
    """Sampled dq rows against the oracle (row i of dq depends on query row i only, so the oracle
    runs each sampled row as a one-row call at its position), and for dk / dv the closed forms that
    hold at any size: per (b, h) the keys' dk sum to 0, and the keys' dv sum to the sum of dout over
    rows."""
    S, g = bwd32k["S"], bwd32k["g"]
    q, k, v, dout = bwd32k["host"]
    dq, dk, dv = bwd32k["dev"]
    rows = [0, 1, 63, 64, 127, 128, 4095, 4096, 16383, 16384, 32766, 32767] + \
        torch.randint(0, S, (6,), generator=g).tolist()
    dq_c = dq.cpu().double()
    for i in rows:
        rq, _, _ = oracle.attention_backward(q[:, i:i + 1].contiguous(), k[:, :i + 1].contiguous(),
                                             v[:, :i + 1].contiguous(), dout[:, i:i + 1].contiguous(),
                                             causal=True, q_pos0=i, k_pos0=0)
        check_grad(dq_c[:, i:i + 1], rq, torch.bfloat16, f"dq row {i}")
    dk_sum = dk.double().sum(dim=1)
    dv_sum = dv.double().sum(dim=1)
    dout_sum = dout.to(DEV).double().sum(dim=1)
    assert dk_sum.abs().max().item() <= 1e-2 * dk.abs().max().item() * math.sqrt(S)
    assert (dv_sum - dout_sum).abs().max().item() <= 2e-2 * dout_sum.abs().max().item()
    assert torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all()


LAST = 4096  # the last query rows: keys at or after their first position see no other query row


@pytest.mark.parametrize("h", list(range(8)))
def test_bwd_ulysses_share_32k_last_chunk(bwd32k, h):
    """Every element of dq for the last 4096 query rows, and of dk and dv for the last 4096 keys, of
    head h at full size.  Under the causal mask key j receives gradient only from query rows i >= j,
    so the oracle's backward of query rows S-4096.. against ALL keys gives those keys' dk and dv in
    full (and those rows' dq).  The oracle runs on blocks of 256 query rows in parallel host threads
    (one single-threaded call each; the test adds the blocks' dk / dv in fp64)."""
    from concurrent.futures import ThreadPoolExecutor

    from parity import host_threads
    S = bwd32k["S"]
    q, k, v, dout = bwd32k["host"]
    dq, dk, dv = bwd32k["dev"]
    say(f"bwd Ulysses share 32k: head {h}, rows and keys {S - LAST}..{S - 1} against the oracle")
    kh, vh = (t[:, :, h:h + 1].contiguous() for t in (k, v))
    blk = 256

    def block(r0):
        qb, db = (t[:, r0:r0 + blk, h:h + 1].contiguous() for t in (q, dout))
        return oracle.attention_backward(qb, kh, vh, db, causal=True, q_pos0=r0, k_pos0=0, nthreads=1)

    with ThreadPoolExecutor(max_workers=host_threads()) as ex:
        res = list(ex.map(block, range(S - LAST, S, blk)))
    rq = torch.cat([r[0] for r in res], dim=1)
    rk = sum(r[1][:, S - LAST:] for r in res)
    rv = sum(r[2][:, S - LAST:] for r in res)
    check_grad(dq[:, S - LAST:, h:h + 1], rq, torch.bfloat16, f"dq rows {S - LAST}.. head {h}")
    check_grad(dk[:, S - LAST:, h:h + 1], rk, torch.bfloat16, f"dk keys {S - LAST}.. head {h}")
    check_grad(dv[:, S - LAST:, h:h + 1], rv, torch.bfloat16, f"dv keys {S - LAST}.. head {h}")

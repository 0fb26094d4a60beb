"""The lazy running-max update on inputs that move it in the middle of a row.  With N(0,1) data a
row's running max is set by its first key tile and almost never raised again, so the rescale of O
and l (taken when a tile's maximum exceeds the running max by more than 2^8 in probability terms)
would only ever act on zeros.  Two recipes add a common direction u (|u| = 1) to every query and,
with a weight per key, to the keys:
  spikes: four keys get weights that put their scores about 8, 11, 15 and 19 times the row's q.u
          (about 1) above the bulk of the row, so the running max is raised mid-row while the keys
          before a spike still hold a large share of the softmax mass, and a wrong rescale shows;
  rising: the weight grows along the sequence, so the scores of a row rise by several units per key
          tile and the running max is raised again and again."""
import pytest
import torch

import oracle
import tensor_head_attention_amd as T
import tha_workloads as W
from parity import check_lse, check_out, say, to_dev

pytestmark = pytest.mark.gpu

KERNELS = [(128, torch.bfloat16, "narrow"), (128, torch.bfloat16, "wide"), (128, torch.bfloat16, "split"),
           (128, torch.bfloat16, "split64"),
           (64, torch.bfloat16, None), (40, torch.float32, None)]


def key_weights(recipe: str, Sk: int, D: int) -> torch.Tensor:
    """Weight of u in each key; a row's score for key j moves by about weight_j * (q.u) / sqrt(D)."""
    if recipe == "rising":
        return 100.0 * torch.arange(Sk, dtype=torch.float32) / Sk * D ** 0.5
    w = torch.zeros(Sk)
    for pos, score in ((150, 8.0), (421, 11.0), (777, 15.0), (1030, 19.0)):
        if pos < Sk:
            w[pos] = score * D ** 0.5
    return w


def inputs(recipe, B, Sq, Sk, H, D, dt, seed):
    g = W.generator(seed)
    u = torch.full((D,), D ** -0.5)
    q = W.randn((B, Sq, H, D), g, torch.float32) + u
    k = W.randn((B, Sk, H, D), g, torch.float32) + key_weights(recipe, Sk, D)[None, :, None, None] * u
    v = W.randn((B, Sk, H, D), g, torch.float32)
    return q.to(dt), k.to(dt), v.to(dt)


def _kid(k):
    D, dt, kn = k
    return f"D{D}_{'bf16' if dt == torch.bfloat16 else 'f32'}_{kn or 'auto'}"


# The fp32 kernel runs on the spikes recipe only: the rising recipe's scores reach several hundred,
# and fp32's own rounding of such scores (about |s| * 2^-24 * sqrt(D), ~1e-4 here) moves the
# output by more than the 1e-5 bound that fits N(0,1)-sized scores.
CASES = [(k, r) for r in ("spikes", "rising") for k in KERNELS if not (r == "rising" and k[1] == torch.float32)]


@pytest.mark.parametrize("kern,recipe", CASES, ids=lambda x: _kid(x) if isinstance(x, tuple) else x)
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_rescale_matches_oracle(kern, recipe, causal):
    D, dt, kn = kern
    say(f"rescale {recipe} {_kid(kern)} causal={causal}")
    q, k, v = inputs(recipe, 2, 300, 1100, 2, D, dt, seed=501 + D)
    ref, ref_lse = oracle.attention(q, k, v, causal=causal, q_pos0=800)
    qd, kd, vd = to_dev(q, k, v)
    out, lse = T.attn_fwd(qd, kd, vd, causal=causal, q_pos0=800, out_dtype=torch.float32, kernel=kn)
    torch.cuda.synchronize()
    check_out(out, ref, dt)
    if dt == torch.float32:
        # the spikes put lse near 50 for some rows, where one fp32 ulp is ~4e-6: the fp32 bound of
        # 1e-5 applies relative to max(1, |lse|) here
        l, r = lse.cpu().double(), ref_lse
        assert torch.equal(torch.isinf(l), torch.isinf(r))
        fin = ~torch.isinf(r)
        rel = ((l[fin] - r[fin]).abs() / r[fin].abs().clamp_min(1.0)).max().item()
        say(f"  lse: max relative error {rel:.3e}")
        assert rel <= 1e-5
    else:
        check_lse(lse, ref_lse, dt)


@pytest.mark.parametrize("recipe", ["spikes", "rising"])
def test_rescale_narrow_wide_bitwise(recipe):
    """The narrow and wide kernels take the same rescale decisions, so they stay bit-identical on
    inputs that rescale mid-row."""
    say(f"rescale narrow vs wide {recipe}")
    q, k, v = inputs(recipe, 1, 520, 1500, 3, 128, torch.bfloat16, seed=777)
    qd, kd, vd = to_dev(q, k, v)
    res = {}
    for kn in ("narrow", "wide"):
        res[kn] = T.attn_fwd(qd, kd, vd, causal=True, q_pos0=1000, out_dtype=torch.float32, kernel=kn)
        torch.cuda.synchronize()
    assert torch.equal(res["narrow"][0], res["wide"][0]) and torch.equal(res["narrow"][1], res["wide"][1])
    ref, ref_lse = oracle.attention(q, k, v, causal=True, q_pos0=1000)
    check_out(res["wide"][0], ref, torch.bfloat16)
    check_lse(res["wide"][1], ref_lse, torch.bfloat16)


@pytest.mark.parametrize("recipe", ["spikes", "rising"])
@pytest.mark.parametrize("fused", [True, False], ids=["fused", "partials"])
def test_ring_share_large_jumps(recipe, fused):
    """A Ring pass over chunks whose scores differ by tens of units between chunks: the merge of
    running results (in the attention epilogue, or by attn_merge_lse) meets weights e^(lse_k - M)
    far from 1 in both directions."""
    say(f"ring share {recipe} fused={fused}")
    q, k, v = inputs(recipe, 1, 256, 1100, 2, 128, torch.bfloat16, seed=913)
    ref, ref_lse = oracle.attention(q, k, v, causal=True, q_pos0=844)
    qd, kd, vd = to_dev(q, k, v)
    cuts = [0, 200, 421, 700, 1030, 1100]
    kc = [kd[:, a:b].contiguous() for a, b in zip(cuts, cuts[1:])]
    vc = [vd[:, a:b].contiguous() for a, b in zip(cuts, cuts[1:])]
    out, lse = T.ring_share(qd, kc, vc, q_pos0=844, k_pos0s=cuts[:-1], fused=fused, out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_out(out, ref, torch.bfloat16)
    check_lse(lse, ref_lse, torch.bfloat16)

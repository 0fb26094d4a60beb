"""Shared comparison helpers for the GPU parity tests (device result vs fp64 oracle).

Tolerances (per the workload definitions):
  fp32 inputs : max |o_dev - o_ref| <= 1e-5 over the whole output; lse <= 1e-5
  bf16 inputs : max |o_dev - o_ref| <= 2e-2 and ||o_dev - o_ref|| / ||o_ref|| <= 5e-3
                over the whole output, on the same bf16-rounded inputs; lse <= 1e-4
A row with no visible key must give o = 0 and lse = -inf on both sides.
"""
import sys

import torch

TOL = {
    torch.float32: dict(max_abs=1e-5, rel_l2=None, lse=1e-5),
    torch.bfloat16: dict(max_abs=2e-2, rel_l2=5e-3, lse=1e-4),
}
DEV = "cuda:0"


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(*ts):
    return [t.to(DEV) for t in ts]


def check_out(dev_out: torch.Tensor, ref: torch.Tensor, in_dtype: torch.dtype, what: str = "out"):
    o = dev_out.detach().float().cpu().double()
    assert o.shape == ref.shape, (o.shape, ref.shape)
    assert torch.isfinite(o).all(), f"{what}: non-finite values"
    tol = TOL[in_dtype]
    diff = (o - ref).abs()
    max_abs = diff.max().item() if diff.numel() else 0.0
    rel = ((o - ref).norm() / ref.norm().clamp_min(1e-300)).item() if ref.numel() else 0.0
    say(f"  {what}: max-abs {max_abs:.3e}, rel-L2 {rel:.3e}")
    assert max_abs <= tol["max_abs"], f"{what}: max-abs {max_abs:.3e} > {tol['max_abs']}"
    if tol["rel_l2"] is not None and ref.numel():
        assert rel <= tol["rel_l2"], f"{what}: rel-L2 {rel:.3e} > {tol['rel_l2']}"
    return max_abs


def check_lse(dev_lse: torch.Tensor, ref: torch.Tensor, in_dtype: torch.dtype, what: str = "lse"):
    l = dev_lse.detach().cpu().double()
    assert l.shape == ref.shape, (l.shape, ref.shape)
    inf_ref = torch.isinf(ref)
    assert torch.equal(torch.isinf(l), inf_ref), f"{what}: -inf pattern differs"
    assert torch.all(l[inf_ref] < 0)
    fin = ~inf_ref
    if fin.any():
        err = (l[fin] - ref[fin]).abs().max().item()
        say(f"  {what}: max-abs {err:.3e}")
        assert err <= TOL[in_dtype]["lse"], f"{what}: max-abs {err:.3e} > {TOL[in_dtype]['lse']}"

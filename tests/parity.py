"""Shared comparison helpers for the GPU parity tests (device result vs fp64 oracle).

Tolerances (per the workload definitions), over the whole output tensor:
  fp32 inputs : max |o_dev - o_ref| <= 1e-5 over the whole output; lse <= 1e-5
  bf16 inputs : max |o_dev - o_ref| <= 2e-2 and ||o_dev - o_ref|| / ||o_ref|| <= 5e-3
                over the whole output, on the same bf16-rounded inputs; lse <= 1e-4
A row with no visible key must give o = 0 and lse = -inf on both sides.
"""
import os
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


def host_threads() -> int:
    """Host threads for the oracle: the CPUs this process may run on, capped by OMP_NUM_THREADS
    when that is set (the CPU share a machine gives one GPU's job)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return max(1, n)


class WholeTensor:
    """Compares one device output with the oracle slice by slice (the oracle runs per head or per
    sequence) and keeps the sums that give max-abs and rel-L2 over the WHOLE tensor: each slice is
    checked at the tolerance as it arrives, and `finish` checks the whole-tensor figures once every
    slice has been seen."""

    def __init__(self, name: str, in_dtype: torch.dtype):
        self.name, self.in_dtype = name, in_dtype
        self.parts = {}

    def add(self, key, dev_out, ref, dev_lse=None, ref_lse=None):
        o = dev_out.detach().float().cpu().double()
        max_abs = check_out(o, ref, self.in_dtype, f"{self.name}[{key}] out")
        lse_err = 0.0
        if dev_lse is not None:
            check_lse(dev_lse, ref_lse, self.in_dtype, f"{self.name}[{key}] lse")
            l = dev_lse.detach().cpu().double()
            fin = ~torch.isinf(ref_lse)
            lse_err = (l[fin] - ref_lse[fin]).abs().max().item() if fin.any() else 0.0
        err2 = (o - ref).pow(2).sum().item()
        ref2 = ref.pow(2).sum().item()
        self.parts[key] = (max_abs, err2, ref2, lse_err, ref.numel())

    def missing(self, keys):
        return [k for k in keys if k not in self.parts]

    def finish(self, keys):
        assert not self.missing(keys), f"{self.name}: slices not compared: {self.missing(keys)}"
        max_abs = max(self.parts[k][0] for k in keys)
        err2 = sum(self.parts[k][1] for k in keys)
        ref2 = sum(self.parts[k][2] for k in keys)
        lse_err = max(self.parts[k][3] for k in keys)
        n = sum(self.parts[k][4] for k in keys)
        rel = (err2 ** 0.5) / max(ref2 ** 0.5, 1e-300)
        say(f"  {self.name}: whole output ({n} elements): max-abs {max_abs:.3e}, rel-L2 {rel:.3e}, "
            f"lse max-abs {lse_err:.3e}")
        tol = TOL[self.in_dtype]
        assert max_abs <= tol["max_abs"]
        if tol["rel_l2"] is not None:
            assert rel <= tol["rel_l2"], f"{self.name}: whole-tensor rel-L2 {rel:.3e} > {tol['rel_l2']}"
        assert lse_err <= tol["lse"]
        return max_abs, rel, lse_err

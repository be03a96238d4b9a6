"""The bf16 rounding allowance of the GPU parity tests is exactly half an ulp of bf16 at each
value's binade: round-to-nearest-even never moves a value further, and the allowance is not
larger than that (so it cannot hide an error of a full ulp)."""
import torch

from tests.gpu_run import bf16_half_ulp


def test_half_ulp_bounds_round_to_nearest_even():
    g = torch.Generator().manual_seed(0)
    x = torch.cat([torch.randn(200000, generator=g) * s for s in (1e-3, 0.3, 1.0, 7.9, 100.0)])
    x = torch.cat([x, torch.tensor([1.0, -2.0, 8.0, 8.03125, 0.0, 3.0e-5])])
    r = x.to(torch.bfloat16).to(torch.float64)
    xd = x.to(torch.float64)
    err = (r - xd).abs()
    bound = bf16_half_ulp(torch.maximum(r.abs(), xd.abs()))
    assert bool((err <= bound).all())
    # tight: some values sit exactly half an ulp from a bf16 neighbour (ties)
    tie = torch.tensor([1.0 + 2.0 ** -8, 8.0 + 2.0 ** -5], dtype=torch.float32)
    assert torch.equal((tie.to(torch.bfloat16).double() - tie.double()).abs(), bf16_half_ulp(tie.double()))


def test_half_ulp_values():
    v = torch.tensor([1.0, 1.99, 2.0, 8.0, 15.9, 0.5, 0.0], dtype=torch.float64)
    want = torch.tensor([2 ** -8, 2 ** -8, 2 ** -7, 2 ** -5, 2 ** -5, 2 ** -9, 0.0], dtype=torch.float64)
    assert torch.equal(bf16_half_ulp(v), want)

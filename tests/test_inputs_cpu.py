"""The seeded input generators (host and on-device draws), on the CPU."""
import numpy as np
import torch

from fusion_residual_add_amd import inputs


def test_generate_is_deterministic_and_seeded():
    wl = inputs.workload("tiny-f32")
    a, b, c = inputs.generate(wl, seed=0), inputs.generate(wl, seed=0), inputs.generate(wl, seed=1)
    assert a.keys() == b.keys()
    for k in a:
        assert torch.equal(a[k], b[k]), k
    assert not torch.equal(a["x"], c["x"])


def test_device_draws_are_seeded_and_rounded_from_float32():
    n = 1 << 20
    x = inputs.device_normal((n,), 0.5, torch.bfloat16, "cpu", seed=7)
    assert x.dtype == torch.bfloat16 and x.shape == (n,)
    assert torch.equal(x, inputs.device_normal((n,), 0.5, torch.bfloat16, "cpu", seed=7))
    assert not torch.equal(x, inputs.device_normal((n,), 0.5, torch.bfloat16, "cpu", seed=8))
    # the same float32 draw, then one round-to-nearest-even cast
    g = torch.Generator(device="cpu")
    g.manual_seed(7)
    ref = torch.empty(n, dtype=torch.float32).normal_(0.0, 0.5, generator=g).to(torch.bfloat16)
    assert torch.equal(x, ref)
    xf = x.double().numpy()
    assert abs(xf.mean()) < 5e-3 and abs(xf.std() - 0.5) < 5e-3
    u = inputs.device_uniform((4, 1000), 0.5, 1.5, torch.float16, "cpu", seed=3).double().numpy()
    assert u.shape == (4, 1000) and u.min() >= 0.5 and u.max() <= 1.5 and abs(u.mean() - 1.0) < 0.02

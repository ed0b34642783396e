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


def test_mxfp4_quantiser_brute_force():
    """Each block's exponent is floor(log2(max |w|)) - 2 and each code the
    nearest E2M1 value of w / 2^e (saturated at 6), ties to the even code:
    checked against a search over the 16 codes."""
    import numpy as np
    import torch
    from fusion_residual_add_amd import inputs
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((6, 96)) * 0.02).astype(np.float32)
    w[1, :32] = 0.0                                       # an all-zero block
    w[2, 5] = 1.5 * 2.0 ** -8                             # ties and exact values in a block
    q, s = inputs.quantize_blocks_mxfp4(w)
    assert q.dtype == torch.float4_e2m1fn_x2 and s.dtype == torch.float8_e8m0fnu
    packed = q.view(torch.uint8).numpy()
    codes = np.stack([packed & 0xF, packed >> 4], -1).reshape(6, 96)
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    vals = np.concatenate([mags, -mags])
    sc = s.view(torch.uint8).numpy().astype(np.int64) - 127
    for j in range(6):
        for b in range(3):
            blk = w[j, 32 * b:32 * b + 32].astype(np.float64)
            amax = np.abs(blk).max()
            e = int(np.floor(np.log2(amax))) - 2 if amax > 0 else 0
            assert sc[j, b] == e
            for k in range(32):
                t = min(max(blk[k] / 2.0 ** e, -6.0), 6.0)
                d = np.abs(vals - t)
                cand = [c for c in range(16) if d[c] == d.min() and (c >= 8) == bool(np.signbit(t))]
                if len(cand) > 1:
                    cand = [c for c in cand if c % 2 == 0]
                assert codes[j, 32 * b + k] == cand[0], (j, b, k, t)

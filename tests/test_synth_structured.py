"""The structured-spectrum input recipe (synth.structured) has the spectra it
claims; checked on the host with numpy's SVD."""
import numpy as np
import pytest
import torch

from newton_schulz_amd import synth


def sv(kind, r, c, **kw):
    y = synth.structured(kind, r, c, seed=7, dtype=torch.float32, **kw).double().numpy()
    return np.linalg.svd(y, compute_uv=False)


@pytest.mark.parametrize("r,c", [(48, 160), (160, 48)])
def test_spectra(r, c):
    s = sv("rank1", r, c)
    assert s[1] / s[0] < 1e-6                      # rank one up to fp32 rounding
    s = sv("rank8_noise", r, c)
    assert s[7] / s[0] > 0.05 and s[8] / s[7] < 1e-2  # eight large values over a floor
    s = sv("geometric", r, c)
    k = min(r, c)
    ratios = s[1:] / s[:-1]
    np.testing.assert_allclose(ratios, 10.0 ** (-6.0 / (k - 1)), rtol=1e-3)
    np.testing.assert_allclose(s[0], 1e-3, rtol=1e-5)


def test_scale_and_determinism():
    a = synth.structured("gauss", 32, 64, seed=3, dtype=torch.float32)
    b = synth.structured("gauss", 32, 64, seed=3, scale=1e6, dtype=torch.float32)
    np.testing.assert_allclose(b.numpy(), (a.double() * 1e6).float().numpy(), rtol=1e-6)
    assert torch.equal(a, synth.structured("gauss", 32, 64, seed=3, dtype=torch.float32))
    # bf16 output is the round-to-nearest-even cast of the fp32 values
    c = synth.structured("rank1", 32, 64, seed=3)
    assert c.dtype == torch.bfloat16
    assert torch.equal(c, synth.structured("rank1", 32, 64, seed=3, dtype=torch.float32).to(torch.bfloat16))

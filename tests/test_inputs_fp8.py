"""The FP8 E4M3 rounding of the input generators, pinned against PyTorch's float8_e4m3fn
conversion (an independent library implementation of the OCP format)."""

import numpy as np
import pytest
import torch

from sub_quadratic_attention_amd import inputs


def test_every_e4m3_value_is_fixed():
    """All 254 finite E4M3 values (decoded by torch) round to themselves."""
    vals = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    vals = vals[np.isfinite(vals)]
    assert len(vals) == 254
    assert np.array_equal(inputs.fp8_round(vals).astype(np.float64), vals)


def test_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200000) * s for s in (1e-3, 0.05, 1.0, 8.0, 60.0)])
    # midpoints between neighbours (ties) and values near the subnormal boundary
    vals = np.unique(torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy())
    vals = vals[np.isfinite(vals)]
    mids = (vals[1:] + vals[:-1]) / 2
    x = np.concatenate([x, mids, rng.uniform(-2 ** -6, 2 ** -6, 10000)])
    x = x[np.abs(x) <= 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = inputs.fp8_round(x).astype(np.float64)
    assert np.array_equal(got, ref)


def test_saturation():
    assert inputs.fp8_round(np.array([500.0, -1e6, 448.0]))[:3].tolist() == [448.0, -448.0, 448.0]

"""The seeded input generator: determinism, layout independence, moments, and
the Irwin-Hall construction checked on its own terms."""
import numpy as np
import pytest

import h3gen


def test_deterministic_and_row_addressable():
    a = h3gen.host_rows("x", 64, 96, "f32", seed=0)
    b = h3gen.host_rows("x", 64, 96, "f32", seed=0)
    assert np.array_equal(a, b)
    sel = [3, 17, 63, 5]
    assert np.array_equal(h3gen.host_rows("x", sel, 96, "f32", seed=0), a[sel])


def test_column_window_matches_full_rows():
    full = h3gen.host_rows("k", 40, 640, "bf16", seed=2)
    assert np.array_equal(h3gen.host_cols("k", 40, 640, 384, 128, "bf16", seed=2), full[:, 384:512])


def test_streams_differ_by_seed_and_tensor():
    a = h3gen.host_rows("x", 4, 64, "f32", seed=0)
    assert not np.array_equal(a, h3gen.host_rows("x", 4, 64, "f32", seed=1))
    assert not np.array_equal(a, h3gen.host_rows("h", 4, 64, "f32", seed=0))


def test_bf16_is_rounded_f32():
    import torch

    a = h3gen.host_rows("gate_up", 16, 128, "f32", seed=0)
    b = h3gen.host_rows("gate_up", 16, 128, "bf16", seed=0)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, ref)


@pytest.mark.parametrize("name,mu,sigma", [("x", 0.0, 1.0), ("gate", 0.0, 0.5),
                                           ("q_weight", 1.0, 0.05), ("shift", 0.0, 0.1)])
def test_moments(name, mu, sigma):
    a = h3gen.host_rows(name, 400, 1000, "f32", seed=0).astype(np.float64)
    n = a.size
    assert abs(a.mean() - mu) < 5 * sigma / np.sqrt(n)
    assert abs(a.std() / sigma - 1) < 5 * np.sqrt(2.0 / n)
    assert np.all(np.abs(a - mu) <= 6 * sigma * (1 + 1e-6))
    # Irwin-Hall(12): excess kurtosis -1.2/12 = -0.1
    z = (a - a.mean()) / a.std()
    assert abs((z ** 4).mean() - 3 + 0.1) < 0.03


def test_values_on_the_irwin_hall_lattice():
    # unit values are integers / 65536 in [-393210, 393210] / 65536
    a = h3gen.host_rows("x", 8, 256, "f32", seed=5).astype(np.float64) * 65536
    assert np.array_equal(a, np.round(a))
    assert np.all(np.abs(a) <= 393210)
    # odd sum of twelve (k + 1/2): numerator sum(k) - 393210 has the parity of sum(k)
    assert len(np.unique(np.mod(a, 2))) == 2

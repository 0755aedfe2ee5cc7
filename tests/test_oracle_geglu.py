"""Pins of the oracle's GEGLU step (gelu(g) = g * Phi(g), out = gelu(gate) * up)
against values and identities fixed by the mathematics, not by the oracle:

  * the standard normal CDF at tabulated points (Phi(1), Phi(2), Phi(-0.5));
  * gelu(x) - gelu(-x) = x for every x (Phi(x) + Phi(-x) = 1);
  * gelu(x) / x -> Phi(0) = 1/2 as x -> 0;
  * the tails: gelu(x) -> x and gelu(-x) -> 0 for large x, with the Mills-ratio
    size of the remainder;
  * geglu64 is the elementwise product gelu(gate) * up, read at FP32 inputs.
A wrong scale inside erf (x instead of x / sqrt 2), a dropped factor 1/2 or a
swapped gate/up each break at least one of these.
"""
import numpy as np
import pytest

import oracle

# Standard normal CDF, tabulated values.
PHI = {1.0: 0.8413447460685429, 2.0: 0.9772498680518208, -0.5: 0.3085375387259869, 0.0: 0.5}


@pytest.mark.parametrize("x,phi", sorted(PHI.items()))
def test_gelu_at_tabulated_points(x, phi):
    assert oracle.gelu64([x])[0] == pytest.approx(x * phi, rel=1e-15, abs=1e-300)


def test_gelu_odd_part_is_identity():
    x = np.random.default_rng(0).normal(0, 3, 1000)
    d = oracle.gelu64(x) - oracle.gelu64(-x)
    assert np.allclose(d, x, rtol=1e-14, atol=1e-14)


def test_gelu_slope_at_zero():
    for h in (1e-3, 1e-6, 1e-9):
        assert oracle.gelu64([h])[0] / h == pytest.approx(0.5, rel=2 * h)


def test_gelu_tails():
    # 1 - Phi(x) ~ phi(x) / x (Mills ratio) for large x.
    x = 8.0
    tail = np.exp(-x * x / 2) / np.sqrt(2 * np.pi) / x
    assert oracle.gelu64([x])[0] == pytest.approx(x, rel=1e-14)
    assert -oracle.gelu64([-x])[0] / x == pytest.approx(tail, rel=0.02)


def test_geglu_is_gelu_of_gate_times_up():
    rng = np.random.default_rng(1)
    gate = rng.normal(0, 2, (7, 13)).astype(np.float32)
    up = rng.normal(0, 2, (7, 13)).astype(np.float32)
    out = oracle.geglu64(gate, up)
    assert out.shape == gate.shape
    assert np.array_equal(out, oracle.gelu64(gate.astype(np.float64)) * up.astype(np.float64))
    # not symmetric in its arguments: swapping gate and up changes the result
    assert not np.allclose(out, oracle.geglu64(up, gate))
    with pytest.raises(ValueError):
        oracle.geglu64(gate, up[:, :5])

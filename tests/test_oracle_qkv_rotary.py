"""Pins of the oracle's Q/K/V packing with rotary multiplication against a
hand-computed case and the properties a rotation fixes:

  * D = 4, theta = 10000, position 1: pair 0 turns by 1 rad, pair 1 by 0.01
    rad (tabulated sines and cosines);
  * position 0 is the identity on q and k; v is always a copy;
  * each rotated pair keeps its length;
  * turning by p and then by r equals turning by p + r;
  * q(p) . k(r) depends on p - r only (the point of rotary embeddings);
  * the packing: head h of q, k, v comes from columns h*D, H*D + h*D and
    2*H*D + h*D of the row.
A swapped sign in the rotation, a wrong pair partner, a wrong frequency
exponent or a wrong head offset breaks at least one of these.
"""
import numpy as np
import pytest

import oracle

SIN1, COS1 = 0.8414709848078965, 0.5403023058681398
SIN01, COS01 = 0.009999833334166665, 0.9999500004166653


def test_hand_case():
    row = np.arange(12, dtype=np.float32).reshape(1, 12)  # q = 0..3, k = 4..7, v = 8..11
    q, k, v = oracle.qkv_rotary(row, H=1, D=4, pos=[1])
    x = [0.0, 1.0, 2.0, 3.0]
    want_q = [x[0] * COS1 - x[2] * SIN1, x[1] * COS01 - x[3] * SIN01,
              x[2] * COS1 + x[0] * SIN1, x[3] * COS01 + x[1] * SIN01]
    assert np.allclose(q[0, 0], want_q, rtol=1e-15, atol=1e-15)
    x = [4.0, 5.0, 6.0, 7.0]
    want_k = [x[0] * COS1 - x[2] * SIN1, x[1] * COS01 - x[3] * SIN01,
              x[2] * COS1 + x[0] * SIN1, x[3] * COS01 + x[1] * SIN01]
    assert np.allclose(k[0, 0], want_k, rtol=1e-15, atol=1e-15)
    assert np.array_equal(v[0, 0], [8.0, 9.0, 10.0, 11.0])


def _rows(T, H, D, seed=0):
    return np.random.default_rng(seed).normal(0, 1, (T, 3 * H * D)).astype(np.float32)


def test_position_zero_is_identity_and_packing():
    T, H, D = 3, 4, 8
    rows = _rows(T, H, D)
    q, k, v = oracle.qkv_rotary(rows, H, D, pos=np.zeros(T, np.int64))
    for h in range(H):
        assert np.array_equal(q[h], rows[:, h * D:(h + 1) * D])
        assert np.array_equal(k[h], rows[:, H * D + h * D:H * D + (h + 1) * D])
        assert np.array_equal(v[h], rows[:, 2 * H * D + h * D:2 * H * D + (h + 1) * D])


def test_pairs_keep_their_length():
    T, H, D = 5, 2, 16
    rows = _rows(T, H, D, 1)
    q, k, _ = oracle.qkv_rotary(rows, H, D, pos=np.arange(T) * 37)
    for h in range(H):
        src = rows[:, h * D:(h + 1) * D].astype(np.float64)
        before = src[:, :D // 2] ** 2 + src[:, D // 2:] ** 2
        after = q[h][:, :D // 2] ** 2 + q[h][:, D // 2:] ** 2
        assert np.allclose(before, after, rtol=1e-13)


def test_turns_compose():
    T, H, D = 4, 1, 8
    rows = _rows(T, H, D, 2)
    p = np.array([3, 10, 100, 7], np.int64)
    r = np.array([5, 1, 23, 0], np.int64)
    q1, _, _ = oracle.qkv_rotary(rows, H, D, pos=p)
    again = rows.copy()
    again[:, :D] = q1[0].astype(np.float32)
    q2, _, _ = oracle.qkv_rotary(again, H, D, pos=r)
    q3, _, _ = oracle.qkv_rotary(rows, H, D, pos=p + r)
    assert np.allclose(q2, q3, rtol=1e-6, atol=1e-6)


def test_scores_depend_on_relative_position():
    H, D = 1, 16
    rows = np.tile(_rows(1, H, D, 3), (4, 1))  # the same token at four positions
    q, k, _ = oracle.qkv_rotary(rows, H, D, pos=np.array([2, 9, 102, 109], np.int64))
    s1 = q[0, 0] @ k[0, 1]    # positions 2, 9
    s2 = q[0, 2] @ k[0, 3]    # positions 102, 109
    assert s1 == pytest.approx(s2, rel=1e-12, abs=1e-12)
    assert not q[0, 0] @ k[0, 0] == pytest.approx(s1, rel=1e-3)

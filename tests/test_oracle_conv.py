"""Pins of the oracle's two-tap dynamic convolution ("DFlash vs DFlash 2", "The
two-tap dynamic convolution": Conv_k(x)_t = k_{t,0} x_t + k_{t,1} x_{t-1}, a
content-dependent kernel per channel group, never across a block boundary,
position 1 reading the anchor).  Answers fixed by construction."""
import numpy as np
import pytest

import oracle


def _x(B=3, G=8, D=48, seed=0):
    return np.random.default_rng(seed).normal(size=(B, G, D))


def test_kernel_one_zero_is_the_identity():
    x = _x()
    k = np.zeros((3, 8, 2, 4))
    k[:, :, 0, :] = 1.0
    assert np.array_equal(oracle.two_tap_conv(x, k), x)


def test_kernel_zero_one_shifts_by_one_position_inside_the_block():
    x = _x()
    k = np.zeros((3, 8, 2, 4))
    k[:, :, 1, :] = 1.0
    y = oracle.two_tap_conv(x, k)
    assert np.array_equal(y[:, 1:], x[:, :-1])      # position t reads position t - 1
    assert np.array_equal(y[:, 0], np.zeros_like(x[:, 0]))  # the anchor's predecessor is zero


def test_blocks_are_independent():
    """Position 0 of block b never reads the last position of block b - 1, and
    changing one block changes no other."""
    x = _x()
    k = np.random.default_rng(1).normal(size=(3, 8, 2, 4))
    y = oracle.two_tap_conv(x, k)
    x2 = x.copy()
    x2[1] += 5.0
    y2 = oracle.two_tap_conv(x2, k)
    assert np.array_equal(y2[0], y[0]) and np.array_equal(y2[2], y[2])
    assert not np.allclose(y2[1], y[1])


@pytest.mark.parametrize("n_groups", [1, 2, 6, 48])
def test_each_channel_group_uses_its_own_kernel(n_groups):
    """Group g's kernel scales exactly the channels [g*D/n, (g+1)*D/n)."""
    B, G, D = 1, 3, 48
    x = np.ones((B, G, D))
    k = np.zeros((B, G, 2, n_groups))
    k[..., 0, :] = np.arange(n_groups) + 1.0
    y = oracle.two_tap_conv(x, k)
    gs = D // n_groups
    want = np.repeat(np.arange(n_groups) + 1.0, gs)
    assert np.array_equal(y[0, 1], want)


def test_linear_in_x():
    x1, x2 = _x(seed=2), _x(seed=3)
    k = np.random.default_rng(4).normal(size=(3, 8, 2, 4))
    y = oracle.two_tap_conv(2.0 * x1 - 3.0 * x2, k)
    assert np.allclose(y, 2.0 * oracle.two_tap_conv(x1, k) - 3.0 * oracle.two_tap_conv(x2, k),
                       rtol=1e-12, atol=1e-12)


def test_rejects_groups_that_do_not_divide_the_width():
    with pytest.raises(ValueError):
        oracle.two_tap_conv(np.zeros((1, 2, 10)), np.zeros((1, 2, 2, 3)))

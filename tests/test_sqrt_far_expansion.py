"""The sqrt-ALiBi kernel's far-tile bias, checked on the host.

On a key tile whose every distance is at least 384, the prefill kernel forms
-slope * sqrt(d) for each 32-key half from a second-order expansion around the
half's centre: d0 = dbase - (32 kb + 13.5), a lane's keys at offsets
dl = 8 (r / 4) + r % 4 - 13.5 (r = 0..15) from it, d = d0 - dl, and
    bias = b0 + b1 dl + b2 dl^2,  b0 = -slope sqrt(d0),
    b1 = slope / (2 sqrt d0),  b2 = slope / (8 d0^1.5).
The dropped remainder is at most 13.5^3 / (16 * 384^2.5) = 5.3e-5 (Lagrange form,
the point between d0 - dl and d0 being >= 384), in units of sqrt(d) times the
slope.  These tests evaluate that formula (in fp64, and in fp32 the way the kernel
does, with one reciprocal square root per half) against sqrt itself over the
tile geometry, so a wrong coefficient, sign or centre fails them."""

import numpy as np

FAR = 384
BOUND = 13.5 ** 3 / (16 * FAR ** 2.5)
DL = np.array([8 * (r // 4) + r % 4 - 13.5 for r in range(16)])


def _far_centres():
    # every half centre a far tile can have: the smallest distance of the half
    # is >= FAR, up to the longest sequences (plus a fine sweep near the edge)
    return np.concatenate([FAR + 13.5 + np.arange(0, 64, 0.5), np.arange(FAR + 13.5, 70000, 7.25)])


def test_bound_value():
    assert abs(BOUND - 5.3e-5) < 1e-6


def test_expansion_error_within_the_stated_bound_fp64():
    d0 = _far_centres()[:, None]
    exact = -np.sqrt(d0 - DL[None, :])
    approx = -np.sqrt(d0) + DL / (2 * np.sqrt(d0)) + DL ** 2 / (8 * d0 ** 1.5)
    err = np.abs(approx - exact)
    assert err.max() <= BOUND
    # the bound is tight to within a factor ~1.1 at the nearest far tile
    assert err.max() >= 0.8 * BOUND


def test_expansion_as_the_kernel_evaluates_it_fp32():
    # fp32, one reciprocal square root per half, Horner in dl, as in the kernel
    # (slope 1): b0 = -d0 * rs, b1 = 0.5 rs, b2 = 0.25 b1 rs^2
    d0 = _far_centres().astype(np.float32)[:, None]
    rs = (1.0 / np.sqrt(d0.astype(np.float64))).astype(np.float32)
    b0 = -d0 * rs
    b1 = np.float32(0.5) * rs
    b2 = np.float32(0.25) * b1 * rs * rs
    dl = DL.astype(np.float32)[None, :]
    approx = (b2 * dl + b1) * dl + b0
    exact = -np.sqrt(d0.astype(np.float64) - DL[None, :])
    err = np.abs(approx.astype(np.float64) - exact)
    # the remainder plus fp32 rounding of values up to sqrt(70000) ~ 265
    assert err.max() <= BOUND + 4 * np.finfo(np.float32).eps * 265


def test_nearer_tiles_would_break_the_bound():
    # the threshold matters: at a distance of 64 the same expansion errs by far
    # more than the bound (the kernel takes the exact square root there)
    d0 = np.array([[64 + 13.5]])
    exact = -np.sqrt(d0 - DL[None, :])
    approx = -np.sqrt(d0) + DL / (2 * np.sqrt(d0)) + DL ** 2 / (8 * d0 ** 1.5)
    assert np.abs(approx - exact).max() > 10 * BOUND

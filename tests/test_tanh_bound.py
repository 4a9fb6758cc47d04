"""The softcap's tanh (csrc/ce_device.hpp: tanh_poly below the split,
tanh_exp above it) against its stated error bounds, evaluated on the CPU in
emulated fp32: every operation is rounded to fp32 as the kernel's are (fused
multiply-adds once), the hardware exp2 and reciprocal are taken as correctly
rounded. The coefficients are read from the kernel source, so the test covers
the constants the GPU uses."""

import os
import re

import numpy as np

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "softmax_cross_entropy_amd", "csrc", "ce_device.hpp")
F = np.float32


def _consts():
    s = open(SRC).read()
    q = [float(re.search(rf"kTanhQ{i} = ([-0-9.e]+)f;", s).group(1)) for i in range(1, 6)]
    split = float(re.search(r"kTanhSplit = ([0-9.]+)f;", s).group(1))
    return [F(c) for c in q], F(split)


def _fma(a, b, c):
    return F(np.float64(a) * np.float64(b) + np.float64(c))


def tanh_poly32(u):
    q, _ = _consts()
    u = F(u)
    s = F(u * u)
    acc = q[4]
    for c in (q[3], q[2], q[1], q[0]):
        acc = _fma(acc, s, c)
    return _fma(F(u * s), acc, u)


def tanh_exp32(u):
    u = F(u)
    au = F(abs(u))
    a = F(15.0) if au > F(15.0) else au        # NaN fails the test: not clamped
    d = F(F(np.exp2(np.float64(F(a * F(2.0 * 1.4426950408889634))))) + F(1.0))
    r = F(1.0 / np.float64(d))
    r = _fma(r, _fma(-d, r, F(1.0)), r)
    return F(np.copysign(_fma(F(-2.0), r, F(1.0)), u))


def test_polynomial_fit_bound_exact_arithmetic():
    q, split = _consts()
    u = np.linspace(1e-6, float(split), 100001)
    s = u * u
    acc = float(q[4])
    for c in (q[3], q[2], q[1], q[0]):
        acc = acc * s + float(c)
    rel = np.abs(u + u * s * acc - np.tanh(u)) / np.tanh(u)
    assert rel.max() <= 3.5e-9, rel.max()


def test_polynomial_branch_fp32_relative_error():
    _, split = _consts()
    us = np.concatenate([np.linspace(1e-30, 1e-3, 300), np.linspace(1e-3, float(split), 3000)])
    worst = 0.0
    for u in us:
        for v in (u, -u):
            t = float(tanh_poly32(v))
            rel = abs(t - np.tanh(float(F(v)))) / abs(np.tanh(float(F(v))))
            worst = max(worst, rel)
    assert worst <= 1e-7, worst


def test_exponential_branch_fp32_error_and_saturation():
    _, split = _consts()
    worst = 0.0
    for u in np.concatenate([np.linspace(float(split), 9.0, 4000), [15.0, 40.0, 1e30]]):
        for v in (u, -u):
            t = float(tanh_exp32(v))
            ref = np.tanh(float(F(v)))
            worst = max(worst, abs(t - ref) / abs(ref))
    assert worst <= 2e-7, worst
    assert tanh_exp32(np.inf) == 1.0 and tanh_exp32(-np.inf) == -1.0
    assert tanh_exp32(1e30) == 1.0


def test_nan_propagates_on_both_branches():
    assert np.isnan(tanh_poly32(np.nan))
    assert np.isnan(tanh_exp32(np.nan))


def test_branches_agree_at_the_split():
    _, split = _consts()
    below = float(tanh_poly32(np.nextafter(split, F(0))))
    above = float(tanh_exp32(split))
    assert abs(above - below) / above <= 4e-7

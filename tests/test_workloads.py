"""The seeded input generators: deterministic, row-addressable, thread-count independent,
and of the stated shapes and distributions."""
from __future__ import annotations

import os

import numpy as np

import workloads


def f32(b):
    return (b.astype(np.uint32) << 16).view(np.float32)


def test_rows_are_independent_of_how_they_are_generated(monkeypatch):
    full = workloads.rows(2, 1, 0, 40, 7168)
    part = workloads.rows(2, 1, 17, 5, 7168)
    assert np.array_equal(full[17:22], part)
    monkeypatch.setenv("OMP_NUM_THREADS", "1")
    one = workloads.rows(2, 1, 0, 40, 7168)
    assert np.array_equal(full, one)


def test_ranks_and_configs_differ():
    a = workloads.rows(2, 0, 0, 4, 1024)
    b = workloads.rows(2, 1, 0, 4, 1024)
    c = workloads.rows(3, 0, 0, 4, 1024)
    assert not np.array_equal(a, b) and not np.array_equal(a, c)


def test_shapes():
    assert workloads.shape(1) == (512, 7168)
    assert workloads.shape(2) == (3072, 7168)
    assert workloads.shape(3) == (3072, 7168)
    assert workloads.shape(4) == (4096, 7168)
    assert workloads.shape(5) == (16384, 7168)


def test_distributions():
    x = f32(workloads.rows(2, 0, 0, 64, 7168)).astype(np.float64)
    assert abs(x.std() - 0.5) < 0.01 and abs(x.mean()) < 0.01
    t = f32(workloads.rows(3, 0, 0, 64, 7168)).astype(np.float64)
    assert abs(np.median(np.abs(t)) - 0.3 * 0.741) < 0.01        # median |t4| ~ 0.741
    c1 = f32(workloads.tensor(1, 0)).reshape(-1, 128).astype(np.float64)
    zero = np.all(c1 == 0, axis=1)
    assert 0.015 < zero.mean() < 0.025
    big = np.abs(c1[~zero]) > 6
    assert 3e-4 < big.mean() < 2e-3                                # the x50 outliers
    g = f32(workloads.rows(4, 0, 0, 256, 512)).astype(np.float64)
    rms = np.sqrt((g ** 2).mean(axis=1))
    assert rms.min() > 1e-4 and rms.max() < 2e2 and rms.max() / rms.min() > 1e3


def test_zero_blocks_coincide_across_ranks():
    z = [np.all(workloads.rows(5, r, 0, 8, 7168).reshape(-1, 128) == 0, axis=1) for r in range(4)]
    assert z[0].any()
    for r in range(1, 4):
        assert np.array_equal(z[0], z[r])
    y = workloads.rows(5, 0, 0, 8, 7168)
    assert not np.array_equal(y, workloads.rows(5, 1, 0, 8, 7168))


def test_truncation_not_rounding():
    # the generator truncates binary32 to bf16; it must never produce NaN or inf
    x = workloads.rows(5, 2, 0, 64, 7168)
    assert np.all(((x >> 7) & 0xFF) != 0xFF)


def test_f16_mode_truncates_the_same_draws():
    """The binary16 mode draws the same doubles as the bf16 mode and truncates them toward
    zero: signs agree, and the two truncations of one value differ by less than a bf16
    ulp plus a binary16 subnormal step."""
    a = workloads.rows(4, 3, 0, 32, 1024, fmt="f16")
    b = workloads.rows(4, 3, 0, 32, 1024)
    fa = a.view(np.float16).astype(np.float64)
    fb = (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.all(np.isfinite(fa))
    assert np.all((fa == 0) | (fb == 0) | (np.sign(fa) == np.sign(fb)))
    assert np.all(np.abs(fa - fb) <= np.abs(fb) * 2.0 ** -7 + 2.0 ** -24)
    assert np.array_equal(workloads.rows(4, 3, 5, 2, 1024, fmt="f16"), a[5:7])

"""Pins of the numerical-quality report's arithmetic (bench.py --quality):
closed forms for the relative L2 error, SNR, cosine and bias."""

import math
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def test_scaled_copy():
    # c = (1 + eps) ref: rel L2 = eps, cosine = 1, bias = eps * mean(ref) / rms(ref)
    ref = np.array([3.0, -4.0, 12.0, 0.0])                 # norm 13, rms 6.5, mean 2.75
    m = bench.quality_metrics(1.01 * ref, ref)
    assert math.isclose(m["rel_l2"], 0.01, rel_tol=1e-9)
    assert math.isclose(m["snr_db"], 40.0, abs_tol=1e-9)
    assert m["cosine"] == 1.0
    assert math.isclose(m["bias"], round(0.01 * 2.75 / 6.5, 7), abs_tol=1e-12)


def test_orthogonal_error():
    # c = ref + n with n orthogonal to ref: rel L2 = |n|/|ref|, cosine = 1/sqrt(1 + rl2^2)
    ref = np.array([1.0, 1.0, 0.0, 0.0])
    n = np.array([0.5, -0.5, 0.0, 0.0])                    # |n| / |ref| = 0.5, mean(n) = 0
    m = bench.quality_metrics(ref + n, ref)
    assert math.isclose(m["rel_l2"], 0.5, rel_tol=1e-9)
    assert math.isclose(m["snr_db"], round(-20 * math.log10(0.5), 2), abs_tol=1e-9)
    assert math.isclose(m["cosine"], round(1 / math.sqrt(1.25), 7), abs_tol=1e-12)
    assert m["bias"] == 0.0


def test_sign_flip_and_constant_offset():
    ref = np.array([2.0, -2.0, 2.0, -2.0])                 # mean 0, rms 2
    m = bench.quality_metrics(-ref, ref)
    assert math.isclose(m["rel_l2"], 2.0, rel_tol=1e-9) and m["cosine"] == -1.0
    m = bench.quality_metrics(ref + 0.5, ref)               # a pure bias: 0.5 / rms 2
    assert math.isclose(m["bias"], 0.25, rel_tol=1e-9)
    assert math.isclose(m["rel_l2"], 0.25, rel_tol=1e-9)

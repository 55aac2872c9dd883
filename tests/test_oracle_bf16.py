"""Pins for the oracle's bf16 conversions (CPU only).

* fp32 -> bf16 (nearest, ties to even) against torch's CPU conversion, a
  library routine, over every one of the 2^32 binary32 bit patterns.
* bf16 -> fp32 widening against torch.
* fp64 -> bf16 single rounding against exact rational rounding.
"""
from fractions import Fraction
import random
import struct

import numpy as np
import pytest
import torch

import oracle
from tests import exact


def test_f32_to_bf16_exhaustive_vs_torch():
    n = 1 << 26
    for c in range(1 << 6):
        u = (np.arange(n, dtype=np.uint64) + np.uint64(c * n)).astype(np.uint32)
        f = u.view(np.float32)
        ours = oracle.f32_to_bf16(f)
        ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        nan = np.isnan(f)
        assert np.array_equal(ours[~nan], ref[~nan]), f"chunk {c}"
        # NaN stays NaN, sign kept
        o = ours[nan]
        assert np.all((o & 0x7F80) == 0x7F80) and np.all((o & 0x7F) != 0)
        assert np.array_equal(o >> 15, (u[nan] >> 31).astype(np.uint16))


def test_bf16_to_f32_all_patterns():
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_to_f32(h)
    ref = torch.from_numpy(h.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin].view(np.uint32), ref[fin].view(np.uint32))
    # round trip is the identity on non-NaN patterns
    back = oracle.f32_to_bf16(ours)
    assert np.array_equal(back[fin], h[fin])


def test_f64_to_bf16_vs_exact_rounding():
    rng = random.Random(7)
    cases = []
    for _ in range(3000):
        e = rng.randint(-120, 120)
        cases.append(rng.uniform(-1, 1) * 2.0 ** e)
    # exact ties at bf16 precision, and values a hair either side of them
    for _ in range(500):
        e = rng.randint(-100, 100)
        m = rng.randint(128, 255)
        tie = (m + 0.5) * 2.0 ** (e - 7)
        cases += [tie, -tie, np.nextafter(tie, np.inf), np.nextafter(tie, -np.inf)]
    for d in cases:
        want = exact.fraction_to_bf16_bits(exact.round_to_bf16(Fraction(d)))
        assert oracle.f64_to_bf16_scalar(d) == want, d


def test_f64_to_bf16_matches_single_rounding_of_f32_values():
    # For a double that is exactly a binary32, a single rounding to bf16 is
    # what torch's fp32 -> bf16 conversion does.
    rng = np.random.default_rng(3)
    f = (rng.standard_normal(20000) * np.exp2(rng.integers(-60, 60, 20000))).astype(np.float32)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = np.array([oracle.f64_to_bf16_scalar(float(v)) for v in f], np.uint16)
    assert np.array_equal(ours, ref)


@pytest.mark.parametrize("d,bits", [(0.0, 0x0000), (-0.0, 0x8000), (1.0, 0x3F80),
                                    (float("inf"), 0x7F80), (-float("inf"), 0xFF80),
                                    (3.5e38, 0x7F80)])
def test_f64_to_bf16_special(d, bits):
    assert oracle.f64_to_bf16_scalar(d) == bits


def test_exact_helper_self_check():
    # the rational rounding agrees with struct's fp32 conversion on random doubles
    rng = random.Random(11)
    for _ in range(2000):
        d = rng.uniform(-1, 1) * 2.0 ** rng.randint(-100, 100)
        f = struct.unpack("<f", struct.pack("<f", d))[0]
        assert exact.round_to_f32(Fraction(d)) == Fraction(f)

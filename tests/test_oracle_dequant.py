"""Pins for the oracle's nibble packing and dequantisation (CPU only).

Dequantisation reads w = alpha * LUT[idx] + beta (the inverse of the
normalisation w_s = (w - beta) / alpha in the 10100.com any4 explainer,
step 2) rounded once to fp32 and then to bf16.  Pins:
  * exact rational evaluation with the two roundings, on tiny inputs and
    on crafted rounding ties;
  * an identity table turns any4 into plain asymmetric int4 (the uniform map
    F = S (Q - Z) of the anything-llm INT4/INT8 article), computed here with
    numpy float32 and torch, not with the oracle;
  * exact scaling by powers of two, table/index permutation invariance,
    alpha = 0 gives beta, and group boundaries land at multiples of g.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import exact


def _rand_inputs(seed, N, K, g):
    return workloads.generic(seed, 1, N, K, g)


def test_pack_roundtrip_and_layout():
    rng = np.random.default_rng(0)
    idx = rng.integers(0, 16, size=(7, 34), dtype=np.uint8)
    p = oracle.pack(idx)
    assert p.shape == (7, 17)
    assert np.array_equal(oracle.unpack(p, 34), idx)
    # byte j: index 2j in the low nibble, 2j+1 in the high nibble
    assert p[3, 5] == idx[3, 10] + 16 * idx[3, 11]
    # only the low 4 bits of an index count
    assert np.array_equal(oracle.pack(idx | 0xF0), p)


def test_pack_brute_force_all_byte_values():
    lo, hi = np.meshgrid(np.arange(16), np.arange(16), indexing="ij")
    idx = np.stack([lo.ravel(), hi.ravel()], axis=1).astype(np.uint8).reshape(1, 512)
    p = oracle.pack(idx).ravel()
    assert sorted(p.tolist()) == list(range(256))
    for b in range(256):
        assert int(p[b]) == int(idx[0, 2 * b]) | (int(idx[0, 2 * b + 1]) << 4)


def _exact_dequant_bits(a, l, b):
    v = exact.bf16_bits_to_fraction(a) * exact.bf16_bits_to_fraction(l) + \
        exact.bf16_bits_to_fraction(b)
    return exact.fraction_to_bf16_bits(exact.round_to_bf16(exact.round_to_f32(v)))


def test_dequant_one_exact_rational_random():
    rng = np.random.default_rng(1)
    a = workloads.to_bf16_bits(rng.uniform(-3, 3, 3000) * np.exp2(rng.integers(-20, 5, 3000)))
    l = workloads.to_bf16_bits(rng.standard_normal(3000) * np.exp2(rng.integers(-20, 5, 3000)))
    b = workloads.to_bf16_bits(rng.standard_normal(3000) * np.exp2(rng.integers(-25, 5, 3000)))
    for i in range(3000):
        assert oracle.dequant_one(int(a[i]), int(l[i]), int(b[i])) == \
            _exact_dequant_bits(int(a[i]), int(l[i]), int(b[i]))


def test_dequant_one_exact_rational_ties():
    # alpha*L lands exactly half way between two bf16 values when beta = 0:
    # 8-bit x 8-bit significands give up to 16 bits; pick products whose 9th
    # significant bit is the last one set.
    rng = np.random.default_rng(2)
    hits = 0
    for _ in range(20000):
        a = int(rng.integers(0x3F80, 0x3FFF))      # significands in [1, 2)
        l = int(rng.integers(0x3F80, 0x3FFF))
        v = exact.bf16_bits_to_fraction(a) * exact.bf16_bits_to_fraction(l)   # in [1, 4)
        want = _exact_dequant_bits(a, l, 0)
        assert oracle.dequant_one(a, l, 0) == want
        # a tie: v sits exactly half way between two bf16 neighbours
        e = 1 if v >= 2 else 0
        scaled = v / Fraction(2) ** (e - 7)
        if scaled.denominator == 2:
            hits += 1
    assert hits > 100     # the sweep really exercised ties


def test_identity_lut_is_int4_asymmetric():
    """LUT[i] = i: w = alpha*q + beta = S*(q - Z) with S = alpha, Z = -beta/alpha."""
    inp = _rand_inputs(3, 32, 256, 128)
    lut = np.tile(workloads.to_bf16_bits(np.arange(16.0)), (32, 1))
    w = oracle.dequant(oracle.pack(inp.idx), lut, inp.alpha, inp.beta, 128)
    # independent three-line int4 dequant: float32 multiply-add, torch bf16
    S = workloads.bf16_bits_to_f64(inp.alpha).astype(np.float32).repeat(128, axis=1)
    B = workloads.bf16_bits_to_f64(inp.beta).astype(np.float32).repeat(128, axis=1)
    ref = workloads.to_bf16_bits(S * inp.idx.astype(np.float32) + B)
    assert np.array_equal(w, ref)


def test_signed_int4_grid():
    """LUT[i] = i - 8 (int4 range -8..7) equals the identity grid with beta - 8*alpha."""
    inp = _rand_inputs(4, 16, 256, 128)
    a = workloads.to_bf16_bits(np.full((16, 2), 0.125))       # exact power of two
    b = workloads.to_bf16_bits(np.full((16, 2), 1.5))
    signed = np.tile(workloads.to_bf16_bits(np.arange(16.0) - 8), (16, 1))
    ident = np.tile(workloads.to_bf16_bits(np.arange(16.0)), (16, 1))
    b_shift = workloads.to_bf16_bits(np.full((16, 2), 1.5 - 8 * 0.125))
    p = oracle.pack(inp.idx)
    assert np.array_equal(oracle.dequant(p, signed, a, b, 128),
                          oracle.dequant(p, ident, a, b_shift, 128))


@pytest.mark.parametrize("j", [-3, 1, 4])
def test_power_of_two_scaling(j):
    inp = _rand_inputs(5, 24, 512, 128)
    p = oracle.pack(inp.idx)
    w = workloads.bf16_bits_to_f64(oracle.dequant(p, inp.lut, inp.alpha, inp.beta, 128))
    s = 2.0 ** j
    a2 = workloads.to_bf16_bits(workloads.bf16_bits_to_f64(inp.alpha) * s)
    b2 = workloads.to_bf16_bits(workloads.bf16_bits_to_f64(inp.beta) * s)
    w2 = workloads.bf16_bits_to_f64(oracle.dequant(p, inp.lut, a2, b2, 128))
    assert np.array_equal(w2, w * s)


def test_permutation_invariance():
    inp = _rand_inputs(6, 20, 384, 128)
    rng = np.random.default_rng(6)
    lut2 = inp.lut.copy()
    idx2 = inp.idx.copy()
    for n in range(20):
        pi = rng.permutation(16)
        lut2[n, pi] = inp.lut[n]           # LUT'[pi(i)] = LUT[i]
        idx2[n] = pi[inp.idx[n]]           # idx' = pi(idx)
    w1 = oracle.dequant(oracle.pack(inp.idx), inp.lut, inp.alpha, inp.beta, 128)
    w2 = oracle.dequant(oracle.pack(idx2), lut2, inp.alpha, inp.beta, 128)
    assert np.array_equal(w1, w2)


def test_alpha_zero_gives_beta():
    inp = _rand_inputs(7, 8, 256, 128)
    z = np.zeros_like(inp.alpha)
    w = oracle.dequant(oracle.pack(inp.idx), inp.lut, z, inp.beta, 128)
    assert np.array_equal(w, inp.beta.repeat(128, axis=1))


@pytest.mark.parametrize("g", [128, 256])
def test_group_boundaries(g):
    """alpha nonzero in group j only, constant LUT, beta 0: w != 0 exactly on group j."""
    N, K = 4, 1024
    rng = np.random.default_rng(8)
    idx = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    lut = np.tile(workloads.to_bf16_bits(np.full(16, 1.0)), (N, 1))
    G = K // g
    for j in range(G):
        a = np.zeros((N, G), np.uint16)
        a[:, j] = workloads.to_bf16_bits(np.array([0.5]))[0]
        w = oracle.dequant(oracle.pack(idx), lut, a, np.zeros((N, G), np.uint16), g)
        nz = np.nonzero(w[0])[0]
        assert nz.min() == j * g and nz.max() == (j + 1) * g - 1 and nz.size == g
        assert np.all(w[:, j * g:(j + 1) * g] == 0x3F00)


def test_lut_lookup_uses_own_row():
    """Row n's weights use row n's table (not a transposed or shared table)."""
    N, K = 16, 128
    idx = np.full((N, K), 5, np.uint8)
    lut = np.zeros((N, 16), np.uint16)
    lut[:, 5] = workloads.to_bf16_bits(np.arange(N, dtype=np.float64) + 1)
    one = workloads.to_bf16_bits(np.ones((N, 1)))
    w = oracle.dequant(oracle.pack(idx), lut, one, np.zeros((N, 1), np.uint16), 128)
    assert np.array_equal(workloads.bf16_bits_to_f64(w), np.repeat(np.arange(1.0, N + 1)[:, None],
                                                                   K, axis=1))

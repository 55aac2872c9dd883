"""The seeded input generators: determinism, shapes and value ranges (CPU only)."""
import numpy as np

import workloads


def test_deterministic_bytes():
    a = workloads.generate(0)
    b = workloads.generate(0)
    for f in ("idx", "lut", "alpha", "beta", "x"):
        assert np.array_equal(getattr(a, f), getattr(b, f))


def test_config0_shapes_and_ranges():
    c = workloads.generate(0)
    assert c.idx.shape == (512, 512) and c.idx.dtype == np.uint8 and c.idx.max() == 15
    assert c.lut.shape == (512, 16) and c.alpha.shape == (512, 4) and c.x.shape == (1, 512)
    L = workloads.bf16_bits_to_f64(c.lut)
    assert np.all(np.diff(L, axis=1) >= 0)                     # sorted rows
    A = workloads.bf16_bits_to_f64(c.alpha)
    assert A.min() >= 0.005 * (1 - 2 ** -8) and A.max() <= 0.02 * (1 + 2 ** -8)
    assert abs(workloads.bf16_bits_to_f64(c.beta).std() - 0.002) < 3e-4
    assert np.bincount(c.idx.ravel(), minlength=16).min() > 0.9 * c.idx.size / 16


def test_config1_outlier_channels():
    c = workloads.generate(1)
    X = np.abs(workloads.bf16_bits_to_f64(c.x[0]))
    # round(0.01 * 4096) = 41 channels scaled by 20
    assert (X > 8).sum() >= 30 and (X > 8).sum() <= 41 + 2


def test_resized_generation_and_prefix_rows():
    c16 = workloads.generate(2, N=64, K=256)
    assert c16.x.shape == (16, 256) and c16.idx.shape == (64, 256)
    g = workloads.generic(5, 3, 40, 384, 128)
    assert g.x.shape == (3, 384) and g.alpha.shape == (40, 3)


def test_config3_student_t_tables_heavier_tails():
    c = workloads.generate(3, N=2048, K=1024)
    L = workloads.bf16_bits_to_f64(c.lut)
    n = workloads.bf16_bits_to_f64(workloads.generate(0).lut)
    assert np.abs(L[:, 0]).mean() > np.abs(n[:, 0]).mean()


def test_raw_layer_prefix_rows_identical():
    # the draw does not depend on how many rows are kept
    r = workloads.raw_layer("qkvo", rows=4)
    assert r.W.shape == (4, 8192) and r.Ex.shape == (8192,) and r.x.shape == (16, 8192)
    assert np.all(r.Ex > 0)


def test_fixed_tables():
    """The baseline 4-bit formats as tables: int4 is the integer grid, fp4 is
    E2M1 (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6, sign in bit 3), nf4 is a
    sorted normal-quantile grid spanning [-1, 1] with an exact zero."""
    f = workloads.bf16_bits_to_f64
    assert np.array_equal(f(workloads.fixed_table("int4")), np.arange(16.0))
    fp4 = f(workloads.fixed_table("fp4"))
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    assert np.array_equal(fp4[:8], mags) and np.array_equal(fp4[8:], -mags)
    assert workloads.fixed_table("fp4")[8] == 0x8000          # -0
    nf4 = f(workloads.fixed_table("nf4"))
    assert nf4[0] == -1.0 and nf4[15] == 1.0 and nf4[7] == 0.0
    assert np.all(np.diff(nf4) > 0)
    # quantile spacing: the steps grow towards the tails on both sides
    d = np.diff(nf4)
    assert np.all(np.diff(d[8:]) > 0) and np.all(np.diff(d[:7]) < 0)

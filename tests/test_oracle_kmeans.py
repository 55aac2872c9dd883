"""Pins for the oracle's any4 quantiser (group scale + weighted k-means), CPU only.

The 10100.com any4 explainer, step 2, describes an E-step (each weight goes
to the nearest of the 16 table values) and an M-step
L_q = sum(alpha * w_s * E|x|) / sum(alpha * E|x|), repeated until
convergence.  Pins:
  * it is weighted Lloyd's algorithm: scikit-learn's KMeans (lloyd, the
    same initial centres, sample_weight = alpha * E|x|) gives the same
    centres and labels;
  * the weighted objective never increases over E and M steps;
  * zero rounds reduce to uniform asymmetric int4 rounding Q = round(F/S + Z)
    (the anything-llm INT4/INT8 article), computed here independently;
  * a row whose values sit near distinct integers converges in one round to
    zero error; a converged row is a fixed point; scaling E|x| by a power of
    two leaves the table unchanged;
  * any3 / any2 (8 / 4 table values): the same weighted Lloyd's algorithm
    against scikit-learn, zero rounds as the uniform 3- / 2-bit grid, the
    objective non-increasing, and the stored table and indices consistent.
"""
import warnings

import numpy as np
import pytest

import oracle
import workloads


def _row(seed, K=2048):
    rng = np.random.default_rng(seed)
    ws = np.concatenate([rng.uniform(0, 15, K // 2),
                         np.clip(rng.normal(7.5, 3.0, K - K // 2), 0, 15)])
    wt = rng.lognormal(0, 1, K) * rng.uniform(0.5, 2.0, K)
    return ws, wt


@pytest.mark.parametrize("seed,iters", [(0, 1), (1, 3), (2, 10), (3, 25)])
def test_matches_sklearn_weighted_lloyd(seed, iters):
    from sklearn.cluster import KMeans
    ws, wt = _row(seed)
    L, idx = oracle.kmeans_row(ws, wt, iters)
    assert np.bincount(idx, minlength=16).min() > 0   # no empty cluster (sklearn relocates)
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")
        km = KMeans(n_clusters=16, init=np.arange(16.0).reshape(-1, 1), n_init=1,
                    max_iter=iters, tol=0.0, algorithm="lloyd")
        km.fit(ws.reshape(-1, 1), sample_weight=wt)
    assert np.allclose(km.cluster_centers_.ravel(), L, rtol=1e-12, atol=1e-12)
    # sklearn's labels_ come from a final E-step against its final centres
    L1, idx_final = oracle.kmeans_row(ws, wt, 0, init=L)
    assert np.array_equal(km.labels_, idx_final)


def test_objective_non_increasing():
    ws, wt = _row(5, K=4096)
    _, _, tr = oracle.kmeans_row(ws, wt, 15, trace=True)
    assert np.all(np.diff(tr) <= 1e-9 * tr[0])
    assert tr[-1] < tr[0]


def test_zero_rounds_is_uniform_int4():
    # group scale then nearest integer grid point = Q = round(F/S + Z), clamped
    rng = np.random.default_rng(6)
    N, K, g = 8, 512, 128
    W = rng.normal(0, 0.02, (N, K))
    Ex = np.ones(K)
    idx, lut, a, b = oracle.kmeans_quantize(W, Ex, g, iters=0, nthreads=2)
    assert np.array_equal(lut, np.tile(workloads.to_bf16_bits(np.arange(16.0)), (N, 1)))
    S = workloads.bf16_bits_to_f64(a).repeat(g, axis=1)
    Z = -workloads.bf16_bits_to_f64(b).repeat(g, axis=1) / S
    F = W
    v = F / S + Z
    q = np.clip(np.ceil(v - 0.5), 0, 15)            # halves go to the lower index
    ok = np.abs(v - np.round(v)) != 0.5             # avoid exact fp64 halves
    assert np.array_equal(idx[ok], q[ok].astype(np.uint8))


def test_group_scale_spans_index_range():
    rng = np.random.default_rng(7)
    W = rng.normal(0, 0.02, (6, 1024))
    a, b = oracle.group_scale(W, 128)
    A = workloads.bf16_bits_to_f64(a).repeat(128, axis=1)
    B = workloads.bf16_bits_to_f64(b).repeat(128, axis=1)
    ws = (W - B) / A
    lo = ws.reshape(6, 8, 128).min(axis=2)
    hi = ws.reshape(6, 8, 128).max(axis=2)
    # bf16 keeps 8 bits: beta within 2^-8 relative of the min, alpha likewise
    assert np.all(np.abs(lo) < 15 * 2.0 ** -7)
    assert np.all(np.abs(hi - 15) < 15 * 2.0 ** -6)


def test_near_integer_row_converges_to_zero_error():
    rng = np.random.default_rng(8)
    centres = np.arange(16) + rng.uniform(-0.4, 0.4, 16)
    ws = np.repeat(centres, 50) + 0.0
    wt = rng.uniform(0.1, 3.0, ws.size)
    L, idx, tr = oracle.kmeans_row(ws, wt, 1, trace=True)
    assert np.allclose(L, centres, rtol=0, atol=1e-13)
    assert tr[-1] < 1e-20


def test_fixed_point_after_convergence():
    ws, wt = _row(9)
    L, idx = oracle.kmeans_row(ws, wt, 200)
    L2, idx2 = oracle.kmeans_row(ws, wt, 1, init=L)
    assert np.array_equal(L, L2) and np.array_equal(idx, idx2)


def test_importance_scale_invariance():
    ws, wt = _row(10)
    L1, i1 = oracle.kmeans_row(ws, wt, 10)
    L2, i2 = oracle.kmeans_row(ws, wt * 4.0, 10)
    assert np.array_equal(L1, L2) and np.array_equal(i1, i2)


def test_importance_pulls_the_table():
    # one heavily weighted point drags its cluster centre onto itself
    ws = np.array([2.0, 2.2, 2.4, 7.0])
    wt = np.array([1.0, 1.0, 1000.0, 1.0])
    L, idx = oracle.kmeans_row(ws, wt, 1)
    assert idx[0] == idx[1] == idx[2] == 2
    assert abs(L[2] - (2.0 + 2.2 + 2400.0) / 1002.0) < 1e-12


def test_quantize_consistency():
    rng = np.random.default_rng(11)
    N, K, g = 5, 1024, 128
    W = rng.normal(0, 0.02, (N, K))
    W[rng.random((N, K)) < 0.001] *= 10
    Ex = rng.lognormal(0, 1, K)
    idx, lut, a, b = oracle.kmeans_quantize(W, Ex, g, iters=10, nthreads=3)
    A = workloads.bf16_bits_to_f64(a).repeat(g, axis=1)
    B = workloads.bf16_bits_to_f64(b).repeat(g, axis=1)
    ws = np.where(A != 0, (W - B) / np.where(A != 0, A, 1), 0)
    Lq = workloads.bf16_bits_to_f64(lut)
    for n in range(N):
        # stored table = bf16 of the fp64 k-means table of this row
        L, _ = oracle.kmeans_row(ws[n], A[n] * Ex, 10)
        assert np.array_equal(lut[n], np.array([oracle.f64_to_bf16_scalar(v) for v in L]))
        # indices are the nearest stored value
        d = np.abs(ws[n][:, None] - Lq[n][None, :])
        assert np.all(d[np.arange(K), idx[n]] <= d.min(axis=1))
    # k-means beats the int4 grid on the weighted objective
    idx0, _, _, _ = oracle.kmeans_quantize(W, Ex, g, iters=0, nthreads=1)
    wt = A * Ex
    J = (wt * (ws - Lq[np.arange(N)[:, None], idx]) ** 2).sum()
    J0 = (wt * (ws - idx0) ** 2).sum()
    assert J < 0.8 * J0


def test_thread_count_does_not_change_quantisation():
    rng = np.random.default_rng(12)
    W = rng.normal(0, 0.02, (9, 256))
    Ex = rng.lognormal(0, 1, 256)
    r1 = oracle.kmeans_quantize(W, Ex, 128, 10, nthreads=1)
    r4 = oracle.kmeans_quantize(W, Ex, 128, 10, nthreads=4)
    for u, v in zip(r1, r4):
        assert np.array_equal(u, v)


# ---- any3 / any2: the same quantiser with 8 / 4 table values ---------------
@pytest.mark.parametrize("levels,seed,iters", [(8, 20, 3), (8, 21, 10), (4, 22, 1), (4, 23, 10)])
def test_low_bit_matches_sklearn_weighted_lloyd(levels, seed, iters):
    from sklearn.cluster import KMeans
    rng = np.random.default_rng(seed)
    K = 2048
    ws = np.concatenate([rng.uniform(0, levels - 1, K // 2),
                         np.clip(rng.normal((levels - 1) / 2, levels / 5, K - K // 2), 0,
                                 levels - 1)])
    wt = rng.lognormal(0, 1, K)
    L, idx = oracle.kmeans_row(ws, wt, iters, levels=levels)
    assert idx.max() < levels and np.bincount(idx, minlength=levels).min() > 0
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")
        km = KMeans(n_clusters=levels, init=np.arange(float(levels)).reshape(-1, 1), n_init=1,
                    max_iter=iters, tol=0.0, algorithm="lloyd")
        km.fit(ws.reshape(-1, 1), sample_weight=wt)
    assert np.allclose(km.cluster_centers_.ravel(), L, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("bits", [3, 2])
def test_low_bit_zero_rounds_is_uniform_grid(bits):
    """Zero rounds: min-max onto [0, 2^bits - 1] and the nearest grid point,
    computed here independently; table entries past 2^bits are zero."""
    Q = 1 << bits
    rng = np.random.default_rng(30 + bits)
    N, K, g = 6, 512, 128
    W = rng.normal(0, 0.02, (N, K))
    idx, lut, a, b = oracle.kmeans_quantize(W, np.ones(K), g, iters=0, nthreads=2, bits=bits)
    grid = np.concatenate([np.arange(float(Q)), np.zeros(16 - Q)])
    assert np.array_equal(lut, np.tile(workloads.to_bf16_bits(grid), (N, 1)))
    # alpha = bf16((max - min) / (Q - 1)), beta = bf16(min): within bf16's
    # half-ulp (2^-9 relative) of the exact values
    Wg = W.reshape(N, K // g, g)
    lo, hi = Wg.min(axis=2), Wg.max(axis=2)
    assert np.all(np.abs(workloads.bf16_bits_to_f64(b) - lo) <= 2.0 ** -8 * np.abs(lo))
    step = (hi - lo) / (Q - 1)
    assert np.all(np.abs(workloads.bf16_bits_to_f64(a) - step) <= 2.0 ** -8 * step)
    S = workloads.bf16_bits_to_f64(a).repeat(g, axis=1)
    B = workloads.bf16_bits_to_f64(b).repeat(g, axis=1)
    v = (W - B) / S
    q = np.clip(np.ceil(v - 0.5), 0, Q - 1)
    ok = np.abs(v - np.round(v)) != 0.5
    assert np.array_equal(idx[ok], q[ok].astype(np.uint8))
    assert idx.max() < Q


@pytest.mark.parametrize("bits", [3, 2])
def test_low_bit_objective_and_consistency(bits):
    Q = 1 << bits
    rng = np.random.default_rng(40 + bits)
    N, K, g = 4, 1024, 128
    W = rng.normal(0, 0.02, (N, K))
    Ex = rng.lognormal(0, 1, K)
    idx, lut, a, b = oracle.kmeans_quantize(W, Ex, g, iters=10, nthreads=2, bits=bits)
    A = workloads.bf16_bits_to_f64(a).repeat(g, axis=1)
    B = workloads.bf16_bits_to_f64(b).repeat(g, axis=1)
    ws = np.where(A != 0, (W - B) / np.where(A != 0, A, 1), 0)
    Lq = workloads.bf16_bits_to_f64(lut)
    assert np.all(lut[:, Q:] == 0) and idx.max() < Q
    for n in range(N):
        L, _, tr = oracle.kmeans_row(ws[n], A[n] * Ex, 10, trace=True, levels=Q)
        assert np.all(np.diff(tr) <= 1e-9 * tr[0])
        assert np.array_equal(lut[n, :Q], np.array([oracle.f64_to_bf16_scalar(v) for v in L]))
        d = np.abs(ws[n][:, None] - Lq[n][None, :Q])
        assert np.all(d[np.arange(K), idx[n]] <= d.min(axis=1))

"""Pins of the oracle's tile layout (CPU only).

The tile layout is the GPU library's own (its header states it); the oracle
restates it with a reshape and a transpose.  Here it is checked against the
per-byte definition, written out with plain loops, on small inputs."""
import numpy as np
import pytest

import oracle


def _tile_by_definition(idx: np.ndarray) -> np.ndarray:
    """byte 16*l + i of tile (b, c) = idx[n][k] | idx[n][k+1] << 4 with
    n = 16b + l % 16 and k = 128c + 32*(l // 16) + 2i; zero for n >= N."""
    N, K = idx.shape
    NB, Kc = -(-N // 16), K // 128
    out = np.zeros(NB * Kc * 1024, np.uint8)
    for b in range(NB):
        for c in range(Kc):
            for l in range(64):
                n = 16 * b + l % 16
                if n >= N:
                    continue
                for i in range(16):
                    k = 128 * c + 32 * (l // 16) + 2 * i
                    lo = int(idx[n, k]) & 15
                    hi = int(idx[n, k + 1]) & 15
                    out[(b * Kc + c) * 1024 + 16 * l + i] = lo | (hi << 4)
    return out


@pytest.mark.parametrize("N,K", [(1, 128), (16, 128), (17, 256), (37, 384), (48, 512)])
def test_tile_matches_the_per_byte_definition(N, K):
    rng = np.random.default_rng(N * 131 + K)
    idx = rng.integers(0, 256, size=(N, K), dtype=np.uint8)   # high bits are ignored
    t = oracle.tile(oracle.pack(idx))
    assert t.size == oracle.tiled_bytes(N, K)
    assert np.array_equal(t, _tile_by_definition(idx))


@pytest.mark.parametrize("N,K", [(5, 128), (33, 640), (64, 1024)])
def test_untile_inverts_tile(N, K):
    rng = np.random.default_rng(N + K)
    p = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    assert np.array_equal(oracle.untile(oracle.tile(p), N, K), p)


def test_one_tile_is_contiguous_per_lane():
    """Lane l of tile (0, 0) holds 32 consecutive k of row l % 16: the first
    byte pairs indices 32*(l//16) and 32*(l//16)+1."""
    N, K = 16, 128
    idx = np.zeros((N, K), np.uint8)
    for n in range(N):
        for k in range(K):
            idx[n, k] = (n + k) % 16
    t = oracle.tile(oracle.pack(idx))
    for l in range(64):
        n, k = l % 16, 32 * (l // 16)
        assert t[16 * l] == ((n + k) % 16) | (((n + k + 1) % 16) << 4)


# ---- any2: 2-bit codes, 512-byte tiles of 16 rows x 128 k -------------------
def _tile2_by_definition(idx: np.ndarray) -> np.ndarray:
    """byte 8*l + i of tile (b, c) = sum_s (idx[n][k + s] & 3) << 2s with
    n = 16b + l % 16 and k = 128c + 32*(l // 16) + 4i; zero for n >= N."""
    N, K = idx.shape
    NB, Kc = -(-N // 16), K // 128
    out = np.zeros(NB * Kc * 512, np.uint8)
    for b in range(NB):
        for c in range(Kc):
            for l in range(64):
                n = 16 * b + l % 16
                if n >= N:
                    continue
                for i in range(8):
                    k = 128 * c + 32 * (l // 16) + 4 * i
                    v = 0
                    for s in range(4):
                        v |= (int(idx[n, k + s]) & 3) << (2 * s)
                    out[(b * Kc + c) * 512 + 8 * l + i] = v
    return out


@pytest.mark.parametrize("N,K", [(1, 128), (16, 128), (17, 256), (37, 384)])
def test_tile2_matches_the_per_byte_definition(N, K):
    rng = np.random.default_rng(N * 7 + K)
    idx = rng.integers(0, 256, size=(N, K), dtype=np.uint8)   # bits above 1 are ignored
    t = oracle.tile2(oracle.pack2(idx))
    assert t.size == oracle.tiled2_bytes(N, K)
    assert np.array_equal(t, _tile2_by_definition(idx))


@pytest.mark.parametrize("N,K", [(5, 128), (33, 640)])
def test_pack2_round_trip(N, K):
    rng = np.random.default_rng(N + 3 * K)
    idx = rng.integers(0, 4, size=(N, K), dtype=np.uint8)
    p = oracle.pack2(idx)
    assert np.array_equal(oracle.unpack2(p, K), idx)
    assert np.array_equal(oracle.untile2(oracle.tile2(p), N, K), p)
    # all 256 byte values decode to their four 2-bit fields
    b = np.arange(256, dtype=np.uint8).reshape(1, 256)
    u = oracle.unpack2(b, 1024).reshape(256, 4)
    assert np.array_equal(u[:, 0] | (u[:, 1] << 2) | (u[:, 2] << 4) | (u[:, 3] << 6), b[0])


# ---- any3: 3-bit codes, 768-byte tiles of 16 rows x 128 k -------------------
def _tile3_by_bits(idx: np.ndarray) -> np.ndarray:
    """The any3 layout of include/any4.h, bit by bit: code bit e of
    code[n][k] (n = 16b + l % 16, k = 128c + 32*(l // 16) + r) is bit
    q = 3*(r % 2) + e of pair i = r // 2; pair i < 12 keeps bit q in byte i,
    bit q; pair 12 + t keeps bit q in byte 4*(q // 2) + t, bit 6 + q % 2."""
    N, K = idx.shape
    NB, Kc = -(-N // 16), K // 128
    out = np.zeros(NB * Kc * 768, np.uint8)
    for n in range(N):
        b, row = divmod(n, 16)
        for k in range(K):
            c, kk = divmod(k, 128)
            l = 16 * (kk // 32) + row
            r = kk % 32
            i = r // 2
            for e in range(3):
                if not (int(idx[n, k]) >> e) & 1:
                    continue
                q = 3 * (r % 2) + e
                if i < 12:
                    byte, bit = i, q
                else:
                    byte, bit = 4 * (q // 2) + (i - 12), 6 + q % 2
                out[(b * Kc + c) * 768 + 12 * l + byte] |= np.uint8(1 << bit)
    return out


@pytest.mark.parametrize("N,K", [(1, 128), (16, 128), (17, 256), (20, 384)])
def test_tile3_matches_the_per_bit_definition(N, K):
    rng = np.random.default_rng(N * 11 + K)
    idx = rng.integers(0, 256, size=(N, K), dtype=np.uint8)   # bits above 2 are ignored
    t = oracle.tile3(idx)
    assert t.size == oracle.tiled3_bytes(N, K) == -(-N // 16) * 16 * K * 3 // 8
    assert np.array_equal(t, _tile3_by_bits(idx & 7))


@pytest.mark.parametrize("N,K", [(5, 128), (33, 640), (16, 4096)])
def test_tile3_round_trip(N, K):
    rng = np.random.default_rng(N + 5 * K)
    idx = rng.integers(0, 8, size=(N, K), dtype=np.uint8)
    assert np.array_equal(oracle.untile3(oracle.tile3(idx), N, K), idx)


def test_tile3_worked_slot():
    """Row 0 with code[k] = k % 8, worked by hand from the layout: the pairs
    of lane 0 are 8, 26, 44, 62 (repeated), so pairs 12..15 are 8, 26, 44,
    62 and their top-bit parts are (0, 2, 0), (2, 2, 1), (0, 3, 2) and
    (2, 3, 3) for bytes (j, 4+j, 8+j)."""
    idx = (np.arange(128) % 8).astype(np.uint8)[None, :]
    t = oracle.tile3(idx)
    assert list(t[:12]) == [8, 154, 44, 190, 136, 154, 236, 254, 8, 90, 172, 254]
    # rows 1..15 are padding: their slots (lanes 1..15, 17..31, ...) are zero
    slots = t.reshape(4, 16, 12)
    assert not slots[:, 1:, :].any()
    # the four quarters of row 0 hold the same codes (k % 8 repeats every 32)
    assert all(np.array_equal(slots[q, 0], slots[0, 0]) for q in range(4))

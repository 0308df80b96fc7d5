"""Pins for O12, the prepacked weight layout: a bijection of the N*K bytes
in which every 2 KiB block is one whole 16-row x 128-column tile of B, the
blocks ordered by row group then K block, each block's two 1 KiB halves
holding every lane's two 16-byte K chunks (g and g + 4 of the 128-byte K
segment, g the lane group), the lanes of a half ordered lane group first (16
rows per group), and the rows of each 64-row group in the GEMM's fragment
order brow.  The device GEMM on prepacked B equalling the plain one bit for bit is
the remaining check (GPU tests)."""
import numpy as np

import oracle


def ids(N, K):
    return np.arange(N * K, dtype=np.int64).reshape(N, K)


def test_prepack_is_a_bijection():
    N, K = 256, 512
    out = oracle.bprepack(ids(N, K))
    assert out.size == N * K
    assert np.array_equal(np.sort(out), np.arange(N * K))


def test_prepack_blocks_are_whole_tiles_in_order():
    N, K = 64, 384
    KB = K // 128
    out = oracle.bprepack(ids(N, K)).reshape(-1, 2048)
    assert out.shape[0] == (N // 16) * KB
    for b in range(out.shape[0]):
        nt, kb = divmod(b, KB)
        rows, cols = np.divmod(out[b], K)
        assert set(rows) <= set(range(64 * (nt // 4), 64 * (nt // 4) + 64)) and len(set(rows)) == 16
        assert set(cols) == set(range(128 * kb, 128 * kb + 128))


def test_prepack_lane_segments():
    """Lane l of a block reads, over its two halves, two 16-byte chunks of one
    row: row brow(16 nt + l % 16), columns 16 g .. +16 and 64 + 16 g .. +16 of
    the K block (g = l / 16): the chunks the GEMM's LDS fragment reads give the
    same lane, so the MFMA sees the same bytes in the same slots."""
    N, K = 128, 256
    B = ids(N, K)
    out = oracle.bprepack(B).reshape(N // 16, K // 128, 2, 64, 16)
    rng = np.random.default_rng(0)
    for _ in range(64):
        nt, kb, l = rng.integers(0, N // 16), rng.integers(0, K // 128), rng.integers(0, 64)
        seg = np.concatenate([out[nt, kb, 0, l], out[nt, kb, 1, l]])
        r, g = int(oracle._brow(16 * nt + l % 16)), l // 16
        k0 = 128 * kb + 16 * g
        assert np.array_equal(seg, np.concatenate([B[r, k0:k0 + 16], B[r, k0 + 64:k0 + 80]]))


def test_prepack_of_uint8_weight():
    rng = np.random.default_rng(1)
    B = rng.integers(0, 256, size=(128, 256), dtype=np.uint8)
    out = oracle.bprepack(B)
    assert out.dtype == np.uint8 and out.size == B.size
    assert np.array_equal(np.sort(out), np.sort(B.ravel()))


def test_fragment_row_order():
    """brow is a permutation of each 64-row group; in it, MFMA sub-tiles 0 and 1
    of a lane group g cover the 8 consecutive rows 8g .. 8g+7, sub-tiles 2 and
    3 the 8 rows 32 + 8g .. (written as columns of C: two 16-byte stores)."""
    R = np.arange(256)
    b = oracle._brow(R)
    for g0 in range(0, 256, 64):
        assert np.array_equal(np.sort(b[g0:g0 + 64]), np.arange(g0, g0 + 64))
    for g in range(4):
        rows01 = [int(oracle._brow(16 * j + 4 * g + e)) for j in (0, 1) for e in range(4)]
        rows23 = [int(oracle._brow(16 * j + 4 * g + e)) for j in (2, 3) for e in range(4)]
        assert rows01 == list(range(8 * g, 8 * g + 8))
        assert rows23 == list(range(32 + 8 * g, 32 + 8 * g + 8))

"""Pins for the oracle's activation quantiser with swizzled block scales
[P39129 "Implementation breakdown", apply_weights of the CUTLASS and
FlashInfer kernels: scaled_fp4_quant(..., is_sf_swizzled_layout=True);
process_weights_after_loading: swizzle_blockscale].

The block codec is the one pinned in the format tests; what is new here is
the placement of the scales, checked against the tile description written a
second way (a block matrix assembled tile by tile), against hand-worked byte
offsets, and for zero padding."""
import numpy as np
import pytest

from oracle import nvfp4_oracle as O


def _bf16(x):
    return O.f32_to_bf16(np.asarray(x, np.float32))


def _tiles_by_blocks(scales: np.ndarray, m: int, k: int) -> np.ndarray:
    """The swizzled buffer built tile by tile: tile (i, j) is a 32 x 16 byte
    matrix whose row b is the 4 scales of rows 128i+b, 128i+32+b, 128i+64+b,
    128i+96+b (columns 4j..4j+3), zero outside the [m, k/16] matrix; tiles
    follow each other with j fastest."""
    nc = k // 16
    mt, ct = -(-m // 128), -(-nc // 4)
    pad = np.zeros((mt * 128, ct * 4), np.uint8)
    pad[:m, :nc] = scales
    chunks = []
    for i in range(mt):
        for j in range(ct):
            t = np.zeros((32, 16), np.uint8)
            for b in range(32):
                t[b] = np.concatenate([pad[128 * i + 32 * a + b, 4 * j: 4 * j + 4] for a in range(4)])
            chunks.append(t.ravel())
    return np.concatenate(chunks)


@pytest.mark.parametrize("m,k", [(1, 16), (33, 80), (128, 64), (200, 272), (257, 1024)])
def test_swizzle_matches_tile_description(m, k):
    rng = np.random.default_rng(m * 1000 + k)
    # per-block magnitudes spread over many binades so the scales differ
    x = rng.standard_normal((m, k)) * np.repeat(np.exp2(rng.integers(-6, 7, (m, k // 16))), 16, axis=1)
    xb = _bf16(x)
    g = np.float32(np.abs(O.bf16_to_f32(xb)).max() / (6 * 448))
    codes_rm, sf_rm = O.quant_activations(xb, g, swizzled=False)
    codes_sw, sf_sw = O.quant_activations(xb, g, swizzled=True)
    assert sf_rm.shape == (m, k // 16)
    assert np.array_equal(codes_rm, codes_sw)
    mp, ncp = O.sf_swizzled_shape(m, k)
    assert sf_sw.shape == (mp * ncp,)
    assert np.array_equal(sf_sw, _tiles_by_blocks(sf_rm, m, k))
    # the row-major form is the scale part of the packed rows, codes the data part
    rows = O.quantize_rows(xb, g)
    assert np.array_equal(codes_rm, rows[:, : k // 2]) and np.array_equal(sf_rm, rows[:, k // 2:])


@pytest.mark.parametrize("r,c,off", [(0, 0, 0), (0, 1, 1), (0, 3, 3), (1, 0, 16), (31, 0, 496), (32, 0, 4),
                                     (32, 4, 516), (127, 2, 510), (130, 0, 1056), (199, 4, 1024 + 512 + 16 * 7 + 8)])
def test_single_block_lands_at_worked_offset(r, c, off):
    """m=200, k=80: 5 scale columns padded to 8 (2 column tiles), 200 rows
    padded to 256 (2 row tiles), 2048 bytes. Only block (r, c) is non-zero:
    sixteen 3.0s under g = 0.25 give amax/(6g) = 2, scale byte 0x40; every
    other block is zero and so is its scale."""
    m, k = 200, 80
    x = np.zeros((m, k), np.float32)
    x[r, 16 * c: 16 * c + 16] = 3.0
    codes, sf = O.quant_activations(_bf16(x), 0.25, swizzled=True)
    assert sf.shape == (2048,)
    nz = np.flatnonzero(sf)
    assert nz.tolist() == [off] and sf[off] == 0x40
    # 3.0 / (2 * 0.25) = 6: every code is E2M1 6 (0x7), two per byte
    assert np.all(codes[r, 8 * c: 8 * c + 8] == 0x77)
    assert np.count_nonzero(codes) == 8


def test_round_trip_exact_blocks_odd_width():
    """Blocks whose values are E2M1 values times a common power of two, and
    one element at +-6, reconstruct exactly from codes and row-major scales
    at a width (k = 48) that is no power of two."""
    rng = np.random.default_rng(7)
    m, k = 37, 48
    vals = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    x = rng.choice(vals, (m, k)) * rng.choice([-1, 1], (m, k))
    x[:, ::16] = 6.0
    x *= np.repeat(np.exp2(rng.integers(-3, 4, (m, k // 16))).astype(np.float32), 16, axis=1)
    g = np.float32(1.0 / 8)  # block scale 8 * 2^e in [1, 64]: inside E4M3
    codes, sf = O.quant_activations(_bf16(x), g, swizzled=False)
    rows = np.concatenate([codes, sf], axis=1)
    back = O.dequantize_rows(rows, g, k)
    assert np.array_equal(back, x.astype(np.float32))

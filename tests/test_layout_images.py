"""The whole-buffer images of gpu_util (reshape + transpose of the oracle's row-major copies)
against the index maps of layout.py, on shapes with ragged rows and contraction tails."""
import numpy as np
import pytest

from mxfp4_block_scaled_cast_amd import layout
from gpu_util import codes_image, codes8_image, scales_image


@pytest.mark.parametrize("rows,k", [(1, 32), (17, 96), (16, 128), (129, 288), (300, 1056), (40, 4096)])
def test_images_match_index_maps(rows, k):
    rng = np.random.default_rng(rows * 7 + k)
    q = rng.integers(0, 256, (rows, k // 2), dtype=np.uint8)
    q8 = rng.integers(0, 256, (rows, k), dtype=np.uint8)
    s = rng.integers(0, 256, (rows, k // 32), dtype=np.uint8)
    assert np.array_equal(codes_image(q, rows, k), layout.codes_from_rowmajor(q, rows, k))
    assert np.array_equal(codes8_image(q8, rows, k), layout.codes8_from_rowmajor(q8, rows, k))
    assert np.array_equal(scales_image(s, rows, k), layout.scales_from_rowmajor(s, rows, k))

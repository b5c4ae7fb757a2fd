"""The inputs of the rounding-point GPU tests (tests/test_gpu_rounding_points.py)
reach what they are built for: block scale values exactly on the E4M3 rounding
points, inside the 16-ulp window where the kernels take the divisions, and just
outside it, where the one-multiply form decides."""
import numpy as np

from test_gpu_rounding_points import (bf16_rows_with_ties, bf16_to_f32, block_scale_value, f32_rows,
                                      near_point, F32, K_RECIPE)


def test_crafted_inputs_reach_the_rounding_points():
    """FP32 rows: ties, near misses inside the window and cases just outside."""
    rng = np.random.default_rng(0)
    for R in (1.0, 3.7e-3, 2.9e4):
        _, amaxes, g = f32_rows(rng, R, 512)
        z = block_scale_value(amaxes, g)
        assert near_point(z, 0).sum() >= 20        # exact ties
        assert near_point(z, 16).sum() >= 500      # inside the window: divisions taken
        assert (~near_point(z, 16)).sum() >= 500   # just outside: the multiply decides




def test_bf16_rows_hit_the_points_exactly():
    """BF16 rows of amax 2688: blocks of amax 6 m give a scale value of m itself."""
    rng = np.random.default_rng(1)
    x = bf16_to_f32(bf16_rows_with_ties(rng, 1024))
    g = F32(2688.0) * K_RECIPE
    blocks = np.abs(x.reshape(x.shape[0], -1, 16)).max(axis=2)[:, 1:].ravel()
    blocks = blocks[blocks > 0]
    z = block_scale_value(blocks, g)
    assert near_point(z, 0).sum() >= 100

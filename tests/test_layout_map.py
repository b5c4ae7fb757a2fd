"""The test-side inverse of the prepared-weight layout equals a literal,
element-by-element construction from the layout's definition in include/pmoe.h."""
import numpy as np
import pytest

from helpers import TILE, canonical_from_prepared, prepared_row_map


@pytest.mark.parametrize("gated,I", [(False, 64), (True, 64), (False, 640), (True, 320)])
def test_inverse_layout_map(gated, I):
    rng = np.random.default_rng(0)
    E, H = 2, 128
    gI = I if gated else 0
    N = 2 * I if gated else I
    canon = rng.integers(0, 256, (E, N, H // 2), dtype=np.uint8)
    canon_s = rng.integers(0, 127, (E, N, H // 16), dtype=np.uint8)
    NB, KC = N // 32, H // 64
    NBp = -(-NB // TILE) * TILE
    NT = NBp // TILE
    prep = np.zeros(E * NBp * 32 * H // 2, np.uint8)
    prep_s = np.zeros(E * NBp * 32 * H // 16, np.uint8)
    rows = prepared_row_map(N, gI)
    for e in range(E):
        for p in range(NB):
            for col in range(32):
                n = rows[p * 32 + col]
                if gated:
                    assert n == (I if p % 2 else 0) + 32 * (p // 2) + col
            for c in range(KC):
                slab = ((e * NT + p // TILE) * KC + c) * TILE + p % TILE
                for lane in range(64):
                    for h in range(2):
                        n = rows[p * 32 + 16 * h + lane % 16]
                        for s_ in range(2):
                            for i in range(8):
                                k = c * 64 + 32 * s_ + 8 * (lane // 16) + i
                                nib = (canon[e, n, k // 2] >> (4 * (k % 2))) & 15
                                off = (slab * 64 + lane) * 16 + (2 * h + s_) * 4 + i // 2
                                prep[off] |= nib << (4 * (i % 2))
                for d in range(32):
                    for h in range(2):
                        n = rows[p * 32 + 16 * h + d % 16]
                        for s_ in range(2):
                            prep_s[(slab * 32 + d) * 4 + 2 * h + s_] = canon_s[e, n, c * 4 + 2 * s_ + d // 16]
    cq, cs = canonical_from_prepared(prep, prep_s, E, N, H, gI)
    assert np.array_equal(cq, canon) and np.array_equal(cs, canon_s)

"""The test-side inverse of the prepared-weight layout equals a literal,
element-by-element construction from the layout's definition in include/pmoe.h."""
import numpy as np
import pytest

from helpers import TILE, canonical_from_prepared, prepared_row_map


@pytest.mark.parametrize("gated,I,H", [(False, 64, 128), (True, 64, 128), (False, 640, 128),
                                       (True, 320, 128), (True, 48, 80), (False, 80, 16),
                                       (True, 16, 208)])
def test_inverse_layout_map(gated, I, H):
    """Literal construction from the header's definition, including shapes whose N is not a
    multiple of 32 and whose reduction is not a multiple of 64 (zero padding rows and k)."""
    rng = np.random.default_rng(0)
    E = 2
    gI = I if gated else 0
    N = 2 * I if gated else I
    canon = rng.integers(0, 256, (E, N, H // 2), dtype=np.uint8)
    canon_s = rng.integers(0, 127, (E, N, H // 16), dtype=np.uint8)
    NB = 2 * -(-I // 32) if gated else -(-N // 32)
    KC = -(-H // 64)
    NBp = -(-NB // TILE) * TILE
    NT = NBp // TILE
    prep = np.zeros(E * NBp * 32 * KC * 32, np.uint8)
    prep_s = np.zeros(E * NBp * 32 * KC * 4, np.uint8)

    def row(p, col):  # the header's row map; None for a padding row
        if gated:
            r = 32 * (p // 2) + col
            return (I if p % 2 else 0) + r if r < I else None
        n = 32 * p + col
        return n if n < N else None

    assert [row(p, c) if row(p, c) is not None else -1 for p in range(NB) for c in range(32)] == \
        prepared_row_map(N, gI).tolist()
    for e in range(E):
        for p in range(NB):
            for c in range(KC):
                slab = ((e * NT + p // TILE) * KC + c) * TILE + p % TILE
                for lane in range(64):
                    for h in range(2):
                        n = row(p, 16 * h + lane % 16)
                        for s_ in range(2):
                            for i in range(8):
                                k = c * 64 + 32 * s_ + 8 * (lane // 16) + i
                                if n is None or k >= H:
                                    continue
                                nib = (canon[e, n, k // 2] >> (4 * (k % 2))) & 15
                                off = (slab * 64 + lane) * 16 + (2 * h + s_) * 4 + i // 2
                                prep[off] |= nib << (4 * (i % 2))
                for d in range(32):
                    for h in range(2):
                        n = row(p, 16 * h + d % 16)
                        for s_ in range(2):
                            blk = c * 4 + 2 * s_ + d // 16
                            if n is not None and blk < H // 16:
                                prep_s[(slab * 32 + d) * 4 + 2 * h + s_] = canon_s[e, n, blk]
    cq, cs = canonical_from_prepared(prep, prep_s, E, N, H, gI)
    assert np.array_equal(cq, canon) and np.array_equal(cs, canon_s)

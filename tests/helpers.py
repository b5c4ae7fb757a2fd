"""Test-side helpers: the prepared-weight layout map and tensor transfers.

The prepared layout is documented in include/pmoe.h; `canonical_from_prepared`
inverts it so prepared bytes can be compared with the oracle's canonical
[E, N, K/2] codes and [E, N, K/16] scales.
"""
import numpy as np

TILE = 8  # column blocks (of 32 rows) per column tile of the prepared layout


def prepared_row_map(N, gated_I):
    """Canonical row index of each prepared row p*32 + col."""
    NB = N // 32
    p = np.repeat(np.arange(NB), 32)
    col = np.tile(np.arange(32), NB)
    if gated_I:
        return np.where(p % 2 == 1, gated_I, 0) + 32 * (p // 2) + col
    return 32 * p + col


def canonical_from_prepared(codes, scales, E, N, Kd, gated_I=0, check_padding=True):
    NB, KC = N // 32, Kd // 64
    NBp = -(-NB // TILE) * TILE
    NT = NBp // TILE
    # codes: lane = 16*g + n16, bytes (2h + s)*4 + b: element k = 32 s + 8 g + 2 b (+1), row 16 h + n16
    c = np.asarray(codes, np.uint8).reshape(E, NT, KC, TILE, 4, 16, 2, 2, 4)  # e ct c pos g n16 h s b
    c = c.transpose(0, 1, 3, 6, 5, 2, 7, 4, 8).reshape(E, NBp * 32, KC * 32)  # e (ct pos h n16) (c s g b)
    # scales: dword d = n16 + 16 jj, byte 2h + s: block 2s + jj of row 16 h + n16
    s = np.asarray(scales, np.uint8).reshape(E, NT, KC, TILE, 2, 16, 2, 2)     # e ct c pos jj n16 h s
    s = s.transpose(0, 1, 3, 6, 5, 2, 7, 4).reshape(E, NBp * 32, KC * 4)       # e (ct pos h n16) (c s jj)
    if check_padding:
        assert not c[:, NB * 32:].any() and not s[:, NB * 32:].any(), "padding blocks must be zero"
    c, s = c[:, :NB * 32], s[:, :NB * 32]
    rows = prepared_row_map(N, gated_I)
    cq = np.empty_like(c)
    cs = np.empty_like(s)
    cq[:, rows] = c
    cs[:, rows] = s
    return cq, cs


def np_u8(t):
    return t.detach().cpu().numpy().view(np.uint8) if t.dtype != __import__("torch").uint8 else t.detach().cpu().numpy()


def bf16_bits(t):
    """torch 2-byte tensor -> numpy uint16 bit patterns."""
    import torch
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def dev_bf16(a, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)


def dev(a, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def per_token_close(got, want, rel):
    """max_n |got - want| <= rel * max_n |want| for every row (want = 0 rows need got == 0)."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    err = np.abs(got - want).max(axis=1)
    scale = np.abs(want).max(axis=1)
    return err <= rel * scale + (scale == 0) * 0.0, err / np.maximum(scale, 1e-30)

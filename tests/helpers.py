"""Test-side helpers: the prepared-weight layout map and tensor transfers.

The prepared layout is documented in include/pmoe.h; `canonical_from_prepared`
inverts it so prepared bytes can be compared with the oracle's canonical
[E, N, K/2] codes and [E, N, K/16] scales.
"""
import numpy as np

TILE = 8  # column blocks (of 32 rows) per column tile of the prepared layout


def prepared_row_map(N, gated_I):
    """Canonical row index of each prepared row p*32 + col (p < NB), or -1 for a zero
    padding row. NB = ceil(N/32), or 2*ceil(I/32) for a gated FC1 (N = 2I)."""
    if gated_I:
        NB = 2 * -(-gated_I // 32)
        p = np.repeat(np.arange(NB), 32)
        r = 32 * (p // 2) + np.tile(np.arange(32), NB)        # row within the gate / up half
        return np.where(r < gated_I, np.where(p % 2 == 1, gated_I, 0) + r, -1)
    n = np.arange(-(-N // 32) * 32)
    return np.where(n < N, n, -1)


def canonical_from_prepared(codes, scales, E, N, Kd, gated_I=0, check_padding=True):
    rows = prepared_row_map(N, gated_I)
    NB, KC = rows.size // 32, -(-Kd // 64)
    NBp = -(-NB // TILE) * TILE
    NT = NBp // TILE
    # codes: lane = 16*g + n16, bytes (2h + s)*4 + b: element k = 32 s + 8 g + 2 b (+1), row 16 h + n16
    c = np.asarray(codes, np.uint8).reshape(E, NT, KC, TILE, 4, 16, 2, 2, 4)  # e ct c pos g n16 h s b
    c = c.transpose(0, 1, 3, 6, 5, 2, 7, 4, 8).reshape(E, NBp * 32, KC * 32)  # e (ct pos h n16) (c s g b)
    # scales: dword d = n16 + 16 jj, byte 2h + s: block 2s + jj of row 16 h + n16
    s = np.asarray(scales, np.uint8).reshape(E, NT, KC, TILE, 2, 16, 2, 2)     # e ct c pos jj n16 h s
    s = s.transpose(0, 1, 3, 6, 5, 2, 7, 4).reshape(E, NBp * 32, KC * 4)       # e (ct pos h n16) (c s jj)
    real = np.nonzero(rows >= 0)[0]
    if check_padding:
        pad = np.ones(NBp * 32, bool)
        pad[real] = False
        assert not c[:, pad].any() and not s[:, pad].any(), "padding rows must be zero"
        assert not c[:, :, Kd // 2:].any() and not s[:, :, Kd // 16:].any(), "padded k must be zero"
    cq = np.zeros((E, N, Kd // 2), np.uint8)
    cs = np.zeros((E, N, Kd // 16), np.uint8)
    cq[:, rows[real]] = c[:, real, :Kd // 2]
    cs[:, rows[real]] = s[:, real, :Kd // 16]
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


# ----------------------------------------------------------------------------- oracle weights
# Quantizing one expert of the full-size workloads takes the oracle a few
# seconds; the GPU tests share one cache per weight set for the whole session
# and fill it from several threads (numpy releases the GIL in its array loops).
_ORACLE_CACHE = {}


def oracle_threads():
    import os
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _prefetch(W, experts):
    from concurrent.futures import ThreadPoolExecutor
    todo = sorted({int(e) for e in experts} - set(W._cache))
    if len(todo) > 1:
        with ThreadPoolExecutor(oracle_threads()) as ex:
            list(ex.map(W.expert, todo))
    for e in todo:
        W.expert(e)
    return W


def oracle_weights(w, experts=()):
    """The oracle's lazily quantized weights of workload w, with `experts` quantized up front."""
    import synth
    from oracle import moe as om
    key = ("per_token", w.index, w.weight_epoch, w.E, w.N1, w.H, w.I, w.weight_std)
    cache = _ORACLE_CACHE.setdefault(key, {})
    W = om.LazyWeights(lambda e: synth.expert_weights(w, e), w.E, w.N1, w.H, w.I, cache=cache)
    return _prefetch(W, experts)


def oracle_weights_per_tensor(w, a1, a2, experts=()):
    import synth
    from oracle import recipes as orc
    key = ("per_tensor", w.index, w.weight_epoch, w.E, w.N1, w.H, w.I, w.weight_std,
           float(a1), float(a2))
    cache = _ORACLE_CACHE.setdefault(key, {})
    W = orc.LazyWeightsPerTensor(lambda e: synth.expert_weights(w, e), w.E, w.N1, w.H, w.I, a1, a2,
                                 cache=cache)
    return _prefetch(W, experts)


def drop_oracle_weights():
    _ORACLE_CACHE.clear()


# ----------------------------------------------------------------------------- sampling
def split_expert(expert_offsets, counters):
    """First local expert of the second part of a two-stream run (counters[3] is its first row)."""
    offs = np.asarray(expert_offsets)
    first_row = int(np.asarray(counters)[3])
    e = int(np.searchsorted(offs, first_row, side="left"))
    while e + 1 < offs.size and offs[e + 1] == offs[e]:   # skip empty experts at the cut
        e += 1
    return e


def sample_experts(counts, split):
    """Experts whose z rows are checked: the first, an ordinary one, both sides of the stream
    split, the two largest (hot) experts and the last one that has rows."""
    counts = np.asarray(counts)
    nz = np.nonzero(counts)[0]
    hot = np.argsort(-counts, kind="stable")[:2]
    picks = {int(nz[0]), int(nz[min(17, nz.size - 1)]), int(nz[-1]), *map(int, hot)}
    below = nz[nz < split]
    above = nz[nz >= split]
    if below.size:
        picks.add(int(below[-1]))
    if above.size:
        picks.add(int(above[0]))
    return sorted(picks)


def sample_tokens(ids, split, have=(), n=8, n_part2=3, expert_offset=0, E=None):
    """n tokens for output checks, chosen to need few extra oracle experts: the first n_part2
    among tokens whose valid routes all run on the second stream (experts >= split), the
    rest among all tokens. Deterministic."""
    ids = np.asarray(ids) - expert_offset
    T = ids.shape[0]
    E = int(ids.max()) + 1 if E is None else E
    valid = (ids >= 0) & (ids < E)
    have = set(int(e) for e in have)
    part2 = [t for t in range(T) if valid[t].any() and (ids[t][valid[t]] >= split).all()]
    chosen = []
    for k in range(min(n, T)):
        pool = part2 if (k < n_part2 and len(part2) > k) else range(T)
        best = min((t for t in pool if t not in chosen),
                   key=lambda t: (len(set(ids[t][valid[t]].tolist()) - have), t))
        chosen.append(best)
        have |= set(ids[best][valid[best]].tolist())
    return chosen, sorted(have)

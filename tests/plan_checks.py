"""Routing-plan checks shared by the oracle tests and the GPU parity tests:
an independent brute-force plan (a stable sort of (local expert, route)) and
the plan invariants."""
import numpy as np


def capacity(M, k, El, T):
    R = M * k
    need = R + min(El, R) * (T - 1)
    return (need + T - 1) // T * T


def brute_force_plan(ids, El, offset, T):
    ids = np.asarray(ids)
    M, k = ids.shape
    flat = ids.reshape(-1)
    local = [(int(flat[r]) - offset, r) for r in range(M * k) if offset <= flat[r] < offset + El]
    order = sorted(local)                       # stable by construction: (expert, route)
    slots = capacity(M, k, El, T)
    e2p = -np.ones(M * k, np.int64)
    p2e = -np.ones(slots, np.int64)
    te = -np.ones(slots // T, np.int64)
    tl = -np.ones(slots // T, np.int64)
    counts = np.zeros(El, np.int64)
    for le, _ in order:
        counts[le] += 1
    offsets = np.zeros(El + 1, np.int64)
    pos = 0
    nt = 0
    i = 0
    for le in range(El):
        offsets[le] = pos
        for j in range(counts[le]):
            _, r = order[i]
            i += 1
            e2p[r] = pos + j
            p2e[pos + j] = r
        ntile = -(-counts[le] // T)
        for tt in range(ntile):
            te[nt] = le
            tl[nt] = min(pos + (tt + 1) * T, pos + counts[le])
            nt += 1
        pos += ntile * T
    offsets[El] = pos
    return dict(expanded_to_permuted=e2p, permuted_to_expanded=p2e, tile_to_expert=te, tile_to_mn_limit=tl,
                num_tiles=nt, expert_offsets=offsets, expert_counts=counts)


def check_invariants(ids, El, offset, T, e2p, p2e, te, tl, num_tiles, offsets, counts):
    M, k = np.asarray(ids).shape
    ids = np.asarray(ids).reshape(-1)
    R = ids.size
    local = (ids >= offset) & (ids < offset + El)
    # per-expert counts equal the histogram of local ids
    hist = np.bincount(ids[local] - offset, minlength=El)
    assert np.array_equal(np.asarray(counts), hist)
    assert hist.sum() <= R
    # non-local routes have no slot; local ones have distinct slots
    e2p = np.asarray(e2p)
    p2e = np.asarray(p2e)
    assert np.all(e2p[~local] == -1)
    s = e2p[local]
    assert np.all(s >= 0) and np.unique(s).size == s.size
    # bijection onto the valid slots
    assert np.array_equal(p2e[s], np.nonzero(local)[0])
    valid = p2e >= 0
    assert valid.sum() == local.sum()
    # capacity
    assert p2e.size == capacity(M, k, El, T)
    assert te.size == p2e.size // T if hasattr(te, "size") else True
    # expert ranges: padded to T, slots increasing in r (stable), padding -1
    offsets = np.asarray(offsets)
    for le in range(El):
        lo, c = offsets[le], counts[le]
        assert lo % T == 0
        assert offsets[le + 1] - lo == -(-c // T) * T
        rows = p2e[lo:lo + c]
        assert np.all(rows >= 0) and np.all(np.diff(rows) > 0)
        assert np.all(ids[rows] - offset == le)
        assert np.all(p2e[lo + c:offsets[le + 1]] == -1)
    assert np.all(p2e[offsets[El]:] == -1)
    # tile tables
    te = np.asarray(te)
    tl = np.asarray(tl)
    assert num_tiles == sum(-(-c // T) for c in counts)
    assert np.all(te[num_tiles:] == -1) and np.all(tl[num_tiles:] == -1)
    for i in range(num_tiles):
        le = te[i]
        start = i * T
        assert offsets[le] <= start < offsets[le + 1]
        assert tl[i] == min(start + T, offsets[le] + counts[le])

"""Pins of the oracle tile planner by brute force on small inputs (CPU only).

The work of a tile is re-derived from the visibility rule itself (count the
KV blocks / Q blocks holding at least one visible (query, key) pair), and the
deal is checked for its defining properties: every tile exactly once, sort
key (work; backward: the estimated time) non-increasing along the deal order,
snake assignment over the workers.
"""
import numpy as np
import pytest

import workloads as W
from oracle import attention as A
from oracle import planner as P


def _brute_work(pass_, b, t, lq_b, lk_b, bm, bn, causal, mask, window=None):
    mask_b = None if mask is None else mask[b]
    if pass_ == P.FWD:
        rows = np.arange(t * bm, min((t + 1) * bm, lq_b))
        vis = A.visibility(lq_b, lk_b, causal=causal, mask_b=mask_b, rows=rows, window=window)
        cols = np.nonzero(vis.any(axis=0))[0]
        return len(set(int(j) // bn for j in cols))
    keys = np.arange(t * bn, min((t + 1) * bn, lk_b))
    vis = A.visibility(lq_b, lk_b, causal=causal, mask_b=mask_b, window=window)[:, keys]
    rows = np.nonzero(vis.any(axis=1))[0]
    return len(set(int(i) // bm for i in rows))


def _simulated_bwd_cost(r, qlens, kvlens, bm, bn, causal, mask, window=None):
    """The backward tile's cost under the plan's cost model, by walking it:
    the Q blocks the tile visits are found from the visibility rule (blocks
    holding a row that sees one of the tile's keys), and each visited block
    costs BWD_BLOCK_FIXED plus one unit per wave (BWD_WAVE_KEYS consecutive
    keys of the tile) that holds at least one key inside the sequence; the
    tile adds BWD_TILE_FIXED. The record's work field is not used."""
    b, _, t, _ = (int(v) for v in r)
    lq_b, lk_b = int(qlens[b]), int(kvlens[b])
    keys = np.arange(t * bn, min((t + 1) * bn, lk_b))
    mask_b = None if mask is None else mask[b]
    vis = A.visibility(lq_b, lk_b, causal=causal, mask_b=mask_b, window=window)[:, keys]
    blocks = sorted(set(int(i) // bm for i in np.nonzero(vis.any(axis=1))[0]))
    cost = P.BWD_TILE_FIXED
    for _ in blocks:
        cost += P.BWD_BLOCK_FIXED
        for wave in range(bn // P.BWD_WAVE_KEYS):
            lo = t * bn + wave * P.BWD_WAVE_KEYS
            if any(lo <= int(k) < lo + P.BWD_WAVE_KEYS for k in keys):
                cost += 1
    return cost


def _cases():
    rng = np.random.default_rng(0)
    lens = rng.integers(1, 700, size=9)
    mask = (rng.random((9, 3, 6)) < 0.5).astype(np.uint8)
    mask[:, :, 0] = 1
    return [
        ("bcast", [300] * 9, lens, False, None),
        ("perseq", lens, lens, False, None),
        ("causal", lens, lens, True, None),
        ("sparse", [300] * 9, lens, False, mask),
    ]


@pytest.mark.parametrize("name,qlens,kvlens,causal,mask", _cases())
@pytest.mark.parametrize("pass_,bm,bn", [(P.FWD, 256, 64), (P.FWD, 128, 64), (P.BWD, 32, 256),
                                         (P.BWD, 64, 128)])
@pytest.mark.parametrize("workers", [1, 7, 16, 255])
def test_plan_properties(name, qlens, kvlens, causal, mask, pass_, bm, bn, workers):
    H = 3
    wp, tiles = P.plan(qlens, kvlens, H, workers, pass_, block_m=bm, block_n=bn,
                       causal=causal, block_mask=mask)
    assert wp[0] == 0 and wp[-1] == len(tiles) and np.all(np.diff(wp) >= 0)
    # every tile of the enumeration exactly once, with its brute-force work
    expect = set()
    for b in range(len(kvlens)):
        n_t = P.cdiv(qlens[b], bm) if pass_ == P.FWD else P.cdiv(kvlens[b], bn)
        for h in range(H):
            for t in range(n_t):
                expect.add((b, h, t, _brute_work(pass_, b, t, qlens[b], kvlens[b], bm, bn,
                                                 causal, mask)))
    got = [tuple(int(x) for x in r) for r in tiles]
    assert len(got) == len(set(got)) == len(expect)
    assert set(got) == expect
    # rebuild the deal order: position i lives on worker snake(i), in increasing i
    n = len(tiles)
    cursor = wp[:-1].copy()
    order = []
    for i in range(n):
        p = i % workers
        w = p if (i // workers) % 2 == 0 else workers - 1 - p
        order.append(got[cursor[w]])
        cursor[w] += 1
    assert np.all(cursor == wp[1:])
    def key(r):
        if pass_ == P.FWD:
            return r[3]
        return _simulated_bwd_cost(r, qlens, kvlens, bm, bn, causal, mask)
    works = [key(r) for r in order]
    assert all(works[i] >= works[i + 1] for i in range(n - 1))
    # stable: equal keys keep (b, h, t) enumeration order
    for i in range(n - 1):
        if works[i] == works[i + 1]:
            assert order[i][:3] < order[i + 1][:3]
    # balance: no worker exceeds the mean by more than one largest tile
    loads = [sum(key(r) for r in got[wp[w]:wp[w + 1]]) for w in range(workers)]
    assert max(loads) <= sum(works) / workers + (max(works) if works else 0)


@pytest.mark.parametrize("name,qlens,kvlens,causal,mask", _cases())
@pytest.mark.parametrize("workers", [1, 7, 16, 255])
def test_dynamic_plan_properties(name, qlens, kvlens, causal, mask, workers):
    """The dynamic forward plan: every tile once, with its brute-force work,
    in non-increasing work with ties in (b, h, t) order; worker w starts with
    tile w. List scheduling of that order (each tile to the first worker to
    be free, as the device counter hands them out) stays within one largest
    tile of the mean load."""
    H = 2
    bm, bn = 256, 64
    wp, tiles = P.plan(qlens, kvlens, H, workers, P.FWD, block_m=bm, block_n=bn,
                       causal=causal, block_mask=mask, dynamic=True)
    n = len(tiles)
    assert list(wp) == [min(w, n) for w in range(workers + 1)]
    expect = set()
    for b in range(len(kvlens)):
        for h in range(H):
            for t in range(P.cdiv(qlens[b], bm)):
                expect.add((b, h, t, _brute_work(P.FWD, b, t, qlens[b], kvlens[b], bm, bn,
                                                 causal, mask)))
    got = [tuple(int(x) for x in r) for r in tiles]
    assert len(got) == len(set(got)) == len(expect) and set(got) == expect
    works = [r[3] for r in got]
    assert all(works[i] >= works[i + 1] for i in range(n - 1))
    for i in range(n - 1):
        if works[i] == works[i + 1]:
            assert got[i][:3] < got[i + 1][:3]
    free = [0] * workers
    for i, wk in enumerate(works):
        w = i if i < workers else min(range(workers), key=lambda x: free[x])
        free[w] += wk
    if works:
        assert max(free) <= sum(works) / workers + max(works)


def test_sparse_lists_by_scan():
    rng = np.random.default_rng(3)
    lens = np.array([5, 129, 256, 900, 1])
    mask = (rng.random((5, 2, 8)) < 0.5).astype(np.uint8)
    qlens = [200] * 5
    ptr, idx = P.sparse_lists(mask, qlens, lens, P.FWD)
    assert len(ptr) == 5 * 2 + 1
    for b in range(5):
        for m in range(2):
            r = b * 2 + m
            want = [4 * c + 1 for c in range(8) if mask[b, m, c] and 128 * c < lens[b]]
            assert list(idx[ptr[r]:ptr[r + 1]]) == want
    # 256-row tiles: the union of the two rows' kept blocks, one bit per row;
    # with 200 query rows both mask rows hold rows of the sequence, with 100
    # only the first does
    for ql in (200, 100):
        ptr, idx = P.sparse_lists(mask, [ql] * 5, lens, P.FWD, block_m=256)
        assert len(ptr) == 5 + 1
        for b in range(5):
            want = []
            for c in range(8):
                if 128 * c >= lens[b]:
                    continue
                bits = int(mask[b, 0, c]) | ((int(mask[b, 1, c]) << 1) if ql > 128 else 0)
                if bits:
                    want.append(4 * c + bits)
            assert list(idx[ptr[b]:ptr[b + 1]]) == want
    ptr, idx = P.sparse_lists(mask, qlens, lens, P.BWD)
    assert len(ptr) == 5 * 8 + 1
    for b in range(5):
        for c in range(8):
            r = b * 8 + c
            want = [4 * m + 1 for m in range(2) if mask[b, m, c] and 128 * m < qlens[b]
                    and 128 * c < lens[b]]
            assert list(idx[ptr[r]:ptr[r + 1]]) == want
    # 256-key tiles: the union of the two columns' kept rows, one bit per
    # column; a column past the sequence keeps nothing
    ptr, idx = P.sparse_lists(mask, qlens, lens, P.BWD, block_n=256)
    assert len(ptr) == 5 * 4 + 1
    for b in range(5):
        for t in range(4):
            want = []
            for m in range(2):
                if 128 * m >= qlens[b]:
                    continue
                bits = sum(1 << k for k in range(2)
                           if mask[b, m, 2 * t + k] and 128 * (2 * t + k) < lens[b])
                if bits:
                    want.append(4 * m + bits)
            assert list(idx[ptr[b * 4 + t]:ptr[b * 4 + t + 1]]) == want


def test_offsets_from_lengths():
    assert list(P.offsets_from_lengths([3, 0, 5])) == [0, 3, 3, 8]
    assert list(P.offsets_from_lengths([])) == [0]
    with pytest.raises(ValueError):
        P.offsets_from_lengths([1, -1])
    x = W.make_inputs(1)
    assert list(P.offsets_from_lengths(x.lengths)) == list(x.kv_offsets)


@pytest.mark.parametrize("workers", [1, 3, 4, 5, 64])
@pytest.mark.parametrize("lq", [0, 100, 256, 600])
def test_dq_plan_grouped(workers, lq):
    """Broadcast-Q dQ plan: every (b, h, t) tile covered once by its chunks
    (consecutive block ranges that partition the tile's brute-force work,
    at most DQ_CHUNK long, the first ones one longer), each worker inside one
    (h, t) group, groups on contiguous disjoint worker ranges, snake deal with
    non-increasing work inside each group."""
    rng = np.random.default_rng(lq + workers)
    lens = rng.integers(0, 3000, size=11)
    lens[3] = 0
    H, bm, bn = 3, 256, 64
    wp, tiles = P.plan_dq([lq] * 11, lens, H, workers, broadcast_q=True, lq=lq,
                          block_m=bm, block_n=bn)
    nqt = P.cdiv(lq, bm)
    G = H * nqt
    # W' = max(G, min(W, G * n)), n the largest chunk count of a group (every
    # group holds the same B sequences here, so all counts are equal)
    n_g = sum(max(1, P.cdiv(_brute_work(P.FWD, b, 0, lq, int(lens[b]), bm, bn, False, None),
                              P.DQ_CHUNK)) for b in range(11)) if G else 0
    Wp = max(G, min(workers, G * n_g)) if G else workers
    assert len(wp) == Wp + 1
    got = [tuple(int(x) for x in r) for r in tiles]
    assert len(got) == len(set(got))
    chunks = {}
    for b, h, f2, n in got:
        t, k0 = f2 % max(nqt, 1), f2 // max(nqt, 1)
        chunks.setdefault((b, h, t), []).append((k0, n))
    expect = {(b, h, t): _brute_work(P.FWD, b, t, lq, int(lens[b]), bm, bn, False, None)
              for b in range(11) for h in range(H) for t in range(nqt)}
    assert set(chunks) == set(expect)
    n_split = 0
    for key, parts in chunks.items():
        w = expect[key]
        parts.sort()
        n = max(1, P.cdiv(w, P.DQ_CHUNK))
        assert len(parts) == n
        n_split += n > 1
        assert parts[0][0] == 0 and sum(p[1] for p in parts) == w
        for (k0, ln), (k1, _) in zip(parts, parts[1:]):
            assert k1 == k0 + ln
        lens_ = [p[1] for p in parts]
        assert max(lens_) <= P.DQ_CHUNK and max(lens_) - min(lens_) <= 1
        assert lens_ == sorted(lens_, reverse=True)
    if lq > 0:
        assert n_split > 0
    for g in range(G):
        h, t = divmod(g, nqt)
        w0, w1 = g * Wp // G, (g + 1) * Wp // G
        assert w1 > w0
        grp = [r for w in range(w0, w1) for r in got[wp[w]:wp[w + 1]]]
        assert all(r[1] == h and r[2] % nqt == t for r in grp)
        assert len(grp) == sum(len(chunks[(b, h, t)]) for b in range(11))
        nw = w1 - w0
        cursor = [wp[w] for w in range(w0, w1)]
        order = []
        for i in range(len(grp)):
            p = i % nw
            w = p if (i // nw) % 2 == 0 else nw - 1 - p
            order.append(got[cursor[w]])
            cursor[w] += 1
        assert cursor == [wp[w + 1] for w in range(w0, w1)]
        works = [r[3] for r in order]
        assert all(works[i] >= works[i + 1] for i in range(len(works) - 1))


def test_dq_plan_per_sequence_is_forward_plan():
    lens = np.array([5, 300, 0, 1000, 257])
    a = P.plan_dq(lens, lens, 2, 3, broadcast_q=False, block_m=256, block_n=64, causal=True)
    b = P.plan(lens, lens, 2, 3, P.FWD, block_m=256, block_n=64, causal=True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("window,causal", [((100, 30), False), ((0, 0), False), ((700, None), False),
                                           ((None, 300), False), ((257, None), True),
                                           ((31, 33), False)])
@pytest.mark.parametrize("pass_,bm,bn", [(P.FWD, 256, 64), (P.BWD, 32, 256)])
def test_band_plan_work_by_brute_force(window, causal, pass_, bm, bn):
    """Sliding-window (band) work: the blocks holding a visible pair, counted
    from the visibility rule itself, for every tile."""
    rng = np.random.default_rng(3)
    lens = list(rng.integers(1, 900, size=7)) + [1, 256, 257]
    wp, tiles = P.plan(lens, lens, 2, 5, pass_, block_m=bm, block_n=bn, causal=causal,
                       window=window)
    got = {(int(r[0]), int(r[1]), int(r[2])): int(r[3]) for r in tiles}
    for b, L in enumerate(lens):
        n_t = P.cdiv(L, bm) if pass_ == P.FWD else P.cdiv(L, bn)
        for t in range(n_t):
            w = _brute_work(pass_, b, t, L, L, bm, bn, causal, None, window=window)
            assert got[(b, 0, t)] == w, (b, t)


def test_bwd_sort_key_puts_partial_tiles_after_full_ones():
    """Equal work (2 Q blocks each), unequal keys: a full 256-key tile (8 waves
    busy) sorts before a 100-key one (4 waves) and a 44-key one (2 waves):
    keys 2*(4+8)+42 = 66, 2*(4+4)+42 = 58, 2*(4+2)+42 = 54."""
    lens = [100, 256, 300]
    wp, tiles = P.plan([64] * 3, lens, 1, 1, P.BWD, block_m=32, block_n=256)
    assert [tuple(int(v) for v in r) for r in tiles] == [(1, 0, 0, 2), (2, 0, 0, 2),
                                                         (0, 0, 0, 2), (2, 0, 1, 2)]
    assert [P.bwd_sort_key(2, t, L, 256) for t, L in ((0, 256), (0, 100), (1, 300))] == [66, 58, 54]


def test_dq_plan_workers_capped_by_chunks():
    """A small broadcast-Q problem gets no more dQ workers than its groups
    have chunks: 2 heads x 2 Q tiles, 3 sequences of one chunk each ->
    W' = 4 * 3 = 12 of the 256 asked for; with more chunks than workers
    per group, W' is the request (or G if larger)."""
    wp, tiles = P.plan_dq([300] * 3, [10, 0, 64], 2, 256, broadcast_q=True, lq=300,
                          block_m=256, block_n=64)
    assert len(wp) == 13 and len(tiles) == 12
    assert all(wp[w + 1] - wp[w] == 1 for w in range(12))
    wp, _ = P.plan_dq([300] * 3, [5000, 4000, 64], 2, 8, broadcast_q=True, lq=300,
                      block_m=256, block_n=64)
    assert len(wp) == 9
    wp, _ = P.plan_dq([300] * 3, [5000, 4000, 64], 2, 3, broadcast_q=True, lq=300,
                      block_m=256, block_n=64)
    assert len(wp) == 5


@pytest.mark.parametrize("name,qlens,kvlens,causal,mask", _cases())
@pytest.mark.parametrize("pass_,bm,bn", [(P.FWD, 256, 64), (P.BWD, 32, 256)])
@pytest.mark.parametrize("workers", [1, 7, 255])
def test_natural_plan_by_enumeration(name, qlens, kvlens, causal, mask, pass_, bm, bn, workers):
    """The natural (ablation) plan: the tiles enumerated by nested loops over
    (b, h, t) with their brute-force work, tile i on worker i mod W, each
    worker's list in enumeration order."""
    H = 2
    wp, tiles = P.plan(qlens, kvlens, H, workers, pass_, block_m=bm, block_n=bn,
                       causal=causal, block_mask=mask, natural=True)
    enum = []
    for b in range(len(kvlens)):
        n_t = P.cdiv(qlens[b], bm) if pass_ == P.FWD else P.cdiv(kvlens[b], bn)
        for h in range(H):
            for t in range(n_t):
                enum.append((b, h, t, _brute_work(pass_, b, t, qlens[b], kvlens[b], bm, bn,
                                                  causal, mask)))
    for w in range(workers):
        got = [tuple(int(x) for x in r) for r in tiles[wp[w]:wp[w + 1]]]
        assert got == enum[w::workers]
    # the same tiles as the sorted plan
    _, sorted_tiles = P.plan(qlens, kvlens, H, workers, pass_, block_m=bm, block_n=bn,
                             causal=causal, block_mask=mask)
    assert sorted(map(tuple, tiles.tolist())) == sorted(map(tuple, sorted_tiles.tolist()))


def test_natural_dq_plan_keeps_groups():
    """Broadcast-Q natural dQ plan: the sorted plan's groups, workers and
    chunks, each group's chunks in (b, chunk) order dealt round-robin."""
    lens = [40, 3000, 700, 0, 1500]
    wp_s, t_s = P.plan_dq([300] * 5, lens, 2, 16, broadcast_q=True, lq=300, block_m=256,
                          block_n=64)
    wp, t = P.plan_dq([300] * 5, lens, 2, 16, broadcast_q=True, lq=300, block_m=256,
                      block_n=64, natural=True)
    assert len(wp) == len(wp_s)
    W_ = len(wp) - 1
    G = 2 * 2
    nqt = 2
    for g in range(G):
        h, tq = divmod(g, nqt)
        w0, w1 = g * W_ // G, (g + 1) * W_ // G
        chunks = [tuple(int(x) for x in r) for r in t_s.tolist()
                  if r[1] == h and r[2] % nqt == tq]
        chunks.sort(key=lambda r: (r[0], r[2] // nqt))       # (b, chunk) order
        for j, w in enumerate(range(w0, w1)):
            got = [tuple(int(x) for x in r) for r in t[wp[w]:wp[w + 1]]]
            assert got == chunks[j::w1 - w0]

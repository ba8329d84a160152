"""Integer reference for the host tile plan -- oracle (test infrastructure only).

The pages describe the forward scheduler as: sort the tiles on the host by KV
workload, largest first, and hand them to the processors in a zigzag pattern,
which recovered about a fifth of the forward time at negligible CPU cost
([bites] section "Optimizations layered on top", item on scheduling jagged
tiles across SMs and the paragraph after the list). The pages fix neither the
tile size, the work measure, the tie order nor the meaning of "zigzag"; the
plainest readings, written out step by step here, are:

 1. Enumerate tiles in row-major (b, h, t) order.
    forward:  t = Q tile of ``block_m`` rows, t < ceil(Lq_b / block_m)
    backward: t = KV tile of ``block_n`` keys, t < ceil(Lk_b / block_n)
 2. Work of a tile = the trip count of its inner loop.
    forward (KV blocks of ``block_n`` keys visited):
      dense        ceil(Lk_b / block_n)
      causal       ceil(min((t+1)*block_m, Lk_b) / block_n)
      band         (sliding window (left, right), causal = (none, 0); Q and KV
                   share lengths): the keys the tile's rows r0..r1 see span
                   jmin = max(0, r0 - left) .. jmax = min(Lk_b - 1, r1 + right),
                   a contiguous range, so work = jmax // block_n - jmin // block_n
                   + 1 (0 if jmax < jmin) and the tile starts at block
                   jmin // block_n
      block-sparse sum over the 128-key mask blocks c kept by any mask row of
                   the tile of ceil((min(128(c+1), Lk_b) - 128c) / block_n)
    backward (Q blocks of ``block_m`` rows visited):
      dense        ceil(Lq_b / block_m)
      causal       ceil(Lq_b / block_m) - floor(t*block_n / block_m)
      band         the rows that see keys k0..k1 span imin = max(0, k0 - right)
                   .. imax = min(Lq_b - 1, k1 + left): work = imax // block_m
                   - imin // block_m + 1 (0 if imax < imin), starting at Q
                   block imin // block_m
      block-sparse sum over the 128-row mask rows m kept by any mask column
                   of the tile of ceil((min(128(m+1), Lq_b) - 128m) / block_m)
 3. Stable sort by a sort key, descending (ties keep enumeration order).
    forward: the work.
    backward: the tile's estimated time on the dK/dV kernel, in units of
    one wave's share of a Q block's matrix products:
      key = work * (BWD_BLOCK_FIXED + ceil(keys / BWD_WAVE_KEYS)) + BWD_TILE_FIXED
    with keys = min(block_n, Lk_b - t*block_n) the tile's keys (a wave holds
    BWD_WAVE_KEYS of them; waves without keys idle), BWD_BLOCK_FIXED the
    per-block copy and barrier time and BWD_TILE_FIXED the tile boundary
    (fetch of K/V, store of dK/dV), both measured on the kernel. The work
    alone would count the partial last tile of every sequence as a full one.
 4. Deal in snake order over W workers: sorted tile i goes to worker i mod W
    when floor(i / W) is even, else to W - 1 - (i mod W).
 5. Emit worker_ptr[W+1] and, per worker in increasing i, tiles[.,4] =
    (b, h, t, work), all int32.

Dynamic forward plan. The pages pair the host sort with the hardware's
cluster launch control, which lets a running program claim its next tile
([bites] sections "What TLX changes" and "Optimizations layered on top",
item on scheduling jagged tiles). Reading: steps 1-3 as above; the plan is
the sorted list itself, worker w starts with sorted tile w (worker_ptr[w] =
min(w, N)), and tiles W, W+1, ... are claimed at run time, in order, by
whichever worker asks first.

dQ pass (the backward's Q-stationary dQ kernel). Tiles are the forward
tiles: (b, h, t) with the forward work.
 * per-sequence Q: the forward plan itself;
 * broadcast Q: every Q tile t of head h gets the contributions of all
   sequences, summed over the batch ([clarity] second paragraph). Tiles are
   grouped by g = h * ceil(Lq / block_m) + t (G groups). The plan uses
   W' = max(G, min(W, G * n)) workers, n the largest number of chunks
   (below) of any group, so that no group gets more workers than it has
   chunks to give them (W' = W when G = 0); group g owns the contiguous workers
   [floor(g W' / G), floor((g+1) W' / G)), and its tiles (b = 0..B-1) are
   stably sorted by work, descending, and dealt in snake order over them.
   Every worker thus sums one group only, into one per-worker partial.
   Because those partials are summed anyway, a long tile can be split at no
   cost: a tile of work w > DQ_CHUNK is cut into n = ceil(w / DQ_CHUNK)
   chunks of consecutive positions of its block list, the first (w mod n)
   of them one block longer, listed in (b, h, t, chunk) order before the
   sort; a chunk starting at position k0 is stored as (b, h, t + nqt * k0,
   length) with nqt = ceil(Lq / block_m).

Natural plan (the ablation baseline). The pages credit the sort and the
zigzag deal with about a fifth of the forward's speed ([bites] section
"Optimizations layered on top"); the plan they are measured against skips
both: steps 1-2 as above, no sort, and enumerated tile i goes to worker
i mod W (broadcast-Q dQ pass: the groups, W' and chunks as above, each
group's tiles in their (b, chunk) order dealt round-robin over its workers).

Block-sparse lists ([radar] section "The turning point": the block-sparse
variant only adds iteration over the selected blocks). The mask is uint8
[B, NQ, NK] over 128-row Q tiles x 128-key blocks, shared by all heads.
  forward  CSR over the Q tiles (b, t) of block_m = R * 128 rows,
           t < ceil(NQ / R): the 128-key blocks c < ceil(Lk_b/128) kept by at
           least one of the tile's mask rows m = R t + k (m < NQ, 128 m < Lq_b),
           ascending, each stored as 4 c + sum_k 2^k [row R t + k keeps c]
           (R <= 2). A tile visits the union of its rows' blocks; each row
           skips the blocks its own mask row drops.
  backward CSC over the KV tiles (b, t) of block_n = C * 128 keys,
           t < ceil(NK / C): the 128-row mask rows m < ceil(Lq_b/128) kept by
           at least one of the tile's mask columns c = C t + k (c < NK,
           128 c < Lk_b), ascending, each stored as 4 m + sum_k 2^k [column
           C t + k keeps m] (C <= 2).
"""
from __future__ import annotations

import numpy as np

MASK_BLOCK = 128
FWD, BWD, DQ = 0, 1, 2
DQ_CHUNK = 16   # longest broadcast-Q dQ chunk, in KV blocks


def cdiv(a: int, b: int) -> int:
    return -(-a // b)


def offsets_from_lengths(lengths):
    """Exclusive prefix sum of the sequence lengths (int32 [B+1])."""
    out = [0]
    for n in lengths:
        if n < 0:
            raise ValueError("negative length")
        out.append(out[-1] + int(n))
    if out[-1] >= 2**31:
        raise ValueError("total length overflows int32")
    return np.array(out, dtype=np.int32)


def _fwd_row_entries(block_mask, b, t, lq_b, lk_b, block_m):
    """Forward list of Q tile (b, t): [(c, bits)] for the kept union, ascending c."""
    _, NQ, NK = block_mask.shape
    R = block_m // MASK_BLOCK
    rows = [m for m in range(R * t, R * t + R) if m < NQ and MASK_BLOCK * m < lq_b]
    out = []
    for c in range(min(cdiv(lk_b, MASK_BLOCK), NK)):
        bits = sum(1 << (m - R * t) for m in rows if block_mask[b, m, c])
        if bits:
            out.append((c, bits))
    return out


def _bwd_col_entries(block_mask, b, t, lq_b, lk_b, block_n):
    """Backward list of KV tile (b, t): [(m, bits)] for the kept union, ascending m."""
    _, NQ, NK = block_mask.shape
    C = block_n // MASK_BLOCK
    cols = [c for c in range(C * t, C * t + C) if c < NK and MASK_BLOCK * c < lk_b]
    out = []
    for m in range(min(cdiv(lq_b, MASK_BLOCK), NQ)):
        bits = sum(1 << (c - C * t) for c in cols if block_mask[b, m, c])
        if bits:
            out.append((m, bits))
    return out


def sparse_lists(block_mask, q_lens, kv_lens, pass_, *, block_m=MASK_BLOCK, block_n=MASK_BLOCK):
    """(ptr, idx) int32: forward CSR over Q tiles (b, t) or backward CSC over KV tiles (b, t)."""
    B, NQ, NK = block_mask.shape
    ptr, idx = [0], []
    if pass_ == FWD:
        R = block_m // MASK_BLOCK
        assert R * MASK_BLOCK == block_m and 1 <= R <= 2
        for b in range(B):
            for t in range(cdiv(NQ, R)):
                for c, bits in _fwd_row_entries(block_mask, b, t, int(q_lens[b]),
                                                int(kv_lens[b]), block_m):
                    idx.append(4 * c + bits)
                ptr.append(len(idx))
    else:
        C = block_n // MASK_BLOCK
        assert C * MASK_BLOCK == block_n and 1 <= C <= 2
        for b in range(B):
            for t in range(cdiv(NK, C)):
                for m, bits in _bwd_col_entries(block_mask, b, t, int(q_lens[b]),
                                                int(kv_lens[b]), block_n):
                    idx.append(4 * m + bits)
                ptr.append(len(idx))
    return np.array(ptr, dtype=np.int32), np.array(idx, dtype=np.int32)


def band(causal, window):
    """(left, right) bounds of the visible band (None: unbounded), or None."""
    left, right = (None, None) if window is None else window
    if causal:
        right = 0 if right is None else min(right, 0)
    if left is None and right is None:
        return None
    return left, right


def band_range(lo, hi, n, left, right):
    """Rows lo..hi see keys (or keys lo..hi are seen by rows) in
    [max(0, lo - left), min(n - 1, hi + right)]: that range as (first, last)."""
    first = 0 if left is None else max(0, lo - left)
    last = n - 1 if right is None else min(n - 1, hi + right)
    return first, last


def _tile_work(pass_, b, t, lq_b, lk_b, *, block_m, block_n, causal, block_mask, window=None):
    bd = band(causal, window)
    if pass_ == FWD:
        if block_mask is not None:
            return sum(cdiv(min(MASK_BLOCK * (c + 1), lk_b) - MASK_BLOCK * c, block_n)
                       for c, _ in _fwd_row_entries(block_mask, b, t, lq_b, lk_b, block_m))
        if bd is not None:
            r0, r1 = t * block_m, min((t + 1) * block_m, lq_b) - 1
            j0, j1 = band_range(r0, r1, lk_b, *bd)
            return 0 if j1 < j0 else j1 // block_n - j0 // block_n + 1
        return cdiv(lk_b, block_n)
    nqb = cdiv(lq_b, block_m)
    if block_mask is not None:
        return sum(cdiv(min(MASK_BLOCK * (m + 1), lq_b) - MASK_BLOCK * m, block_m)
                   for m, _ in _bwd_col_entries(block_mask, b, t, lq_b, lk_b, block_n))
    if bd is not None:
        k0, k1 = t * block_n, min((t + 1) * block_n, lk_b) - 1
        # rows i see key j iff j - right <= i <= j + left
        i0, i1 = band_range(k0, k1, lq_b, bd[1], bd[0])
        return 0 if i1 < i0 else i1 // block_m - i0 // block_m + 1
    return nqb


# backward sort key constants (see step 3)
BWD_WAVE_KEYS = 32
BWD_BLOCK_FIXED = 4
BWD_TILE_FIXED = 42


def bwd_sort_key(work, t, lk_b, block_n):
    """Step 3's backward sort key of KV tile t with the given work."""
    keys = min(block_n, lk_b - t * block_n)
    return work * (BWD_BLOCK_FIXED + cdiv(keys, BWD_WAVE_KEYS)) + BWD_TILE_FIXED


def _snake(order_len, W):
    """Worker (0..W-1) of each position of a sorted list under the snake deal."""
    out = []
    for i in range(order_len):
        p = i % W
        out.append(p if (i // W) % 2 == 0 else W - 1 - p)
    return out


def _round_robin(order_len, W):
    """Worker of each position of a list under the natural plan's deal."""
    return [i % W for i in range(order_len)]


def plan_dq(q_lens, kv_lens, num_heads, num_workers, *, broadcast_q, lq=0, block_m, block_n,
            causal=False, block_mask=None, window=None, natural=False):
    """dQ pass. Returns (worker_ptr int32 [W'+1], tiles int32 [N, 4])."""
    if not broadcast_q:
        return plan(q_lens, kv_lens, num_heads, num_workers, FWD, block_m=block_m,
                    block_n=block_n, causal=causal, block_mask=block_mask, window=window,
                    natural=natural)
    B = len(kv_lens)
    nqt = cdiv(int(lq), block_m)
    G = num_heads * nqt
    if int(num_workers) < 1:
        raise ValueError("need at least one worker")
    groups = []
    for g in range(G):
        h, t = divmod(g, nqt)
        tiles = []
        for b in range(B):
            w = _tile_work(FWD, b, t, int(lq), int(kv_lens[b]), block_m=block_m,
                           block_n=block_n, causal=causal, block_mask=block_mask)
            n = max(1, cdiv(w, DQ_CHUNK))
            k0 = 0
            for c in range(n):
                length = w // n + (1 if c < w % n else 0)
                tiles.append((b, h, t + nqt * k0, length))
                k0 += length
        groups.append(tiles)
    W = int(num_workers)
    if G > 0:
        W = max(G, min(W, G * max(len(tl) for tl in groups)))
    per_worker = [[] for _ in range(W)]
    for g in range(G):
        w0, w1 = (g * W) // G, ((g + 1) * W) // G
        tiles = groups[g]
        if natural:
            order = list(range(len(tiles)))
            owner = _round_robin(len(order), w1 - w0)
        else:
            order = sorted(range(len(tiles)), key=lambda i: -tiles[i][3])   # stable
            owner = _snake(len(order), w1 - w0)
        for i, ti in enumerate(order):
            per_worker[w0 + owner[i]].append(tiles[ti])
    worker_ptr = [0]
    flat = []
    for lst in per_worker:
        flat.extend(lst)
        worker_ptr.append(len(flat))
    return (np.array(worker_ptr, dtype=np.int32),
            np.array(flat, dtype=np.int32).reshape(-1, 4))


def plan(q_lens, kv_lens, num_heads, num_workers, pass_, *, block_m, block_n,
         causal=False, block_mask=None, dynamic=False, window=None, natural=False):
    """Returns (worker_ptr int32 [W+1], tiles int32 [N, 4])."""
    B = len(kv_lens)
    W = int(num_workers)
    if W < 1:
        raise ValueError("need at least one worker")
    tiles, keys = [], []
    for b in range(B):
        lq_b, lk_b = int(q_lens[b]), int(kv_lens[b])
        n_t = cdiv(lq_b, block_m) if pass_ == FWD else cdiv(lk_b, block_n)
        for h in range(num_heads):
            for t in range(n_t):
                w = _tile_work(pass_, b, t, lq_b, lk_b, block_m=block_m, block_n=block_n,
                               causal=causal, block_mask=block_mask, window=window)
                tiles.append((b, h, t, w))
                keys.append(w if pass_ == FWD else bwd_sort_key(w, t, lk_b, block_n))
    if natural:
        if dynamic:
            raise ValueError("a natural plan is static")
        order = list(range(len(tiles)))
        owner = _round_robin(len(order), W)
    else:
        order = sorted(range(len(tiles)), key=lambda i: -keys[i])   # stable
    if dynamic:
        if pass_ != FWD:
            raise ValueError("dynamic plans are forward plans")
        worker_ptr = np.array([min(w, len(order)) for w in range(W + 1)], dtype=np.int32)
        return worker_ptr, np.array([tiles[i] for i in order], dtype=np.int32).reshape(-1, 4)
    if not natural:
        owner = _snake(len(order), W)
    per_worker = [[] for _ in range(W)]
    for i, ti in enumerate(order):
        per_worker[owner[i]].append(tiles[ti])
    worker_ptr = [0]
    flat = []
    for lst in per_worker:
        flat.extend(lst)
        worker_ptr.append(len(flat))
    arr = np.array(flat, dtype=np.int32).reshape(-1, 4)
    return np.array(worker_ptr, dtype=np.int32), arr

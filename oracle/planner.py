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
      block-sparse sum over the kept 128-key mask blocks c of the row of
                   ceil((min(128(c+1), Lk_b) - 128c) / block_n)
    backward (Q blocks of ``block_m`` rows visited):
      dense        ceil(Lq_b / block_m)
      causal       ceil(Lq_b / block_m) - floor(t*block_n / block_m)
      block-sparse number of Q blocks r < ceil(Lq_b / block_m) whose 128-row
                   mask row keeps the tile's 128-key mask column
 3. Stable sort by work, descending (ties keep enumeration order).
 4. Deal in snake order over W workers: sorted tile i goes to worker i mod W
    when floor(i / W) is even, else to W - 1 - (i mod W).
 5. Emit worker_ptr[W+1] and, per worker in increasing i, tiles[.,4] =
    (b, h, t, work), all int32.

Block-sparse lists ([radar] section "The turning point": the block-sparse
variant only adds iteration over the selected blocks). The mask is uint8
[B, NQ, NK] over 128-row Q tiles x 128-key blocks, shared by all heads.
  forward  CSR over rows (b, m), m < NQ: kept c < ceil(Lk_b/128), ascending
  backward CSC over columns (b, c), c < NK: kept m < ceil(Lq_b/128), ascending
"""
from __future__ import annotations

import numpy as np

MASK_BLOCK = 128
FWD, BWD = 0, 1


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


def sparse_lists(block_mask, q_lens, kv_lens, pass_):
    """(ptr, idx) int32: forward CSR over (b, m) or backward CSC over (b, c)."""
    B, NQ, NK = block_mask.shape
    ptr, idx = [0], []
    if pass_ == FWD:
        for b in range(B):
            nk = cdiv(int(kv_lens[b]), MASK_BLOCK)
            for m in range(NQ):
                for c in range(min(nk, NK)):
                    if block_mask[b, m, c]:
                        idx.append(c)
                ptr.append(len(idx))
    else:
        for b in range(B):
            nq = cdiv(int(q_lens[b]), MASK_BLOCK)
            for c in range(NK):
                for m in range(min(nq, NQ)):
                    if block_mask[b, m, c]:
                        idx.append(m)
                ptr.append(len(idx))
    return np.array(ptr, dtype=np.int32), np.array(idx, dtype=np.int32)


def _tile_work(pass_, b, t, lq_b, lk_b, *, block_m, block_n, causal, block_mask):
    if pass_ == FWD:
        if block_mask is not None:
            w = 0
            for c in range(min(cdiv(lk_b, MASK_BLOCK), block_mask.shape[2])):
                if block_mask[b, t * block_m // MASK_BLOCK, c]:
                    w += cdiv(min(MASK_BLOCK * (c + 1), lk_b) - MASK_BLOCK * c, block_n)
            return w
        if causal:
            return cdiv(min((t + 1) * block_m, lk_b), block_n)
        return cdiv(lk_b, block_n)
    nqb = cdiv(lq_b, block_m)
    if block_mask is not None:
        c = t * block_n // MASK_BLOCK
        return sum(1 for r in range(nqb) if block_mask[b, r * block_m // MASK_BLOCK, c])
    if causal:
        return nqb - (t * block_n) // block_m
    return nqb


def plan(q_lens, kv_lens, num_heads, num_workers, pass_, *, block_m, block_n,
         causal=False, block_mask=None):
    """Returns (worker_ptr int32 [W+1], tiles int32 [N, 4])."""
    B = len(kv_lens)
    W = int(num_workers)
    if W < 1:
        raise ValueError("need at least one worker")
    tiles = []
    for b in range(B):
        lq_b, lk_b = int(q_lens[b]), int(kv_lens[b])
        n_t = cdiv(lq_b, block_m) if pass_ == FWD else cdiv(lk_b, block_n)
        for h in range(num_heads):
            for t in range(n_t):
                w = _tile_work(pass_, b, t, lq_b, lk_b, block_m=block_m, block_n=block_n,
                               causal=causal, block_mask=block_mask)
                tiles.append((b, h, t, w))
    order = sorted(range(len(tiles)), key=lambda i: -tiles[i][3])   # stable
    owner = []
    for i in range(len(order)):
        p = i % W
        owner.append(p if (i // W) % 2 == 0 else W - 1 - p)
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

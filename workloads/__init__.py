"""Seeded synthetic inputs for jagged attention.

This module is shared by the test suite, the benchmark and the CPU oracle's
callers. It only draws random numbers and rounds them to bf16; it holds none of
the attention arithmetic, so neither side of a parity check can inherit a
mistake from the other through it.

The five workloads stand in for the packed ("jagged") shapes the pages describe:
  * packed Q/K/V plus an offsets array marking sequence boundaries, no padded
    token ("Meta's TLX Jagged Flash Attention Beats FA4 on Blackwell"
    (ainewsbites.com), section "Why attention in GEM needed a rewrite");
  * one dense Q broadcast over every sequence, dQ summed over the batch
    ("Meta's 3.2K-line Triton kernel outruns FlashAttention-4"
    (theclarity.today), second paragraph);
  * a block-sparse variant that keeps a random half of the KV blocks
    ("TLX porta l'attenzione jagged su Blackwell" (ai-radar.it), section
    "The turning point").
The pages give no shapes; the sizes below are synthetic choices.

Draw order for one workload (seeded numpy PCG64 ``default_rng(seed)``):
lengths -> Q -> K -> V -> dO, all standard normal in float32, then rounded
to bf16 with round-to-nearest-even. The block-sparse mask is drawn from its
own generator (seed 5) as ``random() < 0.5`` in C order over
(sequence, q-tile, kv-block), and block 0 of every row is forced on.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

MASK_BLOCK = 128  # block-sparse granularity (rows and keys)


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape recipe of one synthetic workload."""
    name: str
    batch: int
    heads: int
    head_dim: int
    broadcast_q: bool
    lq: int                 # rows of the shared Q (broadcast only)
    causal: bool
    lengths: str            # "uniform:lo:hi" | "lognormal:mu:sigma:lo:hi" | "const:L"
    seed: int
    mask_seed: Optional[int] = None   # block-sparse when not None
    input_seed: Optional[int] = None  # draw Q/K/V/dO from another workload's seed
    window: Optional[tuple] = None    # sliding window (left, right), None = unbounded side

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


WORKLOADS = {
    1: Workload("tiny-broadcast-q", 4, 2, 64, True, 32, False, "uniform:1:64", seed=1),
    2: Workload("gem-broadcast-q", 256, 4, 128, True, 256, False,
                "lognormal:%r:1.0:16:4096" % math.log(512.0), seed=2),
    3: Workload("jagged-self-causal", 64, 8, 128, False, 0, True, "uniform:128:8192", seed=3),
    4: Workload("dense-causal-4096", 8, 16, 128, False, 0, True, "const:4096", seed=4),
    5: Workload("block-sparse-broadcast-q", 256, 4, 128, True, 256, False,
                "lognormal:%r:1.0:16:4096" % math.log(512.0), seed=2, mask_seed=5),
    # sliding-window variant of the jagged self-attention shape: causal with a
    # 1024-key window (row i sees keys i-1023 .. i)
    6: Workload("jagged-sliding-window", 64, 8, 128, False, 0, True, "uniform:128:8192", seed=6,
                window=(1023, None)),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def draw_lengths(spec: str, batch: int, rng: np.random.Generator) -> np.ndarray:
    kind, *args = spec.split(":")
    if kind == "uniform":
        lo, hi = int(args[0]), int(args[1])
        return rng.integers(lo, hi + 1, size=batch).astype(np.int32)
    if kind == "lognormal":
        mu, sigma, lo, hi = float(args[0]), float(args[1]), float(args[2]), float(args[3])
        x = rng.lognormal(mean=mu, sigma=sigma, size=batch)
        return np.rint(np.clip(x, lo, hi)).astype(np.int32)
    if kind == "const":
        return np.full(batch, int(args[0]), dtype=np.int32)
    raise ValueError(spec)


def offsets_of(lengths: np.ndarray) -> np.ndarray:
    out = np.zeros(len(lengths) + 1, dtype=np.int64)
    np.cumsum(np.asarray(lengths, dtype=np.int64), out=out[1:])
    assert out[-1] < 2**31
    return out.astype(np.int32)


def _normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    """N(0,1) float32 draws rounded to bf16, returned as uint16 bits."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    chunk = 1 << 24
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = f32_to_bf16_bits(rng.standard_normal(e - s, dtype=np.float32))
    return out.reshape(shape)


def draw_block_mask(lengths: np.ndarray, lq_rows: int, seed: int) -> np.ndarray:
    """uint8 [B, ceil(lq/128), ceil(max_len/128)]; block 0 of every row is kept."""
    rng = np.random.default_rng(seed)
    nq = max(1, -(-int(lq_rows) // MASK_BLOCK))
    nk = max(1, -(-int(np.max(lengths)) // MASK_BLOCK)) if len(lengths) else 1
    mask = (rng.random((len(lengths), nq, nk)) < 0.5).astype(np.uint8)
    mask[:, :, 0] = 1
    return mask


@dataclasses.dataclass
class Inputs:
    """One drawn instance. Tensors are bf16 bit patterns (uint16), row-major.

    q:  [lq, H, D] when broadcast_q else [T_q, H, D]
    k, v: [T_k, H, D]
    do: [T_q, H, D]   (T_q = B*lq when broadcast_q; row b*lq + i)
    kv_offsets: int32 [B+1]; q_offsets: int32 [B+1] (per-sequence Q) or None
    block_mask: uint8 [B, nq, nk] or None
    """
    workload: Workload
    lengths: np.ndarray
    kv_offsets: np.ndarray
    q_offsets: Optional[np.ndarray]
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    do: np.ndarray
    block_mask: Optional[np.ndarray]

    @property
    def batch(self) -> int:
        return len(self.lengths)

    @property
    def t_q(self) -> int:
        if self.workload.broadcast_q:
            return self.batch * self.workload.lq
        return int(self.q_offsets[-1])

    def as_f64(self, name: str) -> np.ndarray:
        return bf16_bits_to_f32(getattr(self, name)).astype(np.float64)


def make_inputs(cfg, *, batch: Optional[int] = None, lengths: Optional[np.ndarray] = None,
                lq: Optional[int] = None, heads: Optional[int] = None,
                head_dim: Optional[int] = None, seed: Optional[int] = None,
                mask_seed: Optional[int] = None) -> Inputs:
    """Draw one instance of workload ``cfg`` (an int key of WORKLOADS or a Workload).

    Keyword overrides give smaller instances of the same recipe (used where the
    oracle must finish in seconds); explicit ``lengths`` replace the drawn ones
    but the draw still happens so the rest of the stream is unchanged.
    """
    w = WORKLOADS[cfg] if isinstance(cfg, int) else cfg
    w = dataclasses.replace(
        w,
        batch=w.batch if batch is None else batch,
        lq=w.lq if lq is None else lq,
        heads=w.heads if heads is None else heads,
        head_dim=w.head_dim if head_dim is None else head_dim,
        seed=w.seed if seed is None else seed,
        mask_seed=w.mask_seed if mask_seed is None else mask_seed,
    )
    rng = np.random.default_rng(w.seed if w.input_seed is None else w.input_seed)
    drawn = draw_lengths(w.lengths, w.batch, rng)
    if lengths is not None:
        drawn = np.asarray(lengths, dtype=np.int32)
        w = dataclasses.replace(w, batch=len(drawn))
    kv_off = offsets_of(drawn)
    H, D = w.heads, w.head_dim
    t_k = int(kv_off[-1])
    if w.broadcast_q:
        q_off = None
        q = _normal_bf16(rng, (w.lq, H, D))
        t_q = w.batch * w.lq
    else:
        q_off = kv_off.copy()
        t_q = t_k
        q = _normal_bf16(rng, (t_q, H, D))
    k = _normal_bf16(rng, (t_k, H, D))
    v = _normal_bf16(rng, (t_k, H, D))
    do = _normal_bf16(rng, (t_q, H, D))
    mask = None
    if w.mask_seed is not None:
        mask = draw_block_mask(drawn, w.lq if w.broadcast_q else int(np.max(drawn)), w.mask_seed)
    return Inputs(w, drawn, kv_off, q_off, q, k, v, do, mask)

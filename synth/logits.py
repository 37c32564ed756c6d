"""Seeded synthetic logits.

The model forward pass is not part of the beam step; seeded normal logits
stand in for the LM head's output.  Two sources:

* ``step_logits(cfg, t, b)`` -- the [K, V] block of request b at 0-based step
  t, i.i.d. per config.  Every (t, b) block has its own counter-free PCG64
  stream (``SeedSequence([LOGIT_SEED, seed_id, t, b])``), so any block can be
  regenerated anywhere (a worker process, the host of a GPU run) byte-exactly.
* ``prefix_row(cfg, b, t, prefix)`` -- one row that is a function of the
  beam's token prefix, not of its slot (a "prefix-keyed" fake LM).  Beam
  search over such rows is a well-defined search over sequences, so it can be
  compared against brute-force enumeration of every sequence.

bf16 logits are produced from fp32 by round-to-nearest-even and carried as
uint16 bit patterns.  This module contains no part of the beam step.
"""
from __future__ import annotations

import math
import os
from typing import Iterable, Iterator, Sequence, Tuple

import numpy as np

from .configs import BF16, Config

LOGIT_SEED = 0x106175
PREFIX_SEED = 0xF1E1D
BIAS_SEED = 0xB1A5


def _rng(*words: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(w) for w in words])))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32)
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + r) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def token_bias(cfg: Config) -> np.ndarray | None:
    """The per-token additive bias shared by every row of every step."""
    if cfg.bias_sigma == 0.0 and cfg.sid_shift == 0.0:
        return None
    bias = np.zeros(cfg.vocab, np.float32)
    if cfg.bias_sigma:
        bias += _rng(BIAS_SEED, cfg.seed_id).standard_normal(cfg.vocab, dtype=np.float32) \
            * np.float32(cfg.bias_sigma)
    if cfg.sid_shift:
        lo = cfg.sid_base
        hi = cfg.sid_base + cfg.depth * cfg.codebook
        bias[lo:hi] += np.float32(cfg.sid_shift)
    return bias


def eos_bias(cfg: Config, t: int) -> float:
    """Additive EOS logit bias at 0-based step t: log((t+1)/steps)."""
    if cfg.eos_bias == "log_t_over_T":
        return float(np.float32(math.log((t + 1) / cfg.steps)))
    return 0.0


def _finish(cfg: Config, t: int, x: np.ndarray, bias) -> np.ndarray:
    if bias is not None:
        x += bias
    if cfg.eos >= 0 and cfg.eos_bias:
        x[..., cfg.eos] += np.float32(eos_bias(cfg, t))
    if cfg.dtype == BF16:
        return to_bf16_bits(x)
    return x


def _normal(rng, shape, sigma: float) -> np.ndarray:
    z = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        z *= np.float32(sigma)
    return z


def step_logits(cfg: Config, t: int, b: int, rows: int | None = None) -> np.ndarray:
    """[rows, V] logits of request b at step t (rows defaults to K).

    Row j of the block is the same whatever ``rows`` is (rows are drawn in
    order from one stream), so a caller may ask for only the first few."""
    rows = cfg.beam if rows is None else rows
    x = _normal(_rng(LOGIT_SEED, cfg.seed_id, t, b), (rows, cfg.vocab), cfg.sigma)
    return _finish(cfg, t, x, token_bias(cfg))


def prefix_row(cfg: Config, b: int, t: int, prefix: Sequence[int]) -> np.ndarray:
    """A [V] row keyed by (request, step, token prefix)."""
    words = [PREFIX_SEED, cfg.seed_id, b, t] + [int(p) + 1 for p in prefix]
    x = _normal(_rng(*words), (1, cfg.vocab), cfg.sigma)
    return _finish(cfg, t, x, token_bias(cfg))[0]


def prefix_block(cfg: Config, b: int, t: int, prefixes: Iterable[Sequence[int] | None]) -> np.ndarray:
    """[len(prefixes), V] rows; a None prefix (empty or finished slot, whose
    row is never read) gets zeros."""
    prefixes = list(prefixes)
    dt = np.uint16 if cfg.dtype == BF16 else np.float32
    out = np.zeros((len(prefixes), cfg.vocab), dt)
    for j, p in enumerate(prefixes):
        if p is not None:
            out[j] = prefix_row(cfg, b, t, p)
    return out


def _block_job(args) -> Tuple[int, np.ndarray]:
    cfg, t, b, rows = args
    return b, step_logits(cfg, t, b, rows)


def default_workers() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def iter_step_blocks(cfg: Config, t: int, bs: Iterable[int] | None = None,
                     rows: int | None = None, workers: int | None = None
                     ) -> Iterator[Tuple[int, np.ndarray]]:
    """Yield (b, block) for the requested requests, generated in worker
    processes when the blocks are large.  Order of yield is b order."""
    bs = list(range(cfg.batch) if bs is None else bs)
    rows = cfg.beam if rows is None else rows
    workers = default_workers() if workers is None else workers
    if workers <= 1 or len(bs) <= 1 or rows * cfg.vocab < (1 << 22):
        for b in bs:
            yield b, step_logits(cfg, t, b, rows)
        return
    import concurrent.futures as cf
    import multiprocessing as mp
    ctx = mp.get_context("spawn")
    with cf.ProcessPoolExecutor(max_workers=min(workers, len(bs)), mp_context=ctx) as ex:
        for b, blk in ex.map(_block_job, [(cfg, t, b, rows) for b in bs]):
            yield b, blk


def full_step(cfg: Config, t: int, rows: int | None = None, workers: int | None = None) -> np.ndarray:
    """[B, rows, V] host array of step t (fp32 or bf16 bits)."""
    rows = cfg.beam if rows is None else rows
    dt = np.uint16 if cfg.dtype == BF16 else np.float32
    out = np.empty((cfg.batch, rows, cfg.vocab), dt)
    for b, blk in iter_step_blocks(cfg, t, rows=rows, workers=workers):
        out[b] = blk
    return out

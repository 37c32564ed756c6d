"""Python access to the C oracle of one trie-constrained beam step.

TEST INFRASTRUCTURE ONLY: the slow reference the GPU library is checked
against.  Only the tests, the smoke check and the benchmark's CPU-baseline leg
use it; the GPU library's package never imports it and it never imports that
package.  The definition it implements is written out in oracle/oracle.h.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass, field
from typing import Callable, List, Optional

import numpy as np

from . import build as _build

_lib = None


class _Args(C.Structure):
    _fields_ = [
        ("beam", C.c_int32), ("vocab", C.c_int32), ("eos", C.c_int32), ("dtype", C.c_int32),
        ("row_stride", C.c_int64), ("max_steps", C.c_int32), ("step", C.c_int32),
        ("offsets", C.c_void_p), ("num_nodes", C.c_int64),
        ("tokens", C.c_void_p), ("children", C.c_void_p),
        ("temperature", C.c_float), ("request", C.c_int32), ("seed", C.c_uint64),
        ("alpha", C.c_float), ("min_length", C.c_int32), ("banned", C.c_void_p),
        ("n_banned", C.c_int32), ("norm_mode", C.c_int32), ("norm_lo", C.c_int32),
        ("norm_hi", C.c_int32),
    ]


def lib():
    """Load liboracle.so, building it first only if it is absent."""
    global _lib
    if _lib is None:
        path = os.environ.get("GRO_LIBRARY")  # another build of the oracle (the sanitized one)
        if not path:
            path = _build.LIB
            if not os.path.exists(path):
                _build.build()
        L = C.CDLL(path)
        L.gro_step.restype = C.c_int
        L.gro_step.argtypes = [C.POINTER(_Args)] + [C.c_void_p] * 13
        L.gro_row_lse.restype = C.c_float
        L.gro_row_lse.argtypes = [C.c_void_p, C.c_int32, C.c_int32]
        L.gro_philox4x32_10.restype = None
        L.gro_philox4x32_10.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p]
        L.gro_gumbel.restype = C.c_float
        L.gro_gumbel.argtypes = [C.c_uint64, C.c_int32, C.c_int32, C.c_int64]
        L.gro_length_penalty.restype = C.c_float
        L.gro_length_penalty.argtypes = [C.c_int32, C.c_float]
        L.gro_backward.restype = C.c_int
        L.gro_backward.argtypes = [C.c_int32, C.c_int32, C.c_int32] + [C.c_void_p] * 5 + [C.c_float] + [C.c_void_p] * 3
        L.gro_backward_scatter.restype = C.c_int
        L.gro_backward_scatter.argtypes = [C.c_int32, C.c_int32] + [C.c_void_p] * 4
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def row_lse(row: np.ndarray) -> np.float32:
    """Oracle row normaliser of one fp32 row or bf16-bits (uint16) row."""
    row = np.ascontiguousarray(row)
    dt = 1 if row.dtype == np.uint16 else 0
    if dt == 0:
        row = row.astype(np.float32, copy=False)
    return np.float32(lib().gro_row_lse(_p(row), row.shape[-1], dt))


def philox4x32_10(ctr, key) -> np.ndarray:
    """Philox4x32-10 of one counter block (4 words) under one key (2 words)."""
    c = np.ascontiguousarray(ctr, np.uint32)
    k = np.ascontiguousarray(key, np.uint32)
    out = np.zeros(4, np.uint32)
    lib().gro_philox4x32_10(_p(c), _p(k), _p(out))
    return out


def gumbel(seed: int, request: int, t: int, flat: int) -> np.float32:
    """The Gumbel draw of candidate `flat` of a request at step t."""
    return np.float32(lib().gro_gumbel(seed, request, t, flat))


def length_penalty(length: int, alpha: float) -> np.float32:
    """pen(len) = (float)pow((5 + len) / 6, alpha)."""
    return np.float32(lib().gro_length_penalty(length, alpha))


NORM_MODES = {"full": 0, "range": 1, "slice": 2, "none": 3}


@dataclass
class StepOut:
    score: np.ndarray   # [K] f32
    node: np.ndarray    # [K] i32
    fin: np.ndarray     # [K] u8
    seq: np.ndarray     # [K, T] i32
    parent: np.ndarray  # [K] i32
    token: np.ndarray   # [K] i32
    lse: np.ndarray     # [K] f32, NaN where the row was not read
    n_candidates: int


def step(logits: np.ndarray, score, node, fin, seq, t: int, *, eos: int = -1,
         level: Optional[tuple] = None, temperature: float = 0.0, seed: int = 0,
         request: int = 0, alpha: float = 0.0, min_length: int = 0,
         banned=None, norm: str = "full", norm_range=(0, 0)) -> StepOut:
    """One oracle step of one request.

    logits: [K, V] float32, or uint16 bf16 bit patterns.
    level:  (offsets, tokens, children) of trie level t, or None.
    temperature > 0 samples (Gumbel top-K; see oracle.h) with the Philox key
    `seed`; `request` is the request index in the noise counter.
    alpha, min_length, banned: GNMT length penalty exponent, minimum
    hypothesis length for EOS, tokens never emitted (see oracle.h).
    norm: "full", "range" (over norm_range = (lo, hi)), "slice", or "none"
    (the values are log-probabilities already: lse = 0).
    """
    logits = np.ascontiguousarray(logits)
    dt = 1 if logits.dtype == np.uint16 else 0
    if dt == 0 and logits.dtype != np.float32:
        raise TypeError("logits must be float32 or uint16 (bf16 bits)")
    K, V = logits.shape
    seq = np.ascontiguousarray(seq, np.int32)
    T = seq.shape[1]
    score = np.ascontiguousarray(score, np.float32)
    node = np.ascontiguousarray(node, np.int32)
    fin = np.ascontiguousarray(fin, np.uint8)
    a = _Args(beam=K, vocab=V, eos=eos, dtype=dt, row_stride=V, max_steps=T, step=t,
              temperature=temperature, request=request, seed=seed, alpha=alpha,
              min_length=min_length, norm_mode=NORM_MODES[norm],
              norm_lo=norm_range[0], norm_hi=norm_range[1])
    keep = []
    if banned is not None and len(banned):
        ban = np.ascontiguousarray(banned, np.int32)
        keep.append(ban)
        a.banned, a.n_banned = ban.ctypes.data, len(ban)
    if level is not None:
        off, tok, ch = (np.ascontiguousarray(level[0], np.int64),
                        np.ascontiguousarray(level[1], np.int32),
                        np.ascontiguousarray(level[2], np.int32))
        keep += [off, tok, ch]
        a.offsets, a.num_nodes, a.tokens, a.children = (
            off.ctypes.data, len(off) - 1, tok.ctypes.data, ch.ctypes.data)
    out = StepOut(np.empty(K, np.float32), np.empty(K, np.int32), np.empty(K, np.uint8),
                  np.empty((K, T), np.int32), np.empty(K, np.int32), np.empty(K, np.int32),
                  np.empty(K, np.float32), 0)
    nc = np.zeros(1, np.int64)
    rc = lib().gro_step(C.byref(a), _p(logits), _p(score), _p(node), _p(fin), _p(seq),
                        _p(out.score), _p(out.node), _p(out.fin), _p(out.seq),
                        _p(out.parent), _p(out.token), _p(out.lse), _p(nc))
    if rc != 0:
        raise RuntimeError(f"gro_step failed with code {rc}")
    out.n_candidates = int(nc[0])
    return out


@dataclass
class Search:
    """Oracle beam state of B requests, advanced one step at a time.

    Starts with one live slot per request (score +0.0, the trie root), every
    other slot empty, sequences all -1."""

    batch: int
    beam: int
    vocab: int
    max_steps: int
    eos: int = -1
    trie: object = None   # anything with .offsets/.tokens/.children lists
    temperature: float = 0.0   # > 0: Gumbel top-K sampling with Philox key `seed`
    seed: int = 0
    alpha: float = 0.0         # GNMT length penalty exponent
    min_length: int = 0        # EOS allowed once a hypothesis has this many tokens
    banned: object = None      # token ids never emitted
    norm: str = "full"         # "full", "range" (over norm_range) or "slice"
    norm_range: tuple = (0, 0)
    t: int = 0
    score: np.ndarray = field(init=False)
    node: np.ndarray = field(init=False)
    fin: np.ndarray = field(init=False)
    seq: np.ndarray = field(init=False)
    parents: List[np.ndarray] = field(default_factory=list)
    tokens: List[np.ndarray] = field(default_factory=list)
    lses: List[np.ndarray] = field(default_factory=list)
    n_candidates: List[np.ndarray] = field(default_factory=list)

    def __post_init__(self):
        B, K, T = self.batch, self.beam, self.max_steps
        self.score = np.full((B, K), -np.inf, np.float32)
        self.score[:, 0] = 0.0
        self.node = np.full((B, K), -1, np.int32)
        if self.trie is not None:
            self.node[:, 0] = 0
        self.fin = np.zeros((B, K), np.uint8)
        self.seq = np.full((B, K, T), -1, np.int32)

    def level(self, t: int):
        if self.trie is None:
            return None
        return (self.trie.offsets[t], self.trie.tokens[t], self.trie.children[t])

    def prefixes(self, b: int):
        """Token prefix of every slot of request b; None where the row is
        not read (empty or finished slot)."""
        out = []
        for j in range(self.beam):
            if self.score[b, j] == -np.inf or self.fin[b, j]:
                out.append(None)
            else:
                out.append([int(x) for x in self.seq[b, j, :self.t]])
        return out

    def step(self, logits_of: Callable[[int], np.ndarray], requests=None):
        """Advance requests (default all) by one step; logits_of(b) gives
        the [K, V] block of request b."""
        B, K = self.batch, self.beam
        par = np.full((B, K), -1, np.int32)
        tok = np.full((B, K), -1, np.int32)
        lse = np.full((B, K), np.nan, np.float32)
        nc = np.zeros(B, np.int64)
        lvl = self.level(self.t)
        for b in (range(B) if requests is None else requests):
            o = step(logits_of(b), self.score[b], self.node[b], self.fin[b], self.seq[b],
                     self.t, eos=self.eos, level=lvl, temperature=self.temperature,
                     seed=self.seed, request=b, alpha=self.alpha, min_length=self.min_length,
                     banned=self.banned, norm=self.norm, norm_range=self.norm_range)
            self.score[b], self.node[b], self.fin[b], self.seq[b] = o.score, o.node, o.fin, o.seq
            par[b], tok[b], lse[b], nc[b] = o.parent, o.token, o.lse, o.n_candidates
        self.parents.append(par)
        self.tokens.append(tok)
        self.lses.append(lse)
        self.n_candidates.append(nc)
        self.t += 1


def backward(parents, tokens, score_final, seq_final, grad_final, alpha: float = 0.0):
    """Paths and weights of one request's final beams (gro_backward).

    parents, tokens: [steps, K] history; score_final [K]; seq_final [K, T];
    grad_final [K].  Returns (path_slot [steps, K], path_token [steps, K],
    weight [K]).
    """
    par = np.ascontiguousarray(parents, np.int32)
    tok = np.ascontiguousarray(tokens, np.int32)
    steps, K = par.shape
    seqf = np.ascontiguousarray(seq_final, np.int32)
    T = seqf.shape[1]
    sc = np.ascontiguousarray(score_final, np.float32)
    g = np.ascontiguousarray(grad_final, np.float32)
    ps = np.empty((steps, K), np.int32)
    pt = np.empty((steps, K), np.int32)
    w = np.empty(K, np.float32)
    rc = lib().gro_backward(K, T, steps, _p(par), _p(tok), _p(sc), _p(seqf), _p(g), alpha,
                            _p(ps), _p(pt), _p(w))
    if rc != 0:
        raise RuntimeError(f"gro_backward failed with code {rc}")
    return ps, pt, w


def backward_scatter(path_slot_t, path_token_t, weight, grad: np.ndarray) -> np.ndarray:
    """Add step t's log-probability gradient into grad [K, V] (float32, in
    place; gro_backward_scatter) and return it."""
    ps = np.ascontiguousarray(path_slot_t, np.int32)
    pt = np.ascontiguousarray(path_token_t, np.int32)
    w = np.ascontiguousarray(weight, np.float32)
    assert grad.dtype == np.float32 and grad.flags.c_contiguous
    K, V = grad.shape
    rc = lib().gro_backward_scatter(K, V, _p(ps), _p(pt), _p(w), _p(grad))
    if rc != 0:
        raise RuntimeError(f"gro_backward_scatter failed with code {rc}")
    return grad

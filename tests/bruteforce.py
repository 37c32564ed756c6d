"""Brute-force enumeration of every hypothesis a beam search can reach.

Independent of the oracle: no beam, no truncation, no selection heap.  Every
valid prefix (trie mode) or every token sequence (unconstrained mode, with
finished sequences frozen after EOS) is scored by folding the step
definition along its own path, and the hypotheses of each step are put in
the order beam search uses:

    higher score first, then lower flat index, where
    flat = (rank of the parent hypothesis at the previous step) * V + token

(a finished hypothesis is carried with token slot = EOS and keeps its score).
With a beam width at least the number of hypotheses alive at every step,
beam search keeps every hypothesis and must return exactly this list
(beamgrad README, "How it works": every live beam proposes every token and
the K best survive; nothing is pruned when K is large enough).

Scores use the same arithmetic the pages' step uses: the row normaliser is
m + log(sum exp(x - m)) in fp64 (the sum taken exactly with math.fsum),
rounded once to fp32, and lp = x - lse, c = S + lp are fp32 operations.
"""
from __future__ import annotations

import math
from typing import Callable, Dict, List, Sequence, Tuple

import numpy as np

f32 = np.float32


def lse32(row: np.ndarray) -> np.float32:
    x = np.asarray(row, np.float64)
    m = x.max()
    if m == -np.inf:
        return f32(-np.inf)
    return f32(m + math.log(math.fsum(np.exp(x - m).tolist())))


class Hyp:
    __slots__ = ("score", "tokens", "fin", "flat", "rank", "key")

    def __init__(self, score, tokens, fin, flat, key=None):
        self.score, self.tokens, self.fin, self.flat = score, tokens, fin, flat
        self.key = score if key is None else key   # ranking score
        self.rank = -1


def gnmt_penalty(length: int, alpha: float) -> np.float32:
    """((5 + length) / 6) ** alpha in double, rounded to fp32 (beamgrad
    README, "How it works")."""
    return f32(((5.0 + length) / 6.0) ** float(alpha))


def _order(hyps: List[Hyp]) -> List[Hyp]:
    hyps = sorted(hyps, key=lambda h: (-float(h.key), h.flat))
    for r, h in enumerate(hyps):
        h.rank = r
    return hyps


def trie_hypotheses(codes: np.ndarray, codebook: int, sid_base: int, vocab: int,
                    row_of: Callable[[int, Tuple[int, ...]], np.ndarray],
                    norm: str = "full", norm_range=(0, 0)) -> List[List[Hyp]]:
    """All valid prefixes of a catalog, per step, in beam order.

    codes:   (N, D) catalog of distinct SIDs (any order).
    row_of:  (t, prefix tokens) -> [V] float32 logits of that prefix.
    norm:    the normaliser of each row: "full" (every token), "range" (the
             tokens of norm_range = [lo, hi) only; other tokens are never
             emitted) or "slice" (the prefix's own valid continuations only).
    Returns steps[t] = ordered list of Hyp for prefixes of length t+1.
    """
    N, D = codes.shape
    tokens = sid_base + np.arange(D)[None, :] * codebook + codes.astype(np.int64)
    prev: Dict[Tuple[int, ...], Hyp] = {(): Hyp(f32(0.0), (), False, 0)}
    prev[()].rank = 0
    steps = []
    lo, hi = norm_range
    for t in range(D):
        cur: Dict[Tuple[int, ...], Hyp] = {}
        rows: Dict[Tuple[int, ...], Tuple[np.ndarray, np.float32]] = {}
        kids: Dict[Tuple[int, ...], List[int]] = {}
        for sid in map(tuple, tokens[:, :t + 1].tolist()):
            kids.setdefault(sid[:-1], [])
            if sid[-1] not in kids[sid[:-1]]:
                kids[sid[:-1]].append(sid[-1])
        for sid in map(tuple, tokens[:, :t + 1].tolist()):
            if sid in cur:
                continue
            pre, v = sid[:-1], sid[-1]
            if (norm == "range" and not lo <= v < hi) or pre not in prev:
                continue   # out of range, or continues a prefix that was never emitted
            parent = prev[pre]
            if pre not in rows:
                x = np.asarray(row_of(t, pre), np.float32)
                if norm == "range":
                    rows[pre] = (x, lse32(x[lo:hi]))
                elif norm == "slice":
                    rows[pre] = (x, lse32(x[sorted(kids[pre])]))
                else:
                    rows[pre] = (x, lse32(x))
            x, l = rows[pre]
            c = f32(parent.score + f32(x[v] - l))
            if c == -np.inf:
                continue
            cur[sid] = Hyp(c, sid, False, parent.rank * vocab + v)
        ordered = _order(list(cur.values()))
        steps.append(ordered)
        prev = {h.tokens: h for h in ordered}
    return steps


def free_hypotheses(vocab: int, steps: int, eos: int,
                    row_of: Callable[[int, Tuple[int, ...]], np.ndarray],
                    alpha: float = 0.0, min_length: int = 0, banned=()) -> List[List[Hyp]]:
    """Every token sequence of an unconstrained search, per step, in beam
    order.  A sequence that emitted EOS is finished: at later steps it is
    carried unchanged (token -1) with flat = parent rank * V + eos.
    Ranked by score / gnmt_penalty(length), length = tokens including EOS;
    banned tokens and EOS before min_length are never emitted (beamgrad
    README, "Features")."""
    prev = [Hyp(f32(0.0), (), False, 0)]
    prev[0].rank = 0
    out = []
    for t in range(steps):
        cur = []
        for p in prev:
            if p.fin:
                n = sum(1 for tok in p.tokens if tok != -1)
                cur.append(Hyp(p.score, p.tokens + (-1,), True, p.rank * vocab + eos,
                               f32(p.score / gnmt_penalty(n, alpha))))
                continue
            x = np.asarray(row_of(t, p.tokens), np.float32)
            l = lse32(x)
            pen = gnmt_penalty(t + 1, alpha)
            for v in range(vocab):
                if v in banned or (v == eos and t + 1 < min_length):
                    continue
                c = f32(p.score + f32(x[v] - l))
                if c == -np.inf:
                    continue
                cur.append(Hyp(c, p.tokens + (v,), v == eos, p.rank * vocab + v, f32(c / pen)))
        prev = _order(cur)
        out.append(prev)
    return out


def greedy_path(D: int, children_of: Callable[[int, Tuple[int, ...]], Sequence[int]],
                row_of: Callable[[int, Tuple[int, ...]], np.ndarray]):
    """Textbook greedy decoding: at every step take the valid token with
    the largest logit (lowest token id among equal logits)."""
    pre: Tuple[int, ...] = ()
    score = f32(0.0)
    for t in range(D):
        x = np.asarray(row_of(t, pre), np.float32)
        l = lse32(x)
        valid = list(children_of(t, pre))
        best = max(valid, key=lambda v: (float(f32(score + f32(x[v] - l))), -v))
        score = f32(score + f32(x[best] - l))
        pre = pre + (best,)
    return pre, score

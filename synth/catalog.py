"""Seeded synthetic SID catalogs and their per-level CSR tries.

A catalog is a lexicographically sorted array of distinct semantic IDs, one
row of ``depth`` codes each.  The trie that restricts decoding (FlashRec
README, "Decoding": a dense or CSR-sparse trie restricts decoding to the
catalog of valid SIDs) is stored per level in CSR form:

  level L in [0, depth):
    offsets[L]  int64 [num_nodes[L] + 1]  edges of node n are offsets[n] .. offsets[n+1]-1
    tokens[L]   int32 [E_L]               child token ids, strictly increasing per node
    children[L] int32 [E_L]               child node id at level L+1

Node ids are local to a level; the root is node 0 of level 0; a node at level
``depth`` is a leaf and its id is the SID's row in the sorted catalog.

This module builds inputs only.  It contains no part of the beam step.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List

import numpy as np

from .configs import Config

CATALOG_SEED = 0x5EED


def _rng(*words: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(w) for w in words])))


def _code_dtype(codebook: int):
    if codebook <= 256:
        return np.uint8
    if codebook <= 65536:
        return np.uint16
    return np.int32


@dataclass
class Trie:
    """Per-level CSR trie plus the catalog it was built from."""

    depth: int
    vocab: int
    codebook: int
    sid_base: int
    offsets: List[np.ndarray]
    tokens: List[np.ndarray]
    children: List[np.ndarray]
    codes: np.ndarray = field(default=None, repr=False)  # (N, depth) sorted catalog

    @property
    def num_nodes(self) -> List[int]:
        """Nodes per level 0..depth (level depth = leaves)."""
        return [len(o) - 1 for o in self.offsets] + [len(self.children[-1])]

    def max_fanout(self, level: int) -> int:
        o = self.offsets[level]
        return int(np.max(np.diff(o))) if len(o) > 1 else 0

    def token_of(self, level: int, code):
        return self.sid_base + level * self.codebook + np.asarray(code, np.int64)


def keys_to_codes(keys: np.ndarray, depth: int, codebook: int) -> np.ndarray:
    keys = np.asarray(keys, np.int64)
    out = np.empty((len(keys), depth), _code_dtype(codebook))
    k = keys.copy()
    for L in range(depth - 1, -1, -1):
        out[:, L] = k % codebook
        k //= codebook
    return out


def _zipf_p(codebook: int, s: float) -> np.ndarray:
    r = np.arange(1, codebook + 1, dtype=np.float64)
    p = r ** (-s)
    return p / p.sum()


def _first_distinct(rng, n: int, draw) -> np.ndarray:
    """The first ``n`` distinct keys, in draw order, of a stream of draws."""
    keys = np.empty(0, np.int64)
    have = 0
    while True:
        m = int((n - have) * 1.3) + 4096
        keys = np.concatenate([keys, draw(rng, m)])
        uniq, first = np.unique(keys, return_index=True)
        have = len(uniq)
        if have >= n:
            sel = np.sort(first)[:n]
            return np.sort(keys[sel])


def _subsets(rng, fanouts: np.ndarray, codebook: int, chunk: int = 1 << 16) -> np.ndarray:
    """For each node, ``fanout`` distinct codes chosen uniformly, sorted;
    concatenated in node order."""
    out = []
    base = np.arange(codebook, dtype=np.uint16)
    cols = np.arange(codebook)[None, :]
    for s in range(0, len(fanouts), chunk):
        f = fanouts[s:s + chunk]
        perm = rng.permuted(np.tile(base, (len(f), 1)), axis=1)
        sel = np.where(cols < f[:, None], perm, codebook).astype(np.uint16)
        sel.sort(axis=1)
        out.append(sel[sel < codebook])
    return np.concatenate(out)


def _branching_codes(cfg: Config, rng) -> np.ndarray:
    """Random branching tree: the root draws ``root_fanout`` distinct codes,
    every other inner node 1 + Binomial(codebook-1, (mean-1)/(codebook-1))
    distinct codes; the leaves, in lexicographic order, truncated to n_sids."""
    D, cb = cfg.depth, cfg.codebook
    p = (cfg.mean_fanout - 1) / (cb - 1)
    parents, codes = [], []
    n_nodes = 1
    for L in range(D):
        if L == 0:
            f = np.array([cfg.root_fanout], np.int64)
        else:
            f = 1 + rng.binomial(cb - 1, p, size=n_nodes)
        c = _subsets(rng, f, cb)
        par = np.repeat(np.arange(n_nodes, dtype=np.int32), f)
        parents.append(par)
        codes.append(c.astype(np.uint8 if cb <= 256 else np.uint16))
        n_nodes = len(c)
    n_leaves = n_nodes
    if n_leaves < cfg.n_sids:
        raise RuntimeError(f"branching catalog has {n_leaves} leaves < {cfg.n_sids}")
    N = cfg.n_sids
    out = np.empty((N, D), _code_dtype(cb))
    idx = np.arange(N, dtype=np.int64)
    for L in range(D - 1, -1, -1):
        out[:, L] = codes[L][idx]
        idx = parents[L][idx]
    return out


def make_codes(cfg: Config) -> np.ndarray:
    """The sorted catalog of ``cfg`` as an (n_sids, depth) code array."""
    if not cfg.constrained:
        raise ValueError(f"{cfg.name} has no catalog")
    D, cb, N = cfg.depth, cfg.codebook, cfg.n_sids
    rng = _rng(CATALOG_SEED, cfg.seed_id)
    if cfg.catalog == "uniform":
        space = cb ** D
        keys = np.sort(rng.choice(space, size=N, replace=False)).astype(np.int64)
        return keys_to_codes(keys, D, cb)
    if cfg.catalog in ("zipf0", "zipf01"):
        zl = {"zipf0": (0,), "zipf01": (0, 1)}[cfg.catalog]
        p = _zipf_p(cb, cfg.zipf_s)

        def draw(r, m):
            k = np.zeros(m, np.int64)
            for L in range(D):
                if L in zl:
                    c = r.choice(cb, size=m, p=p)
                else:
                    c = r.integers(0, cb, size=m)
                k = k * cb + c
            return k

        return keys_to_codes(_first_distinct(rng, N, draw), D, cb)
    if cfg.catalog == "branching":
        return _branching_codes(cfg, rng)
    raise ValueError(cfg.catalog)


def csr_from_codes(codes: np.ndarray, codebook: int, sid_base: int, vocab: int) -> Trie:
    """Per-level CSR of the trie of a sorted, duplicate-free catalog."""
    N, D = codes.shape
    new = np.zeros(N, bool)
    if N:
        new[0] = True
    prev_ids = np.zeros(N, np.int32)
    n_prev = 1
    offs, toks, chs = [], [], []
    for L in range(D):
        if N > 1:
            new[1:] |= codes[1:, L] != codes[:-1, L]
        ids = (np.cumsum(new, dtype=np.int64) - 1).astype(np.int32)
        starts = np.flatnonzero(new)
        parent = prev_ids[starts]
        tok = (sid_base + L * codebook + codes[starts, L].astype(np.int64)).astype(np.int32)
        counts = np.bincount(parent, minlength=n_prev)
        off = np.zeros(n_prev + 1, np.int64)
        np.cumsum(counts, out=off[1:])
        offs.append(off)
        toks.append(tok)
        chs.append(np.arange(len(starts), dtype=np.int32))
        prev_ids = ids
        n_prev = len(starts)
    return Trie(depth=D, vocab=vocab, codebook=codebook, sid_base=sid_base,
                offsets=offs, tokens=toks, children=chs, codes=codes)


def make_trie(cfg: Config) -> Trie:
    codes = make_codes(cfg)
    return csr_from_codes(codes, cfg.codebook, cfg.sid_base, cfg.vocab)


def sid_tokens(trie: Trie, codes: np.ndarray) -> np.ndarray:
    """Vocabulary token ids of SIDs given as code rows."""
    codes = np.asarray(codes, np.int64)
    L = np.arange(codes.shape[-1])
    return trie.sid_base + L * trie.codebook + codes


def relabel(trie: Trie, seed: int):
    """The same trie with the node ids of every level below the root
    permuted at random: each level's CSR rows are reordered to the new ids
    and the child ids mapped.  The catalog, its tokens and every path are
    unchanged; only the node numbering differs, so a consumer that follows
    child ids gives the same tokens and the mapped nodes, while one that
    takes an edge's index for its child id does not.  Returns (trie, perms)
    with perms[L][old id] = new id (perms[0] is the root's identity)."""
    rng = np.random.default_rng(seed)
    nn = trie.num_nodes
    perms = [np.zeros(1, np.int64)] + [rng.permutation(n) for n in nn[1:]]
    offs, toks, chs = [], [], []
    for L in range(trie.depth):
        off, tok, ch = trie.offsets[L], trie.tokens[L], trie.children[L]
        inv = np.argsort(perms[L])            # new id -> old id
        cnt = np.diff(off)[inv]
        new_off = np.zeros(len(off), np.int64)
        np.cumsum(cnt, out=new_off[1:])
        # edge i of new node n is old edge off[inv[n]] + (i - new_off[n])
        idx = np.repeat(off[inv] - new_off[:-1], cnt) + np.arange(new_off[-1], dtype=np.int64)
        offs.append(new_off)
        toks.append(tok[idx].astype(np.int32))
        chs.append(perms[L + 1][ch[idx]].astype(np.int32))
    return Trie(trie.depth, trie.vocab, trie.codebook, trie.sid_base, offs, toks, chs,
                trie.codes), perms

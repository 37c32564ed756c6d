"""Pins of the oracle's normalisation variants, on the CPU: RANGE (FlashRec
README, "Decoding": lm_head only over the SID token range) and SLICE
(Qwen-2.5-1B-RLCD-Fast model card, "Sub-Vocabulary Logit Slicing": exact
probabilities over the candidate slice only).

Fixed from outside the oracle by: identities (RANGE over [0, V) is FULL,
SLICE without a trie is FULL), closed forms (a slice's probabilities sum to
one; the card's exp(z/T) / sum exp(z/T) at temperature T; scipy logsumexp over
the range), a hand-worked case (tests/golden/normalisation.json) and
exhaustive enumeration of tiny catalogs (tests/bruteforce.py).
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle
import synth
from bruteforce import trie_hypotheses

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "normalisation.json")
f32 = np.float32


def _one_level_trie(children, V):
    """Level-0 CSR with one node per live beam (node j has children[j])."""
    off = np.zeros(len(children) + 1, np.int64)
    for j, c in enumerate(children):
        off[j + 1] = off[j] + len(c)
    tok = np.array([v for c in children for v in c], np.int32)
    ch = np.arange(len(tok), dtype=np.int32)
    return off, tok, ch


def test_slice_lifts_a_lone_child():
    c = json.load(open(GOLDEN))["cases"][0]
    x = np.array(c["rows"], np.float32)
    K = len(c["rows"])
    level = _one_level_trie(c["children"], c["vocab"])
    st = (np.zeros(K, np.float32), np.arange(K, dtype=np.int32), np.zeros(K, np.uint8),
          np.full((K, 2), -1, np.int32))
    for mode, key in (("full", "expect_full"), ("slice", "expect_slice")):
        o = oracle.step(x, *st, 0, level=level, norm=mode)
        e = c[key]
        assert (int(o.parent[0]), int(o.token[0])) == (e["parent"], e["token"])
        assert abs(float(o.score[0]) - e["approx_score"]) < 1e-5


def test_slice_probabilities_sum_to_one_and_follow_the_card():
    cfg = synth.get("c2").shrink(batch=2, beam=16, n_sids=2000, name="slice")
    trie = synth.make_trie(cfg)
    for T in (0.0, 0.7):
        S = oracle.Search(batch=cfg.batch, beam=cfg.beam, vocab=cfg.vocab, max_steps=cfg.steps,
                          trie=trie, norm="slice", temperature=T, seed=3)
        for t in range(cfg.steps):
            x = synth.full_step(cfg, t)
            node_before = S.node.copy()
            score_before = S.score.copy()
            S.step(lambda b: x[b])
            off, tok = trie.offsets[t], trie.tokens[t]
            for b in range(cfg.batch):
                for j in range(cfg.beam):
                    if not np.isfinite(score_before[b, j]):
                        continue
                    n = node_before[b, j]
                    kids = tok[off[n]:off[n + 1]]
                    inv_t = f32(1.0) / f32(T) if T > 0 else f32(1.0)
                    z = (x[b, j, kids].astype(np.float32) * inv_t).astype(np.float64)
                    lse = float(S.lses[-1][b, j])
                    assert abs(lse - logsumexp(z)) <= 4e-7 * max(1.0, abs(lse))
                    assert abs(math.fsum(np.exp(z - lse)) - 1.0) < 1e-5


def test_range_over_everything_is_full_and_range_lse_is_logsumexp():
    cfg = synth.get("c5").shrink(batch=2, beam=6, vocab=300, steps=3)
    runs = {}
    for mode, rng in (("full", (0, 0)), ("range", (0, cfg.vocab)), ("range", (40, 250))):
        S = oracle.Search(batch=cfg.batch, beam=cfg.beam, vocab=cfg.vocab, max_steps=cfg.steps,
                          eos=cfg.eos if rng[0] == 0 else 45, norm=mode, norm_range=rng)
        for t in range(cfg.steps):
            x = synth.full_step(cfg, t)
            prev = S.score.copy()
            S.step(lambda b: x[b])
            if rng == (40, 250):
                for b in range(cfg.batch):
                    toks = S.seq[b][np.isfinite(S.score[b])]
                    assert np.all((toks == -1) | ((toks >= 40) & (toks < 250)))
                    for j in np.flatnonzero(np.isfinite(prev[b]) & ~np.isnan(S.lses[-1][b])):
                        ref = f32(logsumexp(x[b, j, 40:250].astype(np.float64)))
                        assert abs(float(S.lses[-1][b, j]) - float(ref)) <= 2e-7 * max(1.0, abs(float(ref)))
        runs[(mode, rng)] = (S.score.copy(), S.seq.copy())
    a, b = runs[("full", (0, 0))], runs[("range", (0, cfg.vocab))]
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_slice_without_trie_is_full():
    cfg = synth.get("c5").shrink(batch=2, beam=6, vocab=200, steps=3)
    out = []
    for mode in ("full", "slice"):
        S = oracle.Search(batch=cfg.batch, beam=cfg.beam, vocab=cfg.vocab, max_steps=cfg.steps,
                          eos=cfg.eos, norm=mode)
        for t in range(cfg.steps):
            x = synth.full_step(cfg, t)
            S.step(lambda b: x[b])
        out.append((S.score.copy(), S.seq.copy()))
    assert np.array_equal(out[0][0], out[1][0]) and np.array_equal(out[0][1], out[1][1])


@pytest.mark.parametrize("norm,rng", [("slice", (0, 0)), ("range", None)])
def test_exhaustive_catalog_with_variant_normalisation(norm, rng):
    """K = catalog size: the search keeps every prefix in brute-force order."""
    cfg = synth.get("c1x")
    trie = synth.make_trie(cfg)
    if rng is None:   # the SID range of levels 0-1 only: level-2 tokens are never emitted
        rng = (cfg.sid_base, cfg.sid_base + 2 * cfg.codebook + 5)
    for b in range(cfg.batch):
        row_of = lambda t, pre: synth.prefix_row(cfg, b, t, list(pre))  # noqa: E731
        hyps = trie_hypotheses(trie.codes, cfg.codebook, cfg.sid_base, cfg.vocab, row_of,
                               norm=norm, norm_range=rng)
        S = oracle.Search(batch=1, beam=cfg.beam, vocab=cfg.vocab, max_steps=cfg.steps, trie=trie,
                          norm=norm, norm_range=rng)
        for t in range(cfg.steps):
            blocks = synth.prefix_block(cfg, b, t, S.prefixes(0))
            S.step(lambda _: blocks)
            h = hyps[t]
            n = min(cfg.beam, len(h))
            for i in range(n):
                assert S.score[0, i] == h[i].score, (norm, t, i)
                assert tuple(S.seq[0, i, :t + 1].tolist()) == h[i].tokens
            assert np.all(S.score[0, n:] == -np.inf)

"""Pins of the oracle's length penalty, minimum length and banned tokens
(beamgrad README, "Features" and "How it works": candidates ranked by
raw / ((5 + length) / 6) ** alpha, minimum length, banned tokens), on the CPU.

Fixed from outside the oracle by: closed forms of the penalty, hand-worked
cases (tests/golden/length_penalty.json) and exhaustive enumeration of tiny
EOS searches (tests/bruteforce.py, independent code).
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth
from bruteforce import free_hypotheses

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "length_penalty.json")
f32 = np.float32


def test_penalty_closed_forms():
    assert oracle.length_penalty(1, 1.0) == 1.0           # (5 + 1) / 6
    assert oracle.length_penalty(7, 1.0) == 2.0           # 12 / 6
    assert oracle.length_penalty(19, 0.5) == 2.0          # sqrt(24 / 6)
    assert oracle.length_penalty(3, 2.0) == f32(64.0 / 36.0)
    for n in (1, 4, 30):
        assert oracle.length_penalty(n, 0.0) == 1.0


def _case(name):
    return next(c for c in json.load(open(GOLDEN))["cases"] if c["name"] == name)


@pytest.mark.parametrize("alpha", ["1.0", "0.0"])
def test_penalty_flips_a_finished_beam(alpha):
    c = _case("penalty_flips_a_finished_beam")
    V, K, T = c["vocab"], c["beam"], c["max_steps"]
    x = np.zeros((K, V), np.float32)
    x[1] = [-np.inf if v is None else v for v in c["logits_row1"]]
    o = oracle.step(x, np.array(c["score"], np.float32), np.full(K, -1, np.int32),
                    np.array(c["finished"], np.uint8), np.array(c["sequences"], np.int32),
                    c["step"], eos=c["eos"], alpha=float(alpha))
    e = c["expect"][alpha]
    assert o.parent.tolist() == e["parents"] and o.token.tolist() == e["tokens"]
    assert o.score.tolist() == [float(f32(s)) for s in e["scores"]]
    if alpha == "1.0":
        ranks = [f32(f32(e["scores"][0]) / f32(8.0 / 6.0)), f32(f32(e["scores"][1]) / f32(7.0 / 6.0))]
        assert np.allclose(ranks, c["approx_rank_alpha1"], atol=1e-6)
        assert ranks[0] > ranks[1]


def test_min_length_and_banned():
    c = _case("min_length_and_banned")
    V, K, T = c["vocab"], c["beam"], c["max_steps"]
    x = np.zeros((K, V), np.float32)
    x[0] = c["logits_row0"]
    st = (np.array([0.0, -np.inf], np.float32), np.full(K, -1, np.int32), np.zeros(K, np.uint8),
          np.full((K, T), -1, np.int32))
    o = oracle.step(x, *st, 0, eos=c["eos"], min_length=c["min_length"], banned=c["banned"])
    assert o.token.tolist() == c["expect_tokens"]
    o = oracle.step(x, *st, 0, eos=c["eos"])
    assert o.token.tolist() == c["expect_tokens_unmasked"]


@pytest.mark.parametrize("V,eos,T,alpha,min_len,banned", [
    (3, 0, 3, 1.0, 0, ()), (4, 0, 3, 0.6, 2, ()), (4, 1, 3, 1.3, 0, (2,)),
    (3, 2, 4, 0.8, 3, ()), (5, 0, 2, 2.0, 2, (3, 4)),
])
def test_free_search_with_penalties_equals_bruteforce(V, eos, T, alpha, min_len, banned):
    cfg = synth.Config("pen", 91 + V + 10 * T, batch=2, beam=1, vocab=V, steps=T, sigma=1.5, eos=eos)
    for b in range(cfg.batch):
        row_of = lambda t, pre: synth.prefix_row(cfg, b, t, [p for p in pre if p >= 0])  # noqa: E731
        steps = free_hypotheses(V, T, eos, row_of, alpha=alpha, min_length=min_len, banned=banned)
        K = max(len(s) for s in steps)
        S = oracle.Search(batch=1, beam=K, vocab=V, max_steps=T, eos=eos, alpha=alpha,
                          min_length=min_len, banned=list(banned))
        for t in range(T):
            pre = S.prefixes(0)
            blk = np.zeros((K, V), np.float32)
            for j, p in enumerate(pre):
                if p is not None:
                    blk[j] = row_of(t, tuple(p))
            S.step(lambda _: blk)
            hyps = steps[t]
            for i, h in enumerate(hyps):
                assert S.score[0, i] == h.score, (t, i)
                assert tuple(S.seq[0, i, :t + 1].tolist()) == h.tokens, (t, i)
                assert bool(S.fin[0, i]) == h.fin
            assert np.all(S.score[0, len(hyps):] == -np.inf)
            toks = S.seq[0][np.isfinite(S.score[0])]
            assert not np.isin(toks, list(banned)).any()
            if min_len > 1:
                assert not np.any(toks[:, :min_len - 1] == eos)


def test_penalties_with_sampling_rank_by_penalised_then_noise():
    """Both at once: rank = fl32(fl32(c / pen) + g); scores stay raw."""
    cfg = synth.get("c5").shrink(batch=2, beam=6, vocab=40, steps=3)
    S = oracle.Search(batch=cfg.batch, beam=cfg.beam, vocab=cfg.vocab, max_steps=cfg.steps,
                      eos=cfg.eos, temperature=0.9, seed=4, alpha=0.7)
    for t in range(cfg.steps):
        x = synth.full_step(cfg, t)
        S.step(lambda b: x[b])
        for b in range(cfg.batch):
            keys = []
            for i in range(cfg.beam):
                if S.score[b, i] == -np.inf:
                    continue
                n = int(np.sum(S.seq[b, i] != -1))
                par, tok = S.parents[-1][b, i], S.tokens[-1][b, i]
                flat = par * cfg.vocab + (tok if tok >= 0 else cfg.eos)
                k = f32(f32(S.score[b, i] / oracle.length_penalty(n, 0.7)) + oracle.gumbel(4, b, t, flat))
                keys.append((float(k), flat))
            assert keys == sorted(keys, key=lambda z: (-z[0], z[1]))

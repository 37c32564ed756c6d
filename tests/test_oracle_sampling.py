"""Pins of the oracle's sampling rule (temperature > 0: Gumbel top-K without
replacement; FlashRec README, "Serving", API item), on the CPU.

What fixes it from outside the oracle:
- the generator: the published known-answer vectors of Philox4x32-10;
- the noise: the standard Gumbel law (mean = Euler-Mascheroni constant,
  variance = pi^2/6, CDF exp(-exp(-x)));
- the selection: Gumbel top-k draws without replacement from the tempered
  softmax (Plackett-Luce: P(a then b) = p_a p_b / (1 - p_a)), checked by
  Monte Carlo over seeds;
- the whole step: an independent numpy enumeration of the candidates ranked
  by c + g, and the invariants (unperturbed scores kept, perturbed keys
  non-increasing, valid trie paths, seed determinism).
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox_kat.json")


def test_philox_known_answers():
    data = json.load(open(GOLDEN))
    for v in data["vectors"]:
        ctr = [int(w, 16) for w in v["ctr"]]
        key = [int(w, 16) for w in v["key"]]
        out = oracle.philox4x32_10(ctr, key)
        assert [f"{int(w):08x}" for w in out] == v["out"]


def test_gumbel_moments_and_cdf():
    g = np.array([oracle.gumbel(12345, 3, 1, f) for f in range(200_000)], np.float64)
    assert abs(g.mean() - 0.5772156649015329) < 0.01
    assert abs(g.var() - math.pi ** 2 / 6) < 0.03
    for x in (-1.0, 0.0, 1.0, 3.0):
        assert abs(np.mean(g <= x) - math.exp(-math.exp(-x))) < 0.005
    # distinct counters draw distinct values; the same counter draws the same one
    assert oracle.gumbel(1, 0, 0, 7) == oracle.gumbel(1, 0, 0, 7)
    assert len({float(oracle.gumbel(1, r, s, 5)) for r in range(4) for s in range(4)}) == 16


def _softmax_t(x, T):
    xt = (np.asarray(x, np.float32) * (np.float32(1.0) / np.float32(T))).astype(np.float64)
    p = np.exp(xt - xt.max())
    return p / p.sum()


@pytest.mark.parametrize("T", [1.0, 2.0])
def test_top2_is_plackett_luce(T):
    """K = 2 slots from one beam over 4 tokens: the ordered pair (first,
    second) follows sampling without replacement from softmax(x / T)."""
    x = np.array([[0.0, 1.0, -0.5, 0.3]] + [[0.0] * 4], np.float32)
    score = np.array([0.0, -np.inf], np.float32)
    node = np.full(2, -1, np.int32)
    fin = np.zeros(2, np.uint8)
    seq = np.full((2, 1), -1, np.int32)
    N = 20_000
    counts = {}
    for seed in range(N):
        o = oracle.step(x, score, node, fin, seq, 0, temperature=T, seed=seed)
        key = (int(o.token[0]), int(o.token[1]))
        counts[key] = counts.get(key, 0) + 1
    p = _softmax_t(x[0], T)
    chi2 = 0.0
    for a in range(4):
        for b in range(4):
            if a == b:
                assert (a, b) not in counts      # without replacement
                continue
            e = N * p[a] * p[b] / (1 - p[a])
            chi2 += (counts.get((a, b), 0) - e) ** 2 / e
    assert chi2 < 45.0, (chi2, counts)          # 11 degrees of freedom


def _enumerate_sampled(x, S, node, fin, seq, t, eos, level, T, seed, b, K):
    """Independent numpy version of one sampled step: every candidate's fp32
    c = S + (fl32(x * fl32(1/T)) - lse), ranked by fl32(c + g) then flat."""
    V = x.shape[1]
    inv_t = np.float32(1.0) / np.float32(T)
    cands = []
    for j in range(len(S)):
        if S[j] == -np.inf:
            continue
        if fin[j]:
            flat = j * V + eos
            cands.append((np.float32(S[j] + oracle.gumbel(seed, b, t, flat)), flat, S[j], j, -1))
            continue
        xt = x[j].astype(np.float32) * inv_t
        if np.max(xt) == -np.inf:
            continue
        lse = np.float32(logsumexp(xt.astype(np.float64)))
        toks = range(V) if level is None else level[1][level[0][node[j]]:level[0][node[j] + 1]]
        for v in toks:
            c = np.float32(S[j] + np.float32(xt[v] - lse))
            if c == -np.inf:
                continue
            flat = j * V + int(v)
            cands.append((np.float32(c + oracle.gumbel(seed, b, t, flat)), flat, c, j, int(v)))
    cands.sort(key=lambda z: (-float(z[0]), z[1]))
    return cands[:K]


@pytest.mark.parametrize("T,seed", [(1.0, 1), (0.5, 2), (3.0, 3)])
def test_sampled_step_equals_enumeration(T, seed):
    cfg = synth.get("c2").shrink(batch=2, beam=12, n_sids=3000, name="samp")
    trie = synth.make_trie(cfg)
    S = oracle.Search(batch=cfg.batch, beam=cfg.beam, vocab=cfg.vocab, max_steps=cfg.steps,
                      trie=trie, temperature=T, seed=seed)
    for t in range(cfg.steps):
        x = synth.full_step(cfg, t)
        before = (S.score.copy(), S.node.copy(), S.fin.copy(), S.seq.copy())
        S.step(lambda b: x[b])
        lvl = (trie.offsets[t], trie.tokens[t], trie.children[t])
        for b in range(cfg.batch):
            ref = _enumerate_sampled(x[b], before[0][b], before[1][b], before[2][b], before[3][b],
                                     t, -1, lvl, T, seed, b, cfg.beam)
            n = len(ref)
            assert [r[3] for r in ref] == S.parents[-1][b][:n].tolist()
            assert [r[4] for r in ref] == S.tokens[-1][b][:n].tolist()
            assert np.array_equal(np.array([r[2] for r in ref], np.float32), S.score[b][:n])
            assert np.all(S.score[b][n:] == -np.inf)


def test_sampling_invariants_and_determinism():
    cfg = synth.get("c5").shrink(batch=3, beam=8, vocab=300, steps=4)
    runs = []
    for seed in (7, 7, 8):
        S = oracle.Search(batch=cfg.batch, beam=cfg.beam, vocab=cfg.vocab, max_steps=cfg.steps,
                          eos=cfg.eos, temperature=0.8, seed=seed)
        for t in range(cfg.steps):
            x = synth.full_step(cfg, t)
            prev = S.score.copy()
            S.step(lambda b: x[b])
            for b in range(cfg.batch):
                par, tok = S.parents[-1][b], S.tokens[-1][b]
                keys = []
                for i in range(cfg.beam):
                    if S.score[b, i] == -np.inf:
                        continue
                    flat = par[i] * cfg.vocab + (tok[i] if tok[i] >= 0 else cfg.eos)
                    keys.append((float(np.float32(S.score[b, i] + oracle.gumbel(seed, b, t, flat))), flat))
                    # scores stay cumulative log-probabilities: never above the parent's
                    assert S.score[b, i] <= prev[b, par[i]]
                assert keys == sorted(keys, key=lambda z: (-z[0], z[1]))
        runs.append(S.seq.copy())
    assert np.array_equal(runs[0], runs[1])
    assert not np.array_equal(runs[0], runs[2])


def test_temperature_zero_is_the_deterministic_step():
    cfg = synth.get("c5").shrink(batch=2, beam=6, vocab=200, steps=2)
    x = synth.full_step(cfg, 0)
    K, T = cfg.beam, cfg.steps
    score = np.full(K, -np.inf, np.float32)
    score[0] = 0
    args = (x[0], score, np.full(K, -1, np.int32), np.zeros(K, np.uint8), np.full((K, T), -1, np.int32), 0)
    a = oracle.step(*args, eos=cfg.eos)
    b = oracle.step(*args, eos=cfg.eos, temperature=0.0, seed=99)
    assert np.array_equal(a.score, b.score) and np.array_equal(a.token, b.token)
    with pytest.raises(RuntimeError):
        oracle.step(*args, eos=cfg.eos, temperature=-1.0)

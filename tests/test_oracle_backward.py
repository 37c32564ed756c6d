"""Pins of the oracle's surrogate backward (beamgrad README, "How it works":
with the selection held fixed, d score_k / d log_probs[t, p, v] is
1 / penalty(length_k) on k's path and 0 elsewhere) and of the NONE
normaliser it is checked with.

The finite-difference checks run the oracle's own forward search again on
perturbed inputs, so they do not share the backward's backtracking.  Values
lie on a 2^-10 grid and the perturbation is 2^-12, so every fp32 sum of the
forward search is exact and the difference quotients are exact."""
import numpy as np
import pytest

import oracle

EPS = 2.0 ** -12


def grid_logprobs(rng, T, K, V):
    return (-rng.integers(1, 4096, size=(T, K, V)) * 2.0 ** -10).astype(np.float32)


def run(x, eos=-1, alpha=0.0, norm="none", trie=None, min_length=0):
    T, K, V = x.shape
    s = oracle.Search(1, K, V, T, eos=eos, alpha=alpha, norm=norm, trie=trie, min_length=min_length)
    for _ in range(T):
        s.step(lambda b: x[s.t])
    return s


def history(s):
    return np.stack([p[0] for p in s.parents]), np.stack([t[0] for t in s.tokens])


def grads_of_beam(s, k, alpha):
    """Per-step log-prob gradient [T, K, V] of final beam k's ranked score."""
    par, tok = history(s)
    K = s.beam
    g = np.zeros(K, np.float32)
    g[k] = 1.0
    ps, pt, w = oracle.backward(par, tok, s.score[0], s.seq[0], g, alpha)
    out = np.zeros((s.max_steps, K, s.vocab), np.float32)
    for t in range(s.t):
        oracle.backward_scatter(ps[t], pt[t], w, out[t])
    return out, ps, pt, w


@pytest.mark.parametrize("seed,eos", [(1, -1), (2, 0), (3, 3)])
def test_finite_differences_exact(seed, eos):
    rng = np.random.default_rng(seed)
    T, K, V = 4, 5, 9
    x = grid_logprobs(rng, T, K, V)
    base = run(x, eos=eos)
    par0, tok0 = history(base)
    checked = on_path = 0
    for t in range(T):
        for p in range(K):
            for v in range(V):
                xp = x.copy()
                xp[t, p, v] += EPS
                pert = run(xp, eos=eos)
                par1, tok1 = history(pert)
                if not (np.array_equal(par0, par1) and np.array_equal(tok0, tok1)):
                    continue  # the selection changed: the surrogate does not apply
                fd = (pert.score[0].astype(np.float64) - base.score[0]) / EPS
                for k in range(K):
                    if base.score[0, k] == -np.inf:
                        continue
                    g, _, _, _ = grads_of_beam(base, k, 0.0)
                    assert fd[k] == g[t, p, v], (t, p, v, k, fd[k], g[t, p, v])
                    checked += 1
                    on_path += g[t, p, v] != 0
    assert checked > 500 and on_path >= 10, (checked, on_path)


def test_finite_differences_length_penalty():
    """alpha != 0: the ranked score raw / pen(len) moves by eps / pen(len_k)
    on k's path; beams that ended with EOS early are carried (len < T)."""
    rng = np.random.default_rng(7)
    T, K, V = 5, 6, 8
    x = grid_logprobs(rng, T, K, V)
    x[:, :, 0] += np.float32(1.5)  # EOS (token 0) likely early
    alpha = 0.7
    base = run(x, eos=0, alpha=alpha)
    par0, tok0 = history(base)
    lens = (base.seq[0] != -1).sum(axis=1)
    assert len(set(lens[np.isfinite(base.score[0])].tolist())) > 1  # mixed lengths
    checked = 0
    for (t, p, v) in [(t, p, v) for t in range(T) for p in range(K) for v in range(V)][::3]:
        xp = x.copy()
        xp[t, p, v] += EPS
        pert = run(xp, eos=0, alpha=alpha)
        par1, tok1 = history(pert)
        if not (np.array_equal(par0, par1) and np.array_equal(tok0, tok1)):
            continue
        for k in range(K):
            if base.score[0, k] == -np.inf:
                continue
            pen = np.float64(oracle.length_penalty(int(lens[k]), alpha))
            fd = (np.float64(pert.score[0, k]) - np.float64(base.score[0, k])) / EPS / pen
            g, _, _, _ = grads_of_beam(base, k, alpha)
            assert abs(fd - g[t, p, v]) <= 1e-6 * max(1.0, abs(fd)), (t, p, v, k, fd, g[t, p, v])
            checked += 1
    assert checked > 100


def test_path_reproduces_scores_and_sequences():
    """With the full-row normaliser: each final score is the fp32
    accumulation of (x - lse) along its path (carried steps add nothing),
    and the path's tokens are the final sequence."""
    rng = np.random.default_rng(11)
    T, K, V = 4, 7, 10
    x = rng.normal(0, 2, size=(T, K, V)).astype(np.float32)
    s = run(x, eos=2, norm="full")
    par, tok = history(s)
    ps, pt, w = oracle.backward(par, tok, s.score[0], s.seq[0], np.ones(K, np.float32), 0.0)
    for k in range(K):
        if s.score[0, k] == -np.inf:
            assert np.all(ps[:, k] == -1) and np.all(pt[:, k] == -1) and w[k] == 0
            continue
        acc = np.float32(0.0)
        toks = []
        for t in range(T):
            p, v = ps[t, k], pt[t, k]
            assert 0 <= p < K
            if v < 0:
                continue
            lse = s.lses[t][0, p]
            acc = np.float32(acc + np.float32(x[t, p, v] - lse))
            toks.append(int(v))
        assert acc == s.score[0, k], k
        assert toks == [int(v) for v in s.seq[0, k] if v != -1]
        assert w[k] == 1.0


def test_scatter_sums_and_shared_prefixes():
    rng = np.random.default_rng(5)
    T, K, V = 4, 8, 6
    x = grid_logprobs(rng, T, K, V)
    s = run(x, eos=1)
    par, tok = history(s)
    gfin = rng.integers(-3, 4, size=K).astype(np.float32)  # small integers: every sum exact
    ps, pt, w = oracle.backward(par, tok, s.score[0], s.seq[0], gfin, 0.0)
    for t in range(T):
        g = oracle.backward_scatter(ps[t], pt[t], w, np.zeros((K, V), np.float32))
        on = pt[t] >= 0
        assert g.sum() == w[on].sum()
        ref = np.zeros((K, V), np.float64)
        np.add.at(ref, (ps[t][on], pt[t][on]), w[on].astype(np.float64))
        assert np.array_equal(g.astype(np.float64), ref)
        # two beams through one (p, v) at step t share the whole path before it
        for a in range(K):
            for b in range(a + 1, K):
                if on[a] and on[b] and (ps[t, a], pt[t, a]) == (ps[t, b], pt[t, b]):
                    assert np.array_equal(ps[:t, a], ps[:t, b]) and np.array_equal(pt[:t, a], pt[:t, b])
        # adds to what the buffer holds
        pre = np.full((K, V), 0.5, np.float32)
        oracle.backward_scatter(ps[t], pt[t], w, pre)
        assert np.array_equal(pre, np.float32(0.5) + g)


def test_none_normaliser_is_identity():
    """NONE: lse = 0 and c = S + x exactly."""
    rng = np.random.default_rng(3)
    K, V, T = 4, 7, 2
    x = grid_logprobs(rng, 1, K, V)[0]
    score = np.full(K, -np.inf, np.float32)
    score[0] = 0
    o = oracle.step(x, score, np.full(K, -1, np.int32), np.zeros(K, np.uint8),
                    np.full((K, T), -1, np.int32), 0, norm="none")
    assert o.lse[0] == 0 and np.isnan(o.lse[1:]).all()
    best = np.sort(x[0])[::-1][:K]
    assert np.array_equal(o.score, best)


def test_backward_rejects_broken_history():
    K, T = 3, 2
    par = np.array([[0, -1, -1], [-1, 0, 0]], np.int32)  # slot 0 of step 1 points at -1
    tok = np.array([[4, -1, -1], [5, 6, 7]], np.int32)
    sc = np.array([-1.0, -2.0, -3.0], np.float32)
    seq = np.full((K, T), -1, np.int32)
    with pytest.raises(RuntimeError):
        oracle.backward(par, tok, sc, seq, np.ones(K, np.float32))

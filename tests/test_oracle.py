"""Pins of the oracle against things other than itself.

* hand-worked closed-form cases (tests/golden/worked_examples.json);
* brute-force enumeration of every hypothesis (tests/bruteforce.py): with a
  beam at least as wide as the number of live hypotheses, beam search must
  return all of them in order -- on the exhaustive tiny-SID workload (K =
  2,000 = catalog size), on random tiny tries, and on unconstrained / EOS
  searches over tiny vocabularies;
* K = 1 equals textbook greedy decoding;
* step 0 equals numpy.lexsort of the root's children;
* the row normaliser equals scipy.special.logsumexp rounded to fp32;
* constant logits give the K lowest flat indices with score -log V;
* invariants: emitted SIDs lie in the catalog, scores never increase along a
  beam, slots are best first, #finite slots = min(K, #candidates);
* shift invariance, permutation covariance, a forced EOS is frozen bitwise.
"""
import json
import math
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import synth
from bruteforce import free_hypotheses, greedy_path, lse32, trie_hypotheses
from synth.catalog import csr_from_codes

f32 = np.float32
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


# ---------------------------------------------------------------- helpers

def prefix_search(cfg, trie, K, steps, snap=True, max_steps=None):
    """Oracle search over prefix-keyed logits; returns per-step snapshots."""
    S = oracle.Search(batch=cfg.batch, beam=K, vocab=cfg.vocab, max_steps=max_steps or steps,
                      eos=cfg.eos, trie=trie)
    snaps = []
    for t in range(steps):
        blocks = {b: synth.prefix_block(cfg, b, t, S.prefixes(b)) for b in range(cfg.batch)}
        S.step(lambda b: blocks[b])
        if snap:
            snaps.append(dict(score=S.score.copy(), seq=S.seq.copy(), node=S.node.copy(),
                              fin=S.fin.copy(), parent=S.parents[-1].copy(),
                              token=S.tokens[-1].copy()))
    return S, snaps


def as_f32_row(cfg, row):
    row = np.asarray(row)
    return synth.bf16_bits_to_f32(row) if row.dtype == np.uint16 else row.astype(np.float32)


def compare_to_hyps(snap_b, hyps, t, K):
    """Slots 0.. of one request after step t equal the ordered hypotheses."""
    n = min(K, len(hyps))
    for i in range(n):
        h = hyps[i]
        assert snap_b["score"][i] == h.score, (t, i, snap_b["score"][i], h.score)
        assert tuple(snap_b["seq"][i][:t + 1].tolist()) == tuple(h.tokens), (t, i)
    assert np.all(snap_b["score"][n:] == -np.inf)
    assert np.all(snap_b["seq"][n:] == -1)


# ---------------------------------------------------------------- golden

def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_worked_examples(case):
    V, K, T, eos = case["vocab"], case["beam"], case["steps"], case["eos"]
    trie = None
    if "catalog" in case:
        codes = np.array(case["catalog"], np.uint8)
        trie = csr_from_codes(codes, case["codebook"], case["sid_base"], V)
    S = oracle.Search(batch=1, beam=K, vocab=V, max_steps=T, eos=eos, trie=trie)
    for t in range(T):
        x = np.array(case["logits"][t], np.float32)
        S.step(lambda b: x)
        exp = case["expect"][t]
        assert S.tokens[-1][0].tolist() == exp["tokens"], t
        assert S.parents[-1][0].tolist() == exp["parents"], t
        if "fin" in exp:
            assert S.fin[0].tolist() == exp["fin"], t
        if "nodes" in exp:
            assert S.node[0].tolist() == exp["nodes"], t
    assert S.seq[0].tolist() == case["sequences"]
    assert np.allclose(S.score[0], case["approx_final_scores"], atol=2e-6)
    # exact fp32 closed forms
    L = lambda v: f32(v)  # noqa: E731
    if case["name"] == "constant_unconstrained":
        s0 = f32(0) + (f32(0) - L(math.log(5)))
        s1 = s0 + (f32(0) - L(math.log(5)))
        assert np.all(S.score[0] == s1)
    elif case["name"] == "eos_carry":
        lse0 = L(5 + math.log(1 + 2 * math.exp(-5)))
        assert S.score[0][0] == f32(0) + (f32(5) - lse0)
        assert S.score[0][1] == (f32(0) + (f32(0) - lse0)) + (f32(0) - L(math.log(3)))
    else:
        lse0 = L(9 + math.log(4 + math.exp(-8) + math.exp(-9)))
        la = L(7 + math.log(1 + 3 * math.exp(-7) + math.exp(-6) + math.exp(-5)))
        lb = L(3 + math.log(1 + 5 * math.exp(-3)))
        assert S.score[0][0] == (f32(0) + (f32(0) - lse0)) + (f32(3) - lb)
        assert S.score[0][1] == (f32(0) + (f32(1) - lse0)) + (f32(2) - la)


# ---------------------------------------------------------------- brute force

def test_c1x_exhaustive_equals_bruteforce():
    """K = 2,000 >= every level's number of valid prefixes (16, 256, 2,000):
    beam search must return the whole catalog in brute-force order."""
    cfg = synth.get("c1x")
    trie = synth.make_trie(cfg)
    nn = trie.num_nodes
    assert cfg.beam >= max(nn[1:])
    S, snaps = prefix_search(cfg, trie, cfg.beam, cfg.steps)
    row_index = {tuple(r): i for i, r in enumerate(trie.codes.tolist())}
    for b in range(cfg.batch):
        steps = trie_hypotheses(trie.codes, cfg.codebook, cfg.sid_base, cfg.vocab,
                                lambda t, pre: as_f32_row(cfg, synth.prefix_row(cfg, b, t, pre)))
        for t in range(cfg.steps):
            assert len(steps[t]) == nn[t + 1]
            compare_to_hyps({k: v[b] for k, v in snaps[t].items()}, steps[t], t, cfg.beam)
        # final nodes are leaf ids = rows of the sorted catalog
        for i, h in enumerate(steps[-1]):
            codes = tuple(int(v) - L * cfg.codebook for L, v in enumerate(h.tokens))
            assert S.node[b, i] == row_index[codes]
    # every SID of the catalog appears exactly once per request
    for b in range(cfg.batch):
        assert sorted(S.node[b].tolist()) == list(range(cfg.n_sids))


@st.composite
def tiny_trie(draw):
    D = draw(st.integers(1, 3))
    cb = draw(st.integers(2, 4))
    space = cb ** D
    n = draw(st.integers(1, space))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    rng = np.random.default_rng(seed)
    keys = np.sort(rng.choice(space, size=n, replace=False))
    codes = np.zeros((n, D), np.uint8)
    k = keys.copy()
    for L in range(D - 1, -1, -1):
        codes[:, L] = k % cb
        k //= cb
    extra = draw(st.integers(0, 3))  # non-SID ids before the SID range
    return codes, cb, extra, seed


@settings(max_examples=40, deadline=None)
@given(tiny_trie(), st.sampled_from([0.5, 2.0, 6.0]), st.booleans())
def test_random_tiny_trie_equals_bruteforce(tt, sigma, bf16):
    codes, cb, base, seed = tt
    D = codes.shape[1]
    V = base + D * cb + draw_tail(seed)
    cfg = synth.Config("tiny", 900 + seed % 1000, batch=2, beam=len(codes) + 1, vocab=V,
                       steps=D, dtype="bf16" if bf16 else "f32", depth=D, codebook=cb,
                       sid_base=base, n_sids=len(codes), sigma=sigma)
    trie = csr_from_codes(codes, cb, base, V)
    S, snaps = prefix_search(cfg, trie, cfg.beam, D)
    for b in range(cfg.batch):
        steps = trie_hypotheses(codes, cb, base, V,
                                lambda t, pre: as_f32_row(cfg, synth.prefix_row(cfg, b, t, pre)))
        for t in range(D):
            compare_to_hyps({k: v[b] for k, v in snaps[t].items()}, steps[t], t, cfg.beam)


def draw_tail(seed):
    return seed % 3


@pytest.mark.parametrize("V,eos,T", [(4, 0, 3), (4, -1, 3), (3, 2, 4), (5, 1, 2)])
def test_free_search_equals_bruteforce(V, eos, T):
    cfg = synth.Config("free", 77 + V + 10 * T, batch=2, beam=1, vocab=V, steps=T,
                       sigma=1.5, eos=eos)
    for b in range(cfg.batch):
        row_of = lambda t, pre: synth.prefix_row(cfg, b, t, [p for p in pre if p >= 0])  # noqa: E731
        steps = free_hypotheses(V, T, eos, row_of)
        K = max(len(s) for s in steps)
        if eos == 0 and V == 4 and T == 3:
            assert [len(s) for s in steps] == [4, 13, 40]
        S = oracle.Search(batch=1, beam=K, vocab=V, max_steps=T, eos=eos)
        for t in range(T):
            pre = S.prefixes(0)
            blk = np.zeros((K, V), np.float32)
            for j, p in enumerate(pre):
                if p is not None:
                    blk[j] = row_of(t, tuple(p))
            S.step(lambda _: blk)
            hyps = steps[t]
            for i, h in enumerate(hyps):
                assert S.score[0, i] == h.score
                assert tuple(S.seq[0, i, :t + 1].tolist()) == h.tokens
                assert bool(S.fin[0, i]) == h.fin
            assert np.all(S.score[0, len(hyps):] == -np.inf)


def test_greedy_is_k1():
    cfg = synth.get("c1")
    trie = synth.make_trie(cfg)
    S, _ = prefix_search(cfg, trie, 1, cfg.steps, snap=False)
    toks = synth.sid_tokens(trie, trie.codes)

    def children_of(t, pre):
        m = np.all(toks[:, :t] == np.array(pre, np.int64)[None, :], axis=1) if t else \
            np.ones(len(toks), bool)
        return sorted(set(toks[m, t].tolist()))

    for b in range(cfg.batch):
        path, score = greedy_path(cfg.depth, children_of,
                                  lambda t, pre: synth.prefix_row(cfg, b, t, pre))
        assert tuple(S.seq[b, 0].tolist()) == path
        assert S.score[b, 0] == score


@pytest.mark.parametrize("name", ["c1", "c2"])
def test_step0_is_lexsort_of_root_children(name):
    cfg = synth.get(name)
    trie = synth.make_trie(cfg)
    x = synth.step_logits(cfg, 0, 0)
    o = oracle.step(x, [0.0] + [-np.inf] * (cfg.beam - 1), [0] + [-1] * (cfg.beam - 1),
                    np.zeros(cfg.beam, np.uint8), np.full((cfg.beam, cfg.steps), -1, np.int32),
                    0, level=(trie.offsets[0], trie.tokens[0], trie.children[0]))
    l = lse32(x[0])
    v = trie.tokens[0]
    score = f32(0) + (x[0, v] - l)
    order = np.lexsort((v, -score.astype(np.float64)))[:cfg.beam]
    n = len(order)
    assert o.token[:n].tolist() == v[order].tolist()
    assert np.array_equal(o.score[:n], score[order])
    assert o.node[:n].tolist() == trie.children[0][order].tolist()
    assert o.n_candidates == len(v)


# ---------------------------------------------------------------- closed forms

def test_constant_logits_pick_lowest_flat():
    """All-zero logits on the tiny SID trie: step 0 picks the root's 8
    smallest child tokens in increasing order, each with score -log 48."""
    cfg = synth.get("c1")
    trie = synth.make_trie(cfg)
    K = cfg.beam
    S = oracle.Search(batch=1, beam=K, vocab=cfg.vocab, max_steps=cfg.steps, trie=trie)
    zeros = np.zeros((K, cfg.vocab), np.float32)
    S.step(lambda b: zeros)
    node0 = S.node[0].copy()
    assert S.tokens[0][0].tolist() == sorted(trie.tokens[0].tolist())[:K]
    assert np.all(S.score[0] == f32(0) + (f32(0) - f32(math.log(48))))
    S.step(lambda b: zeros)
    # ties everywhere: the K lowest flat = parent slot * V + token win
    V = cfg.vocab
    flats = []
    lvl = 1
    off, tok = trie.offsets[lvl], trie.tokens[lvl]
    prev_nodes = np.array(node0)
    for j, n in enumerate(prev_nodes):
        flats += [j * V + int(v) for v in tok[off[n]:off[n + 1]]]
    want = sorted(flats)[:K]
    assert S.parents[1][0].tolist() == [f // V for f in want]
    assert S.tokens[1][0].tolist() == [f % V for f in want]


def test_row_lse_matches_scipy():
    from scipy.special import logsumexp
    rng = np.random.default_rng(5)
    for i in range(300):
        V = int(rng.integers(1, 3000))
        x = (rng.standard_normal(V) * rng.choice([0.1, 1, 5, 40]) +
             rng.choice([0, 100, -1e4])).astype(np.float32)
        if i % 7 == 0 and V > 2:
            x[rng.choice(V, V // 2, replace=False)] = -np.inf
        ref = logsumexp(x.astype(np.float64))
        assert oracle.row_lse(x) == f32(ref), i
        assert abs(float(oracle.row_lse(x)) - ref) <= 1e-6 * max(1.0, abs(ref))
    assert oracle.row_lse(np.full(5, -np.inf, np.float32)) == -np.inf
    # a single finite element anywhere: the normaliser is that element
    for V in (1, 2, 7):
        for pos in range(V):
            x = np.full(V, -np.inf, np.float32)
            x[pos] = 3.25
            assert oracle.row_lse(x) == f32(3.25)
    # a huge maximum at either end must not overflow the sum
    for pos in (0, -1):
        x = np.zeros(9, np.float32)
        x[pos] = 1000.0
        assert oracle.row_lse(x) == f32(1000.0 + math.log1p(8 * math.exp(-1000.0)))
        assert oracle.row_lse(-x) == f32(math.log(8 + math.exp(-1000.0)))
    # bf16 path equals the widened fp32 path
    x = synth.to_bf16_bits(rng.standard_normal(4097).astype(np.float32) * 3)
    assert oracle.row_lse(x) == oracle.row_lse(synth.bf16_bits_to_f32(x))


def test_node_ids_are_followed_not_assumed():
    """Relabelling every level's node ids changes nothing but the node
    outputs, which follow the relabelling."""
    cfg = synth.get("c1")
    trie = synth.make_trie(cfg)
    tr2, perms = synth.relabel(trie, 11)
    A = oracle.Search(batch=cfg.batch, beam=cfg.beam, vocab=cfg.vocab, max_steps=3, trie=trie)
    Bq = oracle.Search(batch=cfg.batch, beam=cfg.beam, vocab=cfg.vocab, max_steps=3, trie=tr2)
    for t in range(3):
        A.step(lambda b: synth.step_logits(cfg, t, b))
        Bq.step(lambda b: synth.step_logits(cfg, t, b))
        assert np.array_equal(A.score, Bq.score) and np.array_equal(A.seq, Bq.seq)
        m = A.node >= 0
        assert np.array_equal(perms[t + 1][A.node[m]], Bq.node[m])


def test_bf16_step_equals_widened_step():
    cfg = synth.get("c3").shrink(beam=4, batch=1)
    trie = synth.make_trie(synth.get("c1"))  # any trie; use c1 tokens shifted below
    x = synth.step_logits(cfg, 1, 0)
    K = cfg.beam
    args = ([0.0, -1.0, -2.0, -np.inf], [0, 0, 0, -1], np.zeros(K, np.uint8),
            np.full((K, 3), -1, np.int32), 0)
    lvl = (trie.offsets[0], trie.tokens[0] + cfg.sid_base, trie.children[0])
    a = oracle.step(x, *args, level=lvl)
    b = oracle.step(synth.bf16_bits_to_f32(x), *args, level=lvl)
    for k in ("score", "node", "token", "parent", "seq"):
        assert np.array_equal(getattr(a, k), getattr(b, k))
    assert np.array_equal(a.lse, b.lse, equal_nan=True)


# ---------------------------------------------------------------- invariants

def _check_invariants(cfg, trie, S):
    B, K = S.score.shape
    for t in range(S.t):
        par, tok = S.parents[t], S.tokens[t]
        for b in range(B):
            n_fin = int(np.sum(np.isfinite(S.score[b]))) if t == S.t - 1 else None
            if n_fin is not None:
                assert n_fin == min(K, int(S.n_candidates[t][b]))
    for b in range(B):
        sc = S.score[b]
        finite = sc[np.isfinite(sc)]
        assert np.all(np.diff(finite) <= 0), "best first"
        seqs = [tuple(s) for s, f in zip(S.seq[b].tolist(), np.isfinite(sc)) if f]
        assert len(set(seqs)) == len(seqs), "no duplicate prefixes"
        if trie is not None:
            cat = set(map(tuple, synth.sid_tokens(trie, trie.codes)[:, :S.t].tolist()))
            for s in seqs:
                assert s in cat, "every emitted SID prefix is in the catalog"


def _parent_scores_never_increase(S_hist):
    for prev, cur, par in S_hist:
        m = par >= 0
        assert np.all(cur[m] <= prev[np.where(m, par, 0)][m])


@pytest.mark.parametrize("name,shrink", [
    ("c1", {}),
    ("c2", dict(batch=3, n_sids=30000)),
    ("c4", dict(batch=2, beam=64, n_sids=100000, root_fanout=8, mean_fanout=12)),
    ("c5", dict(batch=2, beam=8, vocab=300, steps=6)),
])
def test_invariants_iid(name, shrink):
    cfg = synth.get(name)
    if shrink:
        cfg = cfg.shrink(**shrink)
    trie = synth.make_trie(cfg) if cfg.constrained else None
    S = oracle.Search(batch=cfg.batch, beam=cfg.beam, vocab=cfg.vocab, max_steps=cfg.steps,
                      eos=cfg.eos, trie=trie)
    hist = []
    for t in range(cfg.steps):
        prev = S.score.copy()
        S.step(lambda b: synth.step_logits(cfg, t, b))
        hist.append((prev, S.score.copy(), S.parents[-1]))
    _check_invariants(cfg, trie, S)
    for prev, cur, par in hist:
        for b in range(cfg.batch):
            m = par[b] >= 0
            assert np.all(cur[b][m] <= prev[b][par[b][m]])


def test_shift_invariance():
    cfg = synth.get("c2").shrink(batch=1, n_sids=20000)
    trie = synth.make_trie(cfg)
    rng = np.random.default_rng(3)
    A = oracle.Search(batch=1, beam=cfg.beam, vocab=cfg.vocab, max_steps=3, trie=trie)
    Bs = oracle.Search(batch=1, beam=cfg.beam, vocab=cfg.vocab, max_steps=3, trie=trie)
    for t in range(3):
        x = synth.step_logits(cfg, t, 0)
        shift = rng.uniform(-20, 20, size=(cfg.beam, 1)).astype(np.float32)
        A.step(lambda b: x)
        Bs.step(lambda b: (x + shift).astype(np.float32))
        assert np.max(np.abs(A.score - Bs.score)[np.isfinite(A.score)]) < 2e-5
        same = A.seq[0, :, :t + 1] == Bs.seq[0, :, :t + 1]
        assert same.all(axis=1).mean() > 0.97  # only near-ties may swap
        Bs.score, Bs.seq, Bs.node, Bs.fin = A.score.copy(), A.seq.copy(), A.node.copy(), A.fin.copy()


def test_permutation_covariance():
    cfg = synth.get("c2").shrink(batch=1, beam=64, n_sids=20000)
    trie = synth.make_trie(cfg)
    S, _ = prefix_search(cfg, trie, cfg.beam, 1, snap=False, max_steps=3)
    state = (S.score[0].copy(), S.node[0].copy(), S.fin[0].copy(), S.seq[0].copy())
    x = synth.prefix_block(cfg, 0, 1, S.prefixes(0))
    lvl = (trie.offsets[1], trie.tokens[1], trie.children[1])
    a = oracle.step(x, *state, 1, level=lvl)
    perm = np.random.default_rng(0).permutation(cfg.beam)
    b = oracle.step(x[perm], state[0][perm], state[1][perm], state[2][perm], state[3][perm], 1,
                    level=lvl)
    key = lambda o: sorted((float(s), tuple(q)) for s, q in zip(o.score, o.seq.tolist())  # noqa
                           if np.isfinite(s))
    assert key(a) == key(b)


def test_forced_eos_frozen_bitwise():
    cfg = synth.get("c5").shrink(batch=2, beam=4, vocab=64, steps=6)
    S = oracle.Search(batch=cfg.batch, beam=cfg.beam, vocab=cfg.vocab, max_steps=cfg.steps,
                      eos=cfg.eos)
    first = None
    for t in range(cfg.steps):
        def blk(b, t=t):
            x = synth.step_logits(cfg, t, b)
            if t == 0:
                x[:, cfg.eos] += 50
            return x
        S.step(blk)
        if t == 0:
            first = S.score[:, 0].copy()
            assert np.all(S.fin[:, 0] == 1) and np.all(S.seq[:, 0, 0] == cfg.eos)
            assert np.all(first <= 0) and np.all(first > -1e-6)
        else:
            assert np.all(S.score[:, 0].view(np.uint32) == first.view(np.uint32))
            assert np.all(S.tokens[-1][:, 0] == -1) and np.all(S.parents[-1][:, 0] == 0)
    assert np.all(S.seq[:, 0, 1:] == -1)


def test_error_codes():
    x = np.zeros((2, 4), np.float32)
    with pytest.raises(RuntimeError, match="-3"):  # step past max_steps
        oracle.step(x, [0, -np.inf], [-1, -1], [0, 0], np.full((2, 1), -1, np.int32), 1)
    with pytest.raises(RuntimeError, match="-3"):  # finished slot without EOS
        oracle.step(x, [0, -np.inf], [-1, -1], [1, 0], np.full((2, 2), -1, np.int32), 0)

"""Helpers of the GPU parity tests: drive the HIP library and the oracle on
the same seeded inputs and compare their steps.

The comparison follows the correctness bar of the method's benchmark:
selected (parent, token) pairs, backpointers, nodes and flags bit-exact, with
one exception -- candidates whose oracle ranking score (the score, or the
score plus its Gumbel draw when sampling) lies within 1e-5 of the K-th
(boundary) one, or of the one they are swapped with, may differ; scores
agree within 1e-4 absolute (fp32).
"""
from __future__ import annotations

import numpy as np

import oracle

TIE = 1e-5
SCORE_TOL = 1e-4


def torch_mod():
    import torch
    return torch


def to_dev(x: np.ndarray):
    torch = torch_mod()
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).cuda()
    return torch.from_numpy(x.astype(np.float32, copy=False)).cuda()


def state_np(beam) -> dict:
    torch = torch_mod()
    st = beam.state()
    torch.cuda.synchronize()
    return {k: (v.cpu().numpy() if hasattr(v, "cpu") else v) for k, v in st.items()}


def set_state_from(beam, step: int, score, node, fin, seq):
    torch = torch_mod()
    beam.set_state(step, torch.from_numpy(np.ascontiguousarray(score, np.float32)).cuda(),
                   torch.from_numpy(np.ascontiguousarray(node, np.int32)).cuda(),
                   torch.from_numpy(np.ascontiguousarray(fin, np.uint8)).cuda(),
                   torch.from_numpy(np.ascontiguousarray(seq, np.int32)).cuda())


def as_f32(x: np.ndarray) -> np.ndarray:
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32)
    return x.astype(np.float32, copy=False)


class Report:
    def __init__(self):
        self.slots = 0
        self.mismatched_slots = 0
        self.excused = 0
        self.rows = 0
        self.lse_equal = 0
        self.max_lse_err = 0.0
        self.max_score_err = 0.0
        self.validated = 0

    def __repr__(self):
        return (f"slots={self.slots} mismatched={self.mismatched_slots} excused={self.excused} "
                f"validated={self.validated} "
                f"rows={self.rows} lse_bit_equal={self.lse_equal} "
                f"max_lse_err={self.max_lse_err:.3g} max_score_err={self.max_score_err:.3g}")


def check_valid_slot(g: dict, b: int, t: int, i: int, pre: dict, V: int, eos: int, where: str,
                     level=None, min_length: int = 0, banned=None, norm_range=None):
    """Slot i of the GPU's request b after step t holds a real candidate of
    its parent slot j: a finished parent is carried (token -1, node -1,
    finished); a live parent's token is a child of its trie node, with that
    edge's child id as the next node (a token of [0, V) without a trie, the
    finished flag set exactly for EOS); the token is not masked; and the
    sequence is the parent's extended by the token."""
    j, tok = int(g["parents"][t][b][i]), int(g["tokens"][t][b][i])
    node, fin, seq = int(g["nodes"][b][i]), int(g["finished"][b][i]), g["sequences"][b][i]
    K = len(pre["score"])
    assert 0 <= j < K and np.isfinite(pre["score"][j]), f"{where}: slot {i} parent {j} is empty"
    if "fin" in pre and pre["fin"][j]:
        assert (tok, node, fin) == (-1, -1, 1), f"{where}: slot {i} carries {j} as {(tok, node, fin)}"
    else:
        assert tok >= 0, f"{where}: slot {i}: a live parent {j} carried"
        if level is not None:
            off, toks, ch = level
            n = int(pre["node"][j])
            a, e_end = int(off[n]), int(off[n + 1])
            e = a + int(np.searchsorted(toks[a:e_end], tok))
            assert e < e_end and toks[e] == tok, f"{where}: slot {i}: token {tok} is no child of node {n}"
            assert node == int(ch[e]), f"{where}: slot {i}: node {node}, the edge's child is {int(ch[e])}"
            assert fin == 0, where
        else:
            assert 0 <= tok < V and node == -1 and fin == int(tok == eos), f"{where}: slot {i}"
        assert banned is None or tok not in set(int(v) for v in banned), f"{where}: banned {tok}"
        assert not (tok == eos and t + 1 < min_length), f"{where}: EOS under the minimum length"
        if norm_range is not None:
            assert norm_range[0] <= tok < norm_range[1], f"{where}: token {tok} outside the range"
    if "seq" in pre:
        want = pre["seq"][j].copy()
        want[t] = tok
        want[t + 1:] = -1
        assert np.array_equal(seq, want), f"{where}: slot {i}: sequence {seq} != {want}"


def compare_request(O, g: dict, b: int, t: int, pre: dict, x: np.ndarray, V: int, eos: int,
                    rep: Report, ctx: str = "", temperature: float = 0.0, seed: int = 0,
                    alpha: float = 0.0, level=None, min_length: int = 0, banned=None,
                    norm_range=None):
    """O: oracle.StepOut of request b; g: GPU state after the step (numpy,
    all requests); pre: the pre-step state of request b (score, node, fin,
    seq); x: [K, V] logits; temperature > 0: both sides sampled with the same
    seed; alpha: the length penalty both sides rank by; level, min_length,
    banned, norm_range: what makes a candidate valid (see check_valid_slot),
    checked for every GPU slot the oracle does not hold in the same place."""
    K = len(O.score)
    gs, gn, gf = g["scores"][b], g["nodes"][b], g["finished"][b]
    gp, gt, gq = g["parents"][t][b], g["tokens"][t][b], g["sequences"][b]
    where = f"{ctx} step {t} request {b}"
    # the row normaliser of every row read
    read = ~np.isnan(O.lse)
    assert np.array_equal(read, ~np.isnan(g["lse"][b])), where + ": rows read differ"
    if read.any():
        ol, gl = O.lse[read].astype(np.float64), g["lse"][b][read].astype(np.float64)
        err = np.abs(ol - gl)
        fin = np.isfinite(ol)
        assert np.array_equal(np.isfinite(gl), fin), where
        if fin.any():
            e = float(np.max(err[fin] / np.maximum(1.0, np.abs(ol[fin]))))
            rep.max_lse_err = max(rep.max_lse_err, e)
            assert e < 4e-6, f"{where}: lse differs by {e}"
        rep.rows += int(read.sum())
        rep.lse_equal += int(np.sum(O.lse[read].view(np.uint32) == g["lse"][b][read].view(np.uint32)))
    nO = int(np.isfinite(O.score).sum())
    nG = int(np.isfinite(gs).sum())
    assert nO == nG, f"{where}: {nO} oracle slots vs {nG} GPU slots"
    rep.slots += nO
    assert np.all(gp[nG:] == -1) and np.all(gt[nG:] == -1) and np.all(gn[nG:] == -1)
    assert np.all(gq[nG:] == -1) and np.all(gf[nG:] == 0) and np.all(np.isneginf(gs[nG:]))
    same = ((O.parent[:nO] == gp[:nO]) & (O.token[:nO] == gt[:nO]) & (O.node[:nO] == gn[:nO]) &
            (O.fin[:nO] == gf[:nO]) & np.all(O.seq[:nO] == gq[:nO], axis=1))
    score_err = np.abs(O.score[:nO].astype(np.float64) - gs[:nO].astype(np.float64))
    if nO:
        rep.max_score_err = max(rep.max_score_err, float(score_err[same].max() if same.any() else 0))
    assert np.all(score_err[same] <= SCORE_TOL), where
    if same.all():
        return
    # near-tie explanation of every difference
    lse_o = O.lse
    inv_t = np.float32(1.0) / np.float32(temperature) if temperature > 0 else np.float32(1.0)

    def oscore(j, tok):
        if tok < 0:  # carried
            return float(pre["score"][j])
        xt = np.float32(as_f32(x[j:j + 1, tok])[0]) * inv_t
        return float(np.float32(pre["score"][j]) + (xt - np.float32(lse_o[j])))

    def orank(j, tok, c):
        """The oracle's ranking score of candidate (j, tok) with score c."""
        k = np.float32(c)
        if alpha != 0:
            n = t + 1 if tok >= 0 else int(np.sum(pre["seq"][j] != -1))
            k = np.float32(k / oracle.length_penalty(n, alpha))
        if temperature > 0:
            flat = j * V + (tok if tok >= 0 else eos)
            k = np.float32(k + oracle.gumbel(seed, b, t, flat))
        return float(k)

    o_c = {(int(O.parent[i]), int(O.token[i])): i for i in range(nO)}
    g_c = {(int(gp[i]), int(gt[i])): i for i in range(nG)}
    boundary = (orank(int(O.parent[nO - 1]), int(O.token[nO - 1]), float(O.score[nO - 1]))
                if nO == K else -np.inf)
    for key in set(o_c) ^ set(g_c):
        rk = orank(*key, oscore(*key))
        assert abs(rk - boundary) <= TIE, f"{where}: candidate {key} ({rk}) differs, boundary {boundary}"
        rep.excused += 1
    for i in np.flatnonzero(~same):
        key = (int(gp[i]), int(gt[i]))
        sc = oscore(*key)
        ro = orank(int(O.parent[i]), int(O.token[i]), float(O.score[i]))
        assert abs(orank(*key, sc) - ro) <= TIE or key not in o_c, \
            f"{where}: slot {i} holds {key} ({sc}) where the oracle has {float(O.score[i])}"
        assert abs(float(gs[i]) - sc) <= SCORE_TOL, where
        if key in o_c:
            k = o_c[key]
            assert gn[i] == O.node[k] and gf[i] == O.fin[k] and np.array_equal(gq[i], O.seq[k]), where
        # whether or not the oracle holds it: a real candidate of its parent
        check_valid_slot(g, b, t, i, pre, V, eos, where, level=level, min_length=min_length,
                         banned=banned, norm_range=norm_range)
        rep.validated += 1
    rep.mismatched_slots += int((~same).sum())


_POOL = None


def oracle_pool():
    """Threads for the oracle: requests are independent and each oracle call
    releases the interpreter lock inside the C library."""
    global _POOL
    if _POOL is None:
        import os
        from concurrent.futures import ThreadPoolExecutor
        _POOL = ThreadPoolExecutor(max_workers=max(1, min(16, os.cpu_count() or 1)))
    return _POOL


def oracle_steps(blocks: dict, st: dict, t: int, level, **kw) -> dict:
    """Oracle step of every request b in blocks (b -> [K, V] logits) from the
    host state st (score, node, fin, seq; [B, ...] arrays), in parallel."""
    futs = {b: oracle_pool().submit(oracle.step, x, st["score"][b], st["node"][b], st["fin"][b],
                                    st["seq"][b], t, level=level, request=b, **kw)
            for b, x in blocks.items()}
    return {b: f.result() for b, f in futs.items()}


def init_state(B, K, T, constrained: bool) -> dict:
    score = np.full((B, K), -np.inf, np.float32)
    score[:, 0] = 0
    node = np.full((B, K), -1, np.int32)
    if constrained:
        node[:, 0] = 0
    return dict(score=score, node=node, fin=np.zeros((B, K), np.uint8),
                seq=np.full((B, K, T), -1, np.int32))


def pre_of(st: dict, b: int) -> dict:
    return dict(score=st["score"][b], node=st["node"][b], fin=st["fin"][b], seq=st["seq"][b])


def mask_kw(cfg, min_length=0, banned=None, norm="full", norm_range=(0, 0)) -> dict:
    """The validity rules of compare_request for a search's options."""
    return dict(min_length=min_length, banned=banned,
                norm_range=tuple(norm_range) if norm == "range" else None)


def level_of(trie, t):
    return (trie.offsets[t], trie.tokens[t], trie.children[t]) if trie is not None else None


def make_beam(gr, cfg, trie, temperature=0.0, seed=0, alpha=0.0, min_length=0, banned=None,
              norm="full", norm_range=(0, 0), dense_levels=(), fused=True):
    """A GPU trie (or None) and beam for cfg with the given options (fused:
    the mode of gr_beam_set_fused; True keeps the default)."""
    gtrie = gr.Trie.from_csr(trie) if trie is not None else None
    for level in dense_levels:
        gtrie.densify(level)
    beam = gr.Beam(cfg.batch, cfg.beam, cfg.vocab, cfg.steps, eos=cfg.eos, dtype=cfg.dtype,
                   trie=gtrie)
    if temperature > 0:
        beam.set_sampling(temperature, seed)
    if alpha or min_length or banned:
        beam.set_penalties(alpha, min_length, banned)
    if norm != "full":
        beam.set_normalization(norm, *norm_range)
    if fused is not True:
        beam.set_fused(fused)
    return gtrie, beam


class Stepwise:
    """The GPU and the oracle stepped side by side on one search: after each
    GPU step every compared request is checked against the oracle's step
    from the same pre-step state.  follow=False re-synchronises the GPU to
    the oracle's state after each step (so an excused near-tie cannot
    cascade; the live bound then comes from that state); follow=True lets
    the GPU run free and takes each pre-step state from the GPU itself (its
    own live bound, as in a real search)."""

    def __init__(self, gr, cfg, trie, rep=None, requests=None, ctx="", follow=False,
                 temperature: float = 0.0, seed: int = 0, alpha: float = 0.0, min_length: int = 0,
                 banned=None, norm: str = "full", norm_range=(0, 0), dense_levels=(), fused=True):
        self.cfg, self.trie, self.ctx, self.follow = cfg, trie, ctx, follow
        self.rep = rep or Report()
        self.reqs = list(range(cfg.batch)) if requests is None else list(requests)
        self.requests = requests
        self.okw = dict(eos=cfg.eos, temperature=temperature, seed=seed, alpha=alpha,
                        min_length=min_length, banned=banned, norm=norm, norm_range=norm_range)
        self.ckw = dict(temperature=temperature, seed=seed, alpha=alpha,
                        **mask_kw(cfg, min_length, banned, norm, norm_range))
        self.gtrie, self.beam = make_beam(gr, cfg, trie, temperature, seed, alpha, min_length,
                                          banned, norm, norm_range, dense_levels, fused)
        self.st = init_state(cfg.batch, cfg.beam, cfg.steps, trie is not None)
        g0 = state_np(self.beam)
        assert np.array_equal(g0["scores"], self.st["score"]) and np.array_equal(g0["nodes"], self.st["node"])
        assert np.all(g0["sequences"] == -1) and np.all(g0["finished"] == 0)
        self.t = 0
        self.last = None

    def step(self, x: np.ndarray, x_dev=None):
        """One step on host logits x [B, K, V] (x_dev: the same on the device)."""
        torch = torch_mod()
        cfg, t = self.cfg, self.t
        xd = to_dev(x) if x_dev is None else x_dev
        self.beam.step(xd)
        torch.cuda.synchronize()
        g = state_np(self.beam)
        lvl = level_of(self.trie, t)
        outs = oracle_steps({b: x[b] for b in self.reqs}, self.st, t, lvl, **self.okw)
        for b in self.reqs:
            compare_request(outs[b], g, b, t, pre_of(self.st, b), x[b], cfg.vocab, cfg.eos, self.rep,
                            self.ctx, level=lvl, **self.ckw)
        self.t += 1
        self.last = g
        if self.follow:
            self.st = dict(score=g["scores"].copy(), node=g["nodes"].copy(), fin=g["finished"].copy(),
                           seq=g["sequences"].copy())
            return g
        new = dict(score=self.st["score"].copy(), node=self.st["node"].copy(), fin=self.st["fin"].copy(),
                   seq=self.st["seq"].copy())
        if self.requests is not None:  # requests not compared keep the GPU's own state
            new = dict(score=g["scores"].copy(), node=g["nodes"].copy(), fin=g["finished"].copy(),
                       seq=g["sequences"].copy())
        for b in self.reqs:
            O = outs[b]
            new["score"][b], new["node"][b], new["fin"][b], new["seq"][b] = O.score, O.node, O.fin, O.seq
        self.st = new
        if self.t < cfg.steps:
            set_state_from(self.beam, self.t, new["score"], new["node"], new["fin"], new["seq"])
        return g

    def close(self):
        self.beam.close()
        if self.gtrie is not None:
            self.gtrie.close()


def run_stepwise(gr, cfg, trie, logits_of, steps=None, rep=None, requests=None, ctx="",
                 follow=False, **opts):
    """Step the GPU and the oracle side by side (Stepwise) for `steps` steps;
    logits_of(t) -> host [B, K, V] array.  opts: temperature, seed, alpha,
    min_length, banned, norm, norm_range, dense_levels, fused."""
    steps = cfg.steps if steps is None else steps
    run = Stepwise(gr, cfg, trie, rep=rep, requests=requests, ctx=ctx, follow=follow, **opts)
    for t in range(steps):
        run.step(logits_of(t))
    run.close()
    return run.rep


def fill_device_step(X, cfg, t, rows, keep=()):
    """Copy step t's seeded logits (first `rows` rows of every request) into
    the device tensor X [B, K, V] block by block; return the host blocks of
    the requests in `keep`."""
    import synth
    torch = torch_mod()
    kept = {}
    for b, blk in synth.iter_step_blocks(cfg, t, rows=rows):
        src = torch.from_numpy(blk.view(np.int16) if blk.dtype == np.uint16 else blk)
        X[b, :rows].copy_(src)
        if b in keep:
            full = np.zeros((cfg.beam, cfg.vocab), blk.dtype)
            full[:rows] = blk
            kept[b] = full
    return kept


def run_sampled(gr, cfg, trie, requests, steps=None, rep=None, ctx="", temperature: float = 0.0,
                seed: int = 0, dense_levels=()):
    """Full-size steps on the GPU; the oracle follows the requests in
    `requests` (all of them, or a sample).  After each step the compared
    requests are re-synchronised to the oracle's state and the others keep
    the GPU's own.  temperature > 0: both sides sampled with the same seed."""
    torch = torch_mod()
    steps = cfg.steps if steps is None else steps
    rep = rep or Report()
    requests = list(requests)
    gtrie, beam = make_beam(gr, cfg, trie, temperature=temperature, seed=seed, dense_levels=dense_levels)
    tdt = torch.int16 if cfg.dtype == "bf16" else torch.float32
    X = torch.zeros((cfg.batch, cfg.beam, cfg.vocab), dtype=tdt, device="cuda")
    st = init_state(cfg.batch, cfg.beam, cfg.steps, trie is not None)
    live = 1
    for t in range(steps):
        rows = min(cfg.beam, live)
        host = fill_device_step(X, cfg, t, rows, keep=set(requests))
        beam.step(X)
        torch.cuda.synchronize()
        g = state_np(beam)
        lvl = level_of(trie, t)
        outs = oracle_steps(host, st, t, lvl, eos=cfg.eos, temperature=temperature, seed=seed)
        for b in requests:
            O = outs[b]
            compare_request(O, g, b, t, pre_of(st, b), host[b], cfg.vocab, cfg.eos, rep, ctx,
                            temperature, seed, level=lvl)
            g["scores"][b], g["nodes"][b], g["finished"][b], g["sequences"][b] = O.score, O.node, O.fin, O.seq
        del host
        st = dict(score=g["scores"], node=g["nodes"], fin=g["finished"], seq=g["sequences"])
        if t + 1 < steps:
            set_state_from(beam, t + 1, st["score"], st["node"], st["fin"], st["seq"])
        mc = trie.max_fanout(t) if trie is not None else cfg.vocab
        live = min(cfg.beam, live * mc)
        print(f"[{ctx}] step {t}: {rep}", flush=True)
    del X
    beam.close()
    if gtrie is not None:
        gtrie.close()
    return rep

"""The seeded input generators: reproducible, well-formed, the stated shapes."""
import numpy as np
import pytest

import synth
from synth.catalog import csr_from_codes


def _check_csr(trie):
    """Every CSR invariant the library's validator also demands."""
    nn = trie.num_nodes
    assert nn[0] == 1
    for L in range(trie.depth):
        off, tok, ch = trie.offsets[L], trie.tokens[L], trie.children[L]
        assert off[0] == 0 and off[-1] == len(tok) == len(ch)
        assert np.all(np.diff(off) >= 1), "every inner node has a child"
        # tokens strictly increasing within a node, inside the level's id range
        lo = trie.sid_base + L * trie.codebook
        assert tok.min() >= lo and tok.max() < lo + trie.codebook
        d = np.diff(tok.astype(np.int64))
        starts = off[1:-1]
        inside = np.ones(len(d), bool)
        inside[starts - 1] = False
        assert np.all(d[inside] > 0)
        assert ch.min() >= 0 and ch.max() < nn[L + 1]


def _walk(trie, codes):
    """Leaf id of each SID found by walking the CSR (binary search per level)."""
    out = []
    for row in codes:
        n = 0
        for L, c in enumerate(row):
            off, tok = trie.offsets[L], trie.tokens[L]
            a, b = off[n], off[n + 1]
            v = trie.sid_base + L * trie.codebook + int(c)
            e = a + np.searchsorted(tok[a:b], v)
            assert e < b and tok[e] == v
            n = trie.children[L][e]
        out.append(n)
    return np.array(out)


@pytest.mark.parametrize("name", ["c1", "c2"])
def test_catalog_csr_matches_codes(name):
    cfg = synth.get(name)
    trie = synth.make_trie(cfg)
    codes = trie.codes
    assert codes.shape == (cfg.n_sids, cfg.depth)
    # distinct and sorted lexicographically
    keys = np.zeros(len(codes), np.int64)
    for L in range(cfg.depth):
        keys = keys * cfg.codebook + codes[:, L]
    assert np.all(np.diff(keys) > 0)
    _check_csr(trie)
    rng = np.random.default_rng(0)
    idx = rng.choice(len(codes), size=min(500, len(codes)), replace=False)
    assert np.array_equal(_walk(trie, codes[idx]), idx), "leaf id = catalog row"


@pytest.mark.parametrize("name", ["c1", "c2", "c4s"])
def test_relabel_keeps_paths_and_moves_node_ids(name):
    """relabel permutes every level's node ids: a well-formed CSR, every
    catalog SID still reaches a leaf, the leaf ids follow the permutation,
    and child ids are no longer the edge ordinals."""
    cfg = (synth.get("c4").shrink(n_sids=10_000, root_fanout=6, mean_fanout=8, name="c4s")
           if name == "c4s" else synth.get(name))
    trie = synth.make_trie(cfg)
    tr2, perms = synth.relabel(trie, 5)
    _check_csr(tr2)
    assert tr2.num_nodes == trie.num_nodes
    rng = np.random.default_rng(1)
    idx = rng.choice(len(trie.codes), size=min(500, len(trie.codes)), replace=False)
    assert np.array_equal(_walk(tr2, trie.codes[idx]), perms[-1][idx])
    for L in range(trie.depth):
        # the same multiset of (parent path, token) edges: sorted tokens per level agree
        assert np.array_equal(np.sort(tr2.tokens[L]), np.sort(trie.tokens[L]))
        if len(tr2.children[L]) > 1:
            assert not np.array_equal(tr2.children[L], np.arange(len(tr2.children[L]))), L


def test_small_csr_by_hand():
    codes = np.array([[0, 1], [0, 2], [2, 0]], np.uint8)
    t = csr_from_codes(codes, 3, 0, 6)
    assert t.num_nodes == [1, 2, 3]
    assert t.offsets[0].tolist() == [0, 2] and t.tokens[0].tolist() == [0, 2]
    assert t.children[0].tolist() == [0, 1]
    assert t.offsets[1].tolist() == [0, 2, 3] and t.tokens[1].tolist() == [4, 5, 3]
    assert t.children[1].tolist() == [0, 1, 2]


def test_zipf_skew_and_seeds():
    cfg = synth.get("c2").shrink(n_sids=20000)
    a = synth.make_codes(cfg)
    b = synth.make_codes(cfg)
    assert np.array_equal(a, b)
    first = np.bincount(a[:, 0].astype(np.int64), minlength=cfg.codebook)
    assert first[0] > 5 * np.median(first), "level 0 is Zipf-skewed toward code 0"
    last = np.bincount(a[:, 2].astype(np.int64), minlength=cfg.codebook)
    assert last.max() < 3 * last.mean(), "last level is uniform"


def test_logits_blocks_reproducible_and_shaped():
    cfg = synth.get("c5")
    x = synth.step_logits(cfg, 3, 7, rows=4)
    y = synth.step_logits(cfg, 3, 7)
    assert x.shape == (4, cfg.vocab) and y.shape == (cfg.beam, cfg.vocab)
    assert np.array_equal(x, y[:4]), "row j is the same whatever the row count"
    z = synth.step_logits(cfg, 3, 8, rows=4)
    assert not np.array_equal(x, z)
    # EOS bias log((t+1)/T) at 0-based t
    big = synth.step_logits(cfg, 0, 0)
    assert abs(float(big[:, 0].mean()) - np.log(1 / 32)) < 0.4
    assert abs(float(big[:, 1:].mean())) < 0.01


def test_bf16_conversion_is_rne():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(100000) * 3).astype(np.float32)
    # exact ties: low 16 bits 0x8000
    ties = (x.view(np.uint32) & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    x = np.concatenate([x, ties.view(np.float32)])
    ours = synth.to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = synth.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_c3_layout():
    cfg = synth.get("c3")
    assert cfg.sid_base + cfg.depth * cfg.codebook == cfg.vocab
    blk = synth.step_logits(cfg.shrink(beam=2), 0, 0)
    assert blk.dtype == np.uint16 and blk.shape == (2, cfg.vocab)
    f = synth.bf16_bits_to_f32(blk)
    assert abs(f[:, cfg.sid_base:].mean() - 2.0) < 0.05
    assert abs(f[:, :cfg.sid_base].mean()) < 0.02

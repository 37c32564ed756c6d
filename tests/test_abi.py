"""The C-ABI library: it loads, exports every function include/gr.h declares,
and its host-only paths (CSR validation, status strings) behave as documented.
No compute call is made here, so these run without a GPU."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gr.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(gr_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def gr():
    import trie_constrained_beam_step_amd as gr
    if not os.path.exists(os.path.join(ROOT, "trie_constrained_beam_step_amd", "libgr.so")):
        from trie_constrained_beam_step_amd import build
        build.build()
    gr.lib()
    return gr


def test_every_declared_symbol_is_exported(gr):
    names = declared_functions()
    assert len(names) >= 20
    lib = C.CDLL(gr._lib.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in gr.h but not exported"
    assert set(names) == set(gr._lib.SIGNATURES), "binding declares exactly the header's functions"


def test_single_hip_runtime(gr):
    maps = gr._lib.hip_runtimes_mapped()
    assert len(maps) <= 1, maps


def test_status_strings_and_version(gr):
    L = gr.lib()
    assert L.gr_status_string(0) == b"GR_OK"
    assert L.gr_status_string(2) == b"GR_ERR_BAD_TRIE"
    assert L.gr_status_string(99) == b"GR_ERR_UNKNOWN"
    assert b"gfx950" in L.gr_version()


def _c1_csr():
    t = synth.make_trie(synth.get("c1"))
    return ([o.copy() for o in t.offsets], [x.copy() for x in t.tokens],
            [c.copy() for c in t.children], t.vocab, t.num_nodes)


def test_validate_accepts_generated_tries(gr):
    o, tk, ch, V, nn = _c1_csr()
    gr.trie_validate(o, tk, ch, V, nn)
    t = synth.make_trie(synth.get("c2").shrink(n_sids=5000))
    gr.trie_validate(t.offsets, t.tokens, t.children, t.vocab, t.num_nodes)
    r, _ = synth.relabel(t, 3)  # node ids permuted per level
    gr.trie_validate(r.offsets, r.tokens, r.children, r.vocab, r.num_nodes)


@pytest.mark.parametrize("mutation,status", [
    ("unsorted_tokens", 2), ("duplicate_token", 2), ("token_out_of_range", 2),
    ("negative_token", 2), ("child_out_of_range", 2), ("offsets_decrease", 2),
    ("offsets_first_nonzero", 2), ("root_two_nodes", 2), ("depth_zero", 1), ("vocab_zero", 1),
])
def test_validate_rejects(gr, mutation, status):
    o, tk, ch, V, nn = _c1_csr()
    nn = list(nn)
    if mutation == "unsorted_tokens":
        tk[1][0], tk[1][1] = tk[1][1], tk[1][0]
    elif mutation == "duplicate_token":
        tk[1][1] = tk[1][0]
    elif mutation == "token_out_of_range":
        tk[2][5] = V
    elif mutation == "negative_token":
        tk[0][0] = -1
    elif mutation == "child_out_of_range":
        ch[1][3] = nn[2]
    elif mutation == "offsets_decrease":
        o[1][3] = o[1][2] - 1
    elif mutation == "offsets_first_nonzero":
        o[2][0] = 1
    elif mutation == "root_two_nodes":
        nn[0] = 2
    if mutation == "depth_zero":
        rc = gr.lib().gr_trie_validate(0, V, np.zeros(1, np.int64).ctypes.data, None, None, None)
        assert rc == status
        return
    if mutation == "vocab_zero":
        V = 0
    with pytest.raises(gr.GrError) as ei:
        gr.trie_validate(o, tk, ch, V, nn)
    assert ei.value.status == status
    assert gr.lib().gr_last_error()  # a message explains it


def test_null_arguments_are_errors(gr):
    L = gr.lib()
    assert L.gr_trie_validate(1, 4, None, None, None, None) == 1
    assert L.gr_beam_step(None, None, None) == 1
    assert L.gr_beam_view_get(None, None) == 1
    assert L.gr_beam_init(None, None, None, None) == 1
    L.gr_beam_free(None)  # NULL-safe
    L.gr_trie_free(None)
    # checked on the host before any device work
    assert L.gr_trie_densify(None, 0, -1, None, None) == 1
    assert L.gr_probe_draw_error(0, 1, None, None) == 1
    assert L.gr_probe_draw_error(0, (1 << 32) + 1, C.c_void_p(16), None) == 1


def test_draw_error_bound_is_the_pruning_margin(gr):
    """The bound the sampled rows' pruning assumes for its fast draw
    estimates: 2^-12 (a worst case measured on the GPU is far below it)."""
    assert gr.draw_error_bound() == 2.0 ** -12


DEMO = os.path.join(ROOT, "tests", "c", "abi_demo")


def _demo():
    if not os.path.exists(DEMO):
        import importlib.util
        spec = importlib.util.spec_from_file_location("build_demo", os.path.join(ROOT, "tests", "c", "build_demo.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    return DEMO


def test_plain_c_program_host_part(gr):
    """A C program linked to libgr.so (no Python, no torch) builds and runs:
    status strings, version and trie validation; without a GPU it stops
    there (exit 77)."""
    import subprocess
    r = subprocess.run([_demo()], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=120)
    assert r.returncode in (0, 77), r.stdout
    assert "catalog: 51 SIDs" in r.stdout


def test_static_step_argument_errors(gr):
    """gr_beam_step_static refuses bad arguments on the host, before any
    device call: NULL io, a bad configuration, a NULL buffer, a step index
    past max_steps, and outputs overlapping inputs."""
    import ctypes as C
    from trie_constrained_beam_step_amd._lib import BeamConfig, StepIO
    L = gr.lib()
    assert L.gr_beam_step_static(None, None) == 1

    def io_with(**kw):
        io = StepIO()
        io.config = BeamConfig(batch=1, beam_width=4, vocab=10, max_steps=2, eos_token=-1, logits_dtype=0,
                               logits_row_stride=0)
        base = 1 << 20
        for i, name in enumerate(["logits", "scores", "nodes", "finished", "sequences", "scores_out",
                                  "nodes_out", "finished_out", "sequences_out", "parents_out", "tokens_out",
                                  "lse_out"]):
            setattr(io, name, base * (i + 1))  # distinct, never dereferenced
        for k, v in kw.items():
            setattr(io, k, v)
        return io

    cases = [
        (dict(config=BeamConfig(batch=0, beam_width=4, vocab=10, max_steps=2, eos_token=-1)), 1),
        (dict(config=BeamConfig(batch=1, beam_width=4, vocab=10, max_steps=2, eos_token=-1,
                                logits_dtype=7)), 1),
        (dict(scores_out=None), 1),
        (dict(lse_out=None), 1),
        (dict(step=2), 3),
        (dict(step=-1), 1),
        (dict(live_bound=-3), 1),
        (dict(temperature=-1.0), 1),
        (dict(scores_out=(1 << 20) * 2 + 4), 1),  # overlaps scores
    ]
    for kw, status in cases:
        io = io_with(**kw)
        assert L.gr_beam_step_static(C.byref(io), None) == status, (kw, L.gr_last_error())

"""The no-allocation step (gr_beam_step_static) against the handle's step
(gr_beam_step): the same kernels on the same inputs, so every output must be
bit-equal.  Two searches in a row on one process's static workspace, the
second smaller than the first, then a step that needs more workspace than
the static buffer holds (refused before anything is enqueued)."""
import numpy as np
import pytest

import synth
from gpu_util import state_np, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gr():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import trie_constrained_beam_step_amd as gr
    gr.lib()
    return gr


def _static_search(gr, cfg, trie_host, live_bound, temperature=0.0, seed=0):
    """Step a handle through the whole search; before each step, run the
    static step on a copy of the handle's state and compare every output."""
    import torch
    gtrie = gr.Trie.from_csr(trie_host) if trie_host is not None else None
    beam = gr.Beam(cfg.batch, cfg.beam, cfg.vocab, cfg.steps, eos=cfg.eos, dtype=cfg.dtype, trie=gtrie)
    if temperature > 0:
        beam.set_sampling(temperature, seed)
    B, K, T = cfg.batch, cfg.beam, cfg.steps
    dev = "cuda"
    for t in range(cfg.steps):
        x = to_dev(synth.full_step(cfg, t))
        pre = beam.state()
        state = {k: pre[k].clone() for k in ("scores", "nodes", "finished", "sequences")}
        out = dict(scores=torch.full((B, K), 7.0, device=dev), nodes=torch.full((B, K), 7, dtype=torch.int32, device=dev),
                   finished=torch.full((B, K), 7, dtype=torch.uint8, device=dev),
                   sequences=torch.full((B, K, T), 7, dtype=torch.int32, device=dev),
                   parents=torch.full((B, K), 7, dtype=torch.int32, device=dev),
                   tokens=torch.full((B, K), 7, dtype=torch.int32, device=dev),
                   lse=torch.full((B, K), 7.0, device=dev))
        gr.beam_step_static(B, K, cfg.vocab, T, t, x, state, out, eos=cfg.eos, dtype=cfg.dtype, trie=gtrie,
                            live_bound=live_bound, temperature=temperature, seed=seed)
        beam.step(x)
        torch.cuda.synchronize()
        g = state_np(beam)
        got = {k: v.cpu().numpy() for k, v in out.items()}
        for k in ("scores", "nodes", "finished", "sequences", "lse"):
            assert np.array_equal(got[k].view(np.uint8), g[k].view(np.uint8)), (cfg.name, t, k)
        assert np.array_equal(got["parents"], g["parents"][t]), (cfg.name, t)
        assert np.array_equal(got["tokens"], g["tokens"][t]), (cfg.name, t)
        print(f"[no-alloc] {cfg.name} step {t}: {int(np.isfinite(got['scores']).sum())} slots bit-equal",
              flush=True)
        del x
    beam.close()
    if gtrie is not None:
        gtrie.close()


def test_static_step_equals_handle_step(gr):
    # first: SID trie rows (B 4, K 256, V 768), every slot allowed live; the
    # tiny catalog (its steps fused); then a smaller unconstrained EOS search
    # (B 2, K 16, V 5,000) with the exact live bound unknown (0 = K), then
    # sampled
    big = synth.get("c2").shrink(batch=4, n_sids=100_000, name="na2")
    _static_search(gr, big, synth.make_trie(big), live_bound=0)
    tiny = synth.get("c1")  # every step fused (one workgroup per request)
    _static_search(gr, tiny, synth.make_trie(tiny), live_bound=0)
    small = synth.get("c5").shrink(batch=2, beam=16, vocab=5000, steps=4, name="na5")
    _static_search(gr, small, None, live_bound=0)
    _static_search(gr, small, None, live_bound=16, temperature=0.8, seed=9)


def test_static_step_refuses_oversized_workspace(gr):
    import torch
    B, K, V, T = 256, 4096, 8, 2
    dev = "cuda"
    x = torch.zeros((B, K, V), device=dev)
    st = dict(scores=torch.zeros((B, K), device=dev), nodes=torch.zeros((B, K), dtype=torch.int32, device=dev),
              finished=torch.zeros((B, K), dtype=torch.uint8, device=dev),
              sequences=torch.zeros((B, K, T), dtype=torch.int32, device=dev))
    out = {k: v.clone() for k, v in st.items()}
    out.update(parents=torch.zeros((B, K), dtype=torch.int32, device=dev),
               tokens=torch.zeros((B, K), dtype=torch.int32, device=dev), lse=torch.zeros((B, K), device=dev))
    with pytest.raises(gr.GrError, match="GR_ERR_UNSUPPORTED.*static workspace"):
        gr.beam_step_static(B, K, V, T, 0, x, st, out)
    torch.cuda.synchronize()

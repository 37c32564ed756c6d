"""The five synthetic workloads of the trie-constrained beam step, as data.

Nothing here computes any part of the beam step: it only names shapes,
distributions and seeds.  Both the oracle side and the GPU side draw their
inputs from this package, so the two see identical bytes.

Workload sources (FlashRec README, "Features" table and "Decoding"; beamgrad
README, "How it works"):
  * SID decoding runs 3-5 steps at beam widths of 50-512+, every continuation
    restricted to a catalog of valid semantic IDs;
  * the plain / EOS-terminated search keeps finished beams competing.
The concrete sizes are the benchmark's: see the ``CONFIGS`` table below.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional

F32 = "f32"
BF16 = "bf16"


@dataclass(frozen=True)
class Config:
    """One synthetic workload.

    Attributes:
      name:       short name ("c1", "c1x", "c2", ...).
      seed_id:    integer mixed into every seed (workloads that share a catalog
                  and logits, like c1 and c1x, share it).
      batch:      B, independent requests.
      beam:       K, beam width (slots per request).
      vocab:      V, logits per row.
      steps:      number of beam steps to run.
      dtype:      "f32" or "bf16" logits.
      depth:      trie depth D (None = unconstrained search).
      codebook:   codes per SID level.
      sid_base:   first vocabulary id used by SID tokens; the token of code c at
                  level L is sid_base + L*codebook + c.
      n_sids:     catalog size.
      catalog:    "uniform", "zipf0" (level 0 Zipf), "zipf01" (levels 0 and 1
                  Zipf) or "branching" (random branching tree).
      zipf_s:     Zipf exponent.
      sigma:      standard deviation of the i.i.d. normal logits.
      bias_sigma: standard deviation of a per-token bias shared by all rows
                  (0 = none).
      sid_shift:  constant added to every SID token's logit.
      eos:        EOS token id, -1 = none.
      eos_bias:   "log_t_over_T" adds log((t+1)/steps) to the EOS logit at
                  0-based step t; "" = no bias.
      root_fanout, mean_fanout: for catalog == "branching".
    """

    name: str
    seed_id: int
    batch: int
    beam: int
    vocab: int
    steps: int
    dtype: str = F32
    depth: Optional[int] = None
    codebook: int = 0
    sid_base: int = 0
    n_sids: int = 0
    catalog: str = ""
    zipf_s: float = 1.1
    sigma: float = 1.0
    bias_sigma: float = 0.0
    sid_shift: float = 0.0
    eos: int = -1
    eos_bias: str = ""
    root_fanout: int = 0
    mean_fanout: int = 0

    @property
    def constrained(self) -> bool:
        return self.depth is not None

    @property
    def itemsize(self) -> int:
        return 2 if self.dtype == BF16 else 4

    def shrink(self, **kw) -> "Config":
        """A smaller variant with its own seeds (name gets a suffix)."""
        name = kw.pop("name", self.name + "-small")
        seed_id = kw.pop("seed_id", self.seed_id * 1000 + 7)
        return replace(self, name=name, seed_id=seed_id, **kw)


CONFIGS = {
    # Tiny SID trie: depth 3, codebook 16 per level, V = 48 (level L uses ids
    # 16L..16L+15); 2,000 distinct SIDs drawn uniformly from the 16^3 space;
    # B = 2, K = 8, 3 steps; fp32 logits N(0, 2).
    "c1": Config("c1", 1, batch=2, beam=8, vocab=48, steps=3, dtype=F32, depth=3,
                 codebook=16, sid_base=0, n_sids=2000, catalog="uniform", sigma=2.0),
    # The exhaustive-check variant of c1: K = 2,000 >= every level's number of
    # valid prefixes, so beam search must return the whole catalog, sorted.
    "c1x": Config("c1x", 1, batch=2, beam=2000, vocab=48, steps=3, dtype=F32, depth=3,
                  codebook=16, sid_base=0, n_sids=2000, catalog="uniform", sigma=2.0),
    # SID-only vocabulary: depth 3, codebook 256 (V = 768); 1M distinct SIDs
    # with Zipf(1.1) first-level codes; B = 32, K = 256; N(0,1) + per-token
    # bias N(0, 0.5).
    "c2": Config("c2", 2, batch=32, beam=256, vocab=768, steps=3, dtype=F32, depth=3,
                 codebook=256, sid_base=0, n_sids=1_000_000, catalog="zipf0",
                 sigma=1.0, bias_sigma=0.5),
    # LLM-vocabulary rows: V = 151,936 bf16; SID tokens are the last
    # 3 x 8,192 ids; 10M distinct depth-3 SIDs with Zipf-skewed prefixes;
    # B = 32, K = 512; N(0,1) with SID tokens shifted by +2.
    "c3": Config("c3", 3, batch=32, beam=512, vocab=151_936, steps=3, dtype=BF16, depth=3,
                 codebook=8192, sid_base=151_936 - 3 * 8192, n_sids=10_000_000,
                 catalog="zipf01", sigma=1.0, sid_shift=2.0),
    # Deep wide trie: depth 5, codebook 256 (V = 1,280 fp32); 50M SIDs from
    # seeded random branching, mean fan-out ~36; B = 64, K = 512; N(0, 1.5).
    "c4": Config("c4", 4, batch=64, beam=512, vocab=1280, steps=5, dtype=F32, depth=5,
                 codebook=256, sid_base=0, n_sids=50_000_000, catalog="branching",
                 sigma=1.5, root_fanout=31, mean_fanout=36),
    # Unconstrained beam search with EOS: V = 50,257 fp32 N(0,1), EOS = 0 with
    # logit bias log(t/32) at 1-based step t; B = 64, K = 64, 32 steps.
    "c5": Config("c5", 5, batch=64, beam=64, vocab=50_257, steps=32, dtype=F32, depth=None,
                 sigma=1.0, eos=0, eos_bias="log_t_over_T"),
}


def get(name: str) -> Config:
    return CONFIGS[name]

"""Workload configurations.

The five named workloads stand in for the pages' evaluation inputs (long
contexts of 2K-32K tokens on Mistral-7B-shaped caches at 25% / 12.5% / 1/128
budgets). They reuse only the shapes; no benchmark item is reproduced.

Shapes: S sequences, Ly layers, H KV heads, G query heads per KV head, d head
dim, P probe queries per query head.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field
from typing import List

import numpy as np


@dataclass
class Config:
    name: str
    S: int
    Ly: int
    H: int
    G: int
    d: int
    lens: List[int]
    dtype: str = "bf16"          # dtype of K/V/queries/hidden: "bf16" or "f32"
    rope_base: float = 1e6
    P: int = 64                  # probe queries per query head
    token_mode: bool = False     # token-level top-B only (no slots, no trees)
    slot_len: int = 64           # fixed slot length; 0 = slots cut by the DP
    slot_min: int = 16
    slot_max: int = 128
    slot_target: int = 64
    lambda_len: float = 1.0
    lambda_curv: float = 4.0
    budget_ratio: float = 0.25
    budget_min: int = 32
    prompt_exact: int = 0
    recent_exact: int = 0
    suffix_exact: int = 0
    floor_frac: float = 0.02
    hybrid_frac: float = 0.0     # head-level hybrid: share of (layer, KV head) units kept whole
    window: int = 64             # step-wise eviction: recent queries behind the features
    n_hops: int = 2
    n_seeds: int = 32
    hop_weight: float = 0.3
    split_mode: int = 0          # 0: midpoint binary trees; 1: curvature-candidate cuts + salient three-way splits
    n_dprobe: int = 64
    w_attn: float = 0.25
    w_value: float = 0.75
    value_base: float = 0.1
    T_dec: int = 1
    vocab: int = 2048
    w_dtype: str = "bf16"
    logit_tau: float = 4.0
    hidden_dim: int = 0          # >0: hidden-state trajectories are drawn
    n_depth: int = 1             # sampled depths of the hidden-state trajectories (shared turns)
    surprisal: bool = False      # draw a per-token surprisal (higher at trajectory turns)
    lambda_surp: float = 1.0     # DP weight of the normalized surprisal at a cut
    plant: str = "spans"         # "evidence" | "spans" | "chains"
    n_plant: int = 64            # evidence tokens / spans / chains per sequence
    span_len: tuple = (4, 16)
    layer_scale: bool = False    # per-layer K/V scale 2^U(-1,1)
    seed: int = 1000

    @property
    def T(self) -> int:
        return int(sum(self.lens))

    @property
    def d_model(self) -> int:
        return self.H * self.G * self.d

    @property
    def n_rows(self) -> int:
        """Probe rows per (layer, KV head)."""
        return self.G * self.P

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


def _ragged_lens(n: int, lo: int, hi: int, seed: int) -> List[int]:
    rng = np.random.default_rng(seed)
    u = rng.random(n)
    return [int(round(lo * (hi / lo) ** x)) for x in u]


CONFIGS = {
    # 1 layer, 1 KV head, GQA 4, d 64, 512 tokens, fp32, 8 evidence tokens.
    "tiny": Config(name="tiny", S=1, Ly=1, H=1, G=4, d=64, lens=[512], dtype="f32",
                   rope_base=1e4, P=16, slot_len=32, T_dec=1, vocab=2048,
                   w_dtype="f32", plant="evidence", n_plant=8, seed=1000),
    # Mistral-7B-shaped single layer, token-level eviction only.
    "mistral1": Config(name="mistral1", S=1, Ly=1, H=8, G=4, d=128, lens=[4096],
                       token_mode=True, slot_len=0, T_dec=32, vocab=32768,
                       plant="spans", n_plant=64, seed=1001),
    # Full depth, one sequence, DP slots over hidden-state trajectories.
    "fulldepth": Config(name="fulldepth", S=1, Ly=32, H=8, G=4, d=128, lens=[16384],
                        slot_len=0, T_dec=64, vocab=32768, hidden_dim=4096,
                        plant="spans", n_plant=64, layer_scale=True, seed=1002),
    # Stress: batch 4 x 32K, budget 1/128 (also run at 1/8), two-hop chains.
    "stress": Config(name="stress", S=4, Ly=32, H=8, G=4, d=128, lens=[32768] * 4,
                     budget_ratio=1.0 / 128, slot_len=64, T_dec=128, vocab=32768,
                     plant="chains", n_plant=8, span_len=(4, 8), seed=1003),
    # The same stress inputs at a budget of 12.5%.
    "stress8": Config(name="stress8", S=4, Ly=32, H=8, G=4, d=128, lens=[32768] * 4,
                      budget_ratio=1.0 / 8, slot_len=64, T_dec=128, vocab=32768,
                      plant="chains", n_plant=8, span_len=(4, 8), seed=1003),
    # Ragged batch of 16 sequences, exact prompt/recent/suffix regions.
    "ragged": Config(name="ragged", S=16, Ly=32, H=8, G=4, d=128,
                     lens=_ragged_lens(16, 2048, 32768, 1004),
                     prompt_exact=256, recent_exact=128, suffix_exact=256,
                     slot_len=64, T_dec=256, vocab=32768, plant="spans", n_plant=64,
                     seed=1004),
}


def get_config(name: str) -> Config:
    return CONFIGS[name]


def small_config(name: str, **kw) -> Config:
    """A reduced copy of a named workload with the same structure, small
    enough for the CPU oracle to finish in seconds while still spanning
    several kernel tiles and a ragged tail."""
    base = CONFIGS[name]
    if name == "tiny":
        c = base
    elif name == "mistral1":
        c = base.replace(H=2, lens=[1000], T_dec=3, vocab=1024, n_plant=8)
    elif name == "fulldepth":
        c = base.replace(Ly=2, H=2, lens=[700], T_dec=2, vocab=1024, hidden_dim=256,
                         n_plant=8)
    elif name == "stress":
        c = base.replace(S=2, Ly=2, H=2, lens=[600, 433], T_dec=2, vocab=1024,
                         n_plant=3, budget_ratio=1.0 / 8)
    elif name == "stress8":
        c = base.replace(S=2, Ly=2, H=2, lens=[600, 433], T_dec=2, vocab=1024, n_plant=3)
    elif name == "ragged":
        c = base.replace(S=3, Ly=2, H=2, lens=[1100, 777, 900], T_dec=2, vocab=1024,
                         n_plant=6, prompt_exact=64, recent_exact=32, suffix_exact=48)
    else:
        raise KeyError(name)
    return c.replace(**kw) if kw else c

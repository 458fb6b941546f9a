"""The five named tree-verify workloads and their knobs.

Each workload is a tree-verify step of DeepSeek-V3/Kimi-style MLA attention in
absorbed form: a latent cache ``kv_c`` (512 wide) plus a decoupled RoPE key
``k_pe`` (64 wide) per token, shared by all heads ("ground_truth_in_silicon"
page, "Input Knowledge Required", item 2), and a draft tree whose nodes attend
to the whole prefix and to their own ancestors ("reading_the_reference_generator"
page, "Output Knowledge Created by This Message").

Readings taken where the pages are silent (all listed in the design notes):
  * scale is 1/sqrt(192) (128 no-RoPE + 64 RoPE dims per head) for every workload;
  * q is stored in the KV dtype; bf16 workloads draw q ~ N(0, 0.5) (std 0.5),
    the fp32 workload q ~ N(0, 1); KV ~ N(0, 1) everywhere;
  * workload k uses numpy ``default_rng(k - 1)``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple


@dataclasses.dataclass(frozen=True)
class VerifyConfig:
    name: str
    batch: int
    heads: int
    tree_nodes: int
    dtype: str                       # "f32" or "bf16" (q, kv_c, k_pe share it)
    prefix: Optional[int] = None     # fixed prefix length for every sequence
    prefix_range: Optional[Tuple[int, int]] = None  # inclusive uniform range
    tree_range: Optional[Tuple[int, int]] = None  # per-sequence tree sizes, inclusive uniform
                                     # range (packed layout); tree_nodes is then the largest
    tree_kind: str = "uniform"       # "uniform": parent of i ~ U{0..i-1}; "bounded"
    max_depth: int = 8               # bounded trees only (node 0 has depth 1)
    max_branch: int = 4              # bounded trees only
    layout: str = "contiguous"       # "contiguous" or "paged" (page_size = 1)
    pool_slots: int = 0              # paged only
    num_splits: int = 0              # 0 = let the planner choose
    q_std: float = 0.5
    kv_std: float = 1.0
    seed: int = 0
    d_latent: int = 512
    d_rope: int = 64
    scale: float = 1.0 / math.sqrt(192.0)

    @property
    def rows(self) -> int:
        """Query rows of a uniform-tree workload (ragged: see VerifyInputs.rows)."""
        return self.batch * self.tree_nodes * self.heads


CONFIGS = {
    c.name: c
    for c in (
        VerifyConfig(name="tiny_f32_b1_h16_p256_t8", batch=1, heads=16, tree_nodes=8,
                     dtype="f32", prefix=256, q_std=1.0, seed=0),
        VerifyConfig(name="b1_h64_p4096_t16_bf16", batch=1, heads=64, tree_nodes=16,
                     dtype="bf16", prefix=4096, seed=1),
        VerifyConfig(name="b4_h64_p32768_t64_bf16", batch=4, heads=64, tree_nodes=64,
                     dtype="bf16", prefix=32768, tree_kind="bounded", seed=2),
        VerifyConfig(name="b1_h64_p200000_t32_bf16_s256", batch=1, heads=64, tree_nodes=32,
                     dtype="bf16", prefix=200000, num_splits=256, seed=3),
        VerifyConfig(name="b8_h64_paged600k_t16_bf16", batch=8, heads=64, tree_nodes=16,
                     dtype="bf16", prefix_range=(8192, 65536), layout="paged",
                     pool_slots=600000, seed=4),
    )
}

# Order used by tests and docs: small parity case first, then the four large ones.
CONFIG_ORDER = list(CONFIGS)

# Further measured workloads (not among the five above): packed trees of 1..256
# nodes per sequence at the 32k prefix, random parents.
EXTRA_WORKLOADS = {
    c.name: c
    for c in (
        VerifyConfig(name="b4_h64_p32768_t1to256_ragged_bf16", batch=4, heads=64, tree_nodes=256,
                     tree_range=(1, 256), dtype="bf16", prefix=32768, seed=5),
    )
}


def get_config(name: str, **overrides) -> VerifyConfig:
    """Return the named workload, optionally with fields replaced (for tests)."""
    cfg = CONFIGS[name] if name in CONFIGS else EXTRA_WORKLOADS[name]
    return dataclasses.replace(cfg, **overrides) if overrides else cfg

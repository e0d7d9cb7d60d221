"""Workload definitions for the ZHA decode hot path (shapes, tree geometry, step counts).

Pure data: no arithmetic of the method lives here. Each workload is described by the
geometry the Zyphra pages give for their trees (blog post "Zyphra Hierarchical Attention",
sections "Building the tree", "Routing through the tree" and "How fast can ZHA get"):
contiguous key blocks of size ``block``, ``levels`` levels of recursive summaries,
``num_ref`` reference queries, per-level top-p ``top_p`` and a sink token.

The five named workloads:

* ``tiny``   1 KV head, 1 query head, head_dim 64, fp32, 4,096 keys, block 4, 3 levels,
             4 reference queries, p=0.95, 8 static decode queries (sum of 3 keys, no noise).
* ``deep``   262,144 bf16 keys, head_dim 128, 32 query heads over 4 KV heads, block 4,
             6 levels (top node spans 4,096 tokens), 16 reference queries, p=0.95,
             256 decode steps each appending one token.
* ``wide``   as ``deep`` but block 256 and 1 level (1,024 summary nodes per KV head).
* ``light``  the light router: 1 reference query, block 8, p=0.75, depth grown until the
             top level holds at most 512 nodes; N in {32K, 64K, 128K, 512K, 1M}.
* ``ultra``  16,777,216 bf16 keys, 1 reference query, block 8, 7 levels, p=0.75,
             128 decode steps, planted mixtures of 1..64 keys.
"""
from __future__ import annotations

import dataclasses


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int              # seed slot; shared by every size of one family
    head_dim: int
    num_kv_heads: int
    num_q_heads: int
    block: int
    levels: int
    num_ref: int
    n_tokens: int            # tokens in the cache before the first decode step
    dtype: str               # "f32" or "bf16"
    top_p: float
    keep_sink: bool = True
    steps: int = 0           # decode steps; each appends one token first when appends=True
    appends: bool = True
    plant_min: int = 1       # planted query = mixture of m keys, m ~ U{plant_min..plant_max}
    plant_max: int = 16
    plant_scale: float = 4.0  # |q| before noise = plant_scale * sqrt(head_dim)
    noise: bool = True       # add N(0, I) to the planted query
    planes: str = "f32"      # storage of the s vectors the router reads: "f32" or "bf16"

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def capacity(self) -> int:
        return self.n_tokens + (self.steps if self.appends else 0)

    def nodes(self, level: int, n_tokens: int | None = None) -> int:
        n = self.n_tokens if n_tokens is None else n_tokens
        return -(-n // self.block ** level)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def light_levels(n_tokens: int, block: int = 8, top_max: int = 512) -> int:
    """Smallest depth whose top level has at most ``top_max`` nodes."""
    lv = 1
    while -(-n_tokens // block ** lv) > top_max:
        lv += 1
    return lv


TINY = Workload("tiny", 0, head_dim=64, num_kv_heads=1, num_q_heads=1, block=4, levels=3,
                num_ref=4, n_tokens=4096, dtype="f32", top_p=0.95, steps=8, appends=False,
                plant_min=3, plant_max=3, noise=False)
DEEP = Workload("deep", 1, head_dim=128, num_kv_heads=4, num_q_heads=32, block=4, levels=6,
                num_ref=16, n_tokens=262_144, dtype="bf16", top_p=0.95, steps=256)
WIDE = Workload("wide", 2, head_dim=128, num_kv_heads=4, num_q_heads=32, block=256, levels=1,
                num_ref=16, n_tokens=262_144, dtype="bf16", top_p=0.95, steps=256)
LIGHT_SIZES = (32_768, 65_536, 131_072, 524_288, 1_048_576)


def light(n_tokens: int, steps: int = 128) -> Workload:
    return Workload(f"light_{n_tokens}", 3, head_dim=128, num_kv_heads=4, num_q_heads=32, block=8,
                    levels=light_levels(n_tokens), num_ref=1, n_tokens=n_tokens, dtype="bf16",
                    top_p=0.75, steps=steps)


ULTRA = Workload("ultra", 4, head_dim=128, num_kv_heads=4, num_q_heads=32, block=8, levels=7,
                 num_ref=1, n_tokens=16_777_216, dtype="bf16", top_p=0.75, steps=128,
                 plant_max=64)

NAMED = {"tiny": TINY, "deep": DEEP, "wide": WIDE, "ultra": ULTRA,
         **{f"light_{n}": light(n) for n in LIGHT_SIZES}}


"""The five link workloads, as shapes and request structure only.

Each entry describes one synthetic link job: the attention-layer shape, the
chunk/prefix/suffix structure of every request, how chunk ids are drawn from a
shared pool, and the value distributions of the seeded inputs. Nothing here
computes any part of the link step.

Sources for the structure: EPIC (atlas.scime.ai summary, "Approach": chunks are
compiled independently and the first k <= 32 tokens of each are recomputed;
"Key results": LegoLink-2 and LegoLink-16, 512-token chunks, ~50k-token
context) and MEPIC (searcharxiv.org abstract: page-aligned chunk KV,
first-block recompute, shared remaining blocks).
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class LinkConfig:
    name: str
    description: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str                  # "f32" or "bf16": storage and tile precision
    rope_theta: float
    page_size: int
    k: int                      # recomputed leading rows per chunk (token mode)
    block_level: bool           # recompute the whole first page of each chunk
    prefix_len: int             # 0 = no prefix segment
    chunk_len: int
    chunks_per_request: int
    suffix_len: int
    n_requests: int
    pool_size: int              # number of distinct chunks in the store
    pool_draw: str              # "sequential" | "uniform" | "zipf"
    zipf_s: float = 0.0
    q_scale: float = 1.0        # q ~ q_scale * N(0, 1)
    kv_scale: float = 1.0       # cached and new K, V ~ kv_scale * N(0, 1)
    seed: int = 0
    pos_offset: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def prefix_id(self, request: int) -> int:
        """Store id of a request's prefix segment (distinct from every pool id)."""
        return (1 << 40) + request


LLAMA3_8B_LAYER = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
                       rope_theta=5e5, page_size=16, q_scale=1.0, kv_scale=0.5)

CONFIGS: dict[str, LinkConfig] = {
    "tiny": LinkConfig(
        name="tiny",
        description="1 layer, 4 q / 2 kv heads, head_dim 64, fp32, theta 1e4; "
                    "16-token prefix + 4 x 64-token chunks + 16-token suffix, k=2",
        num_q_heads=4, num_kv_heads=2, head_dim=64, dtype="f32", rope_theta=1e4,
        page_size=16, k=2, block_level=False, prefix_len=16, chunk_len=64,
        chunks_per_request=4, suffix_len=16, n_requests=1, pool_size=4,
        pool_draw="sequential", q_scale=1.0, kv_scale=1.0, seed=1001),
    "llama3_k2": LinkConfig(
        name="llama3_k2",
        description="Llama-3-8B-shaped layer, bf16; 32-token prefix + 10 x 512-token "
                    "chunks + 64-token suffix (5,216 tokens), k=2, batch 1",
        **LLAMA3_8B_LAYER, k=2, block_level=False, prefix_len=32, chunk_len=512,
        chunks_per_request=10, suffix_len=64, n_requests=1, pool_size=10,
        pool_draw="sequential", seed=1002),
    "batched_k16": LinkConfig(
        name="batched_k16",
        description="8 requests x 24 chunks x 512 tokens drawn uniformly from a "
                    "64-chunk pool, page 16, k=16, 128-token suffix",
        **LLAMA3_8B_LAYER, k=16, block_level=False, prefix_len=0, chunk_len=512,
        chunks_per_request=24, suffix_len=128, n_requests=8, pool_size=64,
        pool_draw="uniform", seed=1003),
    "long50k_k32": LinkConfig(
        name="long50k_k32",
        description="batch 1, 64-token prefix + 98 x 512-token chunks + 64-token "
                    "suffix (50,304 tokens), k=32",
        **LLAMA3_8B_LAYER, k=32, block_level=False, prefix_len=64, chunk_len=512,
        chunks_per_request=98, suffix_len=64, n_requests=1, pool_size=98,
        pool_draw="sequential", seed=1004),
    "block_zipf": LinkConfig(
        name="block_zipf",
        description="block-level recompute (first page of each chunk private), "
                    "64 requests x 8 chunks x 1,024 tokens from a 200-chunk pool "
                    "with Zipf(1.1) reuse, 64-token suffix",
        **LLAMA3_8B_LAYER, k=0, block_level=True, prefix_len=0, chunk_len=1024,
        chunks_per_request=8, suffix_len=64, n_requests=64, pool_size=200,
        pool_draw="zipf", zipf_s=1.1, seed=1005),
}

# Order used when the configs are listed: the small parity tier first.
CONFIG_ORDER = ["tiny", "llama3_k2", "batched_k16", "long50k_k32", "block_zipf"]


@dataclass(frozen=True)
class ModelShape:
    """Decoder layers around the link step, with seeded random weights (no trained model)."""
    name: str
    description: str
    n_layers: int
    d_ff: int
    norm_eps: float = 1e-5
    weight_seed: int = 0


# A reduced configuration the fp64 oracle runs in seconds, for parity; and the Llama-3-8B shape
# (32 layers, d_ff 14,336) that the latency figure uses (EPIC summary, "Limitations": 7-9B models).
MODEL_SHAPES: dict[str, ModelShape] = {
    "small2": ModelShape("small2", "2 layers, d_model 512 (8 q / 2 kv heads x 64), d_ff 1,024", n_layers=2,
                         d_ff=1024, weight_seed=2001),
    "llama3_8b": ModelShape("llama3_8b", "32 layers, d_model 4,096 (32 q / 8 kv heads x 128), d_ff 14,336",
                            n_layers=32, d_ff=14336, weight_seed=2002),
}

# the link workload the reduced model runs on: two requests over a shared pool, LegoLink-4
MODEL_LINK = LinkConfig(
    name="model_small",
    description="8 q / 2 kv heads, head_dim 64, bf16, theta 5e5; 2 requests of a 32-token prefix + 6 x 96-token "
                "chunks (uniform draw from 8) + 40-token suffix, k=4",
    num_q_heads=8, num_kv_heads=2, head_dim=64, dtype="bf16", rope_theta=5e5, page_size=16, k=4,
    block_level=False, prefix_len=32, chunk_len=96, chunks_per_request=6, suffix_len=40, n_requests=2,
    pool_size=8, pool_draw="uniform", q_scale=1.0, kv_scale=1.0, seed=1101)

"""The five workload shapes of the routed-attention layer.

Shapes follow the chunked video-diffusion setting of the Velox article
(sns.style, "Velox: spatial memory speeds up video world models", sections
Background and Deep analysis): a current chunk of ``T`` query tokens attends
over a KV cache holding ``C`` past chunks followed by the current one, routed
at token-block granularity ``blk``.  The article prints no shapes; the sizes
below are the five synthetic workloads this project measures (tiny, small,
mid, headline at chunk 48, stress at chunk 96).
"""
from dataclasses import dataclass, field, replace
from typing import Tuple


@dataclass(frozen=True)
class Config:
    name: str
    batch: int          # B: independent rollouts
    heads: int          # H
    head_dim: int       # d
    chunk_tokens: int   # T: query tokens = tokens per chunk
    past_chunks: int    # C: chunk index; KV tokens N = (C+1)*T
    block: int          # blk: routing block = attention tile
    top_k: int          # kept KV blocks per query block, current blocks included
    alpha: float        # modulation strength
    dtype: str          # "f32" or "bf16"
    overlap: str        # "uniform" | "beta25" | "frustum"
    uncovered_frac: float   # fraction of query blocks forced uncovered
    mean_offset_std: float  # std of the per-chunk mean offset (0 = none)
    seeds: Tuple[int, ...] = field(default=())  # one seed per batch element

    @property
    def kv_tokens(self) -> int:
        return (self.past_chunks + 1) * self.chunk_tokens

    @property
    def nq(self) -> int:
        return self.chunk_tokens // self.block

    @property
    def nk(self) -> int:
        return self.kv_tokens // self.block

    @property
    def ncur(self) -> int:
        return self.chunk_tokens // self.block

    @property
    def k_eff(self) -> int:
        return min(self.top_k, self.nk)

    @property
    def rows(self) -> int:
        return self.batch * self.heads * self.nq

    def flops_exec(self) -> int:
        """QK^T plus PV FLOPs over the executed tiles when every row keeps k_eff blocks."""
        return 4 * self.head_dim * self.chunk_tokens * self.k_eff * self.block * self.heads * self.batch

    def flops_dense(self) -> int:
        """QK^T plus PV FLOPs of dense attention over the whole KV cache."""
        return 4 * self.head_dim * self.chunk_tokens * self.kv_tokens * self.heads * self.batch

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


CONFIGS = {
    "tiny": Config("tiny", 1, 1, 64, 256, 8, 64, 12, 1.0, "f32", "uniform", 0.25, 0.0, (1,)),
    "small": Config("small", 1, 4, 64, 1024, 12, 64, 48, 2.0, "bf16", "beta25", 0.20, 0.5, (2,)),
    "mid": Config("mid", 1, 16, 128, 2048, 24, 128, 64, 2.0, "bf16", "frustum", 0.0, 0.5, (3,)),
    "headline": Config("headline", 1, 24, 128, 4096, 48, 128, 256, 2.0, "bf16", "frustum", 0.0, 0.5, (4,)),
    "stress": Config("stress", 2, 24, 128, 4096, 96, 128, 256, 2.0, "bf16", "frustum", 0.40, 0.5, (5, 1005)),
}


def get_config(name: str) -> Config:
    return CONFIGS[name]

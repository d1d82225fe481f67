"""The synthetic workloads of the fused RMSNorm+MatMul path.

Shapes and value distributions (all seed 0, one generator stream per tensor):
  X ~ N(0,1) (optionally row-scaled), g ~ 1 + 0.1 N(0,1), W ~ N(0, 1/K);
  with a low-rank adapter of rank R: A ~ N(0, 1/K) (R x K), B ~ N(0, 1/R)
  (R x N), so the adapter term has the size of the frozen product.
The pages give no shapes; these stand in for their (unnamed) benchmarks.
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str          # "f32" or "bf16": X, g, W*, Y all stored in this type
    M: int
    K: int
    N: int
    eps: float
    gated: bool
    row_scale: str | None   # None, "pick_x100" (1% of rows x100) or "loguniform"
    lora: int = 0           # adapter rank R (0: none)

    @property
    def n_weights(self) -> int:
        return 2 if self.gated else 1

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def flops(self) -> int:
        """Algorithmic flops: 2*M*N*K per contraction (the adapter: 2*M*R*(K + N))."""
        return 2 * self.M * self.N * self.K * self.n_weights + 2 * self.M * self.lora * (
            self.K + self.N)

    def algo_bytes(self) -> int:
        """Algorithmic HBM bytes: every input once and Y once."""
        return (self.M * self.K + self.K + self.n_weights * self.K * self.N
                + self.lora * (self.K + self.N) + self.M * self.N) * self.elem_bytes


WORKLOADS = {
    w.name: w for w in (
        Workload("f32_m8_k1024_n1024", "f32", 8, 1024, 1024, 1e-6, False, None),
        Workload("decode_m16_k4096_n6144", "bf16", 16, 4096, 6144, 1e-6, False, None),
        Workload("prefill_m4096_k4096_n4096", "bf16", 4096, 4096, 4096, 1e-6, False,
                 "pick_x100"),
        Workload("gated_m64_k4096_n14336", "bf16", 64, 4096, 14336, 1e-6, True, None),
        Workload("large_m8192_k8192_n28672", "bf16", 8192, 8192, 28672, 1e-5, False,
                 "loguniform"),
        # the adapter on the decode shape, so its cost over the plain call shows
        Workload("lora_m16_k4096_n6144_r16", "bf16", 16, 4096, 6144, 1e-6, False, None, 16),
    )
}

ORDER = list(WORKLOADS)


@dataclass(frozen=True)
class AttnWorkload:
    """QKNorm + attention, one query per query head: Q [BH * G, D], K and V
    [BH, S, D] (BH key/value heads, G query heads sharing each), gains [D],
    all bf16.  Q, K, V ~ N(0,1); gains ~ 1 + 0.1 N(0,1)."""
    name: str
    BH: int
    S: int
    D: int
    eps: float
    dtype: str = "bf16"
    G: int = 1

    @property
    def elem_bytes(self) -> int:
        return 2

    def flops(self) -> int:
        """Algorithmic flops: q.k and p.v, 2 * D each per key and query."""
        return 4 * self.BH * self.G * self.S * self.D

    def algo_bytes(self) -> int:
        """Every input once and O once."""
        return (2 * self.BH * self.S * self.D + 2 * self.BH * self.G * self.D + 2 * self.D) * 2


ATTN_WORKLOADS = {
    w.name: w for w in (
        # 8 sequences x 32 heads attending over a 2048-token cache, head dim 128
        AttnWorkload("attn_bh256_s2048_d128", 256, 2048, 128, 1e-6),
        # the same 256 query heads with grouped-query caches: 8 query heads per
        # key/value head (32 key/value heads)
        AttnWorkload("attn_gqa_bh32_g8_s2048_d128", 32, 2048, 128, 1e-6, G=8),
    )
}


def get_workload(name: str):
    return WORKLOADS[name] if name in WORKLOADS else ATTN_WORKLOADS[name]

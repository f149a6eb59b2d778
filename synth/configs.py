"""The named attention workloads: shapes, storage dtype, input scale and seed.

Each workload is non-causal self-attention with Q, K, V of shape [B, H, N, d],
entries drawn iid N(0, 1) (times ``mult``) and rounded to ``dtype``, and
softmax scale 1/sqrt(d).  Seeds follow the workload number.
"""
from __future__ import annotations

import math
from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str
    mult: float
    seed: int
    about: str

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def flops(self) -> int:
        # two N x N x d contractions per (b, h), two flops per multiply-add
        return 4 * self.B * self.H * self.N * self.N * self.d

    @property
    def rows(self) -> int:
        return self.B * self.H * self.N

    def short(self) -> str:
        return f"{self.dtype} B{self.B} H{self.H} N{self.N} d{self.d}" + (
            f" x{self.mult:g}" if self.mult != 1.0 else "")


WORKLOADS = {
    "c1": Workload("c1", 1, 1, 128, 64, "f32", 1.0, 1, "tiny fp32"),
    "c2": Workload("c2", 8, 12, 2048, 128, "f16", 1.0, 2, "fp16 d128"),
    "c3": Workload("c3", 8, 32, 4096, 128, "bf16", 1.0, 3, "bf16 headline shape"),
    "c4": Workload("c4", 16, 16, 4096, 64, "f16", 1.0, 4, "fp16 d64"),
    "c5": Workload("c5", 1, 16, 16384, 128, "bf16", 3.0, 5, "long-sequence bf16, inputs x3"),
}

# Extra workloads taken from the pages' own test recipes (small; parity only).
PAGE_WORKLOADS = {
    # fp16 [2, 4, 512, 64] randn test of the Triton tutorial's correctness section
    "p_randn_2x4x512x64": Workload("p_randn_2x4x512x64", 2, 4, 512, 64, "f16", 1.0, 11,
                                   "tutorial correctness recipe"),
    # N = 64, d = 64 smallest element-wise debug size recommended by the tutorial
    "p_n64_d64": Workload("p_n64_d64", 1, 2, 64, 64, "f16", 1.0, 12, "tutorial N=64 D=64 debug size"),
}

# Head-size variant of the headline shape: d = 256 with the same B*H*N^2*d (equal flops
# and equal tensor bytes), so its throughput compares directly with c3.
HEADDIM_WORKLOADS = {
    "d256": Workload("d256", 4, 32, 4096, 256, "bf16", 1.0, 6, "bf16 d256, c3's flops and bytes"),
}

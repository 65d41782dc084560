"""The workloads as data: the fill shapes and the calibration shape.

Each fill workload names a model shape (hidden size d, L layers, split S, KV heads and
head size), a prompt (N rows, tail T) and how its exact prefix rows are drawn.  Sizes
follow the English RidgeFill review (jaehun.me), section "Two numbers set the skip
range" (split / layer / tail settings of the reference study and of the 27B
deployment) and "Ridge map ..." (d = 4096 for the reference models, 5120 for 27B,
lambda per model).
"""

from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class FillConfig:
    name: str
    d: int
    L: int
    S: int
    n_kv: int
    head_dim: int
    N: int
    T: int
    exact: str            # "count": exact_count rows uniform from the prefix
                          # "none": no exact prefix rows
                          # "blocks": seeded contiguous blocks plus singletons
    exact_count: int
    lam: float
    page_size: int
    seed: int
    calib_rows: int       # rows of synthetic calibration data a map fit may use
    rope_theta: float = 500000.0
    rms_eps: float = 1e-5
    d_in: int = 0         # width of x_S (0: d)

    @property
    def width(self) -> int:
        return self.d_in or self.d

    @property
    def n_upper(self) -> int:
        return self.L - self.S

    @property
    def prefix(self) -> int:
        return self.N - self.T

    @property
    def n_filled(self) -> int:
        return self.prefix - self.exact_count

    @property
    def kv(self) -> int:
        return self.n_kv * self.head_dim

    def fill_flops(self) -> float:
        """Algorithmic multiply-add work of the fill: per filled row and upper layer,
        the d x d map plus the two kv x d projections, 2 flops per multiply-add."""
        per = 2.0 * (self.d * self.width + 2 * self.kv * self.d)
        return per * self.n_filled * self.n_upper


@dataclass(frozen=True)
class CalibConfig:
    name: str
    d: int
    n_layers: int
    rows: int
    chunk: int
    lambdas: tuple = field(default=(1e-4, 1e-3, 0.01, 0.03, 0.1, 1.0))
    noise_scale: float = 0.1
    noise_dof: float = 3.0     # heavy-tailed noise: Student-t with 3 degrees of freedom
    seed: int = 1005

    def accumulate_flops(self) -> float:
        """Gram (lower triangle) plus one cross moment per layer: 2 n (d(d+1)/2 + U d^2)."""
        d = self.d
        return 2.0 * self.rows * (d * (d + 1) / 2 + self.n_layers * d * d)


TINY = FillConfig("tiny", d=256, L=8, S=4, n_kv=2, head_dim=64, N=12, T=3,
                  exact="count", exact_count=2, lam=0.03, page_size=4, seed=1001,
                  calib_rows=2048)

LLAMA8B = FillConfig("llama3.1-8b", d=4096, L=32, S=12, n_kv=8, head_dim=128,
                     N=32768, T=4096, exact="count", exact_count=2867, lam=0.03,
                     page_size=16, seed=1002, calib_rows=8192)

QWEN3_8B = FillConfig("qwen3-8b", d=4096, L=36, S=13, n_kv=8, head_dim=128,
                      N=16384, T=4096, exact="none", exact_count=0, lam=0.01,
                      page_size=16, seed=1003, calib_rows=8192)

QWEN27B = FillConfig("27b-long", d=5120, L=64, S=16, n_kv=8, head_dim=128,
                     N=65536, T=4096, exact="blocks", exact_count=3072, lam=0.03,
                     page_size=16, seed=1004, calib_rows=8192)

# Generic rectangular-map workload: the 8B prompt and layers with a split-layer state twice
# as wide as the layers (d_in = 2 d).
WIDE8B = FillConfig("8b-shape-wide-split", d=4096, L=32, S=12, n_kv=8, head_dim=128,
                    N=32768, T=4096, exact="count", exact_count=2867, lam=0.03,
                    page_size=16, seed=1006, calib_rows=8192, d_in=8192)

CALIB8B = CalibConfig("calib-8b", d=4096, n_layers=20, rows=131072, chunk=16384)

FILL_CONFIGS = {c.name: c for c in (TINY, LLAMA8B, QWEN3_8B, QWEN27B)}

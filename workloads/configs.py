"""The five benchmark workloads of the Muon step, as shapes and recipes.

Shapes are rows x cols = fan_out x fan_in of the weight.  A `MatrixSpec`
with `batch > 1` is a stacked bank of equal-shape matrices, contiguous in
memory (batch, rows, cols); `split_rows > 0` splits every matrix into
row-blocks that are orthogonalised separately (per-head split).
"""

from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class MatrixSpec:
    name: str
    rows: int
    cols: int
    batch: int = 1
    split_rows: int = 0
    grad_dtype: str = "bf16"  # "bf16" or "fp32"

    @property
    def units_per_matrix(self) -> int:
        return self.rows // self.split_rows if self.split_rows else 1

    @property
    def unit_shape(self) -> tuple[int, int]:
        return (self.split_rows or self.rows, self.cols)

    @property
    def numel(self) -> int:
        return self.batch * self.rows * self.cols


@dataclass(frozen=True)
class Workload:
    cfg: int
    title: str
    matrices: tuple[MatrixSpec, ...]
    steps: int
    scale: str  # "spectral" or "unit_rms_norm"
    grad_dist: str  # "normal", "student_t3", "normal_logscale"
    grad_std: float
    ns_paths: tuple[str, ...]  # which NS precisions the workload runs
    zero_fraction: float = 0.0  # fraction of experts with all-zero grads
    w_std: float = 0.02
    extra: dict = field(default_factory=dict)

    @property
    def units(self) -> int:
        return sum(m.batch * m.units_per_matrix for m in self.matrices)

    @property
    def params(self) -> int:
        return sum(m.numel for m in self.matrices)

    def ns_flops(self) -> float:
        """Nominal Newton-Schulz FLOPs of one step over every unit:
        10 iterations of Gram (2 s^2 l) + polynomial square (2 s^3) +
        apply (2 s^2 l), with s the smaller and l the larger unit side."""
        tot = 0.0
        for m in self.matrices:
            r, c = m.unit_shape
            s, l = min(r, c), max(r, c)
            tot += m.batch * m.units_per_matrix * 10 * (4.0 * s * s * l + 2.0 * s**3)
        return tot


def _layer(prefix: str = "", n_layers: int = 1) -> tuple[MatrixSpec, ...]:
    """One transformer layer at hidden 4096: fused QKV of 32 query + 8 key
    + 8 value heads of 128 rows each, split per head; output projection;
    MLP gate and up (14336 x 4096) and down (4096 x 14336)."""
    b = n_layers
    return (
        MatrixSpec(prefix + "qkv", 48 * 128, 4096, batch=b, split_rows=128),
        MatrixSpec(prefix + "o_proj", 4096, 4096, batch=b),
        MatrixSpec(prefix + "gate", 14336, 4096, batch=b),
        MatrixSpec(prefix + "up", 14336, 4096, batch=b),
        MatrixSpec(prefix + "down", 4096, 14336, batch=b),
    )


CONFIGS: dict[int, Workload] = {
    1: Workload(
        1,
        "single fp32 matrix 64x128, 5 steps",
        (MatrixSpec("w", 64, 128, grad_dtype="fp32"),),
        steps=5,
        scale="spectral",
        grad_dist="normal",
        grad_std=1.0,
        ns_paths=("fp32", "bf16"),
    ),
    2: Workload(
        2,
        "32 stacked 1024x1024, bf16 grads, 10 steps",
        (MatrixSpec("stack", 1024, 1024, batch=32),),
        steps=10,
        scale="spectral",
        grad_dist="normal",
        grad_std=1e-3,
        ns_paths=("bf16", "fp32"),
    ),
    3: Workload(
        3,
        "one hidden-4096 transformer layer, per-head QKV split",
        _layer(),
        steps=3,
        scale="spectral",
        grad_dist="student_t3",
        grad_std=1e-3,
        ns_paths=("bf16",),
    ),
    4: Workload(
        4,
        "MoE bank: 128 experts x {gate, up 2048x7168, down 7168x2048}",
        (
            MatrixSpec("gate", 2048, 7168, batch=128),
            MatrixSpec("up", 2048, 7168, batch=128),
            MatrixSpec("down", 7168, 2048, batch=128),
        ),
        steps=3,
        scale="spectral",
        grad_dist="normal",
        grad_std=1e-3,
        ns_paths=("bf16",),
        zero_fraction=0.1,
    ),
    5: Workload(
        5,
        "32 transformer layers (~7B params), unit_rms_norm scale",
        _layer(n_layers=32),
        steps=3,
        scale="unit_rms_norm",
        grad_dist="normal_logscale",
        grad_std=1e-3,
        ns_paths=("bf16", "fp32"),
    ),
}


def workload(cfg: int) -> Workload:
    return CONFIGS[cfg]

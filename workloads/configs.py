"""The five workload configurations of the SLA / SLA2 forward pass.

Shapes follow the video models the pages evaluate on: the Wan2.1-1.3B latent grid
of 21x30x52 tokens (SLA paper summary, section 5 "Datasets"; SLA2 article, the
1.3B timing paragraph) and the Wan2.1-14B-720P grid of 21x45x80 tokens. Head
dim 128, 64-token blocks (SLA explainer, section 2.2 item 1), kh = 5% and
kl = 10% (SLA explainer, section 3.2 deployment advice) or the 97%-sparse SLA2
setting kh = 3%.
"""

from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class WorkloadConfig:
    cid: int
    name: str
    B: int
    H: int
    N: int
    d: int
    grid: Optional[Tuple[int, int, int]]  # (t, h, w) latent grid, raster order, w fastest
    dtype: str                            # "f32" or "bf16": dtype of Q, K, V and O
    kh: float                             # critical fraction per query-block row
    kl: float                             # negligible fraction per query-block row
    router: str                           # "identity" or "learned" (I + 0.1 N(0, 1/d))
    alpha: Tuple                          # ("const", a) or ("uniform", lo, hi), per head
    quant: bool                           # 8-bit sparse branch
    seed: int
    qk: str = "posemb"                    # "normal" or "posemb"
    desc: str = field(default="", compare=False)

    @property
    def Nb(self) -> int:
        return (self.N + 63) // 64

    @property
    def dense_flops(self) -> float:
        """4*B*H*N^2*d: the two N x N x d products of dense attention, 2mnk each."""
        return 4.0 * self.B * self.H * self.N * self.N * self.d


CONFIGS = {
    1: WorkloadConfig(1, "tiny_f32", 1, 2, 1024, 64, None, "f32", 0.25, 0.25,
                      "identity", ("const", 0.5), False, 1001, qk="normal",
                      desc="tiny fp32: B=1 H=2 N=1024 d=64, N(0,1) Q/K/V, identity router"),
    2: WorkloadConfig(2, "mid_bf16", 1, 12, 8192, 128, (4, 32, 64), "bf16", 0.05, 0.10,
                      "learned", ("uniform", 0.2, 0.8), False, 1002,
                      desc="mid bf16: B=1 H=12 N=8192 on a 4x32x64 grid"),
    3: WorkloadConfig(3, "wan13b_sla95", 1, 12, 32760, 128, (21, 30, 52), "bf16", 0.05, 0.10,
                      "identity", ("const", 0.5), False, 1003,
                      desc="Wan2.1-1.3B shape, SLA at 95% sparsity"),
    4: WorkloadConfig(4, "wan13b_sla2_97_cfg", 2, 12, 32760, 128, (21, 30, 52), "bf16", 0.03, 0.10,
                      "learned", ("uniform", 0.0, 1.0), False, 1004,
                      desc="Wan2.1-1.3B shape, SLA2 at 97% sparsity, CFG batch of 2"),
    5: WorkloadConfig(5, "wan14b720p_sla2_97_lowbit", 1, 40, 75600, 128, (21, 45, 80), "bf16",
                      0.03, 0.10, "learned", ("uniform", 0.2, 0.8), True, 1005,
                      desc="Wan2.1-14B-720P shape, SLA2 at 97% with an 8-bit sparse branch"),
}


def get_config(cid: int) -> WorkloadConfig:
    return CONFIGS[int(cid)]

"""The five synthetic workloads, as plain sizes.

Shapes follow the pages' setting: EP=8 at a router-imbalance sweep of maxvio 0.2 to 20
("Moonshot AI Open-Sources MoonEP", paragraph 4), DeepSeek-V3 / Kimi style 384 or 256
experts routed to eight ("Load Balancing in MoE: Stopping Experts Going Idle",
introduction), and a training slot budget of E/R per rank versus 3-4 slots for inference
("Moonshot AI Open-Sources MoonEP", paragraph 5).

Nothing here computes any part of the method; it only names sizes and seeds.
"""

from dataclasses import dataclass, field
from typing import Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    R: int          # simulated expert-parallel ranks (HBM partitions of one GPU)
    E: int          # experts
    K: int          # top-K
    S: int          # tokens per rank
    H: int          # hidden size (bf16 elements)
    slots: int      # prefetch (replica) slots per rank
    maxvio: Tuple[float, ...] = field(default=(1.0,))
    grad_cols: int = 0   # replica-gradient slab is H x grad_cols fp32 per expert (0: none)
    index: int = 0       # position in the workload list, used in seeds

    @property
    def T(self):
        return self.R * self.S

    @property
    def A(self):
        return self.T * self.K

    @property
    def G_el(self):
        return self.H * self.grad_cols

    def seed(self, maxvio_index: int) -> int:
        return 20260000 + 100 * (self.index + 1) + maxvio_index


TINY = Workload("tiny", R=4, E=16, K=2, S=64, H=128, slots=4, maxvio=(2.0,), index=0)
SMALL = Workload("r8-e64-k6", R=8, E=64, K=6, S=1024, H=2048, slots=8, maxvio=(0.2,), index=1)
DSV3 = Workload("dsv3", R=8, E=256, K=8, S=4096, H=7168, slots=32,
                maxvio=(0.2, 1.0, 5.0, 20.0), index=2)
KIMI = Workload("kimi", R=16, E=384, K=8, S=8192, H=7168, slots=24, maxvio=(20.0,),
                grad_cols=512, index=3)
DECODE = Workload("decode", R=64, E=384, K=8, S=128, H=7168, slots=4, maxvio=(1.0, 20.0),
                  index=4)

WORKLOADS = (TINY, SMALL, DSV3, KIMI, DECODE)
BY_NAME = {w.name: w for w in WORKLOADS}

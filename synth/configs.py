"""The five synthetic workloads: shapes, value distributions and seeds.

Shapes follow the model families the pages evaluate on (a 7B multi-head model,
an 8B grouped-query model, a 9B-class pool model).  Their benchmark's prompts
are not available and are not reconstructed; seeded synthetic inputs with the
stated length mixes stand in for them.
"""
from dataclasses import dataclass
from typing import Optional, Tuple

F32, F16, BF16 = 0, 1, 2
ESIZE = {F32: 4, F16: 2, BF16: 2}
DTYPE_NAME = {F32: "f32", F16: "f16", BF16: "bf16"}


@dataclass(frozen=True)
class Config:
    name: str
    seed: int
    B: int                 # rows verified per round (pool size for the pool workload)
    D: int                 # draft length
    V: int                 # vocabulary
    logit_dtype: int
    sigma: float           # std of the logit draws
    plan_mode: int         # 0: independent per-position match, 1: geometric first mismatch
    plan_p: float          # match probability (mode 0) or mismatch probability (mode 1)
    L: int
    H: int
    Dh: int
    kv_dtype: int
    len_lo: int
    len_hi: int
    cap: int
    rounds: int
    fixed_lens: Optional[Tuple[int, ...]] = None
    pool_values: int = 0   # pool workload: number of distinct lengths
    group: int = 0         # pool workload: rows per batch
    temperature: float = 0.0   # sampled workload
    draft_noise: float = 0.0   # sampled workload: std of draft-logit noise
    tie_frac: float = 0.125    # fraction of logit rows with exact ties at the maximum

    @property
    def D1(self):
        return self.D + 1

    @property
    def plant_value(self):
        # above every normal draw (|z| < 6 sigma), exactly representable in bf16/fp16
        return 8.0 * self.sigma

    @property
    def kv_pos_bytes(self):
        """KV bytes of one token position of one row over all layers, K and V."""
        return self.L * 2 * self.H * self.Dh * ESIZE[self.kv_dtype]


CONFIGS = {
    "tiny": Config("tiny", seed=1, B=2, D=4, V=1000, logit_dtype=F32, sigma=1.0, plan_mode=0, plan_p=0.7,
                   L=2, H=2, Dh=16, kv_dtype=F32, len_lo=5, len_hi=9, cap=32, rounds=1, fixed_lens=(5, 9),
                   tie_frac=0.25),
    "7b-mha": Config("7b-mha", seed=2, B=8, D=4, V=32000, logit_dtype=F32, sigma=2.0, plan_mode=1, plan_p=0.3,
                     L=32, H=32, Dh=128, kv_dtype=F16, len_lo=128, len_hi=1024, cap=1024 + 64 * 5, rounds=64),
    "8b-gqa": Config("8b-gqa", seed=3, B=16, D=5, V=151936, logit_dtype=BF16, sigma=2.0, plan_mode=1, plan_p=0.25,
                     L=36, H=8, Dh=128, kv_dtype=BF16, len_lo=256, len_hi=2048, cap=2048 + 64 * 6, rounds=64),
    "exspec": Config("exspec", seed=4, B=256, D=4, V=151552, logit_dtype=BF16, sigma=2.0, plan_mode=1, plan_p=0.3,
                     L=40, H=2, Dh=128, kv_dtype=BF16, len_lo=512, len_hi=4096, cap=4096 + 32 * 5, rounds=32,
                     pool_values=16, group=8),
    "stoch": Config("stoch", seed=5, B=32, D=8, V=32000, logit_dtype=F32, sigma=2.0, plan_mode=-1, plan_p=0.0,
                    L=32, H=32, Dh=128, kv_dtype=F16, len_lo=64, len_hi=2048, cap=2048 + 9, rounds=1,
                    temperature=0.8, draft_noise=0.5),
}

"""The five synthetic workloads of the verification step.

1  toy sampler: V=5, fixed p and q, gamma=1, 200,000 independent trials
   ([P3] section 受理・棄却の規則と出力分布が変わらない理由, the V=5 toy).
2  char-model sampler: B=64, gamma=4, V=96 fp32 (the vocabulary of the numpy
   char model of [P2] section numpyで小さなTransformerを自作する).
3  verify step at the numpy model's shape: B=64, 4 heads, head dim 24, fp32,
   384-token cached prefix ([P2] section プリフィルとデコードの速さの違い),
   gamma+1 = 5 query rows, cache capacity 512 (the model's T), then config 2's
   sampler.
4  LLM-scale verify, one layer: B=32, gamma=4, GQA 32/8, head dim 128, bf16,
   lengths uniform in [1024, 4096]; sampler over V=151,936 (Qwen3's vocabulary
   size quoted in [P3] section vLLMのspeculative-configによる方式と提案数の設定).
5  long context, large batch, one layer: B=256, gamma=8, GQA 64/8, head dim
   128, bf16, lengths uniform in [8192, 32768]; sampler over V=128,256 at
   temperatures 0.7 and 1.0.
"""

from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class Config:
    cid: int
    name: str
    B: int
    gamma: int
    V: int
    dtype: str  # "f32", "bf16" or "f16" (attention only): logits and K/V/Q element type
    temperatures: Tuple[float, ...] = (1.0,)
    # sampler logits: z_t = t_std * N(0,1); z_d = mix * z_t + noise_std * N(0,1)
    t_std: float = 1.0
    mix: float = 1.0
    noise_std: float = 1.0
    # toy distributions (config 1 only)
    p: Optional[Tuple[float, ...]] = None
    q: Optional[Tuple[float, ...]] = None
    # attention (configs 3-5)
    Hq: int = 0
    Hkv: int = 0
    D: int = 0
    L: Tuple[int, int] = (0, 0)  # inclusive range of committed lengths
    max_T: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def n_q(self) -> int:
        return self.gamma + 1

    @property
    def has_attention(self) -> bool:
        return self.Hq > 0

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


def _round_up(x, m):
    return (x + m - 1) // m * m


CONFIGS = {
    1: Config(
        1, "toy-v5", B=200_000, gamma=1, V=5, dtype="f32",
        p=(0.40, 0.25, 0.15, 0.12, 0.08), q=(0.20, 0.40, 0.20, 0.10, 0.10),
    ),
    2: Config(2, "char-sampler", B=64, gamma=4, V=96, dtype="f32", t_std=2.0, mix=1.0, noise_std=1.0),
    3: Config(
        3, "char-verify", B=64, gamma=4, V=96, dtype="f32", t_std=2.0, mix=1.0, noise_std=1.0,
        Hq=4, Hkv=4, D=24, L=(384, 384), max_T=512,
    ),
    4: Config(
        4, "llm-verify", B=32, gamma=4, V=151_936, dtype="bf16", t_std=3.0, mix=0.8, noise_std=1.0,
        Hq=32, Hkv=8, D=128, L=(1024, 4096), max_T=_round_up(4096 + 5, 64),
    ),
    5: Config(
        5, "long-context", B=256, gamma=8, V=128_256, dtype="bf16", temperatures=(0.7, 1.0),
        t_std=3.0, mix=0.8, noise_std=1.0,
        Hq=64, Hkv=8, D=128, L=(8192, 32768), max_T=_round_up(32768 + 9, 64),
    ),
}


def get(cid: int) -> Config:
    return CONFIGS[int(cid)]

"""The five workload shapes the path is measured and checked on."""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int        # tokens
    H: int        # hidden size (bf16 elements per row)
    K: int        # experts per token (top-k)
    E: int        # experts
    S: int        # symmetric slots (stand-ins for ranks)
    I: int        # SwiGLU intermediate size; 0 = identity experts
    routing: str  # routing generator, see synth.gen.routing
    seed: int = 0
    weight_std: float = 0.02

    @property
    def eps(self) -> int:
        return self.E // self.S

    @property
    def cap(self) -> int:
        """Rows per slot the heap must hold (every token may send min(K, E/S)
        distinct-expert rows to one slot)."""
        return self.T * min(self.K, self.eps)

    def with_(self, **kw) -> "MoEConfig":
        return replace(self, **kw)


CONFIGS = {
    # small case: 8 experts over 4 slots, top-2 of softmax(N(0,1) logits)
    "tiny": MoEConfig("tiny", T=128, H=256, K=2, E=8, S=4, I=512, routing="softmax_topk"),
    # Mixtral-shaped: 8 experts, one per slot, near-uniform top-2
    "mixtral": MoEConfig("mixtral", T=4096, H=4096, K=2, E=8, S=8, I=14336,
                         routing="softmax_topk"),
    # dispatch/combine only: identity experts, Zipf(1.2) expert popularity
    "zipf": MoEConfig("zipf", T=16384, H=7168, K=8, E=256, S=8, I=0, routing="zipf"),
    # DeepSeek-V3-shaped: 256 experts over 8 slots, top-8 of biased logits,
    # sigmoid weights normalised over the selected experts
    "dsv3": MoEConfig("dsv3", T=8192, H=7168, K=8, E=256, S=8, I=2048,
                      routing="biased_sigmoid"),
    # decode-shaped: few rows per expert
    "decode": MoEConfig("decode", T=256, H=7168, K=8, E=256, S=8, I=2048,
                        routing="softmax_selected"),
}


def get_config(name: str, **overrides) -> MoEConfig:
    cfg = CONFIGS[name]
    return cfg.with_(**overrides) if overrides else cfg

"""The layer shapes the hot path is measured and checked on.

Model shapes follow the expert matrix sizes the Specter paper names for
fine-grained MoE models (2048x1408 and 4096x6400 expert matrices, in the
paragraph on Marlin and narrow expert GEMMs) and its speculation depths
(K=16 for DeepSeekV2-Lite and Phi-3.5-MoE, K=8 for Qwen1.5-MoE, in the
paragraph on selecting K). The window holds the K candidates plus the
uncached corrected/bonus token (Specter paper, State Manager paragraph), so
T = K + 1. The batched shape follows the batched-execution paragraph
(B up to 32 requests). The single-token step (dsv2_t1) is one call of the
autoregressive draft that proposes those K tokens (Specter paper, the
speculative-decoding paragraphs), and is the latency-bound end of the range.
"""

from dataclasses import dataclass, field


@dataclass(frozen=True)
class MoEConfig:
    name: str
    E: int                 # routed experts
    k: int                 # experts per token (top-k)
    H: int                 # hidden size
    I: int                 # routed expert intermediate size
    G: int                 # INT4 quantisation group size along the reduction dim
    T: int                 # tokens per layer call (K + 1, or B * (K + 1) batched)
    shared_I: int = 0      # always-on FP16 shared expert(s), concatenated intermediate size
    shared_gate: bool = False   # sigmoid gate on the shared expert output
    layers: int = 1
    zipf_s: float = 0.0    # per-expert Zipf(s) log-prior added to router logits
    elb_M: int = 0         # top-M of the activation counter snapshot (0 = none)
    target_fp16: bool = False   # also run the FP16-weight target verification pass
    description: str = field(default="", compare=False)

    @property
    def S(self) -> int:
        """Routed (token, expert) slots per layer."""
        return self.T * self.k


CONFIGS = {
    "tiny": MoEConfig(
        name="tiny", E=8, k=2, H=256, I=512, G=64, T=17,
        description="8 experts, top-2, hidden 256, intermediate 512, 17 tokens, INT4 g64"),
    "dsv2": MoEConfig(
        name="dsv2", E=64, k=6, H=2048, I=1408, G=128, T=17,
        shared_I=2 * 1408, elb_M=32,
        description="DeepSeek-V2-Lite-shaped draft layer: 64 experts, softmax top-6, "
                    "hidden 2048, intermediate 1408, 2 FP16 shared experts, K=16 window "
                    "(17 tokens), INT4 g128, activation counter top-32"),
    "qwen": MoEConfig(
        name="qwen", E=60, k=4, H=2048, I=1408, G=128, T=9,
        shared_I=5632, shared_gate=True,
        description="Qwen1.5-MoE-shaped draft layer: 60 experts, top-4, hidden 2048, "
                    "intermediate 1408, FP16 shared expert 5632 with sigmoid gate, "
                    "K=8 window (9 tokens), INT4 g128"),
    "phi": MoEConfig(
        name="phi", E=16, k=2, H=4096, I=6400, G=128, T=17,
        target_fp16=True,
        description="Phi-3.5-MoE-shaped layer: 16 experts, top-2, hidden 4096, "
                    "intermediate 6400, 17 tokens; INT4 g128 draft pass and FP16 "
                    "target verification pass on the same tokens"),
    "dsv2_t1": MoEConfig(
        name="dsv2_t1", E=64, k=6, H=2048, I=1408, G=128, T=1,
        shared_I=2 * 1408, elb_M=32,
        description="DeepSeek-V2-Lite-shaped single-token draft step: the dsv2 layer at "
                    "T=1, one autoregressive draft token"),
    "batch": MoEConfig(
        name="batch", E=64, k=6, H=2048, I=1408, G=128, T=32 * 17,
        shared_I=2 * 1408, layers=26, zipf_s=1.1, elb_M=32,
        description="Batched DeepSeek-V2-Lite-shaped stack: 26 layers, 32 requests x "
                    "17 tokens = 544 tokens per layer, Zipf(1.1) router skew, "
                    "activation counter top-32 across all layers"),
}


def get_config(name: str) -> MoEConfig:
    try:
        return CONFIGS[name]
    except KeyError:
        raise KeyError(f"unknown config {name!r}; known: {sorted(CONFIGS)}") from None

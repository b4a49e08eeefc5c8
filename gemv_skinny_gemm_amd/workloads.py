"""Linear shapes of the Qwen2.5-72B decode step, as synthetic workloads.

The model has 80 decoder layers and hidden size 8192 ("Developing a custom
Qwen2.5 72B inference engine from scratch", section 1).  Each layer's linears
(y = x . W^T, W stored [N][K]) at tensor-parallel degree 1 and at the per-GPU
shard of degree 8 are:

    TP=1: QKV 10240 x 8192, O 8192 x 8192, gate_up 59136 x 8192, down 8192 x 29568
    TP=8: QKV  1280 x 8192, O 8192 x 1024, gate_up  7392 x 8192, down 8192 x  3696

Every tensor gets its own Philox stream, so a tensor (or any row of it) can be
regenerated anywhere: weights ~ N(0, 0.02) rounded to bf16 (FP8 weights are
those values block-quantized), activations ~ N(0, 1) rounded to bf16.
"""
from __future__ import annotations

from dataclasses import dataclass

from gemv_skinny_gemm_amd.synth import stream_id

BF16 = 0
FP8_BS128 = 1
W_SIGMA = 0.02
X_SIGMA = 1.0
LAYERS = 80

TP1_SHAPES = (("qkv", 10240, 8192), ("o", 8192, 8192), ("gate_up", 59136, 8192),
              ("down", 8192, 29568))
TP8_SHAPES = (("qkv", 1280, 8192), ("o", 8192, 1024), ("gate_up", 7392, 8192),
              ("down", 8192, 3696))


@dataclass(frozen=True)
class LinearSpec:
    name: str
    N: int
    K: int
    dtype: int
    w_stream: int
    x_stream: int

    def weight_bytes(self) -> int:
        return self.N * self.K * (2 if self.dtype == BF16 else 1)

    def scale_bytes(self) -> int:
        if self.dtype == BF16:
            return 0
        return ((self.N + 127) // 128) * ((self.K + 127) // 128) * 4

    def algorithmic_bytes(self, M: int) -> int:
        """W + block scales + x + y, each counted once."""
        return self.weight_bytes() + self.scale_bytes() + 2 * M * self.K + 2 * M * self.N

    def flops(self, M: int) -> int:
        return 2 * M * self.N * self.K


def _spec(tag, layer, name, N, K, dtype):
    return LinearSpec(f"{tag}.L{layer}.{name}" if layer is not None else f"{tag}.{name}", N, K,
                      dtype, stream_id("qwen2.5-72b", tag, layer, name, "w"),
                      stream_id("qwen2.5-72b", tag, layer, name, "x"))


def qkv_tp8_gemv() -> list[LinearSpec]:
    """The TP=8 QKV shard as a single GEMV: W 1280 x 8192 bf16."""
    return [_spec("gemv", None, "qkv", 1280, 8192, BF16)]


def tp8_layer(dtype: int = BF16) -> list[LinearSpec]:
    """One decoder layer's TP=8-shard linears."""
    return [_spec("tp8", 0, n, N, K, dtype) for n, N, K in TP8_SHAPES]


def tp1_stack(dtype: int = BF16, layers: int = LAYERS) -> list[LinearSpec]:
    """The TP=1 decode linear stack: layers x (QKV, O, gate_up, down), distinct weights."""
    tag = "tp1" if dtype == BF16 else "tp1fp8"
    return [_spec(tag, l, n, N, K, dtype) for l in range(layers) for n, N, K in TP1_SHAPES]


# The page gives the vocabulary as ~152k; 152,064 (a multiple of 128, so the
# FP8 scale blocks tile it) is taken as the concrete size.
VOCAB = 152064
HIDDEN = 8192


def lm_head(dtype: int = BF16) -> list[LinearSpec]:
    """The vocabulary projection after the last layer: W VOCAB x HIDDEN (the
    logits of the greedy next token)."""
    return [_spec("head", None, "lm_head", VOCAB, HIDDEN, dtype)]


def mlp(tp: int = 1, dtype: int = BF16) -> list[LinearSpec]:
    """One layer's gated MLP as [gate_up, down] (gate rows first in gate_up);
    the down linear's x is the activation of gate_up's output, not its own."""
    shapes = TP1_SHAPES if tp == 1 else TP8_SHAPES
    tag = f"mlp-tp{tp}" + ("" if dtype == BF16 else "-fp8")
    return [_spec(tag, 0, n, N, K, dtype) for n, N, K in shapes if n in ("gate_up", "down")]


def mlp_algorithmic_bytes(specs, M: int) -> int:
    """W + scales of both linears, x and y once, and the [M][2I] bf16
    intermediate written by gate_up and read by down."""
    gate_up, down = specs
    return (gate_up.weight_bytes() + gate_up.scale_bytes() + down.weight_bytes() +
            down.scale_bytes() + 2 * M * gate_up.K + 2 * M * down.N + 2 * (2 * M * gate_up.N))


def algorithmic_bytes(specs, M: int) -> int:
    return sum(s.algorithmic_bytes(M) for s in specs)


def flops(specs, M: int) -> int:
    return sum(s.flops(M) for s in specs)


# Mixture-of-experts verify step.  The pages route tokens to the top 2 of 8
# experts with hidden size 4096 and two favoured experts ("Multi-GPU Inference
# and Serving at Scale", Example 8) and verify about six draft tokens per step
# ("9% faster GLM-5.3-Flash prefill", section "TileLang: twice as fast, and no
# faster").  They give no expert width; 1536 (a small expert, 3/8 of hidden)
# is taken, a multiple of 128 so FP8 scale blocks never straddle experts.
MOE_EXPERTS = 8
MOE_TOPK = 2
MOE_HIDDEN = 4096
MOE_INTER = 1536
MOE_TOKENS = 6


def moe_experts(dtype: int = FP8_BS128) -> list[LinearSpec]:
    """[gate_up, down] of the MoE layer's experts, each as one [E * N][K]
    tensor (expert e = rows e N .. e N + N - 1, i.e. [E][N][K])."""
    tag = "moe" + ("" if dtype == BF16 else "-fp8")
    E, H, I = MOE_EXPERTS, MOE_HIDDEN, MOE_INTER
    return [_spec(tag, 0, "experts_gate_up", E * 2 * I, H, dtype),
            _spec(tag, 0, "experts_down", E * H, I, dtype)]


def moe_algorithmic_bytes(spec: LinearSpec, ids, experts: int, x_rows: int,
                          x_cols: int) -> int:
    """One MoE linear call: the chosen experts' W and scales once each, x,
    the routes' y and the ids."""
    import numpy as np
    ids = np.asarray(ids)
    chosen = len(set(int(e) for e in ids.ravel() if 0 <= e < experts))
    per_expert = (spec.weight_bytes() + spec.scale_bytes()) // experts
    routes = ids.size
    return chosen * per_expert + 2 * x_rows * x_cols + 2 * routes * (spec.N // experts) + 4 * routes

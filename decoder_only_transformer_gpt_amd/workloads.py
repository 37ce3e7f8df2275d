"""Named workloads: model shape, batch and token law of each configuration.

Shapes follow the depth dial (width 64*depth, heads width/128, head dim 128,
MLP 4x, vocab 65,536, context 2,048: aethryn.com "Nanochat: full-stack LLM
training in 8,000 lines for $72", section "One dial controls everything";
atlas.blal.pro "nanochat — full-stack ChatGPT in ~8k lines", section "How it
works") with one shared K/V head. d20 at batch 32 x 2048 is one GPU's share of
the pages' 8-GPU speedrun batch; the token streams are synthetic stand-ins for
FineWeb-EDU.
"""
from __future__ import annotations

from dataclasses import dataclass

from . import _lib


@dataclass(frozen=True)
class Workload:
    name: str
    depth: int
    model_dim: int
    mlp_dim: int
    vocab_size: int
    seq_len: int
    batch: int
    dtype: str          # "f32" | "bf16" | "fp8" (bf16 with e4m3 QKV / O / MLP products)
    tokens: str         # "uniform" | "zipf"
    window_pattern: str = ""   # sliding-window layer pattern, e.g. "SSSL"; "" = all full
    window_short: int = 0
    x0_lambdas: int = 0        # per-layer resid / x0 scalars
    value_embeds: int = 0      # value embeddings on layers 0, 2, 4, ...

    def config(self) -> _lib.gpt_config:
        dt = {"f32": _lib.GPT_F32, "bf16": _lib.GPT_BF16, "fp8": _lib.GPT_FP8_E4M3}[self.dtype]
        c = _lib.gpt_config_from_depth(self.depth, dt)
        c.model_dim = self.model_dim
        c.n_head = self.model_dim // 128
        c.mlp_dim = self.mlp_dim
        c.vocab_size = self.vocab_size
        c.max_seq_len = max(self.seq_len, 2048)
        c.window_pattern = self.window_pattern.encode()
        c.window_short = self.window_short
        c.x0_lambdas = self.x0_lambdas
        c.value_embeds = self.value_embeds
        return c


WORKLOADS = {
    "tiny": Workload("tiny", 2, 128, 512, 512, 64, 2, "f32", "uniform"),
    "d4": Workload("d4", 4, 256, 1024, 65536, 512, 4, "bf16", "uniform"),
    "d12": Workload("d12", 12, 768, 3072, 65536, 2048, 16, "bf16", "zipf"),
    "d20": Workload("d20", 20, 1280, 5120, 65536, 2048, 32, "bf16", "zipf"),
    # d20 with the pages' sliding-window pattern: SSSL, short windows of 1,024
    # tokens, the last layer full (aethryn.com, section "A Llama-class
    # transformer with ten modern departures")
    "d20-sssl": Workload("d20-sssl", 20, 1280, 5120, 65536, 2048, 32, "bf16", "zipf", "SSSL", 1024),
    # d24 with e4m3 QKV / O / MLP products (repo-explainer.com "karpathy/nanochat:
    # The $100 Full-Stack LLM", section "The Engine Room: Muon and FP8")
    "d24fp8": Workload("d24fp8", 24, 1536, 6144, 65536, 2048, 16, "fp8", "zipf"),
    # d20 with the per-layer residual scalars and value embeddings (aethryn.com,
    # section "A Llama-class transformer with ten modern departures")
    "d20-ve": Workload("d20-ve", 20, 1280, 5120, 65536, 2048, 32, "bf16", "zipf", x0_lambdas=1, value_embeds=1),
}

"""Model shapes and workloads of the decode path (pure data, no arithmetic).

The five named workloads are the synthetic stand-ins for the pages' models:
the 288-dim / 6-layer / 6-head "15M" TinyStories model and the 512-dim /
8-layer / 8-head "44M" model of openai.wiki "llama2.c | Baby LLaMA" (sections
"Environment setup" and "Training example"), the same 15M shape decoded for
many sequences at once, a 768-dim model in between, and the Llama-2-7B shape the
pages mention loading (Xinzhiyuan's llama2.c report, section "Usage").
Weights are N(0, 0.02) drawn from the seed, norm gains 1.0.
"""
from dataclasses import dataclass, field, replace
from typing import Tuple


@dataclass(frozen=True)
class ModelConfig:
    dim: int
    n_layers: int
    n_heads: int
    hidden_dim: int
    vocab_size: int = 32000
    max_seq: int = 256
    tied: bool = True
    rope_theta: float = 10000.0
    norm_eps: float = 1e-5
    max_batch: int = 1
    n_kv_heads: int = 0          # key/value heads (grouped-query attention); 0 = n_heads
    weight_bf16: bool = False    # matrices held as bfloat16 (the fp32 draw rounded to nearest)
    max_pos: int = 0             # positions the model may run through; 0 = max_seq.  Past
                                 # max_seq, attention covers the max_seq most recent positions

    @property
    def head_dim(self):
        return self.dim // self.n_heads

    @property
    def kv_heads(self):
        return self.n_kv_heads or self.n_heads

    @property
    def kv_dim(self):
        return self.kv_heads * self.head_dim

    def n_params(self):
        d, f, V, L = self.dim, self.hidden_dim, self.vocab_size, self.n_layers
        per_layer = 2 * d * d + 2 * self.kv_dim * d + 3 * d * f + 2 * d
        return V * d + L * per_layer + d + (0 if self.tied else V * d)

    @property
    def weight_elem_bytes(self):
        return 2 if self.weight_bf16 else 4

    @property
    def positions(self):
        """positions the model may run through"""
        return self.max_pos or self.max_seq

    def weight_bytes(self):
        """bytes of every matrix the decode step streams once per token."""
        d, f, V, L = self.dim, self.hidden_dim, self.vocab_size, self.n_layers
        return self.weight_elem_bytes * (L * (2 * d * d + 2 * self.kv_dim * d + 3 * d * f) + V * d)


@dataclass(frozen=True)
class Workload:
    """A named decode workload: model, seeds, batch, prompt and positions."""
    name: str
    model: ModelConfig
    model_seed: int
    batch: int
    prompt_len: int            # 0 means "start token only" (see start_token)
    prompt_seed: int
    end_pos: int               # every position < end_pos gets one forward pass
    start_token: int = 1
    description: str = ""
    batches: Tuple[int, ...] = field(default=())

    @property
    def decode_steps(self):
        return self.end_pos - max(self.prompt_len, 1)


M15 = ModelConfig(dim=288, n_layers=6, n_heads=6, hidden_dim=768, max_seq=256)
M44 = ModelConfig(dim=512, n_layers=8, n_heads=8, hidden_dim=1376, max_seq=1024)
M110 = ModelConfig(dim=768, n_layers=12, n_heads=12, hidden_dim=2048, max_seq=1024)
M7B = ModelConfig(dim=4096, n_layers=32, n_heads=32, hidden_dim=11008, max_seq=2048, tied=False)

WORKLOADS = {
    # 15M shape, batch 1, start token 1 at position 0, greedy through position 255
    "C1": Workload("C1", M15, 0, 1, 0, 0, 256,
                   description="15M shape (288/6L/6H), b1, token 1, decode 256 positions"),
    # 44M shape, batch 1, 64 random prompt tokens, greedy to 1024 positions
    "C2": Workload("C2", M44, 1, 1, 64, 1, 1024,
                   description="44M shape (512/8L/8H), b1, 64-token prompt, decode to 1024"),
    # 15M shape, 256 independent sequences in lockstep, 16 prompt tokens each
    "C3": Workload("C3", replace(M15, max_batch=256), 0, 256, 16, 2, 256,
                   description="15M shape, b256 lockstep, 16-token prompts, decode to 256"),
    # 110M shape, 128-token prompts, decode to 1024, at batch 1 and batch 32
    "C4": Workload("C4", replace(M110, max_batch=32), 3, 1, 128, 3, 1024, batches=(1, 32),
                   description="110M shape (768/12L/12H), 128-token prompt, decode to 1024"),
    "C4b32": Workload("C4b32", replace(M110, max_batch=32), 3, 32, 128, 3, 1024,
                      description="110M shape, b32 lockstep, 128-token prompts, decode to 1024"),
    # 7B shape, untied classifier, 512-token prompt then 512 greedy steps
    "C5": Workload("C5", M7B, 4, 1, 512, 4, 1024,
                   description="7B shape (4096/32L/32H, 11008 hidden), b1, 512-token prompt, "
                               "512 decode steps"),
    # the 7B shape with bfloat16 weights (fp32 activations and arithmetic): half the
    # bytes per step
    "C5bf16": Workload("C5bf16", replace(M7B, weight_bf16=True), 4, 1, 512, 4, 1024,
                       description="7B shape, bfloat16 weights, b1, 512-token prompt, "
                                   "512 decode steps"),
    # the 7B shape decoding past its KV cache: a 512-position window (max_seq 512,
    # max_pos 2048), a 1024-token prompt, then positions 1024..1535 over the ring
    "C5w": Workload("C5w", replace(M7B, max_seq=512, max_pos=2048), 4, 1, 1024, 4, 1536,
                    description="7B shape, 512-position sliding window past max_seq, b1, "
                                "1024-token prompt, 512 decode steps"),
    # grouped-query variant of the 7B shape: 8 key/value heads shared by groups of 4
    # query heads (a measurement of the grouped-query row; not one of the five configs)
    "C5g8": Workload("C5g8", replace(M7B, n_kv_heads=8), 4, 1, 512, 4, 1024,
                     description="7B shape with 8 key/value heads (grouped-query), b1, "
                                 "512-token prompt, 512 decode steps"),
}

# Small shapes for element-by-element parity: several tiles and ragged tails.
TINY = ModelConfig(dim=64, n_layers=2, n_heads=4, hidden_dim=96, vocab_size=1003,
                   max_seq=64, max_batch=5)
TINY_UNTIED = replace(TINY, tied=False, n_heads=2, vocab_size=517)
SMALL = ModelConfig(dim=128, n_layers=3, n_heads=2, hidden_dim=352, vocab_size=4099,
                    max_seq=160, max_batch=7)
# grouped-query shapes: 2 key/value heads for 4 query heads (head dim 16), one
# key/value head for 4 query heads (multi-query, head dim 32), and head dim 64
TINY_GQA = replace(TINY, n_kv_heads=2)
SMALL_MQA = ModelConfig(dim=128, n_layers=3, n_heads=4, hidden_dim=352, vocab_size=4099,
                        max_seq=160, max_batch=7, n_kv_heads=1)
GQA_HD64 = ModelConfig(dim=256, n_layers=2, n_heads=4, hidden_dim=320, vocab_size=2011,
                       max_seq=200, max_batch=4, n_kv_heads=2)
# bfloat16 weights: untied classifier (head dim 32), and tied (the classifier
# reads the bfloat16 embedding table)
TINY_BF16 = replace(TINY_UNTIED, weight_bf16=True)
SMALL_BF16 = replace(SMALL, weight_bf16=True)

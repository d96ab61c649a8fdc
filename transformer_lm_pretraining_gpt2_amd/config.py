"""Model/run configurations, the learning-rate schedule and FLOP accounting.

Host-side logic only (no device code).  Shapes follow GPTConfig(vocab_size,
block_size, n_layer, n_head, n_embd) of "A small GPT that writes fairy tales"
(lm-book, code excerpt); block_size is called max_seq_len here.
"""
import math
from dataclasses import dataclass, field

# MI355X published dense bf16 MFMA peak: 256 CUs x 4096 FLOP/clk x 2.4 GHz.
MI355X_BF16_PEAK_FLOPS = 256 * 4096 * 2.4e9
MI355X_FP32_MFMA_PEAK_FLOPS = 157.3e12
MI355X_HBM_BYTES_PER_S = 8.0e12


@dataclass(frozen=True)
class GPT2Config:
    vocab_size: int
    padded_vocab_size: int
    n_layer: int
    n_head: int
    n_embd: int
    max_seq_len: int

    @property
    def head_dim(self):
        return self.n_embd // self.n_head

    def as_tuple(self):
        return (self.vocab_size, self.padded_vocab_size, self.n_layer, self.n_head, self.n_embd, self.max_seq_len)


@dataclass(frozen=True)
class RunConfig:
    name: str
    model: GPT2Config
    B: int
    T: int
    K: int  # micro-steps per optimizer step (gradient accumulation)
    precision: str  # "fp32" or "bf16"
    data: str  # "uniform" or "zipf"
    max_lr: float
    warmup: int
    max_steps: int
    min_lr_ratio: float = 0.1
    beta1: float = 0.9
    beta2: float = 0.95
    eps: float = 1e-8
    weight_decay: float = 0.1
    grad_clip: float = 1.0

    @property
    def tokens_per_step(self):
        return self.K * self.B * self.T


# The five workloads.  Optimizer settings follow "Karpathy's four-hour GPT-2
# reproduction in one post", part 3 (AdamW betas (0.9, 0.95), eps 1e-8, weight
# decay 0.1 on 2-D tensors, clip 1.0, 715 warmup steps, cosine to 10% of a
# 6e-4 peak) and the lm-book code excerpt (peak 1e-3, warmup 200, wd 0.1,
# clip 1.0).  Max steps: 10e9 tokens / 524,288 = 19,073 for GPT-2;
# 14,000 for the story-scale model (its training log).
CONFIGS = {
    "tiny": RunConfig("tiny", GPT2Config(512, 512, 2, 4, 128, 64), B=4, T=64, K=1, precision="fp32",
                      data="uniform", max_lr=6e-4, warmup=715, max_steps=19073),
    "small": RunConfig("small", GPT2Config(4096, 4096, 4, 4, 256, 256), B=64, T=256, K=1, precision="bf16",
                       data="zipf", max_lr=1e-3, warmup=200, max_steps=14000),
    "story": RunConfig("story", GPT2Config(4096, 4096, 8, 8, 512, 512), B=64, T=512, K=1, precision="bf16",
                       data="zipf", max_lr=1e-3, warmup=200, max_steps=14000),
    "gpt2_124m": RunConfig("gpt2_124m", GPT2Config(50257, 50304, 12, 12, 768, 1024), B=16, T=1024, K=1,
                           precision="bf16", data="zipf", max_lr=6e-4, warmup=715, max_steps=19073),
    "gpt2_350m": RunConfig("gpt2_350m", GPT2Config(50257, 50304, 24, 16, 1024, 1024), B=16, T=1024, K=32,
                           precision="bf16", data="zipf", max_lr=6e-4, warmup=715, max_steps=19073),
}


def lr_at(step, max_lr, warmup, max_steps, min_lr_ratio=0.1):
    """Learning rate at 0-based optimizer step: linear warmup lr*(s+1)/W, then a
    cosine from lr down to min_lr_ratio*lr at max_steps, flat after that."""
    min_lr = max_lr * min_lr_ratio
    if step < warmup:
        return max_lr * (step + 1) / warmup
    if step >= max_steps:
        return min_lr
    ratio = (step - warmup) / (max_steps - warmup)
    return min_lr + 0.5 * (1.0 + math.cos(math.pi * ratio)) * (max_lr - min_lr)


def num_params(m: GPT2Config, padded=True):
    """Closed-form parameter count: V*C + Tmax*C + L*(12C^2 + 13C) + 2C."""
    V = m.padded_vocab_size if padded else m.vocab_size
    C = m.n_embd
    return V * C + m.max_seq_len * C + m.n_layer * (12 * C * C + 13 * C) + 2 * C


def flops_per_token(m: GPT2Config, T, causal=True):
    """Training FLOPs per token: 6*N (N over the real vocabulary) plus the
    attention score/value products, 12*L*T*C when every key is counted and
    half of that with the causal mask."""
    att = 12 * m.n_layer * T * m.n_embd
    return 6 * num_params(m, padded=False) + (att // 2 if causal else att)

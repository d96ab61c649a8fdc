"""Seeded synthetic inputs shared by the HIP library's callers and the tests.

This module holds none of the training step's arithmetic: it only draws
numbers.  Token streams stand in for the web-text corpora the pages train on
(not available here): Zipf(s) over the real vocabulary, sampled by inverse CDF
with numpy's PCG64, rank k -> token id k-1.  Initial parameters are the random
draws GPT-2's recipe makes ("Karpathy's four-hour GPT-2 reproduction in one
post", part 1): N(0, 0.02) for 2-D tensors, the two projections that add into
the residual stream scaled by 1/sqrt(2 * n_layer), biases 0, LayerNorm gains
1; padded vocabulary rows of the tied matrix are 0.
"""
import numpy as np

DATA_SEED = 1234
INIT_SEED = 1337


def zipf_stream(n, vocab_size, seed=DATA_SEED, s=1.0):
    """n token ids with P(rank k) proportional to 1/k^s, k = 1..V."""
    rng = np.random.default_rng(seed)
    w = 1.0 / np.arange(1, vocab_size + 1, dtype=np.float64) ** s
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    u = rng.random(n)
    ids = np.searchsorted(cdf, u, side="right")
    return np.minimum(ids, vocab_size - 1).astype(np.int32)


def uniform_stream(n, vocab_size, seed=DATA_SEED):
    rng = np.random.default_rng(seed)
    return rng.integers(0, vocab_size, size=n, dtype=np.int64).astype(np.int32)


def micro_batch(stream, B, T, index):
    """Micro-batch `index` of consecutive, non-overlapping windows:
    row b reads stream[o : o+T] as inputs and stream[o+1 : o+T+1] as targets,
    o = (index*B + b)*T."""
    ids = np.empty((B, T), np.int32)
    tgt = np.empty((B, T), np.int32)
    for b in range(B):
        o = (index * B + b) * T
        ids[b] = stream[o:o + T]
        tgt[b] = stream[o + 1:o + T + 1]
    return ids, tgt


def stream_length(steps, K, B, T):
    return steps * K * B * T + 1


def _is_residual_projection(name):
    return name.endswith("attn.c_proj.weight") or name.endswith("mlp.c_proj.weight")


def init_params(layout, n_layer, vocab_size, seed=INIT_SEED, std=0.02, dtype=np.float32):
    """Flat initial parameters for a layout [{name, offset, rows, cols}, ...]."""
    rng = np.random.default_rng(seed)
    last = layout[-1]
    n = last["offset"] + last["rows"] * (last["cols"] or 1)
    p = np.zeros(n, dtype=np.float64)
    for e in layout:
        size = e["rows"] * (e["cols"] or 1)
        view = p[e["offset"]:e["offset"] + size]
        name = e["name"]
        if e["cols"]:
            s = std / np.sqrt(2.0 * n_layer) if _is_residual_projection(name) else std
            view[:] = rng.standard_normal(size) * s
            if name == "wte":
                view.reshape(e["rows"], e["cols"])[vocab_size:] = 0.0
        elif name.endswith("ln_1.weight") or name.endswith("ln_2.weight") or name == "ln_f.weight":
            view[:] = 1.0
    return p.astype(dtype)


def random_params(layout, vocab_size, seed, scale=0.3, dtype=np.float64):
    """Generic random parameters (every tensor non-trivial) for derivative
    and parity checks: 2-D N(0, scale), LN gains 1 + N(0, scale), other 1-D
    N(0, scale/3).  Padded vocabulary rows stay 0."""
    rng = np.random.default_rng(seed)
    last = layout[-1]
    n = last["offset"] + last["rows"] * (last["cols"] or 1)
    p = np.zeros(n, dtype=np.float64)
    for e in layout:
        size = e["rows"] * (e["cols"] or 1)
        view = p[e["offset"]:e["offset"] + size]
        name = e["name"]
        if e["cols"]:
            view[:] = rng.standard_normal(size) * scale
            if name == "wte":
                view.reshape(e["rows"], e["cols"])[vocab_size:] = 0.0
        elif name.endswith(".weight"):
            view[:] = 1.0 + rng.standard_normal(size) * scale
        else:
            view[:] = rng.standard_normal(size) * scale / 3
    return p.astype(dtype)

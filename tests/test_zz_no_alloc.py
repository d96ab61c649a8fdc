"""gpt2_adamw_step_noalloc (clip + AdamW with the library's static scratch
instead of a workspace) against gpt2_adamw_step on the same state, through the
C ABI: two calls in a row on the same GPU, the second on a smaller model, so
scratch contents left by the first call cannot leak into the second.  Both
entry points run the same kernels in the same order, so the results must be
identical bit for bit (parameters, bf16 copy, moments and norm)."""
import numpy as np
import pytest

from gpu_common import batches
from transformer_lm_pretraining_gpt2_amd import binding, synth
from transformer_lm_pretraining_gpt2_amd.config import CONFIGS, GPT2Config

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(300)]

SMALLER = GPT2Config(vocab_size=509, padded_vocab_size=512, n_layer=1, n_head=2, n_embd=128, max_seq_len=64)


def _one(model, B, T, prec, clip, seed):
    import torch

    lay = binding.param_layout(model)
    p0 = synth.random_params(lay, model.vocab_size, seed=seed, scale=0.05).astype(np.float32)
    (ids, tgt), = batches(model, B, T, 1, seed=seed)
    s = binding.TrainStep(model, B, T, prec)
    s.set_params(p0)
    s.forward(torch.from_numpy(ids.reshape(-1)).cuda(), torch.from_numpy(tgt.reshape(-1)).cuda())
    s.backward(0, 1)
    # a first update on the handle so the moments are nonzero, then the copies
    s.adamw_step(1, 6e-4, grad_clip=clip)
    assert s.sync_status() == 0
    copy = {k: getattr(s, k).clone() for k in ("params", "grads", "m", "v")}
    copy["params_lp"] = s.params_lp.clone() if s.params_lp is not None else None
    n_decay = binding.num_decay_params(model)
    norm_h = torch.zeros(1, device="cuda")
    norm_n = torch.full((1,), float("nan"), device="cuda")
    s.adamw_step(2, 5e-4, grad_clip=clip, grad_norm=norm_h)
    binding.adamw_step_noalloc(copy["params"], copy["params_lp"], copy["grads"], copy["m"], copy["v"], n_decay, 2,
                               5e-4, grad_clip=clip, grad_norm=norm_n)
    assert s.sync_status() == 0
    torch.cuda.synchronize()
    print(f"{model.n_layer} layers, {prec}, clip {clip}: norm {norm_h.item():.6f} / {norm_n.item():.6f}", flush=True)
    assert torch.equal(norm_h, norm_n)
    for k in ("params", "m", "v"):
        assert torch.equal(getattr(s, k), copy[k]), k
    if s.params_lp is not None:
        assert torch.equal(s.params_lp, copy["params_lp"])


@pytest.mark.parametrize("prec,clip", [("bf16", 1.0), ("fp32", 1e3)])
def test_noalloc_update_equals_handle_update_twice(prec, clip):
    # first on the tiny GPT-2, then on a smaller one-layer model
    rc = CONFIGS["tiny"]
    _one(rc.model, rc.B, rc.T, prec, clip, seed=5)
    _one(SMALLER, 2, 64, prec, clip, seed=6)


def test_noalloc_rejects_bad_sizes_before_any_device_work():
    import ctypes

    L = binding.lib()
    a = ctypes.c_void_p(1 << 20)
    args = lambda n, nd, step=1: (a, None, a, a, a, n, nd, step, 6e-4, 0.9, 0.95, 1e-8, 0.1, 1.0, a, None)
    assert L.gpt2_adamw_step_noalloc(*args(6, 4)) == -3  # n not a multiple of 4
    assert L.gpt2_adamw_step_noalloc(*args(8, 12)) == -3  # decayed prefix beyond n
    assert L.gpt2_adamw_step_noalloc(*args((1 << 36) + 4, 0)) == -3  # beyond the limit
    assert L.gpt2_adamw_step_noalloc(*args(8, 4, step=0)) == -3  # steps count from 1
    assert L.gpt2_adamw_step_noalloc(None, None, a, a, a, 8, 4, 1, 6e-4, 0.9, 0.95, 1e-8, 0.1, 1.0, a, None) == -3

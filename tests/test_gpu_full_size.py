"""GPU parity at the full GPT-2 124M size, in the launch configuration the
throughput benchmark times: bf16, B = 16, T = 1024, random GPT-2 init.

The oracle cannot run a whole 16 x 1024 batch in reasonable time, so:
  * forward: a batch of 16 distinct Zipf sequences; the per-position losses of
    two sampled sequences (first and last rows of the batch) are recomputed by
    the oracle one sequence at a time (sequences are independent in the
    forward pass);
  * full step: one sequence repeated 16 times.  The mean loss over 16 x 1024
    identical positions has exactly the gradient of the single sequence's mean
    loss, so the oracle's B = 1 step (forward, backward, clip, AdamW) is the
    reference for every gradient, the norm and the updated parameters, while
    the GPU runs every kernel at its full-size shapes and tiles.
The oracle runs in fp32 here (about 20 s per sequence); its rounding error is
orders of magnitude below the bf16 tolerances.
"""
import numpy as np
import pytest

from gpu_common import TOL, batches, compare, gpu_step, oracle_step
from oracle import oracle
from transformer_lm_pretraining_gpt2_amd import binding, synth
from transformer_lm_pretraining_gpt2_amd.config import CONFIGS

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]

MODEL = CONFIGS["gpt2_124m"].model
B, T = CONFIGS["gpt2_124m"].B, CONFIGS["gpt2_124m"].T


@pytest.fixture(scope="module")
def params():
    return synth.init_params(binding.param_layout(MODEL), MODEL.n_layer, MODEL.vocab_size)


def test_full_size_forward_sampled_rows(params):
    import torch

    ids, tgt = batches(MODEL, B, T, 1, seed=1234)[0]
    s = binding.TrainStep(MODEL, B, T, "bf16")
    s.set_params(params)
    loss = torch.zeros(1, device="cuda")
    rows = torch.zeros(B * T, device="cuda")
    s.forward(torch.from_numpy(ids.reshape(-1)).cuda(), torch.from_numpy(tgt.reshape(-1)).cuda(), loss, rows)
    assert s.sync_status() == 0
    rows = rows.cpu().numpy().astype(np.float64)
    p32 = params.astype(np.float32)
    for b in (0, B - 1):
        rl = np.zeros(T, np.float32)
        lo = oracle.fwd_bwd(MODEL, 1, T, p32, ids[b:b + 1], tgt[b:b + 1], row_loss=rl, R=np.float32)
        got = rows[b * T:(b + 1) * T]
        err = np.max(np.abs(got - rl))
        print(f"sequence {b}: oracle loss {lo:.5f} gpu {got.mean():.5f}, max per-position diff {err:.3e}", flush=True)
        assert abs(got.mean() - lo) <= TOL["bf16"]["loss"]
        assert err <= TOL["bf16"]["rows"]


def test_full_size_step_repeated_sequence(params):
    ids, tgt = batches(MODEL, 1, T, 1, seed=4321)[0]
    rep = (np.repeat(ids, B, axis=0), np.repeat(tgt, B, axis=0))
    print("gpu step (B=16, T=1024, bf16)", flush=True)
    g = gpu_step(MODEL, B, T, "bf16", params, [rep])
    g["loss"] = [g["loss"][0]]
    print("oracle step (B=1, T=1024, fp32)", flush=True)
    o = oracle_step(MODEL, params, [(ids, tgt)], R=np.float32)
    # every copy of the sequence must give the oracle's per-position losses
    g["rows"] = [g["rows"][0][k * T:(k + 1) * T] for k in range(B)]
    o["rows"] = [o["rows"][0]] * B
    compare(MODEL, g, o, "bf16")

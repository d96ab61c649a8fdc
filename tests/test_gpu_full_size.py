"""GPU parity at full size, in each workload's own launch configuration: the
GPT-2 124M step the throughput benchmark times (bf16, B = 16, T = 1024), the
small and story-scale GPTs at their batch sizes, and GPT-2 350M with its
32-step gradient accumulation; random GPT-2 init.

  * 124M, the benchmark's step: a batch of 16 distinct Zipf sequences, every
    gradient, the norm and the updated parameters against the oracle's step on
    the same 16 sequences (fp32 forward/backward, about 5 s of host time per
    sequence), the AdamW update element by element against the fp64 oracle's
    update of the device's own gradients, and the embedding output bit for bit.
  * 350M with K = 32 micro-steps (a 524,288-token batch): micro-steps
    alternate between two batches, each one sequence repeated 16 times; the
    accumulated gradient is then that of the two sequences' mean loss, so the
    oracle's B = 2 step is the reference.
  * The other checks use one sequence repeated B times, whose mean loss has
    exactly the gradient of the single sequence (the oracle's B = 1 step),
    while the device runs every kernel at its full-size shapes and tiles.
The oracle runs its forward and backward in fp32 here; its rounding error is
orders of magnitude below the bf16 tolerances.
"""
import numpy as np
import pytest

from gpu_common import TOL, batches, compare, gpu_step, oracle_step, rel_l2, tensor_views
from optim_check import check_update, reference
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


def test_full_size_eval_equals_training_forward(params):
    # the forward-only path at the benchmark's shapes: same per-position losses
    # as the training forward, bit for bit (the sampled-rows test above pins
    # those to the oracle)
    import torch

    ids, tgt = batches(MODEL, B, T, 1, seed=77)[0]
    s = binding.TrainStep(MODEL, B, T, "bf16")
    s.set_params(params)
    d_ids = torch.from_numpy(ids.reshape(-1)).cuda()
    d_tgt = torch.from_numpy(tgt.reshape(-1)).cuda()
    le, lf = torch.zeros(1, device="cuda"), torch.zeros(1, device="cuda")
    re, rf = torch.zeros(B * T, device="cuda"), torch.zeros(B * T, device="cuda")
    s.evaluate(d_ids, d_tgt, le, re)
    s.forward(d_ids, d_tgt, lf, rf)
    assert s.sync_status() == 0
    print(f"eval loss {le.item():.6f}, training forward loss {lf.item():.6f}", flush=True)
    assert le.item() == lf.item()
    assert torch.equal(re, rf)


def test_full_size_step_distinct_sequences(params):
    # the benchmark's step on 16 distinct sequences: a kernel that mixed up
    # sequences (rows of different batch entries) would show here
    mb = batches(MODEL, B, T, 1, seed=4321)
    ids = mb[0][0]
    assert len({ids[b].tobytes() for b in range(B)}) == B
    print("gpu step (B=16, T=1024, bf16, 16 distinct sequences)", flush=True)
    g = gpu_step(MODEL, B, T, "bf16", params, mb)
    s = g["handle"]
    # the embedding output, bit for bit (both precisions gather fp32 masters)
    x0 = s.residual(0).cpu().numpy()
    p32 = params.astype(np.float32)
    C = MODEL.n_embd
    lay = binding.param_layout(MODEL)
    wpe_off = next(e["offset"] for e in lay if e["name"] == "wpe")
    wte = p32[:MODEL.padded_vocab_size * C].reshape(-1, C)
    wpe = p32[wpe_off:wpe_off + T * C].reshape(T, C)
    want = wte[ids.reshape(-1)] + np.tile(wpe, (B, 1))
    assert np.array_equal(x0.view(np.uint32), want.astype(np.float32).view(np.uint32))
    print("oracle step (B=16, T=1024, fp32)", flush=True)
    o = oracle_step(MODEL, params, mb, R=np.float32)
    compare(MODEL, g, o, "bf16")
    # the update of all 124M parameters, element by element, against the
    # fp64 oracle's clip + AdamW of the device's own gradients
    ref = reference(MODEL, p32.astype(np.float64), g["grads"], np.zeros(p32.size), np.zeros(p32.size), 1, 6e-4, 1.0, 0.1)
    fails = check_update(lay, p32.astype(np.float64), dict(p=g["params"], m=g["m"], v=g["v"], norm=g["norm"]), ref,
                         lp=s.params_lp.float().cpu().numpy())
    assert not fails, fails


def _repeated_step(model, B, T, prec, seed, K=1):
    """GPU step on one sequence repeated B times in each of K micro-steps
    against the oracle's step on that single sequence (same gradient)."""
    p0 = synth.init_params(binding.param_layout(model), model.n_layer, model.vocab_size)
    ids, tgt = batches(model, 1, T, 1, seed=seed)[0]
    rep = (np.repeat(ids, B, axis=0), np.repeat(tgt, B, axis=0))
    print(f"gpu step (B={B}, T={T}, K={K}, {prec})", flush=True)
    handle = binding.TrainStep(model, B, T, "bf16", fp8=True) if prec == "fp8" else None
    g = gpu_step(model, B, T, "bf16" if prec == "fp8" else prec, p0, [rep] * K, handle=handle)
    print("oracle step (B=1, fp32 forward/backward, fp64 update)", flush=True)
    o = oracle_step(model, p0, [(ids, tgt)], R=np.float32)
    g["loss"] = [float(np.mean(g["loss"]))]
    g["rows"] = [r[k * T:(k + 1) * T] for r in g["rows"] for k in range(B)]
    o["rows"] = [o["rows"][0]] * (B * K)
    compare(model, g, o, prec)


def test_full_size_recompute_step_repeated_sequence(params):
    # activation recompute at the benchmark's shapes, against the oracle
    ids, tgt = batches(MODEL, 1, T, 1, seed=2468)[0]
    rep = (np.repeat(ids, B, axis=0), np.repeat(tgt, B, axis=0))
    print("gpu step with activation recompute (B=16, T=1024, bf16)", flush=True)
    g = gpu_step(MODEL, B, T, "bf16", params, [rep], handle=binding.TrainStep(MODEL, B, T, "bf16", recompute=True))
    print("oracle step (B=1, T=1024, fp32)", flush=True)
    o = oracle_step(MODEL, params, [(ids, tgt)], R=np.float32)
    g["rows"] = [g["rows"][0][k * T:(k + 1) * T] for k in range(B)]
    o["rows"] = [o["rows"][0]] * B
    compare(MODEL, g, o, "bf16")


def test_full_size_fp8_step_repeated_sequence(params):
    # FP8 forward products at the benchmark's shapes: against the oracle, and
    # against the bf16 path on the same inputs (FP8 is announced as the next
    # step after the bf16 run, "Reproducing GPT-2 (124M) cheaply with llm.c",
    # FAQ): loss difference and per-tensor gradient relative L2 between the
    # two device modes
    ids, tgt = batches(MODEL, 1, T, 1, seed=2468)[0]
    rep = (np.repeat(ids, B, axis=0), np.repeat(tgt, B, axis=0))
    print("gpu step with FP8 forward products (B=16, T=1024)", flush=True)
    g = gpu_step(MODEL, B, T, "bf16", params, [rep], handle=binding.TrainStep(MODEL, B, T, "bf16", fp8=True))
    print("gpu step in bf16 on the same inputs", flush=True)
    gb = gpu_step(MODEL, B, T, "bf16", params, [rep])
    lay = binding.param_layout(MODEL)
    fv, bv = tensor_views(lay, g["grads"]), tensor_views(lay, gb["grads"])
    worst = max((rel_l2(fv[n], bv[n]), n) for n in fv if np.linalg.norm(bv[n]) > 0)
    dloss = abs(g["loss"][0] - gb["loss"][0])
    print(f"FP8 vs bf16: |loss diff| {dloss:.2e}, worst per-tensor gradient rel L2 {worst[0]:.3e} ({worst[1]}), "
          f"update rel L2 {rel_l2(g['params'] - params, gb['params'] - params):.3e}", flush=True)
    assert dloss <= TOL["fp8"]["loss"]
    assert worst[0] <= TOL["fp8"]["grad"]
    print("oracle step (B=1, T=1024, fp32)", flush=True)
    o = oracle_step(MODEL, params, [(ids, tgt)], R=np.float32)
    g["rows"] = [g["rows"][0][k * T:(k + 1) * T] for k in range(B)]
    o["rows"] = [o["rows"][0]] * B
    compare(MODEL, g, o, "fp8")


def test_story_config_launch_shape():
    # story-scale GPT (27.6M params: V 4096, L 8, nh 8, C 512) at its own B = 64, T = 512
    rc = CONFIGS["story"]
    _repeated_step(rc.model, rc.B, rc.T, "bf16", seed=2024)


def test_gpt2_350m_with_32_accumulated_micro_steps():
    # GPT-2 350M (L 24, nh 16, C 1024) at B = 16, T = 1024 with its own K = 32
    # micro-steps (524,288 tokens, loss / 32 each, the first overwriting the
    # gradients and the rest adding onto them).  Micro-steps alternate between
    # sequence a repeated 16 times and sequence b repeated 16 times, so the
    # accumulated gradient is that of the mean loss over [a, b]: the oracle's
    # B = 2 step.
    rc = CONFIGS["gpt2_350m"]
    model, K = rc.model, rc.K
    assert K == 32
    p0 = synth.init_params(binding.param_layout(model), model.n_layer, model.vocab_size)
    ids, tgt = batches(model, 2, T, 1, seed=350)[0]
    reps = [(np.repeat(ids[k:k + 1], B, axis=0), np.repeat(tgt[k:k + 1], B, axis=0)) for k in (0, 1)]
    print(f"gpu step (B={B}, T={T}, K={K}, bf16)", flush=True)
    g = gpu_step(model, B, T, "bf16", p0, [reps[k % 2] for k in range(K)])
    print("oracle step (B=2, fp32 forward/backward, fp64 update)", flush=True)
    o = oracle_step(model, p0, [(ids, tgt)], R=np.float32)
    # every copy of a sequence in every micro-step gives that sequence's per-position losses
    for k in range(K):
        want = o["rows"][0][(k % 2) * T:(k % 2 + 1) * T]
        got = g["rows"][k].reshape(B, T)
        assert np.max(np.abs(got - want[None, :])) <= TOL["bf16"]["rows"], k
    g["loss"] = [float(np.mean(g["loss"]))]
    g["rows"] = [np.concatenate([g["rows"][k][:T] for k in (0, 1)])]
    compare(model, g, o, "bf16")


def test_gpt2_350m_fp8_step_repeated_sequence():
    # FP8 forward products at GPT-2 350M (C = 1024: MLP rows of 4096 values
    # for the row quantizer), against the oracle
    rc = CONFIGS["gpt2_350m"]
    _repeated_step(rc.model, rc.B, rc.T, "fp8", seed=351)


def test_small_config_launch_shape():
    # small GPT (V 4096, L 4, nh 4, C 256) at its own B = 64, T = 256
    rc = CONFIGS["small"]
    _repeated_step(rc.model, rc.B, rc.T, "bf16", seed=64)


def test_full_size_fp32_step():
    # fp32 mode at the 124M launch shape: operands beyond 2 GiB (the fp32
    # logits are 3.3 GB) against the oracle in fp64, at the fp32 tolerances
    p0 = synth.init_params(binding.param_layout(MODEL), MODEL.n_layer, MODEL.vocab_size)
    ids, tgt = batches(MODEL, 1, T, 1, seed=99)[0]
    rep = (np.repeat(ids, B, axis=0), np.repeat(tgt, B, axis=0))
    print("gpu step (B=16, T=1024, fp32)", flush=True)
    g = gpu_step(MODEL, B, T, "fp32", p0, [rep])
    print("oracle step (B=1, fp64)", flush=True)
    o = oracle_step(MODEL, p0, [(ids, tgt)], R=np.float64)
    g["rows"] = [g["rows"][0][k * T:(k + 1) * T] for k in range(B)]
    o["rows"] = [o["rows"][0]] * B
    compare(MODEL, g, o, "fp32")

"""GPU parity: the HIP training step (through the C ABI) against the CPU
oracle on the same seeded inputs.

Tolerances (fixed by the target contract for this path):
  fp32 mode  |loss diff| <= 1e-4, per-tensor gradient relative L2 <= 1e-4
  bf16 mode  |loss diff| <= 2e-2, parameter and per-tensor gradient relative
             L2 <= 3e-2 after one step
Index handling is exact: which wte rows receive gradient, and which target each
position's loss uses (per-position losses), and the error flags.
"""
import math

import numpy as np
import pytest

from gpu_common import batches, compare, gpu_step, oracle_step, rel_l2, tensor_views
from oracle import oracle
from transformer_lm_pretraining_gpt2_amd import binding, synth
from transformer_lm_pretraining_gpt2_amd.config import CONFIGS, GPT2Config

pytestmark = pytest.mark.gpu

TINY = CONFIGS["tiny"].model
PADDED = GPT2Config(vocab_size=509, padded_vocab_size=512, n_layer=2, n_head=4, n_embd=128, max_seq_len=128)
SMALL = CONFIGS["small"].model
# three layers of C = 384: odd layer count, and at 2048 tokens the bf16 weight
# gradients split their 64 reduction steps into 25 (qkv), 32 (proj) and 21
# (fc, fcproj) parts, uneven for three of the four
MID = GPT2Config(vocab_size=509, padded_vocab_size=512, n_layer=3, n_head=6, n_embd=384, max_seq_len=512)


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
def test_tiny_step_matches_oracle(prec):
    rc = CONFIGS["tiny"]
    p0 = synth.init_params(binding.param_layout(TINY), TINY.n_layer, TINY.vocab_size, dtype=np.float64)
    mb = batches(TINY, rc.B, rc.T, 1, seed=1234, data="uniform")
    g = gpu_step(TINY, rc.B, rc.T, prec, p0, mb)
    o = oracle_step(TINY, p0, mb)
    compare(TINY, g, o, prec)


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
def test_padded_vocab_random_params(prec):
    # larger random weights exercise every nonlinearity; V < Vp exercises the padding mask
    lay = binding.param_layout(PADDED)
    p0 = synth.random_params(lay, PADDED.vocab_size, seed=21, scale=0.05)
    mb = batches(PADDED, 2, 128, 1, seed=5)
    g = gpu_step(PADDED, 2, 128, prec, p0, mb, lr=1e-3)
    o = oracle_step(PADDED, p0, mb, lr=1e-3)
    compare(PADDED, g, o, prec)


def test_zero_tied_matrix_gives_log_vocab():
    lay = binding.param_layout(PADDED)
    p0 = synth.random_params(lay, PADDED.vocab_size, seed=3, scale=0.05)
    p0[:PADDED.padded_vocab_size * PADDED.n_embd] = 0
    mb = batches(PADDED, 2, 64, 1, seed=9)
    g = gpu_step(PADDED, 2, 64, "fp32", p0, mb)
    assert abs(g["loss"][0] - math.log(PADDED.vocab_size)) < 1e-5
    assert np.max(np.abs(g["rows"][0] - math.log(PADDED.vocab_size))) < 1e-5


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
def test_small_config_step(prec):
    # the small workload's shapes (V 4096, L 4, nh 4, C 256, T 256) at B = 8
    lay = binding.param_layout(SMALL)
    p0 = synth.init_params(lay, SMALL.n_layer, SMALL.vocab_size, dtype=np.float64)
    mb = batches(SMALL, 8, 256, 1, seed=1234)
    g = gpu_step(SMALL, 8, 256, prec, p0, mb, lr=1e-3)
    o = oracle_step(SMALL, p0, mb, lr=1e-3)
    compare(SMALL, g, o, prec)


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
def test_grad_accumulation_matches_one_big_batch(prec):
    # K micro-steps of B/K with loss/K == one step of B (both against the oracle)
    lay = binding.param_layout(PADDED)
    p0 = synth.random_params(lay, PADDED.vocab_size, seed=4, scale=0.05)
    big = batches(PADDED, 4, 64, 1, seed=17)[0]
    micro = [(big[0][:2], big[1][:2]), (big[0][2:], big[1][2:])]
    g = gpu_step(PADDED, 2, 64, prec, p0, micro)
    o = oracle_step(PADDED, p0, [big])
    g["loss"] = [float(np.mean(g["loss"]))]
    g["rows"] = [np.concatenate(g["rows"])]
    compare(PADDED, g, o, prec)


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
def test_embedding_output_is_bit_exact(prec):
    # x0[b, t] = wte[id[b, t]] + wpe[t]: one fp32 addition of the fp32 master
    # rows, so the device's residual stream at block 0 equals numpy's sum bit
    # for bit (both precisions gather from the fp32 masters).  Zipf ids put
    # many positions on the same rows; V < Vp leaves padded rows unused.
    import torch

    lay = binding.param_layout(PADDED)
    p0 = synth.random_params(lay, PADDED.vocab_size, seed=13, scale=0.05).astype(np.float32)
    B, T = 4, 128
    ids, tgt = batches(PADDED, B, T, 1, seed=31)[0]
    s = binding.TrainStep(PADDED, B, T, prec)
    s.set_params(p0)
    s.forward(torch.from_numpy(ids.reshape(-1)).cuda(), torch.from_numpy(tgt.reshape(-1)).cuda())
    assert s.sync_status() == 0
    x0 = s.residual(0).cpu().numpy()
    v = {e["name"]: e for e in lay}
    C = PADDED.n_embd
    wte = p0[:PADDED.padded_vocab_size * C].reshape(-1, C)
    wpe = p0[v["wpe"]["offset"]:v["wpe"]["offset"] + PADDED.max_seq_len * C].reshape(-1, C)
    want = (wte[ids.reshape(-1)] + np.tile(wpe[:T], (B, 1))).astype(np.float32)
    assert x0.dtype == np.float32 and x0.shape == want.shape
    assert np.array_equal(x0.view(np.uint32), want.view(np.uint32))
    with pytest.raises(binding.Gpt2Error):
        s.residual_ptr(PADDED.n_layer + 1)


def test_step_is_deterministic():
    lay = binding.param_layout(SMALL)
    p0 = synth.init_params(lay, SMALL.n_layer, SMALL.vocab_size, dtype=np.float64)
    mb = batches(SMALL, 4, 256, 1, seed=77)
    a = gpu_step(SMALL, 4, 256, "bf16", p0, mb)
    b = gpu_step(SMALL, 4, 256, "bf16", p0, mb, handle=a["handle"])
    assert a["loss"] == b["loss"]
    for k in ("grads", "params", "m", "v"):
        assert np.array_equal(a[k], b[k]), k


def test_token_out_of_range_is_reported():
    import torch

    s = binding.TrainStep(PADDED, 2, 64, "fp32")
    s.set_params(synth.random_params(binding.param_layout(PADDED), PADDED.vocab_size, seed=1).astype(np.float32))
    ids = torch.zeros(128, dtype=torch.int32, device="cuda")
    tgt = torch.zeros(128, dtype=torch.int32, device="cuda")
    ids[7] = PADDED.vocab_size  # out of range (a padded row)
    s.forward(ids, tgt)
    assert s.sync_status() == -5
    ids[7] = 3
    tgt[9] = -1
    s.forward(ids, tgt)
    assert s.sync_status() == -5
    tgt[9] = 1
    s.forward(ids, tgt)
    assert s.sync_status() == 0


def test_nonfinite_gradient_skips_the_update():
    import torch

    s = binding.TrainStep(PADDED, 2, 64, "bf16")
    p0 = synth.random_params(binding.param_layout(PADDED), PADDED.vocab_size, seed=1).astype(np.float32)
    s.set_params(p0)
    ids, tgt = batches(PADDED, 2, 64, 1, seed=2)[0]
    s.forward(torch.from_numpy(ids.reshape(-1)).cuda(), torch.from_numpy(tgt.reshape(-1)).cuda())
    s.backward(0, 1)
    s.grads[5] = float("nan")
    s.adamw_step(1, 1e-3)
    assert s.sync_status() == -6
    assert np.array_equal(s.params.cpu().numpy(), p0)
    assert s.sync_status() == 0


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
def test_single_sequence_one_tile(prec):
    # B = 1, T = 128: every matmul is a single 128-row tile, attention two key tiles
    m = GPT2Config(vocab_size=509, padded_vocab_size=512, n_layer=2, n_head=4, n_embd=128, max_seq_len=128)
    p0 = synth.random_params(binding.param_layout(m), m.vocab_size, seed=11, scale=0.05)
    mb = batches(m, 1, 128, 1, seed=12)
    g = gpu_step(m, 1, 128, prec, p0, mb)
    o = oracle_step(m, p0, mb)
    compare(m, g, o, prec)


def test_one_layer_heavy_vocab_padding():
    # one block; V = 130 padded to 256 (most of the last vocabulary tile is padding)
    m = GPT2Config(vocab_size=130, padded_vocab_size=256, n_layer=1, n_head=2, n_embd=128, max_seq_len=128)
    p0 = synth.random_params(binding.param_layout(m), m.vocab_size, seed=13, scale=0.05)
    mb = batches(m, 2, 64, 1, seed=14, data="uniform")
    g = gpu_step(m, 2, 64, "fp32", p0, mb)
    o = oracle_step(m, p0, mb)
    compare(m, g, o, "fp32")


def test_all_positions_same_token():
    # every input position holds the last real id: the embedding scatter sums
    # one segment of all B*T positions (four 64-position pieces)
    lay = binding.param_layout(PADDED)
    p0 = synth.random_params(lay, PADDED.vocab_size, seed=15, scale=0.05)
    ids = np.full((2, 128), PADDED.vocab_size - 1, np.int32)
    tgt = np.random.default_rng(16).integers(0, PADDED.vocab_size, (2, 128)).astype(np.int32)
    g = gpu_step(PADDED, 2, 128, "fp32", p0, [(ids, tgt)])
    o = oracle_step(PADDED, p0, [(ids, tgt)])
    compare(PADDED, g, o, "fp32")


def test_overlapped_weight_gradients_match_serial():
    # the second stream only changes when the weight-gradient products run,
    # never what they compute: both schedules give bit-identical results
    lay = binding.param_layout(SMALL)
    p0 = synth.init_params(lay, SMALL.n_layer, SMALL.vocab_size, dtype=np.float64)
    mb = batches(SMALL, 4, 256, 2, seed=31)
    a = gpu_step(SMALL, 4, 256, "bf16", p0, mb)
    s = binding.TrainStep(SMALL, 4, 256, "bf16")
    s.set_overlap(False)
    b = gpu_step(SMALL, 4, 256, "bf16", p0, mb, handle=s)
    assert a["loss"] == b["loss"]
    for k in ("grads", "params", "m", "v"):
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
def test_sequence_length_not_a_multiple_of_128(prec):
    # T = 192: the attention kernels' second row block of 128 has only its
    # first 64 rows, so half its waves are idle; the key blocks that start on
    # the diagonal walk one (masked) query tile, and the dQ / forward blocks
    # sweep a plain tile before the two masked ones
    m = GPT2Config(vocab_size=509, padded_vocab_size=512, n_layer=2, n_head=4, n_embd=128, max_seq_len=192)
    lay = binding.param_layout(m)
    p0 = synth.random_params(lay, m.vocab_size, seed=21, scale=0.05)
    mb = batches(m, 2, 192, 1, seed=23)
    g = gpu_step(m, 2, 192, prec, p0, mb)
    o = oracle_step(m, p0, mb)
    compare(m, g, o, prec)


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
def test_odd_layer_count_and_uneven_reduction_splits(prec):
    # the backward alternates du, dqkv and LayerNorm 2's copy of dres between
    # two buffers by layer parity and joins the second stream once per layer;
    # with an odd layer count the last layer uses the odd buffers.  Against the
    # oracle, and the overlapped schedule bit-identical to the serial one.
    lay = binding.param_layout(MID)
    p0 = synth.init_params(lay, MID.n_layer, MID.vocab_size, dtype=np.float64)
    mb = batches(MID, 4, 512, 1, seed=77)
    g = gpu_step(MID, 4, 512, prec, p0, mb)
    o = oracle_step(MID, p0, mb)
    compare(MID, g, o, prec)
    s = binding.TrainStep(MID, 4, 512, prec)
    s.set_overlap(False)
    b = gpu_step(MID, 4, 512, prec, p0, mb, handle=s)
    assert g["loss"] == b["loss"]
    for k in ("grads", "params", "m", "v"):
        assert np.array_equal(g[k], b[k]), k


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
def test_eval_matches_forward_and_oracle(prec):
    # forward-only evaluation: the training forward's loss bit for bit (same
    # kernels, fewer stores), the oracle's loss to the parity bar, and no
    # backward allowed after it
    import torch

    lay = binding.param_layout(PADDED)
    p0 = synth.random_params(lay, PADDED.vocab_size, seed=8, scale=0.05)
    (ids, tgt), = batches(PADDED, 2, 128, 1, seed=44)
    s = binding.TrainStep(PADDED, 2, 128, prec)
    s.set_params(p0.astype(np.float32))
    d_ids = torch.from_numpy(ids.reshape(-1).astype(np.int32)).cuda()
    d_tgt = torch.from_numpy(tgt.reshape(-1).astype(np.int32)).cuda()
    le, lf = torch.zeros(1, device="cuda"), torch.zeros(1, device="cuda")
    re, rf = torch.zeros(256, device="cuda"), torch.zeros(256, device="cuda")
    s.evaluate(d_ids, d_tgt, le, re)
    with pytest.raises(RuntimeError):
        s.backward(0, 1)
    s.forward(d_ids, d_tgt, lf, rf)
    assert s.sync_status() == 0
    assert le.item() == lf.item()
    assert torch.equal(re, rf)
    rl = np.zeros(256)
    ref = oracle.fwd_bwd(PADDED, 2, 128, p0, ids, tgt, row_loss=rl)
    tol = {"fp32": 1e-4, "bf16": 2e-2}[prec]
    print(f"eval loss gpu {le.item():.6f} oracle {ref:.6f}", flush=True)
    assert abs(le.item() - ref) <= tol
    assert np.max(np.abs(re.cpu().numpy() - rl)) <= {"fp32": 1e-4, "bf16": 1e-1}[prec]


def test_eval_without_targets_is_rejected():
    import torch

    s = binding.TrainStep(PADDED, 2, 128, "fp32")
    d_ids = torch.zeros(256, dtype=torch.int32, device="cuda")
    with pytest.raises(RuntimeError):
        s.evaluate(d_ids, None)


def test_recompute_fp32_identical_to_default():
    # fp32: rounding the pre-activation to the act type is the identity, so the
    # recompute mode reproduces the default step bit for bit (loss, gradients,
    # updated parameters), which also pins the backward's rebuilt activations
    # to the forward's
    lay = binding.param_layout(SMALL)
    p0 = synth.init_params(lay, SMALL.n_layer, SMALL.vocab_size, dtype=np.float64)
    mb = batches(SMALL, 4, 256, 2, seed=12)
    a = gpu_step(SMALL, 4, 256, "fp32", p0, mb)
    b = gpu_step(SMALL, 4, 256, "fp32", p0, mb, handle=binding.TrainStep(SMALL, 4, 256, "fp32", recompute=True))
    assert a["loss"] == b["loss"]
    for k in ("grads", "params", "m", "v"):
        assert np.array_equal(a[k], b[k]), k


def test_recompute_bf16_matches_oracle():
    # bf16: the activation comes from the rounded pre-activation; the step
    # still meets the parity bar (4 layers, so three layers are rebuilt)
    lay = binding.param_layout(SMALL)
    p0 = synth.init_params(lay, SMALL.n_layer, SMALL.vocab_size, dtype=np.float64)
    mb = batches(SMALL, 8, 256, 1, seed=99)
    g = gpu_step(SMALL, 8, 256, "bf16", p0, mb, lr=1e-3,
                 handle=binding.TrainStep(SMALL, 8, 256, "bf16", recompute=True))
    o = oracle_step(SMALL, p0, mb, lr=1e-3)
    compare(SMALL, g, o, "bf16")


def test_fp8_forward_step_matches_oracle():
    # forward products on FP8 E4M3 copies with per-row scales (4 layers, width 256)
    lay = binding.param_layout(SMALL)
    p0 = synth.init_params(lay, SMALL.n_layer, SMALL.vocab_size, dtype=np.float64)
    mb = batches(SMALL, 8, 256, 1, seed=99)
    g = gpu_step(SMALL, 8, 256, "bf16", p0, mb, lr=1e-3, handle=binding.TrainStep(SMALL, 8, 256, "bf16", fp8=True))
    o = oracle_step(SMALL, p0, mb, lr=1e-3)
    compare(SMALL, g, o, "fp8")


def test_fp8_eval_equals_forward_and_narrow_width_is_rejected():
    import torch

    s = binding.TrainStep(SMALL, 4, 256, "bf16", fp8=True)
    s.set_params(synth.init_params(binding.param_layout(SMALL), SMALL.n_layer, SMALL.vocab_size))
    (ids, tgt), = batches(SMALL, 4, 256, 1, seed=7)
    d_ids = torch.from_numpy(ids.reshape(-1).astype(np.int32)).cuda()
    d_tgt = torch.from_numpy(tgt.reshape(-1).astype(np.int32)).cuda()
    le, lf = torch.zeros(1, device="cuda"), torch.zeros(1, device="cuda")
    s.evaluate(d_ids, d_tgt, le)
    s.forward(d_ids, d_tgt, lf)
    assert s.sync_status() == 0
    assert le.item() == lf.item()
    with pytest.raises(RuntimeError):
        binding.TrainStep(PADDED, 2, 128, "bf16", fp8=True)  # width 128: the fused FP8 layer norm needs 256


def test_fp8_with_recompute_and_accumulation():
    # both flags together, two accumulated micro-steps (the weights' FP8 copies
    # are rebuilt only by the update, so both micro-steps see the same copies)
    lay = binding.param_layout(SMALL)
    p0 = synth.init_params(lay, SMALL.n_layer, SMALL.vocab_size, dtype=np.float64)
    big = batches(SMALL, 8, 256, 1, seed=123)[0]
    micro = [(big[0][:4], big[1][:4]), (big[0][4:], big[1][4:])]
    s = binding.TrainStep(SMALL, 4, 256, "bf16", fp8=True, recompute=True)
    g = gpu_step(SMALL, 4, 256, "bf16", p0, micro, lr=1e-3, handle=s)
    o = oracle_step(SMALL, p0, [big], lr=1e-3)
    g["loss"] = [float(np.mean(g["loss"]))]
    g["rows"] = [np.concatenate(g["rows"])]
    compare(SMALL, g, o, "fp8")


def test_recompute_eval_equals_forward():
    import torch

    s = binding.TrainStep(SMALL, 4, 256, "bf16", recompute=True)
    s.set_params(synth.init_params(binding.param_layout(SMALL), SMALL.n_layer, SMALL.vocab_size))
    (ids, tgt), = batches(SMALL, 4, 256, 1, seed=70)
    d_ids = torch.from_numpy(ids.reshape(-1).astype(np.int32)).cuda()
    d_tgt = torch.from_numpy(tgt.reshape(-1).astype(np.int32)).cuda()
    le, lf = torch.zeros(1, device="cuda"), torch.zeros(1, device="cuda")
    s.evaluate(d_ids, d_tgt, le)
    s.forward(d_ids, d_tgt, lf)
    assert s.sync_status() == 0
    assert le.item() == lf.item()


# head size 64 (the benchmark's), two heads
SHARP = GPT2Config(vocab_size=509, padded_vocab_size=512, n_layer=2, n_head=2, n_embd=128, max_seq_len=256)


def test_sharpened_attention_bf16():
    # The q and k rows of every c_attn weight scaled by 3: attention scores of
    # a few units, a peaked softmax and log-sum-exps far from zero.  The bf16
    # dK/dV kernel adds -LSE*sqrt(hd) and -D to S and dP through the matrix
    # core as three bf16 terms each; with them the step's worst per-tensor
    # gradient error against the fp64 oracle is 2.12e-2, the same as with LSE
    # and D read as fp32 values, while keeping only the leading bf16 term gives
    # 2.43e-2.  The kernels are deterministic, so the bar between the two
    # separates them.  (Scaled by 5 or more, the bf16 rounding of q and k alone
    # puts gradients beyond the bf16 bar, whatever the kernel.)
    B, T = 4, 256
    lay = binding.param_layout(SHARP)
    p0 = synth.random_params(lay, SHARP.vocab_size, seed=31, scale=0.05)
    for e in lay:
        if e["name"].endswith("attn.c_attn.weight"):
            w = p0[e["offset"]:e["offset"] + e["rows"] * e["cols"]].reshape(e["rows"], e["cols"])
            w[:2 * SHARP.n_embd] *= 3.0
    mb = batches(SHARP, B, T, 1, seed=77)
    g = gpu_step(SHARP, B, T, "bf16", p0, mb, lr=1e-3)
    o = oracle_step(SHARP, p0, mb, lr=1e-3)
    compare(SHARP, g, o, "bf16")
    gv, ov = tensor_views(lay, g["grads"]), tensor_views(lay, o["grads"])
    worst = max(rel_l2(gv[n], ov[n]) for n in gv if np.linalg.norm(ov[n]) > 0)
    assert worst <= 2.25e-2, worst

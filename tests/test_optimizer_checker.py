"""The element-wise clip + AdamW check (tests/optim_check.py) that the GPU test
applies, exercised on the CPU: the oracle's own fp32 instantiation passes it,
and each plausible mistake, planted in a CPU copy of the update, fails it in at
least one of the settings the GPU test runs (clip 1.0, 1e3 and 1e-3, steps 1
and 2, one 2-D and one 1-D tensor with zeroed gradients).

The update is the one of "Karpathy's four-hour GPT-2 reproduction in one
post", part 3: clip by global norm, AdamW (0.9, 0.95), eps 1e-8, decay on 2-D
tensors only.
"""
import numpy as np
import pytest

from optim_check import CLIPS, LR, WD, ZEROED, check_update, reference
from oracle import oracle
from transformer_lm_pretraining_gpt2_amd import synth
from transformer_lm_pretraining_gpt2_amd.config import CONFIGS

MODEL = CONFIGS["tiny"].model
B, T = 4, 64


def _views(layout, flat):
    return {e["name"]: flat[e["offset"]:e["offset"] + e["rows"] * (e["cols"] or 1)] for e in layout}


@pytest.fixture(scope="module")
def setup():
    lay = oracle.param_layout(MODEL)
    p0 = synth.init_params(lay, MODEL.n_layer, MODEL.vocab_size, dtype=np.float64)
    s = synth.uniform_stream(synth.stream_length(2, 1, B, T), MODEL.vocab_size, 7)
    grads = []
    for k in range(2):
        ids, tgt = synth.micro_batch(s, B, T, k)
        g = np.zeros_like(p0)
        oracle.fwd_bwd(MODEL, B, T, p0, ids, tgt, 1.0, g)
        grads.append(g)
    # the first step's gradients with one 2-D and one 1-D tensor zeroed
    gv = _views(lay, grads[0])
    for n in ZEROED:
        gv[n][:] = 0.0
    return lay, p0, grads


def _device_like(p0, g, m0, v0, step, clip):
    """What a correct fp32 device computes: the global norm summed in fp64 (a
    sequential fp32 sum of 470K squares is off by about 1e-4), the clip factor
    and the update in fp32 (the oracle's fp32 AdamW)."""
    p, g, m, v = (np.array(a, np.float32) for a in (p0, g, m0, v0))
    n = np.float32(oracle.grad_norm(g.astype(np.float64), R=np.float64))
    if n > np.float32(clip):
        g *= np.float32(clip) / n
    oracle.adamw(MODEL, p, g, m, v, step, LR, 0.9, 0.95, 1e-8, WD, R=np.float32)
    return dict(p=p, m=m, v=v, norm=float(n))


def _mutant(lay, p0, g, m0, v0, step, clip, mistake):
    """A CPU copy of the update with one mistake planted, rounded to fp32."""
    n_decay = sum(e["rows"] * e["cols"] for e in lay if e["decay"])
    g = np.asarray(g, np.float64)
    n = float(np.sqrt(np.sum(g * g)))
    s = clip / n if n > clip else 1.0
    if mistake == "clip_not_applied":
        s = 1.0
    if mistake == "clip_always":
        s = clip / n
    b1, b2, eps = 0.9, 0.95, 1e-8
    if mistake == "betas_swapped":
        b1, b2 = b2, b1
    gs = g * s
    m = b1 * m0 + (1 - b1) * gs
    v = b2 * v0 + (1 - b2) * (g * g * s if mistake == "clip_not_squared_in_v" else gs * gs)
    t = step + 1 if mistake == "bias_correction_wrong_step" else step
    bc1, bc2 = 1 - b1 ** t, 1 - b2 ** t
    if mistake == "no_bias_correction":
        bc1 = bc2 = 1.0
    mh, vh = m / bc1, v / bc2
    den = np.sqrt(vh + eps) if mistake == "eps_inside_sqrt" else np.sqrt(vh) + eps
    d = np.zeros_like(p0)
    d[:n_decay] = WD
    if mistake == "no_weight_decay":
        d[:] = 0.0
    if mistake == "decay_on_1d_tensors":
        d[:] = WD
    if mistake == "decay_not_scaled_by_lr":
        p = p0 - LR * mh / den - d * p0
    else:
        p = p0 - LR * (mh / den + d * p0)
    r = lambda a: np.asarray(a, np.float32).astype(np.float64)
    return dict(p=r(p), m=r(m), v=r(v), norm=n)


def _two_steps(lay, p0, grads, clip, update):
    """Runs `update` for steps 1 and 2 and checks each against the oracle."""
    fails = []
    m0 = np.zeros_like(p0)
    v0 = np.zeros_like(p0)
    state = dict(p=p0, m=m0, v=v0)
    for step, g in ((1, grads[0]), (2, grads[1])):
        got = update(state["p"], g, state["m"], state["v"], step, clip)
        ref = reference(MODEL, state["p"], g, state["m"], state["v"], step, LR, clip, WD)
        fails += [f"step {step}: {f}" for f in check_update(
            lay, state["p"], got, ref, lr=LR, wd=WD, zeroed=ZEROED if step == 1 else ())]
        state = {k: np.asarray(got[k], np.float64) for k in ("p", "m", "v")}
    return fails


@pytest.mark.parametrize("clip", CLIPS)
def test_correct_fp32_update_passes(setup, clip):
    lay, p0, grads = setup
    fails = _two_steps(lay, p0, grads, clip, _device_like)
    assert not fails, fails
    fails = _two_steps(lay, p0, grads, clip, lambda *a: _mutant(lay, *a, mistake=None))
    assert not fails, fails


MISTAKES = ["no_weight_decay", "decay_on_1d_tensors", "decay_not_scaled_by_lr", "no_bias_correction",
            "bias_correction_wrong_step", "eps_inside_sqrt", "betas_swapped", "clip_not_applied", "clip_always",
            "clip_not_squared_in_v"]


@pytest.mark.parametrize("mistake", MISTAKES)
def test_each_planted_mistake_is_caught(setup, mistake):
    lay, p0, grads = setup
    caught = {clip: _two_steps(lay, p0, grads, clip, lambda *a: _mutant(lay, *a, mistake=mistake)) for clip in CLIPS}
    print(mistake, {c: len(f) for c, f in caught.items()})
    assert any(caught.values()), mistake


def test_stale_bf16_copy_is_caught(setup):
    import torch

    lay, p0, grads = setup
    got = _device_like(p0, grads[0], np.zeros_like(p0), np.zeros_like(p0), 1, 1.0)
    ref = reference(MODEL, p0, grads[0], np.zeros_like(p0), np.zeros_like(p0), 1, LR, 1.0, WD)
    bf = lambda a: torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).to(torch.float32).numpy()
    assert not check_update(lay, p0, got, ref, lp=bf(got["p"]))
    assert check_update(lay, p0, got, ref, lp=bf(p0))

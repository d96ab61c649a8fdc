"""GPU pins of global-norm clipping and AdamW ("Karpathy's four-hour GPT-2
reproduction in one post", part 3: betas (0.9, 0.95), eps 1e-8, clip 1.0,
weight decay 0.1 on 2-D tensors only), through the C ABI.

Each case runs two optimizer steps of the tiny GPT-2 on the device.  Before the
first update the gradients of one 2-D tensor and one 1-D tensor are zeroed in
the caller's gradient buffer (the step-1 closed form: the 2-D tensor becomes
p0 (1 - lr wd), the 1-D tensor stays p0, both keep zero moments).  After each
update every parameter, both moments and the pre-clip norm are compared,
element by element, with the fp64 oracle's clip and AdamW applied to exactly
the gradients and state the device used (tests/optim_check.py gives the
bounds and the mistakes they exclude; tests/test_optimizer_checker.py shows on
the CPU that each of those mistakes fails them).  The clip settings cover both
branches: 1.0 and 1e-3 below the gradient norm (scale clip/n) and 1e3 above it
(scale 1).  In bf16 the bf16 parameter copy must equal the rounded updated
parameters, and the agreement of sign(dp) with the oracle's full step (its own
gradients) is reported.
"""
import numpy as np
import pytest

from gpu_common import batches
from optim_check import CLIPS, LR, WD, ZEROED, check_update, reference, sign_agreement
from oracle import oracle
from transformer_lm_pretraining_gpt2_amd import binding, synth
from transformer_lm_pretraining_gpt2_amd.config import CONFIGS

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(300)]

MODEL = CONFIGS["tiny"].model
B, T = CONFIGS["tiny"].B, CONFIGS["tiny"].T


def _views(layout, flat):
    return {e["name"]: flat[e["offset"]:e["offset"] + e["rows"] * (e["cols"] or 1)] for e in layout}


def _state(s):
    out = {k: getattr(s, k).cpu().numpy().astype(np.float64) for k in ("params", "grads", "m", "v")}
    out["p"] = out.pop("params")
    out["lp"] = s.params_lp.float().cpu().numpy() if s.params_lp is not None else None
    return out


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
@pytest.mark.parametrize("clip", CLIPS)
def test_clip_and_adamw_two_steps(prec, clip):
    import torch

    lay = binding.param_layout(MODEL)
    p0 = synth.init_params(lay, MODEL.n_layer, MODEL.vocab_size).astype(np.float32)
    mbs = batches(MODEL, B, T, 2, seed=11, data="uniform")
    s = binding.TrainStep(MODEL, B, T, prec)
    s.set_params(p0)
    norm = torch.zeros(1, device="cuda")
    loss = torch.zeros(1, device="cuda")
    prev = dict(p=p0.astype(np.float64), m=np.zeros(p0.size), v=np.zeros(p0.size))
    for step, (ids, tgt) in enumerate(mbs, start=1):
        print(f"[{prec} clip {clip}] step {step}", flush=True)
        s.forward(torch.from_numpy(ids.reshape(-1)).cuda(), torch.from_numpy(tgt.reshape(-1)).cuda(), loss)
        s.backward(0, 1)
        if step == 1:
            for e in lay:
                if e["name"] in ZEROED:
                    s.grads[e["offset"]:e["offset"] + e["rows"] * (e["cols"] or 1)].zero_()
        s.adamw_step(step, LR, 0.9, 0.95, 1e-8, WD, clip, norm)
        assert s.sync_status() == 0
        got = _state(s)
        got["norm"] = float(norm.item())
        ref = reference(MODEL, prev["p"], got["grads"], prev["m"], prev["v"], step, LR, clip, WD)
        print(f"  norm gpu {got['norm']:.6f} oracle {ref['norm']:.6f} (clip {clip}: "
              f"{'scaled' if ref['norm'] > clip else 'unscaled'})", flush=True)
        fails = check_update(lay, prev["p"], got, ref, lr=LR, wd=WD, zeroed=ZEROED if step == 1 else (),
                             lp=got["lp"])
        assert not fails, fails
        if step == 1:
            gv = _views(lay, got["grads"])
            assert all(np.all(gv[n] == 0) for n in ZEROED)  # the update leaves the gradient buffer alone
        if step == 1 and prec == "bf16" and clip == 1.0:
            # diagnostic: the direction of each parameter's first move against
            # the oracle's whole fp64 step (its own gradients, same zeroed tensors)
            g_or = np.zeros(p0.size)
            oracle.fwd_bwd(MODEL, B, T, p0.astype(np.float64), ids, tgt, 1.0, g_or)
            gov = _views(lay, g_or)
            for n in ZEROED:
                gov[n][:] = 0.0
            full = reference(MODEL, p0.astype(np.float64), g_or, np.zeros(p0.size), np.zeros(p0.size), 1, LR, clip, WD)
            agree, n_el = sign_agreement(got["p"] - prev["p"], full["p"] - prev["p"], g_or)
            print(f"  sign(dp) agreement with the oracle's fp64 step: {agree:.4f} over {n_el} elements", flush=True)
            assert agree >= 0.8
        prev = dict(p=got["p"], m=got["m"], v=got["v"])

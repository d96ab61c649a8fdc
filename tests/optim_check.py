"""Element-wise check of one clip + AdamW update against the fp64 oracle.

The update that "Karpathy's four-hour GPT-2 reproduction in one post" (part 3)
fixes: the gradients are scaled by clip/n when their global norm n exceeds
clip, then AdamW with betas (0.9, 0.95), eps 1e-8, bias correction, and
decoupled, learning-rate-scaled weight decay on the 2-D tensors only.

The reference is the oracle's clip and AdamW in fp64, applied to exactly the
gradients the device used (its gradient buffer, which the update leaves
unchanged) and to the device's parameters and moments before the update.  With
the same inputs the only differences left are fp32 rounding, so every element
is held to a bound of a few units in the last place:

  p:  |p1 - p_ref| <= 2 ulp32(p_ref) + 1e-5 |update terms|
  m:  |m1 - m_ref| <= 1e-5 (b1 |m0| + (1 - b1) |s g|) + 1e-30  (v likewise)
  n:  |n - n_ref|  <= 1e-5 n_ref                 (pre-clip global norm)

(s is the clip factor; the bounds scale with the terms each result sums, so
the cancellation of m's two terms at step 2 does not count as an error.)

A tensor whose gradient was zeroed before the update must follow the step-1
closed form: a 2-D tensor becomes p0 (1 - lr wd) (to 2 ulp), a 1-D tensor
stays p0 exactly, and both keep m = v = 0.

Plausible mistakes this excludes (tests/test_optimizer_checker.py plants each
in a CPU copy of the update and shows the check fails): weight decay dropped,
applied to the 1-D tensors too, or not scaled by the learning rate; bias
correction dropped, or taken at the wrong step; eps inside the square root;
the two betas swapped; the clip factor not applied, applied when n <= clip,
or applied to v only once (not squared); and, for the bf16 copy, a copy that
is not rewritten.
"""
import numpy as np

from oracle import oracle

B1, B2, EPS = 0.9, 0.95, 1e-8


def reference(model, p0, g, m0, v0, step, lr, clip, wd, b1=B1, b2=B2, eps=EPS):
    """fp64 oracle clip + AdamW on the given state; returns p, m, v, norm, and
    the magnitudes of the terms each result sums (mag_p, mag_m, mag_v), which
    scale the rounding bounds: at step 2 the two terms of m may cancel, so an
    fp32 result carries the rounding error of the terms, not of their sum."""
    g = np.array(g, dtype=np.float64)
    p = np.array(p0, dtype=np.float64)
    m = np.array(m0, dtype=np.float64)
    v = np.array(v0, dtype=np.float64)
    norm = oracle.clip_grads(g, clip, R=np.float64)  # g is now the clipped gradient
    oracle.adamw(model, p, g, m, v, step, lr, b1, b2, eps, wd, R=np.float64)
    mag_m = b1 * np.abs(np.asarray(m0, np.float64)) + (1 - b1) * np.abs(g)
    mag_v = b2 * np.asarray(v0, np.float64) + (1 - b2) * g * g
    mag_p = lr * (mag_m / (1 - b1 ** step) / (np.sqrt(v / (1 - b2 ** step)) + eps) + wd * np.abs(p0))
    return dict(p=p, m=m, v=v, norm=norm, mag_p=mag_p, mag_m=mag_m, mag_v=mag_v)


def _views(layout, flat):
    return {e["name"]: flat[e["offset"]:e["offset"] + e["rows"] * (e["cols"] or 1)] for e in layout}


def check_update(layout, p0, got, ref, lr=None, wd=None, zeroed=(), lp=None):
    """Failures (a list of strings; empty when the update matches).

    p0: parameters before the update; got/ref: dicts with p, m, v, norm (got
    in the device's precision, ref from `reference`); zeroed: names of tensors
    whose gradient was zero (closed form, needs lr and wd); lp: the device's
    bf16 parameter copy as float32 values, or None."""
    fails = []
    p0 = np.asarray(p0, np.float64)
    gp, rp = np.asarray(got["p"], np.float64), np.asarray(ref["p"], np.float64)
    ulp = np.spacing(np.abs(rp).astype(np.float32)).astype(np.float64)
    bound = 2 * ulp + 1e-5 * ref["mag_p"]
    err = np.abs(gp - rp)
    bad = err > bound
    if bad.any():
        i = int(np.argmax(err - bound))
        fails.append(f"p: {int(bad.sum())} elements off (worst at {i}: {gp[i]!r} vs {rp[i]!r}, p0 {p0[i]!r})")
    for k in ("m", "v"):
        a, b = np.asarray(got[k], np.float64), np.asarray(ref[k], np.float64)
        e = np.abs(a - b)
        bd = 1e-5 * ref["mag_" + k] + 1e-30
        if (e > bd).any():
            i = int(np.argmax(e - bd))
            fails.append(f"{k}: {int((e > bd).sum())} elements off (worst at {i}: {a[i]!r} vs {b[i]!r})")
    if abs(got["norm"] - ref["norm"]) > 1e-5 * ref["norm"]:
        fails.append(f"norm {got['norm']!r} vs {ref['norm']!r}")
    if zeroed:
        pv, p0v = _views(layout, gp), _views(layout, p0)
        mv, vv = _views(layout, np.asarray(got["m"])), _views(layout, np.asarray(got["v"]))
        dec = {e["name"]: e["decay"] for e in layout}
        for n in zeroed:
            if np.any(mv[n] != 0) or np.any(vv[n] != 0):
                fails.append(f"{n}: zero gradient but nonzero moments")
            if dec[n]:
                want = p0v[n] * (1.0 - lr * wd)
                tol = 2 * np.spacing(np.abs(want).astype(np.float32)).astype(np.float64)
                if np.any(np.abs(pv[n] - want) > tol):
                    fails.append(f"{n}: 2-D tensor with zero gradient is not p0 (1 - lr wd)")
            elif np.any(pv[n] != p0v[n]):
                fails.append(f"{n}: 1-D tensor with zero gradient changed")
    if lp is not None:
        import torch

        want = torch.from_numpy(np.asarray(got["p"], np.float32)).to(torch.bfloat16).to(torch.float32).numpy()
        if np.any(np.asarray(lp, np.float32) != want):
            fails.append("bf16 copy is not the rounded updated parameters")
    return fails


# The settings the GPU test runs (and the CPU test of the checker replays):
# clip 1.0 with the norm above it (scale clip/n), clip 1e3 above the norm
# (scale 1), clip 1e-3 far below it; each at step 1 and at step 2.
CLIPS = (1.0, 1e3, 1e-3)
LR, WD = 6e-4, 0.1
# the tensors whose gradient is zeroed before the first update: one 2-D, one 1-D
ZEROED = ("h.0.attn.c_proj.weight", "h.0.ln_1.weight")


def sign_agreement(dp_a, dp_b, g_ref, rel=1e-2):
    """Fraction of elements where two updates move the parameter the same way,
    over the elements whose reference gradient is not tiny (|g| above rel times
    the RMS gradient): AdamW's first step is about lr sign(g), so near-zero
    gradients may flip legitimately under bf16 rounding."""
    g = np.abs(np.asarray(g_ref, np.float64))
    keep = g > rel * np.sqrt(np.mean(g * g))
    sa, sb = np.sign(dp_a[keep]), np.sign(dp_b[keep])
    return float(np.mean(sa == sb)), int(keep.sum())

"""Helpers for the GPU parity tests: run one training step through the C ABI
and the same step through the CPU oracle, on the same seeded inputs."""
import numpy as np

from oracle import oracle
from transformer_lm_pretraining_gpt2_amd import binding, synth


def tensor_views(layout, flat):
    return {e["name"]: flat[e["offset"]:e["offset"] + e["rows"] * (e["cols"] or 1)] for e in layout}


def rel_l2(a, b):
    d = np.linalg.norm(np.asarray(a, np.float64) - np.asarray(b, np.float64))
    n = np.linalg.norm(np.asarray(b, np.float64))
    return d / n if n > 0 else d


def gpu_step(model, B, T, precision, params, micro_batches, step=1, lr=6e-4, clip=1.0, wd=0.1, handle=None):
    """One optimizer step on cuda:0.  Returns dict with per-micro-batch losses
    and row losses, grads (fp64 copy), params/m/v after the update, norm."""
    import torch

    K = len(micro_batches)
    s = handle or binding.TrainStep(model, B, T, precision)
    s.set_params(params.astype(np.float32))
    out = {"loss": [], "rows": []}
    for k, (ids, tgt) in enumerate(micro_batches):
        d_ids = torch.from_numpy(np.ascontiguousarray(ids, np.int32).reshape(-1)).cuda()
        d_tgt = torch.from_numpy(np.ascontiguousarray(tgt, np.int32).reshape(-1)).cuda()
        loss = torch.zeros(1, device="cuda")
        rows = torch.zeros(B * T, device="cuda")
        s.forward(d_ids, d_tgt, loss, rows)
        s.backward(k, K)
        out["loss"].append(loss)
        out["rows"].append(rows)
    norm = torch.zeros(1, device="cuda")
    s.adamw_step(step, lr, 0.9, 0.95, 1e-8, wd, clip, norm)
    out["status"] = s.sync_status()
    out["loss"] = [float(x.item()) for x in out["loss"]]
    out["rows"] = [x.cpu().numpy().astype(np.float64) for x in out["rows"]]
    out["grads"] = s.grads.cpu().numpy().astype(np.float64)
    out["params"] = s.params.cpu().numpy().astype(np.float64)
    out["m"] = s.m.cpu().numpy().astype(np.float64)
    out["v"] = s.v.cpu().numpy().astype(np.float64)
    out["norm"] = float(norm.item())
    out["handle"] = s
    return out


def oracle_step(model, params, micro_batches, step=1, lr=6e-4, clip=1.0, wd=0.1, R=np.float64):
    """The same step in the CPU oracle.  Grads are reported before clipping."""
    K = len(micro_batches)
    p = params.astype(R).copy()
    g = np.zeros_like(p)
    out = {"loss": [], "rows": []}
    for ids, tgt in micro_batches:
        B, T = ids.shape
        rl = np.zeros(B * T, dtype=R)
        out["loss"].append(oracle.fwd_bwd(model, B, T, p, ids, tgt, 1.0 / K, g, rl, R=R))
        out["rows"].append(rl.astype(np.float64))
    out["grads"] = g.astype(np.float64).copy()
    m = np.zeros_like(p)
    v = np.zeros_like(p)
    out["norm"] = oracle.clip_grads(g, clip, R=R)
    oracle.adamw(model, p, g, m, v, step, lr, 0.9, 0.95, 1e-8, wd, R=R)
    out["params"] = p.astype(np.float64)
    out["m"] = m.astype(np.float64)
    out["v"] = v.astype(np.float64)
    return out


def batches(model, B, T, K, seed, data="zipf", index0=0):
    n = synth.stream_length(1, K, B, T) + index0 * B * T
    stream = synth.zipf_stream(n, model.vocab_size, seed) if data == "zipf" else synth.uniform_stream(
        n, model.vocab_size, seed)
    return [synth.micro_batch(stream, B, T, index0 + k) for k in range(K)]

#!/usr/bin/env python3
"""Throughput of one GPT-2 training step on one MI355X.

A step is the whole path: K micro-steps of forward + backward (token and
position embedding, pre-LN attention/GELU blocks, tied head, fused
cross-entropy, and their gradients) followed by global-norm clipping and
AdamW, all in the HIP library.  Inputs are synthetic Zipf(s=1) token streams
already resident in device memory; weights are a random GPT-2 init.

Prints one JSON line: tokens/s (whole job, from the median step time; the
mean is reported beside it), MFU against the bf16 dense MFMA peak, the
roofline of the dominant kernel measured with HIP events around its launches
in steps of their own after the timed region (the timed steps carry no
per-kernel instrumentation), and the CPU oracle's throughput on a bounded
sample of the same workload.

Only one GPU is supported; --gpus > 1 exits with a message.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "training tokens/sec + MFU, GPT-2 124M bf16 B=16 T=1024, 1×MI355X"
# Per-kernel roofline: which kernel dominates the step (from the rocprofv3
# kernel-trace summary under profiles/) and how it is bounded.
DOMINANT = {"gpt2_124m": "gemm_tn_f32"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


# the sources each measured kernel is built from (its counters go stale when they change)
KERNEL_SOURCES = {"gemm_tn_f32": ("gemm.hip", "common.h"), "attn_bwd_dkv": ("attention.hip", "common.h")}


def kernel_source_hash(kernel="gemm_tn_f32"):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(kernel, ("gemm.hip", "attention.hip", "rowops.hip", "common.h")):
        with open(os.path.join(ROOT, "transformer_lm_pretraining_gpt2_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch (fetched + written) from the committed rocprofv3
    counter runs, or None when they are missing or were taken on a different
    kernel source (see transformer_lm_pretraining_gpt2_amd/traffic.py)."""
    try:
        with open(TRAFFIC_FILE) as fh:
            d = json.load(fh)
    except (OSError, ValueError):
        return None
    e = d.get(workload, {}).get(kernel)
    if not e or e.get("source_hash") != kernel_source_hash(kernel):
        return None
    return e.get("bytes_per_launch")


def host_cpu():
    """Model name of the host CPU, the CPUs this process may run on, and the
    threads the oracle's OpenMP loops use (OMP_NUM_THREADS when set, else one
    per available CPU)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or avail
    return model, avail, threads


def cpu_baseline(model, seed_stream, B, T, B_full):
    """The oracle (plain fp32 C++, not tuned) on a sample of the same workload:
    a full training step (forward, backward, clip, AdamW over all parameters)
    of B sequences of T tokens.  Its forward and backward cost is linear in the
    tokens, so the sample's tokens/s is also the full batch's, except that the
    update over all parameters is spread over fewer tokens (reported
    separately, with the full-batch rate it implies)."""
    import numpy as np

    from oracle import oracle
    from transformer_lm_pretraining_gpt2_amd import synth

    lay = oracle.param_layout(model)
    p = synth.init_params(lay, model.n_layer, model.vocab_size)
    ids, tgt = synth.micro_batch(seed_stream, B, T, 0)
    g = np.zeros_like(p)
    m = np.zeros_like(p)
    v = np.zeros_like(p)
    t0 = time.perf_counter()
    oracle.fwd_bwd(model, B, T, p, ids, tgt, 1.0, g, R=np.float32)
    t1 = time.perf_counter()
    oracle.clip_grads(g, 1.0, R=np.float32)
    oracle.adamw(model, p, g, m, v, 1, 6e-4, R=np.float32)
    t2 = time.perf_counter()
    cpu, avail, threads = host_cpu()
    full = B_full * T / ((t1 - t0) * B_full / B + (t2 - t1))
    return {"value": B * T / (t2 - t0), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"one full step on {B} sequences of {T} tokens of the same model (B={B}): fp32 forward+backward "
                      f"{t1 - t0:.1f} s, clip and AdamW over all {oracle.num_params(model)} parameters {t2 - t1:.1f} s",
            "full_batch_estimate": {"value": full, "B": B_full,
                                    "note": "forward+backward scaled linearly in tokens, one update"},
            "host_cpu": cpu, "nproc": avail, "threads": threads}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="gpt2_124m")
    ap.add_argument("--precision", default=None, help="fp32 or bf16 (default: the workload's)")
    ap.add_argument("--roofline-kernel", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-seqs", type=int, default=4,
                    help="sequences in the oracle's timed sample step (about 5 s each at 124M on 16 cores)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="before warmup, one plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--recompute", action="store_true",
                    help="activation recompute for the MLP (smaller workspace, one extra pass per layer)")
    ap.add_argument("--fp8", action="store_true",
                    help="forward products on FP8 E4M3 copies (per-row scales); reported as its own dtype")
    ap.add_argument("--no-overlap", action="store_true",
                    help="run the whole step on one stream (no second stream for the weight gradients)")
    ap.add_argument("--graph", action="store_true",
                    help="replay each micro-step's forward + backward from a captured HIP graph (AdamW eager)")
    ap.add_argument("--mode", choices=["train", "eval"], default="train",
                    help="eval: forward-only validation loss over held-out batches instead of the training step")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(data parallelism is a design note only).", file=sys.stderr)
        sys.exit(2)

    if args.mode == "eval":
        return run_eval(args)

    import numpy as np
    import torch

    from transformer_lm_pretraining_gpt2_amd import binding, synth
    from transformer_lm_pretraining_gpt2_amd.config import CONFIGS, MI355X_BF16_PEAK_FLOPS, MI355X_FP32_MFMA_PEAK_FLOPS
    from transformer_lm_pretraining_gpt2_amd.config import flops_per_token, lr_at

    rc = CONFIGS[args.config]
    model = rc.model
    prec = args.precision or rc.precision
    B, T, K = rc.B, rc.T, rc.K
    S, W = args.steps, args.warmup
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")

    step = binding.TrainStep(model, B, T, prec, device=dev, recompute=args.recompute, fp8=args.fp8)
    step.set_overlap(not args.no_overlap)
    lay = step.layout
    step.set_params(synth.init_params(lay, model.n_layer, model.vocab_size))
    RT, ISO = 3, 2  # steps after the timed region: the dominant kernel timed in the step, then alone
    n_tok = synth.stream_length(W + S + RT + ISO, K, B, T)
    stream = synth.zipf_stream(n_tok, model.vocab_size) if rc.data == "zipf" else synth.uniform_stream(
        n_tok, model.vocab_size)
    # every micro-batch of the run, resident in HBM before timing starts
    nmb = (W + S + RT + ISO) * K
    ids_all = np.empty((nmb, B * T), np.int32)
    tgt_all = np.empty((nmb, B * T), np.int32)
    for i in range(nmb):
        a, b = synth.micro_batch(stream, B, T, i)
        ids_all[i], tgt_all[i] = a.reshape(-1), b.reshape(-1)
    d_ids = torch.from_numpy(ids_all).to(dev)
    d_tgt = torch.from_numpy(tgt_all).to(dev)
    loss = torch.zeros(1, device=dev)
    norm = torch.zeros(1, device=dev)

    graphs = {}
    if args.graph:
        # One graph per kind of micro-step (the first overwrites the
        # gradients, later ones add), captured on torch's capture stream; the
        # graphs read the micro-batch from fixed buffers, refilled before each
        # replay.  Capturing enqueues nothing.
        g_ids = torch.empty(B * T, dtype=torch.int32, device=dev)
        g_tgt = torch.empty(B * T, dtype=torch.int32, device=dev)
        home = step.stream
        for acc in ((0, 1) if K > 1 else (0,)):
            graphs[acc] = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graphs[acc]):
                step.set_stream(torch.cuda.current_stream())
                step.forward(g_ids, g_tgt, loss)
                step.backward(acc, K)
            step.set_stream(home)

    def one_step(s, graph=False):
        for k in range(K):
            i = s * K + k
            if graph:
                g_ids.copy_(d_ids[i])
                g_tgt.copy_(d_tgt[i])
                graphs[min(k, 1)].replay()
            else:
                step.forward(d_ids[i], d_tgt[i], loss)
                step.backward(k, K)
        step.adamw_step(s + 1, lr_at(s, rc.max_lr, rc.warmup, rc.max_steps), rc.beta1, rc.beta2, rc.eps,
                        rc.weight_decay, rc.grad_clip, norm)

    if args.copy_mib:
        n = args.copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for s in range(W):
        one_step(s, args.graph)
    st = step.sync_status()
    if st != 0:
        raise SystemExit(f"warmup step failed: {binding.ERRORS.get(st, st)}")
    first_loss = loss.item()

    # The timed steps carry no per-kernel instrumentation: only one event on
    # the caller's stream at each step boundary (for the median).
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(S + 1)]
    t0 = time.perf_counter()
    evs[0].record()
    for j, s in enumerate(range(W, W + S)):
        one_step(s, args.graph)
        evs[j + 1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    st = step.sync_status()
    if st != 0:
        raise SystemExit(f"timed step failed: {binding.ERRORS.get(st, st)}")
    step_ms = sorted(evs[j].elapsed_time(evs[j + 1]) for j in range(S))
    median_ms = step_ms[S // 2] if S % 2 else 0.5 * (step_ms[S // 2 - 1] + step_ms[S // 2])
    # The dominant kernel, timed afterwards in steps of their own: with HIP
    # events around each of its launches on the stream it runs on, in the same
    # overlapped schedule, then with overlap off (the kernel alone).
    kname = args.roofline_kernel or DOMINANT.get(args.config, "gemm_tn_f32")
    step.timing_enable(kname, True)
    step.timing_read()
    for s in range(W + S, W + S + RT):
        one_step(s)
    k_ms, k_launches, k_flops = step.timing_read()
    step.set_overlap(False)
    for s in range(W + S + RT, W + S + RT + ISO):
        one_step(s)
    torch.cuda.synchronize()
    i_ms, i_launches, i_flops = step.timing_read()
    step.set_overlap(not args.no_overlap)
    step.timing_enable(kname, False)
    st = step.sync_status()
    if st != 0:
        raise SystemExit(f"roofline step failed: {binding.ERRORS.get(st, st)}")

    wall_ms = (t1 - t0) * 1000 / S
    ev_ms = evs[0].elapsed_time(evs[S]) / S
    mean_ms = max(wall_ms, ev_ms)
    ms = median_ms
    tokens = K * B * T
    tps = tokens / (ms / 1000)
    fpt = flops_per_token(model, T, causal=True)
    peak = MI355X_BF16_PEAK_FLOPS if prec == "bf16" else MI355X_FP32_MFMA_PEAK_FLOPS
    mfu = tps * fpt / peak

    roof = None
    if k_launches:
        achieved = k_flops / (k_ms / 1000)
        traffic = measured_traffic(kname, args.config)
        roof = {"kernel": kname, "bound": "mfma", "achieved": round(achieved / 1e12, 2), "peak": round(peak / 1e12, 1),
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic,
                "avg_launch_us": round(1000 * k_ms / k_launches, 2), "launches_per_step": k_launches / RT,
                "flops_per_launch": k_flops / k_launches,
                "note": f"{RT} steps after the timed region, same schedule, with HIP events around each launch of "
                        "this kernel on the stream it runs on"}
        if i_launches:
            ia = i_flops / (i_ms / 1000)
            roof["isolated"] = {"achieved": round(ia / 1e12, 2), "frac": round(ia / peak, 4),
                                "avg_launch_us": round(1000 * i_ms / i_launches, 2), "steps": ISO,
                                "note": "same kernel with overlap off (nothing runs beside it)"}

    out = {
        "metric": (METRIC if args.config == "gpt2_124m" and not args.fp8 else
                   f"training tokens/sec + MFU, {args.config}" + (" (FP8 E4M3 forward products)" if args.fp8 else "")),
        "value": round(tps, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": S,
        "warmup": W,
        "ms_per_step": round(ms, 3),
        "ms_per_step_median": round(median_ms, 3),
        "ms_per_step_mean": round(mean_ms, 3),
        "ms_per_step_min": round(step_ms[0], 3),
        "ms_per_step_max": round(step_ms[-1], 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "mfu": round(mfu, 4),
        "tflops": round(tps * fpt / 1e12, 1),
        "flops_per_token": fpt,
        "flops_per_token_noncausal": flops_per_token(model, T, causal=False),
        "dtype": "fp8 e4m3 forward products, bf16 backward" if args.fp8 else prec,
        "data": f"synthetic: {'Zipf(s=1.0)' if rc.data == 'zipf' else 'uniform'} token ids over {model.vocab_size}, "
                f"seed {synth.DATA_SEED}; random GPT-2 init, seed {synth.INIT_SEED}",
        "config": {"workload": f"{args.config}: one training step (fwd+bwd+clip+AdamW), B={B} T={T} K={K}, "
                               f"L={model.n_layer} nh={model.n_head} C={model.n_embd} V={model.vocab_size}"
                               f"->{model.padded_vocab_size}",
                   "global_batch": B * K, "seq_len": T, "grad_accum": K, "parallelism": "none (1 GPU)",
                   "activation_recompute": bool(args.recompute), "fp8_forward": bool(args.fp8),
                   "two_streams": not args.no_overlap, "hip_graph": bool(args.graph),
                   "workspace_bytes": int(step.workspace.numel())},
        "roofline": roof,
        "loss_first_timed": round(first_loss, 4),
        "loss_last": round(loss.item(), 4),
        "context": {"a100_pytorch_124m_tok_s": 182000,
                    "note": "pages' single-A100 figure (PyTorch, bf16, compile, flash attention); context only"},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(model, stream, min(args.cpu_sample_seqs, B), T, B * K)
    print(json.dumps(out), flush=True)


def run_eval(args):
    """Forward-only validation: S held-out micro-batches (a stream of its own
    seed) through gpt2_eval after W warmup batches; tokens/s of the timed
    batches, and the mean loss and perplexity they give."""
    import numpy as np
    import torch

    from transformer_lm_pretraining_gpt2_amd import binding, evaluation, synth
    from transformer_lm_pretraining_gpt2_amd.config import CONFIGS, MI355X_BF16_PEAK_FLOPS, MI355X_FP32_MFMA_PEAK_FLOPS
    from transformer_lm_pretraining_gpt2_amd.config import flops_per_token

    rc = CONFIGS[args.config]
    model, prec, B, T = rc.model, args.precision or rc.precision, rc.B, rc.T
    S, W = args.steps, args.warmup
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    step = binding.TrainStep(model, B, T, prec, device=dev)
    step.set_params(synth.init_params(step.layout, model.n_layer, model.vocab_size))
    n = synth.stream_length(W + S, 1, B, T)
    val_seed = synth.DATA_SEED + 1
    stream = synth.zipf_stream(n, model.vocab_size, val_seed) if rc.data == "zipf" else synth.uniform_stream(
        n, model.vocab_size, val_seed)
    mbs = [synth.micro_batch(stream, B, T, i) for i in range(W + S)]
    d = [(torch.from_numpy(a.reshape(-1)).to(dev), torch.from_numpy(b.reshape(-1)).to(dev)) for a, b in mbs]
    losses = torch.zeros(W + S, device=dev)
    for i in range(W):
        step.evaluate(d[i][0], d[i][1], losses[i:i + 1])
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for i in range(W, W + S):
        step.evaluate(d[i][0], d[i][1], losses[i:i + 1])
    ev1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    st = step.sync_status()
    if st != 0:
        raise SystemExit(f"eval failed: {binding.ERRORS.get(st, st)}")
    ms = max((t1 - t0) * 1000 / S, ev0.elapsed_time(ev1) / S)
    tps = B * T / (ms / 1000)
    fpt = flops_per_token(model, T, causal=True) / 3  # forward only: a third of 6N + 6LTC
    peak = MI355X_BF16_PEAK_FLOPS if prec == "bf16" else MI355X_FP32_MFMA_PEAK_FLOPS
    vl = float(np.mean(losses[W:].cpu().numpy().astype(np.float64)))
    out = {
        "metric": f"validation tokens/sec (forward-only loss), {args.config} {prec} B={B} T={T}, 1×MI355X",
        "value": round(tps, 1), "unit": "tokens/s", "n_gpus": 1, "steps": S, "warmup": W,
        "ms_per_step": round(ms, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "mfu": round(tps * fpt / peak, 4), "flops_per_token": fpt, "dtype": prec,
        "data": f"synthetic held-out stream: {'Zipf(s=1.0)' if rc.data == 'zipf' else 'uniform'} token ids, "
                f"seed {val_seed}; random GPT-2 init, seed {synth.INIT_SEED}",
        "config": {"workload": f"{args.config}: forward-only evaluation of one micro-batch, B={B} T={T}",
                   "global_batch": B, "seq_len": T, "parallelism": "none (1 GPU)"},
        "val_loss": round(vl, 4), "perplexity": round(evaluation.perplexity(vl), 2),
        "val_bpb": None, "val_bpb_note": "bits per byte needs the tokenizer's bytes per token; synthetic ids have none",
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

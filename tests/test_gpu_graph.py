"""A micro-step captured into a HIP graph (forward + backward through the C
ABI on torch's capture stream) and replayed over several optimizer steps
equals the same steps run eagerly, bit for bit.

Between replays the program does its own eager work on the same stream
(refilling the graph's input buffers, the AdamW update, which takes the step
and learning rate by value) and synchronises; every replay's loss, and the
gradients and parameters after every step, are compared with the eager run.
With gradient accumulation there are two graphs: the first micro-step
overwrites the gradients, later ones add onto them."""
import numpy as np
import pytest

from gpu_common import batches
from transformer_lm_pretraining_gpt2_amd import binding, synth
from transformer_lm_pretraining_gpt2_amd.config import CONFIGS

STEPS = 3


@pytest.mark.gpu
@pytest.mark.parametrize("name,prec,K", [("tiny", "fp32", 1), ("tiny", "bf16", 2), ("small", "bf16", 2)])
def test_captured_micro_step_replays_equal_eager(name, prec, K):
    import torch

    rc = CONFIGS[name]
    model, B, T = rc.model, rc.B, rc.T
    mbs = batches(model, B, T, STEPS * K, seed=77, data=rc.data)
    d_ids = [torch.from_numpy(np.ascontiguousarray(a, np.int32).reshape(-1)).cuda() for a, _ in mbs]
    d_tgt = [torch.from_numpy(np.ascontiguousarray(b, np.int32).reshape(-1)).cuda() for _, b in mbs]
    p0 = synth.init_params(binding.param_layout(model), model.n_layer, model.vocab_size)
    ids = torch.zeros(B * T, dtype=torch.int32, device="cuda")
    tgt = torch.zeros(B * T, dtype=torch.int32, device="cuda")
    loss = torch.zeros(1, device="cuda")
    norm = torch.zeros(1, device="cuda")

    def handle():
        s = binding.TrainStep(model, B, T, prec)
        s.set_params(p0)
        return s

    def update(s, step):
        s.adamw_step(step + 1, 1e-3, 0.9, 0.95, 1e-8, 0.1, 1.0, norm)

    print(f"[{name} {prec} K={K}] eager steps", flush=True)
    E = handle()
    eager = []
    for step in range(STEPS):
        losses = []
        for k in range(K):
            ids.copy_(d_ids[step * K + k])
            tgt.copy_(d_tgt[step * K + k])
            E.forward(ids, tgt, loss)
            E.backward(k, K)
            losses.append(loss.item())
        grads = E.grads.clone()
        update(E, step)
        torch.cuda.synchronize()
        eager.append((losses, grads, E.params.clone()))
    assert E.sync_status() == 0

    print(f"[{name} {prec} K={K}] capture", flush=True)
    G = handle()
    home = G.stream
    graphs = {}
    for acc in ((0, 1) if K > 1 else (0,)):
        graphs[acc] = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graphs[acc]):
            G.set_stream(torch.cuda.current_stream())
            G.forward(ids, tgt, loss)
            G.backward(acc, K)
        G.set_stream(home)
    torch.cuda.synchronize()

    for step in range(STEPS):
        print(f"[{name} {prec} K={K}] replay step {step}", flush=True)
        losses = []
        for k in range(K):
            ids.copy_(d_ids[step * K + k])
            tgt.copy_(d_tgt[step * K + k])
            graphs[min(k, 1)].replay()
            torch.cuda.synchronize()
            losses.append(loss.item())
        grads = G.grads.clone()
        update(G, step)
        torch.cuda.synchronize()
        e_losses, e_grads, e_params = eager[step]
        assert losses == e_losses, (step, losses, e_losses)
        assert torch.equal(grads, e_grads), step
        assert torch.equal(G.params, e_params), step
    assert G.sync_status() == 0

"""The fwd+bwd step (preallocated workspace, saved buffer, outputs and gradients) captured into
a HIP graph: the library enqueues only kernels on the caller's stream (no allocation, memset or
synchronisation), so the captured step must reproduce the eager step bit for bit on every
replay, with eager work and synchronisations between the replays."""
import numpy as np
import pytest
import torch

from workloads import make_inputs, workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def E():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import delta_rule_sequence_amd as mod
    mod._lib.lib()
    return mod


@pytest.mark.parametrize("gated", [False, True])
def test_graph_replay_matches_eager(E, gated):
    w = workload(2, B=2, H=4, T=64 * 9 + 17)
    inp = make_inputs(w, with_grad=True)
    dev = torch.device("cuda")
    q, k, v, beta, do = (torch.from_numpy(inp[n]).to(dev, torch.bfloat16) for n in ("q", "k", "v", "beta", "do"))
    gate = torch.from_numpy(-np.logaddexp(0.0, -(np.random.default_rng(3).standard_normal(beta.shape) + 2.0))
                            .astype(np.float32)).to(dev, torch.bfloat16)
    p = E.make_problem(q, k, v, beta)
    o = torch.empty_like(v)
    saved = torch.empty(E.efla_saved_bytes(p), dtype=torch.uint8, device=dev)
    ws = torch.empty(max(E.efla_workspace_bytes(p, False), E.efla_workspace_bytes(p, True)),
                     dtype=torch.uint8, device=dev)
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(beta))
    if gated:
        grads = grads + (torch.empty_like(gate),)

    def step():
        if gated:
            E.efla_fwd_gated(q, k, v, beta, gate, 0.9, None, True, ws, o=o, saved=saved)
            E.efla_bwd_gated(q, k, v, beta, gate, do, saved, 0.9, None, ws, grads=grads)
        else:
            E.efla_fwd(q, k, v, beta, 0.9, None, True, ws, o=o, saved=saved)
            E.efla_bwd(q, k, v, beta, do, saved, 0.9, None, ws, grads=grads)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # first calls (kernel attributes) outside the capture
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = [o.clone()] + [t.clone() for t in grads]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in [o] + list(grads):
            t.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip([o] + list(grads), ref)):
            assert torch.equal(a, b), "replay %d, tensor %d differs from the eager step" % (rep, i)
        step()  # eager work between replays
        torch.cuda.synchronize()
        for a, b in zip([o] + list(grads), ref):
            assert torch.equal(a, b)

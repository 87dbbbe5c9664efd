"""Ragged and packed problems wide enough for the scans' 32-column tiling.

With d_v = 128 the scans use 32-column workgroups once sequences x heads reach 64; that tiling's
backward scan is fed by LDS DMA and clears the rows past the end of a partial chunk itself, and
the small parity problems never reach it. These cases do, for d_k = 128 and d_k = 64: a dense
batch whose length is not a multiple of the chunk, and a packed batch with a one-token sequence
and ragged tails, in plain and gated EFLA, forward (saving) and backward, with every
(sequence, head) stream compared against the fp64 oracle (streams are independent, so the
oracle is exact for each of them).
"""
import numpy as np
import pytest
import torch

from oracle_streams import assert_streams, compare_streams
from workloads import make_inputs, workload

pytestmark = pytest.mark.gpu

TOL = 2e-2  # bf16, normwise per tensor and stream, as in the other parity tests

CASES = [
    ("dense_T150", 2, dict(B=4, H=16, T=150), None),
    ("packed", 5, dict(H=16), [150, 64, 1, 100, 300]),
    ("dense_T150_dk64", 2, dict(B=4, H=16, T=150, dk=64), None),
    ("packed_dk64", 5, dict(H=16, dk=64), [150, 64, 1, 100, 300]),
]


@pytest.fixture(scope="module")
def E():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import delta_rule_sequence_amd as mod
    mod._lib.lib()
    return mod


def _dev(x, dt=torch.bfloat16):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda", dtype=dt)


@pytest.mark.parametrize("gated", [False, True], ids=["plain", "gated"])
@pytest.mark.parametrize("name,idx,over,lengths", CASES, ids=[c[0] for c in CASES])
def test_wide_ragged(E, name, idx, over, lengths, gated):
    w = workload(idx, **over)
    inp = make_inputs(w, with_grad=True, lengths=lengths)
    B, H, T, _ = inp["k"].shape
    assert (B if inp["cu_seqlens"] is None else len(inp["cu_seqlens"]) - 1) * H >= 64
    print("%s (%s): B=%d H=%d T=%d" % (name, "gated" if gated else "plain", B, H, T), flush=True)
    q, k, v, beta, do = (_dev(inp[n]) for n in ("q", "k", "v", "beta", "do"))
    cu_np = inp["cu_seqlens"]
    cu = None if cu_np is None else torch.from_numpy(cu_np).cuda()
    if gated:
        x = np.random.default_rng(99).standard_normal((B, H, T)) + 3.0
        a = (-np.logaddexp(0.0, -x)).astype(np.float32)
        a = torch.from_numpy(a).to(torch.bfloat16).float().numpy()  # the values the GPU sees
        g = _dev(a)
        o, saved = E.efla_fwd_gated(q, k, v, beta, g, 1.0, cu, save=True)
        grads = E.efla_bwd_gated(q, k, v, beta, g, do, saved, 1.0, cu)
        names = ("dq", "dk", "dv", "dbeta", "dgate")
    else:
        o, saved = E.efla_fwd(q, k, v, beta, 1.0, cu, save=True)
        grads = E.efla_bwd(q, k, v, beta, do, saved, 1.0, cu)
        names = ("dq", "dk", "dv", "dbeta")
    torch.cuda.synchronize()
    gpu = {"o": o.float().cpu().numpy()}
    gpu.update({nm: t.float().cpu().numpy() for nm, t in zip(names, grads)})
    res = compare_streams(inp, gpu, True, gate=a if gated else None)
    assert_streams(res, TOL)

"""efla_fwd_noalloc: the forward for callers that cannot allocate, through the C ABI.

Its output (and final state) must equal what efla_fwd_state computes with a caller-given
workspace and no saved buffer: the same kernels run in the same order, so the comparison is
bit for bit, and both are within the bf16 / fp32 tolerance of the fp64 oracle. Calls run back
to back on one stream, each later one smaller than the one before, so every call finds the
previous call's leftovers in the static workspace.
"""
import ctypes

import numpy as np
import pytest
import torch

from delta_rule_sequence_amd import _lib
from oracle import efla_oracle as O
from workloads import make_inputs, workload

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
TDT = {"f32": torch.float32, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def L():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import delta_rule_sequence_amd  # noqa: F401
    return _lib.lib()


def _dev(x, dt):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda", dtype=dt)


def _vp(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _run_both(L, inp, dtype, with_state):
    """(o, ht) from efla_fwd_noalloc and from efla_fwd_state with its own workspace."""
    dt = TDT[dtype]
    q, k, v, beta = (_dev(inp[n], dt) for n in ("q", "k", "v", "beta"))
    B, H, T, dk = inp["k"].shape
    dv = inp["v"].shape[-1]
    cu = None if inp["cu_seqlens"] is None else torch.from_numpy(inp["cu_seqlens"]).cuda()
    n_state = B if cu is None else len(inp["cu_seqlens"]) - 1
    p = _lib.problem(B, H, T, dk, dv, _lib.EFLA_F32 if dtype == "f32" else _lib.EFLA_BF16, 1.0,
                     None if cu is None else cu.data_ptr(), 0 if cu is None else n_state)
    h0 = ht_a = ht_b = None
    if with_state:
        h0 = _dev(np.random.default_rng(3).standard_normal((n_state, H, dk, dv)) * 0.2, torch.float32)
        ht_a = torch.empty_like(h0)
        ht_b = torch.empty_like(h0)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    o_a = torch.empty_like(v)
    _lib.check("efla_fwd_noalloc", L.efla_fwd_noalloc(ctypes.byref(p), _vp(q), _vp(k), _vp(v), _vp(beta),
                                                     _vp(h0), _vp(o_a), _vp(ht_a), st))
    o_b = torch.empty_like(v)
    ws_n = int(L.efla_workspace_bytes(ctypes.byref(p), 0))
    assert 0 < ws_n <= _lib.NOALLOC_WS_BYTES
    ws = torch.empty(ws_n, dtype=torch.uint8, device="cuda")
    _lib.check("efla_fwd_state", L.efla_fwd_state(ctypes.byref(p), _vp(q), _vp(k), _vp(v), _vp(beta),
                                                 _vp(h0), _vp(o_b), _vp(ht_b), None, 0, _vp(ws), ws_n, st))
    torch.cuda.synchronize()
    return o_a, o_b, ht_a, ht_b, (None if h0 is None else h0.cpu().numpy().astype(np.float64))


CASES = [  # run in this order, each call smaller than the one before
    ("bf16_segmented", 2, dict(B=1, H=4, T=64 * 40 + 9), None, True),   # 2 segments per sequence
    ("bf16_dense", 2, dict(B=2, H=3, T=700), None, True),
    ("bf16_packed", 5, dict(H=2), [200, 1, 64, 0, 90], True),
    ("f32_small", 4, dict(B=1, H=2, T=150), None, False),
]


def test_noalloc_matches_efla_fwd_state(L):
    sizes = []
    for name, idx, over, lengths, with_state in CASES:
        w = workload(idx, **over)
        inp = make_inputs(w, with_grad=False, lengths=lengths)
        print("%s: %s lengths=%s" % (name, tuple(inp["k"].shape), lengths), flush=True)
        o_a, o_b, ht_a, ht_b, h0 = _run_both(L, inp, w.dtype, with_state)
        assert torch.equal(o_a, o_b), name
        if with_state:
            assert torch.equal(ht_a, ht_b), name
        ref_o, ref_ht = O.forward(inp["q"], inp["k"], inp["v"], inp["beta"],
                                  cu_seqlens=inp["cu_seqlens"], initial_state=h0)
        err = O.rel_err(o_a.float().cpu().numpy(), ref_o)
        print("  o rel err %.3e" % err, flush=True)
        assert np.all(np.isfinite(o_a.float().cpu().numpy())) and err <= TOL[w.dtype], name
        if with_state:
            assert O.rel_err(ht_a.cpu().numpy(), ref_ht) <= TOL[w.dtype], name
        sizes.append(o_a.numel())
    assert all(a > b for a, b in zip(sizes, sizes[1:]))


def test_noalloc_rejects_problems_beyond_its_workspace(L):
    """A problem whose forward workspace exceeds the static array is refused, nothing launched."""
    p = _lib.problem(1, 16, 32768, 128, 128, _lib.EFLA_BF16)
    assert L.efla_workspace_bytes(ctypes.byref(p), 0) > _lib.NOALLOC_WS_BYTES
    t = torch.empty(16, dtype=torch.uint8, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert L.efla_fwd_noalloc(ctypes.byref(p), _vp(t), _vp(t), _vp(t), _vp(t), None, _vp(t), None, st) == 5

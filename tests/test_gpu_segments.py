"""GPU parity of the segment-parallel forward scan (long sequences cut into segments whose
transitions and zero-start states are formed in parallel, then chained), through the C ABI,
against the fp64 oracle: outputs, final states, and gradients computed from the buffer the
segmented forward saved. Tolerances as in test_gpu_parity (normwise, 1e-4 fp32, 2e-2 bf16)."""
import numpy as np
import pytest
import torch

from oracle import efla_oracle as O
from workloads import make_inputs, workload

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
TDT = {"f32": torch.float32, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def E():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import delta_rule_sequence_amd as mod
    mod._lib.lib()
    return mod


def _dev(x, dt):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda", dtype=dt)


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _check(name, gpu, ref, tol):
    err = O.rel_err(gpu, ref)
    print("  %-6s normwise rel err %.3e (tol %.0e)" % (name, err, tol), flush=True)
    assert np.all(np.isfinite(gpu)), name + " has non-finite values"
    assert err <= tol, "%s: %.3e > %.0e" % (name, err, tol)


# (name, workload overrides, segments): ragged tails, one chunk per segment, uneven splits
CASES = [
    ("bf16_T2373_seg2", dict(idx=2, B=2, H=2, T=64 * 37 + 5), 2),
    ("bf16_T2373_seg5", dict(idx=2, B=2, H=2, T=64 * 37 + 5), 5),
    ("bf16_T2373_chunkwise", dict(idx=2, B=1, H=2, T=64 * 37 + 5), 64),
    ("f32_T1280_seg4", dict(idx=4, B=1, H=2, T=64 * 20), 4),
    ("bf16_dk64_dv128", dict(idx=2, B=1, H=3, T=64 * 12 + 40, dk=64, dv=128), 3),
    ("bf16_dk128_dv64", dict(idx=2, B=1, H=3, T=64 * 12 + 40, dk=128, dv=64), 3),
    ("bf16_dk64_dv64", dict(idx=2, B=2, H=1, T=64 * 12 + 40, dk=64, dv=64), 3),
]


@pytest.mark.parametrize("name,wl,segments", CASES, ids=[c[0] for c in CASES])
def test_segmented_forward_and_saved_backward(E, name, wl, segments):
    wl = dict(wl)
    w = workload(wl.pop("idx"), **wl)
    inp = make_inputs(w, with_grad=True)
    dt, tol = TDT[w.dtype], TOL[w.dtype]
    B, H, T, dk = inp["k"].shape
    dv = inp["v"].shape[-1]
    q, k, v, beta, do = (_dev(inp[n], dt) for n in ("q", "k", "v", "beta", "do"))
    r = np.random.default_rng(5)
    h0 = (r.standard_normal((B, H, dk, dv)) * 0.3).astype(np.float32)
    h0_d = _dev(h0, torch.float32)
    print("%s: B=%d H=%d T=%d dk=%d dv=%d segments=%d" % (name, B, H, T, dk, dv, segments), flush=True)
    o, saved, ht = E.efla_fwd(q, k, v, beta, 0.8, None, save=True, initial_state=h0_d,
                              final_state=True, segments=segments)
    g = E.efla_bwd(q, k, v, beta, do, saved, 0.8, None, initial_state=h0_d, segments=segments)
    torch.cuda.synchronize()
    ref_o, ref_ht = O.forward(inp["q"], inp["k"], inp["v"], inp["beta"], scale=0.8,
                              initial_state=h0)
    _check("o", _np(o), ref_o, tol)
    _check("ht", _np(ht), ref_ht, tol)
    ref = O.backward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["do"], scale=0.8,
                     initial_state=h0)
    for nm, t in zip(("dq", "dk", "dv", "dbeta"), g):
        _check(nm, _np(t), ref[nm], tol)
    # the split changes nothing but rounding: same outputs as the sequential scan
    o1, _, ht1 = E.efla_fwd(q, k, v, beta, 0.8, None, save=False, initial_state=h0_d,
                            final_state=True, segments=1)
    torch.cuda.synchronize()
    assert O.rel_err(_np(o), _np(o1)) <= tol / 2
    assert O.rel_err(_np(ht), _np(ht1)) <= tol / 2


def test_segmented_recompute_backward(E):
    """efla_bwd without a saved buffer recomputes the forward with the same segment plan."""
    w = workload(2, B=1, H=2, T=64 * 29 + 17)
    inp = make_inputs(w, with_grad=True)
    q, k, v, beta, do = (_dev(inp[n], torch.bfloat16) for n in ("q", "k", "v", "beta", "do"))
    g = E.efla_bwd(q, k, v, beta, do, None, 1.0, None, segments=6)
    torch.cuda.synchronize()
    ref = O.backward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["do"])
    for nm, t in zip(("dq", "dk", "dv", "dbeta"), g):
        _check(nm, _np(t), ref[nm], TOL["bf16"])


def test_segmented_euler_mode(E):
    """The split is algebra on the chunk maps, so the delta rule goes through it unchanged."""
    w = workload(2, B=1, H=2, T=64 * 24)
    inp = make_inputs(w, with_grad=False)
    kk = inp["k"] / np.maximum(np.linalg.norm(inp["k"], axis=-1, keepdims=True), 1e-30)
    from workloads import round_to_bf16
    inp["k"] = round_to_bf16(kk.astype(np.float32))
    q, k, v, beta = (_dev(inp[n], torch.bfloat16) for n in ("q", "k", "v", "beta"))
    o, _ = E.efla_fwd(q, k, v, beta, 1.0, None, save=False, mode="euler", segments=4)
    torch.cuda.synchronize()
    ref_o, _ = O.forward(inp["q"], inp["k"], inp["v"], inp["beta"], mode="euler")
    _check("o", _np(o), ref_o, TOL["bf16"])


BWD_CASES = [  # name, workload overrides, segments, mode
    ("bf16_seg2", dict(idx=2, B=1, H=2, T=64 * 33 + 7), 2, "exact"),
    ("bf16_seg5", dict(idx=2, B=2, H=1, T=64 * 37 + 5), 5, "exact"),
    ("bf16_seg_per_chunk", dict(idx=2, B=1, H=1, T=64 * 9 + 30), 64, "exact"),
    ("f32_seg3", dict(idx=4, B=1, H=2, T=64 * 20 + 3), 3, "exact"),
    ("bf16_dk64_dv128", dict(idx=2, B=1, H=2, T=64 * 12 + 40, dk=64, dv=128), 3, "exact"),
    ("bf16_dk128_dv64", dict(idx=2, B=1, H=2, T=64 * 12 + 40, dk=128, dv=64), 3, "exact"),
    ("bf16_delta_rule", dict(idx=2, B=1, H=2, T=64 * 16), 4, "euler"),
    # 4 segments x 16 heads: wide enough for the 32-column tiling, whose state-only and full
    # reverse scans are DMA-fed (the unsegmented comparison runs the 16-column tiling)
    ("bf16_wide_seg4", dict(idx=2, B=1, H=16, T=64 * 20 + 7), 4, "exact"),
]


@pytest.mark.parametrize("name,wl,segments,mode", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_segmented_backward_with_state_gradients(E, name, wl, segments, mode):
    """Segment-parallel reverse scan (zero-start gradients of all segments, the chain from the
    last segment to the first with the transposed transitions the segment-parallel forward
    saved, then the full scan from each segment's incoming gradient): every gradient, including
    the one arriving at the final state and the one leaving the initial state, against the
    oracle and against the unsegmented forward and backward. The segment chain applies each
    segment's transition to the incoming gradient as one bf16 product (one extra rounding per
    segment), so the two bf16 paths agree to the parity tolerance, not to rounding (fp32 agrees
    to 5e-5). A saved buffer belongs to its problem's segment plan: the unsegmented backward
    reads the unsegmented forward's buffer."""
    wl = dict(wl)
    w = workload(wl.pop("idx"), **wl)
    inp = make_inputs(w, with_grad=True)
    if mode == "euler":
        from workloads import round_to_bf16
        kk = inp["k"] / np.maximum(np.linalg.norm(inp["k"], axis=-1, keepdims=True), 1e-30)
        inp["k"] = round_to_bf16(kk.astype(np.float32))
    dt, tol = TDT[w.dtype], TOL[w.dtype]
    B, H, T, dk = inp["k"].shape
    dv = inp["v"].shape[-1]
    r = np.random.default_rng(8)
    h0 = (r.standard_normal((B, H, dk, dv)) * 0.3).astype(np.float32)
    dht = (r.standard_normal((B, H, dk, dv)) * 0.2).astype(np.float32)
    q, k, v, beta, do = (_dev(inp[n], dt) for n in ("q", "k", "v", "beta", "do"))
    h0_d, dht_d = _dev(h0, torch.float32), _dev(dht, torch.float32)
    print("%s: B=%d H=%d T=%d dk=%d dv=%d segments=%d mode=%s" % (name, B, H, T, dk, dv, segments, mode),
          flush=True)
    _, saved = E.efla_fwd(q, k, v, beta, 0.8, None, save=True, initial_state=h0_d, mode=mode,
                          segments=segments)
    _, saved1 = E.efla_fwd(q, k, v, beta, 0.8, None, save=True, initial_state=h0_d, mode=mode, segments=1)
    g = E.efla_bwd(q, k, v, beta, do, saved, 0.8, None, mode=mode, initial_state=h0_d,
                   d_final_state=dht_d, d_initial_state=True, segments=segments)
    g1 = E.efla_bwd(q, k, v, beta, do, saved1, 0.8, None, mode=mode, initial_state=h0_d,
                    d_final_state=dht_d, d_initial_state=True, segments=1)
    torch.cuda.synchronize()
    ref = O.backward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["do"], scale=0.8, initial_state=h0,
                     d_final_state=dht, mode=mode)
    for nm, t, t1 in zip(("dq", "dk", "dv", "dbeta", "d_initial_state"), g, g1):
        _check(nm, _np(t), ref[nm], tol)
        assert O.rel_err(_np(t), _np(t1)) <= (tol if w.dtype == "bf16" else tol / 2), \
            nm + " differs from the unsegmented scan"

"""GPU parity of gated EFLA (efla_fwd_gated, efla_bwd_gated, efla_decode_gated) through the C ABI
against the fp64 oracle (oracle.gated_forward, pinned in test_oracle_pins against the dense
decayed ZOH flow; oracle.gated_backward, pinned there by central differences). bf16 problems,
normwise tolerance 2e-2 per tensor as in the other parity tests.

Gate recipe: log-decays a = log sigmoid(x) per (batch, head, token), x ~ N(mu, 1) with mu = 3
(mild decay, e^a about 0.95), 0 (strong decay, e^a about 0.5: e^{-30} and below across a
chunk), rounded to bf16 like every other input."""
import numpy as np
import pytest
import torch

from oracle import efla_oracle as O
from workloads import make_inputs, round_to_bf16, workload

pytestmark = pytest.mark.gpu

TOL = 2e-2


@pytest.fixture(scope="module")
def E():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import delta_rule_sequence_amd as mod
    mod._lib.lib()
    return mod


def _dev(x, dt=torch.bfloat16):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda", dtype=dt)


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _check(name, gpu, ref, tol=TOL):
    err = O.rel_err(gpu, ref)
    print("  %-6s normwise rel err %.3e (tol %.0e)" % (name, err, tol), flush=True)
    assert np.all(np.isfinite(gpu)), name + " has non-finite values"
    assert err <= tol, "%s: %.3e > %.0e" % (name, err, tol)


def _gates(shape, mu, seed):
    x = np.random.default_rng(seed).standard_normal(shape) + mu
    a = -np.logaddexp(0.0, -x)  # log sigmoid(x), <= 0
    return round_to_bf16(a.astype(np.float32))


CASES = [  # name, workload overrides, gate mean, segments, mode
    ("mild_T200", dict(B=2, H=2, T=200), 3.0, 1, "exact"),
    ("strong_T200", dict(B=2, H=2, T=200), 0.0, 1, "exact"),
    ("mild_dk64_dv128", dict(B=1, H=3, T=64 * 5 + 9, dk=64, dv=128), 3.0, 1, "exact"),
    ("mild_dk128_dv64", dict(B=1, H=3, T=64 * 5 + 9, dk=128, dv=64), 3.0, 1, "exact"),
    ("mild_dk64_dv64", dict(B=2, H=1, T=64 * 5 + 9, dk=64, dv=64), 3.0, 1, "exact"),
    ("mild_seg5", dict(B=1, H=2, T=64 * 37 + 5), 3.0, 5, "exact"),
    ("strong_seg3", dict(B=2, H=2, T=64 * 12 + 30), 0.0, 3, "exact"),
    ("mild_delta_rule", dict(B=1, H=2, T=150), 3.0, 1, "euler"),
    # 4 segments x 16 heads: the 32-column tiling (DMA-fed gated reverse scans in every mode)
    ("mild_wide_seg4", dict(B=1, H=16, T=64 * 20 + 7), 3.0, 4, "exact"),
]


@pytest.mark.parametrize("name,wl,mu,segments,mode", CASES, ids=[c[0] for c in CASES])
def test_gated_forward(E, name, wl, mu, segments, mode):
    w = workload(2, **wl)
    inp = make_inputs(w, with_grad=False)
    if mode == "euler":  # the delta rule needs beta ||k||^2 <= 2 (unit keys)
        kk = inp["k"] / np.maximum(np.linalg.norm(inp["k"], axis=-1, keepdims=True), 1e-30)
        inp["k"] = round_to_bf16(kk.astype(np.float32))
    B, H, T, dk = inp["k"].shape
    dv = inp["v"].shape[-1]
    a = _gates((B, H, T), mu, 17)
    h0 = (np.random.default_rng(3).standard_normal((B, H, dk, dv)) * 0.3).astype(np.float32)
    print("%s: B=%d H=%d T=%d dk=%d dv=%d segments=%d mode=%s" % (name, B, H, T, dk, dv, segments, mode),
          flush=True)
    q, k, v, beta, g = (_dev(x) for x in (inp["q"], inp["k"], inp["v"], inp["beta"], a))
    o, _, ht = E.efla_fwd_gated(q, k, v, beta, g, 0.8, mode=mode, initial_state=_dev(h0, torch.float32),
                                final_state=True, segments=segments)
    torch.cuda.synchronize()
    ref_o, ref_ht = O.gated_forward(inp["q"], inp["k"], inp["v"], inp["beta"], a, scale=0.8,
                                    initial_state=h0, mode=mode)
    _check("o", _np(o), ref_o)
    _check("ht", _np(ht), ref_ht)
    # the gate matters: the ungated flow is far from this result
    if mu == 0.0:
        plain, _ = O.forward(inp["q"], inp["k"], inp["v"], inp["beta"], scale=0.8, initial_state=h0)
        assert O.rel_err(plain, ref_o) > 10 * TOL


def test_zero_gate_is_efla(E):
    """a = 0 runs the gated kernels and must give the ungated forward."""
    w = workload(2, B=2, H=2, T=64 * 3 + 11)
    inp = make_inputs(w, with_grad=False)
    q, k, v, beta = (_dev(inp[n]) for n in ("q", "k", "v", "beta"))
    o_g, _ = E.efla_fwd_gated(q, k, v, beta, torch.zeros_like(beta), 1.0)
    o_p, _ = E.efla_fwd(q, k, v, beta, 1.0, None, save=False)
    torch.cuda.synchronize()
    assert O.rel_err(_np(o_g), _np(o_p)) < 1e-2
    ref, _ = O.forward(inp["q"], inp["k"], inp["v"], inp["beta"])
    _check("o", _np(o_g), ref)


@pytest.mark.parametrize("dk,dv,mu", [(128, 128, 3.0), (64, 128, 0.0), (128, 64, 3.0)])
def test_gated_decode(E, dk, dv, mu):
    """Token recurrence from a given state (1 then 7 tokens) against the oracle and against the
    chunked gated forward of the same tokens."""
    w = workload(2, B=2, H=3, T=8, dk=dk, dv=dv)
    inp = make_inputs(w, with_grad=False)
    a = _gates((2, 3, 8), mu, 29)
    h0 = (np.random.default_rng(11).standard_normal((2, 3, dk, dv)) * 0.3).astype(np.float32)
    state = _dev(h0, torch.float32)
    q, k, v, beta, g = (_dev(x) for x in (inp["q"], inp["k"], inp["v"], inp["beta"], a))
    sl = lambda t, lo, hi: t[:, :, lo:hi].contiguous()
    o1 = E.efla_decode_gated(sl(q, 0, 1), sl(k, 0, 1), sl(v, 0, 1), sl(beta, 0, 1), sl(g, 0, 1), state, 0.7)
    o2 = E.efla_decode_gated(sl(q, 1, 8), sl(k, 1, 8), sl(v, 1, 8), sl(beta, 1, 8), sl(g, 1, 8), state, 0.7)
    torch.cuda.synchronize()
    ref_o, ref_s = O.gated_forward(inp["q"], inp["k"], inp["v"], inp["beta"], a, scale=0.7, initial_state=h0)
    _check("o", np.concatenate([_np(o1), _np(o2)], axis=2), ref_o)
    _check("state", _np(state), ref_s)
    o3, _, ht = E.efla_fwd_gated(q, k, v, beta, g, 0.7, initial_state=_dev(h0, torch.float32), final_state=True)
    torch.cuda.synchronize()
    _check("fwd.o", _np(o3), ref_o)
    _check("fwd.ht", _np(ht), ref_s)


GRAD_NAMES = ("dq", "dk", "dv", "dbeta", "dgate", "d_initial_state")


@pytest.mark.parametrize("name,wl,mu,segments,mode", CASES, ids=[c[0] for c in CASES])
def test_gated_backward(E, name, wl, mu, segments, mode):
    """Gradients in q, k, v, beta, the log-decays and the initial state, from the buffer the
    gated forward saved (with the same segment plan), with a gradient arriving at the final
    state."""
    w = workload(2, **wl)
    inp = make_inputs(w, with_grad=True)
    if mode == "euler":
        kk = inp["k"] / np.maximum(np.linalg.norm(inp["k"], axis=-1, keepdims=True), 1e-30)
        inp["k"] = round_to_bf16(kk.astype(np.float32))
    B, H, T, dk = inp["k"].shape
    dv = inp["v"].shape[-1]
    a = _gates((B, H, T), mu, 19)
    r = np.random.default_rng(7)
    h0 = (r.standard_normal((B, H, dk, dv)) * 0.3).astype(np.float32)
    dht = (r.standard_normal((B, H, dk, dv)) * 0.1).astype(np.float32)
    print("%s: B=%d H=%d T=%d dk=%d dv=%d segments=%d mode=%s" % (name, B, H, T, dk, dv, segments, mode),
          flush=True)
    q, k, v, beta, g, do = (_dev(x) for x in (inp["q"], inp["k"], inp["v"], inp["beta"], a, inp["do"]))
    h0_d, dht_d = _dev(h0, torch.float32), _dev(dht, torch.float32)
    _, saved = E.efla_fwd_gated(q, k, v, beta, g, 0.8, save=True, mode=mode, initial_state=h0_d,
                                segments=segments)
    grads = E.efla_bwd_gated(q, k, v, beta, g, do, saved, 0.8, mode=mode, initial_state=h0_d,
                             d_final_state=dht_d, d_initial_state=True, segments=segments)
    torch.cuda.synchronize()
    ref = O.gated_backward(inp["q"], inp["k"], inp["v"], inp["beta"], a, inp["do"], scale=0.8,
                           initial_state=h0, d_final_state=dht, mode=mode)
    for nm, t in zip(GRAD_NAMES, grads):
        _check(nm, _np(t), ref[nm])


def test_gated_recompute_backward(E):
    """Without a saved buffer the gated forward is recomputed inside the workspace."""
    w = workload(2, B=2, H=2, T=64 * 4 + 21)
    inp = make_inputs(w, with_grad=True)
    a = _gates((2, 2, w.T), 1.0, 23)
    q, k, v, beta, g, do = (_dev(x) for x in (inp["q"], inp["k"], inp["v"], inp["beta"], a, inp["do"]))
    grads = E.efla_bwd_gated(q, k, v, beta, g, do, None, 1.0)
    torch.cuda.synchronize()
    ref = O.gated_backward(inp["q"], inp["k"], inp["v"], inp["beta"], a, inp["do"])
    for nm, t in zip(GRAD_NAMES, grads):
        _check(nm, _np(t), ref[nm])


def test_zero_gate_backward_is_efla(E):
    """a = 0: the gated backward gives the ungated gradients, and the log-decay gradient the
    oracle's (it does not vanish at a = 0)."""
    w = workload(2, B=1, H=3, T=64 * 3 + 40)
    inp = make_inputs(w, with_grad=True)
    q, k, v, beta, do = (_dev(inp[n]) for n in ("q", "k", "v", "beta", "do"))
    z = torch.zeros_like(beta)
    gg = E.efla_bwd_gated(q, k, v, beta, z, do, None, 1.0)
    gp = E.efla_bwd(q, k, v, beta, do, None, 1.0, None)
    torch.cuda.synchronize()
    for nm, a_, b_ in zip(("dq", "dk", "dv", "dbeta"), gg, gp):
        assert O.rel_err(_np(a_), _np(b_)) < 1e-2, nm
    ref = O.gated_backward(inp["q"], inp["k"], inp["v"], inp["beta"], np.zeros_like(inp["beta"]), inp["do"])
    assert np.max(np.abs(ref["dgate"])) > 0
    _check("dgate", _np(gg[4]), ref["dgate"])


def test_gated_autograd(E):
    """efla_gated under torch autograd runs the library's gated backward."""
    w = workload(2, B=1, H=2, T=100)
    inp = make_inputs(w, with_grad=True)
    a = _gates((1, 2, 100), 2.0, 31)
    ts = [_dev(x).requires_grad_(True) for x in (inp["q"], inp["k"], inp["v"], inp["beta"], a)]
    o = E.efla_gated(*ts, scale=0.9)
    o.backward(_dev(inp["do"]))
    torch.cuda.synchronize()
    ref = O.gated_backward(inp["q"], inp["k"], inp["v"], inp["beta"], a, inp["do"], scale=0.9)
    for nm, t in zip(GRAD_NAMES, ts):
        _check(nm, _np(t.grad), ref[nm])


def test_gated_packed_sequences(E):
    """Packed batch (cu_seqlens): the state, and the running log-decay sums, restart at every
    sequence; forward and backward against the oracle's packed gated forms, with initial and
    final states per sequence."""
    lens = [70, 200, 1, 64, 133]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    w = workload(2, B=1, H=2, T=T)
    inp = make_inputs(w, with_grad=True)
    a = _gates((1, 2, T), 1.0, 37)
    r = np.random.default_rng(13)
    h0 = (r.standard_normal((len(lens), 2, 128, 128)) * 0.3).astype(np.float32)
    dht = (r.standard_normal((len(lens), 2, 128, 128)) * 0.1).astype(np.float32)
    q, k, v, beta, g, do = (_dev(x) for x in (inp["q"], inp["k"], inp["v"], inp["beta"], a, inp["do"]))
    cu_d = torch.from_numpy(cu).cuda()
    h0_d, dht_d = _dev(h0, torch.float32), _dev(dht, torch.float32)
    o, saved, ht = E.efla_fwd_gated(q, k, v, beta, g, 0.8, cu_d, save=True, initial_state=h0_d,
                                    final_state=True)
    grads = E.efla_bwd_gated(q, k, v, beta, g, do, saved, 0.8, cu_d, initial_state=h0_d,
                             d_final_state=dht_d, d_initial_state=True)
    torch.cuda.synchronize()
    ref_o, ref_ht = O.gated_forward(inp["q"], inp["k"], inp["v"], inp["beta"], a, scale=0.8,
                                    cu_seqlens=cu, initial_state=h0)
    ref = O.gated_backward(inp["q"], inp["k"], inp["v"], inp["beta"], a, inp["do"], scale=0.8,
                           initial_state=h0, d_final_state=dht, cu_seqlens=cu)
    _check("o", _np(o), ref_o)
    _check("ht", _np(ht), ref_ht)
    for nm, t in zip(GRAD_NAMES, grads):
        _check(nm, _np(t), ref[nm])


FACTOR_CASES = [  # name, workload overrides, gate mean, packed sequence lengths
    ("dense_mild", dict(B=2, H=3, T=64 * 3 + 21), 3.0, None),
    ("dense_strong_d64", dict(B=1, H=2, T=64 * 2 + 40, dk=64, dv=64), 0.0, None),
    ("packed", dict(B=1, H=2), 1.0, [70, 200, 1, 64, 133]),
]


@pytest.mark.parametrize("name,wl,mu,lens", FACTOR_CASES, ids=[c[0] for c in FACTOR_CASES])
def test_gated_saved_chunk_factors(E, name, wl, mu, lens):
    """The decayed M = tril(Q K^T) * e^{c_t - c_s} (formed by the forward scan) and X that the gated
    forward saves for the backward, per (chunk slot, head), against oracle.gated_chunk_factors
    (pinned in test_oracle_pins against the token recurrence). X's rows past the end of a sequence
    are padding; M is zero above the diagonal and in those rows."""
    cu = None
    if lens:
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        wl = dict(wl, T=int(cu[-1]))
    w = workload(2, **wl)
    inp = make_inputs(w, with_grad=False)
    B, H, T, dk = inp["k"].shape
    a = _gates((B, H, T), mu, 23)
    print("%s: B=%d H=%d T=%d dk=%d" % (name, B, H, T, dk), flush=True)
    q, k, v, beta, g = (_dev(x) for x in (inp["q"], inp["k"], inp["v"], inp["beta"], a))
    cu_d = None if cu is None else torch.from_numpy(cu).cuda()
    _, saved = E.efla_fwd_gated(q, k, v, beta, g, 0.8, cu_d, save=True)
    views = E.saved_views(saved, q, k, v, beta, 0.8, cu_d)
    gm, gx = _np(views["m"]), _np(views["x"])
    slot, worst = 0, 0.0
    for (b, s0, e0) in O.sequences(B, T, cu):
        for c0 in range(s0, e0, O.CHUNK):
            n = min(e0, c0 + O.CHUNK) - c0
            for h in range(H):
                sl = slice(c0, c0 + n)
                ref = O.gated_chunk_factors(inp["q"][b, h, sl], inp["k"][b, h, sl], inp["beta"][b, h, sl], a[b, h, sl])
                em, ex = O.rel_err(gm[slot, h, :n, :n], ref["M"]), O.rel_err(gx[slot, h, :n, :n], ref["X"])
                worst = max(worst, em, ex)
                assert em <= TOL and ex <= TOL, (slot, h, em, ex)
                assert not np.any(np.triu(gm[slot, h], 1)) and not np.any(gm[slot, h, n:]), ("M zeros", slot, h)
            slot += 1
    print("  M, X worst normwise rel err per (chunk, head) %.3e (tol %.0e)" % (worst, TOL), flush=True)


@pytest.mark.parametrize("segments", [1, 3])
def test_positive_gate_follows_formula(E, segments):
    """Log-decays of either sign, a ~ N(0.01, 0.03): a > 0 is growth, outside the decay reading,
    but the kernels compute it with the same formulas (e^{c_t - c_s} and e^{c_last - c_t} taken
    as they are, masked by index, never clipped at 1). Forward with final state and backward,
    against the oracle; the positive part of the gate changes the result far beyond tolerance."""
    w = workload(2, B=1, H=2, T=64 * 7 + 17)
    inp = make_inputs(w, with_grad=True)
    B, H, T, dk = inp["k"].shape
    a = round_to_bf16((np.random.default_rng(41).standard_normal((B, H, T)) * 0.03 + 0.01).astype(np.float32))
    assert np.mean(a > 0) > 0.5
    q, k, v, beta, g, do = (_dev(x) for x in (inp["q"], inp["k"], inp["v"], inp["beta"], a, inp["do"]))
    o, saved, ht = E.efla_fwd_gated(q, k, v, beta, g, 1.0, save=True, final_state=True, segments=segments)
    grads = E.efla_bwd_gated(q, k, v, beta, g, do, saved, 1.0, segments=segments)
    torch.cuda.synchronize()
    ref_o, ref_ht = O.gated_forward(inp["q"], inp["k"], inp["v"], inp["beta"], a)
    _check("o", _np(o), ref_o)
    _check("ht", _np(ht), ref_ht)
    ref = O.gated_backward(inp["q"], inp["k"], inp["v"], inp["beta"], a, inp["do"])
    for nm, t in zip(GRAD_NAMES[:5], grads):
        _check(nm, _np(t), ref[nm])
    clipped, _ = O.gated_forward(inp["q"], inp["k"], inp["v"], inp["beta"], np.minimum(a, 0.0))
    assert O.rel_err(clipped, ref_o) > 10 * TOL

"""GPU parity of gated EFLA (efla_fwd_gated, efla_decode_gated) through the C ABI against the
fp64 oracle (oracle.gated_forward, pinned in test_oracle_pins against the dense decayed ZOH
flow). bf16 problems, normwise tolerance 2e-2 per tensor as in the other parity tests.

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
    o, ht = E.efla_fwd_gated(q, k, v, beta, g, 0.8, mode=mode, initial_state=_dev(h0, torch.float32),
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
    o_g = E.efla_fwd_gated(q, k, v, beta, torch.zeros_like(beta), 1.0)
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
    o3, ht = E.efla_fwd_gated(q, k, v, beta, g, 0.7, initial_state=_dev(h0, torch.float32), final_state=True)
    torch.cuda.synchronize()
    _check("fwd.o", _np(o3), ref_o)
    _check("fwd.ht", _np(ht), ref_s)

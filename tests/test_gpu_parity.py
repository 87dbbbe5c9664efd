"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Tolerance: normwise relative error max|gpu - oracle| / max|oracle| per tensor of at most
1e-4 for fp32 problems and 2e-2 for bf16 problems (fp32 accumulation), gradients included.
Every tensor is also checked per (batch, head) at the same bound. The oracle is fed the
exact values the GPU consumes (bf16 inputs upcast exactly).
"""
import numpy as np
import pytest
import torch

from oracle import efla_oracle as O
from oracle_streams import TOKEN_FLOORS, TOKEN_TOL_FACTOR, token_ratio
from workloads import make_inputs, workload

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
TDT = {"f32": torch.float32, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def E():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import delta_rule_sequence_amd as mod
    mod._lib.lib()  # fails loudly when libefla.so is missing
    return mod


def _dev(x, dt):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda", dtype=dt)


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _check(name, gpu, ref, tol, per_head=True):
    err = O.rel_err(gpu, ref)
    print("  %-6s normwise rel err %.3e (tol %.0e)" % (name, err, tol), flush=True)
    assert np.all(np.isfinite(gpu)), name + " has non-finite values"
    assert err <= tol, "%s: %.3e > %.0e" % (name, err, tol)
    if per_head and ref.ndim >= 3:
        B, H = ref.shape[:2]
        for b in range(B):
            for h in range(H):
                e = O.rel_err(gpu[b, h], ref[b, h])
                assert e <= tol, "%s[b=%d,h=%d]: %.3e > %.0e" % (name, b, h, e, tol)


def _run(E, inp, dtype, scale=1.0, backward=True):
    dt = TDT[dtype]
    q, k, v, beta = (_dev(inp[n], dt) for n in ("q", "k", "v", "beta"))
    cu = None if inp["cu_seqlens"] is None else torch.from_numpy(inp["cu_seqlens"]).cuda()
    o, saved = E.efla_fwd(q, k, v, beta, scale, cu, save=True)
    out = dict(o=_np(o))
    views = E.saved_views(saved, q, k, v, beta, scale, cu)
    # chunk slots in use (a packed batch's slot count is an upper bound; the rest is never
    # written): ceil(len / 64) per sequence
    B, T = inp["q"].shape[0], inp["q"].shape[2]
    used = sum((e - s + O.CHUNK - 1) // O.CHUNK for (_, s, e) in O.sequences(B, T, inp["cu_seqlens"]))
    out["states"] = _np(views["states"][:used])
    out["ut"] = _np(views["ut"])
    if "w" in views:  # fp32 saves W; bf16 saves X and the column scales alpha~ instead
        out["w"] = _np(views["w"])
    else:
        out["x"] = _np(views["x"][:used])
        out["alpha"] = _np(views["coef"][0, :used])
    if backward:
        do = _dev(inp["do"], dt)
        dq, dk, dv, db = E.efla_bwd(q, k, v, beta, do, saved, scale, cu)
        out.update(dq=_np(dq), dk=_np(dk), dv=_np(dv), dbeta=_np(db))
        # the recompute path (no saved buffer) runs the same kernels in the same order
        g2 = E.efla_bwd(q, k, v, beta, do, None, scale, cu)
        for a, b in zip((dq, dk, dv, db), g2):
            assert torch.equal(a, b)
    torch.cuda.synchronize()
    return out


def _oracle(inp, scale=1.0, backward=True):
    o, _ = O.forward(inp["q"], inp["k"], inp["v"], inp["beta"], scale=scale, cu_seqlens=inp["cu_seqlens"])
    ref = dict(o=o)
    if backward:
        ref.update(O.backward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["do"], scale=scale,
                              cu_seqlens=inp["cu_seqlens"]))
    return ref


def _compare(gpu, ref, dtype, backward=True, token_rows=()):
    tol = TOL[dtype]
    _check("o", gpu["o"], ref["o"], tol)
    if backward:
        for n in ("dq", "dk", "dv", "dbeta"):
            _check(n, gpu[n], ref[n], tol)
    for n in token_rows:  # token by token: ||d_t|| <= tol max(||ref_t||, f max_s ||ref_s||)
        B, H = ref[n].shape[:2]
        f = TOKEN_FLOORS[n]
        worst = max(token_ratio(gpu[n][b, h], ref[n][b, h], f) for b in range(B) for h in range(H))
        tt = tol * TOKEN_TOL_FACTOR.get(n, 1.0)
        print("  %-6s per-token worst ratio %.3e (tol %.0e)" % (n, worst, tt), flush=True)
        assert worst <= tt, "%s per token: %.3e > %.0e" % (n, worst, tt)


# Reduced sizes of the five workloads: several chunks and a ragged tail each.
CASES = [
    ("w1_tiny_f32", 1, dict(), False, 1.0),
    ("w1_ragged_f32_bwd", 1, dict(T=200, backward=True), True, 1.0),
    ("w2_bf16", 2, dict(B=2, H=2, T=209), True, 1.0),
    ("w2_bf16_scale", 2, dict(B=1, H=3, T=130), True, 0.37),
    ("w3_bf16_long", 3, dict(H=2, T=1000), False, 1.0),
    ("w4_stiff_f32", 4, dict(B=2, H=2, T=300), True, 1.0),
    ("w5_varlen_bf16", 5, dict(H=2, n_seqs=6, seq_len_range=(1, 200)), True, 1.0),
    ("bf16_dk64_dv128", 2, dict(B=1, H=2, T=150, dk=64, dv=128), True, 1.0),
    ("bf16_dk128_dv64", 2, dict(B=1, H=2, T=150, dk=128, dv=64), True, 1.0),
    ("bf16_d64", 2, dict(B=2, H=1, T=100, dk=64, dv=64), True, 1.0),
]


@pytest.mark.parametrize("name,idx,over,bwd,scale", CASES, ids=[c[0] for c in CASES])
def test_parity_reduced(E, name, idx, over, bwd, scale):
    w = workload(idx, **over)
    inp = make_inputs(w, with_grad=bwd)
    print("case %s: %s" % (name, w), flush=True)
    gpu = _run(E, inp, w.dtype, scale, bwd)
    ref = _oracle(inp, scale, bwd)
    # stiff keys and outlier values (fp32): the largest rows set the normwise scale, so the
    # tokens are also checked one by one
    rows = ("o", "dk", "dbeta") if w.keys == "loguniform_1e-3_100" else ()
    _compare(gpu, ref, w.dtype, bwd, token_rows=rows)


@pytest.mark.parametrize("widx", [2, 4])
def test_stage_values_match_chunk_oracle(E, widx):
    """Per-stage values: W, U~ and the state entering every chunk (kernels b and c). fp32
    saves W itself; bf16 saves X and the column scales alpha~ (checked against the oracle's
    alpha token by token), and W = X diag(alpha~) K is formed from them here."""
    w = workload(widx, B=2, H=2, T=150)
    inp = make_inputs(w, with_grad=False)
    gpu = _run(E, inp, w.dtype, 1.0, backward=False)
    ref = O.chunk_forward(inp["q"], inp["k"], inp["v"], inp["beta"])
    tol = TOL[w.dtype]
    if "w" in gpu:
        _check("W", gpu["w"], ref["W"], tol)
    else:
        B, H, T = inp["k"].shape[:3]
        ntc = (T + O.CHUNK - 1) // O.CHUNK
        k64 = inp["k"].astype(np.float64)
        alpha_ref = O.coefficients(inp["k"], inp["beta"])["alpha"]
        alpha_gpu = np.zeros_like(alpha_ref)
        w_gpu = np.zeros_like(k64)
        for b in range(B):
            for c in range(ntc):
                t0, n = c * O.CHUNK, min(O.CHUNK, T - c * O.CHUNK)
                for h in range(H):
                    a = gpu["alpha"][b * ntc + c, h, :n].astype(np.float64)
                    alpha_gpu[b, h, t0:t0 + n] = a
                    X = gpu["x"][b * ntc + c, h, :n, :n].astype(np.float64)
                    w_gpu[b, h, t0:t0 + n] = X @ (a[:, None] * k64[b, h, t0:t0 + n])
        err = np.max(np.abs(alpha_gpu - alpha_ref) / np.maximum(np.abs(alpha_ref), 1e-30))
        print("  alpha~ elementwise rel err %.3e" % err, flush=True)
        assert err <= 1e-5, err  # fp32 coefficients: the exact-flow step to fp32 rounding
        _check("W", w_gpu, ref["W"], tol)
    _check("U~", gpu["ut"], ref["Ut"], tol)
    states = np.stack(ref["states"])             # [slots, H, dk, dv]
    _check("S_c", gpu["states"][: len(states)], states, tol, per_head=False)


@pytest.mark.parametrize("widx,over", [(2, dict(B=2, H=2, T=150)), (5, dict(H=2)),
                                       (4, dict(B=1, H=2, T=150))])
def test_saved_chunk_factors_match_oracle(E, widx, over):
    """M = tril(Q K^T) and X = (I + A)^{-1} that the forward saves for the backward, per
    (chunk slot, head), on a ragged dense batch and on a packed batch (bf16: M formed by the
    forward scan), and fp32 (M formed by the UT kernel). X's rows past the end of a sequence are
    padding and are not compared; M is zero above the diagonal and in those rows."""
    w = workload(widx, **over)
    inp = make_inputs(w, with_grad=False)
    dt = TDT[w.dtype]
    q, k, v, beta = (_dev(inp[n], dt) for n in ("q", "k", "v", "beta"))
    cu = None if inp["cu_seqlens"] is None else torch.from_numpy(inp["cu_seqlens"]).cuda()
    _, saved = E.efla_fwd(q, k, v, beta, 1.0, cu, save=True)
    views = E.saved_views(saved, q, k, v, beta, 1.0, cu)
    gm, gx = _np(views["m"]), _np(views["x"])
    tol = TOL[w.dtype]
    slot = 0
    B, H, T = inp["q"].shape[:3]
    for (b, s0, e0) in O.sequences(B, T, inp["cu_seqlens"]):
        for c0 in range(s0, e0, O.CHUNK):
            n = min(e0, c0 + O.CHUNK) - c0
            for h in range(H):
                ref = O.chunk_factors(inp["q"][b, h, c0:c0 + n], inp["k"][b, h, c0:c0 + n],
                                      inp["beta"][b, h, c0:c0 + n])
                assert O.rel_err(gm[slot, h, :n, :n], ref["M"]) <= tol, ("M", slot, h)
                assert O.rel_err(gx[slot, h, :n, :n], ref["X"]) <= tol, ("X", slot, h)
                assert not np.any(np.triu(gm[slot, h], 1)) and not np.any(gm[slot, h, n:]), ("M zeros", slot, h)
            slot += 1


@pytest.mark.parametrize("widx", [4, 2])
def test_chunk_ut_entry_point(E, widx):
    """efla_chunk_ut forms W and U explicitly for fp32 and bf16 (the forward of bf16 problems
    keeps X and the column scales instead)."""
    w = workload(widx, B=1, H=2, T=170)
    inp = make_inputs(w, with_grad=False)
    dt = TDT[w.dtype]
    W, U = E.efla_chunk_ut(_dev(inp["k"], dt), _dev(inp["v"], dt), _dev(inp["beta"], dt))
    ref = O.chunk_forward(inp["q"], inp["k"], inp["v"], inp["beta"])
    _check("W", _np(W), ref["W"], TOL[w.dtype])
    _check("U", _np(U), ref["U"], TOL[w.dtype])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prep_coefficients_log_sweep(E, dtype):
    """Kernel (a): lambda, alpha, e^{-beta lambda} and beta^2 phi'(beta lambda) over
    beta * lambda in [1e-10, 1e4] (lambda -> 0 series, exp underflow), against the oracle
    evaluated at the key energy the kernel computed."""
    dt = TDT[dtype]
    n = 4096
    xs = np.logspace(-10, 4, n)
    beta = np.where(np.arange(n) % 2 == 0, 0.5, 1.0).astype(np.float32)
    lam = xs / beta
    k = np.zeros((1, 1, n, 64), dtype=np.float32)
    k[0, 0, :, 0] = np.sqrt(lam).astype(np.float32)
    k[0, 0, ::3, 1] = 0.25 * k[0, 0, ::3, 0]
    if dtype == "bf16":
        from workloads import round_to_bf16
        k = round_to_bf16(k)
    out = E.efla_prep(_dev(k, dt), _dev(beta[None, None], dt))
    lam_g = _np(out["lam"])[0, 0]
    kk = k.astype(np.float64)[0, 0]
    assert np.allclose(lam_g, np.sum(kk * kk, axis=-1), rtol=2e-7, atol=0)
    co = O.coefficients(np.sqrt(lam_g)[:, None], beta.astype(np.float64))
    for name, key, tol in (("alpha", "alpha", 2e-6), ("dalpha_dbeta", "dalpha_dbeta", 2e-6),
                           ("dalpha_dlam", "dalpha_dlam", 1e-5)):
        g = _np(out[name])[0, 0]
        r = co[key]
        nz = np.abs(r) > 1e-30
        rel = np.max(np.abs(g[nz] - r[nz]) / np.abs(r[nz]))
        print("  %s max elementwise rel err %.2e" % (name, rel), flush=True)
        assert rel < tol, name
        assert np.all(np.abs(g[~nz]) < 1e-30)


def test_edge_cases_packed_batch(E):
    """Length-1 and empty sequences, a sequence of exactly one chunk and one of 65 tokens,
    a zero key row, a zero gate and a gate so large that e^{-beta lambda} underflows."""
    w = workload(5, H=2)
    inp = make_inputs(w, lengths=[1, 0, 64, 65, 1, 130, 0])
    inp["k"][0, 0, 5] = 0.0
    inp["beta"][0, 1, 7] = 0.0
    inp["beta"][0, 0, 70] = 64.0
    gpu = _run(E, inp, w.dtype)
    ref = _oracle(inp)
    _compare(gpu, ref, w.dtype)


def test_single_token_and_one_chunk_dense(E):
    for T in (1, 64):
        w = workload(4, B=1, H=1, T=T)
        inp = make_inputs(w)
        _compare(_run(E, inp, w.dtype), _oracle(inp), w.dtype)


def test_deterministic(E):
    w = workload(2, B=1, H=2, T=200)
    inp = make_inputs(w)
    a = _run(E, inp, w.dtype)
    b = _run(E, inp, w.dtype)
    for n in ("o", "dq", "dk", "dv", "dbeta", "states"):
        assert np.array_equal(a[n], b[n]), n


def test_autograd_function(E):
    w = workload(2, B=1, H=2, T=96)
    inp = make_inputs(w)
    dt = TDT[w.dtype]
    q, k, v, beta = (_dev(inp[n], dt).requires_grad_(True) for n in ("q", "k", "v", "beta"))
    o = E.efla(q, k, v, beta)
    o.backward(_dev(inp["do"], dt))
    ref = _oracle(inp)
    _check("o", _np(o), ref["o"], TOL[w.dtype])
    for t, n in ((q, "dq"), (k, "dk"), (v, "dv"), (beta, "dbeta")):
        _check(n, _np(t.grad), ref[n], TOL[w.dtype])

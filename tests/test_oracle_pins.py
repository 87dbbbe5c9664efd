"""Pins for the fp64 oracle: each test checks it against something other than itself.

The pages (Exact Flow Linear Attention summary page) print no equation and no
worked example, so the pins are the mathematics their statements fix:
the zero-order-hold flow itself (section 3.1, Appendix E) computed by a dense
matrix exponential plus quadrature and by the Van Loan block exponential; the
rank-1 structure (Appendix D); the small-step Euler limit (section 3.4); the
contraction along k and the untouched orthogonal complement (section 3.4);
the exactness of the flow (semigroup property); the chunkwise form (section 3.3)
against the token recurrence; textbook special cases; mpmath for the
coefficient functions; and central finite differences for the backward.
"""
import json
import os

import mpmath
import numpy as np
import pytest
import scipy.integrate
import scipy.linalg

from oracle import efla_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


def _rng(seed):
    return np.random.default_rng(seed)


def _one_seq(S0, ks, vs, betas, qs=None, scale=1.0):
    """Run the oracle on one sequence (B=H=1) from state S0; returns (o [T,dv], S_final)."""
    ks = np.atleast_2d(ks)
    vs = np.atleast_2d(vs)
    T, dk = ks.shape
    if qs is None:
        qs = np.zeros_like(ks)
    o, SF = O.forward(qs[None, None], ks[None, None], vs[None, None],
                      np.asarray(betas, dtype=np.float64).reshape(1, 1, T), scale=scale,
                      initial_state=None if S0 is None else S0[None, None])
    return o[0, 0], SF[0, 0]


def _zoh_dense(S, k, v, beta):
    """Exact ZOH flow by definition: e^{-beta A} S + int_0^beta e^{-(beta - tau) A} dtau (k v^T)."""
    A = np.outer(k, k)
    b = np.outer(k, v)
    E = scipy.linalg.expm(-beta * A)
    integral, _ = scipy.integrate.quad_vec(lambda tau: scipy.linalg.expm(-(beta - tau) * A) @ b,
                                           0.0, beta, epsabs=1e-15, epsrel=1e-13)
    return E @ S + integral


def _zoh_van_loan(S, k, v, beta):
    """Same flow via exp(beta [[-A, k v^T], [0, 0]]) = [[e^{-beta A}, int ...], [0, I]]."""
    dk, dv = len(k), len(v)
    M = np.zeros((dk + dv, dk + dv))
    M[:dk, :dk] = -np.outer(k, k)
    M[:dk, dk:] = np.outer(k, v)
    E = scipy.linalg.expm(beta * M)
    return E[:dk, :dk] @ S + E[:dk, dk:]


# ---------------------------------------------------------------- coefficients

def test_phi_and_dphi_against_mpmath():
    """phi(x) = (1 - e^{-x})/x and phi'(x) at 60 digits over x in [1e-12, 1e4] and small negatives."""
    mpmath.mp.dps = 60
    xs = np.concatenate([np.logspace(-12, 4, 601), -np.logspace(-12, 0.5, 121), [0.0, 1.0, 0.999999]])
    ph, dp = O.phi(xs), O.dphi(xs)
    worst_p = worst_d = 0.0
    for x, p, d in zip(xs, ph, dp):
        X = mpmath.mpf(float(x))
        if X == 0:
            P, D = mpmath.mpf(1), mpmath.mpf(-0.5)
        else:
            P = -mpmath.expm1(-X) / X
            D = (mpmath.exp(-X) * (1 + X) - 1) / X ** 2
        worst_p = max(worst_p, abs(p - float(P)) / abs(float(P)))
        worst_d = max(worst_d, abs(d - float(D)) / abs(float(D)))
    assert worst_p < 1e-15
    assert worst_d < 1e-13


def test_alpha_limits():
    """alpha -> beta as beta*lambda -> 0 (section 3.4), alpha -> 1/lambda when e^{-beta lambda} underflows."""
    beta = np.array([0.3, 0.7, 2.0])
    assert np.allclose(O.alpha(beta, np.zeros(3)), beta, rtol=0, atol=0)
    lam = np.array([1e-9, 1e-9, 1e-9])
    assert np.allclose(O.alpha(beta, lam), beta * (1 - beta * lam / 2), rtol=1e-15)
    assert np.allclose(O.alpha(np.array([50.0]), np.array([100.0])), 1.0 / 100.0, rtol=1e-15)


def test_coefficient_derivatives_by_finite_differences():
    r = _rng(3)
    beta = r.uniform(0.05, 1.5, 50)
    lam = np.exp(r.uniform(np.log(1e-6), np.log(50.0), 50))
    co = O.coefficients(np.sqrt(lam)[:, None] * np.eye(1)[0], beta)
    h = 1e-6
    fd_b = (O.alpha(beta + h, lam) - O.alpha(beta - h, lam)) / (2 * h)
    hl = h * np.maximum(lam, 1.0)
    fd_l = (O.alpha(beta, lam + hl) - O.alpha(beta, lam - hl)) / (2 * hl)
    assert np.allclose(co["dalpha_dbeta"], fd_b, rtol=1e-7, atol=1e-9)
    assert np.allclose(co["dalpha_dlam"], fd_l, rtol=1e-6, atol=1e-9)


# ---------------------------------------------------------------- exact flow

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_token_update_equals_dense_zoh_flow(seed):
    """One token of the oracle equals expm + quadrature of the ZOH integral (d_k=5, d_v=4)."""
    r = _rng(seed)
    S = r.standard_normal((5, 4))
    k = r.standard_normal(5) * r.uniform(0.3, 2.0)
    v = r.standard_normal(4)
    beta = r.uniform(0.1, 1.5)
    _, S1 = _one_seq(S, k[None], v[None], [beta])
    ref = _zoh_dense(S, k, v, beta)
    assert np.max(np.abs(S1 - ref)) < 1e-12 * max(1.0, np.max(np.abs(ref)))


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_sequence_equals_van_loan_flow(seed):
    """Eight tokens, outputs and states, against the Van Loan block exponential, token by token."""
    r = _rng(10 + seed)
    dk, dv, T = 6, 3, 8
    ks = r.standard_normal((T, dk)) * r.uniform(0.2, 3.0, (T, 1))
    vs = r.standard_normal((T, dv))
    qs = r.standard_normal((T, dk))
    betas = r.uniform(0.0, 2.0, T)
    o, SF = _one_seq(None, ks, vs, betas, qs, scale=0.7)
    S = np.zeros((dk, dv))
    for t in range(T):
        S = _zoh_van_loan(S, ks[t], vs[t], betas[t])
        assert np.allclose(o[t], 0.7 * S.T @ qs[t], rtol=1e-12, atol=1e-12)
    assert np.allclose(SF, S, rtol=1e-12, atol=1e-12)


def test_rank1_structure_of_dynamics_matrix():
    """A = k k^T is a scaled projection: A^2 = lambda A, so e^{-beta A} = I - alpha k k^T (Appendix D)."""
    r = _rng(5)
    k = r.standard_normal(7)
    A = np.outer(k, k)
    lam = k @ k
    assert np.allclose(A @ A, lam * A, rtol=1e-14, atol=1e-12)
    beta = 0.9
    a = O.alpha(np.array([beta]), np.array([lam]))[0]
    assert np.allclose(scipy.linalg.expm(-beta * A), np.eye(7) - a * A, rtol=1e-13, atol=1e-13)


def test_semigroup_exact_but_not_euler():
    """Exactness: flowing beta1 then beta2 with the same (k, v) equals flowing beta1 + beta2.
    The Euler step (DeltaNet) does not have this property."""
    r = _rng(7)
    S = r.standard_normal((4, 3))
    k = r.standard_normal(4)
    v = r.standard_normal(3)
    _, S2 = _one_seq(S, np.stack([k, k]), np.stack([v, v]), [0.4, 0.9])
    _, S1 = _one_seq(S, k[None], v[None], [1.3])
    assert np.max(np.abs(S2 - S1)) < 1e-13

    def euler(S, k, v, b):
        return S + b * np.outer(k, v - S.T @ k)
    gap = np.max(np.abs(euler(euler(S, k, v, 0.4), k, v, 0.9) - euler(S, k, v, 1.3)))
    assert gap > 1e-3


def test_fixed_point_when_value_is_recalled():
    """If v = S^T k the memory already maps k to v and the update leaves S unchanged."""
    r = _rng(8)
    S = r.standard_normal((5, 6))
    k = r.standard_normal(5) * 3.0
    _, S1 = _one_seq(S, k[None], (S.T @ k)[None], [0.8])
    assert np.max(np.abs(S1 - S)) < 1e-13


def test_contraction_along_key_and_orthogonal_complement():
    """Section 3.4: the flow scales the component along k by e^{-beta lambda} (pulling it towards v)
    and leaves the orthogonal complement unchanged; with v = 0 it is non-expansive."""
    r = _rng(9)
    for _ in range(20):
        S = r.standard_normal((6, 4))
        k = r.standard_normal(6) * r.uniform(0.1, 5.0)
        v = r.standard_normal(4)
        beta = r.uniform(0.0, 3.0)
        lam = k @ k
        P = np.eye(6) - np.outer(k, k) / lam
        _, S1 = _one_seq(S, k[None], v[None], [beta])
        e = np.exp(-beta * lam)
        assert np.allclose(k @ S1, e * (k @ S) + (1 - e) * v, rtol=1e-12, atol=1e-12)
        assert np.allclose(P @ S1, P @ S, rtol=1e-12, atol=1e-12)
        _, S0v = _one_seq(S, k[None], np.zeros((1, 4)), [beta])
        assert np.linalg.norm(S0v) <= np.linalg.norm(S) * (1 + 1e-14)


def test_overwrite_limit_for_large_step():
    """When beta*lambda is large the memory is overwritten along k: k^T S_t = v_t^T."""
    r = _rng(11)
    S = r.standard_normal((4, 3))
    k = r.standard_normal(4)
    v = r.standard_normal(3)
    _, S1 = _one_seq(S, k[None], v[None], [80.0 / (k @ k)])
    assert np.allclose(k @ S1, v, rtol=1e-13, atol=1e-13)


def test_euler_mode_is_the_delta_rule():
    """mode "euler" of the forward equals the separately written delta-rule loop, on a packed
    batch; the chunked form in that mode agrees as well."""
    r = _rng(15)
    H, dk, dv = 2, 5, 4
    cu = np.array([0, 7, 70, 71, 140], dtype=np.int32)
    T = int(cu[-1])
    q, k = r.standard_normal((1, H, T, dk)), r.standard_normal((1, H, T, dk))
    v, beta = r.standard_normal((1, H, T, dv)), r.uniform(0.0, 1.0, (1, H, T))
    o, _ = O.forward(q, k, v, beta, scale=0.6, cu_seqlens=cu, mode="euler")
    assert O.rel_err(o, O.euler_forward(q, k, v, beta, scale=0.6, cu_seqlens=cu)) < 1e-13
    o_exact, _ = O.forward(q, k, v, beta, scale=0.6, cu_seqlens=cu)
    assert O.rel_err(o, o_exact) > 1e-2   # the two modes do differ at these key norms
    c = O.coefficients(k, beta, mode="euler")
    assert np.array_equal(c["alpha"], beta) and np.all(c["dalpha_dbeta"] == 1.0)
    assert np.all(c["dalpha_dlam"] == 0.0)


def test_euler_limit_is_third_order_in_key_scale():
    """Section 3.4: for small beta*lambda EFLA equals the delta rule up to higher-order terms.
    With k -> s k the one-step gap to the Euler update shrinks like s^3."""
    r = _rng(12)
    S = r.standard_normal((5, 4))
    k = r.standard_normal(5)
    v = r.standard_normal(4)
    beta = 0.8

    def gap(s):
        ks = s * k
        _, S1 = _one_seq(S, ks[None], v[None], [beta])
        return np.max(np.abs(S1 - (S + beta * np.outer(ks, v - S.T @ ks))))
    g1, g2, g3 = gap(1e-1), gap(1e-2), gap(1e-3)
    assert 800 < g1 / g2 < 1200
    assert 800 < g2 / g3 < 1200


# ---------------------------------------------------------------- closed forms

def test_single_token_output():
    """From S_0 = 0 a single token gives o_1 = scale * alpha_1 (k_1 . q_1) v_1."""
    r = _rng(13)
    q, k, v = r.standard_normal(8), r.standard_normal(8), r.standard_normal(5)
    beta = 0.6
    o, _ = _one_seq(None, k[None], v[None], [beta], q[None], scale=1.3)
    a = (1 - np.exp(-beta * (k @ k))) / (k @ k)
    assert np.allclose(o[0], 1.3 * a * (k @ q) * v, rtol=1e-14, atol=1e-14)


def test_orthogonal_keys_reduce_to_masked_linear_attention():
    """Mutually orthogonal keys from S_0 = 0: o_t = sum_{i<=t} alpha_i (k_i . q_t) v_i,
    i.e. causal linear attention with per-token weights alpha (a masked matmul)."""
    r = _rng(14)
    d, T = 16, 12
    Qm, _ = np.linalg.qr(r.standard_normal((d, d)))
    ks = Qm[:, :T].T * r.uniform(0.2, 3.0, (T, 1))
    vs = r.standard_normal((T, 5))
    qs = r.standard_normal((T, d))
    betas = r.uniform(0.1, 1.0, T)
    o, _ = _one_seq(None, ks, vs, betas, qs)
    lam = np.sum(ks * ks, axis=1)
    a = (1 - np.exp(-betas * lam)) / lam
    ref = np.tril(qs @ ks.T) @ (a[:, None] * vs)
    assert np.allclose(o, ref, rtol=1e-12, atol=1e-12)


def test_zero_keys_are_no_ops():
    r = _rng(15)
    S = r.standard_normal((4, 3))
    _, S1 = _one_seq(S, np.zeros((3, 4)), r.standard_normal((3, 3)), [0.5, 0.9, 0.1])
    assert np.array_equal(S1, S)


# ---------------------------------------------------------------- chunk form, layouts

@pytest.mark.parametrize("T", [1, 5, 63, 64, 65, 130, 200])
def test_chunk_form_equals_token_recurrence(T):
    r = _rng(100 + T)
    B, H, dk, dv = 2, 2, 8, 6
    q = r.standard_normal((B, H, T, dk))
    k = r.standard_normal((B, H, T, dk)) * r.uniform(0.3, 3.0, (B, H, T, 1))
    v = r.standard_normal((B, H, T, dv))
    beta = r.uniform(0.0, 1.0, (B, H, T))
    o, _ = O.forward(q, k, v, beta, scale=0.5)
    c = O.chunk_forward(q, k, v, beta, scale=0.5)
    assert O.rel_err(c["o"], o) < 1e-12
    # per-chunk states match the token recurrence at chunk boundaries
    for b in range(B):
        for ci, c0 in enumerate(range(0, T, O.CHUNK)):
            _, S = O.forward(q[b:b + 1, :, :c0], k[b:b + 1, :, :c0], v[b:b + 1, :, :c0],
                             beta[b:b + 1, :, :c0])
            nchunk = (T + O.CHUNK - 1) // O.CHUNK
            assert np.allclose(c["states"][b * nchunk + ci], S[0], rtol=1e-11, atol=1e-11)


def test_chunk_ut_solves_its_triangular_system():
    """T (I + A) ... written as (I + A) T = diag(alpha) with A strictly lower; W = T K, U = T V."""
    r = _rng(21)
    k = r.standard_normal((64, 16)) * r.uniform(0.5, 2.0, (64, 1))
    v = r.standard_normal((64, 8))
    beta = r.uniform(0.0, 1.0, 64)
    f = O.chunk_ut(k, v, beta)
    lam = np.sum(k * k, axis=1)
    a = (1 - np.exp(-beta * lam)) / lam
    A = np.tril(a[:, None] * (k @ k.T), -1)
    assert np.allclose((np.eye(64) + A) @ f["T"], np.diag(a), rtol=1e-10, atol=1e-10)
    assert np.allclose(np.triu(f["T"], 1), 0.0)


def test_chunk_factors_against_ut_and_recurrence():
    """X is the unit lower triangular inverse with X diag(alpha) = T of the UT transform;
    M = tril(Q K^T) keeps the diagonal: from a zero state one chunk reads out
    o = scale M X diag(alpha) V and leaves the state K^T X diag(alpha) V, as the token
    recurrence does."""
    r = _rng(23)
    C, dk, dv = 40, 12, 7
    q = r.standard_normal((C, dk))
    k = r.standard_normal((C, dk)) * r.uniform(0.5, 2.0, (C, 1))
    v = r.standard_normal((C, dv))
    beta = r.uniform(0.05, 1.0, C)
    f = O.chunk_factors(q, k, beta)
    X, M = f["X"], f["M"]
    a = O.alpha(beta, np.sum(k * k, axis=1))
    assert np.allclose(np.triu(X, 1), 0.0) and np.allclose(np.diag(X), 1.0)
    assert np.allclose(X * a[None, :], O.chunk_ut(k, v, beta)["T"], rtol=1e-11, atol=1e-12)
    o, S = O.forward(q[None, None], k[None, None], v[None, None], beta[None, None], scale=0.7)
    U = (X * a[None, :]) @ v
    assert O.rel_err(0.7 * M @ U, o[0, 0]) < 1e-11
    assert O.rel_err(k.T @ U, S[0, 0]) < 1e-11
    # dropping the diagonal of M (a strict causal mask) would not reproduce the read-out
    assert O.rel_err(0.7 * np.tril(q @ k.T, -1) @ U, o[0, 0]) > 1e-3


def test_packed_batch_equals_separate_sequences():
    r = _rng(22)
    H, dk, dv = 2, 6, 5
    lens = [3, 70, 1, 64, 129]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    q = r.standard_normal((1, H, T, dk))
    k = r.standard_normal((1, H, T, dk))
    v = r.standard_normal((1, H, T, dv))
    beta = r.uniform(0.0, 1.0, (1, H, T))
    do = r.standard_normal((1, H, T, dv))
    o, SF = O.forward(q, k, v, beta, cu_seqlens=cu)
    g = O.backward(q, k, v, beta, do, cu_seqlens=cu)
    co = O.chunk_forward(q, k, v, beta, cu_seqlens=cu)
    assert O.rel_err(co["o"], o) < 1e-12
    for i in range(len(lens)):
        s, e = cu[i], cu[i + 1]
        oi, Si = O.forward(q[:, :, s:e], k[:, :, s:e], v[:, :, s:e], beta[:, :, s:e])
        gi = O.backward(q[:, :, s:e], k[:, :, s:e], v[:, :, s:e], beta[:, :, s:e], do[:, :, s:e])
        assert np.array_equal(o[:, :, s:e], oi)
        assert np.array_equal(SF[i], Si[0])
        for name in ("dq", "dk", "dv", "dbeta"):
            assert np.array_equal(g[name][:, :, s:e], gi[name])


def test_split_sequence_with_carried_state():
    """Forward over [0, T) equals [0, T1) then [T1, T) with the state carried; the backward
    of the two halves, chained through the state gradient, equals the full backward."""
    r = _rng(23)
    H, T, T1, dk, dv = 2, 150, 70, 5, 4
    q, k = r.standard_normal((1, H, T, dk)), r.standard_normal((1, H, T, dk))
    v, do = r.standard_normal((1, H, T, dv)), r.standard_normal((1, H, T, dv))
    beta = r.uniform(0.0, 1.0, (1, H, T))
    o, SF = O.forward(q, k, v, beta)
    oa, Sa = O.forward(q[..., :T1, :], k[..., :T1, :], v[..., :T1, :], beta[..., :T1])
    ob, Sb = O.forward(q[..., T1:, :], k[..., T1:, :], v[..., T1:, :], beta[..., T1:], initial_state=Sa)
    assert np.allclose(np.concatenate([oa, ob], axis=2), o, rtol=1e-12, atol=1e-12)
    assert np.allclose(Sb, SF, rtol=1e-12, atol=1e-12)
    g = O.backward(q, k, v, beta, do)
    gb = O.backward(q[..., T1:, :], k[..., T1:, :], v[..., T1:, :], beta[..., T1:], do[..., T1:, :],
                    initial_state=Sa)
    ga = O.backward(q[..., :T1, :], k[..., :T1, :], v[..., :T1, :], beta[..., :T1], do[..., :T1, :],
                    d_final_state=gb["d_initial_state"])
    for name in ("dq", "dk", "dv", "dbeta"):
        assert np.allclose(np.concatenate([ga[name], gb[name]], axis=2), g[name], rtol=1e-11, atol=1e-11)


# ---------------------------------------------------------------- backward

def _loss(q, k, v, beta, do, dSF, S0, scale, cu=None, mode="exact"):
    o, SF = O.forward(q, k, v, beta, scale=scale, cu_seqlens=cu, initial_state=S0, mode=mode)
    return float(np.sum(o * do) + np.sum(SF * dSF))


@pytest.mark.parametrize("mode", ["exact", "euler"])
def test_backward_against_central_differences_every_coordinate(mode):
    r = _rng(31)
    B, H, T, dk, dv = 1, 2, 12, 4, 3
    q, k = r.standard_normal((B, H, T, dk)), r.standard_normal((B, H, T, dk)) * 1.5
    v, do = r.standard_normal((B, H, T, dv)), r.standard_normal((B, H, T, dv))
    beta = r.uniform(0.05, 1.0, (B, H, T))
    S0 = r.standard_normal((B, H, dk, dv))
    dSF = r.standard_normal((B, H, dk, dv))
    scale = 0.8
    g = O.backward(q, k, v, beta, do, scale=scale, initial_state=S0, d_final_state=dSF, mode=mode)
    args = dict(q=q, k=k, v=v, beta=beta, S0=S0)
    names = dict(q="dq", k="dk", v="dv", beta="dbeta", S0="d_initial_state")
    eps = 1e-6
    for name, x in args.items():
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            ap, am = dict(args, **{name: xp}), dict(args, **{name: xm})
            fd[idx] = (_loss(ap["q"], ap["k"], ap["v"], ap["beta"], do, dSF, ap["S0"], scale, mode=mode)
                       - _loss(am["q"], am["k"], am["v"], am["beta"], do, dSF, am["S0"], scale,
                               mode=mode)) / (2 * eps)
        assert np.max(np.abs(fd - g[names[name]])) < 1e-7 * max(1.0, np.max(np.abs(fd))), name


def test_backward_directional_derivative_multi_chunk_packed():
    """Several 64-token blocks and a packed batch: <grad, u> against a central difference along u."""
    r = _rng(32)
    H, dk, dv = 2, 6, 5
    cu = np.array([0, 3, 140, 141, 230], dtype=np.int32)
    T = int(cu[-1])
    q, k = r.standard_normal((1, H, T, dk)), r.standard_normal((1, H, T, dk)) * 1.3
    v, do = r.standard_normal((1, H, T, dv)), r.standard_normal((1, H, T, dv))
    beta = r.uniform(0.0, 1.0, (1, H, T))
    S0 = np.zeros((4, H, dk, dv))
    dSF = np.zeros((4, H, dk, dv))
    g = O.backward(q, k, v, beta, do, scale=1.0, cu_seqlens=cu)
    for trial in range(3):
        u = {n: r.standard_normal(x.shape) for n, x in dict(q=q, k=k, v=v, beta=beta).items()}
        eps = 1e-6
        lp = _loss(q + eps * u["q"], k + eps * u["k"], v + eps * u["v"], beta + eps * u["beta"],
                   do, dSF, S0, 1.0, cu)
        lm = _loss(q - eps * u["q"], k - eps * u["k"], v - eps * u["v"], beta - eps * u["beta"],
                   do, dSF, S0, 1.0, cu)
        fd = (lp - lm) / (2 * eps)
        an = sum(np.sum(g["d" + n] * u[n]) for n in ("q", "k", "v", "beta"))
        assert abs(fd - an) < 1e-6 * max(1.0, abs(an))


def test_backward_at_stiff_and_degenerate_keys():
    """Keys with ||k|| from 1e-3 to 100 and exact zeros (lambda -> 0, e^{-x} underflow)."""
    r = _rng(33)
    H, T, dk, dv = 1, 20, 4, 3
    kdir = r.standard_normal((1, H, T, dk))
    kdir /= np.linalg.norm(kdir, axis=-1, keepdims=True)
    norms = np.exp(r.uniform(np.log(1e-3), np.log(100.0), (1, H, T, 1)))
    k = kdir * norms
    k[0, 0, 4] = 0.0
    q, v, do = r.standard_normal((1, H, T, dk)), r.standard_normal((1, H, T, dv)), r.standard_normal((1, H, T, dv))
    beta = r.uniform(0.0, 1.0, (1, H, T))
    g = O.backward(q, k, v, beta, do)
    zero = np.zeros((1, H, dk, dv))
    for name, x in dict(q=q, k=k, v=v, beta=beta).items():
        for idx in [tuple(r.integers(0, s) for s in x.shape) for _ in range(15)]:
            h = 1e-7 * max(1.0, abs(x[idx]))
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            a = dict(q=q, k=k, v=v, beta=beta)
            lp = _loss(**{**a, name: xp}, do=do, dSF=zero, S0=None, scale=1.0)
            lm = _loss(**{**a, name: xm}, do=do, dSF=zero, S0=None, scale=1.0)
            fd = (lp - lm) / (2 * h)
            assert abs(fd - g["d" + name][idx]) < 2e-5 * max(1.0, abs(fd)), (name, idx)


# ---------------------------------------------------------------- stored regression case

def test_golden_tiny_case_unchanged():
    """tests/golden/tiny_case.json was written by tests/golden/make_golden.py from the oracle."""
    with open(os.path.join(HERE, "golden", "tiny_case.json")) as f:
        gold = json.load(f)
    inp = {n: np.array(gold["inputs"][n]) for n in ("q", "k", "v", "beta", "do")}
    o, _ = O.forward(inp["q"], inp["k"], inp["v"], inp["beta"], scale=gold["scale"])
    g = O.backward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["do"], scale=gold["scale"])
    assert np.allclose(o, np.array(gold["o"]), rtol=1e-13, atol=1e-14)
    for name in ("dq", "dk", "dv", "dbeta"):
        assert np.allclose(g[name], np.array(gold[name]), rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- gated EFLA
# Reading (oracle docstring): the log-decay a_t adds gamma_t I to the dynamics matrix over the
# step interval [0, beta_t], gamma_t beta_t = -a_t. The pins integrate that ODE directly.

def _gated_dense(S, k, v, beta, a):
    """By definition: e^{-beta M} S + int_0^beta e^{-(beta - tau) M} dtau (k v^T), M = gamma I + k k^T."""
    gamma = -a / beta
    M = gamma * np.eye(len(k)) + np.outer(k, k)
    E = scipy.linalg.expm(-beta * M)
    integral, _ = scipy.integrate.quad_vec(lambda tau: scipy.linalg.expm(-(beta - tau) * M) @ np.outer(k, v),
                                           0.0, beta, epsabs=1e-15, epsrel=1e-13)
    return E @ S + integral


def _gated_van_loan(S, k, v, beta, a):
    dk, dv = len(k), len(v)
    Mb = np.zeros((dk + dv, dk + dv))
    Mb[:dk, :dk] = -((-a / beta) * np.eye(dk) + np.outer(k, k))
    Mb[:dk, dk:] = np.outer(k, v)
    E = scipy.linalg.expm(beta * Mb)
    return E[:dk, :dk] @ S + E[:dk, dk:]


def _gated_one_seq(S0, ks, vs, betas, gates, qs=None, scale=1.0):
    ks, vs = np.atleast_2d(ks), np.atleast_2d(vs)
    T = ks.shape[0]
    qs = np.zeros_like(ks) if qs is None else qs
    o, SF = O.gated_forward(qs[None, None], ks[None, None], vs[None, None],
                            np.asarray(betas, dtype=np.float64).reshape(1, 1, T),
                            np.asarray(gates, dtype=np.float64).reshape(1, 1, T), scale=scale,
                            initial_state=None if S0 is None else S0[None, None])
    return o[0, 0], SF[0, 0]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_gated_token_update_equals_dense_flow(seed):
    """One gated token equals expm + quadrature of the decayed ZOH integral (d_k=5, d_v=4)."""
    r = _rng(100 + seed)
    S = r.standard_normal((5, 4))
    k = r.standard_normal(5) * r.uniform(0.3, 2.0)
    v = r.standard_normal(4)
    beta, a = r.uniform(0.1, 1.5), -r.uniform(0.01, 2.0)
    _, S1 = _gated_one_seq(S, k, v, [beta], [a])
    ref = _gated_dense(S, k, v, beta, a)
    assert np.max(np.abs(S1 - ref)) < 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_gated_sequence_equals_van_loan_flow():
    """Ten gated tokens, outputs and states, against the Van Loan block exponential."""
    r = _rng(120)
    dk, dv, T = 6, 3, 10
    ks = r.standard_normal((T, dk)) * r.uniform(0.2, 3.0, (T, 1))
    vs, qs = r.standard_normal((T, dv)), r.standard_normal((T, dk))
    betas, gates = r.uniform(0.05, 2.0, T), -r.uniform(0.0, 3.0, T)
    S0 = r.standard_normal((dk, dv))
    o, SF = _gated_one_seq(S0, ks, vs, betas, gates, qs, scale=0.6)
    S = S0
    for t in range(T):
        S = _gated_van_loan(S, ks[t], vs[t], betas[t], gates[t])
        assert np.allclose(o[t], 0.6 * S.T @ qs[t], rtol=1e-12, atol=1e-12)
    assert np.allclose(SF, S, rtol=1e-12, atol=1e-12)


def test_gated_special_cases():
    """a = 0 is EFLA; k = 0 is pure decay S_t = e^{a_t} S_{t-1}; lambda -> 0 gives the decayed
    Euler-like input b = beta (1 - e^{a}) / (-a)."""
    r = _rng(130)
    B, H, T, dk, dv = 1, 2, 70, 6, 5
    q, k, v = r.standard_normal((B, H, T, dk)), r.standard_normal((B, H, T, dk)), r.standard_normal((B, H, T, dv))
    beta, a = r.uniform(0, 1, (B, H, T)), -r.uniform(0, 1, (B, H, T))
    S0 = r.standard_normal((B, H, dk, dv))
    o_g, f_g = O.gated_forward(q, k, v, beta, np.zeros_like(a), initial_state=S0)
    o_e, f_e = O.forward(q, k, v, beta, initial_state=S0)
    assert O.rel_err(o_g, o_e) < 1e-14 and O.rel_err(f_g, f_e) < 1e-14
    o_z, f_z = O.gated_forward(q, np.zeros_like(k), v, beta, a, initial_state=S0)
    cum = np.cumsum(a, axis=-1)
    ref = np.exp(cum)[..., None] * np.einsum("bhtd,bhdv->bhtv", q, S0)
    assert O.rel_err(o_z, ref) < 1e-13
    co = O.gated_coefficients(np.full((3, 4), 1e-9), np.array([0.5, 1.0, 2.0]), np.array([-0.3, -1.0, -2.5]))
    assert np.allclose(co["b"], np.array([0.5, 1.0, 2.0]) * (1 - np.exp([-0.3, -1.0, -2.5])) / np.array([0.3, 1.0, 2.5]), rtol=1e-12)


def test_gated_chunk_form_equals_token_recurrence():
    """The decayed chunk algebra the kernels use (cumulative log-decays inside each chunk) equals
    the token recurrence, with a ragged tail, a carried initial state and strong decay."""
    r = _rng(140)
    B, H, T, dk, dv = 2, 2, 64 * 3 + 17, 8, 6
    q, k, v = r.standard_normal((B, H, T, dk)), r.standard_normal((B, H, T, dk)) * 0.6, r.standard_normal((B, H, T, dv))
    beta, a = r.uniform(0, 1, (B, H, T)), -r.uniform(0, 2.0, (B, H, T))
    S0 = r.standard_normal((B, H, dk, dv))
    o, f = O.gated_forward(q, k, v, beta, a, scale=0.9, initial_state=S0)
    c = O.gated_chunk_forward(q, k, v, beta, a, scale=0.9, initial_state=S0)
    assert O.rel_err(c["o"], o) < 1e-12 and O.rel_err(c["final"], f) < 1e-12
    # a wrong decay on the output's state term (Gamma_{t-1} instead of Gamma_t) is caught
    ob = O.gated_chunk_forward(q, k, v, beta, np.roll(a, 1, axis=-1), scale=0.9, initial_state=S0)
    assert O.rel_err(ob["o"], o) > 1e-3


@pytest.mark.parametrize("C", [64, 37])
def test_gated_chunk_factors_reproduce_token_recurrence(C):
    """From a zero state one chunk's read-out is o = scale M (X diag(b) V): the decayed M and X of
    gated_chunk_factors against the token recurrence (strong decays; a full and a ragged chunk).
    A zero gate gives chunk_factors' M and X."""
    r = _rng(150 + C)
    dk, dv = 8, 5
    q, k, v = r.standard_normal((C, dk)), r.standard_normal((C, dk)) * 0.7, r.standard_normal((C, dv))
    beta, a = r.uniform(0, 1, C), -r.uniform(0, 1.5, C)
    f = O.gated_chunk_factors(q, k, beta, a)
    b = O.gated_coefficients(k, beta, a)["b"]
    o = 0.7 * f["M"] @ (f["X"] @ (b[:, None] * v))
    ref, _ = O.gated_forward(q[None, None], k[None, None], v[None, None], beta[None, None], a[None, None], scale=0.7)
    assert O.rel_err(o, ref[0, 0]) < 1e-12
    # the decay taken the wrong way round (e^{c_s - c_t}) is caught
    bad = np.tril(q @ k.T) * np.exp(np.tril(np.cumsum(a)[None, :] - np.cumsum(a)[:, None]))
    assert O.rel_err(0.7 * bad @ (f["X"] @ (b[:, None] * v)), ref[0, 0]) > 1e-3
    z = O.gated_chunk_factors(q, k, beta, np.zeros(C))
    u = O.chunk_factors(q, k, beta)
    assert O.rel_err(z["M"], u["M"]) < 1e-14 and O.rel_err(z["X"], u["X"]) < 1e-14


@pytest.mark.parametrize("mode", ["exact", "euler"])
def test_gated_backward_against_central_differences(mode):
    """Every coordinate of every input of gated EFLA (q, k, v, beta, gate, initial state) by
    central differences of sum(o * do) + <final state, d_final>, T = 11 (d_k = 4, d_v = 3)."""
    r = _rng(150)
    B, H, T, dk, dv = 1, 1, 11, 4, 3
    q, k, v = r.standard_normal((B, H, T, dk)), r.standard_normal((B, H, T, dk)) * 0.8, r.standard_normal((B, H, T, dv))
    beta, gate = r.uniform(0.1, 1.0, (B, H, T)), -r.uniform(0.05, 1.5, (B, H, T))
    S0, do, dF = r.standard_normal((B, H, dk, dv)), r.standard_normal((B, H, T, dv)), r.standard_normal((B, H, dk, dv))

    def loss(q_, k_, v_, b_, g_, s_):
        o, f = O.gated_forward(q_, k_, v_, b_, g_, scale=0.7, initial_state=s_, mode=mode)
        return np.sum(o * do) + np.sum(f * dF)

    g = O.gated_backward(q, k, v, beta, gate, do, scale=0.7, initial_state=S0, d_final_state=dF, mode=mode)
    args = [q, k, v, beta, gate, S0]
    names = ["dq", "dk", "dv", "dbeta", "dgate", "d_initial_state"]
    eps = 1e-6
    for i, (x, nm) in enumerate(zip(args, names)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp, xm = [a.copy() for a in args], [a.copy() for a in args]
            xp[i][idx] += eps
            xm[i][idx] -= eps
            num[idx] = (loss(*xp) - loss(*xm)) / (2 * eps)
        assert np.max(np.abs(num - g[nm])) < 1e-7 * max(1.0, np.max(np.abs(num))), (nm, np.max(np.abs(num - g[nm])))


@pytest.mark.parametrize("mode", ["exact", "euler"])
def test_gated_packed_backward_against_central_differences(mode):
    """Packed batch (cu_seqlens with an empty and a one-token sequence): every coordinate of
    every input by central differences of the packed gated forward's loss, states per sequence."""
    r = _rng(151)
    cu = np.array([0, 3, 3, 4, 9])
    H, T, dk, dv, n = 2, 9, 3, 2, 4
    q, k, v = r.standard_normal((1, H, T, dk)), r.standard_normal((1, H, T, dk)) * 0.8, r.standard_normal((1, H, T, dv))
    beta, gate = r.uniform(0.1, 1.0, (1, H, T)), -r.uniform(0.05, 1.5, (1, H, T))
    S0, do, dF = r.standard_normal((n, H, dk, dv)), r.standard_normal((1, H, T, dv)), r.standard_normal((n, H, dk, dv))

    def loss(q_, k_, v_, b_, g_, s_):
        o, f = O.gated_forward(q_, k_, v_, b_, g_, scale=0.7, cu_seqlens=cu, initial_state=s_, mode=mode)
        return np.sum(o * do) + np.sum(f * dF)

    g = O.gated_backward(q, k, v, beta, gate, do, scale=0.7, initial_state=S0, d_final_state=dF,
                         mode=mode, cu_seqlens=cu)
    args = [q, k, v, beta, gate, S0]
    names = ["dq", "dk", "dv", "dbeta", "dgate", "d_initial_state"]
    eps = 1e-6
    for i, (x, nm) in enumerate(zip(args, names)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp, xm = [a.copy() for a in args], [a.copy() for a in args]
            xp[i][idx] += eps
            xm[i][idx] -= eps
            num[idx] = (loss(*xp) - loss(*xm)) / (2 * eps)
        assert np.max(np.abs(num - g[nm])) < 1e-7 * max(1.0, np.max(np.abs(num))), (nm, np.max(np.abs(num - g[nm])))
    # the empty sequence passes its final-state gradient straight through
    assert np.array_equal(g["d_initial_state"][1], dF[1])


def test_gated_packed_equals_separate_sequences():
    """Packed forward and backward equal the same sequences run one by one as dense batches."""
    r = _rng(152)
    lens = [5, 0, 1, 70, 9]
    cu = np.concatenate([[0], np.cumsum(lens)])
    H, T, dk, dv, n = 2, int(cu[-1]), 4, 3, len(lens)
    q, k, v = r.standard_normal((1, H, T, dk)), r.standard_normal((1, H, T, dk)) * 0.7, r.standard_normal((1, H, T, dv))
    beta, gate = r.uniform(0.1, 1.0, (1, H, T)), -r.uniform(0.0, 1.0, (1, H, T))
    S0, do, dF = r.standard_normal((n, H, dk, dv)), r.standard_normal((1, H, T, dv)), r.standard_normal((n, H, dk, dv))
    o, f = O.gated_forward(q, k, v, beta, gate, 0.9, cu_seqlens=cu, initial_state=S0)
    g = O.gated_backward(q, k, v, beta, gate, do, 0.9, S0, dF, cu_seqlens=cu)
    for i in range(n):
        sl = lambda x: x[:, :, cu[i]:cu[i + 1]]
        o1, f1 = O.gated_forward(sl(q), sl(k), sl(v), sl(beta), sl(gate), 0.9, initial_state=S0[i:i + 1])
        g1 = O.gated_backward(sl(q), sl(k), sl(v), sl(beta), sl(gate), sl(do), 0.9, S0[i:i + 1], dF[i:i + 1])
        assert np.array_equal(sl(o), o1) and np.array_equal(f[i], f1[0])
        for nm in ("dq", "dk", "dv", "dbeta", "dgate"):
            assert np.array_equal(sl(g[nm]), g1[nm]), nm
        assert np.array_equal(g["d_initial_state"][i], g1["d_initial_state"][0])


@pytest.mark.parametrize("mode", ["exact", "euler"])
def test_gated_chunk_backward_equals_token_backward(mode):
    """The chunkwise gated backward (decayed UT factors, running log-decay sums) equals the
    hand-written token backward (itself pinned by central differences), ragged tail included."""
    r = _rng(160)
    B, H, T, dk, dv = 1, 2, 64 * 2 + 21, 6, 5
    q, k, v = r.standard_normal((B, H, T, dk)), r.standard_normal((B, H, T, dk)) * 0.6, r.standard_normal((B, H, T, dv))
    beta, a = r.uniform(0, 1, (B, H, T)), -r.uniform(0, 1.5, (B, H, T))
    do, S0, dF = r.standard_normal((B, H, T, dv)), r.standard_normal((B, H, dk, dv)), r.standard_normal((B, H, dk, dv))
    g1 = O.gated_backward(q, k, v, beta, a, do, 0.8, S0, dF, mode=mode)
    g2 = O.gated_chunk_backward(q, k, v, beta, a, do, 0.8, initial_state=S0, d_final_state=dF, mode=mode)
    for n in g1:
        assert O.rel_err(g2[n], g1[n]) < 1e-12, n

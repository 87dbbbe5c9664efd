"""Plain fp64 CPU oracle for Exact Flow Linear Attention (EFLA).

TEST INFRASTRUCTURE. Only the tests, the smoke check and the CPU-baseline leg of
the benchmark may import or run this module. The HIP library never calls it, and
this module shares no code, table or helper with the HIP library.

What is computed (Exact Flow Linear Attention summary page; the pages print no
equation, so the steps below are the plain reading of their statements):

* Memory dynamics (section 3.1): on token t the d_k x d_v state obeys
  dS/dtau = -A_t S + b_t for tau in [0, beta_t], with A_t = k_t k_t^T (the
  rank-1 dynamics matrix named in section 6) and input b_t = k_t v_t^T held
  constant on the interval (zero-order hold).
* Exact flow (sections 3.2 and 6, Appendix E): S_t = e^{-beta A} S_{t-1}
  + int_0^beta e^{-(beta-tau) A} dtau b. Because A^2 = lambda A with
  lambda = k^T k (Appendix D: A is a scaled projection), the exponential is
  I - (1 - e^{-beta lambda})/lambda * k k^T and the integral applied to b is
  (1 - e^{-beta lambda})/lambda * k v^T. The update therefore keeps the delta
  rule's form with beta_t replaced by alpha_t = (1 - e^{-beta_t lambda_t}) / lambda_t
  (section 3.2):  S_t = S_{t-1} + alpha_t k_t (v_t - S_{t-1}^T k_t)^T.
* Read-out: o_t = scale * S_t^T q_t, taken after the update of token t
  (the causal mask of section 2 keeps the diagonal).
* Chunkwise form (section 3.3, UT transform): for a chunk with rows K, V, Q and
  incoming state S, T = (I + strictly_lower(diag(alpha) K K^T))^{-1} diag(alpha),
  W = T K, U = T V, U~ = U - W S, O = scale (Q S + tril(Q K^T) U~),
  S' = S + K^T U~.  Used only to produce per-stage values for tests.
* Backward: reverse-mode differentiation of the token recurrence, written out
  by hand (below); pinned against central finite differences in the tests.

The state starts at zero (or at a given initial state) for every sequence;
packed batches restart the state at every cu_seqlens offset.

Gated EFLA (section 3.4 names it; Appendix E/F apply the exact flow to Gated DeltaNet with an
integrating factor; no formula is printed). Reading taken: a per-token log-decay a_t <= 0
enters the dynamics matrix as a multiple of the identity over the step interval,
dS/dtau = -(gamma_t I + k_t k_t^T) S + k_t v_t^T, tau in [0, beta_t], gamma_t beta_t = -a_t.
The identity part commutes with the rank-1 part, so the exact flow is
  S_t = g_t (I - alpha_t k_t k_t^T) S_{t-1} + b_t k_t v_t^T,
  g_t = e^{a_t},  alpha_t = beta_t phi(beta_t lambda_t),  b_t = beta_t phi(beta_t lambda_t - a_t)
(the input integral int_0^beta e^{-(gamma + lambda) s} ds k v^T). a = 0 is EFLA.
"""
from __future__ import annotations

import numpy as np
import scipy.linalg

CHUNK = 64

# Below this |x| the functions phi and phi' are summed from their Taylor series;
# 25 terms keep the truncation error under 1e-25 for |x| < 1.
_SERIES_BELOW = 1.0
_SERIES_TERMS = 25


def phi(x):
    """phi(x) = (1 - e^{-x}) / x, phi(0) = 1, so alpha = beta * phi(beta * lambda).

    Taylor series sum_{n>=0} (-x)^n / (n+1)! near zero, -expm1(-x)/x elsewhere.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    small = np.abs(x) < _SERIES_BELOW
    xs = x[small]
    term = np.ones_like(xs)
    acc = np.ones_like(xs)
    for n in range(1, _SERIES_TERMS):
        term = term * (-xs) / (n + 1)
        acc = acc + term
    out[small] = acc
    xl = x[~small]
    out[~small] = -np.expm1(-xl) / xl
    return out


def dphi(x):
    """phi'(x) = (e^{-x} (1 + x) - 1) / x^2, phi'(0) = -1/2.

    Taylor series sum_{n>=1} -n (-x)^{n-1} / (n+1)! near zero (the closed form
    cancels catastrophically there), the closed form elsewhere.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    small = np.abs(x) < _SERIES_BELOW
    xs = x[small]
    s = np.full_like(xs, 0.5)          # (-x)^{n-1} / (n+1)! at n = 1
    acc = -1.0 * s
    for n in range(2, _SERIES_TERMS + 1):
        s = s * (-xs) / (n + 1)
        acc = acc - n * s
    out[small] = acc
    xl = x[~small]
    out[~small] = (np.exp(-xl) * (1.0 + xl) - 1.0) / (xl * xl)
    return out


MODES = ("exact", "euler")


def alpha(beta, lam, mode="exact"):
    """Effective step of the exact flow: (1 - e^{-beta lambda}) / lambda; beta when lambda = 0.

    mode "euler" is the delta rule's own step, alpha = beta: the explicit Euler step of the
    same dynamics (summary page, section 2), kept as the comparison mode."""
    beta = np.asarray(beta, dtype=np.float64)
    lam = np.asarray(lam, dtype=np.float64)
    if mode == "euler":
        return beta + 0.0 * lam
    assert mode == "exact", mode
    return beta * phi(beta * lam)


def coefficients(k, beta, mode="exact"):
    """Per-token lambda = ||k||^2, alpha, d alpha / d beta = e^{-beta lambda} and
    d alpha / d lambda = beta^2 phi'(beta lambda) (1 and 0 in mode "euler").
    k: [..., d_k]; beta: [...]."""
    k = np.asarray(k, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    lam = np.sum(k * k, axis=-1)
    if mode == "euler":
        return dict(lam=lam, alpha=beta.copy(), dalpha_dbeta=np.ones_like(beta),
                    dalpha_dlam=np.zeros_like(beta))
    assert mode == "exact", mode
    x = beta * lam
    return dict(lam=lam, alpha=beta * phi(x), dalpha_dbeta=np.exp(-x),
                dalpha_dlam=beta * beta * dphi(x))


# ---------------------------------------------------------------------------
# Token-by-token recurrence over N independent streams of length L.
# ---------------------------------------------------------------------------

def _forward_streams(q, k, v, beta, scale, S0, checkpoint_every=0, mode="exact"):
    """q, k: [N, L, dk]; v: [N, L, dv]; beta: [N, L]; S0: [N, dk, dv] or None.

    Returns o [N, L, dv], final state [N, dk, dv] and, when checkpoint_every > 0,
    the states entering each block of that many tokens.
    """
    N, L, dk = k.shape
    dv = v.shape[-1]
    S = np.zeros((N, dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((N, L, dv))
    checkpoints = []
    a = alpha(beta, np.sum(k * k, axis=-1), mode)      # [N, L]
    for t in range(L):
        if checkpoint_every and t % checkpoint_every == 0:
            checkpoints.append(S.copy())
        kt = k[:, t, :]
        r = v[:, t, :] - np.einsum("nd,ndv->nv", kt, S)   # v_t - S_{t-1}^T k_t
        S = S + a[:, t, None, None] * kt[:, :, None] * r[:, None, :]
        o[:, t, :] = scale * np.einsum("nd,ndv->nv", q[:, t, :], S)
    return o, S, checkpoints


def _backward_streams(q, k, v, beta, do, scale, S0, dS_final, mode="exact"):
    """Reverse-mode gradients of sum(o * do) (+ <S_final, dS_final>) for _forward_streams.

    The state is stored only at block boundaries of CHUNK tokens and rebuilt
    inside each block during the reverse sweep.
    """
    N, L, dk = k.shape
    dv = v.shape[-1]
    co = coefficients(k, beta, mode)
    a = co["alpha"]
    _, _, ckpt = _forward_streams(q, k, v, beta, scale, S0, checkpoint_every=CHUNK, mode=mode)
    dq = np.zeros_like(q)
    dk_ = np.zeros_like(k)
    dv_ = np.zeros_like(v)
    dalpha = np.zeros((N, L))
    dS = np.zeros((N, dk, dv)) if dS_final is None else np.array(dS_final, dtype=np.float64)
    nblk = (L + CHUNK - 1) // CHUNK
    for blk in range(nblk - 1, -1, -1):
        t0, t1 = blk * CHUNK, min(L, (blk + 1) * CHUNK)
        # Rebuild S_{t-1} (states[i]) and S_t (states[i+1]) for the tokens of this block.
        states = [ckpt[blk]]
        for t in range(t0, t1):
            S = states[-1]
            kt = k[:, t, :]
            r = v[:, t, :] - np.einsum("nd,ndv->nv", kt, S)
            states.append(S + a[:, t, None, None] * kt[:, :, None] * r[:, None, :])
        for t in range(t1 - 1, t0 - 1, -1):
            S_prev, S_t = states[t - t0], states[t - t0 + 1]
            kt, qt = k[:, t, :], q[:, t, :]
            # o_t = scale * S_t^T q_t
            dS = dS + scale * qt[:, :, None] * do[:, t, None, :]
            dq[:, t, :] = scale * np.einsum("ndv,nv->nd", S_t, do[:, t, :])
            # S_t = S_{t-1} + alpha_t k_t r_t^T,  r_t = v_t - S_{t-1}^T k_t
            r = v[:, t, :] - np.einsum("nd,ndv->nv", kt, S_prev)
            dS_r = np.einsum("ndv,nv->nd", dS, r)               # dS r
            dalpha[:, t] = np.einsum("nd,nd->n", kt, dS_r)
            dr = a[:, t, None] * np.einsum("ndv,nd->nv", dS, kt)   # alpha dS^T k
            dv_[:, t, :] = dr
            dk_[:, t, :] = a[:, t, None] * dS_r - np.einsum("ndv,nv->nd", S_prev, dr)
            dS = dS - kt[:, :, None] * dr[:, None, :]
    # alpha_t = alpha(beta_t, lambda_t), lambda_t = ||k_t||^2
    dbeta = dalpha * co["dalpha_dbeta"]
    dk_ = dk_ + 2.0 * k * (dalpha * co["dalpha_dlam"])[:, :, None]
    return dq, dk_, dv_, dbeta, dS


# ---------------------------------------------------------------------------
# [B, H, T, d] layout and packed batches.
# ---------------------------------------------------------------------------

def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def sequences(B, T, cu_seqlens):
    """(batch index, start, end) of every sequence; packed batches have B == 1."""
    if cu_seqlens is None:
        return [(b, 0, T) for b in range(B)]
    cu = [int(c) for c in np.asarray(cu_seqlens)]
    if B != 1 or cu[0] != 0 or cu[-1] != T or any(cu[i] > cu[i + 1] for i in range(len(cu) - 1)):
        raise ValueError("cu_seqlens must start at 0, end at T, be non-decreasing, with B == 1")
    return [(0, cu[i], cu[i + 1]) for i in range(len(cu) - 1)]


def forward(q, k, v, beta, scale=1.0, cu_seqlens=None, initial_state=None, mode="exact"):
    """EFLA forward (mode "euler": the delta rule). q, k: [B,H,T,dk]; v: [B,H,T,dv]; beta: [B,H,T].

    initial_state: None or [n_seq, H, dk, dv] (n_seq = B, or the number of packed
    sequences). Returns (o [B,H,T,dv], final_state [n_seq, H, dk, dv]), fp64.
    """
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    o = np.zeros((B, H, T, dv))
    seqs = sequences(B, T, cu_seqlens)
    final = np.zeros((len(seqs), H, dk, dv))
    S0 = _f64(initial_state)
    for i, (b, s, e) in enumerate(seqs):
        o_i, S_i, _ = _forward_streams(q[b, :, s:e], k[b, :, s:e], v[b, :, s:e], beta[b, :, s:e],
                                       scale, None if S0 is None else S0[i], mode=mode)
        o[b, :, s:e] = o_i
        final[i] = S_i
    return o, final


def backward(q, k, v, beta, do, scale=1.0, cu_seqlens=None, initial_state=None,
             d_final_state=None, mode="exact"):
    """Gradients of sum(o * do) (+ <final_state, d_final_state>) for `forward`.

    Returns dict(dq, dk, dv, dbeta, d_initial_state), fp64.
    """
    q, k, v, beta, do = _f64(q), _f64(k), _f64(v), _f64(beta), _f64(do)
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    seqs = sequences(B, T, cu_seqlens)
    S0 = _f64(initial_state)
    dSF = _f64(d_final_state)
    g = dict(dq=np.zeros_like(q), dk=np.zeros_like(k), dv=np.zeros_like(v),
             dbeta=np.zeros_like(beta), d_initial_state=np.zeros((len(seqs), H, dk, dv)))
    for i, (b, s, e) in enumerate(seqs):
        dq, dk_, dv_, dbeta, dS0 = _backward_streams(
            q[b, :, s:e], k[b, :, s:e], v[b, :, s:e], beta[b, :, s:e], do[b, :, s:e], scale,
            None if S0 is None else S0[i], None if dSF is None else dSF[i], mode=mode)
        g["dq"][b, :, s:e] = dq
        g["dk"][b, :, s:e] = dk_
        g["dv"][b, :, s:e] = dv_
        g["dbeta"][b, :, s:e] = dbeta
        g["d_initial_state"][i] = dS0
    return g


# ---------------------------------------------------------------------------
# Chunkwise (UT transform) form: per-stage values for tests of the GPU stages.
# ---------------------------------------------------------------------------

def chunk_ut(k, v, beta, mode="exact"):
    """UT transform of one chunk. k: [C, dk]; v: [C, dv]; beta: [C].

    Returns dict(alpha, T, W, U) with T = (I + strictly_lower(diag(alpha) K K^T))^{-1} diag(alpha).
    """
    k, v, beta = _f64(k), _f64(v), _f64(beta)
    C = k.shape[0]
    a = alpha(beta, np.sum(k * k, axis=-1), mode)
    A = np.tril(a[:, None] * (k @ k.T), -1)
    T = scipy.linalg.solve_triangular(np.eye(C) + A, np.diag(a), lower=True, unit_diagonal=True)
    return dict(alpha=a, T=T, W=T @ k, U=T @ v)


def chunk_factors(q, k, beta, mode="exact"):
    """Per-chunk factors the forward keeps for the backward pass (section 3.3).

    q, k: [C, dk]; beta: [C]. Returns dict(X, M): X = (I + strictly_lower(diag(alpha) K K^T))^{-1},
    the inverse whose product with diag(alpha) is the UT factor T, and M = tril(Q K^T), the
    causal score block (diagonal kept) of the intra-chunk read-out."""
    q, k, beta = _f64(q), _f64(k), _f64(beta)
    C = k.shape[0]
    a = alpha(beta, np.sum(k * k, axis=-1), mode)
    A = np.tril(a[:, None] * (k @ k.T), -1)
    X = scipy.linalg.solve_triangular(np.eye(C) + A, np.eye(C), lower=True, unit_diagonal=True)
    return dict(X=X, M=np.tril(q @ k.T))


def chunk_forward(q, k, v, beta, scale=1.0, cu_seqlens=None, chunk=CHUNK):
    """Chunkwise forward: returns o [B,H,T,dv], W [B,H,T,dk], U [B,H,T,dv],
    U~ = U - W S [B,H,T,dv] and the list of per-chunk incoming states, one entry
    per (sequence, chunk) in sequence order, each [H, dk, dv]."""
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    o = np.zeros((B, H, T, dv))
    Wf = np.zeros((B, H, T, dk))
    Uf = np.zeros((B, H, T, dv))
    Ut = np.zeros((B, H, T, dv))
    states = []
    for (b, s, e) in sequences(B, T, cu_seqlens):
        S = np.zeros((H, dk, dv))
        for c0 in range(s, e, chunk):
            c1 = min(e, c0 + chunk)
            states.append(S.copy())
            for h in range(H):
                f = chunk_ut(k[b, h, c0:c1], v[b, h, c0:c1], beta[b, h, c0:c1])
                Q, K = q[b, h, c0:c1], k[b, h, c0:c1]
                U_t = f["U"] - f["W"] @ S[h]
                o[b, h, c0:c1] = scale * (Q @ S[h] + np.tril(Q @ K.T) @ U_t)
                Wf[b, h, c0:c1], Uf[b, h, c0:c1], Ut[b, h, c0:c1] = f["W"], f["U"], U_t
                S[h] = S[h] + K.T @ U_t
    return dict(o=o, W=Wf, U=Uf, Ut=Ut, states=states)


def euler_forward(q, k, v, beta, scale=1.0, cu_seqlens=None):
    """The Euler (DeltaNet) recurrence with the raw step beta_t, for comparisons."""
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    o = np.zeros((B, H, T, dv))
    for (b, s, e) in sequences(B, T, cu_seqlens):
        S = np.zeros((H, dk, dv))
        for t in range(s, e):
            kt = k[b, :, t]
            r = v[b, :, t] - np.einsum("hd,hdv->hv", kt, S)
            S = S + beta[b, :, t, None, None] * kt[:, :, None] * r[:, None, :]
            o[b, :, t] = scale * np.einsum("hd,hdv->hv", q[b, :, t], S)
    return o


# ---------------------------------------------------------------------------
# Gated EFLA (reading in the module docstring).
# ---------------------------------------------------------------------------

def gated_coefficients(k, beta, gate, mode="exact"):
    """lambda, alpha = beta phi(beta lambda), g = e^a, b = beta phi(beta lambda - a) per token.
    k: [..., d_k]; beta, gate (log-decay a): [...]. mode "euler": alpha = b = beta, the gated
    delta rule's own steps (its explicit-Euler counterpart)."""
    k, beta, gate = _f64(k), _f64(beta), _f64(gate)
    lam = np.sum(k * k, axis=-1)
    if mode == "euler":
        return dict(lam=lam, alpha=beta.copy(), g=np.exp(gate), b=beta.copy())
    assert mode == "exact", mode
    x = beta * lam
    return dict(lam=lam, alpha=beta * phi(x), g=np.exp(gate), b=beta * phi(x - gate))


def gated_forward(q, k, v, beta, gate, scale=1.0, cu_seqlens=None, initial_state=None, mode="exact"):
    """Gated EFLA forward, token by token. gate: log-decay a_t [B,H,T] (a_t <= 0 is a decay).

    Returns (o [B,H,T,dv], final_state [n_seq,H,dk,dv]), fp64."""
    q, k, v, beta, gate = _f64(q), _f64(k), _f64(v), _f64(beta), _f64(gate)
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    c = gated_coefficients(k, beta, gate, mode)
    o = np.zeros((B, H, T, dv))
    seqs = sequences(B, T, cu_seqlens)
    final = np.zeros((len(seqs), H, dk, dv))
    S0 = _f64(initial_state)
    for i, (b, s, e) in enumerate(seqs):
        S = np.zeros((H, dk, dv)) if S0 is None else S0[i].copy()
        for t in range(s, e):
            kt = k[b, :, t]
            kS = np.einsum("hd,hdv->hv", kt, S)                        # k_t^T S_{t-1}
            S = c["g"][b, :, t, None, None] * (S - c["alpha"][b, :, t, None, None] * kt[:, :, None] * kS[:, None, :]) \
                + c["b"][b, :, t, None, None] * kt[:, :, None] * v[b, :, t][:, None, :]
            o[b, :, t] = scale * np.einsum("hd,hdv->hv", q[b, :, t], S)
        final[i] = S
    return o, final


def gated_coefficient_derivatives(k, beta, gate, mode="exact"):
    """Partial derivatives of alpha = beta phi(x) and b = beta phi(x - a), x = beta lambda:
    da/dbeta = e^{-x}, da/dlam = beta^2 phi'(x), db/dbeta = phi(x - a) + x phi'(x - a),
    db/dlam = beta^2 phi'(x - a), db/da = -beta phi'(x - a) (mode "euler": 1, 0, 1, 0, 0)."""
    k, beta, gate = _f64(k), _f64(beta), _f64(gate)
    lam = np.sum(k * k, axis=-1)
    if mode == "euler":
        one, zero = np.ones_like(beta), np.zeros_like(beta)
        return dict(da_dbeta=one, da_dlam=zero, db_dbeta=one, db_dlam=zero, db_da=zero)
    x = beta * lam
    dpg = dphi(x - gate)
    return dict(da_dbeta=np.exp(-x), da_dlam=beta * beta * dphi(x), db_dbeta=phi(x - gate) + x * dpg,
                db_dlam=beta * beta * dpg, db_da=-beta * dpg)


def gated_backward(q, k, v, beta, gate, do, scale=1.0, initial_state=None, d_final_state=None,
                   mode="exact", cu_seqlens=None):
    """Reverse-mode gradients of sum(o * do) (+ <final_state, d_final_state>) for gated_forward
    (dense or packed batches; states per sequence), written out by hand per token:
      S_t = g (S_{t-1} - alpha k y^T) + b k v^T,  y = S_{t-1}^T k,  o_t = scale S_t^T q_t;
      dq = scale S_t do;  dv = b dS^T k;  db = k^T dS v;  dg = <dS, S_{t-1}> - alpha k^T dS y;
      dalpha = -g k^T dS y;  dk = -g alpha (dS y + S_{t-1} dS^T k) + b dS v + 2 k dlambda;
      dS_{t-1} = g (dS - alpha k k^T dS);  da = g dg + db db/da.
    Returns dict(dq, dk, dv, dbeta, dgate, d_initial_state), fp64."""
    q, k, v, beta, gate, do = _f64(q), _f64(k), _f64(v), _f64(beta), _f64(gate), _f64(do)
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    co = gated_coefficients(k, beta, gate, mode)
    de = gated_coefficient_derivatives(k, beta, gate, mode)
    S0 = _f64(initial_state)
    dSF = _f64(d_final_state)
    seqs = sequences(B, T, cu_seqlens)
    out = dict(dq=np.zeros_like(q), dk=np.zeros_like(k), dv=np.zeros_like(v), dbeta=np.zeros_like(beta),
               dgate=np.zeros_like(gate), d_initial_state=np.zeros((len(seqs), H, dk, dv)))
    for i, (b_, s0, s1) in enumerate(seqs):
        Ti = s1 - s0
        for h in range(H):
            tok = (b_, h, slice(s0, s1))
            al, bb, gg = co["alpha"][tok], co["b"][tok], co["g"][tok]
            K, V, Q, dO = k[tok], v[tok], q[tok], do[tok]
            states = [np.zeros((dk, dv)) if S0 is None else S0[i, h].copy()]
            for t in range(Ti):  # all states (tests use short sequences)
                S = states[-1]
                y = S.T @ K[t]
                states.append(gg[t] * (S - al[t] * np.outer(K[t], y)) + bb[t] * np.outer(K[t], V[t]))
            dS = np.zeros((dk, dv)) if dSF is None else dSF[i, h].copy()
            dalpha, dbc, dlg = np.zeros(Ti), np.zeros(Ti), np.zeros(Ti)
            dq_, dk_, dv_ = out["dq"][tok], out["dk"][tok], out["dv"][tok]  # views
            for t in range(Ti - 1, -1, -1):
                Sp, St = states[t], states[t + 1]
                kt = K[t]
                dS = dS + scale * np.outer(Q[t], dO[t])
                dq_[t] = scale * St @ dO[t]
                y = Sp.T @ kt
                dStk = dS.T @ kt
                dv_[t] = bb[t] * dStk
                dbc[t] = kt @ dS @ V[t]
                dg = np.sum(dS * Sp) - al[t] * (kt @ dS @ y)
                dalpha[t] = -gg[t] * (kt @ dS @ y)
                dk_[t] = -gg[t] * al[t] * (dS @ y + Sp @ dStk) + bb[t] * (dS @ V[t])
                dlg[t] = gg[t] * dg
                dS = gg[t] * (dS - al[t] * np.outer(kt, dStk))
            out["d_initial_state"][i, h] = dS
            out["dbeta"][tok] = dalpha * de["da_dbeta"][tok] + dbc * de["db_dbeta"][tok]
            dlam = dalpha * de["da_dlam"][tok] + dbc * de["db_dlam"][tok]
            dk_ += 2.0 * K * dlam[:, None]
            out["dgate"][tok] = dlg + dbc * de["db_da"][tok]
    return out


def gated_chunk_forward(q, k, v, beta, gate, scale=1.0, chunk=CHUNK, initial_state=None, mode="exact"):
    """Chunkwise gated form (dense batches), for tests of the chunk algebra the kernels use.

    Within a chunk with incoming state S, c_t = sum of a over the chunk's tokens up to t,
    Gamma_t = e^{c_t}; A_ts = alpha_t e^{c_t - c_s} k_t . k_s (s < t); X = (I + A)^{-1};
    W = X diag(alpha Gamma) K; U = X diag(b) V; U~ = U - W S;
    O = scale (diag(Gamma) Q S + (tril(Q K^T) * e^{c_t - c_s}) U~);
    S' = Gamma_C S + K^T diag(e^{c_C - c_t}) U~.
    Returns dict(o, final, W, U, Ut, cum) with cum the per-token c (restarting at each chunk)."""
    q, k, v, beta, gate = _f64(q), _f64(k), _f64(v), _f64(beta), _f64(gate)
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    co = gated_coefficients(k, beta, gate, mode)
    o = np.zeros((B, H, T, dv))
    Wf, Uf, Ut = np.zeros((B, H, T, dk)), np.zeros((B, H, T, dv)), np.zeros((B, H, T, dv))
    cum = np.zeros((B, H, T))
    final = np.zeros((B, H, dk, dv))
    S0 = _f64(initial_state)
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else S0[b, h].copy()
            for c0 in range(0, T, chunk):
                c1 = min(T, c0 + chunk)
                K, V, Q = k[b, h, c0:c1], v[b, h, c0:c1], q[b, h, c0:c1]
                al, bb = co["alpha"][b, h, c0:c1], co["b"][b, h, c0:c1]
                cc = np.cumsum(gate[b, h, c0:c1])
                D = np.exp(np.tril(cc[:, None] - cc[None, :]))          # e^{c_t - c_s}, s <= t
                A = np.tril(al[:, None] * D * (K @ K.T), -1)
                X = np.linalg.inv(np.eye(c1 - c0) + A)
                W = X @ ((al * np.exp(cc))[:, None] * K)
                U = X @ (bb[:, None] * V)
                U_t = U - W @ S
                o[b, h, c0:c1] = scale * (np.exp(cc)[:, None] * (Q @ S) + (np.tril(Q @ K.T) * D) @ U_t)
                S = np.exp(cc[-1]) * S + K.T @ (np.exp(cc[-1] - cc)[:, None] * U_t)
                Wf[b, h, c0:c1], Uf[b, h, c0:c1], Ut[b, h, c0:c1], cum[b, h, c0:c1] = W, U, U_t, cc
            final[b, h] = S
    return dict(o=o, final=final, W=Wf, U=Uf, Ut=Ut, cum=cum)


def gated_chunk_factors(q, k, beta, gate, mode="exact"):
    """Per-chunk factors of gated EFLA that the forward keeps for the backward pass (section 3.4
    reading above, in the chunk form of gated_chunk_forward). q, k: [C, dk]; beta, gate: [C].
    With c the running sum of the chunk's log-decays and D_ts = e^{c_t - c_s} (s <= t):
    M = tril(Q K^T) * D, the decayed causal scores of the intra-chunk read-out, and
    X = (I + strictly_lower(diag(alpha) K K^T * D))^{-1}."""
    q, k, beta, gate = _f64(q), _f64(k), _f64(beta), _f64(gate)
    C = k.shape[0]
    co = gated_coefficients(k, beta, gate, mode)
    cc = np.cumsum(gate)
    D = np.exp(np.tril(cc[:, None] - cc[None, :]))
    A = np.tril(co["alpha"][:, None] * D * (k @ k.T), -1)
    X = scipy.linalg.solve_triangular(np.eye(C) + A, np.eye(C), lower=True, unit_diagonal=True)
    return dict(X=X, M=np.tril(q @ k.T) * D)


def gated_chunk_backward(q, k, v, beta, gate, do, scale=1.0, chunk=CHUNK, initial_state=None,
                         d_final_state=None, mode="exact"):
    """Chunkwise gated backward (dense batches): the reverse-mode form of gated_chunk_forward,
    chunk by chunk, for tests of the algebra the kernels would use. Per chunk (c, Gamma = e^c,
    G_C = e^{c_last}, D_ts = e^{c_t - c_s}, r = e^{c_last - c}, P = tril(Q K^T) * D) and the
    gradient G of the outgoing state:
      dU~ = scale P^T dO + diag(r) K G;   G_in = G_C G + scale Q^T diag(Gamma) dO - W^T dU~;
      dP = scale tril(dO U~^T);  dQ = scale diag(Gamma) dO S^T + (dP * D) K;
      dK = (dP * D)^T Q + diag(r) U~ G^T + T_w^T dW + (H + H^T) K + 2 K dlambda;
      W = T_w K, T_w = X diag(alpha Gamma);  U = T_u V, T_u = X diag(b);
      dT_w = -dU~ S^T K^T,  dT_u = dU~ V^T,  dX = dT_w diag(alpha Gamma) + dT_u diag(b),
      dA = -X^T dX X^T (strictly lower),  H = (diag(alpha) dA) * D;
    the log-decay gradient collects every e^{c} factor into dc and sums it backwards over the
    chunk (c_t = sum_{s <= t} a_s). Returns the same dict as gated_backward."""
    q, k, v, beta, gate, do = _f64(q), _f64(k), _f64(v), _f64(beta), _f64(gate), _f64(do)
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    co = gated_coefficients(k, beta, gate, mode)
    de = gated_coefficient_derivatives(k, beta, gate, mode)
    fw = gated_chunk_forward(q, k, v, beta, gate, scale, chunk, initial_state, mode)
    S0 = _f64(initial_state)
    dSF = _f64(d_final_state)
    out = dict(dq=np.zeros_like(q), dk=np.zeros_like(k), dv=np.zeros_like(v), dbeta=np.zeros_like(beta),
               dgate=np.zeros_like(gate), d_initial_state=np.zeros((B, H, dk, dv)))
    for b_ in range(B):
        for h in range(H):
            # incoming states of the chunks, recomputed from the forward's factors
            starts = list(range(0, T, chunk))
            S_in, S = [], (np.zeros((dk, dv)) if S0 is None else S0[b_, h].copy())
            for c0 in starts:
                c1 = min(T, c0 + chunk)
                S_in.append(S)
                cc = fw["cum"][b_, h, c0:c1]
                S = np.exp(cc[-1]) * S + k[b_, h, c0:c1].T @ (np.exp(cc[-1] - cc)[:, None] * fw["Ut"][b_, h, c0:c1])
            G = np.zeros((dk, dv)) if dSF is None else dSF[b_, h].copy()
            for ci in range(len(starts) - 1, -1, -1):
                c0 = starts[ci]
                c1 = min(T, c0 + chunk)
                n = c1 - c0
                K, V, Q, dO = k[b_, h, c0:c1], v[b_, h, c0:c1], q[b_, h, c0:c1], do[b_, h, c0:c1]
                al, bb = co["alpha"][b_, h, c0:c1], co["b"][b_, h, c0:c1]
                Sc = S_in[ci]
                cc = np.cumsum(gate[b_, h, c0:c1])
                Gm = np.exp(cc)
                GC = np.exp(cc[-1])
                D = np.exp(np.tril(cc[:, None] - cc[None, :])) * np.tril(np.ones((n, n)))
                r = np.exp(cc[-1] - cc)
                A = np.tril(al[:, None] * D * (K @ K.T), -1)
                X = np.linalg.inv(np.eye(n) + A)
                Tw = X * (al * Gm)[None, :]
                Tu = X * bb[None, :]
                W = Tw @ K
                Ut = Tu @ V - W @ Sc
                P = np.tril(Q @ K.T) * D
                dUt = scale * P.T @ dO + r[:, None] * (K @ G)
                G_in = GC * G + scale * Q.T @ (Gm[:, None] * dO) - W.T @ dUt
                dP = scale * np.tril(dO @ Ut.T)
                dQs = scale * Gm[:, None] * (dO @ Sc.T)
                dQ = dQs + (dP * D) @ K
                dK = (dP * D).T @ Q + r[:, None] * (Ut @ G.T)
                dc = np.zeros(n)
                dc += np.sum(dQs * Q, axis=1)
                E = dP * P
                dc += E.sum(axis=1)
                dc -= E.sum(axis=0)
                dr = np.sum((K @ G) * Ut, axis=1)
                dc -= r * dr
                dc[-1] += np.sum(r * dr) + GC * np.sum(G * Sc)
                dW = -dUt @ Sc.T
                dTw = dW @ K.T
                dK += Tw.T @ dW
                dTu = dUt @ V.T
                dV = Tu.T @ dUt
                daG = np.sum(dTw * X, axis=0)           # d(alpha Gamma)_j
                db = np.sum(dTu * X, axis=0)
                dX = dTw * (al * Gm)[None, :] + dTu * bb[None, :]
                dA = np.tril(-X.T @ dX @ X.T, -1)
                dal = daG * Gm
                dc += daG * al * Gm
                dal += np.sum(dA * (K @ K.T) * D, axis=1)
                Hm = (al[:, None] * dA) * D
                dK += (Hm + Hm.T) @ K
                F = dA * A
                dc += F.sum(axis=1)
                dc -= F.sum(axis=0)
                dg = np.cumsum(dc[::-1])[::-1]           # c_t = sum_{s<=t} a_s
                out["dq"][b_, h, c0:c1] = dQ
                dlam = dal * de["da_dlam"][b_, h, c0:c1] + db * de["db_dlam"][b_, h, c0:c1]
                out["dk"][b_, h, c0:c1] = dK + 2.0 * K * dlam[:, None]
                out["dv"][b_, h, c0:c1] = dV
                out["dbeta"][b_, h, c0:c1] = dal * de["da_dbeta"][b_, h, c0:c1] + db * de["db_dbeta"][b_, h, c0:c1]
                out["dgate"][b_, h, c0:c1] = dg + db * de["db_da"][b_, h, c0:c1]
                G = G_in
            out["d_initial_state"][b_, h] = G
    return out


def rel_err(x, ref):
    """Normwise relative error max|x - ref| / max|ref| (0 when both are all zero)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    num = np.max(np.abs(x - ref)) if ref.size else 0.0
    if den == 0.0:
        return float(num)
    return float(num / den)

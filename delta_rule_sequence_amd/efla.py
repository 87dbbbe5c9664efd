"""PyTorch binding of the EFLA C ABI: argument marshalling only.

Tensors are only allocated here (outputs, workspaces) and handed to libefla.so
as device pointers together with torch's current HIP stream; every step of the
computation runs in the library's kernels.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib

_DT = {torch.float32: _lib.EFLA_F32, torch.bfloat16: _lib.EFLA_BF16}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, name, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be on the GPU" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))


def _mode(mode):
    if mode not in _lib.MODES:
        raise ValueError("mode must be one of %s" % sorted(_lib.MODES))
    return _lib.MODES[mode]


def make_problem(q, k, v, beta, scale=1.0, cu_seqlens=None, mode="exact", segments=0):
    """Build the efla_problem for tensors q, k [B,H,T,dk], v [B,H,T,dv], beta [B,H,T].
    mode "exact" (the exact flow) or "euler" (the delta rule, alpha = beta). segments: forward
    scan split of long sequences (0 = library's choice, 1 = none, n = at most n segments)."""
    if k.dim() != 4 or v.dim() != 4:
        raise ValueError("k and v must be [B, H, T, d]")
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    if k.dtype not in _DT:
        raise ValueError("dtype must be float32 or bfloat16")
    for t, n, shp in ((q, "q", (B, H, T, dk)), (k, "k", None), (v, "v", (B, H, T, dv)),
                      (beta, "beta", (B, H, T))):
        _need(t, n, k.dtype, shp)
    n_seqs, cu_ptr = 0, None
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32)
        n_seqs = cu_seqlens.numel() - 1
        cu_ptr = cu_seqlens.data_ptr()
    if int(segments) < 0:
        raise ValueError("segments must be >= 0")
    return _lib.problem(B, H, T, dk, dv, _DT[k.dtype], float(scale), cu_ptr, n_seqs,
                        mode=_mode(mode), segments=int(segments))


def efla_workspace_bytes(p, for_backward: bool) -> int:
    return int(_lib.lib().efla_workspace_bytes(ctypes.byref(p), 1 if for_backward else 0))


def efla_saved_bytes(p) -> int:
    return int(_lib.lib().efla_saved_bytes(ctypes.byref(p)))


def efla_get_saved_layout(p) -> dict:
    out = _lib.EflaSavedLayout()
    _lib.check("efla_get_saved_layout", _lib.lib().efla_get_saved_layout(ctypes.byref(p), ctypes.byref(out)))
    return dict(w=out.w, ut=out.ut, states=out.states, table=out.table, m=out.m, x=out.x,
                coef=out.coef, cum=out.cum, segp=out.segp, total=out.total,
                n_chunk_slots=out.n_chunk_slots)


def _bytes(n, device):
    return torch.empty(max(int(n), 1), dtype=torch.uint8, device=device)


def efla_prep(k, beta, mode="exact"):
    """Per-token coefficients: dict(lam, alpha, dalpha_dbeta, dalpha_dlam), fp32 [B,H,T]."""
    if k.dim() != 4 or k.dtype not in _DT:
        raise ValueError("k must be [B, H, T, dk] float32 or bfloat16")
    B, H, T, dk = k.shape
    _need(k, "k", k.dtype)
    _need(beta, "beta", k.dtype, (B, H, T))
    p = _lib.problem(B, H, T, dk, dk, _DT[k.dtype], mode=_mode(mode))
    out = {n: torch.empty((B, H, T), dtype=torch.float32, device=k.device)
           for n in ("lam", "alpha", "dalpha_dbeta", "dalpha_dlam")}

    def fptr(t):
        return ctypes.cast(ctypes.c_void_p(t.data_ptr()), ctypes.POINTER(ctypes.c_float))
    _lib.check("efla_prep", _lib.lib().efla_prep(ctypes.byref(p), _ptr(k), _ptr(beta), fptr(out["lam"]),
                                                fptr(out["alpha"]), fptr(out["dalpha_dbeta"]),
                                                fptr(out["dalpha_dlam"]), _stream()))
    return out


def efla_chunk_ut(k, v, beta, cu_seqlens=None, mode="exact"):
    """UT transform of every chunk: (W [B,H,T,dk], U [B,H,T,dv]) in the input dtype."""
    p = make_problem(k, k, v, beta, 1.0, cu_seqlens, mode)
    w = torch.empty_like(k)
    u = torch.empty_like(v)
    ws_n = efla_workspace_bytes(p, False)
    ws = _bytes(ws_n, k.device)
    _lib.check("efla_chunk_ut", _lib.lib().efla_chunk_ut(ctypes.byref(p), _ptr(k), _ptr(v), _ptr(beta),
                                                        _ptr(w), _ptr(u), _ptr(ws), ws_n, _stream()))
    return w, u


def _n_state(p):
    return p.n_seqs if p.cu_seqlens else p.B


def _state_tensor(t, name, p, device):
    shape = (_n_state(p), p.H, p.dk, p.dv)
    if t is None:
        return None
    _need(t, name, torch.float32, shape)
    return t


def efla_fwd(q, k, v, beta, scale=1.0, cu_seqlens=None, save=True, ws=None, o=None, saved=None,
             mode="exact", initial_state=None, final_state=None, segments=0):
    """Forward. Returns (o, saved) where saved is the uint8 buffer for efla_bwd (or None).
    o, saved and ws may be passed in preallocated. initial_state: fp32 [n_state, H, dk, dv] or
    None (zero). final_state: True (allocate) or a preallocated fp32 tensor of that shape to
    receive the state after each sequence; then (o, saved, final_state) is returned.
    segments: see make_problem."""
    p = make_problem(q, k, v, beta, scale, cu_seqlens, mode, segments)
    if o is None:
        o = torch.empty_like(v)
    else:
        _need(o, "o", v.dtype, v.shape)
    if save and saved is None:
        saved = _bytes(efla_saved_bytes(p), k.device)
    if not save:
        saved = None
    h0 = _state_tensor(initial_state, "initial_state", p, k.device)
    ht = None
    if final_state is True:
        ht = torch.empty((_n_state(p), p.H, p.dk, p.dv), dtype=torch.float32, device=k.device)
    elif final_state is not None and final_state is not False:
        ht = _state_tensor(final_state, "final_state", p, k.device)
    ws_n = efla_workspace_bytes(p, False)
    if ws is None or ws.numel() < ws_n:
        ws = _bytes(ws_n, k.device)
    _lib.check("efla_fwd_state", _lib.lib().efla_fwd_state(
        ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(h0), _ptr(o), _ptr(ht),
        _ptr(saved), 0 if saved is None else saved.numel(), _ptr(ws), ws.numel(), _stream()))
    return (o, saved) if ht is None else (o, saved, ht)


def efla_fwd_gated(q, k, v, beta, gate, scale=1.0, cu_seqlens=None, save=False, ws=None, o=None,
                   saved=None, mode="exact", initial_state=None, final_state=None, segments=0):
    """Gated EFLA forward (efla_fwd_gated in include/efla.h): gate is the per-token log-decay
    [B,H,T] in the input dtype (bf16 only). Returns (o, saved) where saved is the buffer for
    efla_bwd_gated (None unless save), plus final_state as in efla_fwd."""
    p = make_problem(q, k, v, beta, scale, cu_seqlens, mode, segments)
    _need(gate, "gate", k.dtype, tuple(beta.shape))
    if o is None:
        o = torch.empty_like(v)
    else:
        _need(o, "o", v.dtype, v.shape)
    if save and saved is None:
        saved = _bytes(efla_saved_bytes(p), k.device)
    if not save:
        saved = None
    h0 = _state_tensor(initial_state, "initial_state", p, k.device)
    ht = None
    if final_state is True:
        ht = torch.empty((_n_state(p), p.H, p.dk, p.dv), dtype=torch.float32, device=k.device)
    elif final_state is not None and final_state is not False:
        ht = _state_tensor(final_state, "final_state", p, k.device)
    ws_n = efla_workspace_bytes(p, False)
    if ws is None or ws.numel() < ws_n:
        ws = _bytes(ws_n, k.device)
    _lib.check("efla_fwd_gated", _lib.lib().efla_fwd_gated(
        ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(gate), _ptr(h0), _ptr(o),
        _ptr(ht), _ptr(saved), 0 if saved is None else saved.numel(), _ptr(ws), ws.numel(), _stream()))
    return (o, saved) if ht is None else (o, saved, ht)


def efla_bwd(q, k, v, beta, d_o, saved=None, scale=1.0, cu_seqlens=None, ws=None, grads=None,
             mode="exact", initial_state=None, d_final_state=None, d_initial_state=False,
             segments=0):
    """Backward of sum(o * d_o) (+ <final_state, d_final_state>): (dq, dk, dv, dbeta) in the
    input dtype. grads may be a preallocated (dq, dk, dv, dbeta) tuple. initial_state is the
    one the forward used (read only when saved is None). With d_initial_state True (or a
    preallocated fp32 tensor) the gradient at the initial states is returned as a fifth item.
    segments applies to the forward recomputed when saved is None (see make_problem)."""
    p = make_problem(q, k, v, beta, scale, cu_seqlens, mode, segments)
    _need(d_o, "d_o", v.dtype, v.shape)
    if grads is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        dbeta = torch.empty_like(beta)
    else:
        dq, dk, dv, dbeta = grads
        for t, ref, n in ((dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv"), (dbeta, beta, "dbeta")):
            _need(t, n, ref.dtype, ref.shape)
    h0 = _state_tensor(initial_state, "initial_state", p, k.device)
    dht = _state_tensor(d_final_state, "d_final_state", p, k.device)
    dh0 = None
    if d_initial_state is True:
        dh0 = torch.empty((_n_state(p), p.H, p.dk, p.dv), dtype=torch.float32, device=k.device)
    elif d_initial_state is not None and d_initial_state is not False:
        dh0 = _state_tensor(d_initial_state, "d_initial_state", p, k.device)
    ws_n = efla_workspace_bytes(p, True)
    if ws is None or ws.numel() < ws_n:
        ws = _bytes(ws_n, k.device)
    _lib.check("efla_bwd_state", _lib.lib().efla_bwd_state(
        ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(h0), _ptr(d_o), _ptr(dht),
        _ptr(saved), 0 if saved is None else saved.numel(), _ptr(dq), _ptr(dk), _ptr(dv),
        _ptr(dbeta), _ptr(dh0), _ptr(ws), ws.numel(), _stream()))
    return (dq, dk, dv, dbeta) if dh0 is None else (dq, dk, dv, dbeta, dh0)


def efla_bwd_gated(q, k, v, beta, gate, d_o, saved=None, scale=1.0, cu_seqlens=None, ws=None,
                   grads=None, mode="exact", initial_state=None, d_final_state=None,
                   d_initial_state=False, segments=0):
    """Gated EFLA backward (efla_bwd_gated in include/efla.h): (dq, dk, dv, dbeta, dgate) in the
    input dtype, plus the initial-state gradient as in efla_bwd. saved is the buffer
    efla_fwd_gated(save=True) returned, or None to recompute it. grads may be a preallocated
    (dq, dk, dv, dbeta, dgate) tuple."""
    p = make_problem(q, k, v, beta, scale, cu_seqlens, mode, segments)
    _need(gate, "gate", k.dtype, tuple(beta.shape))
    _need(d_o, "d_o", v.dtype, v.shape)
    if grads is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        dbeta, dgate = torch.empty_like(beta), torch.empty_like(gate)
    else:
        dq, dk, dv, dbeta, dgate = grads
        for t, ref, n in ((dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv"), (dbeta, beta, "dbeta"),
                          (dgate, gate, "dgate")):
            _need(t, n, ref.dtype, ref.shape)
    h0 = _state_tensor(initial_state, "initial_state", p, k.device)
    dht = _state_tensor(d_final_state, "d_final_state", p, k.device)
    dh0 = None
    if d_initial_state is True:
        dh0 = torch.empty((_n_state(p), p.H, p.dk, p.dv), dtype=torch.float32, device=k.device)
    elif d_initial_state is not None and d_initial_state is not False:
        dh0 = _state_tensor(d_initial_state, "d_initial_state", p, k.device)
    ws_n = efla_workspace_bytes(p, True)
    if ws is None or ws.numel() < ws_n:
        ws = _bytes(ws_n, k.device)
    _lib.check("efla_bwd_gated", _lib.lib().efla_bwd_gated(
        ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(gate), _ptr(h0), _ptr(d_o),
        _ptr(dht), _ptr(saved), 0 if saved is None else saved.numel(), _ptr(dq), _ptr(dk), _ptr(dv),
        _ptr(dbeta), _ptr(dgate), _ptr(dh0), _ptr(ws), ws.numel(), _stream()))
    out = (dq, dk, dv, dbeta, dgate)
    return out if dh0 is None else out + (dh0,)


def efla_decode(q, k, v, beta, state, scale=1.0, mode="exact", o=None):
    """Recurrent inference over the T tokens of q, k [B,H,T,dk], v [B,H,T,dv], beta [B,H,T]
    (dense batch). state: fp32 [B, H, dk, dv], updated in place. Returns o [B,H,T,dv]."""
    p = make_problem(q, k, v, beta, scale, None, mode)
    _need(state, "state", torch.float32, (p.B, p.H, p.dk, p.dv))
    if o is None:
        o = torch.empty_like(v)
    else:
        _need(o, "o", v.dtype, v.shape)
    _lib.check("efla_decode", _lib.lib().efla_decode(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v),
                                                    _ptr(beta), _ptr(state), _ptr(o), _stream()))
    return o


def efla_decode_gated(q, k, v, beta, gate, state, scale=1.0, mode="exact", o=None):
    """Gated recurrent inference (efla_decode_gated): as efla_decode with the per-token
    log-decay gate [B,H,T] in the input dtype. state is updated in place. Returns o."""
    p = make_problem(q, k, v, beta, scale, None, mode)
    _need(gate, "gate", k.dtype, tuple(beta.shape))
    _need(state, "state", torch.float32, (p.B, p.H, p.dk, p.dv))
    if o is None:
        o = torch.empty_like(v)
    else:
        _need(o, "o", v.dtype, v.shape)
    _lib.check("efla_decode_gated", _lib.lib().efla_decode_gated(
        ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(gate), _ptr(state), _ptr(o),
        _stream()))
    return o


def saved_views(saved, q, k, v, beta, scale=1.0, cu_seqlens=None):
    """Tensor views of a saved buffer: U~ [B,H,T,dv], states [slots,H,dk,dv], M = tril(Q K^T)
    and X = (I + A)^{-1} per chunk [slots,H,64,64], and W [B,H,T,dk] (fp32 problems) or the
    column scales alpha~, b [2,slots,H,64] fp32 (bf16 problems; W = X diag(alpha~) K)."""
    p = make_problem(q, k, v, beta, scale, cu_seqlens)
    L = efla_get_saved_layout(p)
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    es = k.element_size()

    def view(off, shape):
        n = 1
        for s in shape:
            n *= s
        return saved[off:off + n * es].view(k.dtype).view(*shape)
    out = dict(ut=view(L["ut"], (B, H, T, dv)),
               states=view(L["states"], (L["n_chunk_slots"], H, dk, dv)),
               m=view(L["m"], (L["n_chunk_slots"], H, 64, 64)),
               x=view(L["x"], (L["n_chunk_slots"], H, 64, 64)))
    if k.dtype == torch.float32:
        out["w"] = view(L["w"], (B, H, T, dk))
    else:
        n = 2 * L["n_chunk_slots"] * H * 64
        out["coef"] = saved[L["coef"]:L["coef"] + 4 * n].view(torch.float32).view(2, L["n_chunk_slots"], H, 64)
    return out


class EflaFunction(torch.autograd.Function):
    """o = EFLA(q, k, v, beta); the backward runs the library's backward kernels."""

    @staticmethod
    def forward(ctx, q, k, v, beta, scale, cu_seqlens, mode):
        q, k, v, beta = (t.contiguous() for t in (q, k, v, beta))
        o, saved = efla_fwd(q, k, v, beta, scale, cu_seqlens, save=True, mode=mode)
        ctx.save_for_backward(q, k, v, beta, saved, cu_seqlens)
        ctx.scale = scale
        ctx.mode = mode
        return o

    @staticmethod
    def backward(ctx, d_o):
        q, k, v, beta, saved, cu = ctx.saved_tensors
        dq, dk, dv, dbeta = efla_bwd(q, k, v, beta, d_o.contiguous(), saved, ctx.scale, cu,
                                     mode=ctx.mode)
        return dq, dk, dv, dbeta, None, None, None


class EflaGatedFunction(torch.autograd.Function):
    """o = gated EFLA(q, k, v, beta, gate); the backward runs the library's gated kernels."""

    @staticmethod
    def forward(ctx, q, k, v, beta, gate, scale, cu_seqlens, mode):
        q, k, v, beta, gate = (t.contiguous() for t in (q, k, v, beta, gate))
        o, saved = efla_fwd_gated(q, k, v, beta, gate, scale, cu_seqlens, save=True, mode=mode)
        ctx.save_for_backward(q, k, v, beta, gate, saved, cu_seqlens)
        ctx.scale = scale
        ctx.mode = mode
        return o

    @staticmethod
    def backward(ctx, d_o):
        q, k, v, beta, gate, saved, cu = ctx.saved_tensors
        g = efla_bwd_gated(q, k, v, beta, gate, d_o.contiguous(), saved, ctx.scale, cu, mode=ctx.mode)
        return g + (None, None, None)


def efla_gated(q, k, v, beta, gate, scale: float = 1.0, cu_seqlens: Optional[torch.Tensor] = None,
               mode: str = "exact"):
    """Gated EFLA token mixer (per-token log-decays gate [B,H,T], bf16): o [B,H,T,dv],
    differentiable in q, k, v, beta and gate."""
    return EflaGatedFunction.apply(q, k, v, beta, gate, scale, cu_seqlens, mode)


def efla(q, k, v, beta, scale: float = 1.0, cu_seqlens: Optional[torch.Tensor] = None,
         mode: str = "exact"):
    """Exact Flow Linear Attention token mixer: o [B,H,T,dv], differentiable.
    mode "euler" runs the delta rule (alpha = beta) through the same kernels."""
    return EflaFunction.apply(q, k, v, beta, scale, cu_seqlens, mode)


def profile_enable(on: bool):
    _lib.check("efla_profile_enable", _lib.lib().efla_profile_enable(1 if on else 0))


def profile_reset():
    _lib.lib().efla_profile_reset()


def profile_read(max_kernels: int = 32) -> dict:
    """{kernel name: (launches, total ms)} since the last reset."""
    stride = 64
    names = ctypes.create_string_buffer(stride * max_kernels)
    counts = (ctypes.c_int64 * max_kernels)()
    ms = (ctypes.c_double * max_kernels)()
    n = _lib.lib().efla_profile_read(names, stride, counts, ms, max_kernels)
    out = {}
    for i in range(n):
        nm = names.raw[i * stride:(i + 1) * stride].split(b"\0", 1)[0].decode()
        out[nm] = (int(counts[i]), float(ms[i]))
    return out

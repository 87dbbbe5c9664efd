"""Seeded synthetic inputs for the EFLA token mixer.

This module only draws random numbers and shapes them into the five workloads
below. It holds none of the method's arithmetic, so the CPU oracle and the
HIP path can both be fed from it without sharing any part of the computation.

The pages train language models on a SlimPajama subset and evaluate on MAD and
on corrupted-image robustness tasks (Exact Flow Linear Attention summary page,
sections 4.1, 4.3, 4.5). No dataset is used here: synthetic tensors with the
1.3B layer shape (16 heads of width 128, section 4.1) stand in for them, and
the seed family starts at 42, the seed the pages report (Appendix C).

Every array is returned as float32. For bf16 workloads each value is rounded
to the nearest bf16 (ties to even) before it is returned, so the value handed
to the GPU and the value handed to the oracle are the same number.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

BASE_SEED = 42


@dataclass(frozen=True)
class Workload:
    """Shape, dtype and value recipe of one synthetic EFLA workload."""

    name: str
    B: int
    H: int
    T: int
    dk: int
    dv: int
    dtype: str               # "f32" or "bf16": dtype of q, k, v, beta, o and all gradients
    backward: bool           # whether the workload times/checks fwd+bwd or fwd only
    keys: str                # "unif_0.5_2", "unif_0.5_4" or "loguniform_1e-3_100"
    queries: str             # "normal" or "l2norm"
    betas: str               # "sigmoid_normal" or "uniform_0_1"
    value_outliers: float = 0.0   # fraction of tokens whose v is multiplied by 50
    n_seqs: int = 0          # >0: packed variable-length batch (B must be 1)
    seq_len_range: tuple = (0, 0)
    seed_index: int = 0
    chunk: int = 64

    def tokens(self) -> int:
        return self.B * self.T


# The five workloads: a tiny fp32 forward case, the 1.3B-layer fwd+bwd case
# (the throughput workload), a long single sequence, stiff keys in fp32 and a
# packed variable-length batch.
WORKLOADS = {
    1: Workload("tiny_f32_fwd", B=1, H=2, T=256, dk=64, dv=64, dtype="f32", backward=False,
                keys="unif_0.5_2", queries="normal", betas="sigmoid_normal", seed_index=1),
    2: Workload("layer1p3b_bf16_fwdbwd", B=4, H=16, T=2048, dk=128, dv=128, dtype="bf16",
                backward=True, keys="unif_0.5_4", queries="l2norm", betas="sigmoid_normal",
                seed_index=2),
    3: Workload("longctx_bf16_fwd", B=1, H=16, T=32768, dk=128, dv=128, dtype="bf16",
                backward=False, keys="unif_0.5_4", queries="l2norm", betas="sigmoid_normal",
                seed_index=3),
    4: Workload("stiff_f32_fwdbwd", B=8, H=8, T=4096, dk=64, dv=64, dtype="f32", backward=True,
                keys="loguniform_1e-3_100", queries="l2norm", betas="uniform_0_1",
                value_outliers=0.05, seed_index=4),
    5: Workload("varlen_bf16_fwdbwd", B=1, H=16, T=0, dk=128, dv=128, dtype="bf16",
                backward=True, keys="unif_0.5_4", queries="l2norm", betas="sigmoid_normal",
                n_seqs=32, seq_len_range=(128, 8192), seed_index=5),
}


def workload(idx: int, **overrides) -> Workload:
    """Return workload `idx`, optionally with some fields replaced (smaller sizes for tests)."""
    w = WORKLOADS[idx]
    return replace(w, **overrides) if overrides else w


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 value (ties to even), returned as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32).copy()
    nan = np.isnan(x)
    out[nan] = np.nan
    return out


def _l2norm_rows(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True))
    return (x / np.maximum(n, 1e-30)).astype(np.float32)


def seq_lengths(w: Workload, rng: Optional[np.random.Generator] = None) -> np.ndarray:
    """Sequence lengths of a packed batch, drawn uniformly from w.seq_len_range (inclusive)."""
    if rng is None:
        rng = np.random.default_rng(BASE_SEED + w.seed_index)
    lo, hi = w.seq_len_range
    return rng.integers(lo, hi + 1, size=w.n_seqs).astype(np.int64)


def make_inputs(w: Workload, seed: Optional[int] = None, with_grad: Optional[bool] = None,
                lengths=None) -> dict:
    """Draw q, k, v, beta (and grad_out when the workload has a backward) for workload `w`.

    Returns float32 numpy arrays q, k [B,H,T,dk]; v, do [B,H,T,dv]; beta [B,H,T];
    and cu_seqlens (int32 [n_seqs+1]) or None. For a packed batch B is 1 and T is
    the total length; `lengths` replaces the drawn sequence lengths.
    """
    rng = np.random.default_rng(BASE_SEED + w.seed_index if seed is None else seed)
    cu = None
    B, T = w.B, w.T
    if w.n_seqs > 0 or lengths is not None:
        lens = seq_lengths(w, rng) if lengths is None else np.asarray(lengths, dtype=np.int64)
        cu = np.zeros(len(lens) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lens)
        B, T = 1, int(cu[-1])
    H, dk, dv = w.H, w.dk, w.dv

    q = rng.standard_normal((B, H, T, dk), dtype=np.float32)
    if w.queries == "l2norm":
        q = _l2norm_rows(q)

    kdir = _l2norm_rows(rng.standard_normal((B, H, T, dk), dtype=np.float32))
    if w.keys == "unif_0.5_2":
        knorm = rng.uniform(0.5, 2.0, size=(B, H, T, 1))
    elif w.keys == "unif_0.5_4":
        knorm = rng.uniform(0.5, 4.0, size=(B, H, T, 1))
    elif w.keys == "loguniform_1e-3_100":
        knorm = np.exp(rng.uniform(np.log(1e-3), np.log(100.0), size=(B, H, T, 1)))
    else:
        raise ValueError(w.keys)
    k = (kdir * knorm.astype(np.float32)).astype(np.float32)

    v = rng.standard_normal((B, H, T, dv), dtype=np.float32)
    if w.value_outliers > 0:
        hit = rng.random((B, H, T)) < w.value_outliers
        v[hit] *= np.float32(50.0)

    if w.betas == "sigmoid_normal":
        z = rng.standard_normal((B, H, T), dtype=np.float32)
        beta = (1.0 / (1.0 + np.exp(-z.astype(np.float64)))).astype(np.float32)
    elif w.betas == "uniform_0_1":
        beta = rng.uniform(0.0, 1.0, size=(B, H, T)).astype(np.float32)
    else:
        raise ValueError(w.betas)

    out = dict(q=q, k=k, v=v, beta=beta, cu_seqlens=cu)
    if w.backward if with_grad is None else with_grad:
        out["do"] = rng.standard_normal((B, H, T, dv), dtype=np.float32)
    if w.dtype == "bf16":
        for name in ("q", "k", "v", "beta", "do"):
            if name in out:
                out[name] = round_to_bf16(out[name])
    return out

"""Property tests: the HIP path against the fp64 oracle on small random problems drawn by
hypothesis (derandomized, so every run checks the same examples).

Drawn per example: dtype (fp32 with d = 64, or bf16 with any head-size pair), step rule (exact
flow, or the delta rule with unit-norm keys), batch size and heads, either a dense batch with a
length that is usually not a multiple of the chunk (1 to 300 tokens) or a packed batch of up to
five sequences of 0 to 200 tokens (empty and one-token sequences included), a share of key rows
set to zero, and the read-out scale. Forward output and every gradient are compared normwise per
tensor (at five times the tolerance when the whole tensor holds fewer than 64 token-heads), and
per (batch row, head) where the row holds at least one chunk of tokens: below a chunk the
normwise figure degenerates to an elementwise one, ill-conditioned where a dot product cancels.
"""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from oracle import efla_oracle as O
from workloads import make_inputs, round_to_bf16, workload

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


@st.composite
def problems(draw):
    dtype = draw(st.sampled_from(["f32", "bf16"]))
    dk, dv = (64, 64) if dtype == "f32" else (draw(st.sampled_from([64, 128])), draw(st.sampled_from([64, 128])))
    packed = draw(st.booleans())
    H = draw(st.integers(1, 3))
    if packed:
        lengths = draw(st.lists(st.integers(0, 200), min_size=1, max_size=5))
        if sum(lengths) == 0:
            lengths[0] = 1
        B, T = 1, sum(lengths)
    else:
        lengths, B, T = None, draw(st.integers(1, 3)), draw(st.integers(1, 300))
    return dict(dtype=dtype, dk=dk, dv=dv, B=B, H=H, T=T, lengths=lengths,
                mode=draw(st.sampled_from(["exact", "euler"])),
                zero_frac=draw(st.sampled_from([0.0, 0.1, 0.5])),
                scale=draw(st.floats(0.5, 1.5)), seed=draw(st.integers(0, 2 ** 31 - 1)))


@settings(max_examples=30, deadline=None, derandomize=True, database=None,
          suppress_health_check=[HealthCheck.too_slow, HealthCheck.function_scoped_fixture])
@given(prob=problems())
def test_random_problems_match_oracle(E, prob):
    idx = 2 if prob["dtype"] == "bf16" else 4
    w = workload(idx, B=prob["B"], H=prob["H"], T=prob["T"], dk=prob["dk"], dv=prob["dv"],
                 value_outliers=0.0)
    inp = make_inputs(w, seed=prob["seed"], with_grad=True, lengths=prob["lengths"])
    k = inp["k"]
    if prob["mode"] == "euler":  # the delta rule needs beta ||k||^2 <= 2 (reading R13)
        k = k / np.maximum(np.linalg.norm(k, axis=-1, keepdims=True), 1e-30)
    rng = np.random.default_rng(prob["seed"] + 1)
    k = np.where(rng.random(k.shape[:3])[..., None] < prob["zero_frac"], 0.0, k).astype(np.float32)
    inp["k"] = round_to_bf16(k) if prob["dtype"] == "bf16" else k
    print("problem:", {n: prob[n] for n in prob if n != "seed"}, flush=True)
    dt, tol = TDT[prob["dtype"]], TOL[prob["dtype"]]
    q, kk, v, beta, do = (_dev(inp[n], dt) for n in ("q", "k", "v", "beta", "do"))
    cu_np = inp["cu_seqlens"]
    cu = None if cu_np is None else torch.from_numpy(cu_np).cuda()
    o, saved = E.efla_fwd(q, kk, v, beta, prob["scale"], cu, save=True, mode=prob["mode"])
    grads = E.efla_bwd(q, kk, v, beta, do, saved, prob["scale"], cu, mode=prob["mode"])
    torch.cuda.synchronize()
    ref = {"o": O.forward(inp["q"], inp["k"], inp["v"], inp["beta"], scale=prob["scale"],
                          cu_seqlens=cu_np, mode=prob["mode"])[0]}
    ref.update(O.backward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["do"], scale=prob["scale"],
                          cu_seqlens=cu_np, mode=prob["mode"]))
    got = {"o": o}
    got.update(zip(("dq", "dk", "dv", "dbeta"), grads))
    # Reading R9: the normwise figure needs at least one chunk of token-heads behind it. A
    # smaller tensor (a single token of a single head at the extreme) makes it the elementwise
    # relative error, which a nearly cancelling dot product (dO . v in dbeta) inflates with the
    # bf16 factors; those are held at five times the tolerance, as the stiff workload's dbeta.
    tol_t = tol if prob["B"] * prob["H"] * prob["T"] >= 64 else 5 * tol
    for nm, t in got.items():
        g = t.float().cpu().numpy()
        assert np.all(np.isfinite(g)), nm
        err = O.rel_err(g, ref[nm])
        assert err <= tol_t, "%s: %.3e > %.0e" % (nm, err, tol_t)
        if prob["T"] >= 64:
            for b in range(prob["B"]):
                for h in range(prob["H"]):
                    e = O.rel_err(g[b, h], ref[nm][b, h])
                    assert e <= tol, "%s[b=%d,h=%d]: %.3e > %.0e" % (nm, b, h, e, tol)

"""The byte and flop accounting behind bench.py's roofline fields, checked on the CPU.

The method's bytes per token-head are counted here tensor by tensor (what the forward and the
backward must read and write at the boundary). The kernels' interface bytes per (64-token
chunk, head) unit are counted from the tiles each kernel reads and writes in the bf16 factor
form at d_k = d_v = 128. Both are compared with bench.method_model / bench.kernel_model. The
step totals are the figures the bench line reports for B=4 H=16 T=2048.
"""
import bench

C = 64


def _method_bytes(dk, dv, e):
    fwd_in = {"q": dk, "k": dk, "v": dv, "beta": 1}
    fwd_out = {"o": dv}
    bwd_in = {"q": dk, "k": dk, "v": dv, "beta": 1, "dO": dv}
    bwd_out = {"dq": dk, "dk": dk, "dv": dv, "dbeta": 1}
    fwd = e * (sum(fwd_in.values()) + sum(fwd_out.values()))
    bwd = e * (sum(bwd_in.values()) + sum(bwd_out.values()))
    return fwd, bwd


def test_method_bytes_per_token_head():
    for dk, dv, e in ((128, 128, 2), (64, 64, 4), (64, 128, 2)):
        m = bench.method_model(dk, dv, e)
        assert (m["fwd_bytes"], m["bwd_bytes"]) == _method_bytes(dk, dv, e)
    m = bench.method_model(128, 128, 2)
    assert (m["fwd_bytes"], m["bwd_bytes"]) == (1026, 1796)


def test_step_method_totals_of_the_benchmark_workload():
    token_heads = 4 * 16 * 2048
    m = bench.method_model(128, 128, 2)
    assert (m["fwd_bytes"] + m["bwd_bytes"]) * token_heads == 369_885_184
    # dense-tile flops of the chunkwise form, about 82.5 GFLOP per step
    assert abs((m["fwd_flops"] + m["bwd_flops"]) * token_heads - 82.499e9) < 1e6


def _tile(rows, cols, e=2):
    return rows * cols * e


def test_interface_bytes_per_unit_bf16_d128():
    dk = dv = 128
    vec = 4 * C  # one fp32 per token
    tiles = {
        # K, beta in; X (64x64), alpha~ out
        "ut_fwd": _tile(C, dk) + _tile(C, 1) + _tile(C, C) + vec,
        # K, Q, V, X, alpha~ in; O, U~, the chunk state, M out
        "scan_fwd": 2 * _tile(C, dk) + _tile(C, dv) + _tile(C, C) + vec
        + 2 * _tile(C, dv) + _tile(dk, dv) + _tile(C, C),
        # K, Q, X, M, dO, alpha~ in; dU~ and the state gradient out
        "scan_bwd": 2 * _tile(C, dk) + 2 * _tile(C, C) + _tile(C, dv) + vec
        + _tile(C, dv) + _tile(dk, dv),
        # Q, K, V, dO, U~, dU~, beta, state, state gradient, X in; dQ, dK, dV, dbeta out
        "chunk_bwd": 2 * _tile(C, dk) + 4 * _tile(C, dv) + _tile(C, 1) + 2 * _tile(dk, dv)
        + _tile(C, C) + 2 * _tile(C, dk) + _tile(C, dv) + _tile(C, 1),
    }
    for name, b in tiles.items():
        assert bench.kernel_model(name, dk, dv, 2)[0] == b, name
    units = 4 * 16 * 2048 // C
    total = sum(tiles.values()) * units
    assert abs(total / 1e6 - 1009.0) < 0.1  # the step's interface bytes, MB
    assert abs(tiles["chunk_bwd"] * units / 1e6 - 453.5) < 0.1

"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every
symbol include/efla.h declares, and rejects bad arguments before touching HIP."""
import ctypes
import os
import re

import pytest

from delta_rule_sequence_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "efla.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(efla_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def test_header_and_binding_agree():
    assert _declared_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol(L):
    for name in _declared_functions():
        assert hasattr(L, name), name


def test_abi_version(L):
    assert L.efla_abi_version() == 10


def test_status_strings(L):
    for code in range(8):
        assert L.efla_status_str(code)
    assert L.efla_status_str(5) == b"workspace or saved buffer too small"


def _p(**kw):
    base = dict(B=4, H=16, T=2048, dk=128, dv=128, dtype=_lib.EFLA_BF16)
    base.update(kw)
    return _lib.problem(base["B"], base["H"], base["T"], base["dk"], base["dv"], base["dtype"],
                        base.get("scale", 1.0), base.get("cu", None), base.get("n_seqs", 0),
                        base.get("chunk", 64), base.get("mode", 0), base.get("segments", 0))


@pytest.mark.parametrize("kw,code", [
    (dict(), 0),
    (dict(dtype=_lib.EFLA_F32, dk=64, dv=64), 0),
    (dict(dk=64, dv=128), 0),
    (dict(dk=128, dv=64), 0),
    (dict(T=0), 0),
    (dict(T=1), 0),
    (dict(B=0), 2),
    (dict(H=0), 2),
    (dict(T=-1), 2),
    (dict(dtype=7), 3),
    (dict(chunk=32), 4),
    (dict(dk=96), 4),
    (dict(dv=256), 4),
    (dict(dtype=_lib.EFLA_F32), 4),          # fp32 with d = 128 is not built
    (dict(B=2, cu=0x1000, n_seqs=3), 2),     # packed batches need B == 1
    (dict(B=1, cu=0x1000, n_seqs=0), 2),
    (dict(B=4, n_seqs=3), 2),
    (dict(mode=1), 0),
    (dict(mode=2), 4),
    (dict(mode=-1), 4),
    (dict(segments=1), 0),
    (dict(segments=64), 0),
    (dict(segments=-1), 2),
    (dict(B=1, cu=0x1000, n_seqs=3, segments=4), 0),   # packed: accepted, scan not split
    # index limits: B*H*T*max(dk, dv) below 2^40, state slots * H below 2^31
    (dict(B=64, H=64, T=2**21 - 1), 0),
    (dict(B=64, H=64, T=2**21), 4),
    (dict(B=64, H=64, T=2**21, dk=64, dv=64), 0),
    (dict(B=64, H=64, T=2**21, dk=64, dv=128), 4),
    (dict(B=1, H=4, T=1024, cu=0x1000, n_seqs=2**29 - 17), 0),
    (dict(B=1, H=4, T=1024, cu=0x1000, n_seqs=2**29 - 16), 4),
])
def test_problem_validation(L, kw, code):
    p = _p(**kw)
    assert L.efla_check_problem(ctypes.byref(p)) == code


def test_null_problem(L):
    assert L.efla_check_problem(None) == 1
    assert L.efla_workspace_bytes(None, 0) == 0
    assert L.efla_saved_bytes(None) == 0


def test_workspace_and_saved_sizes(L):
    # bf16: the scans read X and the per-token column scales (fp32 [2][slots][H][64]) in place of
    # W and U, so neither is saved nor kept in the workspace; the forward scan forms M itself (and
    # writes it only into a saved buffer, for the backward), so the workspace holds no M either
    p = _p()
    e = 2
    tok = 4 * 16 * 2048
    slots = 4 * 32
    v = tok * 128 * e           # a [B,H,T,128] tensor (U~, dU~)
    states = slots * 16 * 128 * 128 * e
    m = slots * 16 * 64 * 64 * e  # M or X
    cum = slots * 16 * 64 * 4   # running log-decay sums of the gated forward
    coef = 2 * cum
    saved = v + states + 2 * m + coef + cum
    assert L.efla_saved_bytes(ctypes.byref(p)) == saved
    assert L.efla_workspace_bytes(ctypes.byref(p), 0) == m + coef + cum
    assert L.efla_workspace_bytes(ctypes.byref(p), 1) == (v + states) + saved
    lay = _lib.EflaSavedLayout()
    assert L.efla_get_saved_layout(ctypes.byref(p), ctypes.byref(lay)) == 0
    assert (lay.w, lay.ut, lay.states, lay.m, lay.x, lay.coef, lay.cum, lay.n_chunk_slots) == \
        (0, 0, v, v + states, v + states + m, v + states + 2 * m, v + states + 2 * m + coef, slots)
    # fp32: W saved, U and W in the forward workspace, U again for the recompute path
    p32 = _p(dtype=_lib.EFLA_F32, dk=64, dv=64)
    e = 4
    w = tok * 64 * e
    states = slots * 16 * 64 * 64 * e
    m = slots * 16 * 64 * 64 * e
    saved = 2 * w + states + 2 * m + cum
    assert L.efla_saved_bytes(ctypes.byref(p32)) == saved
    assert L.efla_workspace_bytes(ctypes.byref(p32), 0) == 2 * w + m + cum
    assert L.efla_workspace_bytes(ctypes.byref(p32), 1) == (w + states) + saved + w
    assert L.efla_get_saved_layout(ctypes.byref(p32), ctypes.byref(lay)) == 0
    assert (lay.w, lay.ut, lay.states, lay.m, lay.x, lay.coef, lay.cum) == \
        (0, w, 2 * w, 2 * w + states, 2 * w + states + m, 2 * w + states + 2 * m, 2 * w + states + 2 * m)
    # packed batch: chunk slots are bounded by T/64 + n_seqs
    pp = _p(B=1, T=1000, cu=0x1000, n_seqs=7)
    assert L.efla_get_saved_layout(ctypes.byref(pp), ctypes.byref(lay)) == 0
    assert lay.n_chunk_slots == 1000 // 64 + 7


def test_entry_points_reject_bad_arguments_without_launching(L):
    p = _p()
    vp = ctypes.c_void_p
    fake = vp(0x10000)        # never dereferenced: validation fails first
    odd = vp(0x10008)
    ws_need = L.efla_workspace_bytes(ctypes.byref(p), 0)
    # missing pointers
    assert L.efla_fwd(ctypes.byref(p), None, fake, fake, fake, fake, None, 0, fake, ws_need, None) == 1
    assert L.efla_bwd(ctypes.byref(p), fake, fake, fake, fake, fake, None, 0, fake, fake, fake, None,
                      fake, 1 << 40, None) == 1
    assert L.efla_prep(ctypes.byref(p), fake, fake, None, None, None, None, None) == 1
    # misaligned pointer
    assert L.efla_fwd(ctypes.byref(p), odd, fake, fake, fake, fake, None, 0, fake, ws_need, None) == 7
    # workspace too small
    assert L.efla_fwd(ctypes.byref(p), fake, fake, fake, fake, fake, None, 0, fake, ws_need - 1, None) == 5
    sb = L.efla_saved_bytes(ctypes.byref(p))
    assert L.efla_fwd(ctypes.byref(p), fake, fake, fake, fake, fake, fake, sb - 1, fake, ws_need, None) == 5
    assert L.efla_bwd(ctypes.byref(p), fake, fake, fake, fake, fake, None, 0, fake, fake, fake, fake,
                      fake, 16, None) == 5
    assert L.efla_chunk_ut(ctypes.byref(p), fake, fake, fake, fake, fake, fake, 0, None) == 5
    # invalid problem wins over everything else
    bad = _p(dk=96)
    assert L.efla_fwd(ctypes.byref(bad), fake, fake, fake, fake, fake, None, 0, fake, 1 << 40, None) == 4
    # state I/O entry points: the same checks, plus the alignment of the state pointers
    assert L.efla_fwd_state(ctypes.byref(p), fake, fake, fake, fake, odd, fake, None, None, 0, fake,
                            ws_need, None) == 7
    assert L.efla_fwd_state(ctypes.byref(p), fake, fake, fake, fake, None, fake, odd, None, 0, fake,
                            ws_need, None) == 7
    assert L.efla_bwd_state(ctypes.byref(p), fake, fake, fake, fake, None, fake, None, None, 0, fake,
                            fake, fake, fake, odd, fake, 1 << 40, None) == 7
    assert L.efla_bwd_state(ctypes.byref(p), fake, fake, fake, fake, None, None, None, None, 0, fake,
                            fake, fake, fake, None, fake, 1 << 40, None) == 1
    # decode: dense batches only; every pointer required
    assert L.efla_decode(ctypes.byref(p), fake, fake, fake, fake, None, fake, None) == 1
    assert L.efla_decode(ctypes.byref(p), fake, fake, fake, fake, odd, fake, None) == 7
    packed = _p(B=1, T=100, cu=0x1000, n_seqs=2)
    assert L.efla_decode(ctypes.byref(packed), fake, fake, fake, fake, fake, fake, None) == 4
    assert L.efla_decode(ctypes.byref(bad), fake, fake, fake, fake, fake, fake, None) == 4
    # an empty problem is a successful no-op that touches nothing
    empty = _p(T=0)
    assert L.efla_fwd(ctypes.byref(empty), None, None, None, None, None, None, 0, None, 0, None) == 0
    assert L.efla_bwd(ctypes.byref(empty), None, None, None, None, None, None, 0, None, None, None,
                      None, None, 0, None) == 0


def test_profile_api_without_launches(L):
    assert L.efla_profile_enable(1) == 0
    assert L.efla_profile_enable(0) == 0
    L.efla_profile_reset()
    names = ctypes.create_string_buffer(64 * 4)
    counts = (ctypes.c_int64 * 4)()
    ms = (ctypes.c_double * 4)()
    assert L.efla_profile_read(names, 64, counts, ms, 4) == 0


def test_segment_plan_workspace(L):
    """The segment-parallel forward needs R and S_in (fp32 [B*G][H][dk][dv]) and P (fp32
    [B*G][H][dk][dk]) on top of the sequential-scan workspace; G follows the plan."""
    def extra(**kw):
        return (L.efla_workspace_bytes(ctypes.byref(_p(**kw)), 0) -
                L.efla_workspace_bytes(ctypes.byref(_p(**dict(kw, segments=1))), 0))
    per_seg = 16 * 128 * (2 * 128 + 128) * 4       # H * dk * (2 dv + dk) * 4 bytes
    # long context, 16 heads: 512 chunks -> the library picks 4 segments (256 scan workgroups)
    assert extra(B=1, T=32768) == 4 * per_seg
    # 8 heads: 8 segments; 2 heads, 32 chunks: capped at 16 chunks per segment -> 2
    assert extra(B=1, H=8, T=32768) == 8 * per_seg // 2
    assert extra(B=1, H=2, T=64 * 32) == 2 * per_seg // 8
    # a full chip of whole-sequence scans already: no split
    assert extra() == 0
    # explicit requests: at most one segment per chunk, no empty segment
    assert extra(B=1, T=32768, segments=3) == 3 * per_seg
    assert extra(B=1, T=64 * 10, segments=4) == 4 * per_seg      # 10 chunks -> 3,3,3,1
    assert extra(B=1, T=64 * 10, segments=7) == 5 * per_seg      # 10 chunks -> 2 each
    assert extra(B=1, T=64 * 3, segments=50) == 3 * per_seg
    assert extra(B=1, T=64, segments=8) == 0                     # one chunk: nothing to split
    assert extra(B=2, T=64 * 40, segments=4) == 2 * 4 * per_seg
    # a saved buffer keeps each segment's transition, fp32 [B * G][H][dk][dk], for the backward
    lay = _lib.EflaSavedLayout()
    assert L.efla_get_saved_layout(ctypes.byref(_p(B=1, T=32768)), ctypes.byref(lay)) == 0
    assert lay.total - lay.segp == 4 * 16 * 128 * 128 * 4
    assert L.efla_get_saved_layout(ctypes.byref(_p(B=1, T=32768, segments=1)), ctypes.byref(lay)) == 0
    assert lay.total == lay.segp
    # the backward's recompute path runs the same forward
    p, p1 = _p(B=1, T=32768), _p(B=1, T=32768, segments=1)
    assert (L.efla_workspace_bytes(ctypes.byref(p), 1) -
            L.efla_workspace_bytes(ctypes.byref(p1), 1)) == 4 * per_seg


def test_gated_entry_points_reject_bad_arguments(L):
    """Gated forward, backward and decode: bf16 only, gate required, same validation as the others."""
    fake = ctypes.c_void_p(0x100000)
    p = _p(B=1, H=2, T=128)
    ws = L.efla_workspace_bytes(ctypes.byref(p), 0)
    # fp32 problems: not provided
    pf = _p(B=1, H=2, T=128, dtype=_lib.EFLA_F32, dk=64, dv=64)
    assert L.efla_fwd_gated(ctypes.byref(pf), fake, fake, fake, fake, fake, None, fake, None, None, 0, fake, 1 << 40, None) == 4
    # missing gate / missing workspace / short workspace
    assert L.efla_fwd_gated(ctypes.byref(p), fake, fake, fake, fake, None, None, fake, None, None, 0, fake, ws, None) == 1
    assert L.efla_fwd_gated(ctypes.byref(p), fake, fake, fake, fake, fake, None, fake, None, None, 0, None, ws, None) == 1
    assert L.efla_fwd_gated(ctypes.byref(p), fake, fake, fake, fake, fake, None, fake, None, None, 0, fake, ws - 1, None) == 5
    assert L.efla_decode_gated(ctypes.byref(p), fake, fake, fake, fake, None, fake, fake, None) == 1
    packed = _p(B=1, T=128, cu=0x1000, n_seqs=2)
    assert L.efla_decode_gated(ctypes.byref(packed), fake, fake, fake, fake, fake, fake, fake, None) == 4
    # gated backward: q k v beta gate h0 d_o dht saved saved_bytes dq dk dv dbeta dgate dh0 ws ws_bytes
    wb = L.efla_workspace_bytes(ctypes.byref(p), 1)
    sb = L.efla_saved_bytes(ctypes.byref(p))

    def bwd(prob, gate=fake, saved=None, saved_bytes=0, dgate=fake, ws_=fake, ws_bytes=wb):
        return L.efla_bwd_gated(ctypes.byref(prob), fake, fake, fake, fake, gate, None, fake, None,
                                saved, saved_bytes, fake, fake, fake, fake, dgate, None, ws_,
                                ws_bytes, None)
    assert bwd(pf, ws_bytes=1 << 40) == 4
    assert bwd(p, gate=None) == 1
    assert bwd(p, dgate=None) == 1
    assert bwd(p, ws_=None) == 1
    assert bwd(p, ws_bytes=wb - 1) == 5
    assert bwd(p, saved=fake, saved_bytes=sb - 1) == 5


def test_noalloc_entry_point_rejects_without_touching_hip(L):
    """efla_fwd_noalloc validates everything, including the size of its static workspace,
    before it looks up the workspace or enqueues anything."""
    fake, odd = ctypes.c_void_p(0x10000), ctypes.c_void_p(0x10008)
    cap = _lib.NOALLOC_WS_BYTES

    def call(prob, q=fake, h0=None, o=fake, ht=None):
        return L.efla_fwd_noalloc(ctypes.byref(prob), q, fake, fake, fake, h0, o, ht, None)
    big = _p(B=1, H=16, T=32768)
    assert L.efla_workspace_bytes(ctypes.byref(big), 0) > cap
    assert call(big) == 5
    fits = _p(B=1, H=16, T=16384)     # the header's example: 16 heads of 16,384 bf16 tokens
    assert L.efla_workspace_bytes(ctypes.byref(fits), 0) <= cap
    assert call(fits, q=None) == 1
    assert call(fits, o=None) == 1
    assert call(fits, q=odd) == 7
    assert call(fits, h0=odd) == 7
    assert call(fits, ht=odd) == 7
    assert call(_p(B=1, H=16, T=8192, dk=96)) == 4
    assert L.efla_fwd_noalloc(ctypes.byref(_p(T=0)), None, None, None, None, None, None, None, None) == 0

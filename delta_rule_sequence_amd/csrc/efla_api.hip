// C ABI of the EFLA library: argument validation, workspace layout, launch sequencing.
// See include/efla.h for the contract of every entry point.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "efla.h"
#include "efla_internal.hpp"

namespace efla {

// ---------------------------------------------------------------------------
// Profiling: events bracket each launch while enabled.
// ---------------------------------------------------------------------------
namespace {
struct ProfRec {
  std::string name;
  hipEvent_t a, b;
};
bool g_prof_on = false;
std::vector<hipEvent_t> g_prof_free;
std::vector<ProfRec> g_prof_pending;
hipEvent_t g_prof_open = nullptr;
std::map<std::string, std::pair<int64_t, double>> g_prof_totals;

hipEvent_t prof_event() {
  if (!g_prof_free.empty()) {
    hipEvent_t e = g_prof_free.back();
    g_prof_free.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void prof_drain() {
  for (auto& r : g_prof_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) == hipSuccess && hipEventElapsedTime(&ms, r.a, r.b) == hipSuccess) {
      auto& t = g_prof_totals[r.name];
      t.first += 1;
      t.second += ms;
    }
    g_prof_free.push_back(r.a);
    g_prof_free.push_back(r.b);
  }
  g_prof_pending.clear();
}
}  // namespace

int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

int scan_tile(const Shape& s) {
  if (s.dv != 128) return 16;
  static int forced = -1;
  if (forced < 0) {
    const char* e = getenv("EFLA_SCAN_TV");
    forced = (e && (atoi(e) == 16 || atoi(e) == 32)) ? atoi(e) : 0;
  }
  if (forced) return forced;
  const int64_t wgs32 = (int64_t)s.n_seqs * s.H * (s.dv / 32);
  return wgs32 < 256 ? 16 : 32;
}

void prof_begin(hipStream_t st) {
  if (!g_prof_on) return;
  g_prof_open = prof_event();
  if (g_prof_open && hipEventRecord(g_prof_open, st) != hipSuccess) g_prof_open = nullptr;
}

void prof_end(const char* name, hipStream_t st) {
  if (!g_prof_on || !g_prof_open) return;
  hipEvent_t b = prof_event();
  if (!b) return;
  if (hipEventRecord(b, st) != hipSuccess) {
    g_prof_free.push_back(b);
    g_prof_free.push_back(g_prof_open);
    g_prof_open = nullptr;
    return;
  }
  g_prof_pending.push_back(ProfRec{name, g_prof_open, b});
  g_prof_open = nullptr;
  if (g_prof_pending.size() > 4096) prof_drain();
}

// ---------------------------------------------------------------------------
// Validation and sizes.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool head_size_ok(int d) { return d == 64 || d == 128; }

efla_status to_shape(const efla_problem* p, Shape& s) {
  if (!p) return EFLA_ERR_NULL;
  if (p->dtype != EFLA_F32 && p->dtype != EFLA_BF16) return EFLA_ERR_DTYPE;
  if (p->B < 1 || p->H < 1 || p->T < 0 || p->dk < 1 || p->dv < 1) return EFLA_ERR_SHAPE;
  if (p->cu_seqlens) {
    if (p->B != 1 || p->n_seqs < 1) return EFLA_ERR_SHAPE;
  } else if (p->n_seqs != 0 && p->n_seqs != p->B) {
    return EFLA_ERR_SHAPE;
  }
  if (p->chunk != kChunk) return EFLA_ERR_UNSUPPORTED;
  if (p->mode != EFLA_EXACT && p->mode != EFLA_EULER) return EFLA_ERR_UNSUPPORTED;
  if (!head_size_ok(p->dk) || !head_size_ok(p->dv)) return EFLA_ERR_UNSUPPORTED;
  const Dt dt = p->dtype == EFLA_BF16 ? Dt::BF16 : Dt::F32;
  if (lds_ut_fwd(dt, p->dk, p->dv) == 0 || lds_chunk_bwd(dt, p->dk, p->dv) == 0)
    return EFLA_ERR_UNSUPPORTED;
  const int64_t tokens = (int64_t)p->B * p->H * p->T;
  const int64_t dmax = p->dk > p->dv ? p->dk : p->dv;
  if (tokens * dmax >= ((int64_t)1 << 40)) return EFLA_ERR_UNSUPPORTED;
  s.B = p->B;
  s.H = p->H;
  s.T = p->T;
  s.dk = p->dk;
  s.dv = p->dv;
  s.dt = dt;
  s.scale = p->scale;
  s.cu = p->cu_seqlens;
  s.n_seqs = p->cu_seqlens ? p->n_seqs : p->B;
  s.ntc = (p->T + kChunk - 1) / kChunk;
  s.slots = p->cu_seqlens ? (int64_t)(p->T / kChunk) + p->n_seqs : (int64_t)p->B * s.ntc;
  s.euler = p->mode == EFLA_EULER;
  if (s.slots * p->H >= ((int64_t)1 << 31)) return EFLA_ERR_UNSUPPORTED;
  // Segment plan of the forward scan (dense batches): G segments of nc chunks each.
  if (p->segments < 0) return EFLA_ERR_SHAPE;
  s.seg = 1;
  s.seg_nc = 0;
  s.seg_plan = 1;
  s.seg_plan_nc = 0;
  if (!p->cu_seqlens && s.ntc > 1) {
    int want = p->segments;
    if (want == 0) {  // split only when whole-sequence scans would leave compute units idle;
                      // aim at one scan workgroup per compute unit (256)
      const int64_t wgs = (int64_t)p->B * p->H * (p->dv / 32 > 0 ? p->dv / 32 : 1);
      want = (wgs < 128 && s.ntc >= 32) ? (int)(256 / wgs) : 1;
      if (want > s.ntc / 16) want = s.ntc / 16;
    }
    if (want > s.ntc) want = s.ntc;
    if (want > 1) {
      const int nc = (s.ntc + want - 1) / want;
      s.seg_plan = (s.ntc + nc - 1) / nc;  // no empty segment
      s.seg_plan_nc = nc;
    }
  }
  return EFLA_OK;
}

size_t esize(const Shape& s) { return s.dt == Dt::BF16 ? 2 : 4; }
size_t bytes_k(const Shape& s) { return (size_t)s.B * s.H * s.T * s.dk * esize(s); }
size_t bytes_v(const Shape& s) { return (size_t)s.B * s.H * s.T * s.dv * esize(s); }
size_t bytes_states(const Shape& s) { return (size_t)s.slots * s.H * s.dk * s.dv * esize(s); }
size_t bytes_table(const Shape& s) { return s.cu ? (size_t)(s.n_seqs + 1) * 4 : 0; }
size_t bytes_m(const Shape& s) { return (size_t)s.slots * s.H * kChunk * kChunk * esize(s); }
size_t bytes_x(const Shape& s) { return bytes_m(s); }
// Segment-parallel scan: R and S_in, fp32 [B * G][H][dk][dv], and P, fp32 [B * G][H][dk][dk].
size_t bytes_seg_state(const Shape& s) {
  return s.seg_plan > 1 ? (size_t)s.B * s.seg_plan * s.H * s.dk * s.dv * 4 : 0;
}
size_t bytes_seg_p(const Shape& s) {
  return s.seg_plan > 1 ? (size_t)s.B * s.seg_plan * s.H * s.dk * s.dk * 4 : 0;
}
size_t bytes_seg(const Shape& s) {
  return 2 * align_up(bytes_seg_state(s)) + align_up(bytes_seg_p(s));
}
// Gated forward: running log-decay sums per chunk, fp32 [slots][H][64].
size_t bytes_cum(const Shape& s) { return (size_t)s.slots * s.H * kChunk * 4; }
// The chunk factors the scans read. bf16 (xf): X and the per-token column scales alpha~ and b,
// fp32 [2][slots][H][64] (b only when gated); fp32: W and U, whose tiles leave the fp32 scans no
// LDS room for the X form.
bool xform(const Shape& s) { return s.dt == Dt::BF16; }
size_t coef_stride(const Shape& s) { return (size_t)s.slots * s.H * kChunk; }
size_t bytes_coef(const Shape& s) { return xform(s) ? 2 * coef_stride(s) * 4 : 0; }
size_t bytes_w(const Shape& s) { return xform(s) ? 0 : bytes_k(s); }

// Layout of the forward->backward buffer.
struct Saved {
  size_t w, ut, states, table, m, x, coef, cum, segp, total;
};
Saved saved_layout(const Shape& s) {
  Saved L;
  size_t o = 0;
  L.w = o;
  o += align_up(bytes_w(s));
  L.ut = o;
  o += align_up(bytes_v(s));
  L.states = o;
  o += align_up(bytes_states(s));
  L.table = o;
  o += align_up(bytes_table(s));
  L.m = o;
  o += align_up(bytes_m(s));
  L.x = o;
  o += align_up(bytes_x(s));
  L.coef = o;
  o += align_up(bytes_coef(s));
  L.cum = o;
  o += align_up(bytes_cum(s));
  L.segp = o;
  o += align_up(bytes_seg_p(s));
  L.total = o;
  return L;
}

// Forward workspace: U and W (fp32) or X and the column scales (bf16), the chunk table and M
// (fp32; all of them used only when no saved buffer is given, except U), the segment-parallel
// scan's buffers, and the gated forward's decay sums.
size_t bytes_ws_a(const Shape& s) { return xform(s) ? bytes_x(s) : bytes_v(s); }
size_t bytes_ws_b(const Shape& s) { return xform(s) ? bytes_coef(s) : bytes_k(s); }
size_t bytes_ws_m(const Shape& s) { return xform(s) ? 0 : bytes_m(s); }
size_t ws_fwd(const Shape& s) {
  return align_up(bytes_ws_a(s)) + align_up(bytes_ws_b(s)) + align_up(bytes_table(s)) +
         align_up(bytes_ws_m(s)) + bytes_seg(s) + align_up(bytes_cum(s));
}
// Buffers of one forward: saved-buffer regions when a saved buffer is given, workspace otherwise.
struct FwdBufs {
  unsigned char *w, *u, *x;  // W, U (fp32; U always in the workspace); X (bf16; fp32: saved only)
  float* coef;               // alpha~, then b (bf16)
  unsigned char *ut, *states;  // U~ and the chunk states (saved buffer only)
  int* table;
  unsigned char *m, *seg;
  float *cum, *segp;
};
FwdBufs fwd_bufs(const Shape& s, unsigned char* ws, unsigned char* sv) {
  const Saved L = saved_layout(s);
  FwdBufs b;
  unsigned char* a = ws;
  unsigned char* bb = a + align_up(bytes_ws_a(s));
  unsigned char* tb = bb + align_up(bytes_ws_b(s));
  unsigned char* mw = tb + align_up(bytes_table(s));
  b.seg = mw + align_up(bytes_ws_m(s));
  float* cum_ws = (float*)(b.seg + bytes_seg(s));
  b.u = xform(s) ? nullptr : a;
  b.w = xform(s) ? nullptr : (sv ? sv + L.w : bb);
  b.x = sv ? sv + L.x : (xform(s) ? a : nullptr);
  b.coef = xform(s) ? (float*)(sv ? sv + L.coef : bb) : nullptr;
  b.ut = sv ? sv + L.ut : nullptr;
  b.states = sv ? sv + L.states : nullptr;
  b.table = sv ? (int*)(sv + L.table) : (int*)tb;
  // M: fp32, written by the UT kernel and read by the forward scan; bf16, formed by the forward
  // scan itself where it writes O, and written out (for the backward) only into a saved buffer
  b.m = sv ? sv + L.m : (xform(s) ? nullptr : mw);
  b.cum = sv ? (float*)(sv + L.cum) : cum_ws;
  b.segp = sv ? (float*)(sv + L.segp) : nullptr;
  return b;
}
// Backward workspace: dU~ and the per-chunk state gradients, plus a full saved buffer and U for
// the recompute path, plus two segment state buffers (R and the states entering the segments of
// the recomputed forward, then R and the gradients entering the segments of the backward; the
// transitions live in the saved buffer).
size_t bytes_seg_bwd(const Shape& s) { return 2 * align_up(bytes_seg_state(s)); }
size_t ws_bwd(const Shape& s) {
  return align_up(bytes_v(s)) + align_up(bytes_states(s)) + saved_layout(s).total +
         (xform(s) ? 0 : align_up(bytes_v(s))) + bytes_seg_bwd(s);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

efla_status hip_status(hipError_t e) { return e == hipSuccess ? EFLA_OK : EFLA_ERR_HIP; }

bool empty(const Shape& s) { return s.T == 0; }

// Forward stages shared by efla_fwd and the recompute path of efla_bwd. b.seg: bytes_seg(s)
// of workspace for the segment-parallel scan (unused when the plan has one segment). gate (null,
// or log-decays) selects gated EFLA, which then needs b.cum. b.segp (null, or the saved buffer's
// region) receives the segments' transitions P for the backward; without it they stay in the
// workspace.
efla_status run_forward(const Shape& s, const void* q, const void* k, const void* v,
                        const void* beta, void* o, const FwdBufs& b, const float* h0, float* ht,
                        hipStream_t st, const void* gate = nullptr) {
  if (s.cu) {
    if (efla_status r = hip_status(launch_chunk_table(s, b.table, st))) return r;
  }
  const bool xf = xform(s);
  float* ca = b.coef;
  float* cb = xf && gate ? b.coef + coef_stride(s) : nullptr;
  if (efla_status r = hip_status(launch_ut_fwd(s, b.table, q, k, v, beta, gate, b.w, b.u, xf && o ? nullptr : b.m, b.x,
                                               gate ? b.cum : nullptr, ca, cb, st)))
    return r;
  const float* cm = gate ? b.cum : nullptr;
  const void* fa = xf ? (const void*)b.x : (const void*)b.w;  // X or W
  const void* fb = xf ? v : (const void*)b.u;                 // V or U
  if (s.seg_plan <= 1)
    return hip_status(launch_scan_fwd(s, b.table, q, k, fa, fb, b.m, o, b.ut, b.states, h0, ht, st,
                                      cm, ca, cb));
  // Segment-parallel: zero-start states R and transitions P of all segments, the sequential
  // chain S_in, then the output scan over all segments from S_in.
  const Shape sv = segment_view(s);
  float* R = (float*)b.seg;
  float* S_in = (float*)(b.seg + align_up(bytes_seg_state(s)));
  float* P = b.segp ? b.segp : (float*)(b.seg + 2 * align_up(bytes_seg_state(s)));
  if (efla_status r = hip_status(launch_scan_fwd_pair(sv, k, fa, fb, R, P, st, cm, ca, cb))) return r;
  if (efla_status r = hip_status(launch_seg_combine(s, P, R, h0, S_in, ht, st))) return r;
  return hip_status(launch_scan_fwd(sv, b.table, q, k, fa, fb, b.m, o, b.ut, b.states, S_in, nullptr,
                                    st, cm, ca, cb));
}

}  // namespace

// ---------------------------------------------------------------------------
// Workspace of efla_fwd_noalloc: a static device array, one copy per GPU, alive until the
// process ends. In host code `scratch` names a host-side stand-in, not device memory: kernels
// and copies get the device address that hipGetSymbolAddress returns for the current device.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = (size_t)EFLA_NOALLOC_WS_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (looked up once per device, with that device
// current); null if the device index is out of range or the lookup fails.
void* scratch_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}
}  // namespace
}  // namespace efla

using namespace efla;

extern "C" {

int efla_abi_version(void) { return EFLA_ABI_VERSION; }

const char* efla_status_str(efla_status s) {
  switch (s) {
    case EFLA_OK: return "ok";
    case EFLA_ERR_NULL: return "a required pointer is NULL";
    case EFLA_ERR_SHAPE: return "inconsistent problem sizes";
    case EFLA_ERR_DTYPE: return "unknown dtype";
    case EFLA_ERR_UNSUPPORTED: return "unsupported configuration";
    case EFLA_ERR_WORKSPACE: return "workspace or saved buffer too small";
    case EFLA_ERR_HIP: return "HIP launch failed";
    case EFLA_ERR_ALIGN: return "data pointer not 16-byte aligned";
  }
  return "unknown status";
}

efla_status efla_check_problem(const efla_problem* p) {
  Shape s;
  return to_shape(p, s);
}

size_t efla_workspace_bytes(const efla_problem* p, int for_backward) {
  Shape s;
  if (to_shape(p, s) != EFLA_OK) return 0;
  return for_backward ? ws_bwd(s) : ws_fwd(s);
}

size_t efla_saved_bytes(const efla_problem* p) {
  Shape s;
  if (to_shape(p, s) != EFLA_OK) return 0;
  return saved_layout(s).total;
}

efla_status efla_get_saved_layout(const efla_problem* p, efla_saved_layout* out) {
  Shape s;
  if (efla_status r = to_shape(p, s)) return r;
  if (!out) return EFLA_ERR_NULL;
  const Saved L = saved_layout(s);
  out->w = L.w;
  out->ut = L.ut;
  out->states = L.states;
  out->table = L.table;
  out->m = L.m;
  out->x = L.x;
  out->coef = L.coef;
  out->cum = L.cum;
  out->segp = L.segp;
  out->total = L.total;
  out->n_chunk_slots = s.slots;
  return EFLA_OK;
}

efla_status efla_prep(const efla_problem* p, const void* k, const void* beta, float* lam,
                      float* alpha, float* dalpha_dbeta, float* dalpha_dlam, void* stream) {
  Shape s;
  if (efla_status r = to_shape(p, s)) return r;
  if (empty(s)) return EFLA_OK;
  if (!k || !beta || !alpha) return EFLA_ERR_NULL;
  if (!aligned16(k)) return EFLA_ERR_ALIGN;
  return hip_status(launch_prep(s, k, beta, lam, alpha, dalpha_dbeta, dalpha_dlam,
                                (hipStream_t)stream));
}

efla_status efla_chunk_ut(const efla_problem* p, const void* k, const void* v, const void* beta,
                          void* w, void* u, void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  if (efla_status r = to_shape(p, s)) return r;
  if (empty(s)) return EFLA_OK;
  if (!k || !v || !beta || !w || !u) return EFLA_ERR_NULL;
  if (s.cu && !ws) return EFLA_ERR_NULL;
  if (!aligned16(k) || !aligned16(v) || !aligned16(w) || !aligned16(u) || !aligned16(ws))
    return EFLA_ERR_ALIGN;
  if (ws_bytes < ws_fwd(s)) return EFLA_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  int* table = (int*)ws;
  if (s.cu) {
    if (efla_status r = hip_status(launch_chunk_table(s, table, st))) return r;
  }
  return hip_status(launch_ut_fwd(s, table, nullptr, k, v, beta, nullptr, w, u, nullptr, nullptr,
                                  nullptr, nullptr, nullptr, st));
}

efla_status efla_fwd_state(const efla_problem* p, const void* q, const void* k, const void* v,
                           const void* beta, const float* h0, void* o, float* ht, void* saved,
                           size_t saved_bytes, void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  if (efla_status r = to_shape(p, s)) return r;
  if (empty(s)) return EFLA_OK;
  if (!q || !k || !v || !beta || !o || !ws) return EFLA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(ws) ||
      !aligned16(saved) || !aligned16(h0) || !aligned16(ht))
    return EFLA_ERR_ALIGN;
  if (ws_bytes < ws_fwd(s)) return EFLA_ERR_WORKSPACE;
  if (saved && saved_bytes < saved_layout(s).total) return EFLA_ERR_WORKSPACE;
  return run_forward(s, q, k, v, beta, o, fwd_bufs(s, (unsigned char*)ws, (unsigned char*)saved),
                     h0, ht, (hipStream_t)stream);
}

efla_status efla_fwd(const efla_problem* p, const void* q, const void* k, const void* v,
                     const void* beta, void* o, void* saved, size_t saved_bytes, void* ws,
                     size_t ws_bytes, void* stream) {
  return efla_fwd_state(p, q, k, v, beta, nullptr, o, nullptr, saved, saved_bytes, ws, ws_bytes,
                        stream);
}

efla_status efla_fwd_noalloc(const efla_problem* p, const void* q, const void* k, const void* v,
                             const void* beta, const float* h0, void* o, float* ht, void* stream) {
  Shape s;
  if (efla_status r = to_shape(p, s)) return r;
  if (empty(s)) return EFLA_OK;
  if (!q || !k || !v || !beta || !o) return EFLA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(h0) ||
      !aligned16(ht))
    return EFLA_ERR_ALIGN;
  if (ws_fwd(s) > kScratchBytes) return EFLA_ERR_WORKSPACE;
  void* ws = scratch_ptr();
  if (!ws) return EFLA_ERR_HIP;
  // the workspace layout of efla_fwd_state without a saved buffer; nothing in it has to start
  // at zero (every kernel writes what a later one reads)
  return run_forward(s, q, k, v, beta, o, fwd_bufs(s, (unsigned char*)ws, nullptr), h0, ht,
                     (hipStream_t)stream);
}

efla_status efla_fwd_gated(const efla_problem* p, const void* q, const void* k, const void* v,
                           const void* beta, const void* gate, const float* h0, void* o,
                           float* ht, void* saved, size_t saved_bytes, void* ws, size_t ws_bytes,
                           void* stream) {
  Shape s;
  if (efla_status r = to_shape(p, s)) return r;
  if (s.dt != Dt::BF16) return EFLA_ERR_UNSUPPORTED;
  if (empty(s)) return EFLA_OK;
  if (!q || !k || !v || !beta || !gate || !o || !ws) return EFLA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(ws) ||
      !aligned16(saved) || !aligned16(h0) || !aligned16(ht))
    return EFLA_ERR_ALIGN;
  if (ws_bytes < ws_fwd(s)) return EFLA_ERR_WORKSPACE;
  if (saved && saved_bytes < saved_layout(s).total) return EFLA_ERR_WORKSPACE;
  return run_forward(s, q, k, v, beta, o, fwd_bufs(s, (unsigned char*)ws, (unsigned char*)saved),
                     h0, ht, (hipStream_t)stream, gate);
}

}  // extern "C"

namespace efla {
namespace {
// Backward shared by efla_bwd_state and efla_bwd_gated (gate != NULL: gated EFLA, then dgate).
efla_status run_backward(const efla_problem* p, const void* q, const void* k, const void* v,
                         const void* beta, const void* gate, const float* h0, const void* d_o,
                         const float* dht, const void* saved, size_t saved_bytes, void* dq,
                         void* dk, void* dv, void* dbeta, void* dgate, float* dh0, void* ws,
                         size_t ws_bytes, void* stream) {
  Shape s;
  if (efla_status r = to_shape(p, s)) return r;
  if (gate && s.dt != Dt::BF16) return EFLA_ERR_UNSUPPORTED;
  if (empty(s)) return EFLA_OK;
  if (!q || !k || !v || !beta || !d_o || !dq || !dk || !dv || !dbeta || !ws) return EFLA_ERR_NULL;
  if (gate && !dgate) return EFLA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(d_o) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv) || !aligned16(ws) || !aligned16(saved) || !aligned16(h0) ||
      !aligned16(dht) || !aligned16(dh0))
    return EFLA_ERR_ALIGN;
  const Saved L = saved_layout(s);
  const size_t seg_bytes = s.seg_plan > 1 ? bytes_seg_bwd(s) : 0;
  const size_t need =
      saved ? align_up(bytes_v(s)) + align_up(bytes_states(s)) + seg_bytes : ws_bwd(s);
  if (ws_bytes < need) return EFLA_ERR_WORKSPACE;
  if (saved && saved_bytes < L.total) return EFLA_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  unsigned char* wsb = (unsigned char*)ws;
  unsigned char* dut = wsb;
  unsigned char* dstates = dut + align_up(bytes_v(s));
  // segment buffers: after the gradients with a saved buffer, else after the recomputed one
  unsigned char* seg = dstates + align_up(bytes_states(s));
  const unsigned char* sv = (const unsigned char*)saved;
  if (!sv) {
    // recompute: the forward into a saved buffer carved from the workspace; its own workspace
    // (U for fp32, and the segment buffers) after it
    unsigned char* rec = dstates + align_up(bytes_states(s));
    FwdBufs b = fwd_bufs(s, rec + L.total, rec);
    b.u = xform(s) ? nullptr : rec + L.total;
    b.seg = rec + L.total + (xform(s) ? 0 : align_up(bytes_v(s)));
    seg = b.seg;
    if (efla_status r = run_forward(s, q, k, v, beta, nullptr, b, h0, nullptr, st, gate)) return r;
    sv = rec;
  }
  const int* table = (const int*)(sv + L.table);
  const float* cum = gate ? (const float*)(sv + L.cum) : nullptr;
  // the factors of the backward scan: X and alpha~ (bf16) or W (fp32)
  const unsigned char* fa = xform(s) ? sv + L.x : sv + L.w;
  const float* ca = xform(s) ? (const float*)(sv + L.coef) : nullptr;
  if (s.seg_plan > 1) {
    // Segment-parallel reverse scan: zero-start gradients R of all segments, the chain over
    // segments from the last (dht) to the first (dh0) with the transposed forward transitions
    // (a segment maps the state gradient by P^T), then the full scan over all segments from the
    // gradient entering each from its end.
    const Shape svw = segment_view(s);
    float* R = (float*)seg;
    float* G_in = (float*)(seg + align_up(bytes_seg_state(s)));
    const float* A = (const float*)(sv + L.segp);
    if (efla_status r = hip_status(launch_scan_bwd(svw, table, q, k, fa, sv + L.m, d_o, nullptr,
                                                   nullptr, nullptr, R, st, cum, ca, true)))
      return r;
    if (efla_status r = hip_status(launch_seg_combine(s, A, R, dht, G_in, dh0, st, true, true)))
      return r;
    if (efla_status r = hip_status(launch_scan_bwd(svw, table, q, k, fa, sv + L.m, d_o, dut,
                                                   dstates, G_in, nullptr, st, cum, ca, false)))
      return r;
  } else if (efla_status r = hip_status(launch_scan_bwd(s, table, q, k, fa, sv + L.m, d_o, dut,
                                                        dstates, dht, dh0, st, cum, ca, false))) {
    return r;
  }
  return hip_status(launch_chunk_bwd(s, table, q, k, v, beta, d_o, sv + L.ut, dut, sv + L.states,
                                     dstates, sv + L.x, dq, dk, dv, dbeta, st, gate, cum, dgate));
}
}  // namespace
}  // namespace efla

extern "C" {

efla_status efla_bwd_state(const efla_problem* p, const void* q, const void* k, const void* v,
                           const void* beta, const float* h0, const void* d_o, const float* dht,
                           const void* saved, size_t saved_bytes, void* dq, void* dk, void* dv,
                           void* dbeta, float* dh0, void* ws, size_t ws_bytes, void* stream) {
  return run_backward(p, q, k, v, beta, nullptr, h0, d_o, dht, saved, saved_bytes, dq, dk, dv,
                      dbeta, nullptr, dh0, ws, ws_bytes, stream);
}

efla_status efla_bwd_gated(const efla_problem* p, const void* q, const void* k, const void* v,
                           const void* beta, const void* gate, const float* h0, const void* d_o,
                           const float* dht, const void* saved, size_t saved_bytes, void* dq,
                           void* dk, void* dv, void* dbeta, void* dgate, float* dh0, void* ws,
                           size_t ws_bytes, void* stream) {
  if (!gate) return EFLA_ERR_NULL;
  return run_backward(p, q, k, v, beta, gate, h0, d_o, dht, saved, saved_bytes, dq, dk, dv, dbeta,
                      dgate, dh0, ws, ws_bytes, stream);
}

efla_status efla_bwd(const efla_problem* p, const void* q, const void* k, const void* v,
                     const void* beta, const void* d_o, const void* saved, size_t saved_bytes,
                     void* dq, void* dk, void* dv, void* dbeta, void* ws, size_t ws_bytes,
                     void* stream) {
  return efla_bwd_state(p, q, k, v, beta, nullptr, d_o, nullptr, saved, saved_bytes, dq, dk, dv,
                        dbeta, nullptr, ws, ws_bytes, stream);
}

efla_status efla_decode(const efla_problem* p, const void* q, const void* k, const void* v,
                        const void* beta, float* state, void* o, void* stream) {
  Shape s;
  if (efla_status r = to_shape(p, s)) return r;
  if (s.cu) return EFLA_ERR_UNSUPPORTED;
  if (empty(s)) return EFLA_OK;
  if (!q || !k || !v || !beta || !state || !o) return EFLA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(state))
    return EFLA_ERR_ALIGN;
  return hip_status(launch_decode(s, q, k, v, beta, state, o, (hipStream_t)stream));
}

efla_status efla_decode_gated(const efla_problem* p, const void* q, const void* k,
                              const void* v, const void* beta, const void* gate, float* state,
                              void* o, void* stream) {
  Shape s;
  if (efla_status r = to_shape(p, s)) return r;
  if (s.cu) return EFLA_ERR_UNSUPPORTED;
  if (empty(s)) return EFLA_OK;
  if (!q || !k || !v || !beta || !gate || !state || !o) return EFLA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(state))
    return EFLA_ERR_ALIGN;
  return hip_status(launch_decode(s, q, k, v, beta, state, o, (hipStream_t)stream, gate));
}

efla_status efla_profile_enable(int on) {
  if (!on) prof_drain();
  g_prof_on = on != 0;
  return EFLA_OK;
}

int efla_profile_read(char* names, int name_stride, int64_t* counts, double* total_ms,
                      int max_kernels) {
  prof_drain();
  int i = 0;
  for (auto& kv : g_prof_totals) {
    if (i >= max_kernels) break;
    if (names && name_stride > 0) {
      strncpy(names + (size_t)i * name_stride, kv.first.c_str(), (size_t)name_stride - 1);
      names[(size_t)i * name_stride + name_stride - 1] = '\0';
    }
    if (counts) counts[i] = kv.second.first;
    if (total_ms) total_ms[i] = kv.second.second;
    ++i;
  }
  return i;
}

void efla_profile_reset(void) {
  prof_drain();
  g_prof_totals.clear();
}

}  // extern "C"

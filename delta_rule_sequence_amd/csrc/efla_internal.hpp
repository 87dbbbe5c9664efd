// Host-side declarations shared by the EFLA launch code (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "efla_device.hpp"

namespace efla {

enum class Dt { F32 = 0, BF16 = 1 };

// Problem sizes as the launchers see them.
struct Shape {
  int B, H, T, dk, dv;
  Dt dt;
  float scale;
  const int* cu;   // device cu_seqlens or nullptr (then B == 1)
  int n_seqs;      // sequences (B for dense batches)
  int ntc;         // ceil(T/64) (dense)
  int64_t slots;   // chunk slots per head (upper bound for packed batches)
  bool euler;      // step rule: delta rule (alpha = beta) instead of the exact flow
  int seg_plan;    // dense batches: segments per sequence of the forward scan (1 = none)
  int seg_plan_nc; // chunks per segment when seg_plan > 1
  int seg;         // segment view handed to a scan launch (1 = whole sequences): n_seqs is
  int seg_nc;      // then B * seg and sequence s is segment s % seg of batch row s / seg
};

// Optional per-kernel timing (efla_profile_enable): events recorded on the launch stream
// before and after each kernel. No-ops while profiling is off.
void prof_begin(hipStream_t st);
void prof_end(const char* name, hipStream_t st);

// Launchers. Each returns the HIP status of the launch.
hipError_t launch_chunk_table(const Shape& s, int* table, hipStream_t st);
hipError_t launch_prep(const Shape& s, const void* k, const void* beta, float* lam, float* alpha,
                       float* ex, float* dlam, hipStream_t st);
// gate (log-decays, problem dtype, or null) selects gated EFLA; cum then receives the running
// sums of the log-decays inside each chunk, fp32 [slots][H][64]. Every output may be null: W
// and U (w, u), M, X, and the factors' per-token column scales ca = alpha~ (alpha, gated
// alpha e^{c}) and cb = b (gated), fp32 [slots][H][64].
hipError_t launch_ut_fwd(const Shape& s, const int* table, const void* q, const void* k,
                         const void* v, const void* beta, const void* gate, void* w, void* u,
                         void* m, void* x, float* cum, float* ca, float* cb, hipStream_t st);
// The chunk factors the scans read: bf16 problems X ([slots][H][64][64]) with ca, cb as
// written by launch_ut_fwd, fp32 problems W and U. w / u below stand for X / V (the input
// values) in the first case and W / U in the second; ca, cb are unused for fp32.
// h0 / ht (scan_fwd) and dht / dh0 (scan_bwd): fp32 [n_seqs][H][dk][dv] per-sequence
// states entering / leaving the sequence, or null (zero in, not written out).
// cum (null, or the running log-decay sums of launch_ut_fwd) selects gated EFLA.
// m ([slots][H][64][64]): fp32, the M of launch_ut_fwd, read when O is written; bf16, null or
// where the scan writes the M it forms from Q and K (only when O is written).
hipError_t launch_scan_fwd(const Shape& s, const int* table, const void* q, const void* k,
                           const void* w, const void* u, void* m, void* o, void* ut,
                           void* states, const float* h0, float* ht, hipStream_t st,
                           const float* cum, const float* ca, const float* cb);
// For a segment view, in one launch: the zero-start state scan (final states into r, fp32
// [n_seqs][H][dk][dv]) and the transition scan, the product over each sequence's chunks of
// (I - K^T W) (gated: with the decays) into p, fp32 [n_seqs][H][dk][dk] (the scan with U = 0 from
// S = I).
hipError_t launch_scan_fwd_pair(const Shape& s, const void* k, const void* w, const void* u,
                                float* r, float* p, hipStream_t st, const float* cum,
                                const float* ca, const float* cb);
// Chain the segments of every sequence: S_0 = h0 (zero if null), S_{j+1} = P_j S_j + R_j;
// writes S_j of every segment to sin ([B * seg_plan][H][dk][dv]) and the final state to ht
// (if not null). P, R as produced by the transition and state-only scans of segment_view(s).
// reverse walks the segments from the last to the first (backward: state gradients), so
// sin[j] is the value entering segment j from its end; transpose applies P_j^T (the backward
// chains the state gradients with the forward's transitions, transposed).
hipError_t launch_seg_combine(const Shape& s, const float* p, const float* r, const float* h0,
                              float* sin, float* ht, hipStream_t st, bool reverse = false,
                              bool transpose = false);
// cum (null, or the saved running log-decay sums) selects gated EFLA. state_only: neither dU~
// nor the per-chunk gradients are written, only dh0 (first pass of the segment-parallel scan).
// w: X with ca = alpha~ (bf16) or W (fp32), as for launch_scan_fwd.
hipError_t launch_scan_bwd(const Shape& s, const int* table, const void* q, const void* k,
                           const void* w, const void* m, const void* d_o, void* dut,
                           void* dstates, const float* dht, float* dh0, hipStream_t st,
                           const float* cum, const float* ca, bool state_only);
hipError_t launch_decode(const Shape& s, const void* q, const void* k, const void* v,
                         const void* beta, float* state, void* o, hipStream_t st,
                         const void* gate = nullptr);
// gate (null, or log-decays) selects gated EFLA: then cum (saved running log-decay sums) and
// dgate (the log-decay gradient) are used.
hipError_t launch_chunk_bwd(const Shape& s, const int* table, const void* q, const void* k,
                            const void* v, const void* beta, const void* d_o, const void* ut,
                            const void* dut, const void* states, const void* dstates,
                            const void* x, void* dq, void* dk, void* dv, void* dbeta,
                            hipStream_t st, const void* gate = nullptr, const float* cum = nullptr,
                            void* dgate = nullptr);

// Dynamic LDS bytes of each kernel for a head-size pair (0 = combination not built).
size_t lds_ut_fwd(Dt dt, int dk, int dv);
size_t lds_scan_fwd(Dt dt, int dk, int dv);
size_t lds_scan_bwd(Dt dt, int dk, int dv);
size_t lds_chunk_bwd(Dt dt, int dk, int dv);

inline Geom make_geom(const Shape& s, const int* table) {
  Geom g;
  g.B = s.B;
  g.H = s.H;
  g.T = s.T;
  g.n_seqs = s.n_seqs;
  g.ntc = s.ntc;
  g.cu = s.cu;
  g.table = s.cu ? table : nullptr;
  g.max_slots = (int)s.slots;
  g.scale = s.scale;
  g.euler = s.euler ? 1 : 0;
  g.seg = s.seg;
  g.seg_nc = s.seg_nc;
  return g;
}

// The same problem seen by a scan launch as B * seg_plan independent segments.
inline Shape segment_view(const Shape& s) {
  Shape v = s;
  v.seg = s.seg_plan;
  v.seg_nc = s.seg_plan_nc;
  v.n_seqs = s.B * s.seg_plan;
  return v;
}

// Compute units of the current device (cached per device; 256 if the query fails).
int cu_count();

// Width of the d_v slice one scan workgroup owns: 16 when d_v = 64; for d_v = 128, 16 when
// width 32 would leave compute units idle (fewer than 256 workgroups), else 32.
// EFLA_SCAN_TV=16|32 overrides the choice for d_v = 128 (tuning).
int scan_tile(const Shape& s);

}  // namespace efla

// Recurrent inference: the token recurrence of the exact flow, one token after the other.
//
// Exact Flow Linear Attention summary page, section 3.2 (closed-form update with the
// effective step alpha_t) and the recurrent, linear-time inference the pages credit the
// delta-rule family with: per token
//   S <- S + alpha_t k_t (v_t - S^T k_t)^T,   o_t = scale S^T q_t   (state after the update).
// With log-decays (gated EFLA): S <- e^{a} (S - alpha k k^T S) + b k v^T, b the gated input
// coefficient. Column j of the update is S_j <- g S_j + k r_j with g = e^{a} (1 without a gate)
// and r_j = b v_j - g alpha (S^T k)_j, so the read-out after the update needs no second pass
// over the state: o_j = g (S^T q)_j + r_j (k . q), from the state before the update.
//
// The state is [B][H][d_k][d_v] fp32; decoding is bound by reading and writing it once per
// call, which for one token is a single round trip to memory and back. Each (batch row, head) is
// split over d_v / COLS workgroups of one wave each, so a call fills the chip and every reduction
// stays inside a wave: no barrier, no LDS. A wave's COLS columns form COLS / 4 groups of four;
// lane l holds the 16-byte column group l % (COLS / 4) of the rows l / (COLS / 4) + R i
// (R = 256 / COLS lanes share a group) in registers for all T tokens and loads the k and q
// entries of its own rows itself. Per token the partial sums of S^T k, S^T q, ||k||^2 and k . q
// over a lane's rows are reduced over the R lanes that share its column group (xor shuffles).
// The workgroups that cover one 128-byte line of every state row (32 columns) are placed on the
// same XCD (workgroups are dealt to the 8 XCDs round robin), so each line is fetched into one
// L2 only.
#include "efla_internal.hpp"

namespace efla {

constexpr int kDecCols = 16;  // state columns per workgroup (one wave): 16 measured fastest of 8, 16, 32

template <typename E, int DK, int DV, int COLS>
__global__ __launch_bounds__(64) void decode_kernel(Geom g, const E* __restrict__ q,
                                                    const E* __restrict__ k,
                                                    const E* __restrict__ v,
                                                    const E* __restrict__ beta,
                                                    const E* __restrict__ gate,
                                                    float* __restrict__ state,
                                                    E* __restrict__ o, int xcd_map) {
  constexpr int NG = COLS / 4;                  // column groups per wave
  constexpr int R = 64 / NG;                    // lanes sharing a column group (row stride)
  constexpr int RPT = DK / R;                   // rows per lane
  constexpr int NT = DV / COLS;                 // workgroups per (batch row, head)
  constexpr int NPL = 32 / COLS;                // workgroups per 128-byte line of a row
  static_assert(RPT >= 1 && DK % R == 0 && DV % 32 == 0 && NPL >= 1, "decode tiling");
  const int lane = threadIdx.x;
  const int cg = lane % NG, rg = lane / NG;     // column group, first row
  int u = blockIdx.x;
  if (xcd_map && NPL > 1) {  // the NPL consecutive units of one 32-column group share blockIdx % 8
    const int L = u >> 3, x = u & 7;
    u = (L / NPL) * (8 * NPL) + x * NPL + L % NPL;
  }
  const int64_t bh = u / NT;                    // b * H + h
  const int c0 = (u % NT) * COLS + 4 * cg;      // this lane's first column
  float* S = state + bh * DK * DV + c0;
  f32x4 col[RPT];                               // S[rg + R i][c0 .. c0 + 3]
#pragma unroll
  for (int i = 0; i < RPT; ++i) col[i] = *(const f32x4*)(S + (int64_t)(rg + R * i) * DV);
  const int64_t row0 = bh * g.T;
  for (int t = 0; t < g.T; ++t) {
    const int64_t r = row0 + t;
    float kd[RPT], qd[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      kd[i] = to_f(k[r * DK + rg + R * i]);
      qd[i] = to_f(q[r * DK + rg + R * i]);
    }
    const f32x4 vv = ld4f<E>(v + r * DV + c0);
    const float bt = to_f(beta[r]);
    const float lg = gate ? to_f(gate[r]) : 0.f;
    f32x4 y = zero4(), z = zero4();
    float lam = 0.f, kq = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      y += col[i] * kd[i];
      z += col[i] * qd[i];
      lam = fmaf(kd[i], kd[i], lam);
      kq = fmaf(kd[i], qd[i], kq);
    }
    // sum over the R lanes of this column group (every lane ends with the full sums)
#pragma unroll
    for (int off = NG; off < 64; off <<= 1) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        y[e] += __shfl_xor(y[e], off);
        z[e] += __shfl_xor(z[e], off);
      }
      lam += __shfl_xor(lam, off);
      kq += __shfl_xor(kq, off);
    }
    const float alpha = flow_coef(bt, lam, g.euler != 0).alpha;
    float gd = 1.f, bin = alpha;  // state decay and input coefficient (ungated: 1, alpha)
    if (gate) {
      gd = expf(lg);
      bin = gated_input_coef(bt, lam, lg, g.euler != 0);
    }
    const f32x4 rr = bin * vv - (gd * alpha) * y;   // r_j (ungated: alpha (v_j - y_j))
#pragma unroll
    for (int i = 0; i < RPT; ++i) col[i] = gd * col[i] + kd[i] * rr;
    if (rg == 0) {  // o_j = scale (g (S^T q)_j + r_j k . q): the lanes of row 0
      const f32x4 oj = g.scale * (gd * z + kq * rr);
      if constexpr (sizeof(E) == 4) {
        *(f32x4*)(o + r * DV + c0) = oj;
      } else {
        *(bf16x4*)(o + r * DV + c0) = bf16x4{(__bf16)oj[0], (__bf16)oj[1], (__bf16)oj[2], (__bf16)oj[3]};
      }
    }
  }
#pragma unroll
  for (int i = 0; i < RPT; ++i) *(f32x4*)(S + (int64_t)(rg + R * i) * DV) = col[i];
}

template <typename E, int DK, int DV>
static hipError_t decode_go(const Shape& s, const void* q, const void* k, const void* v,
                            const void* beta, const void* gate, float* state, void* o,
                            hipStream_t st) {
  constexpr int COLS = kDecCols, NPL = 32 / COLS;
  const int64_t blocks = (int64_t)s.B * s.H * (DV / COLS);
  if (blocks < 1) return hipSuccess;
  const int xcd_map = blocks % (8 * NPL) == 0 ? 1 : 0;  // the unit mapping is a bijection then
  prof_begin(st);
  hipLaunchKernelGGL((decode_kernel<E, DK, DV, COLS>), dim3((unsigned)blocks), dim3(64), 0, st,
                     make_geom(s, nullptr), (const E*)q, (const E*)k, (const E*)v,
                     (const E*)beta, (const E*)gate, state, (E*)o, xcd_map);
  hipError_t e = hipGetLastError();
  prof_end("decode", st);
  return e;
}

hipError_t launch_decode(const Shape& s, const void* q, const void* k, const void* v,
                         const void* beta, float* state, void* o, hipStream_t st,
                         const void* gate) {
#define EFLA_DC(E_, DK_, DV_) return decode_go<E_, DK_, DV_>(s, q, k, v, beta, gate, state, o, st)
  if (s.dt == Dt::BF16) {
    if (s.dk == 64 && s.dv == 64) EFLA_DC(__bf16, 64, 64);
    if (s.dk == 64 && s.dv == 128) EFLA_DC(__bf16, 64, 128);
    if (s.dk == 128 && s.dv == 64) EFLA_DC(__bf16, 128, 64);
    EFLA_DC(__bf16, 128, 128);
  }
  EFLA_DC(float, 64, 64);
#undef EFLA_DC
}

}  // namespace efla

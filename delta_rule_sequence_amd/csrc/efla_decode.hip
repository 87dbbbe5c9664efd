// Recurrent inference: the token recurrence of the exact flow, one token after the other.
//
// Exact Flow Linear Attention summary page, section 3.2 (closed-form update with the
// effective step alpha_t) and the recurrent, linear-time inference the pages credit the
// delta-rule family with: per token
//   S <- S + alpha_t k_t (v_t - S^T k_t)^T,   o_t = scale S^T q_t   (state after the update).
// One workgroup per (batch row, head); thread j keeps column j of the fp32 d_k x d_v state in
// registers for all T tokens, so the state is read and written once per call. k_t and q_t are
// shared through LDS; every thread forms ||k_t||^2 itself (d_k FMAs, cheaper than a reduction).
// With log-decays (gated EFLA): S <- e^{a} (S - alpha k k^T S) + b k v^T, b the gated input
// coefficient, i.e. column j: S_j <- e^{a} S_j + k (b v_j - e^{a} alpha (S^T k)_j).
#include "efla_internal.hpp"

namespace efla {

template <typename E, int DK, int DV>
__global__ __launch_bounds__(DV) void decode_kernel(Geom g, const E* __restrict__ q,
                                                    const E* __restrict__ k,
                                                    const E* __restrict__ v,
                                                    const E* __restrict__ beta,
                                                    const E* __restrict__ gate,
                                                    float* __restrict__ state,
                                                    E* __restrict__ o) {
  __shared__ float sk[DK], sq[DK];
  const int j = threadIdx.x;
  const int64_t bh = blockIdx.x;               // b * H + h
  float* S = state + bh * DK * DV;
  float col[DK];
#pragma unroll
  for (int d = 0; d < DK; ++d) col[d] = S[(int64_t)d * DV + j];
  const int64_t row0 = bh * g.T;
  for (int t = 0; t < g.T; ++t) {
    const int64_t r = row0 + t;
    __syncthreads();  // the previous token's reads of sk, sq are done
    for (int d = j; d < DK; d += DV) {
      sk[d] = to_f(k[r * DK + d]);
      sq[d] = to_f(q[r * DK + d]);
    }
    __syncthreads();
    float lam = 0.f, skj = 0.f;
#pragma unroll
    for (int d = 0; d < DK; ++d) {
      const float kd = sk[d];
      lam = fmaf(kd, kd, lam);
      skj = fmaf(col[d], kd, skj);  // (S^T k)_j
    }
    const float bt = to_f(beta[r]);
    const float a = flow_coef(bt, lam, g.euler != 0).alpha;
    float oj = 0.f;
    if (gate) {
      const float lg = to_f(gate[r]), gd = expf(lg);
      const float rj = gated_input_coef(bt, lam, lg, g.euler != 0) * to_f(v[r * DV + j]) - gd * a * skj;
#pragma unroll
      for (int d = 0; d < DK; ++d) {
        col[d] = fmaf(sk[d], rj, gd * col[d]);
        oj = fmaf(col[d], sq[d], oj);
      }
    } else {
      const float rj = a * (to_f(v[r * DV + j]) - skj);
#pragma unroll
      for (int d = 0; d < DK; ++d) {
        col[d] = fmaf(sk[d], rj, col[d]);
        oj = fmaf(col[d], sq[d], oj);
      }
    }
    o[r * DV + j] = to_e<E>(g.scale * oj);
  }
#pragma unroll
  for (int d = 0; d < DK; ++d) S[(int64_t)d * DV + j] = col[d];
}

template <typename E, int DK, int DV>
static hipError_t decode_go(const Shape& s, const void* q, const void* k, const void* v,
                            const void* beta, const void* gate, float* state, void* o,
                            hipStream_t st) {
  const int64_t blocks = (int64_t)s.B * s.H;
  if (blocks < 1) return hipSuccess;
  prof_begin(st);
  hipLaunchKernelGGL((decode_kernel<E, DK, DV>), dim3((unsigned)blocks), dim3(DV), 0, st,
                     make_geom(s, nullptr), (const E*)q, (const E*)k, (const E*)v,
                     (const E*)beta, (const E*)gate, state, (E*)o);
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

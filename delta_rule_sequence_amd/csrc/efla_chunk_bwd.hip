// Chunk-parallel gradients of the backward pass, one 64-token chunk per workgroup.
//
// Reverse-mode differentiation of the chunk form of section 3.3 (Exact Flow Linear
// Attention summary page) and of the exact-flow step of section 3.2, given for the chunk:
// S (incoming state), G (gradient of the outgoing state), U~ and dU~ (from the scans).
//   dM  = scale tril(dO U~^T)                 dQ = scale dO S^T + dM K
//   dK  = dM^T Q + U~ G^T                     dW = -dU~ S^T,  dU = dU~
// UT transform W = T K, U = T V, T = X diag(alpha), X = (I + A)^{-1},
// A = strictly_lower(diag(alpha) K K^T):
//   dT = dW K^T + dU V^T,  dK += T^T dW,  dV = T^T dU,
//   dalpha_j += sum_i dT_ij X_ij,  dA = -X^T (dT diag(alpha)) X^T (strictly lower),
//   dalpha_i += sum_j dA_ij (k_i . k_j),  dK += (dG + dG^T) K with dG = diag(alpha) dA.
// Exact-flow step alpha = (1 - e^{-beta lambda}) / lambda, lambda = ||k||^2:
//   dbeta = dalpha e^{-beta lambda},  dk += 2 k dalpha beta^2 phi'(beta lambda).
#include "efla_internal.hpp"

namespace efla {

template <typename E, int DK, int DV>
struct ChunkBwdLds {
  static constexpr int D = DK > DV ? DK : DV;
  static constexpr int LK = pitch<E>(DK), LV = pitch<E>(DV), LT = pitch<E>(64), LF = kPitchF;
  static constexpr size_t r0 = 64 * pitch<E>(D) * sizeof(E);
  static constexpr size_t r1 = D * LT * sizeof(E);
  static constexpr size_t r2 = 64 * LF * 4;
  static constexpr size_t RS = r0 > r1 ? (r0 > r2 ? r0 : r2) : (r1 > r2 ? r1 : r2);
  static constexpr size_t oK = 0;                                  // K   [64][LK]
  static constexpr size_t oKt = oK + 64 * LK * sizeof(E);          // K^T [DK][LT]
  static constexpr size_t oG = oKt + DK * LT * sizeof(E);          // K K^T strictly lower, fp32
  static constexpr size_t oX = oG + 64 * LF * 4;                   // X, fp32
  static constexpr size_t oCo = oX + 64 * LF * 4;                  // alpha, e^-x, dalpha/dlam, dalpha
  static constexpr size_t oScr = oCo + 4 * 64 * 4;                 // inverse scratch
  static constexpr size_t oR0 = oScr + 4 * 16 * 20 * 4;            // four phase regions
  static constexpr size_t oR1 = oR0 + RS;
  static constexpr size_t oR2 = oR1 + RS;
  static constexpr size_t oR3 = oR2 + RS;
  static constexpr size_t bytes = oR3 + RS;
};

template <typename E, int DK, int DV>
__global__ __launch_bounds__(kThreads) void chunk_bwd_kernel(
    Geom g, const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const E* __restrict__ beta, const E* __restrict__ d_o, const E* __restrict__ ut,
    const E* __restrict__ dut, const E* __restrict__ states, const E* __restrict__ dstates,
    E* __restrict__ dq, E* __restrict__ dk, E* __restrict__ dv, E* __restrict__ dbeta) {
  typedef ChunkBwdLds<E, DK, DV> L;
  constexpr int LK = L::LK, LV = L::LV, LT = L::LT, LF = L::LF;
  constexpr int CBK = DK / 64, CBV = DV / 64;  // column blocks per wave of [64][d] outputs
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  E* sK = (E*)(smem + L::oK);
  E* sKt = (E*)(smem + L::oKt);
  float* sG = (float*)(smem + L::oG);
  float* sX = (float*)(smem + L::oX);
  float* alpha = (float*)(smem + L::oCo);
  float* ex = alpha + 64;
  float* dlam = alpha + 128;
  float* dal = alpha + 192;
  float* sScr = (float*)(smem + L::oScr);
  unsigned char* R0 = smem + L::oR0;
  unsigned char* R1 = smem + L::oR1;
  unsigned char* R2 = smem + L::oR2;
  unsigned char* R3 = smem + L::oR3;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int slot = blockIdx.x / g.H, h = blockIdx.x % g.H;
  ChunkInfo ci;
  if (!chunk_info(g, slot, ci)) return;
  const int n = ci.n;
  const int64_t row0 = (int64_t)(ci.b * g.H + h) * g.T + ci.t0;
  const E* Sg = states + ((int64_t)slot * g.H + h) * DK * DV;   // incoming state [DK][DV]
  const E* Gg = dstates + ((int64_t)slot * g.H + h) * DK * DV;  // outgoing-state gradient

  // ---- A: coefficients, K K^T, X = (I + A)^{-1}
  g2s<E, DK>(sK, LK, k + row0 * DK, DK, n, tid);
  g2s_t<E, DK>(sKt, LT, k + row0 * DK, DK, n, tid);
  __syncthreads();
  {
    const int r = tid >> 2, q4 = tid & 3;
    float acc = 0.f;
#pragma unroll 8
    for (int c = q4 * (DK / 4); c < (q4 + 1) * (DK / 4); ++c) {
      const float x = to_f(sK[r * LK + c]);
      acc = fmaf(x, x, acc);
    }
    acc += __shfl_xor(acc, 1);
    acc += __shfl_xor(acc, 2);
    if (q4 == 0) {
      const float bt = r < n ? to_f(beta[row0 + r]) : 0.f;
      const FlowCoef cf = flow_coef(bt, acc);
      alpha[r] = cf.alpha;
      ex[r] = cf.ex;
      dlam[r] = cf.dlam;
      dal[r] = 0.f;
    }
  }
  __syncthreads();
  {
    float* sA = (float*)R0;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      f32x4 acc = zero4();
      if (nb <= wv) acc = mma16<E>(sK + 16 * wv * LK, LK, sK + 16 * nb * LK, LK, 0, DK, acc, lane);
      const int col = 16 * nb + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * wv + 4 * (lane >> 4) + i;
        const float gv = row > col ? acc[i] : 0.f;
        sG[row * LF + col] = gv;
        sA[row * LF + col] = alpha[row] * gv;
      }
    }
    __syncthreads();
    invert_unit_lower64(sA, sX, sScr, tid);
  }

  // ---- E: dU~ (row-major R0, transposed R1); dW = -dU~ S^T (row-major R2, transposed R3)
  E* sdU = (E*)R0;
  E* sdUt = (E*)R1;
  E* sdW = (E*)R2;
  E* sdWt = (E*)R3;
  g2s<E, DV>(sdU, LV, dut + row0 * DV, DV, n, tid);
  g2s_t<E, DV>(sdUt, LT, dut + row0 * DV, DV, n, tid);
  __syncthreads();
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
    for (int cbi = 0; cbi < CBK; ++cbi) {
      const int cb = wv * CBK + cbi;
      f32x4 acc = mma16_gb<E>(sdU + 16 * rb * LV, LV, Sg + (int64_t)16 * cb * DV, DV, 0, DV, zero4(), lane);
      acc = -acc;
      st_frag_lds<E>(sdW + 16 * rb * LK + 16 * cb, LK, acc, lane);
      st_frag_t<E>(sdWt + 16 * cb * LT + 16 * rb, LT, acc, lane);
    }
  }
  __syncthreads();

  // ---- F: dT = dW K^T + dU V^T (lower incl. diagonal), row block wv in registers
  f32x4 dT[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    dT[nb] = zero4();
    if (nb <= wv) dT[nb] = mma16<E>(sdW + 16 * wv * LK, LK, sK + 16 * nb * LK, LK, 0, DK, dT[nb], lane);
  }
  __syncthreads();
  E* sV = (E*)R2;
  g2s<E, DV>(sV, LV, v + row0 * DV, DV, n, tid);
  __syncthreads();
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
    if (nb <= wv) dT[nb] = mma16<E>(sdU + 16 * wv * LV, LV, sV + 16 * nb * LV, LV, 0, DV, dT[nb], lane);
  __syncthreads();

  // ---- G: T^T [j][i] = alpha_j X_ij; dK = T^T dW; dV = T^T dU
  E* sTt = (E*)R2;
  for (int idx = tid; idx < 64 * 64; idx += kThreads) {
    const int j = idx >> 6, i = idx & 63;
    sTt[j * LT + i] = to_e<E>(i >= j ? alpha[j] * sX[i * LF + j] : 0.f);
  }
  __syncthreads();
  f32x4 dKa[4 * CBK];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int k0 = round_down_kc<E>(16 * rb);
#pragma unroll
    for (int cbi = 0; cbi < CBK; ++cbi) {
      const int cb = wv * CBK + cbi;
      dKa[rb * CBK + cbi] = mma16<E>(sTt + 16 * rb * LT, LT, sdWt + 16 * cb * LT, LT, k0, kChunk, zero4(), lane);
    }
#pragma unroll
    for (int cbi = 0; cbi < CBV; ++cbi) {
      const int cb = wv * CBV + cbi;
      const f32x4 acc = mma16<E>(sTt + 16 * rb * LT, LT, sdUt + 16 * cb * LT, LT, k0, kChunk, zero4(), lane);
      st_frag_rows<E>(dv + (row0 + 16 * rb) * DV + 16 * cb, DV, acc, lane, 16 * rb, n);
    }
  }
  __syncthreads();

  // ---- H1: dT to LDS; dalpha from T = X diag(alpha); dX = dT diag(alpha) (strictly lower)
  float* sdT = (float*)R0;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) st_frag_lds<float>(sdT + 16 * wv * LF + 16 * nb, LF, dT[nb], lane);
  __syncthreads();
  E* sdX = (E*)R1;
  E* sXe = (E*)R3;
  E* sXte = (E*)R2;
  if (tid < 64) {
    const int j = tid;
    float s = 0.f;
    for (int i = j; i < 64; ++i) s = fmaf(sdT[i * LF + j], sX[i * LF + j], s);
    dal[j] += s;
  }
  for (int idx = tid; idx < 64 * 64; idx += kThreads) {
    const int i = idx >> 6, j = idx & 63;
    const float x = sX[i * LF + j];
    sdX[i * LT + j] = to_e<E>(i > j ? sdT[i * LF + j] * alpha[j] : 0.f);
    sXe[i * LT + j] = to_e<E>(x);
    sXte[j * LT + i] = to_e<E>(x);
  }
  __syncthreads();

  // ---- H2: Y = dX X^T (row block wv), stored transposed
  E* sYt = (E*)R0;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int k1 = round_up_kc<E>(16 * ((wv < nb ? wv : nb) + 1));
    const f32x4 acc = mma16<E>(sdX + 16 * wv * LT, LT, sXe + 16 * nb * LT, LT, 0, k1, zero4(), lane);
    st_frag_t<E>(sYt + 16 * nb * LT + 16 * wv, LT, acc, lane);
  }
  __syncthreads();

  // ---- H3: dA = -X^T Y (strictly lower); dalpha_i += sum_j dA_ij G_ij; H = dG + dG^T
  E* sH = (E*)R1;
  {
    float rs[4] = {0.f, 0.f, 0.f, 0.f};
    const int k0 = round_down_kc<E>(16 * wv);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      if (nb > wv) continue;
      const f32x4 acc = mma16<E>(sXte + 16 * wv * LT, LT, sYt + 16 * nb * LT, LT, k0, kChunk, zero4(), lane);
      const int col = 16 * nb + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * wv + 4 * (lane >> 4) + i;
        if (row > col) {
          const float da = -acc[i];
          rs[i] = fmaf(da, sG[row * LF + col], rs[i]);
          const E dg = to_e<E>(alpha[row] * da);
          sH[row * LT + col] = dg;
          sH[col * LT + row] = dg;
        } else if (row == col) {
          sH[row * LT + col] = to_e<E>(0.f);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x = rs[i];
      x += __shfl_xor(x, 1);
      x += __shfl_xor(x, 2);
      x += __shfl_xor(x, 4);
      x += __shfl_xor(x, 8);
      if ((lane & 15) == 0) dal[16 * wv + 4 * (lane >> 4) + i] += x;
    }
  }
  __syncthreads();

  // ---- I: dK += H K
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cbi = 0; cbi < CBK; ++cbi) {
      const int cb = wv * CBK + cbi;
      dKa[rb * CBK + cbi] = mma16<E>(sH + 16 * rb * LT, LT, sKt + 16 * cb * LT, LT, 0, kChunk, dKa[rb * CBK + cbi], lane);
    }
  __syncthreads();

  // ---- B: dO (R0), U~ (R2); dM = scale tril(dO U~^T) row-major (R1) and transposed (R3)
  E* sdO = (E*)R0;
  E* sUu = (E*)R2;
  E* sdM = (E*)R1;
  E* sdMt = (E*)R3;
  g2s<E, DV>(sdO, LV, d_o + row0 * DV, DV, n, tid);
  g2s<E, DV>(sUu, LV, ut + row0 * DV, DV, n, tid);
  __syncthreads();
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    f32x4 acc = zero4();
    if (nb <= wv) {
      acc = mma16<E>(sdO + 16 * wv * LV, LV, sUu + 16 * nb * LV, LV, 0, DV, acc, lane);
      if (nb == wv) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if ((lane & 15) > 4 * (lane >> 4) + i) acc[i] = 0.f;
      }
      acc *= g.scale;
    }
    st_frag_lds<E>(sdM + 16 * wv * LT + 16 * nb, LT, acc, lane);
    st_frag_t<E>(sdMt + 16 * nb * LT + 16 * wv, LT, acc, lane);
  }
  __syncthreads();

  // ---- C: dQ = scale dO S^T + dM K
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int k1 = round_up_kc<E>(16 * (rb + 1));
#pragma unroll
    for (int cbi = 0; cbi < CBK; ++cbi) {
      const int cb = wv * CBK + cbi;
      f32x4 acc = mma16_gb<E>(sdO + 16 * rb * LV, LV, Sg + (int64_t)16 * cb * DV, DV, 0, DV, zero4(), lane);
      acc *= g.scale;
      acc = mma16<E>(sdM + 16 * rb * LT, LT, sKt + 16 * cb * LT, LT, 0, k1, acc, lane);
      st_frag_rows<E>(dq + (row0 + 16 * rb) * DK + 16 * cb, DK, acc, lane, 16 * rb, n);
    }
  }
  __syncthreads();

  // ---- D: dK += dM^T Q + U~ G^T
  E* sQt = (E*)R0;
  g2s_t<E, DK>(sQt, LT, q + row0 * DK, DK, n, tid);
  __syncthreads();
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int k0 = round_down_kc<E>(16 * rb);
#pragma unroll
    for (int cbi = 0; cbi < CBK; ++cbi) {
      const int cb = wv * CBK + cbi;
      f32x4 acc = dKa[rb * CBK + cbi];
      acc = mma16<E>(sdMt + 16 * rb * LT, LT, sQt + 16 * cb * LT, LT, k0, kChunk, acc, lane);
      acc = mma16_gb<E>(sUu + 16 * rb * LV, LV, Gg + (int64_t)16 * cb * DV, DV, 0, DV, acc, lane);
      // exact-flow step: lambda = ||k||^2 enters alpha
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * rb + 4 * (lane >> 4) + i;
        const int col = 16 * cb + (lane & 15);
        acc[i] = fmaf(2.f * to_f(sK[row * LK + col]), dal[row] * dlam[row], acc[i]);
      }
      st_frag_rows<E>(dk + (row0 + 16 * rb) * DK + 16 * cb, DK, acc, lane, 16 * rb, n);
    }
  }
  if (tid < n) dbeta[row0 + tid] = to_e<E>(dal[tid] * ex[tid]);
}

template <typename E, int DK, int DV>
static hipError_t chunk_bwd_go(const Shape& s, const int* table, const void* q, const void* k,
                               const void* v, const void* beta, const void* d_o, const void* ut,
                               const void* dut, const void* states, const void* dstates, void* dq,
                               void* dk, void* dv, void* dbeta, hipStream_t st) {
  typedef ChunkBwdLds<E, DK, DV> L;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)chunk_bwd_kernel<E, DK, DV>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)L::bytes);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const int64_t blocks = s.slots * s.H;
  if (blocks < 1) return hipSuccess;
  prof_begin(st);
  hipLaunchKernelGGL((chunk_bwd_kernel<E, DK, DV>), dim3((unsigned)blocks), dim3(kThreads), L::bytes,
                     st, make_geom(s, table), (const E*)q, (const E*)k, (const E*)v,
                     (const E*)beta, (const E*)d_o, (const E*)ut, (const E*)dut,
                     (const E*)states, (const E*)dstates, (E*)dq, (E*)dk, (E*)dv, (E*)dbeta);
  hipError_t e = hipGetLastError();
  prof_end("chunk_bwd", st);
  return e;
}

size_t lds_chunk_bwd(Dt dt, int dk, int dv) {
  if (dt == Dt::BF16) {
    if (dk == 64 && dv == 64) return ChunkBwdLds<__bf16, 64, 64>::bytes;
    if (dk == 64 && dv == 128) return ChunkBwdLds<__bf16, 64, 128>::bytes;
    if (dk == 128 && dv == 64) return ChunkBwdLds<__bf16, 128, 64>::bytes;
    if (dk == 128 && dv == 128) return ChunkBwdLds<__bf16, 128, 128>::bytes;
    return 0;
  }
  if (dk == 64 && dv == 64) return ChunkBwdLds<float, 64, 64>::bytes;
  return 0;
}

hipError_t launch_chunk_bwd(const Shape& s, const int* table, const void* q, const void* k,
                            const void* v, const void* beta, const void* d_o, const void* ut,
                            const void* dut, const void* states, const void* dstates, void* dq,
                            void* dk, void* dv, void* dbeta, hipStream_t st) {
#define EFLA_CB(E_, DK_, DV_)                                                                   \
  return chunk_bwd_go<E_, DK_, DV_>(s, table, q, k, v, beta, d_o, ut, dut, states, dstates, dq, \
                                    dk, dv, dbeta, st)
  if (s.dt == Dt::BF16) {
    if (s.dk == 64 && s.dv == 64) EFLA_CB(__bf16, 64, 64);
    if (s.dk == 64 && s.dv == 128) EFLA_CB(__bf16, 64, 128);
    if (s.dk == 128 && s.dv == 64) EFLA_CB(__bf16, 128, 64);
    EFLA_CB(__bf16, 128, 128);
  }
  EFLA_CB(float, 64, 64);
#undef EFLA_CB
}

}  // namespace efla

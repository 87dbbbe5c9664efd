// UT transform of one 64-token chunk per workgroup.
//
// Exact Flow Linear Attention summary page, section 3.3 (chunkwise form with the UT
// transform; the WY/UT representation is the DeltaNet prior art of the fifth page):
//   alpha_i = exact-flow step of token i,  A = strictly_lower(diag(alpha) K K^T),
//   T = (I + A)^{-1} diag(alpha),  W = T K,  U = T V.
// K K^T, T K and T V are MFMA contractions; the unit lower triangular inverse is a
// blocked forward substitution in fp32 in LDS. Padded rows of a tail chunk read as zero
// (their beta is zero, so alpha = 0 and they do not touch the valid rows).
#include "efla_internal.hpp"

namespace efla {

template <typename E, int DK, int DV>
struct UtFwdLds {
  static constexpr int LK = pitch<E>(DK), LT = pitch<E>(64), LV = pitch<E>(DV), LF = kPitchF;
  static constexpr size_t oK = 0;                                   // K        [64][LK]
  static constexpr size_t oKt = oK + 64 * LK * sizeof(E);           // K^T      [DK][LT]
  static constexpr size_t oVt = oKt + DK * LT * sizeof(E);          // V^T      [DV][LT]
  static constexpr size_t oT = oVt + DV * LT * sizeof(E);           // T        [64][LT]
  static constexpr size_t oA = oT + 64 * LT * sizeof(E);            // A (fp32) [64][LF]
  static constexpr size_t oX = oA + 64 * LF * 4;                    // X (fp32) [64][LF]
  static constexpr size_t oAl = oX + 64 * LF * 4;                   // alpha    [64]
  static constexpr size_t oScr = oAl + 64 * 4;                      // inverse scratch
  static constexpr size_t bytes = oScr + 4 * 16 * 20 * 4;
  static_assert(64 * LV * sizeof(E) <= 64 * LF * 4, "U staging must fit in the A buffer");
};

template <typename E, int DK, int DV>
__global__ __launch_bounds__(kThreads) void ut_fwd_kernel(Geom g, const E* __restrict__ k,
                                                          const E* __restrict__ v,
                                                          const E* __restrict__ beta,
                                                          E* __restrict__ w, E* __restrict__ u) {
  typedef UtFwdLds<E, DK, DV> L;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  E* sK = (E*)(smem + L::oK);
  E* sKt = (E*)(smem + L::oKt);
  E* sVt = (E*)(smem + L::oVt);
  E* sT = (E*)(smem + L::oT);
  float* sA = (float*)(smem + L::oA);
  float* sX = (float*)(smem + L::oX);
  float* sAl = (float*)(smem + L::oAl);
  float* sScr = (float*)(smem + L::oScr);
  E* sU = (E*)(smem + L::oA);  // U staging after the inverse is done

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int slot = blockIdx.x / g.H, h = blockIdx.x % g.H;
  ChunkInfo ci;
  if (!chunk_info(g, slot, ci)) return;
  const int n = ci.n;
  const int64_t row0 = (int64_t)(ci.b * g.H + h) * g.T + ci.t0;
  const E* gk = k + row0 * DK;
  const E* gv = v + row0 * DV;

  g2s<E, DK>(sK, L::LK, gk, DK, n, tid);
  g2s_t<E, DK>(sKt, L::LT, gk, DK, n, tid);
  g2s_t<E, DV>(sVt, L::LT, gv, DV, n, tid);
  __syncthreads();

  {  // alpha per row: 4 threads per row
    const int r = tid >> 2, q4 = tid & 3;
    float acc = 0.f;
#pragma unroll 8
    for (int c = q4 * (DK / 4); c < (q4 + 1) * (DK / 4); ++c) {
      const float x = to_f(sK[r * L::LK + c]);
      acc = fmaf(x, x, acc);
    }
    acc += __shfl_xor(acc, 1);
    acc += __shfl_xor(acc, 2);
    if (q4 == 0) {
      const float bt = r < n ? to_f(beta[row0 + r]) : 0.f;
      sAl[r] = flow_coef(bt, acc).alpha;
    }
  }
  __syncthreads();

  // A = strictly_lower(diag(alpha) K K^T); wave wv owns row block wv.
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    f32x4 acc = zero4();
    if (nb <= wv) acc = mma16<E>(sK + 16 * wv * L::LK, L::LK, sK + 16 * nb * L::LK, L::LK, 0, DK, acc, lane);
    const int col = 16 * nb + (lane & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * wv + 4 * (lane >> 4) + i;
      sA[row * L::LF + col] = row > col ? sAl[row] * acc[i] : 0.f;
    }
  }
  __syncthreads();
  invert_unit_lower64(sA, sX, sScr, tid);

  // T = X diag(alpha)
  for (int i = tid; i < 64 * 64; i += kThreads) {
    const int r = i >> 6, c = i & 63;
    sT[r * L::LT + c] = to_e<E>(sX[r * L::LF + c] * sAl[c]);
  }
  __syncthreads();

  // W = T K, U = T V; T is lower triangular, so row block wv needs columns < 16 (wv + 1).
  const int k1 = round_up_kc<E>(16 * (wv + 1));
#pragma unroll
  for (int nb = 0; nb < DK / 16; ++nb) {
    f32x4 acc = mma16<E>(sT + 16 * wv * L::LT, L::LT, sKt + 16 * nb * L::LT, L::LT, 0, k1, zero4(), lane);
    st_frag_lds<E>(sK + 16 * wv * L::LK + 16 * nb, L::LK, acc, lane);
  }
#pragma unroll
  for (int nb = 0; nb < DV / 16; ++nb) {
    f32x4 acc = mma16<E>(sT + 16 * wv * L::LT, L::LT, sVt + 16 * nb * L::LT, L::LT, 0, k1, zero4(), lane);
    st_frag_lds<E>(sU + 16 * wv * L::LV + 16 * nb, L::LV, acc, lane);
  }
  __syncthreads();
  s2g<E, DK>(w + row0 * DK, DK, sK, L::LK, n, tid);
  s2g<E, DV>(u + row0 * DV, DV, sU, L::LV, n, tid);
}

template <typename E, int DK, int DV>
static hipError_t ut_go(const Shape& s, const int* table, const void* k, const void* v,
                        const void* beta, void* w, void* u, hipStream_t st) {
  typedef UtFwdLds<E, DK, DV> L;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)ut_fwd_kernel<E, DK, DV>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)L::bytes);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const int64_t blocks = s.slots * s.H;
  if (blocks < 1) return hipSuccess;
  prof_begin(st);
  hipLaunchKernelGGL((ut_fwd_kernel<E, DK, DV>), dim3((unsigned)blocks), dim3(kThreads), L::bytes,
                     st, make_geom(s, table), (const E*)k, (const E*)v, (const E*)beta, (E*)w,
                     (E*)u);
  hipError_t e = hipGetLastError();
  prof_end("ut_fwd", st);
  return e;
}

size_t lds_ut_fwd(Dt dt, int dk, int dv) {
  if (dt == Dt::BF16) {
    if (dk == 64 && dv == 64) return UtFwdLds<__bf16, 64, 64>::bytes;
    if (dk == 64 && dv == 128) return UtFwdLds<__bf16, 64, 128>::bytes;
    if (dk == 128 && dv == 64) return UtFwdLds<__bf16, 128, 64>::bytes;
    if (dk == 128 && dv == 128) return UtFwdLds<__bf16, 128, 128>::bytes;
    return 0;
  }
  if (dk == 64 && dv == 64) return UtFwdLds<float, 64, 64>::bytes;
  return 0;
}

hipError_t launch_ut_fwd(const Shape& s, const int* table, const void* k, const void* v,
                         const void* beta, void* w, void* u, hipStream_t st) {
  if (s.dt == Dt::BF16) {
    if (s.dk == 64 && s.dv == 64) return ut_go<__bf16, 64, 64>(s, table, k, v, beta, w, u, st);
    if (s.dk == 64 && s.dv == 128) return ut_go<__bf16, 64, 128>(s, table, k, v, beta, w, u, st);
    if (s.dk == 128 && s.dv == 64) return ut_go<__bf16, 128, 64>(s, table, k, v, beta, w, u, st);
    return ut_go<__bf16, 128, 128>(s, table, k, v, beta, w, u, st);
  }
  return ut_go<float, 64, 64>(s, table, k, v, beta, w, u, st);
}

}  // namespace efla

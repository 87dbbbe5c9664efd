// Reverse inter-chunk recurrence of the backward pass.
//
// Reverse-mode differentiation of the chunk recurrence of section 3.3 (Exact Flow Linear
// Attention summary page): with G the gradient of the state leaving chunk c,
//   dU~_c = scale tril(Q K^T)^T dO_c + K_c G,
//   G    <- G + scale Q_c^T dO_c - W_c^T dU~_c      (gradient of the state entering c).
// One workgroup walks the chunks of one (sequence, head) backwards and owns a d_k x TV
// slice of G in fp32 accumulators. It writes dU~ and, per chunk, the G that entered the
// step (the gradient of the chunk's outgoing state) for the chunk-parallel gradient kernel.
#include "efla_internal.hpp"

namespace efla {

template <typename E, int DK, int DV, int TV>
struct ScanBwdLds {
  static constexpr int LK = pitch<E>(DK), LT = pitch<E>(64);
  static constexpr size_t oQ = 0;                               // Q      [64][LK]
  static constexpr size_t oQt = oQ + 64 * LK * sizeof(E);       // Q^T    [DK][LT]
  static constexpr size_t oK = oQt + DK * LT * sizeof(E);       // K      [64][LK]
  static constexpr size_t oWt = oK + 64 * LK * sizeof(E);       // W^T    [DK][LT]
  static constexpr size_t oOt = oWt + DK * LT * sizeof(E);      // dO^T   [TV][LT]
  static constexpr size_t oGt = oOt + TV * LT * sizeof(E);      // G^T    [TV][LK]
  static constexpr size_t oMt = oGt + TV * LK * sizeof(E);      // tril(QK^T)^T [64][LT]
  static constexpr size_t oDt = oMt + 64 * LT * sizeof(E);      // dU~^T  [TV][LT]
  static constexpr size_t bytes = oDt + TV * LT * sizeof(E);
};

template <typename E, int DK, int DV, int TV>
__global__ __launch_bounds__(kThreads) void scan_bwd_kernel(
    Geom g, const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ w,
    const E* __restrict__ d_o, E* __restrict__ dut, E* __restrict__ dstates) {
  typedef ScanBwdLds<E, DK, DV, TV> L;
  constexpr int NTILE = DV / TV;
  constexpr int NB = TV / 16;
  constexpr int TPW = (DK / 16) * NB / 4;
  static_assert(TPW >= 1 && ((DK / 16) * NB) % 4 == 0, "state tiles must split over 4 waves");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  E* sQ = (E*)(smem + L::oQ);
  E* sQt = (E*)(smem + L::oQt);
  E* sK = (E*)(smem + L::oK);
  E* sWt = (E*)(smem + L::oWt);
  E* sOt = (E*)(smem + L::oOt);
  E* sGt = (E*)(smem + L::oGt);
  E* sMt = (E*)(smem + L::oMt);
  E* sDt = (E*)(smem + L::oDt);

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int sh, tile;
  scan_block(blockIdx.x, g.n_seqs * g.H, NTILE, sh, tile);
  const int s = sh / g.H, h = sh % g.H;
  const SeqInfo si = seq_info(g, s);
  const int nchunks = seq_chunks(g, si);
  const int v0 = tile * TV;
  const int k0M = round_down_kc<E>(16 * wv);  // row block wv of tril(.)^T needs cols >= 16 wv

  f32x4 G[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) G[i] = zero4();

  for (int c = nchunks - 1; c >= 0; --c) {
    const int n = min(kChunk, si.len - c * kChunk);
    const int64_t row0 = (int64_t)(si.b * g.H + h) * g.T + si.bos + c * kChunk;
    g2s<E, DK>(sQ, L::LK, q + row0 * DK, DK, n, tid);
    g2s_t<E, DK>(sQt, L::LT, q + row0 * DK, DK, n, tid);
    g2s<E, DK>(sK, L::LK, k + row0 * DK, DK, n, tid);
    g2s_t<E, DK>(sWt, L::LT, w + row0 * DK, DK, n, tid);
    g2s_t<E, TV>(sOt, L::LT, d_o + row0 * DV + v0, DV, n, tid);
    E* gG = dstates + ((int64_t)(si.slot0 + c) * g.H + h) * DK * DV;
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = wv + 4 * i, mb = t / NB, nb = t % NB;
      st_frag_t<E>(sGt + 16 * nb * L::LK + 16 * mb, L::LK, G[i], lane);
      st_frag_glb<E>(gG + (int64_t)16 * mb * DV + v0 + 16 * nb, DV, G[i], lane);
    }
    __syncthreads();

    // tril(Q K^T)^T [j][i] = k_j . q_i for i >= j; row block wv (j).
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      if (16 * nb >= k0M) {
        f32x4 acc = zero4();
        if (nb >= wv) {
          acc = mma16<E>(sK + 16 * wv * L::LK, L::LK, sQ + 16 * nb * L::LK, L::LK, 0, DK, acc, lane);
          if (nb == wv) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if ((lane & 15) < 4 * (lane >> 4) + i) acc[i] = 0.f;
          }
        }
        st_frag_lds<E>(sMt + 16 * wv * L::LT + 16 * nb, L::LT, acc, lane);
      }
    }
    f32x4 dU[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      dU[nb] = mma16<E>(sK + 16 * wv * L::LK, L::LK, sGt + 16 * nb * L::LK, L::LK, 0, DK, zero4(), lane);
    __syncthreads();

#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const f32x4 m = mma16<E>(sMt + 16 * wv * L::LT, L::LT, sOt + 16 * nb * L::LT, L::LT, k0M, kChunk, zero4(), lane);
      dU[nb] += g.scale * m;
      st_frag_t<E>(sDt + 16 * nb * L::LT + 16 * wv, L::LT, dU[nb], lane);
      st_frag_rows<E>(dut + (row0 + 16 * wv) * DV + v0 + 16 * nb, DV, dU[nb], lane, 16 * wv, n);
    }
    __syncthreads();

#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = wv + 4 * i, mb = t / NB, nb = t % NB;
      const f32x4 a = mma16<E>(sQt + 16 * mb * L::LT, L::LT, sOt + 16 * nb * L::LT, L::LT, 0, kChunk, zero4(), lane);
      const f32x4 b = mma16<E>(sWt + 16 * mb * L::LT, L::LT, sDt + 16 * nb * L::LT, L::LT, 0, kChunk, zero4(), lane);
      G[i] += g.scale * a - b;
    }
    __syncthreads();
  }
}

template <typename E, int DK, int DV>
static hipError_t scan_bwd_go(const Shape& s, const int* table, const void* q, const void* k,
                              const void* w, const void* d_o, void* dut, void* dstates,
                              hipStream_t st) {
  constexpr int TV = DV / 4;
  typedef ScanBwdLds<E, DK, DV, TV> L;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)scan_bwd_kernel<E, DK, DV, TV>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)L::bytes);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const int64_t blocks = (int64_t)s.n_seqs * s.H * (DV / TV);
  if (blocks < 1) return hipSuccess;
  prof_begin(st);
  hipLaunchKernelGGL((scan_bwd_kernel<E, DK, DV, TV>), dim3((unsigned)blocks), dim3(kThreads),
                     L::bytes, st, make_geom(s, table), (const E*)q, (const E*)k, (const E*)w,
                     (const E*)d_o, (E*)dut, (E*)dstates);
  hipError_t e = hipGetLastError();
  prof_end("scan_bwd", st);
  return e;
}

size_t lds_scan_bwd(Dt dt, int dk, int dv) {
  if (dt == Dt::BF16) {
    if (dk == 64 && dv == 64) return ScanBwdLds<__bf16, 64, 64, 16>::bytes;
    if (dk == 64 && dv == 128) return ScanBwdLds<__bf16, 64, 128, 32>::bytes;
    if (dk == 128 && dv == 64) return ScanBwdLds<__bf16, 128, 64, 16>::bytes;
    if (dk == 128 && dv == 128) return ScanBwdLds<__bf16, 128, 128, 32>::bytes;
    return 0;
  }
  if (dk == 64 && dv == 64) return ScanBwdLds<float, 64, 64, 16>::bytes;
  return 0;
}

hipError_t launch_scan_bwd(const Shape& s, const int* table, const void* q, const void* k,
                           const void* w, const void* d_o, void* dut, void* dstates,
                           hipStream_t st) {
  if (s.dt == Dt::BF16) {
    if (s.dk == 64 && s.dv == 64) return scan_bwd_go<__bf16, 64, 64>(s, table, q, k, w, d_o, dut, dstates, st);
    if (s.dk == 64 && s.dv == 128) return scan_bwd_go<__bf16, 64, 128>(s, table, q, k, w, d_o, dut, dstates, st);
    if (s.dk == 128 && s.dv == 64) return scan_bwd_go<__bf16, 128, 64>(s, table, q, k, w, d_o, dut, dstates, st);
    return scan_bwd_go<__bf16, 128, 128>(s, table, q, k, w, d_o, dut, dstates, st);
  }
  return scan_bwd_go<float, 64, 64>(s, table, q, k, w, d_o, dut, dstates, st);
}

}  // namespace efla

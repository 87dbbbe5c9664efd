// Inter-chunk state recurrence fused with the chunk output.
//
// Exact Flow Linear Attention summary page, section 3.3 (chunk-level recurrence and
// outputs). One workgroup walks the chunks of one (sequence, head) in order and owns a
// d_k x TV slice of the state, kept in fp32 MFMA accumulators for the whole sequence:
//   U~ = U - W S,   O = scale (Q S + tril(Q K^T) U~),   S <- S + K^T U~.
// The diagonal of tril is kept because token t reads the state after its own update.
// Optionally the incoming state of every chunk and U~ are written for the backward pass.
#include "efla_internal.hpp"

namespace efla {

template <typename E, int DK, int DV, int TV>
struct ScanFwdLds {
  static constexpr int LK = pitch<E>(DK), LT = pitch<E>(64), LU = pitch<E>(TV);
  static constexpr size_t oQ = 0;                               // Q      [64][LK]
  static constexpr size_t oK = oQ + 64 * LK * sizeof(E);        // K      [64][LK]
  static constexpr size_t oKt = oK + 64 * LK * sizeof(E);       // K^T    [DK][LT]
  static constexpr size_t oW = oKt + DK * LT * sizeof(E);       // W      [64][LK]
  static constexpr size_t oU = oW + 64 * LK * sizeof(E);        // U tile [64][LU]
  static constexpr size_t oM = oU + 64 * LU * sizeof(E);        // tril(QK^T) [64][LT]
  static constexpr size_t oSt = oM + 64 * LT * sizeof(E);       // S^T    [TV][LK]
  static constexpr size_t oUt = oSt + TV * LK * sizeof(E);      // U~^T   [TV][LT]
  static constexpr size_t bytes = oUt + TV * LT * sizeof(E);
};

template <typename E, int DK, int DV, int TV>
__global__ __launch_bounds__(kThreads) void scan_fwd_kernel(
    Geom g, const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ w,
    const E* __restrict__ u, E* __restrict__ o, E* __restrict__ ut, E* __restrict__ states) {
  typedef ScanFwdLds<E, DK, DV, TV> L;
  constexpr int NTILE = DV / TV;
  constexpr int NB = TV / 16;               // column blocks of the state slice
  constexpr int TPW = (DK / 16) * NB / 4;   // state tiles per wave
  static_assert(TPW >= 1 && ((DK / 16) * NB) % 4 == 0, "state tiles must split over 4 waves");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  E* sQ = (E*)(smem + L::oQ);
  E* sK = (E*)(smem + L::oK);
  E* sKt = (E*)(smem + L::oKt);
  E* sW = (E*)(smem + L::oW);
  E* sU = (E*)(smem + L::oU);
  E* sM = (E*)(smem + L::oM);
  E* sSt = (E*)(smem + L::oSt);
  E* sUt = (E*)(smem + L::oUt);

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int sh, tile;
  scan_block(blockIdx.x, g.n_seqs * g.H, NTILE, sh, tile);
  const int s = sh / g.H, h = sh % g.H;
  const SeqInfo si = seq_info(g, s);
  const int nchunks = seq_chunks(g, si);
  const int v0 = tile * TV;
  const int kM = round_up_kc<E>(16 * (wv + 1));  // row block wv of tril(.) needs cols < 16(wv+1)

  f32x4 S[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) S[i] = zero4();

  for (int c = 0; c < nchunks; ++c) {
    const int n = min(kChunk, si.len - c * kChunk);
    const int64_t row0 = (int64_t)(si.b * g.H + h) * g.T + si.bos + c * kChunk;
    g2s<E, DK>(sQ, L::LK, q + row0 * DK, DK, n, tid);
    g2s<E, DK>(sK, L::LK, k + row0 * DK, DK, n, tid);
    g2s_t<E, DK>(sKt, L::LT, k + row0 * DK, DK, n, tid);
    g2s<E, DK>(sW, L::LK, w + row0 * DK, DK, n, tid);
    g2s<E, TV>(sU, L::LU, u + row0 * DV + v0, DV, n, tid);
    E* gS = states ? states + ((int64_t)(si.slot0 + c) * g.H + h) * DK * DV : nullptr;
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = wv + 4 * i, mb = t / NB, nb = t % NB;
      st_frag_t<E>(sSt + 16 * nb * L::LK + 16 * mb, L::LK, S[i], lane);
      if (gS) st_frag_glb<E>(gS + (int64_t)16 * mb * DV + v0 + 16 * nb, DV, S[i], lane);
    }
    __syncthreads();

    // tril(Q K^T), row block wv; zero tiles inside the contraction range above the diagonal.
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      if (16 * nb < kM) {
        f32x4 acc = zero4();
        if (nb <= wv) {
          acc = mma16<E>(sQ + 16 * wv * L::LK, L::LK, sK + 16 * nb * L::LK, L::LK, 0, DK, acc, lane);
          if (nb == wv) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if ((lane & 15) > 4 * (lane >> 4) + i) acc[i] = 0.f;
          }
        }
        st_frag_lds<E>(sM + 16 * wv * L::LT + 16 * nb, L::LT, acc, lane);
      }
    }
    // U~ = U - W S and P = Q S for row block wv.
    f32x4 P[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const f32x4 ws = mma16<E>(sW + 16 * wv * L::LK, L::LK, sSt + 16 * nb * L::LK, L::LK, 0, DK, zero4(), lane);
      P[nb] = mma16<E>(sQ + 16 * wv * L::LK, L::LK, sSt + 16 * nb * L::LK, L::LK, 0, DK, zero4(), lane);
      f32x4 ud;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        ud[i] = to_f(sU[(16 * wv + 4 * (lane >> 4) + i) * L::LU + 16 * nb + (lane & 15)]) - ws[i];
      st_frag_t<E>(sUt + 16 * nb * L::LT + 16 * wv, L::LT, ud, lane);
      if (ut) st_frag_rows<E>(ut + (row0 + 16 * wv) * DV + v0 + 16 * nb, DV, ud, lane, 16 * wv, n);
    }
    __syncthreads();

    if (o) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        f32x4 acc = mma16<E>(sM + 16 * wv * L::LT, L::LT, sUt + 16 * nb * L::LT, L::LT, 0, kM, P[nb], lane);
        acc *= g.scale;
        st_frag_rows<E>(o + (row0 + 16 * wv) * DV + v0 + 16 * nb, DV, acc, lane, 16 * wv, n);
      }
    }
    // S += K^T U~
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = wv + 4 * i, mb = t / NB, nb = t % NB;
      S[i] = mma16<E>(sKt + 16 * mb * L::LT, L::LT, sUt + 16 * nb * L::LT, L::LT, 0, kChunk, S[i], lane);
    }
    __syncthreads();
  }
}

template <typename E, int DK, int DV>
static hipError_t scan_fwd_go(const Shape& s, const int* table, const void* q, const void* k,
                              const void* w, const void* u, void* o, void* ut, void* states,
                              hipStream_t st) {
  constexpr int TV = DV / 4;
  typedef ScanFwdLds<E, DK, DV, TV> L;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)scan_fwd_kernel<E, DK, DV, TV>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)L::bytes);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const int64_t blocks = (int64_t)s.n_seqs * s.H * (DV / TV);
  if (blocks < 1) return hipSuccess;
  prof_begin(st);
  hipLaunchKernelGGL((scan_fwd_kernel<E, DK, DV, TV>), dim3((unsigned)blocks), dim3(kThreads),
                     L::bytes, st, make_geom(s, table), (const E*)q, (const E*)k, (const E*)w,
                     (const E*)u, (E*)o, (E*)ut, (E*)states);
  hipError_t e = hipGetLastError();
  prof_end("scan_fwd", st);
  return e;
}

size_t lds_scan_fwd(Dt dt, int dk, int dv) {
  if (dt == Dt::BF16) {
    if (dk == 64 && dv == 64) return ScanFwdLds<__bf16, 64, 64, 16>::bytes;
    if (dk == 64 && dv == 128) return ScanFwdLds<__bf16, 64, 128, 32>::bytes;
    if (dk == 128 && dv == 64) return ScanFwdLds<__bf16, 128, 64, 16>::bytes;
    if (dk == 128 && dv == 128) return ScanFwdLds<__bf16, 128, 128, 32>::bytes;
    return 0;
  }
  if (dk == 64 && dv == 64) return ScanFwdLds<float, 64, 64, 16>::bytes;
  return 0;
}

hipError_t launch_scan_fwd(const Shape& s, const int* table, const void* q, const void* k,
                           const void* w, const void* u, void* o, void* ut, void* states,
                           hipStream_t st) {
  if (s.dt == Dt::BF16) {
    if (s.dk == 64 && s.dv == 64) return scan_fwd_go<__bf16, 64, 64>(s, table, q, k, w, u, o, ut, states, st);
    if (s.dk == 64 && s.dv == 128) return scan_fwd_go<__bf16, 64, 128>(s, table, q, k, w, u, o, ut, states, st);
    if (s.dk == 128 && s.dv == 64) return scan_fwd_go<__bf16, 128, 64>(s, table, q, k, w, u, o, ut, states, st);
    return scan_fwd_go<__bf16, 128, 128>(s, table, q, k, w, u, o, ut, states, st);
  }
  return scan_fwd_go<float, 64, 64>(s, table, q, k, w, u, o, ut, states, st);
}

}  // namespace efla

// Inter-chunk state recurrence fused with the chunk output.
//
// Exact Flow Linear Attention summary page, section 3.3 (chunk-level recurrence and
// outputs). One workgroup walks the chunks of one (sequence, head) in order and owns a
// d_k x TV slice of the state, kept transposed (S^T, TV x d_k) in fp32 MFMA accumulators
// for the whole sequence:
//   U~ = U - W S,   O = scale (Q S + M U~),   S^T <- S^T + U~^T K,
// with M = tril(Q K^T) from the UT kernel. The diagonal of tril is kept because token t
// reads the state after its own update.
//
// Latency hiding: each wave keeps the W, Q and M rows of its 16 tokens as MFMA A fragments
// in registers. Loads run two chunks ahead in two register stages (the loop is unrolled by
// two so the stages swap roles without copies); K is double-buffered in LDS. Products over
// the token or d_k index read LDS tiles k-major with the LDS transpose read (bf16). O and
// U~ leave through LDS staging as 16-byte stores.
#include "efla_internal.hpp"

namespace efla {

template <typename E, int DK, int DV, int TV>
struct ScanFwdLds {
  static constexpr int LK = pitch<E>(DK), LT = pitch<E>(64), LS = pitch<E>(TV);
  static constexpr size_t oK0 = 0;                              // K, even chunks [64][LK]
  static constexpr size_t oK1 = oK0 + 64 * LK * sizeof(E);      // K, odd chunks  [64][LK]
  static constexpr size_t oS = oK1 + 64 * LK * sizeof(E);       // S slice [DK][LS]
  static constexpr size_t oUt = oS + DK * LS * sizeof(E);       // U~^T    [TV][LT]
  static constexpr size_t oOs = oUt + TV * LT * sizeof(E);      // O staging  [64][LS]
  static constexpr size_t oUs = oOs + 64 * LS * sizeof(E);      // U~ staging [64][LS]
  static constexpr size_t bytes = oUs + 64 * LS * sizeof(E);
};

template <typename E, int DK, int TV>
struct ScanFwdStage {
  typedef typename Mma<E>::vec V;
  static constexpr int KS = DK / Mma<E>::KC, KM = kChunk / Mma<E>::KC, NB = TV / 16;
  static constexpr int KV = 64 * DK * (int)sizeof(E) / 16 / kThreads;
  V w[KS], q[KS], m[KM];
  E u[NB][4];
  u32x4 k[KV];
};

template <typename E, int DK, int DV, int TV>
__global__ __launch_bounds__(kThreads, 1) void scan_fwd_kernel(
    Geom g, const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ w,
    const E* __restrict__ u, const E* __restrict__ m, E* __restrict__ o, E* __restrict__ ut,
    E* __restrict__ states) {
  typedef ScanFwdLds<E, DK, DV, TV> L;
  typedef ScanFwdStage<E, DK, TV> St;
  typedef typename Mma<E>::vec V;
  constexpr int KC = Mma<E>::KC, KS = St::KS, KM = St::KM, NB = St::NB, KV = St::KV;
  constexpr int NTILE = DV / TV;
  constexpr int TPW = (DK / 16) * NB / 4;   // S^T tiles per wave
  constexpr int VE = 16 / (int)sizeof(E);
  static_assert(TPW >= 1 && ((DK / 16) * NB) % 4 == 0, "state tiles must split over 4 waves");
  static_assert(KV >= 1 && (64 * DK / VE) % kThreads == 0, "K tile must split over the threads");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  E* sK0 = (E*)(smem + L::oK0);
  E* sK1 = (E*)(smem + L::oK1);
  E* sS = (E*)(smem + L::oS);
  E* sUt = (E*)(smem + L::oUt);
  E* sOs = (E*)(smem + L::oOs);
  E* sUs = (E*)(smem + L::oUs);

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int sh, tile;
  scan_block(blockIdx.x, g.n_seqs * g.H, NTILE, sh, tile);
  const int s = sh / g.H, h = sh % g.H;
  const SeqInfo si = seq_info(g, s);
  const int nchunks = seq_chunks(g, si);
  const int v0 = tile * TV;
  const int rA = 16 * wv;                         // this wave's 16 token rows
  const int64_t base = (int64_t)(si.b * g.H + h) * g.T + si.bos;

  // Working registers of the current chunk.
  V wA[KS], qA[KS], mA[KM];
  E uA[NB][4];

  // Unconditional loads of chunk c (row indices clamped into the chunk); rows past the end
  // of the sequence are zeroed when the stage is committed, after the data has arrived.
  auto load_chunk = [&](int c, St& P) {
    c = min(c, nchunks - 1);
    const int n = min(kChunk, si.len - c * kChunk);
    const int64_t r0 = base + (int64_t)c * kChunk;
    const int ra = min(rA + (lane & 15), n - 1) - (lane & 15);   // row origin, clamped
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      P.w[ks] = frag_rm<E>(w + (r0 + ra) * DK + ks * KC, DK, lane);
      P.q[ks] = frag_rm<E>(q + (r0 + ra) * DK + ks * KC, DK, lane);
    }
    const E* mc = m + ((int64_t)(si.slot0 + c) * g.H + h) * kChunk * kChunk;
#pragma unroll
    for (int ks = 0; ks < KM; ++ks) P.m[ks] = frag_rm<E>(mc + rA * kChunk + ks * KC, kChunk, lane);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = min(rA + 4 * (lane >> 4) + i, n - 1);
        P.u[nb][i] = u[(r0 + r) * DV + v0 + 16 * nb + (lane & 15)];
      }
#pragma unroll
    for (int it = 0; it < KV; ++it) {
      const int i = it * kThreads + tid;
      const int r = min(i / (DK / VE), n - 1), cc = (i % (DK / VE)) * VE;
      P.k[it] = *(const u32x4*)(k + (r0 + r) * DK + cc);
    }
  };
  // Move stage P (chunk c) into the working registers and the LDS buffer sk.
  auto commit_chunk = [&](int c, const St& P, E* sk) {
    const int n = min(kChunk, si.len - c * kChunk);
    const bool rowok = rA + (lane & 15) < n;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      wA[ks] = keep_if_vec(P.w[ks], rowok);
      qA[ks] = keep_if_vec(P.q[ks], rowok);
    }
#pragma unroll
    for (int ks = 0; ks < KM; ++ks) mA[ks] = P.m[ks];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        uA[nb][i] = rA + 4 * (lane >> 4) + i < n ? P.u[nb][i] : to_e<E>(0.f);
#pragma unroll
    for (int it = 0; it < KV; ++it) {
      const int i = it * kThreads + tid;
      const int r = i / (DK / VE), cc = (i % (DK / VE)) * VE;
      *(u32x4*)(sk + r * L::LK + cc) = keep_if(P.k[it], r < n);
    }
  };

  f32x4 Sacc[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) Sacc[i] = zero4();

  // One chunk: issue the loads of chunk c + 2 into stage Pi, compute chunk c, then commit
  // stage Pc (chunk c + 1, loaded one step earlier).
  auto step = [&](int c, St& Pi, const St& Pc) {
    E* sKc = (c & 1) ? sK1 : sK0;
    E* sKn = (c & 1) ? sK0 : sK1;
    const int n = min(kChunk, si.len - c * kChunk);
    const int64_t r0 = base + (int64_t)c * kChunk;
#pragma unroll
    for (int i = 0; i < TPW; ++i) {  // stage S: S^T tiles written transposed give S [d][v]
      const int t = wv + 4 * i, vb = t % NB, db = t / NB;
      st_frag_t<E>(sS + 16 * db * L::LS + 16 * vb, L::LS, Sacc[i], lane);
    }
    load_chunk(c + 2, Pi);
    __syncthreads();

    if (states) {  // S_c [d][v0 : v0 + TV] of this slot, 16-byte stores
      E* gS = states + ((int64_t)(si.slot0 + c) * g.H + h) * DK * DV + v0;
      constexpr int VPR = TV / VE;
      for (int i = tid; i < DK * VPR; i += kThreads) {
        const int d = i / VPR, cc = (i % VPR) * VE;
        *(u32x4*)(gS + (int64_t)d * DV + cc) = *(const u32x4*)(sS + d * L::LS + cc);
      }
    }
    // U~ = U - W S and P = Q S for this wave's rows.
    f32x4 P[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      f32x4 ws = zero4(), p = zero4();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const V sb = frag_km<E>(sS + ks * KC * L::LS + 16 * nb, L::LS, lane);
        ws = Mma<E>::step(wA[ks], sb, ws);
        p = Mma<E>::step(qA[ks], sb, p);
      }
      P[nb] = p;
      f32x4 ud;
#pragma unroll
      for (int i = 0; i < 4; ++i) ud[i] = to_f(uA[nb][i]) - ws[i];
      st_frag_t<E>(sUt + 16 * nb * L::LT + rA, L::LT, ud, lane);
      if (ut) st_frag_lds<E>(sUs + rA * L::LS + 16 * nb, L::LS, ud, lane);
    }
    __syncthreads();

    if (o) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        f32x4 acc = P[nb];
#pragma unroll
        for (int ks = 0; ks < KM; ++ks)
          acc = Mma<E>::step(mA[ks], frag_rm<E>(sUt + 16 * nb * L::LT + ks * KC, L::LT, lane), acc);
        acc *= g.scale;
        st_frag_lds<E>(sOs + rA * L::LS + 16 * nb, L::LS, acc, lane);
      }
    }
    if (ut) s2g<E, TV>(ut + r0 * DV + v0, DV, sUs, L::LS, n, tid);
    // S^T += U~^T K
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = wv + 4 * i, vb = t % NB, db = t / NB;
      Sacc[i] = mma<E, false, true>(sUt + 16 * vb * L::LT, L::LT, sKc + 16 * db, L::LK, 0, kChunk,
                                    Sacc[i], lane);
    }
    if (c + 1 < nchunks) commit_chunk(c + 1, Pc, sKn);
    if (o) {
      __syncthreads();
      s2g<E, TV>(o + r0 * DV + v0, DV, sOs, L::LS, n, tid);
    }
  };

  St P1, P2;
  if (nchunks > 0) {
    load_chunk(0, P1);
    commit_chunk(0, P1, sK0);
    load_chunk(1, P1);
  }
  for (int c = 0; c < nchunks; c += 2) {
    step(c, P2, P1);
    if (c + 1 < nchunks) step(c + 1, P1, P2);
  }
}

template <typename E, int DK, int DV, int TV>
static hipError_t scan_fwd_go(const Shape& s, const int* table, const void* q, const void* k,
                              const void* w, const void* u, const void* m, void* o, void* ut,
                              void* states, hipStream_t st) {
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
                     (const E*)u, (const E*)m, (E*)o, (E*)ut, (E*)states);
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
                           const void* w, const void* u, const void* m, void* o, void* ut,
                           void* states, hipStream_t st) {
#define EFLA_SF(E_, DK_, DV_, TV_) \
  return scan_fwd_go<E_, DK_, DV_, TV_>(s, table, q, k, w, u, m, o, ut, states, st)
  if (s.dt == Dt::BF16) {
    if (s.dk == 64 && s.dv == 64) EFLA_SF(__bf16, 64, 64, 16);
    if (s.dk == 128 && s.dv == 64) EFLA_SF(__bf16, 128, 64, 16);
    if (scan_tile(s) == 16) {
      if (s.dk == 64) EFLA_SF(__bf16, 64, 128, 16);
      EFLA_SF(__bf16, 128, 128, 16);
    }
    if (s.dk == 64) EFLA_SF(__bf16, 64, 128, 32);
    EFLA_SF(__bf16, 128, 128, 32);
  }
  EFLA_SF(float, 64, 64, 16);
#undef EFLA_SF
}

}  // namespace efla

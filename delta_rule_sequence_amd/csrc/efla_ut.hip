// UT transform of one 64-token chunk per workgroup, plus the chunk's causal score block.
//
// Exact Flow Linear Attention summary page, section 3.3 (chunkwise form with the UT
// transform; the WY/UT representation is the DeltaNet prior art of the fifth page):
//   alpha_i = exact-flow step of token i,  A = strictly_lower(diag(alpha) K K^T),
//   X = (I + A)^{-1},  T = X diag(alpha),  W = T K,  U = T V,   M = tril(Q K^T).
// K K^T, Q K^T, T K and T V are MFMA contractions (products over the token index read the
// row-major K and V tiles k-major); the unit lower triangular inverse is a blocked forward
// substitution in fp32 in LDS. Padded rows of a tail chunk read as zero (their beta is zero,
// so alpha = 0 and they do not touch the valid rows). Every output is optional: W and U (w, u;
// V is read only for them), M (q may be null), X, and the per-token column scales of the two
// factors, alpha~ = alpha (gated: alpha e^{c}) and b (gated). The bf16 forward keeps only X and
// the scales: its scans form U~ = U - W S = X (diag(b) V - diag(alpha~) K S) themselves, which
// moves less data than W and U (X is a quarter of W's size at d = 128), and its forward scan
// forms M from the Q and K tiles it stages anyway, so this kernel reads no Q there (it still
// forms M where no output scan follows: the backward's recomputed forward); X also serves the
// backward pass, which then needs no inverse of its own.
//
// Gated EFLA (GT): with c_t the running sum of the log-decays inside the chunk,
//   A_ts = alpha_t e^{c_t - c_s} k_t . k_s (s < t),  X = (I + A)^{-1},
//   W = X diag(alpha e^{c}) K,  U = X diag(b) V,  M_ts = e^{c_t - c_s} q_t . k_s (s <= t),
// b the gated input coefficient; the c_t are written out for the scan.
#include "efla_internal.hpp"

namespace efla {

// WU: the launch writes W and U (V is read for U). MO: it may form M (q, mout). Without W and U
// (the bf16 factor form) there is no V tile; without M as well, nothing reads K once A is formed,
// so X takes K's place (KX). A bf16 workgroup's LDS then admits three (four with KX) workgroups
// per compute unit.
// Workgroups per compute unit that the LDS admits (the kernel's launch bounds match).
template <typename E> constexpr int ut_per_cu(bool wu, bool mo) {
  return sizeof(E) == 2 && !wu ? (mo ? 3 : 4) : 2;
}

template <typename E, int DK, int DV, bool GT = false, bool WU = true, bool MO = true>
struct UtFwdLds {
  static constexpr bool KX = !WU && !MO;
  // bf16: K and V rows padded by 32 bytes rather than 16 (fewer LDS bank conflicts; measured
  // slightly faster)
  static constexpr int PADE = sizeof(E) == 2 ? 16 / (int)sizeof(E) : 0;
  static constexpr int LK = pitch<E>(DK) + PADE, LT = pitch<E>(64), LV = pitch<E>(DV) + PADE, LF = kPitchF;
  static constexpr size_t TKB = 64 * LK * sizeof(E), TFB = 64 * LF * 4;
  static constexpr size_t oK = 0;                                   // K        [64][LK]
  static constexpr size_t oV = KX && TFB > TKB ? TFB : TKB;         // V        [64][LV] (WU)
  static constexpr size_t oA = oV + (WU ? 64 * LV * sizeof(E) : 0); // A (fp32) [64][LF]; later T
  static constexpr size_t oX = KX ? oK : oA + TFB;                  // X (fp32) [64][LF]; M staging first
  static constexpr size_t oAl = (KX ? oA : oX) + TFB;               // alpha    [64]
  static constexpr size_t oLm = oAl + 64 * 4;                       // lambda   [64]
  static constexpr size_t oBl = oLm + 64 * 4;                       // b, c     [64] each (GT)
  static constexpr size_t oCm = oBl + 64 * 4;
  static constexpr size_t oT2 = oCm + 64 * 4;                       // X diag(b) [64][LT] (GT, WU)
  static constexpr size_t bytes = GT ? (WU ? oT2 + 64 * LT * sizeof(E) : oCm + 64 * 4) : oLm + 64 * 4;
  static constexpr int PER_CU = ut_per_cu<E>(WU, MO);
  static_assert(WU || sizeof(E) == 2, "only the bf16 factor form runs without W and U");
  static_assert(MO || !WU, "W/U launches may form M");
  static_assert(64 * LT * sizeof(E) <= 64 * LF * 4, "T and M must fit in an fp32 work matrix");
  static_assert(sizeof(E) == 4 || PER_CU * bytes <= 160 * 1024, "bf16: workgroups per compute unit");
};

// Persistent: the workgroup walks units u = blockIdx.x, blockIdx.x + gridDim.x, ...; the
// next unit's K, V and Q rows are requested into registers while the current one computes.
template <typename E, int DK, int DV, bool GT, bool WU, bool MO>
__global__ __launch_bounds__(kThreads, (ut_per_cu<E>(WU, MO))) void ut_fwd_kernel(
    Geom g, const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const E* __restrict__ beta, const E* __restrict__ gate, E* __restrict__ w, E* __restrict__ u,
    E* __restrict__ mout, E* __restrict__ xout, float* __restrict__ cum, float* __restrict__ ca,
    float* __restrict__ cb) {
  typedef UtFwdLds<E, DK, DV, GT, WU, MO> L;
  typedef typename Mma<E>::vec Vv;
  if constexpr (!MO) mout = nullptr;  // launched with M only where MO
  constexpr int KC = Mma<E>::KC, KS = DK / KC;
  constexpr int VE = 16 / (int)sizeof(E);
  constexpr int VPR = DK / VE;                  // 16-byte vectors per K row
  constexpr int KIT = 64 * VPR / kThreads;      // K vectors per thread
  constexpr int VIT = 64 * DV / VE / kThreads;  // V vectors per thread
  static_assert(VPR <= 64 && (64 % VPR) == 0 && KIT >= 1 && VIT >= 1, "row split");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  lds_poison(smem);
  E* sK = (E*)(smem + L::oK);
  E* sV = (E*)(smem + L::oV);
  float* sA = (float*)(smem + L::oA);
  E* sT = (E*)(smem + L::oA);
  float* sX = (float*)(smem + L::oX);
  E* sM = (E*)(smem + L::oX);
  float* sAl = (float*)(smem + L::oAl);
  float* sLm = (float*)(smem + L::oLm);
  float* sBl = (float*)(smem + L::oBl);
  float* sCm = (float*)(smem + L::oCm);
  E* sT2 = (E*)(smem + L::oT2);

  int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rA = 16 * wv;
  const int nu = used_slots(g) * g.H;
  int un = blockIdx.x;
  if (un >= nu) return;

  u32x4 kR[KIT], vR[VIT];
  float bN = 0.f, aN = 0.f;  // beta and (gated) log-decay of token `lane` of the requested chunk
  float bC = 0.f, aC = 0.f;  // the same for the chunk in LDS
  Vv qN[KS], qA[KS];
  // Requests for the next chunk's inputs, spread over the current one. Every request is
  // unconditional (row indices are clamped; after the last chunk, one row of the first), and inside
  // the loop the base pointers are opaque copies made each iteration: loads through a read-only
  // kernel argument may be sunk by the compiler to just before the back edge.
  const E *kL = k, *vL = v, *qL = q, *bL = beta, *aL = gate;
  auto issue_k = [&](const ChunkUnit& c) {
#pragma unroll
    for (int it = 0; it < KIT; ++it) {
      const int i = it * kThreads + tid;
      const int r = min(i / VPR, c.n - 1), cc = (i % VPR) * VE;
      kR[it] = *at_byte<u32x4>(kL + c.row0 * DK, (unsigned)((r * DK + cc) * (int)sizeof(E)));
    }
    bN = to_f(bL[c.row0 + min(lane, c.n - 1)]);  // token = lane
    if constexpr (GT) aN = to_f(aL[c.row0 + min(lane, c.n - 1)]);
  };
  auto issue_v = [&](const ChunkUnit& c) {
    if (!WU) return;  // V feeds U = T V only
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      const int i = it * kThreads + tid;
      const int r = min(i / (DV / VE), c.n - 1), cc = (i % (DV / VE)) * VE;
      vR[it] = *(const u32x4*)(vL + (c.row0 + r) * DV + cc);
    }
  };
  auto issue_q = [&](const ChunkUnit& c) {  // this wave's Q rows as A fragments (for M)
    if (!mout) return;
    const int ra = min(rA + (lane & 15), c.n - 1) - (lane & 15);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qN[ks] = frag_rm<E>(qL + (c.row0 + ra) * DK + ks * KC, DK, lane);
  };

  // K and V land in LDS; ||k||^2 is reduced from the K vectors (VPR consecutive threads per
  // row) into LDS (the coefficients follow after the next barrier, one token per lane). Done
  // before the loop for the first chunk and at the end of each iteration for the next one, after
  // that iteration's stores, so the compiler waits for the loads alone there.
  auto land = [&](const ChunkUnit& cu) {
    const int n = cu.n;
#pragma unroll
    for (int it = 0; it < KIT; ++it) {
      const int i = it * kThreads + tid;
      const int r = i / VPR, c = (i % VPR) * VE;
      const u32x4 xr = keep_if(kR[it], r < n);
      *(u32x4*)(sK + r * L::LK + c) = xr;
      const Vv x = __builtin_bit_cast(Vv, xr);
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < VE; ++e) acc = fmaf(to_f(x[e]), to_f(x[e]), acc);
      acc = group_sum<VPR>(acc);
      if (i % VPR == 0) sLm[r] = r < n ? acc : 0.f;
    }
    bC = bN;
    if constexpr (GT) aC = aN;
    if constexpr (WU) {
#pragma unroll
      for (int it = 0; it < VIT; ++it) {
        const int i = it * kThreads + tid;
        const int r = i / (DV / VE), c = (i % (DV / VE)) * VE;
        *(u32x4*)(sV + r * L::LV + c) = keep_if(vR[it], r < n);
      }
    }
    if (mout) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qA[ks] = keep_if_vec(qN[ks], rA + (lane & 15) < n);
    }
    if constexpr (GT) {  // c_t: inclusive running sum of the log-decays (padded rows add 0)
      if (wv == 0) {
        float cs = lane < n ? aN : 0.f;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const float t = __shfl_up(cs, off);
          if (lane >= off) cs += t;
        }
        sCm[lane] = cs;
        if (cum) cum[cu.sh * 64 + lane] = cs;
      }
    }
  };

  ChunkUnit cur = chunk_unit(g, un);
  issue_k(cur);
  issue_v(cur);
  issue_q(cur);
  land(cur);
  for (;;) {
    // Per-lane addresses derive from tid: opaque once per unit so that they are not all
    // hoisted out of the loop (they would hold registers through every step).
    asm volatile("" : "+v"(tid));
    lane = tid & 63;
    kL = opaque_global(k);
    vL = opaque_global(v);
    qL = opaque_global(q);
    bL = opaque_global(beta);
    if constexpr (GT) aL = opaque_global(gate);
    const int n = cur.n;
    const int64_t row0 = cur.row0;
    __syncthreads();
    const int unx = un + (int)gridDim.x;
    const bool more = unx < nu;
    // After the last chunk the requests still go out (every load is unconditional), to one
    // row of the first chunk, which all workgroups then share in L2.
    ChunkUnit nxt = chunk_unit(g, more ? unx : 0);
    if (!more) nxt.n = 1;
    // Flow coefficients, one token per lane, computed by every wave (each needs alpha of the rows
    // it scales; one pass of the coefficient code instead of one per K vector group). Wave 0
    // keeps them in LDS for the later steps. Padded tokens have beta = 0, so alpha = b = 0.
    float al_l;
    {
      const float lam = sLm[lane];
      al_l = flow_coef(lane < n ? bC : 0.f, lam, g.euler).alpha;
      if (wv == 0) {
        sAl[lane] = al_l;
        if constexpr (GT) sBl[lane] = lane < n ? gated_input_coef(bC, lam, aC, g.euler) : 0.f;
      }
    }
    issue_k(nxt);

    // A = strictly_lower(diag(alpha) K K^T) and M = tril(Q K^T), lower blocks only (the
    // inverse never reads A above the diagonal). With M, wave wv takes A's row block 3 - wv and
    // M's row block wv: five block products each; without M the ten blocks of A are dealt 3, 3,
    // 2, 2. Both are formed transposed (operands swapped), so a lane holds four consecutive
    // columns of one row and stores them at once.
    {
      const int c4 = 4 * (lane >> 4);
      auto ablk = [&](int ra, int nb) {
        const int rowa = 16 * ra + (lane & 15);
        const float ala = __shfl(al_l, rowa);
        const float cra = GT ? sCm[rowa] : 0.f;
        f32x4 acc = mma<E, false, false>(sK + 16 * nb * L::LK, L::LK, sK + 16 * ra * L::LK, L::LK, 0, DK, zero4(), lane);
        f32x4 av;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int col = 16 * nb + c4 + i;
          const float dec = GT ? exp_decay(cra - sCm[col]) : 1.f;  // e^{c_t - c_s}, used for s < t
          av[i] = rowa > col ? ala * dec * acc[i] : 0.f;
        }
        *(f32x4*)(sA + rowa * L::LF + 16 * nb + c4) = av;
      };
      if constexpr (MO) {
        const int ra = 3 - wv;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          if (nb <= ra) ablk(ra, nb);
      } else {
        switch (wv) {
          case 0: ablk(3, 0); ablk(3, 1); ablk(3, 2); break;
          case 1: ablk(3, 3); ablk(2, 0); ablk(2, 1); break;
          case 2: ablk(2, 2); ablk(1, 0); break;
          default: ablk(1, 1); ablk(0, 0); break;
        }
      }
    }
    if (mout) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        f32x4 m = zero4();
        if (nb <= wv) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            m = Mma<E>::step(frag_rm<E>(sK + 16 * nb * L::LK + ks * KC, L::LK, lane), qA[ks], m);
          if (nb == wv) {  // keep columns <= row
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (4 * (lane >> 4) + i > (lane & 15)) m[i] = 0.f;
          }
          if constexpr (GT) {
            const float cr = sCm[rA + (lane & 15)];
#pragma unroll
            for (int i = 0; i < 4; ++i) {  // e^{c_t - c_s} for s <= t (above, the factor may overflow)
              const int col = 16 * nb + 4 * (lane >> 4) + i;
              m[i] = col <= rA + (lane & 15) ? m[i] * exp_decay(cr - sCm[col]) : 0.f;
            }
          }
        }
        st_frag_t<E>(sM + rA * L::LT + 16 * nb, L::LT, m, lane);
      }
    }
    __syncthreads();
    if (mout) {  // M [64][64] of this (chunk, head), 16-byte stores
      E* gm = mout + cur.sh * 64 * 64;
      s2g<E, 64>(gm, 64, sM, L::LT, kChunk, tid);
    }
    issue_v(nxt);
    if constexpr (!L::KX) __syncthreads();  // M's staging (X's region) is copied out first
    invert_unit_lower64(sA, sX, tid);
    issue_q(nxt);

    // Column scales of the factors for the scans: alpha~ = alpha (gated alpha e^{c}), b.
    if (ca && tid < 64) {
      ca[cur.sh * 64 + tid] = GT ? sAl[tid] * exp_decay(sCm[tid]) : sAl[tid];
      if constexpr (GT) cb[cur.sh * 64 + tid] = sBl[tid];
    }
    // T = X diag(alpha), written over A (A is no longer needed); X to global memory.
    {
      E* gx = xout ? xout + cur.sh * 64 * 64 : nullptr;
#pragma unroll
      for (int it = 0; it < 2; ++it) {  // 8 consecutive elements of one row per thread
        const int i = it * kThreads + tid;
        const int r = i >> 3, c = (i & 7) * 8;
        // blocks above the diagonal are zero (the inverse leaves them unwritten)
        const bool up = (c >> 4) > (r >> 4);
        f32x4 x0 = *(const f32x4*)(sX + r * L::LF + c);
        f32x4 x1 = *(const f32x4*)(sX + r * L::LF + c + 4);
        if (up) x0 = x1 = zero4();
        f32x4 a0 = *(const f32x4*)(sAl + c), a1 = *(const f32x4*)(sAl + c + 4);
        f32x4 b0 = a0, b1 = a1;  // column scales of the U factor
        if constexpr (GT) {      // W factor X diag(alpha e^{c}), U factor X diag(b)
          const f32x4 c0 = *(const f32x4*)(sCm + c), c1 = *(const f32x4*)(sCm + c + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            a0[e] *= exp_decay(c0[e]);
            a1[e] *= exp_decay(c1[e]);
          }
          b0 = *(const f32x4*)(sBl + c);
          b1 = *(const f32x4*)(sBl + c + 4);
        }
        if constexpr (sizeof(E) == 2) {
          bf16x8 xe, te, tu;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            xe[e] = (__bf16)x0[e];
            xe[e + 4] = (__bf16)x1[e];
            te[e] = (__bf16)(x0[e] * a0[e]);
            te[e + 4] = (__bf16)(x1[e] * a1[e]);
            tu[e] = (__bf16)(x0[e] * b0[e]);
            tu[e + 4] = (__bf16)(x1[e] * b1[e]);
          }
          if (WU) {
            *(bf16x8*)(sT + r * L::LT + c) = te;
            if constexpr (GT) *(bf16x8*)(sT2 + r * L::LT + c) = tu;
          }
          if (gx) *at_byte<bf16x8>(gx, (unsigned)((r * 64 + c) * (int)sizeof(E))) = xe;
        } else {
          if (WU) {
            *(f32x4*)(sT + r * L::LT + c) = x0 * a0;
            *(f32x4*)(sT + r * L::LT + c + 4) = x1 * a1;
            if constexpr (GT) {
              *(f32x4*)(sT2 + r * L::LT + c) = x0 * b0;
              *(f32x4*)(sT2 + r * L::LT + c + 4) = x1 * b1;
            }
          }
          if (gx) {
            *(f32x4*)(gx + r * 64 + c) = x0;
            *(f32x4*)(gx + r * 64 + c + 4) = x1;
          }
        }
      }
    }
    __syncthreads();

    if constexpr (WU) {  // W and U: every thread takes this branch, so the barriers inside match
      // W = T K, U = T V. Wave wv owns a quarter of the columns of each over all four row
      // blocks (equal work per wave); T is lower triangular, so row blocks 0-1 need columns
      // < 32 and row blocks 2-3 all 64. Formed transposed for row-layout stores.
      constexpr int CW = DK / 64, CU = DV / 64;  // 16-column tiles per wave
      f32x4 Wf[4][CW], Uf[4][CU];
      {
        f32x4 (&w01)[2][CW] = *reinterpret_cast<f32x4(*)[2][CW]>(&Wf[0]);
        f32x4 (&w23)[2][CW] = *reinterpret_cast<f32x4(*)[2][CW]>(&Wf[2]);
        f32x4 (&u01)[2][CU] = *reinterpret_cast<f32x4(*)[2][CU]>(&Uf[0]);
        f32x4 (&u23)[2][CU] = *reinterpret_cast<f32x4(*)[2][CU]>(&Uf[2]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int j = 0; j < CW; ++j) Wf[i][j] = zero4();
#pragma unroll
          for (int j = 0; j < CU; ++j) Uf[i][j] = zero4();
        }
        const int k01 = round_up_kc<E>(32);
        mma_blk<E, false, true, 2, CW, kChunk, true>(sT, L::LT, sK + 16 * CW * wv, L::LK, 0, k01, w01, lane);
        mma_blk<E, false, true, 2, CW, kChunk, true>(sT + 32 * L::LT, L::LT, sK + 16 * CW * wv, L::LK, 0, kChunk, w23, lane);
        const E* tU = GT ? sT2 : sT;
        mma_blk<E, false, true, 2, CU, kChunk, true>(tU, L::LT, sV + 16 * CU * wv, L::LV, 0, k01, u01, lane);
        mma_blk<E, false, true, 2, CU, kChunk, true>(tU + 32 * L::LT, L::LT, sV + 16 * CU * wv, L::LV, 0, kChunk, u23, lane);
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < CW; ++j) st_frag_t<E>(sK + 16 * i * L::LK + 16 * (CW * wv + j), L::LK, Wf[i][j], lane);
#pragma unroll
        for (int j = 0; j < CU; ++j) st_frag_t<E>(sV + 16 * i * L::LV + 16 * (CU * wv + j), L::LV, Uf[i][j], lane);
      }
      __syncthreads();
      s2g<E, DK>(w + row0 * DK, DK, sK, L::LK, n, tid);
      s2g<E, DV>(u + row0 * DV, DV, sV, L::LV, n, tid);
    }
    if (!more) break;
    if constexpr (WU) __syncthreads();  // the copies out of sK and sV are done before the next chunk lands
    land(nxt);
    un = unx;
    cur = nxt;
  }
}

template <typename E, int DK, int DV, bool GT, bool WU, bool MO>
static hipError_t ut_go(const Shape& s, const int* table, const void* q, const void* k,
                        const void* v, const void* beta, const void* gate, void* w, void* u,
                        void* m, void* x, float* cum, float* ca, float* cb, hipStream_t st) {
  typedef UtFwdLds<E, DK, DV, GT, WU, MO> L;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)ut_fwd_kernel<E, DK, DV, GT, WU, MO>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)L::bytes);
    if (e != hipSuccess) return e;
    attr = true;
  }
  // Persistent: L::PER_CU workgroups per compute unit walk the chunks.
  const int64_t units = s.slots * s.H;
  if (units < 1) return hipSuccess;
  const int64_t slots = (int64_t)L::PER_CU * cu_count();
  const int64_t blocks = units < slots ? units : slots;
  prof_begin(st);
  hipLaunchKernelGGL((ut_fwd_kernel<E, DK, DV, GT, WU, MO>), dim3((unsigned)blocks), dim3(kThreads), L::bytes,
                     st, make_geom(s, table), (const E*)q, (const E*)k, (const E*)v,
                     (const E*)beta, (const E*)gate, (E*)w, (E*)u, (E*)m, (E*)x, cum, ca, cb);
  hipError_t e = hipGetLastError();
  prof_end(GT ? "ut_fwd_gated" : "ut_fwd", st);
  return e;
}

// W and U are written together (both or neither); without them the kernel reads no V, and
// without M either it keeps X in K's place.
template <typename E, int DK, int DV, bool GT>
static hipError_t ut_gate(const Shape& s, const int* table, const void* q, const void* k,
                          const void* v, const void* beta, const void* gate, void* w, void* u,
                          void* m, void* x, float* cum, float* ca, float* cb, hipStream_t st) {
  if (!w != !u) return hipErrorInvalidValue;
  if (w) return ut_go<E, DK, DV, GT, true, true>(s, table, q, k, v, beta, gate, w, u, m, x, cum, ca, cb, st);
  if constexpr (sizeof(E) == 2) {  // the factor form (bf16) is the only caller without W and U
    if (m) return ut_go<E, DK, DV, GT, false, true>(s, table, q, k, v, beta, gate, w, u, m, x, cum, ca, cb, st);
    return ut_go<E, DK, DV, GT, false, false>(s, table, q, k, v, beta, gate, w, u, m, x, cum, ca, cb, st);
  }
  return hipErrorInvalidValue;
}

template <typename E, int DK, int DV>
static hipError_t ut_dispatch(const Shape& s, const int* table, const void* q, const void* k,
                              const void* v, const void* beta, const void* gate, void* w,
                              void* u, void* m, void* x, float* cum, float* ca, float* cb,
                              hipStream_t st) {
  if (gate) return ut_gate<E, DK, DV, true>(s, table, q, k, v, beta, gate, w, u, m, x, cum, ca, cb, st);
  return ut_gate<E, DK, DV, false>(s, table, q, k, v, beta, gate, w, u, m, x, cum, ca, cb, st);
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

hipError_t launch_ut_fwd(const Shape& s, const int* table, const void* q, const void* k,
                         const void* v, const void* beta, const void* gate, void* w, void* u,
                         void* m, void* x, float* cum, float* ca, float* cb, hipStream_t st) {
#define EFLA_UT(E_, DK_, DV_) \
  return ut_dispatch<E_, DK_, DV_>(s, table, q, k, v, beta, gate, w, u, m, x, cum, ca, cb, st)
  if (s.dt == Dt::BF16) {
    if (s.dk == 64 && s.dv == 64) EFLA_UT(__bf16, 64, 64);
    if (s.dk == 64 && s.dv == 128) EFLA_UT(__bf16, 64, 128);
    if (s.dk == 128 && s.dv == 64) EFLA_UT(__bf16, 128, 64);
    EFLA_UT(__bf16, 128, 128);
  }
  EFLA_UT(float, 64, 64);
#undef EFLA_UT
}

}  // namespace efla

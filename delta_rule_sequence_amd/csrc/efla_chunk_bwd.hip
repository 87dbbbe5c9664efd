// Chunk-parallel gradients of the backward pass: one 64-token chunk of one head per
// workgroup of eight wavefronts.
//
// Reverse-mode differentiation of the chunk form of section 3.3 (Exact Flow Linear
// Attention summary page) and of the exact-flow step of section 3.2, given for the chunk:
// S (incoming state), G (gradient of the outgoing state), U~ and dU~ (from the scans) and
// X = (I + A)^{-1} (saved by the forward UT kernel).
//   dM  = scale tril(dO U~^T)                 dQ = scale dO S^T + dM K
//   dK  = dM^T Q + U~ G^T                     dW = -dU~ S^T,  dU = dU~
// UT transform W = T K, U = T V, T = X diag(alpha), A = strictly_lower(diag(alpha) K K^T):
//   dT = dW K^T + dU V^T,  dK += T^T dW,  dV = T^T dU,
//   dalpha_j += sum_i dT_ij X_ij,  dA = -X^T (dT diag(alpha)) X^T (strictly lower),
//   dalpha_i += sum_j dA_ij (k_i . k_j),  dK += (dG + dG^T) K with dG = diag(alpha) dA.
// Exact-flow step alpha = (1 - e^{-beta lambda}) / lambda, lambda = ||k||^2:
//   dbeta = dalpha e^{-beta lambda},  dk += 2 k dalpha beta^2 phi'(beta lambda).
//
// Every input tile is requested from HBM at the start (held in registers until it lands in
// LDS), so the workgroup pays the memory latency once. S and G are only ever read as
// row-major MFMA operands and go straight from global memory into registers. Products over
// the token index read their row-major LDS tiles k-major (LDS transpose reads for bf16).
// Each wave computes 2x2 (or 2x1) blocks of 16x16 so that every operand fragment it reads
// from LDS feeds two MFMAs: LDS bandwidth, not the matrix cores, bounds the arithmetic.
// Products that end up in LDS row-major are formed transposed (operands swapped), so each
// lane holds four consecutive columns of one row and stores them with one vector write.
// Seven barrier-separated steps:
//   1 loads land; 2 dW, scale dO S^T, U~ G^T, dM, coefficients;
//   3 dT (-> dalpha, dX), T^T dU, T^T dW, dM K, dM^T Q;
//   4 Y = dX X^T;  5 dA = -X^T Y (-> dalpha, H);  6 H K and the outputs.
//
// Gated EFLA (GT): with c the running log-decay sums of the chunk (saved by the forward),
// Gamma = e^c, r = e^{c_last - c}, D_ts = e^{c_t - c_s} and P = tril(Q K^T) * D (formed again
// from the Q and K tiles in LDS, beside dM): dQ's state part is scale diag(Gamma) dO S^T, dK's is diag(r) U~ G^T, dM becomes
// dP * D, the UT factors are T_w = X diag(alpha Gamma) and T_u = X diag(b) (dT split into
// dW K^T and dU V^T), A carries D. Every e^c factor also adds to the log-decay gradient dc
// (accumulated per token in LDS), which a reverse running sum over the chunk turns into the
// gate gradient, plus db db/da. Each contribution to dc has its own LDS slot (no atomics), and
// the slots are summed in a fixed order, so the gate gradient is deterministic.
#include "efla_internal.hpp"

namespace efla {

constexpr int kBwdThreads = 512;

template <typename E, int DK, int DV, bool GT = false>
struct ChunkBwdLds {
  // bf16: d-wide rows padded by 32 bytes rather than 16 (fewer LDS bank conflicts in this
  // kernel's mix of row-major and transposed reads; measured 2% faster at d = 128)
  static constexpr int PADE = sizeof(E) == 2 ? 16 / (int)sizeof(E) : 0;
  static constexpr int LK = pitch<E>(DK) + PADE, LV = pitch<E>(DV) + PADE, LT = pitch<E>(64);
  static constexpr size_t TK = 64 * LK * sizeof(E), TV = 64 * LV * sizeof(E),
                          TT = 64 * LT * sizeof(E);
  static constexpr size_t oK = 0;                // K   [64][LK]
  static constexpr size_t oQ = oK + TK;          // Q;   dQ staging at the end
  static constexpr size_t oW = oQ + TK;          // dW;  dK staging at the end
  static constexpr size_t oDU = oW + TK;         // dU~ [64][LV]; dV staging at the end
  static constexpr size_t oDO = oDU + TV;        // dO;  then dX [64][LT]
  static constexpr size_t oU = oDO + TV;         // U~;  then Y  [64][LT]
  static constexpr size_t oV = oU + TV;          // V;   then H  [64][LT]
  static constexpr size_t oX = oV + TV;          // X   [64][LT]
  static constexpr size_t oM = oX + TT;          // dM  [64][LT]
  static constexpr size_t oC = oM + TT;          // lambda, alpha, e^-x, dalpha/dlam [64]
  static constexpr size_t oP = oC + 4 * 64 * 4;  // dalpha partials [64][8]
  // gated only: c, b, db/dbeta, db/dlam, db/da [64]; dc partials [64][kDcSlots] + <G, S>
  // partials [4]; db column-sum partials [64][4]
  static constexpr int kDcSlots = 20;
  static constexpr size_t oGc = oP + 8 * 64 * 4;
  static constexpr size_t oDc = oGc + 5 * 64 * 4;
  static constexpr size_t oDb = oDc + (64 * kDcSlots + 4) * 4;
  static constexpr size_t bytes = GT ? oDb + 4 * 64 * 4 : oP + 8 * 64 * 4;
  static_assert(TT <= TV, "64x64 work tiles reuse d_v-wide regions");
};

// A [64][COLS] tile on its way from global memory to LDS: rows >= n are clamped on load
// (never out of the chunk's memory) and written as zero.
template <typename E, int COLS>
struct TileRegs {
  static constexpr int VE = 16 / (int)sizeof(E), VPR = COLS / VE, TOT = kChunk * VPR;
  static constexpr int IT = (TOT + kBwdThreads - 1) / kBwdThreads;
  static_assert(TOT % kBwdThreads == 0, "tile split");
  u32x4 v[IT];
  EFLA_DEV void load(const E* __restrict__ g, int n, int tid) {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int i = it * kBwdThreads + tid;
      const int r = min(i / VPR, n - 1), c = (i % VPR) * VE;
      v[it] = *at_byte<u32x4>(g, (unsigned)(r * COLS + c) * (unsigned)sizeof(E));
    }
  }
  EFLA_DEV void store(E* s, int ld, int n, int tid) const {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int i = it * kBwdThreads + tid;
      const int r = i / VPR, c = (i % VPR) * VE;
      *(u32x4*)(s + r * ld + c) = keep_if(v[it], r < n);
    }
  }
};

// Zero a 16x16 block above the diagonal (nb > rb) and, on the diagonal (nb == rb), the
// entries above it (keep_diag) or on and above it.
EFLA_DEV f32x4 tri_mask(f32x4 c, int rb, int nb, bool keep_diag, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * rb + 4 * (lane >> 4) + i, col = 16 * nb + (lane & 15);
    if (keep_diag ? r < col : r <= col) c[i] = 0.f;
  }
  return c;
}

// The same for a block held in row layout (lane owns row lane & 15, columns 4 (lane >> 4)..).
EFLA_DEV f32x4 tri_mask_row(f32x4 c, int rb, int nb, bool keep_diag, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * rb + (lane & 15), col = 16 * nb + 4 * (lane >> 4) + i;
    if (keep_diag ? r < col : r <= col) c[i] = 0.f;
  }
  return c;
}

template <typename E, int DK, int DV, bool GT>
__global__ __launch_bounds__(kBwdThreads, 1) void chunk_bwd_kernel(
    Geom g, const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const E* __restrict__ beta, const E* __restrict__ d_o, const E* __restrict__ ut,
    const E* __restrict__ dut, const E* __restrict__ states, const E* __restrict__ dstates,
    const E* __restrict__ xsav, E* __restrict__ dq, E* __restrict__ dk, E* __restrict__ dv,
    E* __restrict__ dbeta, const E* __restrict__ gate, const float* __restrict__ cum,
    E* __restrict__ dgate) {
  typedef ChunkBwdLds<E, DK, DV, GT> L;
  typedef typename Mma<E>::vec Vv;
  constexpr int LK = L::LK, LV = L::LV, LT = L::LT;
  constexpr int KC = Mma<E>::KC, KSV = DV / KC;
  constexpr int CK = DK / 64, CV = DV / 64;  // column blocks per wave of [64][d] outputs
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  lds_poison(smem);
  E* sK = (E*)(smem + L::oK);
  E* sQ = (E*)(smem + L::oQ);
  E* sW = (E*)(smem + L::oW);
  E* sDU = (E*)(smem + L::oDU);
  E* sDO = (E*)(smem + L::oDO);
  E* sU = (E*)(smem + L::oU);
  E* sV = (E*)(smem + L::oV);
  E* sX = (E*)(smem + L::oX);
  E* sM = (E*)(smem + L::oM);
  E* sDX = sDO;
  E* sY = sU;
  E* sH = sV;
  float* cLam = (float*)(smem + L::oC);
  float* cAl = cLam + 64;
  float* cEx = cLam + 128;
  float* cDl = cLam + 192;
  // dalpha partials [64][8]: slots 0-3 column sums of dT . X per row block, slots 4-7 row
  // sums of dA . KK^T per column block (one token's eight partials are one 32-byte row).
  float* pDa = (float*)(smem + L::oP);
  float* cC = (float*)(smem + L::oGc);     // gated: c, b, db/dbeta, db/dlam, db/da
  float* cB = cC + 64;
  float* cBb = cC + 128;
  float* cBl = cC + 192;
  float* cBa = cC + 256;
  // gated: dc partials per token, slots 0-3 state part of dQ . Q (column group), 4-7
  // r dr (column group), 8-11 dP * P row sums (pair parity, block), 12-15 dP * P column sums
  // (row block), 16-19 dA * A column sums (row block); then <G, S> per column group
  constexpr int NS = L::kDcSlots;
  float* pDc = (float*)(smem + L::oDc);
  float* pGS = pDc + 64 * NS;
  float* pDb = (float*)(smem + L::oDb);    // gated: db partials [64][4]

  int tid = threadIdx.x, lane = tid & 63;
  const int wv0 = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Chunks of all heads are numbered u = slot * H + h; packed batches use a prefix of them.
  const int nu = used_slots(g) * g.H;
  int u = blockIdx.x;
  if (u >= nu) return;

  TileRegs<E, DK> tK, tQ;
  TileRegs<E, DV> tDU, tDO, tU, tV;
  TileRegs<E, 64> tX;
  Vv fS[CK][KSV], fG[CK][KSV];  // rows of S and G for this wave's d_k columns (B^T operands)
  float bt, cR = 0.f, aR = 0.f;  // beta, and (gated) c and log-decay of token lane
  // Requests for a chunk's inputs, issued for the next chunk in small groups spread over
  // the steps of the current one: a large burst would stall the issuing waves until the
  // memory system had taken all of it. The last group goes through opaque copies of its
  // base pointers (fresh each iteration), which keeps the compiler from sinking its loads past
  // the chunk's final stores towards their use in the next iteration.
  const E* qL = q;
  const E* gL = dstates;
  auto issue_k = [&](const ChunkUnit& c) {
    tK.load(k + c.row0 * DK, c.n, tid);
    bt = to_f(beta[c.row0 + min(lane, c.n - 1)]);
    if constexpr (GT) {
      cR = cum[c.sh * kChunk + lane];
      aR = to_f(gate[c.row0 + min(lane, c.n - 1)]);
    }
  };
  auto issue_du_do = [&](const ChunkUnit& c) {
    tDU.load(dut + c.row0 * DV, c.n, tid);
    tDO.load(d_o + c.row0 * DV, c.n, tid);
  };
  auto issue_u = [&](const ChunkUnit& c) { tU.load(ut + c.row0 * DV, c.n, tid); };
  auto issue_v_x = [&](const ChunkUnit& c) {
    tV.load(v + c.row0 * DV, c.n, tid);
    tX.load(xsav + c.sh * 64 * 64, 64, tid);
  };
  auto issue_q = [&](const ChunkUnit& c) { tQ.load(qL + c.row0 * DK, c.n, tid); };
  auto issue_s = [&](const ChunkUnit& c, int cK) {
#pragma unroll
    for (int j = 0; j < CK; ++j)
#pragma unroll
      for (int ks = 0; ks < KSV; ++ks)
        fS[j][ks] = frag_rm_g<E>(states + c.sh * DK * DV + (int64_t)16 * (cK + j) * DV + ks * KC, DV, lane);
  };
  auto issue_g = [&](const ChunkUnit& c, int cK) {
#pragma unroll
    for (int j = 0; j < CK; ++j)
#pragma unroll
      for (int ks = 0; ks < KSV; ++ks)
        fG[j][ks] = frag_rm_g<E>(gL + c.sh * DK * DV + (int64_t)16 * (cK + j) * DV + ks * KC, DV, lane);
  };

  ChunkUnit cur = chunk_unit(g, u);
  issue_k(cur);
  issue_du_do(cur);
  issue_s(cur, CK * (wv0 & 3));
  issue_g(cur, CK * (wv0 & 3));
  issue_u(cur);
  issue_v_x(cur);
  issue_q(cur);
  // ---- 1: a chunk's tiles land in LDS; ||k||^2 is reduced from the loaded K vectors (VPR
  // consecutive threads per row). Done before the loop for the first chunk and at the end of
  // each iteration for the next one, after that iteration's stores: every load and store in the
  // loop is unconditional (after the last chunk, one row of the first), so the compiler knows how many
  // stores follow the loads and waits for the loads alone.
  float bt_cur = 0.f, a_cur = 0.f;
  auto land = [&](const ChunkUnit& c) {
    const int n = c.n;
    tK.store(sK, LK, n, tid);
    {
      typedef TileRegs<E, DK> TKr;
#pragma unroll
      for (int it = 0; it < TKr::IT; ++it) {
        const int i = it * kBwdThreads + tid;
        const Vv x = __builtin_bit_cast(Vv, tK.v[it]);
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < TKr::VE; ++e) acc = fmaf(to_f(x[e]), to_f(x[e]), acc);
        acc = group_sum<TKr::VPR>(acc);
        if (i % TKr::VPR == 0) cLam[i / TKr::VPR] = i / TKr::VPR < n ? acc : 0.f;
      }
    }
    bt_cur = bt;
    a_cur = aR;
    if constexpr (GT) {
      if (tid < 64) cC[tid] = cR;
      for (int i = tid; i < 64 * NS; i += kBwdThreads) pDc[i] = 0.f;
    }
    tDU.store(sDU, LV, n, tid);
    tDO.store(sDO, LV, n, tid);
    tU.store(sU, LV, n, tid);
    tV.store(sV, LV, n, tid);
    tX.store(sX, LT, 64, tid);
    tQ.store(sQ, LK, n, tid);
  };
  land(cur);
  for (;;) {
  // Every per-lane address below derives from tid; making it opaque here keeps the compiler
  // from hoisting dozens of loop-invariant LDS addresses out of the loop (they would hold
  // registers through the whole chunk and spill). Recomputing them costs a few ALU ops.
  asm volatile("" : "+v"(tid));
  lane = tid & 63;
  // The same for the wave index: wave-dependent LDS offsets are formed again in scalar
  // registers where they are used instead of being held (and spilled) across the loop.
  int wv = wv0;
  asm volatile("" : "+s"(wv));
  qL = opaque_global(q);
  gL = opaque_global(dstates);
  // [64][d] outputs: wave wv owns row blocks rb0, rb0 + 1 and column blocks cK.. (cV..).
  const int rb0 = 2 * (wv >> 2), cK = CK * (wv & 3), cV = CV * (wv & 3);
  // 64x64 work matrices: wave wv owns blocks (pr, pn) and (pr, pn + 1).
  const int pr = wv >> 1, pn = 2 * (wv & 1);
  const bool plow = pn <= pr;  // at least one of the two blocks is on or below the diagonal
  const int n = cur.n;
  const int64_t row0 = cur.row0;
  __syncthreads();  // this chunk's tiles are in LDS; the next chunk's are requested from here on
  const int un = u + (int)gridDim.x;
  const bool more = un < nu;
  // After the last chunk the requests still go out (every load is unconditional), to one row
  // of the first chunk, which all workgroups then share in L2.
  ChunkUnit nxt = chunk_unit(g, more ? un : 0);
  if (!more) nxt.n = 1;
  issue_k(nxt);
  __builtin_amdgcn_sched_barrier(0);  // these requests go out now, not after step 2's products

  // ---- 2: dW = -dU~ S^T, dQ = scale dO S^T, dK = U~ G^T (S and G from registers);
  //         dM = scale tril(dO U~^T); per-token coefficients
  f32x4 aQ[2][CK], aK[2][CK];
  if constexpr (GT) {
    // dc_last += e^{c_last} <G, S>: waves 0-3 hold every row of S and G once
    if (wv < 4) {
      float gs = 0.f;
#pragma unroll
      for (int j = 0; j < CK; ++j)
#pragma unroll
        for (int ks = 0; ks < KSV; ++ks)
#pragma unroll
          for (int e = 0; e < 16 / (int)sizeof(E); ++e) gs = fmaf(to_f(fS[j][ks][e]), to_f(fG[j][ks][e]), gs);
      gs = group_sum<16>(gs);
      gs += __shfl_xor(gs, 16);
      gs += __shfl_xor(gs, 32);
      if (lane == 0) pGS[wv] = gs;
    }
  }
  {
    f32x4 aW[2][CK];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < CK; ++j) aW[i][j] = aQ[i][j] = aK[i][j] = zero4();
#pragma unroll
    for (int ks = 0; ks < KSV; ++ks) {
      Vv fu[2], fo[2], fv[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        fu[i] = frag_rm<E>(sDU + 16 * (rb0 + i) * LV + ks * KC, LV, lane);
        fo[i] = frag_rm<E>(sDO + 16 * (rb0 + i) * LV + ks * KC, LV, lane);
        fv[i] = frag_rm<E>(sU + 16 * (rb0 + i) * LV + ks * KC, LV, lane);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < CK; ++j) {
          aW[i][j] = Mma<E>::step(fS[j][ks], fu[i], aW[i][j]);
          aQ[i][j] = Mma<E>::step(fS[j][ks], fo[i], aQ[i][j]);
          aK[i][j] = Mma<E>::step(fG[j][ks], fv[i], aK[i][j]);
        }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < CK; ++j) {
        st_frag_t<E>(sW + 16 * (rb0 + i) * LK + 16 * (cK + j), LK, -aW[i][j], lane);
        aQ[i][j] *= g.scale;
      }
  }
  if constexpr (GT) {
    // dQ's state part scale diag(Gamma) dO S^T adds its row dot with Q to dc; dK's state part
    // diag(r) U~ G^T: with dr_t = k_t . (U~ G^T)_t, dc_t -= r_t dr_t and dc_last += r_t dr_t.
    const float cl = cC[n - 1];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int t = 16 * (rb0 + i) + (lane & 15);
      const float ct = cC[t], gm = exp_decay(ct), rr = exp_decay(cl - ct);
      float p1 = 0.f, p2 = 0.f;
#pragma unroll
      for (int j = 0; j < CK; ++j) {
        const int col = 16 * (cK + j) + 4 * (lane >> 4);
        const f32x4 qv = ld4f<E>(sQ + t * LK + col), kv = ld4f<E>(sK + t * LK + col);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          aQ[i][j][e] *= gm;
          p1 = fmaf(aQ[i][j][e], qv[e], p1);
          p2 = fmaf(aK[i][j][e], kv[e], p2);
          aK[i][j][e] *= rr;
        }
      }
      p1 += __shfl_xor(p1, 16);
      p1 += __shfl_xor(p1, 32);
      p2 += __shfl_xor(p2, 16);
      p2 += __shfl_xor(p2, 32);
      if (lane < 16) {
        pDc[t * NS + (wv & 3)] = p1;
        pDc[t * NS + 4 + (wv & 3)] = rr * p2;
      }
    }
  }
  {
    f32x4 m[1][2] = {{zero4(), zero4()}}, qk[1][2] = {{zero4(), zero4()}};
    if (plow) {
      mma_blk<E, false, false, 1, 2, DV, true>(sDO + 16 * pr * LV, LV, sU + 16 * pn * LV, LV, 0, DV, m, lane);
      if constexpr (GT)
        mma_blk<E, false, false, 1, 2, DK, true>(sQ + 16 * pr * LK, LK, sK + 16 * pn * LK, LK, 0, DK, qk, lane);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      f32x4 mm = tri_mask_row(m[0][j], pr, pn + j, true, lane) * g.scale;
      if constexpr (GT) {  // dP * P adds to dc (rows +, columns -); then dM = dP * D
        const int t = 16 * pr + (lane & 15), s0 = 16 * (pn + j) + 4 * (lane >> 4);
        const float ct = cC[t];
        float rsum = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // D_ts = e^{c_t - c_s} on and below the diagonal only: above it dP * P is zero, and the
          // factor alone may overflow when the log-decays are negative
          const float d = s0 + e <= t ? exp_decay(ct - cC[s0 + e]) : 0.f;
          const float ev = mm[e] * (qk[0][j][e] * d);  // dP * P (mm is zero above the diagonal)
          rsum += ev;
          const float csum = group_sum<16>(ev);
          if ((lane & 15) == 0) pDc[(s0 + e) * NS + 12 + pr] = -csum;
          mm[e] *= d;
        }
        rsum += __shfl_xor(rsum, 16);
        rsum += __shfl_xor(rsum, 32);
        if (lane < 16) pDc[t * NS + 8 + 2 * (wv & 1) + j] = rsum;
      }
      st_frag_t<E>(sM + 16 * pr * LT + 16 * (pn + j), LT, mm, lane);
    }
  }
  if (tid < 64) {
    const FlowCoef cf = flow_coef(tid < n ? bt_cur : 0.f, cLam[tid], g.euler);
    cAl[tid] = cf.alpha;
    cEx[tid] = cf.ex;
    cDl[tid] = cf.dlam;
    if constexpr (GT) {
      const GatedCoef gc = gated_coef(tid < n ? bt_cur : 0.f, cLam[tid], a_cur, g.euler);
      cB[tid] = tid < n ? gc.b : 0.f;
      cBb[tid] = gc.db_dbeta;
      cBl[tid] = gc.db_dlam;
      cBa[tid] = gc.db_da;
    }
  }
  __syncthreads();
  issue_du_do(nxt);

  // ---- 3: dT = dW K^T + dU V^T -> dalpha (columns) and dX = dT diag(alpha) (strictly lower);
  //         dV = T^T dU, dK += T^T dW (T^T = diag(alpha) X^T); dQ += dM K; dK += dM^T Q
  //         (gated: dT_w = dW K^T and dT_u = dU V^T apart; dX = dT_w diag(alpha Gamma) +
  //         dT_u diag(b); column sums of dT_w . X give d(alpha Gamma), of dT_u . X give db)
  {
    f32x4 t[1][2] = {{zero4(), zero4()}}, tu[1][2] = {{zero4(), zero4()}};
    if (plow) {
      mma_blk<E, false, false, 1, 2, DK>(sW + 16 * pr * LK, LK, sK + 16 * pn * LK, LK, 0, DK, t, lane);
      if constexpr (GT)
        mma_blk<E, false, false, 1, 2, DV>(sDU + 16 * pr * LV, LV, sV + 16 * pn * LV, LV, 0, DV, tu, lane);
      else
        mma_blk<E, false, false, 1, 2, DV>(sDU + 16 * pr * LV, LV, sV + 16 * pn * LV, LV, 0, DV, t, lane);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (pn + j > pr) t[0][j] = tu[0][j] = zero4();
      const int col = 16 * (pn + j) + (lane & 15);
      const float al = cAl[col];
      const float gmc = GT ? exp_decay(cC[col]) : 1.f, bc = GT ? cB[col] : 0.f;
      float cs = 0.f, cb = 0.f;
      f32x4 dx;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * pr + 4 * (lane >> 4) + i;
        const float xv = to_f(sX[row * LT + col]);  // X is zero above the diagonal
        cs = fmaf(t[0][j][i], xv, cs);
        if constexpr (GT) {
          cb = fmaf(tu[0][j][i], xv, cb);
          dx[i] = row > col ? t[0][j][i] * (al * gmc) + tu[0][j][i] * bc : 0.f;
        } else {
          dx[i] = row > col ? t[0][j][i] * al : 0.f;
        }
      }
      cs += __shfl_xor(cs, 16);
      cs += __shfl_xor(cs, 32);
      if (lane < 16) pDa[col * 8 + pr] = cs * gmc;  // dalpha part: d(alpha Gamma) Gamma
      if constexpr (GT) {
        cb += __shfl_xor(cb, 16);
        cb += __shfl_xor(cb, 32);
        if (lane < 16) pDb[col * 4 + pr] = cb;
      }
      st_frag_lds<E>(sDX + 16 * pr * LT + 16 * (pn + j), LT, dx, lane);
    }
  }
  f32x4 aV[2][CV];
  {
    f32x4 tw[2][CK];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int j = 0; j < CV; ++j) aV[i][j] = zero4();
#pragma unroll
      for (int j = 0; j < CK; ++j) tw[i][j] = zero4();
    }
    // T^T = diag(alpha) X^T is upper triangular: rows of block rb need k >= 16 rb.
    const int k0 = round_down_kc<E>(16 * rb0);
#pragma unroll
    for (int kk = 0; kk < kChunk; kk += KC) {
      if (kk < k0) continue;
      Vv xa[2], bu[CV], bw[CK];
#pragma unroll
      for (int i = 0; i < 2; ++i) xa[i] = frag_km<E>(sX + 16 * (rb0 + i) + kk * LT, LT, lane);
#pragma unroll
      for (int j = 0; j < CV; ++j) bu[j] = frag_km<E>(sDU + 16 * (cV + j) + kk * LV, LV, lane);
#pragma unroll
      for (int j = 0; j < CK; ++j) bw[j] = frag_km<E>(sW + 16 * (cK + j) + kk * LK, LK, lane);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int j = 0; j < CV; ++j) aV[i][j] = Mma<E>::step(bu[j], xa[i], aV[i][j]);
#pragma unroll
        for (int j = 0; j < CK; ++j) tw[i][j] = Mma<E>::step(bw[j], xa[i], tw[i][j]);
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = 16 * (rb0 + i) + (lane & 15);
      const float al = cAl[row];
      // gated: T_u^T = diag(b) X^T, T_w^T = diag(alpha Gamma) X^T
      const float fu = GT ? cB[row] : al, fw = GT ? al * exp_decay(cC[row]) : al;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
#pragma unroll
        for (int j = 0; j < CV; ++j) aV[i][j][e] *= fu;
#pragma unroll
        for (int j = 0; j < CK; ++j) aK[i][j][e] = fmaf(fw, tw[i][j][e], aK[i][j][e]);
      }
    }
  }
  // dM is lower triangular: dM K for rows of block rb needs k < 16 (rb + 1); dM^T Q needs
  // k >= 16 rb.
  mma_blk<E, false, true, 2, CK, kChunk, true>(sM + 16 * rb0 * LT, LT, sK + 16 * cK, LK, 0,
                                               round_up_kc<E>(16 * (rb0 + 2)), aQ, lane);
  mma_blk<E, true, true, 2, CK, kChunk, true>(sM + 16 * rb0, LT, sQ + 16 * cK, LK,
                                              round_down_kc<E>(16 * rb0), kChunk, aK, lane);
  __syncthreads();
  // S registers are free again; G follows two steps later. The gated kernel, which holds more
  // per-token state, requests S with G so that S is not held through the dA step.
  if constexpr (!GT) issue_s(nxt, cK);

  // ---- 4: Y = dX X^T (only the lower blocks are used: rows t > s), kept transposed
  //         (sY[s][t] = Y[t][s]); stage dQ and dV
  {
    f32x4 y[1][2] = {{zero4(), zero4()}};
    if (plow)
      mma_blk<E, false, false, 1, 2, kChunk>(sDX + 16 * pr * LT, LT, sX + 16 * pn * LT, LT, 0,
                                             round_up_kc<E>(16 * (pn + 2)), y, lane);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const f32x4 yy = pn + j <= pr ? y[0][j] : zero4();
      st_frag_t<E>(sY + 16 * (pn + j) * LT + 16 * pr, LT, yy, lane);
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int j = 0; j < CK; ++j)
      st_frag_t<E>(sQ + 16 * (rb0 + i) * LK + 16 * (cK + j), LK, aQ[i][j], lane);
#pragma unroll
    for (int j = 0; j < CV; ++j)
      st_frag_t<E>(sDU + 16 * (rb0 + i) * LV + 16 * (cV + j), LV, aV[i][j], lane);
  }
  __syncthreads();
  issue_u(nxt);
  issue_v_x(nxt);

  // ---- 5: dA = -X^T Y (strictly lower) -> dalpha (rows) and H = dG + dG^T; write dQ, dV
  {
    f32x4 da[1][2] = {{zero4(), zero4()}}, kk[1][2] = {{zero4(), zero4()}};
    if (plow) {
      mma_blk<E, true, false, 1, 2, kChunk>(sX + 16 * pr, LT, sY + 16 * pn * LT, LT,
                                            round_down_kc<E>(16 * pr), kChunk, da, lane);
      mma_blk<E, false, false, 1, 2, DK>(sK + 16 * pr * LK, LK, sK + 16 * pn * LK, LK, 0, DK, kk, lane);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int nb = pn + j;
      if (nb > pr) {
        if (lane < 16) pDa[(16 * pr + lane) * 8 + 4 + nb] = 0.f;
        continue;
      }
      const int col = 16 * nb + (lane & 15);
      float rs[4], fc = 0.f;
      f32x4 dg;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * pr + 4 * (lane >> 4) + i;
        float a = row > col ? -da[0][j][i] : 0.f;
        if constexpr (GT) a = row > col ? a * exp_decay(cC[row] - cC[col]) : 0.f;  // A carries D
        rs[i] = a * kk[0][j][i];
        dg[i] = a * cAl[row];
        if constexpr (GT) fc = fmaf(cAl[row], rs[i], fc);  // dA . A, column part
      }
      if constexpr (GT) {  // dc_s -= sum_t dA_ts A_ts (the row part enters as alpha dalpha)
        fc += __shfl_xor(fc, 16);
        fc += __shfl_xor(fc, 32);
        if (lane < 16) pDc[col * NS + 16 + pr] = -fc;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) rs[i] = group_sum<16>(rs[i]);
      if ((lane & 15) == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) pDa[(16 * pr + 4 * (lane >> 4) + i) * 8 + 4 + nb] = rs[i];
      }
      if (nb < pr) {
        st_frag_lds<E>(sH + 16 * pr * LT + 16 * nb, LT, dg, lane);
        st_frag_t<E>(sH + 16 * nb * LT + 16 * pr, LT, dg, lane);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * pr + 4 * (lane >> 4) + i;
          if (row > col) {
            sH[row * LT + col] = to_e<E>(dg[i]);
            sH[col * LT + row] = to_e<E>(dg[i]);
          } else if (row == col) {
            sH[row * LT + col] = to_e<E>(0.f);
          }
        }
      }
    }
  }
  s2g<E, DK, kBwdThreads>(dq + row0 * DK, DK, sQ, LK, n, tid);
  s2g<E, DV, kBwdThreads>(dv + row0 * DV, DV, sDU, LV, n, tid);
  __syncthreads();
  issue_q(nxt);
  if constexpr (GT) issue_s(nxt, cK);
  issue_g(nxt, cK);

  // ---- 6: dK += H K; dk += 2 k dalpha dalpha/dlam; dbeta = dalpha e^-x
  mma_blk<E, false, true, 2, CK, kChunk, true>(sH + 16 * rb0 * LT, LT, sK + 16 * cK, LK, 0,
                                               kChunk, aK, lane);
  auto dalpha = [&](int t) {
    const f32x4 a = *(const f32x4*)(pDa + 8 * t), b = *(const f32x4*)(pDa + 8 * t + 4);
    return ((a[0] + a[1]) + (a[2] + a[3])) + ((b[0] + b[1]) + (b[2] + b[3]));
  };
  auto dbsum = [&](int t) {
    const f32x4 a = *(const f32x4*)(pDb + 4 * t);
    return (a[0] + a[1]) + (a[2] + a[3]);
  };
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 16 * (rb0 + i) + (lane & 15);
    float f = 2.f * dalpha(row) * cDl[row];
    if constexpr (GT) f = fmaf(2.f * dbsum(row), cBl[row], f);
#pragma unroll
    for (int j = 0; j < CK; ++j) {
      const f32x4 kv = ld4f<E>(sK + row * LK + 16 * (cK + j) + 4 * (lane >> 4));
#pragma unroll
      for (int e = 0; e < 4; ++e) aK[i][j][e] = fmaf(f, kv[e], aK[i][j][e]);
      st_frag_t<E>(sW + 16 * (rb0 + i) * LK + 16 * (cK + j), LK, aK[i][j], lane);
    }
  }
  if constexpr (GT) {
    if (tid < 64) {
      // dbeta and the gate gradient: dc_t gains alpha_t dalpha_t (the e^{c} in T_w and the row
      // part of dA . A); the last token carries the chunk-end factors; then
      // dgate_t = sum_{s >= t} dc_s + db_t db_t/da_t.
      const float da_t = dalpha(tid), db_t = dbsum(tid);
      float* pt = pDc + tid * NS;
      float sq = 0.f, rdr = 0.f, se = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sq += pt[j];
        rdr += pt[4 + j];
      }
#pragma unroll
      for (int j = 8; j < NS; ++j) se += pt[j];
      float dc = tid < n ? fmaf(cAl[tid], da_t, (sq - rdr) + se) : 0.f;
      float rsum = group_sum<16>(rdr);  // rows >= n hold zeros
      rsum += __shfl_xor(rsum, 16);
      rsum += __shfl_xor(rsum, 32);
      if (tid == n - 1) dc += rsum + exp_decay(cC[tid]) * ((pGS[0] + pGS[1]) + (pGS[2] + pGS[3]));
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const float y = __shfl_down(dc, o);
        if (tid + o < 64) dc += y;
      }
      pt[0] = da_t * cEx[tid] + db_t * cBb[tid];  // dbeta and dgate, stored below by all waves
      pt[1] = fmaf(db_t, cBa[tid], dc);
    }
  }
  __syncthreads();
  {  // every thread stores (see s2g): lanes past the last token repeat it
    const int t = min(tid & 63, n - 1);
    if constexpr (GT) {
      dbeta[row0 + t] = to_e<E>(pDc[t * NS]);
      dgate[row0 + t] = to_e<E>(pDc[t * NS + 1]);
    } else {
      dbeta[row0 + t] = to_e<E>(dalpha(t) * cEx[t]);
    }
  }
  s2g<E, DK, kBwdThreads>(dk + row0 * DK, DK, sW, LK, n, tid);
  if (!more) break;
  __syncthreads();  // every LDS read of this chunk is done before the next one lands
  land(nxt);
  u = un;
  cur = nxt;
  }
}

template <typename E, int DK, int DV, bool GT>
static hipError_t chunk_bwd_go(const Shape& s, const int* table, const void* q, const void* k,
                               const void* v, const void* beta, const void* d_o, const void* ut,
                               const void* dut, const void* states, const void* dstates,
                               const void* x, void* dq, void* dk, void* dv, void* dbeta,
                               const void* gate, const float* cum, void* dgate, hipStream_t st) {
  typedef ChunkBwdLds<E, DK, DV, GT> L;
  static_assert(L::bytes <= 160 * 1024, "LDS budget");
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)chunk_bwd_kernel<E, DK, DV, GT>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)L::bytes);
    if (e != hipSuccess) return e;
    attr = true;
  }
  // Persistent: one workgroup per compute unit walks the chunks, prefetching the next.
  const int64_t units = s.slots * s.H;
  if (units < 1) return hipSuccess;
  const int64_t blocks = units < cu_count() ? units : cu_count();
  prof_begin(st);
  hipLaunchKernelGGL((chunk_bwd_kernel<E, DK, DV, GT>), dim3((unsigned)blocks), dim3(kBwdThreads),
                     L::bytes, st, make_geom(s, table), (const E*)q, (const E*)k, (const E*)v,
                     (const E*)beta, (const E*)d_o, (const E*)ut, (const E*)dut,
                     (const E*)states, (const E*)dstates, (const E*)x, (E*)dq, (E*)dk, (E*)dv,
                     (E*)dbeta, (const E*)gate, cum, (E*)dgate);
  hipError_t e = hipGetLastError();
  prof_end(GT ? "chunk_bwd_gated" : "chunk_bwd", st);
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
                            const void* dut, const void* states, const void* dstates,
                            const void* x, void* dq, void* dk, void* dv, void* dbeta,
                            hipStream_t st, const void* gate, const float* cum, void* dgate) {
#define EFLA_CB(E_, DK_, DV_, GT_)                                                              \
  return chunk_bwd_go<E_, DK_, DV_, GT_>(s, table, q, k, v, beta, d_o, ut, dut, states, dstates, \
                                         x, dq, dk, dv, dbeta, gate, cum, dgate, st)
  if (s.dt == Dt::BF16) {
    if (gate) {
      if (s.dk == 64 && s.dv == 64) EFLA_CB(__bf16, 64, 64, true);
      if (s.dk == 64 && s.dv == 128) EFLA_CB(__bf16, 64, 128, true);
      if (s.dk == 128 && s.dv == 64) EFLA_CB(__bf16, 128, 64, true);
      EFLA_CB(__bf16, 128, 128, true);
    }
    if (s.dk == 64 && s.dv == 64) EFLA_CB(__bf16, 64, 64, false);
    if (s.dk == 64 && s.dv == 128) EFLA_CB(__bf16, 64, 128, false);
    if (s.dk == 128 && s.dv == 64) EFLA_CB(__bf16, 128, 64, false);
    EFLA_CB(__bf16, 128, 128, false);
  }
  if (gate) return hipErrorInvalidValue;  // gated EFLA is built for bf16 only
  EFLA_CB(float, 64, 64, false);
#undef EFLA_CB
}

}  // namespace efla

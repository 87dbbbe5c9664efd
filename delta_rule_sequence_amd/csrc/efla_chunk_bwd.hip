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
// Seven barrier-separated steps:
//   1 loads land; 2 dW, scale dO S^T, U~ G^T, dM, coefficients;
//   3 dT (-> dalpha, dX), T^T dU, T^T dW, dM K, dM^T Q;
//   4 Y = dX X^T;  5 dA = -X^T Y (-> dalpha, H);  6 H K and the outputs.
#include "efla_internal.hpp"

namespace efla {

constexpr int kBwdThreads = 512;
constexpr int kBwdWaves = kBwdThreads / 64;

template <typename E, int DK, int DV>
struct ChunkBwdLds {
  static constexpr int LK = pitch<E>(DK), LV = pitch<E>(DV), LT = pitch<E>(64);
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
  static constexpr size_t oP = oC + 4 * 64 * 4;  // dalpha partials [8][64]
  static constexpr size_t bytes = oP + 8 * 64 * 4;
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
      v[it] = *(const u32x4*)(g + (int64_t)r * COLS + c);
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

// Split of a [64][D] output over the eight waves: column block cb, row blocks rb0..rb0+NRB.
template <int D>
struct Part {
  static constexpr int NCB = D / 16, WPC = kBwdWaves / NCB, NRB = 4 / WPC;
  static_assert(NCB * WPC == kBwdWaves && NRB * WPC == 4, "wave split");
};

// The 16 blocks of a 64x64 matrix, two per wave: the ten lower blocks (diagonal included)
// first, then the six strictly upper ones.
// Entry idx is the nibble 4 rb + nb at bit 4 idx (a register constant, no table in memory).
EFLA_DEV void block_of(int idx, int& rb, int& nb) {
  constexpr uint64_t tab = 0xB76321FEDCA98540ull;
  const int e = (int)(tab >> (4 * idx)) & 15;
  rb = e >> 2;
  nb = e & 3;
}

template <typename E, int DK, int DV>
__global__ __launch_bounds__(kBwdThreads, 1) void chunk_bwd_kernel(
    Geom g, const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const E* __restrict__ beta, const E* __restrict__ d_o, const E* __restrict__ ut,
    const E* __restrict__ dut, const E* __restrict__ states, const E* __restrict__ dstates,
    const E* __restrict__ xsav, E* __restrict__ dq, E* __restrict__ dk, E* __restrict__ dv,
    E* __restrict__ dbeta) {
  typedef ChunkBwdLds<E, DK, DV> L;
  typedef typename Mma<E>::vec Vv;
  typedef Part<DK> PK;
  typedef Part<DV> PV;
  constexpr int LK = L::LK, LV = L::LV, LT = L::LT;
  constexpr int KC = Mma<E>::KC, KSV = DV / KC;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
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
  float* pCol = (float*)(smem + L::oP);  // [4][64]: column sums of dT . X per row block
  float* pRow = pCol + 4 * 64;           // [4][64]: row sums of dA . KK^T per column block

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int slot = blockIdx.x / g.H, h = blockIdx.x % g.H;
  ChunkInfo ci;
  if (!chunk_info(g, slot, ci)) return;
  const int n = ci.n;
  const int64_t row0 = (int64_t)(ci.b * g.H + h) * g.T + ci.t0;
  const int64_t sh = (int64_t)slot * g.H + h;
  const int cbK = wv % PK::NCB, rbK = (wv / PK::NCB) * PK::NRB;
  const int cbV = wv % PV::NCB, rbV = (wv / PV::NCB) * PV::NRB;

  // ---- 1: request everything, in order of first use
  TileRegs<E, DK> tK;
  TileRegs<E, DV> tDU, tDO, tU, tV;
  TileRegs<E, 64> tX;
  TileRegs<E, DK> tQ;
  Vv fS[KSV], fG[KSV];  // rows 16 cbK.. of S and of G (B^T operands, contraction over d_v)
  tK.load(k + row0 * DK, n, tid);
  const float bt = to_f(beta[row0 + min(tid & 63, n - 1)]);
  tDU.load(dut + row0 * DV, n, tid);
  {
    const E* Sg = states + sh * DK * DV + (int64_t)16 * cbK * DV;
#pragma unroll
    for (int ks = 0; ks < KSV; ++ks) fS[ks] = frag_rm<E>(Sg + ks * KC, DV, lane);
  }
  tDO.load(d_o + row0 * DV, n, tid);
  tU.load(ut + row0 * DV, n, tid);
  {
    const E* Gg = dstates + sh * DK * DV + (int64_t)16 * cbK * DV;
#pragma unroll
    for (int ks = 0; ks < KSV; ++ks) fG[ks] = frag_rm<E>(Gg + ks * KC, DV, lane);
  }
  tV.load(v + row0 * DV, n, tid);
  tX.load(xsav + sh * 64 * 64, 64, tid);
  tQ.load(q + row0 * DK, n, tid);

  // K lands first; ||k||^2 is reduced from the loaded vectors (VPR consecutive threads/row).
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
#pragma unroll
      for (int off = TKr::VPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
      if (i % TKr::VPR == 0) cLam[i / TKr::VPR] = i / TKr::VPR < n ? acc : 0.f;
    }
  }
  tDU.store(sDU, LV, n, tid);
  tDO.store(sDO, LV, n, tid);
  tU.store(sU, LV, n, tid);
  tV.store(sV, LV, n, tid);
  tX.store(sX, LT, 64, tid);
  tQ.store(sQ, LK, n, tid);
  __syncthreads();

  // ---- 2: dW = -dU~ S^T, dQ = scale dO S^T, dK = U~ G^T (S and G from registers);
  //         dM = scale tril(dO U~^T); per-token coefficients
  f32x4 aQ[PK::NRB], aK[PK::NRB];
#pragma unroll
  for (int j = 0; j < PK::NRB; ++j) {
    const int rb = rbK + j;
    f32x4 w = zero4(), qq = zero4(), kk = zero4();
#pragma unroll
    for (int ks = 0; ks < KSV; ++ks) {
      w = Mma<E>::step(frag_rm<E>(sDU + 16 * rb * LV + ks * KC, LV, lane), fS[ks], w);
      qq = Mma<E>::step(frag_rm<E>(sDO + 16 * rb * LV + ks * KC, LV, lane), fS[ks], qq);
      kk = Mma<E>::step(frag_rm<E>(sU + 16 * rb * LV + ks * KC, LV, lane), fG[ks], kk);
    }
    st_frag_lds<E>(sW + 16 * rb * LK + 16 * cbK, LK, -w, lane);
    aQ[j] = qq * g.scale;
    aK[j] = kk;
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    int rb, nb;
    block_of(wv + kBwdWaves * t, rb, nb);
    f32x4 acc = zero4();
    if (nb <= rb) {
      acc = mma<E, false, false>(sDO + 16 * rb * LV, LV, sU + 16 * nb * LV, LV, 0, DV, acc, lane);
      if (nb == rb) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if ((lane & 15) > 4 * (lane >> 4) + i) acc[i] = 0.f;
      }
      acc *= g.scale;
    }
    st_frag_lds<E>(sM + 16 * rb * LT + 16 * nb, LT, acc, lane);
  }
  if (tid < 64) {
    const FlowCoef cf = flow_coef(tid < n ? bt : 0.f, cLam[tid]);
    cAl[tid] = cf.alpha;
    cEx[tid] = cf.ex;
    cDl[tid] = cf.dlam;
  }
  __syncthreads();

  // ---- 3: dT = dW K^T + dU V^T -> dalpha (columns) and dX = dT diag(alpha) (strictly lower);
  //         dV = T^T dU, dK += T^T dW (T^T = diag(alpha) X^T); dQ += dM K; dK += dM^T Q
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    int rb, nb;
    block_of(wv + kBwdWaves * t, rb, nb);
    f32x4 acc = zero4();
    if (nb <= rb) {
      acc = mma<E, false, false>(sW + 16 * rb * LK, LK, sK + 16 * nb * LK, LK, 0, DK, acc, lane);
      acc = mma<E, false, false>(sDU + 16 * rb * LV, LV, sV + 16 * nb * LV, LV, 0, DV, acc, lane);
    }
    const int col = 16 * nb + (lane & 15);
    const float al = cAl[col];
    float cs = 0.f;
    f32x4 dx;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * rb + 4 * (lane >> 4) + i;
      cs = fmaf(acc[i], to_f(sX[row * LT + col]), cs);  // X is zero above the diagonal
      dx[i] = row > col ? acc[i] * al : 0.f;
    }
    cs += __shfl_xor(cs, 16);
    cs += __shfl_xor(cs, 32);
    if (lane < 16) pCol[rb * 64 + col] = cs;
    st_frag_lds<E>(sDX + 16 * rb * LT + 16 * nb, LT, dx, lane);
  }
  f32x4 aV[PV::NRB];
#pragma unroll
  for (int j = 0; j < PV::NRB; ++j) {
    const int rb = rbV + j;
    f32x4 acc = mma<E, true, true>(sX + 16 * rb, LT, sDU + 16 * cbV, LV, round_down_kc<E>(16 * rb),
                                   kChunk, zero4(), lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] *= cAl[16 * rb + 4 * (lane >> 4) + i];
    aV[j] = acc;
  }
#pragma unroll
  for (int j = 0; j < PK::NRB; ++j) {
    const int rb = rbK + j;
    f32x4 tw = mma<E, true, true>(sX + 16 * rb, LT, sW + 16 * cbK, LK, round_down_kc<E>(16 * rb),
                                  kChunk, zero4(), lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) aK[j][i] = fmaf(cAl[16 * rb + 4 * (lane >> 4) + i], tw[i], aK[j][i]);
    aQ[j] = mma<E, false, true>(sM + 16 * rb * LT, LT, sK + 16 * cbK, LK, 0,
                                round_up_kc<E>(16 * (rb + 1)), aQ[j], lane);
    aK[j] = mma<E, true, true>(sM + 16 * rb, LT, sQ + 16 * cbK, LK, round_down_kc<E>(16 * rb),
                               kChunk, aK[j], lane);
  }
  __syncthreads();

  // ---- 4: Y = dX X^T (only the lower blocks are used: rows t > s); stage dQ and dV
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    int rb, nb;
    block_of(wv + kBwdWaves * t, rb, nb);
    f32x4 acc = zero4();
    if (nb <= rb)
      acc = mma<E, false, false>(sDX + 16 * rb * LT, LT, sX + 16 * nb * LT, LT, 0,
                                 round_up_kc<E>(16 * (nb + 1)), acc, lane);
    st_frag_lds<E>(sY + 16 * rb * LT + 16 * nb, LT, acc, lane);
  }
#pragma unroll
  for (int j = 0; j < PK::NRB; ++j) st_frag_lds<E>(sQ + 16 * (rbK + j) * LK + 16 * cbK, LK, aQ[j], lane);
#pragma unroll
  for (int j = 0; j < PV::NRB; ++j) st_frag_lds<E>(sDU + 16 * (rbV + j) * LV + 16 * cbV, LV, aV[j], lane);
  __syncthreads();

  // ---- 5: dA = -X^T Y (strictly lower) -> dalpha (rows) and H = dG + dG^T; write dQ, dV
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    int rb, nb;
    block_of(wv + kBwdWaves * t, rb, nb);
    if (nb > rb) {
      if (lane < 16) pRow[nb * 64 + 16 * rb + lane] = 0.f;
      continue;
    }
    const f32x4 da = mma<E, true, true>(sX + 16 * rb, LT, sY + 16 * nb, LT,
                                        round_down_kc<E>(16 * rb), kChunk, zero4(), lane);
    const f32x4 kk = mma<E, false, false>(sK + 16 * rb * LK, LK, sK + 16 * nb * LK, LK, 0, DK,
                                          zero4(), lane);
    const int col = 16 * nb + (lane & 15);
    float rs[4];
    f32x4 dg;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * rb + 4 * (lane >> 4) + i;
      const float a = row > col ? -da[i] : 0.f;
      rs[i] = a * kk[i];
      dg[i] = a * cAl[row];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x = rs[i];
      x += __shfl_xor(x, 1);
      x += __shfl_xor(x, 2);
      x += __shfl_xor(x, 4);
      x += __shfl_xor(x, 8);
      rs[i] = x;
    }
    if ((lane & 15) == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) pRow[nb * 64 + 16 * rb + 4 * (lane >> 4) + i] = rs[i];
    }
    if (nb < rb) {
      st_frag_lds<E>(sH + 16 * rb * LT + 16 * nb, LT, dg, lane);
      st_frag_t<E>(sH + 16 * nb * LT + 16 * rb, LT, dg, lane);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * rb + 4 * (lane >> 4) + i;
        if (row > col) {
          sH[row * LT + col] = to_e<E>(dg[i]);
          sH[col * LT + row] = to_e<E>(dg[i]);
        } else if (row == col) {
          sH[row * LT + col] = to_e<E>(0.f);
        }
      }
    }
  }
  s2g<E, DK, kBwdThreads>(dq + row0 * DK, DK, sQ, LK, n, tid);
  s2g<E, DV, kBwdThreads>(dv + row0 * DV, DV, sDU, LV, n, tid);
  __syncthreads();

  // ---- 6: dK += H K; dk += 2 k dalpha dalpha/dlam; dbeta = dalpha e^-x
#pragma unroll
  for (int j = 0; j < PK::NRB; ++j) {
    const int rb = rbK + j;
    f32x4 acc = mma<E, false, true>(sH + 16 * rb * LT, LT, sK + 16 * cbK, LK, 0, kChunk, aK[j], lane);
    const int col = 16 * cbK + (lane & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * rb + 4 * (lane >> 4) + i;
      const float da = pCol[row] + pCol[64 + row] + pCol[128 + row] + pCol[192 + row] +
                       pRow[row] + pRow[64 + row] + pRow[128 + row] + pRow[192 + row];
      acc[i] = fmaf(2.f * to_f(sK[row * LK + col]), da * cDl[row], acc[i]);
    }
    st_frag_lds<E>(sW + 16 * rb * LK + 16 * cbK, LK, acc, lane);
  }
  if (tid < n) {
    const float da = pCol[tid] + pCol[64 + tid] + pCol[128 + tid] + pCol[192 + tid] + pRow[tid] +
                     pRow[64 + tid] + pRow[128 + tid] + pRow[192 + tid];
    dbeta[row0 + tid] = to_e<E>(da * cEx[tid]);
  }
  __syncthreads();
  s2g<E, DK, kBwdThreads>(dk + row0 * DK, DK, sW, LK, n, tid);
}

template <typename E, int DK, int DV>
static hipError_t chunk_bwd_go(const Shape& s, const int* table, const void* q, const void* k,
                               const void* v, const void* beta, const void* d_o, const void* ut,
                               const void* dut, const void* states, const void* dstates,
                               const void* x, void* dq, void* dk, void* dv, void* dbeta,
                               hipStream_t st) {
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
  hipLaunchKernelGGL((chunk_bwd_kernel<E, DK, DV>), dim3((unsigned)blocks), dim3(kBwdThreads),
                     L::bytes, st, make_geom(s, table), (const E*)q, (const E*)k, (const E*)v,
                     (const E*)beta, (const E*)d_o, (const E*)ut, (const E*)dut,
                     (const E*)states, (const E*)dstates, (const E*)x, (E*)dq, (E*)dk, (E*)dv,
                     (E*)dbeta);
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
                            const void* dut, const void* states, const void* dstates,
                            const void* x, void* dq, void* dk, void* dv, void* dbeta,
                            hipStream_t st) {
#define EFLA_CB(E_, DK_, DV_)                                                                   \
  return chunk_bwd_go<E_, DK_, DV_>(s, table, q, k, v, beta, d_o, ut, dut, states, dstates, x, \
                                    dq, dk, dv, dbeta, st)
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

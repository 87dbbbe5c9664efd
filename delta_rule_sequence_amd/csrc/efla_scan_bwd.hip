// Reverse inter-chunk recurrence of the backward pass.
//
// Reverse-mode differentiation of the chunk recurrence of section 3.3 (Exact Flow Linear
// Attention summary page): with G the gradient of the state leaving chunk c,
//   dU~_c = scale M_c^T dO_c + K_c G,          M_c = tril(Q_c K_c^T) saved by the forward,
//   G    <- G + scale Q_c^T dO_c - W_c^T dU~_c (gradient of the state entering c).
// One workgroup walks the chunks of one (sequence, head) backwards and owns a d_k x TV
// slice of G, kept transposed (G^T, TV x d_k) in fp32 MFMA accumulators. It writes dU~ and,
// per chunk, the G that entered the step (the gradient of the chunk's outgoing state) for
// the chunk-parallel gradient kernel.
//
// Two kernels share this math. The register-fed one (16-column tiles, fp32): the K rows of
// each wave are register A fragments, the previous chunk's K rows and Q, W, M, dO tiles are
// loaded into registers while the current chunk computes, and the LDS tiles are double-
// buffered. The DMA-fed one (bf16, 32-column tiles, further below) has a loader wave fill the
// LDS tiles by DMA and a storer wave write the outputs, as the forward scan does. Products over
// the token or d_k index read LDS tiles k-major with the LDS transpose read (bf16). dU~ and G
// leave through LDS staging as 16-byte stores.
//
// Gated EFLA (GT), with c the running log-decay sums of the chunk, Gamma = e^c,
// r = e^{c_last - c}: dU~ = scale P^T dO + diag(r) K G (P = tril(Q K^T) * e^{c_t - c_s}, saved
// by the forward in place of M) and G <- e^{c_last} G + scale Q^T diag(Gamma) dO - W^T dU~.
// Q rows are scaled by Gamma when they land in LDS; the rest acts on accumulators.
//
// Segment-parallel backward (long sequences, few sequence-head pairs). The chunk step is affine
// in the state gradient, G <- (I - W^T K) G + scale (Q - M W)^T dO (gated: with the decays), so
// a segment of chunks maps the gradient leaving it to the one entering it as A G + R, where A is
// the transpose of the forward's segment transition (kept from the forward). MODE 1 (state only)
// runs from zero and keeps only the result, R. MODE 0 is the full scan that writes dU~ and the
// per-chunk gradients.
#include "efla_internal.hpp"

namespace efla {

// XF (bf16): the stage holds K in W's place, and X and alpha~ (dU~^T W = Z^T K with
// Z = diag(alpha~) X^T dU~, formed in registers); fp32: W, read as it is.
template <typename E, int DK, int DV, int TV, bool GT = false>
struct ScanBwdLds {
  static constexpr bool XF = sizeof(E) == 2;
  static constexpr int LK = pitch<E>(DK), LT = pitch<E>(64), LS = pitch<E>(TV);
  // one stage: Q [64][LK], W or K [64][LK], M [64][LT], X [64][LT] (XF), dO [64][LS]
  static constexpr size_t oQ = 0;
  static constexpr size_t oW = oQ + 64 * LK * sizeof(E);
  static constexpr size_t oM = oW + 64 * LK * sizeof(E);
  static constexpr size_t oX = oM + 64 * LT * sizeof(E);
  static constexpr size_t oO = oX + (XF ? 64 * LT * sizeof(E) : 0);
  static constexpr size_t oCs = oO + 64 * LS * sizeof(E);     // running log-decay sums [64] (GT)
  static constexpr size_t oAl = oCs + (GT ? 64 * 4 : 0);       // alpha~ [64] (XF)
  static constexpr size_t stage = oAl + (XF ? 64 * 4 : 0);
  // bf16 with 16-column tiles: one stage, so that two workgroups share a compute unit
  static constexpr int NSTG = (sizeof(E) == 2 && TV == 16) ? 1 : 2;
  static constexpr size_t oG = NSTG * stage;                    // G slice [DK][LS]
  static constexpr size_t oDt = oG + DK * LS * sizeof(E);       // dU~^T  [TV][LT]
  static constexpr size_t oDu = oDt + TV * LT * sizeof(E);      // dU~ staging [64][LS]
  static constexpr size_t bytes = oDu + 64 * LS * sizeof(E);
};

template <typename E, int DK, int DV, int TV, bool GT, int MODE>
__global__ __launch_bounds__(kThreads, (sizeof(E) == 2 && TV == 16) ? 2 : 1) void scan_bwd_kernel(
    Geom g, const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ w,
    const E* __restrict__ m, const E* __restrict__ d_o, E* __restrict__ dut,
    E* __restrict__ dstates, const float* __restrict__ dht, float* __restrict__ dh0,
    const float* __restrict__ cum, const float* __restrict__ ca) {
  typedef ScanBwdLds<E, DK, DV, TV, GT> L;
  constexpr bool XF = L::XF;
  typedef typename Mma<E>::vec V;
  constexpr int KC = Mma<E>::KC, KS = DK / KC, KT = kChunk / KC;
  constexpr int NTILE = DV / TV;
  constexpr int NB = TV / 16;
  constexpr int TPW = (DK / 16) * NB / 4;
  constexpr int VE = 16 / (int)sizeof(E);
  constexpr int VQ = 64 * DK / VE / kThreads;      // Q (and W) vectors per thread
  constexpr int VM = 64 * 64 / VE / kThreads;      // M vectors per thread
  constexpr int OPR = TV / VE;                     // dO vectors per row
  constexpr int VO = (64 * OPR + kThreads - 1) / kThreads;
  static_assert(TPW >= 1 && ((DK / 16) * NB) % 4 == 0, "state tiles must split over 4 waves");
  static_assert(VQ >= 1 && VM >= 1 && (64 * DK / VE) % kThreads == 0, "tile split");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  lds_poison(smem);
  E* sG = (E*)(smem + L::oG);
  E* sDt = (E*)(smem + L::oDt);
  E* sDu = (E*)(smem + L::oDu);

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int sh, tile;
  scan_block(blockIdx.x, g.n_seqs * g.H, NTILE, sh, tile);
  const int s = sh / g.H, h = sh % g.H;
  const SeqInfo si = seq_info(g, s);
  const int nchunks = seq_chunks(g, si);
  const int v0 = tile * TV;
  const int rA = 16 * wv;
  const int64_t base = (int64_t)(si.b * g.H + h) * g.T + si.bos;

  constexpr bool OUT = MODE == 0;  // write dU~ and dS_c
  V kA[KS], kN[KS];
  u32x4 qR[VQ], wR[VQ], mR[VM], xR[VM], oR[VO];
  float cQ[VQ], cR = 0.f, aR = 0.f;  // gated: running log-decay sums of the Q rows / of token
                                     // lane; XF: alpha~ of token lane

  auto load_chunk = [&](int c) {
    const int n = min(kChunk, si.len - c * kChunk);
    const int64_t r0 = base + (int64_t)c * kChunk;
    const int ra = min(rA + (lane & 15), n - 1) - (lane & 15);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kN[ks] = frag_rm<E>(k + (r0 + ra) * DK + ks * KC, DK, lane);
    const int64_t unit = (int64_t)(si.slot0 + c) * g.H + h;
#pragma unroll
    for (int it = 0; it < VQ; ++it) {
      const int i = it * kThreads + tid;
      const int r = min(i / (DK / VE), n - 1), cc = (i % (DK / VE)) * VE;
      qR[it] = *(const u32x4*)(q + (r0 + r) * DK + cc);
      if constexpr (!XF) wR[it] = *(const u32x4*)(w + (r0 + r) * DK + cc);
      if constexpr (GT) cQ[it] = cum[unit * kChunk + r];
    }
    if constexpr (GT) cR = cum[unit * kChunk + lane];
    if constexpr (XF) {  // X [64][64] of the chunk and alpha~
      const E* xc = w + unit * kChunk * kChunk;
#pragma unroll
      for (int it = 0; it < VM; ++it) xR[it] = *(const u32x4*)(xc + (it * kThreads + tid) * VE);
      aR = ca[unit * kChunk + lane];
    }
    {  // M and dO (the dO term)
      const E* mc = m + ((int64_t)(si.slot0 + c) * g.H + h) * kChunk * kChunk;
#pragma unroll
      for (int it = 0; it < VM; ++it) mR[it] = *(const u32x4*)(mc + (it * kThreads + tid) * VE);
#pragma unroll
      for (int it = 0; it < VO; ++it) {  // unconditional (clamped) so no load sits in a branch
        const int i = min(it * kThreads + tid, 64 * OPR - 1);
        const int r = min(i / OPR, n - 1), cc = (i % OPR) * VE;
        oR[it] = *(const u32x4*)(d_o + (r0 + r) * DV + v0 + cc);
      }
    }
  };
  auto commit_chunk = [&](int c, unsigned char* st) {
    const int n = min(kChunk, si.len - c * kChunk);
    E* sQ = (E*)(st + L::oQ);
    E* sW = (E*)(st + L::oW);
    E* sM = (E*)(st + L::oM);
    E* sO = (E*)(st + L::oO);
    const bool rowok = rA + (lane & 15) < n;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kA[ks] = keep_if_vec(kN[ks], rowok);
    if constexpr (XF) {  // this wave's K rows into the K tile (W's place), rows >= n zero
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        *(V*)(sW + (rA + (lane & 15)) * L::LK + ks * KC + (lane >> 4) * (KC / 4)) = kA[ks];
      E* sX = (E*)(st + L::oX);
#pragma unroll
      for (int it = 0; it < VM; ++it) {
        const int i = (it * kThreads + tid) * VE;
        *(u32x4*)(sX + (i / 64) * L::LT + i % 64) = xR[it];
      }
      if (tid < 64) ((float*)(st + L::oAl))[tid] = aR;
    }
#pragma unroll
    for (int it = 0; it < VQ; ++it) {
      const int i = it * kThreads + tid;
      const int r = i / (DK / VE), cc = (i % (DK / VE)) * VE;
      if constexpr (!XF) *(u32x4*)(sW + r * L::LK + cc) = keep_if(wR[it], r < n);
      u32x4 qv = qR[it];
      if constexpr (GT) {  // Q rows scaled by Gamma = e^c
        const float gm = exp_decay(cQ[it]);
        V x = __builtin_bit_cast(V, qv);
#pragma unroll
        for (int e = 0; e < VE; ++e) x[e] = to_e<E>(to_f(x[e]) * gm);
        qv = __builtin_bit_cast(u32x4, x);
      }
      *(u32x4*)(sQ + r * L::LK + cc) = keep_if(qv, r < n);
    }
    if constexpr (GT) {
      if (tid < 64) ((float*)(st + L::oCs))[tid] = cR;
    }
    {
#pragma unroll
      for (int it = 0; it < VM; ++it) {
        const int i = (it * kThreads + tid) * VE;
        *(u32x4*)(sM + (i / 64) * L::LT + i % 64) = mR[it];
      }
#pragma unroll
      for (int it = 0; it < VO; ++it) {
        const int i = it * kThreads + tid;
        if (i < 64 * OPR) {
          const int r = i / OPR, cc = (i % OPR) * VE;
          *(u32x4*)(sO + r * L::LS + cc) = keep_if(oR[it], r < n);
        }
      }
    }
  };

  // G^T tile t = wv + 4 i holds G[16 db + (lane & 15)][v0 + 16 vb + 4 (lane >> 4) + e];
  // dht / dh0: fp32 [n_seqs][H][DK][DV] gradients at the state leaving / entering the sequence
  f32x4 Gt[TPW];
  auto goff = [&](int i, int e) {
    const int t = wv + 4 * i, vb = t % NB, db = t / NB;
    return ((int64_t)s * g.H + h) * DK * DV + (int64_t)(16 * db + (lane & 15)) * DV + v0 + 16 * vb +
           4 * (lane >> 4) + e;
  };
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    Gt[i] = zero4();
    if (dht) {
#pragma unroll
      for (int e = 0; e < 4; ++e) Gt[i][e] = dht[goff(i, e)];
    }
  }
  // L2 warm-up two chunks ahead of the compute (one word per 128-byte line; the workgroups of
  // the (sequence, head) split the shared tiles): the register loads of chunk c - 1, issued a
  // step later, then hit L2, and HBM keeps a request stream across the barriers. Each warm-up is
  // consumed right after the next step's register loads are issued, so it is waited for there,
  // a step after it was issued, and never together with a load still in flight.
  constexpr int NL = (64 * (DK > DV ? DK : DV) * (int)sizeof(E) / 128 + NTILE * kThreads - 1) /
                     (NTILE * kThreads);
  int pw[5 * NL];
#pragma unroll
  for (int i = 0; i < 5 * NL; ++i) pw[i] = 0;
  auto warm = [&](int c) {
    const int n = min(kChunk, si.len - c * kChunk);
    const int64_t r0 = base + (int64_t)c * kChunk;
    const int bk = n * DK * (int)sizeof(E);
    if constexpr (XF)
      l2_touch<NL, kThreads>(pw, w + ((int64_t)(si.slot0 + c) * g.H + h) * kChunk * kChunk,
                             kChunk * kChunk * (int)sizeof(E), tile, NTILE, tid);
    else
      l2_touch<NL, kThreads>(pw, w + r0 * DK, bk, tile, NTILE, tid);
    l2_touch<NL, kThreads>(pw + NL, k + r0 * DK, bk, tile, NTILE, tid);
    {
      l2_touch<NL, kThreads>(pw + 2 * NL, q + r0 * DK, bk, tile, NTILE, tid);
      l2_touch<NL, kThreads>(pw + 3 * NL, m + ((int64_t)(si.slot0 + c) * g.H + h) * kChunk * kChunk,
                             kChunk * kChunk * (int)sizeof(E), tile, NTILE, tid);
      l2_touch<NL, kThreads>(pw + 4 * NL, d_o + r0 * DV, n * DV * (int)sizeof(E), tile, NTILE, tid);
    }
  };
  if (nchunks > 0) {
    load_chunk(nchunks - 1);
    warm(max(nchunks - 2, 0));  // unconditional, like every warm-up: a load in a branch would
                                // make the compiler's wait counts assume the worst path
    commit_chunk(nchunks - 1, smem + (L::NSTG == 2 ? ((nchunks - 1) & 1) : 0) * L::stage);
  }

  for (int c = nchunks - 1; c >= 0; --c) {
    unsigned char* stc = smem + (L::NSTG == 2 ? (c & 1) : 0) * L::stage;
    const E* sQ = (const E*)(stc + L::oQ);
    const E* sW = (const E*)(stc + L::oW);
    const E* sM = (const E*)(stc + L::oM);
    const E* sO = (const E*)(stc + L::oO);
    const float* sCs = (const float*)(stc + L::oCs);
    const int n = min(kChunk, si.len - c * kChunk);
    const int64_t r0 = base + (int64_t)c * kChunk;
    // Stage G (gradient of the state leaving chunk c): G^T tiles written transposed.
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = wv + 4 * i, vb = t % NB, db = t / NB;
      st_frag_t<E>(sG + 16 * db * L::LS + 16 * vb, L::LS, Gt[i], lane);
    }
    const bool more = c > 0;
    load_chunk(more ? c - 1 : c);
    l2_sink<5 * NL>(pw);
    warm(max(c - 2, 0));
    __syncthreads();

    if constexpr (OUT) {  // G of this slot -> dstates [d][v0 : v0 + TV]
      E* gG = dstates + ((int64_t)(si.slot0 + c) * g.H + h) * DK * DV + v0;
      constexpr int VPR = TV / VE;
      // no store in a branch (see s2g): work past the end repeats the last vector
#pragma unroll
      for (int it = 0; it < (DK * VPR + kThreads - 1) / kThreads; ++it) {
        const int i = min(it * kThreads + tid, DK * VPR - 1), d = i / VPR, cc = (i % VPR) * VE;
        *(u32x4*)(gG + (int64_t)d * DV + cc) = *(const u32x4*)(sG + d * L::LS + cc);
      }
    }
    // dU~ = scale M^T dO + K G for this wave's rows (tokens j).
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      f32x4 kg = zero4(), md = zero4();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kg = Mma<E>::step(kA[ks], frag_km<E>(sG + ks * KC * L::LS + 16 * nb, L::LS, lane), kg);
      md = mma<E, true, true>(sM + rA, L::LT, sO + 16 * nb, L::LS, round_down_kc<E>(rA), kChunk, md, lane);
      if constexpr (GT) {  // rows t of K G decay by e^{c_last - c_t}
        const float cl = sCs[n - 1];
#pragma unroll
        for (int i = 0; i < 4; ++i) kg[i] *= exp_decay(cl - sCs[rA + 4 * (lane >> 4) + i]);
      }
      f32x4 du = kg + g.scale * md;
      st_frag_t<E>(sDt + 16 * nb * L::LT + rA, L::LT, du, lane);
      if constexpr (OUT) st_frag_lds<E>(sDu + rA * L::LS + 16 * nb, L::LS, du, lane);
    }
    // scale dO^T Q for every G^T tile of the wave: independent of dU~, so it runs before the
    // barrier that waits for every wave's dU~
    f32x4 ga[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = wv + 4 * i, vb = t % NB, db = t / NB;
      ga[i] = g.scale * mma<E, true, true>(sO + 16 * vb, L::LS, sQ + 16 * db, L::LK, 0, kChunk, zero4(), lane);
    }
    f32x4 al4[4];  // XF: alpha~ of the rows of Z below (four consecutive rows per tile)
    if constexpr (XF) {
#pragma unroll
      for (int sb = 0; sb < 4; ++sb)
        al4[sb] = *(const f32x4*)((const float*)(stc + L::oAl) + prow<E>(sb, 4 * (lane >> 4)));
    }
    __syncthreads();

    if constexpr (OUT) s2g<E, TV>(dut + r0 * DV + v0, DV, sDu, L::LS, n, tid);
    // XF: dU~^T W = Z^T K with Z = diag(alpha~) X^T dU~, formed by every wave for its columns
    // (vb = wv % NB for all of its G^T tiles) with rows in prow order, packed straight into the
    // A operand of Z^T K; row pair j of Z needs t >= 32 j (X is lower triangular).
    V zA[KT];
    if constexpr (XF) {
      const int vb = wv % NB;
      const E* sX = (const E*)(stc + L::oX);
      f32x4 z[4];
#pragma unroll
      for (int sb = 0; sb < 4; ++sb) {
        z[sb] = zero4();
#pragma unroll
        for (int kt = sb >> 1; kt < KT; ++kt)
          z[sb] = Mma<E>::step(aop_kc_ld<E>(sX, L::LT, sb, kt, lane),
                               frag_rm<E>(sDt + 16 * vb * L::LT + KC * kt, L::LT, lane), z[sb]);
        z[sb] *= al4[sb];
      }
#pragma unroll
      for (int j = 0; j < KT; ++j) zA[j] = bop_acc<E>(z, j);
    }
    // G^T += scale dO^T Q - dU~^T W (gated: G^T <- e^{c_last} G^T + ..., Q pre-scaled)
    const float gC = GT ? exp_decay(sCs[n - 1]) : 1.f;
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = wv + 4 * i, vb = t % NB, db = t / NB;
      f32x4 b = zero4();
      if constexpr (XF) {
#pragma unroll
        for (int j = 0; j < KT; ++j) b = Mma<E>::step(zA[j], frag_km<E>(sW + KC * j * L::LK + 16 * db, L::LK, lane), b);
      } else {
        b = mma<E, false, true>(sDt + 16 * vb * L::LT, L::LT, sW + 16 * db, L::LK, 0, kChunk, zero4(), lane);
      }
      Gt[i] = gC * Gt[i] + (ga[i] - b);
    }
    if constexpr (L::NSTG == 1) __syncthreads();  // every wave is done with the stage
    if (more) commit_chunk(c - 1, smem + (L::NSTG == 2 ? ((c - 1) & 1) : 0) * L::stage);
  }
  if (dh0) {  // gradient at the state entering the sequence
#pragma unroll
    for (int i = 0; i < TPW; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) dh0[goff(i, e)] = Gt[i][e];
  }
}

// DMA-fed variant for bf16 problems with 32-column tiles, organised like the forward
// scan: a loader wave fills swizzled LDS tiles of K, Q, W, M and dO one chunk ahead by LDS DMA
// and warms L2 for the chunk after, and a storer wave copies the staged G and dU~ out, so the
// four compute waves issue no global memory operation in the loop. The loader's barriers are
// bare s_barriers (a fence would wait for every load in flight); before the one that publishes
// a chunk it waits for the DMA only, by a counted vmcnt that leaves the younger warm-up loads in
// flight. Rows past the end of a partial chunk, which the DMA fills with copies of the last row,
// are cleared by the loader (the products over tokens need zeros there). The storer reads the G
// staging between the step's two barriers and dU~ after the second, before the compute waves
// write either again. Gated EFLA (GT) as in the
// register-fed kernel: the loader also stages the chunk's running log-decay sums and Gamma, Q
// elements are scaled by Gamma as they are read (rounded as the register-fed kernel rounds them
// when they land), and the decays of K G and of G act on registers.
template <typename E, int DK, int DV, bool GT = false>
struct ScanBwdDmaLds {
  static constexpr int TV = 32;
  typedef Swz<E, DK> SK;  // K, Q [64][DK]
  typedef Swz<E, 64> SM;  // X, M [64][64]
  typedef Swz<E, TV> SO;  // dO [64][TV] (this tile's columns)
  static constexpr int LS = pitch<E>(TV), LT = pitch<E>(64);
  static constexpr size_t oK = 0, oQ = oK + SK::BYTES, oX = oQ + SK::BYTES, oM = oX + SM::BYTES;
  static constexpr size_t oO = oM + SM::BYTES;
  static constexpr size_t oCs = oO + SO::BYTES;  // running log-decay sums c [64] (GT)
  static constexpr size_t oGm = oCs + 64 * 4;     // Gamma = e^c [64] (GT)
  static constexpr size_t oAl = oCs + (GT ? 2 * 64 * 4 : 0);  // alpha~ [64]
  static constexpr size_t stage = oAl + 64 * 4;
  static constexpr size_t oG = 2 * stage;                   // G slice [DK][LS]
  static constexpr size_t oDt = oG + DK * LS * sizeof(E);   // dU~^T [TV][LT]
  static constexpr size_t oDu = oDt + TV * LT * sizeof(E);  // dU~ staging [64][LS]
  static constexpr size_t oDummy = oDu + 64 * LS * sizeof(E);  // 256 bytes: L2 warm-up landing
  static constexpr size_t bytes = oDummy + 256;
};

constexpr int kScanBwdDmaThreads = 6 * 64;  // four compute waves, the loader and the storer

template <typename E, int DK, int DV, bool GT, int MODE>
__global__ __launch_bounds__(kScanBwdDmaThreads, 1) void scan_bwd_dma_kernel(
    Geom g, const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ x,
    const E* __restrict__ m, const E* __restrict__ d_o, E* __restrict__ dut,
    E* __restrict__ dstates, const float* __restrict__ dht, float* __restrict__ dh0,
    const float* __restrict__ cum, const float* __restrict__ ca) {
  typedef ScanBwdDmaLds<E, DK, DV, GT> L;
  typedef typename Mma<E>::vec V;
  constexpr int TV = L::TV, LS = L::LS, LT = L::LT;
  constexpr int KC = Mma<E>::KC, KS = DK / KC;
  constexpr int NTILE = DV / TV;
  constexpr int NB = TV / 16;
  constexpr int TPW = (DK / 16) * NB / 4;
  constexpr int VE = 16 / (int)sizeof(E);
  constexpr bool OUT = MODE == 0;  // write dU~ and dS_c
  static_assert(TPW >= 1 && ((DK / 16) * NB) % 4 == 0, "state tiles must split over 4 waves");
  static_assert(L::bytes <= 160 * 1024, "LDS budget");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  lds_poison(smem);
  E* sG = (E*)(smem + L::oG);
  E* sDt = (E*)(smem + L::oDt);
  E* sDu = (E*)(smem + L::oDu);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  int sh, tile;
  scan_block(blockIdx.x, g.n_seqs * g.H, NTILE, sh, tile);
  const int s = sh / g.H, h = sh % g.H;
  const SeqInfo si = seq_info(g, s);
  const int nchunks = seq_chunks(g, si);
  const int v0 = tile * TV;
  const int64_t base = (int64_t)(si.b * g.H + h) * g.T + si.bos;
  auto rows_of = [&](int c) { return min(kChunk, si.len - c * kChunk); };
  auto tiles = [&](int c) { return smem + (c & 1) * L::stage; };

  constexpr int NL = (64 * (DK > DV ? DK : DV) * (int)sizeof(E) / 128 + NTILE * 64 - 1) / (NTILE * 64);
  constexpr int NWARM = NL * 5;  // warm-up loads issued after each DMA: X, K, Q, M, dO
  static_assert(NWARM <= 15, "vmcnt field");
  static_assert(sizeof(E) == 2, "bf16 tiles (the transposed products use 32-wide steps)");
  if (wv == 4) {  // ---- loader wave
    // one word per 128-byte line (the head's workgroups split the lines), by LDS DMA into a row
    // that nothing reads: no register waits for these loads, only the counted waits see them
    unsigned char* dummy = smem + L::oDummy;
    auto warm = [&](int c) {
      const int n = rows_of(c);
      const int64_t r0 = base + (int64_t)c * kChunk;
      const int bk = n * DK * (int)sizeof(E);
      l2_touch_lds<NL>(dummy, x + ((int64_t)(si.slot0 + c) * g.H + h) * kChunk * kChunk,
                       kChunk * kChunk * (int)sizeof(E), tile, NTILE, lane);
      l2_touch_lds<NL>(dummy, k + r0 * DK, bk, tile, NTILE, lane);
      l2_touch_lds<NL>(dummy, q + r0 * DK, bk, tile, NTILE, lane);
      l2_touch_lds<NL>(dummy, m + ((int64_t)(si.slot0 + c) * g.H + h) * kChunk * kChunk,
                       kChunk * kChunk * (int)sizeof(E), tile, NTILE, lane);
      l2_touch_lds<NL>(dummy, d_o + r0 * DV, n * DV * (int)sizeof(E), tile, NTILE, lane);
      __builtin_amdgcn_sched_barrier(0);  // every request ahead of what follows (counted waits)
    };
    // the DMA has landed: vmcnt(NWARM) leaves only the younger warm-up loads in flight
    auto wait_dma = [&]() { __builtin_amdgcn_s_waitcnt(0x0F70 | NWARM); };
    auto issue = [&](int c) {
      unsigned char* st = tiles(c);
      const int n = rows_of(c);
      const int64_t r0 = base + (int64_t)c * kChunk;
      const int64_t unit = (int64_t)(si.slot0 + c) * g.H + h;
      dma_tile<E, DK, 1>(st + L::oK, k + r0 * DK, DK, n, 0, lane);
      dma_tile<E, 64, 1>(st + L::oX, x + unit * kChunk * kChunk, kChunk, kChunk, 0, lane);
      {  // Q, M and dO (the dO term)
        dma_tile<E, DK, 1>(st + L::oQ, q + r0 * DK, DK, n, 0, lane);
        dma_tile<E, 64, 1>(st + L::oM, m + ((int64_t)(si.slot0 + c) * g.H + h) * kChunk * kChunk,
                           kChunk, kChunk, 0, lane);
        dma_tile<E, TV, 1>(st + L::oO, d_o + r0 * DV + v0, DV, n, 0, lane);
      }
      // the per-token vectors (64 floats each) by LDS DMA as well: alpha~, and the running
      // log-decay sums (gated)
      dma_vec64(st + L::oAl, ca + unit * kChunk, lane);
      if constexpr (GT) dma_vec64(st + L::oCs, cum + unit * kChunk, lane);
      // the counted waits assume every request above is issued before the warm-up loads that
      // follow: keep the scheduler from moving any of them past this point
      __builtin_amdgcn_sched_barrier(0);
    };
    auto finish = [&](int c) {  // after the wait: Gamma = e^c (gated), rows >= n cleared
      unsigned char* st = tiles(c);
      if constexpr (GT)
        ((float*)(st + L::oGm))[lane] = exp_decay(((const float*)(st + L::oCs))[lane]);
      const int n = rows_of(c);
      if (n >= kChunk) return;  // whole rows are cleared: the swizzle stays inside a row
      const u32x4 z = {0u, 0u, 0u, 0u};
      for (int b = n * L::SK::RB + 16 * lane; b < kChunk * L::SK::RB; b += 16 * 64) {
        *(u32x4*)(st + L::oK + b) = z;
        *(u32x4*)(st + L::oQ + b) = z;
      }
        for (int b = n * L::SO::RB + 16 * lane; b < kChunk * L::SO::RB; b += 16 * 64)
          *(u32x4*)(st + L::oO + b) = z;
    };
    if (nchunks > 0) {
      issue(nchunks - 1);
      warm(max(nchunks - 2, 0));
      wait_dma();
      finish(nchunks - 1);
    }
    for (int c = nchunks - 1; c >= 0; --c) {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): finish's LDS writes are done
      __builtin_amdgcn_s_barrier();  // chunk c is in LDS; every wave is done with chunk c + 1's stage
      if (c > 0) issue(c - 1);
      __builtin_amdgcn_s_barrier();  // the step's second barrier
      warm(max(c - 2, 0));
      if (c > 0) {
        wait_dma();
        finish(c - 1);
      }
    }
    wait_vm_all();
    return;
  }

  if (wv == 5) {  // ---- storer wave (lane: its thread index)
    for (int c = nchunks - 1; c >= 0; --c) {
      __syncthreads();  // G of chunk c is staged
      if constexpr (OUT) {  // G of this slot -> dstates [d][v0 : v0 + TV] (no store in a branch)
        E* gG = dstates + ((int64_t)(si.slot0 + c) * g.H + h) * DK * DV + v0;
        constexpr int VPR = TV / VE;
#pragma unroll
        for (int it = 0; it < (DK * VPR + 63) / 64; ++it) {
          const int i = min(it * 64 + lane, DK * VPR - 1), d = i / VPR, cc = (i % VPR) * VE;
          *(u32x4*)(gG + (int64_t)d * DV + cc) = *(const u32x4*)(sG + d * LS + cc);
        }
      }
      __syncthreads();  // dU~ of chunk c is staged
      if constexpr (OUT) s2g<E, TV, 64>(dut + (base + (int64_t)c * kChunk) * DV + v0, DV, sDu, LS, rows_of(c), lane);
    }
    return;
  }

  // ---- compute waves: G^T tile t = wv + 4 i holds G[16 db + (lane & 15)][v0 + 16 vb + 4 (lane >> 4) + e]
  const int rA = 16 * wv;
  f32x4 Gt[TPW];
  auto goff = [&](int i, int e) {
    const int t = wv + 4 * i, vb = t % NB, db = t / NB;
    return ((int64_t)s * g.H + h) * DK * DV + (int64_t)(16 * db + (lane & 15)) * DV + v0 + 16 * vb +
           4 * (lane >> 4) + e;
  };
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    Gt[i] = zero4();
    if (dht) {
#pragma unroll
      for (int e = 0; e < 4; ++e) Gt[i][e] = dht[goff(i, e)];
    }
  }
  for (int c = nchunks - 1; c >= 0; --c) {
    const unsigned char* st = tiles(c);
    const int n = rows_of(c);
    const float* sCs = (const float*)(st + L::oCs);
    const float* sGm = (const float*)(st + L::oGm);
    // Stage G (gradient of the state leaving chunk c): G^T tiles written transposed.
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = wv + 4 * i, vb = t % NB, db = t / NB;
      st_frag_t<E>(sG + 16 * db * LS + 16 * vb, LS, Gt[i], lane);
    }
    __syncthreads();

    V kA[KS];  // this wave's K rows (A operand of K G)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kA[ks] = frag_rm_sw<E, DK>(st + L::oK, rA, ks * KC, lane);
    // alpha~ of the rows of Z below (four consecutive rows per tile: one 16-byte read each)
    f32x4 al4[4];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) al4[sb] = *(const f32x4*)((const float*)(st + L::oAl) + prow<E>(sb, 4 * (lane >> 4)));
    // dU~ = scale M^T dO + K G for this wave's rows (tokens).
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      f32x4 kg = zero4(), md = zero4();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kg = Mma<E>::step(kA[ks], frag_km<E>(sG + ks * KC * LS + 16 * nb, LS, lane), kg);
      {  // M^T[t][s] = M[s][t]: k-major from M's rows s >= t
        for (int k0 = round_down_kc<E>(rA); k0 < kChunk; k0 += KC)
          md = Mma<E>::step(frag_km_sw<E, 64>(st + L::oM, k0, rA, lane),
                            frag_km_sw<E, TV>(st + L::oO, k0, 16 * nb, lane), md);
      }
      if constexpr (GT) {  // rows t of K G decay by e^{c_last - c_t}
        const float cl = sCs[n - 1];
#pragma unroll
        for (int i = 0; i < 4; ++i) kg[i] *= exp_decay(cl - sCs[rA + 4 * (lane >> 4) + i]);
      }
      f32x4 du = kg + g.scale * md;
      st_frag_t<E>(sDt + 16 * nb * LT + rA, LT, du, lane);
      if constexpr (OUT) st_frag_lds<E>(sDu + rA * LS + 16 * nb, LS, du, lane);
    }
    // scale dO^T Q for every G^T tile of the wave (gated: Q scaled by Gamma): independent of
    // dU~, so it runs before the barrier that waits for every wave's dU~
    f32x4 ga[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = wv + 4 * i, vb = t % NB, db = t / NB;
      f32x4 a = zero4();
#pragma unroll
      for (int k0 = 0; k0 < kChunk; k0 += KC) {
        V qf = frag_km_sw<E, DK>(st + L::oQ, k0, 16 * db, lane);
        if constexpr (GT) {  // element e is token k0 + KC/4 (lane >> 4) + e
          const int t0 = k0 + (KC / 4) * (lane >> 4);
#pragma unroll
          for (int e = 0; e < KC / 4; ++e) qf[e] = to_e<E>(to_f(qf[e]) * sGm[t0 + e]);
        }
        a = Mma<E>::step(frag_km_sw<E, TV>(st + L::oO, k0, 16 * vb, lane), qf, a);
      }
      ga[i] = g.scale * a;
    }
    __syncthreads();

    // dU~^T W with W = X diag(alpha~) K is Z^T K, Z = diag(alpha~) X^T dU~: the wave forms Z for
    // its 16 columns (every G^T tile of the wave has vb = wv % NB), rows in prow order, so that
    // it packs straight into the A operand of Z^T K. Row pair j of Z needs t >= 32 j (X is
    // lower triangular): 6 products.
    V zA[kChunk / KC];
    {
      const int vb = wv % NB;
      f32x4 z[4];
#pragma unroll
      for (int sb = 0; sb < 4; ++sb) {
        z[sb] = zero4();
#pragma unroll
        for (int kt = sb >> 1; kt < kChunk / KC; ++kt)
          z[sb] = Mma<E>::step(aop_kc<E, 64>(st + L::oX, sb, kt, lane),
                               frag_rm<E>(sDt + 16 * vb * LT + KC * kt, LT, lane), z[sb]);
        z[sb] *= al4[sb];
      }
#pragma unroll
      for (int j = 0; j < kChunk / KC; ++j) zA[j] = bop_acc<E>(z, j);
    }
    // G^T <- gC G^T + scale dO^T Q - Z^T K (gated: gC = e^{c_last})
    const float gC = GT ? exp_decay(sCs[n - 1]) : 1.f;
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = wv + 4 * i, db = t / NB;
      f32x4 b = zero4();
#pragma unroll
      for (int k0 = 0; k0 < kChunk; k0 += KC)
        b = Mma<E>::step(zA[k0 / KC], frag_km_sw<E, DK>(st + L::oK, k0, 16 * db, lane), b);
      Gt[i] = gC * Gt[i] + (ga[i] - b);
    }
  }
  if (dh0) {  // gradient at the state entering the sequence
#pragma unroll
    for (int i = 0; i < TPW; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) dh0[goff(i, e)] = Gt[i][e];
  }
}

template <typename E, int DK, int DV, bool GT, int MODE>
static hipError_t scan_bwd_dma_run(const Shape& s, const int* table, const void* q, const void* k,
                                   const void* w, const void* m, const void* d_o, void* dut,
                                   void* dstates, const float* dht, float* dh0, hipStream_t st,
                                   const float* cum, const float* ca) {
  typedef ScanBwdDmaLds<E, DK, DV, GT> L;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)scan_bwd_dma_kernel<E, DK, DV, GT, MODE>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)L::bytes);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const int64_t blocks = (int64_t)s.n_seqs * s.H * (DV / L::TV);
  if (blocks < 1) return hipSuccess;
  prof_begin(st);
  hipLaunchKernelGGL((scan_bwd_dma_kernel<E, DK, DV, GT, MODE>), dim3((unsigned)blocks), dim3(kScanBwdDmaThreads),
                     L::bytes, st, make_geom(s, table), (const E*)q, (const E*)k, (const E*)w,
                     (const E*)m, (const E*)d_o, (E*)dut, (E*)dstates, dht, dh0, cum, ca);
  hipError_t e = hipGetLastError();
  static const char* const names[2][2] = {{"scan_bwd", "scan_bwd_state"},
                                           {"scan_bwd_gated", "scan_bwd_state_gated"}};
  prof_end(names[GT][MODE], st);
  return e;
}

template <typename E, int DK, int DV, int TV, bool GT, int MODE>
static hipError_t scan_bwd_run(const Shape& s, const int* table, const void* q, const void* k,
                               const void* w, const void* m, const void* d_o, void* dut,
                               void* dstates, const float* dht, float* dh0, hipStream_t st,
                               const float* cum, const float* ca) {
  typedef ScanBwdLds<E, DK, DV, TV, GT> L;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)scan_bwd_kernel<E, DK, DV, TV, GT, MODE>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)L::bytes);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const int64_t blocks = (int64_t)s.n_seqs * s.H * (DV / TV);
  if (blocks < 1) return hipSuccess;
  prof_begin(st);
  hipLaunchKernelGGL((scan_bwd_kernel<E, DK, DV, TV, GT, MODE>), dim3((unsigned)blocks), dim3(kThreads),
                     L::bytes, st, make_geom(s, table), (const E*)q, (const E*)k, (const E*)w,
                     (const E*)m, (const E*)d_o, (E*)dut, (E*)dstates, dht, dh0, cum, ca);
  hipError_t e = hipGetLastError();
  static const char* const names[2][2] = {{"scan_bwd", "scan_bwd_state"},
                                           {"scan_bwd_gated", "scan_bwd_state_gated"}};
  prof_end(names[GT][MODE], st);
  return e;
}

template <typename E, int DK, int DV, int TV, int MODE>
static hipError_t scan_bwd_mode(const Shape& s, const int* table, const void* q, const void* k,
                                const void* w, const void* m, const void* d_o, void* dut,
                                void* dstates, const float* dht, float* dh0, hipStream_t st,
                                const float* cum, const float* ca) {
  if (cum) {
    if constexpr (sizeof(E) == 2 && TV == 32)
      return scan_bwd_dma_run<E, DK, DV, true, MODE>(s, table, q, k, w, m, d_o, dut, dstates, dht, dh0, st, cum, ca);
    else if constexpr (sizeof(E) == 2)
      return scan_bwd_run<E, DK, DV, TV, true, MODE>(s, table, q, k, w, m, d_o, dut, dstates, dht, dh0, st, cum, ca);
    else
      return hipErrorInvalidValue;
  }
  if constexpr (sizeof(E) == 2 && TV == 32)
    return scan_bwd_dma_run<E, DK, DV, false, MODE>(s, table, q, k, w, m, d_o, dut, dstates, dht, dh0, st, cum, ca);
  else
    return scan_bwd_run<E, DK, DV, TV, false, MODE>(s, table, q, k, w, m, d_o, dut, dstates, dht, dh0, st, cum, ca);
}

template <typename E, int DK, int DV, int TV>
static hipError_t scan_bwd_go(const Shape& s, const int* table, const void* q, const void* k,
                              const void* w, const void* m, const void* d_o, void* dut,
                              void* dstates, const float* dht, float* dh0, hipStream_t st,
                              const float* cum, const float* ca, int mode) {
  if (mode == 1)
    return scan_bwd_mode<E, DK, DV, TV, 1>(s, table, q, k, w, m, d_o, dut, dstates, dht, dh0, st, cum, ca);
  return scan_bwd_mode<E, DK, DV, TV, 0>(s, table, q, k, w, m, d_o, dut, dstates, dht, dh0, st, cum, ca);
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
                           const void* w, const void* m, const void* d_o, void* dut,
                           void* dstates, const float* dht, float* dh0, hipStream_t st,
                           const float* cum, const float* ca, bool state_only) {
  const int mode = state_only ? 1 : 0;
#define EFLA_SB(E_, DK_, DV_, TV_) \
  return scan_bwd_go<E_, DK_, DV_, TV_>(s, table, q, k, w, m, d_o, dut, dstates, dht, dh0, st, cum, ca, mode)
  if (s.dt == Dt::BF16) {
    if (s.dk == 64 && s.dv == 64) EFLA_SB(__bf16, 64, 64, 16);
    if (s.dk == 128 && s.dv == 64) EFLA_SB(__bf16, 128, 64, 16);
    if (scan_tile(s) == 16) {
      if (s.dk == 64) EFLA_SB(__bf16, 64, 128, 16);
      EFLA_SB(__bf16, 128, 128, 16);
    }
    if (s.dk == 64) EFLA_SB(__bf16, 64, 128, 32);
    EFLA_SB(__bf16, 128, 128, 32);
  }
  EFLA_SB(float, 64, 64, 16);
#undef EFLA_SB
}

}  // namespace efla


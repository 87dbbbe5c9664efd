// Inter-chunk state recurrence fused with the chunk output.
//
// Exact Flow Linear Attention summary page, section 3.3 (chunk-level recurrence and
// outputs). One workgroup walks the chunks of one (sequence, head) in order and owns a
// d_k x TV slice of the state (TV = 16 columns per wave):
//   U~ = U - W S,   O = scale (Q S + M U~),   S <- S + K^T U~,
// with M = tril(Q K^T) (fp32: from the UT kernel; bf16: formed here from the staged Q and K
// tiles, and written out for the backward when a saved buffer is given). The diagonal of tril is
// kept because token t reads the state after its own update. bf16 problems read the UT factor
// X = (I + A)^{-1}, V
// and the per-token scales alpha~ (gated alpha e^{c}) and b instead of W = X diag(alpha~) K
// and U = X diag(b) V, and form U~ = X Y with Y = diag(b) V - diag(alpha~) K S: one more short
// product per chunk (X is lower triangular) for a quarter of W's bytes and no U at all.
//
// Each compute wave owns 16 columns of S for the whole sequence and keeps them in fp32 MFMA
// accumulators. Products whose contraction runs over the rows of an accumulator take that
// accumulator directly as their B operand, so the recurrence S -> W S (or K S -> Y -> X Y) ->
// U~ -> K^T U~ -> S runs inside one wave's registers with no LDS round trip. Accumulator rows (of S, and the
// token rows of U~ and O) are numbered in the contiguous-contraction order (prow), so every
// A operand from LDS is a single 16-byte read. Two further waves move the data, each in a loop
// of its own with the same barrier sequence: the loader wave fills swizzled LDS tiles of K, Q,
// the factor and U (or V), and M (fp32), one chunk ahead by LDS DMA (double-buffered), forms M
// (bf16) once K and Q have landed, and warms L2 for the chunk after; the storer wave copies the
// staged O, U~ and chunk states (and M's rows) out as 16-byte rows. Kept apart from the loads,
// the output stores are never waited for. One barrier per chunk hands the buffers over.
#include "efla_internal.hpp"

namespace efla {

// WO: O is written (Q and M are staged); WSV: U~ and the chunk states are written. The
// output-free modes (the zero-start and transition scans of the segment-parallel forward) stage
// only the factor, K and U (or V), so two of their workgroups fit on a compute unit.
// XF (bf16): the factor tile is X [64][64] and the per-token scales alpha~ (and b, gated) are
// staged; fp32: the factor tile is W [64][DK] (the fp32 tiles leave no room for the X form).
template <typename E, int DK, int DV, int NWC, bool WO, bool WSV, bool GT = false>
struct ScanFwdLds {
  static constexpr bool XF = sizeof(E) == 2;
  static constexpr int TV = 16 * NWC;
  static constexpr int NWL = 1;  // loader waves (one; a second wave stores the outputs)
  // the [64][DK] tiles (K, Q, and W for fp32) take the conflict-free row mask (MXK, in Swz)
  static constexpr int MXK = 1;
  typedef Swz<E, DK, 0, MXK> SK;
  typedef Swz<E, 64> SM;
  typedef Swz<E, TV, 2> SU;  // read in accumulator layout
  static constexpr size_t oW = 0;                              // X [64][64] (XF) or W [64][DK]
  static constexpr size_t oK = oW + (XF ? SM::BYTES : SK::BYTES);  // K  [64][DK]
  static constexpr size_t oU = oK + SK::BYTES;                 // V (XF) or U [64][TV] (this tile's columns)
  static constexpr size_t oQ = oU + SU::BYTES;                 // Q  [64][DK] (WO)
  static constexpr size_t oM = oQ + (WO ? SK::BYTES : 0);      // M  [64][64] (WO)
  static constexpr size_t oC = oM + (WO ? SM::BYTES : 0);      // running log-decay sums [64] (gated)
  static constexpr size_t oA = oC + (GT ? 64 * 4 : 0);         // alpha~ [64], then b [64] (XF, gated)
  static constexpr size_t stage = oA + (XF ? (GT ? 2 : 1) * 64 * 4 : 0);
  // output staging (layout SU): O [64][TV] (WO), U~ [64][TV] and S [DK][TV] (WSV); two buffers
  static constexpr size_t gO = 0, gUt = WO ? SU::BYTES : 0, gS = gUt + (WSV ? SU::BYTES : 0);
  static constexpr size_t sstage = gS + (WSV ? (size_t)DK * SU::RB : 0);
  static constexpr size_t oStg = 2 * stage;
  // WDMA: 256 bytes that the loader's L2 warm-up requests land in (never read; where LDS has no
  // room, the fp32 tiles at d = 64 with every output, the warm-up loads go to registers)
  static constexpr size_t oDummy = oStg + 2 * sstage;
  static constexpr bool WDMA = oDummy + 256 <= 160 * 1024;
  static constexpr size_t bytes = oDummy + (WDMA ? 256 : 0);
};

// WO: write O (also needs Q and M); WSV: write U~ and the chunk states (saved for the
// backward pass). Compile-time, so the inner loops carry no branches on them.
// GT: gated EFLA. With c_t the running log-decay sum inside the chunk (from the UT kernel),
// O = scale (diag(e^{c}) Q S + M U~) (M carries the decay ratios), and
// S <- e^{c_last} S + K^T diag(e^{c_last - c}) U~; the decays are applied to accumulators.
// PM: transition mode for the segment-parallel scan. The chunk step is affine in the state,
// S <- (I - K^T W) S + K^T U, so running it with U = 0 from S = I (DV = DK) leaves in ht the
// product of the (I - K^T W) over the sequence; U (V) is neither read nor needed.
// Factors: bf16 (XF) w = X [slots][H][64][64], u = V [B][H][T][DV], ca = alpha~ and cb = b
// (gated) [slots][H][64]; fp32 w = W [B][H][T][DK], u = U [B][H][T][DV].
// The scan of one workgroup; bid plays the role of the block index.
template <typename E, int DK, int DV, int NWC, bool WO, bool WSV, bool PM, bool GT>
__device__ __forceinline__ void scan_fwd_body(
    int bid, Geom g, const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ w,
    const E* __restrict__ u, E* __restrict__ m, E* __restrict__ o, E* __restrict__ ut,
    E* __restrict__ states, const float* __restrict__ h0, float* __restrict__ ht,
    const float* __restrict__ cum, const float* __restrict__ ca, const float* __restrict__ cb) {
  typedef ScanFwdLds<E, DK, DV, NWC, WO, WSV, GT> L;
  typedef typename L::SU SU;
  typedef typename Mma<E>::vec V;
  constexpr bool XF = L::XF;
  constexpr int TV = L::TV, NWL = L::NWL, NTILE = DV / TV, KC = Mma<E>::KC;
  constexpr int NBK = DK / 16;                 // accumulator tiles of the state slice
  constexpr int KSK = DK / KC, KST = kChunk / KC;
  constexpr int NTL = 64;                      // storer threads (one wave)
  constexpr int VE = 16 / (int)sizeof(E);
  static_assert(DV % TV == 0, "column tiles");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  lds_poison(smem);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wi = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool loader = wi == NWC, storer = wi == NWC + 1;
  int sh, tile;
  scan_block(bid, g.n_seqs * g.H, NTILE, sh, tile);
  const int s = sh / g.H, h = sh % g.H;
  const SeqInfo si = seq_info(g, s);
  const int nchunks = seq_chunks(g, si);
  const int v0 = tile * TV;          // first column of this workgroup
  const int cw = 16 * wi;            // first column of this (compute) wave inside the tile
  const int g4 = 4 * (lane >> 4), cl = lane & 15;
  // h0 / ht: fp32 [n_seqs][H][DK][DV]; this wave's columns
  const int64_t hoff = ((int64_t)s * g.H + h) * DK * DV + v0 + cw + cl;
  if (nchunks <= 0) {  // empty sequence: the state passes through
    if (ht && !loader && !storer) {
#pragma unroll
      for (int b = 0; b < NBK; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t o_ = hoff + (int64_t)prow<E>(b, g4 + i) * DV;
          if constexpr (PM) ht[o_] = prow<E>(b, g4 + i) == v0 + cw + cl ? 1.f : 0.f;
          else ht[o_] = h0 ? h0[o_] : 0.f;
        }
    }
    return;
  }
  const int64_t base = (int64_t)(si.b * g.H + h) * g.T + si.bos;
  auto rows_of = [&](int c) { return min(kChunk, si.len - c * kChunk); };

  // ---- loader wave (wl: its index among the loader waves) and storer wave (tl: its lane)
  const int wl = 0, tl = tid - 64 * (NWC + 1);
  auto issue = [&](int c, int slot) {  // chunk c into LDS stage `slot`
    unsigned char* st = smem + slot * L::stage;
    const int n = rows_of(c);
    const int64_t r0 = base + (int64_t)c * kChunk;
    const int64_t unit = (int64_t)(si.slot0 + c) * g.H + h;
    // K, Q and (gated) the running log-decay sums first: with the output, XF forms M from them
    // (mtile below) while the rest lands. The per-token vectors (64 floats each) by LDS DMA too.
    dma_tile<E, DK, NWL, 0, L::MXK>(st + L::oK, k + r0 * DK, DK, n, wl, lane);
    if constexpr (WO) {
      dma_tile<E, DK, NWL, 0, L::MXK>(st + L::oQ, q + r0 * DK, DK, n, wl, lane);
      if constexpr (!XF) dma_tile<E, 64, NWL>(st + L::oM, m + unit * kChunk * kChunk, kChunk, kChunk, wl, lane);
    }
    if constexpr (GT) dma_vec64(st + L::oC, cum + unit * kChunk, lane);
    if constexpr (XF) dma_tile<E, 64, NWL>(st + L::oW, w + unit * kChunk * kChunk, kChunk, kChunk, wl, lane);
    else dma_tile<E, DK, NWL, 0, L::MXK>(st + L::oW, w + r0 * DK, DK, n, wl, lane);
    if constexpr (!PM) dma_tile<E, TV, NWL, 2>(st + L::oU, u + r0 * DV + v0, DV, n, wl, lane);
    if constexpr (XF) {
      dma_vec64(st + L::oA, ca + unit * kChunk, lane);
      if constexpr (GT) dma_vec64(st + L::oA + 64 * 4, cb + unit * kChunk, lane);
    }
    // the counted wait assumes every request above is issued before the warm-up loads that
    // follow: keep the scheduler from moving any of them past this point
    __builtin_amdgcn_sched_barrier(0);
  };
  // XF with the output, given m: M of chunk c (formed by the loader wave in stage c & 1, which
  // stays put until the next barrier) goes to global memory for the backward. The NTILE
  // workgroups of a (sequence, head) form the same M; each writes 64 / NTILE of its rows. The
  // stage holds only the blocks on and below the diagonal: the others, and rows past the end of
  // the sequence, are written as zeros.
  auto copy_m = [&](int c) {
    if constexpr (XF && WO) {
      if (!m) return;
      typedef Swz<E, 64> SM;
      constexpr int RPT = kChunk / NTILE, CPM = SM::NCH;  // rows per workgroup, 16-byte chunks per row
      static_assert(kChunk % NTILE == 0, "M rows per workgroup");
      const unsigned char* sm = smem + (c & 1) * L::stage + L::oM;
      E* gm = m + ((int64_t)(si.slot0 + c) * g.H + h) * kChunk * kChunk;
      const int n = rows_of(c);
#pragma unroll
      for (int it = 0; it < (RPT * CPM + NTL - 1) / NTL; ++it) {
        const int i = it * NTL + tl, r = tile * RPT + i / CPM, lc = i % CPM;
        if (i < RPT * CPM) {
          u32x4 val = u32x4{0u, 0u, 0u, 0u};
          if (r < n && lc * VE < 16 * (r / 16 + 1)) val = *(const u32x4*)(sm + SM::off(r, lc * VE));
          *at_byte<u32x4>(gm, (unsigned)((r * kChunk + lc * VE) * (int)sizeof(E))) = val;
        }
      }
    }
  };
  // Stores address 32-bit byte offsets from wave-uniform tile bases (scalar-base addressing; no
  // 64-bit address arithmetic per lane).
  auto copy_out = [&](int c) {  // staged outputs of chunk c -> global memory, 16-byte rows
    const unsigned char* stg = smem + L::oStg + (c & 1) * L::sstage;
    const int n = rows_of(c);
    const int64_t r0 = base + (int64_t)c * kChunk;
    constexpr int CPR = SU::NCH;  // 16-byte chunks per row
    if constexpr (WO) {
#pragma unroll
      for (int it = 0; it < (64 * CPR + NTL - 1) / NTL; ++it) {
        const int i = it * NTL + tl, r = i / CPR, lc = i % CPR;
        if (i < 64 * CPR && r < n)
          *at_byte<u32x4>(o + r0 * DV + v0, (unsigned)((r * DV + lc * VE) * (int)sizeof(E))) =
              *(const u32x4*)(stg + L::gO + SU::off(r, lc * VE));
      }
    }
    if constexpr (WSV) {
#pragma unroll
      for (int it = 0; it < (64 * CPR + NTL - 1) / NTL; ++it) {
        const int i = it * NTL + tl, r = i / CPR, lc = i % CPR;
        if (i < 64 * CPR && r < n)
          *at_byte<u32x4>(ut + r0 * DV + v0, (unsigned)((r * DV + lc * VE) * (int)sizeof(E))) =
              *(const u32x4*)(stg + L::gUt + SU::off(r, lc * VE));
      }
    }
    if constexpr (WSV) {
      E* gS = states + ((int64_t)(si.slot0 + c) * g.H + h) * DK * DV + v0;
#pragma unroll
      for (int it = 0; it < (DK * CPR + NTL - 1) / NTL; ++it) {
        const int i = it * NTL + tl, d = i / CPR, lc = i % CPR;
        if (i < DK * CPR)
          *at_byte<u32x4>(gS, (unsigned)((d * DV + lc * VE) * (int)sizeof(E))) =
              *(const u32x4*)(stg + L::gS + SU::off(d, lc * VE));
      }
    }
  };

  // ---- compute waves: S[16 b + g4 + i][v0 + cw + cl] in Sacc[b]
  f32x4 Sacc[NBK];
#pragma unroll
  for (int b = 0; b < NBK; ++b) Sacc[b] = zero4();
  if constexpr (PM) {  // S = I (this wave's columns)
#pragma unroll
    for (int b = 0; b < NBK; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) Sacc[b][i] = prow<E>(b, g4 + i) == v0 + cw + cl ? 1.f : 0.f;
  } else if (h0 && !loader && !storer) {  // state entering the sequence
#pragma unroll
    for (int b = 0; b < NBK; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) Sacc[b][i] = h0[hoff + (int64_t)prow<E>(b, g4 + i) * DV];
  }
  auto compute = [&](int c) {
    const unsigned char* st = smem + (c & 1) * L::stage;
    unsigned char* stg = smem + L::oStg + (c & 1) * L::sstage;
    const int n = rows_of(c);
    // Operands that do not depend on this chunk's results, requested before any product so
    // that their LDS latency overlaps.
    // aw: rows of W (fp32), or of K for the product K S (XF); ax: X for U~ = X Y (XF)
    V aw[4][KSK], aq[4][KSK], ax[4][KST];
    E uv[4][4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
      for (int ks = 0; ks < KSK; ++ks) {
        aw[rb][ks] = aop_rc<E, DK, L::MXK>(st + (XF ? L::oK : L::oW), rb, ks, lane);
        if constexpr (WO) aq[rb][ks] = aop_rc<E, DK, L::MXK>(st + L::oQ, rb, ks, lane);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        uv[rb][i] = PM ? to_e<E>(0.f) : *(const E*)(st + L::oU + SU::off(prow<E>(rb, g4 + i), cw + cl));
    }
    V sb[KSK];
#pragma unroll
    for (int ks = 0; ks < KSK; ++ks) sb[ks] = bop_acc<E>(Sacc, ks);
    // gated: e^{c_t} for the output's state term, e^{c_last - c_t} for the state update
    float gam[4][4], dec[4][4], gC = 1.f;
    if constexpr (GT) {
      const float* cv = (const float*)(st + L::oC);
      const float cl = cv[n - 1];
      gC = exp_decay(cl);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float cr = cv[prow<E>(rb, g4 + i)];
          gam[rb][i] = exp_decay(cr);
          dec[rb][i] = exp_decay(cl - cr);
        }
    }
    if constexpr (WSV) {  // S_c, the state entering chunk c
#pragma unroll
      for (int b = 0; b < NBK; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *(E*)(stg + L::gS + SU::off(prow<E>(b, g4 + i), cw + cl)) = to_e<E>(Sacc[b][i]);
    }
    __builtin_amdgcn_sched_barrier(0);

    // W S (XF: K S) and P = Q S
    f32x4 ws[4], oa[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      ws[rb] = zero4();
      oa[rb] = zero4();
#pragma unroll
      for (int ks = 0; ks < KSK; ++ks) {
        ws[rb] = Mma<E>::step(aw[rb][ks], sb[ks], ws[rb]);
        if constexpr (WO) oa[rb] = Mma<E>::step(aq[rb][ks], sb[ks], oa[rb]);
      }
    }
    if constexpr (GT && WO) {
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) oa[rb][i] *= gam[rb][i];
    }
    V ak[NBK][KST], am[4][KST];
    if constexpr (XF) {  // requested while K S runs (with aw and aq issued, registers are free)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int ks = 0; ks < KST; ++ks)
          if (KC * ks <= 16 * rb + 15) ax[rb][ks] = aop_rc<E, 64>(st + L::oW, rb, ks, lane);
    }
#pragma unroll
    for (int b = 0; b < NBK; ++b)
#pragma unroll
      for (int ks = 0; ks < KST; ++ks) ak[b][ks] = aop_kc<E, DK, L::MXK>(st + L::oK, b, ks, lane);
    if constexpr (WO) {
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int ks = 0; ks < KST; ++ks)
          if (KC * ks <= 16 * rb + 15) am[rb][ks] = aop_rc<E, 64>(st + L::oM, rb, ks, lane);
    }
    __builtin_amdgcn_sched_barrier(0);

    // U~ = U - W S (rows past the end of the sequence zeroed); XF: U~ = X Y with
    // Y = diag(b) V - diag(alpha~) K S (X is lower triangular: row blocks 0-1 need one step)
    f32x4 uta[4];
    if constexpr (XF) {
      // the four rows prow(rb, g4 + i), i < 4, are consecutive: one 16-byte read of each scale
      const float* av = (const float*)(st + L::oA);
      f32x4 y[4];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const f32x4 al = *(const f32x4*)(av + prow<E>(rb, g4));
        const f32x4 bl = GT ? *(const f32x4*)(av + 64 + prow<E>(rb, g4)) : al;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          y[rb][i] = prow<E>(rb, g4 + i) < n ? bl[i] * to_f(uv[rb][i]) - al[i] * ws[rb][i] : 0.f;
      }
      V yb[KST];
#pragma unroll
      for (int ks = 0; ks < KST; ++ks) yb[ks] = bop_acc<E>(y, ks);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        uta[rb] = zero4();
#pragma unroll
        for (int ks = 0; ks < KST; ++ks)
          if (KC * ks <= 16 * rb + 15) uta[rb] = Mma<E>::step(ax[rb][ks], yb[ks], uta[rb]);
      }
    } else {
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          uta[rb][i] = prow<E>(rb, g4 + i) < n ? to_f(uv[rb][i]) - ws[rb][i] : 0.f;
    }
    V ub[KST], ubd[KST];
#pragma unroll
    for (int ks = 0; ks < KST; ++ks) ub[ks] = bop_acc<E>(uta, ks);
    if constexpr (GT) {  // S <- e^{c_last} S + K^T diag(e^{c_last - c}) U~
      f32x4 utd[4];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) utd[rb][i] = uta[rb][i] * dec[rb][i];
#pragma unroll
      for (int ks = 0; ks < KST; ++ks) ubd[ks] = bop_acc<E>(utd, ks);
#pragma unroll
      for (int b = 0; b < NBK; ++b) Sacc[b] *= gC;
    } else {
#pragma unroll
      for (int ks = 0; ks < KST; ++ks) ubd[ks] = ub[ks];
    }
    // S += K^T U~
#pragma unroll
    for (int b = 0; b < NBK; ++b)
#pragma unroll
      for (int ks = 0; ks < KST; ++ks) Sacc[b] = Mma<E>::step(ak[b][ks], ubd[ks], Sacc[b]);
    if constexpr (WO) {  // O = scale (P + M U~); M is lower triangular
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
        for (int ks = 0; ks < KST; ++ks)
          if (KC * ks <= 16 * rb + 15) oa[rb] = Mma<E>::step(am[rb][ks], ub[ks], oa[rb]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *(E*)(stg + L::gO + SU::off(prow<E>(rb, g4 + i), cw + cl)) = to_e<E>(g.scale * oa[rb][i]);
      }
    }
    if constexpr (WSV) {
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *(E*)(stg + L::gUt + SU::off(prow<E>(rb, g4 + i), cw + cl)) = to_e<E>(uta[rb][i]);
    }
  };

  // Three loops, nchunks + 1 barriers each.
  // The loader also warms L2 two chunks ahead (one word per 128-byte line; the workgroups of the
  // (sequence, head) split the shared tiles), so its DMA of chunk c + 1 reads lines requested a
  // step earlier and HBM keeps a request stream across the barriers. Before the barrier that
  // publishes a chunk it waits for the DMA only (a counted vmcnt: the younger warm-up loads stay
  // in flight) and the barrier is a bare s_barrier, whose fence would wait for everything. The
  // warm-up requests are LDS DMA into a row that nothing reads (WDMA), so no register waits for
  // them and the next chunk's warm-up leaves while this chunk's DMA is in flight. Every request
  // is unconditional (clamped chunk index), so the counts stay exact; the last wait before the
  // wave leaves covers them all. The storer never waits for anything but the barriers.
  if (loader) {
    constexpr int NL = (64 * (DK > DV ? DK : DV) * (int)sizeof(E) / 128 + 64 * NTILE - 1) / (64 * NTILE);
    unsigned char* dummy = smem + L::oDummy;
    int pw[L::WDMA ? 1 : 5 * NL];  // register warm-up only
#pragma unroll
    for (int i = 0; i < (L::WDMA ? 1 : 5 * NL); ++i) pw[i] = 0;
    auto touch = [&](int slot, const void* p, int nbytes) {
      if constexpr (L::WDMA) l2_touch_lds<NL>(dummy, p, nbytes, tile, NTILE, lane);
      else l2_touch<NL>(pw + slot * NL, p, nbytes, tile, NTILE, lane);
    };
    auto warm = [&](int c) {
      const int n = rows_of(c);
      const int64_t r0 = base + (int64_t)c * kChunk;
      if constexpr (XF)
        touch(0, w + ((int64_t)(si.slot0 + c) * g.H + h) * kChunk * kChunk, kChunk * kChunk * (int)sizeof(E));
      else
        touch(0, w + r0 * DK, n * DK * (int)sizeof(E));
      touch(1, k + r0 * DK, n * DK * (int)sizeof(E));
      if constexpr (WO) {
        touch(2, q + r0 * DK, n * DK * (int)sizeof(E));
        if constexpr (!XF)
          touch(3, m + ((int64_t)(si.slot0 + c) * g.H + h) * kChunk * kChunk, kChunk * kChunk * (int)sizeof(E));
      }
      if constexpr (!PM) touch(4, u + r0 * DV, n * DV * (int)sizeof(E));
      // keep every warm-up request ahead of the work that follows (the counted waits rely on it)
      __builtin_amdgcn_sched_barrier(0);
    };
    // warm-up loads issued after each DMA: the factor (W or X) and K, Q and M (XF: Q only)
    // with the output, U (or V) unless PM
    constexpr int NWARM = NL * (2 + (WO ? (XF ? 1 : 2) : 0) + (PM ? 0 : 1));
    static_assert(NWARM <= 15, "vmcnt field");
    // XF with the output: once a chunk's K and Q tiles (and gated, its decay sums) have landed,
    // this wave forms its M into the chunk's stage (the compute waves work on the other stage
    // meanwhile); the requests issued after them (X, V, alpha~, b) and the warm-up may still be
    // in flight
    auto mtile = [&](int slot) {
      if constexpr (XF && WO) {
        constexpr int NAFT = NWARM + Swz<E, 64>::BYTES / 1024 / NWL +
                             (PM ? 0 : Swz<E, TV, 2>::BYTES / 1024 / NWL) + 1 + (GT ? 1 : 0);  // warm-up; X, V; alpha~, b
        static_assert(NAFT < 64, "vmcnt field");
        __builtin_amdgcn_s_waitcnt((NAFT & 15) | ((NAFT >> 4) << 14) | 0x0F70);
        unsigned char* st = smem + slot * L::stage;
        m_tile<E, DK, GT, L::MXK>(st + L::oM, st + L::oQ, st + L::oK, (const float*)(st + L::oC), lane);
      }
    };
    issue(0, 0);
    warm(min(1, nchunks - 1));
    mtile(0);
    for (int c = 0; c < nchunks; ++c) {
      // vmcnt(NWARM), lgkmcnt(0): chunk c's DMA has landed (only the younger warm-up loads may
      // still be in flight), and so have this wave's LDS writes
      __builtin_amdgcn_s_waitcnt(0x0070 | NWARM);
      __builtin_amdgcn_s_barrier();
      // after the last chunk the request repeats it into the stage that chunk c + 1 would use,
      // which no wave reads any more (every request is unconditional)
      issue(min(c + 1, nchunks - 1), (c + 1) & 1);
      if constexpr (!L::WDMA) l2_sink<5 * NL>(pw);  // the previous step's register warm-up
      warm(min(c + 2, nchunks - 1));
      mtile((c + 1) & 1);
    }
    wait_vm_all();
    __syncthreads();
    return;
  }
  if (storer) {
    for (int c = 0; c < nchunks; ++c) {
      __syncthreads();  // staging of chunk c - 1 is complete, and M of chunk c is in its stage
      if (c > 0) copy_out(c - 1);
      copy_m(c);
    }
    __syncthreads();
    copy_out(nchunks - 1);
    return;
  }
  for (int c = 0; c < nchunks; ++c) {
    __syncthreads();
    compute(c);
  }
  __syncthreads();
  if (ht) {  // state after the last token
#pragma unroll
    for (int b = 0; b < NBK; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) ht[hoff + (int64_t)prow<E>(b, g4 + i) * DV] = Sacc[b][i];
  }
}

template <typename E, int DK, int DV, int NWC, bool WO, bool WSV, bool PM, bool GT>
__global__ __launch_bounds__(64 * NWC + 128, 1) void scan_fwd_kernel(
    Geom g, const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ w,
    const E* __restrict__ u, E* __restrict__ m, E* __restrict__ o, E* __restrict__ ut,
    E* __restrict__ states, const float* __restrict__ h0, float* __restrict__ ht,
    const float* __restrict__ cum, const float* __restrict__ ca, const float* __restrict__ cb) {
  scan_fwd_body<E, DK, DV, NWC, WO, WSV, PM, GT>(blockIdx.x, g, q, k, w, u, m, o, ut, states, h0, ht,
                                                 cum, ca, cb);
}

// The two independent first passes of the segment-parallel forward in one launch: blocks
// [0, nr) run the zero-start state scan of every segment (R, d_k x d_v per segment), the rest
// the transition scan (P, d_k x d_k). Both use the output-free LDS layout, so two workgroups
// share a compute unit and the passes overlap instead of running one after the other.
template <typename E, int DK, int DV, int NWC, bool GT>
__global__ __launch_bounds__(64 * NWC + 128, 2) void scan_fwd_pair_kernel(
    Geom g, int nr, const E* __restrict__ k, const E* __restrict__ w, const E* __restrict__ u,
    float* __restrict__ R, float* __restrict__ P, const float* __restrict__ cum,
    const float* __restrict__ ca, const float* __restrict__ cb) {
  if ((int)blockIdx.x < nr)
    scan_fwd_body<E, DK, DV, NWC, false, false, false, GT>(blockIdx.x, g, nullptr, k, w, u, nullptr, nullptr,
                                                          nullptr, nullptr, nullptr, R, cum, ca, cb);
  else
    scan_fwd_body<E, DK, DK, NWC, false, false, true, GT>(blockIdx.x - nr, g, nullptr, k, w, nullptr, nullptr,
                                                         nullptr, nullptr, nullptr, nullptr, P, cum, ca, cb);
}

template <typename E, int DK, int DV, int NWC, bool GT>
static hipError_t scan_fwd_pair_run(const Shape& s, const void* k, const void* w, const void* u,
                                    float* R, float* P, hipStream_t st, const float* cum,
                                    const float* ca, const float* cb) {
  typedef ScanFwdLds<E, DK, DV, NWC, false, false, GT> LR;
  typedef ScanFwdLds<E, DK, DK, NWC, false, false, GT> LP;
  constexpr size_t bytes = LR::bytes > LP::bytes ? LR::bytes : LP::bytes;
  static_assert(2 * bytes <= 160 * 1024, "two workgroups per compute unit");
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)scan_fwd_pair_kernel<E, DK, DV, NWC, GT>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const int64_t nr = (int64_t)s.n_seqs * s.H * (DV / LR::TV), np = (int64_t)s.n_seqs * s.H * (DK / LP::TV);
  if (nr + np < 1) return hipSuccess;
  prof_begin(st);
  hipLaunchKernelGGL((scan_fwd_pair_kernel<E, DK, DV, NWC, GT>), dim3((unsigned)(nr + np)),
                     dim3(64 * NWC + 128), bytes, st, make_geom(s, nullptr), (int)nr, (const E*)k,
                     (const E*)w, (const E*)u, R, P, cum, ca, cb);
  hipError_t e = hipGetLastError();
  prof_end(GT ? "scan_fwd_state_transition_gated" : "scan_fwd_state_transition", st);
  return e;
}

template <typename E, int DK, int DV, int NWC, bool WO, bool WSV, bool PM = false, bool GT = false>
static hipError_t scan_fwd_run(const Shape& s, const int* table, const void* q, const void* k,
                               const void* w, const void* u, void* m, void* o, void* ut,
                               void* states, const float* h0, float* ht, hipStream_t st,
                               const float* cum, const float* ca, const float* cb) {
  typedef ScanFwdLds<E, DK, DV, NWC, WO, WSV, GT> L;
  static_assert(L::bytes <= 160 * 1024, "LDS budget");
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)scan_fwd_kernel<E, DK, DV, NWC, WO, WSV, PM, GT>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)L::bytes);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const int64_t blocks = (int64_t)s.n_seqs * s.H * (DV / L::TV);
  if (blocks < 1) return hipSuccess;
  prof_begin(st);
  hipLaunchKernelGGL((scan_fwd_kernel<E, DK, DV, NWC, WO, WSV, PM, GT>), dim3((unsigned)blocks),
                     dim3(64 * NWC + 128), L::bytes, st, make_geom(s, table), (const E*)q, (const E*)k,
                     (const E*)w, (const E*)u, (E*)m, (E*)o, (E*)ut, (E*)states, h0, ht, cum, ca, cb);
  hipError_t e = hipGetLastError();
  prof_end(PM ? (GT ? "scan_fwd_transition_gated" : "scan_fwd_transition")
             : WO || WSV ? (GT ? "scan_fwd_gated" : "scan_fwd") : (GT ? "scan_fwd_state_gated" : "scan_fwd_state"),
           st);
  return e;
}

// Outputs: O alone, O with U~ and the chunk states, U~ and the states alone (recompute), or
// only the final states (first pass of the segment-parallel scan).
template <typename E, int DK, int DV, int NWC>
static hipError_t scan_fwd_go(const Shape& s, const int* table, const void* q, const void* k,
                              const void* w, const void* u, void* m, void* o, void* ut,
                              void* states, const float* h0, float* ht, hipStream_t st,
                              const float* cum, const float* ca, const float* cb) {
  const bool wsv = ut && states;
#define EFLA_SFR(WO_, WSV_, GT_) \
  return scan_fwd_run<E, DK, DV, NWC, WO_, WSV_, false, GT_>(s, table, q, k, w, u, m, o, ut, states, h0, ht, st, cum, ca, cb)
  if (cum) {  // gated
    if constexpr (sizeof(E) == 2) {
      if (o && wsv) EFLA_SFR(true, true, true);
      if (wsv) EFLA_SFR(false, true, true);
      if (o) EFLA_SFR(true, false, true);
      if (ht) EFLA_SFR(false, false, true);
      return hipSuccess;
    } else {
      return hipErrorInvalidValue;  // the fp32 tiles leave no LDS room for the decays
    }
  }
  if (o && wsv) EFLA_SFR(true, true, false);
  if (o) EFLA_SFR(true, false, false);
  if (wsv) EFLA_SFR(false, true, false);
  if (ht) EFLA_SFR(false, false, false);
#undef EFLA_SFR
  return hipSuccess;
}

// bf16: two compute waves (32 state columns), a loader and a storer wave per workgroup; fp32:
// one compute wave (the double-buffered fp32 tiles leave LDS room for 16 columns of staging).
size_t lds_scan_fwd(Dt dt, int dk, int dv) {
  if (dt == Dt::BF16) {
    if (dk == 64 && dv == 64) return ScanFwdLds<__bf16, 64, 64, 2, true, true>::bytes;
    if (dk == 64 && dv == 128) return ScanFwdLds<__bf16, 64, 128, 2, true, true>::bytes;
    if (dk == 128 && dv == 64) return ScanFwdLds<__bf16, 128, 64, 2, true, true>::bytes;
    if (dk == 128 && dv == 128) return ScanFwdLds<__bf16, 128, 128, 2, true, true>::bytes;
    return 0;
  }
  if (dk == 64 && dv == 64) return ScanFwdLds<float, 64, 64, 1, true, true>::bytes;
  return 0;
}

hipError_t launch_scan_fwd(const Shape& s, const int* table, const void* q, const void* k,
                           const void* w, const void* u, void* m, void* o, void* ut,
                           void* states, const float* h0, float* ht, hipStream_t st,
                           const float* cum, const float* ca, const float* cb) {
#define EFLA_SF(E_, DK_, DV_, NWC_) \
  return scan_fwd_go<E_, DK_, DV_, NWC_>(s, table, q, k, w, u, m, o, ut, states, h0, ht, st, cum, ca, cb)
  if (s.dt == Dt::BF16) {
    if (s.dk == 64 && s.dv == 64) EFLA_SF(__bf16, 64, 64, 2);
    if (s.dk == 64 && s.dv == 128) EFLA_SF(__bf16, 64, 128, 2);
    if (s.dk == 128 && s.dv == 64) EFLA_SF(__bf16, 128, 64, 2);
    EFLA_SF(__bf16, 128, 128, 2);
  }
  EFLA_SF(float, 64, 64, 1);
#undef EFLA_SF
}

hipError_t launch_scan_fwd_pair(const Shape& s, const void* k, const void* w, const void* u,
                                float* r, float* p, hipStream_t st, const float* cum,
                                const float* ca, const float* cb) {
#define EFLA_SP(E_, DK_, DV_, NWC_, GT_) \
  return scan_fwd_pair_run<E_, DK_, DV_, NWC_, GT_>(s, k, w, u, r, p, st, cum, ca, cb)
  if (s.dt == Dt::BF16) {
    if (cum) {
      if (s.dk == 64 && s.dv == 64) EFLA_SP(__bf16, 64, 64, 2, true);
      if (s.dk == 64 && s.dv == 128) EFLA_SP(__bf16, 64, 128, 2, true);
      if (s.dk == 128 && s.dv == 64) EFLA_SP(__bf16, 128, 64, 2, true);
      EFLA_SP(__bf16, 128, 128, 2, true);
    }
    if (s.dk == 64 && s.dv == 64) EFLA_SP(__bf16, 64, 64, 2, false);
    if (s.dk == 64 && s.dv == 128) EFLA_SP(__bf16, 64, 128, 2, false);
    if (s.dk == 128 && s.dv == 64) EFLA_SP(__bf16, 128, 64, 2, false);
    EFLA_SP(__bf16, 128, 128, 2, false);
  }
  if (cum) return hipErrorInvalidValue;  // gated EFLA is built for bf16 only
  EFLA_SP(float, 64, 64, 1, false);
#undef EFLA_SP
}

}  // namespace efla

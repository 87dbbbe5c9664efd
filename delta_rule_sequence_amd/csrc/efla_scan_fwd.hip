// Inter-chunk state recurrence fused with the chunk output.
//
// Exact Flow Linear Attention summary page, section 3.3 (chunk-level recurrence and
// outputs). One workgroup walks the chunks of one (sequence, head) in order and owns a
// d_k x TV slice of the state (TV = 16 columns per wave):
//   U~ = U - W S,   O = scale (Q S + M U~),   S <- S + K^T U~,
// with M = tril(Q K^T) from the UT kernel. The diagonal of tril is kept because token t
// reads the state after its own update.
//
// Each compute wave owns 16 columns of S for the whole sequence and keeps them in fp32 MFMA
// accumulators. Products whose contraction runs over the rows of an accumulator take that
// accumulator directly as their B operand, so the recurrence S -> W S -> U~ -> K^T U~ -> S
// runs inside one wave's registers with no LDS round trip. Accumulator rows (of S, and the
// token rows of U~ and O) are numbered in the contiguous-contraction order (prow), so every
// A operand from LDS is a single 16-byte read. Two further waves move the data, each in a loop
// of its own with the same barrier sequence: the loader wave fills swizzled LDS tiles of W, Q,
// K, M and U one chunk ahead by LDS DMA (double-buffered) and warms L2 for the chunk after; the
// storer wave copies the staged O, U~ and chunk states out as 16-byte rows. Kept apart from the
// loads, the output stores are never waited for. One barrier per chunk hands the buffers over.
#include "efla_internal.hpp"

namespace efla {

template <typename E, int DK, int DV, int NWC, bool GT = false>
struct ScanFwdLds {
  static constexpr int TV = 16 * NWC;
  static constexpr int NWL = 1;  // loader waves (one; a second wave stores the outputs)
  typedef Swz<E, DK> SK;
  typedef Swz<E, 64> SM;
  typedef Swz<E, TV, 2> SU;  // read in accumulator layout
  static constexpr size_t oW = 0;                       // W  [64][DK]
  static constexpr size_t oQ = oW + SK::BYTES;          // Q  [64][DK]
  static constexpr size_t oK = oQ + SK::BYTES;          // K  [64][DK]
  static constexpr size_t oM = oK + SK::BYTES;          // M  [64][64]
  static constexpr size_t oU = oM + SM::BYTES;          // U  [64][TV] (this tile's columns)
  static constexpr size_t oC = oU + SU::BYTES;         // running log-decay sums [64] (gated)
  static constexpr size_t stage = oC + (GT ? 64 * 4 : 0);
  // output staging (layout SU): O [64][TV], U~ [64][TV], S [DK][TV]; two buffers
  static constexpr size_t gO = 0, gUt = SU::BYTES, gS = 2 * SU::BYTES;
  static constexpr size_t sstage = gS + (size_t)DK * SU::RB;
  static constexpr size_t oStg = 2 * stage;
  static constexpr size_t bytes = oStg + 2 * sstage;
};

// WO: write O (also needs Q and M); WSV: write U~ and the chunk states (saved for the
// backward pass). Compile-time, so the inner loops carry no branches on them.
// GT: gated EFLA. With c_t the running log-decay sum inside the chunk (from the UT kernel),
// O = scale (diag(e^{c}) Q S + M U~) (M carries the decay ratios), and
// S <- e^{c_last} S + K^T diag(e^{c_last - c}) U~; the decays are applied to accumulators.
// PM: transition mode for the segment-parallel scan. The chunk step is affine in the state,
// S <- (I - K^T W) S + K^T U, so running it with U = 0 from S = I (DV = DK) leaves in ht the
// product of the (I - K^T W) over the sequence; U is neither read nor needed.
template <typename E, int DK, int DV, int NWC, bool WO, bool WSV, bool PM, bool GT>
__global__ __launch_bounds__(64 * NWC + 128, 1) void scan_fwd_kernel(
    Geom g, const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ w,
    const E* __restrict__ u, const E* __restrict__ m, E* __restrict__ o, E* __restrict__ ut,
    E* __restrict__ states, const float* __restrict__ h0, float* __restrict__ ht,
    const float* __restrict__ cum) {
  typedef ScanFwdLds<E, DK, DV, NWC, GT> L;
  typedef typename L::SU SU;
  typedef typename Mma<E>::vec V;
  constexpr int TV = L::TV, NWL = L::NWL, NTILE = DV / TV, KC = Mma<E>::KC;
  constexpr int NBK = DK / 16;                 // accumulator tiles of the state slice
  constexpr int KSK = DK / KC, KST = kChunk / KC;
  constexpr int NTL = 64;                      // storer threads (one wave)
  constexpr int VE = 16 / (int)sizeof(E);
  static_assert(DV % TV == 0, "column tiles");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wi = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool loader = wi == NWC, storer = wi == NWC + 1;
  int sh, tile;
  scan_block(blockIdx.x, g.n_seqs * g.H, NTILE, sh, tile);
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
    dma_tile<E, DK, NWL>(st + L::oW, w + r0 * DK, DK, n, wl, lane);
    if constexpr (!PM) dma_tile<E, TV, NWL, 2>(st + L::oU, u + r0 * DV + v0, DV, n, wl, lane);
    dma_tile<E, DK, NWL>(st + L::oK, k + r0 * DK, DK, n, wl, lane);
    if constexpr (WO) {
      dma_tile<E, DK, NWL>(st + L::oQ, q + r0 * DK, DK, n, wl, lane);
      dma_tile<E, 64, NWL>(st + L::oM, m + ((int64_t)(si.slot0 + c) * g.H + h) * kChunk * kChunk,
                           kChunk, kChunk, wl, lane);
    }
    if constexpr (GT) {  // 64 floats: one plain load per lane of the loader wave
      if (wl == 0) ((float*)(st + L::oC))[lane] = cum[((int64_t)(si.slot0 + c) * g.H + h) * kChunk + lane];
    }
  };
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
          *(u32x4*)(o + (r0 + r) * DV + v0 + lc * VE) = *(const u32x4*)(stg + L::gO + SU::off(r, lc * VE));
      }
    }
    if constexpr (WSV) {
#pragma unroll
      for (int it = 0; it < (64 * CPR + NTL - 1) / NTL; ++it) {
        const int i = it * NTL + tl, r = i / CPR, lc = i % CPR;
        if (i < 64 * CPR && r < n)
          *(u32x4*)(ut + (r0 + r) * DV + v0 + lc * VE) = *(const u32x4*)(stg + L::gUt + SU::off(r, lc * VE));
      }
    }
    if constexpr (WSV) {
      E* gS = states + ((int64_t)(si.slot0 + c) * g.H + h) * DK * DV + v0;
#pragma unroll
      for (int it = 0; it < (DK * CPR + NTL - 1) / NTL; ++it) {
        const int i = it * NTL + tl, d = i / CPR, lc = i % CPR;
        if (i < DK * CPR)
          *(u32x4*)(gS + (int64_t)d * DV + lc * VE) = *(const u32x4*)(stg + L::gS + SU::off(d, lc * VE));
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
    V aw[4][KSK], aq[4][KSK];
    E uv[4][4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
      for (int ks = 0; ks < KSK; ++ks) {
        aw[rb][ks] = aop_rc<E, DK>(st + L::oW, rb, ks, lane);
        if constexpr (WO) aq[rb][ks] = aop_rc<E, DK>(st + L::oQ, rb, ks, lane);
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
          dec[rb][i] = exp_decay(fminf(cl - cr, 0.f));
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

    // W S and P = Q S
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
#pragma unroll
    for (int b = 0; b < NBK; ++b)
#pragma unroll
      for (int ks = 0; ks < KST; ++ks) ak[b][ks] = aop_kc<E, DK>(st + L::oK, b, ks, lane);
    if constexpr (WO) {
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int ks = 0; ks < KST; ++ks)
          if (KC * ks <= 16 * rb + 15) am[rb][ks] = aop_rc<E, 64>(st + L::oM, rb, ks, lane);
    }
    __builtin_amdgcn_sched_barrier(0);

    // U~ = U - W S (rows past the end of the sequence zeroed)
    f32x4 uta[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        uta[rb][i] = prow<E>(rb, g4 + i) < n ? to_f(uv[rb][i]) - ws[rb][i] : 0.f;
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
  // in flight) and the barrier is a bare s_barrier, whose fence would wait for everything; each
  // warm-up is consumed a step later. Every request is unconditional (clamped chunk index), so
  // the compiler's counts stay exact. The storer then never waits for anything but the barriers.
  if (loader) {
    constexpr int NL = (64 * (DK > DV ? DK : DV) * (int)sizeof(E) / 128 + 64 * NTILE - 1) / (64 * NTILE);
    int pw[5 * NL];
#pragma unroll
    for (int i = 0; i < 5 * NL; ++i) pw[i] = 0;
    auto warm = [&](int c) {
      const int n = rows_of(c);
      const int64_t r0 = base + (int64_t)c * kChunk;
      l2_touch<NL>(pw, w + r0 * DK, n * DK * (int)sizeof(E), tile, NTILE, lane);
      l2_touch<NL>(pw + NL, k + r0 * DK, n * DK * (int)sizeof(E), tile, NTILE, lane);
      if constexpr (WO) {
        l2_touch<NL>(pw + 2 * NL, q + r0 * DK, n * DK * (int)sizeof(E), tile, NTILE, lane);
        l2_touch<NL>(pw + 3 * NL, m + ((int64_t)(si.slot0 + c) * g.H + h) * kChunk * kChunk,
                     kChunk * kChunk * (int)sizeof(E), tile, NTILE, lane);
      }
      if constexpr (!PM) l2_touch<NL>(pw + 4 * NL, u + r0 * DV, n * DV * (int)sizeof(E), tile, NTILE, lane);
    };
    // warm-up loads issued after each DMA: W and K, Q and M with the output, U unless PM
    constexpr int NWARM = NL * (2 + (WO ? 2 : 0) + (PM ? 0 : 1));
    static_assert(NWARM <= 15, "vmcnt field");
    issue(0, 0);
    warm(min(1, nchunks - 1));
    for (int c = 0; c < nchunks; ++c) {
      // vmcnt(NWARM), lgkmcnt(0): chunk c's DMA has landed (only the younger warm-up loads may
      // still be in flight), and so has the gated loader's LDS store
      __builtin_amdgcn_s_waitcnt(0x0070 | NWARM);
      __builtin_amdgcn_s_barrier();
      // after the last chunk the request repeats it into the stage that chunk c + 1 would use,
      // which no wave reads any more (every request is unconditional)
      issue(min(c + 1, nchunks - 1), (c + 1) & 1);
      l2_sink<5 * NL>(pw);
      warm(min(c + 2, nchunks - 1));
    }
    wait_vm_all();
    __syncthreads();
    return;
  }
  if (storer) {
    for (int c = 0; c < nchunks; ++c) {
      __syncthreads();  // staging of chunk c - 1 is complete
      if (c > 0) copy_out(c - 1);
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

template <typename E, int DK, int DV, int NWC, bool WO, bool WSV, bool PM = false, bool GT = false>
static hipError_t scan_fwd_run(const Shape& s, const int* table, const void* q, const void* k,
                               const void* w, const void* u, const void* m, void* o, void* ut,
                               void* states, const float* h0, float* ht, hipStream_t st,
                               const float* cum = nullptr) {
  typedef ScanFwdLds<E, DK, DV, NWC, GT> L;
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
                     (const E*)w, (const E*)u, (const E*)m, (E*)o, (E*)ut, (E*)states, h0, ht, cum);
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
                              const void* w, const void* u, const void* m, void* o, void* ut,
                              void* states, const float* h0, float* ht, hipStream_t st,
                              const float* cum) {
  const bool wsv = ut && states;
  if (cum) {  // gated
    if constexpr (sizeof(E) == 2) {
      if (o && wsv)
        return scan_fwd_run<E, DK, DV, NWC, true, true, false, true>(s, table, q, k, w, u, m, o, ut, states, h0, ht, st, cum);
      if (wsv)
        return scan_fwd_run<E, DK, DV, NWC, false, true, false, true>(s, table, q, k, w, u, m, o, ut, states, h0, ht, st, cum);
      if (o)
        return scan_fwd_run<E, DK, DV, NWC, true, false, false, true>(s, table, q, k, w, u, m, o, ut, states, h0, ht, st, cum);
      if (ht)
        return scan_fwd_run<E, DK, DV, NWC, false, false, false, true>(s, table, q, k, w, u, m, o, ut, states, h0, ht, st, cum);
      return hipSuccess;
    } else {
      return hipErrorInvalidValue;  // the fp32 tiles leave no LDS room for the decays
    }
  }
  if (o && wsv)
    return scan_fwd_run<E, DK, DV, NWC, true, true>(s, table, q, k, w, u, m, o, ut, states, h0, ht, st);
  if (o) return scan_fwd_run<E, DK, DV, NWC, true, false>(s, table, q, k, w, u, m, o, ut, states, h0, ht, st);
  if (wsv)
    return scan_fwd_run<E, DK, DV, NWC, false, true>(s, table, q, k, w, u, m, o, ut, states, h0, ht, st);
  if (ht)
    return scan_fwd_run<E, DK, DV, NWC, false, false>(s, table, q, k, w, u, m, o, ut, states, h0, ht, st);
  return hipSuccess;
}

// bf16: two compute waves (32 state columns), a loader and a storer wave per workgroup; fp32:
// one compute wave (the double-buffered fp32 tiles leave LDS room for 16 columns of staging).
size_t lds_scan_fwd(Dt dt, int dk, int dv) {
  if (dt == Dt::BF16) {
    if (dk == 64 && dv == 64) return ScanFwdLds<__bf16, 64, 64, 2>::bytes;
    if (dk == 64 && dv == 128) return ScanFwdLds<__bf16, 64, 128, 2>::bytes;
    if (dk == 128 && dv == 64) return ScanFwdLds<__bf16, 128, 64, 2>::bytes;
    if (dk == 128 && dv == 128) return ScanFwdLds<__bf16, 128, 128, 2>::bytes;
    return 0;
  }
  if (dk == 64 && dv == 64) return ScanFwdLds<float, 64, 64, 1>::bytes;
  return 0;
}

hipError_t launch_scan_fwd(const Shape& s, const int* table, const void* q, const void* k,
                           const void* w, const void* u, const void* m, void* o, void* ut,
                           void* states, const float* h0, float* ht, hipStream_t st,
                           const float* cum) {
#define EFLA_SF(E_, DK_, DV_, NWC_) \
  return scan_fwd_go<E_, DK_, DV_, NWC_>(s, table, q, k, w, u, m, o, ut, states, h0, ht, st, cum)
  if (s.dt == Dt::BF16) {
    if (s.dk == 64 && s.dv == 64) EFLA_SF(__bf16, 64, 64, 2);
    if (s.dk == 64 && s.dv == 128) EFLA_SF(__bf16, 64, 128, 2);
    if (s.dk == 128 && s.dv == 64) EFLA_SF(__bf16, 128, 64, 2);
    EFLA_SF(__bf16, 128, 128, 2);
  }
  EFLA_SF(float, 64, 64, 1);
#undef EFLA_SF
}

hipError_t launch_scan_fwd_transition(const Shape& s, const void* k, const void* w, float* p,
                                      hipStream_t st, const float* cum) {
#define EFLA_ST(E_, DK_, NWC_)                                                               \
  return scan_fwd_run<E_, DK_, DK_, NWC_, false, false, true>(s, nullptr, nullptr, k, w, nullptr, \
                                                             nullptr, nullptr, nullptr, nullptr, \
                                                             nullptr, p, st)
  if (cum) {
    if (s.dt != Dt::BF16) return hipErrorInvalidValue;
    if (s.dk == 64)
      return scan_fwd_run<__bf16, 64, 64, 2, false, false, true, true>(s, nullptr, nullptr, k, w, nullptr, nullptr,
                                                                      nullptr, nullptr, nullptr, nullptr, p, st, cum);
    return scan_fwd_run<__bf16, 128, 128, 2, false, false, true, true>(s, nullptr, nullptr, k, w, nullptr, nullptr,
                                                                      nullptr, nullptr, nullptr, nullptr, p, st, cum);
  }
  if (s.dt == Dt::BF16) {
    if (s.dk == 64) EFLA_ST(__bf16, 64, 2);
    EFLA_ST(__bf16, 128, 2);
  }
  EFLA_ST(float, 64, 1);
#undef EFLA_ST
}

}  // namespace efla

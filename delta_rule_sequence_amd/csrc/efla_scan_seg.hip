// Segment-parallel inter-chunk scan: the sequential combine step.
//
// Exact Flow Linear Attention summary page, section 3.3: across chunks the state obeys
// S <- S + K^T (U - W S) = (I - K^T W) S + K^T U, an affine map of S. Over a segment of
// consecutive chunks the maps compose to S_out = P S_in + R, where P is the product of the
// (I - K^T W) and R is the state the segment reaches from S_in = 0. Long sequences are cut
// into segments whose P and R are formed in parallel (transition and state-only scans);
// this kernel then walks the segments of each sequence in order,
//   S_0 = h0 (or 0),  S_{j+1} = P_j S_j + R_j,
// writing the state entering every segment (the initial state of the second, output-writing
// scan over the segments) and the state after the last one. The backward pass chains its state
// gradients the same way with the segments taken from the last to the first. States, P and R are held in
// fp32; P_j and S enter the products in the problem dtype, as W and S do in the scan.
//
// One workgroup per (batch row, head). Each wave owns 16 state columns and keeps them in
// fp32 MFMA accumulators, exactly as the scan's compute waves do, so P_j S is formed like the
// scan's W S: S enters as the B operand straight from the accumulators, P_j (staged one
// segment ahead into a swizzled LDS tile, in the problem dtype) is the A operand, and R_j
// (fetched one segment ahead into registers) seeds the accumulation.
#include "efla_internal.hpp"

namespace efla {

template <typename E, int DK>
struct SegLds {
  typedef Swz<E, DK> SP;                             // P_j: DK rows = DK / 64 stacked tiles
  static constexpr size_t TILE = (size_t)SP::BYTES * (DK / 64);
  static constexpr size_t bytes = 2 * TILE;          // double-buffered
};

// rev: walk the segments from the last to the first (state gradients). tr: apply P_j^T instead of
// P_j. Going backwards a segment maps the gradient by the product of the (I - W^T K) of its
// chunks in forward order, which is the transpose of the forward transition (the product of the
// (I - K^T W) in reverse order; with decays both carry e^{c_last} I in place of I), so the
// backward chains with the forward's P.
template <typename E, int DK, int DV>
__global__ __launch_bounds__(64 * (DV / 16)) void seg_combine_kernel(
    int H, int G, int rev, int tr, const float* __restrict__ P, const float* __restrict__ R,
    const float* __restrict__ h0, float* __restrict__ sin, float* __restrict__ ht) {
  typedef SegLds<E, DK> L;
  typedef typename L::SP SP;
  typedef typename Mma<E>::vec V;
  constexpr int NW = DV / 16, NT = 64 * NW, NBK = DK / 16, KSK = DK / Mma<E>::KC;
  constexpr int VE = 16 / (int)sizeof(E);
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  lds_poison(smem);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wi = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.x / H, h = blockIdx.x % H;
  const int col = 16 * wi + (lane & 15), g4 = 4 * (lane >> 4);
  // this lane's entries of a state slice: rows prow(bb, g4 + i), column col
  auto at = [&](const float* base, int64_t seq, int bb, int i) {
    return base + ((seq * H + h) * DK + prow<E>(bb, g4 + i)) * (int64_t)DV + col;
  };
  // processing step j handles segment seg(j): j itself, or G - 1 - j when walking backwards
  auto seg = [&](int j) { return rev ? G - 1 - j : j; };
  auto stage = [&](int j) {  // P of step j (fp32) -> LDS buffer j & 1 in the problem dtype
    unsigned char* dst = smem + (j & 1) * L::TILE;
    const float* Pj = P + (((int64_t)b * G + seg(j)) * H + h) * DK * DK;
    if (tr) {  // tile element (r, c) = P_j[c][r]: rows of P_j read whole, written as columns
      for (int i = tid; i < DK * DK / VE; i += NT) {
        const int rr = i / (DK / VE), cc = (i % (DK / VE)) * VE;
        const f32x4 x0 = *(const f32x4*)(Pj + (int64_t)rr * DK + cc);
        f32x4 x1 = zero4();
        if constexpr (VE == 8) x1 = *(const f32x4*)(Pj + (int64_t)rr * DK + cc + 4);
#pragma unroll
        for (int e = 0; e < VE; ++e)
          *(E*)(dst + SP::off(cc + e, rr)) = to_e<E>(e < 4 ? x0[e & 3] : x1[e & 3]);
      }
      return;
    }
    for (int i = tid; i < DK * DK / VE; i += NT) {
      const int r = i / (DK / VE), c = (i % (DK / VE)) * VE;
      if constexpr (sizeof(E) == 2) {
        const f32x4 x0 = *(const f32x4*)(Pj + (int64_t)r * DK + c);
        const f32x4 x1 = *(const f32x4*)(Pj + (int64_t)r * DK + c + 4);
        *(bf16x8*)(dst + SP::off(r, c)) =
            bf16x8{(__bf16)x0[0], (__bf16)x0[1], (__bf16)x0[2], (__bf16)x0[3],
                   (__bf16)x1[0], (__bf16)x1[1], (__bf16)x1[2], (__bf16)x1[3]};
      } else {
        *(f32x4*)(dst + SP::off(r, c)) = *(const f32x4*)(Pj + (int64_t)r * DK + c);
      }
    }
  };
  f32x4 S[NBK], Rn[NBK];
  auto fetch_r = [&](int j) {
#pragma unroll
    for (int bb = 0; bb < NBK; ++bb)
#pragma unroll
      for (int i = 0; i < 4; ++i) Rn[bb][i] = *at(R, (int64_t)b * G + seg(j), bb, i);
  };
#pragma unroll
  for (int bb = 0; bb < NBK; ++bb)
#pragma unroll
    for (int i = 0; i < 4; ++i) S[bb][i] = h0 ? *at(h0, b, bb, i) : 0.f;
  // segment j's map is needed for j < G - 1, and for the last one only to form ht
  const int used = ht ? G : G - 1;
  if (used > 0) {
    stage(0);
    fetch_r(0);
  }
  __syncthreads();
  for (int j = 0; j < G; ++j) {
    const int64_t sj = (int64_t)b * G + seg(j);
#pragma unroll
    for (int bb = 0; bb < NBK; ++bb)
#pragma unroll
      for (int i = 0; i < 4; ++i) *(float*)at(sin, sj, bb, i) = S[bb][i];
    if (j >= used) break;
    f32x4 acc[NBK];
#pragma unroll
    for (int bb = 0; bb < NBK; ++bb) acc[bb] = Rn[bb];
    if (j + 1 < used) {  // next segment's operands, requested before this one's products
      stage(j + 1);
      fetch_r(j + 1);
    }
    const unsigned char* pt = smem + (j & 1) * L::TILE;
    V sb[KSK];
#pragma unroll
    for (int ks = 0; ks < KSK; ++ks) sb[ks] = bop_acc<E>(S, ks);
#pragma unroll
    for (int rb = 0; rb < NBK; ++rb)
#pragma unroll
      for (int ks = 0; ks < KSK; ++ks) acc[rb] = Mma<E>::step(aop_rc<E, DK>(pt, rb, ks, lane), sb[ks], acc[rb]);
#pragma unroll
    for (int bb = 0; bb < NBK; ++bb) S[bb] = acc[bb];
    __syncthreads();  // P_{j+1} staged for every wave; buffer j & 1 free for P_{j+2}
  }
  if (ht) {
#pragma unroll
    for (int bb = 0; bb < NBK; ++bb)
#pragma unroll
      for (int i = 0; i < 4; ++i) *(float*)at(ht, b, bb, i) = S[bb][i];
  }
}

template <typename E, int DK, int DV>
static hipError_t seg_combine_go(const Shape& s, const float* p, const float* r, const float* h0,
                                 float* sin, float* ht, hipStream_t st, bool rev, bool tr) {
  typedef SegLds<E, DK> L;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)seg_combine_kernel<E, DK, DV>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)L::bytes);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const int64_t blocks = (int64_t)s.B * s.H;
  if (blocks < 1) return hipSuccess;
  prof_begin(st);
  hipLaunchKernelGGL((seg_combine_kernel<E, DK, DV>), dim3((unsigned)blocks), dim3(64 * (DV / 16)),
                     L::bytes, st, s.H, s.seg_plan, rev ? 1 : 0, tr ? 1 : 0, p, r, h0, sin, ht);
  hipError_t e = hipGetLastError();
  prof_end("seg_combine", st);
  return e;
}

hipError_t launch_seg_combine(const Shape& s, const float* p, const float* r, const float* h0,
                              float* sin, float* ht, hipStream_t st, bool rev, bool tr) {
  if (s.dt == Dt::BF16) {
    if (s.dk == 64 && s.dv == 64) return seg_combine_go<__bf16, 64, 64>(s, p, r, h0, sin, ht, st, rev, tr);
    if (s.dk == 64 && s.dv == 128) return seg_combine_go<__bf16, 64, 128>(s, p, r, h0, sin, ht, st, rev, tr);
    if (s.dk == 128 && s.dv == 64) return seg_combine_go<__bf16, 128, 64>(s, p, r, h0, sin, ht, st, rev, tr);
    return seg_combine_go<__bf16, 128, 128>(s, p, r, h0, sin, ht, st, rev, tr);
  }
  return seg_combine_go<float, 64, 64>(s, p, r, h0, sin, ht, st, rev, tr);
}

}  // namespace efla

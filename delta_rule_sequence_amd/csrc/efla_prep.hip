// Per-token coefficient kernel (key energy and exact-flow step) and the chunk-start
// table of packed batches.
//
// Exact Flow Linear Attention summary page, section 3.2: the closed-form update keeps the
// delta rule's form with beta_t replaced by alpha_t; section 3.4: the denominator is the
// key energy lambda_t = ||k_t||^2. Each token's row is reduced by 16 (or 8) lanes with
// wavefront shuffles; the coefficients come from flow_coef (series near zero).
#include "efla_internal.hpp"

namespace efla {

template <typename E, int DK>
__global__ __launch_bounds__(kThreads) void prep_kernel(int64_t ntok, int euler, const E* __restrict__ k,
                                                        const E* __restrict__ beta,
                                                        float* __restrict__ lam,
                                                        float* __restrict__ alpha,
                                                        float* __restrict__ ex,
                                                        float* __restrict__ dlam) {
  constexpr int V = 16 / sizeof(E);
  constexpr int VPR = DK / V;                  // 16-byte vectors per row
  constexpr int LPR = VPR < 16 ? VPR : 16;     // lanes per row
  constexpr int VPL = VPR / LPR;               // vectors per lane
  constexpr int RPB = kThreads / LPR;          // rows per workgroup pass
  typedef typename Mma<E>::vec VT;
  const int tid = threadIdx.x, sub = tid % LPR;
  for (int64_t row = (int64_t)blockIdx.x * RPB + tid / LPR; row < ntok;
       row += (int64_t)gridDim.x * RPB) {
    const E* p = k + row * DK;
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const VT x = *(const VT*)(p + (sub + j * LPR) * V);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const float f = to_f(x[e]);
        acc = fmaf(f, f, acc);
      }
    }
    acc = group_sum<LPR>(acc);
    if (sub == 0) {
      const FlowCoef c = flow_coef(to_f(beta[row]), acc, euler != 0);
      if (lam) lam[row] = acc;
      alpha[row] = c.alpha;
      if (ex) ex[row] = c.ex;
      if (dlam) dlam[row] = c.dlam;
    }
  }
}

// table[s] = sum over s' < s of ceil(len_s' / 64); table[n] = total. One workgroup.
__global__ __launch_bounds__(kThreads) void chunk_table_kernel(const int* __restrict__ cu, int n,
                                                               int T, int* __restrict__ table) {
  __shared__ int part[kThreads];
  const int tid = threadIdx.x;
  const int per = (n + kThreads - 1) / kThreads;
  const int s0 = min(n, tid * per), s1 = min(n, s0 + per);
  auto nchunk = [&](int s) {
    const int a = min(max(cu[s], 0), T);
    const int b = max(min(max(cu[s + 1], 0), T), a);
    return (b - a + kChunk - 1) / kChunk;
  };
  int sum = 0;
  for (int s = s0; s < s1; ++s) sum += nchunk(s);
  part[tid] = sum;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int i = 0; i < kThreads; ++i) {
      const int x = part[i];
      part[i] = run;
      run += x;
    }
    table[n] = run;
  }
  __syncthreads();
  int run = part[tid];
  for (int s = s0; s < s1; ++s) {
    table[s] = run;
    run += nchunk(s);
  }
}

hipError_t launch_chunk_table(const Shape& s, int* table, hipStream_t st) {
  prof_begin(st);
  hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(kThreads), 0, st, s.cu, s.n_seqs, s.T,
                     table);
  hipError_t e = hipGetLastError();
  prof_end("chunk_table", st);
  return e;
}

template <typename E, int DK>
static hipError_t prep_go(const Shape& s, const void* k, const void* beta, float* lam,
                          float* alpha, float* ex, float* dlam, hipStream_t st) {
  const int64_t ntok = (int64_t)s.B * s.H * s.T;
  constexpr int VPR = DK * (int)sizeof(E) / 16;
  constexpr int LPR = VPR < 16 ? VPR : 16;
  constexpr int RPB = kThreads / LPR;
  int64_t blocks = (ntok + RPB - 1) / RPB;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) return hipSuccess;
  prof_begin(st);
  hipLaunchKernelGGL((prep_kernel<E, DK>), dim3((unsigned)blocks), dim3(kThreads), 0, st, ntok,
                     s.euler ? 1 : 0, (const E*)k, (const E*)beta, lam, alpha, ex, dlam);
  hipError_t e = hipGetLastError();
  prof_end("prep", st);
  return e;
}

hipError_t launch_prep(const Shape& s, const void* k, const void* beta, float* lam, float* alpha,
                       float* ex, float* dlam, hipStream_t st) {
  if (s.dt == Dt::BF16) {
    if (s.dk == 64) return prep_go<__bf16, 64>(s, k, beta, lam, alpha, ex, dlam, st);
    return prep_go<__bf16, 128>(s, k, beta, lam, alpha, ex, dlam, st);
  }
  if (s.dk == 64) return prep_go<float, 64>(s, k, beta, lam, alpha, ex, dlam, st);
  return prep_go<float, 128>(s, k, beta, lam, alpha, ex, dlam, st);
}

}  // namespace efla

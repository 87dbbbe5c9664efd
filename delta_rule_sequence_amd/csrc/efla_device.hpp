// Device-side building blocks shared by the EFLA kernels (gfx950 / CDNA4).
//
// Every kernel runs 256 threads = 4 wavefronts of 64 lanes. Dense contractions use
// 16x16 MFMA tiles: v_mfma_f32_16x16x32_bf16 for bf16 problems and
// v_mfma_f32_16x16x4_f32 for fp32 problems, always accumulating in fp32.
//
// Operand convention for a 16x16 output tile C = A * B:
//   A is read as 16 rows of A (row-major, the contraction index contiguous),
//   B is read as 16 rows of B^T (row-major, the contraction index contiguous).
//   Lane l reads row (l & 15) and 16 contiguous bytes of the contraction range
//   starting at (l >> 4) * KC/4 inside each KC-wide step. A and B use the same
//   mapping, so each k-slot pairs the same contraction index in both operands.
//   The accumulator element i of lane l is C[4 * (l >> 4) + i][l & 15].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace efla {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));  // 16 raw bytes in registers

constexpr int kChunk = 64;
constexpr int kThreads = 256;

#define EFLA_DEV __device__ __forceinline__

// Debug build (-DEFLA_LDS_POISON): a kernel with dynamic LDS first fills its whole dynamic LDS
// allocation with all-ones bytes, which read as NaN in fp32 and bf16, and then waits at a
// barrier. A location the kernel reads before writing it in this launch then turns its results
// into NaN instead of silently reusing whatever an earlier workgroup left there. The size comes
// from the dispatch packet (group_segment_size: static + dynamic LDS of this launch). In the
// normal build this is empty. No kernel keeps integers in dynamic LDS, so the poison cannot
// become an address.
EFLA_DEV void lds_poison(unsigned char* smem) {
#ifdef EFLA_LDS_POISON
  const char* pkt = (const char*)__builtin_amdgcn_dispatch_ptr();
  const uint32_t total = *(const uint32_t*)(pkt + 28);
  uint32_t n = (total - __builtin_amdgcn_groupstaticsize()) / 16;
  if (n > 160u * 1024u / 16u) n = 160u * 1024u / 16u;
  const uint32_t nt = blockDim.x;
  for (uint32_t i = threadIdx.x; i < n; i += nt) ((u32x4*)smem)[i] = u32x4{~0u, ~0u, ~0u, ~0u};
  __syncthreads();
#else
  (void)smem;
#endif
}

template <typename E> EFLA_DEV E to_e(float x);
template <> EFLA_DEV float to_e<float>(float x) { return x; }
template <> EFLA_DEV __bf16 to_e<__bf16>(float x) { return (__bf16)x; }
EFLA_DEV float to_f(float x) { return x; }
EFLA_DEV float to_f(__bf16 x) { return (float)x; }

EFLA_DEV f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Row pitch (in elements) of an LDS tile whose rows hold `cols` elements: 16 bytes of
// padding per row spreads consecutive rows over different LDS banks.
template <typename E> constexpr int pitch(int cols) { return cols + 16 / (int)sizeof(E); }
constexpr int kPitchF = 68;  // fp32 64x64 work matrices

// ---------------------------------------------------------------------------
// MFMA step: one 16-byte operand load per lane covers KC contraction indices.
// ---------------------------------------------------------------------------
template <typename E> struct Mma;

template <> struct Mma<float> {
  static constexpr int KC = 16;  // 4 fp32 per lane x 4 lane groups
  typedef f32x4 vec;
  EFLA_DEV static f32x4 step(vec a, vec b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
    return c;
  }
};

template <> struct Mma<__bf16> {
  static constexpr int KC = 32;  // 8 bf16 per lane x 4 lane groups
  typedef bf16x8 vec;
  EFLA_DEV static f32x4 step(vec a, vec b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <typename E> EFLA_DEV constexpr int round_down_kc(int k) { return k - k % Mma<E>::KC; }
template <typename E> EFLA_DEV constexpr int round_up_kc(int k) {
  return (k + Mma<E>::KC - 1) / Mma<E>::KC * Mma<E>::KC;
}

// acc += A[0:16, k0:k1] * B[k0:k1, 0:16]; `a` points at row 0 of A (pitch lda), `bt` at
// row 0 of B^T (pitch ldb). k0 and k1 are multiples of Mma<E>::KC. Works on LDS and
// global pointers alike.
template <typename E>
EFLA_DEV f32x4 mma16(const E* a, int lda, const E* bt, int ldb, int k0, int k1, f32x4 acc,
                     int lane) {
  typedef typename Mma<E>::vec V;
  const int r = lane & 15;
  const int kq = (lane >> 4) * (Mma<E>::KC / 4);
  const E* pa = a + r * lda + kq;
  const E* pb = bt + r * ldb + kq;
  for (int k = k0; k < k1; k += Mma<E>::KC)
    acc = Mma<E>::step(*(const V*)(pa + k), *(const V*)(pb + k), acc);
  return acc;
}

// Same with B^T in global memory addressed with a 64-bit pitch.
template <typename E>
EFLA_DEV f32x4 mma16_gb(const E* a, int lda, const E* __restrict__ bt, int64_t ldb, int k0, int k1,
                        f32x4 acc, int lane) {
  typedef typename Mma<E>::vec V;
  const int r = lane & 15;
  const int kq = (lane >> 4) * (Mma<E>::KC / 4);
  const E* pa = a + r * lda + kq;
  const E* pb = bt + r * ldb + kq;
  for (int k = k0; k < k1; k += Mma<E>::KC)
    acc = Mma<E>::step(*(const V*)(pa + k), *(const V*)(pb + k), acc);
  return acc;
}

// ---------------------------------------------------------------------------
// Fragment loads. The operand X[m][k] of a 16-row tile is either stored "row-major"
// (k contiguous: row m at src + m * ld) or "k-major" (m contiguous: row k at src + k * ld).
// frag_rm: src points at X[m0][k0]; frag_km: src points at storage row k0, column m0.
// Lane l receives X[m0 + (l & 15)][k0 + (l >> 4) * KC/4 + t] for t < KC/4.
// bf16 k-major fragments use the gfx950 LDS transpose read ds_read_b64_tr_b16: within each
// 16-lane group, output lane j, slot s holds element j % 4 of the 8-byte row addressed by
// lane 4 s + j / 4; addressing rows k0 + 8 g + i / 4 (+4) at column m0 + 4 (i % 4) from lane
// i of group g therefore yields the standard operand layout. k-major loads must come from LDS.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

template <typename E>
EFLA_DEV typename Mma<E>::vec frag_rm(const E* src, int ld, int lane) {
  return *(const typename Mma<E>::vec*)(src + (lane & 15) * ld + (lane >> 4) * (Mma<E>::KC / 4));
}

template <typename E> EFLA_DEV typename Mma<E>::vec frag_km(const E* src, int ld, int lane);

// Global memory addressed as a wave-uniform base plus a 32-bit unsigned byte offset per lane:
// the access can then use the scalar-base form (no 64-bit address arithmetic per lane).
template <typename T, typename E> EFLA_DEV T* at_byte(E* base, unsigned byte_off) {
  return (T*)((char*)base + byte_off);
}
template <typename T, typename E> EFLA_DEV const T* at_byte(const E* base, unsigned byte_off) {
  return (const T*)((const char*)base + byte_off);
}

// A copy of a global pointer that the compiler cannot trace back to its kernel argument. Loads
// through it are ordinary loads, ordered with the stores around them; loads through a read-only
// kernel argument may be moved anywhere, e.g. sunk from a loop body to just before the back edge.
template <typename E> EFLA_DEV const E* opaque_global(const E* p) {
  typedef const E __attribute__((address_space(1)))* G;
  G g = (G)p;
  asm volatile("" : "+s"(g));
  return (const E*)g;
}

// frag_rm from global memory, src uniform across the wave.
template <typename E>
EFLA_DEV typename Mma<E>::vec frag_rm_g(const E* __restrict__ src, int ld, int lane) {
  const unsigned off = ((unsigned)(lane & 15) * (unsigned)ld + (unsigned)(lane >> 4) * (Mma<E>::KC / 4)) *
                       (unsigned)sizeof(E);
  return *at_byte<typename Mma<E>::vec>(src, off);
}

template <> EFLA_DEV f32x4 frag_km<float>(const float* src, int ld, int lane) {
  const float* p = src + (lane >> 4) * 4 * ld + (lane & 15);
  return f32x4{p[0], p[ld], p[2 * ld], p[3 * ld]};
}

template <> EFLA_DEV bf16x8 frag_km<__bf16>(const __bf16* src, int ld, int lane) {
  const int gq = lane >> 4, i = lane & 15;
  const __bf16* p = src + (8 * gq + (i >> 2)) * ld + 4 * (i & 3);
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + 4 * ld));
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// acc += A[0:16, k0:k1] * B[k0:k1, 0:16]. A is stored row-major (AK = false; a points at
// row m0) or k-major (AK = true; a points at column m0 of storage row 0). B is given as B^T
// row-major (BK = false; b points at row n0 of B^T) or as B itself, k-major for this
// product (BK = true; b points at column n0 of storage row 0).
template <typename E, bool AK, bool BK>
EFLA_DEV f32x4 mma(const E* a, int lda, const E* b, int ldb, int k0, int k1, f32x4 acc,
                   int lane) {
  for (int k = k0; k < k1; k += Mma<E>::KC) {
    typename Mma<E>::vec av, bv;
    if constexpr (AK) av = frag_km<E>(a + k * lda, lda, lane); else av = frag_rm<E>(a + k, lda, lane);
    if constexpr (BK) bv = frag_km<E>(b + k * ldb, ldb, lane); else bv = frag_rm<E>(b + k, ldb, lane);
    acc = Mma<E>::step(av, bv, acc);
  }
  return acc;
}

// Register-blocked product: acc[i][j] += A_i B_j for NA row blocks and NB column blocks,
// contraction index k in [k0, k1) (multiples of KC inside [0, K)). Row block i of A starts
// 16 i rows (AK = false) or 16 i columns (AK = true, k-major) after a; column block j of B
// likewise after b (BK = false: rows of B^T; BK = true: columns of k-major B). Every operand
// fragment is read from memory once per k step and feeds NB (or NA) products.
// TR = true hands the two operands to the matrix core the other way round, which yields the
// transposed product: the accumulator then holds each block in row layout (lane l owns row
// l & 15, columns 4 (l >> 4) .. + 3), ready for one vector store per lane (st_frag_t).
template <typename E, bool AK, bool BK, int NA, int NB, int K, bool TR = false>
EFLA_DEV void mma_blk(const E* a, int lda, const E* b, int ldb, int k0, int k1,
                      f32x4 (&acc)[NA][NB], int lane) {
  constexpr int KC = Mma<E>::KC;
#pragma unroll
  for (int k = 0; k < K; k += KC) {
    if (k < k0 || k >= k1) continue;
    typename Mma<E>::vec av[NA], bv[NB];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      if constexpr (AK) av[i] = frag_km<E>(a + 16 * i + k * lda, lda, lane);
      else av[i] = frag_rm<E>(a + 16 * i * lda + k, lda, lane);
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if constexpr (BK) bv[j] = frag_km<E>(b + 16 * j + k * ldb, ldb, lane);
      else bv[j] = frag_rm<E>(b + 16 * j * ldb + k, ldb, lane);
    }
#pragma unroll
    for (int i = 0; i < NA; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
        acc[i][j] = TR ? Mma<E>::step(bv[j], av[i], acc[i][j]) : Mma<E>::step(av[i], bv[j], acc[i][j]);
  }
}

template <typename E> EFLA_DEV typename Mma<E>::vec zero_vec() {
  typename Mma<E>::vec v;
#pragma unroll
  for (int i = 0; i < 16 / (int)sizeof(E); ++i) v[i] = to_e<E>(0.f);
  return v;
}

// Store an accumulator tile transposed: s[n][m] = C[m][n] (s points at the tile origin of
// C^T, pitch ld). Four consecutive m per lane become one 8- or 16-byte store.
template <typename E> EFLA_DEV void st_frag_t(E* s, int ld, f32x4 c, int lane);
template <> EFLA_DEV void st_frag_t<float>(float* s, int ld, f32x4 c, int lane) {
  *(f32x4*)(s + (lane & 15) * ld + 4 * (lane >> 4)) = c;
}
template <> EFLA_DEV void st_frag_t<__bf16>(__bf16* s, int ld, f32x4 c, int lane) {
  bf16x4 v = {(__bf16)c[0], (__bf16)c[1], (__bf16)c[2], (__bf16)c[3]};
  *(bf16x4*)(s + (lane & 15) * ld + 4 * (lane >> 4)) = v;
}

// Cross-lane sums inside a 16-lane row with DPP moves folded into the adds (VALU only, no
// LDS-pipe permutes): quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror.
template <int CTRL> EFLA_DEV float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                               0xF, 0xF, false));
}
// Sum over each aligned group of N consecutive lanes (N = 1, 2, 4, 8 or 16); every lane of
// the group receives the sum.
template <int N> EFLA_DEV float group_sum(float x) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16, "group of 1..16 lanes");
  if constexpr (N >= 2) x += dpp_mov<0xB1>(x);
  if constexpr (N >= 4) x += dpp_mov<0x4E>(x);
  if constexpr (N >= 8) x += dpp_mov<0x141>(x);
  if constexpr (N >= 16) x += dpp_mov<0x140>(x);
  return x;
}

// Four consecutive elements as fp32 (8- or 16-byte aligned LDS or global address).
template <typename E> EFLA_DEV f32x4 ld4f(const E* p);
template <> EFLA_DEV f32x4 ld4f<float>(const float* p) { return *(const f32x4*)p; }
template <> EFLA_DEV f32x4 ld4f<__bf16>(const __bf16* p) {
  const bf16x4 v = *(const bf16x4*)p;
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}

// Store an accumulator tile row-major into LDS: s[m][n] = C[m][n]. The ROCm 7.2 LLVM
// backend was seen to pair two such fp32 stores of MFMA results into a ds_write2_b32 with a
// wrong first offset (scaled down by four), silently corrupting the tile. bf16 stores cannot
// be paired (there is no 16-bit ds_write2); between fp32 stores an empty asm statement with a
// memory clobber keeps the backend from pairing them. It costs no instruction.
template <typename E>
EFLA_DEV void st_frag_lds(E* s, int ld, f32x4 c, int lane) {
  E* p = s + 4 * (lane >> 4) * ld + (lane & 15);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    p[i * ld] = to_e<E>(c[i]);
    if constexpr (sizeof(E) == 4) asm volatile("" ::: "memory");
  }
}

// Store an accumulator tile row-major to global memory: g[m][n] = C[m][n].
template <typename E>
EFLA_DEV void st_frag_glb(E* __restrict__ g, int64_t ld, f32x4 c, int lane) {
  E* p = g + (int64_t)(4 * (lane >> 4)) * ld + (lane & 15);
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i * ld] = to_e<E>(c[i]);
}

// Row-major store to global memory keeping only rows < nvalid (relative to the tile origin).
template <typename E>
EFLA_DEV void st_frag_rows(E* __restrict__ g, int64_t ld, f32x4 c, int lane, int row0, int nvalid) {
  const int rb = 4 * (lane >> 4);
  E* p = g + (int64_t)rb * ld + (lane & 15);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (row0 + rb + i < nvalid) p[i * ld] = to_e<E>(c[i]);
}

// ---------------------------------------------------------------------------
// A 16-byte vector, or zero unless `keep`. Written as a bitwise mask: a conditional
// expression over register arrays can otherwise become a select between two private-memory
// addresses (the arrays then live in scratch).
EFLA_DEV u32x4 keep_if(u32x4 x, bool keep) {
  const unsigned m = keep ? ~0u : 0u;
  return x & m;
}
template <typename Vt> EFLA_DEV Vt keep_if_vec(Vt x, bool keep) {
  static_assert(sizeof(Vt) == 16, "16-byte vectors only");
  return __builtin_bit_cast(Vt, keep_if(__builtin_bit_cast(u32x4, x), keep));
}

// Global -> LDS tile copies (64 rows, rows >= nvalid read as zero).
// ---------------------------------------------------------------------------
template <typename E, int COLS>
EFLA_DEV void g2s(E* s, int ld, const E* __restrict__ g, int64_t gld, int nvalid, int tid) {
  constexpr int V = 16 / sizeof(E);
  constexpr int VPR = COLS / V;
  constexpr int TOT = kChunk * VPR;
#pragma unroll
  for (int it = 0; it < (TOT + kThreads - 1) / kThreads; ++it) {
    const int i = it * kThreads + tid;
    if (TOT % kThreads == 0 || i < TOT) {
      const int r = i / VPR, c = (i % VPR) * V;
      u32x4 val = u32x4{0u, 0u, 0u, 0u};
      if (r < nvalid) val = *(const u32x4*)(g + (int64_t)r * gld + c);
      *(u32x4*)(s + r * ld + c) = val;
    }
  }
}

// Transposed copy: s[c][r] = g[r][c] for r < 64, c < COLS.
template <typename E, int COLS>
EFLA_DEV void g2s_t(E* s, int ld, const E* __restrict__ g, int64_t gld, int nvalid, int tid);

template <int COLS>
EFLA_DEV void g2s_t_impl_f32(float* s, int ld, const float* __restrict__ g, int64_t gld, int nvalid,
                             int tid) {
  constexpr int VPR = COLS / 4;
  constexpr int TOT = kChunk * VPR;
#pragma unroll
  for (int it = 0; it < (TOT + kThreads - 1) / kThreads; ++it) {
    const int i = it * kThreads + tid;
    if (TOT % kThreads == 0 || i < TOT) {
      const int r = i % kChunk, c = (i / kChunk) * 4;
      f32x4 val = zero4();
      if (r < nvalid) val = *(const f32x4*)(g + (int64_t)r * gld + c);
#pragma unroll
      for (int e = 0; e < 4; ++e) s[(c + e) * ld + r] = val[e];
    }
  }
}

template <int COLS>
EFLA_DEV void g2s_t_impl_bf16(__bf16* s, int ld, const __bf16* __restrict__ g, int64_t gld,
                              int nvalid, int tid) {
  // Each thread moves two rows x 8 columns and writes eight 4-byte row pairs.
  constexpr int VPR = COLS / 8;
  constexpr int TOT = (kChunk / 2) * VPR;
#pragma unroll
  for (int it = 0; it < (TOT + kThreads - 1) / kThreads; ++it) {
    const int i = it * kThreads + tid;
    if (TOT % kThreads == 0 || i < TOT) {
      const int rp = i % (kChunk / 2), c = (i / (kChunk / 2)) * 8;
      const int r = 2 * rp;
      bf16x8 v0, v1;
      for (int e = 0; e < 8; ++e) { v0[e] = (__bf16)0.f; v1[e] = (__bf16)0.f; }
      if (r < nvalid) v0 = *(const bf16x8*)(g + (int64_t)r * gld + c);
      if (r + 1 < nvalid) v1 = *(const bf16x8*)(g + (int64_t)(r + 1) * gld + c);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bf16x2 pr = {v0[e], v1[e]};
        *(bf16x2*)(s + (c + e) * ld + r) = pr;
      }
    }
  }
}

template <typename E, int COLS>
EFLA_DEV void g2s_t(E* s, int ld, const E* __restrict__ g, int64_t gld, int nvalid, int tid) {
  if constexpr (sizeof(E) == 4)
    g2s_t_impl_f32<COLS>((float*)s, ld, (const float*)g, gld, nvalid, tid);
  else
    g2s_t_impl_bf16<COLS>((__bf16*)s, ld, (const __bf16*)g, gld, nvalid, tid);
}

// Copy rows [0, nvalid) of a 64-row LDS tile to global memory with 16-byte stores (NT threads
// cooperate, 1 <= nvalid <= 64). Every thread stores on every step: work past the end is
// clamped onto the last row and chunk, so those lanes write the same bytes again. With no store
// inside a branch the compiler knows how many stores follow an earlier load and waits for that
// load alone, not for the stores.
template <typename E, int COLS, int NT = kThreads>
EFLA_DEV void s2g(E* __restrict__ g, int64_t gld, const E* s, int ld, int nvalid, int tid) {
  constexpr int V = 16 / sizeof(E);
  constexpr int VPR = COLS / V;
  constexpr int TOT = kChunk * VPR;
#pragma unroll
  for (int it = 0; it < (TOT + NT - 1) / NT; ++it) {
    const int i = TOT % NT == 0 ? it * NT + tid : min(it * NT + tid, TOT - 1);
    const int r = min(i / VPR, nvalid - 1), c = (i % VPR) * V;
    // 32-bit unsigned element offset from the (uniform) tile base: the store can use the
    // scalar-base addressing form instead of a 64-bit address per lane.
    const unsigned off = ((unsigned)r * (unsigned)gld + (unsigned)c) * (unsigned)sizeof(E);
    *at_byte<u32x4>(g, off) = *(const u32x4*)(s + r * ld + c);
  }
}

// ---------------------------------------------------------------------------
// Swizzled [64][COLS] LDS tiles filled by LDS DMA (global_load_lds_dwordx4). One DMA
// instruction writes 1 KiB of LDS contiguously (16 bytes per lane), so the rows carry no
// padding; instead 16-byte chunk c of row r sits at chunk c ^ (r mod NCH), NCH = chunks per
// row, which spreads the 16 rows of one MFMA operand fetch over the LDS banks.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;

template <typename E, int COLS, int SH = 0, int MX = 0>
struct Swz {
  static constexpr int RB = COLS * (int)sizeof(E);  // bytes per row
  static constexpr int NCH = RB / 16;
  static constexpr int BYTES = 64 * RB;
  static_assert((NCH & (NCH - 1)) == 0 && BYTES % 1024 == 0, "swizzled tile shape");
  // The 16-byte chunk index of row r is XORed with mask(r): bits SH.. of the row (SH = 2 for
  // tiles read in accumulator layout, whose lanes hold rows 4 (lane >> 4) + i). MX = 1 selects,
  // for bf16 rows of 128 elements, a mask built so that none of the tile's readers meets a bank
  // conflict it can avoid: with row bits r0..r4 the mask bits are (r2 ^ r3, r0, r1, r3 ^ r4). It
  // is one-to-one on any 16 consecutive rows (16-byte row-major reads), on the rows
  // prow(b, 0..15) of an A operand, and, in bits 1..3, on the rows {0..3, 8..11} + const of a
  // transposed read of two adjacent chunks. (It costs a few more instructions per address than
  // the plain mask, which some kernels cannot spare.)
  EFLA_DEV static int mask(int r) {
    if constexpr (MX == 1 && sizeof(E) == 2 && COLS == 128 && SH == 0)
      return (((r >> 2) ^ (r >> 3)) & 1) | ((r & 3) << 1) | ((((r >> 3) ^ (r >> 4)) & 1) << 3);
    else
      return (r >> SH) & (NCH - 1);
  }
  // byte offset of element (r, c)
  EFLA_DEV static int off(int r, int c) {
    const int b = c * (int)sizeof(E);
    return r * RB + (((b >> 4) ^ mask(r)) << 4) + (b & 15);
  }
};

// Request rows [0, 64) of a [64][COLS] tile (row r at g + r * gld; rows >= n repeat row n - 1,
// so every address stays inside the chunk) into the swizzled LDS tile at dst. The NW waves
// that call it share the instructions: wave wi issues numbers wi, wi + NW, ...
template <typename E, int COLS, int NW, int SH = 0, int MX = 0>
EFLA_DEV void dma_tile(unsigned char* dst, const E* __restrict__ g, int64_t gld, int n, int wi,
                       int lane) {
  typedef Swz<E, COLS, SH, MX> S;
  constexpr int NI = S::BYTES / 1024;
  static_assert(NI % NW == 0, "DMA split");
#pragma unroll
  for (int jj = 0; jj < NI / NW; ++jj) {
    const int j = jj * NW + wi;
    const int byte = j * 1024 + lane * 16;
    const int r = byte / S::RB, pc = (byte % S::RB) >> 4;
    const int lc = pc ^ S::mask(r);
    // a 32-bit byte offset from the wave-uniform base: scalar-base addressing, no per-lane
    // 64-bit address arithmetic (the tile spans under 64 rows of gld elements)
    const unsigned off = (unsigned)(min(r, n - 1) * (int)gld * (int)sizeof(E) + 16 * lc);
    __builtin_amdgcn_global_load_lds((const void*)at_byte<unsigned char>(g, off),
                                     (lds_void*)(dst + j * 1024), 16, 0, 0);
  }
}

// Request 64 consecutive floats (one per lane) into LDS at dst by LDS DMA: lane l's word lands
// at dst + 4 l. No register takes the value, so nothing but the counted wait for the DMA has
// to precede its use (a plain load followed by an LDS store makes the compiler wait for every
// load in flight, the L2 warm-up loads included).
EFLA_DEV void dma_vec64(unsigned char* dst, const float* __restrict__ g, int lane) {
  __builtin_amdgcn_global_load_lds((const void*)at_byte<unsigned char>(g, 4u * (unsigned)lane),
                                   (lds_void*)dst, 4, 0, 0);
}

// Wait until this wave's outstanding vector memory operations (loads, stores, LDS DMA) are
// done: s_waitcnt vmcnt(0).
EFLA_DEV void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// L2 warm-up for a later read of bytes [0, nbytes) at p (nbytes > 0). Part `part` of `nparts`
// (the workgroups that will all read the range) is shared by NT threads; thread `lane` of them
// takes the 128-byte lines part + nparts (lane + NT i), i < N, and loads one word of each into
// w. A line index past the end is clamped to the last line, so every address stays inside the
// range. The caller leaves w alone until l2_sink, so no wait for these loads is placed before
// that point.
template <int N, int NT = 64>
EFLA_DEV void l2_touch(int* w, const void* p, int nbytes, int part, int nparts, int lane) {
  const int last = (nbytes - 1) >> 7;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int j = min(part + nparts * (lane + NT * i), last);
    w[i] = *(const int*)((const char*)p + (j << 7));
  }
}
// Consumes the words of l2_touch: the compiler waits for those loads here and nowhere earlier.
template <int N>
EFLA_DEV void l2_sink(const int* w) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" ::"v"(w[i]));
}
// The same warm-up by LDS DMA into `dummy` (256 bytes of LDS that nothing reads; each request
// writes one word per lane there): no register receives the data, so the compiler places no
// wait for these loads anywhere (a register load consumed in the next loop iteration gets a
// wait for every vector memory operation in flight). The caller's counted vmcnt waits see them
// as ordinary loads, N per call, issued in order.
template <int N, int NT = 64>
EFLA_DEV void l2_touch_lds(unsigned char* dummy, const void* p, int nbytes, int part, int nparts,
                           int lane) {
  const int last = (nbytes - 1) >> 7;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int j = min(part + nparts * (lane + NT * i), last);
    __builtin_amdgcn_global_load_lds((const void*)at_byte<unsigned char>((const unsigned char*)p, (unsigned)j << 7),
                                     (lds_void*)dummy, 4, 0, 0);
  }
}

// MFMA operands in the accumulator-compatible contraction order. A 16x16 accumulator tile
// holds rows 4 (lane >> 4) + i of column lane & 15, so for a product whose contraction index
// runs over accumulator rows the k slots of one step are taken as
//   bf16 (KC = 32): k = 32 ks + 16 h + 4 (lane >> 4) + i   (h = 0, 1; i < 4)
//   fp32 (KC = 16): k = 16 ks + 4 (lane >> 4) + i
// bop_acc builds the B operand straight from accumulator tiles c[] (tile b = rows 16 b..);
// aop_rm / aop_km read the matching A operand from a swizzled LDS tile stored with the
// contraction index along columns (aop_rm: A[m][k] at (m, k)) or along rows (aop_km:
// A[m][k] at (k, m), LDS transpose reads for bf16).
template <typename E> EFLA_DEV typename Mma<E>::vec bop_acc(const f32x4* c, int ks);
template <> EFLA_DEV f32x4 bop_acc<float>(const f32x4* c, int ks) { return c[ks]; }
template <> EFLA_DEV bf16x8 bop_acc<__bf16>(const f32x4* c, int ks) {
  const f32x4 a = c[2 * ks], b = c[2 * ks + 1];
  return bf16x8{(__bf16)a[0], (__bf16)a[1], (__bf16)a[2], (__bf16)a[3],
                (__bf16)b[0], (__bf16)b[1], (__bf16)b[2], (__bf16)b[3]};
}

template <typename E, int COLS>
EFLA_DEV typename Mma<E>::vec aop_rm(const unsigned char* t, int m0, int ks, int lane) {
  typedef Swz<E, COLS> S;
  const int r = m0 + (lane & 15), g4 = 4 * (lane >> 4);
  if constexpr (sizeof(E) == 2) {
    const bf16x4 lo = *(const bf16x4*)(t + S::off(r, 32 * ks + g4));
    const bf16x4 hi = *(const bf16x4*)(t + S::off(r, 32 * ks + 16 + g4));
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  } else {
    return *(const f32x4*)(t + S::off(r, 16 * ks + g4));
  }
}

// Contiguous-contraction order. bop_acc hands lane group g of a bf16 B operand the rows
// 4 g + i of accumulator tiles 2 ks and 2 ks + 1, so its A operand needs columns
// 32 ks + 4 g.. and 32 ks + 16 + 4 g.. (two 8-byte LDS reads, which the compiler pairs into
// the slow ds_read2 forms). Numbering the accumulator rows instead so that tile b, MFMA row
// r stands for row prow(b, r) of the matrix (tiles 2j and 2j + 1 of each 32-row block
// interleave in runs of four) gives every lane group 8 consecutive rows, 32 ks + 8 g.., and
// the matching A operand is one 16-byte read. The numbering is chosen by the rows the
// producing product's A operand is fed in (aop_rc / aop_kc below), so it costs nothing; only
// the code that moves accumulator entries to or from memory must use prow. fp32 operands
// (KC = 16) are contiguous already.
template <typename E> EFLA_DEV constexpr int prow(int b, int r) {
  if constexpr (sizeof(E) == 2) return 32 * (b >> 1) + 8 * (r >> 2) + 4 * (b & 1) + (r & 3);
  else return 16 * b + r;
}

// A operand, row-major in a swizzled tile, for a product whose B operand is bop_acc of
// prow-ordered accumulators and whose result is prow-ordered: output tile rb takes rows
// prow(rb, lane & 15), contraction slots ks.
template <typename E, int COLS, int MX = 0>
EFLA_DEV typename Mma<E>::vec aop_rc(const unsigned char* t, int rb, int ks, int lane) {
  typedef Swz<E, COLS, 0, MX> S;
  const int r = prow<E>(rb, lane & 15), g = lane >> 4;
  if constexpr (sizeof(E) == 2) return *(const bf16x8*)(t + S::off(r, 32 * ks + 8 * g));
  else return *(const f32x4*)(t + S::off(r, 16 * ks + 4 * g));
}

// The same with the contraction index along the tile's rows (k-major, LDS transpose reads
// for bf16): output tile b takes columns prow(b, lane & 15).
template <typename E, int COLS, int MX = 0>
EFLA_DEV typename Mma<E>::vec aop_kc(const unsigned char* t, int b, int ks, int lane) {
  typedef Swz<E, COLS, 0, MX> S;
  const int i = lane & 15, g = lane >> 4;
  if constexpr (sizeof(E) == 2) {
    // transpose read: output lane j, slot s gets element j % 4 of the 8-byte row that lane
    // 4 s + j / 4 addresses; lane i addresses row 32 ks + 8 g + i / 4 (then + 4) at column
    // prow(b, 4 (i & 3)), so lane j receives column prow(b, j) of rows 32 ks + 8 g + s.
    const int r = 32 * ks + 8 * g + (i >> 2), c = prow<E>(b, 4 * (i & 3));
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(t + S::off(r, c)));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(t + S::off(r + 4, c)));
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  } else {
    const int r = 16 * ks + 4 * g, c = 16 * b + i;
    return f32x4{*(const float*)(t + S::off(r, c)), *(const float*)(t + S::off(r + 1, c)),
                 *(const float*)(t + S::off(r + 2, c)), *(const float*)(t + S::off(r + 3, c))};
  }
}

// aop_kc for a plain row-major tile with leading dimension ld (no swizzle).
template <typename E>
EFLA_DEV typename Mma<E>::vec aop_kc_ld(const E* t, int ld, int b, int ks, int lane) {
  const int i = lane & 15, g = lane >> 4;
  if constexpr (sizeof(E) == 2) {
    const int r = 32 * ks + 8 * g + (i >> 2), c = prow<E>(b, 4 * (i & 3));
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(t + r * ld + c));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(t + (r + 4) * ld + c));
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  } else {
    const int r = 16 * ks + 4 * g, c = 16 * b + i;
    return f32x4{t[r * ld + c], t[(r + 1) * ld + c], t[(r + 2) * ld + c], t[(r + 3) * ld + c]};
  }
}

// Standard-order fragments (as frag_rm / frag_km: lane group g takes k0 + KC/4 g..) from a
// swizzled LDS tile (swizzle keyed on row >> SH): frag_rm_sw reads A[m0 + (lane & 15)][k0..] with
// A[m][k] at (m, k); frag_km_sw reads X[k0..][m0 + (lane & 15)] with X stored at (k, m), by
// transpose reads.
template <typename E, int COLS, int SH = 0, int MX = 0>
EFLA_DEV typename Mma<E>::vec frag_rm_sw(const unsigned char* t, int m0, int k0, int lane) {
  typedef Swz<E, COLS, SH, MX> S;
  return *(const typename Mma<E>::vec*)(t + S::off(m0 + (lane & 15), k0 + (lane >> 4) * (Mma<E>::KC / 4)));
}
template <typename E, int COLS, int SH = 0, int MX = 0>
EFLA_DEV typename Mma<E>::vec frag_km_sw(const unsigned char* t, int k0, int m0, int lane) {
  typedef Swz<E, COLS, SH, MX> S;
  const int gq = lane >> 4, i = lane & 15;
  if constexpr (sizeof(E) == 2) {
    const int r = k0 + 8 * gq + (i >> 2), c = m0 + 4 * (i & 3);
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(t + S::off(r, c)));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(t + S::off(r + 4, c)));
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  } else {
    const int r = k0 + 4 * gq, c = m0 + i;
    return f32x4{*(const float*)(t + S::off(r, c)), *(const float*)(t + S::off(r + 1, c)),
                 *(const float*)(t + S::off(r + 2, c)), *(const float*)(t + S::off(r + 3, c))};
  }
}

template <typename E, int COLS>
EFLA_DEV typename Mma<E>::vec aop_km(const unsigned char* t, int m0, int ks, int lane) {
  typedef Swz<E, COLS> S;
  const int i = lane & 15, g = lane >> 4;
  if constexpr (sizeof(E) == 2) {
    const int r = 32 * ks + 4 * g + (i >> 2), c = m0 + 4 * (i & 3);
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(t + S::off(r, c)));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(t + S::off(r + 16, c)));
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  } else {
    const int r = 16 * ks + 4 * g, c = m0 + i;
    return f32x4{*(const float*)(t + S::off(r, c)), *(const float*)(t + S::off(r + 1, c)),
                 *(const float*)(t + S::off(r + 2, c)), *(const float*)(t + S::off(r + 3, c))};
  }
}

// ---------------------------------------------------------------------------
// Per-token coefficients of the exact flow.
//   x = beta * lambda, phi(x) = (1 - e^-x) / x,
//   alpha = beta phi(x), d alpha / d beta = e^-x, d alpha / d lambda = beta^2 phi'(x).
// With euler set the step is the delta rule's own: alpha = beta, d alpha / d beta = 1,
// d alpha / d lambda = 0.
// For |x| < 1 phi and phi' are Taylor polynomials (degree 11; truncation < 2e-10
// relative), which avoids the cancellation of the closed forms near zero; elsewhere
// the closed forms with expm1 are used. Overflow for large negative x follows IEEE.
// ---------------------------------------------------------------------------
struct FlowCoef {
  float alpha, ex, dlam;
};

// Decay factors of gated EFLA (e^{c} for running log-decay sums c): the hardware base-2
// exponential after one multiply by log2(e), two instructions instead of the libm sequence.
// The product's rounding gives a relative error of about |x| 2^-24 on top of the instruction's
// ~1 ulp, far below the resolution of bf16 data; results below the normal range may flush to 0.
EFLA_DEV float exp_decay(float x) { return __builtin_amdgcn_exp2f(x * 1.44269504088896341f); }

// M = tril(Q K^T) of one chunk (gated: M_ts = e^{c_t - c_s} q_t . k_s for s <= t) from the
// swizzled [64][DK] Q and K tiles (mask MX) into the swizzled [64][64] M tile, by one wave: the ten blocks
// on and below the diagonal, and zeros in blocks (0,1) and (2,3), which readers that step over
// the columns 32 at a time also read. Formed transposed (K Q^T), so that a lane holds four
// consecutive columns of one row and stores them at once; every K and Q fragment is read from
// LDS once (K's for the whole tile, Q's per row block). c: the chunk's running log-decay sums in
// LDS (gated). The scans' loader waves call it once a chunk's tiles have landed.
template <typename E, int DK, bool GT, int MX = 0>
EFLA_DEV void m_tile(unsigned char* sm, const unsigned char* sq, const unsigned char* sk,
                     const float* c, int lane) {
  typedef Swz<E, 64> SM;
  typedef typename Mma<E>::vec V;
  constexpr int KC = Mma<E>::KC, KS = DK / KC;
  const int g4 = 4 * (lane >> 4), cl = lane & 15;
  V kf[4][KS];
#pragma unroll
  for (int sb = 0; sb < 4; ++sb)
#pragma unroll
    for (int kd = 0; kd < KS; ++kd) kf[sb][kd] = frag_rm_sw<E, DK, 0, MX>(sk, 16 * sb, kd * KC, lane);
  // gated: every decay sum this lane needs, read up front (rows t = 16 tb + cl, columns
  // s = 16 sb + g4 + i), so the decay factors below wait for no LDS read
  // (scaled by log2 e once, so that each factor e^{c_t - c_s} is one subtraction and one exp2)
  float crow[4];
  f32x4 ccol[4];
  if constexpr (GT) {
    constexpr float kLog2e = 1.44269504088896341f;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      crow[b] = c[16 * b + cl] * kLog2e;
      ccol[b] = *(const f32x4*)(c + 16 * b + g4) * kLog2e;
    }
  }
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    const int t = 16 * tb + cl;
    const float ct = GT ? crow[tb] : 0.f;
    V qf[KS];
#pragma unroll
    for (int kd = 0; kd < KS; ++kd) qf[kd] = frag_rm_sw<E, DK, 0, MX>(sq, 16 * tb, kd * KC, lane);
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
      const bool zero_blk = (tb == 0 && sb == 1) || (tb == 2 && sb == 3);
      if (sb > tb && !zero_blk) continue;
      f32x4 m = zero4();
      if (sb <= tb) {
#pragma unroll
        for (int kd = 0; kd < KS; ++kd) m = Mma<E>::step(kf[sb][kd], qf[kd], m);
#pragma unroll
        for (int i = 0; i < 4; ++i) {  // element i: row t, column s = 16 sb + g4 + i
          const int s = 16 * sb + g4 + i;
          if constexpr (GT) m[i] *= __builtin_amdgcn_exp2f(ct - ccol[sb][i]);
          if (sb == tb) m[i] = s <= t ? m[i] : 0.f;  // below the diagonal blocks, s < t always
        }
      }
      if constexpr (sizeof(E) == 2)
        *(bf16x4*)(sm + SM::off(t, 16 * sb + g4)) = bf16x4{(__bf16)m[0], (__bf16)m[1], (__bf16)m[2], (__bf16)m[3]};
      else
        *(f32x4*)(sm + SM::off(t, 16 * sb + g4)) = m;
    }
  }
}

// phi(x) = (1 - e^{-x}) / x (phi(0) = 1): Taylor polynomial for |x| < 1 (degree 11), else the
// closed form with expm1.
EFLA_DEV float phi_f(float x) {
  if (fabsf(x) < 1.0f) {
    // phi(x)  = sum_{n>=0} (-1)^n x^n / (n+1)!
    float ph = -1.0f / 479001600.0f;
    ph = fmaf(ph, x, 1.0f / 39916800.0f);
    ph = fmaf(ph, x, -1.0f / 3628800.0f);
    ph = fmaf(ph, x, 1.0f / 362880.0f);
    ph = fmaf(ph, x, -1.0f / 40320.0f);
    ph = fmaf(ph, x, 1.0f / 5040.0f);
    ph = fmaf(ph, x, -1.0f / 720.0f);
    ph = fmaf(ph, x, 1.0f / 120.0f);
    ph = fmaf(ph, x, -1.0f / 24.0f);
    ph = fmaf(ph, x, 1.0f / 6.0f);
    ph = fmaf(ph, x, -0.5f);
    return fmaf(ph, x, 1.0f);
  }
  return -expm1f(-x) / x;
}

// phi'(x) = (e^{-x} (1 + x) - 1) / x^2 (phi'(0) = -1/2): Taylor polynomial for |x| < 1
// (the closed form cancels there), else the closed form.
EFLA_DEV float dphi_f(float x) {
  if (fabsf(x) < 1.0f) {
    // phi'(x) = sum_{n>=0} (n+1) (-1)^(n+1) x^n / (n+2)!
    float d = 1.0f / 518918400.0f;
    d = fmaf(d, x, -1.0f / 43545600.0f);
    d = fmaf(d, x, 1.0f / 3991680.0f);
    d = fmaf(d, x, -1.0f / 403200.0f);
    d = fmaf(d, x, 1.0f / 45360.0f);
    d = fmaf(d, x, -1.0f / 5760.0f);
    d = fmaf(d, x, 1.0f / 840.0f);
    d = fmaf(d, x, -1.0f / 144.0f);
    d = fmaf(d, x, 1.0f / 30.0f);
    d = fmaf(d, x, -1.0f / 8.0f);
    d = fmaf(d, x, 1.0f / 3.0f);
    return fmaf(d, x, -0.5f);
  }
  return (expf(-x) * (1.0f + x) - 1.0f) / (x * x);
}

// Input coefficient of gated EFLA: with the log-decay a added to the dynamics as -a / beta
// times the identity over the step interval, the exact flow's input term is
// int_0^beta e^{-(gamma + lambda) s} ds = beta phi(beta lambda - a) (beta in the delta-rule mode,
// the gated delta rule's own input step).
EFLA_DEV float gated_input_coef(float beta, float lam, float a, bool euler) {
  return euler ? beta : beta * phi_f(beta * lam - a);
}

// b = beta phi(beta lambda - a) and its partial derivatives: db/dbeta = phi(y) + beta lambda
// phi'(y), db/dlambda = beta^2 phi'(y), db/da = -beta phi'(y), y = beta lambda - a
// (delta-rule mode: b = beta, 1, 0, 0).
struct GatedCoef {
  float b, db_dbeta, db_dlam, db_da;
};
EFLA_DEV GatedCoef gated_coef(float beta, float lam, float a, bool euler) {
  if (euler) return GatedCoef{beta, 1.0f, 0.0f, 0.0f};
  const float y = beta * lam - a, ph = phi_f(y), dph = dphi_f(y);
  return GatedCoef{beta * ph, ph + beta * lam * dph, beta * beta * dph, -beta * dph};
}

EFLA_DEV FlowCoef flow_coef(float beta, float lam, bool euler = false) {
  if (euler) return FlowCoef{beta, 1.0f, 0.0f};  // delta rule: alpha = beta
  const float x = beta * lam;
  float ph, dph;
  const float ex = expf(-x);
  if (fabsf(x) < 1.0f) {
    ph = phi_f(x);
    // phi'(x) = sum_{n>=0} (n+1) (-1)^(n+1) x^n / (n+2)!
    dph = 1.0f / 518918400.0f;
    dph = fmaf(dph, x, -1.0f / 43545600.0f);
    dph = fmaf(dph, x, 1.0f / 3991680.0f);
    dph = fmaf(dph, x, -1.0f / 403200.0f);
    dph = fmaf(dph, x, 1.0f / 45360.0f);
    dph = fmaf(dph, x, -1.0f / 5760.0f);
    dph = fmaf(dph, x, 1.0f / 840.0f);
    dph = fmaf(dph, x, -1.0f / 144.0f);
    dph = fmaf(dph, x, 1.0f / 30.0f);
    dph = fmaf(dph, x, -1.0f / 8.0f);
    dph = fmaf(dph, x, 1.0f / 3.0f);
    dph = fmaf(dph, x, -0.5f);
  } else {
    ph = -expm1f(-x) / x;
    dph = (ex * (1.0f + x) - 1.0f) / (x * x);
  }
  return FlowCoef{beta * ph, ex, beta * beta * dph};
}

// ---------------------------------------------------------------------------
// Chunk geometry. A "sequence" is one batch row (dense) or one packed segment.
// Chunk slots number the chunks of all sequences: slot = b * ntc + c (dense) or
// table[s] + c (packed), with table[s] = sum of ceil(len/64) over earlier sequences.
// ---------------------------------------------------------------------------
struct Geom {
  int B, H, T;
  int n_seqs;          // B for dense batches
  int ntc;             // ceil(T / 64) for dense batches
  const int* cu;       // packed: cu_seqlens, else nullptr
  const int* table;    // packed: chunk start table [n_seqs + 1], else nullptr
  int max_slots;       // chunk slots the state buffers hold per head
  float scale;
  int euler;           // step rule: 0 exact flow, 1 delta rule (alpha = beta)
  int seg;             // dense batches only: > 1 splits every sequence into seg segments of
  int seg_nc;          // seg_nc chunks (the last one shorter); sequence index = b * seg + j
};

struct SeqInfo {
  int b, bos, len, slot0;
};

// Offsets are clamped into [0, T] so that a malformed cu_seqlens cannot send a kernel
// outside the tensors (the result is then meaningless but memory stays in bounds).
EFLA_DEV int clamp_t(const Geom& g, int x) { return min(max(x, 0), g.T); }

EFLA_DEV SeqInfo seq_info(const Geom& g, int s) {
  if (g.cu) {
    const int bos = clamp_t(g, g.cu[s]);
    const int end = max(clamp_t(g, g.cu[s + 1]), bos);
    return SeqInfo{0, bos, end - bos, g.table[s]};
  }
  if (g.seg > 1) {
    const int b = s / g.seg, j = s - b * g.seg;
    const int bos = min(j * g.seg_nc * kChunk, g.T);
    return SeqInfo{b, bos, min(g.seg_nc * kChunk, g.T - bos), b * g.ntc + j * g.seg_nc};
  }
  return SeqInfo{s, 0, g.T, s * g.ntc};
}

// Number of chunks of a sequence that fit in the state buffers.
EFLA_DEV int seq_chunks(const Geom& g, const SeqInfo& si) {
  const int nc = (si.len + kChunk - 1) / kChunk;
  return max(0, min(nc, g.max_slots - si.slot0));
}

struct ChunkInfo {
  int b, t0, n;   // batch row, first token (absolute T index), valid rows
};

// Returns false when the slot is past the last chunk of a packed batch.
EFLA_DEV bool chunk_info(const Geom& g, int slot, ChunkInfo& ci) {
  if (!g.cu) {
    const int c = slot % g.ntc;
    ci.b = slot / g.ntc;
    ci.t0 = c * kChunk;
    ci.n = min(kChunk, g.T - ci.t0);
    return true;
  }
  if (slot >= g.max_slots || slot >= g.table[g.n_seqs]) return false;
  int lo = 0, hi = g.n_seqs - 1;  // largest s with table[s] <= slot
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (g.table[mid] <= slot) lo = mid; else hi = mid - 1;
  }
  const SeqInfo si = seq_info(g, lo);
  const int c = slot - si.slot0;
  ci.b = 0;
  ci.t0 = si.bos + c * kChunk;
  ci.n = min(kChunk, si.len - c * kChunk);
  return ci.n > 0;
}

// Work unit u = slot * H + h of the chunk-parallel kernels: valid rows of the chunk, its
// first row in the [B,H,T,*] tensors and the index of its [slot][H] blocks.
struct ChunkUnit {
  int n;
  int64_t row0, sh;
};

// Chunk slots in use: a packed batch may leave the tail of the slot range empty, and the
// used units u < used_slots * H are then exactly the valid ones.
EFLA_DEV int used_slots(const Geom& g) {
  return g.cu ? min(g.table[g.n_seqs], g.max_slots) : g.max_slots;
}

EFLA_DEV ChunkUnit chunk_unit(const Geom& g, int u) {
  const int slot = u / g.H, h = u % g.H;
  ChunkInfo ci;
  chunk_info(g, slot, ci);
  ChunkUnit r;
  r.n = max(ci.n, 1);
  r.row0 = (int64_t)(ci.b * g.H + h) * g.T + ci.t0;
  r.sh = (int64_t)slot * g.H + h;
  return r;
}

// Map a linear workgroup id to (sequence*H + head, d_v tile) so that the tiles of one
// (sequence, head) land on the same XCD (workgroups are dealt to the 8 XCDs round-robin)
// and share its L2 for the K, Q, W tiles they all read.
EFLA_DEV void scan_block(int bid, int nsh, int ntile, int& sh, int& tile) {
  if (nsh % 8 == 0) {
    const int xcd = bid & 7, local = bid >> 3;
    sh = (local / ntile) * 8 + xcd;
    tile = local % ntile;
  } else {
    sh = bid / ntile;
    tile = bid % ntile;
  }
}

// ---------------------------------------------------------------------------
// X = (I + A)^{-1} for a strictly lower triangular 64x64 fp32 A (LDS, pitch kPitchF).
// Blocked forward substitution over 16x16 blocks:
//   diagonal blocks X_ii = (I + A_ii)^{-1} by column substitution, all four in wave 3 (lane
//   16 i + c solves column c of block i; each solved row at once updates every later row, so
//   the FMAs form short independent chains; the other waves leave their issue slots to the
//   other workgroups on the compute unit, and wave 3 has no block column below),
//   then wave j fills block column j downwards, X_ij = -X_ii sum_{k=j}^{i-1} A_ik X_kj,
//   with fp32 MFMA: an accumulator tile has exactly the layout of a B operand, so the
//   X_kj already computed stay in registers and feed the next products.
// All 256 threads must call it. On return the diagonal and lower 16x16 blocks of X are in
// LDS; the blocks above the diagonal are NOT written (they are zero by definition and the
// caller masks them when it reads whole rows).
// ---------------------------------------------------------------------------
EFLA_DEV void invert_unit_lower64(const float* sA, float* sX, int tid) {
  constexpr int ld = kPitchF;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (wv == 3) {
    const int o = 16 * (lane >> 4), c = lane & 15;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = (r == c) ? 1.f : 0.f;
#pragma unroll
    for (int m = 0; m < 15; ++m)
#pragma unroll
      for (int r = m + 1; r < 16; ++r) x[r] = fmaf(-sA[(o + r) * ld + o + m], x[m], x[r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) sX[(o + r) * ld + o + c] = x[r];
  }
  __syncthreads();
  const int j = wv;
  if (j < 3) {
    f32x4 xc[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
    for (int kb = 0; kb < 3; ++kb)
      if (kb == j) xc[kb] = frag_km<float>(sX + 16 * j * ld + 16 * j, ld, lane);
#pragma unroll
    for (int i = 1; i < 4; ++i) {
      if (i <= j) continue;
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < 3; ++kb)
        if (kb >= j && kb < i)
          acc = Mma<float>::step(frag_rm<float>(sA + 16 * i * ld + 16 * kb, ld, lane), xc[kb], acc);
      xc[i] = -Mma<float>::step(frag_rm<float>(sX + 16 * i * ld + 16 * i, ld, lane), acc, zero4());
      st_frag_lds<float>(sX + 16 * i * ld + 16 * j, ld, xc[i], lane);
    }
  }
  __syncthreads();
}

}  // namespace efla

// KDA backward in chunk form (training).
//
// The pages give the chunkwise algorithm as the training form of the
// recurrence ("Kimi Linear、独自の土俵でFull Attentionを上回る" (remio.ai),
// section "Kimi Linearがより賢いRecurrent Memoryを使う方法") but print neither
// it nor its gradient.  This is the reverse mode of the chunk form the prefill
// uses, taken through its matrices.  Per chunk of 64 tokens, per key channel,
// with gamma_r the product of alpha over rows 0..r and rho_r = gamma_r /
// gamma_mR the decay of row r relative to the reference row m_R = 16R + 7 of
// its 16-row block R (products of alpha, no logarithms):
//   Kr = k rho,  Kh = k / rho,  Qr = q rho                 (per row and channel)
//   X = strict_lower(G_K),  P = lower(G_Q)     G[r,s] = Kr_r . Kh_s D_rs
//   M = (I + Diag(beta) X)^-1,  T = M Diag(beta)
//   Kg = k gamma,  Qg = q gamma,  Ke = k gamma_C / gamma   (Kr, Qr, Kh rescaled)
//   W = T Kg,  U = T V,  Vn = U - W S
//   O = Qg S + P Vn,   S' = Diag(gamma_C) S + Ke^T Vn
// D_rs = gamma_mR / gamma_mI for rows r of block R and s of block I < R,
// applied to the column operand in two steps (S1_I, then E_RI) and to the row
// operand of the transposed sums in two steps (P1_R, then F_RI), so that no
// intermediate leaves the range of the entries it builds (the forward's
// factoring; see kda_prefill.hip).  S is the state entering the chunk (the
// forward's snapshot).  The adjoint of the state entering a chunk is affine in
// the adjoint of the state leaving it, dS = b_c + A_c dS' with
// A_c = Diag(gamma_C) - W^T Ke and b_c = (Qg - P W)^T dO, so the reverse pass
// is three launches per window of chunks:
//   prep   one workgroup per chunk-head: A_c, b_c, M, Vn, P and X, the decays;
//   chain  one workgroup per (sequence, head, 16 value columns): the adjoints
//          dS' at every chunk end, sequentially from the last chunk;
//   post   one workgroup per chunk-head: dq, dk, dv, dalpha, dbeta from S, dS',
//          M, Vn, P and X (the solve's adjoint dA = -M^T dM M^T, the decays'
//          gradient as a reverse cumulative sum within the chunk).
// The gradient of the log-decays per row is
//   dg = AQ Qr + AR Kr - AH Kh   (+ the chunk-end decay's terms on the last row)
// with AQ, AR, AH the row and column sums of the factored products.  The
// diagonal of P carries no decay (gamma_r / gamma_r): its contributions to dq
// and dk are added apart, so that dg holds no pair of equal and opposite terms
// that would cancel in fp32 (dalpha = d log(alpha) / alpha would magnify the
// rounding of such a pair by 1 / alpha).
// All products are fp32 MFMA (16x16x4) on LDS operands.
#include <hip/hip_runtime.h>

#include "kda_internal.h"

namespace kda {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kC = 64;      // chunk
// Decay buffer of a chunk-head ([kDecayRows][DK] floats): rho (rows 0..63),
// then per-channel vectors (row indices):
constexpr int kGM = 64;     // gamma_mR, R = 0..3           (rows 0 .. 16R + 7)
constexpr int kGNM = 68;    // gamma_C / gamma_mI, I = 0..3 (rows 16I + 8 .. 63)
constexpr int kS1 = 72;     // S1_I, I = 0..3               (rows 16I + 8 .. 16I + 15)
constexpr int kE = 76;      // E_RI, 6 pairs I < R          (rows 16I + 16 .. 16R + 7)
constexpr int kP1 = 82;     // P1_R, R = 0..3               (rows 16R .. 16R + 7)
constexpr int kF = 86;      // F_RI, 6 pairs I < R          (rows 16I + 8 .. 16R - 1)
constexpr int kGC = 92;     // gamma_C                      (rows 0 .. 63)
constexpr int kDecayRows = 93;
constexpr int kVecRows = kDecayRows - 64;
// index of the block pair (R, I), I < R, among the six
__host__ __device__ constexpr int pidx(int R, int I) { return R * (R - 1) / 2 + I; }
constexpr int kNW = 8;      // waves per workgroup (prep, post)
constexpr int kNT = 64 * kNW;
constexpr int kLS = 20;     // pitch (floats) of a 16-column slab
constexpr int kL64 = 68;    // pitch of a 64-column array

// Workgroup barrier that orders LDS only: global loads (prefetches) and stores
// stay in flight across it.  No kernel here reads global memory that another
// thread of the same launch writes.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <bool BF16>
__device__ __forceinline__ float ld_in(const void* p, int64_t i) {
  if constexpr (BF16) {
    const uint16_t b = static_cast<const uint16_t*>(p)[i];
    return __uint_as_float(uint32_t(b) << 16);
  } else {
    return static_cast<const float*>(p)[i];
  }
}

// Row r of a chunk with nv >= 1 rows, clamped into the chunk.  Loads of rows
// past the end read the last row and their values are discarded where they
// are used: a load under a per-lane branch makes the compiler wait for it
// before the branches join, which turns a loop of such loads into one memory
// round trip per iteration.
__device__ __forceinline__ int in_rows(int r, int nv) { return r < nv ? r : nv - 1; }

// acc[s] += A(tile rows, 0:K) B(0:K, tile cols) for the tiles t = wv + 8 s of
// the (M/16) x (N/16) tile grid (row-major), wv being the caller's wave slot
// (wave-uniform; a slot past the grid does nothing).  All tiles of a wave
// share one column block, so each B fragment is loaded once for them.
//   A(m, k) = AK ? a[m * lda + k] : a[k * lda + m]
//   B(k, n) = BK ? b[n * ldb + k] : b[k * ldb + n]
// Within each 16-wide block of K, lane group g takes k = 4g .. 4g + 3 over the
// four products (lane i = row of A / column of B); the result lane holds rows
// 4g + q of column i of its tile.  The fragments of KG blocks of K are loaded
// before their products.  Triangular operands are stored with their zeros, so
// the products may run over the whole of K (exact zeros do not change a sum).
// TRI (used where the tiles' rows are known at compile time, N == 16 * kNW:
// tile s starts at row 16 s) skips the blocks of K where a triangular A is
// zero: 2 = A lower triangular (k <= m), 3 = A upper triangular (k >= m).
template <int M, int N, int K, bool AK, bool BK, int NT, int TRI = 0>
__device__ __forceinline__ void mm(f4 (&acc)[NT], const float* a, int lda, const float* b, int ldb,
                                   int wv) {
  constexpr int TN = N / 16, NTILE = (M / 16) * TN, KB = K / 16;
  static_assert(kNW % TN == 0, "a wave's tiles share one column block");
  static_assert(NTILE % kNW == 0 ? NT == NTILE / kNW : (NT == 1 && NTILE < kNW), "tiles per wave");
  constexpr int KG0 = NT >= 8 ? 1 : (NT >= 4 ? 2 : 4);
  constexpr int KG = KB < KG0 ? KB : KG0;
  static_assert(KB % KG == 0, "K blocks in whole groups");
  static_assert(TRI == 0 || N / 16 == kNW, "triangular skips need compile-time tile rows");
  if (NTILE < kNW && wv >= NTILE) return;
  // block k0 of tile s contributes (compile-time after unrolling)
  auto need = [](int s, int k0) {
    return TRI == 0 || (TRI == 2 && k0 <= 16 * s) || (TRI == 3 && k0 >= 16 * s);
  };
  const int l = threadIdx.x & 63, i = l & 15, g = l >> 4;
  const int n0 = (wv % TN) * 16;
#pragma unroll
  for (int kg = 0; kg < KB; kg += KG) {
    f4 bv[KG], av[KG][NT];
#pragma unroll
    for (int u = 0; u < KG; ++u) {
      const int k0 = 16 * (kg + u);
      bool any = false;
#pragma unroll
      for (int s = 0; s < NT; ++s) any = any || need(s, k0);
      if (!any) continue;
      if constexpr (BK) {
        bv[u] = *reinterpret_cast<const f4*>(b + (n0 + i) * ldb + k0 + 4 * g);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) bv[u][j] = b[(k0 + 4 * g + j) * ldb + n0 + i];
      }
#pragma unroll
      for (int s = 0; s < NT; ++s) {
        if (!need(s, k0)) continue;
        const int m0 = ((wv + kNW * s) / TN) * 16;
        if constexpr (AK) {
          av[u][s] = *reinterpret_cast<const f4*>(a + (m0 + i) * lda + k0 + 4 * g);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) av[u][s][j] = a[(k0 + 4 * g + j) * lda + m0 + i];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < KG; ++u)
#pragma unroll
      for (int s = 0; s < NT; ++s) {
        if (!need(s, 16 * (kg + u))) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[s] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[u][s][j], bv[u][j], acc[s], 0, 0, 0);
      }
  }
}

// A triangular skip for products with DK output columns: only where a wave's
// tiles have compile-time rows (DK == 16 * kNW).
template <int DK>
constexpr int tri_dk(int t) {
  return DK == 16 * kNW ? t : 0;
}

template <int NT>
__device__ __forceinline__ void zero(f4 (&acc)[NT]) {
#pragma unroll
  for (int s = 0; s < NT; ++s) acc[s] = f4{0.f, 0.f, 0.f, 0.f};
}

// Tile s of a wave: first row m0, first column n0 (N columns in the grid).
template <int N>
__device__ __forceinline__ void tile_origin(int wv, int s, int& m0, int& n0) {
  const int t = wv + kNW * s;
  m0 = (t / (N / 16)) * 16;
  n0 = (t % (N / 16)) * 16;
}
template <int M, int N>
__device__ __forceinline__ bool tile_live(int wv, int s) {
  return wv + kNW * s < (M / 16) * (N / 16);
}

// Layouts of the chain's operands, in its fragment order so that each wave
// instruction moves one contiguous block.  A_c: wave w (rows 16w..16w+15)
// takes DK/16 float4 per lane, lane (i, g) holding A_c[16w + i][4j + g] for
// j = 0 .. DK/4 - 1.  b_c and dS': per 16-column slab and wave, one float4
// per lane holding rows 16w + 4g .. 16w + 4g + 3 of column i.
template <int DK>
__device__ __forceinline__ int frag_a(int r, int c) {
  const int j = c >> 2;
  return (((r >> 4) * (DK / 16) + (j >> 2)) * 64 + (r & 15) + 16 * (c & 3)) * 4 + (j & 3);
}
template <int DK>
__device__ __forceinline__ int64_t frag_s(int js, int w, int l) {
  return ((int64_t(js) * (DK / 16) + w) * 64 + l) * 4;
}

// The chunk a workgroup works on: sequence n, chunk c counted from the start
// (the window holds reverse indices win_lo .. win_lo + win_k - 1).
struct Chunk {
  int64_t n, c, s0, tok0, wi;
  int nv, h;
};

__device__ __forceinline__ bool locate(const BwdChunkArgs& p, int64_t n, int64_t jw, int h,
                                       Chunk& ck) {
  int64_t s0, len;
  if (p.cu_seqlens) {
    s0 = p.cu_seqlens[n];
    len = p.cu_seqlens[n + 1] - s0;
  } else {
    s0 = n * p.T;
    len = p.T;
  }
  const int64_t nch = (len + kC - 1) / kC;
  ck.n = n;
  ck.h = h;
  ck.s0 = s0;
  ck.c = nch - 1 - (p.win_lo + jw);
  if (ck.c < 0) return false;
  ck.tok0 = s0 + ck.c * kC;
  const int64_t rem = len - ck.c * kC;
  ck.nv = int(rem < kC ? rem : kC);
  ck.wi = (n * p.H + h) * p.win_k + jw;
  return true;
}

// The state entering chunk c: state_in for the first chunk (nullptr = zero),
// else the forward's snapshot after chunk c - 1.
template <int DK>
__device__ __forceinline__ const float* chunk_state(const BwdChunkArgs& p, const Chunk& ck) {
  const int64_t hs = int64_t(DK) * p.DV;
  if (ck.c == 0) return p.state_in ? p.state_in + (ck.n * p.H + ck.h) * hs : nullptr;
  const int64_t base = p.cu_seqlens ? ck.s0 / kC : ck.n * (p.T / kC);
  return p.snapshots + ((base + ck.c - 1) * p.H + ck.h) * hs;
}

// The chunk's decays: rho into rho[64][ld] (LDS), the vectors into
// vec[kVecRows][DK] (LDS, rows counted from kGM), all of it into the global
// buffer dg ([kDecayRows][DK]).  Threads 0..DK-1, one channel each; rows past
// the chunk's end take alpha = 1.  Every value is a product of alpha over
// consecutive rows (or its reciprocal for rho above the reference row).
template <int DK, bool SG>
__device__ __forceinline__ void decays(const BwdChunkArgs& p, const Chunk& ck, float* rho, int ld,
                                       float* vec, float* dg) {
  const int c = threadIdx.x;
  if (c >= DK) return;
  float a[kC];
#pragma unroll
  for (int r = 0; r < kC; ++r) {
    const int64_t row = (ck.tok0 + in_rows(r, ck.nv)) * p.H + ck.h;
    a[r] = SG ? p.alpha[row] : p.alpha[row * DK + c];
  }
#pragma unroll
  for (int r = 0; r < kC; ++r)
    if (r >= ck.nv) a[r] = 1.f;
  auto put = [&](int row, float v) {
    dg[row * DK + c] = v;
    if (row < kC) rho[row * ld + c] = v;
    else vec[(row - kGM) * DK + c] = v;
  };
  // product of alpha over rows r0 .. r1 (inclusive)
  auto prod = [&](int r0, int r1) {
    float x = 1.f;
#pragma unroll
    for (int r = 0; r < kC; ++r)
      if (r >= r0 && r <= r1) x *= a[r];
    return x;
  };
#pragma unroll
  for (int R = 0; R < 4; ++R) {
    const int m = 16 * R + 7;
    float x = 1.f;
    put(m, 1.f);
#pragma unroll
    for (int r = m - 1; r >= 16 * R; --r) {   // 1 / prod_{r < s <= m} alpha_s
      x *= a[r + 1];
      put(r, 1.f / x);
    }
    x = 1.f;
#pragma unroll
    for (int r = m + 1; r < 16 * R + 16; ++r) {   // prod_{m < s <= r} alpha_s
      x *= a[r];
      put(r, x);
    }
  }
#pragma unroll
  for (int R = 0; R < 4; ++R) {
    put(kGM + R, prod(0, 16 * R + 7));
    put(kGNM + R, prod(16 * R + 8, kC - 1));
    put(kS1 + R, prod(16 * R + 8, 16 * R + 15));
    put(kP1 + R, prod(16 * R, 16 * R + 7));
#pragma unroll
    for (int I = 0; I < R; ++I) {
      put(kE + pidx(R, I), prod(16 * I + 16, 16 * R + 7));
      put(kF + pidx(R, I), prod(16 * I + 8, 16 * R - 1));
    }
  }
  put(kGC, prod(0, kC - 1));
}

// The two 64 x 64 Gram tiles of wave wv, G = lower(Ar Kh^T) with the decay
// factors of the off-diagonal blocks (row block R = wv / 4 + 2 s, column
// block I = wv % 4): for I < R the column operand is scaled by S1_I and then
// E_RI per channel (vec rows from kGM, LDS); blocks above the diagonal are
// left zero.  On diagonal blocks the entries above the diagonal may be
// infinite: the caller selects them away.
template <int DK>
__device__ __forceinline__ void gram_bw(f4 (&acc)[2], const float* ar, const float* kh, int ld,
                                        const float* vec, int wv) {
  const int l = threadIdx.x & 63, i = l & 15, g = l >> 4;
  const int I = wv & 3;
#pragma unroll
  for (int kb = 0; kb < DK / 16; ++kb) {
    const int k0 = 16 * kb + 4 * g;
    const f4 bv = *reinterpret_cast<const f4*>(kh + (16 * I + i) * ld + k0);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int R = (wv >> 2) + 2 * s;
      if (I > R) continue;
      f4 b = bv;
      if (I < R) {
        const f4 s1 = *reinterpret_cast<const f4*>(vec + (kS1 - kGM + I) * DK + k0);
        const f4 e = *reinterpret_cast<const f4*>(vec + (kE - kGM + pidx(R, I)) * DK + k0);
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = (b[j] * s1[j]) * e[j];
      }
      const f4 av = *reinterpret_cast<const f4*>(ar + (16 * R + i) * ld + k0);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[s] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[j], b[j], acc[s], 0, 0, 0);
    }
  }
}

// acc[s] += A B for the wave's tiles of a 64 x DK output, K = the 64 tokens,
// where the product of output row (token) r and K token u carries the decay
// between them in factored form:
//   ROWS (AK: A(m,k) = a[m * lda + k], lower triangular):  row block R, K
//        block I < R: B rows scaled by S1_I, then E_RI (per output column);
//   COLS (A(m,k) = a[k * lda + m], i.e. A^T of a lower-triangular array):
//        row block I, K block R > I: B rows scaled by P1_R, then F_RI.
// Diagonal K blocks are unscaled, K blocks on the zero side are skipped.
// B(k, n) = b[k * ldb + n].  Tile s: rows 16 (wv / TN + (8 / TN) s)..,
// columns 16 (wv % TN).., TN = DK / 16; the scales of the lane's column are
// read from the chunk's global decay buffer dg.
template <int DK, bool COLS>
__device__ __forceinline__ void gsum(f4 (&acc)[(4 * (DK / 16) + kNW - 1) / kNW], const float* a, int lda,
                                     const float* b, int ldb, int wv, const float* dg) {
  constexpr int TN = DK / 16, NT = (4 * TN + kNW - 1) / kNW;
  const int l = threadIdx.x & 63, i = l & 15, g = l >> 4;
  const int n0 = (wv % TN) * 16;
  // COLS: P1_R (R = 1..3) and F_RI;  rows: S1_I (I = 0..2) and E_RI
  float s1v[4], s2v[6];
#pragma unroll
  for (int x = 0; x < 3; ++x) s1v[x + (COLS ? 1 : 0)] = dg[((COLS ? kP1 + 1 : kS1) + x) * DK + n0 + i];
#pragma unroll
  for (int x = 0; x < 6; ++x) s2v[x] = dg[((COLS ? kF : kE) + x) * DK + n0 + i];
#pragma unroll
  for (int u = 0; u < 4; ++u) {   // K block (16 tokens)
    f4 bv;
#pragma unroll
    for (int j = 0; j < 4; ++j) bv[j] = b[(16 * u + 4 * g + j) * ldb + n0 + i];
#pragma unroll
    for (int s = 0; s < NT; ++s) {
      const int ro = (wv + kNW * s) / TN;   // output row block
      if (COLS ? (u < ro) : (u > ro)) continue;
      f4 bs = bv;
      if (u != ro) {
        const float s1 = s1v[u];
        const float s2 = s2v[COLS ? pidx(u, ro) : pidx(ro, u)];
#pragma unroll
        for (int j = 0; j < 4; ++j) bs[j] = (bs[j] * s1) * s2;
      }
      f4 av;
      if constexpr (COLS) {
#pragma unroll
        for (int j = 0; j < 4; ++j) av[j] = a[(16 * u + 4 * g + j) * lda + 16 * ro + i];
      } else {
        // one 16-byte read: four scalar reads of this pattern conflict 4 ways
        av = *reinterpret_cast<const f4*>(a + (16 * ro + i) * lda + 16 * u + 4 * g);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[s] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[j], bs[j], acc[s], 0, 0, 0);
    }
  }
}

// ---------------------------------------------------------------- prep ------
template <int DK, bool BF16, bool SG>
__global__ __launch_bounds__(kNT, 1) void kda_bwdc_prep_kernel(BwdChunkArgs p) {
  constexpr int LD = DK + 4;
  constexpr int NTW = (4 * (DK / 16) + kNW - 1) / kNW;          // 64 x DK tiles per wave
  constexpr int NTA = ((DK / 16) * (DK / 16) + kNW - 1) / kNW;  // DK x DK
  __shared__ __attribute__((aligned(16))) float sm[3 * 64 * LD + 2 * 64 * kL64 + 2 * DK + 64 +
                                                   (128 + DK) * kLS];
  float* const sKr = sm;             // Kr, then W
  float* const sKh = sKr + 64 * LD;
  float* const sQr = sKh + 64 * LD;
  float* const sM = sQr + 64 * LD;   // Diag(beta) X, then M, then T
  float* const sP = sM + 64 * kL64;
  float* const sgc = sP + 64 * kL64;   // gamma_C
  float* const sb = sgc + 2 * DK;
  float* const sV = sb + 64;         // decay vectors, V slab, then Z slab (also the solve's scratch)
  float* const sO = sV + 64 * kLS;   // dO slab
  float* const sS = sO + 64 * kLS;   // S slab [DK][16]
  float* const sVec = sV;            // steps 1-2: [kVecRows][DK] from kGM
  static_assert(kVecRows * DK <= (128 + DK) * kLS, "decay vectors fit the slab space");

  const int t = threadIdx.x, w = __builtin_amdgcn_readfirstlane(t >> 6), l = t & 63, li = l & 15,
            g = l >> 4;
  const int H = p.H, DV = p.DV;
  const int64_t bid = blockIdx.x;
  const int h = int(bid % H);
  const int64_t jw = (bid / H) % p.win_k, n = bid / H / p.win_k;
  Chunk ck;
  if (!locate(p, n, jw, h, ck)) return;
  const int nv = ck.nv;

  // 1. decays, scaled keys and queries, beta (the keys and queries are loaded
  // before the decays' products, so that both latencies overlap)
  constexpr int NE = 64 * DK / kNT;
  float pk[NE], pq[NE];
#pragma unroll
  for (int u = 0; u < NE; ++u) {
    const int e = t + u * kNT;
    const int r = e / DK, c = e % DK;
    const int64_t x = ((ck.tok0 + in_rows(r, nv)) * H + h) * int64_t(DK) + c;
    pk[u] = ld_in<BF16>(p.k, x);
    pq[u] = ld_in<BF16>(p.q, x);
  }
  float* const rho_g = p.rho + ck.wi * (kDecayRows * DK);
  decays<DK, SG>(p, ck, sQr, LD, sVec, rho_g);   // rho parked in sQr
  {
    const float bv = p.beta[(ck.tok0 + in_rows(t & 63, nv)) * H + h];
    if (t < 64) sb[t] = t < nv ? bv : 0.f;
  }
  lds_barrier();
#pragma unroll
  for (int u = 0; u < NE; ++u) {
    const int e = t + u * kNT;
    const int r = e / DK, c = e % DK;
    const float rh = sQr[r * LD + c];
    const float kv = r < nv ? pk[u] : 0.f, qv = r < nv ? pq[u] : 0.f;
    sKr[r * LD + c] = kv * rh;
    sKh[r * LD + c] = kv / rh;
    sQr[r * LD + c] = qv * rh;
  }
  lds_barrier();

  // 2. Diag(beta) X and P; both also to the global P/X array (P on and below
  // the diagonal, X transposed above it) for the post kernel.
  {
    f4 ax[2], ap[2];
    zero(ax);
    zero(ap);
    gram_bw<DK>(ax, sKr, sKh, LD, sVec, w);
    gram_bw<DK>(ap, sQr, sKh, LD, sVec, w);
    float* const PXg = p.PX + ck.wi * (64 * 64);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      int m0, n0;
      tile_origin<64>(w, s, m0, n0);
      f4 xt;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = m0 + 4 * g + q, c = n0 + li;
        // (selected, not multiplied by a zero: above the diagonal the factored
        // products may be infinite)
        const float x = c < r ? ax[s][q] : 0.f;
        const float pv = c <= r ? ap[s][q] : 0.f;
        sM[r * kL64 + c] = sb[r] * x;
        sP[r * kL64 + c] = pv;
        if (c <= r) PXg[r * 64 + c] = pv;
        xt[q] = x;
      }
      // X^T above the diagonal: row c, columns r = m0 + 4g .. +3 (> c)
      if (n0 < m0 || (n0 == m0 && 4 * g > li)) {
        *reinterpret_cast<f4*>(PXg + (n0 + li) * 64 + m0 + 4 * g) = xt;
      } else if (n0 == m0) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (4 * g + q > li) PXg[(n0 + li) * 64 + m0 + 4 * g + q] = xt[q];
      }
    }
    if (t < DK) sgc[t] = sVec[(kGC - kGM) * DK + t];
  }
  lds_barrier();
  // Kr -> Kg = Kr Diag(gamma_mR), Qr -> Qg, Kh -> Ke = Kh Diag(gamma_C / gamma_mR)
  // (rows of block R): the operands of W, b_c and A_c.
#pragma unroll
  for (int u = 0; u < NE; ++u) {
    const int e = t + u * kNT;
    const int r = e / DK, c = e % DK;
    const float gm = sVec[(kGM - kGM + (r >> 4)) * DK + c];
    const float gq = sVec[(kGNM - kGM + (r >> 4)) * DK + c];
    sKr[r * LD + c] *= gm;
    sQr[r * LD + c] *= gm;
    sKh[r * LD + c] *= gq;
  }
  lds_barrier();

  // 3. M = (I + Diag(beta) X)^-1 in place: the four diagonal 16x16 blocks by
  // forward substitution (wave 0, lane = column of a block), then block rows
  // 1..3: M_ij = -M_ii sum_{j <= k < i} A_ik M_kj.
  if (w == 0) {
    const int o = 16 * g;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float s = r == li ? 1.f : 0.f;
#pragma unroll
      for (int u = 0; u < r; ++u) s -= sM[(o + r) * kL64 + o + u] * x[u];
      x[r] = s;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) sM[(o + r) * kL64 + o + li] = x[r];
  }
  lds_barrier();
  for (int bi = 1; bi < 4; ++bi) {
    f4 acc = f4{0.f, 0.f, 0.f, 0.f};
    const int bj = w;
    if (bj < bi) {
      for (int bk = bj; bk < bi; ++bk) {
        const f4 av = *reinterpret_cast<const f4*>(sM + (16 * bi + li) * kL64 + 16 * bk + 4 * g);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[j], sM[(16 * bk + 4 * g + j) * kL64 + 16 * bj + li],
                                                     acc, 0, 0, 0);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) sV[(16 * bj + 4 * g + q) * kLS + li] = acc[q];
    }
    lds_barrier();
    f4 acc2 = f4{0.f, 0.f, 0.f, 0.f};
    if (bj < bi) {
      const f4 av = *reinterpret_cast<const f4*>(sM + (16 * bi + li) * kL64 + 16 * bi + 4 * g);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc2 = __builtin_amdgcn_mfma_f32_16x16x4f32(av[j], sV[(16 * bj + 4 * g + j) * kLS + li], acc2, 0, 0,
                                                    0);
    }
    lds_barrier();
    if (bj < bi) {
#pragma unroll
      for (int q = 0; q < 4; ++q) sM[(16 * bi + 4 * g + q) * kL64 + 16 * bj + li] = -acc2[q];
    }
    lds_barrier();
  }

  // 4. M out; T = M Diag(beta) in place
  float* const Mg = p.Mb + ck.wi * (64 * 64);
#pragma unroll
  for (int u = 0; u < 64 * 64 / kNT; ++u) {
    const int e = t + u * kNT;
    const int r = e >> 6, c = e & 63;
    const float m = sM[r * kL64 + c];
    Mg[e] = m;
    sM[r * kL64 + c] = m * sb[c];
  }
  lds_barrier();

  // Inputs of the value-column loop (step 7); the first slab is fetched here,
  // ahead of steps 5 and 6.
  const float* const S = chunk_state<DK>(p, ck);
  float* const Vng = p.Vnb + ck.wi * (64 * int64_t(DV));
  float* const bg = p.bc + ck.wi * (int64_t(DK) * DV);
  // (the next slab's inputs are fetched into registers during this slab's
  // products; past the last slab the last one is fetched again)
  constexpr int NR = 64 * 16 / kNT, NS = DK * 16 / kNT;
  struct Slab {
    float v[NR], o[NR], s[NS];
  };
  auto fetch = [&](Slab& R, int js) {
    if (js >= DV / 16) js = DV / 16 - 1;
#pragma unroll
    for (int u = 0; u < NR; ++u) {
      const int e = t + u * kNT;
      const int r = e >> 4, j = e & 15;
      const int64_t x = ((ck.tok0 + in_rows(r, nv)) * H + h) * int64_t(DV) + 16 * js + j;
      R.v[u] = ld_in<BF16>(p.v, x);   // rows past the end: zeroed where stored
      R.o[u] = p.d_o[x];
    }
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int e = t + u * kNT;
      R.s[u] = S ? S[int64_t(e >> 4) * DV + 16 * js + (e & 15)] : 0.f;
    }
  };
  Slab R;
  fetch(R, 0);

  // 5. W = T Kg, over Kg
  {
    f4 aw[NTW];
    zero(aw);
    mm<64, DK, 64, true, false, NTW, tri_dk<DK>(2)>(aw, sM, kL64, sKr, LD, w);
    lds_barrier();
#pragma unroll
    for (int s = 0; s < NTW; ++s) {
      if (!tile_live<64, DK>(w, s)) break;
      int m0, n0;
      tile_origin<DK>(w, s, m0, n0);
#pragma unroll
      for (int q = 0; q < 4; ++q) sKr[(m0 + 4 * g + q) * LD + n0 + li] = aw[s][q];
    }
  }
  lds_barrier();
  float* const sW = sKr;

  // 6. A_c = Diag(gamma_C) - W^T Ke, stored in the chain's fragment order.
  {
    f4 aa[NTA];
    zero(aa);
    mm<DK, DK, 64, false, false>(aa, sW, LD, sKh, LD, w);
    float* const Ag = p.Ac + ck.wi * (int64_t(DK) * DK);
#pragma unroll
    for (int s = 0; s < NTA; ++s) {
      if (!tile_live<DK, DK>(w, s)) break;
      int m0, n0;
      tile_origin<DK>(w, s, m0, n0);
      const int c = n0 + li;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = m0 + 4 * g + q;
        float v = -aa[s][q];
        if (r == c) v += sgc[r];
        Ag[frag_a<DK>(r, c)] = v;
      }
    }
  }

  // 7. per 16 value columns: Vn = T V - W S;  b_c = Qg^T dO - W^T (P^T dO)
  for (int js = 0; js < DV / 16; ++js) {
#pragma unroll
    for (int u = 0; u < NR; ++u) {
      const int e = t + u * kNT;
      sV[(e >> 4) * kLS + (e & 15)] = (e >> 4) < nv ? R.v[u] : 0.f;
      sO[(e >> 4) * kLS + (e & 15)] = (e >> 4) < nv ? R.o[u] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int e = t + u * kNT;
      sS[(e >> 4) * kLS + (e & 15)] = R.s[u];
    }
    fetch(R, js + 1);
    lds_barrier();
    f4 au[1], an[1], az[1];
    zero(au);
    zero(an);
    zero(az);
    mm<64, 16, 64, true, false>(au, sM, kL64, sV, kLS, w);
    mm<64, 16, DK, true, false>(an, sW, LD, sS, kLS, w);
    mm<64, 16, 64, false, false>(az, sP, kL64, sO, kLS, (w + 4) & 7);
    if (w < 4) {
#pragma unroll
      for (int q = 0; q < 4; ++q) Vng[(16 * w + 4 * g + q) * DV + 16 * js + li] = au[0][q] - an[0][q];
    }
    lds_barrier();
    if (w >= 4) {
#pragma unroll
      for (int q = 0; q < 4; ++q) sV[(16 * (w - 4) + 4 * g + q) * kLS + li] = az[0][q];
    }
    lds_barrier();
    f4 b1[1], b2[1];
    zero(b1);
    zero(b2);
    mm<DK, 16, 64, false, false>(b1, sQr, LD, sO, kLS, w);
    mm<DK, 16, 64, false, false>(b2, sW, LD, sV, kLS, w);
    if (tile_live<DK, 16>(w, 0)) {
      f4 v;
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = b1[0][q] - b2[0][q];
      *reinterpret_cast<f4*>(bg + frag_s<DK>(js, w, l)) = v;
    }
    lds_barrier();
  }
}

// ---------------------------------------------------------------- chain -----
// dS (adjoint of the state entering a chunk) = b_c + A_c dS'.  One workgroup
// per (sequence, head, 16 value columns); wave w holds rows 16w .. 16w + 15 of
// the slab in the MFMA result layout.  dS' of every chunk goes to dSend.
template <int DK>
__global__ __launch_bounds__(64 * (DK / 16), 1) void kda_bwdc_chain_kernel(BwdChunkArgs p) {
  constexpr int KQ = DK / 4;
  __shared__ __attribute__((aligned(16))) float sD[2][DK * 16];
  const int t = threadIdx.x, w = __builtin_amdgcn_readfirstlane(t >> 6), l = t & 63, li = l & 15,
            g = l >> 4;
  const int H = p.H, DV = p.DV, nsl = DV / 16;
  // Workgroups go to the 8 XCDs round-robin; remap so that the slabs of one
  // (sequence, head), which read the same A_c, run on one XCD and share its L2.
  int64_t bid = blockIdx.x;
  const int64_t G = gridDim.x;
  if ((G & 7) == 0) bid = (bid & 7) * (G >> 3) + (bid >> 3);
  const int slab = int(bid % nsl);
  const int64_t pr = bid / nsl;
  const int h = int(pr % H);
  const int64_t n = pr / H;
  const int64_t len = p.cu_seqlens ? p.cu_seqlens[n + 1] - p.cu_seqlens[n] : p.T;
  const int64_t nch = (len + kC - 1) / kC;
  const int64_t c_hi = nch - 1 - p.win_lo;
  const int64_t hs = (n * H + h) * int64_t(DK) * DV;
  const int col = 16 * slab + li;
  f4 dS;
  if (p.win_lo == 0 || c_hi < 0) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      dS[q] = p.d_state_out ? p.d_state_out[hs + int64_t(16 * w + 4 * g + q) * DV + col] : 0.f;
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) dS[q] = p.carry[hs + int64_t(16 * w + 4 * g + q) * DV + col];
  }
  if (c_hi < 0) {   // no chunk in this window: only an empty sequence writes (window 0)
    if (p.win_lo == 0 && p.d_state_in) {
#pragma unroll
      for (int q = 0; q < 4; ++q) p.d_state_in[hs + int64_t(16 * w + 4 * g + q) * DV + col] = dS[q];
    }
    return;
  }
  const int64_t steps = c_hi + 1 < p.win_k ? c_hi + 1 : p.win_k;
  // Operands of a step: this lane's A_c fragments and b_c values.  Three sets
  // in rotation: the loads for the next two chunks are in flight during this
  // chunk's products (past the last step the last chunk is loaded again, so
  // the loads stay unconditional).
  struct Ops {
    f4 a[KQ / 4];
    f4 b;
  };
  auto load = [&](Ops& o, int64_t jw) {
    if (jw >= steps) jw = steps - 1;
    const int64_t wi = (n * H + h) * p.win_k + jw;
    const float* const ar = p.Ac + wi * (int64_t(DK) * DK) + (w * (KQ / 4) * 64 + l) * 4;
#pragma unroll
    for (int j = 0; j < KQ / 4; ++j) o.a[j] = *reinterpret_cast<const f4*>(ar + j * 256);
    o.b = *reinterpret_cast<const f4*>(p.bc + wi * (int64_t(DK) * DV) + frag_s<DK>(slab, w, l));
  };
  auto step = [&](const Ops& o, int64_t jw) {
    const int64_t wi = (n * H + h) * p.win_k + jw;
    float* const sd = sD[jw & 1];
#pragma unroll
    for (int q = 0; q < 4; ++q) sd[(16 * w + 4 * g + q) * 16 + li] = dS[q];
    *reinterpret_cast<f4*>(p.dSend + wi * (int64_t(DK) * DV) + frag_s<DK>(slab, w, l)) = dS;
    lds_barrier();
    f4 acc0 = o.b, acc1 = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KQ; j += 2) {
      acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(o.a[j >> 2][j & 3], sd[(4 * j + g) * 16 + li], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(o.a[(j + 1) >> 2][(j + 1) & 3],
                                                  sd[(4 * (j + 1) + g) * 16 + li], acc1, 0, 0, 0);
    }
    dS = acc0 + acc1;
  };
  Ops A, B, C;
  load(A, 0);
  load(B, 1);
  int64_t jw = 0;
  for (; jw + 2 < steps; jw += 3) {
    load(C, jw + 2);
    step(A, jw);
    load(A, jw + 3);
    step(B, jw + 1);
    load(B, jw + 4);
    step(C, jw + 2);
  }
  if (jw < steps) step(A, jw);
  if (jw + 1 < steps) step(B, jw + 1);
  const int64_t c = c_hi - steps;   // last chunk done: c + 1
  if (c < 0 && !p.d_state_in) return;
  // chunks remain but no later window will take them: the caller's max_seqlen
  // was below this sequence's length (nothing to carry to, nothing written)
  if (c >= 0 && !p.carry) return;
  float* const dst = c < 0 ? p.d_state_in + hs : p.carry + hs;
#pragma unroll
  for (int q = 0; q < 4; ++q) dst[int64_t(16 * w + 4 * g + q) * DV + col] = dS[q];
}

// ---------------------------------------------------------------- post ------
// Ke dS' for the wave's 16 rows (row block rb = wave): acc += (Kh_rb Diag(gq)) D,
// Kh [64][LD] (rows = tokens, K = channels), D [DK][kLS] (K = channels, 16
// columns), gq the block's gamma_C / gamma_mR per channel.
template <int DK, int LD>
__device__ __forceinline__ f4 ke_ds(f4 acc, const float* kh, const float* d, const float* gq, int rb) {
  const int l = threadIdx.x & 63, i = l & 15, g = l >> 4;
#pragma unroll
  for (int kb = 0; kb < DK / 16; ++kb) {
    const int k0 = 16 * kb + 4 * g;
    const f4 a = *reinterpret_cast<const f4*>(kh + (16 * rb + i) * LD + k0);
    const f4 sc = *reinterpret_cast<const f4*>(gq + k0);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j] * sc[j], d[(k0 + j) * kLS + i], acc, 0, 0, 0);
  }
  return acc;
}

template <int DK, bool BF16, bool SG>
__global__ __launch_bounds__(kNT, 1) void kda_bwdc_post_kernel(BwdChunkArgs p) {
  constexpr int LD = DK + 4;
  constexpr int NT4 = (4 * (DK / 16) + kNW - 1) / kNW;   // 64 x DK tiles per wave
  constexpr int RED = 4 * DK > kNT ? 4 * DK : kNT;
  __shared__ __attribute__((aligned(16))) float sm[3 * 64 * LD + 3 * 64 * kL64 + 9 * DK + 3 * 64 +
                                                   RED];
  float* const R1 = sm;               // Kh
  float* const R2 = R1 + 64 * LD;     // slabs (with R3), then dW, then Qr, then dg
  float* const R3 = R2 + 64 * LD;     // slabs, then Kr
  float* const sM = R3 + 64 * LD;     // M
  float* const sP = sM + 64 * kL64;   // P, then strict dP, then dM M^T
  float* const sX = sP + 64 * kL64;   // dT, then dM, then Diag(beta) dA
  float* const sGM = sX + 64 * kL64;  // gamma_mR [4][DK]
  float* const sGQ = sGM + 4 * DK;    // gamma_C / gamma_mR [4][DK]
  float* const sdgc = sGQ + 4 * DK;
  float* const sb = sdgc + DK;
  float* const sdb = sb + 64;
  float* const sdpd = sdb + 64;       // diagonal of dP
  float* const red = sdpd + 64;       // [4][DK] or [kNT] partial sums
  // slab buffers (inside R2 .. R3)
  float* const sO = R2;
  float* const sVn = sO + 64 * kLS;
  float* const sV = sVn + 64 * kLS;
  float* const sdVn = sV + 64 * kLS;
  float* const sD = sdVn + 64 * kLS;  // dS' rows, [DK][16]
  float* const sS = sD + DK * kLS;    // S rows

  const int t = threadIdx.x, w = __builtin_amdgcn_readfirstlane(t >> 6), l = t & 63, li = l & 15,
            g = l >> 4;
  const int H = p.H, DV = p.DV;
  const int64_t bid = blockIdx.x;
  const int h = int(bid % H);
  const int64_t jw = (bid / H) % p.win_k, n = bid / H / p.win_k;
  Chunk ck;
  if (!locate(p, n, jw, h, ck)) return;
  const int nv = ck.nv;
  const float* const rho = p.rho + ck.wi * (kDecayRows * DK);
  const float* const PXg = p.PX + ck.wi * (64 * 64);

  // Inputs of the value-column loop (step 2); the first slab is fetched here,
  // ahead of step 1.
  const float* const S = chunk_state<DK>(p, ck);
  const float* const dSe = p.dSend + ck.wi * (int64_t(DK) * DV);
  const float* const Vng = p.Vnb + ck.wi * (64 * int64_t(DV));
  // The next slab's operands are fetched into registers during this slab's
  // products (past the last slab the last one is fetched again).
  constexpr int NR = 64 * 16 / kNT, NS = DK * 16 / kNT;
  struct Slab {
    float o[NR], v[NR], vn[NR], s[NS];
    f4 d;   // dS' of rows 16 (t / 64) + 4 g .. + 3, column t % 16 (t < 4 DK)
  };
  auto fetch = [&](Slab& R, int js) {
    if (js >= DV / 16) js = DV / 16 - 1;
#pragma unroll
    for (int u = 0; u < NR; ++u) {
      const int e = t + u * kNT;
      const int r = e >> 4, j = e & 15;
      const int64_t x = ((ck.tok0 + in_rows(r, nv)) * H + h) * int64_t(DV) + 16 * js + j;
      R.o[u] = p.d_o[x];   // rows past the end: zeroed where stored
      R.v[u] = ld_in<BF16>(p.v, x);
      R.vn[u] = Vng[r * DV + 16 * js + j];
    }
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int e = t + u * kNT;
      R.s[u] = S ? S[int64_t(e >> 4) * DV + 16 * js + (e & 15)] : 0.f;
    }
    if (t < DK * 4) R.d = *reinterpret_cast<const f4*>(dSe + frag_s<DK>(js, t >> 6, t & 63));
  };
  Slab R;
  fetch(R, 0);

  // 1. decay vectors, beta, Kh, M, P
  for (int e = t; e < 8 * DK; e += kNT)
    sGM[e] = rho[(e < 4 * DK ? kGM * DK + e : kGNM * DK + e - 4 * DK)];
  {
    const float bv = p.beta[(ck.tok0 + in_rows(t & 63, nv)) * H + h];
    if (t < 64) sb[t] = t < nv ? bv : 0.f;
  }
#pragma unroll 8
  for (int u = 0; u < 64 * DK / kNT; ++u) {
    const int e = t + u * kNT;
    const int r = e / DK, c = e % DK;
    const float rh = rho[e];
    const float kv = ld_in<BF16>(p.k, ((ck.tok0 + in_rows(r, nv)) * H + h) * int64_t(DK) + c);
    R1[r * LD + c] = (r < nv ? kv : 0.f) / rh;
  }
  {
    const float* const Mg = p.Mb + ck.wi * (64 * 64);
    constexpr int NU = 64 * 64 / kNT;
    float mv[NU], pv[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {   // all loads first (P's upper part is read and dropped)
      mv[u] = Mg[t + u * kNT];
      pv[u] = PXg[t + u * kNT];
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int e = t + u * kNT;
      const int r = e >> 6, c = e & 63;
      sM[r * kL64 + c] = mv[u];
      sP[r * kL64 + c] = c <= r ? pv[u] : 0.f;
    }
  }
  lds_barrier();

  // 2. over the value columns, 16 at a time
  f4 aq[NT4], ah[NT4], awn[NT4], adp[2], adt[2];
  zero(aq);
  zero(ah);
  zero(awn);
  zero(adp);
  zero(adt);
  float dgcs = 0.f;
  for (int js = 0; js < DV / 16; ++js) {
#pragma unroll
    for (int u = 0; u < NR; ++u) {
      const int e = t + u * kNT;
      const int r = e >> 4, j = e & 15;
      sO[r * kLS + j] = r < nv ? R.o[u] : 0.f;
      sV[r * kLS + j] = r < nv ? R.v[u] : 0.f;
      sVn[r * kLS + j] = R.vn[u];
    }
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int e = t + u * kNT;
      const int r = e >> 4, j = e & 15;
      sS[r * kLS + j] = R.s[u];
    }
    if (t < DK * 4) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 16 * (t >> 6) + 4 * (g) + q;
        sD[r * kLS + li] = R.d[q];
      }
    }
    fetch(R, js + 1);
    lds_barrier();
    {
      // dVn = P^T dO + Ke dS'
      f4 adv[1];
      zero(adv);
      mm<64, 16, 64, false, false>(adv, sP, kL64, sO, kLS, w);
      if (w < 4) {
        adv[0] = ke_ds<DK, LD>(adv[0], R1, sD, sGQ + w * DK, w);
#pragma unroll
        for (int q = 0; q < 4; ++q) sdVn[(16 * w + 4 * g + q) * kLS + li] = adv[0][q];
      }
      if (t < DK) {
#pragma unroll
        for (int j = 0; j < 16; ++j) dgcs += sS[t * kLS + j] * sD[t * kLS + j];
      }
    }
    lds_barrier();
    mm<64, DK, 16, true, true>(aq, sO, kLS, sS, kLS, w);      // dO S^T
    mm<64, DK, 16, true, true>(awn, sdVn, kLS, sS, kLS, w);   // dVn S^T = -dW
    mm<64, DK, 16, true, true>(ah, sVn, kLS, sD, kLS, w);     // Vn dS'^T = dKe
    mm<64, 64, 16, true, true>(adp, sO, kLS, sVn, kLS, w);
    mm<64, 64, 16, true, true>(adt, sdVn, kLS, sV, kLS, w);
    {
      f4 adv2[1];
      zero(adv2);
      const int wv = (w + 4) & 7;
      mm<64, 16, 64, false, false>(adv2, sM, kL64, sdVn, kLS, wv);
      if (wv < 4) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = 16 * wv + 4 * g + q;
          if (r < nv) p.dv[((ck.tok0 + r) * H + h) * int64_t(DV) + 16 * js + li] = sb[r] * adv2[0][q];
        }
      }
    }
    lds_barrier();
  }

  // 3. Into the factored forms: AQ = (dO S^T) Diag(gamma_mR) and
  // AHe = dKe Diag(gamma_C / gamma_mR) per row block R (kept apart from the
  // other terms of AH: AHe * Kh = dKe * Ke is the gradient through the
  // chunk-end decays gamma_C / gamma_r, which enters d log(alpha)_t as the sum
  // over the rows before t; folding it into the per-row sums instead would
  // pair it with its own total on the last row, and the pair cancels).
  // gamma_C's other gradient: gamma_C sum_j S dS'.  dW, strict dP and its
  // diagonal, dT to LDS.  The inputs of Kr and Qr (rebuilt below) are loaded
  // first, so that their latency overlaps this work.
  constexpr int NE = 64 * DK / kNT;
  float pk[NE], pr[NE];
#pragma unroll
  for (int u = 0; u < NE; ++u) {
    const int e = t + u * kNT;
    const int r = e / DK, c = e % DK;
    pk[u] = ld_in<BF16>(p.k, ((ck.tok0 + in_rows(r, nv)) * H + h) * int64_t(DK) + c);
    pr[u] = rho[e];
  }
  f4 ahe[NT4];
#pragma unroll
  for (int s = 0; s < NT4; ++s) {
    if (!tile_live<64, DK>(w, s)) break;
    int m0, n0;
    tile_origin<DK>(w, s, m0, n0);
    const int c = n0 + li, rb = m0 >> 4;
    const float gm = sGM[rb * DK + c], gq = sGQ[rb * DK + c];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      aq[s][q] *= gm;
      ahe[s][q] = ah[s][q] * gq;
      ah[s][q] = 0.f;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) R2[(m0 + 4 * g + q) * LD + c] = -awn[s][q];
  }
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    int m0, n0;
    tile_origin<64>(w, s, m0, n0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = m0 + 4 * g + q, c = n0 + li;
      sP[r * kL64 + c] = c < r ? adp[s][q] : 0.f;
      if (c == r) sdpd[r] = adp[s][q];
      sX[r * kL64 + c] = adt[s][q];
    }
  }
  lds_barrier();
  if (t < DK) sdgc[t] = rho[kGC * DK + t] * dgcs;
#pragma unroll
  for (int u = 0; u < NE; ++u) {   // Kr
    const int e = t + u * kNT;
    R3[(e / DK) * LD + e % DK] = (e / DK < nv ? pk[u] : 0.f) * pr[u];
  }
  lds_barrier();

  // 4. dT += dW Kg^T (Kg rows of block R: Kr Diag(gamma_mR));
  //    AR = Diag(gamma_mR) applied to dKg = Diag(beta) M^T dW
  float pq[NE];
#pragma unroll
  for (int u = 0; u < NE; ++u) {
    const int e = t + u * kNT;
    const int r = e / DK, c = e % DK;
    pq[u] = ld_in<BF16>(p.q, ((ck.tok0 + in_rows(r, nv)) * H + h) * int64_t(DK) + c);
  }
  f4 ar[NT4];
  zero(ar);
  {
    f4 at[2];
    zero(at);
    // (A = dW rows r, B = Kr rows s of column block n0: B scaled by gamma_m of
    // that block, per channel k)
    const int i = li;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      int m0, n0;
      tile_origin<64>(w, s2, m0, n0);
      const float* const gmb = sGM + (n0 >> 4) * DK;
#pragma unroll 2
      for (int kb = 0; kb < DK / 16; ++kb) {
        const int k0 = 16 * kb + 4 * g;
        const f4 av = *reinterpret_cast<const f4*>(R2 + (m0 + i) * LD + k0);
        const f4 bv = *reinterpret_cast<const f4*>(R3 + (n0 + i) * LD + k0);
        const f4 sc = *reinterpret_cast<const f4*>(gmb + k0);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          at[s2] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[j], bv[j] * sc[j], at[s2], 0, 0, 0);
      }
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      int m0, n0;
      tile_origin<64>(w, s, m0, n0);
#pragma unroll
      for (int q = 0; q < 4; ++q) sX[(m0 + 4 * g + q) * kL64 + n0 + li] += at[s][q];
    }
  }
  mm<64, DK, 64, false, false, NT4, tri_dk<DK>(3)>(ar, sM, kL64, R2, LD, w);
#pragma unroll
  for (int s = 0; s < NT4; ++s) {
    if (!tile_live<64, DK>(w, s)) break;
    int m0, n0;
    tile_origin<DK>(w, s, m0, n0);
    const float gm = sGM[(m0 >> 4) * DK + n0 + li];
#pragma unroll
    for (int q = 0; q < 4; ++q) ar[s][q] *= sb[m0 + 4 * g + q] * gm;
  }
  lds_barrier();
#pragma unroll
  for (int u = 0; u < NE; ++u) {   // Qr
    const int e = t + u * kNT;
    R2[(e / DK) * LD + e % DK] = (e / DK < nv ? pq[u] : 0.f) * pr[u];
  }
  lds_barrier();

  // 5. AH += dP^T Qr;  AQ += dP Kh (strict dP, factored);  dbeta from T
  gsum<DK, true>(ah, sP, kL64, R2, LD, w, rho);
  gsum<DK, false>(aq, sP, kL64, R1, LD, w, rho);
  {   // column sums of M o dT (M is lower triangular), 8 rows per thread
    const int col = t & 63, part = t >> 6;
    float s = 0.f;
#pragma unroll
    for (int r = 8 * part; r < 8 * part + 8; ++r) s += sM[r * kL64 + col] * sX[r * kL64 + col];
    red[part * 64 + col] = s;
  }
  lds_barrier();
  if (t < 64) {
    float s = 0.f;
#pragma unroll
    for (int part = 0; part < kNT / 64; ++part) s += red[part * 64 + t];
    sdb[t] = s;
  }
#pragma unroll
  for (int u = 0; u < 64 * 64 / kNT; ++u) {   // dM = dT Diag(beta)
    const int e = t + u * kNT;
    const int r = e >> 6, c = e & 63;
    sX[r * kL64 + c] *= sb[c];
  }
  lds_barrier();
  {
    f4 atm[2];
    zero(atm);
    mm<64, 64, 64, true, true>(atm, sX, kL64, sM, kL64, w);   // dM M^T
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      int m0, n0;
      tile_origin<64>(w, s, m0, n0);
#pragma unroll
      for (int q = 0; q < 4; ++q) sP[(m0 + 4 * g + q) * kL64 + n0 + li] = atm[s][q];
    }
  }
  lds_barrier();
  {
    f4 ada[2];
    zero(ada);
    mm<64, 64, 64, false, false>(ada, sM, kL64, sP, kL64, w);   // M^T (dM M^T)
    // dA = -M^T dM M^T (strictly lower); dbeta_r += sum_s dA_rs X_rs, X from
    // the prep kernel (stored transposed above the diagonal)
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      int m0, n0;
      tile_origin<64>(w, s, m0, n0);
      float v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = m0 + 4 * g + q, c = n0 + li;
        const float da = c < r ? -ada[s][q] : 0.f;
        ada[s][q] = da;
        v[q] = c < r ? da * PXg[c * 64 + r] : 0.f;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float x = v[q];
        x += __shfl_xor(x, 1);
        x += __shfl_xor(x, 2);
        x += __shfl_xor(x, 4);
        x += __shfl_xor(x, 8);
        if (li == 0) red[(n0 >> 4) * 64 + m0 + 4 * g + q] = x;
      }
    }
    lds_barrier();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      int m0, n0;
      tile_origin<64>(w, s, m0, n0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = m0 + 4 * g + q;
        sX[r * kL64 + n0 + li] = sb[r] * ada[s][q];
      }
    }
    if (t < 64) sdb[t] += red[t] + red[64 + t] + red[128 + t] + red[192 + t];
  }
  lds_barrier();

  // 6. AR += B Kh;  AH += B^T Kr  (B = Diag(beta) dA, factored).  The decays
  // of this lane's output elements are loaded first, the alphas of step 8
  // after the products.
  float rh[NT4][4];
#pragma unroll
  for (int s = 0; s < NT4; ++s) {
    int m0, n0;
    tile_origin<DK>(w, s, m0, n0);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      rh[s][q] = tile_live<64, DK>(w, s) ? rho[(m0 + 4 * g + q) * DK + n0 + li] : 1.f;
  }
  gsum<DK, false>(ar, sX, kL64, R1, LD, w, rho);
  gsum<DK, true>(ah, sX, kL64, R3, LD, w, rho);
  constexpr int NP = kNT / DK, RP = 64 / NP;
  float al[SG ? 1 : RP];
  if constexpr (SG) {
    const int r = t >> 3;
    al[0] = p.alpha[(ck.tok0 + in_rows(r, nv)) * H + h];   // used for rows < nv only
  } else {
    const int c = t % DK, pp = t / DK;
#pragma unroll
    for (int i = 0; i < RP; ++i) {
      const int r = pp * RP + i;
      al[i] = p.alpha[((ck.tok0 + in_rows(r, nv)) * H + h) * int64_t(DK) + c];   // rows < nv only
    }
  }

  // 7. dq, dk (the diagonal of dP added apart: q_r . k_r carries no decay);
  // dg = AQ Qr + AR Kr - AH Kh without AHe (+ gamma_C S dS' on the last row);
  // z = AHe Kh into R1 (each lane overwrites only the Kh entries it read)
  float dgv[NT4][4];
#pragma unroll
  for (int s = 0; s < NT4; ++s) {
    if (!tile_live<64, DK>(w, s)) break;
    int m0, n0;
    tile_origin<DK>(w, s, m0, n0);
    const int c = n0 + li;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = m0 + 4 * g + q;
      const float kr = R3[r * LD + c], kh = R1[r * LD + c], qr = R2[r * LD + c];
      float dg = aq[s][q] * qr + ar[s][q] * kr - ah[s][q] * kh;
      if (r == kC - 1) dg += sdgc[c];
      dgv[s][q] = dg;
      R1[r * LD + c] = ahe[s][q] * kh;
      if (r < nv) {
        const int64_t x = ((ck.tok0 + r) * H + h) * int64_t(DK) + c;
        const float pd = sdpd[r];
        p.dq[x] = aq[s][q] * rh[s][q] + pd * (kh * rh[s][q]);
        p.dk[x] = ar[s][q] * rh[s][q] + (ah[s][q] + ahe[s][q]) / rh[s][q] + pd * (qr / rh[s][q]);
      }
    }
  }
  lds_barrier();
#pragma unroll
  for (int s = 0; s < NT4; ++s) {
    if (!tile_live<64, DK>(w, s)) break;
    int m0, n0;
    tile_origin<DK>(w, s, m0, n0);
#pragma unroll
    for (int q = 0; q < 4; ++q) R2[(m0 + 4 * g + q) * LD + n0 + li] = dgv[s][q];
  }
  if (t < 64 && t < nv) p.dbeta[(ck.tok0 + t) * H + h] = sdb[t];
  lds_barrier();
  // 8. dlog(alpha)_t = sum_{r >= t} dg_r + sum_{r < t} z_r within the chunk;
  // dalpha = that / alpha.  Each channel's 64 rows in NP parts of RP rows:
  // sums from the end (dg) and from the start (z) within a part, plus the
  // totals of the later (dg) and earlier (z) parts.
  {
    const int c = t % DK, pp = t / DK;
    float* const red2 = sGM;   // [NP][DK] over sGM and sGQ (no longer needed)
    static_assert(NP * DK <= 8 * DK && NP * DK <= RED, "partial sums fit");
    float v[RP];
    float run = 0.f, zr = 0.f;
#pragma unroll
    for (int i = RP - 1; i >= 0; --i) {
      run += R2[(pp * RP + i) * LD + c];
      v[i] = run;
    }
#pragma unroll
    for (int i = 0; i < RP; ++i) {
      v[i] += zr;
      zr += R1[(pp * RP + i) * LD + c];
    }
    red[pp * DK + c] = run;
    red2[pp * DK + c] = zr;
    lds_barrier();
    float off = 0.f;
    for (int q2 = pp + 1; q2 < NP; ++q2) off += red[q2 * DK + c];
    for (int q2 = 0; q2 < pp; ++q2) off += red2[q2 * DK + c];
    if constexpr (SG) {
#pragma unroll
      for (int i = 0; i < RP; ++i) R2[(pp * RP + i) * LD + c] = v[i] + off;
    } else {
#pragma unroll
      for (int i = 0; i < RP; ++i) {
        const int r = pp * RP + i;
        if (r < nv) {
          const int64_t x = ((ck.tok0 + r) * H + h) * int64_t(DK) + c;
          p.dalpha[x] = (v[i] + off) / al[i];
        }
      }
    }
  }
  if constexpr (SG) {   // one gate per token: the sum over the channels, 8 threads per row
    lds_barrier();
    const int r = t >> 3, part = t & 7;
    float s = 0.f;
#pragma unroll
    for (int c = part * (DK / 8); c < (part + 1) * (DK / 8); ++c) s += R2[r * LD + c];
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    s += __shfl_xor(s, 4);
    if (part == 0 && r < nv) {
      const int64_t row = (ck.tok0 + r) * H + h;
      p.dalpha[row] = s / al[0];
    }
  }
}

template <int DK, bool BF16, bool SG>
void launch_t(const BwdChunkArgs& a, int stage, hipStream_t st) {
  const unsigned nchunk = unsigned(int64_t(a.N) * a.win_k * a.H);
  if (stage == 0) {
    hipLaunchKernelGGL((kda_bwdc_prep_kernel<DK, BF16, SG>), dim3(nchunk), dim3(kNT), 0, st, a);
  } else if (stage == 1) {
    const unsigned nb = unsigned(int64_t(a.N) * a.H * (a.DV / 16));
    hipLaunchKernelGGL((kda_bwdc_chain_kernel<DK>), dim3(nb), dim3(64 * (DK / 16)), 0, st, a);
  } else {
    hipLaunchKernelGGL((kda_bwdc_post_kernel<DK, BF16, SG>), dim3(nchunk), dim3(kNT), 0, st, a);
  }
}

template <int DK>
void launch_dk(const BwdChunkArgs& a, int stage, hipStream_t st) {
  if (a.alpha_scalar) {
    if (a.in_bf16) launch_t<DK, true, true>(a, stage, st);
    else launch_t<DK, false, true>(a, stage, st);
  } else {
    if (a.in_bf16) launch_t<DK, true, false>(a, stage, st);
    else launch_t<DK, false, false>(a, stage, st);
  }
}

}  // namespace

size_t backward_chunk_floats(int DK, int DV) {
  // A_c, b_c, dS', M, Vn, the decays, P and X per chunk-head
  return size_t(DK) * DK + 2 * size_t(DK) * DV + 64 * 64 + 64 * size_t(DV) + kDecayRows * size_t(DK) +
         64 * 64;
}

int launch_backward_chunk(const BwdChunkArgs& a, int stage, void* stream, const char** msg) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (a.DK == 128) launch_dk<128>(a, stage, st);
  else if (a.DK == 64) launch_dk<64>(a, stage, st);
  else {
    *msg = "unsupported DK";
    return 1;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    *msg = hipGetErrorString(e);
    return 1;
  }
  return 0;
}

}  // namespace kda

// KDA chunked prefill on gfx950 (MI355X).
//
// The chunk form of the KDA recurrence ("Kimi Delta Attention 徹底解説"
// (tech-tide.dev), section "Kimi Delta Attention の仕組み": prefill regroups
// the token recurrence into chunked matrix products; "Kimi Linear、独自の土俵で
// Full Attentionを上回る" (remio.ai), section "Kimi Linearがより賢いRecurrent
// Memoryを使う方法": the chunkwise algorithm rests on a diagonal-plus-low-rank
// transition).  The pages print no chunk formula; the one used here follows
// from unrolling the recurrence inside a chunk of n <= 64 tokens with
// incoming state S (d_k x d_v, rows = key channels).  Per key channel, with
// gamma_r the product of alpha over the chunk's rows 0..r:
//     K_g = K * gamma,  Q_g = Q * gamma,  K_e = K * (gamma_n / gamma)
//     A   = Diag(beta) strict_lower(G_K),  P = lower(G_Q),
//           G_K[r,i] = sum_c k_rc k_ic gamma_rc / gamma_ic  (G_Q: q_r)
//     T   = (I + A)^-1 Diag(beta)                 (unit-lower solve)
//     U   = T (V - K_g S)                         (values actually written)
//     O   = Q_g S + P U
//     S'  = Diag(gamma_n) S + K_e^T U
// All products are dense MFMA contractions.  bf16 inputs use split bf16
// operands (x = hi + lo, three MFMAs per product) so that the products carry
// ~16 significant bits; fp32 inputs use the fp32 MFMA.  Accumulation is fp32.
//
// Decay factors are products of alpha (no exp / log).  The Gram matrices need
// gamma_r / gamma_i split into a row factor and a column factor; each 16-row
// block R takes its own reference row m_R = 16 R + 7, so a factor spans at
// most 8 tokens and stays within alpha^-8 (finite in fp32 down to alpha ~ 2e-5):
//     Kl = K * rho,  Ql = Q * rho,  Kr = K / rho,   rho_r = gamma_r / gamma_m(R(r))
// Diagonal 16x16 blocks are Kl_R Kr_R^T.  An off-diagonal block (R, I < R)
// also needs gamma_mR / gamma_mI, which can underflow where the block's
// entries do not; its column operand is therefore rescaled in two steps,
// first to the end of block I (Kr_I * S1_I <= 1), then on to m_R (* E_RI):
// every intermediate stays within the range of the true entries.
//
// One workgroup (4 waves) per (sequence, head, value slab): the value columns
// of the state evolve independently, so the sequential pass over the chunks
// is split into slabs of 16..128 columns to give enough workgroups; a
// workgroup holds its slab of S in registers for the whole sequence.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "kda_internal.h"

namespace kda {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));

constexpr int kC = 64;    // chunk length

struct Params {
  int N;
  int64_t T_fixed;
  const int32_t* cu;
  int H, DV, nslab;
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;
  const float* s_in;
  float* o;
  float* s_out;
  float* snap;        // state snapshots [rows][H][DK][DV] (SNAP kernels)
  int snap_every;     // a snapshot after every snap_every-th full chunk
  int64_t snap_per_seq;   // fixed length: sequence n's snapshot j is row n * snap_per_seq + j
  const int32_t* snap_off;  // varlen: row snap_off[n] + j, j < snap_off[n+1] - snap_off[n]
                            // (NULL: row cu[n] / 64 + j)
  int64_t snap_rows;        // varlen: rows of snap (rows outside [0, snap_rows) are skipped)
  int alpha_scalar;   // alpha is [tokens][H] (one gate per token and head)
  int states_only;    // with snapshots: o is not needed (NOO kernels)
};

// ---------------------------------------------------------------- layout ----
// Operand arrays are [rows][K] with the contraction index K contiguous.  In
// bf16 mode every group of 8 consecutive K holds 8 hi parts (16 B) followed by
// the 8 lo parts (16 B); in fp32 mode an element is one float.  Either way an
// element takes 4 bytes and a row has a 16-byte pad (conflict-free 128-bit
// fragment reads).
template <int DK>
struct Lay {
  static constexpr int NW = DK / 16;        // waves: one 16-row tile of the state each
  static constexpr int NT = 64 * NW;        // threads
  static constexpr int P_OP = DK * 4 + 16;  // rows of DK elements
  static constexpr int P_T = kC * 4 + 16;   // rows of 64 elements (272 B)
  static constexpr int P_AF = kC + 4;       // fp32 pitch (floats) of A and L^-1 (272 B)
  static constexpr int OFF_KL = 0;
  static constexpr int OFF_QL = OFF_KL + kC * P_OP;
  static constexpr int OFF_KRT = OFF_QL + kC * P_OP;         // Kr^T [DK][64]
  static constexpr int OFF_X = OFF_KRT + DK * P_T;           // Kr, then A + P
  static constexpr int SZ_X = (kC * P_OP > 2 * kC * P_T) ? kC * P_OP : 2 * kC * P_T;
  static constexpr int OFF_A = OFF_X;                        // fp32 [64][68]
  static constexpr int OFF_P = OFF_X + kC * P_T;             // [64][64]
  static constexpr int OFF_SBT = OFF_X;                      // S^T [16][DK]  (after the solve)
  static constexpr int OFF_XT = OFF_SBT + 16 * P_OP;         // X^T [16][64]
  static constexpr int OFF_UT = OFF_XT + 16 * P_T;           // U^T [16][64]
  static constexpr int OFF_T = OFF_X + SZ_X;                 // T [64][64] (fp32 L^-1 first)
  static constexpr int RG = 16;                              // row groups (4 rows) of the decay prep
  // Steps 1-2 only (the T space is free until the solve):
  static constexpr int OFF_GP = OFF_T;                       // group products [RG][DK]
  static constexpr int OFF_S1 = OFF_GP + RG * DK * 4;        // S1_I = gamma_(16I+15) / gamma_mI [4][DK]
  static constexpr int OFF_E = OFF_S1 + 4 * DK * 4;          // E_RI = gamma_mR / gamma_(16I+15) [6][DK]
  static constexpr int OFF_GNM = OFF_E + 6 * DK * 4;         // gamma_n / gamma_mI [4][DK]
  // Kept for the whole chunk:
  static constexpr int OFF_GM = OFF_T + kC * P_T;           // gamma_mR [4][DK]
  static constexpr int OFF_GN = OFF_GM + 4 * DK * 4;         // gamma_n [DK]
  static constexpr int OFF_BE = OFF_GN + DK * 4;             // beta [64]
  static constexpr int TOTAL = OFF_BE + kC * 4;
  static_assert(OFF_GNM + 4 * DK * 4 <= OFF_T + kC * P_T, "decay vectors fit the T space");
  static_assert(NT == RG * DK / 4, "decay prep: one thread per (channel quad, row group)");
  static_assert(RG * DK * 4 <= kC * P_T, "group products fit the T space");
  static_assert(OFF_UT + 16 * P_T <= OFF_X + kC * P_T, "step buffers fit in A's space");
  static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

// Workgroup barrier that orders LDS only: pending global loads (prefetches)
// and stores stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// --------------------------------------------------------------- MFMA ops ---
template <bool BF>
struct Mma;

template <>
struct Mma<true> {  // split bf16: x = hi + lo, products hi*hi + hi*lo + lo*hi
  static constexpr int KU = 32;
  struct Frag {
    bf8 hi, lo;
  };
  // Fragment of rows row0..row0+15 (row = row0 + lane%16), K chunk kc.
  __device__ static Frag load(const char* base, int pitch, int row0, int kc) {
    const int l = lane_id();
    const char* p = base + (row0 + (l & 15)) * pitch + (kc * 4 + (l >> 4)) * 32;
    Frag f;
    f.hi = *reinterpret_cast<const bf8*>(p);
    f.lo = *reinterpret_cast<const bf8*>(p + 16);
    return f;
  }
  __device__ static f4 mma(const Frag& a, const Frag& b, f4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.hi, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.lo, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, c, 0, 0, 0);
    return c;
  }
};

template <>
struct Mma<false> {  // fp32 MFMA
  static constexpr int KU = 4;
  typedef float Frag;
  __device__ static Frag load(const char* base, int pitch, int row0, int kc) {
    const int l = lane_id();
    return *reinterpret_cast<const float*>(base + (row0 + (l & 15)) * pitch +
                                           (kc * 4 + (l >> 4)) * 4);
  }
  __device__ static f4 mma(Frag a, Frag b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

// acc += A[arow0.., 0:K] * B[brow0.., 0:K]^T  (both stored [row][K]).  All
// fragments are loaded before the first product, so the LDS latency is paid
// once per call rather than once per K chunk.
template <bool BF, int K>
__device__ __forceinline__ f4 gemm(f4 acc, const char* A, int ap, int arow0, const char* B,
                                   int bp, int brow0) {
  using M = Mma<BF>;
  constexpr int NKC = K / M::KU;
  typename M::Frag a[NKC], b[NKC];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) {
    a[kc] = M::load(A, ap, arow0, kc);
    b[kc] = M::load(B, bp, brow0, kc);
  }
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) acc = M::mma(a[kc], b[kc], acc);
  return acc;
}

// ------------------------------------------------------- operand stores -----
__device__ __forceinline__ uint16_t bf_bits(__bf16 x) { return __builtin_bit_cast(uint16_t, x); }

__device__ __forceinline__ void split(float x, uint16_t& h, uint16_t& l) {
  const __bf16 hb = static_cast<__bf16>(x);
  const __bf16 lb = static_cast<__bf16>(x - static_cast<float>(hb));
  h = bf_bits(hb);
  l = bf_bits(lb);
}

// Two elements at once: h and l hold (x0, x1) as packed bf16 pairs, x0 in the
// low half.  One packed conversion per part, and the hi parts are widened
// back by a shift and a mask: the same bits as split() on each element, in
// three instructions per element instead of four.
typedef float f2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& h, uint32_t& l) {
  h = __builtin_bit_cast(uint32_t, __builtin_convertvector((f2v{x0, x1}), bf2v));
  const float r0 = x0 - __uint_as_float(h << 16);
  const float r1 = x1 - __uint_as_float(h & 0xffff0000u);
  l = __builtin_bit_cast(uint32_t, __builtin_convertvector((f2v{r0, r1}), bf2v));
}

// c + A B for 16x16 blocks: lane (lr, lg) holds a[j] = A[lr][4lg + j] and
// b[j] = B[4lg + j][lr]; the result lane holds rows 4lg + q of column lr.
// Four 16x16x4 fp32 MFMAs for either input dtype: the operands are fp32
// values in registers (the triangular solve's blocks), and splitting them into
// bf16 parts for the bf16 MFMA costs more VALU time on the solve's dependent
// chain than the fp32 MFMA's extra passes.
__device__ __forceinline__ f4 mm16x16(const f4& a, const f4& b, f4 c) {
#pragma unroll
  for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
  return c;
}

// One element (row, kk).
template <bool BF>
__device__ __forceinline__ void st1(char* base, int pitch, int row, int kk, float x) {
  if constexpr (BF) {
    uint16_t h, l;
    split(x, h, l);
    char* p = base + row * pitch + (kk >> 3) * 32 + (kk & 7) * 2;
    *reinterpret_cast<uint16_t*>(p) = h;
    *reinterpret_cast<uint16_t*>(p + 16) = l;
  } else {
    *reinterpret_cast<float*>(base + row * pitch + kk * 4) = x;
  }
}

// Two consecutive elements (row, kk), (row, kk+1); kk even.
template <bool BF>
__device__ __forceinline__ void st2(char* base, int pitch, int row, int kk, float x0, float x1) {
  if constexpr (BF) {
    uint32_t h, l;
    split2(x0, x1, h, l);
    char* p = base + row * pitch + (kk >> 3) * 32 + (kk & 7) * 2;
    *reinterpret_cast<uint32_t*>(p) = h;
    *reinterpret_cast<uint32_t*>(p + 16) = l;
  } else {
    *reinterpret_cast<float2*>(base + row * pitch + kk * 4) = make_float2(x0, x1);
  }
}

// Four consecutive elements starting at kk (kk % 4 == 0).
template <bool BF>
__device__ __forceinline__ void st4(char* base, int pitch, int row, int kk, const float* x) {
  if constexpr (BF) {
    char* p = base + row * pitch + (kk >> 3) * 32 + (kk & 7) * 2;
    uint2 hv, lv;
    split2(x[0], x[1], hv.x, lv.x);
    split2(x[2], x[3], hv.y, lv.y);
    *reinterpret_cast<uint2*>(p) = hv;
    *reinterpret_cast<uint2*>(p + 16) = lv;
  } else {
    *reinterpret_cast<float4*>(base + row * pitch + kk * 4) = make_float4(x[0], x[1], x[2], x[3]);
  }
}

// Eight consecutive elements starting at kk (kk % 8 == 0): one 8-group.
template <bool BF>
__device__ __forceinline__ void st8(char* base, int pitch, int row, int kk, const float* x) {
  if constexpr (BF) {
    char* p = base + row * pitch + (kk >> 3) * 32;
    uint4 hv, lv;
    split2(x[0], x[1], hv.x, lv.x);
    split2(x[2], x[3], hv.y, lv.y);
    split2(x[4], x[5], hv.z, lv.z);
    split2(x[6], x[7], hv.w, lv.w);
    *reinterpret_cast<uint4*>(p) = hv;
    *reinterpret_cast<uint4*>(p + 16) = lv;
  } else {
    st4<BF>(base, pitch, row, kk, x);
    st4<BF>(base, pitch, row, kk + 4, x + 4);
  }
}

// -------------------------------------------------------- global inputs -----
template <bool BF>
__device__ __forceinline__ float2 ld2(const void* p, int64_t i) {
  if constexpr (BF) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p) + i);
    return make_float2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
  } else {
    return *reinterpret_cast<const float2*>(static_cast<const float*>(p) + i);
  }
}

template <bool BF>
__device__ __forceinline__ float ld1(const void* p, int64_t i) {
  if constexpr (BF) {
    return __uint_as_float(uint32_t(static_cast<const uint16_t*>(p)[i]) << 16);
  } else {
    return static_cast<const float*>(p)[i];
  }
}

__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Raw (unconverted) input words, so that prefetched loads are not consumed
// before they are needed: a bf16 pair / bf16 value, or fp32.
template <bool BF> struct Raw { typedef uint2 four; typedef uint32_t two; typedef uint32_t one; };
template <> struct Raw<false> { typedef float4 four; typedef float2 two; typedef float one; };

template <bool BF>
__device__ __forceinline__ typename Raw<BF>::two ldraw2(const void* p, uint32_t i) {
  if constexpr (BF) return *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p) + i);
  else return *reinterpret_cast<const float2*>(static_cast<const float*>(p) + i);
}
template <bool BF>
__device__ __forceinline__ typename Raw<BF>::one ldraw1(const void* p, uint32_t i) {
  if constexpr (BF) return uint32_t(static_cast<const uint16_t*>(p)[i]);
  else return static_cast<const float*>(p)[i];
}
template <bool BF>
__device__ __forceinline__ typename Raw<BF>::four ldraw4(const void* p, uint32_t i) {
  if constexpr (BF) return *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i);
  else return *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
}
template <bool BF>
__device__ __forceinline__ float4 cvt4(typename Raw<BF>::four r) {
  if constexpr (BF)
    return make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
                       __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u));
  else return r;
}
template <bool BF>
__device__ __forceinline__ float2 cvt2(typename Raw<BF>::two r) {
  if constexpr (BF) return make_float2(__uint_as_float(r << 16), __uint_as_float(r & 0xffff0000u));
  else return r;
}
template <bool BF>
__device__ __forceinline__ float cvt1(typename Raw<BF>::one r) {
  if constexpr (BF) return __uint_as_float(r << 16);
  else return r;
}


// ------------------------------------------------------ MFMA transposes -----
// Transposing through the MFMA: with B a column selector (B[n][k] = s_n when k
// is column n, else 0), A B^T picks out columns of A, scaled by s, in the
// result layout, where a lane holds four consecutive rows of one column, i.e.
// four consecutive elements of one row of the transposed array.  One 8-byte
// LDS store per hi/lo part and lane then writes the transposed tile without
// bank conflicts (stores of a [channel][token] array from a per-thread block
// of channels x tokens conflict many ways).
//   dst[16cb + lr][16rb + 4lg + q] = A[16rb + 4lg + q][16cb + lr] * s
__device__ __forceinline__ uint32_t bf16_bits_rne(float x) {
  return uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(x)));
}

// Split bf16: `a` covers the 32 columns 32kc.. (tiles cb = 2kc, 2kc+1) of row
// block rb; s0 / s1 are this lane's column scales for the two tiles (column
// 16cb + lr).  With hi_only the lo parts of `a` are zero and s0 = s1 = 1.
template <bool HI_ONLY>
__device__ __forceinline__ void xpose32_bf(const Mma<true>::Frag& a, int rb, int kc, float s0, float s1,
                                           char* dst, int dpitch) {
  const int l = lane_id(), lr = l & 15, lg = l >> 4;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float sc = h ? s1 : s0;
    const bool mine = lg == 2 * h + (lr >> 3);
    const int e = lr & 7;
    const uint32_t sh = bf16_bits_rne(sc);
    const uint32_t sl = HI_ONLY ? 0u : bf16_bits_rne(sc - __uint_as_float(sh << 16));
    uint32_t wh[4], wl[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool here = mine && (e >> 1) == j;
      wh[j] = here ? ((e & 1) ? (sh << 16) : sh) : 0u;
      wl[j] = here ? ((e & 1) ? (sl << 16) : sl) : 0u;
    }
    Mma<true>::Frag b;
    b.hi = __builtin_bit_cast(bf8, make_uint4(wh[0], wh[1], wh[2], wh[3]));
    b.lo = __builtin_bit_cast(bf8, make_uint4(wl[0], wl[1], wl[2], wl[3]));
    f4 acc = f4{0.f, 0.f, 0.f, 0.f};
    if constexpr (HI_ONLY) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, acc, 0, 0, 0);
    else acc = Mma<true>::mma(a, b, acc);
    const float x[4] = {acc[0], acc[1], acc[2], acc[3]};
    st4<true>(dst, dpitch, 32 * kc + 16 * h + lr, 16 * rb + 4 * lg, x);
  }
}

// fp32: a4[j] is this lane's element of row 16rb + lr, column 16cb + 4lg + j;
// s is this lane's column scale (column 16cb + lr).
__device__ __forceinline__ void xpose16_f32(const float (&a4)[4], int rb, int cb, float s, char* dst,
                                            int dpitch) {
  const int l = lane_id(), lr = l & 15, lg = l >> 4;
  f4 acc = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; ++j)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[j], 4 * lg + j == lr ? s : 0.f, acc, 0, 0, 0);
  const float x[4] = {acc[0], acc[1], acc[2], acc[3]};
  st4<false>(dst, dpitch, 16 * cb + lr, 16 * rb + 4 * lg, x);
}

// Transposes the columns of a [64][DK] LDS operand array (rows = tokens) into
// a [DK][64] array, scaled per column by scale[] (LDS; with PER_RB, rows of
// 16-row block rb by scale[rb * DK + column]): the work is spread over the NW
// waves.
template <bool BF, int DK, int NW, bool PER_RB>
__device__ __forceinline__ void xpose_lds(const char* src, int spitch, const float* scale, char* dst,
                                          int dpitch) {
  const int l = lane_id(), lr = l & 15, lg = l >> 4, w = threadIdx.x >> 6;
  if constexpr (BF) {
    constexpr int NU = 4 * (DK / 32);   // (row block, 32-column chunk) units
    static_assert(NU % NW == 0, "equal share per wave");
#pragma unroll
    for (int i = 0; i < NU / NW; ++i) {
      const int u = w + NW * i, rb = u & 3, kc = u >> 2;
      const float* sc = PER_RB ? scale + rb * DK : scale;
      const Mma<true>::Frag a = Mma<true>::load(src, spitch, 16 * rb, kc);
      xpose32_bf<false>(a, rb, kc, sc[32 * kc + lr], sc[32 * kc + 16 + lr], dst, dpitch);
    }
  } else {
    constexpr int NU = 4 * (DK / 16);   // (row block, 16-column block) units
    static_assert(NU % NW == 0, "equal share per wave");
#pragma unroll
    for (int i = 0; i < NU / NW; ++i) {
      const int u = w + NW * i, rb = u & 3, cb = u >> 2;
      const float* sc = PER_RB ? scale + rb * DK : scale;
      const float4 v = *reinterpret_cast<const float4*>(src + (16 * rb + lr) * spitch + 4 * (16 * cb + 4 * lg));
      const float a4[4] = {v.x, v.y, v.z, v.w};
      xpose16_f32(a4, rb, cb, sc[16 * cb + lr], dst, dpitch);
    }
  }
}

// A fragment of the column operand Kr with every K (channel) element scaled
// by s1[k] and then by e[k] (two roundings, so that no intermediate leaves the
// range of the result).  Split bf16: the lane's 8 channels 32kc + 8lg .. +7
// are rebuilt in fp32, scaled and split again; fp32: channel 4kc + lg.
__device__ __forceinline__ float bf_lo16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ Mma<true>::Frag rescale_frag(const Mma<true>::Frag& f, const float* s1,
                                                       const float* e, int kc) {
  const int k0 = 32 * kc + 8 * (lane_id() >> 4);
  const float4 sa = *reinterpret_cast<const float4*>(s1 + k0), sb = *reinterpret_cast<const float4*>(s1 + k0 + 4);
  const float4 ea = *reinterpret_cast<const float4*>(e + k0), eb = *reinterpret_cast<const float4*>(e + k0 + 4);
  const float sv[8] = {sa.x, sa.y, sa.z, sa.w, sb.x, sb.y, sb.z, sb.w};
  const float ev[8] = {ea.x, ea.y, ea.z, ea.w, eb.x, eb.y, eb.z, eb.w};
  const uint4 hi = __builtin_bit_cast(uint4, f.hi), lo = __builtin_bit_cast(uint4, f.lo);
  const uint32_t hw[4] = {hi.x, hi.y, hi.z, hi.w}, lw[4] = {lo.x, lo.y, lo.z, lo.w};
  uint32_t nh[4], nl[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float x0 = ((bf_lo16(hw[j]) + bf_lo16(lw[j])) * sv[2 * j]) * ev[2 * j];
    const float x1 = ((bf_hi16(hw[j]) + bf_hi16(lw[j])) * sv[2 * j + 1]) * ev[2 * j + 1];
    split2(x0, x1, nh[j], nl[j]);
  }
  Mma<true>::Frag r;
  r.hi = __builtin_bit_cast(bf8, make_uint4(nh[0], nh[1], nh[2], nh[3]));
  r.lo = __builtin_bit_cast(bf8, make_uint4(nl[0], nl[1], nl[2], nl[3]));
  return r;
}

__device__ __forceinline__ float rescale_frag(float f, const float* s1, const float* e, int kc) {
  const int k = 4 * kc + (lane_id() >> 4);
  return (f * s1[k]) * e[k];
}

// Destination of output stores for rows past the end of a sequence, and of
// the mirrored stores below (never read): 32 stores of 64 lanes per workgroup
// slot, workgroups taken modulo 256.
constexpr int kSinkStores = 32;
}  // namespace
// (external linkage: stores to it are not dead to the compiler)
__device__ float g_kda_sink[256 * kSinkStores * 64];
namespace {

// N stores to distinct sink addresses (plain stores: the compiler keeps them,
// since they reach memory other code could read, and does not wait for them).
// Issued after a kernel's first prefetch, they stand in for the stores that
// follow the prefetch in every later iteration, so that the compiler's
// memory-counter waits for prefetched values need not cover those stores.
template <int N>
__device__ __forceinline__ void mirror_stores() {
  static_assert(N <= kSinkStores, "sink size");
  float* sink = g_kda_sink + (blockIdx.x & 255) * (kSinkStores * 64) + (threadIdx.x & 63);
#pragma unroll
  for (int i = 0; i < N; ++i) sink[64 * i] = 0.f;
}

// Thread -> (column quad cq, group grp of consecutive rows) of a 64-row chunk
// with QUADS column quads: consecutive threads take consecutive quads
// of one row group (a wave's loads read whole rows).  (A wave-blocked mapping,
// 8 quads x 8 groups per wave, measured slower.)
template <int QUADS>
__device__ __forceinline__ void quad_map(int t, int& cq, int& grp) {
  cq = t % QUADS;
  grp = t / QUADS;
}

// Index of the off-diagonal block (R, I), I < R, in the [6][DK] E vectors.
__host__ __device__ constexpr int eidx(int R, int I) { return R * (R - 1) / 2 + I; }

// One wave's tiles of the intra-chunk Gram matrices A = Kl Kr^T (type 0) and
// P = Ql Kr^T (type 1) for the block pair (R, I), plus with XD >= 0 the
// diagonal tile (type XD, R, R).  For I < R the column operand Kr_I is scaled
// by S1_I and then E_RI (the decay from the tokens of block I to the
// reference row of block R, see the top of the file).  Tiles are computed
// transposed (Kr rows as the first operand) so that a lane ends up with four
// consecutive columns of one row; operands shared by the tiles are loaded once
// per K chunk (this step is bound by LDS read bandwidth, not by the MFMA rate).
template <bool BF, int DK, int R, int I, int XD>
__device__ __forceinline__ void gram_group(const char* sKl, const char* sQl, const char* sKr,
                                           const float* sS1, const float* sE, f4 (&acc)[3]) {
  using M = Mma<BF>;
  constexpr int P = DK * 4 + 16;
#pragma unroll
  for (int kc = 0; kc < DK / M::KU; ++kc) {
    auto c = M::load(sKr, P, 16 * I, kc);
    if constexpr (I < R) c = rescale_frag(c, sS1 + I * DK, sE + eidx(R, I) * DK, kc);
    const auto rk = M::load(sKl, P, 16 * R, kc);
    const auto rq = M::load(sQl, P, 16 * R, kc);
    acc[0] = M::mma(c, rk, acc[0]);
    acc[1] = M::mma(c, rq, acc[1]);
    if constexpr (XD >= 0) {
      const auto cd = M::load(sKr, P, 16 * R, kc);
      acc[2] = M::mma(cd, XD == 0 ? rk : rq, acc[2]);
    }
  }
}

// Steps 1-3 of one chunk (everything that does not depend on the state):
// decay factors and decayed operands, the Gram tiles A and P, and
// T = (I + A)^-1 Diag(beta).  On return the LDS holds Kl, Ql (CONVERT: K_g and
// Q_g in their place), K_e^T (in the Kr^T array), T, P, gamma_mR of the four
// row blocks and gamma_n.  av/kv/qv are this thread's 4 rows (4g .. 4g+3) of
// 4 channels (4c .. 4c+3), c = t % (DK/4), g = t / (DK/4) (rows past the
// sequence end: alpha = 1, k = q = 0), bev is beta of token (threadIdx.x & 63)
// (0 past the end).
// after_gram() runs between steps 2 and 3 (callers issue global loads there,
// when the memory pipeline is idle).
template <int DK, bool BF, bool CONVERT, typename Hook>
__device__ __forceinline__ void prep_chunk(char* smem, const float4 (&av)[4], const float4 (&kv)[4],
                                           const float4 (&qv)[4], float bev, Hook&& after_gram) {
  using L = Lay<DK>;
  constexpr int NW = L::NW;
  constexpr int NT = L::NT;
  char* const sKl = smem + L::OFF_KL;
  char* const sQl = smem + L::OFF_QL;
  char* const sKrT = smem + L::OFF_KRT;
  char* const sKr = smem + L::OFF_X;
  float* const sA = reinterpret_cast<float*>(smem + L::OFF_A);
  char* const sP = smem + L::OFF_P;
  char* const sT = smem + L::OFF_T;
  float* const sLi = reinterpret_cast<float*>(smem + L::OFF_T);
  float* const sGP = reinterpret_cast<float*>(smem + L::OFF_GP);
  float* const sS1 = reinterpret_cast<float*>(smem + L::OFF_S1);
  float* const sE = reinterpret_cast<float*>(smem + L::OFF_E);
  float* const sGNM = reinterpret_cast<float*>(smem + L::OFF_GNM);
  float* const sGM = reinterpret_cast<float*>(smem + L::OFF_GM);
  float* const sGN = reinterpret_cast<float*>(smem + L::OFF_GN);
  float* const sBe = reinterpret_cast<float*>(smem + L::OFF_BE);
  const int t = threadIdx.x;
  const int l = t & 63;
  const int w = t >> 6;
  const int lr = l & 15;
  const int lg = l >> 4;
  int cq, grp;
  quad_map<DK / 4>(t, cq, grp);
  const int c0 = 4 * cq;           // this thread's channels c0 .. c0+3
  const int r0 = 4 * grp;          // this thread's rows r0 .. r0+3
  (void)l;
  auto mul4 = [](float4 a, float4 b) { return make_float4(a.x * b.x, a.y * b.y, a.z * b.z, a.w * b.w); };
  auto gp4 = [&](int g) { return *reinterpret_cast<const float4*>(sGP + g * DK + c0); };
  const float4 one4 = make_float4(1.f, 1.f, 1.f, 1.f);
  // product of the group products g0 .. g1 (inclusive; empty: 1)
  auto gprod = [&](int g0, int g1) {
    float4 x = one4;
    for (int g = g0; g <= g1; ++g) x = mul4(x, gp4(g));
    return x;
  };
  auto st4v = [&](float* dst, float4 x) { *reinterpret_cast<float4*>(dst + c0) = x; };

  // ---- step 1: decay factors and decayed operands ------------------------
  {
    float4 gp = mul4(mul4(av[0], av[1]), mul4(av[2], av[3]));
    *reinterpret_cast<float4*>(sGP + grp * DK + c0) = gp;
    if (t < kC) sBe[t] = bev;
  }
  lds_barrier();
  {
    // Row r of block R = r / 16 (reference row m_R = 16R + 7, the last row of
    // group 4R + 1): rho_r = gamma_r / gamma_mR.
    const int R = grp >> 2;
    if ((grp & 3) >= 2) {
      // rows after the reference: rho = prod_{m_R < s <= r} alpha_s <= 1
      float4 P = gprod(4 * R + 2, grp - 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        P = mul4(P, av[i]);
        const float4 iv = make_float4(rcp(P.x), rcp(P.y), rcp(P.z), rcp(P.w));
        const int r = r0 + i;
        const float4 a = mul4(kv[i], P), b = mul4(qv[i], P), c = mul4(kv[i], iv);
        const float xa[4] = {a.x, a.y, a.z, a.w}, xb[4] = {b.x, b.y, b.z, b.w};
        const float xc[4] = {c.x, c.y, c.z, c.w};
        st4<BF>(sKl, L::P_OP, r, c0, xa);
        st4<BF>(sQl, L::P_OP, r, c0, xb);
        st4<BF>(sKr, L::P_OP, r, c0, xc);
      }
    } else {
      // rows up to the reference: 1/rho = prod_{r < s <= m_R} alpha_s <= 1
      float4 Q = gprod(grp + 1, 4 * R + 1);
#pragma unroll
      for (int i = 3; i >= 0; --i) {
        const float4 f = make_float4(rcp(Q.x), rcp(Q.y), rcp(Q.z), rcp(Q.w));
        const int r = r0 + i;
        const float4 a = mul4(kv[i], f), b = mul4(qv[i], f), c = mul4(kv[i], Q);
        const float xa[4] = {a.x, a.y, a.z, a.w}, xb[4] = {b.x, b.y, b.z, b.w};
        const float xc[4] = {c.x, c.y, c.z, c.w};
        st4<BF>(sKl, L::P_OP, r, c0, xa);
        st4<BF>(sQl, L::P_OP, r, c0, xb);
        st4<BF>(sKr, L::P_OP, r, c0, xc);
        Q = mul4(Q, av[i]);
      }
    }
    // Per-channel decay vectors, one set of threads each (chains of products,
    // every one of them a product over consecutive tokens, so none leaves the
    // range of what it stands for).  The sets are the first row group of
    // waves 0-3, so that no wave runs two of the chains one after the other.
    constexpr int GPW = 256 / DK;   // row groups per wave
    if (grp == 0) {
      // gamma_mR = gamma at row 16R + 7; gamma_n at row 63
      float4 x = gprod(0, 1);
      st4v(sGM, x);
#pragma unroll
      for (int RR = 1; RR < 4; ++RR) {
        x = mul4(x, gprod(4 * RR - 2, 4 * RR + 1));
        st4v(sGM + RR * DK, x);
      }
      st4v(sGN, mul4(x, gprod(14, 15)));
    } else if (grp == GPW) {
      // gamma_n / gamma_mI = product over rows 16I + 8 .. 63
      float4 x = gprod(14, 15);
      st4v(sGNM + 3 * DK, x);
#pragma unroll
      for (int II = 2; II >= 0; --II) {
        x = mul4(x, gprod(4 * II + 2, 4 * II + 5));
        st4v(sGNM + II * DK, x);
      }
    } else if (grp == 2 * GPW) {
      // S1_I: rows 16I + 8 .. 16I + 15;  E_(I+1),I: rows 16I + 16 .. 16I + 23
#pragma unroll
      for (int II = 0; II < 3; ++II) {
        st4v(sS1 + II * DK, gprod(4 * II + 2, 4 * II + 3));
        st4v(sE + eidx(II + 1, II) * DK, gprod(4 * II + 4, 4 * II + 5));
      }
    } else if (grp == 3 * GPW) {
      // E_RI for R >= I + 2: rows 16I + 16 .. 16R + 7
      const float4 x10 = gprod(4, 5), x21 = gprod(8, 9), x32 = gprod(12, 13);
      const float4 m1 = gprod(6, 7), m2 = gprod(10, 11);
      const float4 e20 = mul4(mul4(x10, m1), x21);
      const float4 e31 = mul4(mul4(x21, m2), x32);
      st4v(sE + eidx(2, 0) * DK, e20);
      st4v(sE + eidx(3, 1) * DK, e31);
      st4v(sE + eidx(3, 0) * DK, mul4(mul4(e20, m2), x32));
    }
  }
  lds_barrier();

  // ---- step 2: A = beta * strict_lower(G_K), P = lower(G_Q) --------------
  {
    // The 20 lower 16x16 tiles (10 of A, 10 of P) in eight groups: per row
    // block pair (R, I < R) the A and P tiles share the rescaled column
    // operand; a diagonal tile joins four of the groups.  Waves w and w + 4
    // share a SIMD and together take 5 tiles.
    f4 acc[2][3];
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int j = 0; j < 3; ++j) acc[g][j] = f4{0.f, 0.f, 0.f, 0.f};
    int tT[2][3], tR[2][3], tI[2][3];
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int j = 0; j < 3; ++j) tT[g][j] = -1, tR[g][j] = 0, tI[g][j] = 0;
#define KDA_GROUP(g, R_, I_, XD_)                                                      \
  gram_group<BF, DK, R_, I_, XD_>(sKl, sQl, sKr, sS1, sE, acc[g]);                     \
  tT[g][0] = 0; tR[g][0] = R_; tI[g][0] = I_;                                          \
  tT[g][1] = 1; tR[g][1] = R_; tI[g][1] = I_;                                          \
  tT[g][2] = XD_; tR[g][2] = R_; tI[g][2] = R_;
    if constexpr (NW >= 8) {
      switch (w) {
        case 0: KDA_GROUP(0, 3, 0, 0) break;
        case 1: KDA_GROUP(0, 3, 1, 1) break;
        case 2: KDA_GROUP(0, 2, 0, 0) break;
        case 3: KDA_GROUP(0, 2, 1, 1) break;
        case 4: KDA_GROUP(0, 0, 0, -1) break;
        case 5: KDA_GROUP(0, 1, 1, -1) break;
        case 6: KDA_GROUP(0, 3, 2, -1) break;
        default: KDA_GROUP(0, 1, 0, -1) break;
      }
    } else {
      switch (w) {
        case 0: KDA_GROUP(0, 3, 0, 0) KDA_GROUP(1, 0, 0, -1) break;
        case 1: KDA_GROUP(0, 3, 1, 1) KDA_GROUP(1, 1, 1, -1) break;
        case 2: KDA_GROUP(0, 2, 0, 0) KDA_GROUP(1, 3, 2, -1) break;
        default: KDA_GROUP(0, 2, 1, 1) KDA_GROUP(1, 1, 0, -1) break;
      }
    }
#undef KDA_GROUP
    // K_e^T = Diag(gamma_n / gamma_mI) Kr_I^T, rows = key channels (from the Kr rows)
    xpose_lds<BF, DK, NW, true>(sKr, L::P_OP, sGNM, sKrT, L::P_T);
    lds_barrier();  // every read of Kr is done: A and P overwrite it
    // Tile (R, I) transposed: lane (lr, lg) holds row 16R + lr, columns
    // 16I + 4lg .. +3.  On diagonal tiles the entries above the diagonal may
    // be infinite (factors up to alpha^-15): they are selected away, never
    // multiplied.
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        if (tT[g][j] >= 0) {
          const int r = 16 * tR[g][j] + lr;
          const int i0 = 16 * tI[g][j] + 4 * lg;
          float x[4];
          if (tT[g][j] == 1) {
#pragma unroll
            for (int q = 0; q < 4; ++q) x[q] = i0 + q <= r ? acc[g][j][q] : 0.f;
            st4<BF>(sP, L::P_T, r, i0, x);
          } else {
            const float be = sBe[r];
#pragma unroll
            for (int q = 0; q < 4; ++q) x[q] = i0 + q < r ? be * acc[g][j][q] : 0.f;
            *reinterpret_cast<float4*>(sA + r * L::P_AF + i0) = make_float4(x[0], x[1], x[2], x[3]);
          }
        }
      }
    // Upper tiles of P are zero (the P U product runs over the whole chunk).
    if (w >= NW - 2) {
      const float z[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 3; ++e) {
        const int blk = (w - (NW - 2)) * 3 + e;  // (0,1) (0,2) (0,3) (1,2) (1,3) (2,3)
        const int R = blk < 3 ? 0 : (blk < 5 ? 1 : 2);
        const int I = blk < 3 ? blk + 1 : (blk < 5 ? blk - 1 : 3);
        st4<BF>(sP, L::P_T, 16 * R + lr, 16 * I + 4 * lg, z);
      }
    }
  }
  lds_barrier();
  after_gram();

  // ---- step 3: T = (I + A)^-1 Diag(beta) ---------------------------------
  // 3a: inverses D_R = (I + N)^-1 of the four 16x16 unit-lower diagonal
  // blocks (N = A_RR strictly lower, so N^16 = 0):
  //     (I + N)^-1 = (I - N)(I + N^2)(I + N^4)(I + N^8),
  // wave R < 4 for block R, entirely in registers.  In the result layout a
  // lane holds M[4lg + q][lr] of a 16x16 matrix M (its B-operand quad for
  // mm16x16); the same layout of M^T holds M[lr][4lg + q] (M's A-operand
  // quad).  Every factor is a polynomial in N, so all of them commute: X P is
  // computed as P X from P^T's copy and X's, and each power P is kept with its
  // transpose, (P P)^T = mm(P's copy, P^T's copy).  Waves 4.. (or all waves
  // after their block) clear the upper blocks of L^-1.
  if (w < 4) {
    const int R = w;
    const float* const Nb = sA + 16 * R * L::P_AF + 16 * R;
    float* const Xb = sLi + 16 * R * L::P_AF + 16 * R;
    f4 No, Nt, Xo;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      No[q] = Nb[(4 * lg + q) * L::P_AF + lr];
      Nt[q] = Nb[lr * L::P_AF + 4 * lg + q];
      Xo[q] = (4 * lg + q == lr ? 1.f : 0.f) - No[q];
    }
    const f4 zero = f4{0.f, 0.f, 0.f, 0.f};
    f4 Po = mm16x16(Nt, No, zero), Pt = mm16x16(No, Nt, zero);   // N^2
#pragma unroll
    for (int e = 0; e < 3; ++e) {
      // X <- X + P X with P = N^(2^(e+1)); then P <- P P
      Xo = mm16x16(Pt, Xo, Xo);
      if (e < 2) {
        const f4 Po2 = mm16x16(Pt, Po, zero), Pt2 = mm16x16(Po, Pt, zero);
        Po = Po2;
        Pt = Pt2;
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) Xb[(4 * lg + q) * L::P_AF + lr] = Xo[q];
  }
  constexpr int w0 = NW > 4 ? 4 : 0;
  if (w >= w0) {
    // blocks (R, I) with I > R: (0,1) (0,2) (0,3) (1,2) (1,3) (2,3); waves
    // 4.. when there are 8, else every wave after its block
    for (int e = t - 64 * w0; e < 6 * 256; e += NT - 64 * w0) {
      const int blk = e >> 8, rr = (e >> 4) & 15, cc = e & 15;
      const int R = blk < 3 ? 0 : (blk < 5 ? 1 : 2);
      const int I = blk < 3 ? blk + 1 : (blk < 5 ? blk - 1 : 3);
      sLi[(16 * R + rr) * L::P_AF + 16 * I + cc] = 0.f;
    }
    if constexpr (CONVERT) {
      // Kl -> K_g = Kl Diag(gamma_mR), Ql -> Q_g in place (rows of block R),
      // one group of 8 channels at a time, while waves 0-3 invert.
      constexpr int G8 = DK / 8;
      for (int e = t - 64 * w0; e < 2 * kC * G8; e += NT - 64 * w0) {
        char* const base = e < kC * G8 ? sKl : sQl;
        const int e2 = e < kC * G8 ? e : e - kC * G8;
        const int r = e2 / G8, g8 = e2 - r * G8;
        const float* gm = sGM + (r >> 4) * DK + 8 * g8;
        float x[8];
        if constexpr (BF) {
          const char* src = base + r * L::P_OP + g8 * 32;
          const uint4 hi = *reinterpret_cast<const uint4*>(src);
          const uint4 lo = *reinterpret_cast<const uint4*>(src + 16);
          const uint32_t hw[4] = {hi.x, hi.y, hi.z, hi.w}, lw[4] = {lo.x, lo.y, lo.z, lo.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            x[2 * j] = (bf_lo16(hw[j]) + bf_lo16(lw[j])) * gm[2 * j];
            x[2 * j + 1] = (bf_hi16(hw[j]) + bf_hi16(lw[j])) * gm[2 * j + 1];
          }
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) x[j] = reinterpret_cast<const float*>(base + r * L::P_OP)[8 * g8 + j] * gm[j];
        }
        st8<BF>(base, L::P_OP, r, 8 * g8, x);
      }
    }
  }
  lds_barrier();
  // 3b: off-diagonal blocks row block by row block:
  //     L^-1_{R,I} = -D_R (sum_{I<=J<R} A_{R,J} L^-1_{J,I}),  wave I
  // (the sum, in the result layout, is directly the B operand of the
  // product with D_R).
#pragma unroll
  for (int R = 1; R < 4; ++R) {
    if (w < R) {
      const int I = w;
      f4 y = f4{0.f, 0.f, 0.f, 0.f};
      for (int J = I; J < R; ++J) {
        const float4 a4 = *reinterpret_cast<const float4*>(sA + (16 * R + lr) * L::P_AF + 16 * J + 4 * lg);
        const float* bb = sLi + (16 * J + 4 * lg) * L::P_AF + 16 * I + lr;
        const f4 a = f4{a4.x, a4.y, a4.z, a4.w};
        const f4 b = f4{bb[0], bb[L::P_AF], bb[2 * L::P_AF], bb[3 * L::P_AF]};
        y = mm16x16(a, b, y);
      }
      const float4 d4 = *reinterpret_cast<const float4*>(sLi + (16 * R + lr) * L::P_AF + 16 * R + 4 * lg);
      const f4 x = mm16x16(f4{d4.x, d4.y, d4.z, d4.w}, y, f4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int q = 0; q < 4; ++q) sLi[(16 * R + 4 * lg + q) * L::P_AF + 16 * I + lr] = -x[q];
    }
    lds_barrier();
  }
  // 3c: T = L^-1 Diag(beta), converted in place to the operand format
  // (an 8-element group of fp32 occupies exactly the bytes of its hi/lo form).
#pragma unroll
  for (int e = t; e < kC * 8; e += NT) {
    const int r = e >> 3, g8 = e & 7;
    float x[8];
    const float* src = sLi + r * L::P_AF + 8 * g8;
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = src[i] * sBe[8 * g8 + i];
    st8<BF>(sT, L::P_T, r, 8 * g8, x);
  }
  lds_barrier();
}

// ------------------------------------------------------------------ kernel --
// Store the state slab S[js][q] (rows 16w + 4lg + q, columns col0 + 16js + lr)
// as snapshot row `row` of head h.
template <int DK, int NSUB>
__device__ __forceinline__ void store_snapshot(float* snap, int64_t row, int h, int H, int DV, int col0,
                                               const f4 (&S)[NSUB]) {
  const int l = lane_id(), w = threadIdx.x >> 6;
  float* dst = snap + (row * H + h) * int64_t(DK) * DV + col0 + (l & 15);
#pragma unroll
  for (int js = 0; js < NSUB; ++js)
#pragma unroll
    for (int q = 0; q < 4; ++q) dst[uint32_t((16 * w + 4 * (l >> 4) + q) * DV + 16 * js)] = S[js][q];
}

// NOO: states and snapshots only (no output products; o is not written).
// Packed batches of up to this many sequences are taken longest first.
constexpr int kRankedSeqs = 256;

template <int DK, int NSUB, bool BF, bool SNAP, bool NOO>
__global__ __launch_bounds__(64 * (DK / 16), 1) void kda_prefill_kernel(Params p) {
  using L = Lay<DK>;
  constexpr int NW = L::NW;         // waves; wave w owns rows 16w..16w+15 of the state
  constexpr int VS = 16 * NSUB;     // value columns of this workgroup

  __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
  char* const sKl = smem + L::OFF_KL;
  char* const sQl = smem + L::OFF_QL;
  char* const sKrT = smem + L::OFF_KRT;
  char* const sP = smem + L::OFF_P;
  char* const sSBT = smem + L::OFF_SBT;
  char* const sXT = smem + L::OFF_XT;
  char* const sUT = smem + L::OFF_UT;
  char* const sT = smem + L::OFF_T;
  float* const sGN = reinterpret_cast<float*>(smem + L::OFF_GN);

  const int t = threadIdx.x;
  const int l = t & 63;
  const int w = t >> 6;
  const int lr = l & 15;   // fragment row / accumulator column
  const int lg = l >> 4;   // lane group

  // Workgroup -> (sequence, head, slab).  Workgroups are dispatched to the 8
  // XCDs round-robin; remap so that the slabs of one (sequence, head), which
  // read the same q/k/alpha, run on one XCD and share its L2.
  int64_t b = blockIdx.x;
  const int64_t G = gridDim.x;
  // The remap hands each XCD a contiguous range of sequences, so it is used
  // only when there are several slabs per head to share: with one slab,
  // a packed batch sorted by length would put its longest sequences on one
  // XCD and leave the others idle (1.6x slower than round-robin).
  if ((G & 7) == 0 && p.nslab > 1) b = (b & 7) * (G >> 3) + (b >> 3);
  const int slab = int(b % p.nslab);
  const int64_t pr = b / p.nslab;
  const int h = int(pr % p.H);
  int n = int(pr / p.H);
  // Packed sequences: the workgroups take the sequences longest first (the
  // n-th workgroup row gets the sequence of rank n by length, ties in pack
  // order), so that the longest chains start first and the short ones fill in
  // behind them, whatever the order of the pack.  The ranks are counted from
  // cu_seqlens staged in LDS (before the LDS takes anything else), up to
  // kRankedSeqs sequences; past that the pack order stands.
  if (p.cu != nullptr && p.N <= kRankedSeqs) {
    int* const sLen = reinterpret_cast<int*>(smem);
    int* const sPick = sLen + kRankedSeqs;
    for (int i = t; i < p.N; i += L::NT) sLen[i] = p.cu[i + 1] - p.cu[i];
    if (t == 0) *sPick = n;
    __syncthreads();
    for (int i = t; i < p.N; i += L::NT) {
      const int li = sLen[i];
      int rank = 0;
      for (int j = 0; j < p.N; ++j) rank += (sLen[j] > li || (sLen[j] == li && j < i)) ? 1 : 0;
      if (rank == n) *sPick = i;
    }
    __syncthreads();
    n = *sPick;
    __syncthreads();
  }
  const int H = p.H, DV = p.DV;
  const int col0 = slab * VS;

  int64_t s0, s1;
  int64_t snap_base = 0, snap_cnt = 0;   // varlen snapshot rows of sequence n
  if (SNAP && p.snap_off != nullptr) {
    snap_base = p.snap_off[n];
    snap_cnt = p.snap_off[n + 1] - snap_base;
  }
  if (p.cu != nullptr) {
    s0 = p.cu[n];
    s1 = p.cu[n + 1];
  } else {
    s0 = int64_t(n) * p.T_fixed;
    s1 = s0 + p.T_fixed;
  }

  // State slab in registers: S[js][q] = S[16w + 4lg + q][col0 + 16js + lr].
  f4 S[NSUB];
  const int64_t sbase = (int64_t(n) * H + h) * DK * DV;
#pragma unroll
  for (int js = 0; js < NSUB; ++js)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      S[js][q] = p.s_in ? p.s_in[sbase + int64_t(16 * w + 4 * lg + q) * DV + col0 + 16 * js + lr]
                        : 0.f;

  // Decay prep: thread = (channel quad, group of 4 rows).
  int cq, grp;
  quad_map<DK / 4>(t, cq, grp);
  const int c0 = 4 * cq, r0 = 4 * grp;

  // Raw inputs of the next chunk, loaded one chunk ahead.  Every load is
  // unconditional: rows past the sequence end are clamped to its last row
  // and their values discarded.
  typename Raw<BF>::four pk[4], pq[4];
  float4 pa[4];
  float pb = 0.f;
  typename Raw<BF>::one pv[NSUB][4];
  const int rsk = H * DK, rsv = H * DV;  // token strides (elements)
  constexpr int ESZ = BF ? 2 : 4;        // bytes per q/k/v element
  auto load_chunk = [&](int64_t tk0, int nvv) {
    // Wave-uniform base pointers for the chunk and 32-bit per-lane offsets
    // (scalar-base addressing: one vector add per load).
    const int64_t row0 = tk0 * H + h;
    const bool sg = p.alpha_scalar != 0;
    const float* ab = p.alpha + (sg ? row0 : row0 * DK);
    const char* kb = static_cast<const char*>(p.k) + row0 * DK * ESZ;
    const char* qb = static_cast<const char*>(p.q) + row0 * DK * ESZ;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = r0 + i < nvv ? r0 + i : nvv - 1;
      const uint32_t off = uint32_t(r * rsk + c0);
      // (a scalar gate stays in .x until the values are taken: a broadcast
      // here would make the wave wait for the load right away)
      if (sg) pa[i].x = ab[uint32_t(r * H)];
      else pa[i] = *reinterpret_cast<const float4*>(ab + off);
      pk[i] = ldraw4<BF>(kb, off);
      pq[i] = ldraw4<BF>(qb, off);
    }
    pb = p.beta[row0 + uint32_t(((t & 63) < nvv ? (t & 63) : nvv - 1) * H)];
    {
      // (waves 4.. load the rows of waves 0..3 again: keeps the loads unconditional)
      const char* vb = static_cast<const char*>(p.v) + (row0 * DV + col0) * ESZ;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int rv = 16 * (w & 3) + 4 * lg + q;
        const int r = rv < nvv ? rv : nvv - 1;
#pragma unroll
        for (int js = 0; js < NSUB; ++js) pv[js][q] = ldraw1<BF>(vb, uint32_t(r * rsv + 16 * js + lr));
      }
    }
  };
  if (s0 < s1) load_chunk(s0, int(s1 - s0 < kC ? s1 - s0 : kC));
  // Mirror the output stores that follow the prefetch in every later chunk,
  // so that the first chunk and the steady state agree on how many memory
  // operations are in flight after the prefetched loads (otherwise the
  // compiler's wait for them degrades to waiting for every store).  Plain
  // stores to distinct addresses: volatile ones would each be followed by a
  // wait for every memory operation in flight, the prefetch included.
  mirror_stores<4 * NSUB>();

  for (int64_t tok0 = s0; tok0 < s1; tok0 += kC) {
    const int nv = int(s1 - tok0 < kC ? s1 - tok0 : kC);

    // ---- take this chunk's inputs, start loading the next chunk's --------
    float4 av[4], kv[4], qv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = r0 + i < nv;
      const float4 ai = p.alpha_scalar ? make_float4(pa[i].x, pa[i].x, pa[i].x, pa[i].x) : pa[i];
      av[i] = ok ? ai : make_float4(1.f, 1.f, 1.f, 1.f);
      const float4 kk = cvt4<BF>(pk[i]), qq = cvt4<BF>(pq[i]);
      kv[i] = ok ? kk : make_float4(0.f, 0.f, 0.f, 0.f);
      qv[i] = ok ? qq : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const float bev = (t & 63) < nv ? pb : 0.f;
    float vreg[NSUB][4];
#pragma unroll
    for (int js = 0; js < NSUB; ++js)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        vreg[js][q] = (16 * (w & 3) + 4 * lg + q) < nv ? cvt1<BF>(pv[js][q]) : 0.f;
    if (tok0 + kC < s1) load_chunk(tok0 + kC, int(s1 - tok0 - kC < kC ? s1 - tok0 - kC : kC));

    prep_chunk<DK, BF, true>(smem, av, kv, qv, bev, [] {});

    // ---- step 4: the state pass, 16 value columns at a time ----------------
    // Waves 0..3 compute X and U for rows 16w..; the output rows 16*ow.. are
    // computed by waves 4..7 when there are eight waves (their Q_g S product
    // overlaps X and U), else by waves 0..3 after U.
    constexpr bool kSplitO = NW >= 8;
    const bool xw = w < 4;
    const bool owave = NOO ? false : (kSplitO ? (w >= 4) : (w < 4));
    const int ow = w & 3;
#pragma unroll
    for (int js = 0; js < NSUB; ++js) {
      // 4a: S^T for these columns.
      {
        const int kr = 16 * w + 4 * lg;
        const float x[4] = {S[js][0], S[js][1], S[js][2], S[js][3]};
        st4<BF>(sSBT, L::P_OP, lr, kr, x);
      }
      lds_barrier();
      // 4b: X = V - K_g S; the output waves start O = Q_g S.
      f4 acco = f4{0.f, 0.f, 0.f, 0.f};
      if (xw) {
        f4 acc = gemm<BF, DK>(f4{0.f, 0.f, 0.f, 0.f}, sKl, L::P_OP, 16 * w, sSBT, L::P_OP, 0);
        float x[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) x[q] = vreg[js][q] - acc[q];
        st4<BF>(sXT, L::P_T, lr, 16 * w + 4 * lg, x);
      }
      if (kSplitO && owave)
        acco = gemm<BF, DK>(acco, sQl, L::P_OP, 16 * ow, sSBT, L::P_OP, 0);
      lds_barrier();
      // 4c: U = T X  (T is lower triangular: K up to the end of this row block)
      if (xw) {
        f4 acc = gemm<BF, kC>(f4{0.f, 0.f, 0.f, 0.f}, sT, L::P_T, 16 * w, sXT, L::P_T, 0);
        float x[4] = {acc[0], acc[1], acc[2], acc[3]};
        st4<BF>(sUT, L::P_T, lr, 16 * w + 4 * lg, x);
      }
      lds_barrier();
      // 4d: O = Q_g S + P U
      if (owave) {
        if constexpr (!kSplitO)
          acco = gemm<BF, DK>(acco, sQl, L::P_OP, 16 * ow, sSBT, L::P_OP, 0);
        acco = gemm<BF, kC>(acco, sP, L::P_T, 16 * ow, sUT, L::P_T, 0);
      }
      {
        // Every wave issues the stores; rows past the end of the sequence and
        // waves without output rows store into a sink.  Unconditional stores
        // stay visible to the compiler's memory-counter bookkeeping, so taking
        // the prefetched inputs never waits for output stores to drain.
        float* ob = p.o + (tok0 * H + h) * int64_t(DV) + col0 + 16 * js;  // uniform
        float* sink = g_kda_sink + (blockIdx.x & 255) * (kSinkStores * 64) + l;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = 16 * ow + 4 * lg + q;
          float* dst = owave && r < nv ? ob + uint32_t(r * rsv + lr) : sink;
          *dst = acco[q];
        }
      }
      // 4e: S' = Diag(gamma_n) S + K_e^T U  (rows 16w..)
      {
        f4 acc = gemm<BF, kC>(f4{0.f, 0.f, 0.f, 0.f}, sKrT, L::P_T, 16 * w, sUT, L::P_T, 0);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = 16 * w + 4 * lg + q;
          S[js][q] = sGN[c] * S[js][q] + acc[q];
        }
      }
      // With 8 waves the next column block rewrites S^T, X^T and U^T only
      // after barriers that every wave reaches after its reads of them here
      // (S^T is last read in 4b).  With 4 waves S^T is read in 4d, and the
      // next chunk's steps 1-3 overwrite everything: barrier.
      if (js == NSUB - 1 || !kSplitO) lds_barrier();
    }
    if constexpr (SNAP) {
      // State after a complete interval of snap_every full chunks.
      const int64_t done = (tok0 - s0) / kC + 1;
      if (nv == kC && done % p.snap_every == 0) {
        const int64_t j = done / p.snap_every - 1;
        if (p.snap_off == nullptr && p.cu == nullptr) {
          store_snapshot<DK, NSUB>(p.snap, n * p.snap_per_seq + j, h, H, DV, col0, S);
        } else if (p.snap_off == nullptr) {
          // packed sequences without offsets: chunk j of the sequence starting
          // at token s0 goes to row s0 / 64 + j (rows of consecutive sequences
          // never meet, and all are below T_total / 64)
          if (s0 / kC + j < p.snap_rows) store_snapshot<DK, NSUB>(p.snap, s0 / kC + j, h, H, DV, col0, S);
        } else if (j < snap_cnt && snap_base + j >= 0 && snap_base + j < p.snap_rows) {
          store_snapshot<DK, NSUB>(p.snap, snap_base + j, h, H, DV, col0, S);
        }
      }
    }
  }

  if (p.s_out) {
#pragma unroll
    for (int js = 0; js < NSUB; ++js)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        p.s_out[sbase + int64_t(16 * w + 4 * lg + q) * DV + col0 + 16 * js + lr] = S[js][q];
  }
}


// ==================================================================== staged ==
// Staged form for workloads with few (sequence, head) chains.  The fused
// kernel above repeats steps 1-3 in every value slab of a chain; here they run
// once per chunk, for all chunks at once (kda_stage_kernel), together with the
// state-independent parts of steps 4b-4e folded into four matrices:
//     W  = T K_g                  [64 x DK]    so that  U = Uv - W S
//     Uv = T V                    [64 x DV]
//     Qg = Q_g                    [64 x DK]    so that  O = Qg S + P U
//     Kg = K_e^T                  [DK x 64]    so that  S' = Diag(gamma_n) S + Kg U
// The sequential pass (kda_chain_kernel) then
// streams them from a workspace straight into MFMA registers: two dependent
// products and two barriers per chunk.
//
// Workspace slot of one (chunk, sequence, head), "fragment order": every
// matrix is stored as the MFMA A-operand fragments of its 16-row blocks, in
// the order a wave loads them, so that each load instruction reads 1 KiB of
// consecutive bytes.
//   split bf16: fragment (rb, kc) covers rows 16rb.., K 32kc.. and takes
//     2 KiB: lane l's 8 hi parts at 16l, its 8 lo parts at 1024 + 16l (lane l:
//     row 16rb + l%16, K 32kc + 8(l/16) + e).
//   fp32: unit (rb, g) covers rows 16rb.., K 16g.. and takes 1 KiB: lane l
//     holds 4 floats, fragment kc = 4g + i at row 16rb + l%16, K 4kc + l/16.
// Uv is stored as MFMA result tiles (rb, 16-column block): 1 KiB, lane l's 4
// floats (rows 16rb + 4(l/16) + q, column l%16) at 16l.  gamma_n last.
template <int DK, int DV>
struct Slot {
  static constexpr int OFF_W = 0;
  static constexpr int OFF_Q = OFF_W + 64 * DK * 4;
  static constexpr int OFF_K = OFF_Q + 64 * DK * 4;
  static constexpr int OFF_P = OFF_K + DK * 64 * 4;
  static constexpr int OFF_U = OFF_P + 64 * 64 * 4;
  static constexpr int OFF_G = OFF_U + 64 * DV * 4;
  static constexpr int BYTES = OFF_G + DK * 4;
  static_assert(BYTES % 256 == 0, "slot alignment");
};

struct StageParams {
  int H, DV, nslab;
  int64_t T_fixed;   // tokens per sequence
  int64_t pairs;     // sequences x heads
  int64_t c_begin;   // first chunk (of every sequence) of this segment
  int64_t nseg;      // chunks per sequence in this segment
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;
  const float* s_in;
  float* o;
  float* s_out;
  char* ws;          // slot of item i = (c - c_begin) * pairs + pair
  float* snap;       // state snapshots [N][snap_per_seq][H][DK][DV] (SNAP chain kernels)
  int snap_every;
  int64_t snap_per_seq;
  int alpha_scalar;  // alpha is [tokens][H]
  int states_only;   // o is not written (NOO kernels)
};

template <bool BF> struct FL;
template <> struct FL<true> {
  static constexpr int KU = 32;       // K per fragment
  static constexpr int UNIT = 2048;   // bytes per fragment
  // Fragments kc < n of a row block (n wave-uniform; the rest untouched).
  template <int NKC>
  __device__ static void load(Mma<true>::Frag (&f)[NKC], const char* rb, int n = NKC) {
    const int l = lane_id();
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      if (kc < n) {
        f[kc].hi = *reinterpret_cast<const bf8*>(rb + kc * 2048 + 16 * l);
        f[kc].lo = *reinterpret_cast<const bf8*>(rb + kc * 2048 + 1024 + 16 * l);
      }
    }
  }
};
template <> struct FL<false> {
  static constexpr int KU = 16;       // K per 1 KiB unit (four fragments)
  static constexpr int UNIT = 1024;
  template <int NKC>
  __device__ static void load(float (&f)[NKC], const char* rb, int n = NKC) {
    static_assert(NKC % 4 == 0, "fp32 fragments come in fours");
    const int l = lane_id();
#pragma unroll
    for (int g = 0; g < NKC / 4; ++g) {
      if (4 * g >= n) continue;
      const float4 x = *reinterpret_cast<const float4*>(rb + g * 1024 + 16 * l);
      f[4 * g] = x.x;
      f[4 * g + 1] = x.y;
      f[4 * g + 2] = x.z;
      f[4 * g + 3] = x.w;
    }
  }
};

// Writes an LDS operand array (ROWS x K, layout of the operand arrays above)
// to global memory in fragment order, each element times rs[row] (RS) and
// cs[k] (CS; cs[rb * K + k] for the rows of 16-row block rb with CS_RB).  The
// fragments are dealt out to the waves round-robin; every wave writes the
// same number.
template <bool BF, int K, int ROWS, int NW, bool RS, bool CS, bool CS_RB = false>
__device__ __forceinline__ void export_frags(char* dst, const char* src, int pitch, const float* rs,
                                             const float* cs_all) {
  using F = FL<BF>;
  constexpr int NU = K / F::KU;                 // units per row block
  constexpr int NF = (ROWS / 16) * NU;
  static_assert(NF % NW == 0, "equal share per wave");
  const int l = lane_id(), w = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < NF / NW; ++i) {
    const int f = w + NW * i;
    const int rb = f / NU, u = f - rb * NU;
    const int row = 16 * rb + (l & 15);
    const float r = RS ? rs[row] : 1.f;
    const float* cs = CS_RB ? cs_all + rb * K : cs_all;
    if constexpr (BF) {
      const char* s = src + row * pitch + (u * 4 + (l >> 4)) * 32;
      uint4 hi = *reinterpret_cast<const uint4*>(s);
      uint4 lo = *reinterpret_cast<const uint4*>(s + 16);
      if constexpr (RS || CS) {
        const int k0 = u * 32 + 8 * (l >> 4);
        const uint32_t hw[4] = {hi.x, hi.y, hi.z, hi.w}, lw[4] = {lo.x, lo.y, lo.z, lo.w};
        uint32_t nh[4], nl[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float x0 = bf_lo16(hw[j]) + bf_lo16(lw[j]);
          float x1 = bf_hi16(hw[j]) + bf_hi16(lw[j]);
          x0 *= r * (CS ? cs[k0 + 2 * j] : 1.f);
          x1 *= r * (CS ? cs[k0 + 2 * j + 1] : 1.f);
          split2(x0, x1, nh[j], nl[j]);
        }
        hi = make_uint4(nh[0], nh[1], nh[2], nh[3]);
        lo = make_uint4(nl[0], nl[1], nl[2], nl[3]);
      }
      *reinterpret_cast<uint4*>(dst + f * 2048 + 16 * l) = hi;
      *reinterpret_cast<uint4*>(dst + f * 2048 + 1024 + 16 * l) = lo;
    } else {
      float x[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k = (4 * u + j) * 4 + (l >> 4);
        x[j] = *reinterpret_cast<const float*>(src + row * pitch + 4 * k) * r * (CS ? cs[k] : 1.f);
      }
      *reinterpret_cast<float4*>(dst + f * 1024 + 16 * l) = make_float4(x[0], x[1], x[2], x[3]);
    }
  }
}

// Steps 1-3 and the folded products for every (chunk, sequence, head) of a
// segment.  Persistent: workgroup b takes items b, b + G, ...; the raw inputs
// of its next item are loaded while it works on the current one.
// NOO: the call needs the states only, so Q_g and P (used by o alone) are not
// stored.
template <int DK, int DV, bool BF, bool NOO>
__global__ __launch_bounds__(64 * (DK / 16), 1) void kda_stage_kernel(StageParams p) {
  using L = Lay<DK>;
  using SL = Slot<DK, DV>;
  using M = Mma<BF>;
  constexpr int NW = L::NW;
  // V is loaded straight in MFMA operand layout, one unit per (16-row block,
  // 32 (fp32: 16) columns): lane (lr, lg) holds row 16rb + lr, columns
  // 32kc + 8lg .. +7 (fp32: 16cb + 4lg .. +3).
  constexpr int NUV = 4 * (BF ? DV / 32 : DV / 16);
  static_assert(NUV % NW == 0, "V units per wave");
  constexpr int UV = NUV / NW;
  constexpr int KCC = kC / M::KU;
  constexpr int ESZ = BF ? 2 : 4;
  __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
  static_assert(DV * L::P_T <= L::SZ_X, "V^T fits the A/P space");

  const int t = threadIdx.x;
  const int l = t & 63;
  const int w = t >> 6;
  const int lr = l & 15, lg = l >> 4;
  const int H = p.H;
  const int64_t items = p.nseg * p.pairs;

  int cq, grp;
  quad_map<DK / 4>(t, cq, grp);
  const int c0 = 4 * cq, r0 = 4 * grp;       // prep: channels c0.., rows r0..
  typename Raw<BF>::four pk[4], pq[4];
  uint4 pv[UV];
  float4 pa[4];
  float pb = 0.f;
  // V of item `it`: loaded after steps 1-3 (it is first needed by the folded
  // products; keeping it in registers through steps 1-3 would spill).
  // Item it = (chunk c_begin + it / pairs, pair it % pairs); items < 2^31 (the
  // host checks), so the index arithmetic is 32-bit.
  const uint32_t npairs = uint32_t(p.pairs), uH = uint32_t(H);
  auto item_of = [&](int64_t it, int64_t& c, int& h, int64_t& n) {
    const uint32_t cr = uint32_t(it) / npairs;
    const uint32_t pr = uint32_t(it) - cr * npairs;
    const uint32_t nn = pr / uH;
    c = p.c_begin + cr;
    h = int(pr - nn * uH);
    n = nn;
  };
  auto load_v = [&](int64_t it) {
    int64_t c, n;
    int h;
    item_of(it, c, h, n);
    const int64_t tok0 = n * p.T_fixed + c * kC;
    const int64_t rem = p.T_fixed - c * kC;
    const int nvv = int(rem < kC ? rem : kC);
    const char* vb = static_cast<const char*>(p.v) + (tok0 * H + h) * DV * ESZ;
    const int rsv = H * DV;
#pragma unroll
    for (int i = 0; i < UV; ++i) {
      const int u = w + NW * i, rb = u & 3, cu = u >> 2;
      const int r0v = 16 * rb + lr;
      const int r = r0v < nvv ? r0v : nvv - 1;
      const int col = BF ? 32 * cu + 8 * lg : 16 * cu + 4 * lg;
      pv[i] = *reinterpret_cast<const uint4*>(vb + uint32_t(r * rsv + col) * ESZ);
    }
  };
  auto load_item = [&](int64_t it) {
    int64_t c, n;
    int h;
    item_of(it, c, h, n);
    const int64_t tok0 = n * p.T_fixed + c * kC;
    const int64_t rem = p.T_fixed - c * kC;
    const int nvv = int(rem < kC ? rem : kC);
    const int64_t row0 = tok0 * H + h;
    const bool sg = p.alpha_scalar != 0;
    const float* ab = p.alpha + (sg ? row0 : row0 * DK);
    const char* kb = static_cast<const char*>(p.k) + row0 * DK * ESZ;
    const char* qb = static_cast<const char*>(p.q) + row0 * DK * ESZ;
    const int rsk = H * DK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = r0 + i < nvv ? r0 + i : nvv - 1;
      const uint32_t off = uint32_t(r * rsk + c0);
      // (a scalar gate stays in .x until the values are taken: a broadcast
      // here would make the wave wait for the load right away)
      if (sg) pa[i].x = ab[uint32_t(r * H)];
      else pa[i] = *reinterpret_cast<const float4*>(ab + off);
      pk[i] = ldraw4<BF>(kb, off);
      pq[i] = ldraw4<BF>(qb, off);
    }
    pb = p.beta[row0 + uint32_t((l < nvv ? l : nvv - 1) * H)];
  };

  if (int64_t(blockIdx.x) < items) load_item(blockIdx.x);
  {
    // Every item's slot stores follow the prefetch of the next item's inputs.
    // The same number of stores, mirrored before the first item, keeps the
    // compiler's memory-counter waits for the prefetched inputs from also
    // waiting for the previous item's slot stores.
    using F = FL<BF>;
    constexpr int SPF = BF ? 2 : 1;                    // stores per fragment
    constexpr int NQ = 4 * (DK / F::KU) / NW;          // Qg and W fragments per wave
    constexpr int NK = (DK / 16) * (kC / F::KU) / NW;  // Kg
    constexpr int NP = 4 * (kC / F::KU) / NW;          // P
    constexpr int NBU = (DV / 16) * 4 / NW;            // Uv tiles
    mirror_stores<(2 * NQ + NK + NP) * SPF + 1 + NBU>();
  }
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int64_t c = p.c_begin + uint32_t(it) / npairs;
    const int64_t rem = p.T_fixed - c * kC;
    const int nv = int(rem < kC ? rem : kC);

    float4 av[4], kv[4], qv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = r0 + i < nv;
      const float4 ai = p.alpha_scalar ? make_float4(pa[i].x, pa[i].x, pa[i].x, pa[i].x) : pa[i];
      av[i] = ok ? ai : make_float4(1.f, 1.f, 1.f, 1.f);
      const float4 kk = cvt4<BF>(pk[i]), qq = cvt4<BF>(pq[i]);
      kv[i] = ok ? kk : make_float4(0.f, 0.f, 0.f, 0.f);
      qv[i] = ok ? qq : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const float bev = l < nv ? pb : 0.f;

    // The next item's raw inputs and this item's V are requested between
    // steps 2 and 3: behind this item's computation, not behind the previous
    // item's slot stores.
    prep_chunk<DK, BF, false>(smem, av, kv, qv, bev, [&] {
      load_v(it);
      if (it + gridDim.x < items) load_item(it + gridDim.x);
    });

    char* slot = p.ws + it * int64_t(SL::BYTES);
    const float* sGM = reinterpret_cast<const float*>(smem + L::OFF_GM);
    const float* sGN = reinterpret_cast<const float*>(smem + L::OFF_GN);

    // F1: Qg = Q_g (Ql Diag(gamma_mR) per row block R), Kg = K_e^T (scaled in
    // step 2), P, gamma_n.
    if constexpr (!NOO)
      export_frags<BF, DK, kC, NW, false, true, true>(slot + SL::OFF_Q, smem + L::OFF_QL, L::P_OP, nullptr, sGM);
    export_frags<BF, kC, DK, NW, false, false>(slot + SL::OFF_K, smem + L::OFF_KRT, L::P_T, nullptr, nullptr);
    if constexpr (!NOO)
      export_frags<BF, kC, kC, NW, false, false>(slot + SL::OFF_P, smem + L::OFF_P, L::P_T, nullptr, nullptr);
    reinterpret_cast<float*>(slot + SL::OFF_G)[t % DK] = sGN[t % DK];
    lds_barrier();

    // F2: K_g^T (Kl Diag(gamma_mR) per row block R) into the Kr^T space, V^T
    // into the A/P space.
    char* const sKgT = smem + L::OFF_KRT;
    char* const sVT = smem + L::OFF_X;
    xpose_lds<BF, DK, NW, true>(smem + L::OFF_KL, L::P_OP, sGM, sKgT, L::P_T);
#pragma unroll
    for (int i = 0; i < UV; ++i) {
      const int u = w + NW * i, rb = u & 3, cu = u >> 2;
      const uint4 x = 16 * rb + lr < nv ? pv[i] : make_uint4(0u, 0u, 0u, 0u);
      if constexpr (BF) {
        Mma<true>::Frag a;
        a.hi = __builtin_bit_cast(bf8, x);
        a.lo = __builtin_bit_cast(bf8, make_uint4(0u, 0u, 0u, 0u));
        xpose32_bf<true>(a, rb, cu, 1.f, 1.f, sVT, L::P_T);
      } else {
        const float a4[4] = {__uint_as_float(x.x), __uint_as_float(x.y), __uint_as_float(x.z),
                             __uint_as_float(x.w)};
        xpose16_f32(a4, rb, cu, 1.f, sVT, L::P_T);
      }
    }
    lds_barrier();

    // F3: W = T K_g into a staging array (the Ql space);
    // Uv = T V straight to the slot.  Wave w takes row block rb of T (rb = w
    // for waves 0-3, 3 - (w - 4) for waves 4-7, so that the two waves of a
    // SIMD together cover 3 of the 4 nonzero K blocks of the lower-triangular
    // T) and skips the K chunks above the diagonal.
    char* const sW = smem + L::OFF_QL;
    {
      const int rb = w < 4 ? w : 3 - (w & 3);
      const int kmax = 16 * rb + 16;   // K (tokens) past which T's row block is zero
      typename M::Frag ta[KCC];
#pragma unroll
      for (int kc = 0; kc < KCC; ++kc) ta[kc] = M::load(smem + L::OFF_T, L::P_T, 16 * rb, kc);
      constexpr int NBW = (DK / 16) * 4 / NW;   // column blocks of W per wave
      constexpr int NBU = (DV / 16) * 4 / NW;   // column blocks of Uv per wave
#pragma unroll
      for (int i = 0; i < NBW; ++i) {
        const int nb = NBW * (w >> 2) + i;
        // W^T tile: lane (lr, lg) holds W[16rb + lr][16nb + 4lg .. +3]
        f4 acc = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < KCC; ++kc)
          if (kc * M::KU < kmax) acc = M::mma(M::load(sKgT, L::P_T, 16 * nb, kc), ta[kc], acc);
        const float x[4] = {acc[0], acc[1], acc[2], acc[3]};
        st4<BF>(sW, L::P_OP, 16 * rb + lr, 16 * nb + 4 * lg, x);
      }
#pragma unroll
      for (int i = 0; i < NBU; ++i) {
        const int nb = NBU * (w >> 2) + i;
        f4 acc = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < KCC; ++kc)
          if (kc * M::KU < kmax) acc = M::mma(ta[kc], M::load(sVT, L::P_T, 16 * nb, kc), acc);
        *reinterpret_cast<f4*>(slot + SL::OFF_U + (rb * (DV / 16) + nb) * 1024 + 16 * l) = acc;
      }
    }
    lds_barrier();

    // F4: W to the slot.
    export_frags<BF, DK, kC, NW, false, false>(slot + SL::OFF_W, sW, L::P_OP, nullptr, nullptr);
    lds_barrier();
  }
}

// ------------------------------------------------ stage kernel, d = 128 ----
// The slots of kda_stage_kernel for d_k = d_v = 128 with bf16 inputs, from a
// workgroup of eight waves in 79.6 KB of LDS and at most 128 VGPRs, one
// workgroup per item: two workgroups share a compute unit, four waves per
// SIMD, so one item's barriers and memory latency are covered by the other
// item's work (measured: the B=1, H=32, T=8192 prefill in 415 us against
// 451 us with the one-workgroup-per-CU kernel).  What makes it fit: the
// decayed operands Kl, Ql and Kr go through the LDS one half of the key
// channels at a time (the Gram tiles accumulate over the halves in
// registers; Q_g and K_e^T are exported per half), and after the solve K_g
// is rebuilt per half from the keys and decays the threads keep in
// registers.  Without a loop over items (and so without a prefetch of the
// next one) the compiler keeps nothing in registers across items, which
// holds the register count under 128 without spills.
//
// Decay prep: thread t takes half ht = t / 256 of the key channels, its
// channel quad cq = t % 16 and rows 4 g4 .. 4 g4 + 3, g4 = (t / 16) % 16; the
// two threads of an 8-row group (rows 8G .. 8G + 7) are lanes l and l ^ 16
// of one wave.  The reference row of block R, 16R + 7, is the last row of
// group 2R, so every per-block vector is a product of whole 8-row groups.
struct Lay2 {
  static constexpr int NT = 512;
  static constexpr int P_H = 64 * 4 + 16;   // rows of 64 elements (272 B)
  static constexpr int P_AF = 68;           // fp32 pitch of A and L^-1 (floats)
  static constexpr int ARR = 64 * P_H;      // one 64 x 64 array
  static constexpr int OFF_O0 = 0;          // Kl_h; A; K_g_h / W staging / K_g^T / V^T
  static constexpr int OFF_O1 = ARR;        // Ql_h; P; K_g^T / W staging / V^T
  static constexpr int OFF_O2 = 2 * ARR;    // Kr_h; L^-1 then T
  static constexpr int OFF_XS = 3 * ARR;    // K_e^T of a half
  static constexpr int OFF_GM = 4 * ARR;    // gamma_mR [4][128]
  static constexpr int OFF_GN = OFF_GM + 4 * 128 * 4;    // gamma_n [128]
  static constexpr int OFF_GNM = OFF_GN + 128 * 4;       // gamma_n / gamma_mI [4][128]
  static constexpr int OFF_S1 = OFF_GNM + 4 * 128 * 4;   // S1_I [4][128]
  static constexpr int OFF_E = OFF_S1 + 4 * 128 * 4;     // E_RI [6][128]
  static constexpr int OFF_BE = OFF_E + 6 * 128 * 4;     // beta [64]
  static constexpr int OFF_GP = OFF_O0;                  // 8-row group products [8][128] (steps 1-2)
  static constexpr int TOTAL = OFF_BE + 64 * 4;
  static_assert(2 * TOTAL <= 160 * 1024, "two workgroups per compute unit");
  static_assert(ARR == 64 * P_AF * 4, "A and L^-1 fill one array");
};

// acc += the Gram tiles of block pair (R, I) over one half of the key
// channels (K = 64, two 32-channel fragments); the half's operands are
// [64][64] arrays of pitch Lay2::P_H, and s1 / e point at the half's
// channels of S1_I and E_RI.
template <int R, int I, int XD>
__device__ __forceinline__ void gram_group_half(const char* sKl, const char* sQl, const char* sKr,
                                                const float* s1, const float* e, f4 (&acc)[3]) {
  using M = Mma<true>;
  constexpr int P = Lay2::P_H;
#pragma unroll 1
  for (int kc = 0; kc < 2; ++kc) {
    auto c = M::load(sKr, P, 16 * I, kc);
    if constexpr (I < R) c = rescale_frag(c, s1, e, kc);
    const auto rk = M::load(sKl, P, 16 * R, kc);
    const auto rq = M::load(sQl, P, 16 * R, kc);
    acc[0] = M::mma(c, rk, acc[0]);
    acc[1] = M::mma(c, rq, acc[1]);
    if constexpr (XD >= 0) {
      const auto cd = M::load(sKr, P, 16 * R, kc);
      acc[2] = M::mma(cd, XD == 0 ? rk : rq, acc[2]);
    }
  }
}

// One fragment (16 rows, 32 K) of a [rows][64] split-bf16 LDS array (pitch
// Lay2::P_H) to global memory in fragment order, each element times
// cs[row block][k] when cs is given (row stride 128 floats).
__device__ __forceinline__ void export_frag_half(char* dst, const char* src, int rb, int u, const float* cs) {
  const int l = lane_id();
  const int row = 16 * rb + (l & 15);
  const char* s = src + row * Lay2::P_H + (u * 4 + (l >> 4)) * 32;
  uint4 hi = *reinterpret_cast<const uint4*>(s);
  uint4 lo = *reinterpret_cast<const uint4*>(s + 16);
  if (cs != nullptr) {
    const float* c = cs + rb * 128 + u * 32 + 8 * (l >> 4);
    const uint32_t hw[4] = {hi.x, hi.y, hi.z, hi.w}, lw[4] = {lo.x, lo.y, lo.z, lo.w};
    uint32_t nh[4], nl[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float x0 = (bf_lo16(hw[j]) + bf_lo16(lw[j])) * c[2 * j];
      const float x1 = (bf_hi16(hw[j]) + bf_hi16(lw[j])) * c[2 * j + 1];
      split2(x0, x1, nh[j], nl[j]);
    }
    hi = make_uint4(nh[0], nh[1], nh[2], nh[3]);
    lo = make_uint4(nl[0], nl[1], nl[2], nl[3]);
  }
  *reinterpret_cast<uint4*>(dst + 16 * l) = hi;
  *reinterpret_cast<uint4*>(dst + 1024 + 16 * l) = lo;
}

// NOO: the call needs the states only (Q_g and P are not stored).  SG: one
// gate per token and head (alpha is [tokens][H]); a template parameter, so
// that the input loads are straight-line code: a run-time branch around each
// alpha load made the compiler wait for every row's loads before issuing the
// next row's.
template <bool NOO, bool SG>
__global__ __launch_bounds__(Lay2::NT, 4) void kda_stage2_kernel(StageParams p) {
  using L = Lay2;
  using M = Mma<true>;
  using SL = Slot<128, 128>;
  constexpr int DK = 128, DV = 128;
  __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
  char* const sO0 = smem + L::OFF_O0;
  char* const sO1 = smem + L::OFF_O1;
  char* const sO2 = smem + L::OFF_O2;
  char* const sXS = smem + L::OFF_XS;
  float* const sGP = reinterpret_cast<float*>(smem + L::OFF_GP);
  float* const sGM = reinterpret_cast<float*>(smem + L::OFF_GM);
  float* const sGN = reinterpret_cast<float*>(smem + L::OFF_GN);
  float* const sGNM = reinterpret_cast<float*>(smem + L::OFF_GNM);
  float* const sS1 = reinterpret_cast<float*>(smem + L::OFF_S1);
  float* const sE = reinterpret_cast<float*>(smem + L::OFF_E);
  float* const sBe = reinterpret_cast<float*>(smem + L::OFF_BE);
  float* const sA = reinterpret_cast<float*>(sO0);
  char* const sP = sO1;
  char* const sT = sO2;
  float* const sLi = reinterpret_cast<float*>(sO2);

  const int t = threadIdx.x;
  const int l = t & 63;
  const int w = t >> 6;
  const int lr = l & 15, lg = l >> 4;
  // decay prep: half ht of the key channels (waves 4ht .. 4ht + 3), channel
  // quad cq of the half, rows 4 g4 .. 4 g4 + 3
  const int ht = t >> 8, cq = t & 15, g4 = (t >> 4) & 15;
  const int r0 = 4 * g4;
  const int pos = g4 & 3;   // place of the thread's 4 rows in their 16-row block
  const int wr = w & 3;     // row block of T for the folded products
  const int H = p.H;
  const int64_t items = p.nseg * p.pairs;
  const uint32_t npairs = uint32_t(p.pairs), uH = uint32_t(H);
  auto mul4 = [](float4 a, float4 b) { return make_float4(a.x * b.x, a.y * b.y, a.z * b.z, a.w * b.w); };
  const float4 one4 = make_float4(1.f, 1.f, 1.f, 1.f);
  auto rcp4 = [](float4 a) { return make_float4(rcp(a.x), rcp(a.y), rcp(a.z), rcp(a.w)); };
  auto shfl4 = [](float4 a) {
    return make_float4(__shfl_xor(a.x, 16), __shfl_xor(a.y, 16), __shfl_xor(a.z, 16), __shfl_xor(a.w, 16));
  };

  {
    const int64_t it = blockIdx.x;
    if (it >= items) return;
    const uint32_t crel = uint32_t(it) / npairs;
    const uint32_t pr = uint32_t(it) - crel * npairs;
    const uint32_t nn = pr / uH;
    const int h = int(pr - nn * uH);
    const int64_t c = p.c_begin + crel;
    const int64_t tok0 = int64_t(nn) * p.T_fixed + c * kC;
    const int64_t rem = p.T_fixed - c * kC;
    const int nv = int(rem < kC ? rem : kC);
    const int64_t row0 = tok0 * H + h;
    const int rsk = H * DK, rsv = H * DV;
    char* const slot = p.ws + it * int64_t(SL::BYTES);

    // ---- inputs (rows past the end: alpha = 1, k = q = 0) -----------------
    // All loads are issued first, the alphas (needed first) ahead of k and q,
    // then the rows past the end are masked.
    const float* ab = p.alpha + (SG ? row0 : row0 * DK);
    const char* kb = static_cast<const char*>(p.k) + row0 * DK * 2;
    const char* qb = static_cast<const char*>(p.q) + row0 * DK * 2;
    uint2 kraw[4], qraw[4];
    float4 av[4];
    uint32_t roff[4];
    // (beta first: it is stored to LDS before the barrier that the alphas
    // need, and loads complete in order)
    const float bev = p.beta[row0 + uint32_t((t & 63) < nv ? (t & 63) : nv - 1) * H];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = r0 + i < nv ? r0 + i : nv - 1;
      roff[i] = uint32_t(r * rsk + 64 * ht + 4 * cq);
      if constexpr (SG) av[i].x = ab[uint32_t(r * H)];
      else av[i] = *reinterpret_cast<const float4*>(ab + roff[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kraw[i] = ldraw4<true>(kb, roff[i]);
      qraw[i] = ldraw4<true>(qb, roff[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (SG) av[i] = make_float4(av[i].x, av[i].x, av[i].x, av[i].x);
      if (r0 + i >= nv) {
        av[i] = one4;
        kraw[i] = make_uint2(0u, 0u);
        qraw[i] = make_uint2(0u, 0u);
      }
    }
    if (t < kC) sBe[t] = t < nv ? bev : 0.f;

    // ---- step 1: 8-row group products, then the decays of the own rows ----
    const float4 own = mul4(mul4(av[0], av[1]), mul4(av[2], av[3]));
    const float4 par = shfl4(own);   // the other 4 rows of the 8-row group
    if ((g4 & 1) == 0) *reinterpret_cast<float4*>(sGP + (g4 >> 1) * DK + 64 * ht + 4 * cq) = mul4(own, par);
    lds_barrier();
    // rho_r = gamma_r / gamma_(16R+7), the decay of row r relative to its
    // block's reference row, kept as the exact product ex: 1/rho for the rows
    // up to the reference (prod_{r < s <= 16R+7} alpha_s), rho after it
    // (prod_{16R+7 < s <= r} alpha_s); the other one is its reciprocal.
    float4 ex[4];
    const bool before = pos < 2;
    if (before) {
      float4 Q = pos == 0 ? par : one4;
#pragma unroll
      for (int i = 3; i >= 0; --i) {
        ex[i] = Q;
        Q = mul4(Q, av[i]);
      }
    } else {
      float4 P = pos == 3 ? par : one4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        P = mul4(P, av[i]);
        ex[i] = P;
      }
    }
    auto rho_of = [&](int i) { return before ? rcp4(ex[i]) : ex[i]; };
    auto irho_of = [&](int i) { return before ? ex[i] : rcp4(ex[i]); };
    // Per-channel block vectors from the group products gp[G] (rows 8G..8G+7),
    // one chain per wave of waves 0-3, lanes 0-31 = the 32 channel quads.
    if (w < 4 && l < 32) {
      const int c0 = 4 * l;
      auto gp = [&](int G) { return *reinterpret_cast<const float4*>(sGP + G * DK + c0); };
      auto st = [&](float* dst, float4 x) { *reinterpret_cast<float4*>(dst + c0) = x; };
      if (w == 0) {
        // gamma_mR = groups 0..2R; gamma_n = all groups
        float4 x = gp(0);
        st(sGM, x);
        x = mul4(x, mul4(gp(1), gp(2)));
        st(sGM + DK, x);
        x = mul4(x, mul4(gp(3), gp(4)));
        st(sGM + 2 * DK, x);
        x = mul4(x, mul4(gp(5), gp(6)));
        st(sGM + 3 * DK, x);
        st(sGN, mul4(x, gp(7)));
      } else if (w == 1) {
        // gamma_n / gamma_mI = groups 2I+1 .. 7
        float4 x = gp(7);
        st(sGNM + 3 * DK, x);
        x = mul4(x, mul4(gp(5), gp(6)));
        st(sGNM + 2 * DK, x);
        x = mul4(x, mul4(gp(3), gp(4)));
        st(sGNM + DK, x);
        st(sGNM, mul4(x, mul4(gp(1), gp(2))));
      } else if (w == 2) {
        // S1_I = group 2I+1;  E_(I+1),I = group 2I+2
#pragma unroll
        for (int II = 0; II < 3; ++II) {
          st(sS1 + II * DK, gp(2 * II + 1));
          st(sE + eidx(II + 1, II) * DK, gp(2 * II + 2));
        }
      } else {
        // E_RI for R >= I + 2: groups 2I+2 .. 2R
        const float4 e20 = mul4(mul4(gp(2), gp(3)), gp(4));
        const float4 e31 = mul4(mul4(gp(4), gp(5)), gp(6));
        st(sE + eidx(2, 0) * DK, e20);
        st(sE + eidx(3, 1) * DK, e31);
        st(sE + eidx(3, 0) * DK, mul4(e20, mul4(gp(5), gp(6))));
      }
    }
    lds_barrier();
    if (t < DK) reinterpret_cast<float*>(slot + SL::OFF_G)[t] = sGN[t];

    // ---- step 2: Gram tiles over the two halves of the key channels -------
    f4 acc[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) acc[j] = f4{0.f, 0.f, 0.f, 0.f};
    int tT[3], tR[3], tI[3];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      if (ht == hh) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 kv = cvt4<true>(kraw[i]), qv = cvt4<true>(qraw[i]);
          const float4 rh = rho_of(i);
          const float4 a = mul4(kv, rh), b = mul4(qv, rh), cc = mul4(kv, irho_of(i));
          const float xa[4] = {a.x, a.y, a.z, a.w}, xb[4] = {b.x, b.y, b.z, b.w};
          const float xc[4] = {cc.x, cc.y, cc.z, cc.w};
          st4<true>(sO0, L::P_H, r0 + i, 4 * cq, xa);
          st4<true>(sO1, L::P_H, r0 + i, 4 * cq, xb);
          st4<true>(sO2, L::P_H, r0 + i, 4 * cq, xc);
        }
      }
      lds_barrier();
      const float* s1h = sS1 + 64 * hh;
      const float* eh = sE + 64 * hh;
#define KDA_GROUP2(R_, I_, XD_)                                                                              \
  gram_group_half<R_, I_, XD_>(sO0, sO1, sO2, s1h + (I_) * DK, eh + eidx(R_ > I_ ? R_ : 1, I_) * DK, acc); \
  tT[0] = 0; tR[0] = R_; tI[0] = I_;                                                                          \
  tT[1] = 1; tR[1] = R_; tI[1] = I_;                                                                          \
  tT[2] = XD_; tR[2] = R_; tI[2] = R_;
      switch (w) {
        case 0: KDA_GROUP2(3, 0, 0) break;
        case 1: KDA_GROUP2(3, 1, 1) break;
        case 2: KDA_GROUP2(2, 0, 0) break;
        case 3: KDA_GROUP2(2, 1, 1) break;
        case 4: KDA_GROUP2(0, 0, -1) break;
        case 5: KDA_GROUP2(1, 1, -1) break;
        case 6: KDA_GROUP2(3, 2, -1) break;
        default: KDA_GROUP2(1, 0, -1) break;
      }
#undef KDA_GROUP2
      // K_e^T of this half = (Kr Diag(gamma_n / gamma_mI) per row block)^T:
      // unit w = (row block w & 3, 32 channels w >> 2)
      {
        const int rb = w & 3, kc = w >> 2;
        const float* sc = sGNM + rb * DK + 64 * hh;
        const M::Frag a = M::load(sO2, L::P_H, 16 * rb, kc);
        xpose32_bf<false>(a, rb, kc, sc[32 * kc + lr], sc[32 * kc + 16 + lr], sXS, L::P_H);
      }
      // Q_g of this half = Ql Diag(gamma_mR) per row block: fragment w
      if constexpr (!NOO)
        export_frag_half(slot + SL::OFF_Q + ((w >> 1) * 4 + 2 * hh + (w & 1)) * 2048, sO1, w >> 1, w & 1,
                         sGM + 64 * hh);
      lds_barrier();
      // K_e^T rows (channels) 64hh.. to the slot: row blocks 4hh + (w >> 1)
      export_frag_half(slot + SL::OFF_K + ((4 * hh + (w >> 1)) * 2 + (w & 1)) * 2048, sXS, w >> 1, w & 1,
                       nullptr);
    }

    // A = beta * strict_lower, P = lower (the halves' operands are no longer
    // read: the last barrier followed the last Gram products)
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      if (tT[j] >= 0) {
        const int r = 16 * tR[j] + lr;
        const int i0 = 16 * tI[j] + 4 * lg;
        float x[4];
        if (tT[j] == 1) {
#pragma unroll
          for (int q = 0; q < 4; ++q) x[q] = i0 + q <= r ? acc[j][q] : 0.f;
          st4<true>(sP, L::P_H, r, i0, x);
        } else {
          const float be = sBe[r];
#pragma unroll
          for (int q = 0; q < 4; ++q) x[q] = i0 + q < r ? be * acc[j][q] : 0.f;
          *reinterpret_cast<float4*>(sA + r * L::P_AF + i0) = make_float4(x[0], x[1], x[2], x[3]);
        }
      }
    }
    if (w >= 6) {   // upper tiles of P are zero
      const float z[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 3; ++e) {
        const int blk = (w - 6) * 3 + e;   // (0,1) (0,2) (0,3) (1,2) (1,3) (2,3)
        const int R = blk < 3 ? 0 : (blk < 5 ? 1 : 2);
        const int I = blk < 3 ? blk + 1 : (blk < 5 ? blk - 1 : 3);
        st4<true>(sP, L::P_H, 16 * R + lr, 16 * I + 4 * lg, z);
      }
    }
    lds_barrier();

    // ---- step 3: T = (I + A)^-1 Diag(beta) (as in prep_chunk) -------------
    // (fragments 1 and 3, K = 32..63 of row blocks 0 and 1, are zero and never
    // read: the state pass takes the nonzero K chunks of P only)
    if constexpr (!NOO)
      if (w != 1 && w != 3) export_frag_half(slot + SL::OFF_P + w * 2048, sP, w >> 1, w & 1, nullptr);
    if (w < 4) {
      const int R = w;
      const float* const Nb = sA + 16 * R * L::P_AF + 16 * R;
      float* const Xb = sLi + 16 * R * L::P_AF + 16 * R;
      f4 No, Nt, Xo;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        No[q] = Nb[(4 * lg + q) * L::P_AF + lr];
        Nt[q] = Nb[lr * L::P_AF + 4 * lg + q];
        Xo[q] = (4 * lg + q == lr ? 1.f : 0.f) - No[q];
      }
      const f4 zero = f4{0.f, 0.f, 0.f, 0.f};
      f4 Po = mm16x16(Nt, No, zero), Pt = mm16x16(No, Nt, zero);
#pragma unroll
      for (int e = 0; e < 3; ++e) {
        Xo = mm16x16(Pt, Xo, Xo);
        if (e < 2) {
          const f4 Po2 = mm16x16(Pt, Po, zero), Pt2 = mm16x16(Po, Pt, zero);
          Po = Po2;
          Pt = Pt2;
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) Xb[(4 * lg + q) * L::P_AF + lr] = Xo[q];
    } else {
      for (int e = t - 256; e < 6 * 256; e += 256) {
        const int blk = e >> 8, rr = (e >> 4) & 15, cc = e & 15;
        const int R = blk < 3 ? 0 : (blk < 5 ? 1 : 2);
        const int I = blk < 3 ? blk + 1 : (blk < 5 ? blk - 1 : 3);
        sLi[(16 * R + rr) * L::P_AF + 16 * I + cc] = 0.f;
      }
    }
    lds_barrier();
#pragma unroll
    for (int R = 1; R < 4; ++R) {
      if (w < R) {
        const int I = w;
        f4 y = f4{0.f, 0.f, 0.f, 0.f};
        for (int J = I; J < R; ++J) {
          const float4 a4 = *reinterpret_cast<const float4*>(sA + (16 * R + lr) * L::P_AF + 16 * J + 4 * lg);
          const float* bb = sLi + (16 * J + 4 * lg) * L::P_AF + 16 * I + lr;
          y = mm16x16(f4{a4.x, a4.y, a4.z, a4.w}, f4{bb[0], bb[L::P_AF], bb[2 * L::P_AF], bb[3 * L::P_AF]}, y);
        }
        const float4 d4 = *reinterpret_cast<const float4*>(sLi + (16 * R + lr) * L::P_AF + 16 * R + 4 * lg);
        const f4 x = mm16x16(f4{d4.x, d4.y, d4.z, d4.w}, y, f4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int q = 0; q < 4; ++q) sLi[(16 * R + 4 * lg + q) * L::P_AF + 16 * I + lr] = -x[q];
      }
      lds_barrier();
    }
    // T = L^-1 Diag(beta) in place (split), while K_g of half 0 = Kl
    // Diag(gamma_mR) goes into the A space (A is no longer read)
    {
      const int r = t >> 3, g8 = t & 7;
      float x[8];
      const float* src = sLi + r * L::P_AF + 8 * g8;
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = src[i] * sBe[8 * g8 + i];
      st8<true>(sT, L::P_H, r, 8 * g8, x);
    }
    auto put_kg = [&](char* dst, int hh) {
      if (ht != hh) return;
      const float4 gm = *reinterpret_cast<const float4*>(sGM + (g4 >> 2) * DK + 64 * hh + 4 * cq);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 a = mul4(mul4(cvt4<true>(kraw[i]), rho_of(i)), gm);
        const float x[4] = {a.x, a.y, a.z, a.w};
        st4<true>(dst, L::P_H, r0 + i, 4 * cq, x);
      }
    };
    put_kg(sO0, 0);
    // V in MFMA operand layout: lane (lr, lg) of wave w holds row 16 wr + lr,
    // columns 32 cu + 8 lg .. +7 with cu = (w >> 2) + 2 vh, vh = 0, 1.
    uint4 pv[2];
    {
      const char* vb = static_cast<const char*>(p.v) + row0 * DV * 2;
      const int rv = 16 * wr + lr < nv ? 16 * wr + lr : nv - 1;
#pragma unroll
      for (int vh = 0; vh < 2; ++vh) {
        const int cu = (w >> 2) + 2 * vh;
        pv[vh] = *reinterpret_cast<const uint4*>(vb + uint32_t(rv * rsv + 32 * cu + 8 * lg) * 2);
        if (16 * wr + lr >= nv) pv[vh] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
    lds_barrier();

    // ---- folded products: W = T K_g, Uv = T V, per half -------------------
    // Wave w: row block wr = w & 3 of T (zero past token 16 wr + 15), column
    // blocks 2 (w >> 2) and 2 (w >> 2) + 1 of the half.
    const int kmax = 16 * wr + 16;
    M::Frag ta[2];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) ta[kc] = M::load(sT, L::P_H, 16 * wr, kc);
    auto xpose_kg = [&](const char* src, char* dst) {   // K_g (gamma_mR applied in put_kg) transposed
      const int rb = w & 3, kc = w >> 2;
      const M::Frag a = M::load(src, L::P_H, 16 * rb, kc);
      xpose32_bf<false>(a, rb, kc, 1.f, 1.f, dst, L::P_H);
    };
    auto w_half = [&](const char* kgt, char* stage) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int nb = 2 * (w >> 2) + j;
        f4 a = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
          if (kc * 32 < kmax) a = M::mma(M::load(kgt, L::P_H, 16 * nb, kc), ta[kc], a);
        const float x[4] = {a[0], a[1], a[2], a[3]};
        st4<true>(stage, L::P_H, 16 * wr + lr, 16 * nb + 4 * lg, x);
      }
    };
    auto w_export = [&](const char* stage, int hh) {
      export_frag_half(slot + SL::OFF_W + ((w >> 1) * 4 + 2 * hh + (w & 1)) * 2048, stage, w >> 1, w & 1,
                       nullptr);
    };
    auto v_xpose = [&](char* dst, int vh) {
      M::Frag a;
      a.hi = __builtin_bit_cast(bf8, pv[vh]);
      a.lo = __builtin_bit_cast(bf8, make_uint4(0u, 0u, 0u, 0u));
      xpose32_bf<true>(a, wr, w >> 2, 1.f, 1.f, dst, L::P_H);
    };
    auto u_half = [&](const char* vt, int vh) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int nb = 2 * (w >> 2) + j;
        f4 a = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
          if (kc * 32 < kmax) a = M::mma(ta[kc], M::load(vt, L::P_H, 16 * nb, kc), a);
        *reinterpret_cast<f4*>(slot + SL::OFF_U + (wr * (DV / 16) + 4 * vh + nb) * 1024 + 16 * l) = a;
      }
    };
    xpose_kg(sO0, sO1);   // K_g^T half 0 -> O1
    lds_barrier();
    w_half(sO1, sO0);     // W half 0 -> O0
    lds_barrier();
    w_export(sO0, 0);
    put_kg(sO1, 1);       // K_g half 1 -> O1
    lds_barrier();
    xpose_kg(sO1, sO0);   // K_g^T half 1 -> O0
    lds_barrier();
    w_half(sO0, sO1);     // W half 1 -> O1
    lds_barrier();
    w_export(sO1, 1);
    v_xpose(sO0, 0);      // V^T of value columns 0-63 -> O0
    lds_barrier();
    u_half(sO0, 0);
    v_xpose(sO1, 1);      // V^T of value columns 64-127 -> O1
    lds_barrier();
    u_half(sO1, 1);
    lds_barrier();
  }
}

// acc += A B^T with the A fragments already in registers and B [16][K] in LDS;
// K chunks kc >= n (wave-uniform) are zero in A and skipped.  Every B read is
// issued before the first product: the scheduling barrier keeps the compiler
// from interleaving one read per K chunk with the products, which waited for
// the LDS once per K chunk on the state pass's critical path.
template <bool BF, int NKC>
__device__ __forceinline__ f4 gemm_ra(f4 acc, const typename Mma<BF>::Frag (&a)[NKC],
                                      const char* B, int bp, int n = NKC) {
  using M = Mma<BF>;
  typename M::Frag b[NKC];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc)
    if (kc < n) b[kc] = M::load(B, bp, 0, kc);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc)
    if (kc < n) acc = M::mma(a[kc], b[kc], acc);
  return acc;
}

// The state pass over the chunks of a segment, operands from the slots.  One
// workgroup per (sequence, head, value slab of 16*NSUB columns); the slab of S
// lives in registers, wave w holding rows 16w..16w+15.
// NOO: states (and snapshots) only; no o, so no Q_g, P or output products.
template <int DK, int NSUB, bool BF, bool SNAP, bool NOO>
__global__ __launch_bounds__(64 * (DK / 16), 1) void kda_chain_kernel(StageParams p) {
  using M = Mma<BF>;
  using F = FL<BF>;
  using Frag = typename M::Frag;
  constexpr int NW = DK / 16;
  constexpr int VS = 16 * NSUB;
  constexpr int KCK = DK / M::KU;               // fragments over the key channels
  constexpr int KCC = kC / M::KU;               // fragments over the tokens of a chunk
  constexpr int RBK = DK / F::KU * F::UNIT;     // bytes per 16-row block, K = DK
  constexpr int RBC = kC / F::KU * F::UNIT;     // bytes per 16-row block, K = 64
  constexpr int SP_S = DK * 4 + 16, SP_U = kC * 4 + 16;
  constexpr int OFF_W = 0, OFF_Q = 64 * DK * 4, OFF_K = 128 * DK * 4, OFF_P = 192 * DK * 4;
  constexpr int OFF_U = OFF_P + 64 * 64 * 4;
  __shared__ __attribute__((aligned(16))) char smem[VS * SP_S + VS * SP_U];
  char* const sS = smem;               // S^T of the slab [VS][DK]
  char* const sU = smem + VS * SP_S;   // U^T of the slab [VS][64]

  const int t = threadIdx.x;
  const int l = t & 63;
  const int w = t >> 6;
  const int lr = l & 15;
  const int lg = l >> 4;

  int64_t b = blockIdx.x;
  const int64_t G = gridDim.x;
  if ((G & 7) == 0) b = (b & 7) * (G >> 3) + (b >> 3);
  const int slab = int(b % p.nslab);
  const int64_t pr = b / p.nslab;
  const int H = p.H, DV = p.DV;
  const int h = int(pr % H);
  const int64_t n = pr / H;
  const int col0 = slab * VS;
  const int rsv = H * DV;
  const int64_t slot_bytes = OFF_U + 64 * DV * 4 + DK * 4;
  const int off_g = OFF_U + 64 * DV * 4;

  f4 S[NSUB];
  const int64_t sbase = pr * DK * DV;
#pragma unroll
  for (int js = 0; js < NSUB; ++js)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      S[js][q] = p.s_in ? p.s_in[sbase + int64_t(16 * w + 4 * lg + q) * DV + col0 + 16 * js + lr]
                        : 0.f;

  // With 8 waves, waves 0-3 compute X and U for token rows 16w.. and waves
  // 4-7 the output rows 16(w-4)..; with 4 waves every wave does both.
  constexpr bool kSplitO = NW >= 8;
  const bool xw = w < 4;
  const bool owave = NOO ? false : (kSplitO ? (w >= 4) : true);
  const int ow = w & 3;
  constexpr int NA = kSplitO ? 1 : 2;   // row blocks of W / Qg held by a wave
  // P is lower triangular: its row block ow is zero past token 16 ow + 15.
  const int npk = (16 * ow + 16 + M::KU - 1) / M::KU;

  // Operands of a chunk: two sets, ping-ponged between consecutive chunks
  // (no register copies, so the wait for each prefetched part sits at its
  // first use, not at the start of the chunk).
  struct Ops {
    Frag a[NA][KCK], pp[KCC], kg[KCC];
    f4 u[NSUB];
    float4 g;
  };
  // The loads are issued in three parts spread over the chunk, so that the
  // memory pipeline works while the waves compute: K_e^T and gamma_n (part 2,
  // last used at the end of a chunk) at the start of the previous chunk, W or
  // Q_g (part 1) after its first barrier, P and Uv (part 3) after its second.
  // (Measured at B=1, H=32, T=8192: 2% faster than parts 1, 2, 3 in order;
  // the other four orders were slower.)
  auto slot_of = [&](int64_t c) { return p.ws + ((c - p.c_begin) * p.pairs + pr) * slot_bytes; };
  auto load_part1 = [&](Ops& o, const char* slot) {
#pragma unroll
    for (int a = 0; a < NA; ++a) {
      const bool wside = kSplitO ? xw : (a == 0);
      if (NOO && !wside) continue;
      F::load(o.a[a], slot + (wside ? OFF_W : OFF_Q) + ow * RBK);
    }
  };
  auto load_part2 = [&](Ops& o, const char* slot) {
    F::load(o.kg, slot + OFF_K + w * RBC);
    o.g = *reinterpret_cast<const float4*>(slot + off_g + (16 * w + 4 * lg) * 4);
  };
  auto load_part3 = [&](Ops& o, const char* slot) {
    if (owave) F::load(o.pp, slot + OFF_P + ow * RBC, npk);
    if (xw) {
#pragma unroll
      for (int js = 0; js < NSUB; ++js)
        o.u[js] = *reinterpret_cast<const f4*>(slot + OFF_U + (ow * (DV / 16) + (col0 >> 4) + js) * 1024 + 16 * l);
    }
  };
  const int64_t c_end = p.c_begin + p.nseg;
  Ops A, B;
  {
    const char* s0 = slot_of(p.c_begin);
    load_part1(A, s0);
    load_part2(A, s0);
    load_part3(A, s0);
  }
  // The output stores that follow the prefetch in every chunk, mirrored
  // before the first one (keeps the compiler's memory-counter waits for the
  // prefetched operands from covering the stores as well).  Plain stores to
  // distinct addresses: volatile ones would each be followed by a wait for
  // every memory operation in flight, the prefetch included.
  mirror_stores<4 * NSUB>();

  // One chunk with operands `cur`; the next chunk's operands go to `nxt`
  // (past the last chunk the last one is loaded again: loads stay
  // unconditional).
  auto step = [&](int64_t c, Ops& cur, Ops& nxt) {
    const int64_t tok0 = n * p.T_fixed + c * kC;
    const int64_t rem = p.T_fixed - c * kC;
    const int nv = int(rem < kC ? rem : kC);
    const char* sn = slot_of(c + 1 < c_end ? c + 1 : c);
    load_part2(nxt, sn);

    // S^T of the slab to LDS.
#pragma unroll
    for (int js = 0; js < NSUB; ++js) {
      const float x[4] = {S[js][0], S[js][1], S[js][2], S[js][3]};
      st4<BF>(sS, SP_S, 16 * js + lr, 16 * w + 4 * lg, x);
    }
    lds_barrier();
    load_part1(nxt, sn);
    // U = Uv - W S  (X side);  O = Qg S  (O side).
    f4 acco[NSUB];
#pragma unroll
    for (int js = 0; js < NSUB; ++js) acco[js] = f4{0.f, 0.f, 0.f, 0.f};
    if (xw) {
#pragma unroll
      for (int js = 0; js < NSUB; ++js) {
        const f4 x = gemm_ra<BF, KCK>(f4{0.f, 0.f, 0.f, 0.f}, cur.a[0], sS + 16 * js * SP_S, SP_S);
        const float y[4] = {cur.u[js][0] - x[0], cur.u[js][1] - x[1], cur.u[js][2] - x[2],
                            cur.u[js][3] - x[3]};
        st4<BF>(sU, SP_U, 16 * js + lr, 16 * ow + 4 * lg, y);
      }
    }
    if (owave) {
#pragma unroll
      for (int js = 0; js < NSUB; ++js)
        acco[js] = gemm_ra<BF, KCK>(acco[js], cur.a[NA - 1], sS + 16 * js * SP_S, SP_S);
    }
    lds_barrier();
    load_part3(nxt, sn);
    // O += P U, stored;  S' = Diag(gamma_n) S + Kg U.
    if (owave) {
#pragma unroll
      for (int js = 0; js < NSUB; ++js)
        acco[js] = gemm_ra<BF, KCC>(acco[js], cur.pp, sU + 16 * js * SP_U, SP_U, npk);
    }
#pragma unroll
    for (int js = 0; js < NSUB; ++js) {
      float* ob = p.o + (tok0 * H + h) * int64_t(DV) + col0 + 16 * js;
      float* sink = g_kda_sink + (blockIdx.x & 255) * (kSinkStores * 64) + l;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 16 * ow + 4 * lg + q;
        float* dst = owave && r < nv ? ob + uint32_t(r * rsv + lr) : sink;
        *dst = acco[js][q];
      }
    }
#pragma unroll
    for (int js = 0; js < NSUB; ++js) {
      const f4 y = gemm_ra<BF, KCC>(f4{0.f, 0.f, 0.f, 0.f}, cur.kg, sU + 16 * js * SP_U, SP_U);
      S[js][0] = cur.g.x * S[js][0] + y[0];
      S[js][1] = cur.g.y * S[js][1] + y[1];
      S[js][2] = cur.g.z * S[js][2] + y[2];
      S[js][3] = cur.g.w * S[js][3] + y[3];
    }
    if constexpr (SNAP) {
      if (nv == kC && (c + 1) % p.snap_every == 0)
        store_snapshot<DK, NSUB>(p.snap, n * p.snap_per_seq + (c + 1) / p.snap_every - 1, h, H, DV, col0, S);
    }
  };

  // The first chunk is peeled: it is the only one that reads the state as
  // loaded from state_in, so the loop's waits never cover that load.
  step(p.c_begin, A, B);
  for (int64_t c = p.c_begin + 1; c < c_end; c += 2) {
    step(c, B, A);
    if (c + 1 >= c_end) break;
    step(c + 1, A, B);
  }

  if (p.s_out) {
#pragma unroll
    for (int js = 0; js < NSUB; ++js)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        p.s_out[sbase + int64_t(16 * w + 4 * lg + q) * DV + col0 + 16 * js + lr] = S[js][q];
  }
}

template <int DK, int NSUB, bool BF>
void launch_t(const Params& p, int64_t nblocks, hipStream_t st) {
  if (p.snap && p.states_only)   // the backward's checkpoints
    hipLaunchKernelGGL((kda_prefill_kernel<DK, NSUB, BF, true, true>), dim3(unsigned(nblocks)),
                       dim3(Lay<DK>::NT), 0, st, p);
  else if (p.snap)
    hipLaunchKernelGGL((kda_prefill_kernel<DK, NSUB, BF, true, false>), dim3(unsigned(nblocks)),
                       dim3(Lay<DK>::NT), 0, st, p);
  else
    hipLaunchKernelGGL((kda_prefill_kernel<DK, NSUB, BF, false, false>), dim3(unsigned(nblocks)),
                       dim3(Lay<DK>::NT), 0, st, p);
}

template <int DK, bool BF>
void launch_dk(const Params& p, int nsub, int64_t nblocks, hipStream_t st) {
  switch (nsub) {
    case 8: launch_t<DK, 8, BF>(p, nblocks, st); break;
    case 4: launch_t<DK, 4, BF>(p, nblocks, st); break;
    case 2: launch_t<DK, 2, BF>(p, nblocks, st); break;
    default: launch_t<DK, 1, BF>(p, nblocks, st); break;
  }
}

// Columns per workgroup: as many as possible while the launch still has a
// workgroup for every compute unit (256 on MI355X).
int choose_nsub(int64_t pairs, int DV) {
  if (const int v = tuning().prefill_nsub; v > 0 && 16 * v <= DV) return v;
  // The widest slab that still gives every compute unit a workgroup: a
  // wider slab repeats steps 1-3 for fewer slabs (d=128, bf16: NSUB 8 over 4
  // is 11-13% faster from 256 chains up, although its registers spill).
  for (int nsub = DV / 16 < 8 ? DV / 16 : 8; nsub > 1; nsub >>= 1)
    if (pairs * (DV / (16 * nsub)) >= 256) return nsub;
  return 1;
}

// The staged form pays off when the chains are too few to fill the GPU
// without value slabs, i.e. when the fused kernel would repeat steps 1-3 per
// slab.  Fixed-length batches only.
bool use_staged(bool varlen, int64_t pairs, int64_t nchunks) {
  if (varlen || nchunks < 2) return false;
  if (const int f = tuning().prefill_form; f != 0) return f == 2;
  return pairs < 128;
}

size_t slot_bytes(int DK, int DV) { return size_t(4) * (3 * 64 * DK + 64 * 64 + 64 * DV + DK); }

// Chunks per sequence handled by one stage + chain pair of launches.  Every
// value slab's chain workgroup reads each slot, so the slots are read many
// times; when one segment's slots fit in the memory-side cache (256 MB on
// MI355X, budget 160 MiB of it) the chain kernel is served from there rather
// than from HBM (B=1, H=32, T=8192, d=128: 527 -> 442 us).  The chunks are
// split into equal segments, so that no stage launch ends on a short segment.
// The tuning override prefill_seg forces that many chunks per segment (at
// most 1 GiB of slots, and at most `budget` bytes when one is given).
constexpr int64_t kSegBudget = int64_t(160) << 20;
int64_t seg_chunks(int64_t pairs, int64_t nchunks, int DK, int DV, int64_t budget = 0) {
  const int64_t per_chunk = pairs * int64_t(slot_bytes(DK, DV));
  const int64_t limit = budget > 0 ? budget : (int64_t(1) << 30);
  if (const int64_t v = tuning().prefill_seg; v > 0 && v <= limit / per_chunk)
    return v < nchunks ? v : nchunks;
  int64_t cap = (budget > 0 && budget < kSegBudget ? budget : kSegBudget) / per_chunk;
  if (cap < 1) cap = 1;
  if (cap >= nchunks) return nchunks;
  const int64_t nseg = (nchunks + cap - 1) / cap;
  return (nchunks + nseg - 1) / nseg;
}

// Compute units of the current device (persistent stage kernel grid).
int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    cus[dev] = v;
  }
  return cus[dev];
}

template <int DK, int DV, bool BF>
void launch_staged_t(const Params& base, int64_t T, int nsub, hipStream_t st, char* ws, int64_t seg,
                     int64_t nchunks, float* state_ws) {
  StageParams sp;
  sp.H = base.H;
  sp.DV = DV;
  sp.nslab = DV / (16 * nsub);
  sp.T_fixed = T;
  sp.pairs = int64_t(base.N) * base.H;
  sp.q = base.q;
  sp.k = base.k;
  sp.v = base.v;
  sp.alpha = base.alpha;
  sp.beta = base.beta;
  sp.o = base.o;
  sp.ws = ws;
  sp.snap = base.snap;
  sp.snap_every = base.snap_every;
  sp.snap_per_seq = base.snap_per_seq;
  sp.alpha_scalar = base.alpha_scalar;
  sp.states_only = base.states_only;
  const int64_t nsegs = (nchunks + seg - 1) / seg;
  const int64_t cus = device_cus();
  for (int64_t si = 0; si < nsegs; ++si) {
    sp.c_begin = si * seg;
    sp.nseg = (si + 1) * seg <= nchunks ? seg : nchunks - si * seg;
    sp.s_in = si == 0 ? base.s_in : state_ws;
    sp.s_out = si == nsegs - 1 ? base.s_out : state_ws;
    const int64_t items = sp.pairs * sp.nseg;
    const bool noo = sp.snap && sp.states_only;   // the backward's checkpoints
    if constexpr (DK == 128 && DV == 128 && BF) {
      // one workgroup per item, two per compute unit
      const dim3 grid{unsigned(items)}, block{unsigned(Lay2::NT)};
      if (noo) {
        if (sp.alpha_scalar) hipLaunchKernelGGL((kda_stage2_kernel<true, true>), grid, block, 0, st, sp);
        else hipLaunchKernelGGL((kda_stage2_kernel<true, false>), grid, block, 0, st, sp);
      } else {
        if (sp.alpha_scalar) hipLaunchKernelGGL((kda_stage2_kernel<false, true>), grid, block, 0, st, sp);
        else hipLaunchKernelGGL((kda_stage2_kernel<false, false>), grid, block, 0, st, sp);
      }
    } else {
      const unsigned ns = unsigned(items < cus ? items : cus);
      if (noo)
        hipLaunchKernelGGL((kda_stage_kernel<DK, DV, BF, true>), dim3(ns), dim3(Lay<DK>::NT), 0, st, sp);
      else
        hipLaunchKernelGGL((kda_stage_kernel<DK, DV, BF, false>), dim3(ns), dim3(Lay<DK>::NT), 0, st, sp);
    }
    const unsigned nb = unsigned(sp.pairs * sp.nslab);
    if (noo) {
      if (nsub == 4)
        hipLaunchKernelGGL((kda_chain_kernel<DK, 4, BF, true, true>), dim3(nb), dim3(Lay<DK>::NT), 0, st, sp);
      else if (nsub == 2)
        hipLaunchKernelGGL((kda_chain_kernel<DK, 2, BF, true, true>), dim3(nb), dim3(Lay<DK>::NT), 0, st, sp);
      else
        hipLaunchKernelGGL((kda_chain_kernel<DK, 1, BF, true, true>), dim3(nb), dim3(Lay<DK>::NT), 0, st, sp);
    } else if (nsub == 4) {
      if (sp.snap)
        hipLaunchKernelGGL((kda_chain_kernel<DK, 4, BF, true, false>), dim3(nb), dim3(Lay<DK>::NT), 0, st, sp);
      else
        hipLaunchKernelGGL((kda_chain_kernel<DK, 4, BF, false, false>), dim3(nb), dim3(Lay<DK>::NT), 0, st, sp);
    } else if (nsub == 2) {
      if (sp.snap)
        hipLaunchKernelGGL((kda_chain_kernel<DK, 2, BF, true, false>), dim3(nb), dim3(Lay<DK>::NT), 0, st, sp);
      else
        hipLaunchKernelGGL((kda_chain_kernel<DK, 2, BF, false, false>), dim3(nb), dim3(Lay<DK>::NT), 0, st, sp);
    } else {
      if (sp.snap)
        hipLaunchKernelGGL((kda_chain_kernel<DK, 1, BF, true, false>), dim3(nb), dim3(Lay<DK>::NT), 0, st, sp);
      else
        hipLaunchKernelGGL((kda_chain_kernel<DK, 1, BF, false, false>), dim3(nb), dim3(Lay<DK>::NT), 0, st, sp);
    }
  }
}

template <int DK, bool BF>
void launch_staged(const Params& base, int64_t T, int nsub, hipStream_t st, char* ws, int64_t seg,
                   int64_t nchunks, float* state_ws) {
  if (base.DV == 128) launch_staged_t<DK, 128, BF>(base, T, nsub, st, ws, seg, nchunks, state_ws);
  else launch_staged_t<DK, 64, BF>(base, T, nsub, st, ws, seg, nchunks, state_ws);
}

// Value columns per chain workgroup of the staged form (1 or 2 blocks of 16).
int staged_nsub(int64_t pairs, int DV) {
  if (const int v = tuning().prefill_nsub; (v == 1 || v == 2 || v == 4) && 16 * v <= DV) return v;
  (void)pairs;
  (void)DV;
  return 1;
}

}  // namespace

// The staged form's workspace for callers that cannot allocate
// (kda_chunk_prefill_noalloc): one array per device, reserved with the code
// object while the process lives.  Host code never passes `scratch` itself to
// a kernel (on the host it names a stand-in, not device memory): it takes the
// device address from hipGetSymbolAddress, once per device.
static __device__ __align__(256) char scratch[kNoallocScratchBytes];

void* noalloc_scratch(const char** msg) {
  static std::mutex mu;
  static void* addr[64] = {nullptr};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= 64) {
    *msg = e != hipSuccess ? hipGetErrorString(e) : "device index out of range";
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      *msg = e != hipSuccess ? hipGetErrorString(e) : "no device address for the scratch array";
      return nullptr;
    }
    addr[dev] = ptr;
  }
  return addr[dev];
}

size_t prefill_workspace_bytes(int N, int64_t T_total, int H, int DK, int DV, bool varlen,
                               int64_t seg_budget) {
  const int64_t pairs = int64_t(N) * H;
  if (pairs == 0 || varlen) return 0;
  const int64_t T = T_total / N;
  const int64_t nchunks = (T + kC - 1) / kC;
  if (!use_staged(varlen, pairs, nchunks)) return 0;
  const int64_t seg = seg_chunks(pairs, nchunks, DK, DV, seg_budget);
  size_t bytes = size_t(pairs) * size_t(seg) * slot_bytes(DK, DV);
  if (seg < nchunks) bytes += size_t(pairs) * DK * DV * 4;  // state carried between segments
  return bytes;
}

int launch_prefill(const PrefillArgs& a, void* stream, const char** msg) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (a.DK != 128 && a.DK != 64) {
    *msg = "unsupported DK";
    return 1;
  }
  Params p;
  p.N = a.N;
  p.T_fixed = a.T_fixed;
  p.cu = a.cu_seqlens;
  p.H = a.H;
  p.DV = a.DV;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.alpha = a.alpha;
  p.beta = a.beta;
  p.s_in = a.state_in;
  p.o = a.o;
  p.s_out = a.state_out;
  p.snap = a.snapshots;
  p.snap_every = a.snap_every > 0 ? a.snap_every : 1;
  p.snap_per_seq = a.snapshots ? a.T_fixed / (int64_t(kC) * p.snap_every) : 0;
  p.snap_off = a.snap_offsets;
  p.snap_rows = a.snap_rows;
  p.alpha_scalar = a.alpha_scalar ? 1 : 0;
  p.states_only = a.states_only ? 1 : 0;
  const int64_t pairs = int64_t(a.N) * a.H;
  const bool varlen = a.cu_seqlens != nullptr;
  const int64_t nchunks = varlen ? 0 : (a.T_fixed + kC - 1) / kC;
  (void)hipGetLastError();
  if (use_staged(varlen, pairs, nchunks)) {
    const int nsub = staged_nsub(pairs, a.DV);
    const int64_t seg = seg_chunks(pairs, nchunks, a.DK, a.DV, a.seg_budget);
    if (pairs * seg >= (int64_t(1) << 31)) {   // the stage kernel indexes items in 32 bits
      *msg = "staged prefill: more than 2^31 items in one segment";
      return 1;
    }
    char* ws = static_cast<char*>(a.workspace);
    float* state_ws = seg < nchunks
        ? reinterpret_cast<float*>(ws + size_t(pairs) * size_t(seg) * slot_bytes(a.DK, a.DV))
        : nullptr;
    if (a.DK == 128) {
      if (a.in_bf16) launch_staged<128, true>(p, a.T_fixed, nsub, st, ws, seg, nchunks, state_ws);
      else launch_staged<128, false>(p, a.T_fixed, nsub, st, ws, seg, nchunks, state_ws);
    } else {
      if (a.in_bf16) launch_staged<64, true>(p, a.T_fixed, nsub, st, ws, seg, nchunks, state_ws);
      else launch_staged<64, false>(p, a.T_fixed, nsub, st, ws, seg, nchunks, state_ws);
    }
  } else {
    const int nsub = choose_nsub(pairs, a.DV);
    p.nslab = a.DV / (16 * nsub);
    const int64_t nblocks = pairs * p.nslab;
    if (a.DK == 128) {
      if (a.in_bf16) launch_dk<128, true>(p, nsub, nblocks, st);
      else launch_dk<128, false>(p, nsub, nblocks, st);
    } else {
      if (a.in_bf16) launch_dk<64, true>(p, nsub, nblocks, st);
      else launch_dk<64, false>(p, nsub, nblocks, st);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    *msg = hipGetErrorString(e);
    return 1;
  }
  return 0;
}

}  // namespace kda

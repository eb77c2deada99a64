// KDA chunked prefill on gfx950 (MI355X).
//
// The chunk form of the KDA recurrence ("Kimi Delta Attention 徹底解説"
// (tech-tide.dev), section "Kimi Delta Attention の仕組み": prefill regroups
// the token recurrence into chunked matrix products; "Kimi Linear、独自の土俵で
// Full Attentionを上回る" (remio.ai), section "Kimi Linearがより賢いRecurrent
// Memoryを使う方法": the chunkwise algorithm rests on a diagonal-plus-low-rank
// transition).  The pages print no chunk formula; the one used here follows
// from unrolling the recurrence inside a chunk of n <= 64 tokens with
// incoming state S (d_k x d_v, rows = key channels).  With m = 31 the chunk's
// reference position and f_r = prod_{s<=r} alpha_s / prod_{s<=m} alpha_s
// (per key channel; > 1 before m, <= 1 after it):
//     Kl = K * f,   Ql = Q * f,   Kr = K / f           (row-wise, per channel)
//     A  = Diag(beta) strict_lower(Kl Kr^T)            (= beta_r k_r.(decayed k_i))
//     P  = lower(Ql Kr^T)
//     T  = (I + A)^-1 Diag(beta)                       (unit-lower solve)
//     S_B = Diag(gamma_m) S                            (state decayed to m)
//     X  = V - Kl S_B ;  U = T X                       (values actually written)
//     O  = Ql S_B + P U
//     S' = Diag(gamma_n) S + Diag(gamma_n / gamma_m) Kr^T U
// All products are dense MFMA contractions.  bf16 inputs use split bf16
// operands (x = hi + lo, three MFMAs per product) so that the products carry
// ~16 significant bits; fp32 inputs use the fp32 MFMA.  Accumulation is fp32.
//
// One workgroup (4 waves) per (sequence, head, value slab): the value columns
// of the state evolve independently, so the sequential pass over the chunks
// is split into slabs of 16..128 columns to give enough workgroups; a
// workgroup holds its slab of S in registers for the whole sequence.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "kda_internal.h"

namespace kda {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));

constexpr int kC = 64;    // chunk length
constexpr int kNT = 256;  // threads per workgroup (4 waves)
constexpr int kRef = 31;  // reference position inside a chunk (rows 0..31 | 32..63)

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
};

// ---------------------------------------------------------------- layout ----
// Operand arrays are [rows][K] with the contraction index K contiguous.  In
// bf16 mode every group of 8 consecutive K holds 8 hi parts (16 B) followed by
// the 8 lo parts (16 B); in fp32 mode an element is one float.  Either way an
// element takes 4 bytes and a row has a 16-byte pad (conflict-free 128-bit
// fragment reads).
template <int DK>
struct Lay {
  static constexpr int P_OP = DK * 4 + 16;  // rows of DK elements
  static constexpr int P_T = kC * 4 + 16;   // rows of 64 elements (272 B)
  static constexpr int P_AF = kC + 4;       // fp32 pitch (floats) of A / L^-1 (272 B)
  static constexpr int OFF_KL = 0;
  static constexpr int OFF_QL = OFF_KL + kC * P_OP;
  static constexpr int OFF_KRT = OFF_QL + kC * P_OP;         // Kr^T [DK][64]
  static constexpr int OFF_X = OFF_KRT + DK * P_T;           // Kr, then A + P
  static constexpr int SZ_X = (kC * P_OP > 2 * kC * P_T) ? kC * P_OP : 2 * kC * P_T;
  static constexpr int OFF_A = OFF_X;                        // fp32 [64][68]
  static constexpr int OFF_P = OFF_X + kC * P_T;             // [64][64]
  static constexpr int OFF_SBT = OFF_X;                      // S_B^T [16][DK]  (after the solve)
  static constexpr int OFF_XT = OFF_SBT + 16 * P_OP;         // X^T [16][64]
  static constexpr int OFF_UT = OFF_XT + 16 * P_T;           // U^T [16][64]
  static constexpr int OFF_T = OFF_X + SZ_X;                 // T [64][64] (fp32 L^-1 first)
  static constexpr int OFF_TMP = OFF_T + kC * P_T;           // 3 x 16x16 fp32
  static constexpr int RG = 512 / DK;                        // row groups in the decay prep
  static constexpr int OFF_GP = OFF_TMP + 3 * 256 * 4;       // group products [RG][DK]
  static constexpr int OFF_GM = OFF_GP + RG * DK * 4;        // gamma_m [DK]
  static constexpr int OFF_DL = OFF_GM + DK * 4;             // gamma_n / gamma_m [DK]
  static constexpr int OFF_GN = OFF_DL + DK * 4;             // gamma_n [DK]
  static constexpr int OFF_BE = OFF_GN + DK * 4;             // beta [64]
  static constexpr int TOTAL = OFF_BE + kC * 4;
  static_assert(OFF_UT + 16 * P_T <= OFF_X + kC * P_T, "step buffers fit in A's space");
  static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

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

// acc += A[arow0.., k0:k1] * B[brow0.., k0:k1]^T  (both stored [row][K]).
template <bool BF>
__device__ __forceinline__ f4 gemm(f4 acc, const char* A, int ap, int arow0, const char* B,
                                   int bp, int brow0, int k0, int k1) {
  using M = Mma<BF>;
#pragma unroll 4
  for (int kc = k0 / M::KU; kc < k1 / M::KU; ++kc) {
    auto a = M::load(A, ap, arow0, kc);
    auto b = M::load(B, bp, brow0, kc);
    acc = M::mma(a, b, acc);
  }
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
    uint16_t h0, l0, h1, l1;
    split(x0, h0, l0);
    split(x1, h1, l1);
    char* p = base + row * pitch + (kk >> 3) * 32 + (kk & 7) * 2;
    *reinterpret_cast<uint32_t*>(p) = uint32_t(h0) | (uint32_t(h1) << 16);
    *reinterpret_cast<uint32_t*>(p + 16) = uint32_t(l0) | (uint32_t(l1) << 16);
  } else {
    *reinterpret_cast<float2*>(base + row * pitch + kk * 4) = make_float2(x0, x1);
  }
}

// Four consecutive elements starting at kk (kk % 4 == 0).
template <bool BF>
__device__ __forceinline__ void st4(char* base, int pitch, int row, int kk, const float* x) {
  if constexpr (BF) {
    uint16_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) split(x[i], h[i], l[i]);
    char* p = base + row * pitch + (kk >> 3) * 32 + (kk & 7) * 2;
    uint2 hv, lv;
    hv.x = uint32_t(h[0]) | (uint32_t(h[1]) << 16);
    hv.y = uint32_t(h[2]) | (uint32_t(h[3]) << 16);
    lv.x = uint32_t(l[0]) | (uint32_t(l[1]) << 16);
    lv.y = uint32_t(l[2]) | (uint32_t(l[3]) << 16);
    *reinterpret_cast<uint2*>(p) = hv;
    *reinterpret_cast<uint2*>(p + 16) = lv;
  } else {
    *reinterpret_cast<float4*>(base + row * pitch + kk * 4) = make_float4(x[0], x[1], x[2], x[3]);
  }
}

// Eight consecutive elements starting at kk (kk % 8 == 0).
template <bool BF>
__device__ __forceinline__ void st8(char* base, int pitch, int row, int kk, const float* x) {
  st4<BF>(base, pitch, row, kk, x);
  st4<BF>(base, pitch, row, kk + 4, x + 4);
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

// ------------------------------------------------------------------ kernel --
template <int DK, int NSUB, bool BF>
__global__ __launch_bounds__(kNT, 1) void kda_prefill_kernel(Params p) {
  using L = Lay<DK>;
  using M = Mma<BF>;
  constexpr int NP = DK / 2;        // channel pairs in the decay prep
  constexpr int RG = L::RG;         // row groups in the decay prep
  constexpr int RPG = kC / RG;      // rows per group
  constexpr int TPW = DK / 64;      // 16-row tiles of the state per wave
  constexpr int VS = 16 * NSUB;     // value columns of this workgroup

  __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
  char* const sKl = smem + L::OFF_KL;
  char* const sQl = smem + L::OFF_QL;
  char* const sKrT = smem + L::OFF_KRT;
  char* const sKr = smem + L::OFF_X;
  float* const sA = reinterpret_cast<float*>(smem + L::OFF_A);
  char* const sP = smem + L::OFF_P;
  char* const sSBT = smem + L::OFF_SBT;
  char* const sXT = smem + L::OFF_XT;
  char* const sUT = smem + L::OFF_UT;
  char* const sT = smem + L::OFF_T;
  float* const sLi = reinterpret_cast<float*>(smem + L::OFF_T);
  float* const sTmp = reinterpret_cast<float*>(smem + L::OFF_TMP);
  float* const sGP = reinterpret_cast<float*>(smem + L::OFF_GP);
  float* const sGM = reinterpret_cast<float*>(smem + L::OFF_GM);
  float* const sDL = reinterpret_cast<float*>(smem + L::OFF_DL);
  float* const sGN = reinterpret_cast<float*>(smem + L::OFF_GN);
  float* const sBe = reinterpret_cast<float*>(smem + L::OFF_BE);

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
  if ((G & 7) == 0) b = (b & 7) * (G >> 3) + (b >> 3);
  const int slab = int(b % p.nslab);
  const int64_t pr = b / p.nslab;
  const int h = int(pr % p.H);
  const int n = int(pr / p.H);
  const int H = p.H, DV = p.DV;
  const int col0 = slab * VS;

  int64_t s0, s1;
  if (p.cu != nullptr) {
    s0 = p.cu[n];
    s1 = p.cu[n + 1];
  } else {
    s0 = int64_t(n) * p.T_fixed;
    s1 = s0 + p.T_fixed;
  }

  // State slab in registers: S[js][tt][q] = S[c][col0 + 16 js + lr] with
  // c = 16 (w*TPW + tt) + 4 lg + q.
  f4 S[NSUB][TPW];
  const int64_t sbase = (int64_t(n) * H + h) * DK * DV;
#pragma unroll
  for (int js = 0; js < NSUB; ++js)
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = 16 * (w * TPW + tt) + 4 * lg + q;
        S[js][tt][q] = p.s_in ? p.s_in[sbase + int64_t(c) * DV + col0 + 16 * js + lr] : 0.f;
      }

  const int cp = t % NP, grp = t / NP;
  const int ch0 = 2 * cp;
  const int rb = grp * RPG;

  for (int64_t tok0 = s0; tok0 < s1; tok0 += kC) {
    const int nv = int(s1 - tok0 < kC ? s1 - tok0 : kC);

    // ---- values of this workgroup's columns, in accumulator layout -------
    float vreg[NSUB][4];
#pragma unroll
    for (int js = 0; js < NSUB; ++js)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 16 * w + 4 * lg + q;
        vreg[js][q] = r < nv ? ld1<BF>(p.v, ((tok0 + r) * H + h) * int64_t(DV) + col0 + 16 * js + lr)
                             : 0.f;
      }

    // ---- step 1: decay factors and decayed operands ------------------------
    float2 av[RPG], kv[RPG], qv[RPG];
    float2 gp = make_float2(1.f, 1.f);
#pragma unroll
    for (int i = 0; i < RPG; ++i) {
      const int r = rb + i;
      if (r < nv) {
        const int64_t idx = ((tok0 + r) * H + h) * int64_t(DK) + ch0;
        av[i] = *reinterpret_cast<const float2*>(p.alpha + idx);
        kv[i] = ld2<BF>(p.k, idx);
        qv[i] = ld2<BF>(p.q, idx);
      } else {
        av[i] = make_float2(1.f, 1.f);
        kv[i] = make_float2(0.f, 0.f);
        qv[i] = make_float2(0.f, 0.f);
      }
      gp.x *= av[i].x;
      gp.y *= av[i].y;
    }
    sGP[grp * DK + ch0] = gp.x;
    sGP[grp * DK + ch0 + 1] = gp.y;
    if (t < kC) sBe[t] = t < nv ? p.beta[(tok0 + t) * H + h] : 0.f;
    __syncthreads();

    {
      float2 krs[RPG];
      constexpr int half = RG / 2;
      if (grp >= half) {
        // rows after the reference: f = prod_{m < s <= r} alpha_s <= 1
        float2 P = make_float2(1.f, 1.f);
        for (int g2 = half; g2 < grp; ++g2) {
          P.x *= sGP[g2 * DK + ch0];
          P.y *= sGP[g2 * DK + ch0 + 1];
        }
#pragma unroll
        for (int i = 0; i < RPG; ++i) {
          P.x *= av[i].x;
          P.y *= av[i].y;
          const float ix = rcp(P.x), iy = rcp(P.y);
          const int r = rb + i;
          st2<BF>(sKl, L::P_OP, r, ch0, kv[i].x * P.x, kv[i].y * P.y);
          st2<BF>(sQl, L::P_OP, r, ch0, qv[i].x * P.x, qv[i].y * P.y);
          krs[i] = make_float2(kv[i].x * ix, kv[i].y * iy);
          st2<BF>(sKr, L::P_OP, r, ch0, krs[i].x, krs[i].y);
        }
      } else {
        // rows up to the reference: 1/f = prod_{r < s <= m} alpha_s <= 1
        float2 Q = make_float2(1.f, 1.f);
        for (int g2 = grp + 1; g2 < half; ++g2) {
          Q.x *= sGP[g2 * DK + ch0];
          Q.y *= sGP[g2 * DK + ch0 + 1];
        }
#pragma unroll
        for (int i = RPG - 1; i >= 0; --i) {
          const float fx = rcp(Q.x), fy = rcp(Q.y);
          const int r = rb + i;
          st2<BF>(sKl, L::P_OP, r, ch0, kv[i].x * fx, kv[i].y * fy);
          st2<BF>(sQl, L::P_OP, r, ch0, qv[i].x * fx, qv[i].y * fy);
          krs[i] = make_float2(kv[i].x * Q.x, kv[i].y * Q.y);
          st2<BF>(sKr, L::P_OP, r, ch0, krs[i].x, krs[i].y);
          Q.x *= av[i].x;
          Q.y *= av[i].y;
        }
      }
      // Kr^T rows (= key channels), 8 tokens at a time.
#pragma unroll
      for (int j = 0; j < RPG / 8; ++j) {
        float x0[8], x1[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          x0[e] = krs[8 * j + e].x;
          x1[e] = krs[8 * j + e].y;
        }
        st8<BF>(sKrT, L::P_T, ch0, rb + 8 * j, x0);
        st8<BF>(sKrT, L::P_T, ch0 + 1, rb + 8 * j, x1);
      }
      if (grp == 0) {
        float2 gm = make_float2(1.f, 1.f), dl = make_float2(1.f, 1.f);
        for (int g2 = 0; g2 < RG; ++g2) {
          const float a0 = sGP[g2 * DK + ch0], a1 = sGP[g2 * DK + ch0 + 1];
          if (g2 < half) {
            gm.x *= a0;
            gm.y *= a1;
          } else {
            dl.x *= a0;
            dl.y *= a1;
          }
        }
        sGM[ch0] = gm.x;
        sGM[ch0 + 1] = gm.y;
        sDL[ch0] = dl.x;
        sDL[ch0 + 1] = dl.y;
        sGN[ch0] = gm.x * dl.x;
        sGN[ch0 + 1] = gm.y * dl.y;
      }
    }
    __syncthreads();

    // ---- step 2: A = beta * strict_lower(Kl Kr^T), P = lower(Ql Kr^T) -------
    {
      // 16x16 tile pairs (R, I), I <= R, spread over the waves.
      int tr[3], ti[3], np;
      if (w == 0) { tr[0] = 3; ti[0] = 0; tr[1] = 3; ti[1] = 1; tr[2] = 0; ti[2] = 0; np = 3; }
      else if (w == 1) { tr[0] = 3; ti[0] = 2; tr[1] = 3; ti[1] = 3; tr[2] = 1; ti[2] = 0; np = 3; }
      else if (w == 2) { tr[0] = 2; ti[0] = 0; tr[1] = 2; ti[1] = 1; tr[2] = 0; ti[2] = 0; np = 2; }
      else { tr[0] = 2; ti[0] = 2; tr[1] = 1; ti[1] = 1; tr[2] = 0; ti[2] = 0; np = 2; }
      f4 accA[3], accP[3];
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        accA[j] = f4{0.f, 0.f, 0.f, 0.f};
        accP[j] = accA[j];
        if (j < np) {
#pragma unroll 2
          for (int kc = 0; kc < DK / M::KU; ++kc) {
            auto bk = M::load(sKr, L::P_OP, 16 * ti[j], kc);
            auto ak = M::load(sKl, L::P_OP, 16 * tr[j], kc);
            auto aq = M::load(sQl, L::P_OP, 16 * tr[j], kc);
            accA[j] = M::mma(ak, bk, accA[j]);
            accP[j] = M::mma(aq, bk, accP[j]);
          }
        }
      }
      __syncthreads();  // every read of Kr is done: A and P overwrite it
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        if (j < np) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r = 16 * tr[j] + 4 * lg + q;
            const int i = 16 * ti[j] + lr;
            sA[r * L::P_AF + i] = i < r ? sBe[r] * accA[j][q] : 0.f;
            st1<BF>(sP, L::P_T, r, i, i <= r ? accP[j][q] : 0.f);
          }
        }
      }
      // Upper tiles of P that the 32-wide K chunks of the P U product touch.
      if (w == 2 || w == 3) {
        const int R = w == 2 ? 0 : 2;
#pragma unroll
        for (int q = 0; q < 4; ++q) st1<BF>(sP, L::P_T, 16 * R + 4 * lg + q, 16 * (R + 1) + lr, 0.f);
      }
    }
    __syncthreads();

    // ---- step 3: T = (I + A)^-1 Diag(beta) ---------------------------------
    // 3a: inverses of the four 16x16 unit-lower diagonal blocks by forward
    // substitution (lane = (block, column)); the other waves clear the upper
    // blocks.
    if (w == 0) {
      const int R = lg, j = lr;
      const float* Ab = sA + 16 * R * L::P_AF + 16 * R;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float s = r == j ? 1.f : 0.f;
#pragma unroll
        for (int i = 0; i < r; ++i) s -= Ab[r * L::P_AF + i] * x[i];
        x[r] = s;
      }
      float* Lb = sLi + 16 * R * L::P_AF + 16 * R;
#pragma unroll
      for (int r = 0; r < 16; ++r) Lb[r * L::P_AF + j] = x[r];
    } else {
      // blocks (R, I) with I > R: (0,1) (0,2) (0,3) (1,2) (1,3) (2,3)
      for (int e = t - 64; e < 6 * 256; e += 192) {
        const int blk = e >> 8, rr = (e >> 4) & 15, cc = e & 15;
        const int R = blk < 3 ? 0 : (blk < 5 ? 1 : 2);
        const int I = blk < 3 ? blk + 1 : (blk < 5 ? blk - 1 : 3);
        sLi[(16 * R + rr) * L::P_AF + 16 * I + cc] = 0.f;
      }
    }
    __syncthreads();
    // 3b: off-diagonal blocks, L^-1_RI = -D_R sum_{I<=J<R} A_RJ L^-1_JI,
    // level by level; each thread computes one element of each 16x16 block.
    {
      const int rr = t >> 4, cc = t & 15;
      auto Ab = [&](int R, int I) { return sA + 16 * R * L::P_AF + 16 * I; };
      auto Lb = [&](int R, int I) { return sLi + 16 * R * L::P_AF + 16 * I; };
      auto mm = [&](const float* X, int xp, const float* Y, int yp) {
        float s = 0.f;
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) s += X[rr * xp + kk] * Y[kk * yp + cc];
        return s;
      };
      constexpr int pf = L::P_AF;
      // level 1: X_{s,s-1} = -D_s A_{s,s-1} D_{s-1}
#pragma unroll
      for (int s = 1; s < 4; ++s) sTmp[(s - 1) * 256 + t] = mm(Ab(s, s - 1), pf, Lb(s - 1, s - 1), pf);
      __syncthreads();
#pragma unroll
      for (int s = 1; s < 4; ++s) Lb(s, s - 1)[rr * pf + cc] = -mm(Lb(s, s), pf, sTmp + (s - 1) * 256, 16);
      __syncthreads();
      // level 2: X_20 = -D_2 (A_20 D_0 + A_21 X_10), X_31 = -D_3 (A_31 D_1 + A_32 X_21)
      sTmp[t] = mm(Ab(2, 0), pf, Lb(0, 0), pf) + mm(Ab(2, 1), pf, Lb(1, 0), pf);
      sTmp[256 + t] = mm(Ab(3, 1), pf, Lb(1, 1), pf) + mm(Ab(3, 2), pf, Lb(2, 1), pf);
      __syncthreads();
      Lb(2, 0)[rr * pf + cc] = -mm(Lb(2, 2), pf, sTmp, 16);
      Lb(3, 1)[rr * pf + cc] = -mm(Lb(3, 3), pf, sTmp + 256, 16);
      __syncthreads();
      // level 3: X_30 = -D_3 (A_30 D_0 + A_31 X_10 + A_32 X_20)
      sTmp[t] = mm(Ab(3, 0), pf, Lb(0, 0), pf) + mm(Ab(3, 1), pf, Lb(1, 0), pf) +
                mm(Ab(3, 2), pf, Lb(2, 0), pf);
      __syncthreads();
      Lb(3, 0)[rr * pf + cc] = -mm(Lb(3, 3), pf, sTmp, 16);
      __syncthreads();
    }
    // 3c: T = L^-1 Diag(beta), converted in place to the operand format
    // (an 8-element group of fp32 occupies exactly the bytes of its hi/lo form).
#pragma unroll
    for (int e = t; e < kC * 8; e += kNT) {
      const int r = e >> 3, g8 = e & 7;
      float x[8];
      const float* src = sLi + r * L::P_AF + 8 * g8;
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = src[i] * sBe[8 * g8 + i];
      st8<BF>(sT, L::P_T, r, 8 * g8, x);
    }
    __syncthreads();

    // ---- step 4: the state pass, 16 value columns at a time ----------------
#pragma unroll
    for (int js = 0; js < NSUB; ++js) {
      // 4a: S_B^T = (Diag(gamma_m) S)^T for these columns.
#pragma unroll
      for (int tt = 0; tt < TPW; ++tt) {
        const int c0 = 16 * (w * TPW + tt) + 4 * lg;
        float x[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) x[q] = S[js][tt][q] * sGM[c0 + q];
        st4<BF>(sSBT, L::P_OP, lr, c0, x);
      }
      __syncthreads();
      // 4b: X = V - Kl S_B  (rows 16w..16w+15)
      {
        f4 acc = gemm<BF>(f4{0.f, 0.f, 0.f, 0.f}, sKl, L::P_OP, 16 * w, sSBT, L::P_OP, 0, 0, DK);
        float x[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) x[q] = vreg[js][q] - acc[q];
        st4<BF>(sXT, L::P_T, lr, 16 * w + 4 * lg, x);
      }
      __syncthreads();
      // 4c: U = T X  (T is lower triangular: K up to the end of this row block)
      const int kend = BF ? 32 * ((w + 2) >> 1) : 16 * (w + 1);
      {
        f4 acc = gemm<BF>(f4{0.f, 0.f, 0.f, 0.f}, sT, L::P_T, 16 * w, sXT, L::P_T, 0, 0, kend);
        float x[4] = {acc[0], acc[1], acc[2], acc[3]};
        st4<BF>(sUT, L::P_T, lr, 16 * w + 4 * lg, x);
      }
      __syncthreads();
      // 4d: O = Ql S_B + P U
      {
        f4 acc = gemm<BF>(f4{0.f, 0.f, 0.f, 0.f}, sQl, L::P_OP, 16 * w, sSBT, L::P_OP, 0, 0, DK);
        acc = gemm<BF>(acc, sP, L::P_T, 16 * w, sUT, L::P_T, 0, 0, kend);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = 16 * w + 4 * lg + q;
          if (r < nv) p.o[((tok0 + r) * H + h) * int64_t(DV) + col0 + 16 * js + lr] = acc[q];
        }
      }
      // 4e: S' = Diag(gamma_n) S + Diag(gamma_n / gamma_m) Kr^T U
#pragma unroll
      for (int tt = 0; tt < TPW; ++tt) {
        const int tc = w * TPW + tt;
        f4 acc = gemm<BF>(f4{0.f, 0.f, 0.f, 0.f}, sKrT, L::P_T, 16 * tc, sUT, L::P_T, 0, 0, kC);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = 16 * tc + 4 * lg + q;
          S[js][tt][q] = sGN[c] * S[js][tt][q] + sDL[c] * acc[q];
        }
      }
      __syncthreads();
    }
  }

  if (p.s_out) {
#pragma unroll
    for (int js = 0; js < NSUB; ++js)
#pragma unroll
      for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = 16 * (w * TPW + tt) + 4 * lg + q;
          p.s_out[sbase + int64_t(c) * DV + col0 + 16 * js + lr] = S[js][tt][q];
        }
  }
}

template <int DK, int NSUB, bool BF>
void launch_t(const Params& p, int64_t nblocks, hipStream_t st) {
  hipLaunchKernelGGL((kda_prefill_kernel<DK, NSUB, BF>), dim3(unsigned(nblocks)), dim3(kNT), 0,
                     st, p);
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
  if (const char* e = getenv("KDA_PREFILL_NSUB")) {
    const int v = atoi(e);
    if ((v == 1 || v == 2 || v == 4 || v == 8) && 16 * v <= DV) return v;
  }
  for (int nsub = DV / 16; nsub > 1; nsub >>= 1)
    if (pairs * (DV / (16 * nsub)) >= 256) return nsub;
  return 1;
}

}  // namespace

size_t prefill_workspace_bytes(int, int64_t, int, int, int) { return 0; }

int launch_prefill(const PrefillArgs& a, void* stream, const char** msg) {
  hipStream_t st = static_cast<hipStream_t>(stream);
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
  const int64_t pairs = int64_t(a.N) * a.H;
  const int nsub = choose_nsub(pairs, a.DV);
  p.nslab = a.DV / (16 * nsub);
  const int64_t nblocks = pairs * p.nslab;
  (void)hipGetLastError();
  if (a.DK == 128) {
    if (a.in_bf16) launch_dk<128, true>(p, nsub, nblocks, st);
    else launch_dk<128, false>(p, nsub, nblocks, st);
  } else if (a.DK == 64) {
    if (a.in_bf16) launch_dk<64, true>(p, nsub, nblocks, st);
    else launch_dk<64, false>(p, nsub, nblocks, st);
  } else {
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

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
  static constexpr int OFF_SBT = OFF_X;                      // S_B^T [16][DK]  (after the solve)
  static constexpr int OFF_XT = OFF_SBT + 16 * P_OP;         // X^T [16][64]
  static constexpr int OFF_UT = OFF_XT + 16 * P_T;           // U^T [16][64]
  static constexpr int OFF_T = OFF_X + SZ_X;                 // T [64][64] (fp32 L^-1 first)
  static constexpr int OFF_TMP = OFF_T + kC * P_T;           // 3 x 16x16 fp32 (solve)
  static constexpr int RG = 8;                               // row groups of the decay prep
  static constexpr int OFF_GP = OFF_TMP + 3 * 256 * 4;       // group products [RG][DK]
  static constexpr int OFF_GM = OFF_GP + RG * DK * 4;        // gamma_m [DK]
  static constexpr int OFF_DL = OFF_GM + DK * 4;             // gamma_n / gamma_m [DK]
  static constexpr int OFF_GN = OFF_DL + DK * 4;             // gamma_n [DK]
  static constexpr int OFF_BE = OFF_GN + DK * 4;             // beta [64]
  static constexpr int TOTAL = OFF_BE + kC * 4;
  static_assert(NT == RG * DK / 2, "decay prep: one thread per (channel pair, row group)");
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

// Raw (unconverted) input words, so that prefetched loads are not consumed
// before they are needed: a bf16 pair / bf16 value, or fp32.
template <bool BF> struct Raw { typedef uint32_t two; typedef uint32_t one; };
template <> struct Raw<false> { typedef float2 two; typedef float one; };

template <bool BF>
__device__ __forceinline__ typename Raw<BF>::two ldraw2(const void* p, int64_t i) {
  if constexpr (BF) return *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p) + i);
  else return *reinterpret_cast<const float2*>(static_cast<const float*>(p) + i);
}
template <bool BF>
__device__ __forceinline__ typename Raw<BF>::one ldraw1(const void* p, int64_t i) {
  if constexpr (BF) return uint32_t(static_cast<const uint16_t*>(p)[i]);
  else return static_cast<const float*>(p)[i];
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


// Destination of output stores for rows past the end of a sequence (never read).
__device__ float g_sink[256 * 64];

// A and P tiles of up to three (R, I) pairs (R < 0: unused) of one wave.
// Each row block of Kl/Ql and column block of Kr is loaded once per K chunk
// and shared by the pair's two products (the LDS read bandwidth, not the
// MFMA rate, bounds this step).
template <bool BF, int DK, int R0, int I0, int R1, int I1, int R2, int I2>
__device__ __forceinline__ void ap_tiles(const char* sKl, const char* sQl, const char* sKr,
                                         f4 (&accA)[3], f4 (&accP)[3]) {
  using M = Mma<BF>;
  constexpr int P = DK * 4 + 16;
#pragma unroll
  for (int kc = 0; kc < DK / M::KU; ++kc) {
    const auto kr0 = M::load(sKr, P, 16 * I0, kc);
    const auto kl0 = M::load(sKl, P, 16 * R0, kc);
    const auto ql0 = M::load(sQl, P, 16 * R0, kc);
    accA[0] = M::mma(kl0, kr0, accA[0]);
    accP[0] = M::mma(ql0, kr0, accP[0]);
    if constexpr (R1 >= 0) {
      const auto kr1 = M::load(sKr, P, 16 * I1, kc);
      const auto kl1 = (R1 == R0) ? kl0 : M::load(sKl, P, 16 * R1, kc);
      const auto ql1 = (R1 == R0) ? ql0 : M::load(sQl, P, 16 * R1, kc);
      accA[1] = M::mma(kl1, kr1, accA[1]);
      accP[1] = M::mma(ql1, kr1, accP[1]);
      if constexpr (R2 >= 0) {
        const auto kr2 = (I2 == I0) ? kr0 : ((I2 == I1) ? kr1 : M::load(sKr, P, 16 * I2, kc));
        const auto kl2 = (R2 == R1) ? kl1 : M::load(sKl, P, 16 * R2, kc);
        const auto ql2 = (R2 == R1) ? ql1 : M::load(sQl, P, 16 * R2, kc);
        accA[2] = M::mma(kl2, kr2, accA[2]);
        accP[2] = M::mma(ql2, kr2, accP[2]);
      }
    }
  }
}


// ------------------------------------------------------------------ kernel --
template <int DK, int NSUB, bool BF>
__global__ __launch_bounds__(64 * (DK / 16), 1) void kda_prefill_kernel(Params p) {
  using L = Lay<DK>;
  using M = Mma<BF>;
  constexpr int NW = L::NW;         // waves; wave w owns rows 16w..16w+15 of the state
  constexpr int NT = L::NT;
  constexpr int NP = DK / 2;        // channel pairs in the decay prep
  constexpr int RG = L::RG;         // row groups in the decay prep
  constexpr int RPG = kC / RG;      // rows per group (8)
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

  // State slab in registers: S[js][q] = S[16w + 4lg + q][col0 + 16js + lr].
  f4 S[NSUB];
  const int64_t sbase = (int64_t(n) * H + h) * DK * DV;
#pragma unroll
  for (int js = 0; js < NSUB; ++js)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      S[js][q] = p.s_in ? p.s_in[sbase + int64_t(16 * w + 4 * lg + q) * DV + col0 + 16 * js + lr]
                        : 0.f;

  // Decay prep: thread = (channel pair, group of 8 rows).
  const int cp = t % NP, grp = t / NP;
  const int ch0 = 2 * cp;
  const int rb = grp * RPG;

  // Raw inputs of the next chunk, loaded one chunk ahead.  Every load is
  // unconditional: rows past the sequence end are clamped to its last row
  // and their values discarded.
  typename Raw<BF>::two pk[RPG], pq[RPG];
  float2 pa[RPG];
  float pb = 0.f;
  typename Raw<BF>::one pv[NSUB][4];
  const int rsk = H * DK, rsv = H * DV;  // token strides (elements)
  auto load_chunk = [&](int64_t c0, int nvv) {
    const int64_t kb = (c0 * H + h) * int64_t(DK) + ch0;
#pragma unroll
    for (int i = 0; i < RPG; ++i) {
      const int r = rb + i < nvv ? rb + i : nvv - 1;
      const int64_t idx = kb + r * rsk;
      pa[i] = *reinterpret_cast<const float2*>(p.alpha + idx);
      pk[i] = ldraw2<BF>(p.k, idx);
      pq[i] = ldraw2<BF>(p.q, idx);
    }
    pb = p.beta[(c0 + ((t & 63) < nvv ? (t & 63) : nvv - 1)) * H + h];
    {
      // (waves 4.. load the rows of waves 0..3 again: keeps the loads unconditional)
      const int64_t vb = (c0 * H + h) * int64_t(DV) + col0 + lr;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r0 = 16 * (w & 3) + 4 * lg + q;
        const int r = r0 < nvv ? r0 : nvv - 1;
#pragma unroll
        for (int js = 0; js < NSUB; ++js) pv[js][q] = ldraw1<BF>(p.v, vb + r * rsv + 16 * js);
      }
    }
  };
  if (s0 < s1) load_chunk(s0, int(s1 - s0 < kC ? s1 - s0 : kC));
  {
    // Mirror the output stores that follow the prefetch in every later chunk,
    // so that the first chunk and the steady state agree on how many memory
    // operations are in flight after the prefetched loads (otherwise the
    // compiler's wait for them degrades to waiting for every store).
    volatile float* sink = g_sink + ((blockIdx.x & 255) << 6) + l;
#pragma unroll
    for (int i = 0; i < 4 * NSUB; ++i) *sink = 0.f;
  }

  for (int64_t tok0 = s0; tok0 < s1; tok0 += kC) {
    const int nv = int(s1 - tok0 < kC ? s1 - tok0 : kC);

    // ---- take this chunk's inputs, start loading the next chunk's --------
    float2 av[RPG], kv[RPG], qv[RPG];
#pragma unroll
    for (int i = 0; i < RPG; ++i) {
      const bool ok = rb + i < nv;
      av[i] = ok ? pa[i] : make_float2(1.f, 1.f);
      const float2 kk = cvt2<BF>(pk[i]), qq = cvt2<BF>(pq[i]);
      kv[i] = ok ? kk : make_float2(0.f, 0.f);
      qv[i] = ok ? qq : make_float2(0.f, 0.f);
    }
    const float bev = (t & 63) < nv ? pb : 0.f;
    float vreg[NSUB][4];
#pragma unroll
    for (int js = 0; js < NSUB; ++js)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        vreg[js][q] = (16 * (w & 3) + 4 * lg + q) < nv ? cvt1<BF>(pv[js][q]) : 0.f;
    if (tok0 + kC < s1) load_chunk(tok0 + kC, int(s1 - tok0 - kC < kC ? s1 - tok0 - kC : kC));

    // ---- step 1: decay factors and decayed operands ------------------------
    {
      float2 gp = make_float2(1.f, 1.f);
#pragma unroll
      for (int i = 0; i < RPG; ++i) {
        gp.x *= av[i].x;
        gp.y *= av[i].y;
      }
      sGP[grp * DK + ch0] = gp.x;
      sGP[grp * DK + ch0 + 1] = gp.y;
      if (t < kC) sBe[t] = bev;
    }
    lds_barrier();
    {
      float2 krs[RPG];
      constexpr int half = RG / 2;  // groups before / after the reference row
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
      // Kr^T rows (= key channels): this thread's 8 tokens of two channels.
      float x0[RPG], x1[RPG];
#pragma unroll
      for (int e = 0; e < RPG; ++e) {
        x0[e] = krs[e].x;
        x1[e] = krs[e].y;
      }
      st8<BF>(sKrT, L::P_T, ch0, rb, x0);
      st8<BF>(sKrT, L::P_T, ch0 + 1, rb, x1);
      if (grp == 0) {
        float2 gm = make_float2(1.f, 1.f), dl = make_float2(1.f, 1.f);
#pragma unroll
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
    lds_barrier();

    // ---- step 2: A = beta * strict_lower(Kl Kr^T), P = lower(Ql Kr^T) -------
    {
      // The 10 tile pairs (R, I), I <= R, grouped per wave by shared blocks.
      f4 accA[3], accP[3];
#pragma unroll
      for (int j = 0; j < 3; ++j) accA[j] = accP[j] = f4{0.f, 0.f, 0.f, 0.f};
      int pR[3] = {-1, -1, -1}, pI[3] = {0, 0, 0};
      if constexpr (NW >= 8) {
        switch (w) {
          case 0: ap_tiles<BF, DK, 3, 0, 3, 1, -1, 0>(sKl, sQl, sKr, accA, accP); pR[0] = 3; pI[0] = 0; pR[1] = 3; pI[1] = 1; break;
          case 1: ap_tiles<BF, DK, 3, 2, 3, 3, -1, 0>(sKl, sQl, sKr, accA, accP); pR[0] = 3; pI[0] = 2; pR[1] = 3; pI[1] = 3; break;
          case 2: ap_tiles<BF, DK, 2, 0, 2, 1, -1, 0>(sKl, sQl, sKr, accA, accP); pR[0] = 2; pI[0] = 0; pR[1] = 2; pI[1] = 1; break;
          case 3: ap_tiles<BF, DK, 2, 2, -1, 0, -1, 0>(sKl, sQl, sKr, accA, accP); pR[0] = 2; pI[0] = 2; break;
          case 4: ap_tiles<BF, DK, 1, 0, 1, 1, -1, 0>(sKl, sQl, sKr, accA, accP); pR[0] = 1; pI[0] = 0; pR[1] = 1; pI[1] = 1; break;
          case 5: ap_tiles<BF, DK, 0, 0, -1, 0, -1, 0>(sKl, sQl, sKr, accA, accP); pR[0] = 0; pI[0] = 0; break;
          default: break;
        }
      } else {
        switch (w) {
          case 0: ap_tiles<BF, DK, 3, 0, 3, 1, 3, 2>(sKl, sQl, sKr, accA, accP); pR[0] = 3; pI[0] = 0; pR[1] = 3; pI[1] = 1; pR[2] = 3; pI[2] = 2; break;
          case 1: ap_tiles<BF, DK, 3, 3, 2, 2, 1, 1>(sKl, sQl, sKr, accA, accP); pR[0] = 3; pI[0] = 3; pR[1] = 2; pI[1] = 2; pR[2] = 1; pI[2] = 1; break;
          case 2: ap_tiles<BF, DK, 2, 0, 2, 1, 1, 0>(sKl, sQl, sKr, accA, accP); pR[0] = 2; pI[0] = 0; pR[1] = 2; pI[1] = 1; pR[2] = 1; pI[2] = 0; break;
          default: ap_tiles<BF, DK, 0, 0, -1, 0, -1, 0>(sKl, sQl, sKr, accA, accP); pR[0] = 0; pI[0] = 0; break;
        }
      }
      lds_barrier();  // every read of Kr is done: A and P overwrite it
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        if (pR[j] >= 0) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r = 16 * pR[j] + 4 * lg + q;
            const int i = 16 * pI[j] + lr;
            st1<BF>(sP, L::P_T, r, i, i <= r ? accP[j][q] : 0.f);
            sA[r * L::P_AF + i] = i < r ? sBe[r] * accA[j][q] : 0.f;
          }
        }
      }
      // Upper tiles of P that the 32-wide K chunks of the P U product touch.
      if (w == NW - 1) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          st1<BF>(sP, L::P_T, 4 * lg + q, 16 + lr, 0.f);
          st1<BF>(sP, L::P_T, 32 + 4 * lg + q, 48 + lr, 0.f);
        }
      }
    }
    lds_barrier();

    // ---- step 3: T = (I + A)^-1 Diag(beta) ---------------------------------
    // 3a: inverses D_R of the four 16x16 unit-lower diagonal blocks by forward
    // substitution (wave 0, lane = (block, column)); the other waves clear the
    // upper blocks of L^-1.
    if (w == 0) {
      const int R = lg, j = lr;
      const float* Ab = sA + 16 * R * L::P_AF + 16 * R;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float s = r == j ? 1.f : 0.f;
#pragma unroll
        for (int i4 = 0; i4 < r; i4 += 4) {
          const float4 a4 = *reinterpret_cast<const float4*>(Ab + r * L::P_AF + i4);
          s -= a4.x * x[i4];
          if (i4 + 1 < r) s -= a4.y * x[i4 + 1];
          if (i4 + 2 < r) s -= a4.z * x[i4 + 2];
          if (i4 + 3 < r) s -= a4.w * x[i4 + 3];
        }
        x[r] = s;
      }
      float* Lb = sLi + 16 * R * L::P_AF + 16 * R;
#pragma unroll
      for (int r = 0; r < 16; ++r) Lb[r * L::P_AF + j] = x[r];
    } else {
      // blocks (R, I) with I > R: (0,1) (0,2) (0,3) (1,2) (1,3) (2,3)
      for (int e = t - 64; e < 6 * 256; e += NT - 64) {
        const int blk = e >> 8, rr = (e >> 4) & 15, cc = e & 15;
        const int R = blk < 3 ? 0 : (blk < 5 ? 1 : 2);
        const int I = blk < 3 ? blk + 1 : (blk < 5 ? blk - 1 : 3);
        sLi[(16 * R + rr) * L::P_AF + 16 * I + cc] = 0.f;
      }
    }
    lds_barrier();
    // 3b: off-diagonal blocks row block by row block:
    //     L^-1_{R,I} = -D_R (sum_{I<=J<R} A_{R,J} L^-1_{J,I}),  wave I, fp32 MFMA.
#pragma unroll
    for (int R = 1; R < 4; ++R) {
      if (w < R) {
        const int I = w;
        f4 y = f4{0.f, 0.f, 0.f, 0.f};
        for (int J = I; J < R; ++J) {
#pragma unroll
          for (int s4 = 0; s4 < 4; ++s4) {
            const float a = sA[(16 * R + lr) * L::P_AF + 16 * J + 4 * s4 + lg];
            const float bb = sLi[(16 * J + 4 * s4 + lg) * L::P_AF + 16 * I + lr];
            y = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bb, y, 0, 0, 0);
          }
        }
        float* tmp = sTmp + 256 * I;
#pragma unroll
        for (int q = 0; q < 4; ++q) tmp[(4 * lg + q) * 16 + lr] = y[q];
        f4 x = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const float a = sLi[(16 * R + lr) * L::P_AF + 16 * R + 4 * s4 + lg];
          const float bb = tmp[(4 * s4 + lg) * 16 + lr];
          x = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bb, x, 0, 0, 0);
        }
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

    // ---- step 4: the state pass, 16 value columns at a time ----------------
    // Waves 0..3 compute X and U for rows 16w..; the output rows 16*ow.. are
    // computed by waves 4..7 when there are eight waves (their Ql S_B product
    // overlaps X and U), else by waves 0..3 after U.
    constexpr bool kSplitO = NW >= 8;
    const bool xw = w < 4;
    const bool owave = kSplitO ? (w >= 4) : (w < 4);
    const int ow = w & 3;
    const int kend_u = BF ? 32 * ((w + 2) >> 1) : 16 * (w + 1);
    const int kend_o = BF ? 32 * ((ow + 2) >> 1) : 16 * (ow + 1);
#pragma unroll
    for (int js = 0; js < NSUB; ++js) {
      // 4a: S_B^T = (Diag(gamma_m) S)^T for these columns.
      {
        const int c0 = 16 * w + 4 * lg;
        float x[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) x[q] = S[js][q] * sGM[c0 + q];
        st4<BF>(sSBT, L::P_OP, lr, c0, x);
      }
      lds_barrier();
      // 4b: X = V - Kl S_B; the output waves start O = Ql S_B.
      f4 acco = f4{0.f, 0.f, 0.f, 0.f};
      if (xw) {
        f4 acc = gemm<BF>(f4{0.f, 0.f, 0.f, 0.f}, sKl, L::P_OP, 16 * w, sSBT, L::P_OP, 0, 0, DK);
        float x[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) x[q] = vreg[js][q] - acc[q];
        st4<BF>(sXT, L::P_T, lr, 16 * w + 4 * lg, x);
      }
      if (kSplitO && owave)
        acco = gemm<BF>(acco, sQl, L::P_OP, 16 * ow, sSBT, L::P_OP, 0, 0, DK);
      lds_barrier();
      // 4c: U = T X  (T is lower triangular: K up to the end of this row block)
      if (xw) {
        f4 acc = gemm<BF>(f4{0.f, 0.f, 0.f, 0.f}, sT, L::P_T, 16 * w, sXT, L::P_T, 0, 0, kend_u);
        float x[4] = {acc[0], acc[1], acc[2], acc[3]};
        st4<BF>(sUT, L::P_T, lr, 16 * w + 4 * lg, x);
      }
      lds_barrier();
      // 4d: O = Ql S_B + P U
      if (owave) {
        if constexpr (!kSplitO)
          acco = gemm<BF>(acco, sQl, L::P_OP, 16 * ow, sSBT, L::P_OP, 0, 0, DK);
        acco = gemm<BF>(acco, sP, L::P_T, 16 * ow, sUT, L::P_T, 0, 0, kend_o);
      }
      {
        // Every wave issues the stores; rows past the end of the sequence and
        // waves without output rows store into a sink.  Unconditional stores
        // stay visible to the compiler's memory-counter bookkeeping, so taking
        // the prefetched inputs never waits for output stores to drain.
        float* orow = p.o + ((tok0 + 16 * ow + 4 * lg) * H + h) * int64_t(DV) + col0 + 16 * js + lr;
        float* sink = g_sink + ((blockIdx.x & 255) << 6) + l;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float* dst = owave && 16 * ow + 4 * lg + q < nv ? orow + int64_t(q) * H * DV : sink;
          *dst = acco[q];
        }
      }
      // 4e: S' = Diag(gamma_n) S + Diag(gamma_n / gamma_m) Kr^T U  (rows 16w..)
      {
        f4 acc = gemm<BF>(f4{0.f, 0.f, 0.f, 0.f}, sKrT, L::P_T, 16 * w, sUT, L::P_T, 0, 0, kC);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = 16 * w + 4 * lg + q;
          S[js][q] = sGN[c] * S[js][q] + sDL[c] * acc[q];
        }
      }
      lds_barrier();
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

template <int DK, int NSUB, bool BF>
void launch_t(const Params& p, int64_t nblocks, hipStream_t st) {
  hipLaunchKernelGGL((kda_prefill_kernel<DK, NSUB, BF>), dim3(unsigned(nblocks)),
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

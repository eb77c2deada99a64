// KDA backward pass on gfx950: gradients of the operator's outputs with
// respect to q, k, v, alpha, beta and the initial state.
//
// The chunk algorithm regroups the token recurrence of "Kimi Delta Attention
// 徹底解説" (tech-tide.dev), section "Kimi Delta Attention の仕組み"; its gradient
// is the gradient of that recurrence.  Reverse mode of one token
//     St = Diag(a) S;  p = St^T k;  u = b (v - p);  S' = St + k u^T;  o = S'^T q
// with G the adjoint of S' (including o's term q do^T) gives
//     dq = S' do;  du = G^T k;  dv = b du;  db = du . (v - p);  dp = -b du
//     dSt = G + k dp^T;  dk = G u + St dp;  da = rowsum(dSt * S);  G <- Diag(a) dSt
//
// Plan of a call:
//   1. the forward prefill with a state snapshot after every chunk (the
//      states at chunk starts are the checkpoints);
//   2. kda_bwd_kernel: one workgroup per (sequence, head, 16 value columns).
//      Every step above keeps value columns apart except the row sums (dq,
//      dk, da) and db, so the slab of G and of the state needs no exchange;
//      the row sums go to per-slab partial buffers.  Chunks are visited from
//      the last to the first.  While chunk c is walked backwards, chunk c-1's
//      token states are recomputed forward from its checkpoint into the other
//      half of a per-workgroup scratch: the two token chains are independent,
//      so their latencies overlap;
//   3. kda_bwd_reduce_kernel: sums the per-slab partials (a fixed order, so
//      the result is deterministic).
//
// Layout: wave w of a workgroup owns value columns 4w .. 4w+3 of the
// workgroup's 16 and every key row (lane l holds rows DK/64 * l ..), so the
// column sums of a step (St^T k and G^T k) are reductions inside one wave
// (DPP within rows of 16 lanes, then row broadcasts into the last row, whose
// lane 63 is read out): no barrier for them.  The row sums (dq, dk, da, over
// the wave's 4 columns) and db are
// outputs only: each wave stages them in LDS and after one barrier per token
// the workgroup adds the four waves' values in a fixed order and writes the
// slab's partials.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kC = 64;     // chunk length (checkpoint interval)
constexpr int kVS = 16;    // value columns per workgroup
constexpr int kCPW = 4;    // value columns per wave
constexpr int kNW = kVS / kCPW;   // waves per workgroup
constexpr int kNT = 64 * kNW;     // threads per workgroup

__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int N>
__device__ __forceinline__ void ld_f(const float* p, float (&x)[N]) {
  if constexpr (N == 2) {
    const float2 a = *reinterpret_cast<const float2*>(p);
    x[0] = a.x;
    x[1] = a.y;
  } else {
    x[0] = p[0];
  }
}

// N = 2 or 4 consecutive floats (8- or 16-byte aligned).
template <int N>
__device__ __forceinline__ void ldfn(const float* p, float* x) {
  if constexpr (N == 4) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  } else {
    static_assert(N == 2, "two or four floats");
    const float2 a = *reinterpret_cast<const float2*>(p);
    x[0] = a.x; x[1] = a.y;
  }
}

template <int N>
__device__ __forceinline__ void stfn(float* p, const float* x) {
  if constexpr (N == 4) {
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  } else {
    static_assert(N == 2, "two or four floats");
    *reinterpret_cast<float2*>(p) = make_float2(x[0], x[1]);
  }
}

// E floats in pieces of at most four.
template <int E>
__device__ __forceinline__ void ld_elems(const float* p, float* x) {
#pragma unroll
  for (int e = 0; e < E; e += (E >= 4 ? 4 : E)) ldfn<(E >= 4 ? 4 : E)>(p + e, x + e);
}

template <int E>
__device__ __forceinline__ void st_elems(float* p, const float* x) {
#pragma unroll
  for (int e = 0; e < E; e += (E >= 4 ? 4 : E)) stfn<(E >= 4 ? 4 : E)>(p + e, x + e);
}

// Key rows (RPL of them) or four value columns of a bf16 or float input, kept
// as loaded and converted at use (so that a prefetched value is not waited
// for where it is loaded).
template <bool BF16, int RPL>
struct RowsIn;
template <int RPL>
struct RowsIn<true, RPL> {
  uint32_t w;
  __device__ void load(const void* p, int64_t i) {
    const uint16_t* b = static_cast<const uint16_t*>(p) + i;
    if constexpr (RPL == 2) w = *reinterpret_cast<const uint32_t*>(b);
    else w = *b;
  }
  __device__ float operator[](int r) const {
    return r == 0 ? __uint_as_float(w << 16) : __uint_as_float(w & 0xffff0000u);
  }
};
template <int RPL>
struct RowsIn<false, RPL> {
  float x[RPL];
  __device__ void load(const void* p, int64_t i) { ld_f<RPL>(static_cast<const float*>(p) + i, x); }
  __device__ float operator[](int r) const { return x[r]; }
};
template <bool BF16>
struct ColsIn;
template <>
struct ColsIn<true> {
  uint32_t w[kCPW / 2];
  __device__ void load(const void* p, int64_t i) {
    const uint16_t* b = static_cast<const uint16_t*>(p) + i;
    if constexpr (kCPW == 4) {
      const uint2 r = *reinterpret_cast<const uint2*>(b);
      w[0] = r.x;
      w[kCPW / 2 - 1] = r.y;
    } else {
      w[0] = *reinterpret_cast<const uint32_t*>(b);
    }
  }
  __device__ float operator[](int e) const {
    const uint32_t x = w[e >> 1];
    return (e & 1) ? __uint_as_float(x & 0xffff0000u) : __uint_as_float(x << 16);
  }
};
template <>
struct ColsIn<false> {
  float x[kCPW];
  __device__ void load(const void* p, int64_t i) { ldfn<kCPW>(static_cast<const float*>(p) + i, x); }
  __device__ float operator[](int e) const { return x[e]; }
};

// Sum of the kNW per-wave values r[0], r[stride], ..., pairwise.
__device__ __forceinline__ float sum_waves(const float* r, int stride) {
  float x[kNW];
#pragma unroll
  for (int i = 0; i < kNW; ++i) x[i] = r[i * stride];
#pragma unroll
  for (int h = 1; h < kNW; h <<= 1)
#pragma unroll
    for (int i = 0; i + h < kNW; i += 2 * h) x[i] += x[i + h];
  return x[0];
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                                0xF, 0xF, false));
}

__device__ __forceinline__ float lane_val(float x, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_rows(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                                ROWS, 0xF, false));
}

// Sums over the 64 lanes of a wave of N values each (every lane gets the
// totals): lane pairs and quads, then rotations by 4 and 8 inside each row
// of 16 lanes (every lane holds its row's sum), then lane 15 of rows 0 and 2
// added into rows 1 and 3 and lane 31 into rows 2 and 3, so that lane 63
// holds (r2 + r3) + (r0 + r1); it is read out for all lanes.
template <int N>
__device__ __forceinline__ void wave_sums(float (&x)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] += dpp<0xB1>(x[i]);    // quad_perm [1,0,3,2]
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] += dpp<0x4E>(x[i]);    // quad_perm [2,3,0,1]
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] += dpp<0x124>(x[i]);   // row_ror:4
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] += dpp<0x128>(x[i]);   // row_ror:8
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] += dpp_rows<0x142, 0xA>(x[i]);   // row_bcast:15 into rows 1, 3
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] += dpp_rows<0x143, 0xC>(x[i]);   // row_bcast:31 into rows 2, 3
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = lane_val(x[i], 63);
}

// SG: one gate per token and head (alpha [rows]), the same for every key row.
template <int DK, bool BF16, bool SG>
__global__ __launch_bounds__(kNT) void kda_bwd_kernel(BackwardArgs p) {
  constexpr int RPL = DK / 64;       // key rows per lane
  constexpr int E = RPL * kCPW;      // state elements per lane
  __shared__ float sU[2][kC][kVS];   // u of a chunk's tokens (this slab), two chunks
  __shared__ float sR[2][kC][kVS];   // v - p
  __shared__ float ring[2][3][kNW][DK];   // dq, dk, da per wave, two tokens
  __shared__ float ringb[2][kNW];         // db per wave

  const int t = threadIdx.x;
  const int l = t & 63;
  const int w = t >> 6;
  const int i0 = RPL * l;                // first key row of this lane
  const int jc = kCPW * w;               // first of this wave's columns in the slab
  const int H = p.H, DV = p.DV;
  const int nslab = DV / kVS;

  // Workgroups of one (sequence, head) run on one XCD (they read the same
  // q, k, alpha rows).
  int64_t b = blockIdx.x;
  const int64_t G_ = gridDim.x;
  if ((G_ & 7) == 0) b = (b & 7) * (G_ >> 3) + (b >> 3);
  const int slab = int(b % nslab);
  const int64_t pr = b / nslab;
  const int h = int(pr % H);
  const int64_t n = pr / H;
  const int col = slab * kVS + jc;       // first value column of this wave
  // this sequence's tokens: fixed length, or packed by cu_seqlens
  const int64_t tok0 = p.cu_seqlens ? int64_t(p.cu_seqlens[n]) : n * p.T;
  const int64_t T = p.cu_seqlens ? int64_t(p.cu_seqlens[n + 1]) - tok0 : p.T;
  const int64_t nchunks = T > 0 ? (T + kC - 1) / kC : 0;
  const int64_t state_off = pr * DK * DV + int64_t(i0) * DV + col;
  // token states: [2 chunk buffers][64 tokens][kNT threads][E floats]
  float* scratch = p.scratch + b * (2 * int64_t(kC) * kNT * E) + int64_t(t) * E;
  auto slot = [&](int64_t c, int s) { return scratch + ((c & 1) * kC + s) * int64_t(kNT) * E; };
  auto row_of = [&](int64_t c, int s) { return (tok0 + c * kC + s) * H + h; };

  auto ld_state = [&](const float* src, float (&S)[E]) {
#pragma unroll
    for (int r = 0; r < RPL; ++r) ldfn<kCPW>(src + int64_t(r) * DV, S + r * kCPW);
  };
  // state at the start of chunk c (snapshot c-1 is the state after chunk c-1)
  auto checkpoint = [&](int64_t c, float (&S)[E]) {
    if (c > 0) {
      // snapshot of chunk c-1: row n * snap_per_seq + c - 1, or tok0 / 64 + c - 1 when packed
      const int64_t srow = (p.cu_seqlens ? tok0 / kC : n * p.snap_per_seq) + (c - 1);
      ld_state(p.snapshots + (srow * H + h) * int64_t(DK) * DV + int64_t(i0) * DV + col, S);
    } else if (p.state_in) {
      ld_state(p.state_in + state_off, S);
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) S[e] = 0.f;
    }
  };

  // This launch's window: the chunks c_lo .. c_hi, counted from the
  // sequence's end (reverse indices win_lo .. win_lo + win_k - 1).  The
  // adjoint G comes from d_state_out in the first window and from the
  // previous window's carry otherwise.
  const int64_t c_hi = nchunks - 1 - p.win_lo;
  const int64_t c_lo = c_hi - p.win_k + 1 > 0 ? c_hi - p.win_k + 1 : 0;
  float G[E], S[E];
  if (p.win_lo > 0) {
    ld_state(p.g_carry + state_off, G);
  } else if (p.d_state_out) {
    ld_state(p.d_state_out + state_off, G);
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) G[e] = 0.f;
  }
  if (c_hi < 0) {
    // nothing of this sequence in the window; an empty sequence passes the
    // final state's gradient through (once, in the first window)
    if (nchunks == 0 && p.win_lo == 0 && p.d_state_in) {
#pragma unroll
      for (int r = 0; r < RPL; ++r)
        stfn<kCPW>(p.d_state_in + state_off + int64_t(r) * DV, G + r * kCPW);
    }
    return;
  }
  // row of the window's partial sums for token sb of chunk c
  auto prow_of = [&](int64_t c, int sb) {
    return ((n * p.win_k + (nchunks - 1 - c - p.win_lo)) * kC + sb) * H + h;
  };

  // Inputs of one forward token and of one backward token, loaded a step
  // ahead of their use (within a chunk: the backward token's state was
  // stored when its chunk was recomputed, a pass earlier).
  struct FIn {
    float a[RPL], b;
    RowsIn<BF16, RPL> k;
    ColsIn<BF16> v;
  };
  struct BIn {
    float a[RPL], b, dout[kCPW], Sp[E];
    RowsIn<BF16, RPL> k, q;
  };
  auto load_alpha = [&](int64_t row, float (&a)[RPL]) {
    if constexpr (SG) {
      const float g = p.alpha[row];
#pragma unroll
      for (int r = 0; r < RPL; ++r) a[r] = g;
    } else {
      ld_f<RPL>(p.alpha + row * DK + i0, a);
    }
  };
  auto load_f = [&](int64_t c, int s, FIn& x) {
    const int64_t row = row_of(c, s);
    load_alpha(row, x.a);
    x.k.load(p.k, row * DK + i0);
    x.b = p.beta[row];
    x.v.load(p.v, row * DV + col);
  };
  auto load_b = [&](int64_t c, int sb, BIn& x) {
    const int64_t row = row_of(c, sb);
    load_alpha(row, x.a);
    x.k.load(p.k, row * DK + i0);
    x.q.load(p.q, row * DK + i0);
    x.b = p.beta[row];
    ldfn<kCPW>(p.d_o + row * DV + col, x.dout);
    const float* src = slot(c, sb);
    ld_elems<E>(src, x.Sp);
  };

  // One forward token of chunk c: keeps S before the token, then
  // S <- Diag(a) S + k u^T with u = b (v - St^T k).
  auto fwd_token = [&](int64_t c, int s, const FIn& f) {
    float* dst = slot(c, s);
    st_elems<E>(dst, S);
    float x[kCPW];
#pragma unroll
    for (int e = 0; e < kCPW; ++e) {
      x[e] = 0.f;
#pragma unroll
      for (int r = 0; r < RPL; ++r) {
        S[r * kCPW + e] *= f.a[r];
        x[e] += S[r * kCPW + e] * f.k[r];
      }
    }
    wave_sums<kCPW>(x);
#pragma unroll
    for (int e = 0; e < kCPW; ++e) {
      const float r_ = f.v[e] - x[e];   // v - p
      const float u = f.b * r_;
#pragma unroll
      for (int r = 0; r < RPL; ++r) S[r * kCPW + e] += f.k[r] * u;
      if (l == 0) {
        sU[c & 1][s][jc + e] = u;
        sR[c & 1][s][jc + e] = r_;
      }
    }
  };

  // Backward token sb of chunk c with inputs x (and, when f is given, the
  // forward token s of chunk c-1 between its two halves).  Every memory
  // instruction is issued by every lane, so each step issues the same number
  // of them and the memory-counter waits for loads issued a step earlier do
  // not cover the stores in between: the per-wave row sums go through LDS
  // (one barrier per token) and all threads write the slab's sums; values
  // that are the same in every lane (dv, db) are stored by all lanes.
  int par = 0;
  auto bwd_token = [&](int64_t c, int sb, const BIn& x, int64_t cf_c, int cf_s, const FIn* f) {
    const int64_t brow = row_of(c, sb);
    float u[kCPW], rr[kCPW], St[E];
#pragma unroll
    for (int e = 0; e < kCPW; ++e) {
      u[e] = sU[c & 1][sb][jc + e];
      rr[e] = sR[c & 1][sb][jc + e];
    }
    // G += q do^T (o_t = S'^T q_t); dq = S' do; du = G^T k
    float dq[RPL], du[kCPW];
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      float xq = 0.f;
#pragma unroll
      for (int e = 0; e < kCPW; ++e) {
        const int q_ = r * kCPW + e;
        St[q_] = x.a[r] * x.Sp[q_];
        G[q_] += x.q[r] * x.dout[e];
        xq += (St[q_] + x.k[r] * u[e]) * x.dout[e];
      }
      dq[r] = xq;
    }
#pragma unroll
    for (int e = 0; e < kCPW; ++e) {
      du[e] = 0.f;
#pragma unroll
      for (int r = 0; r < RPL; ++r) du[e] += G[r * kCPW + e] * x.k[r];
    }
    // the forward token of chunk c-1 at the same step: its column sum is
    // independent of this one, so the two reductions overlap
    if (f) fwd_token(cf_c, cf_s, *f);
    wave_sums<kCPW>(du);
    float dk[RPL], da[RPL], db = 0.f;
#pragma unroll
    for (int r = 0; r < RPL; ++r) dk[r] = da[r] = 0.f;
#pragma unroll
    for (int e = 0; e < kCPW; ++e) {
      const float dp = -x.b * du[e];
      db += du[e] * rr[e];
#pragma unroll
      for (int r = 0; r < RPL; ++r) {
        const int q_ = r * kCPW + e;
        const float dSt = G[q_] + x.k[r] * dp;
        dk[r] += G[q_] * u[e] + St[q_] * dp;
        da[r] += dSt * x.Sp[q_];
        G[q_] = x.a[r] * dSt;
      }
    }
    float dv4[kCPW];
#pragma unroll
    for (int e = 0; e < kCPW; ++e) dv4[e] = x.b * du[e];
    stfn<kCPW>(p.dv + brow * DV + col, dv4);
    if (l == 0) ringb[par][w] = db;
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      ring[par][0][w][i0 + r] = dq[r];
      ring[par][1][w][i0 + r] = dk[r];
      ring[par][2][w][i0 + r] = da[r];
    }
    lds_sync();
    // the slab's sums over the waves, in a fixed order: index x = t + kNT j
    // is quantity min(x / DK, 2) (dq, dk, da) of row x % DK (indices past
    // 3 DK write da values again), and every thread writes the same db
    {
      const int64_t lrow = prow_of(c, sb);
      constexpr int NPASS = (3 * DK + kNT - 1) / kNT;
#pragma unroll
      for (int j = 0; j < NPASS; ++j) {
        const int x = t + kNT * j;
        const int i = x % DK;
        const int qn = x / DK < 2 ? x / DK : 2;
        const float v = sum_waves(&ring[par][qn][0][i], DK);
        const int64_t prow = (slab * p.part_rows + lrow) * DK + i;   // slab-major: one row is 512 B
        (qn == 0 ? p.part_dq : (qn == 1 ? p.part_dk : p.part_da))[prow] = v;
      }
      p.part_db[slab * p.part_rows + lrow] = sum_waves(ringb[par], 1);
    }
    par ^= 1;
  };

  FIn cf, nf;
  BIn cb, nb;
  // prologue: the token states of the window's last chunk
  {
    const int64_t c = c_hi;
    const int len = int(T - c * kC < kC ? T - c * kC : kC);
    checkpoint(c, S);
    for (int s = 0; s < len; ++s) {
      load_f(c, s, cf);
      fwd_token(c, s, cf);
    }
  }

  for (int64_t c = c_hi; c >= c_lo; --c) {
    const int len = int(T - c * kC < kC ? T - c * kC : kC);
    const bool fwd = c > c_lo;              // chunk c-1 is recomputed meanwhile (always full)
    if (fwd) checkpoint(c - 1, S);
    if (fwd && len == kC) {
      // the steady state: both tokens in every step, inputs a step ahead in
      // two sets used alternately (no register copies, so each wait sits at
      // the first use of its input; the loads past the chunk's end repeat
      // its last token: no branch)
      load_f(c - 1, 0, cf);
      load_b(c, kC - 1, cb);
      for (int s = 0; s < kC; s += 2) {
        load_b(c, kC - 2 - s, nb);
        load_f(c - 1, s + 1, nf);
        bwd_token(c, kC - 1 - s, cb, c - 1, s, &cf);
        const int sn = s + 2 < kC ? s + 2 : kC - 1;
        load_b(c, kC - 1 - sn, cb);
        load_f(c - 1, sn, cf);
        bwd_token(c, kC - 2 - s, nb, c - 1, s + 1, &nf);
      }
    } else {
      const int steps = fwd ? kC : len;
      for (int s = 0; s < steps; ++s) {
        if (fwd) load_f(c - 1, s, cf);
        if (s < len) {
          load_b(c, len - 1 - s, cb);
          bwd_token(c, len - 1 - s, cb, c - 1, s, fwd ? &cf : nullptr);
        } else {
          fwd_token(c - 1, s, cf);
        }
      }
    }
  }
  // after chunk 0 the initial state's gradient; otherwise the carry for
  // the next window
  float* gdst = c_lo == 0 ? p.d_state_in : p.g_carry;
#pragma unroll
  for (int r = 0; r < RPL; ++r)
    if (gdst) stfn<kCPW>(gdst + state_off + int64_t(r) * DV, G + r * kCPW);
}

// The global token row of row lrow of a window's partial sums, or -1 when
// that row is past its sequence (or before its first chunk).
__device__ __forceinline__ int64_t window_row(const BackwardArgs& p, int64_t lrow) {
  const int64_t h = lrow % p.H;
  int64_t x = lrow / p.H;
  const int s = int(x % 64);
  x /= 64;
  const int64_t jj = x % p.win_k;
  const int64_t n = x / p.win_k;
  const int64_t tok0 = p.cu_seqlens ? int64_t(p.cu_seqlens[n]) : n * p.T;
  const int64_t T = p.cu_seqlens ? int64_t(p.cu_seqlens[n + 1]) - tok0 : p.T;
  const int64_t nch = (T + 63) / 64;
  const int64_t c = nch - 1 - (p.win_lo + jj);
  const int64_t t = c * 64 + s;
  if (c < 0 || t >= T) return -1;
  return (tok0 + t) * p.H + h;
}

// dq, dk, dalpha (per element) and dbeta: sums of the NS per-slab partials,
// which are stored slab-major (the walk writes whole 512-byte rows), so a
// thread reads NS values `stride` apart and a wave reads NS contiguous
// streams; the slabs are added pairwise in a fixed order.
template <int NS>
__device__ __forceinline__ float sum_ns(const float* p, int64_t stride) {
  float x[NS];
#pragma unroll
  for (int v = 0; v < NS; ++v) x[v] = p[v * stride];
#pragma unroll
  for (int h = 1; h < NS; h <<= 1)
#pragma unroll
    for (int v = 0; v + h < NS; v += 2 * h) x[v] += x[v + h];
  return x[0];
}

template <int DK, int NS, bool SG>
__global__ __launch_bounds__(256) void kda_bwd_reduce_kernel(BackwardArgs p) {
  const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;   // window row * DK + key row
  if (idx >= p.part_rows * DK) return;
  const int64_t lrow = idx / DK;
  const int i = int(idx % DK);
  const int64_t grow = window_row(p, lrow);
  if (grow < 0) return;
  const int64_t o = grow * DK + i;
  const int64_t st = p.part_rows * DK;
  p.dq[o] = sum_ns<NS>(p.part_dq + idx, st);
  p.dk[o] = sum_ns<NS>(p.part_dk + idx, st);
  if constexpr (!SG) p.dalpha[o] = sum_ns<NS>(p.part_da + idx, st);
  if (i == 0) p.dbeta[grow] = sum_ns<NS>(p.part_db + lrow, p.part_rows);
}

// A scalar gate's gradient: the sum over key rows and slabs of the per-row
// partials (chain rule: the gate is every row's decay), one wave per token
// row; each lane adds the slabs of its DK / 64 key rows, then the lanes are
// added in a fixed order (deterministic).
template <int DK, int NS>
__global__ __launch_bounds__(256) void kda_bwd_dgate_kernel(BackwardArgs p) {
  constexpr int PER = DK / 64;   // key rows per lane
  const int64_t lrow = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  if (lrow >= p.part_rows) return;
  const int64_t row = window_row(p, lrow);
  if (row < 0) return;
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < PER; ++r) s += sum_ns<NS>(p.part_da + lrow * DK + l * PER + r, p.part_rows * DK);
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) s += __shfl_xor(s, off);
  if (l == 0) p.dalpha[row] = s;
}

template <int DK, bool BF16, bool SG>
void launch_bwd_t(const BackwardArgs& a, hipStream_t st) {
  const unsigned nb = unsigned(int64_t(a.N) * a.H * (a.DV / kVS));
  hipLaunchKernelGGL((kda_bwd_kernel<DK, BF16, SG>), dim3(nb), dim3(kNT), 0, st, a);
  if (a.rows == 0) return;   // no tokens: only d_state_in (= d_state_out) is written
  const int64_t threads = a.part_rows * DK;
  const dim3 grid(unsigned((threads + 255) / 256));
  const dim3 grid_g(unsigned((a.part_rows + 3) / 4));
  if (a.DV == 128) {
    hipLaunchKernelGGL((kda_bwd_reduce_kernel<DK, 8, SG>), grid, dim3(256), 0, st, a);
    if (SG) hipLaunchKernelGGL((kda_bwd_dgate_kernel<DK, 8>), grid_g, dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL((kda_bwd_reduce_kernel<DK, 4, SG>), grid, dim3(256), 0, st, a);
    if (SG) hipLaunchKernelGGL((kda_bwd_dgate_kernel<DK, 4>), grid_g, dim3(256), 0, st, a);
  }
}

}  // namespace

size_t backward_scratch_bytes(int N, int H, int DK, int DV) {
  return size_t(N) * H * (DV / kVS) * 2 * size_t(kC) * DK * kVS * 4;
}

int launch_backward(const BackwardArgs& a, void* stream, const char** msg) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (a.DK == 128) {
    if (a.alpha_scalar) {
      if (a.in_bf16) launch_bwd_t<128, true, true>(a, st);
      else launch_bwd_t<128, false, true>(a, st);
    } else {
      if (a.in_bf16) launch_bwd_t<128, true, false>(a, st);
      else launch_bwd_t<128, false, false>(a, st);
    }
  } else if (a.DK == 64) {
    if (a.alpha_scalar) {
      if (a.in_bf16) launch_bwd_t<64, true, true>(a, st);
      else launch_bwd_t<64, false, true>(a, st);
    } else {
      if (a.in_bf16) launch_bwd_t<64, true, false>(a, st);
      else launch_bwd_t<64, false, false>(a, st);
    }
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

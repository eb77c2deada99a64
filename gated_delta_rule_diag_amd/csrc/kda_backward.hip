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
//      so their latencies overlap and one column-sum barrier serves both;
//   3. kda_bwd_reduce_kernel: sums the per-slab partials (a fixed order, so
//      the result is deterministic).
//
// Thread layout: thread t owns key rows 2 (t / 4) and 2 (t / 4) + 1 and value
// columns 4 (t % 4) .. +3 of the workgroup's 16: row sums are four local adds
// and two lane exchanges, column sums two local adds, four lane exchanges and
// the waves through LDS (double-buffered by step parity: one barrier per step).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kC = 64;    // chunk length (checkpoint interval)
constexpr int kVS = 16;   // value columns per workgroup
constexpr int kCPT = 4;   // value columns per thread
constexpr int kRPT = 2;   // key rows per thread
constexpr int kTPR = kVS / kCPT;   // threads per row pair
constexpr int kE = kRPT * kCPT;    // state elements per thread

__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <bool BF16>
__device__ __forceinline__ float ld_in(const void* p, int64_t i) {
  if constexpr (BF16) {
    return __uint_as_float(uint32_t(static_cast<const uint16_t*>(p)[i]) << 16);
  } else {
    return static_cast<const float*>(p)[i];
  }
}

// Four consecutive values (8-byte aligned for bf16, 16-byte for float).
template <bool BF16>
__device__ __forceinline__ void ld4(const void* p, int64_t i, float (&x)[kCPT]) {
  if constexpr (BF16) {
    const uint2 r = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i);
    x[0] = __uint_as_float(r.x << 16);
    x[1] = __uint_as_float(r.x & 0xffff0000u);
    x[2] = __uint_as_float(r.y << 16);
    x[3] = __uint_as_float(r.y & 0xffff0000u);
  } else {
    const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  }
}

__device__ __forceinline__ void ldf4(const float* p, float* x) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
}

__device__ __forceinline__ void stf4(float* p, const float* x) {
  *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
}

// The thread's 2 x 4 slab elements of a [DK][DV] state (row stride DV).
__device__ __forceinline__ void ld_slab(const float* p, int DV, float (&x)[kE]) {
  ldf4(p, x);
  ldf4(p + DV, x + kCPT);
}

__device__ __forceinline__ void st_slab(float* p, int DV, const float (&x)[kE]) {
  stf4(p, x);
  stf4(p + DV, x + kCPT);
}

// Sum over the workgroup's 16 columns of a row: 4 local values and the 3
// partner lanes.
__device__ __forceinline__ float row_sum(const float* x) {
  float s = (x[0] + x[1]) + (x[2] + x[3]);
  s += __shfl_xor(s, 1);
  return s + __shfl_xor(s, 2);
}

// Column sums over all DK rows for NV vectors of this thread's four columns
// (x[v][e]: vector v, column e, already summed over the thread's two rows).
template <int NW, int NV>
__device__ __forceinline__ void col_sums(float (&x)[NV][kCPT], float (*red)[NW][NV][kVS],
                                         int parity) {
  const int t = threadIdx.x, l = t & 63, w = t >> 6;
#pragma unroll
  for (int v = 0; v < NV; ++v)
#pragma unroll
    for (int e = 0; e < kCPT; ++e)
#pragma unroll
      for (int off = kTPR; off < 64; off <<= 1) x[v][e] += __shfl_xor(x[v][e], off);
  if (l < kTPR) {
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
      for (int e = 0; e < kCPT; ++e) red[parity][w][v][kCPT * l + e] = x[v][e];
  }
  lds_sync();
  const int c0 = kCPT * (t % kTPR);
#pragma unroll
  for (int v = 0; v < NV; ++v)
#pragma unroll
    for (int e = 0; e < kCPT; ++e) {
      float s = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) s += red[parity][ww][v][c0 + e];
      x[v][e] = s;
    }
}

template <int DK, bool BF16>
__global__ __launch_bounds__(DK / kRPT * kTPR) void kda_bwd_kernel(BackwardArgs p) {
  constexpr int NT = DK / kRPT * kTPR;
  constexpr int NW = NT / 64;
  __shared__ float red[2][NW][2][kVS];
  __shared__ float sU[2][kC][kVS];   // u of a chunk's tokens (this slab), two chunks
  __shared__ float sR[2][kC][kVS];   // v - p

  const int t = threadIdx.x;
  const int i0 = kRPT * (t / kTPR);      // first key row
  const int jc = kCPT * (t % kTPR);      // first of this thread's columns in the slab
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
  const int col = slab * kVS + jc;       // first value column of this thread
  const int64_t T = p.T;
  const int64_t nchunks = (T + kC - 1) / kC;
  const int64_t state_off = pr * DK * DV + int64_t(i0) * DV + col;
  // token states: [2 chunk buffers][64 tokens][NT threads][8 floats]
  float* scratch = p.scratch + b * (2 * int64_t(kC) * NT * kE) + int64_t(t) * kE;
  auto slot = [&](int64_t c, int s) { return scratch + ((c & 1) * kC + s) * int64_t(NT) * kE; };
  auto row_of = [&](int64_t c, int s) { return (n * T + c * kC + s) * H + h; };

  // state at the start of chunk c (snapshot c-1 is the state after chunk c-1)
  auto checkpoint = [&](int64_t c, float (&S)[kE]) {
    if (c > 0) {
      ld_slab(p.snapshots + ((n * p.snap_per_seq + (c - 1)) * H + h) * int64_t(DK) * DV +
                  int64_t(i0) * DV + col, DV, S);
    } else if (p.state_in) {
      ld_slab(p.state_in + state_off, DV, S);
    } else {
#pragma unroll
      for (int e = 0; e < kE; ++e) S[e] = 0.f;
    }
  };

  float G[kE], S[kE];
  if (p.d_state_out) {
    ld_slab(p.d_state_out + state_off, DV, G);
  } else {
#pragma unroll
    for (int e = 0; e < kE; ++e) G[e] = 0.f;
  }

  // One forward token of chunk c (full or the last one): keeps S before the
  // token, then S <- Diag(a) S + k u^T.  The column sum p = St^T k is shared
  // with the backward token of the same step (slot 1 of the sums).
  float fa[kRPT], fk[kRPT], fb = 0.f, fv[kCPT];
  auto fwd_pre = [&](int64_t c, int s, float (&x)[kCPT]) {
    const int64_t row = row_of(c, s);
#pragma unroll
    for (int r = 0; r < kRPT; ++r) {
      fa[r] = p.alpha[row * DK + i0 + r];
      fk[r] = ld_in<BF16>(p.k, row * DK + i0 + r);
    }
    fb = p.beta[row];
    ld4<BF16>(p.v, row * DV + col, fv);
    float* dst = slot(c, s);
    stf4(dst, S);
    stf4(dst + kCPT, S + kCPT);
#pragma unroll
    for (int r = 0; r < kRPT; ++r)
#pragma unroll
      for (int e = 0; e < kCPT; ++e) S[r * kCPT + e] *= fa[r];
#pragma unroll
    for (int e = 0; e < kCPT; ++e) x[e] = S[e] * fk[0] + S[kCPT + e] * fk[1];
  };
  auto fwd_post = [&](int64_t c, int s, const float (&pcol)[kCPT]) {
#pragma unroll
    for (int e = 0; e < kCPT; ++e) {
      const float r_ = fv[e] - pcol[e];   // v - p
      const float u = fb * r_;
#pragma unroll
      for (int r = 0; r < kRPT; ++r) S[r * kCPT + e] += fk[r] * u;
      if (i0 == 0) {
        sU[c & 1][s][jc + e] = u;
        sR[c & 1][s][jc + e] = r_;
      }
    }
  };

  // prologue: the last chunk's token states
  {
    const int64_t c = nchunks - 1;
    const int len = int(T - c * kC);
    checkpoint(c, S);
    int parity = 0;
    for (int s = 0; s < len; ++s) {
      float x[2][kCPT];
      fwd_pre(c, s, x[1]);
#pragma unroll
      for (int e = 0; e < kCPT; ++e) x[0][e] = 0.f;
      col_sums<NW, 2>(x, red, parity);
      parity ^= 1;
      fwd_post(c, s, x[1]);
    }
  }
  lds_sync();

  int parity = 0;
  for (int64_t c = nchunks - 1; c >= 0; --c) {
    const int len = int(T - c * kC < kC ? T - c * kC : kC);
    const bool fwd = c > 0;                 // chunk c-1 is recomputed meanwhile (always full)
    if (fwd) checkpoint(c - 1, S);
    const int steps = fwd ? kC : len;
    for (int s = 0; s < steps; ++s) {
      const bool bwd = s < len;
      const int sb = len - 1 - s;           // backward token of chunk c
      float x[2][kCPT];
      // backward, first half: G += q do^T, dq = S' do, du partial = G^T k
      float a[kRPT], kk[kRPT], qq[kRPT], bt = 0.f, dout[kCPT], Sp[kE], u[kCPT], rr[kCPT];
      float St[kE], dq[kRPT] = {0.f, 0.f};
      int64_t brow = 0;
      if (bwd) {
        brow = row_of(c, sb);
#pragma unroll
        for (int r = 0; r < kRPT; ++r) {
          a[r] = p.alpha[brow * DK + i0 + r];
          kk[r] = ld_in<BF16>(p.k, brow * DK + i0 + r);
          qq[r] = ld_in<BF16>(p.q, brow * DK + i0 + r);
        }
        bt = p.beta[brow];
        ldf4(p.d_o + brow * DV + col, dout);
        const float* src = slot(c, sb);
        ldf4(src, Sp);
        ldf4(src + kCPT, Sp + kCPT);
#pragma unroll
        for (int e = 0; e < kCPT; ++e) {
          u[e] = sU[c & 1][sb][jc + e];
          rr[e] = sR[c & 1][sb][jc + e];
        }
#pragma unroll
        for (int r = 0; r < kRPT; ++r) {
          float xq[kCPT];
#pragma unroll
          for (int e = 0; e < kCPT; ++e) {
            const int q_ = r * kCPT + e;
            St[q_] = a[r] * Sp[q_];
            G[q_] += qq[r] * dout[e];                  // o_t = S'^T q_t
            xq[e] = (St[q_] + kk[r] * u[e]) * dout[e];  // dq: S' do
          }
          dq[r] = row_sum(xq);
        }
#pragma unroll
        for (int e = 0; e < kCPT; ++e) x[0][e] = G[e] * kk[0] + G[kCPT + e] * kk[1];
      } else {
#pragma unroll
        for (int e = 0; e < kCPT; ++e) x[0][e] = 0.f;
      }
      if (fwd) {
        fwd_pre(c - 1, s, x[1]);
      } else {
#pragma unroll
        for (int e = 0; e < kCPT; ++e) x[1][e] = 0.f;
      }
      col_sums<NW, 2>(x, red, parity);
      parity ^= 1;
      if (fwd) fwd_post(c - 1, s, x[1]);
      if (bwd) {
        // backward, second half
        const float* du = x[0];
        float xk[kRPT][kCPT], xa[kRPT][kCPT], xb[kCPT];
#pragma unroll
        for (int e = 0; e < kCPT; ++e) {
          const float dp = -bt * du[e];
          xb[e] = du[e] * rr[e];
#pragma unroll
          for (int r = 0; r < kRPT; ++r) {
            const int q_ = r * kCPT + e;
            const float dSt = G[q_] + kk[r] * dp;
            xk[r][e] = G[q_] * u[e] + St[q_] * dp;
            xa[r][e] = dSt * Sp[q_];
            G[q_] = a[r] * dSt;
          }
        }
        float dk[kRPT], da[kRPT];
#pragma unroll
        for (int r = 0; r < kRPT; ++r) {
          dk[r] = row_sum(xk[r]);
          da[r] = row_sum(xa[r]);
        }
        if ((t % kTPR) == 0) {
          // partials are slab-minor: [token row][key row][slab]
          const int64_t prow = (brow * DK + i0) * nslab + slab;
#pragma unroll
          for (int r = 0; r < kRPT; ++r) {
            p.part_dq[prow + r * nslab] = dq[r];
            p.part_dk[prow + r * nslab] = dk[r];
            p.part_da[prow + r * nslab] = da[r];
          }
        }
        if (i0 == 0) {
          float dv4[kCPT];
#pragma unroll
          for (int e = 0; e < kCPT; ++e) dv4[e] = bt * du[e];
          stf4(p.dv + brow * DV + col, dv4);
          const float db = row_sum(xb);
          if (t == 0) p.part_db[brow * nslab + slab] = db;
        }
      }
    }
    lds_sync();   // chunk c-1's u, v - p visible; chunk c's buffers free
  }
  if (p.d_state_in) st_slab(p.d_state_in + state_off, DV, G);
}

// dq, dk, dalpha (per element) and dbeta: sums of the NS per-slab partials,
// which are stored slab-minor, so a thread reads NS consecutive floats per
// output and a wave streams contiguous memory.
template <int NS>
__device__ __forceinline__ float sum_ns(const float* p) {
  float s = 0.f;
#pragma unroll
  for (int v = 0; v < NS; v += 4) {
    const float4 x = *reinterpret_cast<const float4*>(p + v);
    s += (x.x + x.y) + (x.z + x.w);
  }
  return s;
}

template <int DK, int NS>
__global__ __launch_bounds__(256) void kda_bwd_reduce_kernel(BackwardArgs p) {
  const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;   // token row * DK + key row
  if (idx < p.rows * DK) {
    p.dq[idx] = sum_ns<NS>(p.part_dq + idx * NS);
    p.dk[idx] = sum_ns<NS>(p.part_dk + idx * NS);
    p.dalpha[idx] = sum_ns<NS>(p.part_da + idx * NS);
  }
  if (idx < p.rows) p.dbeta[idx] = sum_ns<NS>(p.part_db + idx * NS);
}

template <int DK, bool BF16>
void launch_bwd_t(const BackwardArgs& a, hipStream_t st) {
  const unsigned nb = unsigned(int64_t(a.N) * a.H * (a.DV / kVS));
  hipLaunchKernelGGL((kda_bwd_kernel<DK, BF16>), dim3(nb), dim3(DK / kRPT * kTPR), 0, st, a);
  const int64_t threads = a.rows * DK;
  const dim3 grid(unsigned((threads + 255) / 256));
  if (a.DV == 128) hipLaunchKernelGGL((kda_bwd_reduce_kernel<DK, 8>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((kda_bwd_reduce_kernel<DK, 4>), grid, dim3(256), 0, st, a);
}

}  // namespace

size_t backward_scratch_bytes(int N, int H, int DK, int DV) {
  return size_t(N) * H * (DV / kVS) * 2 * size_t(kC) * DK * kVS * 4;
}

int launch_backward(const BackwardArgs& a, void* stream, const char** msg) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (a.DK == 128) {
    if (a.in_bf16) launch_bwd_t<128, true>(a, st);
    else launch_bwd_t<128, false>(a, st);
  } else if (a.DK == 64) {
    if (a.in_bf16) launch_bwd_t<64, true>(a, st);
    else launch_bwd_t<64, false>(a, st);
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

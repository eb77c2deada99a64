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
//      the last to the first: the chunk's token states are recomputed from its
//      checkpoint into a per-workgroup scratch, then the chunk is walked
//      backwards;
//   3. kda_bwd_reduce_kernel: sums the per-slab partials (a fixed order, so
//      the result is deterministic).
//
// Thread layout: thread t owns key row i = t / 2 and value columns
// 8 (t % 2) .. +7 of the workgroup's 16, so row sums are eight local adds and
// one lane exchange; column sums reduce 32 rows per wave by lane exchanges and
// the waves through LDS (double-buffered by step parity: one barrier per sum).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kC = 64;    // chunk length (checkpoint interval)
constexpr int kVS = 16;   // value columns per workgroup
constexpr int kCPT = 8;   // value columns per thread
constexpr int kTPR = kVS / kCPT;

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

// Eight consecutive values (16-byte aligned for float, 16-byte for bf16).
template <bool BF16>
__device__ __forceinline__ void ld8(const void* p, int64_t i, float (&x)[kCPT]) {
  if constexpr (BF16) {
    const uint4 r = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + i);
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __uint_as_float(w[e] << 16);
      x[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
    const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

__device__ __forceinline__ void ldf8(const float* p, float (&x)[kCPT]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

__device__ __forceinline__ void stf8(float* p, const float (&x)[kCPT]) {
  *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
}

// Sum over the workgroup's 16 columns of a row: 8 local values + the partner lane.
__device__ __forceinline__ float row_sum(const float (&x)[kCPT]) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < kCPT; ++e) s += x[e];
  return s + __shfl_xor(s, 1);
}

// Column sums over all DK rows of the workgroup: x holds this row's eight
// columns; the result (all rows' sum for the same eight columns) lands in x.
template <int NW>
__device__ __forceinline__ void col_sum(float (&x)[kCPT], float (*red)[NW][kVS], int parity) {
  const int t = threadIdx.x, l = t & 63, w = t >> 6;
#pragma unroll
  for (int e = 0; e < kCPT; ++e) {
#pragma unroll
    for (int off = kTPR; off < 64; off <<= 1) x[e] += __shfl_xor(x[e], off);
  }
  if (l < kTPR) {
#pragma unroll
    for (int e = 0; e < kCPT; ++e) red[parity][w][kCPT * l + e] = x[e];
  }
  lds_sync();
  const int c0 = kCPT * (t & (kTPR - 1));
#pragma unroll
  for (int e = 0; e < kCPT; ++e) {
    float s = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) s += red[parity][ww][c0 + e];
    x[e] = s;
  }
}

template <int DK, bool BF16>
__global__ __launch_bounds__(DK * kTPR) void kda_bwd_kernel(BackwardArgs p) {
  constexpr int NT = DK * kTPR;
  constexpr int NW = NT / 64;
  __shared__ float red[2][NW][kVS];
  __shared__ float sU[kC][kVS];   // u of the chunk's tokens (this slab)
  __shared__ float sP[kC][kVS];   // p of the chunk's tokens

  const int t = threadIdx.x;
  const int i = t / kTPR;                 // key row
  const int jc = kCPT * (t % kTPR);       // first of this thread's columns in the slab
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
  const int col = slab * kVS + jc;        // first value column of this thread
  const int64_t T = p.T;
  const int64_t nchunks = (T + kC - 1) / kC;
  const int64_t state_off = pr * DK * DV + int64_t(i) * DV + col;
  float* scratch = p.scratch + b * (int64_t(kC) * NT * kCPT) + int64_t(t) * kCPT;

  float G[kCPT], S[kCPT];
  if (p.d_state_out) {
    ldf8(p.d_state_out + state_off, G);
  } else {
#pragma unroll
    for (int e = 0; e < kCPT; ++e) G[e] = 0.f;
  }

  int parity = 0;
  for (int64_t c = nchunks - 1; c >= 0; --c) {
    const int64_t t0 = c * kC;
    const int len = int(T - t0 < kC ? T - t0 : kC);
    // checkpoint: the state at the chunk start
    // (snapshot c-1 is the state after chunk c-1; every chunk before the last is full)
    if (c > 0) {
      ldf8(p.snapshots + ((n * p.snap_per_seq + (c - 1)) * H + h) * int64_t(DK) * DV +
               int64_t(i) * DV + col, S);
    } else if (p.state_in) {
      ldf8(p.state_in + state_off, S);
    } else {
#pragma unroll
      for (int e = 0; e < kCPT; ++e) S[e] = 0.f;
    }

    // ---- forward through the chunk: keep S before every token ----
    for (int s = 0; s < len; ++s) {
      const int64_t row = (n * T + t0 + s) * H + h;
      const float a = p.alpha[row * DK + i];
      const float kk = ld_in<BF16>(p.k, row * DK + i);
      const float bt = p.beta[row];
      float v[kCPT];
      ld8<BF16>(p.v, row * DV + col, v);
      stf8(scratch + int64_t(s) * NT * kCPT, S);
      float x[kCPT];
#pragma unroll
      for (int e = 0; e < kCPT; ++e) {
        S[e] *= a;
        x[e] = S[e] * kk;
      }
      col_sum<NW>(x, red, parity);
      parity ^= 1;
#pragma unroll
      for (int e = 0; e < kCPT; ++e) {
        const float u = bt * (v[e] - x[e]);
        S[e] += kk * u;
        if (i == 0) {
          sU[s][jc + e] = u;
          sP[s][jc + e] = x[e];
        }
      }
    }
    lds_sync();   // sU, sP of the chunk visible to every thread

    // ---- backward through the chunk ----
    for (int s = len - 1; s >= 0; --s) {
      const int64_t row = (n * T + t0 + s) * H + h;
      const float a = p.alpha[row * DK + i];
      const float kk = ld_in<BF16>(p.k, row * DK + i);
      const float qq = ld_in<BF16>(p.q, row * DK + i);
      const float bt = p.beta[row];
      float dout[kCPT], Sp[kCPT], u[kCPT], pp[kCPT], v[kCPT];
      ldf8(p.d_o + row * DV + col, dout);
      ld8<BF16>(p.v, row * DV + col, v);
      ldf8(scratch + int64_t(s) * NT * kCPT, Sp);
#pragma unroll
      for (int e = 0; e < kCPT; ++e) {
        u[e] = sU[s][jc + e];
        pp[e] = sP[s][jc + e];
      }
      float St[kCPT], x[kCPT], du[kCPT];
#pragma unroll
      for (int e = 0; e < kCPT; ++e) {
        St[e] = a * Sp[e];
        G[e] += qq * dout[e];                  // o_t = S'^T q_t
        x[e] = (St[e] + kk * u[e]) * dout[e];  // dq: S' do
        du[e] = G[e] * kk;
      }
      const float dq = row_sum(x);
      col_sum<NW>(du, red, parity);
      parity ^= 1;
      float xk[kCPT], xa[kCPT], xb[kCPT];
#pragma unroll
      for (int e = 0; e < kCPT; ++e) {
        const float dp = -bt * du[e];
        const float dSt = G[e] + kk * dp;
        xk[e] = G[e] * u[e] + St[e] * dp;
        xa[e] = dSt * Sp[e];
        xb[e] = du[e] * (v[e] - pp[e]);
        G[e] = a * dSt;
      }
      const float dk = row_sum(xk), da = row_sum(xa);
      const int64_t prow = (int64_t(slab) * p.rows + row) * DK + i;
      if ((t % kTPR) == 0) {
        p.part_dq[prow] = dq;
        p.part_dk[prow] = dk;
        p.part_da[prow] = da;
      }
      if (i == 0) {
        float dv8[kCPT];
#pragma unroll
        for (int e = 0; e < kCPT; ++e) dv8[e] = bt * du[e];
        stf8(p.dv + row * DV + col, dv8);
        const float db = row_sum(xb);
        if (t == 0) p.part_db[int64_t(slab) * p.rows + row] = db;
      }
    }
    lds_sync();   // the next chunk rewrites sU, sP
  }
  if (p.d_state_in) stf8(p.d_state_in + state_off, G);
}

// dq, dk, dalpha (per row) and dbeta: sums of the per-slab partials.
template <int DK>
__global__ __launch_bounds__(256) void kda_bwd_reduce_kernel(BackwardArgs p) {
  const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;   // (token row, key row)
  const int64_t total = p.rows * DK;
  const int nslab = p.DV / kVS;
  if (idx < total) {
    float q = 0.f, k = 0.f, a = 0.f;
    for (int s = 0; s < nslab; ++s) {
      q += p.part_dq[s * total + idx];
      k += p.part_dk[s * total + idx];
      a += p.part_da[s * total + idx];
    }
    p.dq[idx] = q;
    p.dk[idx] = k;
    p.dalpha[idx] = a;
  }
  if (idx < p.rows) {
    float b = 0.f;
    for (int s = 0; s < nslab; ++s) b += p.part_db[s * p.rows + idx];
    p.dbeta[idx] = b;
  }
}

template <int DK, bool BF16>
void launch_bwd_t(const BackwardArgs& a, hipStream_t st) {
  const unsigned nb = unsigned(int64_t(a.N) * a.H * (a.DV / kVS));
  hipLaunchKernelGGL((kda_bwd_kernel<DK, BF16>), dim3(nb), dim3(DK * kTPR), 0, st, a);
  const int64_t total = a.rows * DK;
  hipLaunchKernelGGL((kda_bwd_reduce_kernel<DK>), dim3(unsigned((total + 255) / 256)), dim3(256),
                     0, st, a);
}

}  // namespace

size_t backward_scratch_bytes(int N, int H, int DK, int DV) {
  return size_t(N) * H * (DV / kVS) * size_t(kC) * DK * kTPR * kCPT * 4;
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

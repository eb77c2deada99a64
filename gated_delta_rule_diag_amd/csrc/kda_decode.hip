// KDA recurrent decode step on gfx950: one token for each (sequence, head).
//
// Token-wise mode of "Kimi Delta Attention 徹底解説" (tech-tide.dev), section
// "Kimi Delta Attention の仕組み": decay the state per key channel, write the
// delta-rule error, read.  One pass over the state is enough because
//     p  = S^T (alpha * k)            prediction from the decayed state
//     r  = S^T (alpha * q)
//     u  = beta (v - p)               the value actually written
//     S' = Diag(alpha) S + k u^T
//     o  = S'^T q = r + (k . q) u
// so every state element is read once and written once: the step is bound by
// HBM bandwidth (64 KiB read + 64 KiB written per (sequence, head) at d=128).
//
// One workgroup of 256 threads per (sequence, head).  Thread t owns value
// columns 4*(t % CG) .. +3 (CG = DV/4 column groups, 16-byte accesses) and
// key rows r = t / CG + RG*m (RG = 256/CG row groups), so each wave reads
// whole 512-byte rows per instruction.  The two column reductions go through
// LDS; the update is applied in registers and written back in place.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(uint32_t(b) << 16);
}

template <bool BF16>
__device__ __forceinline__ float load_in(const void* p, int64_t i) {
  if constexpr (BF16) {
    return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  } else {
    return static_cast<const float*>(p)[i];
  }
}

template <int DK, int DV, bool BF16>
__global__ __launch_bounds__(kThreads) void kda_decode_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, float* __restrict__ state,
    float* __restrict__ o) {
  constexpr int CG = DV / 4;          // column groups of 4 floats
  constexpr int RG = kThreads / CG;   // row groups
  constexpr int RPT = DK / RG;        // rows per thread
  static_assert(RPT * RG == DK, "layout");

  __shared__ float s_ak[DK];          // alpha * k
  __shared__ float s_aq[DK];          // alpha * q
  __shared__ float s_a[DK];           // alpha
  __shared__ float s_k[DK];
  __shared__ float s_part[2][RG][DV]; // partial column sums of p and r
  __shared__ float s_u[DV];
  __shared__ float s_kq[kThreads / 64];

  const int t = threadIdx.x;
  const int64_t pair = blockIdx.x;    // (sequence, head) flattened
  const int cg = t % CG;
  const int rg = t / CG;

  // Small per-pair vectors.
  float kq_part = 0.f;
  if (t < DK) {
    const float kk = load_in<BF16>(k, pair * DK + t);
    const float qq = load_in<BF16>(q, pair * DK + t);
    const float aa = alpha[pair * DK + t];
    s_ak[t] = aa * kk;
    s_aq[t] = aa * qq;
    s_a[t] = aa;
    s_k[t] = kk;
    kq_part = kk * qq;
  }
  // k . q: wave reduction then LDS.
  for (int off = 32; off > 0; off >>= 1) kq_part += __shfl_xor(kq_part, off);
  if ((t & 63) == 0) s_kq[t >> 6] = kq_part;

  // Stream this thread's slice of the state into registers.
  float4* S4 = reinterpret_cast<float4*>(state + pair * DK * DV);
  float4 s[RPT];
#pragma unroll
  for (int m = 0; m < RPT; ++m) s[m] = S4[(rg + RG * m) * CG + cg];
  __syncthreads();

  // Partial column sums over this thread's rows.
  float4 pp = make_float4(0.f, 0.f, 0.f, 0.f), rr = pp;
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int row = rg + RG * m;
    const float ak = s_ak[row], aq = s_aq[row];
    pp.x += ak * s[m].x; pp.y += ak * s[m].y; pp.z += ak * s[m].z; pp.w += ak * s[m].w;
    rr.x += aq * s[m].x; rr.y += aq * s[m].y; rr.z += aq * s[m].z; rr.w += aq * s[m].w;
  }
  *reinterpret_cast<float4*>(&s_part[0][rg][4 * cg]) = pp;
  *reinterpret_cast<float4*>(&s_part[1][rg][4 * cg]) = rr;
  __syncthreads();

  if (t < DV) {
    float p = 0.f, r = 0.f;
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      p += s_part[0][g][t];
      r += s_part[1][g][t];
    }
    float kq = 0.f;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) kq += s_kq[w];
    const float u = beta[pair] * (load_in<BF16>(v, pair * DV + t) - p);
    s_u[t] = u;
    o[pair * DV + t] = r + kq * u;
  }
  __syncthreads();

  const float4 u4 = *reinterpret_cast<const float4*>(&s_u[4 * cg]);
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int row = rg + RG * m;
    const float a = s_a[row], kk = s_k[row];
    float4 x = s[m];
    x.x = a * x.x + kk * u4.x;
    x.y = a * x.y + kk * u4.y;
    x.z = a * x.z + kk * u4.z;
    x.w = a * x.w + kk * u4.w;
    S4[row * CG + cg] = x;
  }
}

// ------------------------------------------------------------ pooled decode --
// Up to L tokens per sequence, states gathered from a pool by slot index
// (continuous batching; speculative drafts).  Same thread layout as above; the
// state slice stays in registers across the sequence's tokens, so the pool is
// read once and written once whatever L is.  Each token costs three barriers:
// its small vectors are double-buffered by token parity, so the writes for
// token j+1 never meet the reads of token j (every thread has passed token j's
// last barrier before anyone writes them, and token j-1's buffer is free).
template <int DK, int DV, bool BF16>
__global__ __launch_bounds__(kThreads) void kda_decode_pool_kernel(PoolDecodeArgs p) {
  constexpr int CG = DV / 4;
  constexpr int RG = kThreads / CG;
  constexpr int RPT = DK / RG;
  static_assert(RPT * RG == DK, "layout");

  __shared__ float s_ak[2][DK];
  __shared__ float s_aq[2][DK];
  __shared__ float s_a[2][DK];
  __shared__ float s_k[2][DK];
  __shared__ float s_part[2][RG][DV];
  __shared__ float s_u[DV];
  __shared__ float s_kq[2][kThreads / 64];

  const int t = threadIdx.x;
  const int cg = t % CG;
  const int rg = t / CG;
  const int H = p.H, L = p.L;
  const int64_t n = int64_t(blockIdx.x) / H;
  const int h = int(int64_t(blockIdx.x) % H);
  const int slot = p.state_idx ? p.state_idx[n] : int(n);
  int len = p.num_tokens ? p.num_tokens[n] : L;
  len = len < 0 ? 0 : (len > L ? L : len);
  if (slot < 0 || slot >= p.pool_size) len = 0;   // padding row

  // Outputs of tokens that are not processed are zero.
  if (t < DV)
    for (int j = len; j < L; ++j) p.o[((n * L + j) * H + h) * DV + t] = 0.f;
  if (len == 0) return;   // uniform over the workgroup, before any barrier

  // Token j of this (sequence, head) is row (n*L + j)*H + h of the inputs.
  auto row_of = [&](int j) { return (n * L + j) * H + h; };
  float pk = 0.f, pq = 0.f, pa = 0.f, pv = 0.f, pb = 0.f;   // next token's inputs
  auto load_token = [&](int64_t r) {
    if (t < DK) {
      pk = load_in<BF16>(p.k, r * DK + t);
      pq = load_in<BF16>(p.q, r * DK + t);
      pa = p.alpha[r * DK + t];
    }
    if (t < DV) {
      pv = load_in<BF16>(p.v, r * DV + t);
      pb = p.beta[r];
    }
  };
  load_token(row_of(0));

  float4* S4 = reinterpret_cast<float4*>(p.pool + (int64_t(slot) * H + h) * DK * DV);
  float4 s[RPT];
#pragma unroll
  for (int m = 0; m < RPT; ++m) s[m] = S4[(rg + RG * m) * CG + cg];

  for (int j = 0; j < len; ++j) {
    const int b = j & 1;
    const int64_t row = row_of(j);
    const float kk = pk, qq = pq, aa = pa, vv = pv, bb = pb;
    if (j + 1 < len) load_token(row_of(j + 1));
    float kq_part = 0.f;
    if (t < DK) {
      s_ak[b][t] = aa * kk;
      s_aq[b][t] = aa * qq;
      s_a[b][t] = aa;
      s_k[b][t] = kk;
      kq_part = kk * qq;
    }
    for (int off = 32; off > 0; off >>= 1) kq_part += __shfl_xor(kq_part, off);
    if ((t & 63) == 0) s_kq[b][t >> 6] = kq_part;
    __syncthreads();

    float4 pp = make_float4(0.f, 0.f, 0.f, 0.f), rr = pp;
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
      const int r = rg + RG * m;
      const float ak = s_ak[b][r], aq = s_aq[b][r];
      pp.x += ak * s[m].x; pp.y += ak * s[m].y; pp.z += ak * s[m].z; pp.w += ak * s[m].w;
      rr.x += aq * s[m].x; rr.y += aq * s[m].y; rr.z += aq * s[m].z; rr.w += aq * s[m].w;
    }
    *reinterpret_cast<float4*>(&s_part[0][rg][4 * cg]) = pp;
    *reinterpret_cast<float4*>(&s_part[1][rg][4 * cg]) = rr;
    __syncthreads();

    if (t < DV) {
      float pr = 0.f, rs = 0.f;
#pragma unroll
      for (int g = 0; g < RG; ++g) {
        pr += s_part[0][g][t];
        rs += s_part[1][g][t];
      }
      float kq = 0.f;
#pragma unroll
      for (int w = 0; w < kThreads / 64; ++w) kq += s_kq[b][w];
      const float u = bb * (vv - pr);
      s_u[t] = u;
      p.o[row * DV + t] = rs + kq * u;
    }
    __syncthreads();

    const float4 u4 = *reinterpret_cast<const float4*>(&s_u[4 * cg]);
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
      const int r = rg + RG * m;
      const float a = s_a[b][r], kr = s_k[b][r];
      s[m].x = a * s[m].x + kr * u4.x;
      s[m].y = a * s[m].y + kr * u4.y;
      s[m].z = a * s[m].z + kr * u4.z;
      s[m].w = a * s[m].w + kr * u4.w;
    }
    if (p.token_states) {
      float4* T4 = reinterpret_cast<float4*>(p.token_states + row * DK * DV);
#pragma unroll
      for (int m = 0; m < RPT; ++m) T4[(rg + RG * m) * CG + cg] = s[m];
    }
  }
#pragma unroll
  for (int m = 0; m < RPT; ++m) S4[(rg + RG * m) * CG + cg] = s[m];
}

template <int DK, int DV>
int launch_decode_t(const DecodeArgs& a, hipStream_t st) {
  dim3 grid(unsigned(int64_t(a.N) * a.H)), block(kThreads);
  if (a.in_bf16)
    hipLaunchKernelGGL((kda_decode_kernel<DK, DV, true>), grid, block, 0, st, a.q, a.k, a.v,
                       a.alpha, a.beta, a.state, a.o);
  else
    hipLaunchKernelGGL((kda_decode_kernel<DK, DV, false>), grid, block, 0, st, a.q, a.k, a.v,
                       a.alpha, a.beta, a.state, a.o);
  return 0;
}

template <int DK, int DV>
void launch_pool_t(const PoolDecodeArgs& a, hipStream_t st) {
  dim3 grid(unsigned(int64_t(a.N) * a.H)), block(kThreads);
  if (a.in_bf16)
    hipLaunchKernelGGL((kda_decode_pool_kernel<DK, DV, true>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((kda_decode_pool_kernel<DK, DV, false>), grid, block, 0, st, a);
}

}  // namespace

int launch_decode_pool(const PoolDecodeArgs& a, void* stream, const char** msg) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (a.DK == 128 && a.DV == 128) launch_pool_t<128, 128>(a, st);
  else if (a.DK == 128 && a.DV == 64) launch_pool_t<128, 64>(a, st);
  else if (a.DK == 64 && a.DV == 128) launch_pool_t<64, 128>(a, st);
  else if (a.DK == 64 && a.DV == 64) launch_pool_t<64, 64>(a, st);
  else {
    *msg = "unsupported DK/DV";
    return 1;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    *msg = hipGetErrorString(e);
    return 1;
  }
  return 0;
}

int launch_decode(const DecodeArgs& a, void* stream, const char** msg) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (a.DK == 128 && a.DV == 128) launch_decode_t<128, 128>(a, st);
  else if (a.DK == 128 && a.DV == 64) launch_decode_t<128, 64>(a, st);
  else if (a.DK == 64 && a.DV == 128) launch_decode_t<64, 128>(a, st);
  else if (a.DK == 64 && a.DV == 64) launch_decode_t<64, 64>(a, st);
  else {
    *msg = "unsupported DK/DV";
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

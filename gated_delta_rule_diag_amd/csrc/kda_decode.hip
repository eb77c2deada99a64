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

}  // namespace

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

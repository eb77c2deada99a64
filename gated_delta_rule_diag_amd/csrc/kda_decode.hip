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
// The reductions run over the key rows, so the value columns could split
// freely, but they do not: one workgroup of 256 threads owns the whole state
// of a (sequence, head), 64 KiB at d=128, i.e. whole 512-byte rows.  Thread t
// owns columns 4*(t % CG) .. +3 (CG = DV/4 column groups, 16-byte accesses)
// and key rows r = t / CG + RG*m (RG = 256/CG row groups), so a wave reads two
// whole rows per instruction and a workgroup streams one contiguous 64 KiB
// block.  The two column reductions go through LDS; the update is applied in
// registers and written back in place with non-temporal accesses both ways.
// Measured on a 256 x 32 step at d=128 that follows an 8192-token, 32-head
// prefill: whole rows cut the pair from 650 to 643 us against
// half rows (64 columns, two workgroups per state).  Ordinary loads make the
// decode alone faster when it runs back to back (159 against 191 us), but
// they leave the caches full of state lines that the following prefill must
// write back first, so the pair gets slower (667 us).  The
// state of sequence n is slot state_idx[n] of a pool (slot n without an
// index); a slot outside the pool, or a token count of 0, marks a padding row
// whose output is zero.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

typedef float f4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 ld_nt(const float4* p) {
  const f4v v = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}


__device__ __forceinline__ void st_nt(float4* p, float4 x) {
  const f4v v = {x.x, x.y, x.z, x.w};
  __builtin_nontemporal_store(v, reinterpret_cast<f4v*>(p));
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(uint32_t(b) << 16);
}

// Column sums of a wave's row groups: lanes l, l + CG, l + 2 CG, ... of a wave
// hold the same four columns for different rows.
template <int CG>
__device__ __forceinline__ float4 wave_colsum(float4 x) {
#pragma unroll
  for (int off = CG; off < 64; off <<= 1) {
    x.x += __shfl_xor(x.x, off);
    x.y += __shfl_xor(x.y, off);
    x.z += __shfl_xor(x.z, off);
    x.w += __shfl_xor(x.w, off);
  }
  return x;
}

template <bool BF16>
__device__ __forceinline__ float load_in(const void* p, int64_t i) {
  if constexpr (BF16) {
    return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  } else {
    return static_cast<const float*>(p)[i];
  }
}

template <int DK, int DV, int kVC, bool BF16>
__global__ __launch_bounds__(kThreads) void kda_decode_kernel(PoolDecodeArgs p) {
  constexpr int CS = DV / kVC;        // workgroups per (sequence, head)
  constexpr int CG = kVC / 4;         // column groups of 4 floats
  constexpr int RG = kThreads / CG;   // row groups
  constexpr int RPT = DK / RG;        // rows per thread
  static_assert(RPT * RG == DK && CS * kVC == DV, "layout");

  __shared__ float s_ak[DK];          // alpha * k
  __shared__ float s_aq[DK];          // alpha * q
  __shared__ float s_a[DK];           // alpha
  __shared__ float s_k[DK];
  __shared__ float s_part[2][kWaves][kVC]; // per-wave column sums of p and r
  __shared__ float s_u[kVC];
  __shared__ float s_kq[kThreads / 64];

  const int t = threadIdx.x;
  const int64_t pair = blockIdx.x / CS;  // (sequence, head) flattened: token row of the inputs
  const int c0 = int(blockIdx.x % CS) * kVC;
  const int cg = t % CG;
  const int rg = t / CG;
  const void* __restrict__ q = p.q;
  const void* __restrict__ k = p.k;
  const void* __restrict__ v = p.v;
  const float* __restrict__ alpha = p.alpha;
  const float* __restrict__ beta = p.beta;
  float* __restrict__ o = p.o;
  const int64_t n = pair / p.H;
  const int slot = p.state_idx ? p.state_idx[n] : int(n);
  if (slot < 0 || slot >= p.pool_size || (p.num_tokens && p.num_tokens[n] <= 0)) {
    if (t < kVC) o[pair * DV + c0 + t] = 0.f;   // padding row
    return;
  }
  float* __restrict__ state = p.pool + (int64_t(slot) * p.H + (pair - n * p.H)) * DK * DV + c0;

  // The small per-pair vectors and this thread's slice of the state are all
  // loaded before any of them is used, so that the workgroup waits for one
  // memory latency, not three.  (Threads past DK or kVC read a valid element
  // they do not use.)
  const int tk = t < DK ? t : DK - 1;
  const float kk = load_in<BF16>(k, pair * DK + tk);
  const float qq = load_in<BF16>(q, pair * DK + tk);
  const float aa = alpha[p.alpha_scalar ? pair : pair * DK + tk];
  const float vv = load_in<BF16>(v, pair * DV + c0 + (t < kVC ? t : 0));
  const float bb = beta[pair];
  float4* S4 = reinterpret_cast<float4*>(state);
  float4 s[RPT];
#pragma unroll
  for (int m = 0; m < RPT; ++m) s[m] = ld_nt(&S4[(rg + RG * m) * (DV / 4) + cg]);

  float kq_part = 0.f;
  if (t < DK) {
    s_ak[t] = aa * kk;
    s_aq[t] = aa * qq;
    s_a[t] = aa;
    s_k[t] = kk;
    kq_part = kk * qq;
  }
  // k . q: wave reduction then LDS.
  for (int off = 32; off > 0; off >>= 1) kq_part += __shfl_xor(kq_part, off);
  if ((t & 63) == 0) s_kq[t >> 6] = kq_part;
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
  pp = wave_colsum<CG>(pp);
  rr = wave_colsum<CG>(rr);
  if ((t & 63) < CG) {
    *reinterpret_cast<float4*>(&s_part[0][t >> 6][4 * cg]) = pp;
    *reinterpret_cast<float4*>(&s_part[1][t >> 6][4 * cg]) = rr;
  }
  __syncthreads();

  if (t < kVC) {
    float p = 0.f, r = 0.f;
#pragma unroll
    for (int g = 0; g < kWaves; ++g) {
      p += s_part[0][g][t];
      r += s_part[1][g][t];
    }
    float kq = 0.f;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) kq += s_kq[w];
    const float u = bb * (vv - p);
    s_u[t] = u;
    o[pair * DV + c0 + t] = r + kq * u;
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
    st_nt(&S4[row * (DV / 4) + cg], x);
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
template <int DK, int DV, int kVC, bool BF16, bool TS>
__global__ __launch_bounds__(kThreads) void kda_decode_pool_kernel(PoolDecodeArgs p) {
  constexpr int CS = DV / kVC;
  constexpr int CG = kVC / 4;
  constexpr int RG = kThreads / CG;
  constexpr int RPT = DK / RG;
  static_assert(RPT * RG == DK && CS * kVC == DV, "layout");

  __shared__ float s_ak[2][DK];
  __shared__ float s_aq[2][DK];
  __shared__ float s_a[2][DK];
  __shared__ float s_k[2][DK];
  __shared__ float s_part[2][kWaves][kVC];
  __shared__ float s_u[kVC];
  __shared__ float s_kq[2][kThreads / 64];

  const int t = threadIdx.x;
  const int cg = t % CG;
  const int rg = t / CG;
  const int H = p.H, L = p.L;
  const int64_t pair = blockIdx.x / CS;
  const int c0 = int(blockIdx.x % CS) * kVC;
  const int64_t n = pair / H;
  const int h = int(pair % H);
  const int slot = p.state_idx ? p.state_idx[n] : int(n);
  int len = p.num_tokens ? p.num_tokens[n] : L;
  len = len < 0 ? 0 : (len > L ? L : len);
  if (slot < 0 || slot >= p.pool_size) len = 0;   // padding row

  // Outputs of tokens that are not processed are zero.
  if (t < kVC)
    for (int j = len; j < L; ++j) p.o[((n * L + j) * H + h) * DV + c0 + t] = 0.f;
  if (len == 0) return;   // uniform over the workgroup, before any barrier

  // Token j of this (sequence, head) is row (n*L + j)*H + h of the inputs.
  auto row_of = [&](int j) { return (n * L + j) * H + h; };
  float pk = 0.f, pq = 0.f, pa = 0.f, pv = 0.f, pb = 0.f;   // next token's inputs
  // Unconditional loads (threads past DK or kVC read an element they do not
  // use): loads under a branch make the compiler wait for them at the join,
  // before the state loads that follow are issued.
  const int tk = t < DK ? t : DK - 1, tv = t < kVC ? t : 0;
  auto load_token = [&](int64_t r) {
    pk = load_in<BF16>(p.k, r * DK + tk);
    pq = load_in<BF16>(p.q, r * DK + tk);
    pa = p.alpha[p.alpha_scalar ? r : r * DK + tk];
    pv = load_in<BF16>(p.v, r * DV + c0 + tv);
    pb = p.beta[r];
  };
  load_token(row_of(0));

  float4* S4 = reinterpret_cast<float4*>(p.pool + (int64_t(slot) * H + h) * DK * DV + c0);
  float4 s[RPT];
#pragma unroll
  for (int m = 0; m < RPT; ++m) s[m] = ld_nt(&S4[(rg + RG * m) * (DV / 4) + cg]);

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
    pp = wave_colsum<CG>(pp);
    rr = wave_colsum<CG>(rr);
    if ((t & 63) < CG) {
      *reinterpret_cast<float4*>(&s_part[0][t >> 6][4 * cg]) = pp;
      *reinterpret_cast<float4*>(&s_part[1][t >> 6][4 * cg]) = rr;
    }
    __syncthreads();

    if (t < kVC) {
      float pr = 0.f, rs = 0.f;
#pragma unroll
      for (int g = 0; g < kWaves; ++g) {
        pr += s_part[0][g][t];
        rs += s_part[1][g][t];
      }
      float kq = 0.f;
#pragma unroll
      for (int w = 0; w < kThreads / 64; ++w) kq += s_kq[b][w];
      const float u = bb * (vv - pr);
      s_u[t] = u;
      p.o[row * DV + c0 + t] = rs + kq * u;
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
    if constexpr (TS) {
      float4* T4 = reinterpret_cast<float4*>(p.token_states + row * DK * DV + c0);
#pragma unroll
      for (int m = 0; m < RPT; ++m) st_nt(&T4[(rg + RG * m) * (DV / 4) + cg], s[m]);
    }
  }
#pragma unroll
  for (int m = 0; m < RPT; ++m) st_nt(&S4[(rg + RG * m) * (DV / 4) + cg], s[m]);
}

// One token per sequence without per-token states: the single-step kernel;
// otherwise the multi-token kernel.
// Value columns per workgroup: the whole row, for the single step (contiguous
// 64 KiB per workgroup streams best) and for several tokens (the per-token
// barriers and small-vector loads are paid once per (sequence, head)).
constexpr int kStepVC = 128;

template <int DK, int DV>
void launch_pool_t(const PoolDecodeArgs& a, hipStream_t st) {
  const int64_t pairs = int64_t(a.N) * a.H;
  dim3 block(kThreads);
  if (a.L == 1 && !a.token_states) {
    constexpr int VC = DV < kStepVC ? DV : kStepVC;
    dim3 grid(unsigned(pairs * (DV / VC)));
    if (a.in_bf16) hipLaunchKernelGGL((kda_decode_kernel<DK, DV, VC, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((kda_decode_kernel<DK, DV, VC, false>), grid, block, 0, st, a);
  } else if (a.token_states) {
    dim3 grid(static_cast<unsigned>(pairs));
    if (a.in_bf16) hipLaunchKernelGGL((kda_decode_pool_kernel<DK, DV, DV, true, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((kda_decode_pool_kernel<DK, DV, DV, false, true>), grid, block, 0, st, a);
  } else {
    dim3 grid(static_cast<unsigned>(pairs));
    if (a.in_bf16) hipLaunchKernelGGL((kda_decode_pool_kernel<DK, DV, DV, true, false>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((kda_decode_pool_kernel<DK, DV, DV, false, false>), grid, block, 0, st, a);
  }
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
  PoolDecodeArgs pa{};
  pa.N = a.N; pa.L = 1; pa.H = a.H; pa.DK = a.DK; pa.DV = a.DV;
  pa.in_bf16 = a.in_bf16;
  pa.q = a.q; pa.k = a.k; pa.v = a.v; pa.alpha = a.alpha; pa.beta = a.beta;
  pa.state_idx = nullptr; pa.num_tokens = nullptr;
  pa.pool = a.state; pa.pool_size = a.N;
  pa.o = a.o; pa.token_states = nullptr;
  pa.alpha_scalar = a.alpha_scalar;
  return launch_decode_pool(pa, stream, msg);
}

}  // namespace kda

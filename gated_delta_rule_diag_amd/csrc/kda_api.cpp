// Host side of the KDA C ABI: argument checks and dispatch.
//
// Every check runs before the first HIP call, so an invalid call returns its
// status having enqueued nothing and touched no output.  This file has no HIP
// dependency; the launchers live in the .hip sources.

#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <rocprofiler-sdk-roctx/roctx.h>

#include <atomic>
#include <string>

#include "kda.h"
#include "kda_internal.h"

namespace {

// A roctx range over one ABI call (its name), so that a rocprofv3 trace with
// markers shows which entry point launched which kernels.
struct TraceRange {
  explicit TraceRange(const char* name) { roctxRangePushA(name); }
  ~TraceRange() { roctxRangePop(); }
  TraceRange(const TraceRange&) = delete;
  TraceRange& operator=(const TraceRange&) = delete;
};

std::atomic<int> g_prefill_form{0}, g_prefill_nsub{0}, g_prefill_seg{0}, g_bwd_window{0};

thread_local std::string g_last_error;

kda_status_t fail(kda_status_t s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

kda_status_t fail(kda_status_t s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

kda_status_t ok() {
  g_last_error.clear();
  return KDA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
  if (a == nullptr || b == nullptr || an == 0 || bn == 0) return false;
  uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + bn && b0 < a0 + an;
}

bool dims_ok(int d) { return d == 64 || d == 128; }

// Shared checks of the prefill entry points.  `ntok` is the number of tokens
// on the packed axis, `nseq` the number of states.
kda_status_t check_prefill(int nseq, int64_t ntok, int H, int DK, int DV, int chunk,
                           kda_dtype_t dt, const void* q, const void* k, const void* v,
                           const float* alpha, const float* beta, const float* s_in,
                           const float* o, const float* s_out, bool alpha_scalar) {
  if (nseq < 0 || ntok < 0 || H < 0)
    return fail(KDA_ERR_SHAPE, "negative size (sequences=%d tokens=%lld H=%d)", nseq,
                (long long)ntok, H);
  if (!dims_ok(DK) || !dims_ok(DV))
    return fail(KDA_ERR_UNSUPPORTED, "DK=%d DV=%d: only 64 and 128 are supported", DK, DV);
  if (chunk != 64) return fail(KDA_ERR_UNSUPPORTED, "chunk=%d: only 64 is supported", chunk);
  if (dt != KDA_F32 && dt != KDA_BF16) return fail(KDA_ERR_DTYPE, "unknown in_dtype %d", (int)dt);
  // (the kernels address the rows of one chunk with 32-bit offsets:
  // 64 * H * 128 elements of 4 bytes stay below 2^31 for H <= 65536)
  if (ntok > (int64_t(1) << 31) - 1 || int64_t(nseq) * H > (int64_t(1) << 24) || H > 65536)
    return fail(KDA_ERR_UNSUPPORTED, "too large: tokens=%lld sequences*H=%lld H=%d (at most 65536)",
                (long long)ntok, (long long)nseq * H, H);
  const size_t esz = dt == KDA_BF16 ? 2 : 4;
  const size_t nk = size_t(ntok) * H * DK, nv = size_t(ntok) * H * DV, nb = size_t(ntok) * H;
  const size_t ns = size_t(nseq) * H * DK * DV;
  const size_t na = (alpha_scalar ? nb : nk) * 4;   // bytes of alpha
  if (nk > 0) {
    if (!q || !k || !v || !alpha || !beta || !o)
      return fail(KDA_ERR_NULL, "q, k, v, alpha, beta and o must be non-NULL");
  }
  const void* ptrs[] = {q, k, v, alpha, beta, s_in, o, s_out};
  const char* names[] = {"q", "k", "v", "alpha", "beta", "state_in", "o", "state_out"};
  for (int i = 0; i < 8; ++i)
    if (ptrs[i] && !aligned16(ptrs[i]))
      return fail(KDA_ERR_ALIGN, "%s is not 16-byte aligned", names[i]);
  // o must not overlap any input or state; state_out may only equal state_in.
  const size_t obytes = nv * 4;
  if (overlaps(o, obytes, q, nk * esz) || overlaps(o, obytes, k, nk * esz) ||
      overlaps(o, obytes, v, nv * esz) || overlaps(o, obytes, alpha, na) ||
      overlaps(o, obytes, beta, nb * 4) || overlaps(o, obytes, s_in, ns * 4) ||
      overlaps(o, obytes, s_out, ns * 4))
    return fail(KDA_ERR_SHAPE, "o overlaps an input or a state");
  if (s_out && s_out != s_in &&
      (overlaps(s_out, ns * 4, q, nk * esz) || overlaps(s_out, ns * 4, k, nk * esz) ||
       overlaps(s_out, ns * 4, v, nv * esz) || overlaps(s_out, ns * 4, alpha, na) ||
       overlaps(s_out, ns * 4, beta, nb * 4) || overlaps(s_out, ns * 4, s_in, ns * 4)))
    return fail(KDA_ERR_SHAPE, "state_out overlaps an input (only state_out == state_in is allowed)");
  return KDA_OK;
}

}  // namespace

namespace kda {
Tuning tuning() {
  return Tuning{g_prefill_form.load(std::memory_order_relaxed), g_prefill_nsub.load(std::memory_order_relaxed),
                g_prefill_seg.load(std::memory_order_relaxed), g_bwd_window.load(std::memory_order_relaxed)};
}
}  // namespace kda

extern "C" {

int kda_abi_version(void) { return (1 << 16) | 1; }

kda_status_t kda_internal_set_tuning(int prefill_form, int prefill_nsub, int prefill_seg,
                                     int bwd_window) {
  if (prefill_form < 0 || prefill_form > 2)
    return fail(KDA_ERR_SHAPE, "prefill_form=%d: 0 (by shape), 1 (fused) or 2 (staged)", prefill_form);
  if (prefill_nsub != 0 && prefill_nsub != 1 && prefill_nsub != 2 && prefill_nsub != 4 &&
      prefill_nsub != 8)
    return fail(KDA_ERR_SHAPE, "prefill_nsub=%d: 0, 1, 2, 4 or 8", prefill_nsub);
  if (prefill_seg < 0 || bwd_window < 0)
    return fail(KDA_ERR_SHAPE, "prefill_seg=%d bwd_window=%d: must be >= 0", prefill_seg, bwd_window);
  g_prefill_form.store(prefill_form, std::memory_order_relaxed);
  g_prefill_nsub.store(prefill_nsub, std::memory_order_relaxed);
  g_prefill_seg.store(prefill_seg, std::memory_order_relaxed);
  g_bwd_window.store(bwd_window, std::memory_order_relaxed);
  return ok();
}

const char* kda_status_string(kda_status_t s) {
  switch (s) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_NULL: return "KDA_ERR_NULL";
    case KDA_ERR_SHAPE: return "KDA_ERR_SHAPE";
    case KDA_ERR_DTYPE: return "KDA_ERR_DTYPE";
    case KDA_ERR_ALIGN: return "KDA_ERR_ALIGN";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
    case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE";
    case KDA_ERR_HIP: return "KDA_ERR_HIP";
  }
  return "KDA_ERR_UNKNOWN";
}

const char* kda_last_error_message(void) { return g_last_error.c_str(); }

size_t kda_chunk_prefill_workspace_size(int B, int T, int H, int DK, int DV, int chunk) {
  if (B < 0 || T < 0 || H < 0 || !dims_ok(DK) || !dims_ok(DV) || chunk != 64) return 0;
  return kda::prefill_workspace_bytes(B, int64_t(B) * T, H, DK, DV, false);
}

size_t kda_chunk_prefill_varlen_workspace_size(int N, int T_total, int H, int DK, int DV,
                                               int chunk) {
  if (N < 0 || T_total < 0 || H < 0 || !dims_ok(DK) || !dims_ok(DV) || chunk != 64) return 0;
  return kda::prefill_workspace_bytes(N, T_total, H, DK, DV, true);
}

static kda_status_t run_prefill(kda::PrefillArgs& a, size_t need, void* stream) {
  if (need > 0 && (a.workspace == nullptr || a.workspace_bytes < need))
    return fail(KDA_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given", need,
                a.workspace ? a.workspace_bytes : size_t(0));
  if (a.workspace && !aligned16(a.workspace))
    return fail(KDA_ERR_ALIGN, "workspace is not 16-byte aligned");
  if (need > 0) {
    const size_t esz = a.in_bf16 ? 2 : 4;
    const size_t nk = size_t(a.T_total) * a.H * a.DK, nv = size_t(a.T_total) * a.H * a.DV;
    const size_t nb = size_t(a.T_total) * a.H, ns = size_t(a.N) * a.H * a.DK * a.DV;
    const size_t nsnap = !a.snapshots ? 0
                         : (a.snap_offsets ? size_t(a.snap_rows)
                                           : size_t(a.N) * size_t(a.T_fixed / (64 * a.snap_every))) *
                               a.H * a.DK * a.DV;
    const void* ptrs[] = {a.q, a.k, a.v, a.alpha, a.beta, a.state_in, a.o, a.state_out, a.snapshots};
    const size_t sizes[] = {nk * esz, nk * esz, nv * esz, (a.alpha_scalar ? nb : nk) * 4, nb * 4,
                            ns * 4, nv * 4, ns * 4, nsnap * 4};
    for (int i = 0; i < 9; ++i)
      if (overlaps(a.workspace, need, ptrs[i], sizes[i]))
        return fail(KDA_ERR_SHAPE, "workspace overlaps another argument");
  }
  if (a.N == 0 || a.H == 0) return ok();
  const char* msg = nullptr;
  if (kda::launch_prefill(a, stream, &msg) != 0)
    return fail(KDA_ERR_HIP, "prefill launch failed: %s", msg ? msg : "?");
  return ok();
}

static kda_status_t prefill_fixed(int B, int T, int H, int DK, int DV, int chunk,
                                  kda_dtype_t in_dtype, const void* q, const void* k,
                                  const void* v, const float* alpha, const float* beta,
                                  const float* state_in, float* o, float* state_out,
                                  void* workspace, size_t workspace_bytes, void* stream,
                                  bool alpha_scalar) {
  if (B < 0 || T < 0) return fail(KDA_ERR_SHAPE, "negative size (B=%d T=%d)", B, T);
  kda_status_t s = check_prefill(B, int64_t(B) * T, H, DK, DV, chunk, in_dtype, q, k, v, alpha,
                                 beta, state_in, o, state_out, alpha_scalar);
  if (s != KDA_OK) return s;
  kda::PrefillArgs a{};
  a.N = B;
  a.T_fixed = T;
  a.cu_seqlens = nullptr;
  a.T_total = int64_t(B) * T;
  a.H = H; a.DK = DK; a.DV = DV;
  a.in_bf16 = in_dtype == KDA_BF16;
  a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta;
  a.state_in = state_in; a.o = o; a.state_out = state_out;
  a.workspace = workspace; a.workspace_bytes = workspace_bytes;
  a.alpha_scalar = alpha_scalar;
  return run_prefill(a, kda::prefill_workspace_bytes(B, a.T_total, H, DK, DV, false), stream);
}

kda_status_t kda_chunk_prefill(int B, int T, int H, int DK, int DV, int chunk,
                               kda_dtype_t in_dtype, const void* q, const void* k,
                               const void* v, const float* alpha, const float* beta,
                               const float* state_in, float* o, float* state_out,
                               void* workspace, size_t workspace_bytes, void* stream) {
  TraceRange trace_range("kda_chunk_prefill");
  return prefill_fixed(B, T, H, DK, DV, chunk, in_dtype, q, k, v, alpha, beta, state_in, o,
                       state_out, workspace, workspace_bytes, stream, false);
}

kda_status_t kda_chunk_prefill_noalloc(int B, int T, int H, int DK, int DV, int chunk,
                                       kda_dtype_t in_dtype, const void* q, const void* k,
                                       const void* v, const float* alpha, const float* beta,
                                       const float* state_in, float* o, float* state_out,
                                       void* stream) {
  TraceRange trace_range("kda_chunk_prefill_noalloc");
  if (B < 0 || T < 0) return fail(KDA_ERR_SHAPE, "negative size (B=%d T=%d)", B, T);
  kda_status_t s = check_prefill(B, int64_t(B) * T, H, DK, DV, chunk, in_dtype, q, k, v, alpha,
                                 beta, state_in, o, state_out, false);
  if (s != KDA_OK) return s;
  kda::PrefillArgs a{};
  a.N = B;
  a.T_fixed = T;
  a.cu_seqlens = nullptr;
  a.T_total = int64_t(B) * T;
  a.H = H; a.DK = DK; a.DV = DV;
  a.in_bf16 = in_dtype == KDA_BF16;
  a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta;
  a.state_in = state_in; a.o = o; a.state_out = state_out;
  // The staged form's slots go to the static scratch in segments short enough
  // that one segment's slots and the carried state fit it.
  const size_t cap = kda::kNoallocScratchBytes;
  const size_t carry = size_t(B) * H * DK * DV * 4;
  const int64_t budget = carry < cap ? int64_t(cap - carry) : 1;
  const size_t need = kda::prefill_workspace_bytes(B, a.T_total, H, DK, DV, false, budget);
  if (need > cap)
    return fail(KDA_ERR_UNSUPPORTED,
                "B*H=%d pairs: the staged form needs %zu bytes of scratch (one chunk of slots "
                "and the carried state), the static scratch holds %zu",
                B * H, need, cap);
  if (a.N == 0 || a.H == 0) return ok();
  const char* msg = nullptr;
  if (need > 0) {
    void* ptr = kda::noalloc_scratch(&msg);
    if (ptr == nullptr) return fail(KDA_ERR_HIP, "static scratch: %s", msg ? msg : "?");
    a.workspace = ptr;
    a.workspace_bytes = cap;
    a.seg_budget = budget;
  }
  if (kda::launch_prefill(a, stream, &msg) != 0)
    return fail(KDA_ERR_HIP, "prefill launch failed: %s", msg ? msg : "?");
  return ok();
}

kda_status_t kda_chunk_prefill_scalar_gate(int B, int T, int H, int DK, int DV, int chunk,
                                           kda_dtype_t in_dtype, const void* q, const void* k,
                                           const void* v, const float* gate, const float* beta,
                                           const float* state_in, float* o, float* state_out,
                                           void* workspace, size_t workspace_bytes,
                                           void* stream) {
  TraceRange trace_range("kda_chunk_prefill_scalar_gate");
  return prefill_fixed(B, T, H, DK, DV, chunk, in_dtype, q, k, v, gate, beta, state_in, o,
                       state_out, workspace, workspace_bytes, stream, true);
}

kda_status_t kda_chunk_prefill_snapshots(int B, int T, int H, int DK, int DV, int chunk,
                                         kda_dtype_t in_dtype, const void* q, const void* k,
                                         const void* v, const float* alpha, const float* beta,
                                         const float* state_in, float* o, float* state_out,
                                         int every, float* snapshots, void* workspace,
                                         size_t workspace_bytes, void* stream) {
  TraceRange trace_range("kda_chunk_prefill_snapshots");
  if (B < 0 || T < 0) return fail(KDA_ERR_SHAPE, "negative size (B=%d T=%d)", B, T);
  if (every < 1) return fail(KDA_ERR_SHAPE, "every=%d: must be >= 1", every);
  kda_status_t s = check_prefill(B, int64_t(B) * T, H, DK, DV, chunk, in_dtype, q, k, v, alpha,
                                 beta, state_in, o, state_out, false);
  if (s != KDA_OK) return s;
  const int64_t nsnap = int64_t(T) / (int64_t(64) * every);
  const size_t sbytes = size_t(B) * size_t(nsnap) * H * DK * DV * 4;
  if (sbytes > 0) {
    if (!snapshots) return fail(KDA_ERR_NULL, "snapshots must be non-NULL (%lld per sequence)",
                                (long long)nsnap);
    if (!aligned16(snapshots)) return fail(KDA_ERR_ALIGN, "snapshots is not 16-byte aligned");
    const size_t esz = in_dtype == KDA_BF16 ? 2 : 4;
    const size_t nk = size_t(B) * T * H * DK, nv = size_t(B) * T * H * DV, nb = size_t(B) * T * H;
    const size_t ns = size_t(B) * H * DK * DV;
    if (overlaps(snapshots, sbytes, q, nk * esz) || overlaps(snapshots, sbytes, k, nk * esz) ||
        overlaps(snapshots, sbytes, v, nv * esz) || overlaps(snapshots, sbytes, alpha, nk * 4) ||
        overlaps(snapshots, sbytes, beta, nb * 4) || overlaps(snapshots, sbytes, state_in, ns * 4) ||
        overlaps(snapshots, sbytes, o, nv * 4) || overlaps(snapshots, sbytes, state_out, ns * 4))
      return fail(KDA_ERR_SHAPE, "snapshots overlaps another argument");
  }
  kda::PrefillArgs a{};
  a.N = B;
  a.T_fixed = T;
  a.cu_seqlens = nullptr;
  a.T_total = int64_t(B) * T;
  a.H = H; a.DK = DK; a.DV = DV;
  a.in_bf16 = in_dtype == KDA_BF16;
  a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta;
  a.state_in = state_in; a.o = o; a.state_out = state_out;
  a.workspace = workspace; a.workspace_bytes = workspace_bytes;
  a.snapshots = sbytes > 0 ? snapshots : nullptr;
  a.snap_every = every;
  return run_prefill(a, kda::prefill_workspace_bytes(B, a.T_total, H, DK, DV, false), stream);
}

static kda_status_t prefill_varlen(int N, int T_total, const int32_t* cu_seqlens, int H,
                                   int DK, int DV, int chunk, kda_dtype_t in_dtype,
                                   const void* q, const void* k, const void* v,
                                   const float* alpha, const float* beta,
                                   const float* state_in, float* o, float* state_out,
                                   void* workspace, size_t workspace_bytes, void* stream,
                                   bool alpha_scalar) {
  if (N < 0 || T_total < 0) return fail(KDA_ERR_SHAPE, "negative size (N=%d T_total=%d)", N, T_total);
  if (N > 0 && cu_seqlens == nullptr) return fail(KDA_ERR_NULL, "cu_seqlens must be non-NULL");
  if (cu_seqlens && (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u))
    return fail(KDA_ERR_ALIGN, "cu_seqlens is not 4-byte aligned");
  kda_status_t s = check_prefill(N, T_total, H, DK, DV, chunk, in_dtype, q, k, v, alpha, beta,
                                 state_in, o, state_out, alpha_scalar);
  if (s != KDA_OK) return s;
  kda::PrefillArgs a{};
  a.N = N;
  a.T_fixed = 0;
  a.cu_seqlens = cu_seqlens;
  a.T_total = T_total;
  a.H = H; a.DK = DK; a.DV = DV;
  a.in_bf16 = in_dtype == KDA_BF16;
  a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta;
  a.state_in = state_in; a.o = o; a.state_out = state_out;
  a.workspace = workspace; a.workspace_bytes = workspace_bytes;
  a.alpha_scalar = alpha_scalar;
  return run_prefill(a, kda::prefill_workspace_bytes(N, T_total, H, DK, DV, true), stream);
}

kda_status_t kda_chunk_prefill_varlen(int N, int T_total, const int32_t* cu_seqlens, int H,
                                      int DK, int DV, int chunk, kda_dtype_t in_dtype,
                                      const void* q, const void* k, const void* v,
                                      const float* alpha, const float* beta,
                                      const float* state_in, float* o, float* state_out,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  TraceRange trace_range("kda_chunk_prefill_varlen");
  return prefill_varlen(N, T_total, cu_seqlens, H, DK, DV, chunk, in_dtype, q, k, v, alpha, beta,
                        state_in, o, state_out, workspace, workspace_bytes, stream, false);
}

kda_status_t kda_chunk_prefill_varlen_snapshots(int N, int T_total, const int32_t* cu_seqlens,
                                                int H, int DK, int DV, int chunk,
                                                kda_dtype_t in_dtype, const void* q, const void* k,
                                                const void* v, const float* alpha,
                                                const float* beta, const float* state_in,
                                                float* o, float* state_out, int every,
                                                const int32_t* snap_offsets, int num_snapshots,
                                                float* snapshots, void* workspace,
                                                size_t workspace_bytes, void* stream) {
  TraceRange trace_range("kda_chunk_prefill_varlen_snapshots");
  if (N < 0 || T_total < 0) return fail(KDA_ERR_SHAPE, "negative size (N=%d T_total=%d)", N, T_total);
  if (every < 1) return fail(KDA_ERR_SHAPE, "every=%d: must be >= 1", every);
  if (num_snapshots < 0) return fail(KDA_ERR_SHAPE, "num_snapshots=%d is negative", num_snapshots);
  if (N > 0 && cu_seqlens == nullptr) return fail(KDA_ERR_NULL, "cu_seqlens must be non-NULL");
  if (N > 0 && snap_offsets == nullptr) return fail(KDA_ERR_NULL, "snap_offsets must be non-NULL");
  if ((reinterpret_cast<uintptr_t>(cu_seqlens) | reinterpret_cast<uintptr_t>(snap_offsets)) & 3u)
    return fail(KDA_ERR_ALIGN, "cu_seqlens and snap_offsets must be 4-byte aligned");
  kda_status_t s = check_prefill(N, T_total, H, DK, DV, chunk, in_dtype, q, k, v, alpha, beta,
                                 state_in, o, state_out, false);
  if (s != KDA_OK) return s;
  const size_t sbytes = size_t(num_snapshots) * H * DK * DV * 4;
  if (sbytes > 0) {
    if (!snapshots) return fail(KDA_ERR_NULL, "snapshots must be non-NULL (%d rows)", num_snapshots);
    if (!aligned16(snapshots)) return fail(KDA_ERR_ALIGN, "snapshots is not 16-byte aligned");
    const size_t esz = in_dtype == KDA_BF16 ? 2 : 4;
    const size_t nk = size_t(T_total) * H * DK, nv = size_t(T_total) * H * DV, nb = size_t(T_total) * H;
    const size_t ns = size_t(N) * H * DK * DV;
    const void* others[] = {q, k, v, alpha, beta, state_in, o, state_out, cu_seqlens, snap_offsets};
    const size_t ob[] = {nk * esz, nk * esz, nv * esz, nk * 4, nb * 4, ns * 4, nv * 4, ns * 4,
                         size_t(N + 1) * 4, size_t(N + 1) * 4};
    for (int i = 0; i < 10; ++i)
      if (overlaps(snapshots, sbytes, others[i], ob[i]))
        return fail(KDA_ERR_SHAPE, "snapshots overlaps another argument");
  }
  kda::PrefillArgs a{};
  a.N = N;
  a.T_fixed = 0;
  a.cu_seqlens = cu_seqlens;
  a.T_total = T_total;
  a.H = H; a.DK = DK; a.DV = DV;
  a.in_bf16 = in_dtype == KDA_BF16;
  a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta;
  a.state_in = state_in; a.o = o; a.state_out = state_out;
  a.workspace = workspace; a.workspace_bytes = workspace_bytes;
  a.snapshots = sbytes > 0 ? snapshots : nullptr;
  a.snap_every = every;
  a.snap_offsets = snap_offsets;
  a.snap_rows = num_snapshots;
  return run_prefill(a, kda::prefill_workspace_bytes(N, T_total, H, DK, DV, true), stream);
}

kda_status_t kda_chunk_prefill_varlen_scalar_gate(int N, int T_total, const int32_t* cu_seqlens,
                                                  int H, int DK, int DV, int chunk,
                                                  kda_dtype_t in_dtype, const void* q,
                                                  const void* k, const void* v, const float* gate,
                                                  const float* beta, const float* state_in,
                                                  float* o, float* state_out, void* workspace,
                                                  size_t workspace_bytes, void* stream) {
  TraceRange trace_range("kda_chunk_prefill_varlen_scalar_gate");
  return prefill_varlen(N, T_total, cu_seqlens, H, DK, DV, chunk, in_dtype, q, k, v, gate, beta,
                        state_in, o, state_out, workspace, workspace_bytes, stream, true);
}

static kda_status_t decode_step(int N, int H, int DK, int DV, kda_dtype_t in_dtype, const void* q,
                                const void* k, const void* v, const float* alpha,
                                const float* beta, float* state, float* o, void* stream,
                                bool alpha_scalar) {
  if (N < 0 || H < 0) return fail(KDA_ERR_SHAPE, "negative size (N=%d H=%d)", N, H);
  if (!dims_ok(DK) || !dims_ok(DV))
    return fail(KDA_ERR_UNSUPPORTED, "DK=%d DV=%d: only 64 and 128 are supported", DK, DV);
  if (in_dtype != KDA_F32 && in_dtype != KDA_BF16)
    return fail(KDA_ERR_DTYPE, "unknown in_dtype %d", (int)in_dtype);
  if (int64_t(N) * H > (int64_t(1) << 30))
    return fail(KDA_ERR_UNSUPPORTED, "too large: N*H=%lld", (long long)N * H);
  if (N == 0 || H == 0) return ok();
  if (!q || !k || !v || !alpha || !beta || !state || !o)
    return fail(KDA_ERR_NULL, "q, k, v, alpha, beta, state and o must be non-NULL");
  const void* ptrs[] = {q, k, v, alpha, beta, state, o};
  const char* names[] = {"q", "k", "v", "alpha", "beta", "state", "o"};
  for (int i = 0; i < 7; ++i)
    if (!aligned16(ptrs[i])) return fail(KDA_ERR_ALIGN, "%s is not 16-byte aligned", names[i]);
  const size_t esz = in_dtype == KDA_BF16 ? 2 : 4;
  const size_t nh = size_t(N) * H;
  const size_t obytes = nh * DV * 4, sbytes = nh * DK * DV * 4;
  const size_t abytes = (alpha_scalar ? nh : nh * DK) * 4;
  if (overlaps(o, obytes, q, nh * DK * esz) || overlaps(o, obytes, k, nh * DK * esz) ||
      overlaps(o, obytes, v, nh * DV * esz) || overlaps(o, obytes, alpha, abytes) ||
      overlaps(o, obytes, beta, nh * 4) || overlaps(o, obytes, state, sbytes))
    return fail(KDA_ERR_SHAPE, "o overlaps an input or the state");
  if (overlaps(state, sbytes, q, nh * DK * esz) || overlaps(state, sbytes, k, nh * DK * esz) ||
      overlaps(state, sbytes, v, nh * DV * esz) || overlaps(state, sbytes, alpha, abytes) ||
      overlaps(state, sbytes, beta, nh * 4))
    return fail(KDA_ERR_SHAPE, "state overlaps an input");
  kda::DecodeArgs a{};
  a.N = N; a.H = H; a.DK = DK; a.DV = DV;
  a.in_bf16 = in_dtype == KDA_BF16;
  a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta; a.state = state; a.o = o;
  a.alpha_scalar = alpha_scalar;
  const char* msg = nullptr;
  if (kda::launch_decode(a, stream, &msg) != 0)
    return fail(KDA_ERR_HIP, "decode launch failed: %s", msg ? msg : "?");
  return ok();
}

kda_status_t kda_decode_step(int N, int H, int DK, int DV, kda_dtype_t in_dtype, const void* q,
                             const void* k, const void* v, const float* alpha,
                             const float* beta, float* state, float* o, void* stream) {
  TraceRange trace_range("kda_decode_step");
  return decode_step(N, H, DK, DV, in_dtype, q, k, v, alpha, beta, state, o, stream, false);
}

kda_status_t kda_decode_step_scalar_gate(int N, int H, int DK, int DV, kda_dtype_t in_dtype,
                                         const void* q, const void* k, const void* v,
                                         const float* gate, const float* beta, float* state,
                                         float* o, void* stream) {
  TraceRange trace_range("kda_decode_step_scalar_gate");
  return decode_step(N, H, DK, DV, in_dtype, q, k, v, gate, beta, state, o, stream, true);
}

kda_status_t kda_decode_pool(int N, int L, int H, int DK, int DV, kda_dtype_t in_dtype,
                             const void* q, const void* k, const void* v, const float* alpha,
                             const float* beta, const int32_t* state_idx,
                             const int32_t* num_tokens, float* state_pool, int pool_size,
                             float* o, float* token_states, void* stream) {
  TraceRange trace_range("kda_decode_pool");
  if (N < 0 || H < 0 || pool_size < 0)
    return fail(KDA_ERR_SHAPE, "negative size (N=%d H=%d pool_size=%d)", N, H, pool_size);
  if (L < 1 || L > 64) return fail(KDA_ERR_UNSUPPORTED, "L=%d: 1 <= L <= 64 tokens per sequence", L);
  if (!dims_ok(DK) || !dims_ok(DV))
    return fail(KDA_ERR_UNSUPPORTED, "DK=%d DV=%d: only 64 and 128 are supported", DK, DV);
  if (in_dtype != KDA_F32 && in_dtype != KDA_BF16)
    return fail(KDA_ERR_DTYPE, "unknown in_dtype %d", (int)in_dtype);
  if (int64_t(N) * H > (int64_t(1) << 30) || int64_t(pool_size) * H > (int64_t(1) << 30))
    return fail(KDA_ERR_UNSUPPORTED, "too large: N*H=%lld pool_size*H=%lld", (long long)N * H,
                (long long)pool_size * H);
  if (!state_idx && pool_size < N)
    return fail(KDA_ERR_SHAPE, "state_idx is NULL, so pool_size (%d) must be >= N (%d)",
                pool_size, N);
  if (N == 0 || H == 0) return ok();
  if (!q || !k || !v || !alpha || !beta || !o || (!state_pool && pool_size > 0))
    return fail(KDA_ERR_NULL, "q, k, v, alpha, beta, o and state_pool must be non-NULL");
  const void* ptrs[] = {q, k, v, alpha, beta, state_pool, o, token_states};
  const char* names[] = {"q", "k", "v", "alpha", "beta", "state_pool", "o", "token_states"};
  for (int i = 0; i < 8; ++i)
    if (ptrs[i] && !aligned16(ptrs[i])) return fail(KDA_ERR_ALIGN, "%s is not 16-byte aligned", names[i]);
  if ((reinterpret_cast<uintptr_t>(state_idx) | reinterpret_cast<uintptr_t>(num_tokens)) & 3u)
    return fail(KDA_ERR_ALIGN, "state_idx and num_tokens must be 4-byte aligned");
  const size_t esz = in_dtype == KDA_BF16 ? 2 : 4;
  const size_t rows = size_t(N) * L * H;
  const size_t bk = rows * DK * esz, bv = rows * DV * esz, ba = rows * DK * 4, bb = rows * 4;
  const size_t bo = rows * DV * 4, bp = size_t(pool_size) * H * DK * DV * 4;
  const size_t bt = token_states ? rows * DK * DV * 4 : 0, bi = size_t(N) * 4;
  const void* in[] = {q, k, v, alpha, beta, state_idx, num_tokens};
  const size_t in_b[] = {bk, bk, bv, ba, bb, bi, bi};
  const void* out[] = {state_pool, o, token_states};
  const size_t out_b[] = {bp, bo, bt};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 7; ++j)
      if (overlaps(out[i], out_b[i], in[j], in_b[j]))
        return fail(KDA_ERR_SHAPE, "an output (state_pool, o, token_states) overlaps an input");
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(out[i], out_b[i], out[j], out_b[j]))
        return fail(KDA_ERR_SHAPE, "state_pool, o and token_states must not overlap");
  }
  kda::PoolDecodeArgs a{};
  a.N = N; a.L = L; a.H = H; a.DK = DK; a.DV = DV;
  a.in_bf16 = in_dtype == KDA_BF16;
  a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta;
  a.state_idx = state_idx; a.num_tokens = num_tokens;
  a.pool = state_pool; a.pool_size = pool_size; a.o = o; a.token_states = token_states;
  const char* msg = nullptr;
  if (kda::launch_decode_pool(a, stream, &msg) != 0)
    return fail(KDA_ERR_HIP, "decode launch failed: %s", msg ? msg : "?");
  return ok();
}

namespace {

// Byte offsets of the backward workspace: [forward prefill workspace, later the
// window buffers | snapshots | adjoint carried between windows].
struct BwdLayout {
  size_t fwd_or_win, snaps, carry, total;
  int64_t win_k, nwin;   // chunks per window of the reverse pass, windows
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Workspace of a backward call: the forward's workspace (fixed length only) or
// the buffers of one window of chunks, whichever is larger (they are not live
// at the same time), one state per full chunk, and the adjoint carried between
// windows.  (The forward runs in its states-only form, which writes no o.)
// The reverse pass goes through the chunks in windows of win_k chunks counted
// from each sequence's end, so that the window buffers (backward_chunk_floats
// per chunk-head) take at most 4 GiB whatever the length (the tuning override
// bwd_window forces a window size).  Packed sequences: T_fixed = 0,
// max_chunks from the longest sequence, and the snapshot rows are T_total / 64
// (chunk j of the sequence starting at token s is row s / 64 + j).
BwdLayout bwd_layout(int N, int T_fixed, int64_t T_total, int64_t max_chunks, int H, int DK,
                     int DV, bool varlen) {
  BwdLayout L{};
  const size_t per_chunk = size_t(N) * H * kda::backward_chunk_floats(DK, DV) * 4;
  int64_t k = int64_t((size_t(4) << 30) / per_chunk);
  if (const int v = kda::tuning().bwd_window; v > 0) k = v;
  if (k < 1) k = 1;
  if (max_chunks < 1) max_chunks = 1;
  if (k > max_chunks) k = max_chunks;
  L.win_k = k;
  L.nwin = (max_chunks + k - 1) / k;
  const size_t pw = varlen ? 0 : kda::prefill_workspace_bytes(N, T_total, H, DK, DV, false);
  const size_t win = size_t(k) * per_chunk;
  const size_t snap_rows = varlen ? size_t(T_total / 64) : size_t(N) * size_t(T_fixed / 64);
  L.fwd_or_win = 0;
  L.snaps = align256(pw > win ? pw : win);
  L.carry = L.snaps + align256(snap_rows * H * DK * DV * 4);
  L.total = L.carry + (L.nwin > 1 ? align256(size_t(N) * H * DK * DV * 4) : 0);
  return L;
}

int64_t chunks_of(int64_t len) { return (len + 63) / 64; }

kda_status_t run_backward(int N, int T_fixed, const int32_t* cu_seqlens, int64_t T_total,
                          int64_t max_chunks, int H,
                          int DK, int DV, int chunk, kda_dtype_t in_dtype, const void* q,
                          const void* k, const void* v, const float* alpha, const float* beta,
                          const float* state_in, const float* d_o, const float* d_state_out,
                          float* dq, float* dk, float* dv, float* dalpha, float* dbeta,
                          float* d_state_in, void* workspace, size_t workspace_bytes,
                          void* stream, bool alpha_scalar) {
  const bool varlen = cu_seqlens != nullptr;
  const size_t nalpha = alpha_scalar ? 1 : size_t(DK);   // alpha (and dalpha) values per token row
  if (!dims_ok(DK) || !dims_ok(DV))
    return fail(KDA_ERR_UNSUPPORTED, "DK=%d DV=%d: only 64 and 128 are supported", DK, DV);
  if (chunk != 64) return fail(KDA_ERR_UNSUPPORTED, "chunk=%d: only 64 is supported", chunk);
  if (in_dtype != KDA_F32 && in_dtype != KDA_BF16)
    return fail(KDA_ERR_DTYPE, "unknown in_dtype %d", (int)in_dtype);
  // (the same limits as the prefill: the forward runs first; the reverse
  // pass indexes with 64-bit offsets and its reductions cover one window)
  if (T_total > (int64_t(1) << 31) - 1 || int64_t(N) * H > (int64_t(1) << 24) || H > 65536)
    return fail(KDA_ERR_UNSUPPORTED, "too large: tokens=%lld sequences*H=%lld H=%d",
                (long long)T_total, (long long)N * H, H);
  if (N == 0 || H == 0) return ok();
  const size_t ns = size_t(N) * H * DK * DV * 4;
  if (T_total == 0) {
    // no tokens: the initial state's gradient is the final state's
    if (!d_state_in) return ok();
    if (!aligned16(d_state_in) || (d_state_out && !aligned16(d_state_out)))
      return fail(KDA_ERR_ALIGN, "d_state_in and d_state_out must be 16-byte aligned");
    if (d_state_out && d_state_out != d_state_in && overlaps(d_state_in, ns, d_state_out, ns))
      return fail(KDA_ERR_SHAPE, "d_state_in overlaps d_state_out");
    const char* msg = nullptr;
    kda::BwdChunkArgs c{};
    c.N = N; c.H = H; c.DK = DK; c.DV = DV; c.T = 0; c.cu_seqlens = cu_seqlens;
    c.in_bf16 = in_dtype == KDA_BF16;
    c.alpha_scalar = alpha_scalar;
    c.win_lo = 0; c.win_k = 1;
    c.d_state_out = d_state_out; c.d_state_in = d_state_in;
    if (kda::launch_backward_chunk(c, 1, stream, &msg) != 0)
      return fail(KDA_ERR_HIP, "backward launch failed: %s", msg ? msg : "?");
    return ok();
  }
  const void* need[] = {q, k, v, alpha, beta, d_o, dq, dk, dv, dalpha, dbeta};
  for (const void* x : need)
    if (!x)
      return fail(KDA_ERR_NULL,
                  "q, k, v, alpha, beta, d_o, dq, dk, dv, dalpha and dbeta must be non-NULL");
  const size_t esz = in_dtype == KDA_BF16 ? 2 : 4;
  const size_t rows = size_t(T_total) * H;
  const void* in[] = {q, k, v, alpha, beta, state_in, d_o, d_state_out, cu_seqlens};
  const size_t in_b[] = {rows * DK * esz, rows * DK * esz, rows * DV * esz, rows * nalpha * 4,
                         rows * 4, ns, rows * DV * 4, ns, size_t(N + 1) * 4};
  const char* in_n[] = {"q", "k", "v", "alpha", "beta", "state_in", "d_o", "d_state_out",
                        "cu_seqlens"};
  const void* out[] = {dq, dk, dv, dalpha, dbeta, d_state_in};
  const size_t out_b[] = {rows * DK * 4, rows * DK * 4, rows * DV * 4, rows * nalpha * 4, rows * 4, ns};
  const char* out_n[] = {"dq", "dk", "dv", "dalpha", "dbeta", "d_state_in"};
  for (int i = 0; i < 8; ++i)
    if (in[i] && !aligned16(in[i])) return fail(KDA_ERR_ALIGN, "%s is not 16-byte aligned", in_n[i]);
  for (int i = 0; i < 6; ++i)
    if (out[i] && !aligned16(out[i]))
      return fail(KDA_ERR_ALIGN, "%s is not 16-byte aligned", out_n[i]);
  for (int i = 0; i < 6; ++i) {
    for (int j = 0; j < 9; ++j)
      if (overlaps(out[i], out_b[i], in[j], in_b[j]))
        return fail(KDA_ERR_SHAPE, "%s overlaps %s", out_n[i], in_n[j]);
    for (int j = i + 1; j < 6; ++j)
      if (overlaps(out[i], out_b[i], out[j], out_b[j]))
        return fail(KDA_ERR_SHAPE, "%s overlaps %s", out_n[i], out_n[j]);
  }
  const BwdLayout L = bwd_layout(N, T_fixed, T_total, max_chunks, H, DK, DV, varlen);
  if (!workspace || workspace_bytes < L.total)
    return fail(KDA_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given", L.total,
                workspace ? workspace_bytes : size_t(0));
  if (!aligned16(workspace)) return fail(KDA_ERR_ALIGN, "workspace is not 16-byte aligned");
  for (int j = 0; j < 9; ++j)
    if (overlaps(workspace, L.total, in[j], in_b[j]))
      return fail(KDA_ERR_SHAPE, "workspace overlaps %s", in_n[j]);
  for (int j = 0; j < 6; ++j)
    if (overlaps(workspace, L.total, out[j], out_b[j]))
      return fail(KDA_ERR_SHAPE, "workspace overlaps %s", out_n[j]);

  char* ws = static_cast<char*>(workspace);
  // 1. forward with a snapshot after every chunk
  kda::PrefillArgs f{};
  f.N = N; f.T_fixed = varlen ? 0 : T_fixed; f.cu_seqlens = cu_seqlens; f.T_total = T_total;
  f.H = H; f.DK = DK; f.DV = DV; f.in_bf16 = in_dtype == KDA_BF16;
  f.q = q; f.k = k; f.v = v; f.alpha = alpha; f.beta = beta; f.alpha_scalar = alpha_scalar;
  // (states only: o is never written, but must be a valid address)
  f.state_in = state_in; f.o = reinterpret_cast<float*>(ws); f.state_out = nullptr;
  f.workspace = ws + L.fwd_or_win; f.workspace_bytes = L.snaps;
  const int64_t snap_rows = varlen ? T_total / 64 : int64_t(N) * (T_fixed / 64);
  f.snapshots = snap_rows > 0 ? reinterpret_cast<float*>(ws + L.snaps) : nullptr;
  f.snap_every = 1;
  f.snap_offsets = nullptr;
  f.states_only = true;   // the reverse pass reads the checkpoints only
  f.snap_rows = snap_rows;
  const char* msg = nullptr;
  if (kda::launch_prefill(f, stream, &msg) != 0)
    return fail(KDA_ERR_HIP, "backward: forward launch failed: %s", msg ? msg : "?");
  // 2. per window of chunks: per-chunk matrices, the adjoint's pass, gradients
  kda::BwdChunkArgs c{};
  c.N = N; c.H = H; c.DK = DK; c.DV = DV; c.T = varlen ? 0 : T_fixed; c.cu_seqlens = cu_seqlens;
  c.in_bf16 = in_dtype == KDA_BF16;
  c.alpha_scalar = alpha_scalar;
  c.q = q; c.k = k; c.v = v; c.alpha = alpha; c.beta = beta; c.state_in = state_in;
  c.d_o = d_o; c.d_state_out = d_state_out;
  c.snapshots = reinterpret_cast<const float*>(ws + L.snaps);
  c.dq = dq; c.dk = dk; c.dv = dv; c.dalpha = dalpha; c.dbeta = dbeta; c.d_state_in = d_state_in;
  c.carry = L.nwin > 1 ? reinterpret_cast<float*>(ws + L.carry) : nullptr;
  c.win_k = L.win_k;
  const size_t per = size_t(N) * size_t(L.win_k) * H;   // chunk-heads of a window
  c.Ac = reinterpret_cast<float*>(ws + L.fwd_or_win);
  c.bc = c.Ac + per * DK * DK;
  c.dSend = c.bc + per * DK * DV;
  c.Mb = c.dSend + per * DK * DV;
  c.PX = c.Mb + per * 64 * 64;
  c.Vnb = c.PX + per * 64 * 64;
  c.rho = c.Vnb + per * 64 * DV;
  for (int64_t w = 0; w < L.nwin; ++w) {
    c.win_lo = w * L.win_k;
    for (int stage = 0; stage < 3; ++stage)
      if (kda::launch_backward_chunk(c, stage, stream, &msg) != 0)
        return fail(KDA_ERR_HIP, "backward launch failed: %s", msg ? msg : "?");
  }
  return ok();
}

}  // namespace

size_t kda_chunk_backward_workspace_size(int B, int T, int H, int DK, int DV, int chunk) {
  if (B <= 0 || T <= 0 || H <= 0 || !dims_ok(DK) || !dims_ok(DV) || chunk != 64) return 0;
  return bwd_layout(B, T, int64_t(B) * T, chunks_of(T), H, DK, DV, false).total;
}

kda_status_t kda_chunk_backward(int B, int T, int H, int DK, int DV, int chunk,
                                kda_dtype_t in_dtype, const void* q, const void* k,
                                const void* v, const float* alpha, const float* beta,
                                const float* state_in, const float* d_o,
                                const float* d_state_out, float* dq, float* dk, float* dv,
                                float* dalpha, float* dbeta, float* d_state_in, void* workspace,
                                size_t workspace_bytes, void* stream) {
  TraceRange trace_range("kda_chunk_backward");
  if (B < 0 || T < 0 || H < 0) return fail(KDA_ERR_SHAPE, "negative size (B=%d T=%d H=%d)", B, T, H);
  return run_backward(B, T, nullptr, int64_t(B) * T, chunks_of(T), H, DK, DV, chunk, in_dtype, q, k, v, alpha,
                      beta, state_in, d_o, d_state_out, dq, dk, dv, dalpha, dbeta, d_state_in,
                      workspace, workspace_bytes, stream, false);
}

kda_status_t kda_chunk_backward_scalar_gate(int B, int T, int H, int DK, int DV, int chunk,
                                            kda_dtype_t in_dtype, const void* q, const void* k,
                                            const void* v, const float* gate, const float* beta,
                                            const float* state_in, const float* d_o,
                                            const float* d_state_out, float* dq, float* dk,
                                            float* dv, float* dgate, float* dbeta,
                                            float* d_state_in, void* workspace,
                                            size_t workspace_bytes, void* stream) {
  TraceRange trace_range("kda_chunk_backward_scalar_gate");
  if (B < 0 || T < 0 || H < 0) return fail(KDA_ERR_SHAPE, "negative size (B=%d T=%d H=%d)", B, T, H);
  return run_backward(B, T, nullptr, int64_t(B) * T, chunks_of(T), H, DK, DV, chunk, in_dtype, q, k, v, gate,
                      beta, state_in, d_o, d_state_out, dq, dk, dv, dgate, dbeta, d_state_in,
                      workspace, workspace_bytes, stream, true);
}

size_t kda_chunk_backward_varlen_workspace_size(int N, int T_total, int max_seqlen, int H, int DK,
                                                int DV, int chunk) {
  if (N <= 0 || T_total <= 0 || H <= 0 || !dims_ok(DK) || !dims_ok(DV) || chunk != 64) return 0;
  const int64_t ml = max_seqlen > 0 && max_seqlen < T_total ? max_seqlen : T_total;
  return bwd_layout(N, 0, T_total, chunks_of(ml), H, DK, DV, true).total;
}

kda_status_t kda_chunk_backward_varlen(int N, int T_total, const int32_t* cu_seqlens,
                                       int max_seqlen, int H, int DK, int DV, int chunk,
                                       kda_dtype_t in_dtype,
                                       const void* q, const void* k, const void* v,
                                       const float* alpha, const float* beta,
                                       const float* state_in, const float* d_o,
                                       const float* d_state_out, float* dq, float* dk, float* dv,
                                       float* dalpha, float* dbeta, float* d_state_in,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  TraceRange trace_range("kda_chunk_backward_varlen");
  if (N < 0 || T_total < 0 || H < 0)
    return fail(KDA_ERR_SHAPE, "negative size (N=%d T_total=%d H=%d)", N, T_total, H);
  if (N > 0 && cu_seqlens == nullptr) return fail(KDA_ERR_NULL, "cu_seqlens must be non-NULL");
  if (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u)
    return fail(KDA_ERR_ALIGN, "cu_seqlens must be 4-byte aligned");
  const int64_t ml = max_seqlen > 0 && max_seqlen < T_total ? max_seqlen : T_total;
  return run_backward(N, 0, N > 0 ? cu_seqlens : nullptr, T_total, chunks_of(ml), H, DK, DV, chunk,
                      in_dtype, q, k, v, alpha, beta, state_in, d_o, d_state_out, dq, dk, dv, dalpha, dbeta,
                      d_state_in, workspace, workspace_bytes, stream, false);
}

kda_status_t kda_chunk_backward_varlen_scalar_gate(
    int N, int T_total, const int32_t* cu_seqlens, int max_seqlen, int H, int DK, int DV,
    int chunk, kda_dtype_t in_dtype, const void* q, const void* k, const void* v,
    const float* gate, const float* beta, const float* state_in, const float* d_o,
    const float* d_state_out, float* dq, float* dk, float* dv, float* dgate, float* dbeta,
    float* d_state_in, void* workspace, size_t workspace_bytes, void* stream) {
  TraceRange trace_range("kda_chunk_backward_varlen_scalar_gate");
  if (N < 0 || T_total < 0 || H < 0)
    return fail(KDA_ERR_SHAPE, "negative size (N=%d T_total=%d H=%d)", N, T_total, H);
  if (N > 0 && cu_seqlens == nullptr) return fail(KDA_ERR_NULL, "cu_seqlens must be non-NULL");
  if (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u)
    return fail(KDA_ERR_ALIGN, "cu_seqlens must be 4-byte aligned");
  const int64_t ml = max_seqlen > 0 && max_seqlen < T_total ? max_seqlen : T_total;
  return run_backward(N, 0, N > 0 ? cu_seqlens : nullptr, T_total, chunks_of(ml), H, DK, DV, chunk,
                      in_dtype, q, k, v, gate, beta, state_in, d_o, d_state_out, dq, dk, dv, dgate, dbeta,
                      d_state_in, workspace, workspace_bytes, stream, true);
}

}  // extern "C"

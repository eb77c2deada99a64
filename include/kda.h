/*
 * kda.h — C ABI of the Kimi Delta Attention (KDA) operator for AMD Instinct
 * MI355X (gfx950).
 *
 * The operator (per sequence n and head h, state S of d_k x d_v, fp32):
 *     for every token t, in order:
 *         S   <- Diag(alpha_t) S                       channel-wise forget, first
 *         S   <- S + beta_t k_t (v_t - S^T k_t)^T      delta-rule write
 *         o_t  = S^T q_t                                read after the write
 * as defined by "Kimi Delta Attention 徹底解説" (tech-tide.dev), section
 * "Kimi Delta Attention の仕組み — 「忘れ方」を鍛える": DeltaNet writes the
 * prediction error scaled by a write strength beta; Gated DeltaNet decays the
 * state before writing; KDA makes the decay a diagonal (per-channel) matrix;
 * decode is the token recurrence and prefill the same computation regrouped
 * into chunked matrix products.  The decay is given per token ("Kimi Linear、
 * 独自の土俵でFull Attentionを上回る" (remio.ai), section "Kimi Linearがより
 * 賢いRecurrent Memoryを使う方法").
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a DEVICE pointer owned by the caller, C-contiguous
 *     (row-major), 16-byte aligned.  The library never allocates, frees or
 *     synchronises, and never reads device memory on the host.
 *   - q, k, v are KDA_F32 (float) or KDA_BF16 (bfloat16 bit patterns);
 *     alpha, beta, states and o are always float (fp32).
 *   - State layout: S[n][h][i][j] at ((n*H + h)*DK + i)*DV + j, where i is the
 *     KEY channel (the axis Diag(alpha) scales) and j the VALUE channel.
 *   - Supported sizes: DK, DV in {64, 128}; chunk == 64; prefill and backward
 *     at most 65536 heads.
 *   - Data domain (not checked: violating it gives unspecified output):
 *     alpha in [1e-4, 1] and finite inputs.  The chunked forms split the decay
 *     between two tokens of a chunk through a reference row in each block of
 *     16 tokens, so every factor they build is a product of at most 8 alphas
 *     or its reciprocal (at most 1e32 at alpha = 1e-4, within fp32).
 *   - Errors: argument errors are detected on the host before anything is
 *     enqueued; the call then returns a non-zero status, enqueues nothing and
 *     leaves every output untouched.  KDA_ERR_HIP means a launch failed.
 *     kda_last_error_message() gives a thread-local description.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream).
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KDA_OK = 0,
  KDA_ERR_NULL = 1,        /* a required pointer is NULL                          */
  KDA_ERR_SHAPE = 2,       /* a size is negative or tensors overlap illegally     */
  KDA_ERR_DTYPE = 3,       /* unknown kda_dtype_t                                 */
  KDA_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned                    */
  KDA_ERR_UNSUPPORTED = 5, /* DK/DV not in {64,128}, chunk != 64, or too large    */
  KDA_ERR_WORKSPACE = 6,   /* workspace missing or smaller than required          */
  KDA_ERR_HIP = 7          /* a HIP launch failed                                 */
} kda_status_t;

/* dtype of q, k, v only.  The two range markers are not dtypes: they make
 * every int a value of the type, so a caller may pass any int and an unknown
 * one is rejected with KDA_ERR_DTYPE (rather than being out of the enum's
 * range, which C++ does not define). */
typedef enum {
  KDA_F32 = 0,
  KDA_BF16 = 1,
  KDA_DTYPE_RANGE_MIN_ = -2147483647 - 1,
  KDA_DTYPE_RANGE_MAX_ = 2147483647
} kda_dtype_t;

/* Version of this ABI: (major << 16) | minor. */
int kda_abi_version(void);

/*
 * Chunked prefill, fixed length: B sequences of T tokens, H heads.
 *   q, k       [B,T,H,DK]  (in_dtype)
 *   v          [B,T,H,DV]  (in_dtype)
 *   alpha      [B,T,H,DK]  float, per-token per-channel decay
 *   beta       [B,T,H]     float, per-token write strength (any finite value)
 *   state_in   [B,H,DK,DV] float, or NULL for a zero initial state
 *   o          [B,T,H,DV]  float output; must not overlap any input
 *   state_out  [B,H,DK,DV] float, or NULL; may be equal to state_in (in place)
 *   workspace  device scratch of at least kda_chunk_prefill_workspace_size()
 *              bytes, 16-byte aligned, not overlapping any other argument;
 *              may be NULL when that size is 0.  Its contents on entry are
 *              ignored and on return are unspecified.  The size is nonzero
 *              when B*H < 128 and T > 64: the per-chunk operands of the
 *              state pass are then computed for all chunks at once and staged
 *              here.  Long sequences are processed in equal segments of
 *              chunks whose operands take at most 160 MiB (so that they stay
 *              in the memory-side cache between the two kernels), plus one
 *              B*H*DK*DV float state carried between segments.
 * Computes exactly the token recurrence (up to rounding) by the chunk form:
 * per chunk a unit-lower-triangular solve and dense products, and a
 * sequential pass of the state over the chunks.
 */
size_t kda_chunk_prefill_workspace_size(int B, int T, int H, int DK, int DV, int chunk);
kda_status_t kda_chunk_prefill(int B, int T, int H, int DK, int DV, int chunk,
                               kda_dtype_t in_dtype, const void* q, const void* k,
                               const void* v, const float* alpha, const float* beta,
                               const float* state_in, float* o, float* state_out,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_chunk_prefill for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same arguments without the workspace, and the same result (bit for bit).
 * Where kda_chunk_prefill would stage per-chunk operands in the workspace
 * (B*H < 128, T > 64), this call stages them in a static device array of
 * 64 MiB that the library keeps on every device it runs on until the process
 * ends, in segments short enough for one segment's operands and the carried
 * state to fit (more segments than with a workspace: somewhat slower).
 * Returns KDA_ERR_UNSUPPORTED, enqueuing nothing, when even one chunk does
 * not fit (only possible under the internal tuning override that forces the
 * staged form on 128 or more (sequence, head) pairs); KDA_ERR_HIP if the
 * array's device address cannot be obtained.  It allocates nothing and needs
 * nothing zeroed: every call writes the parts it reads.  All calls on one
 * device share the array: calls that overlap in time on one device (e.g. on
 * two streams) race and give undefined results.
 */
kda_status_t kda_chunk_prefill_noalloc(int B, int T, int H, int DK, int DV, int chunk,
                                       kda_dtype_t in_dtype, const void* q, const void* k,
                                       const void* v, const float* alpha, const float* beta,
                                       const float* state_in, float* o, float* state_out,
                                       void* stream);

/*
 * Chunked prefill with state snapshots at chunk boundaries (prefix caching):
 * the same computation as kda_chunk_prefill, and in addition the state after
 * every `every`-th chunk, i.e. after the first 64*every*(j+1) tokens of each
 * sequence, for j = 0 .. T/(64*every) - 1 (complete intervals only):
 *   snapshots  [B, T/(64*every), H, DK, DV] float (row = key channel), device,
 *              16-byte aligned, not overlapping any other argument; may be NULL
 *              only when T < 64*every (nothing to write).
 *   every      >= 1 chunks of 64 tokens.
 * A prefill started from snapshot j over the tokens that follow it continues
 * the sequence exactly (up to rounding).  Workspace: as for kda_chunk_prefill
 * (kda_chunk_prefill_workspace_size with the same arguments).
 * Serving stacks cache prefixes of KDA sequences as states at block
 * boundaries: "Kimi Linearは広がりつつある：検証できるすべてのモデルが実際に
 * KDAを実行する" (orcarouter.ai), section "既に起こった採用はサービングスタッ
 * クの中にあります" (KDA prefix caching went into the serving engine), and
 * "Kimi Linear、独自の土俵でFull Attentionを上回る" (remio.ai), section
 * "オープンコードにより主張は検証可能になる" (prefix caching and the state
 * across chunk boundaries are what deployments must test).
 */
kda_status_t kda_chunk_prefill_snapshots(int B, int T, int H, int DK, int DV, int chunk,
                                         kda_dtype_t in_dtype, const void* q, const void* k,
                                         const void* v, const float* alpha, const float* beta,
                                         const float* state_in, float* o, float* state_out,
                                         int every, float* snapshots, void* workspace,
                                         size_t workspace_bytes, void* stream);

/*
 * Packed variable-length prefill with snapshots (prefix caching for a
 * continuous-batching prefill): as kda_chunk_prefill_varlen, and sequence n's
 * state after its first 64*every*(j+1) tokens is written to row
 * snap_offsets[n] + j of `snapshots`, for j < floor(len_n / (64*every)) and
 * j < snap_offsets[n+1] - snap_offsets[n] (rows the offsets do not provide
 * are skipped).
 *   snap_offsets   int32 DEVICE [N+1], 4-byte aligned, non-decreasing
 *                  (normally snap_offsets[n+1] - snap_offsets[n] =
 *                  floor(len_n / (64*every)))
 *   num_snapshots  host int = snap_offsets[N], the rows of `snapshots`; rows
 *                  outside [0, num_snapshots) are never written, whatever the
 *                  device offsets hold
 *   snapshots      [num_snapshots, H, DK, DV] float, may be NULL when
 *                  num_snapshots == 0
 * Prefix reuse and the state at chunk boundaries under continuous batching
 * are what serving has to get right ("Kimi Linear、独自の土俵でFull Attention
 * を上回る" (remio.ai), section "Kimi Linearリリース後に注目すべき点").
 */
kda_status_t kda_chunk_prefill_varlen_snapshots(int N, int T_total, const int32_t* cu_seqlens,
                                                int H, int DK, int DV, int chunk,
                                                kda_dtype_t in_dtype, const void* q, const void* k,
                                                const void* v, const float* alpha,
                                                const float* beta, const float* state_in,
                                                float* o, float* state_out, int every,
                                                const int32_t* snap_offsets, int num_snapshots,
                                                float* snapshots, void* workspace,
                                                size_t workspace_bytes, void* stream);

/*
 * Chunked prefill, packed variable length: N sequences concatenated on the
 * token axis; sequence n owns tokens [cu_seqlens[n], cu_seqlens[n+1]).
 *   cu_seqlens  int32 DEVICE array [N+1], cu_seqlens[0] == 0, non-decreasing,
 *               cu_seqlens[N] == T_total (not checked: it is never read on
 *               the host)
 *   q, k, alpha [T_total,H,DK];  v, o [T_total,H,DV];  beta [T_total,H]
 *   state_in / state_out  [N,H,DK,DV] as above (one state per sequence)
 * Chunks restart at every sequence start; a zero-length sequence passes its
 * state through.  The order of the sequences in the pack only affects speed:
 * longest first finishes soonest (the long chains start first).
 */
size_t kda_chunk_prefill_varlen_workspace_size(int N, int T_total, int H, int DK, int DV,
                                               int chunk);
kda_status_t kda_chunk_prefill_varlen(int N, int T_total, const int32_t* cu_seqlens, int H,
                                      int DK, int DV, int chunk, kda_dtype_t in_dtype,
                                      const void* q, const void* k, const void* v,
                                      const float* alpha, const float* beta,
                                      const float* state_in, float* o, float* state_out,
                                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * One recurrent decode step for N sequences x H heads (one token each); the
 * explainer's token-wise mode.
 *   q, k, alpha [N,H,DK];  v [N,H,DV];  beta [N,H]
 *   state       [N,H,DK,DV] float, read and updated IN PLACE
 *   o           [N,H,DV] float output; must not overlap any input or state
 */
kda_status_t kda_decode_step(int N, int H, int DK, int DV, kda_dtype_t in_dtype, const void* q,
                             const void* k, const void* v, const float* alpha,
                             const float* beta, float* state, float* o, void* stream);

/*
 * Scalar-gate (Gated DeltaNet) forms: the same operator with one decay gate
 * per token and head instead of one per key channel, i.e. alpha_t = g_t * 1.
 * Gated DeltaNet decays the whole state by one scalar before the delta write,
 * and KDA generalises that scalar to a diagonal ("Kimi Delta Attention 徹底
 * 解説" (tech-tide.dev), section "Kimi Delta Attention の仕組み — 「忘れ方」を
 * 鍛える").  Arguments as in the per-channel entry points above, except
 *   gate  [B,T,H] (fixed), [T_total,H] (varlen), [N,H] (decode) float, in the
 *         same data domain as alpha.
 * Same kernels, same results as passing alpha with every channel equal to the
 * gate (bit for bit); the gate costs 4 bytes per token-head instead of 4*DK.
 * Workspace sizes: kda_chunk_prefill_workspace_size and
 * kda_chunk_prefill_varlen_workspace_size.
 */
kda_status_t kda_chunk_prefill_scalar_gate(int B, int T, int H, int DK, int DV, int chunk,
                                           kda_dtype_t in_dtype, const void* q, const void* k,
                                           const void* v, const float* gate, const float* beta,
                                           const float* state_in, float* o, float* state_out,
                                           void* workspace, size_t workspace_bytes,
                                           void* stream);
kda_status_t kda_chunk_prefill_varlen_scalar_gate(int N, int T_total, const int32_t* cu_seqlens,
                                                  int H, int DK, int DV, int chunk,
                                                  kda_dtype_t in_dtype, const void* q,
                                                  const void* k, const void* v, const float* gate,
                                                  const float* beta, const float* state_in,
                                                  float* o, float* state_out, void* workspace,
                                                  size_t workspace_bytes, void* stream);
kda_status_t kda_decode_step_scalar_gate(int N, int H, int DK, int DV, kda_dtype_t in_dtype,
                                         const void* q, const void* k, const void* v,
                                         const float* gate, const float* beta, float* state,
                                         float* o, void* stream);

/*
 * Decode of up to L tokens per sequence over a pool of states (continuous
 * batching: the batch's sequences index their states in a shared pool;
 * speculative decoding: L draft tokens are run and the state after each is
 * kept for the verifier).  Deployment tools must support both without
 * breaking KDA's state handling ("Kimi Linear、独自の土俵でFull Attentionを
 * 上回る" (remio.ai), section "Kimi Linearリリース後に注目すべき点"); each
 * token is one step of the token recurrence defined above.
 *   q, k, alpha  [N,L,H,DK];  v [N,L,H,DV];  beta [N,L,H]   (token j of
 *                sequence n is row n*L + j)
 *   state_idx    int32 DEVICE [N], 4-byte aligned, or NULL (sequence n uses
 *                slot n; then pool_size >= N).  A slot outside
 *                [0, pool_size) marks a padding row: its o rows are set to 0
 *                and nothing else is read or written for it.  Valid slots
 *                must be distinct (not checked: two sequences on one slot race).
 *   num_tokens   int32 DEVICE [N], 4-byte aligned, or NULL (L each): sequence
 *                n runs its first min(max(num_tokens[n], 0), L) tokens; the o
 *                rows of the others are set to 0.
 *   state_pool   [pool_size,H,DK,DV] float, read and updated IN PLACE: a slot
 *                ends holding the state after its sequence's last token.
 *   o            [N,L,H,DV] float output.
 *   token_states [N,L,H,DK,DV] float or NULL: the state after each processed
 *                token (entries of unprocessed tokens are not written).
 *   1 <= L <= 64.  No output may overlap an input or another output.
 * With L = 1, state_idx = NULL and num_tokens = NULL this is kda_decode_step.
 */
kda_status_t kda_decode_pool(int N, int L, int H, int DK, int DV, kda_dtype_t in_dtype,
                             const void* q, const void* k, const void* v, const float* alpha,
                             const float* beta, const int32_t* state_idx,
                             const int32_t* num_tokens, float* state_pool, int pool_size,
                             float* o, float* token_states, void* stream);

/*
 * Backward pass (training): gradients of L = sum(o * d_o) + sum(S_T * d_state_out)
 * for a fixed-length prefill with per-channel alpha.  The chunk algorithm is
 * the training form of the recurrence ("Kimi Linear、独自の土俵でFull Attention
 * を上回る" (remio.ai), section "Kimi Linearがより賢いRecurrent Memoryを使う方法");
 * its gradient is that of the token recurrence defined above.
 *   q, k, v, alpha, beta, state_in   as for kda_chunk_prefill (state_in may be NULL)
 *   d_o          [B,T,H,DV] float, gradient of o
 *   d_state_out  [B,H,DK,DV] float or NULL (zero), gradient of the final state
 *   dq, dk, dalpha [B,T,H,DK], dv [B,T,H,DV], dbeta [B,T,H]  float outputs
 *   d_state_in   [B,H,DK,DV] float or NULL: gradient of the initial state
 *   workspace    at least kda_chunk_backward_workspace_size() bytes, 16-byte
 *                aligned, not overlapping any argument (holds the forward's
 *                chunk-boundary states, DK DV / 64 floats per token-head; per chunk-head of a window of chunks
 *                DK^2 + 2 DK DV + 64 DV + 93 DK + 8192 floats (310 KB at
 *                d = 128), the windows sized to keep this at most 4 GiB; one
 *                state per (sequence, head) when there are several windows).
 * Outputs must not overlap inputs or each other.  The forward is recomputed
 * (with a state checkpoint per chunk).  The reverse pass is in chunk form: the
 * adjoint of the state at every chunk boundary comes from one sequential pass
 * over the chunks (an affine map per chunk), then every chunk's gradients are
 * computed independently from its checkpoint.  The result is deterministic.
 * With T == 0 only d_state_in is written (= d_state_out, or zeros) and no
 * workspace is needed.
 */
size_t kda_chunk_backward_workspace_size(int B, int T, int H, int DK, int DV, int chunk);
kda_status_t kda_chunk_backward(int B, int T, int H, int DK, int DV, int chunk,
                                kda_dtype_t in_dtype, const void* q, const void* k,
                                const void* v, const float* alpha, const float* beta,
                                const float* state_in, const float* d_o,
                                const float* d_state_out, float* dq, float* dk, float* dv,
                                float* dalpha, float* dbeta, float* d_state_in, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * Backward pass of the packed variable-length prefill (training on packed
 * sequences): as kda_chunk_backward, for the N sequences of
 * kda_chunk_prefill_varlen (same cu_seqlens, token tensors [T_total,H,*],
 * states [N,H,DK,DV]).
 *   cu_seqlens   int32 DEVICE [N+1], 4-byte aligned, non-decreasing, from 0 to
 *                T_total (not checked on the device)
 *   max_seqlen   host int: at least the longest sequence's length, or 0 if
 *                unknown (then T_total is assumed; correct, but the reverse
 *                pass may run more, empty, windows).  Not checked: with a
 *                smaller value the reverse pass covers only the last chunks
 *                of a longer sequence (at least ceil(max_seqlen / 64); their
 *                gradients are right); the gradients of its earlier tokens and
 *                its d_state_in are not written.
 *   workspace    at least kda_chunk_backward_varlen_workspace_size() bytes for
 *                the same N, T_total, max_seqlen (the host never reads the
 *                lengths)
 * A sequence of length 0 passes d_state_out through to d_state_in.
 */
size_t kda_chunk_backward_varlen_workspace_size(int N, int T_total, int max_seqlen, int H, int DK,
                                                int DV, int chunk);
kda_status_t kda_chunk_backward_varlen(int N, int T_total, const int32_t* cu_seqlens,
                                       int max_seqlen, int H, int DK, int DV, int chunk,
                                       kda_dtype_t in_dtype,
                                       const void* q, const void* k, const void* v,
                                       const float* alpha, const float* beta,
                                       const float* state_in, const float* d_o,
                                       const float* d_state_out, float* dq, float* dk, float* dv,
                                       float* dalpha, float* dbeta, float* d_state_in,
                                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward pass with a scalar gate (Gated DeltaNet, as
 * kda_chunk_prefill_scalar_gate): as kda_chunk_backward and
 * kda_chunk_backward_varlen, with the gate and its gradient one float per
 * token and head:
 *   gate, dgate  [B,T,H] (packed: [T_total,H]) float
 * The gate decays every key channel, so dgate is the sum over the channels
 * of the per-channel gradient ("Kimi Delta Attention 徹底解説"
 * (tech-tide.dev), section "Kimi Delta Attention の仕組み": KDA turns Gated
 * DeltaNet's scalar into a diagonal).  Workspace sizes: the queries of the
 * per-channel calls.
 */
kda_status_t kda_chunk_backward_scalar_gate(int B, int T, int H, int DK, int DV, int chunk,
                                            kda_dtype_t in_dtype, const void* q, const void* k,
                                            const void* v, const float* gate, const float* beta,
                                            const float* state_in, const float* d_o,
                                            const float* d_state_out, float* dq, float* dk,
                                            float* dv, float* dgate, float* dbeta,
                                            float* d_state_in, void* workspace,
                                            size_t workspace_bytes, void* stream);
kda_status_t kda_chunk_backward_varlen_scalar_gate(
    int N, int T_total, const int32_t* cu_seqlens, int max_seqlen, int H, int DK, int DV,
    int chunk, kda_dtype_t in_dtype, const void* q, const void* k, const void* v,
    const float* gate, const float* beta, const float* state_in, const float* d_o,
    const float* d_state_out, float* dq, float* dk, float* dv, float* dgate, float* dbeta,
    float* d_state_in, void* workspace, size_t workspace_bytes, void* stream);

const char* kda_status_string(kda_status_t s);
const char* kda_last_error_message(void);

/*
 * Internal: tuning overrides for tests and measurements.  Callers never need
 * them (every entry point chooses its launch shapes from the sizes); they
 * exist so that both prefill forms, every slab width, segment length and
 * backward window can be exercised on small inputs.  Process-wide, taking
 * effect at the next call; a workspace size queried before a change does not
 * hold for calls after it.  0 restores the choice by shape:
 *   prefill_form  0, 1 = one-kernel form, 2 = staged form (fixed-length
 *                 batches of more than one chunk; packed batches always take
 *                 the one-kernel form)
 *   prefill_nsub  0, or 1, 2, 4, 8 blocks of 16 value columns per workgroup
 *   prefill_seg   0, or chunks per segment of the staged form
 *   bwd_window    0, or chunks per window of the backward's reverse pass
 * Returns KDA_ERR_SHAPE, changing nothing, for values outside these.
 */
kda_status_t kda_internal_set_tuning(int prefill_form, int prefill_nsub, int prefill_seg,
                                     int bwd_window);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */

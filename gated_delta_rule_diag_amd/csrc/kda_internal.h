// Internal contract between the host-side argument checks (kda_api.cpp, plain
// C++ with no HIP dependency) and the kernel launchers (*.hip).
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace kda {

// One prefill launch.  Fixed-length batches are described by cu_seqlens ==
// nullptr and T_fixed > 0 (sequence n owns tokens [n*T_fixed, (n+1)*T_fixed)).
struct PrefillArgs {
  int N;                       // number of sequences
  int64_t T_fixed;             // tokens per sequence when cu_seqlens == nullptr
  const int32_t* cu_seqlens;   // device [N+1] or nullptr
  int64_t T_total;             // tokens on the packed axis
  int H, DK, DV;
  bool in_bf16;
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;
  const float* state_in;       // may be nullptr (zero state)
  float* o;
  float* state_out;            // may be nullptr
  void* workspace;
  size_t workspace_bytes;
  float* snapshots;            // fixed: [N, T_fixed / (64 * snap_every), H, DK, DV]; varlen:
                               // [snap_rows, H, DK, DV]; or nullptr
  int snap_every;              // chunks between snapshots (with snapshots != nullptr)
  const int32_t* snap_offsets; // varlen: device [N+1], sequence n owns rows [off[n], off[n+1])
  int64_t snap_rows;           // varlen: rows of snapshots
  bool alpha_scalar;           // alpha is [tokens, H]: one gate per token and head
  bool states_only;            // with snapshots: o is not written (the caller needs the
                               // snapshots only; o must still point at valid memory)
  int64_t seg_budget;          // staged form: bytes of slots per segment at most (0: default)
};

struct DecodeArgs {
  int N, H, DK, DV;
  bool in_bf16;
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;
  float* state;
  float* o;
  bool alpha_scalar;           // alpha is [N, H]
};

// Decode of up to L tokens per sequence over a pool of states.
struct PoolDecodeArgs {
  int N, L, H, DK, DV;
  bool in_bf16;
  const void* q;               // [N, L, H, DK]
  const void* k;
  const void* v;               // [N, L, H, DV]
  const float* alpha;          // [N, L, H, DK]
  const float* beta;           // [N, L, H]
  const int32_t* state_idx;    // device [N] or nullptr (slot n)
  const int32_t* num_tokens;   // device [N] or nullptr (L each)
  float* pool;                 // [pool_size, H, DK, DV]
  int pool_size;
  float* o;                    // [N, L, H, DV]
  float* token_states;         // [N, L, H, DK, DV] or nullptr
  bool alpha_scalar;           // alpha is [N, L, H]
};

// Backward pass in chunk form: three launches per window of chunks (stage 0 =
// per-chunk matrices, 1 = the adjoint's pass over the chunks, 2 = per-chunk
// gradients).  Window buffers hold, per chunk-head of the window (index
// (n * H + h) * win_k + j, j = reverse index within the window):
//   Ac [DK][DK], bc [DK][DV], dSend [DK][DV] (these three in the pass's
//   fragment order), Mb [64][64], PX [64][64] (P on and below the diagonal,
//   X^T above it), Vnb [64][DV], rho [93][DK] (the chunk's decays: rows 0..63
//   relative to each 16-row block's reference row, then per-channel vectors).
struct BwdChunkArgs {
  int N, H, DK, DV;
  int64_t T;                   // tokens per sequence (fixed length)
  const int32_t* cu_seqlens;   // packed sequences: device [N + 1], or nullptr
  bool in_bf16;
  bool alpha_scalar;
  int64_t win_lo, win_k;
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;
  const float* state_in;
  const float* d_o;
  const float* d_state_out;
  const float* snapshots;      // state after every full chunk: [N, T / 64, H, DK, DV];
                               // packed: chunk j of the sequence starting at token s is
                               // row s / 64 + j
  float* dq;
  float* dk;
  float* dv;
  float* dalpha;
  float* dbeta;
  float* d_state_in;
  float* carry;                // [N, H, DK, DV] between windows, or nullptr
  float* Ac;
  float* bc;
  float* dSend;
  float* Mb;
  float* PX;
  float* Vnb;
  float* rho;
};

// Tuning overrides (kda_internal_set_tuning); 0 everywhere = choose by shape.
struct Tuning {
  int prefill_form;   // 0 by shape, 1 one-kernel (fused), 2 staged
  int prefill_nsub;   // 0 by shape, else value blocks of 16 per workgroup
  int prefill_seg;    // 0 by size, else chunks per staged segment
  int bwd_window;     // 0 by size, else chunks per backward window
};
Tuning tuning();

// Launchers return 0 on success, else a non-zero code and a static message.
int launch_prefill(const PrefillArgs& a, void* stream, const char** msg);
int launch_decode(const DecodeArgs& a, void* stream, const char** msg);
int launch_decode_pool(const PoolDecodeArgs& a, void* stream, const char** msg);
int launch_backward_chunk(const BwdChunkArgs& a, int stage, void* stream, const char** msg);
size_t backward_chunk_floats(int DK, int DV);   // window-buffer floats per chunk-head
size_t prefill_workspace_bytes(int N, int64_t T_total, int H, int DK, int DV, bool varlen,
                               int64_t seg_budget = 0);
// Static per-device scratch of kda_chunk_prefill_noalloc: its size, and its
// device address on the current device (nullptr and a message on failure).
constexpr size_t kNoallocScratchBytes = size_t(64) << 20;
void* noalloc_scratch(const char** msg);

}  // namespace kda

// Internal launch interface between the C ABI (attn_api.hip) and the kernel files.
// Every launcher assumes its arguments were validated by the C ABI and only enqueues work.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

struct FwdProblem {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;      // may be null
  int B, Hq, Hkv, Sq, Sk, D;
  int causal;
  float scale;
  int nsplit;        // bf16: key-range splits per query tile (<= 1: none)
  void* workspace;   // bf16 with nsplit > 1: fwd_bf16_workspace_bytes(p, nsplit) bytes
  int mapping;       // bf16 without splits: FwdMapping, or -1 to choose by the problem
  int cus = 256;     // compute units of the device (for the choice of mapping)
  // bf16 wide kernel without splits: wide_claim_words(items) words that no other launch uses
  // at the same time, and a launch mark (even, larger than any earlier launch's on them); null
  // runs each item on its own workgroup only
  unsigned long long* claim = nullptr;
  unsigned long long epoch = 0;
};

// Words of the wide kernel's claim block for `items` work items: the per-XCD counters and the
// "nothing left" word, each on its own 128-byte line, then a mark per item.
inline size_t wide_claim_words(long long items) { return 9 * 16 + (size_t)items; }

// Work items of the bf16 wide kernel for a problem (0 when the problem does not run on it
// without key-range splits).
long long fwd_wide_items(const FwdProblem& p);

// Work mappings of the bf16 forward without key-range splits.
enum FwdMapping { kMapTile = 0, kMapPair = 1, kMapWide = 2 };

// The mapping the bf16 forward uses for p (without key-range splits) when none is forced.
int fwd_bf16_mapping(const FwdProblem& p, int cus);

// Key-range splits the bf16 forward uses on a device with cus compute units (1 when the
// query tiles alone fill it), and the workspace bytes those splits need.
int fwd_bf16_splits(const FwdProblem& p, int cus);
size_t fwd_bf16_workspace_bytes(const FwdProblem& p, int nsplit);
// bf16 Q/K/V/O, fp32 LSE; MFMA kernel. D in {64, 128}.
hipError_t launch_fwd_bf16(const FwdProblem& p, hipStream_t stream);
// The wide mapping of the bf16 forward (one wave per SIMD, 256 query rows per workgroup);
// D = 128, no key-range splits.
hipError_t launch_fwd_bf16_wide(const FwdProblem& p, hipStream_t stream);
// fp32 Q/K/V/O, fp32 LSE; vector-ALU kernel. D in {64, 128}.
hipError_t launch_fwd_f32(const FwdProblem& p, hipStream_t stream);

// Prefill of packed query tokens against a paged KV cache (several sequences of any lengths).
struct PagedProblem {
  const void* q;               // [T, Hq, D] bf16, sequence b's tokens at rows cu_seqlens_q[b..b+1)
  const void* k_cache;         // [num_blocks, Hkv, 16, D] bf16
  const void* v_cache;
  const int32_t* block_table;  // [B, table_stride]
  const int32_t* cu_seqlens_q; // [B + 1]
  const int32_t* ctx_lens;     // [B] keys of each sequence (its new tokens included)
  void* o;                     // [T, Hq, D] bf16
  float* lse;                  // [T, Hq] fp32 or null
  int B, T, Hq, Hkv, D;
  int max_q, max_ctx;          // bounds on the query tokens and keys of any one sequence
  int table_stride;
  int num_blocks;              // <= 0: block ids unchecked
  int causal;
  float scale;
  int nsplit;                  // key-range splits per query tile (<= 1: none)
  void* workspace;             // nsplit > 1: fwd_paged_workspace_bytes(p, nsplit) bytes
};

int fwd_paged_splits(const PagedProblem& p, int cus);
size_t fwd_paged_workspace_bytes(const PagedProblem& p, int nsplit);
hipError_t launch_fwd_paged(const PagedProblem& p, hipStream_t stream);

struct DecodeProblem {
  const void* q;            // [B, Hq, D] bf16
  const void* k_cache;      // [num_blocks, Hkv, block_size, D] bf16
  const void* v_cache;
  const int32_t* block_table;  // [B, table_stride] int32
  const int32_t* ctx_lens;     // [B] int32
  void* o;                  // [B, Hq, D] bf16
  float* lse;               // [B, Hq] fp32 or null
  int B, Hq, Hkv, D, block_size;
  int table_stride;         // <= 0: derived on the device as max_b ceil(ctx_b / block_size)
  int num_blocks;           // <= 0: unknown (no physical-block range check)
  int workers;              // worker waves that split the batch's K/V blocks between them
  float scale;
  void* workspace;          // decode_workspace_bytes(B, Hkv, Hq / Hkv, D, workers) bytes
};

// Bytes of partial results the decode needs (16-byte aligned start assumed).
size_t decode_workspace_bytes(int B, int Hkv, int group, int D, int workers);
hipError_t launch_decode_paged(const DecodeProblem& p, hipStream_t stream);

struct NormProblem {
  const void* x;            // [M, d] bf16
  const void* residual;     // [M, d] bf16
  const void* weight;       // [d] bf16
  void* out;                // [M, d] bf16 (may be x)
  void* residual_out;       // [M, d] bf16 (may be residual)
  int M, d;                 // d a multiple of 8, 8 <= d <= 65536
  float eps;
};

// Threads per row the residual-add RMS norm launches for a row of d elements.
int add_rms_norm_threads(int d);
hipError_t launch_add_rms_norm(const NormProblem& p, hipStream_t stream);

struct RopeProblem {
  const void* q;            // [T, Hq, D] bf16
  const void* k;            // [T, Hkv, D] bf16
  const void* v;            // [T, Hkv, D] bf16
  void* q_out;              // [T, Hq, D] bf16 (may be q)
  void* k_cache;            // [num_blocks, Hkv, 16, D] bf16
  void* v_cache;
  const int32_t* block_table;  // [num_seqs, table_stride]
  const int32_t* positions;    // [T]
  const int32_t* seq_ids;      // [T] or null (token t is sequence t)
  int T, num_seqs, Hq, Hkv, D;
  int table_stride;
  int num_blocks;           // <= 0: unchecked
  float base;
};

hipError_t launch_rope_cache_write(const RopeProblem& p, hipStream_t stream);

}  // namespace attn

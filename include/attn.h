/* Fused exact attention for AMD Instinct MI355X (gfx950): C ABI of libattn.so.
 *
 * What is computed. For every batch b, query head h and query row i,
 *     O[b,h,i,:] = sum_j softmax_j( scale * q[b,h,i,:] . k[b,hk,j,:] + mask[i,j] ) v[b,hk,j,:]
 *     LSE[b,h,i] = ln sum_j exp( scale * q[b,h,i,:] . k[b,hk,j,:] + mask[i,j] )
 * with hk = h / (Hq / Hkv). This is the attention equation of "Fused Kernel Compiler"
 * (Candle paper), §FlashAttention Integration, with the scale passed explicitly (1/sqrt(d_k)
 * in the usual case) and an optional causal mask (the "scale, mask, softmax" pattern of that
 * page's table "Kernel fusion opportunities"). It is computed in a single pass over K/V with
 * an online softmax, so no score or probability matrix is ever written to memory (same
 * section; also "Optimizing Large Language Model Inference Through Kernel Fusion and Advanced
 * Memory Management", §FlashAttention and the Memory-Efficiency Revolution). Results equal
 * the plain definition up to floating-point rounding order.
 *
 * Conventions shared by every call:
 *   - All tensors are dense, row-major, in device memory owned by the caller; the library
 *     never allocates, frees or retains them.
 *   - q, o: [B, Hq, Sq, D]; k, v: [B, Hkv, Sk, D]; lse: [B, Hq, Sq] float32.
 *   - Grouped-query attention: Hq must be a multiple of Hkv; query head h uses KV head
 *     h / (Hq / Hkv) (contiguous groups).
 *   - causal != 0 masks key j for query i unless j <= i + (Sk - Sq) (aligned to the bottom
 *     right corner; the usual lower triangle when Sq == Sk). A row that sees no key gets
 *     O = 0 and LSE = -inf.
 *   - scale must be finite and >= 0 (scale 0 gives uniform weights over the visible keys).
 *     scale * |score| must stay finite in float32.
 *   - Softmax statistics and accumulation are float32 on every path.
 *   - stream is a hipStream_t (NULL = the null stream). Calls only enqueue work on it and
 *     never synchronise; faults inside a kernel surface at the caller's next synchronisation.
 *   - Every argument is checked on the host before anything is launched; on any error the
 *     call returns a nonzero ATTN_* code, launches nothing and records a message that
 *     attn_last_error() returns on the calling thread.
 *   - B == 0, Sq == 0 (or, for decode, B == 0) is a valid empty problem: nothing is launched.
 *   - The calls are thread-safe.
 *
 * Library workspace. The split-KV decode, and the forward when it splits key ranges, keep
 * partial results in device memory. Without a caller workspace (the _ex entry points) they use
 * one owned by the library per (device, stream), allocated on first use and replaced by a
 * larger one when a call needs more. A call holds it from taking it until all of its kernels
 * are enqueued, so calls from several host threads on one stream never mix their partials.
 * A replaced buffer is not freed until attn_release_workspace (kernels enqueued earlier may
 * still read it). The library workspace is never used on a stream that is being captured into
 * a graph: such a call returns ATTN_ERR_WORKSPACE; pass a caller workspace instead.
 *
 * Claim block. A bf16 forward with D = 128 and more 256-row work items than the device has
 * compute units lets workgroups that finish early take the last items of slower XCDs. The
 * items' claim marks live in a small block the library owns per (device, stream), at least
 * 8 * (144 + items) bytes, allocated and cleared on first use, replaced (like the workspace)
 * when a call needs more, never cleared again (every launch takes larger marks) and freed by
 * attn_release_workspace. On a stream being captured, or on the per-thread default stream, or
 * if the block cannot be allocated, the call runs without it: each item on its own workgroup,
 * with the same results bit for bit.
 */
#ifndef EXACT_ATTENTION_ATTN_H
#define EXACT_ATTENTION_ATTN_H

#include <stddef.h>
#include <stdint.h>

/* The HIP runtime's stream handle, declared exactly as <hip/hip_runtime_api.h> declares it (an
 * identical redeclaration, valid C11 and C++), so that this header needs no HIP include. */
typedef struct ihipStream_t* hipStream_t;

#ifdef __cplusplus
extern "C" {
#endif

enum attn_status {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,         /* a required pointer is NULL */
  ATTN_ERR_SHAPE = 2,        /* negative size, Hq or Hkv < 1, Hq % Hkv != 0, size overflow */
  ATTN_ERR_UNSUPPORTED = 3,  /* D not in {64, 128}; block_size != 16; decode Hq/Hkv > 16 */
  ATTN_ERR_ALIGN = 4,        /* q/k/v/o/cache pointer not 16-byte aligned, or lse/table/ctx
                                pointer not 4-byte aligned */
  ATTN_ERR_SCALE = 5,        /* scale is NaN, infinite or negative */
  ATTN_ERR_HIP = 6,          /* the HIP runtime reported an error (text in attn_last_error) */
  ATTN_ERR_NOMEM = 7,        /* the library workspace could not be allocated */
  ATTN_ERR_WORKSPACE = 8     /* caller workspace too small or misaligned, or the library
                                workspace was needed on a stream under graph capture */
};

/* Prefill / full-sequence forward, bfloat16 q, k, v, o (float32 lse).
 * lse may be NULL (not written). Layouts and semantics as above. D in {64, 128}.
 * One head's K (and V) must be under 2 GiB: Sk * D * 2 < 2^31, else ATTN_ERR_SHAPE.
 * When B * Hq * ceil(Sq / 128) query tiles are too few to fill the device (a short query
 * chunk against a long prefix, say), each tile's keys are split into up to 8 ranges whose
 * partial results are merged by a second kernel (the same online-softmax merge), through a
 * library-owned workspace (see "Library workspace" above). attn_fwd_ex takes a caller
 * workspace instead. */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int Hq, int Hkv, int Sq, int Sk, int D,
             int causal, float scale, hipStream_t stream);

/* attn_fwd with a caller-owned workspace for the key-range splits: at least
 * attn_fwd_workspace_bytes(B, Hq, Hkv, Sq, Sk, D, causal) bytes, 16-byte aligned
 * (ATTN_ERR_WORKSPACE otherwise); NULL = the library workspace. Calls sharing one workspace
 * must not overlap in time. For callers that capture graphs. */
int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal, float scale,
                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes attn_fwd / attn_fwd_ex need on the current device for this problem
 * (0 when it runs without key-range splits or the arguments are invalid). */
size_t attn_fwd_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal);

/* Work mapping of the bf16 forward, for measurement and testing:
 *   0 "tile": one 4-wave workgroup per 128-row query tile;
 *   1 "pair": causal light/heavy tile pairs in one 8-wave workgroup (causal calls only; others
 *      run the tile kernel);
 *   2 "wide": one wave per SIMD, 64 rows per wave, 256-row workgroups (D = 128 only; other D
 *      run the tile kernel);
 *   anything else: chosen per problem (the default). ATTN_FWD_MAPPING = tile / pair / wide sets
 *   the initial value.
 * A forced mapping never splits key ranges. Process-wide; returns the previous setting
 * (-1 = chosen per problem). Every mapping computes the same result up to rounding order. */
int attn_fwd_force_mapping(int mapping);

/* The same computation with float32 q, k, v, o (full-precision path; no workspace). */
int attn_fwd_f32(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int Hq, int Hkv, int Sq, int Sk, int D,
                 int causal, float scale, hipStream_t stream);

/* Prefill over a paged KV cache, for several sequences of any lengths at once (a chunked
 * prefill: the new tokens of each sequence attend to its whole cached context). Prefill and
 * decode are two schedules of the same attention ("Kernel Fusion, Softmax, and Attention");
 * the cache is the paged one of "Optimizing Large Language Model Inference ...", §Paged
 * Attention and Dynamic KV Cache Management, which attn_rope_cache_write fills.
 *   q, o:      [T, Hq, D] bfloat16, token-major; sequence b's query tokens are rows
 *              cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1
 *   lse:       [T, Hq] float32, or NULL
 *   k_cache, v_cache: [num_blocks, Hkv, block_size, D] bfloat16; key t of sequence b is slot
 *              t % block_size of physical block block_table[b * table_stride + t / block_size]
 *   block_table: [B, table_stride] int32
 *   cu_seqlens_q: [B + 1] int32, nondecreasing, cu_seqlens_q[B] <= T
 *   ctx_lens:  [B] int32, keys of each sequence in the cache, its own query tokens included
 *              (they are its last cu_seqlens_q[b+1] - cu_seqlens_q[b] keys)
 * Query i of sequence b is at position ctx_lens[b] - n_b + i (n_b its query count); causal != 0
 * lets it see keys 0 .. that position (the bottom-right alignment of attn_fwd), causal == 0
 * all ctx_lens[b] keys. A row that sees no key gets O = 0 and LSE = -inf.
 *   max_q:     an upper bound on n_b (sizes the grid; a longer sequence is still done whole,
 *              by fewer workgroups); max_q == 0 launches nothing
 *   max_ctx:   an upper bound on ctx_lens[b] (with max_q, decides the key-range splits)
 *   num_blocks: pool size; > 0 makes a table entry outside [0, num_blocks) mask its block's
 *              keys (they take no part) instead of being read; <= 0 = unchecked
 * Keys at or past table_stride * block_size have no table entry and are masked the same way.
 * Cache rows past ctx_lens[b] are never read, whatever they hold.
 * A sequence whose row range is invalid (cu_seqlens_q[b] < 0, decreasing, or past T) is
 * skipped; rows of q outside [cu_seqlens_q[0], cu_seqlens_q[B]) are not written.
 * Few query tiles (a short chunk) split each tile's keys into up to 8 ranges whose partial
 * results a second kernel merges; the partials go to workspace (caller-owned, 16-byte aligned,
 * at least attn_fwd_paged_workspace_bytes(...) bytes) or, when workspace is NULL, to the
 * library workspace (see above). block_size must be 16, D 64 or 128. */
int attn_fwd_paged(const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* block_table, const int32_t* cu_seqlens_q,
                   const int32_t* ctx_lens, void* o, float* lse, int B, int T, int Hq, int Hkv,
                   int D, int block_size, int max_q, int max_ctx, int table_stride,
                   int num_blocks, int causal, float scale, void* workspace,
                   size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes attn_fwd_paged needs for these sizes (0 when it does not split, or for
 * invalid arguments). */
size_t attn_fwd_paged_workspace_bytes(int B, int T, int Hq, int Hkv, int D, int max_q,
                                      int max_ctx, int causal);

/* One-token decode over a paged KV cache ("Optimizing Large Language Model Inference ...",
 * §Paged Attention and Dynamic KV Cache Management: fixed-size blocks of the cache are placed
 * anywhere in a physical pool and a block table maps each sequence's logical blocks to them).
 *   q, o:      [B, Hq, D] bfloat16 (the newest token of each sequence)
 *   k_cache, v_cache: [num_blocks, Hkv, block_size, D] bfloat16; token t of sequence b is
 *              slot t % block_size of physical block block_table[b, t / block_size]
 *   block_table: [B, stride] int32. Here stride = max_b ceil(ctx_lens[b] / block_size),
 *              derived on the device (no host synchronisation). Entries at or past a
 *              sequence's last block are never read.
 *   ctx_lens:  [B] int32, number of cached tokens of each sequence (the new token included).
 *              Values <= 0 give O = 0. No mask is applied inside the context.
 * block_size must be 16. Hq / Hkv must be at most 16. The call runs two kernels on stream:
 * a streaming kernel in which W worker waves split the batch's (sequence, KV head, block)
 * list into equal contiguous shares and write partial results (running max, sum and
 * unnormalised output) to the library workspace (see above), and a combine kernel merging each sequence's
 * partials with the running-softmax algebra. The caller must keep physical block ids valid;
 * they are not range-checked here (attn_decode_paged_full can check them). */
int attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_table, const int32_t* ctx_lens, void* o,
                      int B, int Hq, int Hkv, int D, int block_size, float scale,
                      hipStream_t stream);

/* attn_decode_paged with an explicit block-table row stride and a caller workspace (graph
 * capture, callers that manage their own memory):
 *   block_table_stride: row stride of block_table in entries; <= 0 derives it as above
 *   workspace:          caller-owned device buffer of at least
 *                       attn_decode_workspace_bytes(B, Hq, D) bytes, 16-byte aligned; NULL =
 *                       the library-owned workspace. Calls sharing one workspace must not
 *                       overlap in time.
 * Block ids are not range-checked and no LSE is written (attn_decode_paged_full has both). */
int attn_decode_paged_ex(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_table, const int32_t* ctx_lens, void* o,
                         int B, int Hq, int Hkv, int D, int block_size, float scale,
                         int block_table_stride, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/* attn_decode_paged with every control:
 *   lse:             [B, Hq] float32 log-sum-exp per head, or NULL
 *   table_stride:    row stride of block_table in entries; <= 0 derives it as above
 *   num_blocks:      size of the physical pool; > 0 makes the kernels skip (treat as empty)
 *                    any block-table entry outside [0, num_blocks); <= 0 = unchecked
 *   num_workers:     worker waves W that split the blocks, 1..65536; 0 = the default
 *                    (attn_decode_default_workers()). Any W gives the same result up to
 *                    rounding; it only changes how the work is spread.
 *   workspace:       caller-owned device buffer of at least
 *                    attn_decode_workspace_bytes_ex(B, Hq, Hkv, D, num_workers) bytes, 16-byte
 *                    aligned; NULL = use the library-owned workspace. Calls sharing one
 *                    workspace must not overlap in time. */
int attn_decode_paged_full(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_table, const int32_t* ctx_lens, void* o,
                           float* lse, int B, int Hq, int Hkv, int D, int block_size,
                           float scale, int table_stride, int num_blocks, int num_workers,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* attn_decode_paged_full for callers that cannot allocate device memory (code under graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same kernels and result,
 * but the partial results live in a fixed device array of attn_decode_noalloc_max_bytes()
 * bytes (8 MiB) inside the library, one per device, held until the process ends. The call
 * allocates and frees nothing. Arguments as for attn_decode_paged_full, without a workspace.
 * A problem whose attn_decode_workspace_bytes_ex(B, Hq, Hkv, D, num_workers) exceeds that size
 * returns ATTN_ERR_WORKSPACE (e.g. B = 64, Hq = 32, Hkv = 8, D = 128 at the default 768
 * workers needs 2.7 MB). Nothing in the array needs clearing between calls. Every call on a
 * device shares that device's array: calls that overlap in time on one device (two streams,
 * or two host threads) race on it and give wrong results; serialise them. */
int attn_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* ctx_lens, void* o,
                              float* lse, int B, int Hq, int Hkv, int D, int block_size,
                              float scale, int table_stride, int num_blocks, int num_workers,
                              hipStream_t stream);

/* Size in bytes of the fixed array attn_decode_paged_noalloc uses. */
size_t attn_decode_noalloc_max_bytes(void);

/* Bytes of workspace the decode needs (num_workers 0 = the default):
 * (W + B * Hkv) partial results of (Hq / Hkv) heads x (D + 2) floats, 16-byte padded, plus
 * 2 int32 per (sequence, KV head). 0 for invalid arguments. */
size_t attn_decode_workspace_bytes_ex(int B, int Hq, int Hkv, int D, int num_workers);

/* Bytes of workspace attn_decode_paged_ex needs for B sequences of Hq query heads of size D,
 * whatever Hkv (the largest attn_decode_workspace_bytes_ex(B, Hq, Hkv, D, 0) over the Hkv that
 * divide Hq with Hq / Hkv <= 16). 0 for invalid arguments. */
size_t attn_decode_workspace_bytes(int B, int Hq, int D);

/* Default worker-wave count for the current device: 3 per compute unit. The environment
 * variable ATTN_DECODE_WORKERS = 1..65536 overrides it. */
int attn_decode_default_workers(void);

/* Fused residual add + RMS normalisation of M rows of d elements ("Kernel and Operator
 * Fusion -- Inference Optimization", §4 Tiny example, §5 Why add_rms_norm returns two
 * things): per row,
 *   residual_out = x + residual
 *   out          = residual_out * rsqrt(mean(residual_out^2) + eps) * weight
 * with the mean over the row's d elements.
 *   x, residual:        [M, d] bf16, row-major, read only (unless aliased below)
 *   weight:             [d] bf16
 *   out, residual_out:  [M, d] bf16, written. out may be the same buffer as x and
 *                       residual_out the same buffer as residual (in place); any other
 *                       overlap is undefined.
 * The add, the sum of squares and the scaling are done in fp32; residual_out and out are
 * rounded to bf16 (nearest even) once, at their stores.
 * Requirements: d a multiple of 8 with 8 <= d <= 65536 (else ATTN_ERR_UNSUPPORTED); M >= 0
 * (M == 0 is a no-op); all pointers non-NULL (ATTN_ERR_NULL) and 16-byte aligned
 * (ATTN_ERR_ALIGN); eps finite and >= 0 (ATTN_ERR_SCALE). One kernel on stream, no
 * synchronisation; the caller owns every buffer. */
int attn_add_rms_norm(const void* x, const void* residual, const void* weight, void* out,
                      void* residual_out, int M, int d, float eps, hipStream_t stream);

/* Fused rotary position embedding + paged KV-cache store, the step before decode attention
 * ("Kernel and Operator Fusion -- Inference Optimization", §2 item 6, RoPE then KV store).
 * For every token t at position p = positions[t] of sequence s = seq_ids[t] (s = t when
 * seq_ids is NULL), with theta_i = base^(-2i/D) for i < D/2:
 *   every query head and key head: element i and element i + D/2 turn by p * theta_i
 *     (y_i = x_i cos - x_{i+D/2} sin, y_{i+D/2} = x_{i+D/2} cos + x_i sin);
 *   q_out[t] = rotated q[t];
 *   k_cache[b, h, p % 16, :] = rotated k[t, h], v_cache[b, h, p % 16, :] = v[t, h], where
 *     b = block_table[s * table_stride + p / 16] -- the layout attn_decode_paged reads.
 *   q, q_out:          [T, Hq, D] bf16 (q_out may be q: in place)
 *   k, v:              [T, Hkv, D] bf16
 *   k_cache, v_cache:  [num_blocks, Hkv, block_size, D] bf16, updated in place
 *   block_table:       [num_seqs, table_stride] int32; positions [T] int32;
 *   seq_ids:           [T] int32 or NULL (then T <= num_seqs)
 *   num_blocks:        pool size; > 0 makes the kernel skip the store of a token whose table
 *                      entry is outside [0, num_blocks); <= 0 = unchecked
 * A token stores nothing when p < 0, p / 16 >= table_stride, s is outside [0, num_seqs) or
 * (checked) its entry is outside the pool; its query is rotated regardless. The angle and its
 * sine and cosine are evaluated in fp64, the rotation in fp32, each output rounded to bf16
 * (nearest even) once; values are copied exactly. Two tokens that map to the same slot race.
 * Requirements: D in {64, 128}, block_size 16 (ATTN_ERR_UNSUPPORTED); T, num_seqs >= 0,
 * Hq, Hkv, table_stride >= 1 (ATTN_ERR_SHAPE); base finite and > 0 (ATTN_ERR_SCALE);
 * pointers non-NULL (seq_ids may be NULL) and aligned: 16 bytes for the bf16 tensors, 4 for
 * the int32 arrays (ATTN_ERR_NULL, ATTN_ERR_ALIGN). T == 0 is a no-op. One kernel on stream. */
int attn_rope_cache_write(const void* q, const void* k, const void* v, void* q_out,
                          void* k_cache, void* v_cache, const int32_t* block_table,
                          const int32_t* positions, const int32_t* seq_ids, int T,
                          int num_seqs, int Hq, int Hkv, int D, int block_size,
                          int table_stride, int num_blocks, float base, hipStream_t stream);

/* Static text for a status code. */
const char* attn_status_string(int status);

/* Detail of the last failed call on this thread ("" if none). */
const char* attn_last_error(void);

/* Frees every library-owned workspace and claim block, including replaced ones (synchronises
 * the devices that hold them). No call may be running or enqueued-and-unfinished when it is
 * called. */
void attn_release_workspace(void);

/* ABI version of this header: 10. */
int attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTENTION_ATTN_H */

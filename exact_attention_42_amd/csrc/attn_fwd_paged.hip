// Prefill over a paged KV cache: the queries of a chunk of new tokens (or of a whole prompt)
// of several sequences at once attend to each sequence's cached keys and values, read through
// its block table. This is one schedule of the same attention equation as the contiguous
// forward ("Kernel Fusion, Softmax, and Attention": prefill and decode are different schedules
// of one computation), on the cache layout of "Optimizing Large Language Model Inference
// Through Kernel Fusion and Advanced Memory Management", §Paged Attention and Dynamic KV Cache
// Management (fixed-size blocks anywhere in a physical pool, a table per sequence).
//
// Layouts: q and o are packed token-major, [T, Hq, D], the tokens of sequence b being rows
// cu_q[b] .. cu_q[b+1]-1; lse is [T, Hq]; the caches are [num_blocks, Hkv, 16, D]. Query i of
// sequence b sits at position ctx[b] - (cu_q[b+1] - cu_q[b]) + i of that sequence (its keys
// are already in the cache), so with the causal mask it sees keys 0 .. that position.
//
// The kernel is the 4-wave tile kernel of the contiguous forward (128 query rows per
// workgroup, 32 per wave, 64-key tiles double buffered in LDS through direct-to-LDS loads) with
// another K/V loader: each wave's share of a 64-key tile is exactly one 16-token cache block,
// so a wave looks up one block-table entry per tile and loads its block through a buffer
// resource based at that block, sized to the block's live rows. Rows past a sequence's context
// therefore arrive as zeros whatever the pool holds there, and the pool can be any size. The
// block-table entries of the tile after next are fetched while the current tile is computed.
// A block whose table entry is missing (past the row's stride) or outside the pool (when the
// pool size is given) takes no part: its keys are masked.
//
// Short chunks (few query tiles) split each tile's keys into ranges; the ranges' partial
// results go to a workspace and a second kernel merges them (the same merge as the contiguous
// forward's key-range splits).
#include "fwd_tiles.hpp"

namespace attn {
namespace {

using namespace cdna4;

constexpr int kPage = 16;   // tokens per cache block

struct PagedArgs {
  const uint16_t* q;        // [T, Hq, D]
  const char* kc;           // [num_blocks, Hkv, 16, D]
  const char* vc;
  uint16_t* o;              // [T, Hq, D]
  float* lse;               // [T, Hq] or null
  const int32_t* table;     // [B, stride]
  const int32_t* cu_q;      // [B + 1]
  const int32_t* ctx;       // [B]
  int B, Hq, Hkv, T, group;
  int ntq;                  // query-tile ranks of the grid: ceil(max_q / 128)
  int stride;               // block-table row stride
  int num_blocks;           // pool size; <= 0: entries are not range-checked
  float c;                  // scale * log2(e), > 0
  int nsplit;
  uint16_t* part_o;         // [nsplit][T * Hq][D] bf16 output of each key range alone
  float* part_ml;           // [nsplit][T * Hq][2]
};

// Direct-to-LDS loads of this wave's cache block of a tile. Each lane owns, per load, the byte
// offset within the 16-row block of the chunk that belongs in its LDS slot (the tile's chunk
// permutations depend on the row modulo 16 or less, so a block's rows permute as the tile's).
template <int D>
struct PageDma {
  using G = Geo<D, 4>;
  static_assert(G::kIPW * G::kRPI == kPage, "one cache block per wave and tile");
  uint32_t koff[G::kIPW];
  uint32_t voff[G::kIPW];
  const char* kc;
  const char* vc;
  size_t head_bytes;   // offset of this KV head within a block
  size_t blk_bytes;    // bytes of one physical block (all KV heads)
  int wave;

  __device__ __forceinline__ void init(int wave_, int lane, const PagedArgs& a, int hk) {
    wave = wave_;
    kc = a.kc;
    vc = a.vc;
    head_bytes = (size_t)hk * kPage * G::kRow;
    blk_bytes = (size_t)a.Hkv * kPage * G::kRow;
    const int pos = lane % G::kCPR;
    const int rsub = lane / G::kCPR;
#pragma unroll
    for (int i = 0; i < G::kIPW; ++i) {
      const int row = i * G::kRPI + rsub;    // row within the block (tile row 16 * wave + row)
      koff[i] = row * G::kRow + ((pos ^ kswz<D>(row)) * 16);
      voff[i] = row * G::kRow + ((pos ^ vswz<D>(row)) * 16);
    }
  }

  // Block id (wave-uniform) with `rows` live rows (0..16; 0 loads nothing from memory).
  __device__ __forceinline__ void issue(char* sk, char* sv, int id, int rows) const {
    const size_t base = (size_t)(rows > 0 ? id : 0) * blk_bytes + head_bytes;
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void*)(kc + base), 0, rows * G::kRow, kRawBufferFlags);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc((void*)(vc + base), 0, rows * G::kRow, kRawBufferFlags);
#pragma unroll
    for (int i = 0; i < G::kIPW; ++i) {
      const int blk = wave * G::kIPW + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(sk + blk * 1024), 16, koff[i], 0,
                                               0, 0);
    }
#pragma unroll
    for (int i = 0; i < G::kIPW; ++i) {
      const int blk = wave * G::kIPW + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(sv + blk * 1024), 16, voff[i], 0,
                                               0, 0);
    }
  }
};

// Block-table entries of the four cache blocks of the tile at key kt: lanes 0..3 load one
// each (vector loads, so that waiting for them is part of the wait for the tile's K/V).
// Entries past the sequence's blocks or the table row read as -1.
__device__ __forceinline__ int load_page_ids(const int32_t* row, int kt, int nblk, int lane) {
  const int lb = kt / kPage + lane;
  return (lane < 4 && lb < nblk) ? row[lb] : -1;
}

// From the entries loaded by load_page_ids: bit i set when block i of the tile takes part
// (it exists and, with a pool size given, lies in the pool); this wave's own id.
__device__ __forceinline__ int page_valid_bits(int id, int lane, int num_blocks) {
  const bool ok = lane < 4 && id >= 0 && (num_blocks <= 0 || id < num_blocks);
  return (int)(__builtin_amdgcn_ballot_w64(ok) & 0xFull);
}

template <int D, bool CAUSAL, bool SPLIT>
__device__ __forceinline__ void fwd_paged_body(const PagedArgs& a) {
  using G = Geo<D, 4>;
  __shared__ __attribute__((aligned(1024))) char sk0[G::kTile];
  __shared__ __attribute__((aligned(1024))) char sv0[G::kTile];
  __shared__ __attribute__((aligned(1024))) char sk1[G::kTile];
  __shared__ __attribute__((aligned(1024))) char sv1[G::kTile];
  lds_poison(sk0, G::kTile);
  lds_poison(sv0, G::kTile);
  lds_poison(sk1, G::kTile);
  lds_poison(sv1, G::kTile);
  lds_poison_done();

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_uniform(tid >> 6);
  const int l32 = lane & 31;
  const int h = lane >> 5;

  // ---- work item: (rank, split) major, then (sequence, query head) ----
  const int BH = a.B * a.Hq;
  const int id = blockIdx.x;
  const int unit = id / BH;
  const int bh = id - unit * BH;
  const int rank0 = SPLIT ? unit / a.nsplit : unit;
  const int split = SPLIT ? unit - rank0 * a.nsplit : 0;
  const int b = bh / a.Hq;
  const int hq = bh - b * a.Hq;
  const int hk = hq / a.group;

  const int qs = a.cu_q[b];
  const int qe = a.cu_q[b + 1];
  if (qs < 0 || qe < qs || qe > a.T) return;   // not a valid row range: nothing to do
  const int Sq = qe - qs;
  const int Sk = max(0, a.ctx[b]);
  const int off = Sk - Sq;                      // position of query 0
  const int ntq_b = (Sq + kBM - 1) / kBM;
  if (rank0 >= ntq_b) return;
  // blocks that can have a table entry: those of the context, within the row
  const int nblk = min((Sk + kPage - 1) / kPage, a.stride);
  const int32_t* trow = a.table + (size_t)b * a.stride;
  const size_t R = (size_t)a.T * a.Hq;          // rows of o / lse / one split's partials

  // Out-of-range loads leave LDS bytes untouched or zero; clear the stages once so that every
  // byte a masked key reads is finite.
  {
    u32x4* z[4] = {(u32x4*)sk0, (u32x4*)sv0, (u32x4*)sk1, (u32x4*)sv1};
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < G::kTile / 16 / 256; ++i) z[s][i * 256 + tid] = u32x4{0, 0, 0, 0};
    __syncthreads();
  }

  PageDma<D> dma;
  dma.init(wave, lane, a, hk);

  // K operand: row l32 (+32kb), chunk 2kk+h at its permuted slot; V^T operand offsets of the
  // transposing reads (as in the contiguous tile kernel)
  WaveState<D> w;
#pragma unroll
  for (int kk = 0; kk < G::KS; ++kk)
    w.koff[kk] = l32 * G::kRow + (((2 * kk + h) ^ kswz<D>(l32)) * 16);
  {
    const int g = lane >> 4, j = lane & 15;
    const int keyl = 4 * (g >> 1) + (j >> 2);
    const int small = 2 * (g & 1) + ((j & 3) >> 1);
#pragma unroll
    for (int db = 0; db < G::DB; ++db)
      w.voff[db] = keyl * G::kRow + (((4 * db + small) ^ vswz<D>(keyl)) * 16) + 8 * (j & 1);
  }
  const float c = a.c;

  constexpr int kQBytes = 32 * G::kRow;             // Q of one wave's rows
  static_assert(2 * kQBytes == G::kTile, "two waves' rows per tile");
  auto q_read = [&](const char* st) {
#pragma unroll
    for (int kk = 0; kk < G::KS; ++kk)
      w.qf[kk] = *reinterpret_cast<const u32x4*>(st + (wave & 1) * kQBytes + w.koff[kk]);
  };

  // Every rank of this sequence that the grid leaves over (the grid has a.ntq ranks; a
  // sequence with more query tiles wraps around) is done by the workgroups of the first ranks.
  for (int rank = rank0; rank < ntq_b; rank += a.ntq) {
    const int tile = CAUSAL ? (ntq_b - 1 - rank) : rank;
    const int q0 = tile * kBM;
    const int qw = q0 + wave * 32;
    const int my_q = qw + l32;
    const int wave_last_key = qw + 31 + off;

    int kv_end = Sk;
    if (CAUSAL) kv_end = min(Sk, max(0, q0 + kBM + off));
    const int nall = (kv_end + kBN - 1) / kBN;
    const int t0 = SPLIT ? split * nall / a.nsplit : 0;
    const int ntiles = SPLIT ? (split + 1) * nall / a.nsplit - t0 : nall;

    // Q of the wave's 32 rows passes through LDS, with whole rows per load (one row per lane
    // would touch each row's bytes in 32-byte pieces): wave w's rows go to half w % 2 of stage
    // 1's K (w < 2) or V tile, which the loop first loads into after the barrier below, in the
    // K tiles' layout, so that the fragments are read with the K operand offsets. Rows past Sq
    // load row Sq - 1: they are computed like it, and never stored. (The loads are assembly,
    // which the compiler does not track: the wait for the first tile covers them. They take
    // per-lane addresses: a token's rows are Hq * D elements apart, more than a buffer offset
    // spans for large Hq.)
    {
      char* const qst = (wave < 2 ? sk1 : sv1) + (wave & 1) * kQBytes;
      const int pos = lane % G::kCPR;
      const int rsub = lane / G::kCPR;
#pragma unroll
      for (int i = 0; i < kQBytes / 1024; ++i) {
        const int r = i * G::kRPI + rsub;             // row among the wave's 32
        const int t = qs + min(qw + r, Sq - 1);       // its token
        lds_dma16_global(a.q + ((size_t)t * a.Hq + hq) * D + (pos ^ kswz<D>(r)) * 8,
                         lds_addr(qst) + i * 1024);
      }
    }
#pragma unroll
    for (int i = 0; i < G::DB; ++i) w.o[i] = f32x16{};
    w.mref = -INFINITY;
    w.l_run = 0.f;

    // live rows of this wave's block in the tile at key kt
    auto rows_of = [&](int kt) { return min(kPage, max(0, Sk - (kt + kPage * wave))); };

    // valid_cur: valid bits of the tile in the stage computed next; ent_next: the block-table
    // entries of the tile after it (loaded one tile ahead of their use)
    int valid_cur = 0, ent_next = 0;
    if (ntiles > 0) {
      const int kt0 = t0 * kBN;
      const int ent = load_page_ids(trow, kt0, nblk, lane);
      valid_cur = page_valid_bits(ent, lane, a.num_blocks);
      dma.issue(sk0, sv0, __builtin_amdgcn_readlane(ent, wave),
                ((valid_cur >> wave) & 1) ? rows_of(kt0) : 0);
      if (ntiles > 1) ent_next = load_page_ids(trow, kt0 + kBN, nblk, lane);
    }
    wait_dma_and_barrier();
    // Q, the table entries and the first tile were in flight together. Each wave reads its
    // fragments (its stage named in a branch of its own, so that the reads carry that stage's
    // alias information); the waves that held Q in the V tile clear it again (a masked key
    // must find finite bytes there); the loop first loads into stage 1 after the barrier.
    if (wave < 2) {
      q_read(sk1);
    } else {
      q_read(sv1);
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
#pragma unroll
      for (int i = 0; i < kQBytes / 1024; ++i)
        lds_zero16(lds_addr(sv1 + (wave & 1) * kQBytes) + i * 1024 + lane * 16);
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __syncthreads();

    for (int j = 0; j < ntiles; j += 2) {
      const int kt = (t0 + j) * kBN;
      // stage 0 holds tile j; tile j+1 goes to stage 1
      int valid_next = 0, ent_after = 0;
      if (j + 1 < ntiles) {
        valid_next = page_valid_bits(ent_next, lane, a.num_blocks);
        dma.issue(sk1, sv1, __builtin_amdgcn_readlane(ent_next, wave),
                  ((valid_next >> wave) & 1) ? rows_of(kt + kBN) : 0);
        if (j + 2 < ntiles) ent_after = load_page_ids(trow, kt + 2 * kBN, nblk, lane);
      }
      compute_tile<D, CAUSAL>(w, sk0, sv0, kt, Sk, qw, wave_last_key, my_q, off, h, c,
                              valid_cur);
      wait_dma_and_barrier();
      if (j + 1 >= ntiles) break;
      // stage 1 holds tile j+1; tile j+2 goes to stage 0
      int valid_after = 0, ent_far = 0;
      if (j + 2 < ntiles) {
        valid_after = page_valid_bits(ent_after, lane, a.num_blocks);
        dma.issue(sk0, sv0, __builtin_amdgcn_readlane(ent_after, wave),
                  ((valid_after >> wave) & 1) ? rows_of(kt + 2 * kBN) : 0);
        if (j + 3 < ntiles) ent_far = load_page_ids(trow, kt + 3 * kBN, nblk, lane);
      }
      compute_tile<D, CAUSAL>(w, sk1, sv1, kt + kBN, Sk, qw, wave_last_key, my_q, off, h, c,
                              valid_next);
      wait_dma_and_barrier();
      valid_cur = valid_after;
      ent_next = ent_far;
    }

    const float l_tot = xor32_sum(w.l_run);
    const size_t row = (size_t)(qs + min(my_q, Sq - 1)) * a.Hq + hq;   // (Sq >= 1 here)
    // O leaves through LDS as whole rows (stage_o_group): wave w's 32 rows go to half w % 2 of
    // stage 0's (w < 2) or stage 1's K tile. The loop ended with a barrier, so no wave reads a
    // stage any more and no load is writing one.
    char* const os = (wave < 2 ? sk0 : sk1) + (wave & 1) * kQBytes;
    stage_o_group<D>(os, 0, w.o, (l_tot > 0.f) ? 1.f / l_tot : 0.f, h, l32);
    const size_t row0 = (size_t)(qs + qw) * a.Hq + hq;   // (an address only when qw >= Sq)
    const size_t stride = (size_t)a.Hq * D;              // (tokens are Hq rows apart)
    if (SPLIT) {
      // this key range's own output (bf16), reference max (base 2, scaled) and sum
      store_staged_rows<D, 32>(a.part_o + ((size_t)split * R + row0) * D, stride, os, Sq - qw,
                               lane);
      if (my_q < Sq && h == 0)
        *reinterpret_cast<f32x2*>(a.part_ml + ((size_t)split * R + row) * 2) =
            f32x2{l_tot > 0.f ? w.mref : -INFINITY, l_tot};
    } else {
      store_staged_rows<D, 32>(a.o + row0 * D, stride, os, Sq - qw, lane);
      if (my_q < Sq && a.lse != nullptr && h == 0)
        a.lse[row] = (l_tot > 0.f) ? (w.mref + log2_fast(l_tot)) * kLn2 : -INFINITY;
    }
    // (the next rank's first loads go into the stages that held O)
    if (rank + a.ntq < ntq_b) __syncthreads();
  }
}

// Merge of the key-range splits for the rows of the packed tokens cu_q[0] .. cu_q[B]-1 (the
// rows of all sequences when cu_q is a valid cumulative count); other rows are not touched.
template <int D>
__device__ __forceinline__ void fwd_paged_combine_body(const PagedArgs& a) {
  const int lo = a.cu_q[0], hi = a.cu_q[a.B];
  FwdArgs f{};
  f.o = a.o;
  f.lse = a.lse;
  f.B = 1;
  f.Hq = a.Hq;
  f.Sq = a.T;
  f.nsplit = a.nsplit;
  f.part_o = a.part_o;
  f.part_ml = a.part_ml;
  const size_t row_lo = (size_t)max(0, min(lo, a.T)) * a.Hq;
  const size_t row_hi = (size_t)max(0, min(hi, a.T)) * a.Hq;
  fwd_split_combine_body<D>(f, row_lo, row_hi);
}

#define ATTN_PAGED_KERNEL(NAME, D, CAUSAL, SPLIT)                     \
  __global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) \
  void NAME(PagedArgs a) { fwd_paged_body<D, CAUSAL, SPLIT>(a); }
ATTN_PAGED_KERNEL(fwd_paged_d128_causal, 128, true, false)
ATTN_PAGED_KERNEL(fwd_paged_d128, 128, false, false)
ATTN_PAGED_KERNEL(fwd_paged_d64_causal, 64, true, false)
ATTN_PAGED_KERNEL(fwd_paged_d64, 64, false, false)
ATTN_PAGED_KERNEL(fwd_paged_d128_causal_split, 128, true, true)
ATTN_PAGED_KERNEL(fwd_paged_d128_split, 128, false, true)
ATTN_PAGED_KERNEL(fwd_paged_d64_causal_split, 64, true, true)
ATTN_PAGED_KERNEL(fwd_paged_d64_split, 64, false, true)
#undef ATTN_PAGED_KERNEL

__global__ __launch_bounds__(256) void fwd_paged_d128_split_combine(PagedArgs a) {
  fwd_paged_combine_body<128>(a);
}
__global__ __launch_bounds__(256) void fwd_paged_d64_split_combine(PagedArgs a) {
  fwd_paged_combine_body<64>(a);
}

}  // namespace

int fwd_paged_splits(const PagedProblem& p, int cus) {
  FwdProblem f{};
  f.B = p.B;
  f.Hq = p.Hq;
  f.Hkv = p.Hkv;
  f.Sq = p.max_q;
  f.Sk = p.max_ctx;
  f.D = p.D;
  f.causal = p.causal;
  return fwd_bf16_splits(f, cus);
}

size_t fwd_paged_workspace_bytes(const PagedProblem& p, int nsplit) {
  if (nsplit <= 1) return 0;
  const size_t rows = (size_t)nsplit * p.T * p.Hq;
  return rows * p.D * sizeof(uint16_t) + rows * 2 * sizeof(float);
}

hipError_t launch_fwd_paged(const PagedProblem& p, hipStream_t stream) {
  PagedArgs a;
  a.q = static_cast<const uint16_t*>(p.q);
  a.kc = static_cast<const char*>(p.k_cache);
  a.vc = static_cast<const char*>(p.v_cache);
  a.o = static_cast<uint16_t*>(p.o);
  a.lse = p.lse;
  a.table = p.block_table;
  a.cu_q = p.cu_seqlens_q;
  a.ctx = p.ctx_lens;
  a.B = p.B; a.Hq = p.Hq; a.Hkv = p.Hkv; a.T = p.T;
  a.group = p.Hq / p.Hkv;
  a.ntq = (p.max_q + kBM - 1) / kBM;
  a.stride = p.table_stride;
  a.num_blocks = p.num_blocks;
  float c = p.scale * kLog2e;
  if (!(c > 0.f)) c = 1.17549435e-38f;   // scale 0: uniform weights, masked keys stay -inf
  a.c = c;
  a.nsplit = p.nsplit > 1 ? p.nsplit : 1;
  a.part_o = nullptr;
  a.part_ml = nullptr;
  const long long nwg = (long long)a.ntq * a.nsplit * p.B * p.Hq;
  if (nwg == 0) return hipSuccess;
  if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  dim3 grid((unsigned)nwg), block(256);
  if (a.nsplit > 1) {
    const size_t rows = (size_t)a.nsplit * p.T * p.Hq;
    a.part_o = static_cast<uint16_t*>(p.workspace);
    a.part_ml = reinterpret_cast<float*>(a.part_o + rows * p.D);
    const size_t nrows = (size_t)p.T * p.Hq;
    const int rows_per_block = 256 / (p.D / 4);
    dim3 cgrid((unsigned)((nrows + rows_per_block - 1) / rows_per_block)), cblock(256);
    if (p.D == 128) {
      if (p.causal) hipLaunchKernelGGL(fwd_paged_d128_causal_split, grid, block, 0, stream, a);
      else hipLaunchKernelGGL(fwd_paged_d128_split, grid, block, 0, stream, a);
      hipLaunchKernelGGL(fwd_paged_d128_split_combine, cgrid, cblock, 0, stream, a);
    } else {
      if (p.causal) hipLaunchKernelGGL(fwd_paged_d64_causal_split, grid, block, 0, stream, a);
      else hipLaunchKernelGGL(fwd_paged_d64_split, grid, block, 0, stream, a);
      hipLaunchKernelGGL(fwd_paged_d64_split_combine, cgrid, cblock, 0, stream, a);
    }
    return hipGetLastError();
  }
  if (p.D == 128) {
    if (p.causal) hipLaunchKernelGGL(fwd_paged_d128_causal, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(fwd_paged_d128, grid, block, 0, stream, a);
  } else {
    if (p.causal) hipLaunchKernelGGL(fwd_paged_d64_causal, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(fwd_paged_d64, grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace attn

// One-token decode attention over a paged KV cache on gfx950.
//
// The cache is a pool of fixed-size blocks; a per-sequence block table maps logical block n
// of sequence b to a physical block ("Optimizing Large Language Model Inference ...",
// §Paged Attention and Dynamic KV Cache Management). Physical block p, KV head hk holds its
// block_size tokens as a contiguous [block_size, D] bf16 tile (cache layout
// [num_blocks, Hkv, block_size, D]).
//
// Kernel 1 (stream): the batch's K/V work is the list of units (sequence b, KV head hk,
// block n), ordered by b, then hk, then n. W worker waves split that list into W contiguous,
// equal shares (whatever the mix of context lengths), so every wave streams the same number of
// bytes. Runs of one (b, hk) are "segments"; a wave's share covers one or a few of them, and for
// each it keeps a running max and sum and writes one partial result (its max, sum and
// unnormalised output for the g = Hq / Hkv query heads of hk) to workspace slot (wave +
// segment index); a segment's slots are therefore consecutive. The wave that starts a segment
// and the one that ends it record the segment's first and last slot.
// A wave walks its share as one pipeline: it describes up to 256 units at a time (block-table
// entry, live tokens, segment) in registers, and keeps NS blocks in per-wave LDS slots, filled
// by direct-to-LDS loads NS - 1 blocks ahead of the block it processes; segment changes do not
// stall the pipeline (the next segment's query is fetched when its first block is issued).
// A unit:
//   S^T[tok][h] = K[tok][:] . q[h][:]      MFMA 16x16x32, K rows read from the slot as the A
//                                          operand, q^T resident as B (heads padded to 16)
//   O^T[d][h]  += V^T[d][tok] P^T[tok][h]  MFMA 16x16x16; P^T is the first product's
//                                          accumulator as is; V^T comes from the slot through
//                                          the transposing LDS read.
// All g query heads of hk ride in one wave, so every K/V byte is read from HBM once.
// Kernel 2 (combine): per (query head, sequence), merges the segment's partial results:
// M = max m_s, L = sum l_s 2^(m_s - M), O = sum O_s 2^(m_s - M) / L -- the running-softmax
// algebra of the online softmax ("Fused Kernel Compiler" (Candle paper), §FlashAttention
// Integration).
#include "cdna4.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

using namespace cdna4;

constexpr int kBS = 16;              // tokens per cache block
constexpr int kDecWaves = 4;         // independent worker waves per workgroup
constexpr int kDecThreads = 64 * kDecWaves;

#ifndef ATTN_DEC_WAVES_PER_EU
#define ATTN_DEC_WAVES_PER_EU 2
#endif

struct DecArgs {
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const int32_t* table;
  const int32_t* ctx;
  uint16_t* o;
  float* lse;
  int B, Hq, Hkv, group;
  int stride;        // <= 0: derive from ctx_lens
  int num_blocks;    // <= 0: unchecked
  int workers;       // worker waves W
  float c;           // scale * log2(e), > 0
  float* part_o;     // [W + B*Hkv][group][D] unnormalised partial outputs
  float* part_ml;    // [W + B*Hkv][group][2] partial (max * c, sum)
  int* seg;          // [B*Hkv][2] first and last partial slot of each segment
};

__device__ __forceinline__ int ctx_blocks(int ctx) { return ctx > 0 ? (ctx + kBS - 1) / kBS : 0; }

// Blocks of sequence b that are read: its context, cut to an explicit table row length.
__device__ __forceinline__ int seq_blocks(int ctx, int stride) {
  const int n = ctx_blocks(ctx);
  return (stride > 0 && n > stride) ? stride : n;
}

// Byte geometry of one cache block in a wave's LDS slot. A slot holds the K block, then the V
// block, each as 16 rows of D bf16, written by 1 KiB direct-to-LDS loads (lane l of a load
// fills bytes 16 l .. 16 l + 15 of its KiB). The 16-byte chunks of a row are XOR-swizzled by a
// key that differs between rows sharing a 256-byte bank line, so both the row-wise K reads
// (the 16x16x32 A operand) and the column-wise transposing V reads hit every bank equally.
template <int D>
struct DecGeo {
  static constexpr int kRow = D * 2;             // bytes per token row
  static constexpr int kCPR = kRow / 16;         // 16-byte chunks per row
  static constexpr int kRPI = 1024 / kRow;       // rows per 1 KiB load
  static constexpr int kIPB = kBS / kRPI;        // loads per K (or V) block
  static constexpr int kBlock = kBS * kRow;      // bytes of one K (or V) block
  static constexpr int kSlot = 2 * kBlock;       // K block, then V block
  static constexpr int kLPU = 2 * kIPB;          // loads per unit (block)
  static __device__ __forceinline__ int swz(int row) { return (row * kRow / 256) & (kCPR - 1); }
};

// Buffer resource word 3 for raw (untyped) loads on gfx9-family parts.
constexpr int kRawBufferFlags = 0x00020000;

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// One pipeline stage: a block in flight to the stage's LDS slot, and its description
// (wave-uniform).
struct DecStage {
  int info;      // live tokens | first block of its segment << 5 | last block << 6 | hk << 8
  int sid;       // segment b * Hkv + hk
};

typedef __attribute__((address_space(3))) char lds_char;

// One 1 KiB direct-to-LDS load: lane l copies 16 bytes from buffer offset voff to LDS byte
// lds + 16 l (zeros when voff is past the buffer's size). Written as assembly so that the
// compiler, which would otherwise make every later LDS read wait for all such loads, leaves
// the ordering to the explicit waits below.
__device__ __forceinline__ void lds_dma16(const u32x4& rsrc, uint32_t lds, int voff) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "{m0}"(lds)
               : "memory");
}

// Raw buffer descriptor (base, no stride, size in bytes) for lds_dma16.
__device__ __forceinline__ u32x4 raw_rsrc(const void* base, int bytes) {
  const uint64_t a = (uint64_t)base;
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, (uint32_t)bytes,
               (uint32_t)kRawBufferFlags};
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_char*)p;
}

// Waits until at most N vector-memory operations of this wave are outstanding (they retire
// in issue order). The memory clobber keeps LDS reads of the awaited slot below it.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Info word of a unit: live tokens (0..16), first / last block of the segment, KV head.
constexpr int kInfoFirst = 32;
constexpr int kInfoLast = 64;
constexpr int kInfoHeadShift = 8;

// Units described per round: lane j of register r describes unit 64 r + j of the round.
constexpr int kRound = 256;
constexpr int kRoundRegs = kRound / 64;

// s_waitcnt immediate: vmcnt(0), expcnt and lgkmcnt left free (gfx9 encoding).
constexpr int kWaitVmcnt0 = 0x0F70;

// Blocks per wave between issue and use: one in flight while one is processed measured
// fastest (deeper pipelines only add memory-side contention once ~750 waves stream at once).
#ifndef ATTN_DEC_STAGES
#define ATTN_DEC_STAGES 2
#endif

// Sum over the wave (every lane gets the result).
__device__ __forceinline__ long long wave_sum(long long x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// A 64-bit value that is the same on every lane, moved to scalar registers (the compiler
// cannot tell that cross-lane sums are uniform; buffer descriptors built from them would
// otherwise be wrapped in per-lane loops).
__device__ __forceinline__ long long wave_uniform64(long long x) {
  const unsigned long long u = (unsigned long long)x;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)u);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(u >> 32));
  return (long long)(((unsigned long long)hi << 32) | lo);
}

template <int D, int NS>
__global__ __launch_bounds__(kDecThreads)
__attribute__((amdgpu_waves_per_eu(ATTN_DEC_WAVES_PER_EU))) void decode_stream_kernel(DecArgs a) {
  using G = DecGeo<D>;
  using St = DecStage;
  constexpr int KS = D / 32;        // 16x16x32 k-steps of the score product
  constexpr int DT = D / 16;        // 16-row d tiles of O^T
  __shared__ __attribute__((aligned(1024))) char smem[kDecWaves * NS * G::kSlot];
  lds_poison(smem, sizeof(smem));
  lds_poison_done();

  const int lane = threadIdx.x & 63;
  const int wave = wave_uniform(threadIdx.x >> 6);   // scalar: block addresses are per wave
  const int wid = blockIdx.x * kDecWaves + wave;
  if (wid >= a.workers) return;                      // (waves of a workgroup never meet)
  // ---- one pass over ctx_lens: U = Hkv * sum_b nblk_b units and the longest sequence. The
  // first 64 lengths stay in registers for the search below (all of them when B <= 64). ----
  const int ctx0 = lane < a.B ? a.ctx[lane] : 0;
  const int nbl0 = seq_blocks(ctx0, a.stride);
  long long U = 0;
  int maxblk = 0;
  for (int base = 0; base < a.B; base += 64) {
    const int bb = base + lane;
    const int cb = base == 0 ? ctx0 : (bb < a.B ? a.ctx[bb] : 0);
    U += wave_sum(seq_blocks(cb, a.stride));
    maxblk = max(maxblk, ctx_blocks(cb));
  }
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) maxblk = max(maxblk, __shfl_xor(maxblk, x, 64));
  const int stride = wave_uniform(a.stride > 0 ? a.stride : maxblk);
  U = wave_uniform64(U * a.Hkv);
  // at most one worker per unit, so that every share is non-empty: the waves that meet a
  // segment then fill its whole slot range first..last
  const long long W = min((long long)a.workers, U);
  if (wid >= W) return;
  const long long u0 = (long long)wid * U / W;
  const long long len = (long long)(wid + 1) * U / W - u0;

  // ---- locate unit u0: sequence mb (mnb blocks, mctx tokens), KV head mhk, block mn ----
  int mb = 0, mnb = 0, mctx = 0;
  long long off = 0;
  {
    long long acc = 0;
    for (int base = 0; base < a.B; base += 64) {
      const int bb = base + lane;
      const int cb = base == 0 ? ctx0 : (bb < a.B ? a.ctx[bb] : 0);
      const int nbl = base == 0 ? nbl0 : seq_blocks(cb, a.stride);
      const long long ub = (long long)a.Hkv * nbl;
      long long incl = ub;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const long long t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
      }
      const long long tot = __shfl(incl, 63, 64);
      if (u0 < acc + tot) {
        const unsigned long long hit = __builtin_amdgcn_ballot_w64(acc + incl > u0);
        const int l = (int)__builtin_ctzll(hit);
        mb = base + l;
        mnb = __shfl(nbl, l, 64);
        mctx = __shfl(cb, l, 64);
        off = u0 - (acc + __shfl(incl - ub, l, 64));
        break;
      }
      acc += tot;
    }
  }
  mb = wave_uniform(mb);
  mnb = wave_uniform(mnb);
  mctx = wave_uniform(mctx);
  off = wave_uniform64(off);
  int mhk = wave_uniform((int)(off / mnb));
  int mn = wave_uniform((int)(off - (long long)mhk * mnb));

  const int g = a.group;
  const int r16 = lane & 15;        // MFMA row/column index within a 16-wide tile
  const int grp = lane >> 4;        // k-slot group
  const float c = a.c;
  char* wslots = smem + wave * NS * G::kSlot;   // this wave's NS slots
  const size_t tile_elems = (size_t)kBS * D;
  const size_t phys_elems = (size_t)a.Hkv * tile_elems;
  // direct-to-LDS loads: lane l of load i fetches the chunk that the swizzle places at its
  // 16 bytes, row i * kRPI + l / kCPR
  int dma_off[G::kIPB];
#pragma unroll
  for (int i = 0; i < G::kIPB; ++i) {
    const int row = i * G::kRPI + lane / G::kCPR;
    dma_off[i] = row * G::kRow + (((lane % G::kCPR) ^ G::swz(row)) * 16);
  }
  // K as the A operand: lane (grp, r16) reads row r16, chunk 4 kk + grp
  int krd[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) krd[kk] = r16 * G::kRow + (((4 * kk + grp) ^ G::swz(r16)) * 16);
  // the transposing V read: lane (grp, r16) addresses key 4 grp + r16 / 4, columns
  // 16 dt + 4 (r16 % 4) .. + 3, i.e. half (r16 & 1) of chunk 2 dt + (r16 & 3) / 2
  int vrd[DT];
  {
    const int row = 4 * grp + (r16 >> 2);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      vrd[dt] = G::kBlock + row * G::kRow + ((((r16 & 3) >> 1) + 2 * dt) ^ G::swz(row)) * 16 +
                (r16 & 1) * 8;
  }

  // ---- per-round unit descriptions (table entry, info word, segment), 64 units a register ----
  int mphys[kRoundRegs], minfo[kRoundRegs], msid[kRoundRegs];
  auto describe = [&](long long r0, int rl) {
#pragma unroll
    for (int k = 0; k < kRoundRegs; ++k) { mphys[k] = 0; minfo[k] = 0; msid[k] = 0; }
    int j0 = 0;
    while (j0 < rl) {
      const int take = min(mnb - mn, rl - j0);
      const int sidv = mb * a.Hkv + mhk;
      const int32_t* trow = a.table + (size_t)mb * stride;
#pragma unroll
      for (int k = 0; k < kRoundRegs; ++k) {
        const int jj = 64 * k + lane - j0;
        if (jj >= 0 && jj < take) {
          const int nn = mn + jj;
          mphys[k] = trow[nn];
          minfo[k] = min(kBS, mctx - nn * kBS) | (nn == 0 ? kInfoFirst : 0) |
                     (nn == mnb - 1 ? kInfoLast : 0) | (mhk << kInfoHeadShift);
          msid[k] = sidv;
        }
      }
      j0 += take;
      mn += take;
      if (mn == mnb && r0 + j0 < len) {   // next segment (only while units remain)
        mn = 0;
        if (++mhk == a.Hkv) {
          mhk = 0;
          do {
            ++mb;
            mctx = a.ctx[mb];
            mnb = seq_blocks(mctx, a.stride);   // sequences without blocks have no units
          } while (mnb == 0);
        }
      }
    }
  };

  // ---- consumer state ----
  u32x4 qf[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) qf[kk] = u32x4{0, 0, 0, 0};
  f32x4 acc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) acc[i] = f32x4{};
  float m_run = -INFINITY;  // running max of raw scores for head r16 (same on its 4 lanes)
  float l_run = 0.f;        // running sum over this lane's token slots
  bool has_first = false;   // this wave holds the first block of the current segment
  int cur_sid = -1;         // segment whose query is in qf
  int prod_sid = -1;        // segment of the last block produced
  u32x4 qn[KS];             // prefetched query of segment qn_sid
  int qn_sid = -1;
  bool qn_pending = false;

  // query rows of segment sid (KV head hk) as the 16x16x32 B operand. Columns r16 >= g of
  // the 16-wide tile repeat head g - 1: each column's softmax and output stay its own, and
  // those columns are never written out.
  const int qrow = min(r16, g - 1);
  auto load_q = [&](u32x4 (&dst)[KS], int sid, int hk) {
    const int b = sid / a.Hkv;
    const uint16_t* qh = a.q + ((size_t)b * a.Hq + (size_t)hk * g + qrow) * D;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) dst[kk] = *reinterpret_cast<const u32x4*>(qh + kk * 32 + grp * 8);
  };

  // starts the loads of block p of the round into stage st, slot sl (p >= rl: an empty stage,
  // whose loads still issue but touch no memory)
  auto produce = [&](St& st, int sl, int p, int rl) {
    const int r = p >> 6, lp = p & 63;
    int ph = __builtin_amdgcn_readlane(mphys[0], lp);
    int inf = __builtin_amdgcn_readlane(minfo[0], lp);
    int sd = __builtin_amdgcn_readlane(msid[0], lp);
#pragma unroll
    for (int k = 1; k < kRoundRegs; ++k) {
      if (r == k) {
        ph = __builtin_amdgcn_readlane(mphys[k], lp);
        inf = __builtin_amdgcn_readlane(minfo[k], lp);
        sd = __builtin_amdgcn_readlane(msid[k], lp);
      }
    }
    const bool in = p < rl;
    const bool ok = in && (a.num_blocks <= 0 || (ph >= 0 && ph < a.num_blocks));
    const int live = ok ? (inf & 31) : 0;
    st.info = in ? ((inf & ~31) | live) : 0;
    st.sid = sd;
    if (in && sd != prod_sid) {   // a new segment: prefetch its query unless one is pending
      prod_sid = sd;
      if (!qn_pending) {
        load_q(qn, sd, inf >> kInfoHeadShift);
        qn_sid = sd;
        qn_pending = true;
      }
    }
    const int hk = inf >> kInfoHeadShift;
    const size_t po = ok ? (size_t)ph * phys_elems + (size_t)hk * tile_elems : 0;
    const int bytes = live * G::kRow;   // rows past the context read as zeros
    const u32x4 rk = raw_rsrc(a.kc + po, bytes);
    const u32x4 rv = raw_rsrc(a.vc + po, bytes);
    const uint32_t slot = lds_addr(wslots + sl * G::kSlot);
#pragma unroll
    for (int i = 0; i < G::kIPB; ++i) lds_dma16(rk, slot + i * 1024, dma_off[i]);
#pragma unroll
    for (int i = 0; i < G::kIPB; ++i) lds_dma16(rv, slot + G::kBlock + i * 1024, dma_off[i]);
  };

  // the partial result of the current segment: per head (max * c, sum) and the unnormalised O
  auto emit = [&](int sid, bool last) {
    float l_head = l_run + wave_xor(l_run, 16);
    l_head += wave_xor(l_head, 32);
    const int slot = wid + sid;
    if (r16 < g) {
      float* po = a.part_o + ((size_t)slot * g + r16) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        *reinterpret_cast<f32x4*>(po + 16 * dt + 4 * grp) = acc[dt];
      if (grp == 0) {
        float* pm = a.part_ml + ((size_t)slot * g + r16) * 2;
        pm[0] = (m_run == -INFINITY) ? -INFINITY : m_run * c;
        pm[1] = l_head;
      }
    }
    if (lane == 0) {
      if (has_first) a.seg[2 * sid] = slot;   // this wave starts the segment
      if (last) a.seg[2 * sid + 1] = slot;    // this wave ends it
    }
#pragma unroll
    for (int i = 0; i < DT; ++i) acc[i] = f32x4{};
    m_run = -INFINITY;
    l_run = 0.f;
    has_first = false;
  };

  // processes the block in stage st, slot sl (unit tg of the share); the NS - 1 later stages
  // may still be in flight
  auto consume = [&](const St& st, int sl, long long tg) {
    if (st.sid != cur_sid) {   // segment switch: the prefetched query, else load it now
      cur_sid = st.sid;
      if (qn_pending && qn_sid == st.sid) {
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) qf[kk] = qn[kk];
        qn_pending = false;
      } else {
        load_q(qf, st.sid, st.info >> kInfoHeadShift);
        // wait here, on this rare path, so that the compiler sees qf complete on every path
        // into the products below
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      }
    }
    if (st.info & kInfoFirst) has_first = true;
    const int live = st.info & 31;
    const char* slot = wslots + sl * G::kSlot;
    wait_vmem<(NS - 1) * G::kLPU>();
    u32x4 kf[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) kf[kk] = *reinterpret_cast<const u32x4*>(slot + krd[kk]);
    f32x4 sc = f32x4{};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) sc = mfma16x16x32(kf[kk], qf[kk], sc);

    // lane holds tokens 4*grp + t of this block for head r16
#pragma unroll
    for (int t = 0; t < 4; ++t) sc[t] = (4 * grp + t < live) ? sc[t] : -INFINITY;
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mx = fmaxf(mx, wave_xor(mx, 16));
    mx = fmaxf(mx, wave_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float mc = (m_new == -INFINITY) ? 0.f : m_new * c;
    const float alpha = exp2_fast(m_run * c - mc);
    m_run = m_new;
    float p[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) p[t] = exp2_fast(__builtin_fmaf(sc[t], c, -mc));
    l_run = l_run * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
#pragma unroll
    for (int i = 0; i < DT; ++i) acc[i] *= alpha;
    const u32x2 pb = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};

#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const i16x4 vt = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(slot + vrd[dt]));
      acc[dt] = mfma16x16x16(__builtin_bit_cast(u32x2, vt), pb, acc[dt]);
    }

    if ((st.info & kInfoLast) || tg == len - 1) emit(st.sid, (st.info & kInfoLast) != 0);
  };

  // ---- rounds of up to kRound units; within a round, NS - 1 blocks stay in flight ----
  St st[NS];
  for (long long r0 = 0; r0 < len; r0 += kRound) {
    const int rl = (int)min((long long)kRound, len - r0);
    describe(r0, rl);
#pragma unroll
    for (int s = 0; s < NS - 1; ++s) produce(st[s], s, s, rl);
    for (int t = 0; t < rl; t += NS) {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        produce(st[(s + NS - 1) % NS], (s + NS - 1) % NS, t + s + NS - 1, rl);
        consume(st[s], s, r0 + t + s);
        if (t + s + 1 >= rl) goto round_done;
      }
    }
  round_done:
    // stages past the round's end were empty loads; retire them before the next round reuses
    // their registers
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  }
}

template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecArgs a) {
  constexpr int kBatch = 8;          // partial results whose loads are issued together
  const int hq = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int g = a.group;
  const int s = b * a.Hkv + hq / g, hh = hq % g;
  const bool empty = seq_blocks(a.ctx[b], a.stride) == 0;
  float M = -INFINITY, L = 0.f, O = 0.f;   // running max (base 2, scaled), sum, output
  if (!empty) {
    const int first = a.seg[2 * s], last = a.seg[2 * s + 1];
    for (int base = first; base <= last; base += kBatch) {
      float m[kBatch], l[kBatch], o[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int sl = min(base + i, last);   // past the range: a repeat, weighted 0 below
        const f32x2 ml = *reinterpret_cast<const f32x2*>(a.part_ml + ((size_t)sl * g + hh) * 2);
        m[i] = (base + i <= last) ? ml[0] : -INFINITY;
        l[i] = ml[1];
        o[i] = a.part_o[((size_t)sl * g + hh) * D + d];
      }
      float mb = M;
#pragma unroll
      for (int i = 0; i < kBatch; ++i) mb = fmaxf(mb, m[i]);
      if (mb != -INFINITY) {
        const float r = (M == -INFINITY) ? 0.f : exp2_fast(M - mb);
        L *= r;
        O *= r;
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
          const float w = (m[i] == -INFINITY) ? 0.f : exp2_fast(m[i] - mb);
          L += w * l[i];
          O += w * o[i];
        }
        M = mb;
      }
    }
  }
  const float out = (L > 0.f) ? O / L : 0.f;
  __bf16 ob = (__bf16)out;
  a.o[((size_t)b * a.Hq + hq) * D + d] = __builtin_bit_cast(uint16_t, ob);
  if (a.lse != nullptr && d == 0)
    a.lse[(size_t)b * a.Hq + hq] = (L > 0.f) ? (M + log2_fast(L)) * kLn2 : -INFINITY;
}

}  // namespace

size_t decode_workspace_bytes(int B, int Hkv, int group, int D, int workers) {
  const size_t slots = (size_t)workers + (size_t)B * Hkv;
  size_t bytes = slots * group * (D + 2) * sizeof(float);  // partial outputs, then (max, sum)
  bytes = (bytes + 15) / 16 * 16;
  bytes += (size_t)B * Hkv * 2 * sizeof(int);              // segment slot ranges
  return bytes;
}

hipError_t launch_decode_paged(const DecodeProblem& p, hipStream_t stream) {
  DecArgs a;
  a.q = static_cast<const uint16_t*>(p.q);
  a.kc = static_cast<const uint16_t*>(p.k_cache);
  a.vc = static_cast<const uint16_t*>(p.v_cache);
  a.table = p.block_table;
  a.ctx = p.ctx_lens;
  a.o = static_cast<uint16_t*>(p.o);
  a.lse = p.lse;
  a.B = p.B; a.Hq = p.Hq; a.Hkv = p.Hkv; a.group = p.Hq / p.Hkv;
  a.stride = p.table_stride;
  a.num_blocks = p.num_blocks;
  a.workers = p.workers;
  float c = p.scale * kLog2e;
  if (!(c > 0.f)) c = 1.17549435e-38f;   // scale 0: uniform weights
  a.c = c;
  const size_t slots = (size_t)p.workers + (size_t)p.B * p.Hkv;
  char* ws = static_cast<char*>(p.workspace);
  a.part_o = reinterpret_cast<float*>(ws);
  a.part_ml = a.part_o + slots * a.group * p.D;
  const size_t head = ((slots * a.group * (p.D + 2) * sizeof(float)) + 15) / 16 * 16;
  a.seg = reinterpret_cast<int*>(ws + head);
  if (p.B == 0) return hipSuccess;
  dim3 g1((p.workers + kDecWaves - 1) / kDecWaves), b1(kDecThreads);
  dim3 g2(p.Hq, p.B);
  if (p.D == 128) {
    hipLaunchKernelGGL((decode_stream_kernel<128, ATTN_DEC_STAGES>), g1, b1, 0, stream, a);
    hipLaunchKernelGGL(decode_combine_kernel<128>, g2, dim3(128), 0, stream, a);
  } else {
    hipLaunchKernelGGL((decode_stream_kernel<64, ATTN_DEC_STAGES>), g1, b1, 0, stream, a);
    hipLaunchKernelGGL(decode_combine_kernel<64>, g2, dim3(64), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace attn

// Pieces shared by the bf16 forward kernels on gfx950: K/V tile geometry in LDS, the
// direct-to-LDS tile loader, the kernel argument block and small wave-level helpers.
// The tile scheme: K and V move from global memory to LDS in tiles of 64 keys with
// direct-to-LDS buffer loads (each lane's 16 bytes land at base + 16*lane). Rows are stored
// unpadded with their 16-byte chunks XOR-permuted: K by chunk ^ (row % 16), which makes the
// row-per-lane ds_read_b128 operand reads conflict-free; V by chunk ^ 4*(row % 4), which
// spreads the transposing ds_read_b64_tr_b16 reads that form the V^T operand over all banks.
#pragma once

#include "cdna4.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

using namespace cdna4;

constexpr int kBN = 64;            // keys per K/V tile
constexpr int kBM = 128;           // query rows per tile of the 4-wave tile kernels
constexpr float kLazy = 8.0f;      // log2 of the largest probability allowed before rescaling

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

template <int D, int WAVES>
struct Geo {
  static constexpr int kRow = 2 * D;              // bytes per K or V row in LDS
  static constexpr int kTile = kBN * kRow;        // one K or V tile
  static constexpr int kCPR = D / 8;              // 16-byte chunks per row
  static constexpr int kRPI = 1024 / kRow;        // rows per 1 KiB direct load
  static constexpr int kIPW = kTile / 1024 / WAVES;  // direct loads per wave, tensor and tile
  static constexpr int KS = D / 16;               // MFMA k-steps over the head dimension
  static constexpr int DB = D / 32;               // 32-wide d blocks of O^T
};

// Chunk permutations (XOR masks) of K and V rows in LDS.
template <int D>
__device__ __forceinline__ int kswz(int row) { return row % (D / 8); }
template <int D>
__device__ __forceinline__ int vswz(int row) {
  return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int B, Hq, Hkv, Sq, Sk;
  int group;       // Hq / Hkv
  int ntq;         // number of 128-query tiles
  int npairs;      // pair kernel: work items per (batch, query head)
  int nitems;      // pair kernel: B * Hq * npairs
  float c;         // scale * log2(e), > 0
  int nsplit;      // split kernel: key-range splits per query tile
  uint16_t* part_o;  // split kernels: [nsplit][B*Hq*Sq][D] bf16 output of each key range alone
  float* part_ml;     // split kernels: [nsplit][B*Hq*Sq][2] (reference max, sum) of each range
  // wide kernel: per-XCD claim counters, the launch's "nothing left" word and the work items'
  // claim marks (null: no workgroup takes another's item), and this launch's mark
  unsigned long long* claim;
  unsigned long long epoch;
};

// Buffer resource word 3 for raw (untyped) loads on gfx9-family parts.
constexpr int kRawBufferFlags = 0x00020000;

// s_waitcnt immediate: lgkmcnt(0), vmcnt and expcnt left free
constexpr int kWaitLgkm0 = 0xC07F;

typedef __attribute__((address_space(3))) char lds_char;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_char*)p;
}

// Raw buffer descriptor (base, no stride, size in bytes) for lds_dma16.
__device__ __forceinline__ u32x4 raw_rsrc(const void* base, int bytes) {
  const uint64_t p = (uint64_t)base;
  return u32x4{(uint32_t)p, (uint32_t)(p >> 32) & 0xffffu, (uint32_t)bytes,
               (uint32_t)kRawBufferFlags};
}

// A 1 KiB direct-to-LDS load (lane l copies 16 bytes from buffer offset voff to LDS byte
// lds + 16 l) and a 16-byte LDS store of zeros, written as assembly: the compiler does not see
// them, and their ordering is left to explicit waits.
__device__ __forceinline__ void lds_dma16(const u32x4& rsrc, uint32_t lds, int voff) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "{m0}"(lds)
               : "memory");
}
// The same load from per-lane 64-bit addresses: lane l copies the 16 bytes at src to LDS byte
// lds + 16 l.
__device__ __forceinline__ void lds_dma16_global(const void* src, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void lds_zero16(uint32_t lds) {
  asm volatile("ds_write_b128 %0, %1" : : "v"(lds), "v"(u32x4{0, 0, 0, 0}) : "memory");
}

// Direct-to-LDS staging of K/V tiles; each wave issues its share of a tile. Each lane owns,
// per direct load, the byte offset within a K (or V) tile of the global chunk it moves: row
// blk*RPI + lane/CPR, chunk (lane%CPR) ^ permutation(row), so that the chunk lands in its
// permuted LDS slot. The loads go through buffer resources over this head's K and V, so a
// tile is addressed by a scalar offset and the per-lane offsets stay fixed.
template <int D, int WAVES>
struct TileDma {
  using G = Geo<D, WAVES>;
  uint32_t koff[G::kIPW];
  uint32_t voff[G::kIPW];
  __amdgpu_buffer_rsrc_t rk, rv;
  int wave;   // wave-uniform
  int lane;

  __device__ __forceinline__ void init(int wave_, int lane_, const uint16_t* kbase,
                                       const uint16_t* vbase, int Sk) {
    wave = wave_;
    lane = lane_;
    const int bytes = Sk * G::kRow;   // the C ABI keeps this below 2^31
    rk = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, 0, bytes, kRawBufferFlags);
    rv = __builtin_amdgcn_make_buffer_rsrc((void*)vbase, 0, bytes, kRawBufferFlags);
    const int pos = lane % G::kCPR;
    const int rsub = lane / G::kCPR;
#pragma unroll
    for (int i = 0; i < G::kIPW; ++i) {
      const int row = (wave * G::kIPW + i) * G::kRPI + rsub;
      koff[i] = row * G::kRow + ((pos ^ kswz<D>(row)) * 16);
      voff[i] = row * G::kRow + ((pos ^ vswz<D>(row)) * 16);
    }
  }

  // This wave's share of the loads of one tensor's tile (K through rk and koff, or V) at key
  // kt. A tile that runs past Sk clamps those keys to Sk-1: they are masked out of the scores,
  // and their (finite) V rows are multiplied by a probability of exactly 0.
  // (v is a constant at every call site; inlining folds the selection)
  __device__ __forceinline__ void issue_one(bool v, char* dst, int kt, int Sk) const {
    const int tile_off = kt * G::kRow;
    const int last = Sk - 1 - kt;                 // last valid row of this tile
    if (last >= kBN - 1) {
#pragma unroll
      for (int i = 0; i < G::kIPW; ++i) {
        const int blk = wave * G::kIPW + i;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(v ? rv : rk, (lds_void*)(dst + blk * 1024), 16,
                                                 v ? voff[i] : koff[i], tile_off, 0, 0);
      }
    } else {
      // (the empty asm keeps this a branch: folded into straight-line code, the clamping
      //  below would run on every tile)
      asm volatile("");
#pragma unroll
      for (int i = 0; i < G::kIPW; ++i) {
        const int blk = wave * G::kIPW + i;
        const int row = blk * G::kRPI + lane / G::kCPR;
        const uint32_t shift = row > last ? (uint32_t)((row - last) * G::kRow) : 0u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(v ? rv : rk, (lds_void*)(dst + blk * 1024), 16,
                                                 (v ? voff[i] : koff[i]) - shift, tile_off, 0, 0);
      }
    }
  }

  // Load j (0..2*kIPW-1: K parts then V parts) of this wave's share of the tile at key kt,
  // with the same clamping of rows past Sk as issue_one.
  __device__ __forceinline__ void issue_part(char* sk, char* sv, int kt, int Sk, int j) const {
    const bool v = j >= G::kIPW;
    const int i = v ? j - G::kIPW : j;
    const int blk = wave * G::kIPW + i;
    const int tile_off = kt * G::kRow;
    const int last = Sk - 1 - kt;
    const uint32_t base = v ? voff[i] : koff[i];
    char* dst = (v ? sv : sk) + blk * 1024;
    if (last >= kBN - 1) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(v ? rv : rk, (lds_void*)dst, 16, base, tile_off, 0,
                                               0);
    } else {
      asm volatile("");
      const int row = blk * G::kRPI + lane / G::kCPR;
      const uint32_t shift = row > last ? (uint32_t)((row - last) * G::kRow) : 0u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(v ? rv : rk, (lds_void*)dst, 16, base - shift,
                                               tile_off, 0, 0);
    }
  }

  // Load j as issue_part, without clamping: rows at or past Sk are out of the buffer's range
  // and land in LDS as whatever the hardware gives for out-of-range loads (zero, or the stage
  // left as it was); callers keep those LDS bytes finite and mask those keys.
  __device__ __forceinline__ void issue_part_unclamped(char* sk, char* sv, int kt, int j) const {
    const bool v = j >= G::kIPW;
    const int i = v ? j - G::kIPW : j;
    const int blk = wave * G::kIPW + i;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(v ? rv : rk, (lds_void*)((v ? sv : sk) + blk * 1024),
                                             16, v ? voff[i] : koff[i], kt * G::kRow, 0, 0);
  }

  // both tensors' tiles at key kt
  __device__ __forceinline__ void issue(char* sk, char* sv, int kt, int Sk) const {
    issue_one(false, sk, kt, Sk);
    issue_one(true, sv, kt, Sk);
  }
};

__device__ __forceinline__ void wait_dma_and_barrier() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

template <int D>
struct WaveState {
  using G = Geo<D, 4>;
  u32x4 qf[G::KS];          // Q^T fragments (B operand)
  f32x16 o[G::DB];          // O^T accumulators
  float mref;               // reference max (scaled, base 2) of this lane's query
  float l_run;              // sum of probabilities over this lane's half of the keys
  int koff[G::KS];          // per-lane K operand offsets within a tile
  int voff[G::DB];          // per-lane V^T transposed-read offsets within a tile
};

// Marks the Q fragments as used (an empty assembly block that reads and writes them), so that
// the compiler waits for their loads at this point and at no later one. Placed after a wait
// for all loads in flight, it costs nothing.
template <int D>
__device__ __forceinline__ void consume_q(WaveState<D>& w) {
#pragma unroll
  for (int kk = 0; kk < Geo<D, 4>::KS; ++kk) asm volatile("" : "+v"(w.qf[kk]));
}

// max / sum of x over lanes l and l ^ 32. v_permlane32_swap returns the low half of x in
// both halves of one register and the high half in both halves of the other, so the pair
// (l, l ^ 32) meets in every lane with no LDS round trip.
__device__ __forceinline__ float xor32_max(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// Normalised O of one 32-query column group as bf16 into its rows. The accumulators hold O^T:
// lane (l32, h) has element r of block db at d = 32 db + 8 (r / 4) + 4 h + r % 4 for query l32,
// i.e. half of every 16-byte chunk of the row. Lanes l and l ^ 32 (the same query) swap halves
// with v_permlane32_swap so that each lane holds whole chunks (the even ones on h = 0, the odd
// ones on h = 1) and stores 16 bytes at a time: half the store instructions, and 32 contiguous
// bytes of a row per instruction instead of 8-byte pieces. Every lane runs the swaps; only
// lanes whose query exists (store) write.
template <int DB>
__device__ __forceinline__ void store_o_group(uint16_t* orow, const f32x16 (&o)[DB], float inv,
                                              int h, bool store) {
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int e0 = 2 * k, e1 = 2 * k + 1;
      const uint32_t x0 = pack_bf16x2(o[db][4 * e0 + 0] * inv, o[db][4 * e0 + 1] * inv);
      const uint32_t x1 = pack_bf16x2(o[db][4 * e0 + 2] * inv, o[db][4 * e0 + 3] * inv);
      const uint32_t y0 = pack_bf16x2(o[db][4 * e1 + 0] * inv, o[db][4 * e1 + 1] * inv);
      const uint32_t y1 = pack_bf16x2(o[db][4 * e1 + 2] * inv, o[db][4 * e1 + 3] * inv);
      // upper lanes of x take the lower lanes of y and vice versa: h = 0 ends with chunk e0
      // (its own first half in x, the partner's second half in y), h = 1 with chunk e1
      const auto s0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
      const auto s1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
      if (store)
        *reinterpret_cast<u32x4*>(orow + 32 * db + 8 * (h ? e1 : e0)) =
            u32x4{s0[0], s1[0], s0[1], s1[1]};
    }
}

// O through LDS, so that every store instruction covers whole rows. Stored straight from the
// accumulators (store_o_group), one instruction writes 32 bytes into each of 32 rows: four
// times as many partial-line writes as the same bytes in whole rows.
//
// stage_o_group: normalised O of one 32-row group into the wave's LDS region, one row per
// query (G::kRow bytes, 16-byte chunk c of row r at slot c ^ kswz(r)). The lane's chunks are
// formed as in store_o_group: after the half swap, lane (l32, h) holds chunks 4 db + 2 k + h of
// row row0 + l32.
template <int D>
__device__ __forceinline__ void stage_o_group(char* st, int row0, const f32x16 (&o)[D / 32],
                                              float inv, int h, int l32) {
  using G = Geo<D, 4>;
  int r = row0 + l32;
  asm volatile("" : "+v"(r), "+v"(h));   // (addresses formed here, not hoisted above the loop)
#pragma unroll
  for (int db = 0; db < G::DB; ++db)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int e0 = 2 * k, e1 = 2 * k + 1;
      const uint32_t x0 = pack_bf16x2(o[db][4 * e0 + 0] * inv, o[db][4 * e0 + 1] * inv);
      const uint32_t x1 = pack_bf16x2(o[db][4 * e0 + 2] * inv, o[db][4 * e0 + 3] * inv);
      const uint32_t y0 = pack_bf16x2(o[db][4 * e1 + 0] * inv, o[db][4 * e1 + 1] * inv);
      const uint32_t y1 = pack_bf16x2(o[db][4 * e1 + 2] * inv, o[db][4 * e1 + 3] * inv);
      const auto s0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
      const auto s1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
      const int ch = 4 * db + 2 * k + h;
      *reinterpret_cast<u32x4*>(st + r * G::kRow + ((ch ^ kswz<D>(r)) * 16)) =
          u32x4{s0[0], s1[0], s0[1], s1[1]};
    }
}
// store_staged_rows: the wave's NROWS staged rows back out, G::kCPR lanes per row, so that one
// store covers 64 / kCPR rows (1 KiB at D = 128, consecutive where `stride`, the elements from
// one row of O to the next, is D). Rows from `nvalid` on are not stored.
template <int D, int NROWS>
__device__ __forceinline__ void store_staged_rows(uint16_t* obase, size_t stride, const char* st,
                                                  int nvalid, int lane) {
  using G = Geo<D, 4>;
  static_assert(NROWS % (64 / G::kCPR) == 0, "whole stores");
  constexpr int kRowsPerStore = 64 / G::kCPR;
  asm volatile("" : "+v"(lane));         // (addresses formed here, not hoisted above the loop)
  const int cc = lane % G::kCPR;
#pragma unroll
  for (int i = 0; i < NROWS / kRowsPerStore; ++i) {
    const int r = kRowsPerStore * i + lane / G::kCPR;
    const u32x4 x = *reinterpret_cast<const u32x4*>(st + r * G::kRow + ((cc ^ kswz<D>(r)) * 16));
    if (r < nvalid) *reinterpret_cast<u32x4*>(obase + (size_t)r * stride + cc * 8) = x;
  }
}

// Work item -> (batch, query head, pair). Workgroups are dispatched to the 8 XCDs round
// robin; this gives XCD x a contiguous run of items, so the items of one KV head (adjacent
// query heads of one batch) share that XCD's L2.
__device__ __forceinline__ int xcd_item(int id, int n) {
  constexpr int kXcd = 8;
  const int x = id % kXcd, s = id / kXcd;
  const int q = n / kXcd, r = n % kXcd;
  return x < r ? x * (q + 1) + s : r * (q + 1) + (x - r) * q + s;
}


// O^T += V^T P^T for the first NKB 32-key blocks of the tile. Slots (h, 0..3) of P^T hold
// keys 32kb+16t+4h+{0..3} and slots (h, 4..7) the same + 8: one transposed read each.
template <int D, int NKB>
__device__ __forceinline__ void pv_blocks(WaveState<D>& w, const char* sv,
                                          const u32x4 (&pb)[2][2]) {
  using G = Geo<D, 4>;
#pragma unroll
  for (int db = 0; db < G::DB; ++db) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const char* vp = sv + w.voff[db] + (32 * kb + 16 * t) * G::kRow;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vp));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vp + 8 * G::kRow));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
        const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
        w.o[db] = mfma32x32x16(u32x4{l2[0], l2[1], h2[0], h2[1]}, pb[kb][t], w.o[db]);
      }
    }
  }
}

// One K/V tile: S^T = K Q^T, mask, online softmax, O^T += V^T P^T. Bit i of kvalid clears
// keys 16i..16i+15 of the tile when 0 (a paged cache block that takes no part).
template <int D, bool CAUSAL>
__device__ __forceinline__ void compute_tile(WaveState<D>& w, const char* sk, const char* sv,
                                             int kt, int Sk, int qw, int wave_last_key,
                                             int my_q, int off, int h, float c,
                                             int kvalid = 0xF) {
  using G = Geo<D, 4>;
  bool act[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
    act[kb] = (kt + 32 * kb < Sk) && (!CAUSAL || kt + 32 * kb <= wave_last_key);

  // ---- S^T = K Q^T ----
  // (computed for every block: a block no query of this wave can see is masked below, and
  //  skipping it would cost a register copy of every score on all the other tiles)
  u32x4 kf[2][G::KS];
#pragma unroll
  for (int kk = 0; kk < G::KS; ++kk)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      kf[kb][kk] = *reinterpret_cast<const u32x4*>(sk + 32 * kb * G::kRow + w.koff[kk]);
  f32x16 s[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) s[kb] = mfma32x32x16(kf[kb][0], w.qf[0], f32x16{});
#pragma unroll
  for (int kk = 1; kk < G::KS; ++kk)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) s[kb] = mfma32x32x16(kf[kb][kk], w.qf[kk], s[kb]);

  // ---- mask: causal diagonal, key tail, inactive blocks ----
  const bool need_mask = (kt + kBN > Sk) || (CAUSAL && kt + kBN - 1 > qw + off) || kvalid != 0xF;
  if (need_mask) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kt + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
        bool vis = act[kb] && key < Sk && ((kvalid >> ((key - kt) >> 4)) & 1);
        if (CAUSAL) vis = vis && (key <= my_q + off);
        s[kb][r] = vis ? s[kb][r] : -INFINITY;
      }
    }
  }

  // ---- online softmax (per lane = per query) with a lazily moved reference ----
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; r += 2) mx = fmax3(mx, s[kb][r], s[kb][r + 1]);
  mx = xor32_max(mx);
  const float mxc = mx * c;                       // -inf stays -inf (c > 0)
  const bool move = mxc > w.mref + kLazy;
  if (__builtin_amdgcn_ballot_w64(move)) {
    // (the empty asm keeps this a branch: folded into straight-line code, the 64 multiplies
    //  below would run on every tile)
    asm volatile("");
    // lanes that keep their reference use 1 (not exp2(mref - mref): NaN while mref = -inf);
    // a lane moving away from -inf gets 0, which clears its empty state
    const float alpha = move ? exp2_fast(w.mref - mxc) : 1.f;
    w.mref = move ? mxc : w.mref;
    w.l_run *= alpha;
#pragma unroll
    for (int i = 0; i < G::DB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) w.o[i][r] *= alpha;
  }
  const float mu = (w.mref == -INFINITY) ? 0.f : w.mref;

  // ---- P^T as bf16 B operands; fp32 row sums (the LSE needs them unrounded) ----
  u32x4 pb[2][2];
  float ls[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = exp2_fast(__builtin_fmaf(s[kb][8 * t + 2 * e], c, -mu));
        const float p1 = exp2_fast(__builtin_fmaf(s[kb][8 * t + 2 * e + 1], c, -mu));
        if (kb == 0 && t == 0 && e == 0) {
          ls[0] = p0;
          ls[1] = p1;
        } else {
          ls[0] += p0;
          ls[1] += p1;
        }
        pb[kb][t][e] = pack_bf16x2(p0, p1);
      }
  w.l_run += ls[0] + ls[1];

  // ---- O^T += V^T P^T over the active 32-key blocks (a uniform choice per tile) ----
  pv_blocks<D, 2>(w, sv, pb);
}

// Merges the key-range splits of each query row: M = max m_s, L = sum l_s 2^(m_s - M),
// O = sum O_s 2^(m_s - M) / L (the online-softmax merge), then O in bf16 and the natural-log
// LSE. D/4 threads per row, each with 4 consecutive columns. Rows outside [row_lo, row_hi)
// are left alone.
template <int D>
__device__ __forceinline__ void fwd_split_combine_body(const FwdArgs& a, size_t row_lo = 0,
                                                       size_t row_hi = ~(size_t)0) {
  constexpr int TPR = D / 4;
  const size_t nrows = (size_t)a.B * a.Hq * a.Sq;
  const size_t row = (size_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int c4 = (threadIdx.x % TPR) * 4;
  if (row >= nrows || row < row_lo || row >= row_hi) return;
  float M = -INFINITY;
  for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, a.part_ml[((size_t)s * nrows + row) * 2]);
  float L = 0.f;
  f32x4 O = f32x4{};
  if (M != -INFINITY) {
    for (int s = 0; s < a.nsplit; ++s) {
      const size_t pr = (size_t)s * nrows + row;
      const f32x2 ml = *reinterpret_cast<const f32x2*>(a.part_ml + pr * 2);
      if (ml[0] == -INFINITY) continue;
      // (each range's output is its own softmax-weighted sum: weight it by its share of the
      //  whole row's sum)
      const float wl = exp2_fast(ml[0] - M) * ml[1];
      L += wl;
      const u32x2 ov = *reinterpret_cast<const u32x2*>(a.part_o + pr * D + c4);
      O += wl * f32x4{__builtin_bit_cast(float, ov[0] << 16),
                      __builtin_bit_cast(float, ov[0] & 0xffff0000u),
                      __builtin_bit_cast(float, ov[1] << 16),
                      __builtin_bit_cast(float, ov[1] & 0xffff0000u)};
    }
  }
  const float inv = (L > 0.f) ? 1.f / L : 0.f;
  u32x2 v = {pack_bf16x2(O[0] * inv, O[1] * inv), pack_bf16x2(O[2] * inv, O[3] * inv)};
  *reinterpret_cast<u32x2*>(a.o + row * D + c4) = v;
  if (a.lse != nullptr && c4 == 0)
    a.lse[row] = (L > 0.f) ? (M + log2_fast(L)) * kLn2 : -INFINITY;
}

}  // namespace
}  // namespace attn

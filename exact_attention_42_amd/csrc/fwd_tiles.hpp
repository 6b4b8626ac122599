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
  float* part_o;   // split kernel: [nsplit][B*Hq*Sq][D] unnormalised partial outputs
  float* part_ml;  // split kernel: [nsplit][B*Hq*Sq][2] (reference max, sum)
};

// Buffer resource word 3 for raw (untyped) loads on gfx9-family parts.
constexpr int kRawBufferFlags = 0x00020000;

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

// Work item -> (batch, query head, pair). Workgroups are dispatched to the 8 XCDs round
// robin; this gives XCD x a contiguous run of items, so the items of one KV head (adjacent
// query heads of one batch) share that XCD's L2.
__device__ __forceinline__ int xcd_item(int id, int n) {
  constexpr int kXcd = 8;
  const int x = id % kXcd, s = id / kXcd;
  const int q = n / kXcd, r = n % kXcd;
  return x < r ? x * (q + 1) + s : r * (q + 1) + (x - r) * q + s;
}

}  // namespace
}  // namespace attn

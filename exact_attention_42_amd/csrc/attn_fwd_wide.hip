// Fused exact-attention forward for bf16 Q/K/V with D = 128 on gfx950, "wide" mapping: one
// wave per SIMD and 64 query rows per wave. The method is the one of "Fused Kernel Compiler"
// (Candle paper), §FlashAttention Integration: Q, K and V are tiled on chip, scores, softmax
// and the weighted sum run in a single pass with an online softmax, and only O (plus the
// per-row log-sum-exp) is written, so memory stays O(N).
//
// Work item: (batch, query head, 256-row query tile), one workgroup of 4 waves; wave w owns
// rows 64w..64w+63 of the tile as two 32-row column groups g = 0, 1 of the matrix-core
// products. Each XCD (one L2 each) works through a contiguous range of KV heads, all query
// tiles and heads of one KV head together, causal tiles heaviest first.
//
// Products (transposed, as in the other bf16 forward kernels):
//   S^T[key][q] = K[key][:] . Q[q][:]      v_mfma_f32_32x32x16_bf16, A = K rows from LDS,
//                                          B = Q^T held in VGPRs for the whole item
//   O^T[d][q]  += V^T[d][key] P^T[key][q]   A = V^T from the transposing LDS read,
//                                          B = P^T straight from the score accumulators
// Both column groups use the same K and V operand reads, so each LDS byte read feeds two
// matrix-core instructions, and the 128 O accumulators per lane live in the accumulation
// registers (one wave per SIMD has all 512 registers per lane).
//
// Pipeline. Every 32-key block i passes three phases: scores (matrix cores), softmax (vector
// ALU: max, reference decision, exponentials, bf16 P^T) and the product with V (matrix cores).
// Iteration i runs, in two stretches of code:
//   1. the scores of block i for both groups, interleaved with the exponentials of block
//      i-1's group 1 and then the max / reference decision of block i's group 0;
//   2. the products with V of block i-1 for both groups, interleaved with the exponentials of
//      block i's group 0 and then the max / reference decision of block i's group 1.
// So the vector work of one block always issues between matrix-core instructions of another.
// The reference max moves lazily (only when a row's max exceeds it by more than 2^8); when it
// does, O is rescaled after the products of the previous block have been added, which keeps
// every pending P^T valid without rescaling it.
//
// K/V staging: 64-key tiles in 4 LDS stages (32 KiB each: K then V), filled by the four waves'
// direct-to-LDS buffer loads. A wave's 8 loads of a tile go out one at a time between its
// matrix-core instructions (the four waves reach a load together, and a few of them at once
// already stall in-order issue while the address unit works through them), starting after the
// workgroup barrier in the middle of tile T - 3's second block, into the stage tile T - 4 used;
// that barrier also guarantees tile T - 2 has landed.
// Each stage is a separate LDS object so the compiler can tell the in-flight loads into one
// stage from reads of another.
#include <type_traits>

#include "fwd_tiles.hpp"

namespace attn {
namespace {

using namespace cdna4;

constexpr int kWideRows = 64;                  // query rows per wave
constexpr int kWideBM = 4 * kWideRows;         // query rows per workgroup
// K/V tiles resident in LDS. Four: a wave's last tile is at most 3 tiles before the
// workgroup's last, so its stage is never reloaded and the wave can finish its last block
// after the loop.
constexpr int kStages = 4;
// Workgroups per XCD that take other XCDs' last items (a fast XCD's share of the spread between
// XCDs, in light items of a few to a few tens of microseconds each).
constexpr int kTakers = 128;
// Words of the claim block before the item marks (the counters and the "nothing left" mark).
constexpr int kClaimHead = 9 * 16;

// s_waitcnt immediates, gfx9 encoding (vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt free)
constexpr int kWaitVm0 = 0x0F70;
constexpr int kWaitVm8 = 0x0F78;
constexpr int kWaitVm11 = 0x0F7B;
constexpr int kWaitVm16 = 0x4F70;   // (vmcnt's two high bits sit at 15:14)

template <int D>
struct WideWave {
  using G = Geo<D, 4>;
  u32x4 qf[2][G::KS];    // Q^T fragments of the two column groups (B operands)
  f32x16 o[2][G::DB];    // O^T accumulators
  float m[2];            // reference max (scaled, base 2) of this lane's query, per group
  float l[2];            // running sum over this lane's half of the keys, per group
  float thr[2];          // raw score above which the reference moves, per group
  int lim[2];            // keys below lim are visible to this lane's query, per group
  int koff[G::KS];       // per-lane K operand offsets within a 32-key block
  int voff[G::DB];       // per-lane V^T transposed-read offsets within a 32-key block
};

// Registers carried from one iteration to the next. The pending scores and P^T are double
// buffered by block parity (an even block reads slot 1 and writes slot 0, an odd block the
// reverse), so the new values never have to be copied over the old ones, which are still being
// read while the new ones are produced.
template <int D>
struct WidePipe {
  using G = Geo<D, 4>;
  u32x4 kf[G::KS];       // K fragments of the block scored next
  f32x16 s1[2];          // group 1 scores of the previous block (exponentials pending)
  float mu1[2];          // the reference those exponentials subtract
  u32x4 p0[2][2];        // group 0 P^T of the previous block (product with V pending)
};

template <int D, int FIRST = 0, int LAST = Geo<D, 4>::KS>
__device__ __forceinline__ void read_k(const WideWave<D>& w, const char* kblk,
                                       u32x4 (&kf)[Geo<D, 4>::KS]) {
#pragma unroll
  for (int kk = FIRST; kk < LAST; ++kk)
    kf[kk] = *reinterpret_cast<const u32x4*>(kblk + w.koff[kk]);
}

// V^T fragments of a 32-key block, index 2*db + t: keys 16t + 4h + {0..3} in slots (h, 0..3)
// and 16t + 8 + 4h + {0..3} in slots (h, 4..7), matching the P^T slots.
template <int D, int FIRST = 0, int LAST = 2 * Geo<D, 4>::DB>
__device__ __forceinline__ void read_v(const WideWave<D>& w, const char* vblk,
                                       u32x4 (&vf)[2 * Geo<D, 4>::DB]) {
  using G = Geo<D, 4>;
#pragma unroll
  for (int i = FIRST; i < LAST; ++i) {
    const char* vp = vblk + w.voff[i >> 1] + 16 * (i & 1) * G::kRow;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vp));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vp + 8 * G::kRow));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
    const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
    vf[i] = u32x4{l2[0], l2[1], h2[0], h2[1]};
  }
}

// Accumulator element r of a lane holds key k0 + 4h + 8(r/4) + r%4: keys at or past lim
// become -inf.
__device__ __forceinline__ void mask_block(f32x16& s, int lim, int k0, int h) {
  const int d = lim - k0 - 4 * h;
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = (8 * (r >> 2) + (r & 3) < d) ? s[r] : -INFINITY;
}

// Row max of a block (raw scores; the lane pair l, l ^ 32 holds one query's 32 keys), in
// pieces that can be spread between matrix-core instructions.
struct RowMax {
  float m[5];
  float mx;
};
__device__ __forceinline__ void row_max_a(RowMax& r, const f32x16& s) {
  r.m[0] = fmax3(s[0], s[1], s[2]);
  r.m[1] = fmax3(s[3], s[4], s[5]);
  r.m[2] = fmax3(s[6], s[7], s[8]);
}
__device__ __forceinline__ void row_max_b(RowMax& r, const f32x16& s) {
  r.m[3] = fmax3(s[9], s[10], s[11]);
  r.m[4] = fmax3(s[12], s[13], s[14]);
  r.mx = fmax3(fmax3(r.m[0], r.m[1], r.m[2]), fmax3(r.m[3], r.m[4], s[15]), -INFINITY);
}
__device__ __forceinline__ void row_max_c(RowMax& r) { r.mx = xor32_max(r.mx); }

// The reference max of a lane's query (scaled scores, base 2) starts at kNoRef, a finite
// stand-in for "no key seen yet": a block with a finite score always moves it, masked scores
// (-inf) never do, and exponentials against it are only ever taken of -inf (giving 0).
constexpr float kNoRef = -1e30f;

// Whether a block's row max mx (raw scores) moves the reference: when it exceeds it by more
// than 2^kLazy after scaling, i.e. when mx > thr = (m + kLazy) / c. Returns whether any lane of
// the wave moves (wave-uniform); the move itself is apply_move, on the rare path.
__device__ __forceinline__ bool must_move(float mx, float thr, bool& move) {
  move = mx > thr;
  return __builtin_amdgcn_ballot_w64(move) != 0;
}

// Moves the reference of the lanes that must (a lane moving away from kNoRef gets factor 0,
// which clears its empty state): returns the factor O must be scaled by (1 on other lanes),
// scales the running sum and recomputes the threshold.
__device__ __forceinline__ float apply_move(float& m, float& l, float& thr, float mx, bool move,
                                            float c, float inv_c) {
  const float mxc = mx * c;
  const float alpha = move ? exp2_fast(m - mxc) : 1.f;
  m = move ? mxc : m;
  l *= alpha;
  thr = (m + kLazy) * inv_c;
  return alpha;
}

// Probabilities of two adjacent accumulator elements (2e, 2e + 1 of half t) against the
// reference mu: one packed bf16 word of P^T, and the fp32 values added to the running sums.
__device__ __forceinline__ uint32_t exp_pair(const f32x16& s, int t, int e, float c, float mu,
                                             float& l0, float& l1) {
  const float p0 = exp2_fast(__builtin_fmaf(s[8 * t + 2 * e], c, -mu));
  const float p1 = exp2_fast(__builtin_fmaf(s[8 * t + 2 * e + 1], c, -mu));
  l0 += p0;
  l1 += p1;
  return pack_bf16x2(p0, p1);
}

__device__ __forceinline__ void scale_acc(f32x16& o, float a) {
#pragma unroll
  for (int r = 0; r < 16; ++r) o[r] *= a;
}

// Keeps a value computed before this point: the compiler may not sink its computation past
// it (pure computations otherwise drift to their first use and undo the schedule).
template <typename T>
__device__ __forceinline__ void pin(T& x) { asm volatile("" : "+v"(x)); }

// Ends a stretch: nothing moves across it in the machine scheduler either.
__device__ __forceinline__ void stretch_end() { __builtin_amdgcn_sched_barrier(0); }

// The same with the LDS reads early: DS after each of the first two matrix-core instructions.
template <int DS, int T, int V>
__device__ __forceinline__ void stretch_pattern_early_ds() {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (i < 2) __builtin_amdgcn_sched_group_barrier(0x100, DS, 0);
    if (V > 0) __builtin_amdgcn_sched_group_barrier(0x002, V, 0);
    if (T > 0) __builtin_amdgcn_sched_group_barrier(0x400, T, 0);
  }
}

// Issue pattern of one stretch of 8 matrix-core instructions: after each one, DS LDS reads,
// T transcendental (exponential) and V other vector instructions. (Sched-group masks: 0x008
// matrix core, 0x100 LDS read, 0x400 transcendental, 0x002 vector ALU.)
template <int DS, int T, int V>
__device__ __forceinline__ void stretch_pattern() {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (DS > 0) __builtin_amdgcn_sched_group_barrier(0x100, DS, 0);
    if (V > 0) __builtin_amdgcn_sched_group_barrier(0x002, V, 0);
    if (T > 0) __builtin_amdgcn_sched_group_barrier(0x400, T, 0);
  }
}

// One iteration for block i (see the file comment): the scores and decisions of block i and
// the pending exponentials and products of block i-1. mask: block i needs the causal /
// key-tail mask (wave-uniform). vprev: LDS rows of block i-1's V; knext: LDS rows of block
// i+1's K (read for the next iteration); k0: first key of block i. mid() runs between
// stretches 1b and 2a (the workgroup barrier and the next loads, on odd blocks).
// Four stretches, each one group's 8 matrix-core instructions with vector work written in
// between them, in the order it should issue:
//   1a  scores of group 0            | exponentials of block i-1, group 1, first half
//   1b  scores of group 1            | the second half; max / decision of group 0
//   2a  products of block i-1, grp 0 | exponentials of group 0, first half
//   2b  products of block i-1, grp 1 | the second half; max / decision of group 1
// The K operands of block i+1 are read during 2b. (EVEN: block i is the first of its tile.)
template <int D, bool EVEN, typename Mid, typename Hook>
__device__ __forceinline__ void wide_iter(WideWave<D>& w, WidePipe<D>& p, const char* vprev,
                                          const char* knext, int k0, bool mask, int h, float c,
                                          float inv_c, Mid&& mid, Hook&& hook) {
  using G = Geo<D, 4>;
  constexpr int KS = G::KS;
  constexpr int NV = 2 * G::DB;
  static_assert(KS == 8 && NV == 8, "D = 128");
  constexpr int IN = EVEN ? 1 : 0, OUT = 1 - IN;   // pending-state slots read and written
  stretch_end();

  // ---- 1a ----
  u32x4 vf[NV];
  read_v<D>(w, vprev, vf);
  u32x4 p1[2];
  float la = 0.f, lb = 0.f;
  f32x16 s0 = f32x16{};
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    s0 = mfma32x32x16(p.kf[kk], w.qf[0][kk], s0);
    if (kk & 1) p1[0][kk >> 1] = exp_pair(p.s1[IN], 0, kk >> 1, c, p.mu1[IN], la, lb);
    hook(0, kk);
  }
  stretch_pattern<2, 1, 3>();
  pin(s0);
  pin(p1[0]);
  pin(la);
  pin(lb);
  stretch_end();

  // ---- 1b ---- (the mask, rare, between the stretches)
  if (__builtin_expect(mask, 0)) mask_block(s0, w.lim[0], k0, h);
  stretch_end();
  f32x16 s1 = f32x16{};
  RowMax r0;
  bool move0, any0;
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    s1 = mfma32x32x16(p.kf[kk], w.qf[1][kk], s1);
    if (kk == 0) p1[1][0] = exp_pair(p.s1[IN], 1, 0, c, p.mu1[IN], la, lb);
    if (kk == 1) row_max_a(r0, s0);
    if (kk == 2) p1[1][1] = exp_pair(p.s1[IN], 1, 1, c, p.mu1[IN], la, lb);
    if (kk == 3) row_max_b(r0, s0);
    if (kk == 4) p1[1][2] = exp_pair(p.s1[IN], 1, 2, c, p.mu1[IN], la, lb);
    if (kk == 5) row_max_c(r0);
    if (kk == 6) p1[1][3] = exp_pair(p.s1[IN], 1, 3, c, p.mu1[IN], la, lb);
    if (kk == 7) any0 = must_move(r0.mx, w.thr[0], move0);
    hook(1, kk);
  }
  w.l[1] += la + lb;
  stretch_pattern<0, 1, 5>();
  pin(s0);
  pin(s1);
  pin(p1[1]);
  pin(w.l[1]);
  stretch_end();
  // (rare) group 0's reference moves: before its exponentials below
  float alpha0 = 1.f;
  if (__builtin_expect(any0, 0)) alpha0 = apply_move(w.m[0], w.l[0], w.thr[0], r0.mx, move0, c, inv_c);
  const float mu0 = w.m[0];
  stretch_end();

  mid();
  asm volatile("" ::: "memory");
  stretch_end();

  // ---- 2a ----
  u32x4 (&p0n)[2] = p.p0[OUT];
  la = 0.f;
  lb = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    w.o[0][i >> 1] = mfma32x32x16(vf[i], p.p0[IN][i & 1], w.o[0][i >> 1]);
    if (i & 1) p0n[0][i >> 1] = exp_pair(s0, 0, i >> 1, c, mu0, la, lb);
    hook(2, i);
  }
  stretch_pattern<0, 1, 3>();
  pin(p0n[0]);
  pin(la);
  pin(lb);
  stretch_end();

  // ---- 2b ---- (the mask, rare, between the stretches)
  if (__builtin_expect(mask, 0)) mask_block(s1, w.lim[1], k0, h);
  stretch_end();
  // (the current K fragments were last used in 1b: the next block's go into the same registers)
  read_k<D>(w, knext, p.kf);
  RowMax r1;
  bool move1, any1;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    w.o[1][i >> 1] = mfma32x32x16(vf[i], p1[i & 1], w.o[1][i >> 1]);
    if (i == 0) p0n[1][0] = exp_pair(s0, 1, 0, c, mu0, la, lb);
    if (i == 1) row_max_a(r1, s1);
    if (i == 2) p0n[1][1] = exp_pair(s0, 1, 1, c, mu0, la, lb);
    if (i == 3) row_max_b(r1, s1);
    if (i == 4) p0n[1][2] = exp_pair(s0, 1, 2, c, mu0, la, lb);
    if (i == 5) row_max_c(r1);
    if (i == 6) p0n[1][3] = exp_pair(s0, 1, 3, c, mu0, la, lb);
    if (i == 7) any1 = must_move(r1.mx, w.thr[1], move1);
    hook(3, i);
  }
  w.l[0] += la + lb;
  stretch_pattern_early_ds<4, 1, 5>();
  pin(p0n[1]);
  pin(s1);
  pin(w.l[0]);
  stretch_end();

  // ---- rescale (rare), after the products of block i-1 were added ----
  if (__builtin_expect(any0, 0)) {
#pragma unroll
    for (int db = 0; db < G::DB; ++db) scale_acc(w.o[0][db], alpha0);
  }
  if (__builtin_expect(any1, 0)) {
    const float alpha1 = apply_move(w.m[1], w.l[1], w.thr[1], r1.mx, move1, c, inv_c);
#pragma unroll
    for (int db = 0; db < G::DB; ++db) scale_acc(w.o[1][db], alpha1);
  }
  p.s1[OUT] = s1;
  p.mu1[OUT] = w.m[1];
  stretch_end();
}

// The pending work of a wave's last block: exponentials of its group 1 and both products.
template <int D, int SLOT>
__device__ __forceinline__ void wide_drain(WideWave<D>& w, WidePipe<D>& p, const char* vlast,
                                           float c) {
  using G = Geo<D, 4>;
  constexpr int NV = 2 * G::DB;
  u32x4 vf[NV];
  read_v<D>(w, vlast, vf);
  u32x4 p1[2];
  float la = 0.f, lb = 0.f;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) p1[t][e] = exp_pair(p.s1[SLOT], t, e, c, p.mu1[SLOT], la, lb);
  w.l[1] += la + lb;
#pragma unroll
  for (int i = 0; i < NV; ++i)
    w.o[0][i >> 1] = mfma32x32x16(vf[i], p.p0[SLOT][i & 1], w.o[0][i >> 1]);
#pragma unroll
  for (int i = 0; i < NV; ++i) w.o[1][i >> 1] = mfma32x32x16(vf[i], p1[i & 1], w.o[1][i >> 1]);
}

// Work item -> (query tile rank, batch * query head). Workgroups are dispatched to the 8 XCDs
// round robin (workgroup id mod 8), and each XCD (one L2) works through its own KV heads: when
// the B * Hkv KV heads split evenly, XCD x takes KV heads x * n .. x * n + n - 1, in bundles of
// ceil(4 / group) consecutive ones; within a bundle the items go tile rank by tile rank,
// heaviest first, each rank listing all query heads of the bundle. So the workgroups running
// at once on an XCD read the K/V of a few KV heads through its L2, and at least 4 consecutive
// workgroups of an XCD's queue (one per shader engine) have the same amount of work. (Within an XCD the hardware hands
// workgroups to its shader engines in a fixed rotation and in order: a workgroup whose engine
// has no free CU holds back the ones behind it, so when heavy and light tiles alternate in the
// queue, CUs wait for their next workgroup; equal neighbours avoid that.) Otherwise the items
// are ordered KV head by KV head (heaviest tile first, the query heads of a tile together) and
// XCD x takes a contiguous eighth of that order.
__device__ __forceinline__ void wide_item(int id, int nitems, int ntq, int group, int nkv,
                                          int& rank, int& bh) {
  constexpr int kXcd = 8;
  if (nkv % kXcd == 0) {
    const int x = id % kXcd, j = id / kXcd;
    const int hpx = nkv / kXcd;                     // KV heads of this XCD
    const int nb = (4 + group - 1) / group;         // KV heads per bundle
    const int per_bundle = nb * group * ntq;
    const int bundle = j / per_bundle;
    const int nbb = min(nb, hpx - bundle * nb);     // KV heads in this bundle (the last: fewer)
    const int r = j - bundle * per_bundle;
    rank = r / (nbb * group);
    const int rem = r - rank * (nbb * group);       // (KV head in bundle) * group + g
    bh = (x * hpx + bundle * nb) * group + rem;     // (b * Hkv + hk) * group + g = b * Hq + hq
    return;
  }
  const int item = xcd_item(id, nitems);
  const int per_kv = group * ntq;
  const int kvh = item / per_kv;                    // batch * Hkv + KV head
  const int r = item - kvh * per_kv;
  rank = r / group;
  bh = kvh * group + (r - rank * group);
}

// One work item on the workgroup. SPLIT: the workgroup covers one of a.nsplit contiguous ranges
// of its query tile's key tiles and writes that range's own output (bf16, normalised by the
// range's sum), reference max and sum to the workspace; a merge kernel combines the ranges
// (for problems with too few query tiles to fill the device). `claimed`: the item is this workgroup's own, marked in the claim
// block as the work starts; if a workgroup of another XCD took it first, this one stops there.
template <int D, bool CAUSAL, bool SPLIT>
__device__ __forceinline__ void wide_item_body(const FwdArgs& a, int id, bool claimed) {
  using G = Geo<D, 4>;
  // (The V stages are placed in the low 64 KiB, where a stage's base fits the 16-bit offset
  //  field of the transposing reads; the LDS layout orders these objects by name.)
  __shared__ __attribute__((aligned(1024))) char a_v0[G::kTile];
  __shared__ __attribute__((aligned(1024))) char a_v1[G::kTile];
  __shared__ __attribute__((aligned(1024))) char a_v2[G::kTile];
  __shared__ __attribute__((aligned(1024))) char a_v3[G::kTile];
  __shared__ __attribute__((aligned(1024))) char b_k0[G::kTile];
  __shared__ __attribute__((aligned(1024))) char b_k1[G::kTile];
  __shared__ __attribute__((aligned(1024))) char b_k2[G::kTile];
  __shared__ __attribute__((aligned(1024))) char b_k3[G::kTile];
  char* const KS[kStages] = {b_k0, b_k1, b_k2, b_k3};
  char* const VS[kStages] = {a_v0, a_v1, a_v2, a_v3};
#pragma unroll
  for (int st = 0; st < kStages; ++st) {
    lds_poison(KS[st], G::kTile);
    lds_poison(VS[st], G::kTile);
  }
  lds_poison_done();

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_uniform(tid >> 6);
  const int l32 = lane & 31;
  const int h = lane >> 5;

  int rank, bh;
  wide_item(id, a.nitems, SPLIT ? a.ntq * a.nsplit : a.ntq, a.group, a.B * a.Hkv, rank,
            bh);
  // (with splits, the ranges of one query tile are neighbours in the order, equal in work)
  const int split = SPLIT ? rank % a.nsplit : 0;
  if (SPLIT) rank /= a.nsplit;
  const int tile = CAUSAL ? (a.ntq - 1 - rank) : rank;
  const int b = bh / a.Hq;
  const int hq = bh - b * a.Hq;
  const int hk = hq / a.group;
  const int q0 = tile * kWideBM;
  const int qw = q0 + wave * kWideRows;
  const int off = a.Sk - a.Sq;

  const uint16_t* qbase = a.q + ((size_t)(b * a.Hq + hq) * a.Sq) * D;
  const uint16_t* kbase = a.k + ((size_t)(b * a.Hkv + hk) * a.Sk) * D;
  const uint16_t* vbase = a.v + ((size_t)(b * a.Hkv + hk) * a.Sk) * D;

  // ---- key tiles of the workgroup, and blocks of this wave ----
  const int qend = min(q0 + kWideBM, a.Sq);         // rows of the workgroup end here
  int kend = a.Sk;
  if (CAUSAL) kend = min(a.Sk, max(0, qend + off));
  const int nt_all = (kend + kBN - 1) / kBN;        // key tiles the query tile sees
  // this workgroup's key tiles t0 .. t0 + nt - 1 (all of them without splits); below, tile and
  // block indices count from t0, and kt0 is the first key
  const int t0 = SPLIT ? split * nt_all / a.nsplit : 0;
  const int nt = SPLIT ? (split + 1) * nt_all / a.nsplit - t0 : nt_all;
  const int kt0 = t0 * kBN;
  int nblk = 0;                                     // 32-key blocks this wave scores
  int nunm = 0;                                     // leading blocks needing no mask
  if (qw < a.Sq) {
    const int qlast = min(qw + kWideRows, a.Sq) - 1;
    int kw = a.Sk;
    if (CAUSAL) kw = min(a.Sk, max(0, qlast + off + 1));
    nblk = (kw + 31) / 32;
    nunm = a.Sk / 32;
    if (CAUSAL) nunm = min(nunm, max(0, qw + off + 1) / 32);
    // (rows past Sq see every key of the tile: they need no mask, and are never stored)
    nunm = min(nunm, nblk);
    if (SPLIT) {
      nblk = max(0, min(nblk, 2 * (t0 + nt)) - 2 * t0);
      nunm = min(max(0, nunm - 2 * t0), nblk);
    }
  }

  WideWave<D> w;
  const float a_inv_c = 1.f / a.c;
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int qi = qw + 32 * g + l32;
    w.lim[g] = CAUSAL ? min(a.Sk, qi + off + 1) : a.Sk;
#pragma unroll
    for (int i = 0; i < G::DB; ++i) w.o[g][i] = f32x16{};
    w.m[g] = kNoRef;
    w.l[g] = 0.f;
    w.thr[g] = (kNoRef + kLazy) * a_inv_c;
  }
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

  // (the item's claim mark goes out first, and has returned by the wait for tile 0)
  __shared__ int s_stolen;
  unsigned long long took = 0;
  if (claimed && wave == 0 && lane == 0) took = atomicMax(a.claim + kClaimHead + id, a.epoch);

  // Every V stage starts cleared (stages 2 and 3 once Q has passed through them, below): the
  // dummy block before the first reads "V" from the second half of the last stage (0 * V must
  // stay 0), and rows past Sk of a partial tile are loaded out of range, which leaves finite V
  // bytes (cleared, or an earlier tile's) beside the masked keys. Keys past Sk are cut out of
  // the scores by selection, so the K stages may hold anything; each still takes a store here,
  // ahead of every load into LDS, as do stages 2 and 3: without a store into each stage before
  // the first such load, the compiler's tracking of these loads puts waits for loads in flight
  // in front of reads inside the loop.
  {
#pragma unroll
    for (int st = 0; st < kStages; ++st) {
      u32x4* kz = reinterpret_cast<u32x4*>(KS[st]);
      u32x4* vz = reinterpret_cast<u32x4*>(VS[st]);
      kz[tid] = u32x4{0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < (st < 2 ? G::kTile / 16 / 256 : 1); ++i)
        vz[i * 256 + tid] = u32x4{0, 0, 0, 0};
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }

  // Q of the wave (its 64 rows, 16 KiB) passes through LDS, with whole rows per load (one row
  // per lane would touch each row's 256 bytes in 16 pieces): into a quarter of stages 2 and 3,
  // which the first tiles leave free, in the K tiles' layout, so that the fragments are read
  // with the K operand offsets. Rows past Sq load row Sq - 1 (every tile has a row below Sq):
  // they are computed like it, and never stored. (Written as assembly: seen by the compiler
  // ahead of the tiles' loads into stages 2 and 3, these loads would bring back the waits.)
  char* const qs = wave == 0 ? KS[2] : wave == 1 ? KS[3] : wave == 2 ? VS[2] : VS[3];
  {
    const u32x4 rq = raw_rsrc(qbase + (size_t)q0 * D, kWideBM * G::kRow);
    const int pos = lane % G::kCPR;
    const int rsub = lane / G::kCPR;
#pragma unroll
    for (int i = 0; i < kWideRows / G::kRPI; ++i) {
      const int r = i * G::kRPI + rsub;             // row among the wave's 64
      const int src = min(qw + r, a.Sq - 1) - q0;
      lds_dma16(rq, lds_addr(qs) + i * 1024, src * G::kRow + ((pos ^ kswz<D>(r)) * 16));
    }
  }
  static_assert(kWideRows / G::kRPI == 16, "D = 128: 16 Q loads per wave");
  TileDma<D, 4> dma;
  dma.init(wave, lane, kbase, vbase, a.Sk);
  // Loads: a wave's 8 loads of tile X go out one at a time between the matrix-core instructions
  // of iterations 2X - 5 (after its barrier: loads 0..2) and 2X - 4 (loads 3..7), into the stage
  // of tile X - 4, which no wave reads after barrier X - 3. Every load is issued, so the count of
  // loads in flight after tile T + 1's is always 8 at barrier T: a tile past the workgroup's
  // last loads, instead, the tile its stage already holds (X - 4, the same bytes), or for X < 4
  // tile X itself into a stage no tile uses. Tiles 0 and 1 and the first three loads of tile 2
  // are issued here (tile 2's once Q has been read out of the stages); then wait for tile 0.
  constexpr int kParts = 2 * G::kIPW;      // loads per wave and tile
  static_assert(kParts == 8, "D = 128: 4 K and 4 V loads per wave and tile");
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int j = 0; j < kParts; ++j) dma.issue_part_unclamped(KS[t], VS[t], kt0 + t * kBN, j);
  }
  // The wave's Q has landed (the tiles' 16 loads are still out). Each wave reads its fragments
  // (its stage named in a branch of its own, so that the reads carry that stage's alias
  // information), those holding Q in a V stage clear it, and tile 2 may overwrite stage 2 once
  // every wave is past the barrier.
  __builtin_amdgcn_s_waitcnt(kWaitVm16);
  asm volatile("" ::: "memory");
  auto q_read = [&](const char* st) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
#pragma unroll
      for (int kk = 0; kk < G::KS; ++kk)
        w.qf[g][kk] = *reinterpret_cast<const u32x4*>(st + 32 * g * G::kRow + w.koff[kk]);
    }
  };
  if (wave == 0) {
    q_read(KS[2]);
  } else if (wave == 1) {
    q_read(KS[3]);
  } else {
    q_read(wave == 2 ? VS[2] : VS[3]);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
#pragma unroll
    for (int i = 0; i < G::kTile / 1024; ++i) lds_zero16(lds_addr(qs) + i * 1024 + lane * 16);
  }
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
#pragma unroll
  for (int j = 0; j < 3; ++j) dma.issue_part_unclamped(KS[2], VS[2], kt0 + 2 * kBN, j);
  __builtin_amdgcn_s_waitcnt(kWaitVm11);
  if (claimed && wave == 0 && lane == 0) s_stolen = took == (a.epoch | 1ull);
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  if (claimed && s_stolen) {
    // another XCD's workgroup runs this item: no load may still be writing LDS at the end
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    return;
  }

  // the dummy block before the first (slot 1, read by block 0): scores -inf, P^T zero
  WidePipe<D> p;
  if (nblk > 0) read_k<D>(w, KS[0], p.kf);
#pragma unroll
  for (int r = 0; r < 16; ++r) p.s1[1][r] = -INFINITY;
  p.mu1[1] = kNoRef;
  p.p0[1][0] = u32x4{0, 0, 0, 0};
  p.p0[1][1] = u32x4{0, 0, 0, 0};

  // barrier in the middle of tile T's second block: tile T + 1 has landed for every wave (its
  // loads were all issued before tile T + 2's 8) and nobody reads the stage of tile T - 1 any more
  auto mid_for = [&](int T) {
    return [&, T]() {
      if (__builtin_expect(T + 1 >= nt, 0)) return;
      __builtin_amdgcn_s_waitcnt(kWaitVm8);
      __builtin_amdgcn_s_barrier();
    };
  };
  // the tile whose bytes a load for tile X fetches (see above)
  auto load_tile = [&](int X) { return X < nt ? X : (X >= 4 ? X - 4 : X); };
  auto nothing = []() {};

  // one 64-key tile (blocks 2T and 2T + 1) with its stages fixed at compile time
  auto run_tile = [&](auto st_tag, int T) {
    constexpr int ST = decltype(st_tag)::value;
    char* const kc = KS[ST];                               // K/V of tile T
    char* const vc = VS[ST];
    char* const vp = VS[(ST + kStages - 1) % kStages];     // V of tile T - 1
    char* const kn = KS[(ST + 1) % kStages];               // K of tile T + 1
    char* const k2 = KS[(ST + 2) % kStages];               // tile T + 2 (loads 3..7 now)
    char* const v2 = VS[(ST + 2) % kStages];
    char* const k3 = KS[(ST + 3) % kStages];               // tile T + 3 (loads 0..2 now)
    char* const v3 = VS[(ST + 3) % kStages];
    const int k0 = kt0 + T * kBN;
    const int kt2 = kt0 + load_tile(T + 2) * kBN, kt3 = kt0 + load_tile(T + 3) * kBN;
    // loads 3..7 of tile T + 2 spread over block 2T (stretches 1a, 1a, 2a, 2a, 2b), loads 0..2
    // of tile T + 3 over the stretches of block 2T + 1 after its barrier (2a, 2b, 2b)
    auto hook0 = [&](int st, int slot) {
      if (st == 0 && slot == 1) dma.issue_part_unclamped(k2, v2, kt2, 3);
      if (st == 0 && slot == 5) dma.issue_part_unclamped(k2, v2, kt2, 4);
      if (st == 2 && slot == 1) dma.issue_part_unclamped(k2, v2, kt2, 5);
      if (st == 2 && slot == 5) dma.issue_part_unclamped(k2, v2, kt2, 6);
      if (st == 3 && slot == 3) dma.issue_part_unclamped(k2, v2, kt2, 7);
    };
    auto hook1 = [&](int st, int slot) {
      if (st == 2 && slot == 3) dma.issue_part_unclamped(k3, v3, kt3, 0);
      if (st == 3 && slot == 1) dma.issue_part_unclamped(k3, v3, kt3, 1);
      if (st == 3 && slot == 5) dma.issue_part_unclamped(k3, v3, kt3, 2);
    };
    auto mid = mid_for(T);
    const int i = 2 * T;
    if (__builtin_expect(i < nblk, 1)) {
      wide_iter<D, true>(w, p, vp + 32 * G::kRow, kc + 32 * G::kRow, k0, i >= nunm, h, c,
                         a_inv_c, nothing, hook0);
    } else {
#pragma unroll
      for (int j = 3; j < kParts; ++j) dma.issue_part_unclamped(k2, v2, kt2, j);
    }
    if (__builtin_expect(i + 1 < nblk, 1)) {
      wide_iter<D, false>(w, p, vc, kn, k0 + 32, i + 1 >= nunm, h, c, a_inv_c, mid, hook1);
    } else {
      mid();
#pragma unroll
      for (int j = 0; j < 3; ++j) dma.issue_part_unclamped(k3, v3, kt3, j);
    }
  };

  for (int T = 0; T < nt; T += kStages) {
    run_tile(std::integral_constant<int, 0>{}, T);
    if (__builtin_expect(T + 1 >= nt, 0)) break;
    run_tile(std::integral_constant<int, 1>{}, T + 1);
    if (__builtin_expect(T + 2 >= nt, 0)) break;
    run_tile(std::integral_constant<int, 2>{}, T + 2);
    if (__builtin_expect(T + 3 >= nt, 0)) break;
    run_tile(std::integral_constant<int, 3>{}, T + 3);
  }
  // The last block's pending work. Its V tile (tile (nblk - 1) / 2, within the last 4 tiles
  // of the workgroup: a wave's rows end at most 192 rows before the workgroup's) is never
  // overwritten, and every load has completed by now.
  if (nblk > 0) {
    const int tl = (nblk - 1) >> 1;
    const int st = tl % kStages;
    const char* vl = st == 0 ? VS[0] : st == 1 ? VS[1] : st == 2 ? VS[2] : VS[3];
    // (the last block wrote slot 0 if it was even, else slot 1)
    if ((nblk - 1) & 1) wide_drain<D, 1>(w, p, vl + 32 * G::kRow, c);
    else wide_drain<D, 0>(w, p, vl, c);
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm0);   // (no load may still be writing LDS at the end)

  // ---- epilogue: normalise O and stage it as rows in the wave's K stage (at the barrier every
  //      wave is past its last read of the K stages, and every load has landed), then store
  //      whole rows ----
  static_assert(kWideRows * G::kRow == G::kTile, "a wave's rows of O fill one K stage");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  char* const os = wave == 0 ? KS[0] : wave == 1 ? KS[1] : wave == 2 ? KS[2] : KS[3];
  float l_tot[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    l_tot[g] = xor32_sum(w.l[g]);
    stage_o_group<D>(os, 32 * g, w.o[g], (l_tot[g] > 0.f) ? 1.f / l_tot[g] : 0.f, h, l32);
  }
  const int nvalid = min(kWideRows, a.Sq - qw);
  if (SPLIT) {
    // ---- partial result: this key range's own output (bf16), reference max (base 2,
    //      scaled) and sum ----
    const size_t prow0 =
        (size_t)split * a.B * a.Hq * a.Sq + (size_t)(b * a.Hq + hq) * a.Sq + qw;
    store_staged_rows<D, kWideRows>(a.part_o + prow0 * D, D, os, nvalid, lane);
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int r = 32 * g + l32;
      if (r < nvalid && h == 0)
        *reinterpret_cast<f32x2*>(a.part_ml + (prow0 + r) * 2) =
            f32x2{l_tot[g] > 0.f ? w.m[g] : -INFINITY, l_tot[g]};
    }
    return;
  }
  const size_t orow0 = (size_t)(b * a.Hq + hq) * a.Sq + qw;
  store_staged_rows<D, kWideRows>(a.o + orow0 * D, D, os, nvalid, lane);
  // LSE (natural log)
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int r = 32 * g + l32;
    if (r < nvalid && a.lse != nullptr && h == 0) {
      const float lse = (l_tot[g] > 0.f) ? (w.m[g] + log2_fast(l_tot[g])) * kLn2 : -INFINITY;
      a.lse[orow0 + r] = lse;
    }
  }
}

// Claims the last unclaimed item of another XCD (one lane; a.nitems when nothing is left). The
// claim block holds per XCD x a word at 16 * x counting this launch's claims from the back of
// x's order, at 16 * 8 the launch's "nothing left" mark, and from kClaimHead on a mark per item.
// Launch marks grow from launch to launch, so an item mark below a.epoch is unclaimed; owners
// raise it to a.epoch and takers to a.epoch + 1, with an atomic maximum, so a mark never lowers
// another (a taker that finds the owner there leaves the owner's claim as it is). A counter word
// carries the launch (a.epoch / 2) in its upper half; the first claim of a launch finds an
// earlier launch's there and restarts it.
__device__ __forceinline__ int wide_take(const FwdArgs& a, int xs) {
  unsigned long long* const ctr = a.claim;
  if (__hip_atomic_load(ctr + 16 * 8, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.epoch)
    return a.nitems;
  const unsigned long long launch = a.epoch >> 1;
  for (int j = 1; j < 8; ++j) {
    const int x = (xs + j) & 7;
    const int cnt = (a.nitems - x + 7) >> 3;   // items of XCD x
    unsigned long long w = atomicAdd(ctr + 16 * x, 1ull);
    long long b;
    if ((w >> 32) == (launch & 0xffffffffull)) {
      b = (long long)(w & 0xffffffffull);
    } else {
      const unsigned long long fresh = ((launch & 0xffffffffull) << 32) | 1ull;
      if (atomicCAS(ctr + 16 * x, w + 1, fresh) == w + 1) {
        b = 0;
      } else {
        w = atomicAdd(ctr + 16 * x, 1ull);
        if ((w >> 32) != (launch & 0xffffffffull)) continue;   // (left to others)
        b = (long long)(w & 0xffffffffull);
      }
    }
    if (b >= cnt) continue;
    const int id = x + 8 * (cnt - 1 - (int)b);
    if (atomicMax(a.claim + kClaimHead + id, a.epoch | 1ull) < a.epoch) return id;
    // its owner has it: XCD x's owners have reached the back of its order
  }
  atomicExch(ctr + 16 * 8, a.epoch);
  return a.nitems;
}

// The wide kernel's workgroups, one item each. Items are workgroups 0 .. nitems - 1; with a
// claim block, the workgroups past them each take the last unclaimed item of another XCD, or
// end at once when none is left. They are dispatched after all of their own XCD's items, so
// they start as that XCD finishes its share: under this load the XCDs run at clocks up to
// several percent apart, and the faster ones then take over the slower ones' last (lightest)
// items. (Each takes one item: a loop over items here would be a second copy of the item code,
// and with two copies the compiler lays out the tile loop less well.)
template <int D, bool CAUSAL, bool SPLIT>
__device__ __forceinline__ void fwd_wide_body(const FwdArgs& a) {
  int id = blockIdx.x;
  const bool taker = !SPLIT && a.claim != nullptr && id >= a.nitems;
  if (taker) {
    __shared__ int s_take;
    if (threadIdx.x == 0) s_take = wide_take(a, blockIdx.x & 7);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    id = s_take;
    if (id >= a.nitems) return;
  }
  wide_item_body<D, CAUSAL, SPLIT>(a, id, !SPLIT && a.claim != nullptr && !taker);
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fwd_bf16_d128_causal_wide(FwdArgs a) { fwd_wide_body<128, true, false>(a); }
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fwd_bf16_d128_wide(FwdArgs a) { fwd_wide_body<128, false, false>(a); }
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fwd_bf16_d128_causal_wide_split(FwdArgs a) { fwd_wide_body<128, true, true>(a); }
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fwd_bf16_d128_wide_split(FwdArgs a) { fwd_wide_body<128, false, true>(a); }
__global__ __launch_bounds__(256) void fwd_bf16_d128_wide_split_combine(FwdArgs a) {
  fwd_split_combine_body<128>(a);
}

}  // namespace

hipError_t launch_fwd_bf16_wide(const FwdProblem& p, hipStream_t stream) {
  FwdArgs a{};
  a.q = static_cast<const uint16_t*>(p.q);
  a.k = static_cast<const uint16_t*>(p.k);
  a.v = static_cast<const uint16_t*>(p.v);
  a.o = static_cast<uint16_t*>(p.o);
  a.lse = p.lse;
  a.B = p.B; a.Hq = p.Hq; a.Hkv = p.Hkv; a.Sq = p.Sq; a.Sk = p.Sk;
  a.group = p.Hq / p.Hkv;
  a.ntq = (p.Sq + kWideBM - 1) / kWideBM;
  float c = p.scale * kLog2e;
  if (!(c > 0.f)) c = 1.17549435e-38f;   // scale 0: uniform weights, -inf * c stays -inf
  a.c = c;
  a.nsplit = p.nsplit > 1 ? p.nsplit : 1;
  const long long nwg = (long long)a.ntq * a.nsplit * p.B * p.Hq;
  if (nwg == 0) return hipSuccess;
  if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  a.nitems = (int)nwg;
  if (a.nsplit > 1) {
    // the key ranges of each query tile, then their merge (workspace as for the other forward
    // kernels' splits: fwd_bf16_workspace_bytes)
    const size_t nrows = (size_t)p.B * p.Hq * p.Sq;
    a.part_o = static_cast<uint16_t*>(p.workspace);
    a.part_ml = reinterpret_cast<float*>(a.part_o + (size_t)a.nsplit * nrows * p.D);
    dim3 grid((unsigned)nwg), block(256);
    if (p.causal) hipLaunchKernelGGL(fwd_bf16_d128_causal_wide_split, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(fwd_bf16_d128_wide_split, grid, block, 0, stream, a);
    const int rows_per_block = 256 / (p.D / 4);
    dim3 cgrid((unsigned)((nrows + rows_per_block - 1) / rows_per_block)), cblock(256);
    hipLaunchKernelGGL(fwd_bf16_d128_wide_split_combine, cgrid, cblock, 0, stream, a);
    return hipGetLastError();
  }
  // with a claim block, kTakers workgroups per XCD after the items take over other XCDs' last
  // items (those that find none end at once)
  a.claim = p.claim;
  a.epoch = p.epoch;
  const long long ngrid = nwg + (a.claim != nullptr ? 8 * kTakers : 0);
  if (ngrid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  dim3 grid((unsigned)ngrid), block(256);
  if (p.causal) hipLaunchKernelGGL(fwd_bf16_d128_causal_wide, grid, block, 0, stream, a);
  else hipLaunchKernelGGL(fwd_bf16_d128_wide, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace attn

// Fused exact-attention forward for bf16 Q/K/V on gfx950: O = softmax(scale * Q K^T + mask) V
// and the per-row log-sum-exp, in one pass over K/V with an online softmax, so no score or
// probability matrix ever reaches HBM ("Fused Kernel Compiler" (Candle paper), §FlashAttention
// Integration: tile Q, K, V on chip; scores, softmax and the weighted sum in a single pass;
// online softmax; O(N) memory).
//
// Queries are cut into 128-row tiles and each wave owns 32 rows of a tile. Query head h reads
// KV head h / (Hq / Hkv) (grouped-query attention). Two work mappings share the tile code:
//
//  * Tile kernel: a workgroup of 4 waves per (batch, query head, tile), two workgroups per CU.
//    With a causal mask tiles are issued heaviest first, which balances the CUs when there are
//    many more workgroups than CU slots (long sequences).
//  * Pair kernel (causal launches with few tiles per head, where one round of workgroups would
//    be set by its heaviest tile): a workgroup of 8 waves, one per CU, takes the pair of tiles
//    (p, T-1-p), a light one that sees few keys and a heavy one that sees many, and splits it
//    so that all 8 waves do the same number of K/V tiles: waves 4..7 ("H") take the heavy
//    tile's rows over the first x key tiles; waves 0..3 ("L") take the light tile's rows over
//    the same key tiles (loaded once for both), then the heavy tile's rows over the remaining
//    key tiles, last tile first. At the end each L wave hands its partial softmax state to the
//    H wave with the same rows through LDS, where the two are merged with the online-softmax
//    rescaling. Every workgroup then does about the same work. Work items of one KV head are
//    placed on one XCD so they share its L2. Each wave software-pipelines its 32-key blocks
//    (scores of one block, softmax of the previous, product with V of the one before, in one
//    stretch of code) and the L waves issue all the direct loads (see the pipelined pair body).
//
// Each wave works on the transposed problem so that the softmax runs inside each lane:
//   S^T[key][q] = K[key][:] . Q[q][:]        (MFMA 32x32x16: A = K from LDS, B = Q^T in VGPRs)
//   O^T[d][q]  += V^T[d][key] P^T[key][q]    (MFMA 32x32x16: A = V^T from LDS, B = P^T in VGPRs)
// A lane's accumulator column is one query, so the running max and sum are per lane: a row max
// needs one exchange with lane l^32 (v_permlane32_swap), and P^T leaves the first product's
// accumulators in exactly the B-operand layout of the second (no LDS round trip).
//
// K/V staging: tiles of 64 keys go from global memory straight into LDS with direct-to-LDS
// buffer loads (each lane's 16 bytes land at base + 16*lane), double buffered (the pair kernel
// keeps a second stream for the heavy tail). Rows are stored unpadded with their 16-byte chunks
// XOR-permuted; each lane fetches the global chunk that belongs in its LDS slot. The K
// permutation (chunk ^ row%16) makes the row-per-lane ds_read_b128 operand reads conflict-free;
// V stays row-major and its V^T operand comes from the transposing read ds_read_b64_tr_b16
// (each group of 16 lanes turns 4 keys x 16 columns into 16 lanes x 4 keys), with the V
// permutation (chunk ^ 4*(row%4)) spreading those reads over all banks.
//
// Softmax: base 2 with scale*log2(e) folded into one FMA per score. The running reference
// max is only moved when a row's max exceeds it by more than 2^8 (lazy rescale): until then
// the probabilities are at most 256, far from overflow, and the result is the same up to
// rounding, while the O accumulators are rescaled only a handful of times per row.
//
// Causal masking is bottom-right aligned (key j visible to query i iff j <= i + Sk - Sq);
// tiles wholly above a wave's diagonal are skipped by that wave, and tiles no row of the
// workgroup sees are never loaded.
#include "fwd_tiles.hpp"

namespace attn {
namespace {

using namespace cdna4;

constexpr int kWideRows = 256;     // query rows per workgroup of the wide kernel
// Pair kernel is used for causal launches with at most this many tiles per head.
constexpr int kPairMaxTiles = 64;
// Most key-range splits per query tile (the split path serves few-tile problems, such as a
// prefill chunk against a long prefix, whose query tiles alone would leave CUs idle).
constexpr int kMaxFwdSplits = 8;

// SPLIT: the workgroup covers one of a.nsplit contiguous ranges of the query tile's key tiles
// and writes that range's own output (bf16, normalised by the range's sum), reference max and
// sum to the workspace; the split combine kernel merges the ranges. Otherwise it covers all
// the tile's keys.
template <int D, bool CAUSAL, bool SPLIT>
__device__ __forceinline__ void fwd_tile_body(const FwdArgs& a) {
  using G = Geo<D, 4>;
  // two stages, each a K tile and a V tile; separate objects so the compiler can tell the
  // in-flight direct loads into one stage from the reads of the other
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

  // ---- work item: heaviest tiles first, all heads of one rank together ----
  const int BH = a.B * a.Hq;
  const int id = blockIdx.x;
  const int unit = id / BH;                // rank * nsplit + split
  const int bh = id - unit * BH;
  const int rank = SPLIT ? unit / a.nsplit : unit;
  const int split = SPLIT ? unit - rank * a.nsplit : 0;
  const int tile = CAUSAL ? (a.ntq - 1 - rank) : rank;
  const int b = bh / a.Hq;
  const int hq = bh - b * a.Hq;
  const int hk = hq / a.group;
  const int q0 = tile * kBM;
  const int qw = q0 + wave * 32;           // first query of this wave
  const int off = a.Sk - a.Sq;             // causal diagonal offset

  const uint16_t* qbase = a.q + ((size_t)(b * a.Hq + hq) * a.Sq) * D;
  const uint16_t* kbase = a.k + ((size_t)(b * a.Hkv + hk) * a.Sk) * D;
  const uint16_t* vbase = a.v + ((size_t)(b * a.Hkv + hk) * a.Sk) * D;

  // ---- keys this workgroup visits ----
  int kv_end = a.Sk;
  if (CAUSAL) kv_end = min(a.Sk, max(0, q0 + kBM + off));
  const int nall = (kv_end + kBN - 1) / kBN;
  // this workgroup's key tiles [t0, t0 + ntiles)
  const int t0 = SPLIT ? split * nall / a.nsplit : 0;
  const int ntiles = SPLIT ? (split + 1) * nall / a.nsplit - t0 : nall;

  WaveState<D> w;
  {
    const int qi = qw + l32;
#pragma unroll
    for (int kk = 0; kk < G::KS; ++kk) {
      if (qi < a.Sq)
        w.qf[kk] = *reinterpret_cast<const u32x4*>(qbase + (size_t)qi * D + kk * 16 + h * 8);
      else
        w.qf[kk] = u32x4{0, 0, 0, 0};
    }
  }
#pragma unroll
  for (int i = 0; i < G::DB; ++i) w.o[i] = f32x16{};
  w.mref = -INFINITY;
  w.l_run = 0.f;
  // K operand: row l32 (+32kb), chunk 2kk+h at its permuted slot
#pragma unroll
  for (int kk = 0; kk < G::KS; ++kk)
    w.koff[kk] = l32 * G::kRow + (((2 * kk + h) ^ kswz<D>(l32)) * 16);
  // V^T operand via transposed reads: source lane (group g, index j) points at key
  // 4*(g/2) + j/4 (+ the block's first key) and columns 32db + 16*(g%2) + 4*(j%4) .. +3
  {
    const int g = lane >> 4, j = lane & 15;
    const int keyl = 4 * (g >> 1) + (j >> 2);
    const int small = 2 * (g & 1) + ((j & 3) >> 1);
#pragma unroll
    for (int db = 0; db < G::DB; ++db)
      w.voff[db] = keyl * G::kRow + (((4 * db + small) ^ vswz<D>(keyl)) * 16) + 8 * (j & 1);
  }
  const float c = a.c;
  const int my_q = qw + l32;
  const int wave_last_key = qw + 31 + off;   // last key any query of this wave may see

  TileDma<D, 4> dma;
  dma.init(wave, lane, kbase, vbase, a.Sk);
  if (ntiles > 0) dma.issue(sk0, sv0, t0 * kBN, a.Sk);
  wait_dma_and_barrier();
  // Q and the first tile were in flight together. Consume the Q loads here, where they have
  // landed: otherwise the loop's first use of qf waits for every load in flight then,
  // including the next tile's prefetch.
  consume_q(w);

  for (int j = 0; j < ntiles; j += 2) {
    const int kt = (t0 + j) * kBN;
    // stage 0 holds tile j; prefetch tile j+1 into stage 1
    if (j + 1 < ntiles) dma.issue(sk1, sv1, kt + kBN, a.Sk);
    compute_tile<D, CAUSAL>(w, sk0, sv0, kt, a.Sk, qw, wave_last_key, my_q, off, h, c);
    wait_dma_and_barrier();
    if (j + 1 >= ntiles) break;
    // stage 1 holds tile j+1; prefetch tile j+2 into stage 0
    if (j + 2 < ntiles) dma.issue(sk0, sv0, kt + 2 * kBN, a.Sk);
    compute_tile<D, CAUSAL>(w, sk1, sv1, kt + kBN, a.Sk, qw, wave_last_key, my_q, off, h, c);
    wait_dma_and_barrier();
  }

  if (SPLIT) {
    // ---- partial result: this key range's own output (bf16), reference max (base 2,
    //      scaled) and sum ----
    const float l_tot = xor32_sum(w.l_run);
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    const size_t prow = (size_t)split * BH * a.Sq + (size_t)bh * a.Sq + min(my_q, a.Sq - 1);
    store_o_group<G::DB>(a.part_o + prow * D, w.o, inv, h, my_q < a.Sq);
    if (my_q < a.Sq && h == 0)
      *reinterpret_cast<f32x2*>(a.part_ml + prow * 2) =
          f32x2{l_tot > 0.f ? w.mref : -INFINITY, l_tot};
    return;
  }

  // ---- epilogue: normalise, store O (bf16) and LSE (natural log) ----
  const float l_tot = xor32_sum(w.l_run);
  const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  store_o_group<G::DB>(a.o + ((size_t)(b * a.Hq + hq) * a.Sq + min(my_q, a.Sq - 1)) * D, w.o,
                       inv, h, my_q < a.Sq);
  if (my_q < a.Sq) {
    if (a.lse != nullptr && h == 0) {
      const float lse = (l_tot > 0.f) ? (w.mref + log2_fast(l_tot)) * kLn2 : -INFINITY;
      a.lse[(size_t)(b * a.Hq + hq) * a.Sq + my_q] = lse;
    }
  }
}

// ---- software-pipelined pair kernel ----
// Each 32-key block of a wave's rows passes three phases: its scores S^T = K Q^T (matrix
// cores), its softmax (vector ALU: max, exponentials, bf16 P^T) and its product O^T += V^T P^T
// (matrix cores). Slot t runs the scores of block t, the softmax of block t-1 and the product
// of block t-2: the three are independent, so the exponentials issue between the matrix-core
// instructions of the same wave instead of after them (on gfx950 a wave's own interleaved
// vector work hides under its matrix-core work far better than the other wave's does).
// The two blocks of the key tile at step j are slots (j, 0) and (j, 1); both products in step
// j are of tile j - 1, so a step reads K of tile j and V of tile j - 1, and the V tile is
// loaded one step after its K tile, into the other stage.

template <int D>
struct Pipe {
  f32x16 s;       // scores of the block waiting for its softmax
  u32x4 pb[2];    // P^T (bf16) of the block waiting for its product with V
  int s_k0;       // first key of the block in s
  bool has_s;
  bool has_p;
  bool pv_b;      // the block in pb is from the second K/V stream
};

// Mask the block in p.s, take its row max and move the reference if needed (rescaling O, the
// running sum and the P^T still waiting for its product, all relative to the old reference).
// Returns the reference to subtract (0 while it is still -inf).
template <int D, bool CAUSAL>
__device__ __forceinline__ float pipe_prep(WaveState<D>& w, Pipe<D>& p, int Sk, int qw, int off,
                                           int l32, int h, float c) {
  using G = Geo<D, 4>;
  const int k0 = p.s_k0;
  const bool need_mask = (k0 + 32 > Sk) || (CAUSAL && k0 + 31 > qw + off);
  if (need_mask) {
    const int my_q = qw + l32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = k0 + 8 * (r >> 2) + 4 * h + (r & 3);
      bool vis = key < Sk;
      if (CAUSAL) vis = vis && (key <= my_q + off);
      p.s[r] = vis ? p.s[r] : -INFINITY;
    }
  }
  // (a tree: three dependent steps instead of eight)
  const float m0 = fmax3(p.s[0], p.s[1], p.s[2]), m1 = fmax3(p.s[3], p.s[4], p.s[5]);
  const float m2 = fmax3(p.s[6], p.s[7], p.s[8]), m3 = fmax3(p.s[9], p.s[10], p.s[11]);
  const float m4 = fmax3(p.s[12], p.s[13], p.s[14]);
  float mx = fmax3(fmax3(m0, m1, m2), fmax3(m3, m4, p.s[15]), -INFINITY);
  mx = xor32_max(mx);
  const float mxc = mx * c;
  const bool move = mxc > w.mref + kLazy;
  if (__builtin_amdgcn_ballot_w64(move)) {
    asm volatile("");
    const float alpha = move ? exp2_fast(w.mref - mxc) : 1.f;
    w.mref = move ? mxc : w.mref;
    w.l_run *= alpha;
#pragma unroll
    for (int i = 0; i < G::DB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) w.o[i][r] *= alpha;
    if (p.has_p) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t u = p.pb[t][e];
          p.pb[t][e] = pack_bf16x2(bf16lo_to_f32(u) * alpha, bf16hi_to_f32(u) * alpha);
        }
    }
  }
  return (w.mref == -INFINITY) ? 0.f : w.mref;
}

// One slot: with QK the scores of the 32-key block at kblk (K rows in LDS) into p.s; with EX the
// softmax of the block in p.s (reference mu) into p.pb; with PV, O^T += V^T P^T for the block in
// p.pb, whose V rows start at vblk. The matrix-core instructions of the scores and of the product
// alternate, with one group of exponentials after each pair.
template <int D, bool QK, bool EX, bool PV>
__device__ __forceinline__ void pipe_slot(WaveState<D>& w, Pipe<D>& p, const char* kblk,
                                          const char* vblk, float c, float mu) {
  using G = Geo<D, 4>;
  constexpr int KS = G::KS;            // score k-steps
  constexpr int NP = 2 * G::DB;        // product instructions (as many as score k-steps)
  static_assert(KS == NP, "one score and one product instruction per step");
  constexpr int NM = KS;
  // (a compiler barrier: the next slot's operand reads would otherwise be hoisted into this
  //  one, which doubles the live fragments and undoes the schedule below)
  asm volatile("" ::: "memory");
  u32x4 kf[KS];
  u32x4 vf[NP];
  if (QK) {
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) kf[kk] = *reinterpret_cast<const u32x4*>(kblk + w.koff[kk]);
  }
  if (PV) {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int db = i >> 1, t = i & 1;
      const char* vp = vblk + w.voff[db] + 16 * t * G::kRow;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vp));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vp + 8 * G::kRow));
      const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
      const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
      vf[i] = u32x4{l2[0], l2[1], h2[0], h2[1]};
    }
  }
  f32x16 sn;
  u32x4 pn[2];
  float ls0 = 0.f, ls1 = 0.f;
  // the score products first, so that the next slot's max finds them complete; the products
  // with V after them; the 8 exponential items spread over all of them
  constexpr int NI = (QK ? NM : 0) + (PV ? NM : 0);
#pragma unroll
  for (int i = 0; i < (NI > 0 ? NI : 1); ++i) {
    if (QK && i < NM) sn = mfma32x32x16(kf[i], w.qf[i], i == 0 ? f32x16{} : sn);
    const int ip = QK ? i - NM : i;
    if (PV && ip >= 0 && ip < NM) w.o[ip >> 1] = mfma32x32x16(vf[ip], p.pb[ip & 1], w.o[ip >> 1]);
    if (EX) {
#pragma unroll
      for (int it = NI > 0 ? (8 * i) / NI : 0; it < (NI > 0 ? (8 * (i + 1)) / NI : 8); ++it) {
        const int t = it >> 2, e = it & 3;
        const float p0 = exp2_fast(__builtin_fmaf(p.s[8 * t + 2 * e], c, -mu));
        const float p1 = exp2_fast(__builtin_fmaf(p.s[8 * t + 2 * e + 1], c, -mu));
        ls0 += p0;
        ls1 += p1;
        pn[t][e] = pack_bf16x2(p0, p1);
      }
    }
  }
  if (EX) {
    w.l_run += ls0 + ls1;
    p.pb[0] = pn[0];
    p.pb[1] = pn[1];
  }
  if (QK) p.s = sn;
  // Schedule: every LDS operand read first (they complete in order while the first products
  // run), then per step its matrix-core instructions followed by its vector work. (Group masks:
  // 0x100 LDS read, 0x008 matrix core, 0x002 vector ALU.)
  constexpr int NDS = (QK ? KS : 0) + (PV ? 2 * NP : 0);
  // 7 vector instructions per exponential item (2 FMA, 2 exp, 2 adds, 1 pack): 56 over NI
  // matrix-core instructions, alternately rounded down and up
  __builtin_amdgcn_sched_group_barrier(0x100, NDS, 0);
  constexpr int VA = NI > 0 ? (112 / NI + 1) / 2 : 0, VB = NI > 0 ? 112 / NI - VA : 0;
#pragma unroll
  for (int i = 0; i < NI; i += 2) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (EX) __builtin_amdgcn_sched_group_barrier(0x002, VA, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (EX) __builtin_amdgcn_sched_group_barrier(0x002, VB, 0);
  }
}

template <int D, bool CAUSAL>
__device__ __forceinline__ void fwd_pair_pipe_body(const FwdArgs& a) {
  using G = Geo<D, 8>;
  // K stages k?0 / k?1 and V stages v?0 / v?1 of streams a and b; at step j the wave reads K
  // stage j % 2 and V stage (j - 1) % 2 while K of step j + 1 and V of step j load into the
  // other two (separate objects, so the compiler tells the in-flight direct loads apart)
  __shared__ __attribute__((aligned(1024))) char ka0[G::kTile];
  __shared__ __attribute__((aligned(1024))) char va0[G::kTile];
  __shared__ __attribute__((aligned(1024))) char ka1[G::kTile];
  __shared__ __attribute__((aligned(1024))) char va1[G::kTile];
  __shared__ __attribute__((aligned(1024))) char kb0[G::kTile];
  __shared__ __attribute__((aligned(1024))) char vb0[G::kTile];
  __shared__ __attribute__((aligned(1024))) char kb1[G::kTile];
  __shared__ __attribute__((aligned(1024))) char vb1[G::kTile];
  __shared__ float xml[4][2][64];     // hand-over of (mref, l_run) from the L waves
  {
    char* const st[8] = {ka0, va0, ka1, va1, kb0, vb0, kb1, vb1};
#pragma unroll
    for (int i = 0; i < 8; ++i) lds_poison(st[i], G::kTile);
    lds_poison(xml, sizeof(xml));
    lds_poison_done();
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_uniform(tid >> 6);
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const bool lwave = wave < 4;
  const int wr = wave & 3;

  const int item = xcd_item(blockIdx.x, a.nitems);
  const int pair = item % a.npairs;
  const int bh = item / a.npairs;
  const int b = bh / a.Hq;
  const int hq = bh - b * a.Hq;
  const int hk = hq / a.group;
  int tl, th;
  bool single;
  if (CAUSAL) {
    tl = pair;
    th = a.ntq - 1 - pair;
    single = tl == th;
  } else {
    tl = 2 * pair;
    th = 2 * pair + 1;
    single = th >= a.ntq;
  }
  if (single) th = tl;
  const int off = a.Sk - a.Sq;

  auto tiles_for = [&](int t) -> int {
    const int last = min(t * kBM + kBM, a.Sq) - 1;
    int kend = a.Sk;
    if (CAUSAL) kend = min(a.Sk, max(0, last + off + 1));
    return (kend + kBN - 1) / kBN;
  };
  const int nH = tiles_for(th);
  const int nL = single ? 0 : tiles_for(tl);
  const int x = (nL + nH + 1) / 2;       // steps with a key tile; step x only drains
  const int nB = nH - x;

  const uint16_t* qbase = a.q + ((size_t)(b * a.Hq + hq) * a.Sq) * D;
  const uint16_t* kbase = a.k + ((size_t)(b * a.Hkv + hk) * a.Sk) * D;
  const uint16_t* vbase = a.v + ((size_t)(b * a.Hkv + hk) * a.Sk) * D;

  WaveState<D> w;
#pragma unroll
  for (int kk = 0; kk < G::KS; ++kk)
    w.koff[kk] = l32 * G::kRow + (((2 * kk + h) ^ kswz<D>(l32)) * 16);
  {
    const int g = lane >> 4, jj = lane & 15;
    const int keyl = 4 * (g >> 1) + (jj >> 2);
    const int small = 2 * (g & 1) + ((jj & 3) >> 1);
#pragma unroll
    for (int db = 0; db < G::DB; ++db)
      w.voff[db] = keyl * G::kRow + (((4 * db + small) ^ vswz<D>(keyl)) * 16) + 8 * (jj & 1);
  }
  const float c = a.c;

  // O and the softmax state reset for new rows
  auto reset_rows = [&]() {
#pragma unroll
    for (int i = 0; i < G::DB; ++i) w.o[i] = f32x16{};
    w.mref = -INFINITY;
    w.l_run = 0.f;
  };
  // Q of 32 rows from qw straight into the fragments (one row per lane; rows past Sq zero)
  auto load_q = [&](int qw) {
    const int qi = qw + l32;
#pragma unroll
    for (int kk = 0; kk < G::KS; ++kk) {
      if (qi < a.Sq)
        w.qf[kk] = *reinterpret_cast<const u32x4*>(qbase + (size_t)qi * D + kk * 16 + h * 8);
      else
        w.qf[kk] = u32x4{0, 0, 0, 0};
    }
  };
  auto store_rows = [&](int qw) {
    const int my_q = qw + l32;
    const float l_tot = xor32_sum(w.l_run);
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    store_o_group<G::DB>(a.o + ((size_t)(b * a.Hq + hq) * a.Sq + min(my_q, a.Sq - 1)) * D,
                         w.o, inv, h, my_q < a.Sq);
    if (my_q < a.Sq) {
      if (a.lse != nullptr && h == 0) {
        const float lse = (l_tot > 0.f) ? (w.mref + log2_fast(l_tot)) * kLn2 : -INFINITY;
        a.lse[(size_t)(b * a.Hq + hq) * a.Sq + my_q] = lse;
      }
    }
  };

  const int qlight = tl * kBM + 32 * wr;
  const int qheavy = th * kBM + 32 * wr;
  int qw;
  if (lwave && !single) {
    qw = qlight;
    reset_rows();
    if (nL == 0) {
      store_rows(qw);
      qw = qheavy;
      reset_rows();
    }
  } else {
    qw = qheavy;
    reset_rows();
  }
  // The first rows' Q passes through LDS, with whole rows per load (one row per lane would
  // touch each row's bytes in 32-byte pieces): wave w's 32 rows go to half w % 2 of the V stage
  // of steps 0 and 1 (va0, vb0, va1, vb1 for w / 2 = 0..3), which no load uses before the loop,
  // in the K tiles' layout, so that the fragments are read with the K operand offsets. Rows
  // past Sq load row Sq - 1: they are computed like it, and never stored. (The loads are
  // assembly, which the compiler does not track: the wait before the loop covers them.)
  constexpr int kQBytes = 32 * G::kRow;
  static_assert(2 * kQBytes == G::kTile, "two waves' rows per stage");
  {
    char* const qs = (wave < 2 ? va0 : wave < 4 ? vb0 : wave < 6 ? va1 : vb1) +
                     (wave & 1) * kQBytes;
    const int rb = min(qw, a.Sq - 1);               // first row loaded
    const u32x4 rq = raw_rsrc(qbase + (size_t)rb * D, kQBytes);
    const int pos = lane % G::kCPR;
    const int rsub = lane / G::kCPR;
#pragma unroll
    for (int i = 0; i < kQBytes / 1024; ++i) {
      const int r = i * G::kRPI + rsub;             // row among the wave's 32
      const int src = min(qw + r, a.Sq - 1) - rb;
      lds_dma16(rq, lds_addr(qs) + i * 1024, src * G::kRow + ((pos ^ kswz<D>(r)) * 16));
    }
  }

  Pipe<D> p;
  p.has_s = false;
  p.has_p = false;
  p.pv_b = false;
  p.s_k0 = 0;

  // The L waves issue all the direct loads: issued by all eight waves right after a barrier
  // they queue behind each other for ~600 cycles, which the L waves (lighter per step) absorb
  // while the H waves go straight to their matrix-core work.
  TileDma<D, 4> dma;
  dma.init(wr, lane, kbase, vbase, a.Sk);
  // key tile of stream b at step j (the heavy rows' tail, walked from its end)
  auto ktb = [&](int j) { return (nH + nL - 1 - j) * kBN; };
  auto in_b = [&](int j) { return j >= nL && j - nL < nB; };
  // loads started at step j: K of step j + 1 and V of step j
  auto dma_step = [&](int j, char* kan, char* kbn, char* vac, char* vbc) {
    if (!lwave) return;
    if (j + 1 < x) dma.issue_one(false, kan, (j + 1) * kBN, a.Sk);
    if (in_b(j + 1)) dma.issue_one(false, kbn, ktb(j + 1), a.Sk);
    if (j < x) dma.issue_one(true, vac, j * kBN, a.Sk);
    if (in_b(j)) dma.issue_one(true, vbc, ktb(j), a.Sk);
  };

  // finishes the block pipeline of the current rows (V of the last key tile in vprev)
  auto drain = [&](const char* vprev) {
    if (!p.has_s) return;
    const float mu = pipe_prep<D, CAUSAL>(w, p, a.Sk, qw, off, l32, h, c);
    pipe_slot<D, false, true, true>(w, p, nullptr, vprev, c, mu);
    pipe_slot<D, false, false, true>(w, p, nullptr, vprev + 32 * G::kRow, c, 0.f);
    p.has_s = false;
    p.has_p = false;
  };

  // the wave's work at step j: K of the step's tile in k{a,b}, V of the previous step's tile in
  // v{a,b}
  auto step = [&](int j, const char* kac, const char* kbc, const char* vap, const char* vbp) {
    int kt = -1;
    bool sb = false;
    if (j < x) {
      if (!lwave || j < nL) {
        kt = j * kBN;
      } else if (j - nL < nB) {
        kt = ktb(j);
        sb = true;
      }
    }
    const bool row_switch = lwave && !single && nL > 0 && j == nL;
    const int rows = row_switch ? qheavy : qw;
    const bool vis = kt >= 0 && (!CAUSAL || kt <= rows + 31 + off);
    if (p.has_s && (!vis || row_switch)) drain(p.pv_b ? vbp : vap);
    if (row_switch) {
      store_rows(qw);
      qw = qheavy;
      if (nB > 0) {
        reset_rows();
        load_q(qw);
        consume_q(w);
      }
    }
    if (!vis) return;
    const char* kt_lds = sb ? kbc : kac;
    const char* vp = p.pv_b ? vbp : vap;
    // slot (j, 0)
    if (p.has_s) {
      const float mu = pipe_prep<D, CAUSAL>(w, p, a.Sk, qw, off, l32, h, c);
      pipe_slot<D, true, true, true>(w, p, kt_lds, vp, c, mu);
    } else {
      pipe_slot<D, true, false, false>(w, p, kt_lds, nullptr, c, 0.f);
    }
    const bool had_p = p.has_s;          // a P^T of the previous tile is now waiting
    p.s_k0 = kt;
    p.has_s = true;
    // slot (j, 1)
    {
      const float mu = pipe_prep<D, CAUSAL>(w, p, a.Sk, qw, off, l32, h, c);
      if (had_p)
        pipe_slot<D, true, true, true>(w, p, kt_lds + 32 * G::kRow, vp + 32 * G::kRow, c, mu);
      else
        pipe_slot<D, true, true, false>(w, p, kt_lds + 32 * G::kRow, nullptr, c, mu);
    }
    p.s_k0 = kt + 32;
    p.has_p = true;
    p.pv_b = sb;
  };

  if (lwave && x > 0) dma.issue_one(false, ka0, 0, a.Sk);
  if (lwave && in_b(0)) dma.issue_one(false, kb0, ktb(0), a.Sk);
  wait_dma_and_barrier();
  // Q and the first K tile were in flight together. Each wave reads its fragments (its stage
  // named in a branch of its own, so that the reads carry that stage's alias information);
  // the loop's first loads overwrite va0 and vb0 once every wave is past the barrier.
  {
    auto q_read = [&](const char* st) {
#pragma unroll
      for (int kk = 0; kk < G::KS; ++kk)
        w.qf[kk] = *reinterpret_cast<const u32x4*>(st + (wave & 1) * kQBytes + w.koff[kk]);
    };
    if (wave < 2) q_read(va0);
    else if (wave < 4) q_read(vb0);
    else if (wave < 6) q_read(va1);
    else q_read(vb1);
    consume_q(w);
    __syncthreads();
  }
  for (int j = 0; j <= x; j += 2) {
    dma_step(j, ka1, kb1, va0, vb0);
    step(j, ka0, kb0, va1, vb1);
    wait_dma_and_barrier();
    if (j + 1 > x) break;
    dma_step(j + 1, ka0, kb0, va1, vb1);
    step(j + 1, ka1, kb1, va0, vb0);
    wait_dma_and_barrier();
  }

  if (nB > 0) {
    float* xo = reinterpret_cast<float*>(wr == 0 ? ka0 : wr == 1 ? va0 : wr == 2 ? ka1 : va1);
    if (lwave) {
#pragma unroll
      for (int db = 0; db < G::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) xo[(16 * db + r) * 64 + lane] = w.o[db][r];
      xml[wr][0][lane] = w.mref;
      xml[wr][1][lane] = w.l_run;
    }
    __syncthreads();
    if (!lwave) {
      const float m2 = xml[wr][0][lane], l2 = xml[wr][1][lane];
      const float mn = fmaxf(w.mref, m2);
      const float a1 = (w.mref == -INFINITY) ? 0.f : exp2_fast(w.mref - mn);
      const float a2 = (m2 == -INFINITY) ? 0.f : exp2_fast(m2 - mn);
      w.mref = mn;
      w.l_run = w.l_run * a1 + l2 * a2;
#pragma unroll
      for (int db = 0; db < G::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          w.o[db][r] = w.o[db][r] * a1 + xo[(16 * db + r) * 64 + lane] * a2;
    }
  }
  if (!lwave) {
    // the heavy rows leave through LDS as whole rows (stage_o_group), each wave's through the
    // stage it took the hand-over in, which no other wave reads; the loop ended with a barrier,
    // so no wave reads a stage any more and no load is writing one
    char* const os = wr == 0 ? ka0 : wr == 1 ? va0 : wr == 2 ? ka1 : va1;
    const float l_tot = xor32_sum(w.l_run);
    stage_o_group<D>(os, 0, w.o, (l_tot > 0.f) ? 1.f / l_tot : 0.f, h, l32);
    const size_t orow0 = (size_t)(b * a.Hq + hq) * a.Sq + qw;
    store_staged_rows<D, 32>(a.o + orow0 * D, D, os, a.Sq - qw, lane);
    if (qw + l32 < a.Sq && a.lse != nullptr && h == 0)
      a.lse[orow0 + l32] = (l_tot > 0.f) ? (w.mref + log2_fast(l_tot)) * kLn2 : -INFINITY;
  }
}

template <int D, bool CAUSAL>
__device__ __forceinline__ void fwd_tile_full(const FwdArgs& a) { fwd_tile_body<D, CAUSAL, false>(a); }
template <int D, bool CAUSAL>
__device__ __forceinline__ void fwd_tile_split(const FwdArgs& a) { fwd_tile_body<D, CAUSAL, true>(a); }

// Plain kernels (not kernel templates): their host-side launch stubs then depend only on these
// signatures.
#define ATTN_FWD_KERNEL(NAME, BODY, WAVES, D, CAUSAL)                      \
  __global__ __launch_bounds__(64 * WAVES)                                 \
  __attribute__((amdgpu_waves_per_eu(2, 2)))                               \
  void NAME(FwdArgs a) { BODY<D, CAUSAL>(a); }
ATTN_FWD_KERNEL(fwd_bf16_d128_causal, fwd_tile_full, 4, 128, true)
ATTN_FWD_KERNEL(fwd_bf16_d128, fwd_tile_full, 4, 128, false)
ATTN_FWD_KERNEL(fwd_bf16_d64_causal, fwd_tile_full, 4, 64, true)
ATTN_FWD_KERNEL(fwd_bf16_d64, fwd_tile_full, 4, 64, false)
ATTN_FWD_KERNEL(fwd_bf16_d128_causal_split, fwd_tile_split, 4, 128, true)
ATTN_FWD_KERNEL(fwd_bf16_d128_split, fwd_tile_split, 4, 128, false)
ATTN_FWD_KERNEL(fwd_bf16_d64_causal_split, fwd_tile_split, 4, 64, true)
ATTN_FWD_KERNEL(fwd_bf16_d64_split, fwd_tile_split, 4, 64, false)
ATTN_FWD_KERNEL(fwd_bf16_d128_causal_pairs, fwd_pair_pipe_body, 8, 128, true)
ATTN_FWD_KERNEL(fwd_bf16_d64_causal_pairs, fwd_pair_pipe_body, 8, 64, true)
#undef ATTN_FWD_KERNEL

__global__ __launch_bounds__(256) void fwd_bf16_d128_split_combine(FwdArgs a) {
  fwd_split_combine_body<128>(a);
}
__global__ __launch_bounds__(256) void fwd_bf16_d64_split_combine(FwdArgs a) {
  fwd_split_combine_body<64>(a);
}

}  // namespace

int fwd_bf16_splits(const FwdProblem& p, int cus) {
  const long long ntq = (p.Sq + kBM - 1) / kBM;
  const long long items = ntq * p.B * p.Hq;
  if (items <= 0 || items * 2 >= 3LL * cus) return 1;   // enough query tiles to fill the chip
  // key tiles of the heaviest query tile; at least four per split
  const int kv = p.causal ? std::min(p.Sk, std::max(0, (int)ntq * kBM + p.Sk - p.Sq)) : p.Sk;
  const int tmax = (kv + kBN - 1) / kBN;
  long long s = (2LL * cus + items - 1) / items;
  s = std::min<long long>(s, kMaxFwdSplits);
  s = std::min<long long>(s, std::max(1, tmax / 4));
  return (int)std::max<long long>(s, 1);
}

int fwd_bf16_mapping(const FwdProblem& p, int cus) {
  // The wide kernel (one wave per SIMD, 256-row workgroups, one per CU) when its items fill the
  // CUs at least four times over, so that the causal spread of item sizes evens out.
  const long long wide_items = (long long)((p.Sq + kWideRows - 1) / kWideRows) * p.B * p.Hq;
  if (p.D == 128 && wide_items >= 4LL * cus) return kMapWide;
  const int ntq = (p.Sq + kBM - 1) / kBM;
  return (p.causal && ntq <= kPairMaxTiles) ? kMapPair : kMapTile;
}

long long fwd_wide_items(const FwdProblem& p) {
  if (p.nsplit > 1 || p.D != 128) return 0;
  const int mapping = p.mapping >= 0 ? p.mapping : fwd_bf16_mapping(p, p.cus);
  if (mapping != kMapWide) return 0;
  return (long long)((p.Sq + kWideRows - 1) / kWideRows) * p.B * p.Hq;
}

size_t fwd_bf16_workspace_bytes(const FwdProblem& p, int nsplit) {
  if (nsplit <= 1) return 0;
  const size_t rows = (size_t)nsplit * p.B * p.Hq * p.Sq;
  return rows * p.D * sizeof(uint16_t) + rows * 2 * sizeof(float);
}

hipError_t launch_fwd_bf16(const FwdProblem& p, hipStream_t stream) {
  FwdArgs a;
  a.q = static_cast<const uint16_t*>(p.q);
  a.k = static_cast<const uint16_t*>(p.k);
  a.v = static_cast<const uint16_t*>(p.v);
  a.o = static_cast<uint16_t*>(p.o);
  a.lse = p.lse;
  a.B = p.B; a.Hq = p.Hq; a.Hkv = p.Hkv; a.Sq = p.Sq; a.Sk = p.Sk;
  a.group = p.Hq / p.Hkv;
  a.ntq = (p.Sq + kBM - 1) / kBM;
  a.npairs = (a.ntq + 1) / 2;
  float c = p.scale * kLog2e;
  // scale == 0 means uniform weights; any tiny positive c gives exactly that (every exp2
  // argument rounds to 0) while keeping -inf * c = -inf for masked keys.
  if (!(c > 0.f)) c = 1.17549435e-38f;
  a.c = c;
  a.nsplit = p.nsplit > 1 ? p.nsplit : 1;
  a.part_o = nullptr;
  a.part_ml = nullptr;
  // key-range splits of a problem with D = 128 and query tiles of at least the wide kernel's
  // 256 rows run on the wide kernel: the same split count gives it half as many workgroups,
  // one per CU where the tile kernel has two
  if (a.nsplit > 1 && p.D == 128 && p.Sq >= kWideRows) return launch_fwd_bf16_wide(p, stream);
  if (a.nsplit > 1) {
    const size_t rows = (size_t)a.nsplit * p.B * p.Hq * p.Sq;
    a.part_o = static_cast<uint16_t*>(p.workspace);
    a.part_ml = reinterpret_cast<float*>(a.part_o + rows * p.D);
    const long long nwg = (long long)a.ntq * a.nsplit * p.B * p.Hq;
    if (nwg == 0) return hipSuccess;
    if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)nwg), block(256);
    const size_t nrows = (size_t)p.B * p.Hq * p.Sq;
    const int rows_per_block = 256 / (p.D / 4);
    dim3 cgrid((unsigned)((nrows + rows_per_block - 1) / rows_per_block)), cblock(256);
    if (p.D == 128) {
      if (p.causal) hipLaunchKernelGGL(fwd_bf16_d128_causal_split, grid, block, 0, stream, a);
      else hipLaunchKernelGGL(fwd_bf16_d128_split, grid, block, 0, stream, a);
      hipLaunchKernelGGL(fwd_bf16_d128_split_combine, cgrid, cblock, 0, stream, a);
    } else {
      if (p.causal) hipLaunchKernelGGL(fwd_bf16_d64_causal_split, grid, block, 0, stream, a);
      else hipLaunchKernelGGL(fwd_bf16_d64_split, grid, block, 0, stream, a);
      hipLaunchKernelGGL(fwd_bf16_d64_split_combine, cgrid, cblock, 0, stream, a);
    }
    return hipGetLastError();
  }
  const int mapping = p.mapping >= 0 ? p.mapping : fwd_bf16_mapping(p, p.cus);
  if (mapping == kMapWide && p.D == 128) return launch_fwd_bf16_wide(p, stream);
  const bool pairs = mapping == kMapPair && p.causal;   // (the pair kernel is causal only)
  const long long nwg = (long long)(pairs ? a.npairs : a.ntq) * p.B * p.Hq;
  if (nwg == 0) return hipSuccess;
  if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  a.nitems = (int)nwg;
  if (pairs) {
    dim3 grid((unsigned)nwg), block(512);
    if (p.D == 128) hipLaunchKernelGGL(fwd_bf16_d128_causal_pairs, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(fwd_bf16_d64_causal_pairs, grid, block, 0, stream, a);
  } else {
    dim3 grid((unsigned)nwg), block(256);
    if (p.D == 128) {
      if (p.causal) hipLaunchKernelGGL(fwd_bf16_d128_causal, grid, block, 0, stream, a);
      else hipLaunchKernelGGL(fwd_bf16_d128, grid, block, 0, stream, a);
    } else {
      if (p.causal) hipLaunchKernelGGL(fwd_bf16_d64_causal, grid, block, 0, stream, a);
      else hipLaunchKernelGGL(fwd_bf16_d64, grid, block, 0, stream, a);
    }
  }
  return hipGetLastError();
}

}  // namespace attn

// Fused exact-attention forward for bf16 Q/K/V on gfx950: O = softmax(scale * Q K^T + mask) V
// and the per-row log-sum-exp, in one pass over K/V with an online softmax, so no score or
// probability matrix ever reaches HBM ("Fused Kernel Compiler" (Candle paper), §FlashAttention
// Integration: tile Q, K, V on chip; scores, softmax and the weighted sum in a single pass;
// online softmax; O(N) memory).
//
// Work mapping: one workgroup of 4 waves per (batch, query head, 128-query tile); each wave
// owns 32 queries. Query head h reads KV head h / (Hq / Hkv) (grouped-query attention).
// The kernel works on the transposed problem so that the softmax runs inside each lane:
//   S^T[key][q] = K[key][:] . Q[q][:]        (MFMA 32x32x16: A = K from LDS, B = Q^T in VGPRs)
//   O^T[d][q]  += V^T[d][key] P^T[key][q]    (MFMA 32x32x16: A = V^T from LDS, B = P^T in VGPRs)
// With this orientation a lane's accumulator column is one query, so the running max and
// sum are per lane: a row max needs one exchange with lane l^32, and P^T leaves the first
// product's accumulators in exactly the B-operand layout of the second (no LDS round trip).
//
// K/V tiles of 64 keys are staged through LDS, double-buffered: the global loads for tile
// j+1 are in flight while tile j is consumed. K is stored row-major with a 16-byte row pad;
// V is transposed on the way in (V^T rows of 64 keys, 8-byte granules XOR-swizzled) so the
// PV operand reads are two ds_read_b64 per MFMA without bank conflicts.
//
// Causal masking is bottom-right aligned (key j visible to query i iff j <= i + Sk - Sq);
// tiles wholly above the diagonal are never loaded, and 32-key blocks above a wave's
// diagonal are skipped by that wave. Tiles are issued heaviest first.
#include "cdna4.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

using namespace cdna4;

#ifndef ATTN_FWD_WAVES_PER_EU
#define ATTN_FWD_WAVES_PER_EU 2
#endif
#ifndef ATTN_FWD_ZIGZAG
#define ATTN_FWD_ZIGZAG 0
#endif

constexpr int kBM = 128;
constexpr int kBN = 64;
constexpr int kThreads = 256;

template <int D>
struct FwdLds {
  static constexpr int kPitch = D * 2 + 16;        // K row: D bf16 + 16 B pad
  static constexpr int kKBytes = kBN * kPitch;
  static constexpr int kVBytes = D * kBN * 2;      // V^T: D rows x 64 keys bf16
  static constexpr int kStage = kKBytes + kVBytes;
  static constexpr int kTotal = 2 * kStage;
};

// Position of the 8-byte granule g (keys 4g..4g+3) inside V^T row d.
__device__ __forceinline__ int vt_swz(int d) { return (d & 15) ^ (((d >> 4) & 3) << 2); }

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int B, Hq, Hkv, Sq, Sk;
  int group;       // Hq / Hkv
  int ntq;         // number of 128-query tiles
  int causal;
  float c;         // scale * log2(e), > 0
};

template <int D>
struct TileRegs {
  // global -> LDS staging registers for one K/V tile
  static constexpr int kKLoads = D / 32;           // 16-byte K chunks per thread
  u32x4 kreg[kKLoads];
  u32x4 vreg[4];
};

template <int D>
__device__ __forceinline__ void load_tile(TileRegs<D>& r, const uint16_t* kbase,
                                          const uint16_t* vbase, int kt, int Sk, int tid) {
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int RPP = kThreads / CPR;        // rows per pass
  const int c = tid % CPR;
#pragma unroll
  for (int i = 0; i < TileRegs<D>::kKLoads; ++i) {
    const int row = tid / CPR + RPP * i;
    const int key = kt + row;
    if (key < Sk)
      r.kreg[i] = *reinterpret_cast<const u32x4*>(kbase + (size_t)key * D + c * 8);
    else
      r.kreg[i] = u32x4{0, 0, 0, 0};
  }
  // V: thread (dc, kg) reads keys 4kg..4kg+3 at d-chunk dc
  const int dc = tid % CPR;
  const int kg = tid / CPR;
  if (kg < 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = kt + 4 * kg + i;
      if (key < Sk)
        r.vreg[i] = *reinterpret_cast<const u32x4*>(vbase + (size_t)key * D + dc * 8);
      else
        r.vreg[i] = u32x4{0, 0, 0, 0};
    }
  }
}

template <int D>
__device__ __forceinline__ void store_tile(const TileRegs<D>& r, char* stage, int tid) {
  using L = FwdLds<D>;
  constexpr int CPR = D / 8;
  constexpr int RPP = kThreads / CPR;
  const int c = tid % CPR;
#pragma unroll
  for (int i = 0; i < TileRegs<D>::kKLoads; ++i) {
    const int row = tid / CPR + RPP * i;
    *reinterpret_cast<u32x4*>(stage + row * L::kPitch + c * 16) = r.kreg[i];
  }
  const int dc = tid % CPR;
  const int kg = tid / CPR;
  if (kg < 16) {
    char* vt = stage + L::kKBytes;
    // transpose the 4 keys x 8 d block: for each d, the 4 keys form one 8-byte granule
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t a = r.vreg[0][w], b = r.vreg[1][w], cc = r.vreg[2][w], dd = r.vreg[3][w];
      // d = 8dc + 2w (low halves) and 8dc + 2w + 1 (high halves)
      const int d0 = 8 * dc + 2 * w;
      const int d1 = d0 + 1;
      u32x2 g0 = {pack_lo16(a, b), pack_lo16(cc, dd)};
      u32x2 g1 = {pack_hi16(a, b), pack_hi16(cc, dd)};
      *reinterpret_cast<u32x2*>(vt + d0 * (kBN * 2) + ((kg ^ vt_swz(d0)) * 8)) = g0;
      *reinterpret_cast<u32x2*>(vt + d1 * (kBN * 2) + ((kg ^ vt_swz(d1)) * 8)) = g1;
    }
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(ATTN_FWD_WAVES_PER_EU, ATTN_FWD_WAVES_PER_EU)))
void fwd_bf16_kernel(FwdArgs a) {
  using L = FwdLds<D>;
  constexpr int KS = D / 16;        // MFMA k-steps over the head dimension
  constexpr int DB = D / 32;        // 32-wide d blocks of O^T
  __shared__ __attribute__((aligned(16))) char smem[L::kTotal];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int h = lane >> 5;

  // ---- work item: heaviest tiles first, all heads of one rank together ----
  const int BH = a.B * a.Hq;
  const int id = blockIdx.x;
  const int rank = id / BH;
  const int bh = id - rank * BH;
  int tile = rank;
  if (CAUSAL) {
    // heaviest tiles first; with ZIGZAG the second half of the ranks runs lightest-first,
    // so the two workgroups that share a CU early on carry complementary amounts of work
    const int half = (a.ntq + 1) / 2;
    if (ATTN_FWD_ZIGZAG && rank >= half) tile = rank - half;
    else tile = a.ntq - 1 - rank;
  }
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
  const int ntiles = (kv_end + kBN - 1) / kBN;

  // ---- Q^T fragments (B operand), resident for the whole loop ----
  u32x4 qf[KS];
  {
    const int qi = qw + l32;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      if (qi < a.Sq)
        qf[kk] = *reinterpret_cast<const u32x4*>(qbase + (size_t)qi * D + kk * 16 + h * 8);
      else
        qf[kk] = u32x4{0, 0, 0, 0};
    }
  }

  f32x16 o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) o[i] = f32x16{};
  float m_run = -INFINITY;     // running max of raw scores of this lane's query
  float l_run = 0.f;           // running sum of exp over this lane's half of the keys
  const float c = a.c;
  const int my_q = qw + l32;
  const int wave_last_key = qw + 31 + off;   // last key any query of this wave may see

  TileRegs<D> tr;
  if (ntiles > 0) {
    load_tile<D>(tr, kbase, vbase, 0, a.Sk, tid);
    store_tile<D>(tr, smem, tid);
  }
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int kt = j * kBN;
    char* stage = smem + (j & 1) * L::kStage;
    const bool more = (j + 1) < ntiles;
    if (more) load_tile<D>(tr, kbase, vbase, kt + kBN, a.Sk, tid);

    // which 32-key blocks of this tile can be visible to this wave
    bool act[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      act[kb] = (kt + 32 * kb < a.Sk) && (!CAUSAL || kt + 32 * kb <= wave_last_key);

    // ---- S^T = K Q^T ----
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      if (act[kb]) {
        const char* krow = stage + (32 * kb + l32) * L::kPitch + h * 16;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
          const u32x4 kf = *reinterpret_cast<const u32x4*>(krow + kk * 32);
          s[kb] = mfma32x32x16(kf, qf[kk], s[kb]);
        }
      }
    }

    // ---- mask: causal diagonal, key tail, inactive blocks ----
    const bool need_mask = (kt + kBN > a.Sk) || (CAUSAL && kt + kBN - 1 > qw + off);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
          bool vis = act[kb] && key < a.Sk;
          if (CAUSAL) vis = vis && (key <= my_q + off);
          s[kb][r] = vis ? s[kb][r] : -INFINITY;
        }
      }
    }

    // ---- online softmax (per lane = per query) ----
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) mx = fmax3(mx, s[kb][r], s[kb][r + 1]);
    mx = fmaxf(mx, wave_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float mc = (m_new == -INFINITY) ? 0.f : m_new * c;
    const float alpha = exp2_fast(m_run * c - mc);     // m_run = -inf -> 0
    m_run = m_new;

    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2_fast(__builtin_fmaf(s[kb][r], c, -mc));
        s[kb][r] = p;
        rs += p;
      }
    l_run = l_run * alpha + rs;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
      for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
    }

    // ---- P^T as bf16 B operands ----
    u32x4 pb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t)
        pb[kb][t] = u32x4{pack_bf16x2(s[kb][8 * t + 0], s[kb][8 * t + 1]),
                          pack_bf16x2(s[kb][8 * t + 2], s[kb][8 * t + 3]),
                          pack_bf16x2(s[kb][8 * t + 4], s[kb][8 * t + 5]),
                          pack_bf16x2(s[kb][8 * t + 6], s[kb][8 * t + 7])};

    // ---- O^T += V^T P^T ----
    const char* vt = stage + L::kKBytes;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int d = 32 * db + l32;
      const int sw = vt_swz(d);
      const char* vrow = vt + d * (kBN * 2);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (!act[kb]) continue;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int g1 = 8 * kb + 4 * t + h;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + ((g1 ^ sw) * 8));
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + (((g1 + 2) ^ sw) * 8));
          const u32x4 vf = {lo[0], lo[1], hi[0], hi[1]};
          o[db] = mfma32x32x16(vf, pb[kb][t], o[db]);
        }
      }
    }

    if (more) store_tile<D>(tr, smem + ((j + 1) & 1) * L::kStage, tid);
    __syncthreads();
  }

  // ---- epilogue: normalise, store O (bf16) and LSE (natural log) ----
  const float l_tot = l_run + wave_xor(l_run, 32);
  const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  if (my_q < a.Sq) {
    uint16_t* orow = a.o + ((size_t)(b * a.Hq + hq) * a.Sq + my_q) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * db + 8 * g + 4 * h;
        u32x2 w = {pack_bf16x2(o[db][4 * g + 0] * inv, o[db][4 * g + 1] * inv),
                   pack_bf16x2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + d) = w;
      }
    if (a.lse != nullptr && h == 0) {
      const float lse = (l_tot > 0.f) ? (m_run * c + log2_fast(l_tot)) * kLn2 : -INFINITY;
      a.lse[(size_t)(b * a.Hq + hq) * a.Sq + my_q] = lse;
    }
  }
}

}  // namespace

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
  a.causal = p.causal;
  float c = p.scale * kLog2e;
  // scale == 0 means uniform weights; any tiny positive c gives exactly that (every exp2
  // argument rounds to 0) while keeping -inf * c = -inf for masked keys.
  if (!(c > 0.f)) c = 1.17549435e-38f;
  a.c = c;
  const long long nwg = (long long)a.ntq * p.B * p.Hq;
  if (nwg == 0) return hipSuccess;
  if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  dim3 grid((unsigned)nwg), block(kThreads);
  if (p.D == 128) {
    if (p.causal) hipLaunchKernelGGL((fwd_bf16_kernel<128, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((fwd_bf16_kernel<128, false>), grid, block, 0, stream, a);
  } else {
    if (p.causal) hipLaunchKernelGGL((fwd_bf16_kernel<64, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((fwd_bf16_kernel<64, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace attn

// One-token decode attention over a paged KV cache on gfx950, split over the context.
//
// The cache is a pool of fixed-size blocks; a per-sequence block table maps logical block n
// of sequence b to a physical block ("Optimizing Large Language Model Inference ...",
// §Paged Attention and Dynamic KV Cache Management). Physical block p, KV head hk holds its
// block_size tokens as a contiguous [block_size, D] bf16 tile (cache layout
// [num_blocks, Hkv, block_size, D]).
//
// Kernel 1 (split): one workgroup per (split, KV head, sequence). It serves all
// g = Hq / Hkv query heads of that KV head, so every K/V byte is read from HBM once. Its
// four waves walk disjoint blocks of the split, each with its own running max/sum:
//   S^T[tok][h] = K[tok][:] . q[h][:]      MFMA 16x16x32, K straight from global into the
//                                          A operand (no LDS), q^T resident as B (heads
//                                          padded to 16 with zeros)
//   O^T[d][h]  += V^T[d][tok] P^T[tok][h]  MFMA 16x16x16; P^T is the first product's
//                                          accumulator as is; V^T is read from a per-wave
//                                          LDS copy of the block with 2-byte column reads.
// The four wave states are merged through LDS and the split writes its normalised partial
// output and its log-sum-exp to a workspace.
// Kernel 2 (combine): per (query head, sequence), merges the splits by their log-sum-exps:
// L = log sum_s exp(lse_s), O = sum_s exp(lse_s - L) O_s -- the same running-softmax algebra
// as the online softmax ("Fused Kernel Compiler" (Candle paper), §FlashAttention Integration).
#include "cdna4.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

using namespace cdna4;

constexpr int kBS = 16;              // tokens per cache block
constexpr int kDecThreads = 256;
constexpr int kDecWaves = 4;
#ifndef ATTN_DEC_MIN_BPS
#define ATTN_DEC_MIN_BPS 8
#endif
constexpr int kMinBlocksPerSplit = ATTN_DEC_MIN_BPS;
constexpr int kMaxGroup = 16;        // query heads per KV head handled by one MFMA column set

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
  int max_splits;
  float c;           // scale * log2(e), > 0
  float* ws_o;
  float* ws_lse;
};

__device__ __forceinline__ int num_splits(int nblk, int max_splits) {
  if (nblk <= 0) return 0;
  const int s = (nblk + kMinBlocksPerSplit - 1) / kMinBlocksPerSplit;
  return s < max_splits ? s : max_splits;
}

__device__ __forceinline__ int ctx_blocks(int ctx) { return ctx > 0 ? (ctx + kBS - 1) / kBS : 0; }

// Blocks of sequence b that are read: its context, cut to an explicit table row length.
__device__ __forceinline__ int seq_blocks(int ctx, int stride) {
  const int n = ctx_blocks(ctx);
  return (stride > 0 && n > stride) ? stride : n;
}

// max_b ceil(ctx_b / kBS), computed by one wave (every lane gets the result).
__device__ int derived_stride(const int32_t* ctx, int B, int lane) {
  int mx = 0;
  for (int i = lane; i < B; i += 64) mx = max(mx, ctx_blocks(ctx[i]));
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) mx = max(mx, __shfl_xor(mx, x, 64));
  return mx;
}

template <int D>
struct DecLds {
  static constexpr int kVPitch = D * 2 + 8;                   // bytes per token row of V
  static constexpr int kVBytes = kBS * kVPitch;               // one block, one wave
  static constexpr int kVAll = kDecWaves * kVBytes;
  static constexpr int kMerge = kDecWaves * kMaxGroup * D * 4;
  static constexpr int kMain = kVAll > kMerge ? kVAll : kMerge;
  static constexpr int kTotal = kMain + 2 * kDecWaves * kMaxGroup * 4;
};

template <int D>
__global__ __launch_bounds__(kDecThreads) void decode_split_kernel(DecArgs a) {
  using L = DecLds<D>;
  constexpr int KS = D / 32;        // 16x16x32 k-steps for q.K
  constexpr int DT = D / 16;        // 16-row d tiles of O^T
  constexpr int VCH = D / 8;        // 16-byte chunks per token row
  constexpr int VLD = kBS * VCH / 64;  // 16-byte V loads per lane per block
  __shared__ __attribute__((aligned(16))) char smem[L::kTotal];

  const int sp = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ctx = a.ctx[b];
  const int nblk = seq_blocks(ctx, a.stride);
  const int ns = num_splits(nblk, a.max_splits);
  if (sp >= ns) return;                       // uniform for the whole workgroup
  const int stride = a.stride > 0 ? a.stride : derived_stride(a.ctx, a.B, lane);
  const int bps = (nblk + ns - 1) / ns;
  const int n0 = sp * bps;
  const int n1 = min(nblk, n0 + bps);
  const int g = a.group;

  const int r16 = lane & 15;        // MFMA row/column index within a 16-wide tile
  const int grp = lane >> 4;        // k-slot group

  // q^T as the B operand: lane (head r16, slot group grp)
  u32x4 qf[KS];
  {
    const uint16_t* qh = a.q + ((size_t)b * a.Hq + (size_t)hk * g + r16) * D;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
      qf[kk] = (r16 < g) ? *reinterpret_cast<const u32x4*>(qh + kk * 32 + grp * 8)
                         : u32x4{0, 0, 0, 0};
  }

  f32x4 acc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) acc[i] = f32x4{};
  float m_run = -INFINITY;  // running max of raw scores for head r16 (same on its 4 lanes)
  float l_run = 0.f;        // running sum over this lane's token slots
  const float c = a.c;
  char* vl = smem + wave * L::kVBytes;
  const int32_t* trow = a.table + (size_t)b * stride;

  for (int n = n0 + wave; n < n1; n += kDecWaves) {
    const int phys = trow[n];
    if (a.num_blocks > 0 && (phys < 0 || phys >= a.num_blocks)) continue;   // invalid entry
    const size_t tile = ((size_t)phys * a.Hkv + hk) * kBS * D;
    const uint16_t* kt = a.kc + tile;
    const uint16_t* vt = a.vc + tile;
    u32x4 kf[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
      kf[kk] = *reinterpret_cast<const u32x4*>(kt + r16 * D + kk * 32 + grp * 8);
    u32x4 vr[VLD];
#pragma unroll
    for (int i = 0; i < VLD; ++i) {
      const int ci = lane + 64 * i;
      vr[i] = *reinterpret_cast<const u32x4*>(vt + (ci / VCH) * D + (ci % VCH) * 8);
    }
    // slots past the end of the context hold stale data (possibly NaN): the matrix core
    // would multiply them by p = 0 and still produce NaN, so they are staged as zeros
#pragma unroll
    for (int i = 0; i < VLD; ++i) {
      const int ci = lane + 64 * i;
      const bool live = n * kBS + ci / VCH < ctx;
      char* dst = vl + (ci / VCH) * L::kVPitch + (ci % VCH) * 16;
      *reinterpret_cast<u32x2*>(dst) = live ? u32x2{vr[i][0], vr[i][1]} : u32x2{0, 0};
      *reinterpret_cast<u32x2*>(dst + 8) = live ? u32x2{vr[i][2], vr[i][3]} : u32x2{0, 0};
    }

    f32x4 s = f32x4{};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) s = mfma16x16x32(kf[kk], qf[kk], s);

    // lane holds tokens 4*grp + j of this block for head r16
    const int tok0 = n * kBS + 4 * grp;
#pragma unroll
    for (int j = 0; j < 4; ++j) s[j] = (tok0 + j < ctx) ? s[j] : -INFINITY;
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = fmaxf(mx, wave_xor(mx, 16));
    mx = fmaxf(mx, wave_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float mc = (m_new == -INFINITY) ? 0.f : m_new * c;
    const float alpha = exp2_fast(m_run * c - mc);
    m_run = m_new;
    float p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) p[j] = exp2_fast(__builtin_fmaf(s[j], c, -mc));
    l_run = l_run * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
#pragma unroll
    for (int i = 0; i < DT; ++i) acc[i] *= alpha;
    const u32x2 pb = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};

    wave_lds_fence();
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const char* col = vl + (4 * grp) * L::kVPitch + (16 * dt + r16) * 2;
      const uint32_t t0 = *reinterpret_cast<const uint16_t*>(col);
      const uint32_t t1 = *reinterpret_cast<const uint16_t*>(col + L::kVPitch);
      const uint32_t t2 = *reinterpret_cast<const uint16_t*>(col + 2 * L::kVPitch);
      const uint32_t t3 = *reinterpret_cast<const uint16_t*>(col + 3 * L::kVPitch);
      const u32x2 va = {t0 | (t1 << 16), t2 | (t3 << 16)};
      acc[dt] = mfma16x16x16(va, pb, acc[dt]);
    }
    wave_lds_fence();
  }

  // ---- merge the four wave states of this split ----
  float l_head = l_run + wave_xor(l_run, 16);
  l_head += wave_xor(l_head, 32);
  __syncthreads();                           // V staging area is reused below
  float* ow = reinterpret_cast<float*>(smem);                       // [wave][head][D]
  float* mw = reinterpret_cast<float*>(smem + L::kMain);            // [wave][head]
  float* lw = mw + kDecWaves * kMaxGroup;                           // [wave][head]
  if (r16 < g) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        ow[(wave * kMaxGroup + r16) * D + 16 * dt + 4 * grp + j] = acc[dt][j];
    if (grp == 0) {
      mw[wave * kMaxGroup + r16] = m_run;
      lw[wave * kMaxGroup + r16] = l_head;
    }
  }
  __syncthreads();
  for (int i = tid; i < g * D; i += kDecThreads) {
    const int hh = i / D, d = i - hh * D;
    float mt = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) mt = fmaxf(mt, mw[w * kMaxGroup + hh]);
    float lt = 0.f, ot = 0.f;
    if (mt != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) {
        const float wt = exp2_fast((mw[w * kMaxGroup + hh] - mt) * c);
        lt += lw[w * kMaxGroup + hh] * wt;
        ot += ow[(w * kMaxGroup + hh) * D + d] * wt;
      }
    }
    const size_t row = ((size_t)b * a.Hq + (size_t)hk * g + hh) * a.max_splits + sp;
    a.ws_o[row * D + d] = (lt > 0.f) ? ot / lt : 0.f;
    if (d == 0) a.ws_lse[row] = (lt > 0.f) ? (mt * c + log2_fast(lt)) * kLn2 : -INFINITY;
  }
}

template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecArgs a) {
  const int hq = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int ns = num_splits(seq_blocks(a.ctx[b], a.stride), a.max_splits);
  const size_t row0 = ((size_t)b * a.Hq + hq) * a.max_splits;
  float mt = -INFINITY;
  for (int s = 0; s < ns; ++s) mt = fmaxf(mt, a.ws_lse[row0 + s]);
  float wsum = 0.f, ot = 0.f;
  if (mt != -INFINITY) {
    for (int s = 0; s < ns; ++s) {
      const float w = exp2_fast((a.ws_lse[row0 + s] - mt) * kLog2e);
      wsum += w;
      ot += w * a.ws_o[(row0 + s) * D + d];
    }
  }
  const float out = (wsum > 0.f) ? ot / wsum : 0.f;
  __bf16 ob = (__bf16)out;
  a.o[((size_t)b * a.Hq + hq) * D + d] = __builtin_bit_cast(uint16_t, ob);
  if (a.lse != nullptr && d == 0)
    a.lse[(size_t)b * a.Hq + hq] = (wsum > 0.f) ? mt + log2_fast(wsum) * kLn2 : -INFINITY;
}

}  // namespace

size_t decode_workspace_floats(int B, int Hq, int D, int max_splits) {
  return (size_t)B * Hq * max_splits * (size_t)(D + 1);
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
  a.max_splits = p.max_splits;
  float c = p.scale * kLog2e;
  if (!(c > 0.f)) c = 1.17549435e-38f;   // scale 0: uniform weights
  a.c = c;
  a.ws_o = p.ws_o;
  a.ws_lse = p.ws_lse;
  if (p.B == 0) return hipSuccess;
  dim3 g1(p.max_splits, p.Hkv, p.B), b1(kDecThreads);
  dim3 g2(p.Hq, p.B);
  if (p.D == 128) {
    hipLaunchKernelGGL(decode_split_kernel<128>, g1, b1, 0, stream, a);
    hipLaunchKernelGGL(decode_combine_kernel<128>, g2, dim3(128), 0, stream, a);
  } else {
    hipLaunchKernelGGL(decode_split_kernel<64>, g1, b1, 0, stream, a);
    hipLaunchKernelGGL(decode_combine_kernel<64>, g2, dim3(64), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace attn

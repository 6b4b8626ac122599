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
  // V rows padded by 32 bytes: the 16-byte row writes and the transposing 8-byte column
  // reads both spread over all 64 banks (D = 128; D = 64 leaves a 2-way conflict on writes)
  static constexpr int kVPitch = D * 2 + 32;
  static constexpr int kVBytes = kBS * kVPitch;               // one block, one wave
  static constexpr int kVAll = kDecWaves * kVBytes;
  static constexpr int kMerge = kDecWaves * kMaxGroup * D * 4;
  static constexpr int kMain = kVAll > kMerge ? kVAll : kMerge;
  static constexpr int kTotal = kMain + 2 * kDecWaves * kMaxGroup * 4;
};

// Buffer resource word 3 for raw (untyped) loads on gfx9-family parts.
constexpr int kRawBufferFlags = 0x00020000;

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// The K and V registers of one cache block for one wave.
template <int D>
struct DecFrag {
  static constexpr int KS = D / 32;                 // K: 16x16x32 A-operand k-steps
  static constexpr int VLD = kBS * D * 2 / 16 / 64;  // V: 16-byte loads per lane
  u32x4 k[KS];
  u32x4 v[VLD];
};

// Loads one block through buffer resources whose size is the block's live bytes: rows past
// the context, and whole blocks whose table entry is invalid (size 0), come back as zeros
// without touching memory. Zero V rows keep 0 * stale-NaN out of the matrix core.
template <int D>
__device__ __forceinline__ void dec_load(DecFrag<D>& f, const uint16_t* kbase,
                                         const uint16_t* vbase, int bytes, int koff, int voff) {
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc((void*)kbase, 0, bytes, kRawBufferFlags);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc((void*)vbase, 0, bytes, kRawBufferFlags);
#pragma unroll
  for (int kk = 0; kk < DecFrag<D>::KS; ++kk)
    f.k[kk] = __builtin_amdgcn_raw_buffer_load_b128(rk, koff + kk * 64, 0, 0);
#pragma unroll
  for (int i = 0; i < DecFrag<D>::VLD; ++i)
    f.v[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, voff + i * 1024, 0, 0);
}

#ifndef ATTN_DEC_WAVES_PER_EU
#define ATTN_DEC_WAVES_PER_EU 3
#endif

template <int D>
__global__ __launch_bounds__(kDecThreads)
__attribute__((amdgpu_waves_per_eu(ATTN_DEC_WAVES_PER_EU))) void decode_split_kernel(DecArgs a) {
  using L = DecLds<D>;
  using F = DecFrag<D>;
  constexpr int KS = F::KS;
  constexpr int DT = D / 16;        // 16-row d tiles of O^T
  constexpr int VCH = D / 8;        // 16-byte chunks per token row
  __shared__ __attribute__((aligned(16))) char smem[L::kTotal];

  const int sp = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = wave_uniform(tid >> 6);   // scalar: the block addresses below are per wave
  const int ctx = a.ctx[b];
  const int stride = a.stride > 0 ? a.stride : derived_stride(a.ctx, a.B, lane);
  const int nblk = seq_blocks(ctx, a.stride);
  const int ns = num_splits(nblk, a.max_splits);
  if (sp >= ns) return;                       // uniform for the whole workgroup
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
  const size_t tile_elems = (size_t)kBS * D;
  const uint16_t* kc = a.kc + (size_t)hk * tile_elems;
  const uint16_t* vc = a.vc + (size_t)hk * tile_elems;
  const size_t phys_elems = (size_t)a.Hkv * tile_elems;
  const int koff = r16 * 2 * D + grp * 16;   // K: row r16, 8 columns of slot group grp
  const int voff = lane * 16;                // V: contiguous 1 KiB per load
  // the transposing read: lane (grp, r16) addresses key 4*grp + r16/4, columns 4*(r16%4)..+3
  const char* vtr = vl + (4 * grp + (r16 >> 2)) * L::kVPitch + (r16 & 3) * 8;

  // this wave's blocks are first + 4j, j < cnt; table entries are fetched 64 at a time
  const int first = n0 + wave;
  const int cnt = first < n1 ? (n1 - first + 3) / 4 : 0;
  for (int c0 = 0; c0 < cnt; c0 += 64) {
    const int cc = min(64, cnt - c0);
    const int tv = lane < cc ? trow[first + 4 * (c0 + lane)] : 0;

    // live bytes of block j of this chunk (0 past the chunk or for an invalid entry)
    auto block_src = [&](int j, const uint16_t*& kb, const uint16_t*& vb) -> int {
      const int phys = __builtin_amdgcn_readlane(tv, j & 63);
      const int n = first + 4 * (c0 + j);
      const bool ok = j < cc && (a.num_blocks <= 0 || (phys >= 0 && phys < a.num_blocks));
      const size_t off = ok ? (size_t)phys * phys_elems : 0;
      kb = kc + off;
      vb = vc + off;
      return ok ? min(kBS, ctx - n * kBS) * 2 * D : 0;
    };

    auto process = [&](const F& f, int j) {
      const uint16_t *kb, *vb;
      const int live = block_src(j, kb, vb) / (2 * D);   // live tokens of this block
#pragma unroll
      for (int i = 0; i < F::VLD; ++i) {
        const int ci = lane + 64 * i;
        *reinterpret_cast<u32x4*>(vl + (ci / VCH) * L::kVPitch + (ci % VCH) * 16) = f.v[i];
      }
      f32x4 s = f32x4{};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) s = mfma16x16x32(f.k[kk], qf[kk], s);

      // lane holds tokens 4*grp + j of this block for head r16
#pragma unroll
      for (int t = 0; t < 4; ++t) s[t] = (4 * grp + t < live) ? s[t] : -INFINITY;
      float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
      mx = fmaxf(mx, wave_xor(mx, 16));
      mx = fmaxf(mx, wave_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float mc = (m_new == -INFINITY) ? 0.f : m_new * c;
      const float alpha = exp2_fast(m_run * c - mc);
      m_run = m_new;
      float p[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) p[t] = exp2_fast(__builtin_fmaf(s[t], c, -mc));
      l_run = l_run * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
#pragma unroll
      for (int i = 0; i < DT; ++i) acc[i] *= alpha;
      const u32x2 pb = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};

      wave_lds_fence();
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const i16x4 vt = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vtr + 32 * dt));
        acc[dt] = mfma16x16x16(__builtin_bit_cast(u32x2, vt), pb, acc[dt]);
      }
      wave_lds_fence();
    };

    // two register sets: block j+1 is in flight while block j is processed
    F fa, fb;
    {
      const uint16_t *kb, *vb;
      const int bytes = block_src(0, kb, vb);
      dec_load<D>(fa, kb, vb, bytes, koff, voff);
    }
    for (int j = 0; j < cc; j += 2) {
      {
        const uint16_t *kb, *vb;
        const int bytes = block_src(j + 1, kb, vb);
        dec_load<D>(fb, kb, vb, bytes, koff, voff);
      }
      process(fa, j);
      if (j + 1 >= cc) break;
      {
        const uint16_t *kb, *vb;
        const int bytes = block_src(j + 2, kb, vb);
        dec_load<D>(fa, kb, vb, bytes, koff, voff);
      }
      process(fb, j + 1);
    }
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

// Exact-attention forward for fp32 Q/K/V/O on the vector ALUs (gfx950).
//
// Same single-pass, tiled online-softmax schedule as the bf16 kernel ("Fused Kernel
// Compiler" (Candle paper), §FlashAttention Integration), kept in fp32 end to end: this path
// exists for full-precision checks, so it favours exactness over speed.
//
// Mapping: D/32 lanes share one query, each holding 32 of its D components of q and of the
// output accumulator; a 128-thread workgroup covers 128*32/D queries. K/V tiles of 32 keys
// are staged in LDS and every lane reads them as broadcasts.
#include "cdna4.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

using namespace cdna4;

constexpr int kThreadsF = 128;
constexpr int kTileF = 32;

struct FwdF32Args {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  int B, Hq, Hkv, Sq, Sk, group, ntq;
  float c;   // scale * log2(e), > 0
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreadsF) void fwd_f32_kernel(FwdF32Args a) {
  constexpr int TPQ = D / 32;                 // lanes per query
  constexpr int QPB = kThreadsF / TPQ;        // queries per workgroup
  __shared__ float ks[kTileF][D];
  __shared__ float vs[kTileF][D];
  lds_poison(ks, sizeof(ks));
  lds_poison(vs, sizeof(vs));
  lds_poison_done();

  const int tid = threadIdx.x;
  const int part = tid % TPQ;
  const int BH = a.B * a.Hq;
  const int rank = blockIdx.x / BH;
  const int bh = blockIdx.x - rank * BH;
  const int tile = CAUSAL ? (a.ntq - 1 - rank) : rank;
  const int b = bh / a.Hq;
  const int hq = bh - b * a.Hq;
  const int hk = hq / a.group;
  const int q0 = tile * QPB;
  const int qi = q0 + tid / TPQ;
  const int off = a.Sk - a.Sq;

  const float* qrow = a.q + ((size_t)(b * a.Hq + hq) * a.Sq + qi) * D + part * 32;
  const float* kb = a.k + (size_t)(b * a.Hkv + hk) * a.Sk * D;
  const float* vb = a.v + (size_t)(b * a.Hkv + hk) * a.Sk * D;

  float qv[32], acc[32];
#pragma unroll
  for (int d = 0; d < 32; ++d) {
    qv[d] = (qi < a.Sq) ? qrow[d] : 0.f;
    acc[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const float c = a.c;

  int kv_end = a.Sk;
  if (CAUSAL) kv_end = min(a.Sk, max(0, q0 + QPB + off));

  for (int kt = 0; kt < kv_end; kt += kTileF) {
    __syncthreads();
    for (int i = tid; i < kTileF * D; i += kThreadsF) {
      const int r = i / D, d = i % D;
      const bool ok = kt + r < a.Sk;
      ks[r][d] = ok ? kb[(size_t)(kt + r) * D + d] : 0.f;
      vs[r][d] = ok ? vb[(size_t)(kt + r) * D + d] : 0.f;
    }
    __syncthreads();

    float s[kTileF];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kTileF; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < 32; ++d) dot = __builtin_fmaf(qv[d], ks[j][part * 32 + d], dot);
#pragma unroll
      for (int x = 1; x < TPQ; x <<= 1) dot += __shfl_xor(dot, x, 64);
      const int key = kt + j;
      bool vis = key < a.Sk;
      if (CAUSAL) vis = vis && key <= qi + off;
      s[j] = vis ? dot * c : -INFINITY;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m, mx);
    const float mu = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2_fast(m - mu);
    m = m_new;
    float rs = 0.f;
#pragma unroll
    for (int j = 0; j < kTileF; ++j) {
      s[j] = exp2_fast(s[j] - mu);
      rs += s[j];
    }
    l = l * alpha + rs;
#pragma unroll
    for (int d = 0; d < 32; ++d) {
      float t = acc[d] * alpha;
#pragma unroll
      for (int j = 0; j < kTileF; ++j) t = __builtin_fmaf(s[j], vs[j][part * 32 + d], t);
      acc[d] = t;
    }
  }

  if (qi < a.Sq) {
    float* orow = a.o + ((size_t)(b * a.Hq + hq) * a.Sq + qi) * D + part * 32;
    const float inv = (l > 0.f) ? 1.f / l : 0.f;
#pragma unroll
    for (int d = 0; d < 32; ++d) orow[d] = acc[d] * inv;
    if (a.lse != nullptr && part == 0)
      a.lse[(size_t)(b * a.Hq + hq) * a.Sq + qi] =
          (l > 0.f) ? (m + log2_fast(l)) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_fwd_f32(const FwdProblem& p, hipStream_t stream) {
  FwdF32Args a;
  a.q = static_cast<const float*>(p.q);
  a.k = static_cast<const float*>(p.k);
  a.v = static_cast<const float*>(p.v);
  a.o = static_cast<float*>(p.o);
  a.lse = p.lse;
  a.B = p.B; a.Hq = p.Hq; a.Hkv = p.Hkv; a.Sq = p.Sq; a.Sk = p.Sk;
  a.group = p.Hq / p.Hkv;
  const int qpb = kThreadsF / (p.D / 32);
  a.ntq = (p.Sq + qpb - 1) / qpb;
  float c = p.scale * kLog2e;
  if (!(c > 0.f)) c = 1.17549435e-38f;   // scale 0: uniform weights, masked keys stay -inf
  a.c = c;
  const long long nwg = (long long)a.ntq * p.B * p.Hq;
  if (nwg == 0) return hipSuccess;
  if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  dim3 grid((unsigned)nwg), block(kThreadsF);
  if (p.D == 128) {
    if (p.causal) hipLaunchKernelGGL((fwd_f32_kernel<128, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((fwd_f32_kernel<128, false>), grid, block, 0, stream, a);
  } else {
    if (p.causal) hipLaunchKernelGGL((fwd_f32_kernel<64, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((fwd_f32_kernel<64, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace attn

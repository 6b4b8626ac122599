// Fused residual add + RMS normalisation on gfx950 ("Kernel and Operator Fusion -- Inference
// Optimization", §4 Tiny example and §6-9 Under the hood): per row of d elements,
//   t   = x + residual                       (returned: the next layer's residual input)
//   out = t * rsqrt(mean(t^2) + eps) * weight
// in one pass over HBM: x and the residual are read once, t and out written once (the weight
// row is read by every row and stays in L2).
//
// One workgroup per row. Thread i of T holds the 16-byte vectors v*T + i (v < VPT) of the
// row, so every load and store instruction covers T*16 contiguous bytes. The add, the sum of
// squares and the scaling run in fp32 registers; t and out are rounded to bfloat16 once, at
// their stores. The row's sum of squares is reduced across the wave with lane exchanges,
// then across the workgroup's waves through LDS. Each thread writes only the elements it
// read, so out may be x and residual_out may be residual (in place).
#include "cdna4.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

using namespace cdna4;

constexpr int kNormMaxThreads = 1024;

struct NormArgs {
  const uint16_t* x;
  const uint16_t* r;
  const uint16_t* w;
  uint16_t* out;
  uint16_t* t_out;
  int d;          // row length, a multiple of 8
  int nvec;       // d / 8 16-byte vectors per row
  float eps;
  float inv_d;
};

// The eight bf16 of a 16-byte vector, widened to fp32 (exact).
__device__ __forceinline__ void widen8(const u32x4& v, float (&f)[8]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[2 * j] = bf16lo_to_f32(v[j]);
    f[2 * j + 1] = bf16hi_to_f32(v[j]);
  }
}

__device__ __forceinline__ u32x4 narrow8(const float (&f)[8]) {
  return u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
               pack_bf16x2(f[6], f[7])};
}

template <int VPT>
__global__ __launch_bounds__(kNormMaxThreads) void add_rms_norm_kernel(NormArgs a) {
  __shared__ float part[kNormMaxThreads / 64];
  lds_poison(part, sizeof(part));
  lds_poison_done();
  const int T = blockDim.x;
  const int tid = threadIdx.x;
  const size_t row = (size_t)blockIdx.x * a.d;
  const u32x4* xr = reinterpret_cast<const u32x4*>(a.x + row);
  const u32x4* rr = reinterpret_cast<const u32x4*>(a.r + row);
  const u32x4* wr = reinterpret_cast<const u32x4*>(a.w);

  // all loads first (x, residual and weight vectors), so their latencies overlap and so a
  // thread has read every element it will overwrite in place
  u32x4 xv[VPT], rv[VPT], wv[VPT];
#pragma unroll
  for (int v = 0; v < VPT; ++v) {
    const int vi = v * T + tid;
    const bool in = vi < a.nvec;
    xv[v] = in ? xr[vi] : u32x4{0, 0, 0, 0};
    rv[v] = in ? rr[vi] : u32x4{0, 0, 0, 0};
    wv[v] = in ? wr[vi] : u32x4{0, 0, 0, 0};
  }

  float t[VPT][8];
  float ss = 0.f;
#pragma unroll
  for (int v = 0; v < VPT; ++v) {
    float xf[8], rf[8];
    widen8(xv[v], xf);
    widen8(rv[v], rf);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      t[v][j] = xf[j] + rf[j];
      ss = __builtin_fmaf(t[v][j], t[v][j], ss);
    }
  }
  // the new residual: t rounded once
  u32x4* tr = reinterpret_cast<u32x4*>(a.t_out + row);
#pragma unroll
  for (int v = 0; v < VPT; ++v) {
    const int vi = v * T + tid;
    if (vi < a.nvec) tr[vi] = narrow8(t[v]);
  }

  // sum of squares over the row: within the wave, then across the waves through LDS
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += wave_xor(ss, m);
  if ((tid & 63) == 0) part[tid >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
  for (int i = 0; i < (T >> 6); ++i) tot += part[i];
  const float rs = rsqrtf(__builtin_fmaf(tot, a.inv_d, a.eps));

  u32x4* orow = reinterpret_cast<u32x4*>(a.out + row);
#pragma unroll
  for (int v = 0; v < VPT; ++v) {
    const int vi = v * T + tid;
    float wf[8], o[8];
    widen8(wv[v], wf);
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = t[v][j] * rs * wf[j];
    if (vi < a.nvec) orow[vi] = narrow8(o);
  }
}

}  // namespace

int add_rms_norm_threads(int d) {
  const int nvec = d / 8;
  int vpt = (nvec + 255) / 256;   // up to 256 threads per row, more vectors per thread beyond
  if (vpt > 8) vpt = 8;
  const int per = (nvec + vpt - 1) / vpt;
  return ((per + 63) / 64) * 64;
}

hipError_t launch_add_rms_norm(const NormProblem& p, hipStream_t stream) {
  if (p.M == 0) return hipSuccess;
  NormArgs a;
  a.x = static_cast<const uint16_t*>(p.x);
  a.r = static_cast<const uint16_t*>(p.residual);
  a.w = static_cast<const uint16_t*>(p.weight);
  a.out = static_cast<uint16_t*>(p.out);
  a.t_out = static_cast<uint16_t*>(p.residual_out);
  a.d = p.d;
  a.nvec = p.d / 8;
  a.eps = p.eps;
  a.inv_d = 1.0f / (float)p.d;
  const int T = add_rms_norm_threads(p.d);
  const int vpt = (a.nvec + T - 1) / T;
  dim3 grid(p.M), block(T);
  switch (vpt) {
    case 1: hipLaunchKernelGGL(add_rms_norm_kernel<1>, grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL(add_rms_norm_kernel<2>, grid, block, 0, stream, a); break;
    case 3:
    case 4: hipLaunchKernelGGL(add_rms_norm_kernel<4>, grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL(add_rms_norm_kernel<8>, grid, block, 0, stream, a); break;
  }
  return hipGetLastError();
}

}  // namespace attn

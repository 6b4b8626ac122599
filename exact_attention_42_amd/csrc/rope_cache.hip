// Fused rotary position embedding + paged KV-cache store on gfx950 -- the step just before
// decode attention, "RoPE then KV store" in one pass ("Kernel and Operator Fusion --
// Inference Optimization", §2 item 6; RoPE as sin, cos, rotate in the fusion table of "Fused
// Kernel Compiler" (Candle paper)). The pages print no formula; the rotate-half form is used:
// pair (i, i + D/2) of every query and key head turns by p * base^(-2i/D).
//
// One workgroup per token. Its first D/2 threads form the token's cos/sin table in LDS: the
// angle p * theta_i and its sine and cosine are evaluated in fp64, so the angle keeps full
// accuracy at long positions, then rounded to fp32. The work items are (head, j) for the
// query heads, the key heads and the value heads: an item covers 16-byte vectors j and
// j + D/16 of the head (elements 8j..8j+7 and D/2+8j..D/2+8j+7, which are rotation partners).
// Query items rotate and store to q_out; key items rotate and store into the cache slot;
// value items copy into the cache slot. The slot is block_table[seq, p / 16], row p % 16 of
// the [num_blocks, Hkv, 16, D] cache -- where the paged decode reads it.
#include "cdna4.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

using namespace cdna4;

constexpr int kRopeThreads = 256;
constexpr int kRopeBS = 16;

struct RopeArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* q_out;
  uint16_t* kc;
  uint16_t* vc;
  const int32_t* table;
  const int32_t* pos;
  const int32_t* seq;       // may be null: token t is sequence t
  int num_seqs;             // rows of the block table
  int Hq, Hkv, D;
  int stride;
  int num_blocks;           // <= 0: unchecked
  double base;
};

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

template <int D>
__global__ __launch_bounds__(kRopeThreads) void rope_cache_kernel(RopeArgs a) {
  constexpr int H2 = D / 2;          // rotation pairs
  constexpr int VP = D / 16;         // vector pairs per head
  __shared__ float cs[H2], sn[H2];
  lds_poison(cs, sizeof(cs));
  lds_poison(sn, sizeof(sn));
  lds_poison_done();
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int p = a.pos[t];
  const int nq = a.Hq * VP, nk = a.Hkv * VP;
  const int nitems = nq + 2 * nk;

  // the cache row of this token (null when nothing is stored)
  size_t row = 0;
  bool store = false;
  const int s = a.seq != nullptr ? a.seq[t] : t;
  if (p >= 0 && p / kRopeBS < a.stride && s >= 0 && s < a.num_seqs) {
    const int phys = a.table[(size_t)s * a.stride + p / kRopeBS];
    store = a.num_blocks <= 0 || (phys >= 0 && phys < a.num_blocks);
    row = ((size_t)phys * a.Hkv) * kRopeBS * D + (size_t)(p % kRopeBS) * D;
  }

  // item it: vectors j and j + D/16 of a query, key or value head
  auto src_of = [&](int it, int& j) -> const uint16_t* {
    if (it < nq) {
      j = it % VP;
      return a.q + ((size_t)t * a.Hq + it / VP) * D;
    }
    const int kv = it - nq;
    const bool isv = kv >= nk;
    const int w = isv ? kv - nk : kv;
    j = w % VP;
    return (isv ? a.v : a.k) + ((size_t)t * a.Hkv + w / VP) * D;
  };
  // the first two items' loads go out before the table and before any store, so that each
  // thread keeps four 16-byte loads in flight
  u32x4 lo0 = u32x4{0, 0, 0, 0}, hi0 = u32x4{0, 0, 0, 0};
  u32x4 lo1 = u32x4{0, 0, 0, 0}, hi1 = u32x4{0, 0, 0, 0};
  if (tid < nitems) {
    int j;
    const uint16_t* src = src_of(tid, j);
    lo0 = *reinterpret_cast<const u32x4*>(src + 8 * j);
    hi0 = *reinterpret_cast<const u32x4*>(src + H2 + 8 * j);
  }
  if (tid + kRopeThreads < nitems) {
    int j;
    const uint16_t* src = src_of(tid + kRopeThreads, j);
    lo1 = *reinterpret_cast<const u32x4*>(src + 8 * j);
    hi1 = *reinterpret_cast<const u32x4*>(src + H2 + 8 * j);
  }

  if (tid < H2) {
    const double theta = pow(a.base, -2.0 * (double)tid / (double)D);
    double sd, cd;
    sincos((double)p * theta, &sd, &cd);
    cs[tid] = (float)cd;
    sn[tid] = (float)sd;
  }
  __syncthreads();

  for (int it = tid; it < nitems; it += kRopeThreads) {
    int j;
    const uint16_t* src = src_of(it, j);
    u32x4 lo, hi;
    if (it == tid) {
      lo = lo0;
      hi = hi0;
    } else if (it == tid + kRopeThreads) {
      lo = lo1;
      hi = hi1;
    } else {
      lo = *reinterpret_cast<const u32x4*>(src + 8 * j);
      hi = *reinterpret_cast<const u32x4*>(src + H2 + 8 * j);
    }
    uint16_t* dst;
    bool rotate = true;
    if (it < nq) {
      dst = a.q_out + ((size_t)t * a.Hq + it / VP) * D;
    } else {
      if (!store) continue;
      const int kv = it - nq;
      const bool isv = kv >= nk;
      const int w = isv ? kv - nk : kv;
      dst = (isv ? a.vc : a.kc) + row + (size_t)(w / VP) * kRopeBS * D;
      rotate = !isv;
    }
    if (!rotate) {
      *reinterpret_cast<u32x4*>(dst + 8 * j) = lo;
      *reinterpret_cast<u32x4*>(dst + H2 + 8 * j) = hi;
      continue;
    }
    float x1[8], x2[8], y1[8], y2[8];
    widen8(lo, x1);
    widen8(hi, x2);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float c = cs[8 * j + e], sa = sn[8 * j + e];
      y1[e] = x1[e] * c - x2[e] * sa;
      y2[e] = x2[e] * c + x1[e] * sa;
    }
    *reinterpret_cast<u32x4*>(dst + 8 * j) = narrow8(y1);
    *reinterpret_cast<u32x4*>(dst + H2 + 8 * j) = narrow8(y2);
  }
}

}  // namespace

hipError_t launch_rope_cache_write(const RopeProblem& p, hipStream_t stream) {
  if (p.T == 0) return hipSuccess;
  RopeArgs a;
  a.q = static_cast<const uint16_t*>(p.q);
  a.k = static_cast<const uint16_t*>(p.k);
  a.v = static_cast<const uint16_t*>(p.v);
  a.q_out = static_cast<uint16_t*>(p.q_out);
  a.kc = static_cast<uint16_t*>(p.k_cache);
  a.vc = static_cast<uint16_t*>(p.v_cache);
  a.table = p.block_table;
  a.pos = p.positions;
  a.seq = p.seq_ids;
  a.num_seqs = p.num_seqs;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.D = p.D;
  a.stride = p.table_stride;
  a.num_blocks = p.num_blocks;
  a.base = (double)p.base;
  dim3 grid(p.T), block(kRopeThreads);
  if (p.D == 128)
    hipLaunchKernelGGL(rope_cache_kernel<128>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(rope_cache_kernel<64>, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace attn

// CDNA4 (gfx950) building blocks for the attention kernels: vector types, MFMA wrappers,
// bfloat16 packing, exp2/log2 and wave-level exchanges.
//
// Matrix-core fragment layouts used throughout (wave64; l = lane id):
//   v_mfma_f32_32x32x16_bf16  A: lane l holds A[m = l%32][k-slot (l/32, i)], i = 0..7
//                             B: lane l holds B[k-slot (l/32, i)][n = l%32]
//                             C: lane l, reg j holds C[m = 8*(j/4) + 4*(l/32) + j%4][n = l%32]
//   v_mfma_f32_16x16x32_bf16  A: lane l holds A[m = l%16][k-slot (l/16, i)], i = 0..7
//                             B: lane l holds B[k-slot (l/16, i)][n = l%16]
//                             C: lane l, reg j holds C[m = 4*(l/16) + j][n = l%16]
//   v_mfma_f32_16x16x16_bf16  A: lane l holds A[m = l%16][k = 4*(l/16) + i], i = 0..3
//                             B: lane l holds B[k = 4*(l/16) + i][n = l%16]
//                             C: as for 16x16x32.
// A and B always share the same k-slot -> k assignment, so a contraction only needs the
// two operands to agree on which logical index sits in slot (l/32, i) (or (l/16, i)); the
// kernels choose that assignment to match where the data already lives in registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cdna4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32x32x16(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mfma16x16x16(const u32x2& a, const u32x2& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                   __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
}

// Two fp32 -> one dword of two bfloat16 (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

// acc + lo + hi of a dword holding two bfloat16 values (v_dot2_f32_bf16 against 1.0, 1.0).
__device__ __forceinline__ float bf16x2_sum_acc(uint32_t w, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), one, acc, false);
}

__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// Byte permute: result byte n = byte sel[n] of the 8-byte value {hi:lo}.
__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}
// {lo16(a), lo16(b)} and {hi16(a), hi16(b)}
__device__ __forceinline__ uint32_t pack_lo16(uint32_t a, uint32_t b) { return perm_b32(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pack_hi16(uint32_t a, uint32_t b) { return perm_b32(b, a, 0x07060302u); }

// A value that is the same on every lane, moved to a scalar register.
__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ float wave_xor(float x, int mask) { return __shfl_xor(x, mask, 64); }

__device__ __forceinline__ float fmax3(float a, float b, float c) { return fmaxf(a, fmaxf(b, c)); }

// Orders LDS accesses of one wave (no workgroup barrier): what the wave wrote before is
// visible to what it reads after.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Debug builds (-DATTN_POISON_LDS): a kernel first fills the LDS arrays it uses with 0xff bytes
// (NaN as fp32 and as bf16), then synchronises the workgroup, so that reading any LDS byte the
// kernel has not written itself shows in its results. In normal builds both calls are empty.
#ifdef ATTN_POISON_LDS
__device__ __forceinline__ void lds_poison(void* p, size_t bytes) {
  uint32_t* w = static_cast<uint32_t*>(p);
  for (size_t i = threadIdx.x; i < bytes / 4; i += blockDim.x) w[i] = 0xffffffffu;
}
__device__ __forceinline__ void lds_poison_done() { __syncthreads(); }
#else
__device__ __forceinline__ void lds_poison(void*, size_t) {}
__device__ __forceinline__ void lds_poison_done() {}
#endif

}  // namespace cdna4

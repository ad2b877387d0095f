// Device-side building blocks shared by the gfx950 attention kernels.
//
// MFMA tile shapes used here (CDNA4, wave64):
//   v_mfma_f32_32x32x16_bf16: A is 32(m) x 16(k), B is 16(k) x 32(n), C is
//   32 x 32 fp32.  Lane l holds A[m = l%32][k-group l/32] (8 bf16), B[k-group
//   l/32][n = l%32] (8 bf16) and C rows m = 8*(r/4) + 4*(l/32) + r%4 of column
//   n = l%32 in its 16 result registers r.
// The contraction index k may be permuted freely as long as A and B agree, so
// every kernel chooses the k order that makes its memory reads contiguous and
// lets an accumulator be reused as the next product's B operand without a
// round trip through LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma_32x32x16_bf16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// fp32 pair -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Low 16-bit halves of a and b packed as (a.lo, b.lo); high halves likewise.
__device__ __forceinline__ uint32_t pack_lo16(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi16(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Exchange with the lane 32 positions away (the other half of the wave).
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

template <typename T>
__device__ __forceinline__ T ldg(const void* p) {
  return *reinterpret_cast<const T*>(p);
}
template <typename T>
__device__ __forceinline__ void stg(void* p, T v) {
  *reinterpret_cast<T*>(p) = v;
}
template <typename T>
__device__ __forceinline__ T lds_read(const char* base, int off) {
  return *reinterpret_cast<const T*>(base + off);
}
template <typename T>
__device__ __forceinline__ void lds_write(char* base, int off, T v) {
  *reinterpret_cast<T*>(base + off) = v;
}

}  // namespace fa

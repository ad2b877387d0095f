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

// Accumulating product with the accumulator pinned to the accumulation
// registers (AGPRs), for long-lived accumulators (O in the forward, dK/dV in
// the backward).  Left to itself the compiler assigns MFMA results to one
// register file for the whole kernel and, when the short-lived products
// (whose results feed VALU work) compete for it, shuffles the long-lived
// accumulators between files around every product.  The hardware needs two
// wait states between a VALU write of an operand (or of the accumulator) and
// its read by a matrix instruction, and the compiler does not look inside
// inline assembly for that hazard: callers pass only operands produced well
// before the product (fragments from LDS reads, whose waits the compiler
// inserts as for any other use, and bf16 values packed in an earlier phase).
// A CPU test compiles the kernels to assembly and checks that no VALU
// instruction writes a register of a pinned product in the two instructions
// before it.
__device__ __forceinline__ void mfma_acc_pinned(f32x16& c, u32x4 a, u32x4 b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
// Wait states between the last pinned product into c and any read of c by a
// non-matrix instruction (more than the 19 the longest product needs).
__device__ __forceinline__ void mfma_acc_drain(f32x16& c) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(c));
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

// max / sum of x over lanes l and l^32, in every lane (v_permlane32_swap:
// one result holds the lower half's values, the other the upper half's).
__device__ __forceinline__ float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

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

// Work order of query-tile work units.  Workgroups are dealt round-robin over
// the 8 XCDs (workgroup t runs on XCD t % 8), each with its own L2.  Causal:
// longest first ([L21] slides 27-46), consecutive units walking the (b,h)
// index fastest, so that the units of one (b,h) land on the same XCD and
// share K/V in its L2.  Equal-cost units (not causal, BH a multiple of 8):
// XCD x takes every query tile of (b,h) x, then of x + 8, ..., so that its
// compute units stream one (b,h)'s K/V at the same time instead of several
// (b,h)'s at once.
constexpr int kXcds = 8;
__host__ __device__ inline void query_tile_of(int t, int BH, int nqt, bool causal, int* bh,
                                              int* qt) {
  if (!causal && BH % kXcds == 0) {
    const int j = t / kXcds;
    *bh = t % kXcds + kXcds * (j / nqt);
    *qt = j % nqt;
    return;
  }
  *bh = t % BH;
  *qt = causal ? (nqt - 1 - t / BH) : (t / BH);
}

// Persistent grids: workgroup w of G takes the positions of the longest-first
// unit list in snake order, w, 2G-1-w, 2G+w, 4G-1-w, ... (round i).  On a
// list sorted by non-increasing cost this pairs the longest remaining units
// of one round with the shortest of the next ([L21] slides 26-46: a
// persistent grid whose work is handed out longest first).  Positions grow
// with i, so a workgroup stops at its first position past the list.
__host__ __device__ inline int persistent_position(int i, int w, int G) {
  const int r = i >> 1;
  return (i & 1) ? (2 * r + 2) * G - 1 - w : 2 * r * G + w;
}

template <int N>
struct IntConst {
  static constexpr int value = N;
};

// ---------------------------------------------------------------------------
// Direct global -> LDS loads and transposing LDS reads (gfx950).

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

// Buffer resource over [base, base + bytes): loads past the end return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// One wave copies 64 x 16 bytes: lane i reads rsrc[voff_i + soff] and writes
// LDS bytes [lds + 16*i, lds + 16*i + 16).  `lds` must be wave-uniform.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, char* lds, int voff,
                                                  int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, voff, soff, 0, 0);
}
// The same with 4 bytes per lane: LDS bytes [lds + 4*i, lds + 4*i + 4).
__device__ __forceinline__ void buffer_load_lds4(__amdgpu_buffer_rsrc_t r, char* lds, int voff,
                                                 int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 4, voff, soff, 0, 0);
}

// Waits for this wave's vector-memory loads, issued through the builtin so
// that the compiler's own wait bookkeeping knows about them (it then does not
// re-wait for loads these calls have already covered).  The empty asm
// statements pin each wait between the loads around it.
constexpr int vmcnt_wait_bits(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  // at most N loads outstanding (they complete in issue order for this counter)
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(vmcnt_wait_bits(N));
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void wait_vmem() { wait_vmem_le<0>(); }
// Make the compiler wait for a register loaded from memory here.  Placed
// before a main loop for the loads issued ahead of it (register operands),
// so that the compiler does not carry them as pending across the loop
// back-edge and wait for them inside the loop, where that wait would also
// wait for the prefetches.
template <typename T>
__device__ __forceinline__ void settle(const T& x) {
  asm volatile("" ::"v"(x));
}
// Workgroup barrier for LDS tiles: this wave's LDS reads have returned, then
// s_barrier.  Outstanding direct-to-LDS loads are waited for separately.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ds_read_b64_tr_b16: within each group of 16 lanes, output lane i element e
// is element (i % 4) of the 8-byte chunk addressed by lane 4*e + i/4.
__device__ __forceinline__ u32x2 lds_read_tr16(const char* p) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p);
  return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ float fdot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// ---------------------------------------------------------------------------
// fp8 operands (gfx950 32x32x64 scaled MFMA).
//   v_mfma_scale_f32_32x32x64_f8f6f4: lane l holds 32 bytes of A row m = l%32
//   (B column n = l%32); bytes 0-15 belong to k-block 0 and bytes 16-31 to
//   k-block 1 (32 k each), the lane half l/32 choosing which 16 of each
//   block's 32 k it holds.  The block scale of A (row m, k-block kb) is byte 0
//   (e8m0: 2^(byte - 127)) of lane m + 32*kb's scale operand, and likewise
//   for B.  Within a block, k may be permuted freely as long as A and B agree.

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2_t;

// Both operands e4m3, unit block scales (e8m0 byte 127 is 2^0).
__device__ __forceinline__ f32x16 mfma_32x32x64_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
// A e4m3, B e5m2, per-lane e8m0 block scales sa, sb (byte 0).
__device__ __forceinline__ f32x16 mfma_32x32x64_fp8_bf8_scaled(i32x8 a, i32x8 b, f32x16 c,
                                                               int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 1, 0, sa, 0, sb);
}
// A e5m2, B e4m3, scales sa, sb, into an accumulator pinned to the
// accumulation registers (as mfma_acc_pinned).  The wait states the hardware
// needs between a VALU write of an operand or scale and its read by the
// product are placed inside the statement (s_nop 4: five), since the compiler
// does not look inside it.
__device__ __forceinline__ void mfma_scale_bf8_fp8_pinned(f32x16& c, i32x8 a, i32x8 b, int sa,
                                                          int sb) {
  asm("s_nop 4\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0] cbsz:1"
      : "+a"(c)
      : "v"(a), "v"(b), "v"(sa), "v"(sb));
}

// Four fp32 values (already within +-448) -> four e4m3 codes, value i in
// byte i (round to nearest even).  Each conversion writes one 16-bit half
// and keeps the other, and the two together write both, so the register
// they start from is arbitrary: a's bits, which lets the result take a's
// register (a zero there would cost a move per call).
__device__ __forceinline__ int cvt_fp8x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __float_as_int(a), false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}
// The same, starting from a register the caller names (one whose value is
// dead, where a itself is still read afterwards).
__device__ __forceinline__ int cvt_fp8x4_from(int start, float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, start, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}
// Four fp32 values (within +-57344) -> four e5m2 codes, value i in byte i
// (round to nearest even); the starting register as in cvt_fp8x4.
__device__ __forceinline__ int cvt_bf8x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, __float_as_int(a), false);
  return __builtin_amdgcn_cvt_pk_bf8_f32(c, d, lo, true);
}

// Power-of-two block scale: the smallest e with amax <= fmt_max * 2^e (0 for
// amax = 0), kept >= -126 (so that 2^e is a normal float, and its e8m0 code
// e + 127 is at least 1).  fmt_max = 0.875 * 2^T (T = 9 for e4m3's 448, 16 for
// e5m2's 57344): with amax = 1.f * 2^(E-127), amax <= 0.875 * 2^(T+e) holds
// from e = E - 127 - T + 1 when 1.f <= 1.75 and from one more otherwise.
// Subnormal maxima fall to the clamp.
template <int T>
__device__ __forceinline__ int pow2_block_exp(float amax) {
  const uint32_t u = __float_as_uint(amax);
  const int E = (int)(u >> 23);
  const int e = E - 126 - T + ((u & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return amax > 0.f ? (e > -126 ? e : -126) : 0;
}
// 2^-e as a float, for -126 <= e <= 126.
__device__ __forceinline__ float exp2_neg(int e) { return __int_as_float((127 - e) << 23); }
// 2^e as a float, for -126 <= e <= 127.
__device__ __forceinline__ float exp2_pos(int e) { return __int_as_float((127 + e) << 23); }

typedef short s16x2_t __attribute__((ext_vector_type(2)));
// Four fp32 values -> four e5m2 codes of x / s (s a power of two, the
// quotients within +-57344), value i in byte i: v_cvt_scalef32_pk_bf8_f32
// divides by its scale operand exactly for a power of two and rounds to
// nearest even, like cvt_bf8x4 on the quotients.
__device__ __forceinline__ int cvt_bf8x4_div(float a, float b, float c, float d, float s) {
  // (starting register as in cvt_fp8x4)
  s16x2_t r = __builtin_bit_cast(s16x2_t, __float_as_int(a));
  r = __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(r, a, b, s, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(r, c, d, s, true);
  return __builtin_bit_cast(int, r);
}

// Chunk swizzle of an fp8 tile (128-byte rows, 16-byte chunks) read through
// the transposing byte read below (two lanes per row, 8 rows, one chunk per
// lane pair): the read pattern spreads over all 64 banks.
__device__ __forceinline__ int f8_swz_t(int r) { return 2 * (((r >> 1) & 1) | (((r >> 3) & 1) << 1)); }

// ds_read_b64_tr_b8: within each group of 16 lanes, lanes 2r and 2r+1 address
// the two 8-byte halves of row r (r = 0..7) of an 8 x 16-byte tile, and output
// lane i receives byte i of rows 0..7 (byte k of the result from row k).
__device__ __forceinline__ i32x2_t lds_read_tr8(const char* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t*)p);
}

}  // namespace fa

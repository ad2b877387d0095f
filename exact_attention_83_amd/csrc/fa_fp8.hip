// FP8 path for gfx950: quantisation pre-pass and the e4m3 forward.
//
// Method: [CH18] "第 18 章 FlashAttention" §18.6.2 (1)(2) (E4M3 operands with
// range +-448 and a per-block scale s = amax/448, FP32 accumulation and
// softmax) and [L21] "CMU 11-868 L21 FlashAttention" slide 24 (incoherent
// processing: Q and K are multiplied by the same random orthogonal matrix
// J = diag(sign) H / sqrt(d); (QJ)(KJ)^T = QK^T while outliers are spread over
// the whole row).
//
// Quantiser, one workgroup (128 threads) per (b, h, 128-row block): the block
// is staged through LDS with coalesced loads, each thread then owns one row,
// applies the sign flip and an in-register fast Walsh-Hadamard transform, the
// block's amax is reduced across the workgroup, and the codes are written
// through LDS with coalesced stores.
//
// Forward: the bf16 kernel's structure (S^T = K Q^T with queries on the MFMA
// n axis, P^T reused as the B operand of O^T += V^T P^T) on the gfx950
// 32x32x64 fp8 MFMA.  Per-block scales fold into the exp2 argument (Q, K) and
// into the running-output rescale factor (V).  P is rounded to e4m3 after
// multiplication by 2^8, which keeps small probabilities out of the subnormal
// range; the factor cancels in O / l.

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x16 mfma_32x32x64_fp8(i32x8 a, i32x8 b, f32x16 c) {
  // unit block scales: the e8m0 exponent 127 is 2^0
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Four fp32 values (already within +-448) -> four e4m3 codes, value i in byte i.
__device__ __forceinline__ int cvt_fp8x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

constexpr int kQBlk = 128;  // rows per quantisation block

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(128) void quantize_fp8_kernel(const uint16_t* __restrict__ X,
                                                           const int8_t* __restrict__ signs,
                                                           uint8_t* __restrict__ X8,
                                                           float* __restrict__ scales, int N,
                                                           int nblk) {
  constexpr int D = 128;
  constexpr int IP = D * 2 + 16;  // bf16 staging pitch
  constexpr int OP = D + 16;      // code staging pitch
  __shared__ __attribute__((aligned(16))) char stage[kQBlk * IP];
  __shared__ float wmax[2];
  const int tid = threadIdx.x;
  const int bh = blockIdx.x / nblk;
  const int blk = blockIdx.x - bh * nblk;
  const int r0 = blk * kQBlk;
  const int rows = min(kQBlk, N - r0);
  const uint16_t* xp = X + ((size_t)bh * N + r0) * D;
  uint8_t* yp = X8 + ((size_t)bh * N + r0) * D;

  // coalesced block load: 16 chunks of 16 bytes per row
  for (int c = tid; c < kQBlk * 16; c += 128) {
    const int r = c >> 4, col = c & 15;
    u32x4 v = r < rows ? ldg<u32x4>(xp + (size_t)r * D + col * 8) : u32x4{0, 0, 0, 0};
    lds_write<u32x4>(stage, r * IP + col * 16, v);
  }
  __syncthreads();

  float x[D];
#pragma unroll
  for (int c = 0; c < D / 8; ++c) {
    u32x4 v = lds_read<u32x4>(stage, tid * IP + c * 16);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      x[c * 8 + 2 * w] = bf16_lo(v[w]);
      x[c * 8 + 2 * w + 1] = bf16_hi(v[w]);
    }
  }
  if (signs) {
#pragma unroll
    for (int i = 0; i < D; ++i) x[i] = signs[i] < 0 ? -x[i] : x[i];
    // natural-order fast Walsh-Hadamard transform (Sylvester H_128)
#pragma unroll
    for (int len = 1; len < D; len <<= 1)
#pragma unroll
      for (int i = 0; i < D; i += 2 * len)
#pragma unroll
        for (int j = i; j < i + len; ++j) {
          const float a = x[j], b = x[j + len];
          x[j] = a + b;
          x[j + len] = a - b;
        }
    const float inv_sqrt = 0.088388347648318440550f;  // 1/sqrt(128)
#pragma unroll
    for (int i = 0; i < D; ++i) x[i] *= inv_sqrt;
  }
  float amax = 0.f;
  if (tid < rows) {
#pragma unroll
    for (int i = 0; i < D; ++i) amax = fmaxf(amax, fabsf(x[i]));
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
  if ((tid & 63) == 0) wmax[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(wmax[0], wmax[1]);
  const bool zero = amax == 0.f;
  const float r = zero ? 0.f : 448.f / amax;

  // codes for this thread's row -> LDS (reusing the staging buffer)
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    int w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        v[e] = fminf(fmaxf(x[c * 16 + q * 4 + e] * r, -448.f), 448.f);
      w[q] = cvt_fp8x4(v[0], v[1], v[2], v[3]);
    }
    lds_write<u32x4>(stage, tid * OP + c * 16,
                     u32x4{(uint32_t)w[0], (uint32_t)w[1], (uint32_t)w[2], (uint32_t)w[3]});
  }
  __syncthreads();
  for (int c = tid; c < kQBlk * 8; c += 128) {
    const int rr = c >> 3, col = c & 7;
    if (rr < rows) stg<u32x4>(yp + (size_t)rr * D + col * 16, lds_read<u32x4>(stage, rr * OP + col * 16));
  }
  if (tid == 0) scales[blockIdx.x] = zero ? 1.f : amax / 448.f;
}

// ---------------------------------------------------------------------------
namespace {
constexpr int kF8Br = 128;
constexpr int kF8Bc = 64;
}  // namespace

template <bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fwd_fp8_kernel(
    const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ V,
    const float* __restrict__ QS, const float* __restrict__ KS, const float* __restrict__ VS,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int Hq, int Hkv, int Nq, int Nk,
    float scale_log2, int BH, int nqt) {
  constexpr int D = 128;
  constexpr int BC = kF8Bc;
  constexpr int KP = D + 16;      // K row pitch (bytes)
  constexpr int VP = BC + 4;      // V^T row pitch (bytes)
  constexpr int KSLOT = BC * KP;
  constexpr int VSLOT = D * VP;
  constexpr int DBLK = D / 32;
  __shared__ __attribute__((aligned(16))) char smem[2 * (KSLOT + VSLOT)];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  const int bh = blockIdx.x % BH;
  const int qt = CAUSAL ? (nqt - 1 - blockIdx.x / BH) : (blockIdx.x / BH);
  const int b = bh / Hq;
  const int h = bh - b * Hq;
  const int hk = h / (Hq / Hkv);
  const int bhk = b * Hkv + hk;
  const uint8_t* Qp = Q + (size_t)bh * Nq * D;
  const uint8_t* Kp = K + (size_t)bhk * Nk * D;
  const uint8_t* Vp = V + (size_t)bhk * Nk * D;
  const int nkb = (Nk + kQBlk - 1) / kQBlk;

  const int q0 = qt * kF8Br;
  const int qrow = q0 + wave * 32 + l32;
  const int qrow_c = qrow < Nq ? qrow : Nq - 1;
  const float sq = QS[(size_t)bh * ((Nq + kQBlk - 1) / kQBlk) + qt];

  // Q8 fragments: k-step s, lane half hf holds head dims 64*s + 32*hf .. +32.
  i32x8 qf[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const uint8_t* p = Qp + (size_t)qrow_c * D + s * 64 + hf * 32;
    u32x4 a = ldg<u32x4>(p), c = ldg<u32x4>(p + 16);
    qf[s] = i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)c[0], (int)c[1], (int)c[2], (int)c[3]};
  }

  const int kv_end = CAUSAL ? min(Nk, q0 + kF8Br) : Nk;
  const int ntiles = (kv_end + BC - 1) / BC;

  // staging: K 2 chunks/thread; V: 128 threads x (4 keys x 16 bytes)
  u32x4 kreg[2], vreg[4];
  const int v_rg = tid >> 3;   // 0..31 for tid < 128 -> keys 4*v_rg..
  const int v_col = tid & 7;   // 16-byte column
  const bool v_active = tid < 128;
  auto load_tile = [&](int j) {
    const int kv0 = j * BC;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i;
      const int row = c >> 3, col = c & 7;
      int key = kv0 + row;
      key = key < Nk ? key : Nk - 1;
      kreg[i] = ldg<u32x4>(Kp + (size_t)key * D + col * 16);
    }
    if (v_active) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int key = kv0 + (v_rg & 15) * 4 + i;
        key = key < Nk ? key : Nk - 1;
        // threads 0..127: 16 key groups x 8 columns
        vreg[i] = ldg<u32x4>(Vp + (size_t)key * D + v_col * 16);
      }
    }
  };
  auto store_tile = [&](int slot) {
    char* ks = smem + slot * (KSLOT + VSLOT);
    char* vs = ks + KSLOT;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i;
      const int row = c >> 3, col = c & 7;
      lds_write<u32x4>(ks, row * KP + col * 16, kreg[i]);
    }
    if (v_active) {
      const int rg = v_rg & 15;
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // byte e of word w of each of the 4 key rows -> one dword of 4 keys
          const uint32_t sel = 0x0c0c0000u | ((e + 4) << 8) | e;  // (k0.e, k1.e, 0, 0)
          const uint32_t lo = __builtin_amdgcn_perm(vreg[1][w], vreg[0][w], sel);
          const uint32_t hi = __builtin_amdgcn_perm(vreg[3][w], vreg[2][w], sel);
          const uint32_t v4 = (lo & 0xffffu) | (hi << 16);
          lds_write<uint32_t>(vs, (v_col * 16 + w * 4 + e) * VP + rg * 4, v4);
        }
    }
  };

  f32x16 o[DBLK];
#pragma unroll
  for (int i = 0; i < DBLK; ++i) o[i] = f32x16{0};
  float m_run = -INFINITY;  // running max in log2 units
  float l_run = 0.f;
  float sv_prev = 1.f;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int slot = j & 1;
    if (j + 1 < ntiles) load_tile(j + 1);
    const char* ks = smem + slot * (KSLOT + VSLOT);
    const char* vs = ks + KSLOT;
    const int kv0 = j * BC;
    const int kblk = kv0 / kQBlk;
    const float cj = sq * KS[(size_t)bhk * nkb + kblk] * scale_log2;
    const float sv = VS[(size_t)bhk * nkb + kblk];

    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{0};
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int off = (kb * 32 + l32) * KP + st * 64 + hf * 32;
        u32x4 a0 = lds_read<u32x4>(ks, off), a1 = lds_read<u32x4>(ks, off + 16);
        i32x8 a = i32x8{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                        (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
        s[kb] = mfma_32x32x64_fp8(a, qf[st], s[kb]);
      }
    }
    const bool need_mask = (kv0 + BC > Nk) || (CAUSAL && kv0 + BC - 1 > q0 + wave * 32);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + kb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
          if (key >= Nk || (CAUSAL && key > qrow)) s[kb][r] = -INFINITY;
        }
    }
    float mt = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kb][r]);
    mt = fmaxf(mt, xor32(mt)) * cj;
    const float m_new = fmaxf(m_run, mt);
    const float m_ref = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_ref);
    const float bias = 8.f - m_ref;  // P is produced as 2^8 * p
    m_run = m_new;
    // O is kept in units of the current tile's V scale.
    const float f = alpha * (sv_prev / sv);
    sv_prev = sv;
#pragma unroll
    for (int i = 0; i < DBLK; ++i) o[i] *= f;

    float psum = 0.f;
    int pw[8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float p[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          p[e] = fast_exp2(fmaf(s[kb][4 * g + e], cj, bias));
          psum += p[e];
        }
        pw[kb * 4 + g] = cvt_fp8x4(p[0], p[1], p[2], p[3]);
      }
    l_run = l_run * alpha + psum;
    // B element i = 16*kb + 4*g + e of lane half hf is key kb*32 + 8*g + 4*hf + e.
    const i32x8 pb = i32x8{pw[0], pw[1], pw[2], pw[3], pw[4], pw[5], pw[6], pw[7]};
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
      int a[8];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          a[kb * 4 + g] = (int)lds_read<uint32_t>(vs, (db * 32 + l32) * VP + kb * 32 + g * 8 + hf * 4);
      o[db] = mfma_32x32x64_fp8(i32x8{a[0], a[1], a[2], a[3], a[4], a[5], a[6], a[7]}, pb, o[db]);
    }
    if (j + 1 < ntiles) store_tile(slot ^ 1);
    __syncthreads();
  }

  const float l_tot = l_run + xor32(l_run);
  const float inv = sv_prev / l_tot;
  if (qrow < Nq) {
    uint16_t* Op = O + ((size_t)bh * Nq + qrow) * D;
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = db * 32 + g * 8 + hf * 4;
        stg<u32x2>(Op + d0, u32x2{pack_bf16(o[db][4 * g] * inv, o[db][4 * g + 1] * inv),
                                  pack_bf16(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv)});
      }
    if (hf == 0) LSE[(size_t)bh * Nq + qrow] = (m_run - 8.f) * kLn2 + __logf(l_tot);
  }
}

hipError_t launch_quantize_fp8(const void* x, const int8_t* signs, uint8_t* x8, float* scales,
                               int B, int H, int N, int d, hipStream_t stream) {
  const int nblk = (N + kQBlk - 1) / kQBlk;
  hipLaunchKernelGGL(quantize_fp8_kernel, dim3(B * H * nblk), dim3(128), 0, stream,
                     (const uint16_t*)x, signs, x8, scales, N, nblk);
  return hipGetLastError();
}

hipError_t launch_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                          const float* qs, const float* ks, const float* vs, void* o,
                          float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                          float scale, bool causal, hipStream_t stream) {
  const int BH = B * Hq;
  const int nqt = (Nq + kF8Br - 1) / kF8Br;
  dim3 grid(BH * nqt), block(256);
  const float sl2 = scale * kLog2e;
  if (causal)
    hipLaunchKernelGGL((fwd_fp8_kernel<true>), grid, block, 0, stream, q8, k8, v8, qs, ks, vs,
                       (uint16_t*)o, lse, Hq, Hkv, Nq, Nk, sl2, BH, nqt);
  else
    hipLaunchKernelGGL((fwd_fp8_kernel<false>), grid, block, 0, stream, q8, k8, v8, qs, ks, vs,
                       (uint16_t*)o, lse, Hq, Hkv, Nq, Nk, sl2, BH, nqt);
  return hipGetLastError();
}

}  // namespace fa

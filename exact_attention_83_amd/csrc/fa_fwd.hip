// Forward attention kernels for gfx950.
//
// Method: [CH18] "第 18 章 FlashAttention" §18.4.3 (tiled forward, Fig. 18-16)
// and §18.5.1-18.5.2 (work split per query tile, causal tile skipping); the
// rescaling step is the two-block identity of [L21] "CMU 11-868 L21
// FlashAttention" slide 12.
//
// bf16 kernel layout (one workgroup = 4 waves = 128 query rows, KV tiles of 64
// keys):
//   * each wave owns 32 query rows.  It computes S^T = K Q^T with the keys on
//     the MFMA m axis and its queries on the n axis, so every lane owns one
//     query column: the row max is an in-register reduction plus one exchange
//     with the other wave half, and the rescale factor is lane-local.
//   * Q stays in registers for the whole tile as the B operand.
//   * P^T (the S^T accumulator rounded to bf16) is directly the B operand of
//     O^T += V^T P^T: the keys of the accumulator become the k index of the
//     next product.  V^T comes from LDS, where V is stored transposed.
//   * K and V^T tiles are double-buffered in LDS; the next tile's global loads
//     are issued before the current tile's math so their latency is hidden.
//   * exp is exp2 with scale*log2(e) folded into one FMA; O is divided by the
//     row sum once at the end ([CH18] §18.4.3 step 9).

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kFwdWaves = 4;
constexpr int kFwdBr = 32 * kFwdWaves;  // query rows per workgroup
constexpr int kFwdBc = 64;              // keys per KV tile

}  // namespace

// Dispatch order of the forward's work units: longest first for causal
// ([L21] slides 27-46).  Consecutive units walk the (b,h) index fastest, so
// units of one (b,h) land on the same XCD (workgroups are dealt round-robin
// over the 8 XCDs) and share K/V in its L2.
__host__ __device__ inline void fwd_tile_of(int t, int BH, int nqt, bool causal, int* bh,
                                            int* qt) {
  *bh = t % BH;
  *qt = causal ? (nqt - 1 - t / BH) : (t / BH);
}

int fwd_kv_tiles(int qt, int Nk, bool causal, int br, int bc) {
  int last = causal ? ((qt + 1) * br < Nk ? (qt + 1) * br : Nk) : Nk;
  return (last + bc - 1) / bc;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE,
    int Hq, int Hkv, int Nq, int Nk, float scale, float scale_log2, int BH, int nqt) {
  constexpr int BC = kFwdBc;
  constexpr int KP = D * 2 + 16;   // K row pitch in LDS (bytes): conflict-free b128 reads
  constexpr int VP = BC * 2 + 8;   // V^T row pitch in LDS (bytes): conflict-free b64 reads
  constexpr int KSLOT = BC * KP;
  constexpr int VSLOT = D * VP;
  constexpr int KCH = BC * D / 8 / 256;  // 16-byte K chunks per thread per tile
  constexpr int DCH = D / 8;             // 16-byte chunks per row
  constexpr int KSTEPS = D / 16;         // MFMA k-steps over the head dim
  constexpr int DBLK = D / 32;           // 32-wide blocks of the head dim
  __shared__ __attribute__((aligned(16))) char smem[2 * (KSLOT + VSLOT)];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  int bh, qt;
  fwd_tile_of(blockIdx.x, BH, nqt, CAUSAL, &bh, &qt);
  const int b = bh / Hq;
  const int h = bh - b * Hq;
  const int hk = h / (Hq / Hkv);
  const uint16_t* Qp = Q + (size_t)bh * Nq * D;
  const uint16_t* Kp = K + (size_t)(b * Hkv + hk) * Nk * D;
  const uint16_t* Vp = V + (size_t)(b * Hkv + hk) * Nk * D;

  const int q0 = qt * kFwdBr;
  const int qrow = q0 + wave * 32 + l32;
  const int qrow_c = qrow < Nq ? qrow : Nq - 1;

  // Q fragments (B operand of S^T = K Q^T): k-step ks covers head dims
  // 16*ks + 8*hf .. +8.
  u32x4 qf[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks)
    qf[ks] = ldg<u32x4>(Qp + (size_t)qrow_c * D + ks * 16 + hf * 8);

  const int kv_end = CAUSAL ? min(Nk, q0 + kFwdBr) : Nk;
  const int ntiles = (kv_end + BC - 1) / BC;

  // Global -> register staging for one K/V tile.
  u32x4 kreg[KCH];
  u32x4 vreg[4];
  // V is read in groups of 4 consecutive keys x 8 head dims per thread so that
  // it can be written transposed as 8-byte runs of keys.
  const int v_rg = tid / DCH;          // key group (4 keys)
  const int v_col = tid - v_rg * DCH;  // 16-byte column chunk
  const bool v_active = v_rg < BC / 4;

  auto load_tile = [&](int j) {
    const int kv0 = j * BC;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      int c = tid + 256 * i;
      int row = c / DCH, col = c - row * DCH;
      int key = kv0 + row;
      key = key < Nk ? key : Nk - 1;
      kreg[i] = ldg<u32x4>(Kp + (size_t)key * D + col * 8);
    }
    if (v_active) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int key = kv0 + v_rg * 4 + i;
        key = key < Nk ? key : Nk - 1;
        vreg[i] = ldg<u32x4>(Vp + (size_t)key * D + v_col * 8);
      }
    }
  };
  auto store_tile = [&](int slot) {
    char* ks = smem + slot * (KSLOT + VSLOT);
    char* vs = ks + KSLOT;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      int c = tid + 256 * i;
      int row = c / DCH, col = c - row * DCH;
      lds_write<u32x4>(ks, row * KP + col * 16, kreg[i]);
    }
    if (v_active) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e >> 1;
        uint32_t lo, hi;
        if (e & 1) {
          lo = pack_hi16(vreg[0][w], vreg[1][w]);
          hi = pack_hi16(vreg[2][w], vreg[3][w]);
        } else {
          lo = pack_lo16(vreg[0][w], vreg[1][w]);
          hi = pack_lo16(vreg[2][w], vreg[3][w]);
        }
        lds_write<u32x2>(vs, (v_col * 8 + e) * VP + v_rg * 8, u32x2{lo, hi});
      }
    }
  };

  f32x16 o[DBLK];
#pragma unroll
  for (int i = 0; i < DBLK; ++i) o[i] = f32x16{0};
  float m_run = -INFINITY;  // running max of raw q.k (unscaled)
  float l_run = 0.f;        // this lane's share of the running row sum

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int slot = j & 1;
    if (j + 1 < ntiles) load_tile(j + 1);
    const char* ks = smem + slot * (KSLOT + VSLOT);
    const char* vs = ks + KSLOT;
    const int kv0 = j * BC;

    // S^T for the wave: two 32-key blocks x 32 queries.
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{0};
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        u32x4 a = lds_read<u32x4>(ks, (kb * 32 + l32) * KP + (kk * 16 + hf * 8) * 2);
        s[kb] = mfma_32x32x16_bf16(a, qf[kk], s[kb]);
      }
    }

    // Mask keys past the end (ragged tail) and, on diagonal tiles, keys after
    // the query ([CH18] §18.5.2: only tiles crossing the diagonal need it).
    const bool need_mask = (kv0 + BC > Nk) || (CAUSAL && kv0 + BC - 1 > q0 + wave * 32);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          int key = kv0 + kb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
          bool dead = key >= Nk || (CAUSAL && key > qrow);
          if (dead) s[kb][r] = -INFINITY;
        }
    }

    float mt = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kb][r]);
    mt = fmaxf(mt, xor32(mt));
    // A row with no visible key so far keeps m = -inf; use 0 as its reference
    // so that no (-inf) - (-inf) is ever formed.
    const float m_new = fmaxf(m_run, mt);
    const float m_ref = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2((m_run - m_ref) * scale_log2);
    const float mb = m_ref * scale_log2;
    m_run = m_new;

    float psum = 0.f;
    u32x4 pb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = fast_exp2(fmaf(s[kb][r], scale_log2, -mb));
        psum += p[r];
      }
#pragma unroll
      for (int st = 0; st < 2; ++st)
        pb[kb][st] = u32x4{pack_bf16(p[8 * st + 0], p[8 * st + 1]),
                           pack_bf16(p[8 * st + 2], p[8 * st + 3]),
                           pack_bf16(p[8 * st + 4], p[8 * st + 5]),
                           pack_bf16(p[8 * st + 6], p[8 * st + 7])};
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int i = 0; i < DBLK; ++i) o[i] *= alpha;

    // O^T += V^T P^T.  B element e of lane half hf in k-step (kb, st) is key
    // kb*32 + 16*st + 8*(e/4) + 4*hf + e%4 (the accumulator's row order).
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          int off = (db * 32 + l32) * VP + (kb * 32 + st * 16 + hf * 4) * 2;
          u32x2 a0 = lds_read<u32x2>(vs, off);
          u32x2 a1 = lds_read<u32x2>(vs, off + 16);
          o[db] = mfma_32x32x16_bf16(u32x4{a0[0], a0[1], a1[0], a1[1]}, pb[kb][st], o[db]);
        }

    if (j + 1 < ntiles) store_tile(slot ^ 1);
    __syncthreads();
  }

  // Epilogue: O = O^T / l, LSE = m*scale + ln l.
  const float l_tot = l_run + xor32(l_run);
  const float inv = 1.f / l_tot;
  if (qrow < Nq) {
    uint16_t* Op = O + ((size_t)bh * Nq + qrow) * D;
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        int d0 = db * 32 + g * 8 + hf * 4;
        stg<u32x2>(Op + d0, u32x2{pack_bf16(o[db][4 * g] * inv, o[db][4 * g + 1] * inv),
                                  pack_bf16(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv)});
      }
    if (hf == 0) LSE[(size_t)bh * Nq + qrow] = m_run * scale + __logf(l_tot);
  }
}

// ---------------------------------------------------------------------------
// fp32 forward (d = 64): plain VALU kernel, one query row per thread, 64-row
// query tiles and 64-key KV tiles staged in LDS.  Exact expf/logf keep the
// result within fp32 rounding of the definition.
constexpr int kF32D = 64;
constexpr int kF32B = 64;

__global__ __launch_bounds__(64) void fwd_f32_kernel(const float* __restrict__ Q,
                                                     const float* __restrict__ K,
                                                     const float* __restrict__ V,
                                                     float* __restrict__ O,
                                                     float* __restrict__ LSE, int Hq, int Hkv,
                                                     int Nq, int Nk, float scale, int causal) {
  constexpr int D = kF32D;
  __shared__ float ks[kF32B][D + 1];
  __shared__ float vs[kF32B][D + 1];
  const int bh = blockIdx.y;
  const int b = bh / Hq, h = bh - (bh / Hq) * Hq;
  const int hk = h / (Hq / Hkv);
  const int t = threadIdx.x;
  const int row = blockIdx.x * kF32B + t;
  const int rowc = row < Nq ? row : Nq - 1;
  const float* Kp = K + (size_t)(b * Hkv + hk) * Nk * D;
  const float* Vp = V + (size_t)(b * Hkv + hk) * Nk * D;
  float q[D], o[D];
  for (int c = 0; c < D; ++c) {
    q[c] = Q[((size_t)bh * Nq + rowc) * D + c];
    o[c] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int kv_end = causal ? min(Nk, (int)(blockIdx.x + 1) * kF32B) : Nk;
  for (int j0 = 0; j0 < kv_end; j0 += kF32B) {
    __syncthreads();
    for (int i = t; i < kF32B * D; i += 64) {
      int r = i / D, c = i - (i / D) * D;
      int key = min(j0 + r, Nk - 1);
      ks[r][c] = Kp[(size_t)key * D + c];
      vs[r][c] = Vp[(size_t)key * D + c];
    }
    __syncthreads();
    float s[kF32B];
    float mt = -INFINITY;
    for (int j = 0; j < kF32B; ++j) {
      float acc = 0.f;
      for (int c = 0; c < D; ++c) acc = fmaf(q[c], ks[j][c], acc);
      const int key = j0 + j;
      s[j] = (key < Nk && (!causal || key <= row)) ? acc * scale : -INFINITY;
      mt = fmaxf(mt, s[j]);
    }
    const float mn = fmaxf(m, mt);
    const float a = expf(m - mn);
    l *= a;
    for (int c = 0; c < D; ++c) o[c] *= a;
    for (int j = 0; j < kF32B; ++j) {
      const float p = expf(s[j] - mn);
      l += p;
      for (int c = 0; c < D; ++c) o[c] = fmaf(p, vs[j][c], o[c]);
    }
    m = mn;
  }
  if (row < Nq) {
    for (int c = 0; c < D; ++c) O[((size_t)bh * Nq + row) * D + c] = o[c] / l;
    LSE[(size_t)bh * Nq + row] = m + logf(l);
  }
}

// ---------------------------------------------------------------------------

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                           bool causal, hipStream_t stream) {
  const int BH = B * Hq;
  const int nqt = (Nq + kFwdBr - 1) / kFwdBr;
  dim3 grid(BH * nqt), block(256);
  const float sl2 = scale * kLog2e;
  auto Qp = (const uint16_t*)q;
  auto Kp = (const uint16_t*)k;
  auto Vp = (const uint16_t*)v;
  auto Op = (uint16_t*)o;
  if (d == 128) {
    if (causal)
      hipLaunchKernelGGL((fwd_bf16_kernel<128, true>), grid, block, 0, stream, Qp, Kp, Vp, Op,
                         lse, Hq, Hkv, Nq, Nk, scale, sl2, BH, nqt);
    else
      hipLaunchKernelGGL((fwd_bf16_kernel<128, false>), grid, block, 0, stream, Qp, Kp, Vp, Op,
                         lse, Hq, Hkv, Nq, Nk, scale, sl2, BH, nqt);
  } else {
    if (causal)
      hipLaunchKernelGGL((fwd_bf16_kernel<64, true>), grid, block, 0, stream, Qp, Kp, Vp, Op,
                         lse, Hq, Hkv, Nq, Nk, scale, sl2, BH, nqt);
    else
      hipLaunchKernelGGL((fwd_bf16_kernel<64, false>), grid, block, 0, stream, Qp, Kp, Vp, Op,
                         lse, Hq, Hkv, Nq, Nk, scale, sl2, BH, nqt);
  }
  return hipGetLastError();
}

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          int B, int Hq, int Hkv, int Nq, int Nk, float scale, bool causal,
                          hipStream_t stream) {
  dim3 grid((Nq + kF32B - 1) / kF32B, B * Hq), block(64);
  hipLaunchKernelGGL(fwd_f32_kernel, grid, block, 0, stream, q, k, v, o, lse, Hq, Hkv, Nq, Nk,
                     scale, causal ? 1 : 0);
  return hipGetLastError();
}

int fwd_schedule(int B, int Hq, int Nq, int Nk, bool causal, int* bh_out, int* qt_out,
                 int* cost_out, int capacity) {
  const int BH = B * Hq;
  const int nqt = (Nq + kFwdBr - 1) / kFwdBr;
  const int n = BH * nqt;
  if (bh_out || qt_out || cost_out) {
    if (capacity < n) return -1;
    for (int t = 0; t < n; ++t) {
      int bh, qt;
      fwd_tile_of(t, BH, nqt, causal, &bh, &qt);
      if (bh_out) bh_out[t] = bh;
      if (qt_out) qt_out[t] = qt;
      if (cost_out) cost_out[t] = fwd_kv_tiles(qt, Nk, causal, kFwdBr, kFwdBc);
    }
  }
  return n;
}

}  // namespace fa

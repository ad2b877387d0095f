// Backward attention kernels for gfx950.
//
// Method: [CH18] "第 18 章 FlashAttention" §18.2.4 (gradients: dV = P^T dO,
// dP = dO V^T, dS = P * (dP - rowsum(P * dP)), dQ = dS K, dK = dS^T Q, each
// with one factor of the score scale) and §18.4.4 (recomputation: P is rebuilt
// tile by tile from the saved logsumexp, so no rescaling is needed; only O(N)
// row statistics are kept from the forward).  The row term rowsum(P * dP)
// equals dO_i . O_i, which a pre-pass computes from O and dO.
//
// bf16 main kernel, one workgroup per (b, KV head, 128-key tile):
//   * wave w owns keys kv0 + 32w .. +32.  Its K and V rows stay in registers
//     as MFMA B operands for S = Q K^T and dP = dO V^T (queries on the MFMA m
//     axis, keys on n), and it accumulates dK and dV for those keys in
//     registers over every query tile of every query head of the group.
//   * the S and dP accumulators (query rows in registers, one key per lane)
//     are directly the A operands of dV += P^T dO and dK += dS^T Q: their
//     query index becomes the contraction index.  The other operands, dO^T and
//     Q^T, are read from LDS where the query tile is also stored transposed.
//   * dQ needs the contraction over all 128 keys, so each wave writes its dS
//     block to LDS; after a barrier the waves split the 64 x d dQ tile, compute
//     it from dS and K^T (resident in LDS) and add it into the fp32
//     accumulator with atomics.
//   * the next query tile is fetched into registers while the current one is
//     processed.
// Causal: KV tile j only visits query tiles that reach its keys, and only the
// tiles crossing the diagonal are masked ([CH18] §18.5.2 (4): the skipped
// gradients are structurally zero).  Work units are launched in ascending KV
// tile order, i.e. longest first.

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

// ---------------------------------------------------------------------------
// delta_i = sum_c dO_ic * O_ic; also zeroes the fp32 dQ accumulator row.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const T* __restrict__ O,
                                                        const T* __restrict__ dO,
                                                        float* __restrict__ delta,
                                                        float* __restrict__ dq_accum,
                                                        int rows) {
  // 16 threads per row, each owns D/16 consecutive elements.
  constexpr int E = D / 16;
  const int row = blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  float acc = 0.f;
  if (row < rows) {
    const T* op = O + (size_t)row * D + sub * E;
    const T* gp = dO + (size_t)row * D + sub * E;
#pragma unroll
    for (int e = 0; e < E; ++e) acc = fmaf((float)op[e], (float)gp[e], acc);
    if (dq_accum) {
      float* zp = dq_accum + (size_t)row * D + sub * E;
#pragma unroll
      for (int e = 0; e < E; e += 4) stg<f32x4>(zp + e, f32x4{0.f, 0.f, 0.f, 0.f});
    }
  }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 16);
  if (row < rows && sub == 0) delta[row] = acc;
}

// dq_accum (fp32) -> dq (bf16), 8 elements per thread.
__global__ __launch_bounds__(256) void bwd_dq_convert_kernel(const float* __restrict__ acc,
                                                             uint16_t* __restrict__ dq,
                                                             size_t n8) {
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  f32x4 a = ldg<f32x4>(acc + i * 8);
  f32x4 b = ldg<f32x4>(acc + i * 8 + 4);
  stg<u32x4>(dq + i * 8, u32x4{pack_bf16(a[0], a[1]), pack_bf16(a[2], a[3]),
                               pack_bf16(b[0], b[1]), pack_bf16(b[2], b[3])});
}

// ---------------------------------------------------------------------------
// fp32 backward (d = 64), plain VALU, deterministic.
constexpr int kBF32D = 64;
constexpr int kBF32T = 64;

// dQ: one query row per thread.
__global__ __launch_bounds__(64) void bwd_f32_dq_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ LSE,
    const float* __restrict__ delta, float* __restrict__ dQ, int Hq, int Hkv, int Nq, int Nk,
    float scale, int causal) {
  constexpr int D = kBF32D;
  __shared__ float ks[kBF32T][D + 1];
  __shared__ float vs[kBF32T][D + 1];
  const int bh = blockIdx.y;
  const int b = bh / Hq, h = bh - (bh / Hq) * Hq;
  const int hk = h / (Hq / Hkv);
  const int t = threadIdx.x;
  const int row = blockIdx.x * kBF32T + t;
  const int rowc = row < Nq ? row : Nq - 1;
  const float* Kp = K + (size_t)(b * Hkv + hk) * Nk * D;
  const float* Vp = V + (size_t)(b * Hkv + hk) * Nk * D;
  float q[D], g[D], dq[D];
  for (int c = 0; c < D; ++c) {
    q[c] = Q[((size_t)bh * Nq + rowc) * D + c];
    g[c] = dO[((size_t)bh * Nq + rowc) * D + c];
    dq[c] = 0.f;
  }
  const float lse = LSE[(size_t)bh * Nq + rowc];
  const float dl = delta[(size_t)bh * Nq + rowc];
  const int kv_end = causal ? min(Nk, (int)(blockIdx.x + 1) * kBF32T) : Nk;
  for (int j0 = 0; j0 < kv_end; j0 += kBF32T) {
    __syncthreads();
    for (int i = t; i < kBF32T * D; i += 64) {
      int r = i / D, c = i - (i / D) * D;
      int key = min(j0 + r, Nk - 1);
      ks[r][c] = Kp[(size_t)key * D + c];
      vs[r][c] = Vp[(size_t)key * D + c];
    }
    __syncthreads();
    for (int j = 0; j < kBF32T; ++j) {
      const int key = j0 + j;
      if (key >= Nk || (causal && key > row)) continue;
      float s = 0.f, dp = 0.f;
      for (int c = 0; c < D; ++c) {
        s = fmaf(q[c], ks[j][c], s);
        dp = fmaf(g[c], vs[j][c], dp);
      }
      const float p = expf(s * scale - lse);
      const float ds = p * (dp - dl) * scale;
      for (int c = 0; c < D; ++c) dq[c] = fmaf(ds, ks[j][c], dq[c]);
    }
  }
  if (row < Nq)
    for (int c = 0; c < D; ++c) dQ[((size_t)bh * Nq + row) * D + c] = dq[c];
}

// dK, dV: one (key row, half of the head dim) per thread; sums over the query
// heads of the GQA group.
__global__ __launch_bounds__(64) void bwd_f32_dkv_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ LSE,
    const float* __restrict__ delta, float* __restrict__ dK, float* __restrict__ dV, int Hq,
    int Hkv, int Nq, int Nk, float scale, int causal) {
  constexpr int D = kBF32D;
  constexpr int HD = D / 2;
  __shared__ float qs[kBF32T][D + 1];
  __shared__ float gs[kBF32T][D + 1];
  __shared__ float ls[kBF32T], dls[kBF32T];
  const int bhk = blockIdx.y;
  const int b = bhk / Hkv, hk = bhk - (bhk / Hkv) * Hkv;
  const int G = Hq / Hkv;
  const int t = threadIdx.x;
  const int key = blockIdx.x * 32 + (t >> 1);
  const int half = t & 1;
  const int keyc = key < Nk ? key : Nk - 1;
  float k[D], v[D], dk[HD], dv[HD];
  for (int c = 0; c < D; ++c) {
    k[c] = K[((size_t)bhk * Nk + keyc) * D + c];
    v[c] = V[((size_t)bhk * Nk + keyc) * D + c];
  }
  for (int c = 0; c < HD; ++c) dk[c] = dv[c] = 0.f;
  const int q_begin = causal ? (int)(blockIdx.x * 32) / kBF32T * kBF32T : 0;
  for (int gi = 0; gi < G; ++gi) {
    const int bh = b * Hq + hk * G + gi;
    for (int i0 = q_begin; i0 < Nq; i0 += kBF32T) {
      __syncthreads();
      for (int i = t; i < kBF32T * D; i += 64) {
        int r = i / D, c = i - (i / D) * D;
        int qr = min(i0 + r, Nq - 1);
        qs[r][c] = Q[((size_t)bh * Nq + qr) * D + c];
        gs[r][c] = dO[((size_t)bh * Nq + qr) * D + c];
      }
      {
        int qr = min(i0 + t, Nq - 1);
        ls[t] = LSE[(size_t)bh * Nq + qr];
        dls[t] = delta[(size_t)bh * Nq + qr];
      }
      __syncthreads();
      for (int r = 0; r < kBF32T; ++r) {
        const int qi = i0 + r;
        if (qi >= Nq || (causal && key > qi)) continue;
        float s = 0.f, dp = 0.f;
        for (int c = 0; c < D; ++c) {
          s = fmaf(qs[r][c], k[c], s);
          dp = fmaf(gs[r][c], v[c], dp);
        }
        const float p = expf(s * scale - ls[r]);
        const float ds = p * (dp - dls[r]) * scale;
        for (int c = 0; c < HD; ++c) {
          dv[c] = fmaf(p, gs[r][half * HD + c], dv[c]);
          dk[c] = fmaf(ds, qs[r][half * HD + c], dk[c]);
        }
      }
    }
  }
  if (key < Nk)
    for (int c = 0; c < HD; ++c) {
      dK[((size_t)bhk * Nk + key) * D + half * HD + c] = dk[c];
      dV[((size_t)bhk * Nk + key) * D + half * HD + c] = dv[c];
    }
}

// ---------------------------------------------------------------------------
// bf16 main backward kernel.
namespace {
constexpr int kBwdBkv = 128;  // keys per workgroup (4 waves x 32)
constexpr int kBwdBq = 64;    // query rows per inner tile
}  // namespace

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ Delta,
    float* __restrict__ dq_accum, uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
    int Hq, int Hkv, int Nq, int Nk, float scale, float scale_log2, int BHkv) {
  constexpr int BQ = kBwdBq;
  constexpr int KSTEPS = D / 16;
  constexpr int DBLK = D / 32;
  constexpr int DCH = D / 8;                // 16-byte chunks per row
  constexpr int RP = D * 2 + 16;            // row-major tile pitch (Q, dO)
  constexpr int TP = BQ * 2 + 8;            // transposed tile pitch (Q^T, dO^T)
  constexpr int SP = kBwdBkv * 2 + 16;      // dS pitch [q][key]
  constexpr int KTP = kBwdBkv * 2 + 16;     // K^T pitch [d][key]
  constexpr int OFF_Q = 0;
  constexpr int OFF_QT = OFF_Q + BQ * RP;
  constexpr int OFF_G = OFF_QT + D * TP;
  constexpr int OFF_GT = OFF_G + BQ * RP;
  constexpr int OFF_L = OFF_GT + D * TP;    // lse * log2(e)
  constexpr int OFF_DL = OFF_L + BQ * 4;    // delta
  constexpr int OFF_S = OFF_DL + BQ * 4;
  constexpr int OFF_KT = OFF_S + BQ * SP;
  constexpr int SMEM = OFF_KT + D * KTP;
  __shared__ __attribute__((aligned(16))) char smem[SMEM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  const int t = blockIdx.x;
  const int bhk = t % BHkv;
  const int jt = t / BHkv;  // ascending KV tiles = longest first under causal
  const int b = bhk / Hkv;
  const int hk = bhk - b * Hkv;
  const int G = Hq / Hkv;
  const int kv0 = jt * kBwdBkv;
  const int mykey = kv0 + wave * 32 + l32;
  const int mykey_c = mykey < Nk ? mykey : Nk - 1;

  const uint16_t* Kp = K + (size_t)bhk * Nk * D;
  const uint16_t* Vp = V + (size_t)bhk * Nk * D;

  // Resident K, V fragments (B operands with n = key, k = head dim).
  u32x4 kf[KSTEPS], vf[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    kf[ks] = ldg<u32x4>(Kp + (size_t)mykey_c * D + ks * 16 + hf * 8);
    vf[ks] = ldg<u32x4>(Vp + (size_t)mykey_c * D + ks * 16 + hf * 8);
  }
  // K^T for the whole workgroup in LDS (B operand of dQ = dS K).
  {
    // thread: 4 keys x 8 head dims, written as 8-byte runs of keys.
    for (int gidx = tid; gidx < (kBwdBkv / 4) * DCH; gidx += 256) {
      const int rg = gidx / DCH, col = gidx - (gidx / DCH) * DCH;
      u32x4 r[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int key = kv0 + rg * 4 + i;
        key = key < Nk ? key : Nk - 1;
        r[i] = ldg<u32x4>(Kp + (size_t)key * D + col * 8);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e >> 1;
        uint32_t lo = (e & 1) ? pack_hi16(r[0][w], r[1][w]) : pack_lo16(r[0][w], r[1][w]);
        uint32_t hi = (e & 1) ? pack_hi16(r[2][w], r[3][w]) : pack_lo16(r[2][w], r[3][w]);
        lds_write<u32x2>(smem + OFF_KT, (col * 8 + e) * KTP + rg * 8, u32x2{lo, hi});
      }
    }
  }

  f32x16 dk[DBLK], dv[DBLK];
#pragma unroll
  for (int i = 0; i < DBLK; ++i) {
    dk[i] = f32x16{0};
    dv[i] = f32x16{0};
  }

  const int nqt = (Nq + BQ - 1) / BQ;
  const int qt_begin = CAUSAL ? kv0 / BQ : 0;
  const int per_head = nqt - qt_begin;
  const int total = per_head * G;

  // Query-tile staging: thread owns 4 consecutive rows x 8 head dims of Q and dO.
  const int st_rg = tid / DCH;                 // row group
  const int st_col = tid - st_rg * DCH;
  const bool st_active = st_rg < BQ / 4;
  u32x4 qreg[4], greg[4];
  float lreg = 0.f;

  auto tile_head = [&](int it, int* bh, int* q0) {
    const int gi = it / per_head;
    *bh = b * Hq + hk * G + gi;
    *q0 = (qt_begin + (it - gi * per_head)) * BQ;
  };
  auto load_q = [&](int it) {
    int bh, q0;
    tile_head(it, &bh, &q0);
    if (st_active) {
      const uint16_t* qp = Q + (size_t)bh * Nq * D;
      const uint16_t* gp = dO + (size_t)bh * Nq * D;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int r = q0 + st_rg * 4 + i;
        r = r < Nq ? r : Nq - 1;
        qreg[i] = ldg<u32x4>(qp + (size_t)r * D + st_col * 8);
        greg[i] = ldg<u32x4>(gp + (size_t)r * D + st_col * 8);
      }
    }
    if (tid < 2 * BQ) {
      int r = q0 + (tid & (BQ - 1));
      r = r < Nq ? r : Nq - 1;
      lreg = tid < BQ ? LSE[(size_t)bh * Nq + r] * kLog2e : Delta[(size_t)bh * Nq + r];
    }
  };
  auto store_q = [&]() {
    if (st_active) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lds_write<u32x4>(smem + OFF_Q, (st_rg * 4 + i) * RP + st_col * 16, qreg[i]);
        lds_write<u32x4>(smem + OFF_G, (st_rg * 4 + i) * RP + st_col * 16, greg[i]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e >> 1;
        uint32_t lo = (e & 1) ? pack_hi16(qreg[0][w], qreg[1][w]) : pack_lo16(qreg[0][w], qreg[1][w]);
        uint32_t hi = (e & 1) ? pack_hi16(qreg[2][w], qreg[3][w]) : pack_lo16(qreg[2][w], qreg[3][w]);
        lds_write<u32x2>(smem + OFF_QT, (st_col * 8 + e) * TP + st_rg * 8, u32x2{lo, hi});
        lo = (e & 1) ? pack_hi16(greg[0][w], greg[1][w]) : pack_lo16(greg[0][w], greg[1][w]);
        hi = (e & 1) ? pack_hi16(greg[2][w], greg[3][w]) : pack_lo16(greg[2][w], greg[3][w]);
        lds_write<u32x2>(smem + OFF_GT, (st_col * 8 + e) * TP + st_rg * 8, u32x2{lo, hi});
      }
    }
    if (tid < 2 * BQ) lds_write<float>(smem, OFF_L + tid * 4, lreg);
  };

  if (total > 0) {
    load_q(0);
    store_q();
  }
  __syncthreads();

  for (int it = 0; it < total; ++it) {
    int bh, q0;
    tile_head(it, &bh, &q0);
    if (it + 1 < total) load_q(it + 1);

    // S = Q K^T and dP = dO V^T for this wave's 32 keys: two 32-row blocks.
    f32x16 s[2], dp[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      s[qb] = f32x16{0};
      dp[qb] = f32x16{0};
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const int off = (qb * 32 + l32) * RP + (ks * 16 + hf * 8) * 2;
        s[qb] = mfma_32x32x16_bf16(lds_read<u32x4>(smem + OFF_Q, off), kf[ks], s[qb]);
        dp[qb] = mfma_32x32x16_bf16(lds_read<u32x4>(smem + OFF_G, off), vf[ks], dp[qb]);
      }
    }

    // P = exp(S*scale - lse) and dS = P (dP - delta).  Accumulator register r
    // of block qb holds query row 32*qb + 8*(r/4) + 4*hf + r%4.
    const bool need_mask = (kv0 + wave * 32 + 32 > Nk) || (q0 + BQ > Nq) ||
                           (CAUSAL && kv0 + wave * 32 + 31 > q0);
    u32x4 pa[2][2], dsa[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float p[16], ds[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int qr = qb * 32 + g * 8 + hf * 4;
        f32x4 lv = lds_read<f32x4>(smem, OFF_L + qr * 4);
        f32x4 dl = lds_read<f32x4>(smem, OFF_DL + qr * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = g * 4 + e;
          float sv = s[qb][r];
          if (need_mask) {
            const int qi = q0 + qr + e;
            if (mykey >= Nk || qi >= Nq || (CAUSAL && mykey > qi)) sv = -INFINITY;
          }
          p[r] = fast_exp2(fmaf(sv, scale_log2, -lv[e]));
          ds[r] = p[r] * (dp[qb][r] - dl[e]);
        }
      }
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        pa[qb][st] = u32x4{pack_bf16(p[8 * st + 0], p[8 * st + 1]),
                           pack_bf16(p[8 * st + 2], p[8 * st + 3]),
                           pack_bf16(p[8 * st + 4], p[8 * st + 5]),
                           pack_bf16(p[8 * st + 6], p[8 * st + 7])};
        dsa[qb][st] = u32x4{pack_bf16(ds[8 * st + 0], ds[8 * st + 1]),
                            pack_bf16(ds[8 * st + 2], ds[8 * st + 3]),
                            pack_bf16(ds[8 * st + 4], ds[8 * st + 5]),
                            pack_bf16(ds[8 * st + 6], ds[8 * st + 7])};
      }
    }

    // dV += P^T dO and dK += dS^T Q.  k-step (qb, st) element e of lane half
    // hf is query row 32*qb + 16*st + 8*(e/4) + 4*hf + e%4.
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const int off = (db * 32 + l32) * TP + (qb * 32 + st * 16 + hf * 4) * 2;
          u32x2 g0 = lds_read<u32x2>(smem + OFF_GT, off);
          u32x2 g1 = lds_read<u32x2>(smem + OFF_GT, off + 16);
          dv[db] = mfma_32x32x16_bf16(pa[qb][st], u32x4{g0[0], g0[1], g1[0], g1[1]}, dv[db]);
          u32x2 q0v = lds_read<u32x2>(smem + OFF_QT, off);
          u32x2 q1v = lds_read<u32x2>(smem + OFF_QT, off + 16);
          dk[db] = mfma_32x32x16_bf16(dsa[qb][st], u32x4{q0v[0], q0v[1], q1v[0], q1v[1]}, dk[db]);
        }

    // dS -> LDS as [q][key] bf16 for the dQ product.  This wave's keys are
    // columns 32*wave + l32; register r of block qb is query row
    // 32*qb + 8*(r/4) + 4*hf + r%4.  The transposed register layout is
    // recovered from the packed pairs: each packed word holds two query rows.
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t word = dsa[qb][st][w];
          const int e0 = 2 * w;  // elements e0 and e0+1 of this k-step
          const int r0 = qb * 32 + st * 16 + 8 * (e0 >> 2) + 4 * hf + (e0 & 3);
          const int col = (wave * 32 + l32) * 2;
          lds_write<uint16_t>(smem + OFF_S, r0 * SP + col, (uint16_t)(word & 0xffff));
          lds_write<uint16_t>(smem + OFF_S, (r0 + 1) * SP + col, (uint16_t)(word >> 16));
        }
    __syncthreads();

    // Next query tile into LDS (Q, dO regions are free now; dS and K^T are
    // still being read below).
    if (it + 1 < total) store_q();

    // dQ = dS K over all 128 keys, then fp32 atomics.  The (query block,
    // head-dim block) pairs of the 64 x D output are dealt to the 4 waves.
    {
      constexpr int PAIRS = 2 * DBLK;
      constexpr int PPW = PAIRS / 4;
#pragma unroll
      for (int pi = 0; pi < PPW; ++pi) {
        const int pr = wave * PPW + pi;
        const int qb = pr / DBLK;
        const int db = pr - qb * DBLK;
        f32x16 dq = f32x16{0};
#pragma unroll
        for (int kk = 0; kk < kBwdBkv / 16; ++kk) {
          const u32x4 bk =
              lds_read<u32x4>(smem + OFF_KT, (db * 32 + l32) * KTP + (kk * 16 + hf * 8) * 2);
          const u32x4 a =
              lds_read<u32x4>(smem + OFF_S, (qb * 32 + l32) * SP + (kk * 16 + hf * 8) * 2);
          dq = mfma_32x32x16_bf16(a, bk, dq);
        }
        float* dqp = dq_accum + (size_t)bh * Nq * D + db * 32 + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qi = q0 + qb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
          if (qi < Nq) atomicAdd(dqp + (size_t)qi * D, dq[r] * scale);
        }
      }
    }
    __syncthreads();
  }

  // dK = scale * sum dS^T Q, dV = sum P^T dO.  Accumulator register r of block
  // db holds key 32*wave + 8*(r/4) + 4*hf + r%4 at head dim 32*db + l32.
  uint16_t* dkp = dK + (size_t)bhk * Nk * D;
  uint16_t* dvp = dV + (size_t)bhk * Nk * D;
#pragma unroll
  for (int db = 0; db < DBLK; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kv0 + wave * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
      if (key < Nk) {
        const size_t off = (size_t)key * D + db * 32 + l32;
        dkp[off] = (uint16_t)(pack_bf16(dk[db][r] * scale, 0.f) & 0xffff);
        dvp[off] = (uint16_t)(pack_bf16(dv[db][r], 0.f) & 0xffff);
      }
    }
}

// ---------------------------------------------------------------------------

hipError_t launch_bwd_f32(const float* q, const float* k, const float* v, const float* o,
                          const float* dout, const float* lse, float* dq, float* dk, float* dv,
                          float* delta, int B, int Hq, int Hkv, int Nq, int Nk, float scale,
                          bool causal, hipStream_t stream) {
  const int rows = B * Hq * Nq;
  hipLaunchKernelGGL((bwd_delta_kernel<float, 64>), dim3((rows + 15) / 16), dim3(256), 0,
                     stream, o, dout, delta, (float*)nullptr, rows);
  hipLaunchKernelGGL(bwd_f32_dq_kernel, dim3((Nq + kBF32T - 1) / kBF32T, B * Hq), dim3(64), 0,
                     stream, q, k, v, dout, lse, delta, dq, Hq, Hkv, Nq, Nk, scale,
                     causal ? 1 : 0);
  hipLaunchKernelGGL(bwd_f32_dkv_kernel, dim3((Nk + 31) / 32, B * Hkv), dim3(64), 0, stream, q,
                     k, v, dout, lse, delta, dk, dv, Hq, Hkv, Nq, Nk, scale, causal ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_bwd_pre(const void* o, const void* dout, float* dq_accum, float* delta, int B,
                          int Hq, int Nq, int d, hipStream_t stream) {
  const int rows = B * Hq * Nq;
  const __bf16* ob = (const __bf16*)o;
  const __bf16* gb = (const __bf16*)dout;
  if (d == 128)
    hipLaunchKernelGGL((bwd_delta_kernel<__bf16, 128>), dim3((rows + 15) / 16), dim3(256), 0,
                       stream, ob, gb, delta, dq_accum, rows);
  else
    hipLaunchKernelGGL((bwd_delta_kernel<__bf16, 64>), dim3((rows + 15) / 16), dim3(256), 0,
                       stream, ob, gb, delta, dq_accum, rows);
  return hipGetLastError();
}

hipError_t launch_bwd_main(const void* q, const void* k, const void* v, const void* dout,
                           const float* lse, const float* delta, float* dq_accum, void* dk,
                           void* dv, int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                           bool causal, hipStream_t stream) {
  const int BHkv = B * Hkv;
  dim3 grid(BHkv * ((Nk + kBwdBkv - 1) / kBwdBkv)), block(256);
  auto Q = (const uint16_t*)q;
  auto K = (const uint16_t*)k;
  auto V = (const uint16_t*)v;
  auto G = (const uint16_t*)dout;
  auto dK = (uint16_t*)dk;
  auto dV = (uint16_t*)dv;
  const float sl2 = scale * kLog2e;
  if (d == 128) {
    if (causal)
      hipLaunchKernelGGL((bwd_bf16_kernel<128, true>), grid, block, 0, stream, Q, K, V, G, lse,
                         delta, dq_accum, dK, dV, Hq, Hkv, Nq, Nk, scale, sl2, BHkv);
    else
      hipLaunchKernelGGL((bwd_bf16_kernel<128, false>), grid, block, 0, stream, Q, K, V, G, lse,
                         delta, dq_accum, dK, dV, Hq, Hkv, Nq, Nk, scale, sl2, BHkv);
  } else {
    if (causal)
      hipLaunchKernelGGL((bwd_bf16_kernel<64, true>), grid, block, 0, stream, Q, K, V, G, lse,
                         delta, dq_accum, dK, dV, Hq, Hkv, Nq, Nk, scale, sl2, BHkv);
    else
      hipLaunchKernelGGL((bwd_bf16_kernel<64, false>), grid, block, 0, stream, Q, K, V, G, lse,
                         delta, dq_accum, dK, dV, Hq, Hkv, Nq, Nk, scale, sl2, BHkv);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_post(const float* dq_accum, void* dq, int B, int Hq, int Nq, int d,
                           hipStream_t stream) {
  const size_t n8 = (size_t)B * Hq * Nq * d / 8;
  hipLaunchKernelGGL(bwd_dq_convert_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0,
                     stream, dq_accum, (uint16_t*)dq, n8);
  return hipGetLastError();
}

}  // namespace fa

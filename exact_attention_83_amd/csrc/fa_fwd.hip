// Forward attention kernels for gfx950.
//
// Method: [CH18] "第 18 章 FlashAttention" §18.4.3 (tiled forward, Fig. 18-16)
// and §18.5.1-18.5.2 (work split per query tile, causal tile skipping); the
// rescaling step is the two-block identity of [L21] "CMU 11-868 L21
// FlashAttention" slide 12.
//
// bf16 kernel layout (one workgroup = 4 waves = 128 query rows, KV tiles of 64
// keys, two workgroups per compute unit):
//   * each wave owns 32 query rows.  It computes S^T = K Q^T with the keys on
//     the MFMA m axis and its queries on the n axis, so every lane owns one
//     query column: the row max is an in-register reduction plus one exchange
//     with the other wave half, and the rescale factor is lane-local.
//   * Q stays in registers for the whole tile as the B operand.
//   * P^T (the S^T accumulator rounded to bf16) is directly the B operand of
//     O^T += V^T P^T: the keys of the accumulator become the k index of the
//     next product.  The V^T fragments are read from the row-major V tile with
//     the transposing LDS read (ds_read_b64_tr_b16).
//   * K and V tiles go from HBM straight into LDS (buffer loads with the LDS
//     destination bit), double-buffered: the next tile's loads are issued
//     right after the barrier and land while the current tile is computed.
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
  constexpr int ROWB = D * 2;               // bytes per K/V row in LDS (no padding)
  constexpr int NCH = D / 8;                // 16-byte chunks per row
  constexpr int TILE = BC * ROWB;           // bytes of one K or V tile
  constexpr int LPW = TILE / 1024 / 4;      // 1 KB direct loads per wave per tile
  constexpr int RPL = 1024 / ROWB;          // rows per 1 KB load
  constexpr int KSTEPS = D / 16;            // MFMA k-steps over the head dim
  constexpr int DBLK = D / 32;              // 32-wide blocks of the head dim
  // LDS: [slot 0: K | V][slot 1: K | V].  Rows are stored unpadded with the
  // 16-byte chunks XOR-swizzled per row, so that both the b128 reads of K and
  // the transposing b64 reads of V hit distinct banks:
  //   K: chunk c of row r sits at position c ^ (r & 7)
  //   V: chunk c of row r sits at position c ^ ((2 r) & (NCH - 1))
  __shared__ __attribute__((aligned(1024))) char smem[4 * TILE];

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
  const size_t kv_off = (size_t)(b * Hkv + hk) * Nk * D;
  // rows past Nk read as zero (and are masked below)
  const __amdgpu_buffer_rsrc_t rK = make_rsrc(K + kv_off, (uint32_t)Nk * ROWB);
  const __amdgpu_buffer_rsrc_t rV = make_rsrc(V + kv_off, (uint32_t)Nk * ROWB);

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

  // Per-lane source offsets of this wave's direct loads (same for every tile):
  // LDS block (wave*LPW + i) holds tile rows r, lane -> position p.
  int koff[LPW], voff[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int r = (wave * LPW + i) * RPL + lane / NCH;
    const int p = lane % NCH;
    koff[i] = r * ROWB + ((p ^ (r & 7)) << 4);
    voff[i] = r * ROWB + ((p ^ ((2 * r) & (NCH - 1))) << 4);
  }
  auto issue_tile = [&](int j, int slot) {
    char* kd = smem + slot * 2 * TILE + wave * LPW * 1024;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      buffer_load_lds16(rK, kd + i * 1024, koff[i], j * TILE);
      buffer_load_lds16(rV, kd + TILE + i * 1024, voff[i], j * TILE);
    }
  };

  // Per-lane LDS read offsets.  K (A operand, row kb*32 + l32, chunk 2*kk + hf):
  int krd[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) krd[kk] = l32 * ROWB + (((2 * kk + hf) ^ (l32 & 7)) << 4);
  // V^T via ds_read_b64_tr_b16.  In each 16-lane group g (= lane/16), source
  // lane j addresses key row 4*(g/2) + j/4 (+ 16*st + 32*kb, + 8 for the
  // second read) at head dims dbase + 4*(j%4) with dbase = 32*db + 16*(g%2);
  // the group's output lane i then holds V[row(e)][dbase + i] for e = 0..3.
  const int g16 = lane >> 4;
  const int j16 = lane & 15;
  const int vrow = 4 * (g16 >> 1) + (j16 >> 2);
  const int vsw = (2 * vrow) & (NCH - 1);
  int vrd[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) {
    const int c = 4 * db + 2 * (g16 & 1) + ((j16 & 3) >> 1);
    vrd[db] = vrow * ROWB + ((c ^ vsw) << 4) + (j16 & 1) * 8;
  }

  f32x16 o[DBLK];
#pragma unroll
  for (int i = 0; i < DBLK; ++i) o[i] = f32x16{0};
  // Running reference max in log2 units (scale*log2e folded in).  It is only
  // raised when some row's max grows by more than 2^8, so O and l are rescaled
  // rarely; probabilities are then at most 2^8, which fp32 and bf16 hold with
  // unchanged relative precision.  The final O/l and LSE do not depend on the
  // reference.  A finite start keeps (-inf) - (-inf) from ever forming.
  float M = -1e30f;
  float l_run = 0.f;  // this lane's share of the row sum

  issue_tile(0, 0);
  for (int j = 0; j < ntiles; ++j) {
    const int slot = j & 1;
    wait_vmem();
    __syncthreads();
    if (j + 1 < ntiles) issue_tile(j + 1, slot ^ 1);
    const int kv0 = j * BC;
    if (CAUSAL && kv0 > q0 + wave * 32 + 31) continue;  // every key after every row
    const char* ks = smem + slot * 2 * TILE;
    const char* vs = ks + TILE;

    // S^T for the wave: two 32-key blocks x 32 queries.
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{0};
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk)
        s[kb] = mfma_32x32x16_bf16(lds_read<u32x4>(ks, kb * 32 * ROWB + krd[kk]), qf[kk], s[kb]);
    }

    // Mask keys past the end (ragged tail) and, on diagonal tiles, keys after
    // the query ([CH18] §18.5.2: only tiles crossing the diagonal need it).
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
    const float mts = max_halves(mt) * scale_log2;
    if (__builtin_amdgcn_ballot_w64(mts > M + 8.f)) {
      const float Mn = fmaxf(M, mts);
      const float alpha = fast_exp2(M - Mn);
      M = Mn;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DBLK; ++i) o[i] *= alpha;
    }

    u32x4 pb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = fast_exp2(fmaf(s[kb][r], scale_log2, -M));
        l_run += p[r];  // fp32 sum of the unrounded p: LSE stays exact to fp32
      }
#pragma unroll
      for (int st = 0; st < 2; ++st)
        pb[kb][st] = u32x4{pack_bf16(p[8 * st + 0], p[8 * st + 1]),
                           pack_bf16(p[8 * st + 2], p[8 * st + 3]),
                           pack_bf16(p[8 * st + 4], p[8 * st + 5]),
                           pack_bf16(p[8 * st + 6], p[8 * st + 7])};
    }

    // O^T += V^T P^T.  B element e of lane half hf in k-step (kb, st) is key
    // kb*32 + 16*st + 8*(e/4) + 4*hf + e%4 (the accumulator's row order).
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const char* vp = vs + (kb * 32 + st * 16) * ROWB + vrd[db];
          const u32x2 a0 = lds_read_tr16(vp);
          const u32x2 a1 = lds_read_tr16(vp + 8 * ROWB);
          o[db] = mfma_32x32x16_bf16(u32x4{a0[0], a0[1], a1[0], a1[1]}, pb[kb][st], o[db]);
        }
  }

  // Epilogue: O = O^T / l, LSE = (M + log2 l) ln 2.
  const float l_tot = sum_halves(l_run);
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
    if (hf == 0) LSE[(size_t)bh * Nq + qrow] = (M + __log2f(l_tot)) * kLn2;
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

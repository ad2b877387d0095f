// Backward attention kernels for gfx950.
//
// Method: [CH18] "第 18 章 FlashAttention" §18.2.4 (gradients: dV = P^T dO,
// dP = dO V^T, dS = P * (dP - rowsum(P * dP)), dQ = dS K, dK = dS^T Q, each
// with one factor of the score scale) and §18.4.4 (recomputation: P is rebuilt
// tile by tile from the saved logsumexp, so no rescaling is needed; only O(N)
// row statistics are kept from the forward).  The row term rowsum(P * dP)
// equals dO_i . O_i, which the dQ kernel forms from its rows' O and dO (or a
// pre-pass computes) and writes for the dK/dV kernel.  Both kernels start
// their dP accumulators at that delta and feed dO V^T one factor negated, so
// dS = P * (dP - delta) is a single multiply by -P.
//
// The bf16 path runs the dQ kernel (forming delta) and then the dK/dV kernel
// (see the comments above both).  Causal: a KV tile only visits the query
// tiles that reach its keys, a query tile only the key tiles up to its last
// row, and only tiles crossing the diagonal are masked ([CH18] §18.5.2 (4):
// the skipped gradients are structurally zero).  Work units are launched
// longest first.

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

// ---------------------------------------------------------------------------
// delta_i = sum_c dO_ic * O_ic.
// Rows are (token, head) pairs in memory order; with heads > 1 (packed
// token-major input, row = token * heads + head) delta is written head-major,
// delta[head][token], the layout of the forward's LSE.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const T* __restrict__ O,
                                                        const T* __restrict__ dO,
                                                        float* __restrict__ delta, int rows,
                                                        int heads) {
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
  }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 16);
  if (row < rows && sub == 0) delta[(size_t)(row % heads) * (rows / heads) + row / heads] = acc;
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
// bf16 backward: two kernels, no atomics.
//   bwd_dkdv_kernel: one workgroup per (b, KV head, 256-key tile); dK and dV
//     are accumulated on chip over every query tile of every query head of the
//     group (4 products per tile pair: S, dP, dV, dK).
//   bwd_dq_kernel: one workgroup per (b, query head, 256-row tile); dQ is
//     accumulated on chip over the key tiles, exactly like O in the forward
//     (3 products per tile pair: S, dP, dQ).
// Recomputing S and dP in the dQ kernel costs 7 products per tile pair instead
// of the 5 of a single kernel, but removes the fp32 dQ atomics (whose traffic,
// B*H*(#tile pairs)*BQ*d*4 bytes, goes to memory on this multi-XCD device)
// and the dS round trip through LDS.
namespace {
constexpr int kKvWaves = 4;
constexpr int kKvKb = 2;                         // 32-key blocks per wave
constexpr int kKvBkv = 32 * kKvKb * kKvWaves;    // keys per dK/dV work unit
// Bytes of dynamic LDS of the dK/dV kernel: each wave's V rows.
constexpr int dkdv_vbuf_bytes(int d) { return kKvWaves * 32 * kKvKb * 2 * d; }
constexpr int kKvBq = 32;              // query rows per inner tile
constexpr int kDqWaves = 8;
constexpr int kDqBr = 32 * kDqWaves;   // query rows per dQ work unit
constexpr int kDqBc = 64;              // keys per KV tile
constexpr int kSpBq = 256;             // query rows per block of a sparse pattern
constexpr int kSpBk = 64;              // keys per block of a sparse pattern
}  // namespace

// Chunk swizzle of an LDS tile with ROWB-byte rows: chunk c of row r sits at
// position c ^ bwd_swz<ROWB>(r).  Both b128 reads of 16 consecutive rows (one
// chunk) and transposing reads of 4 consecutive rows x 4 chunks are free of
// bank conflicts on the 64-bank LDS.
template <int ROWB>
__device__ __forceinline__ int bwd_swz(int r) {
  return ROWB == 256 ? (((r & 3) << 2) | ((r >> 2) & 3))
                     : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// Byte offset, within a row-major tile, that lane `lane` passes to the
// transposing read (ds_read_b64_tr_b16) so that output lane i of its 16-lane
// group receives elements (row r0 + e, col c0 + 16*((lane>>4)&1) + i), e=0..3,
// with r0 = rb + 4*(lane>>5) (the lane half) and c0 a multiple of 32.
template <int ROWB>
__device__ __forceinline__ int tr_offset(int lane, int rb, int c0) {
  const int g = lane >> 4, j = lane & 15;
  const int row = rb + 4 * (g >> 1) + (j >> 2);
  const int col = c0 + 16 * (g & 1) + 4 * (j & 3);  // elements (bf16)
  return row * ROWB + (((col >> 3) ^ bwd_swz<ROWB>(row)) << 4) + (col & 7) * 2;
}

// Source offset of direct-load block `blk` (1 KB) of a row-major tile with
// ROWB-byte rows, for this lane: LDS position p of row r receives source
// chunk p ^ swz(r).
template <int ROWB>
__device__ __forceinline__ int swz_src_offset(int lane, int blk, int stride = ROWB) {
  // stride: bytes between consecutive source rows (ROWB when rows are dense)
  const int r = blk * (1024 / ROWB) + lane / (ROWB / 16);
  const int p = lane % (ROWB / 16);
  return r * stride + ((p ^ bwd_swz<ROWB>(r)) << 4);
}

// Slot schedule of the bf16 dK/dV tile's elementwise work.  Slot g is the
// product g of phases 2-4 (dP: 0-15, dV: 16-31, dK: 32-47); after issuing it
// the wave packs to bf16 the pairs finished in slot g - 1 and then computes
// the next elements of P and of dS due in slot g, in element order.
// P ends in slot 22 (a dV product of k-step 1 first runs in slot 24) and dS
// in slot 37 (a dK product of k-step 1 first runs in slot 40), so the
// exponentials spread over the dP and dV products and the dS arithmetic over
// the dV and dK products instead of piling up in one phase each.
// P: one element per slot in slots 0-22, two in those with g % 5 = 1 or 3;
// dS: two per slot in slots 22-37.  The counts below are the elements
// finished by the end of slot g (none for g < 0).
__host__ __device__ constexpr int dkdv_p_cum(int g) {
  return g < 0 ? 0
               : (g < 22 ? g : 22) + 1 + 2 * (((g < 22 ? g : 22) + 1) / 5) +
                     (((g < 22 ? g : 22) + 1) % 5 > 1) + (((g < 22 ? g : 22) + 1) % 5 > 3);
}
__host__ __device__ constexpr int dkdv_ds_cum(int g) {
  return g < 22 ? 0 : 2 * ((g < 37 ? g : 37) - 21);
}
// every P element done (and packed) before the first dV product that reads
// it, every dS element before its dK product: rows 0-15 are elements 0-15
static_assert(dkdv_p_cum(0) == 1 && dkdv_p_cum(1) == 3 && dkdv_p_cum(4) == 7 &&
                  dkdv_p_cum(21) == 31 && dkdv_p_cum(22) == 32 && dkdv_p_cum(47) == 32 &&
                  dkdv_p_cum(14) >= 16,
              "P schedule");
static_assert(dkdv_ds_cum(21) == 0 && dkdv_ds_cum(22) == 2 && dkdv_ds_cum(37) == 32 &&
                  dkdv_ds_cum(47) == 32 && dkdv_ds_cum(30) >= 16,
              "dS schedule");

// ---------------------------------------------------------------------------
// dK, dV.  Wave w owns KB blocks of 32 keys, kv0 + 32*KB*w + 32*kb + (0..31).
// Their K rows stay in registers and their V rows in the wave's own LDS
// region, as the MFMA B operands of S = Q K^T and dP = dO V^T (queries on the
// m axis, keys on n).  Each A operand read from
// LDS (a Q or dO row chunk) feeds one product per key block, which halves the
// LDS read traffic per product at KB = 2: with one LDS operand per product
// the LDS read bandwidth, not the matrix cores, bounds the kernel.  The S and
// dP accumulators (query rows in registers, one key per lane) are directly the
// A operands of dV += P^T dO and dK += dS^T Q; their B operands are
// transposing reads of the row-major dO and Q tiles, again shared by the key
// blocks.  The dK/dV accumulators (256 registers at d = 128) live in the
// accumulation registers, so one wave runs per SIMD.
// WIN: sliding window (key j visible to query i iff i - win_l <= j <= i +
// win_r; negative = unbounded): only the query tiles whose windows reach this
// work unit's keys are visited.
// FP8DS: dK += dS^T Q runs on the 32x32x64 scaled fp8 MFMA ([CH18] §18.6.2
// (3)), two query tiles per product: the first tile of each pair keeps its
// dS (e5m2, one power-of-two scale per (key, 32-query tile)) and its half of
// the Q fragments in registers, and the second tile's products take the two
// tiles as their two 32-query k-blocks; Q comes in e4m3 from the quantiser's
// per-32-row blocks (Q8, e8m0 scale words QE), staged in each slot beside the
// bf16 Q and read with transposing byte reads.  A last tile without a partner
// pairs with zeros.
template <int D, bool CAUSAL, bool WIN, bool VARLEN, bool SPARSE, bool FP8DS>
__device__ __forceinline__ void bwd_dkdv_unit(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ Delta,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int Hq, int Hkv, int Nq_arg,
    int Nk_arg, float scale, float scale_log2, int BHkv, int win_l, int win_r,
    const int* __restrict__ cu_q, const int* __restrict__ cu_k, int total_q,
    const uint8_t* __restrict__ sp_map, int sp_nkb, const uint8_t* __restrict__ Q8,
    const int32_t* __restrict__ QE, int unit) {
  static_assert(!FP8DS || (D == 128 && !WIN && !VARLEN && !SPARSE), "fp8 dS: dense, d = 128");
  constexpr int NW = kKvWaves;
  constexpr int KB = kKvKb;
  constexpr int BQ = kKvBq;
  constexpr int BKV = kKvBkv;
  constexpr int KSTEPS = D / 16;
  constexpr int DBLK = D / 32;
  constexpr int ROWB = D * 2;
  constexpr int QTILE = BQ * ROWB;
  constexpr int LPW = QTILE / 1024 / NW;  // direct loads per wave per Q (or dO) tile
  // Q, dO, lse, delta; FP8DS: the e4m3 Q tile (1 KB-aligned) and each wave's
  // copy of its scale word
  constexpr int Q8OFF = 2 * QTILE + 1024;
  constexpr int QEOFF = Q8OFF + BQ * D;
  constexpr int SLOT = FP8DS ? QEOFF + NW * 256 : 2 * QTILE + 2 * BQ * 4;
  static_assert(2 * SLOT <= 64 * 1024, "slot bases within a read's immediate offset");
  // One variable per slot: with the slot a compile-time constant in the loop
  // body, the compiler sees that the direct loads into one slot cannot alias
  // the reads of the other and does not wait for them.
  __shared__ __attribute__((aligned(1024))) char s0[SLOT], s1[SLOT];
  auto sslot = [&](int sl) -> char* { return sl == 0 ? s0 : s1; };

  // (opaque to the optimiser: per-lane offsets derived from it are then
  // recomputed for each unit of a persistent loop instead of being kept
  // live, and spilled, across it)
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  const int t = unit;
  const int bhk = t % BHkv;
  const int jt = t / BHkv;  // ascending KV tiles = longest first under causal
  const int b = bhk / Hkv;
  const int hk = bhk - b * Hkv;
  const int G = Hq / Hkv;
  const int kv0 = jt * BKV;
  const int kbase = kv0 + wave * 32 * KB;
  // This unit's sequence lengths, the element offset of its K/V rows and the
  // row strides in elements (D for [B][H][N][D]; H*D for a packed
  // token-major batch, VARLEN, whose sequence b spans cu_q/cu_k[b] .. [b+1]).
  int Nq = Nq_arg, Nk = Nk_arg, qs0 = 0;
  size_t kv_off = (size_t)bhk * Nk * D;
  const int SQ = VARLEN ? Hq * D : D;
  const int SK = VARLEN ? Hkv * D : D;
  if constexpr (VARLEN) {
    qs0 = cu_q[b];
    const int ks0 = cu_k[b];
    Nq = cu_q[b + 1] - qs0;
    Nk = cu_k[b + 1] - ks0;
    if (kv0 >= Nk) return;  // the whole workgroup: past this sequence's keys
    kv_off = ((size_t)ks0 * Hkv + hk) * D;
  }
  // Element offsets of query head bh's Q/dO rows and of its lse/delta.
  auto q_off = [&](int bh) -> size_t {
    if constexpr (VARLEN) return ((size_t)qs0 * Hq + (bh - b * Hq)) * D;
    return (size_t)bh * Nq * D;
  };
  auto l_off = [&](int bh) -> size_t {
    if constexpr (VARLEN) return (size_t)(bh - b * Hq) * total_q + qs0;
    return (size_t)bh * Nq;
  };

  // This lane's K and V rows: B operands with n = key, k = head dim.
  u32x4 kf[KB][KSTEPS];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int key = min(kbase + kb * 32 + l32, Nk - 1);
    const uint16_t* kr = K + kv_off + (size_t)key * SK;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) kf[kb][ks] = ldg<u32x4>(kr + ks * 16 + hf * 8);
  }
  // This wave's V rows go to its own LDS region (row-major, chunks swizzled
  // like the query tiles), read back as B operands of dP = dO V^T: that frees
  // the registers for deeper prefetching of the LDS operands below.  The
  // region is dynamic LDS, which follows the static slots, so the slots sit
  // below 64 KB, where a read's immediate offset can hold the slot base.
  constexpr int VROWS = 32 * KB;
  static_assert(NW * VROWS * ROWB == dkdv_vbuf_bytes(D), "V region size");
  static_assert(2 * SLOT + NW * VROWS * ROWB <= 160 * 1024, "LDS per workgroup");
  extern __shared__ __attribute__((aligned(1024))) char vbuf[];  // dkdv_vbuf_bytes(D)
  char* vw = vbuf + wave * VROWS * ROWB;
  {
    const __amdgpu_buffer_rsrc_t rV = make_rsrc(V + kv_off, (uint32_t)Nk * SK * 2);
#pragma unroll
    for (int blk = 0; blk < VROWS * ROWB / 1024; ++blk)
      buffer_load_lds16(rV, vw + blk * 1024, swz_src_offset<ROWB>(lane, blk, SK * 2),
                        kbase * SK * 2);
  }

  const int nqt = (Nq + BQ - 1) / BQ;
  int qt_begin = CAUSAL ? kv0 / BQ : 0;
  int qt_end = nqt;
  if constexpr (WIN) {
    if (win_r >= 0) qt_begin = max(qt_begin, max(0, kv0 - win_r) / BQ);
    if (win_l >= 0) qt_end = min(qt_end, (kv0 + BKV - 1 + win_l) / BQ + 1);
  }
  // SPARSE: the query blocks (kSpBq rows) whose list holds one of this
  // unit's four key blocks (wave w's 64 keys are key block kv0/64 + w),
  // compacted into LDS as block | (4-bit set of listed waves) << 16.
  __shared__ int sp_list[SPARSE ? 256 : 1];
  __shared__ int sp_cnt[SPARSE ? NW : 1];
  int nact = 0;
  if constexpr (SPARSE) {
    static_assert(BKV == kSpBq && 32 * KB == kSpBk && NW * 64 == 256, "sparse block shapes");
    const int nqb = (Nq + kSpBq - 1) / kSpBq;  // <= 256, checked on the host
    const int kc0 = kv0 / kSpBk;
    int bits = 0;
    // causal: query blocks before this unit's keys see none of them
    if (tid < nqb && (!CAUSAL || tid >= jt)) {
      const uint8_t* row = sp_map + (size_t)tid * sp_nkb;
#pragma unroll
      for (int w = 0; w < NW; ++w)
        if (kc0 + w < sp_nkb && row[kc0 + w]) bits |= 1 << w;
    }
    const uint64_t act = __builtin_amdgcn_ballot_w64(bits != 0);
    if (lane == 0) sp_cnt[wave] = __builtin_popcountll(act);
    __syncthreads();
    int before = 0;
    for (int w = 0; w < NW; ++w) {
      const int c = sp_cnt[w];
      if (w < wave) before += c;
      nact += c;
    }
    nact = __builtin_amdgcn_readfirstlane(nact);
    if (bits) {
      const int pos = before + (int)__builtin_amdgcn_mbcnt_hi(
                                   (uint32_t)(act >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)act, 0));
      sp_list[pos] = tid | (bits << 16);
    }
    __syncthreads();
  }
  const int per_head = SPARSE ? nact * (kSpBq / BQ) : max(0, qt_end - qt_begin);
  const int total = per_head * G;
  // query tile `it` of the loop: head bh, first row q0, and (SPARSE) whether
  // this wave's key block is listed for it.  Tiles run from the last query
  // tile down: every work unit of a head then starts on the same tile
  // and the units running side by side (one XCD holds all of a head's
  // units) read the same Q and dO rows at about the same time, from L2
  // (causal: 14% less HBM fetch than starting each unit at its diagonal).
  auto tile_head = [&](int it, int* bh, int* q0, bool* listed = nullptr) {
    const int gi = it / per_head;
    const int x = it - gi * per_head;
    *bh = b * Hq + hk * G + gi;
    if constexpr (SPARSE) {
      // the listed blocks' tiles in the same descending order
      const int xr = per_head - 1 - x;
      const int e = __builtin_amdgcn_readfirstlane(sp_list[xr / (kSpBq / BQ)]);
      *q0 = (e & 0xffff) * kSpBq + (xr % (kSpBq / BQ)) * BQ;
      if (listed) *listed = (e >> (16 + wave)) & 1;
    } else {
      *q0 = (qt_end - 1 - x) * BQ;
    }
  };
  int qoff[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) qoff[i] = swz_src_offset<ROWB>(lane, wave * LPW + i, SQ * 2);
  static_assert(!FP8DS || BQ * D == NW * 1024, "one 1 KB e4m3 load per wave per tile");
  const int q8row = wave * 8 + (lane >> 3);
  const int q8off = q8row * D + (((lane & 7) ^ f8_swz_t(q8row)) << 4);
  auto issue = [&](int it, int slot) {
    int bh, q0;
    tile_head(it, &bh, &q0);
    const __amdgpu_buffer_rsrc_t rQ = make_rsrc(Q + q_off(bh), (uint32_t)Nq * SQ * 2);
    const __amdgpu_buffer_rsrc_t rG = make_rsrc(dO + q_off(bh), (uint32_t)Nq * SQ * 2);
    char* qd = sslot(slot) + wave * LPW * 1024;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      buffer_load_lds16(rQ, qd + i * 1024, qoff[i], q0 * SQ * 2);
      buffer_load_lds16(rG, qd + QTILE + i * 1024, qoff[i], q0 * SQ * 2);
    }
    // wave 0: lse, wave 1: delta (each with its own uniform descriptor; a
    // pointer chosen per wave would make the descriptor look divergent)
    // (descriptors built outside the lane-divergent branches, so that they
    // stay scalar)
    char* ld = sslot(slot) + 2 * QTILE;
    const __amdgpu_buffer_rsrc_t rL = make_rsrc(LSE + l_off(bh), (uint32_t)Nq * 4);
    const __amdgpu_buffer_rsrc_t rD = make_rsrc(Delta + l_off(bh), (uint32_t)Nq * 4);
    if (wave == 0 && lane < BQ)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rL, (lds_void_t*)ld, 4, lane * 4, q0 * 4, 0, 0);
    if (wave == 1 && lane < BQ)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rD, (lds_void_t*)(ld + BQ * 4), 4, lane * 4, q0 * 4,
                                               0, 0);
    if constexpr (FP8DS) {
      // wave w: e4m3 rows 8w .. 8w+7 (lane -> row 8w + lane/8, LDS chunk
      // position lane%8 holding source chunk (lane%8) ^ swz), and the tile's
      // scale word into its own 256-byte copy
      const __amdgpu_buffer_rsrc_t rQ8 = make_rsrc(Q8 + q_off(bh), (uint32_t)Nq * D);
      buffer_load_lds16(rQ8, sslot(slot) + Q8OFF + wave * 1024, q8off, q0 * D);
      const int nqb8 = (Nq + 31) / 32;
      const __amdgpu_buffer_rsrc_t rQE = make_rsrc(QE + (size_t)bh * nqb8, (uint32_t)nqb8 * 4);
      buffer_load_lds4(rQE, sslot(slot) + QEOFF + wave * 256, 0, (q0 / 32) * 4);
    }
  };

  // A-operand rows of S / dP (b128): query l32, chunk 2*ks + hf.
  int ard[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks)
    ard[ks] = l32 * ROWB + (((2 * ks + hf) ^ bwd_swz<ROWB>(l32)) << 4);
  // B operands of dV / dK (transposing reads of dO / Q), k-step st: query rows
  // 16*st + 8*(e/4) + 4*hf + e%4, head dims 32*db + lane.
  int trd0[DBLK], trd1[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) {
    trd0[db] = tr_offset<ROWB>(lane, 0, 32 * db);
    trd1[db] = tr_offset<ROWB>(lane, 8, 32 * db);
  }

  // FP8DS: B operand of dK (k = query, n = head dim 32*db + l32), one tile's
  // half: bytes 16*th .. 16*th+15 of the 32 come from tile th of the pair,
  // byte i of lane half hf being query 8*(i/4) + 4*hf + i%4 of that tile
  // (the S accumulator's row order).  Source lane 2r + half of 16-lane group
  // g16 addresses row 8*(r/4) + 4*hf + r%4 (+16 for the second read), head
  // dims 32*db + 16*(g16%2) + 8*half.
  int q8rd[FP8DS ? DBLK : 1];
  if constexpr (FP8DS) {
    const int g16 = lane >> 4, j16 = lane & 15;
    const int vr = j16 >> 1;
    const int row = 8 * (vr >> 2) + 4 * hf + (vr & 3);
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
      q8rd[db] = row * D + (((2 * db + (g16 & 1)) ^ f8_swz_t(row)) << 4) + 8 * (j16 & 1);
  }
  // the first tile of a pair: dS codes, dS scale codes, Q fragment halves and
  // Q scale word
  constexpr int F8N = FP8DS ? 1 : 0;
  int dsc_prev[KB][4 * F8N + 1 - F8N], esc_prev[KB], q8h_prev[DBLK][4 * F8N + 1 - F8N];
  int qe_prev = 0;

  f32x16 dk[KB][DBLK], dv[KB][DBLK];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int i = 0; i < DBLK; ++i) {
      dk[kb][i] = f32x16{0};
      dv[kb][i] = f32x16{0};
    }

#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) settle(kf[kb][ks]);
  // V enters dP = dO V^T negated and the dP accumulators start at delta, so
  // that they end at delta - dP and dS = P (dP - delta) is one multiply by
  // -P: each wave flips the sign bits of its own V rows once, when they have
  // landed (before the first tile's products; LDS operations of one wave run
  // in order).
  auto negate_v = [&]() {
    constexpr int NCHK = VROWS * ROWB / 16 / 64;  // 16-byte chunks per lane
#pragma unroll
    for (int c = 0; c < NCHK; ++c) {
      const int off = (c * 64 + lane) * 16;
      u32x4 x = lds_read<u32x4>(vw, off);
      x ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
      lds_write<u32x4>(vw, off, x);
    }
    asm volatile("" ::: "memory");
  };
  if (total > 0) issue(0, 0);
  auto body = [&](int it, auto S) {
    constexpr int slot = decltype(S)::value;
    int bh, q0;
    bool listed = true;
    tile_head(it, &bh, &q0, &listed);
    wait_vmem();
    lds_barrier();
    if (it == 0) negate_v();
    // FP8DS: first (slot 0) or second (slot 1) tile of a pair; a first tile
    // with no second one runs the products itself, against zeros
    const bool lone = FP8DS && slot == 0 && it + 1 >= total;
    const char* qs = sslot(slot);
    const char* gs = qs + QTILE;
    const char* ls = qs + 2 * QTILE;

    // Four phases of NPH products each: (1) S = Q K^T; (2) dP = dO V^T;
    // (3) dV += P^T dO; (4) dK += dS^T Q.  P = exp(S*scale - lse) of the
    // finished S and dS = P (dP - delta) are computed between the products of
    // phases 2-4 (bf16 at d = 128: on the slot schedule of dkdv_p_cum; else P
    // in phase 2 and dS in phase 3, EPP elements per product).  LDS operands are read
    // two product pairs ahead (Q in phase 1 three), and each phase's first
    // ones during the last products of the phase before it (this kernel has
    // one wave per SIMD, so nothing else hides LDS latency).
    // Element x (of 32 per lane) is register r = 4*(x/8) + x%4 of block kb =
    // (x/4)%2; register r holds query row 8*(r/4) + 4*hf + r%4.
    constexpr int NPH = KB * KSTEPS;  // products per phase
    constexpr int EPP = 32 / NPH;     // elements per product (per lane)
    constexpr int NPR = NPH / 2;      // product pairs per phase
    static_assert(KB == 2 && 2 * DBLK * KB == NPH && EPP * NPH == 32, "phase shapes");
    // the slot schedule is laid out for 16 products per phase (d = 128)
    constexpr bool SPREAD = !FP8DS && NPH == 16;
    f32x16 sb[KB], dpb[KB];  // dpb: set to delta at the end of phase 1
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) sb[kb] = f32x16{0};
    // Transposed B operand (dO^T or Q^T rows) of pair j of phases 3/4:
    // st = j / DBLK, db = j % DBLK.
    auto trB = [&](const char* base, int j) {
      const int ro = (j / DBLK) * 16 * ROWB;
      const u32x2 v0 = lds_read_tr16(base + ro + trd0[j % DBLK]);
      const u32x2 v1 = lds_read_tr16(base + ro + trd1[j % DBLK]);
      return u32x4{v0[0], v0[1], v1[0], v1[1]};
    };
    // The first LDS operands of each phase are read during the last products
    // of the phase before it, so that no phase starts by waiting for LDS.
    u32x4 ga[2], va[2][KB];  // phase 2: dO and V fragments, two pairs ahead
    f32x4 lvn;               // phase 2: lse of the current row group
    u32x4 gb[2], qb[2];      // phases 3 / 4: first two transposed B operands
    // (1) S: pair ks shares the Q fragment, read PF1 pairs ahead.
    {
      constexpr int PF1 = 3;
      static_assert(KSTEPS >= PF1, "phase 1 prefetch depth");
      u32x4 qa[PF1];
#pragma unroll
      for (int p = 0; p < PF1; ++p) qa[p] = lds_read<u32x4>(qs, ard[p]);
      // the next tile's loads after this tile's first LDS reads, so that
      // their address work runs while the reads are in flight
      asm volatile("" ::: "memory");
      if (it + 1 < total) issue(it + 1, slot ^ 1);
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const u32x4 a = qa[ks % PF1];
        if (ks + PF1 < KSTEPS) {
          qa[ks % PF1] = lds_read<u32x4>(qs, ard[ks + PF1]);
        } else {
          const int pp = ks + PF1 - KSTEPS;
          if (pp < 2) {
            ga[pp] = lds_read<u32x4>(gs, ard[pp]);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) va[pp][kb] = lds_read<u32x4>(vw, kb * 32 * ROWB + ard[pp]);
          } else {
            lvn = lds_read<f32x4>(ls, (hf * 4) * 4);
            // the dP accumulators start at the delta of this lane's rows
            // (register 4g + e: row 8g + 4*hf + e)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
              for (int g = 0; g < 4; ++g) {
                const f32x4 d4 = lds_read<f32x4>(ls, BQ * 4 + (g * 8 + hf * 4) * 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) dpb[kb][4 * g + e] = d4[e];
              }
          }
        }
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) sb[kb] = mfma_32x32x16_bf16(a, kf[kb][ks], sb[kb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // Mask keys past Nk, rows past Nq and (causal) keys after the query.
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int key = kbase + kb * 32 + l32;
      const int kb0 = kbase + kb * 32;
      bool need = (kb0 + 32 > Nk) || (q0 + BQ > Nq) || (CAUSAL && kb0 + 31 > q0);
      if constexpr (SPARSE) need = need || !listed;
      if constexpr (WIN)
        need = need || (win_l >= 0 && kb0 < q0 + BQ - 1 - win_l) ||
               (win_r >= 0 && kb0 + 31 > q0 + win_r);
      if (need) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qi = q0 + 8 * (r >> 2) + 4 * hf + (r & 3);
          bool out = key >= Nk || qi >= Nq || (CAUSAL && key > qi);
          if constexpr (WIN)
            out = out || (win_l >= 0 && key < qi - win_l) || (win_r >= 0 && key > qi + win_r);
          if constexpr (SPARSE) out = out || !listed;
          sb[kb][r] = out ? -INFINITY : sb[kb][r];
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    u32x4 pa[KB][2], dsa[KB][2];  // [kb][k-step]
    f32x4 nl;  // -lse * log2(e) of P's current row group
    // P of element x (in place of S); the next row group's lse is read when
    // a row group starts
    auto elem_p = [&](int x) {
      const int gr = x >> 3, kbe = (x >> 2) & 1, e = x & 3, r = 4 * gr + e;
      if ((x & 7) == 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          nl[q] = -lvn[q] * kLog2e;
          // a row that sees no key (lse = -inf, possible only with a
          // sparse pattern) gets P = 0 rather than exp(-inf + inf)
          if constexpr (SPARSE) nl[q] = lvn[q] == -INFINITY ? -INFINITY : nl[q];
        }
        if (gr < 3) lvn = lds_read<f32x4>(ls, ((gr + 1) * 8 + hf * 4) * 4);
      }
      sb[kbe][r] = fast_exp2(fmaf(sb[kbe][r], scale_log2, nl[e]));
    };
    // bf16 A operand of the element pair (x - 1, x), x odd
    auto pack_p = [&](int x) {
      const int gr = x >> 3, kbe = (x >> 2) & 1, e = x & 3, r = 4 * gr + e;
      pa[kbe][gr >> 1][2 * (gr & 1) + (e >> 1)] = pack_bf16(sb[kbe][r - 1], sb[kbe][r]);
    };
    // dS of element x (in place of dP, which holds delta - dP here)
    auto elem_ds = [&](int x) {
      const int kbe = (x >> 2) & 1, r = 4 * (x >> 3) + (x & 3);
      dpb[kbe][r] = -sb[kbe][r] * dpb[kbe][r];
    };
    auto pack_ds = [&](int x) {
      const int gr = x >> 3, kbe = (x >> 2) & 1, e = x & 3, r = 4 * gr + e;
      dsa[kbe][gr >> 1][2 * (gr & 1) + (e >> 1)] = pack_bf16(dpb[kbe][r - 1], dpb[kbe][r]);
    };
    // SPREAD: the elementwise work of slot g (see dkdv_p_cum).  A pair is
    // packed one slot after its second element: right behind it the pack
    // would wait for the result.
    auto slot_work = [&](int g) {
#pragma unroll
      for (int x = 1; x < 32; x += 2)
        if (x >= dkdv_p_cum(g - 2) && x < dkdv_p_cum(g - 1)) pack_p(x);
#pragma unroll
      for (int x = 1; x < 32; x += 2)
        if (x >= dkdv_ds_cum(g - 2) && x < dkdv_ds_cum(g - 1)) pack_ds(x);
#pragma unroll
      for (int x = 0; x < 32; ++x)
        if (x >= dkdv_p_cum(g - 1) && x < dkdv_p_cum(g)) elem_p(x);
#pragma unroll
      for (int x = 0; x < 32; ++x)
        if (x >= dkdv_ds_cum(g - 1) && x < dkdv_ds_cum(g)) elem_ds(x);
    };
    // (2) dP, with P (in place of S) and its bf16 A operands.  Pair ks uses
    // the dO fragment ga and the V fragments of both key blocks.
    {
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const u32x4 g = ga[ks & 1];
        u32x4 v[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) v[kb] = va[ks & 1][kb];
        if (ks + 2 < KSTEPS) {
          ga[ks & 1] = lds_read<u32x4>(gs, ard[ks + 2]);
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
            va[ks & 1][kb] = lds_read<u32x4>(vw, kb * 32 * ROWB + ard[ks + 2]);
        } else {
          // phase 3's first operands
          gb[ks + 2 - KSTEPS] = trB(gs, ks + 2 - KSTEPS);
        }
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const int m = 2 * ks + kb;
          dpb[kb] = mfma_32x32x16_bf16(g, v[kb], dpb[kb]);
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (SPREAD) {
            slot_work(m);
          } else {
            // all of P here, EPP elements per product; the previous
            // product's pairs are packed one product after their exp
#pragma unroll
            for (int t = 0; t < EPP; ++t) elem_p(EPP * m + t);
            if (m > 0) {
#pragma unroll
              for (int t = 1; t < EPP; t += 2) pack_p(EPP * (m - 1) + t);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if constexpr (!SPREAD) {
#pragma unroll
        for (int t = 1; t < EPP; t += 2) pack_p(EPP * (NPH - 1) + t);
      }
    }
    // (3) dV += P^T dO, with dS = P (dP - delta) and its bf16 A operands
    // (FP8DS: the largest |dS| of each key block, over this lane's rows).
    float am[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) am[kb] = 0.f;
    {
#pragma unroll
      for (int j = 0; j < NPR; ++j) {
        const u32x4 b = gb[j & 1];
        if (j + 2 < NPR) gb[j & 1] = trB(gs, j + 2);
        else if (!FP8DS) qb[j + 2 - NPR] = trB(qs, j + 2 - NPR);  // phase 4's first operands
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const int m = 2 * j + kb;
          mfma_acc_pinned(dv[kb][j % DBLK], pa[kb][j / DBLK], b);
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (SPREAD) {
            slot_work(NPH + m);
          } else {
            // all of dS here (FP8DS: with the largest magnitude per key
            // block; else each pair packed right behind its second element)
#pragma unroll
            for (int t = 0; t < EPP; ++t) {
              const int x = EPP * m + t, kbe = (x >> 2) & 1, r = 4 * (x >> 3) + (x & 3);
              elem_ds(x);
              if constexpr (FP8DS) am[kbe] = fmaxf(am[kbe], fabsf(dpb[kbe][r]));
              else if (x & 1) pack_ds(x);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    // (4) dK += dS^T Q.
    if constexpr (FP8DS) {
      // this tile's dS in e5m2 with one power-of-two scale per (key, tile)
      // (the maximum over both lane halves), its Q fragment halves and scale.
      // The second tile of a pair quantises key block 1 between key block
      // 0's products.
      int dsc[KB][4], esc[KB], q8h[DBLK][4];
      float scl[KB];
      auto block_scale = [&](int kb) {
        const int e = pow2_block_exp<16>(max_halves(am[kb]));
        scl[kb] = exp2_pos(e);
        esc[kb] = e + 127;
      };
      auto quant = [&](int kb, int i) {
        dsc[kb][i] = cvt_bf8x4_div(dpb[kb][4 * i], dpb[kb][4 * i + 1], dpb[kb][4 * i + 2],
                                   dpb[kb][4 * i + 3], scl[kb]);
      };
      const char* q8s = qs + Q8OFF;
#pragma unroll
      for (int db = 0; db < DBLK; ++db) {
        const i32x2_t x0 = lds_read_tr8(q8s + q8rd[db]);
        const i32x2_t x1 = lds_read_tr8(q8s + 16 * D + q8rd[db]);
        q8h[db][0] = x0[0];
        q8h[db][1] = x0[1];
        q8h[db][2] = x1[0];
        q8h[db][3] = x1[1];
      }
      const int qe = lds_read<int>(qs + QEOFF + wave * 256, 0);
      block_scale(0);
#pragma unroll
      for (int i = 0; i < 4; ++i) quant(0, i);
      block_scale(1);
      if (slot == 0 && !lone) {
#pragma unroll
        for (int i = 0; i < 4; ++i) quant(1, i);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          esc_prev[kb] = esc[kb];
#pragma unroll
          for (int i = 0; i < 4; ++i) dsc_prev[kb][i] = dsc[kb][i];
        }
#pragma unroll
        for (int db = 0; db < DBLK; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) q8h_prev[db][i] = q8h[db][i];
        qe_prev = qe;
      } else {
        // k-block 0 = the pair's first tile (or this lone tile), k-block 1 =
        // the second tile (or zeros with unit scales); lane half hf supplies
        // k-block hf's scales
        const int sb = lone ? (hf ? 127 : qe) : (hf ? qe : qe_prev);
        auto operand_b = [&](int db) {
          return lone ? i32x8{q8h[db][0], q8h[db][1], q8h[db][2], q8h[db][3], 0, 0, 0, 0}
                      : i32x8{q8h_prev[db][0], q8h_prev[db][1], q8h_prev[db][2],
                              q8h_prev[db][3], q8h[db][0], q8h[db][1], q8h[db][2], q8h[db][3]};
        };
        auto operand_a = [&](int kb) {
          return lone ? i32x8{dsc[kb][0], dsc[kb][1], dsc[kb][2], dsc[kb][3], 0, 0, 0, 0}
                      : i32x8{dsc_prev[kb][0], dsc_prev[kb][1], dsc_prev[kb][2], dsc_prev[kb][3],
                              dsc[kb][0], dsc[kb][1], dsc[kb][2], dsc[kb][3]};
        };
        auto scale_a = [&](int kb) {
          return lone ? (hf ? 127 : esc[kb]) : (hf ? esc[kb] : esc_prev[kb]);
        };
        {
          const i32x8 a = operand_a(0);
          const int sa = scale_a(0);
#pragma unroll
          for (int db = 0; db < DBLK; ++db) {
            mfma_scale_bf8_fp8_pinned(dk[0][db], a, operand_b(db), sa, sb);
            __builtin_amdgcn_sched_barrier(0);
            quant(1, db);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        {
          const i32x8 a = operand_a(1);
          const int sa = scale_a(1);
#pragma unroll
          for (int db = 0; db < DBLK; ++db)
            mfma_scale_bf8_fp8_pinned(dk[1][db], a, operand_b(db), sa, sb);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < NPR; ++j) {
        const u32x4 b = qb[j & 1];
        if (j + 2 < NPR) qb[j & 1] = trB(qs, j + 2);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const int g = 2 * NPH + 2 * j + kb;
          mfma_acc_pinned(dk[kb][j % DBLK], dsa[kb][j / DBLK], b);
          if (SPREAD && g <= 38) {
            __builtin_amdgcn_sched_barrier(0);
            slot_work(g);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    }
  };

  int it = 0;
  for (; it + 1 < total; it += 2) {
    body(it, IntConst<0>{});
    body(it + 1, IntConst<1>{});
  }
  if (it < total) body(it, IntConst<0>{});
  wait_vmem();  // the V rows when the loop ran no iteration
  // dK = scale * sum dS^T Q, dV = sum P^T dO.  Accumulator register r of
  // block (kb, db) holds key kbase + 32*kb + 8*(r/4) + 4*hf + r%4 at head dim
  // 32*db + l32.
  uint16_t* dkp = dK + kv_off;
  uint16_t* dvp = dV + kv_off;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
      mfma_acc_drain(dk[kb][db]);
      mfma_acc_drain(dv[kb][db]);
    }
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kbase + kb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
        if (key < Nk) {
          const size_t off = (size_t)key * SK + db * 32 + l32;
          dkp[off] = (uint16_t)(pack_bf16(dk[kb][db][r] * scale, 0.f) & 0xffff);
          dvp[off] = (uint16_t)(pack_bf16(dv[kb][db][r], 0.f) & 0xffff);
        }
      }
}

// The dK/dV kernel: one workgroup per key tile, launched in longest-first
// order (a persistent grid over the same list measured no faster here).
template <int D, bool CAUSAL, bool WIN = false, bool VARLEN = false, bool SPARSE = false,
          bool FP8DS = false>
__global__ __launch_bounds__(kKvWaves * 64, 1) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ Delta,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int Hq, int Hkv, int Nq_arg,
    int Nk_arg, float scale, float scale_log2, int BHkv, int win_l = -1, int win_r = -1,
    const int* __restrict__ cu_q = nullptr, const int* __restrict__ cu_k = nullptr,
    int total_q = 0, const uint8_t* __restrict__ sp_map = nullptr, int sp_nkb = 0,
    const uint8_t* __restrict__ Q8 = nullptr, const int32_t* __restrict__ QE = nullptr) {
  bwd_dkdv_unit<D, CAUSAL, WIN, VARLEN, SPARSE, FP8DS>(
      Q, K, V, dO, LSE, Delta, dK, dV, Hq, Hkv, Nq_arg, Nk_arg, scale, scale_log2, BHkv, win_l,
      win_r, cu_q, cu_k, total_q, sp_map, sp_nkb, Q8, QE, blockIdx.x);
}

// ---------------------------------------------------------------------------
// dQ.  The forward's structure with keys on the MFMA m axis: S^T = K Q^T and
// dP^T = V dO^T with this wave's 32 queries on n (Q and dO rows in registers),
// so lse and delta are per-lane scalars; dS^T (rounded to bf16) is the B
// operand of dQ^T += K^T dS^T, whose A operand is a transposing read of the
// row-major K tile.  K/V tiles of 64 keys are double-buffered in LDS.
// WIN: sliding window as for bwd_dkdv_kernel; only the key tiles that some
// row's window reaches are visited.
// DELTA: the kernel forms its rows' delta = dO . O itself (from O, beside the
// dO rows it holds) and writes it to Delta for the dK/dV kernel that runs after
// it; otherwise it reads Delta from the pre-pass.
// FP8DS: dQ^T += K^T dS^T runs on the 32x32x64 scaled fp8 MFMA ([CH18]
// §18.6.2 (3)): dS^T in e5m2 with one power-of-two scale per (query, 32-key
// block) -- both k-blocks of one product are the tile's two key blocks -- and
// K in e4m3 from the quantiser's per-32-row blocks (K8, e8m0 scale words KE),
// its tile and the tile's two scale words staged in LDS beside the bf16 K
// and V (the tile is read with transposing byte reads).  S and dP stay bf16
// products.
template <int D, bool CAUSAL, bool WIN, bool VARLEN, bool SPARSE, bool DELTA, bool FP8DS>
__device__ __forceinline__ void bwd_dq_unit(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ LSE, float* __restrict__ Delta,
    uint16_t* __restrict__ dQ, int Hq, int Hkv, int Nq_arg, int Nk_arg, float scale,
    float scale_log2, int BH, int nqt, int win_l, int win_r, const int* __restrict__ cu_q,
    const int* __restrict__ cu_k, int total_q, const int* __restrict__ sp_ptr,
    const int* __restrict__ sp_idx, const uint16_t* __restrict__ O,
    const uint8_t* __restrict__ K8, const int32_t* __restrict__ KE, int unit) {
  static_assert(!FP8DS || (D == 128 && !WIN && !VARLEN && !SPARSE), "fp8 dS: dense, d = 128");
  constexpr int NW = kDqWaves;
  constexpr int BR = kDqBr;
  constexpr int BC = kDqBc;
  constexpr int KSTEPS = D / 16;
  constexpr int DBLK = D / 32;
  constexpr int ROWB = D * 2;
  constexpr int TILE = BC * ROWB;
  constexpr int LPW = TILE / 1024 / NW;
  // Three slots, one LDS variable each holding the tile's K and V (and, with
  // FP8DS, its e4m3 K rows and the two K scale words, one 256-byte copy per
  // wave).  The compiler tracks only a few direct-to-LDS destinations one by
  // one; with one variable per slot it sees that a slot being read is not the
  // one in flight and adds no waits of its own.
  constexpr int TILE8 = FP8DS ? BC * D : 0;
  constexpr int KEW = FP8DS ? NW * 256 : 0;
  constexpr int SLOT = 2 * TILE + TILE8 + KEW;
  __shared__ __attribute__((aligned(1024))) char sl0[SLOT], sl1[SLOT], sl2[SLOT];
  auto slot_base = [&](int sl) -> char* { return sl == 0 ? sl0 : sl == 1 ? sl1 : sl2; };
  auto kslot = [&](int sl) -> char* { return slot_base(sl); };
  auto vslot = [&](int sl) -> char* { return slot_base(sl) + TILE; };
  auto k8slot = [&](int sl) -> char* { return slot_base(sl) + 2 * TILE; };
  auto keslot = [&](int sl) -> char* { return slot_base(sl) + 2 * TILE + TILE8; };

  // (opaque to the optimiser: per-lane offsets derived from it are then
  // recomputed for each unit of a persistent loop instead of being kept
  // live, and spilled, across it)
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  int bh, qt;
  query_tile_of(unit, BH, nqt, CAUSAL, &bh, &qt);
  const int b = bh / Hq;
  const int h = bh - b * Hq;
  const int hk = h / (Hq / Hkv);
  const int q0 = qt * BR;
  // Sequence lengths, element offsets and row strides of this unit (as in
  // bwd_dkdv_kernel).
  int Nq = Nq_arg, Nk = Nk_arg;
  size_t q_off = (size_t)bh * Nq * D, kv_off = (size_t)(b * Hkv + hk) * Nk * D;
  size_t l_off = (size_t)bh * Nq;
  const int SQ = VARLEN ? Hq * D : D;
  const int SK = VARLEN ? Hkv * D : D;
  if constexpr (VARLEN) {
    const int qs0 = cu_q[b], ks0 = cu_k[b];
    Nq = cu_q[b + 1] - qs0;
    Nk = cu_k[b + 1] - ks0;
    if (q0 >= Nq) return;  // the whole workgroup: past this sequence's rows
    q_off = ((size_t)qs0 * Hq + h) * D;
    kv_off = ((size_t)ks0 * Hkv + hk) * D;
    l_off = (size_t)h * total_q + qs0;
  }
  const __amdgpu_buffer_rsrc_t rK = make_rsrc(K + kv_off, (uint32_t)Nk * SK * 2);
  const __amdgpu_buffer_rsrc_t rV = make_rsrc(V + kv_off, (uint32_t)Nk * SK * 2);
  // FP8DS: e4m3 K rows (dense [b][hkv][Nk][128]) and their 32-row scale bytes
  const __amdgpu_buffer_rsrc_t rK8 =
      make_rsrc(FP8DS ? (const void*)(K8 + kv_off) : (const void*)K, FP8DS ? (uint32_t)Nk * D : 0u);
  const int nkb8 = (Nk + 31) / 32;
  // (a tile's second key block past the end reads 0 here: a scale of 2^-127
  // on codes that are all zero)
  const __amdgpu_buffer_rsrc_t rKE =
      make_rsrc(FP8DS ? (const void*)(KE + (size_t)(b * Hkv + hk) * nkb8) : (const void*)K,
                FP8DS ? (uint32_t)nkb8 * 4 : 0u);

  const int qrow = q0 + wave * 32 + l32;
  const int qrow_c = qrow < Nq ? qrow : Nq - 1;
  u32x4 qf[KSTEPS], gf[KSTEPS];
  u32x4 of[DELTA ? KSTEPS : 1];
  {
    const uint16_t* qr = Q + q_off + (size_t)qrow_c * SQ;
    const uint16_t* gr = dO + q_off + (size_t)qrow_c * SQ;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      qf[ks] = ldg<u32x4>(qr + ks * 16 + hf * 8);
      gf[ks] = ldg<u32x4>(gr + ks * 16 + hf * 8);
    }
    if constexpr (DELTA) {
      // this lane's half of its row of O, in the layout of its dO elements
      const uint16_t* orow = O + q_off + (size_t)qrow_c * SQ;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) of[ks] = ldg<u32x4>(orow + ks * 16 + hf * 8);
    }
  }
  float lse2 = LSE[l_off + qrow_c] * kLog2e;
  // a row that sees no key (lse = -inf, possible only with a sparse pattern)
  // gets P = 0: every score of it is masked, and -inf - (+inf) = -inf
  if constexpr (SPARSE) lse2 = lse2 == -INFINITY ? INFINITY : lse2;
  float dlt;
  if constexpr (DELTA) {
    // delta_i = dO_i . O_i ([CH18] §18.4.4: rowsum(P * dP) = dO_i . O_i);
    // the two lane halves hold the two halves of the row
    float acc = 0.f;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        acc = fmaf(bf16_lo(of[ks][w]), bf16_lo(gf[ks][w]), acc);
        acc = fmaf(bf16_hi(of[ks][w]), bf16_hi(gf[ks][w]), acc);
      }
    dlt = sum_halves(acc);
  } else {
    dlt = Delta[l_off + qrow_c];
  }
  // dO enters dP^T = V dO^T negated and the dP accumulators start at delta,
  // so that they end at delta - dP and dS = P (dP - delta) is one multiply by
  // -P (the sign flip is exact; the dO fragments serve nothing else below)
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) gf[ks] ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};

  int kv_end = CAUSAL ? min(Nk, q0 + BR) : Nk;
  int jf = 0;  // first key tile visited
  if constexpr (WIN) {
    if (win_r >= 0) kv_end = min(kv_end, q0 + BR + win_r);
    if (win_l >= 0) jf = max(0, q0 - win_l) / BC;
  }
  int ntiles = (kv_end + BC - 1) / BC - jf;
  // SPARSE: this query tile's list of key blocks, one entry per lane and
  // register, read back with readlane (as in the forward).
  int spc[4] = {0, 0, 0, 0};
  if constexpr (SPARSE) {
    static_assert(BR == kSpBq && BC == kSpBk, "sparse block shapes");
    const int lo = sp_ptr[qt];
    ntiles = min(max(sp_ptr[qt + 1] - lo, 0), 256);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (r * 64 + lane < ntiles) spc[r] = sp_idx[lo + r * 64 + lane];
  }
  // key tile visited at loop position j
  auto tile_of = [&](int j) -> int {
    if constexpr (SPARSE) {
      const int v = j < 64 ? spc[0] : j < 128 ? spc[1] : j < 192 ? spc[2] : spc[3];
      return __builtin_amdgcn_readlane(v, j & 63);
    } else {
      return jf + j;
    }
  };

  int ldo[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) ldo[i] = swz_src_offset<ROWB>(lane, wave * LPW + i, SK * 2);
  // FP8DS: wave w moves e4m3 rows 8w .. 8w+7 of a tile (lane -> row 8w +
  // lane/8, LDS chunk position lane%8 holding source chunk (lane%8) ^ swz),
  // and the tile's two scale words into its own LDS copy (lane l: key block
  // l%2 of the tile, at word l).
  static_assert(!FP8DS || BC * D / 1024 == NW, "one 1 KB e4m3 load per wave per tile");
  const int k8row = wave * 8 + (lane >> 3);
  const int k8off = k8row * D + (((lane & 7) ^ f8_swz_t(k8row)) << 4);
  auto issue = [&](int j, int slot) {
    char* dk_ = kslot(slot) + wave * LPW * 1024;
    char* dv_ = vslot(slot) + wave * LPW * 1024;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      buffer_load_lds16(rK, dk_ + i * 1024, ldo[i], tile_of(j) * BC * SK * 2);
      buffer_load_lds16(rV, dv_ + i * 1024, ldo[i], tile_of(j) * BC * SK * 2);
    }
    if constexpr (FP8DS) {
      buffer_load_lds16(rK8, k8slot(slot) + wave * 1024, k8off, tile_of(j) * BC * D);
      buffer_load_lds4(rKE, keslot(slot) + wave * 256, 4 * (lane & 1), tile_of(j) * 8);
    }
  };
  constexpr int LOADS = 2 * LPW + (FP8DS ? 2 : 0);  // per tile and wave
  // A operands of S^T / dP^T (b128): key row kb*32 + l32, chunk 2*ks + hf.
  int ard[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks)
    ard[ks] = l32 * ROWB + (((2 * ks + hf) ^ bwd_swz<ROWB>(l32)) << 4);
  // A operand of dQ^T (transposing read of K): k-step (kb, st) element e of
  // lane half hf is key kb*32 + 16*st + 8*(e/4) + 4*hf + e%4.
  int trd0[DBLK], trd1[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) {
    trd0[db] = tr_offset<ROWB>(lane, 0, 32 * db);
    trd1[db] = tr_offset<ROWB>(lane, 8, 32 * db);
  }

  // FP8DS: A operand of dQ^T from the e4m3 K tile (transposing byte reads):
  // byte i of lane half hf is key 32*(i/16) + 8*((i/4)%4) + 4*hf + i%4 of
  // head dim 32*db + l32.  Source lane 2r + half of 16-lane group g16 addresses
  // key row 8*(r/4) + 4*hf + r%4 (+ 16*(read%2) + 32*(read/2)), head dims
  // 32*db + 16*(g16%2) + 8*half.
  int k8rd[FP8DS ? DBLK : 1];
  if constexpr (FP8DS) {
    const int g16 = lane >> 4, j16 = lane & 15;
    const int vr = j16 >> 1;
    const int row = 8 * (vr >> 2) + 4 * hf + (vr & 3);
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
      k8rd[db] = row * D + (((2 * db + (g16 & 1)) ^ f8_swz_t(row)) << 4) + 8 * (j16 & 1);
  }
  auto k8frag = [&](const char* k8s, int db) {
    int w[8];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const i32x2_t x = lds_read_tr8(k8s + ((t >> 1) * 32 + (t & 1) * 16) * D + k8rd[db]);
      w[2 * t] = x[0];
      w[2 * t + 1] = x[1];
    }
    return i32x8{w[0], w[1], w[2], w[3], w[4], w[5], w[6], w[7]};
  };

  f32x16 dq[DBLK];
#pragma unroll
  for (int i = 0; i < DBLK; ++i) dq[i] = f32x16{0};

#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    settle(qf[ks]);
    settle(gf[ks]);
  }
  settle(lse2);
  settle(dlt);
  // Two K/V tiles in flight while one is computed.  Past the last tile the
  // last one is loaded again into the free slot, so that every step issues
  // the same loads: the wait below is then exact, and the compiler's view of
  // which slot is in flight stays precise enough not to add waits of its own.
  if (ntiles > 0) {
    issue(0, 0);
    issue(min(1, ntiles - 1), 1);
  }
  // One iteration per KV tile; S = slot (a compile-time constant).
  auto body = [&](int j, auto S) {
    constexpr int slot = decltype(S)::value;
    // tile j has landed once at most the next step's loads remain
    wait_vmem_le<LOADS>();
    lds_barrier();
    const char* ks_ = kslot(slot);
    const char* vs_ = vslot(slot);
    const int kv0 = tile_of(j) * BC;

    // Three phases so that the elementwise work runs beside matrix products:
    // (A) S^T = K Q^T; (B) dP^T = V dO^T with P = exp(S*scale - lse) of the
    // finished S computed in place between its products; (C) dS = P (dP -
    // delta) of key block 0, then dQ^T += K^T dS^T for block 0 with block 1's
    // dS computed between its products, then block 1's products.
    constexpr int NAB = 2 * KSTEPS;      // products of phase A (and B)
    constexpr int EPB = 32 / NAB;        // elements per phase-B product
    constexpr int NCB = 2 * DBLK;        // phase-C products per key block
    constexpr int EPC = 16 / NCB;        // block-1 elements per block-0 product
    f32x16 s[2], dp[2];  // dp: set to delta just before phase B
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) s[kb] = f32x16{0};
    // LDS operands are read PF products ahead of their use (the latency of
    // a read is several products long, and only one other wave shares the
    // SIMD to hide it).  Operand m of phases A and B: key block m % 2, k-step
    // m / 2.
    constexpr int PFA = 4, PFB = 3;
    auto ka_of = [&](int m) { return lds_read<u32x4>(ks_, (m & 1) * 32 * ROWB + ard[m >> 1]); };
    auto va_of = [&](int m) { return lds_read<u32x4>(vs_, (m & 1) * 32 * ROWB + ard[m >> 1]); };
    // Phase B's operand order: FP8DS takes key block 0's eight products
    // first, so that block 0's dS can be formed and quantised beside block
    // 1's products; otherwise the blocks alternate.
    auto vb_of = [&](int m) { return va_of(FP8DS ? (((m & 7) << 1) | (m >> 3)) : m); };
    // (A)
    u32x4 va[PFB];
    {
      u32x4 ka[PFA];
#pragma unroll
      for (int p = 0; p < PFA; ++p) ka[p] = ka_of(p);
      // next tile's loads after this tile's first LDS reads
      asm volatile("" ::: "memory");
      issue(min(j + 2, ntiles - 1), (slot + 2) % 3);
#pragma unroll
      for (int m = 0; m < NAB; ++m) {
        const int kk = m >> 1, kb = m & 1;
        const u32x4 a = ka[m % PFA];
        if (m + PFA < NAB) ka[m % PFA] = ka_of(m + PFA);
        else if (m + PFA - NAB < PFB) va[m + PFA - NAB] = vb_of(m + PFA - NAB);
        s[kb] = mfma_32x32x16_bf16(a, qf[kk], s[kb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    const int rw0 = q0 + wave * 32;  // this wave's first row
    bool need_mask = (kv0 + BC > Nk) || (CAUSAL && kv0 + BC - 1 > rw0);
    if constexpr (WIN)
      need_mask = need_mask || (win_l >= 0 && kv0 < rw0 + 31 - win_l) ||
                  (win_r >= 0 && kv0 + BC - 1 > rw0 + win_r);
    if constexpr (SPARSE) need_mask = need_mask || kv0 < 0;  // a bad list entry
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + kb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
          bool out = key >= Nk || (CAUSAL && key > qrow);
          if constexpr (WIN)
            out = out || (win_l >= 0 && key < qrow - win_l) || (win_r >= 0 && key > qrow + win_r);
          if constexpr (SPARSE) out = out || key < 0;
          s[kb][r] = out ? -INFINITY : s[kb][r];
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    // (B)
    // FP8DS: dS = P (dP - delta) in fp32 with one power-of-two scale per
    // (query, 32-key block), the block maximum taken over this lane's 16 keys
    // and the other half's 16; codes in e5m2.  Byte i of this lane's 32 is
    // key 32*(i/16) + 8*((i/4)%4) + 4*hf + i%4, the order of the S
    // accumulator (and of the K^T fragments).  Key block 0 is done between
    // block 1's dP products, block 1 after them.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      dp[kb] = f32x16{dlt, dlt, dlt, dlt, dlt, dlt, dlt, dlt,
                      dlt, dlt, dlt, dlt, dlt, dlt, dlt, dlt};
    float am0 = 0.f, am1 = 0.f, sc0 = 1.f;
    int e0 = 0;
    int w8[FP8DS ? 8 : 1];
    auto ds_slice = [&](int kb, int i) {  // elements 4i .. 4i+3 of key block kb
#pragma unroll
      for (int r = 4 * i; r < 4 * i + 4; ++r) {
        dp[kb][r] = -s[kb][r] * dp[kb][r];
        if (kb == 0) am0 = fmaxf(am0, fabsf(dp[0][r]));
        else am1 = fmaxf(am1, fabsf(dp[1][r]));
      }
    };
    auto cvt_slice = [&](int kb, int i, float sc) {  // dword 4*kb + i of the codes
      const int r0 = 4 * i;
      w8[4 * kb + i] = cvt_bf8x4_div(dp[kb][r0], dp[kb][r0 + 1], dp[kb][r0 + 2], dp[kb][r0 + 3], sc);
    };
    {
#pragma unroll
      for (int m = 0; m < NAB; ++m) {
        const int kk = FP8DS ? (m & 7) : (m >> 1), kb = FP8DS ? (m >> 3) : (m & 1);
        const u32x4 a = va[m % PFB];
        if (m + PFB < NAB) va[m % PFB] = vb_of(m + PFB);
        dp[kb] = mfma_32x32x16_bf16(a, gf[kk], dp[kb]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < EPB; ++t) {
          const int x = EPB * m + t;
          s[x >> 4][x & 15] = fast_exp2(fmaf(s[x >> 4][x & 15], scale_log2, -lse2));
        }
        if constexpr (FP8DS) {
          static_assert(NAB == 16, "block 0's work spread over block 1's eight products");
          if (m >= 8 && m < 12) ds_slice(0, m - 8);
          if (m == 12) {
            e0 = pow2_block_exp<16>(max_halves(am0));
            sc0 = exp2_pos(e0);
          }
          if (m == 13) { cvt_slice(0, 0, sc0); cvt_slice(0, 1, sc0); }
          if (m == 14) { cvt_slice(0, 2, sc0); cvt_slice(0, 3, sc0); }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // (C)
    if constexpr (FP8DS) {
      const char* k8s = k8slot(slot);
      i32x8 ka8 = k8frag(k8s, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) ds_slice(1, i);
      const int e1 = pow2_block_exp<16>(max_halves(am1));
      const float sc1 = exp2_pos(e1);
#pragma unroll
      for (int i = 0; i < 4; ++i) cvt_slice(1, i, sc1);
      const i32x8 ds8 = i32x8{w8[0], w8[1], w8[2], w8[3], w8[4], w8[5], w8[6], w8[7]};
      // scale operands: lane half hf supplies key block hf's scale
      const int sb = (hf ? e1 : e0) + 127;
      const int sa = lds_read<int>(keslot(slot) + wave * 256, 4 * hf);
#pragma unroll
      for (int db = 0; db < DBLK; ++db) {
        const i32x8 a = ka8;
        if (db + 1 < DBLK) ka8 = k8frag(k8s, db + 1);
        dq[db] = mfma_32x32x64_fp8_bf8_scaled(a, ds8, dq[db], sa, sb);
        __builtin_amdgcn_sched_barrier(0);
      }
      return;
    }
    u32x4 dsb[2][2];
    auto ds_elem = [&](int kb, int r) {
      dp[kb][r] = -s[kb][r] * dp[kb][r];
      if (r & 1) {
        const int st = r >> 3, w = (r & 7) >> 1;
        dsb[kb][st][w] = pack_bf16(dp[kb][r - 1], dp[kb][r]);
      }
    };
    auto kfragT = [&](int kb, int st, int db) {
      const char* kp = ks_ + (kb * 32 + st * 16) * ROWB;
      const u32x2 a0 = lds_read_tr16(kp + trd0[db]);
      const u32x2 a1 = lds_read_tr16(kp + trd1[db]);
      return u32x4{a0[0], a0[1], a1[0], a1[1]};
    };
    {
      // operand m: key block m / NCB, k-step (m / DBLK) % 2, head-dim block m % DBLK
      auto kt_of = [&](int m) { return kfragT(m / NCB, (m / DBLK) & 1, m % DBLK); };
      u32x4 kt[2] = {kt_of(0), kt_of(1)};
#pragma unroll
      for (int r = 0; r < 16; ++r) ds_elem(0, r);
#pragma unroll
      for (int m = 0; m < 2 * NCB; ++m) {
        const int kb = m / NCB, st = (m / DBLK) & 1, db = m % DBLK;
        const u32x4 a = kt[m & 1];
        if (m + 2 < 2 * NCB) kt[m & 1] = kt_of(m + 2);
        dq[db] = mfma_32x32x16_bf16(a, dsb[kb][st], dq[db]);
        __builtin_amdgcn_sched_barrier(0);
        if (m < NCB) {
#pragma unroll
          for (int t = 0; t < EPC; ++t) ds_elem(1, EPC * m + t);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  if constexpr (FP8DS) {
    // (in this form the compiler's waits in the fp8 variant are already
    // exact, and peeling the remainder as below makes it spill)
    for (int j = 0; j < ntiles; j += 3) {
      body(j, IntConst<0>{});
      if (j + 1 < ntiles) body(j + 1, IntConst<1>{});
      if (j + 2 < ntiles) body(j + 2, IntConst<2>{});
    }
  } else {
    // Whole rounds of three in the loop and the remainder after it: the
    // loop's back edge then always follows the same three steps, so the
    // compiler's view of which slots are in flight at the loop head is exact
    // (with a partial round able to reach the back edge it waited there for
    // every load in flight, the next tiles' included).
    int j = 0;
    for (; j + 3 <= ntiles; j += 3) {
      body(j, IntConst<0>{});
      body(j + 1, IntConst<1>{});
      body(j + 2, IntConst<2>{});
    }
    if (j < ntiles) body(j, IntConst<0>{});
    if (j + 1 < ntiles) body(j + 1, IntConst<1>{});
  }
  wait_vmem();  // the reloads of the last tile

  // (written last: a store among the loop's loads would upset its exact
  // load-count waits)
  if constexpr (DELTA)
    if (hf == 0 && qrow < Nq) Delta[l_off + qrow] = dlt;
  // dQ = scale * dQ^T, written as bf16 rows.
  if (qrow < Nq) {
    uint16_t* op = dQ + q_off + (size_t)qrow * SQ;
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = db * 32 + g * 8 + hf * 4;
        stg<u32x2>(op + d0, u32x2{pack_bf16(dq[db][4 * g] * scale, dq[db][4 * g + 1] * scale),
                                  pack_bf16(dq[db][4 * g + 2] * scale, dq[db][4 * g + 3] * scale)});
      }
  }
}

// The dQ kernel: one workgroup per query tile in longest-first order, or
// (PERSIST) a persistent grid walking that list in snake order, as for the
// forward.
template <int D, bool CAUSAL, bool WIN = false, bool VARLEN = false, bool SPARSE = false,
          bool DELTA = false, bool PERSIST = false, bool FP8DS = false>
__global__ __launch_bounds__(kDqWaves * 64, 1) void bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ LSE, float* __restrict__ Delta,
    uint16_t* __restrict__ dQ, int Hq, int Hkv, int Nq_arg, int Nk_arg, float scale,
    float scale_log2, int BH, int nqt, int win_l = -1, int win_r = -1,
    const int* __restrict__ cu_q = nullptr, const int* __restrict__ cu_k = nullptr,
    int total_q = 0, const int* __restrict__ sp_ptr = nullptr,
    const int* __restrict__ sp_idx = nullptr, const uint16_t* __restrict__ O = nullptr,
    const uint8_t* __restrict__ K8 = nullptr, const int32_t* __restrict__ KE = nullptr) {
  if constexpr (PERSIST) {
    const int n = BH * nqt;
    for (int i = 0;; ++i) {
      const int p = persistent_position(i, blockIdx.x, gridDim.x);
      if (p >= n) break;
      bwd_dq_unit<D, CAUSAL, WIN, VARLEN, SPARSE, DELTA, FP8DS>(
          Q, K, V, dO, LSE, Delta, dQ, Hq, Hkv, Nq_arg, Nk_arg, scale, scale_log2, BH, nqt, win_l,
          win_r, cu_q, cu_k, total_q, sp_ptr, sp_idx, O, K8, KE, p);
      __syncthreads();  // every wave is done with the LDS slots before the next unit
    }
  } else {
    bwd_dq_unit<D, CAUSAL, WIN, VARLEN, SPARSE, DELTA, FP8DS>(
        Q, K, V, dO, LSE, Delta, dQ, Hq, Hkv, Nq_arg, Nk_arg, scale, scale_log2, BH, nqt, win_l,
        win_r, cu_q, cu_k, total_q, sp_ptr, sp_idx, O, K8, KE, blockIdx.x);
  }
}

// ---------------------------------------------------------------------------

hipError_t launch_bwd_f32(const float* q, const float* k, const float* v, const float* o,
                          const float* dout, const float* lse, float* dq, float* dk, float* dv,
                          float* delta, int B, int Hq, int Hkv, int Nq, int Nk, float scale,
                          bool causal, hipStream_t stream) {
  const int rows = B * Hq * Nq;
  hipLaunchKernelGGL((bwd_delta_kernel<float, 64>), dim3((rows + 15) / 16), dim3(256), 0,
                     stream, o, dout, delta, rows, 1);
  hipLaunchKernelGGL(bwd_f32_dq_kernel, dim3((Nq + kBF32T - 1) / kBF32T, B * Hq), dim3(64), 0,
                     stream, q, k, v, dout, lse, delta, dq, Hq, Hkv, Nq, Nk, scale,
                     causal ? 1 : 0);
  hipLaunchKernelGGL(bwd_f32_dkv_kernel, dim3((Nk + 31) / 32, B * Hkv), dim3(64), 0, stream, q,
                     k, v, dout, lse, delta, dk, dv, Hq, Hkv, Nq, Nk, scale, causal ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_bwd_pre(const void* o, const void* dout, float* delta, int B, int Hq, int Nq,
                          int d, hipStream_t stream, int heads) {
  const int rows = B * Hq * Nq;
  const __bf16* ob = (const __bf16*)o;
  const __bf16* gb = (const __bf16*)dout;
  if (d == 128)
    hipLaunchKernelGGL((bwd_delta_kernel<__bf16, 128>), dim3((rows + 15) / 16), dim3(256), 0,
                       stream, ob, gb, delta, rows, heads);
  else
    hipLaunchKernelGGL((bwd_delta_kernel<__bf16, 64>), dim3((rows + 15) / 16), dim3(256), 0,
                       stream, ob, gb, delta, rows, heads);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout,
                           const float* lse, const float* delta, void* dk, void* dv, int B,
                           int Hq, int Hkv, int Nq, int Nk, int d, float scale, bool causal,
                           hipStream_t stream, int win_l, int win_r) {
  const int BHkv = B * Hkv;
  dim3 grid(BHkv * ((Nk + kKvBkv - 1) / kKvBkv)), block(kKvWaves * 64);
  auto Q = (const uint16_t*)q;
  auto K = (const uint16_t*)k;
  auto V = (const uint16_t*)v;
  auto G = (const uint16_t*)dout;
  auto dK = (uint16_t*)dk;
  auto dV = (uint16_t*)dv;
  const float sl2 = scale * kLog2e;
#define FA_LAUNCH_DKDV(DD, CC, WW)                                                          \
  hipLaunchKernelGGL((bwd_dkdv_kernel<DD, CC, WW>), grid, block, dkdv_vbuf_bytes(DD), stream, \
                     Q, K, V, G, lse, delta, dK, dV, Hq, Hkv, Nq, Nk, scale, sl2, BHkv, win_l,  \
                     win_r)
  const bool win = win_l >= 0 || win_r >= 0;
  if (d == 128) {
    if (win) {
      if (causal) FA_LAUNCH_DKDV(128, true, true);
      else FA_LAUNCH_DKDV(128, false, true);
    } else {
      if (causal) FA_LAUNCH_DKDV(128, true, false);
      else FA_LAUNCH_DKDV(128, false, false);
    }
  } else {
    if (win) {
      if (causal) FA_LAUNCH_DKDV(64, true, true);
      else FA_LAUNCH_DKDV(64, false, true);
    } else {
      if (causal) FA_LAUNCH_DKDV(64, true, false);
      else FA_LAUNCH_DKDV(64, false, false);
    }
  }
#undef FA_LAUNCH_DKDV
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, const void* dout,
                         const float* lse, float* delta, void* dq, int B, int Hq, int Hkv,
                         int Nq, int Nk, int d, float scale, bool causal, hipStream_t stream,
                         int win_l, int win_r, const void* o) {
  const int BH = B * Hq;
  const int nqt = (Nq + kDqBr - 1) / kDqBr;
  dim3 grid(BH * nqt), block(kDqWaves * 64);
  auto Q = (const uint16_t*)q;
  auto K = (const uint16_t*)k;
  auto V = (const uint16_t*)v;
  auto G = (const uint16_t*)dout;
  auto dQ = (uint16_t*)dq;
  auto Op = (const uint16_t*)o;
  const float sl2 = scale * kLog2e;
#define FA_LAUNCH_DQ(DD, CC, WW)                                                                 \
  do {                                                                                           \
    if (Op)                                                                                      \
      hipLaunchKernelGGL((bwd_dq_kernel<DD, CC, WW, false, false, true>), grid, block, 0, stream, \
                         Q, K, V, G, lse, delta, dQ, Hq, Hkv, Nq, Nk, scale, sl2, BH, nqt, win_l,  \
                         win_r, nullptr, nullptr, 0, nullptr, nullptr, Op);                        \
    else                                                                                         \
      hipLaunchKernelGGL((bwd_dq_kernel<DD, CC, WW>), grid, block, 0, stream, Q, K, V, G, lse,     \
                         delta, dQ, Hq, Hkv, Nq, Nk, scale, sl2, BH, nqt, win_l, win_r);           \
  } while (0)
  // causal: a persistent grid over the longest-first list (as for the forward)
#define FA_LAUNCH_DQ_PERSIST(DD)                                                                 \
  do {                                                                                           \
    const dim3 pg(persistent_grid(BH * nqt));                                                    \
    if (Op)                                                                                      \
      hipLaunchKernelGGL((bwd_dq_kernel<DD, true, false, false, false, true, true>), pg, block, 0, \
                         stream, Q, K, V, G, lse, delta, dQ, Hq, Hkv, Nq, Nk, scale, sl2, BH, nqt, \
                         -1, -1, nullptr, nullptr, 0, nullptr, nullptr, Op);                      \
    else                                                                                         \
      hipLaunchKernelGGL((bwd_dq_kernel<DD, true, false, false, false, false, true>), pg, block,  \
                         0, stream, Q, K, V, G, lse, delta, dQ, Hq, Hkv, Nq, Nk, scale, sl2, BH,  \
                         nqt);                                                                   \
  } while (0)
  const bool win = win_l >= 0 || win_r >= 0;
  if (d == 128) {
    if (win) {
      if (causal) FA_LAUNCH_DQ(128, true, true);
      else FA_LAUNCH_DQ(128, false, true);
    } else {
      if (causal) FA_LAUNCH_DQ_PERSIST(128);
      else FA_LAUNCH_DQ(128, false, false);
    }
  } else {
    if (win) {
      if (causal) FA_LAUNCH_DQ(64, true, true);
      else FA_LAUNCH_DQ(64, false, true);
    } else {
      if (causal) FA_LAUNCH_DQ_PERSIST(64);
      else FA_LAUNCH_DQ(64, false, false);
    }
  }
#undef FA_LAUNCH_DQ
#undef FA_LAUNCH_DQ_PERSIST
  return hipGetLastError();
}

hipError_t launch_bwd_dq_fp8(const void* q, const void* k, const void* v, const void* dout,
                             const float* lse, float* delta, void* dq, const uint8_t* k8,
                             const int32_t* ke, const void* o, int B, int Hq, int Hkv, int Nq,
                             int Nk, float scale, bool causal, hipStream_t stream) {
  const int BH = B * Hq;
  const int nqt = (Nq + kDqBr - 1) / kDqBr;
  const dim3 block(kDqWaves * 64);
  auto Q = (const uint16_t*)q;
  auto K = (const uint16_t*)k;
  auto V = (const uint16_t*)v;
  auto G = (const uint16_t*)dout;
  auto dQ = (uint16_t*)dq;
  auto Op = (const uint16_t*)o;
  const float sl2 = scale * kLog2e;
  if (causal)
    hipLaunchKernelGGL((bwd_dq_kernel<128, true, false, false, false, true, true, true>),
                       dim3(persistent_grid(BH * nqt)), block, 0, stream, Q, K, V, G, lse, delta,
                       dQ, Hq, Hkv, Nq, Nk, scale, sl2, BH, nqt, -1, -1, nullptr, nullptr, 0,
                       nullptr, nullptr, Op, k8, ke);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<128, false, false, false, false, true, false, true>),
                       dim3(BH * nqt), block, 0, stream, Q, K, V, G, lse, delta, dQ, Hq, Hkv, Nq,
                       Nk, scale, sl2, BH, nqt, -1, -1, nullptr, nullptr, 0, nullptr, nullptr, Op,
                       k8, ke);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv_fp8(const void* q, const void* k, const void* v, const void* dout,
                               const float* lse, const float* delta, void* dk, void* dv,
                               const uint8_t* q8, const int32_t* qe, int B, int Hq, int Hkv,
                               int Nq, int Nk, float scale, bool causal, hipStream_t stream) {
  const int BHkv = B * Hkv;
  const dim3 grid(BHkv * ((Nk + kKvBkv - 1) / kKvBkv)), block(kKvWaves * 64);
  auto Q = (const uint16_t*)q;
  auto K = (const uint16_t*)k;
  auto V = (const uint16_t*)v;
  auto G = (const uint16_t*)dout;
  auto dK = (uint16_t*)dk;
  auto dV = (uint16_t*)dv;
  const float sl2 = scale * kLog2e;
  if (causal)
    hipLaunchKernelGGL((bwd_dkdv_kernel<128, true, false, false, false, true>), grid, block,
                       dkdv_vbuf_bytes(128), stream, Q, K, V, G, lse, delta, dK, dV, Hq, Hkv, Nq,
                       Nk, scale, sl2, BHkv, -1, -1, nullptr, nullptr, 0, nullptr, 0, q8, qe);
  else
    hipLaunchKernelGGL((bwd_dkdv_kernel<128, false, false, false, false, true>), grid, block,
                       dkdv_vbuf_bytes(128), stream, Q, K, V, G, lse, delta, dK, dV, Hq, Hkv, Nq,
                       Nk, scale, sl2, BHkv, -1, -1, nullptr, nullptr, 0, nullptr, 0, q8, qe);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv_varlen(const void* q, const void* k, const void* v, const void* dout,
                                  const float* lse, const float* delta, void* dk, void* dv,
                                  const int* cu_q, const int* cu_k, int batch, int Hq, int Hkv,
                                  int total_q, int max_seqlen_k, int d, float scale, bool causal,
                                  hipStream_t stream) {
  const int BHkv = batch * Hkv;
  dim3 grid(BHkv * ((max_seqlen_k + kKvBkv - 1) / kKvBkv)), block(kKvWaves * 64);
  auto Q = (const uint16_t*)q;
  auto K = (const uint16_t*)k;
  auto V = (const uint16_t*)v;
  auto G = (const uint16_t*)dout;
  auto dK = (uint16_t*)dk;
  auto dV = (uint16_t*)dv;
  const float sl2 = scale * kLog2e;
#define FA_LAUNCH_DKDV_VL(DD, CC)                                                            \
  hipLaunchKernelGGL((bwd_dkdv_kernel<DD, CC, false, true>), grid, block, dkdv_vbuf_bytes(DD), \
                     stream, Q, K, V, G, lse, delta, dK, dV, Hq, Hkv, 0, 0, scale, sl2, BHkv,   \
                     -1, -1, cu_q, cu_k, total_q)
  if (d == 128) {
    if (causal) FA_LAUNCH_DKDV_VL(128, true);
    else FA_LAUNCH_DKDV_VL(128, false);
  } else {
    if (causal) FA_LAUNCH_DKDV_VL(64, true);
    else FA_LAUNCH_DKDV_VL(64, false);
  }
#undef FA_LAUNCH_DKDV_VL
  return hipGetLastError();
}

hipError_t launch_bwd_dq_varlen(const void* q, const void* k, const void* v, const void* dout,
                                const float* lse, float* delta, void* dq, const int* cu_q,
                                const int* cu_k, int batch, int Hq, int Hkv, int total_q,
                                int max_seqlen_q, int d, float scale, bool causal,
                                hipStream_t stream, const void* o) {
  const int BH = batch * Hq;
  const int nqt = (max_seqlen_q + kDqBr - 1) / kDqBr;
  dim3 grid(BH * nqt), block(kDqWaves * 64);
  auto Q = (const uint16_t*)q;
  auto K = (const uint16_t*)k;
  auto V = (const uint16_t*)v;
  auto G = (const uint16_t*)dout;
  auto dQ = (uint16_t*)dq;
  auto Op = (const uint16_t*)o;
  const float sl2 = scale * kLog2e;
#define FA_LAUNCH_DQ_VL(DD, CC)                                                                  \
  do {                                                                                           \
    if (Op)                                                                                      \
      hipLaunchKernelGGL((bwd_dq_kernel<DD, CC, false, true, false, true>), grid, block, 0,      \
                         stream, Q, K, V, G, lse, delta, dQ, Hq, Hkv, 0, 0, scale, sl2, BH, nqt, \
                         -1, -1, cu_q, cu_k, total_q, nullptr, nullptr, Op);                     \
    else                                                                                         \
      hipLaunchKernelGGL((bwd_dq_kernel<DD, CC, false, true>), grid, block, 0, stream, Q, K, V,  \
                         G, lse, delta, dQ, Hq, Hkv, 0, 0, scale, sl2, BH, nqt, -1, -1, cu_q,     \
                         cu_k, total_q);                                                         \
  } while (0)
  if (d == 128) {
    if (causal) FA_LAUNCH_DQ_VL(128, true);
    else FA_LAUNCH_DQ_VL(128, false);
  } else {
    if (causal) FA_LAUNCH_DQ_VL(64, true);
    else FA_LAUNCH_DQ_VL(64, false);
  }
#undef FA_LAUNCH_DQ_VL
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Block-sparse backward.  The dQ kernel walks each query tile's list as the
// forward does; the dK/dV kernel needs the opposite direction (which query
// blocks list a key block), read from a byte map map[t][c] = 1 iff key block
// c is in query tile t's list (entries past 256 and outside [0, nkb) are
// ignored, as the forward ignores them).  One workgroup per query tile.
__global__ __launch_bounds__(256) void sparse_block_map_kernel(const int* __restrict__ sp_ptr,
                                                               const int* __restrict__ sp_idx,
                                                               uint8_t* __restrict__ map,
                                                               int nkb) {
  const int t = blockIdx.x;
  uint8_t* row = map + (size_t)t * nkb;
  for (int c = threadIdx.x; c < nkb; c += 256) row[c] = 0;
  __syncthreads();  // the zeros land before any entry is set
  const int lo = sp_ptr[t];
  const int n = min(max(sp_ptr[t + 1] - lo, 0), 256);
  for (int e = threadIdx.x; e < n; e += 256) {
    const int c = sp_idx[lo + e];
    if (c >= 0 && c < nkb) row[c] = 1;
  }
}

hipError_t launch_bwd_bf16_sparse(const void* q, const void* k, const void* v, const void* dout,
                                  const float* lse, float* delta, uint8_t* map, void* dq,
                                  void* dk, void* dv, const int* sp_ptr, const int* sp_idx, int B,
                                  int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                                  bool causal, hipStream_t stream, const void* o) {
  const int nqb = (Nq + kSpBq - 1) / kSpBq;
  const int nkb = (Nk + kSpBk - 1) / kSpBk;
  hipLaunchKernelGGL(sparse_block_map_kernel, dim3(nqb), dim3(256), 0, stream, sp_ptr, sp_idx,
                     map, nkb);
  auto Q = (const uint16_t*)q;
  auto K = (const uint16_t*)k;
  auto V = (const uint16_t*)v;
  auto G = (const uint16_t*)dout;
  auto Op = (const uint16_t*)o;
  const float sl2 = scale * kLog2e;
  // dQ first: with o given it also writes delta, which dK/dV then reads
  const int BH = B * Hq;
  const int nqt = (Nq + kDqBr - 1) / kDqBr;
  dim3 grid_q(BH * nqt), block_q(kDqWaves * 64);
  auto dQ = (uint16_t*)dq;
#define FA_LAUNCH_DQ_SP(DD, CC)                                                                  \
  do {                                                                                           \
    if (Op)                                                                                      \
      hipLaunchKernelGGL((bwd_dq_kernel<DD, CC, false, false, true, true>), grid_q, block_q, 0,  \
                         stream, Q, K, V, G, lse, delta, dQ, Hq, Hkv, Nq, Nk, scale, sl2, BH,    \
                         nqt, -1, -1, nullptr, nullptr, 0, sp_ptr, sp_idx, Op);                  \
    else                                                                                         \
      hipLaunchKernelGGL((bwd_dq_kernel<DD, CC, false, false, true>), grid_q, block_q, 0, stream, \
                         Q, K, V, G, lse, delta, dQ, Hq, Hkv, Nq, Nk, scale, sl2, BH, nqt, -1,    \
                         -1, nullptr, nullptr, 0, sp_ptr, sp_idx);                               \
  } while (0)
  if (d == 128) {
    if (causal) FA_LAUNCH_DQ_SP(128, true);
    else FA_LAUNCH_DQ_SP(128, false);
  } else {
    if (causal) FA_LAUNCH_DQ_SP(64, true);
    else FA_LAUNCH_DQ_SP(64, false);
  }
#undef FA_LAUNCH_DQ_SP
  const int BHkv = B * Hkv;
  dim3 grid_kv(BHkv * ((Nk + kKvBkv - 1) / kKvBkv)), block_kv(kKvWaves * 64);
  auto dK = (uint16_t*)dk;
  auto dV = (uint16_t*)dv;
#define FA_LAUNCH_DKDV_SP(DD, CC)                                                              \
  hipLaunchKernelGGL((bwd_dkdv_kernel<DD, CC, false, false, true>), grid_kv, block_kv,          \
                     dkdv_vbuf_bytes(DD), stream, Q, K, V, G, lse, delta, dK, dV, Hq, Hkv, Nq, \
                     Nk, scale, sl2, BHkv, -1, -1, nullptr, nullptr, 0, map, nkb)
  if (d == 128) {
    if (causal) FA_LAUNCH_DKDV_SP(128, true);
    else FA_LAUNCH_DKDV_SP(128, false);
  } else {
    if (causal) FA_LAUNCH_DKDV_SP(64, true);
    else FA_LAUNCH_DKDV_SP(64, false);
  }
#undef FA_LAUNCH_DKDV_SP
  return hipGetLastError();
}

}  // namespace fa

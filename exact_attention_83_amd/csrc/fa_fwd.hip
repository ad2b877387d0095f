// Forward attention kernels for gfx950.
//
// Method: [CH18] "第 18 章 FlashAttention" §18.4.3 (tiled forward, Fig. 18-16)
// and §18.5.1-18.5.2 (work split per query tile, causal tile skipping); the
// rescaling step is the two-block identity of [L21] "CMU 11-868 L21
// FlashAttention" slide 12.
//
// bf16 kernel layout (one workgroup = 8 waves = 256 query rows, two waves per
// SIMD, KV tiles of 64 keys):
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
//     destination bit) through two slots each, K two tiles ahead of use and V
//     one; each iteration interleaves the QK^T products of tile i+1 and the
//     PV products of tile i-1 with the softmax work of tile i (one barrier
//     per tile).
//   * the running max is lazy: p is computed against a reference that moves
//     only when a tile's sum of p grows past a bound.
//   * exp is exp2 with scale*log2(e) folded into one FMA; O is divided by the
//     row sum once at the end ([CH18] §18.4.3 step 9).

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kFwdWaves = 8;
constexpr int kFwdBr = 32 * kFwdWaves;  // query rows per workgroup
constexpr int kFwdBc = 64;              // keys per KV tile
constexpr int kFwdStages = 2;           // K/V slots

}  // namespace

int fwd_kv_tiles(int qt, int Nk, bool causal, int br, int bc) {
  int last = causal ? ((qt + 1) * br < Nk ? (qt + 1) * br : Nk) : Nk;
  return (last + bc - 1) / bc;
}

// Chunk swizzles of the K and V tiles (see fwd_bf16_kernel).  K: rows r..r+15
// read one chunk each; V: rows 4i..4i+3 read four consecutive chunks each.
template <int D>
__device__ __forceinline__ int fwd_swz_k(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int fwd_swz_v(int r) {
  return D == 128 ? (4 * (r & 3)) : (4 * ((r >> 1) & 1));
}

// VARLEN: packed variable-length batch ([CH18] §18.7.1): Q/O are token-major
// [total_q][Hq][D], K/V [total_k][Hkv][D]; sequence b owns query rows
// cu_q[b] .. cu_q[b+1]-1 and key rows cu_k[b] .. cu_k[b+1]-1, and its
// attention (causal: top-left) stays inside them; LSE is [Hq][total_q].  The
// grid covers batch x Hq x (query tiles of the longest sequence); tiles past
// a sequence's end exit at once.
// WIN: sliding window ([CH18] §18.7.1, window_size = (left, right)): key j is
// visible to query i only if i - win_l <= j <= i + win_r (a negative bound is
// unbounded); only the key tiles that intersect some row's window are
// visited.
// SPARSE: block-sparse pattern ([CH18] §18.8.1): query tile t (BR rows)
// visits only the 64-key tiles sp_idx[sp_ptr[t] .. sp_ptr[t+1]-1] (at most
// 256 of them), the same list for every (b, head).  A row that sees no key
// gets O = 0 and LSE = -inf.
// One work unit (one query tile of one (b, head)); `unit` is its position in
// the longest-first list.
template <int D, bool CAUSAL, int NW, int NS, bool VARLEN, bool WIN, bool SPARSE>
__device__ __forceinline__ void fwd_bf16_unit(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE,
    int Hq, int Hkv, int Nq_arg, int Nk_arg, float scale, float scale_log2, int BH, int nqt,
    const int* __restrict__ cu_q, const int* __restrict__ cu_k, int total_q, int win_l,
    int win_r, const int* __restrict__ sp_ptr, const int* __restrict__ sp_idx, int unit) {
  constexpr int BC = kFwdBc;
  constexpr int ROWB = D * 2;               // bytes per K/V row in LDS (no padding)
  constexpr int NCH = D / 8;                // 16-byte chunks per row
  constexpr int TILE = BC * ROWB;           // bytes of one K or V tile
  constexpr int BR = 32 * NW;               // query rows per workgroup
  constexpr int LPW = TILE / 1024 / NW;     // 1 KB direct loads per wave per tile
  constexpr int RPL = 1024 / ROWB;          // rows per 1 KB load
  constexpr int KSTEPS = D / 16;            // MFMA k-steps over the head dim
  constexpr int DBLK = D / 32;              // 32-wide blocks of the head dim
  // LDS: NS K slots and NS V slots.  Rows are stored unpadded
  // with the 16-byte chunks XOR-swizzled per row (chunk c of row r at position
  // c ^ sw(r)), so that the b128 reads of K (16 consecutive rows, one chunk)
  // and the transposing b64 reads of V (4 consecutive rows x 4 chunks) hit
  // distinct banks of the 64-bank LDS.
  //
  // Every K and V slot is an LDS variable of its own: the compiler then knows
  // which slot a direct load writes and does not make the reads of the other
  // slots wait for it (with one array it would wait for every outstanding
  // load before any LDS read).  Slot indices are compile-time constants.
  static_assert(NS == 2 || NS == 4, "stages");
  __shared__ __attribute__((aligned(1024))) char kb0[TILE], kb1[TILE], kb2[TILE], kb3[TILE];
  __shared__ __attribute__((aligned(1024))) char vb0[TILE], vb1[TILE], vb2[TILE], vb3[TILE];
  auto kslot = [&](int s) -> char* { return s == 0 ? kb0 : s == 1 ? kb1 : s == 2 ? kb2 : kb3; };
  auto vslot = [&](int s) -> char* { return s == 0 ? vb0 : s == 1 ? vb1 : s == 2 ? vb2 : vb3; };

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
  // This work unit's query and key counts, bases and row strides (elements
  // between consecutive rows: D for [B][H][N][D], H*D when packed).
  int Nq = Nq_arg, Nk = Nk_arg;
  size_t q_base = (size_t)bh * Nq * D;
  size_t kv_off = (size_t)(b * Hkv + hk) * Nk * D;
  size_t lse_base = (size_t)bh * Nq;
  const int SQ = VARLEN ? Hq * D : D;
  const int SKVB = (VARLEN ? Hkv * D : D) * 2;  // bytes
  const int q0 = qt * BR;
  const int qrow = q0 + wave * 32 + l32;
  if constexpr (VARLEN) {
    const int qs0 = cu_q[b], ks0 = cu_k[b];
    Nq = cu_q[b + 1] - qs0;
    Nk = cu_k[b + 1] - ks0;
    if (q0 >= Nq) return;  // the whole workgroup: past this sequence's rows
    q_base = ((size_t)qs0 * Hq + h) * D;
    kv_off = ((size_t)ks0 * Hkv + hk) * D;
    lse_base = (size_t)h * total_q + qs0;
    if (Nk <= 0) {  // no visible key: O = 0, LSE = -inf
      if (qrow < Nq) {
        uint16_t* Op = O + q_base + (size_t)qrow * SQ;
#pragma unroll
        for (int db = 0; db < DBLK; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) stg<u32x2>(Op + db * 32 + g * 8 + hf * 4, u32x2{0u, 0u});
        if (hf == 0) LSE[lse_base + qrow] = -INFINITY;
      }
      return;
    }
  }
  const uint16_t* Qp = Q + q_base;
  // rows past Nk read as zero (and are masked below)
  const __amdgpu_buffer_rsrc_t rK = make_rsrc(K + kv_off, (uint32_t)Nk * SKVB);
  const __amdgpu_buffer_rsrc_t rV = make_rsrc(V + kv_off, (uint32_t)Nk * SKVB);

  const int qrow_c = qrow < Nq ? qrow : Nq - 1;

  // Q fragments (B operand of S^T = K Q^T): k-step ks covers head dims
  // 16*ks + 8*hf .. +8.
  u32x4 qf[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks)
    qf[ks] = ldg<u32x4>(Qp + (size_t)qrow_c * SQ + ks * 16 + hf * 8);

  int kv_end = CAUSAL ? min(Nk, q0 + BR) : Nk;
  int jf = 0;  // first key tile visited
  if constexpr (WIN) {
    if (win_r >= 0) kv_end = min(kv_end, q0 + BR + win_r);
    if (win_l >= 0) jf = max(0, q0 - win_l) / BC;
  }
  int ntiles = (kv_end + BC - 1) / BC - jf;
  // The sparse list of this query tile, one entry per lane and register
  // (list position p in register p/64, lane p%64), read back with readlane.
  int spc[4] = {0, 0, 0, 0};
  if constexpr (SPARSE) {
    const int lo = sp_ptr[qt];
    ntiles = min(max(sp_ptr[qt + 1] - lo, 0), 256);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (r * 64 + lane < ntiles) spc[r] = sp_idx[lo + r * 64 + lane];
    if (ntiles == 0) {  // nothing visible: O = 0, LSE = -inf
      if (qrow < Nq) {
        uint16_t* Op = O + q_base + (size_t)qrow * SQ;
#pragma unroll
        for (int db = 0; db < DBLK; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) stg<u32x2>(Op + db * 32 + g * 8 + hf * 4, u32x2{0u, 0u});
        if (hf == 0) LSE[lse_base + qrow] = -INFINITY;
      }
      return;
    }
  }
  // Key tile (of BC keys) visited at loop position j.
  auto tile_of = [&](int j) -> int {
    if constexpr (SPARSE) {
      const int v = j < 64 ? spc[0] : j < 128 ? spc[1] : j < 192 ? spc[2] : spc[3];
      return __builtin_amdgcn_readlane(v, j & 63);
    } else {
      return jf + j;
    }
  };

  // Per-lane source offsets of this wave's direct loads (same for every tile):
  // LDS block (wave*LPW + i) of a tile holds rows r, lane -> position p.
  int koff[LPW], voff[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int r = (wave * LPW + i) * RPL + lane / NCH;
    const int p = lane % NCH;
    koff[i] = r * SKVB + ((p ^ fwd_swz_k<D>(r)) << 4);
    voff[i] = r * SKVB + ((p ^ fwd_swz_v<D>(r)) << 4);
  }
  auto issue_k = [&](int j, int slot) {
    char* d = kslot(slot) + wave * LPW * 1024;
#pragma unroll
    for (int i = 0; i < LPW; ++i)
      buffer_load_lds16(rK, d + i * 1024, koff[i], tile_of(j) * BC * SKVB);
  };
  auto issue_v = [&](int j, int slot) {
    char* d = vslot(slot) + wave * LPW * 1024;
#pragma unroll
    for (int i = 0; i < LPW; ++i)
      buffer_load_lds16(rV, d + i * 1024, voff[i], tile_of(j) * BC * SKVB);
  };

  // Per-lane LDS read offsets.  K (A operand, row kb*32 + l32, chunk 2*kk + hf):
  int krd[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk)
    krd[kk] = l32 * ROWB + (((2 * kk + hf) ^ fwd_swz_k<D>(l32)) << 4);
  // V^T via ds_read_b64_tr_b16.  In each 16-lane group g (= lane/16), source
  // lane j addresses key row 4*(g/2) + j/4 (+ 16*st + 32*kb, + 8 for the
  // second read) at head dims dbase + 4*(j%4) with dbase = 32*db + 16*(g%2);
  // the group's output lane i then holds V[row(e)][dbase + i] for e = 0..3.
  const int g16 = lane >> 4;
  const int j16 = lane & 15;
  const int vrow = 4 * (g16 >> 1) + (j16 >> 2);
  const int vsw = fwd_swz_v<D>(vrow);  // rows vrow + 8, +16, ... share it
  int vrd[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) {
    const int c = 4 * db + 2 * (g16 & 1) + ((j16 & 3) >> 1);
    vrd[db] = vrow * ROWB + ((c ^ vsw) << 4) + (j16 & 1) * 8;
  }

  // S^T = K Q^T for one K slot: two 32-key blocks x this wave's 32 queries.
  auto qk = [&](int slot, f32x16* s) {
    const char* ks = kslot(slot);
    s[0] = f32x16{0};
    s[1] = f32x16{0};
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        s[kb] = mfma_32x32x16_bf16(lds_read<u32x4>(ks, kb * 32 * ROWB + krd[kk]), qf[kk], s[kb]);
  };

  f32x16 o[DBLK];
#pragma unroll
  for (int i = 0; i < DBLK; ++i) o[i] = f32x16{0};
  // Reference max M in log2 units (scale*log2e folded in), per query row, and
  // this lane's share of the row sum.  p = exp2(s*c - M) is computed against
  // the current reference without taking each tile's max first; the tile's
  // per-lane sum of p bounds every p it holds, and only when some lane's sum
  // exceeds kLazyLimit (or is inf) is the tile's true max taken, O and l
  // rescaled and the tile's p recomputed.  The final O/l and LSE do not depend
  // on the reference ([L21] slide 12: any common shift cancels).
  constexpr float kLazyLimit = 65536.f;
  float M;
  float l_run = 0.f;

  // Mask one S^T tile: keys past the end (ragged tail) and, on tiles crossing
  // the diagonal, keys after the query ([CH18] §18.5.2).
  auto mask = [&](int j, f32x16* s) {
    const int kv0 = tile_of(j) * BC;
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
  };
  // Row max of a masked tile in log2 units, the same in both lane halves.
  auto tile_max = [&](const f32x16* s) {
    float mt = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kb][r]);
    return max_halves(mt) * scale_log2;
  };

  // Software pipeline, one barrier per tile, two LDS slots each for K and V.
  // Iteration i issues, op by op, the 16 products of S_{i+1} = K_{i+1} Q^T and
  // the 16 products of O^T += V_{i-1}^T P_{i-1}^T (tile i-1's P, kept from the
  // previous iteration), and after each product the fma/exp/sum/convert of one
  // element of tile i's S; every product thus has about four VALU ops beside
  // it, and the matrix pipe never waits for a VALU-only phase.  The loads
  // issued at the start of iteration i fetch K_{i+2} (into the slot K_i left)
  // and V_i (into the slot V_{i-2} left); both have one iteration to arrive.
  // S^T tiles and P fragments alternate by iteration parity.
  static_assert(NS == 2, "stages");
  f32x16 sbuf[2][2];
  u32x4 pbuf[2][2][2];  // [parity][kb][k-step]: P^T B operands
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int st = 0; st < 2; ++st) pbuf[1][kb][st] = u32x4{0, 0, 0, 0};
  // prologue: K_0, K_1; V slot 1 is zeroed so that the first iteration's
  // product with "tile -1" (P = 0) adds exactly zero.
  issue_k(0, 0);
  if (ntiles > 1) issue_k(1, 1);
  {
    char* z = vslot(1);
    for (int off = tid * 16; off < TILE; off += NW * 64 * 16) lds_write<u32x4>(z, off, u32x4{0, 0, 0, 0});
  }
  wait_vmem();
  __syncthreads();
  qk(0, sbuf[0]);
  mask(0, sbuf[0]);
  // Start the reference at tile 0's max (finite without a window: key 0 is
  // visible to every row).  The floor covers rows that see nothing in tile 0
  // (past Nq, or outside a sliding window): their first visible tile then
  // overflows the lazy bound and takes the rescale path, which moves the
  // reference to that tile's max and zeroes the (empty) O and l.
  M = fmaxf(tile_max(sbuf[0]), -1e30f);
  lds_barrier();  // K slot 0 is refilled below

  // Products per tile: NQK of S = K Q^T (h -> kb = h%2, kk = h/2) and NPV of
  // O^T += V^T P^T (h -> kb = h/(2*DBLK), st = (h/DBLK)%2, db = h%DBLK).
  constexpr int NQK = 2 * KSTEPS;
  constexpr int NPV = 4 * DBLK;
  static_assert(NQK == NPV && 32 % (2 * NQK) == 0, "product interleave");
  constexpr int EPG = 32 / (2 * NQK);  // elements of S_i per product (per lane)
  // V^T fragment of PV product h.
  auto vfrag = [&](const char* vs, int h) {
    const char* vp = vs + ((h / (2 * DBLK)) * 32 + ((h / DBLK) & 1) * 16) * ROWB + vrd[h % DBLK];
    const u32x2 a0 = lds_read_tr16(vp);
    const u32x2 a1 = lds_read_tr16(vp + 8 * ROWB);
    return u32x4{a0[0], a0[1], a1[0], a1[1]};
  };
  // K fragment of S product h: kb = h%2, kk = h/2.
  auto kfrag = [&](const char* ks, int h) {
    return lds_read<u32x4>(ks, (h & 1) * 32 * ROWB + krd[h >> 1]);
  };

  // The first AHEAD K and V fragments of a step are read at the end of the
  // step before it (or in the prologue), after that step's barrier: a step
  // starts with its first operands in flight rather than waiting for them.
  constexpr int AHEAD = 2;
  u32x4 kfr[AHEAD], vfr[AHEAD];
#pragma unroll
  for (int h = 0; h < AHEAD; ++h) {
    kfr[h] = kfrag(kslot(1), h);  // K_1
    vfr[h] = vfrag(vslot(1), h);  // zeros ("V_{-1}")
  }
  // One pipeline step; U = i % 2 makes slots and buffers compile-time
  // constants, so the LDS fragment addresses are a per-lane register plus an
  // immediate.
  auto step = [&](int i, auto U) {
    constexpr int u = decltype(U)::value;
    f32x16* s_cur = sbuf[u];
    f32x16* s_nxt = sbuf[u ^ 1];
    u32x4 (*pb_cur)[2] = pbuf[u];
    u32x4 (*pb_prev)[2] = pbuf[u ^ 1];
    const bool more_k = i + 2 < ntiles;
    float lt = 0.f;  // this lane's sum of p over tile i
    {
      const char* ks = kslot(u ^ 1);   // K_{i+1}
      const char* vs = vslot(u ^ 1);   // V_{i-1}
      s_nxt[0] = f32x16{0};
      s_nxt[1] = f32x16{0};
      // This step's loads go out after its first LDS reads (issued at the
      // end of the previous step).
      asm volatile("" ::: "memory");
      if (more_k) issue_k(i + 2, u);
      issue_v(i, u);
      // The elementwise chain of one element (fma -> exp -> sum/convert) is
      // spread over three product groups: group g does the fma of group g+1's
      // elements, the exp of its own and the sum/convert of group g-1's, so no
      // result is consumed by the instruction right after it (an exp result
      // read at once costs a wait state).
      constexpr int NG = 2 * NQK;
      float p[32];
      auto F = [&](int gg) {
#pragma unroll
        for (int e = gg * EPG; e < (gg + 1) * EPG; ++e)
          p[e] = fmaf(s_cur[e >> 4][e & 15], scale_log2, -M);
      };
      auto X = [&](int gg) {
#pragma unroll
        for (int e = gg * EPG; e < (gg + 1) * EPG; ++e) p[e] = fast_exp2(p[e]);
      };
      auto A = [&](int gg) {
#pragma unroll
        for (int e = gg * EPG; e < (gg + 1) * EPG; ++e) {
          lt += p[e];  // fp32 sum of the unrounded p: LSE stays exact to fp32
          if (e & 1) {
            const int r = e & 15;
            pb_cur[e >> 4][r >> 3][(r & 7) >> 1] = pack_bf16(p[e - 1], p[e]);
            // Pinned here: left alone, the compiler sinks the conversions
            // below the rare-rescale branch (they are dead on that path),
            // out of the product interleave.
            settle(pb_cur[e >> 4][r >> 3][(r & 7) >> 1]);
          }
        }
      };
      F(0);
      // After group GB every LDS read of this step has been issued (the last
      // K and V fragments are read AHEAD products before their use): wait for
      // this step's loads (K_{i+2}, V_i) and the other waves there, then read
      // the next step's first fragments while the last products run.
      constexpr int GB = NG - 2 * AHEAD;
      u32x4 kn[AHEAD], vn[AHEAD];
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const int h = g >> 1;
        if (g == GB) {
          wait_vmem();
          lds_barrier();
#pragma unroll
          for (int hh = 0; hh < AHEAD; ++hh) {
            kn[hh] = kfrag(kslot(u), hh);
            vn[hh] = vfrag(vslot(u), hh);
          }
        }
        if ((g & 1) == 0) {
          s_nxt[h & 1] = mfma_32x32x16_bf16(kfr[h % AHEAD], qf[h >> 1], s_nxt[h & 1]);
          if (h + AHEAD < NQK) kfr[h % AHEAD] = kfrag(ks, h + AHEAD);
        } else {
          o[h % DBLK] = mfma_32x32x16_bf16(vfr[h % AHEAD],
                                           pb_prev[h / (2 * DBLK)][(h / DBLK) & 1], o[h % DBLK]);
          if (h + AHEAD < NPV) vfr[h % AHEAD] = vfrag(vs, h + AHEAD);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (g + 1 < NG) F(g + 1);
        X(g);
        if (g > 0) A(g - 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      A(NG - 1);
#pragma unroll
      for (int hh = 0; hh < AHEAD; ++hh) {
        kfr[hh] = kn[hh];
        vfr[hh] = vn[hh];
      }
    }
    // Rare: the reference is too low for tile i.  Move it to the tile's max,
    // rescale O (which now holds tiles up to i-1) and l, and redo tile i's p.
    if (__builtin_amdgcn_ballot_w64(lt > kLazyLimit)) {
      const float Mn = fmaxf(M, tile_max(s_cur));
      const float alpha = fast_exp2(M - Mn);
      M = Mn;
      l_run *= alpha;
#pragma unroll
      for (int d4 = 0; d4 < DBLK; ++d4) o[d4] *= alpha;
      lt = 0.f;
#pragma unroll
      for (int e = 0; e < 32; e += 2) {
        const float p0 = fast_exp2(fmaf(s_cur[e >> 4][e & 15], scale_log2, -M));
        const float p1 = fast_exp2(fmaf(s_cur[e >> 4][(e & 15) + 1], scale_log2, -M));
        lt += p0 + p1;
        const int r = e & 15;
        pb_cur[e >> 4][r >> 3][(r & 7) >> 1] = pack_bf16(p0, p1);
      }
    }
    l_run += lt;
    if (i + 1 < ntiles) mask(i + 1, s_nxt);
  };
  for (int i0 = 0; i0 < ntiles; i0 += 2) {
    step(i0, IntConst<0>{});
    if (i0 + 1 < ntiles) step(i0 + 1, IntConst<1>{});
  }
  // The last tile's O^T += V^T P^T.
  auto pv_last = [&](auto U) {
    constexpr int u = decltype(U)::value;
    const char* vs = vslot(u);
#pragma unroll
    for (int h = 0; h < NPV; ++h)
      o[h % DBLK] =
          mfma_32x32x16_bf16(vfrag(vs, h), pbuf[u][h / (2 * DBLK)][(h / DBLK) & 1], o[h % DBLK]);
  };
  if ((ntiles - 1) & 1) pv_last(IntConst<1>{});
  else pv_last(IntConst<0>{});

  // Epilogue: O = O^T / l, LSE = (M + log2 l) ln 2 (a row that saw no key,
  // possible with a block-sparse list: O = 0, LSE = -inf).
  const float l_tot = sum_halves(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qrow < Nq) {
    uint16_t* Op = O + q_base + (size_t)qrow * SQ;
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        int d0 = db * 32 + g * 8 + hf * 4;
        stg<u32x2>(Op + d0, u32x2{pack_bf16(o[db][4 * g] * inv, o[db][4 * g + 1] * inv),
                                  pack_bf16(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv)});
      }
    if (hf == 0) LSE[lse_base + qrow] = l_tot > 0.f ? (M + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// The bf16 forward kernel.  One workgroup per work unit, launched in the
// longest-first order (the dispatcher hands the next unit to the next free
// compute unit), or, PERSIST, a persistent grid of one workgroup per compute
// unit that walks the same list in snake order (persistent_position).  Unit
// results do not depend on which workgroup computes them.
template <int D, bool CAUSAL, int NW, int NS, bool VARLEN = false, bool WIN = false,
          bool SPARSE = false, bool PERSIST = false>
__global__ __launch_bounds__(NW * 64, 8 / NW) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE,
    int Hq, int Hkv, int Nq_arg, int Nk_arg, float scale, float scale_log2, int BH, int nqt,
    const int* __restrict__ cu_q = nullptr, const int* __restrict__ cu_k = nullptr,
    int total_q = 0, int win_l = -1, int win_r = -1, const int* __restrict__ sp_ptr = nullptr,
    const int* __restrict__ sp_idx = nullptr) {
  if constexpr (PERSIST) {
    const int n = BH * nqt;
    for (int i = 0;; ++i) {
      const int p = persistent_position(i, blockIdx.x, gridDim.x);
      if (p >= n) break;
      fwd_bf16_unit<D, CAUSAL, NW, NS, VARLEN, WIN, SPARSE>(Q, K, V, O, LSE, Hq, Hkv, Nq_arg,
                                                            Nk_arg, scale, scale_log2, BH, nqt,
                                                            cu_q, cu_k, total_q, win_l, win_r,
                                                            sp_ptr, sp_idx, p);
      __syncthreads();  // every wave is done with the LDS slots before the next unit
    }
  } else {
    fwd_bf16_unit<D, CAUSAL, NW, NS, VARLEN, WIN, SPARSE>(Q, K, V, O, LSE, Hq, Hkv, Nq_arg,
                                                          Nk_arg, scale, scale_log2, BH, nqt,
                                                          cu_q, cu_k, total_q, win_l, win_r,
                                                          sp_ptr, sp_idx, blockIdx.x);
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
                           bool causal, hipStream_t stream, int win_l, int win_r) {
  constexpr int NW = kFwdWaves, NS = kFwdStages;
  const int BH = B * Hq;
  const int nqt = (Nq + kFwdBr - 1) / kFwdBr;
  dim3 grid(BH * nqt), block(NW * 64);
  const float sl2 = scale * kLog2e;
  auto Qp = (const uint16_t*)q;
  auto Kp = (const uint16_t*)k;
  auto Vp = (const uint16_t*)v;
  auto Op = (uint16_t*)o;
#define FA_LAUNCH_FWD(DD, CC, WW)                                                               \
  hipLaunchKernelGGL((fwd_bf16_kernel<DD, CC, NW, NS, false, WW>), grid, block, 0, stream, Qp, \
                     Kp, Vp, Op, lse, Hq, Hkv, Nq, Nk, scale, sl2, BH, nqt, nullptr, nullptr, 0, \
                     win_l, win_r)
  // Causal units have unequal costs: a persistent grid (one workgroup per
  // compute unit) walks the longest-first list, which hides each unit's
  // start-up behind the previous one's (measured 1.3% faster than one
  // workgroup per unit at B2 H16 N8192 d128; equal-cost non-causal units
  // gain nothing and keep one workgroup each).
#define FA_LAUNCH_FWD_PERSIST(DD)                                                              \
  hipLaunchKernelGGL((fwd_bf16_kernel<DD, true, NW, NS, false, false, false, true>),          \
                     dim3(persistent_grid(BH * nqt)), block, 0, stream, Qp, Kp, Vp, Op, lse, Hq, \
                     Hkv, Nq, Nk, scale, sl2, BH, nqt)
  const bool win = win_l >= 0 || win_r >= 0;
  if (d == 128) {
    if (win) {
      if (causal) FA_LAUNCH_FWD(128, true, true);
      else FA_LAUNCH_FWD(128, false, true);
    } else {
      if (causal) FA_LAUNCH_FWD_PERSIST(128);
      else FA_LAUNCH_FWD(128, false, false);
    }
  } else {
    if (win) {
      if (causal) FA_LAUNCH_FWD(64, true, true);
      else FA_LAUNCH_FWD(64, false, true);
    } else {
      if (causal) FA_LAUNCH_FWD_PERSIST(64);
      else FA_LAUNCH_FWD(64, false, false);
    }
  }
#undef FA_LAUNCH_FWD
#undef FA_LAUNCH_FWD_PERSIST
  return hipGetLastError();
}

hipError_t launch_fwd_bf16_sparse(const void* q, const void* k, const void* v, void* o,
                                  float* lse, const int* sp_ptr, const int* sp_idx, int B,
                                  int Hq, int Hkv, int Nq, int Nk, int d, float scale, bool causal,
                                  hipStream_t stream) {
  constexpr int NW = kFwdWaves, NS = kFwdStages;
  const int BH = B * Hq;
  const int nqt = (Nq + kFwdBr - 1) / kFwdBr;
  dim3 grid(BH * nqt), block(NW * 64);
  const float sl2 = scale * kLog2e;
  auto Qp = (const uint16_t*)q;
  auto Kp = (const uint16_t*)k;
  auto Vp = (const uint16_t*)v;
  auto Op = (uint16_t*)o;
#define FA_LAUNCH_SPARSE(DD, CC)                                                                \
  hipLaunchKernelGGL((fwd_bf16_kernel<DD, CC, NW, NS, false, false, true>), grid, block, 0,     \
                     stream, Qp, Kp, Vp, Op, lse, Hq, Hkv, Nq, Nk, scale, sl2, BH, nqt, nullptr, \
                     nullptr, 0, -1, -1, sp_ptr, sp_idx)
  if (d == 128) {
    if (causal) FA_LAUNCH_SPARSE(128, true);
    else FA_LAUNCH_SPARSE(128, false);
  } else {
    if (causal) FA_LAUNCH_SPARSE(64, true);
    else FA_LAUNCH_SPARSE(64, false);
  }
#undef FA_LAUNCH_SPARSE
  return hipGetLastError();
}

hipError_t launch_fwd_bf16_varlen(const void* q, const void* k, const void* v, void* o,
                                  float* lse, const int* cu_q, const int* cu_k, int batch,
                                  int Hq, int Hkv, int total_q, int max_seqlen_q, int d,
                                  float scale, bool causal, hipStream_t stream) {
  constexpr int NW = kFwdWaves, NS = kFwdStages;
  const int BH = batch * Hq;
  const int nqt = (max_seqlen_q + kFwdBr - 1) / kFwdBr;
  dim3 grid(BH * nqt), block(NW * 64);
  const float sl2 = scale * kLog2e;
  auto Qp = (const uint16_t*)q;
  auto Kp = (const uint16_t*)k;
  auto Vp = (const uint16_t*)v;
  auto Op = (uint16_t*)o;
#define FA_LAUNCH_VARLEN(DD, CC)                                                              \
  hipLaunchKernelGGL((fwd_bf16_kernel<DD, CC, NW, NS, true>), grid, block, 0, stream, Qp, Kp, \
                     Vp, Op, lse, Hq, Hkv, 0, 0, scale, sl2, BH, nqt, cu_q, cu_k, total_q)
  if (d == 128) {
    if (causal) FA_LAUNCH_VARLEN(128, true);
    else FA_LAUNCH_VARLEN(128, false);
  } else {
    if (causal) FA_LAUNCH_VARLEN(64, true);
    else FA_LAUNCH_VARLEN(64, false);
  }
#undef FA_LAUNCH_VARLEN
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

int persistent_schedule(int n_units, int grid, int* worker_out, int capacity) {
  if (n_units < 0 || grid <= 0 || (worker_out && capacity < n_units)) return -1;
  if (worker_out) {
    for (int w = 0; w < grid; ++w)
      for (int i = 0;; ++i) {
        const int p = persistent_position(i, w, grid);
        if (p >= n_units) break;
        worker_out[p] = w;
      }
  }
  return n_units;
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
      query_tile_of(t, BH, nqt, causal, &bh, &qt);
      if (bh_out) bh_out[t] = bh;
      if (qt_out) qt_out[t] = qt;
      if (cost_out) cost_out[t] = fwd_kv_tiles(qt, Nk, causal, kFwdBr, kFwdBc);
    }
  }
  return n;
}

}  // namespace fa

// Split-KV decode and its combine step for gfx950.
//
// Method: [CH18] "第 18 章 FlashAttention" §18.8.2 (Flash-Decoding: cut the KV
// length into chunks handled in parallel, then merge the partial softmax
// statistics with the online-softmax formula) and [L21] "CMU 11-868 L21
// FlashAttention" slides 57-60 (GQA packing: the query heads that share one KV
// head fill the rows of one tile, so K and V are streamed once per group).
//
// Split kernel, one workgroup (4 waves) per (b, KV head, chunk):
//   * the G = Hq/Hkv query heads of the group, times the Nq query tokens, are
//     the n axis of S^T = K Q^T on the 32x32x16 MFMA (column n = g*Nq + t; n =
//     32 >= G*Nq; the columns past it hold zero queries).
//   * each wave streams 32-key blocks of the chunk (blocks w, w+4, ...)
//     through one K and one V slot of its own in LDS: direct global-to-LDS
//     loads, each instruction moving 1 KB of consecutive rows, marked
//     non-temporal (every key row is read once); K fragments are b128 reads,
//     V^T fragments transposing reads (ds_read_b64_tr_b16), both from
//     chunk-swizzled rows.
//   * the next block's K is loaded as soon as the current block's K reads
//     are done (after S), its V after the current PV products; the wave waits
//     for both at the top of the next iteration.
//   * the 4 waves' (max, sum, O) are merged in LDS and the chunk's normalised
//     output and logsumexp are written.
// The work is bound by HBM reads of K and V (about 4 FLOP per byte); MFMA
// waste on the padded n axis costs nothing that matters.

#include <atomic>
#include <mutex>

#include "fa_device.h"
#include "fa_launch.h"

// Scratch for the no-allocation decode (fa_decode_splitkv_noalloc): the split
// partials of one call, o_part then lse_part at the next 256-byte boundary.
// Each GPU the library runs on holds its own copy until the process ends.  In
// host code the name is only a stand-in for the symbol: its device address is
// looked up once per device (fa::noalloc_scratch) and only that address is
// passed to kernels.
static __device__ __align__(256) unsigned char scratch[fa::kNoAllocScratchBytes];

namespace fa {

namespace {
// Cache-policy bits of the K/V loads: nt (non-temporal).
constexpr int kStreamPolicy = 2;
// Chunk swizzles of the K and V block rows (the forward's tile swizzles):
// K rows l32 = 0..15 read one chunk each, V rows 4i..4i+3 read four
// consecutive chunks each, without bank conflicts.
template <int D>
__device__ __forceinline__ int dec_swz_k(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int dec_swz_v(int r) {
  return D == 128 ? (4 * (r & 3)) : (4 * ((r >> 1) & 1));
}
typedef __attribute__((address_space(1))) void glb_void_t;
// One wave copies 64 x 16 bytes from global memory to LDS: lane i reads 16
// bytes at its own address `src` and writes LDS bytes [lds + 16*i, +16);
// `lds` must be wave-uniform.  Non-temporal: streamed data.
__device__ __forceinline__ void global_load_lds16_stream(const uint16_t* src, char* lds) {
  __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)lds, 16, 0, kStreamPolicy);
}
// Waits for this wave's outstanding LDS reads.
__device__ __forceinline__ void wait_lds_reads() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
}  // namespace

namespace {
constexpr int kDecWaves = 4;
constexpr int kDecBlk = 32;  // keys per wave iteration
}  // namespace

// PAGED: K and V are paged caches [num_pages][page_size][Hkv][D] and batch
// entry b's logical key t sits in page table[b][t / page_size] at row
// t % page_size ([CH18] §18.8.2 (3), §18.8.3 (1)); its length is seqlens[b]
// and chunk c covers logical keys [c*L, (c+1)*L) of it (possibly none).  The
// dense layout is [B][Hkv][Nk][D] with L = Nk / num_splits.
template <int D, bool PAGED>
__global__ __launch_bounds__(256, 2) void decode_split_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, float* __restrict__ o_part, float* __restrict__ lse_part,
    int Hq, int Hkv, int Nk, int num_splits, float scale, float scale_log2,
    const int* __restrict__ table, const int* __restrict__ seqlens, int page_shift,
    int max_pages, int num_pages, int chunk, int Nq = 1, int causal = 0) {
  constexpr int KS = D / 16;          // k-steps over the head dim
  constexpr int DBLK = D / 32;
  constexpr int ROWB = D * 2;         // bytes per key row
  constexpr int NCH = ROWB / 16;      // 16-byte chunks per row
  constexpr int RPL = 64 / NCH;       // rows per 1 KB direct load
  constexpr int LPB = kDecBlk / RPL;  // direct loads per 32-row block
  constexpr int SLOT = kDecBlk * ROWB;
  // Per wave: one K and one V slot of a 32-key block (row-major, swizzled).
  // After the loop the same bytes hold the merge buffer red_o[32][D + 1].
  __shared__ __attribute__((aligned(1024))) char slots[kDecWaves][2][SLOT];
  __shared__ float red_m[kDecWaves][32];
  __shared__ float red_l[kDecWaves][32];
  static_assert(32 * (D + 1) * 4 <= (int)sizeof(slots), "merge buffer fits in the slots");
  float (*red_o)[D + 1] = reinterpret_cast<float (*)[D + 1]>(&slots[0][0][0]);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hf = lane >> 5;
  const int G = Hq / Hkv;
  // Columns of the n axis in use: the G heads of the group times the Nq query
  // tokens, column n = g * Nq + t (<= 32, checked on the host).
  const int NC = G * Nq;

  const int c = blockIdx.x % num_splits;
  const int bhk = blockIdx.x / num_splits;
  const int b = bhk / Hkv;
  const int hk = bhk - b * Hkv;
  const int L = PAGED ? chunk : Nk / num_splits;
  const int key_begin = c * L;
  // (paged: the length is clamped to what the table can address and page ids
  // to the cache, so bad table data reads wrong rows but never out of bounds)
  // this entry's key count and the end of this chunk's keys
  const int kv_len = PAGED ? min(seqlens[b], max_pages << page_shift) : Nk;
  const int key_end = PAGED ? min(key_begin + L, kv_len) : key_begin + L;

  const uint16_t* Kp = PAGED ? K : K + (size_t)bhk * Nk * D;
  const uint16_t* Vp = PAGED ? V : V + (size_t)bhk * Nk * D;
  const int* trow = PAGED ? table + (size_t)b * max_pages : nullptr;
  // Element offset of key row `key` of this KV head.  Paged: a 32-key block
  // starting at k0 (a multiple of 32; pages are at least 16 keys) touches at
  // most the pages of k0 and k0 + 31, looked up once per block (pg0, pg1).
  auto row_off = [&](int key, int k0, int pg0, int pg1) -> size_t {
    if constexpr (PAGED) {
      const int pg = (key >> page_shift) == (k0 >> page_shift) ? pg0 : pg1;
      const int slot = (pg << page_shift) | (key & ((1 << page_shift) - 1));
      return ((size_t)slot * Hkv + hk) * D;
    } else {
      (void)k0; (void)pg0; (void)pg1;
      return (size_t)key * D;
    }
  };
  char* kslot = slots[wave][0];
  char* vslot = slots[wave][1];

  // Q^T B operand: column n = l32 is query head hk*G + l32 (zero past G).
  // k-step ks, element i of lane half hf is head dim 16*ks + 8*hf + i.
  u32x4 qf[KS];
  {
    const bool valid = l32 < NC;
    const uint16_t* qp = Q + (((size_t)b * Hq + hk * G) * Nq + (valid ? l32 : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 x = ldg<u32x4>(qp + ks * 16 + hf * 8);
      qf[ks] = valid ? x : u32x4{0, 0, 0, 0};
    }
  }

  const int nblk = key_end > key_begin ? (key_end - key_begin + kDecBlk - 1) / kDecBlk : 0;
  // Direct loads of one 32-key block (K or V) into this wave's slot: load i
  // moves rows RPL*i .. RPL*i + RPL-1, lane -> row RPL*i + lane/NCH, LDS
  // chunk position lane%NCH holding source chunk (lane%NCH) ^ swz(row).  Rows
  // past the chunk's keys repeat its last key (their scores are masked), and
  // the loads are non-temporal: every key row is read by this workgroup only.
  // Paged: the block's two page ids (looked up once per block, ahead of its
  // loads, so that the table reads are not waited for at the load).
  auto block_pages = [&](int blk, int* pg0, int* pg1) {
    *pg0 = 0;
    *pg1 = 0;
    if constexpr (PAGED) {
      const int k0 = key_begin + blk * kDecBlk;
      *pg0 = min(max(trow[k0 >> page_shift], 0), num_pages - 1);
      *pg1 = min(max(trow[(min(k0 + kDecBlk, key_end) - 1) >> page_shift], 0), num_pages - 1);
    }
  };
  auto issue_blk = [&](char* dst, const uint16_t* base, int blk, bool is_v, int pg0, int pg1) {
    const int k0 = key_begin + blk * kDecBlk;
#pragma unroll
    for (int i = 0; i < LPB; ++i) {
      const int r = RPL * i + lane / NCH;
      const int pos = lane % NCH;
      int key = k0 + r;
      key = key < key_end ? key : key_end - 1;
      const int src = pos ^ (is_v ? dec_swz_v<D>(r) : dec_swz_k<D>(r));
      global_load_lds16_stream(base + row_off(key, k0, pg0, pg1) + src * 8, dst + i * 1024);
    }
  };
  // K A operand of k-step ks: row l32, head dims 16*ks + 8*hf .. +8 (chunk
  // 2*ks + hf).
  int krd[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) krd[ks] = l32 * ROWB + (((2 * ks + hf) ^ dec_swz_k<D>(l32)) << 4);
  // V^T A operand (head-dim block db, keys 16*st ..): two ds_read_b64_tr_b16.
  // In each 16-lane group g (= lane/16), source lane j addresses key row
  // 4*(g/2) + j/4 (+ 16*st, + 8 for the second read) at head dims
  // 32*db + 16*(g%2) + 4*(j%4); output lane i of the group then holds head
  // dim 32*db + 16*(g%2) + i of those four keys, which is the key order of the
  // P^T B operand below.
  const int g16 = lane >> 4;
  const int j16 = lane & 15;
  const int vrow = 4 * (g16 >> 1) + (j16 >> 2);
  const int vsw = dec_swz_v<D>(vrow);  // rows vrow + 8, +16, +24 share it
  int vrd[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) {
    const int c = 4 * db + 2 * (g16 & 1) + ((j16 & 3) >> 1);
    vrd[db] = vrow * ROWB + ((c ^ vsw) << 4) + (j16 & 1) * 8;
  }

  f32x16 o[DBLK];
#pragma unroll
  for (int i = 0; i < DBLK; ++i) o[i] = f32x16{0};
  float m_run = -INFINITY, l_run = 0.f;

  int blk = wave;
  if (blk < nblk) {
    int pg0, pg1;
    block_pages(blk, &pg0, &pg1);
    issue_blk(kslot, Kp, blk, false, pg0, pg1);
    issue_blk(vslot, Vp, blk, true, pg0, pg1);
  }
  for (; blk < nblk; blk += kDecWaves) {
    const bool more = blk + kDecWaves < nblk;
    int npg0 = 0, npg1 = 0;  // the next block's pages
    if (more) block_pages(blk + kDecWaves, &npg0, &npg1);
    wait_vmem();  // this block's K and V are in the slots
    f32x16 s = f32x16{0};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) s = mfma_32x32x16_bf16(lds_read<u32x4>(kslot, krd[ks]), qf[ks], s);
    // the K slot is free once this wave's reads of it are done
    wait_lds_reads();
    if (more) issue_blk(kslot, Kp, blk + kDecWaves, false, npg0, npg1);

    const int k0 = key_begin + blk * kDecBlk;

    if (k0 + kDecBlk > key_end) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (k0 + 8 * (r >> 2) + 4 * hf + (r & 3) >= key_end) s[r] = -INFINITY;
    }
    // Several query tokens, causal: they are the newest Nq positions, so token
    // t sees keys up to kv_len - Nq + t (a mask aligned to the end of the keys).
    if (causal && k0 + kDecBlk - 1 > kv_len - Nq) {
      const int lim = kv_len - Nq + l32 % Nq;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (k0 + 8 * (r >> 2) + 4 * hf + (r & 3) > lim) s[r] = -INFINITY;
    }
    float mt = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mt = fmaxf(mt, s[r]);
    mt = fmaxf(mt, xor32(mt));
    const float m_new = fmaxf(m_run, mt);
    const float m_ref = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2((m_run - m_ref) * scale_log2);
    const float mb = m_ref * scale_log2;
    m_run = m_new;
    float p[16], psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = fast_exp2(fmaf(s[r], scale_log2, -mb));
      psum += p[r];
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int i = 0; i < DBLK; ++i) o[i] *= alpha;
    u32x4 pb[2];
#pragma unroll
    for (int st = 0; st < 2; ++st)
      pb[st] = u32x4{pack_bf16(p[8 * st + 0], p[8 * st + 1]), pack_bf16(p[8 * st + 2], p[8 * st + 3]),
                     pack_bf16(p[8 * st + 4], p[8 * st + 5]), pack_bf16(p[8 * st + 6], p[8 * st + 7])};

#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const char* vp = vslot + st * 16 * ROWB + vrd[db];
        const u32x2 a0 = lds_read_tr16(vp);
        const u32x2 a1 = lds_read_tr16(vp + 8 * ROWB);
        o[db] = mfma_32x32x16_bf16(u32x4{a0[0], a0[1], a1[0], a1[1]}, pb[st], o[db]);
      }
    wait_lds_reads();
    if (more) issue_blk(vslot, Vp, blk + kDecWaves, true, npg0, npg1);
  }

  // Merge the four waves.  Lane (l32, hf) holds head column l32 and head dims
  // 32*db + 8*(r/4) + 4*hf + r%4.  (red_o reuses the slots: every wave has
  // waited for its last loads and passes the barrier below before any write.)  Each wave rescales its partial output to
  // the merged max and sum, then the waves add into one LDS buffer in a fixed
  // order (deterministic).
  const float l_tot = l_run + xor32(l_run);
  if (l32 < NC && hf == 0) {
    red_m[wave][l32] = m_run;
    red_l[wave][l32] = l_tot;
  }
  __syncthreads();
  float M = -INFINITY;
  float Lsum = 0.f;
  if (l32 < NC) {
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, red_m[w][l32]);
    const float Mr = M == -INFINITY ? 0.f : M;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w)
      Lsum += red_l[w][l32] * fast_exp2((red_m[w][l32] - Mr) * scale_log2);
    // (a chunk with no keys -- possible when paged -- gives O = 0, lse = -inf)
    const float f = Lsum > 0.f ? fast_exp2((m_run - Mr) * scale_log2) / Lsum : 0.f;
#pragma unroll
    for (int db = 0; db < DBLK; ++db) o[db] *= f;
  }
#pragma unroll
  for (int w = 0; w < kDecWaves; ++w) {
    if (wave == w && l32 < NC) {
#pragma unroll
      for (int db = 0; db < DBLK; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float* dst = &red_o[l32][db * 32 + 8 * (r >> 2) + 4 * hf + (r & 3)];
          *dst = (w == 0) ? o[db][r] : *dst + o[db][r];
        }
    }
    __syncthreads();
  }
  // rows of the partials: ((b*Hq + h) * Nq + t) * num_splits + c, and the
  // group's rows are consecutive: (b*Hq + hk*G) * Nq + n
  for (int idx = tid; idx < NC * D; idx += 256) {
    const int n = idx / D, dd = idx - (idx / D) * D;
    const size_t row = (((size_t)b * Hq + hk * G) * Nq + n) * num_splits + c;
    o_part[row * D + dd] = red_o[n][dd];
  }
  if (wave == 0 && hf == 0 && l32 < NC) {
    const size_t row = (((size_t)b * Hq + hk * G) * Nq + l32) * num_splits + c;
    lse_part[row] = Lsum > 0.f ? M * scale + __logf(Lsum) : -INFINITY;
  }
}

// Combine of the split partials ([CH18] §18.8.2 (2), reduction step).
template <int VW>
__global__ __launch_bounds__(256) void decode_combine_kernel(const float* __restrict__ o_part,
                                                             const float* __restrict__ lse_part,
                                                             uint16_t* __restrict__ O,
                                                             float* __restrict__ LSE, int d,
                                                             int S) {
  // One workgroup per (b, hq) row.  lse = M + ln sum_c exp(lse_c - M) over the
  // whole workgroup; then thread t sums VW consecutive output elements
  // (vector j = t % NV) over the splits c = g, g + G, ... (g = t / NV), and
  // the G partial sums meet in LDS.  Reads of o_part are VW*4-byte vectors,
  // consecutive across the threads of a group.
  __shared__ float red[1024];
  __shared__ float wred[4];
  const int row = blockIdx.x;  // b*Hq + hq
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const float* lp = lse_part + (size_t)row * S;

  float m = -INFINITY;
  for (int c = t; c < S; c += 256) m = fmaxf(m, lp[c]);
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) m = fmaxf(m, __shfl_xor(m, k, 64));
  if (lane == 0) wred[wave] = m;
  __syncthreads();
  const float M = fmaxf(fmaxf(wred[0], wred[1]), fmaxf(wred[2], wred[3]));
  const float Mr = M == -INFINITY ? 0.f : M;
  __syncthreads();
  float z = 0.f;
  for (int c = t; c < S; c += 256) z += __expf(lp[c] - Mr);
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) z += __shfl_xor(z, k, 64);
  if (lane == 0) wred[wave] = z;
  __syncthreads();
  const float lse = Mr + __logf(wred[0] + wred[1] + wred[2] + wred[3]);

  const int NV = d / VW;          // vectors per output row (<= 256)
  const int G = 256 / NV;         // split groups
  const int j = t % NV, g = t / NV;
  float acc[VW];
#pragma unroll
  for (int e = 0; e < VW; ++e) acc[e] = 0.f;
  if (g < G) {
    const float* op = o_part + (size_t)row * S * d + j * VW;
#pragma unroll 4
    for (int c = g; c < S; c += G) {
      // a row no split saw (every lse_c = -inf, so lse = -inf) gets O = 0
      const float w = lse == -INFINITY ? 0.f : __expf(lp[c] - lse);
      if constexpr (VW == 4) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(op + (size_t)c * d);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = fmaf(w, v[e], acc[e]);
      } else {
        acc[0] = fmaf(w, op[(size_t)c * d], acc[0]);
      }
    }
#pragma unroll
    for (int e = 0; e < VW; ++e) red[g * d + j * VW + e] = acc[e];
  }
  __syncthreads();
  for (int dd = t; dd < d; dd += 256) {
    float sum = 0.f;
    for (int gg = 0; gg < G; ++gg) sum += red[gg * d + dd];
    O[(size_t)row * d + dd] = (uint16_t)(pack_bf16(sum, 0.f) & 0xffff);
  }
  if (t == 0) LSE[row] = lse;
}

hipError_t launch_decode_split(const void* q, const void* k, const void* v, float* o_part,
                               float* lse_part, int B, int Hq, int Hkv, int Nk, int d,
                               float scale, int num_splits, hipStream_t stream, int Nq,
                               bool causal) {
  dim3 grid(B * Hkv * num_splits), block(256);
  const float sl2 = scale * kLog2e;
  if (d == 128)
    hipLaunchKernelGGL((decode_split_kernel<128, false>), grid, block, 0, stream,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, o_part,
                       lse_part, Hq, Hkv, Nk, num_splits, scale, sl2, nullptr, nullptr, 0, 0, 0, 0,
                       Nq, causal ? 1 : 0);
  else
    hipLaunchKernelGGL((decode_split_kernel<64, false>), grid, block, 0, stream,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, o_part,
                       lse_part, Hq, Hkv, Nk, num_splits, scale, sl2, nullptr, nullptr, 0, 0, 0, 0,
                       Nq, causal ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_decode_split_paged(const void* q, const void* k_cache, const void* v_cache,
                                     const int* block_table, const int* seqlens, float* o_part,
                                     float* lse_part, int B, int Hq, int Hkv, int page_shift,
                                     int max_pages, int num_pages, int chunk, int d, float scale,
                                     int num_splits, hipStream_t stream, int Nq, bool causal) {
  dim3 grid(B * Hkv * num_splits), block(256);
  const float sl2 = scale * kLog2e;
  if (d == 128)
    hipLaunchKernelGGL((decode_split_kernel<128, true>), grid, block, 0, stream,
                       (const uint16_t*)q, (const uint16_t*)k_cache, (const uint16_t*)v_cache,
                       o_part, lse_part, Hq, Hkv, 0, num_splits, scale, sl2, block_table,
                       seqlens, page_shift, max_pages, num_pages, chunk, Nq, causal ? 1 : 0);
  else
    hipLaunchKernelGGL((decode_split_kernel<64, true>), grid, block, 0, stream,
                       (const uint16_t*)q, (const uint16_t*)k_cache, (const uint16_t*)v_cache,
                       o_part, lse_part, Hq, Hkv, 0, num_splits, scale, sl2, block_table,
                       seqlens, page_shift, max_pages, num_pages, chunk, Nq, causal ? 1 : 0);
  return hipGetLastError();
}

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_lock;
}  // namespace

hipError_t noalloc_scratch(void** addr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> guard(g_scratch_lock);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      // with this device current: the address of its own copy of the array
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *addr = p;
  return hipSuccess;
}

hipError_t launch_decode_noalloc(const void* q, const void* k, const void* v, void* o,
                                 float* lse, int B, int Hq, int Hkv, int Nk, int d, float scale,
                                 int num_splits, hipStream_t stream) {
  void* base = nullptr;
  hipError_t e = noalloc_scratch(&base);
  if (e != hipSuccess) return e;
  // same layout as a caller's workspace of fa_decode_workspace_size bytes
  const size_t rows = (size_t)B * Hq * num_splits;
  const size_t o_bytes = (rows * d * sizeof(float) + 255) & ~size_t(255);
  float* o_part = static_cast<float*>(base);
  float* lse_part = reinterpret_cast<float*>(static_cast<char*>(base) + o_bytes);
  e = launch_decode_split(q, k, v, o_part, lse_part, B, Hq, Hkv, Nk, d, scale, num_splits,
                          stream);
  if (e != hipSuccess) return e;
  return launch_decode_combine(o_part, lse_part, o, lse, B, Hq, d, num_splits, stream);
}

hipError_t launch_decode_combine(const float* o_part, const float* lse_part, void* o,
                                 float* lse, int B, int Hq, int d, int num_splits,
                                 hipStream_t stream) {
  // (d <= 256 is checked by the caller; G * d <= 1024 floats of LDS)
  if (d % 4 == 0)
    hipLaunchKernelGGL(decode_combine_kernel<4>, dim3(B * Hq), dim3(256), 0, stream, o_part,
                       lse_part, (uint16_t*)o, lse, d, num_splits);
  else
    hipLaunchKernelGGL(decode_combine_kernel<1>, dim3(B * Hq), dim3(256), 0, stream, o_part,
                       lse_part, (uint16_t*)o, lse, d, num_splits);
  return hipGetLastError();
}

}  // namespace fa

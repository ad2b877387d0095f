// Host-side launchers of the gfx950 kernels (internal to the library).  Each
// returns the HIP status of its launches; arguments are validated by the C ABI
// layer before any launcher is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

// Workgroups of a persistent grid over `units` work units: one per compute
// unit of the current device (the forward and dQ kernels each hold a whole
// compute unit), never more than there are units.
inline int persistent_grid(int units) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  return units < cus ? units : cus;
}

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                           bool causal, hipStream_t stream, int win_l = -1, int win_r = -1);
hipError_t launch_fwd_bf16_sparse(const void* q, const void* k, const void* v, void* o,
                                  float* lse, const int* sp_ptr, const int* sp_idx, int B,
                                  int Hq, int Hkv, int Nq, int Nk, int d, float scale, bool causal,
                                  hipStream_t stream);
hipError_t launch_fwd_bf16_varlen(const void* q, const void* k, const void* v, void* o,
                                  float* lse, const int* cu_q, const int* cu_k, int batch,
                                  int Hq, int Hkv, int total_q, int max_seqlen_q, int d,
                                  float scale, bool causal, hipStream_t stream);
hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          int B, int Hq, int Hkv, int Nq, int Nk, float scale, bool causal,
                          hipStream_t stream);
int fwd_schedule(int B, int Hq, int Nq, int Nk, bool causal, int* bh_out, int* qt_out,
                 int* cost_out, int capacity);
// Workgroup of a persistent grid of `grid` workgroups that takes each list
// position (persistent_position); returns n_units, or -1 on bad arguments.
int persistent_schedule(int n_units, int grid, int* worker_out, int capacity);

hipError_t launch_bwd_f32(const float* q, const float* k, const float* v, const float* o,
                          const float* dout, const float* lse, float* dq, float* dk, float* dv,
                          float* delta, int B, int Hq, int Hkv, int Nq, int Nk, float scale,
                          bool causal, hipStream_t stream);
// heads > 1: the rows are a packed token-major [tokens][heads][d] batch and
// delta is written head-major [heads][tokens] (call with B = Hq = 1, Nq =
// tokens * heads).
hipError_t launch_bwd_pre(const void* o, const void* dout, float* delta, int B, int Hq, int Nq,
                          int d, hipStream_t stream, int heads = 1);
hipError_t launch_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout,
                           const float* lse, const float* delta, void* dk, void* dv, int B,
                           int Hq, int Hkv, int Nq, int Nk, int d, float scale, bool causal,
                           hipStream_t stream, int win_l = -1, int win_r = -1);
// o given: the dQ kernel forms delta = dO . O itself and writes it to `delta`
// (launch it before dK/dV, which reads it); o null: it reads `delta`.
hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, const void* dout,
                         const float* lse, float* delta, void* dq, int B, int Hq, int Hkv,
                         int Nq, int Nk, int d, float scale, bool causal, hipStream_t stream,
                         int win_l = -1, int win_r = -1, const void* o = nullptr);
// FP8 dS products: the dQ kernel (d = 128, delta formed from o) with
// dQ = dS K on e5m2 dS x e4m3 K8 (e8m0 scale words ke, one per 32 key rows).
hipError_t launch_bwd_dq_fp8(const void* q, const void* k, const void* v, const void* dout,
                             const float* lse, float* delta, void* dq, const uint8_t* k8,
                             const int32_t* ke, const void* o, int B, int Hq, int Hkv, int Nq,
                             int Nk, float scale, bool causal, hipStream_t stream);
// FP8 dS products: the dK/dV kernel (d = 128) with dK = dS^T Q on e5m2 dS x
// e4m3 Q8 (e8m0 scale words qe, one per 32 query rows).
hipError_t launch_bwd_dkdv_fp8(const void* q, const void* k, const void* v, const void* dout,
                               const float* lse, const float* delta, void* dk, void* dv,
                               const uint8_t* q8, const int32_t* qe, int B, int Hq, int Hkv,
                               int Nq, int Nk, float scale, bool causal, hipStream_t stream);
hipError_t launch_bwd_dkdv_varlen(const void* q, const void* k, const void* v, const void* dout,
                                  const float* lse, const float* delta, void* dk, void* dv,
                                  const int* cu_q, const int* cu_k, int batch, int Hq, int Hkv,
                                  int total_q, int max_seqlen_k, int d, float scale, bool causal,
                                  hipStream_t stream);
hipError_t launch_bwd_dq_varlen(const void* q, const void* k, const void* v, const void* dout,
                                const float* lse, float* delta, void* dq, const int* cu_q,
                                const int* cu_k, int batch, int Hq, int Hkv, int total_q,
                                int max_seqlen_q, int d, float scale, bool causal,
                                hipStream_t stream, const void* o = nullptr);
// map: nqb * nkb bytes of scratch (query tiles of 256 rows x key blocks of 64).
// o given: the dQ kernel (launched first) writes delta; else delta is read.
hipError_t launch_bwd_bf16_sparse(const void* q, const void* k, const void* v, const void* dout,
                                  const float* lse, float* delta, uint8_t* map, void* dq,
                                  void* dk, void* dv, const int* sp_ptr, const int* sp_idx, int B,
                                  int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                                  bool causal, hipStream_t stream, const void* o = nullptr);

// Nq query tokens per (b, head) ([B][Hq][Nq][d]; G*Nq <= 32), partials
// [B][Hq][Nq][S][d] / [B][Hq][Nq][S]; causal: token t sees keys <= Nk-Nq+t.
hipError_t launch_decode_split(const void* q, const void* k, const void* v, float* o_part,
                               float* lse_part, int B, int Hq, int Hkv, int Nk, int d,
                               float scale, int num_splits, hipStream_t stream, int Nq = 1,
                               bool causal = false);
hipError_t launch_decode_split_paged(const void* q, const void* k_cache, const void* v_cache,
                                     const int* block_table, const int* seqlens, float* o_part,
                                     float* lse_part, int B, int Hq, int Hkv, int page_shift,
                                     int max_pages, int num_pages, int chunk, int d, float scale,
                                     int num_splits, hipStream_t stream, int Nq = 1,
                                     bool causal = false);
hipError_t launch_decode_combine(const float* o_part, const float* lse_part, void* o,
                                 float* lse, int B, int Hq, int d, int num_splits,
                                 hipStream_t stream);
// Bytes of the fixed device scratch of the no-allocation decode (one copy per
// GPU); equal to FA_NOALLOC_SCRATCH_BYTES of the C ABI.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
// Device address of this GPU's scratch (looked up once per device, with that
// device current; no allocation).
hipError_t noalloc_scratch(void** addr);
// Split + combine with the partials in the scratch (the caller has checked
// that fa_decode_workspace_size(B, Hq, d, num_splits) fits in it).
hipError_t launch_decode_noalloc(const void* q, const void* k, const void* v, void* o,
                                 float* lse, int B, int Hq, int Hkv, int Nk, int d, float scale,
                                 int num_splits, hipStream_t stream);

hipError_t launch_quantize_fp8(const void* x, const int8_t* signs, uint8_t* x8, float* scales,
                               int B, int H, int N, int d, hipStream_t stream);
// Power-of-two e4m3 quantisation of bf16 [BH][N][128] in blocks of 32 rows:
// codes x8 (same layout), e8m0 scale bytes xe[BH][ceil(N/32)].
hipError_t launch_quantize_pow2_e4m3(const void* x, uint8_t* x8, uint8_t* xe, int BH, int N,
                                     hipStream_t stream);
// The same for two tensors in one launch, each scale code in a 32-bit word
// (xe[BH][ceil(N/32)]).
hipError_t launch_quantize_pow2_e4m3_words2(const void* x0, uint8_t* x8_0, int32_t* xe0, int BH0,
                                            int N0, const void* x1, uint8_t* x8_1, int32_t* xe1,
                                            int BH1, int N1, hipStream_t stream);
hipError_t launch_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                          const float* qs, const float* ks, const float* vs, void* o,
                          float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                          float scale, bool causal, hipStream_t stream);

}  // namespace fa

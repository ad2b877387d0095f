// C ABI of the attention library: argument validation and dispatch to the
// gfx950 kernels.  Every check runs before anything is enqueued, so an invalid
// call leaves the stream untouched.

#include "fa.h"

#include <cmath>
#include <cstdint>

#include "fa_launch.h"

namespace {

constexpr int kVersion = 1 * 10000 + 0 * 100 + 0;

bool aligned16(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool good_scale(float s) { return std::isfinite(s) && s > 0.f; }

size_t round256(size_t n) { return (n + 255) & ~size_t(255); }

fa_status hip_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

// Shape checks shared by the attention entry points.  elem_bytes is the size
// of one Q/K/V element on the path (2 bf16, 4 fp32, 1 fp8).
fa_status check_shape(int B, int Hq, int Hkv, int Nq, int Nk, int d, int elem_bytes = 2) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0 || d <= 0) return FA_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return FA_ERR_INVALID_ARG;
  // element offsets are formed in 64-bit, per-(b,h) row counts in 32-bit
  if ((int64_t)B * Hq > (1 << 24) || (int64_t)B * Hkv > (1 << 24)) return FA_ERR_UNSUPPORTED;
  // One (b, head) slab of Q, K or V is addressed through a buffer descriptor
  // with a 32-bit size and signed 32-bit offsets: it must stay below 2 GiB.
  const int64_t n_max = Nq > Nk ? Nq : Nk;
  if (n_max * d * elem_bytes >= ((int64_t)1 << 31)) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

}  // namespace

extern "C" {

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG: invalid argument";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: unsupported configuration";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace missing or too small";
    case FA_ERR_HIP: return "FA_ERR_HIP: HIP runtime error";
    default: return "unknown fa_status";
  }
}

int fa_version(void) { return kVersion; }

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                 int Hkv, int Nq, int Nk, int d, float scale, int causal, hipStream_t stream) {
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_INVALID_ARG;
  if (fa_status s = check_shape(B, Hq, Hkv, Nq, Nk, d)) return s;
  if (!good_scale(scale)) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (causal && Nq != Nk) return FA_ERR_UNSUPPORTED;
  return hip_status(
      fa::launch_fwd_bf16(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal != 0, stream));
}

static bool good_window(int win_l, int win_r) { return win_l >= -1 && win_r >= -1; }

fa_status fa_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                        int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                        int window_left, int window_right, hipStream_t stream) {
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_INVALID_ARG;
  if (fa_status s = check_shape(B, Hq, Hkv, Nq, Nk, d)) return s;
  if (!good_scale(scale) || !good_window(window_left, window_right)) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (Nq != Nk) return FA_ERR_UNSUPPORTED;  // window positions are defined for Nq == Nk
  return hip_status(fa::launch_fwd_bf16(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale,
                                        causal != 0, stream, window_left, window_right));
}

fa_status fa_fwd_block_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                              int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                              int causal, const int* q_tile_ptr, const int* kv_block_idx,
                              int max_blocks_per_tile, hipStream_t stream) {
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      q_tile_ptr == nullptr || kv_block_idx == nullptr ||
      (reinterpret_cast<uintptr_t>(q_tile_ptr) & 3u) ||
      (reinterpret_cast<uintptr_t>(kv_block_idx) & 3u))
    return FA_ERR_INVALID_ARG;
  if (fa_status s = check_shape(B, Hq, Hkv, Nq, Nk, d)) return s;
  if (!good_scale(scale)) return FA_ERR_INVALID_ARG;
  if (max_blocks_per_tile < 0) return FA_ERR_INVALID_ARG;
  if (max_blocks_per_tile > 256) return FA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (causal && Nq != Nk) return FA_ERR_UNSUPPORTED;
  return hip_status(fa::launch_fwd_bf16_sparse(q, k, v, o, lse, q_tile_ptr, kv_block_idx, B, Hq,
                                               Hkv, Nq, Nk, d, scale, causal != 0, stream));
}

fa_status fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                        const int* cu_seqlens_q, const int* cu_seqlens_k, int batch, int Hq,
                        int Hkv, int total_q, int total_k, int max_seqlen_q, int max_seqlen_k,
                        int d, float scale, int causal, hipStream_t stream) {
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      cu_seqlens_q == nullptr || cu_seqlens_k == nullptr ||
      (reinterpret_cast<uintptr_t>(cu_seqlens_q) & 3u) ||
      (reinterpret_cast<uintptr_t>(cu_seqlens_k) & 3u))
    return FA_ERR_INVALID_ARG;
  if (batch <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || total_q <= 0 || total_k <= 0 ||
      max_seqlen_q <= 0 || max_seqlen_k <= 0 || max_seqlen_q > total_q ||
      max_seqlen_k > total_k || d <= 0)
    return FA_ERR_INVALID_ARG;
  if (!good_scale(scale)) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  // 32-bit buffer offsets: every K/V row of the pack must be addressable.
  if ((int64_t)total_k * Hkv * d * 2 >= ((int64_t)1 << 31)) return FA_ERR_UNSUPPORTED;
  const int64_t units = (int64_t)batch * Hq * ((max_seqlen_q + 255) / 256);
  if (units >= ((int64_t)1 << 31)) return FA_ERR_UNSUPPORTED;
  return hip_status(fa::launch_fwd_bf16_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k,
                                               batch, Hq, Hkv, total_q, max_seqlen_q, d, scale,
                                               causal != 0, stream));
}

fa_status fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                     int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                     hipStream_t stream) {
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_INVALID_ARG;
  if (fa_status s = check_shape(B, Hq, Hkv, Nq, Nk, d, 4)) return s;
  if (!good_scale(scale)) return FA_ERR_INVALID_ARG;
  if (d != 64) return FA_ERR_UNSUPPORTED;
  if (causal && Nq != Nk) return FA_ERR_UNSUPPORTED;
  return hip_status(
      fa::launch_fwd_f32(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, scale, causal != 0, stream));
}

size_t fa_bwd_workspace_size(int B, int Hq, int Nq, int d) {
  if (B <= 0 || Hq <= 0 || Nq <= 0 || d <= 0) return 0;
  return round256((size_t)B * Hq * Nq * sizeof(float));
}

static fa_status bwd_common(const void* q, const void* k, const void* v, const void* o,
                            const void* dout, const float* lse, const void* dq, const void* dk,
                            const void* dv, void* ws, size_t ws_bytes, int B, int Hq, int Hkv,
                            int Nq, int Nk, int d, float scale, int causal,
                            int elem_bytes = 2) {
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(lse) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return FA_ERR_INVALID_ARG;
  if (fa_status s = check_shape(B, Hq, Hkv, Nq, Nk, d, elem_bytes)) return s;
  if (!good_scale(scale)) return FA_ERR_INVALID_ARG;
  if (causal && Nq != Nk) return FA_ERR_UNSUPPORTED;
  if (ws == nullptr || !aligned16(ws)) return FA_ERR_WORKSPACE;
  if (ws_bytes < fa_bwd_workspace_size(B, Hq, Nq, d)) return FA_ERR_WORKSPACE;
  return FA_OK;
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, void* workspace,
                 size_t workspace_bytes, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                 float scale, int causal, hipStream_t stream) {
  if (fa_status s = bwd_common(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B,
                               Hq, Hkv, Nq, Nk, d, scale, causal))
    return s;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  // dQ first: it also forms delta = dO . O for its rows (no pre-pass), which
  // the dK/dV kernel then reads
  float* delta = static_cast<float*>(workspace);
  hipError_t e = fa::launch_bwd_dq(q, k, v, dout, lse, delta, dq, B, Hq, Hkv, Nq, Nk, d, scale,
                                   causal != 0, stream, -1, -1, o);
  if (e == hipSuccess)
    e = fa::launch_bwd_dkdv(q, k, v, dout, lse, delta, dk, dv, B, Hq, Hkv, Nq, Nk, d, scale,
                            causal != 0, stream);
  return hip_status(e);
}

fa_status fa_bwd_window(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int Nq,
                        int Nk, int d, float scale, int causal, int window_left,
                        int window_right, hipStream_t stream) {
  if (fa_status s = bwd_common(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B,
                               Hq, Hkv, Nq, Nk, d, scale, causal))
    return s;
  if (!good_window(window_left, window_right)) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (Nq != Nk) return FA_ERR_UNSUPPORTED;
  float* delta = static_cast<float*>(workspace);
  hipError_t e = fa::launch_bwd_dq(q, k, v, dout, lse, delta, dq, B, Hq, Hkv, Nq, Nk, d, scale,
                                   causal != 0, stream, window_left, window_right, o);
  if (e == hipSuccess)
    e = fa::launch_bwd_dkdv(q, k, v, dout, lse, delta, dk, dv, B, Hq, Hkv, Nq, Nk, d, scale,
                            causal != 0, stream, window_left, window_right);
  return hip_status(e);
}

fa_status fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        void* workspace, size_t workspace_bytes, const int* cu_seqlens_q,
                        const int* cu_seqlens_k, int batch, int Hq, int Hkv, int total_q,
                        int total_k, int max_seqlen_q, int max_seqlen_k, int d, float scale,
                        int causal, hipStream_t stream) {
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(lse) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
      cu_seqlens_q == nullptr || cu_seqlens_k == nullptr ||
      (reinterpret_cast<uintptr_t>(cu_seqlens_q) & 3u) ||
      (reinterpret_cast<uintptr_t>(cu_seqlens_k) & 3u))
    return FA_ERR_INVALID_ARG;
  if (batch <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || total_q <= 0 || total_k <= 0 ||
      max_seqlen_q <= 0 || max_seqlen_k <= 0 || max_seqlen_q > total_q ||
      max_seqlen_k > total_k || d <= 0)
    return FA_ERR_INVALID_ARG;
  if (!good_scale(scale)) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  // 32-bit buffer offsets: every row of the packs must be addressable.
  if ((int64_t)total_k * Hkv * d * 2 >= ((int64_t)1 << 31) ||
      (int64_t)total_q * Hq * d * 2 >= ((int64_t)1 << 31))
    return FA_ERR_UNSUPPORTED;
  if ((int64_t)batch * Hq * ((max_seqlen_q + 255) / 256) >= ((int64_t)1 << 31) ||
      (int64_t)batch * Hkv * ((max_seqlen_k + 255) / 256) >= ((int64_t)1 << 31))
    return FA_ERR_UNSUPPORTED;
  if (workspace == nullptr || !aligned16(workspace)) return FA_ERR_WORKSPACE;
  if (workspace_bytes < fa_bwd_workspace_size(1, Hq, total_q, d)) return FA_ERR_WORKSPACE;
  float* delta = static_cast<float*>(workspace);
  hipError_t e = fa::launch_bwd_dq_varlen(q, k, v, dout, lse, delta, dq, cu_seqlens_q,
                                          cu_seqlens_k, batch, Hq, Hkv, total_q, max_seqlen_q, d,
                                          scale, causal != 0, stream, o);
  if (e == hipSuccess)
    e = fa::launch_bwd_dkdv_varlen(q, k, v, dout, lse, delta, dk, dv, cu_seqlens_q,
                                   cu_seqlens_k, batch, Hq, Hkv, total_q, max_seqlen_k, d,
                                   scale, causal != 0, stream);
  return hip_status(e);
}

size_t fa_bwd_block_sparse_workspace_size(int B, int Hq, int Nq, int Nk, int d) {
  if (B <= 0 || Hq <= 0 || Nq <= 0 || Nk <= 0 || d <= 0) return 0;
  const size_t nqb = (size_t)(Nq + FA_SPARSE_BLOCK_Q - 1) / FA_SPARSE_BLOCK_Q;
  const size_t nkb = (size_t)(Nk + FA_SPARSE_BLOCK_K - 1) / FA_SPARSE_BLOCK_K;
  return fa_bwd_workspace_size(B, Hq, Nq, d) + round256(nqb * nkb);
}

fa_status fa_bwd_block_sparse(const void* q, const void* k, const void* v, const void* o,
                              const void* dout, const float* lse, void* dq, void* dk, void* dv,
                              void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv,
                              int Nq, int Nk, int d, float scale, int causal,
                              const int* q_tile_ptr, const int* kv_block_idx,
                              int max_blocks_per_tile, hipStream_t stream) {
  if (q_tile_ptr == nullptr || kv_block_idx == nullptr ||
      (reinterpret_cast<uintptr_t>(q_tile_ptr) & 3u) ||
      (reinterpret_cast<uintptr_t>(kv_block_idx) & 3u))
    return FA_ERR_INVALID_ARG;
  if (fa_status s = bwd_common(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B,
                               Hq, Hkv, Nq, Nk, d, scale, causal))
    return s;
  if (max_blocks_per_tile < 0) return FA_ERR_INVALID_ARG;
  if (max_blocks_per_tile > 256) return FA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  // the dK/dV work units hold the list of query tiles they visit in 256 slots
  if ((Nq + FA_SPARSE_BLOCK_Q - 1) / FA_SPARSE_BLOCK_Q > 256) return FA_ERR_UNSUPPORTED;
  if (workspace_bytes < fa_bwd_block_sparse_workspace_size(B, Hq, Nq, Nk, d))
    return FA_ERR_WORKSPACE;
  float* delta = static_cast<float*>(workspace);
  uint8_t* map = static_cast<uint8_t*>(workspace) + fa_bwd_workspace_size(B, Hq, Nq, d);
  return hip_status(fa::launch_bwd_bf16_sparse(q, k, v, dout, lse, delta, map, dq, dk, dv,
                                               q_tile_ptr, kv_block_idx, B, Hq, Hkv, Nq, Nk, d,
                                               scale, causal != 0, stream, o));
}

fa_status fa_bwd_pre(const void* o, const void* dout, void* workspace, size_t workspace_bytes,
                     int B, int Hq, int Nq, int d, hipStream_t stream) {
  if (!aligned16(o) || !aligned16(dout)) return FA_ERR_INVALID_ARG;
  if (B <= 0 || Hq <= 0 || Nq <= 0 || d <= 0) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (workspace == nullptr || !aligned16(workspace)) return FA_ERR_WORKSPACE;
  if (workspace_bytes < fa_bwd_workspace_size(B, Hq, Nq, d)) return FA_ERR_WORKSPACE;
  return hip_status(
      fa::launch_bwd_pre(o, dout, static_cast<float*>(workspace), B, Hq, Nq, d, stream));
}

fa_status fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout,
                      const float* lse, void* dk, void* dv, const void* workspace,
                      size_t workspace_bytes, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                      float scale, int causal, hipStream_t stream) {
  // o and dq are not touched by this stage; q stands in for them in the checks
  if (fa_status s = bwd_common(q, k, v, q, dout, lse, q, dk, dv, const_cast<void*>(workspace),
                               workspace_bytes, B, Hq, Hkv, Nq, Nk, d, scale, causal))
    return s;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  return hip_status(fa::launch_bwd_dkdv(q, k, v, dout, lse, static_cast<const float*>(workspace),
                                        dk, dv, B, Hq, Hkv, Nq, Nk, d, scale, causal != 0,
                                        stream));
}

fa_status fa_bwd_dq(const void* q, const void* k, const void* v, const void* dout,
                    const float* lse, void* dq, const void* workspace, size_t workspace_bytes,
                    int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                    hipStream_t stream) {
  // o, dk and dv are not touched by this stage; q stands in for them
  if (fa_status s = bwd_common(q, k, v, q, dout, lse, dq, q, q, const_cast<void*>(workspace),
                               workspace_bytes, B, Hq, Hkv, Nq, Nk, d, scale, causal))
    return s;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  // (reads the delta fa_bwd_pre wrote; nothing is written to the workspace)
  return hip_status(fa::launch_bwd_dq(q, k, v, dout, lse,
                                      static_cast<float*>(const_cast<void*>(workspace)), dq, B,
                                      Hq, Hkv, Nq, Nk, d, scale, causal != 0, stream));
}

fa_status fa_bwd_dq_delta(const void* q, const void* k, const void* v, const void* o,
                          const void* dout, const float* lse, void* dq, void* workspace,
                          size_t workspace_bytes, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                          float scale, int causal, hipStream_t stream) {
  // dk and dv are not touched by this stage; q stands in for them
  if (fa_status s = bwd_common(q, k, v, o, dout, lse, dq, q, q, workspace, workspace_bytes, B,
                               Hq, Hkv, Nq, Nk, d, scale, causal))
    return s;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  return hip_status(fa::launch_bwd_dq(q, k, v, dout, lse, static_cast<float*>(workspace), dq, B,
                                      Hq, Hkv, Nq, Nk, d, scale, causal != 0, stream, -1, -1, o));
}

size_t fa_bwd_fp8_workspace_size(int B, int Hq, int Hkv, int Nq, int Nk, int d) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0 || d <= 0) return 0;
  // delta, e4m3 K and its 32-row scale words, e4m3 Q and its scale words
  return round256((size_t)B * Hq * Nq * sizeof(float)) + round256((size_t)B * Hkv * Nk * d) +
         round256((size_t)B * Hkv * ((Nk + 31) / 32) * 4) + round256((size_t)B * Hq * Nq * d) +
         round256((size_t)B * Hq * ((Nq + 31) / 32) * 4);
}

fa_status fa_bwd_fp8(const void* q, const void* k, const void* v, const void* o,
                     const void* dout, const float* lse, void* dq, void* dk, void* dv,
                     void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int Nq,
                     int Nk, int d, float scale, int causal, hipStream_t stream) {
  if (fa_status s = bwd_common(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B,
                               Hq, Hkv, Nq, Nk, d, scale, causal))
    return s;
  if (d != 128) return FA_ERR_UNSUPPORTED;
  if (workspace_bytes < fa_bwd_fp8_workspace_size(B, Hq, Hkv, Nq, Nk, d)) return FA_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  float* delta = reinterpret_cast<float*>(ws);
  ws += round256((size_t)B * Hq * Nq * sizeof(float));
  uint8_t* k8 = reinterpret_cast<uint8_t*>(ws);
  ws += round256((size_t)B * Hkv * Nk * d);
  int32_t* ke = reinterpret_cast<int32_t*>(ws);
  ws += round256((size_t)B * Hkv * ((Nk + 31) / 32) * 4);
  uint8_t* q8 = reinterpret_cast<uint8_t*>(ws);
  ws += round256((size_t)B * Hq * Nq * d);
  int32_t* qe = reinterpret_cast<int32_t*>(ws);
  hipError_t e = fa::launch_quantize_pow2_e4m3_words2(k, k8, ke, B * Hkv, Nk, q, q8, qe, B * Hq,
                                                      Nq, stream);
  if (e == hipSuccess)
    e = fa::launch_bwd_dq_fp8(q, k, v, dout, lse, delta, dq, k8, ke, o, B, Hq, Hkv, Nq, Nk, scale,
                              causal != 0, stream);
  if (e == hipSuccess)
    e = fa::launch_bwd_dkdv_fp8(q, k, v, dout, lse, delta, dk, dv, q8, qe, B, Hq, Hkv, Nq, Nk,
                                scale, causal != 0, stream);
  return hip_status(e);
}

fa_status fa_quantize_pow2_e4m3(const void* x, uint8_t* x8, uint8_t* x_scale, int B, int H,
                                int N, int d, hipStream_t stream) {
  if (!aligned16(x) || !aligned16(x8) || x_scale == nullptr) return FA_ERR_INVALID_ARG;
  // (codes are stored 8 bytes at a time)
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0) return FA_ERR_INVALID_ARG;
  if (d != 128) return FA_ERR_UNSUPPORTED;
  if ((int64_t)B * H * ((N + 31) / 32) >= ((int64_t)1 << 31)) return FA_ERR_UNSUPPORTED;
  return hip_status(fa::launch_quantize_pow2_e4m3(x, x8, x_scale, B * H, N, stream));
}

fa_status fa_bwd_f32(const float* q, const float* k, const float* v, const float* o,
                     const float* dout, const float* lse, float* dq, float* dk, float* dv,
                     void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int Nq,
                     int Nk, int d, float scale, int causal, hipStream_t stream) {
  if (fa_status s = bwd_common(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B,
                               Hq, Hkv, Nq, Nk, d, scale, causal, 4))
    return s;
  if (d != 64) return FA_ERR_UNSUPPORTED;
  float* delta = static_cast<float*>(workspace);
  return hip_status(fa::launch_bwd_f32(q, k, v, o, dout, lse, dq, dk, dv, delta, B, Hq, Hkv, Nq,
                                       Nk, scale, causal != 0, stream));
}

size_t fa_decode_workspace_size(int B, int Hq, int d, int num_splits) {
  if (B <= 0 || Hq <= 0 || d <= 0 || num_splits <= 0) return 0;
  const size_t rows = (size_t)B * Hq * num_splits;
  return round256(rows * d * sizeof(float)) + round256(rows * sizeof(float));
}

fa_status fa_decode_splitkv(const void* q, const void* k, const void* v, float* o_part,
                            float* lse_part, int B, int Hq, int Hkv, int Nk, int d, float scale,
                            int num_splits, hipStream_t stream) {
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o_part) ||
      !aligned16(lse_part))
    return FA_ERR_INVALID_ARG;
  if (fa_status s = check_shape(B, Hq, Hkv, 1, Nk, d)) return s;
  if (!good_scale(scale)) return FA_ERR_INVALID_ARG;
  if (num_splits <= 0 || num_splits > Nk || Nk % num_splits != 0) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (Hq / Hkv > 32) return FA_ERR_UNSUPPORTED;
  if ((int64_t)B * Hkv * num_splits > (int64_t)1 << 30) return FA_ERR_UNSUPPORTED;
  return hip_status(fa::launch_decode_split(q, k, v, o_part, lse_part, B, Hq, Hkv, Nk, d, scale,
                                            num_splits, stream));
}

fa_status fa_decode_splitkv_q(const void* q, const void* k, const void* v, float* o_part,
                              float* lse_part, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                              float scale, int causal, int num_splits, hipStream_t stream) {
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o_part) ||
      !aligned16(lse_part))
    return FA_ERR_INVALID_ARG;
  if (fa_status s = check_shape(B, Hq, Hkv, Nq, Nk, d)) return s;
  if (!good_scale(scale)) return FA_ERR_INVALID_ARG;
  if (Nq > Nk) return FA_ERR_INVALID_ARG;
  if (num_splits <= 0 || num_splits > Nk || Nk % num_splits != 0) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  // the group's heads times the tokens fill at most the 32 columns of a tile
  if ((int64_t)(Hq / Hkv) * Nq > 32) return FA_ERR_UNSUPPORTED;
  if ((int64_t)B * Hkv * num_splits > (int64_t)1 << 30) return FA_ERR_UNSUPPORTED;
  return hip_status(fa::launch_decode_split(q, k, v, o_part, lse_part, B, Hq, Hkv, Nk, d, scale,
                                            num_splits, stream, Nq, causal != 0));
}

static fa_status decode_paged_impl(const void* q, const void* k_cache, const void* v_cache,
                                   const int* block_table, const int* seqlens, float* o_part,
                                   float* lse_part, int B, int Hq, int Hkv, int Nq, int num_pages,
                                   int page_size, int max_pages, int max_seqlen, int d,
                                   float scale, int causal, int num_splits, hipStream_t stream) {
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o_part) ||
      !aligned16(lse_part) || block_table == nullptr || seqlens == nullptr ||
      (reinterpret_cast<uintptr_t>(block_table) & 3u) || (reinterpret_cast<uintptr_t>(seqlens) & 3u))
    return FA_ERR_INVALID_ARG;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || num_pages <= 0 || max_pages <= 0 ||
      max_seqlen <= 0 || num_splits <= 0 || d <= 0)
    return FA_ERR_INVALID_ARG;
  if (!good_scale(scale)) return FA_ERR_INVALID_ARG;
  int shift = 0;
  while ((1 << shift) < page_size && shift < 30) ++shift;
  if ((1 << shift) != page_size || page_size < 16 || page_size > 4096) return FA_ERR_UNSUPPORTED;
  if ((int64_t)max_pages * page_size < max_seqlen) return FA_ERR_INVALID_ARG;
  if ((int64_t)num_pages * page_size * Hkv * d >= ((int64_t)1 << 31)) return FA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (Nq <= 0 || Nq > max_seqlen) return FA_ERR_INVALID_ARG;
  if ((int64_t)(Hq / Hkv) * Nq > 32) return FA_ERR_UNSUPPORTED;
  if ((int64_t)B * Hkv * num_splits > (int64_t)1 << 30) return FA_ERR_UNSUPPORTED;
  // Keys per chunk: the longest sequence cut in num_splits pieces, rounded up
  // to the kernel's 32-key block (trailing chunks of shorter sequences are
  // empty and come out as lse = -inf).
  const int per = (max_seqlen + num_splits - 1) / num_splits;
  const int chunk = (per + 31) / 32 * 32;
  return hip_status(fa::launch_decode_split_paged(q, k_cache, v_cache, block_table, seqlens,
                                                  o_part, lse_part, B, Hq, Hkv, shift, max_pages,
                                                  num_pages, chunk, d, scale, num_splits, stream, Nq,
                                                  causal != 0));
}

fa_status fa_decode_splitkv_paged(const void* q, const void* k_cache, const void* v_cache,
                                  const int* block_table, const int* seqlens, float* o_part,
                                  float* lse_part, int B, int Hq, int Hkv, int num_pages,
                                  int page_size, int max_pages, int max_seqlen, int d, float scale,
                                  int num_splits, hipStream_t stream) {
  return decode_paged_impl(q, k_cache, v_cache, block_table, seqlens, o_part, lse_part, B, Hq,
                           Hkv, 1, num_pages, page_size, max_pages, max_seqlen, d, scale, 0,
                           num_splits, stream);
}

fa_status fa_decode_splitkv_paged_q(const void* q, const void* k_cache, const void* v_cache,
                                    const int* block_table, const int* seqlens, float* o_part,
                                    float* lse_part, int B, int Hq, int Hkv, int Nq,
                                    int num_pages, int page_size, int max_pages, int max_seqlen,
                                    int d, float scale, int causal, int num_splits,
                                    hipStream_t stream) {
  return decode_paged_impl(q, k_cache, v_cache, block_table, seqlens, o_part, lse_part, B, Hq,
                           Hkv, Nq, num_pages, page_size, max_pages, max_seqlen, d, scale, causal,
                           num_splits, stream);
}

fa_status fa_decode_combine(const float* o_part, const float* lse_part, void* o, float* lse,
                            int B, int Hq, int d, int num_splits, hipStream_t stream) {
  if (!aligned16(o_part) || !aligned16(lse_part) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_INVALID_ARG;
  if (B <= 0 || Hq <= 0 || d <= 0 || num_splits <= 0) return FA_ERR_INVALID_ARG;
  if (d > 256) return FA_ERR_UNSUPPORTED;
  return hip_status(
      fa::launch_decode_combine(o_part, lse_part, o, lse, B, Hq, d, num_splits, stream));
}

fa_status fa_decode_splitkv_noalloc(const void* q, const void* k, const void* v, void* o,
                                   float* lse, int B, int Hq, int Hkv, int Nk, int d, float scale,
                                   int num_splits, hipStream_t stream) {
  static_assert(fa::kNoAllocScratchBytes == FA_NOALLOC_SCRATCH_BYTES, "scratch size");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_INVALID_ARG;
  if (fa_status s = check_shape(B, Hq, Hkv, 1, Nk, d)) return s;
  if (!good_scale(scale)) return FA_ERR_INVALID_ARG;
  if (num_splits <= 0 || num_splits > Nk || Nk % num_splits != 0) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (Hq / Hkv > 32) return FA_ERR_UNSUPPORTED;
  if ((int64_t)B * Hkv * num_splits > (int64_t)1 << 30) return FA_ERR_UNSUPPORTED;
  if (fa_decode_workspace_size(B, Hq, d, num_splits) > FA_NOALLOC_SCRATCH_BYTES)
    return FA_ERR_WORKSPACE;
  return hip_status(fa::launch_decode_noalloc(q, k, v, o, lse, B, Hq, Hkv, Nk, d, scale,
                                              num_splits, stream));
}

fa_status fa_quantize_fp8(const void* x, const int8_t* signs, uint8_t* x8, float* scales, int B,
                          int H, int N, int d, hipStream_t stream) {
  if (!aligned16(x) || !aligned16(x8) || !aligned16(scales)) return FA_ERR_INVALID_ARG;
  if (signs != nullptr && !aligned16(signs)) return FA_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0) return FA_ERR_INVALID_ARG;
  if (d != 128) return FA_ERR_UNSUPPORTED;
  return hip_status(fa::launch_quantize_fp8(x, signs, x8, scales, B, H, N, d, stream));
}

fa_status fa_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                     const float* q_scale, const float* k_scale, const float* v_scale, void* o,
                     float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                     int causal, hipStream_t stream) {
  if (!aligned16(q8) || !aligned16(k8) || !aligned16(v8) || !aligned16(q_scale) ||
      !aligned16(k_scale) || !aligned16(v_scale) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_INVALID_ARG;
  if (fa_status s = check_shape(B, Hq, Hkv, Nq, Nk, d, 1)) return s;
  if (!good_scale(scale)) return FA_ERR_INVALID_ARG;
  if (d != 128) return FA_ERR_UNSUPPORTED;
  if (causal && Nq != Nk) return FA_ERR_UNSUPPORTED;
  return hip_status(fa::launch_fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, o, lse, B, Hq, Hkv,
                                       Nq, Nk, d, scale, causal != 0, stream));
}

int fa_persistent_schedule(int n_units, int grid, int* worker_out, int capacity) {
  return fa::persistent_schedule(n_units, grid, worker_out, capacity);
}

int fa_fwd_schedule(int B, int Hq, int Nq, int Nk, int d, int causal, int* bh_out,
                    int* qtile_out, int* cost_out, int capacity) {
  if (B <= 0 || Hq <= 0 || Nq <= 0 || Nk <= 0 || (d != 64 && d != 128)) return -1;
  if (causal && Nq != Nk) return -1;
  return fa::fwd_schedule(B, Hq, Nq, Nk, causal != 0, bh_out, qtile_out, cost_out, capacity);
}

}  // extern "C"

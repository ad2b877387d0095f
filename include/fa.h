/*
 * fa.h -- C ABI of the exact-attention library for AMD MI355X (gfx950).
 *
 * The library computes exact scaled-dot-product attention
 *     O = softmax(scale * Q K^T + M) V
 * the FlashAttention way: Q and K/V are split into tiles, a running row max and
 * row sum rescale the partial output (online softmax), and the N x N score
 * matrix never reaches device memory.  The forward stores only the per-row
 * logsumexp; the backward recomputes the scores from it.
 *
 * Pages the operations follow (cited by title and section):
 *   [CH18] "第 18 章 FlashAttention" (AI algorithm guide, theaiera.top)
 *   [L21]  "CMU 11-868 L21 FlashAttention" lecture digest (quidproquo.cc)
 *
 * Conventions shared by every entry point
 *   - Tensors are device pointers to contiguous row-major [B][H][N][d] arrays
 *     ("BHSD"): element (b,h,n,c) sits at ((b*H + h)*N + n)*d + c, unless an
 *     entry point states another layout (packed batches, paged caches).
 *   - bf16 tensors are IEEE bfloat16 stored as 16-bit words; fp32 tensors are
 *     float.  Every tensor pointer must be 16-byte aligned.
 *   - Grouped-query attention: Hq must be a multiple of Hkv and query head hq
 *     reads KV head hq / (Hq / Hkv)  ([CH18] §18.2.2).
 *   - scale multiplies Q K^T; it must be finite and > 0 (the usual value is
 *     1/sqrt(d)).
 *   - causal: key j is visible to query i iff j <= i ([CH18] §18.2.2 item 3);
 *     it requires Nq == Nk.  The few-token decode entry points align their
 *     causal mask to the end of the keys instead (stated there).
 *   - lse is fp32 [B][Hq][Nq]: lse_i = ln sum_j exp(scale * q_i . k_j) over the
 *     visible keys (natural log).
 *   - Ownership: the caller allocates and owns every buffer, workspaces
 *     included.  The library allocates no device memory and keeps no mutable
 *     global state, so concurrent calls on different streams are safe.  The
 *     one exception is fa_decode_splitkv_noalloc, which keeps its partials in
 *     a fixed per-GPU scratch array (see there).
 *   - Calls are asynchronous on `stream`.  Argument errors are detected before
 *     anything is enqueued and return FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED or
 *     FA_ERR_WORKSPACE; a failed kernel launch returns FA_ERR_HIP.  Faults in a
 *     running kernel surface at the caller's next synchronisation.
 *   - Outputs are overwritten, never accumulated into.
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1, /* null/misaligned pointer, non-positive size, bad scale */
  FA_ERR_UNSUPPORTED = 2, /* valid but not implemented: head dim, causal Nq != Nk */
  FA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than *_workspace_size */
  FA_ERR_HIP = 4          /* the HIP runtime rejected a launch */
} fa_status;

/* Static, human-readable name of a status code (never NULL). */
const char* fa_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int fa_version(void);

/*
 * Forward, bf16.  [CH18] §18.4.3 (tiled forward with online softmax, Fig.
 * 18-16), §18.5.2 (causal tile skipping); [L21] slides 9-12.
 *   q [B][Hq][Nq][d], k,v [B][Hkv][Nk][d], o [B][Hq][Nq][d]: bf16.
 *   lse [B][Hq][Nq]: fp32.
 *   d in {64, 128}.  Softmax and accumulation are fp32; O is rounded to
 *   bf16 (nearest-even).
 * Work units (query tiles) are ordered longest first ([L21] slides 27-46);
 * causal, a persistent grid of one workgroup per compute unit walks that list
 * (fa_persistent_schedule; [L21] slide 26).  Otherwise every unit costs the
 * same and one workgroup per unit is launched, in an order that gives each
 * XCD (workgroup t runs on XCD t % 8) the query tiles of one (b, h) after
 * another when B*Hq is a multiple of 8 (fa_fwd_schedule shows the order).
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int Hq, int Hkv, int Nq, int Nk, int d,
                 float scale, int causal, hipStream_t stream);

/*
 * Forward with a sliding window, bf16 ([CH18] §18.7.1, window_size =
 * (left, right); §18.8.1: a sliding window is a block-sparse pattern, and
 * only the key tiles inside some row's window are visited).  Same tensors and
 * meaning as fa_fwd, with key j visible to query i only if
 * i - window_left <= j <= i + window_right (and j <= i when causal); -1
 * leaves a side unbounded, so (-1, -1) is plain fa_fwd.  Requires Nq == Nk
 * (positions are aligned top-left); window values below -1 are
 * FA_ERR_INVALID_ARG.  d in {64, 128}.
 */
fa_status fa_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int Hq, int Hkv, int Nq, int Nk, int d,
                        float scale, int causal, int window_left, int window_right,
                        hipStream_t stream);

/*
 * Block-sparse forward, bf16 ([CH18] §18.8.1: query block i attends only to
 * the key blocks in its list; skipped blocks contribute nothing).  Same
 * tensors and meaning as fa_fwd, plus one pattern shared by every (b, head):
 *   query tile t is rows t*FA_SPARSE_BLOCK_Q .. +FA_SPARSE_BLOCK_Q-1, key
 *   block c is keys c*FA_SPARSE_BLOCK_K .. +FA_SPARSE_BLOCK_K-1;
 *   q_tile_ptr: device int32 [ceil(Nq/FA_SPARSE_BLOCK_Q) + 1], CSR row
 *   offsets; kv_block_idx: device int32, the listed key blocks of each query
 *   tile (distinct within a tile; any order, ascending is fastest).
 *   max_blocks_per_tile: the longest list (<= 256; FA_ERR_UNSUPPORTED above).
 * causal additionally masks j > i (requires Nq == Nk).  A row that sees no
 * key gets O = 0 and LSE = -inf.  The lists are device data and are not
 * checked on the host; a block index outside [0, ceil(Nk/64)) reads zeros
 * and is masked, and a tile's list is cut at 256 entries.  d in {64, 128}.
 */
#define FA_SPARSE_BLOCK_Q 256
#define FA_SPARSE_BLOCK_K 64
fa_status fa_fwd_block_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                              int B, int Hq, int Hkv, int Nq, int Nk, int d,
                              float scale, int causal, const int* q_tile_ptr,
                              const int* kv_block_idx, int max_blocks_per_tile,
                              hipStream_t stream);

/*
 * Forward over a packed variable-length batch, bf16 ([CH18] §18.7.1: the
 * sequences are concatenated along the token axis and cumulative offsets
 * give each one's rows; attention never crosses a sequence boundary and the
 * causal mask applies inside each sequence).
 *   q, o [total_q][Hq][d] and k, v [total_k][Hkv][d], bf16, token-major (the
 *   page's (total_tokens, nheads, headdim)).
 *   cu_seqlens_q, cu_seqlens_k: device int32 [batch+1], non-decreasing, from
 *   0 to total_q / total_k; sequence b owns query rows cu_seqlens_q[b] ..
 *   cu_seqlens_q[b+1]-1 and key rows cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1.
 *   lse [Hq][total_q] fp32 (natural log).
 *   max_seqlen_q / max_seqlen_k: the longest sequence (sizes the launch;
 *   must be >= every sequence's length).
 * causal: key j visible to query i of the same sequence iff j <= i
 * (top-left, as for fa_fwd; meant for equal query and key lengths).  A
 * sequence with queries but no keys gets O = 0 and LSE = -inf.  The offsets
 * are device data and are not checked on the host; they must satisfy the
 * above.  d in {64, 128}; total_k * Hkv * d * 2 < 2^31.
 */
fa_status fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                        const int* cu_seqlens_q, const int* cu_seqlens_k,
                        int batch, int Hq, int Hkv, int total_q, int total_k,
                        int max_seqlen_q, int max_seqlen_k, int d,
                        float scale, int causal, hipStream_t stream);

/*
 * Forward, fp32 in and out: the tiled forward of [CH18] §18.4.3 (online
 * softmax across key tiles, Fig. 18-16) with the same layout and meaning as
 * fa_fwd, everything in fp32.  d == 64.  Query and key tiles are 64 rows,
 * so Nk = 256 exercises four rounds of online rescaling.
 */
fa_status fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                     int B, int Hq, int Hkv, int Nq, int Nk, int d,
                     float scale, int causal, hipStream_t stream);

/*
 * Bytes of workspace fa_bwd / fa_bwd_f32 need: the fp32 row term delta
 * [B][Hq][Nq], rounded up to 256 bytes.
 */
size_t fa_bwd_workspace_size(int B, int Hq, int Nq, int d);

/*
 * Backward, bf16.  [CH18] §18.2.4 (gradients of attention), §18.4.4
 * (recomputation: P is rebuilt from the saved logsumexp, no rescaling).
 *   q,k,v,o,dout: bf16, o and lse as written by fa_fwd for the same inputs.
 *   dq [B][Hq][Nq][d], dk,dv [B][Hkv][Nk][d]: bf16 outputs.  A KV head's
 *   gradient is summed over the query heads of its group.
 *   workspace: at least fa_bwd_workspace_size(B,Hq,Nq,d) bytes, 16-byte
 *   aligned; its contents on entry do not matter.
 * Two launches on `stream`: dQ, one work unit per query tile accumulating
 * over the KV tiles, which also forms delta_i = dO_i . O_i (equal to
 * rowsum(P * dP), [CH18] §18.4.4) from its rows' dO and O and writes it to the
 * workspace; then dK and dV, one work unit per KV tile accumulating over the
 * query tiles.  No atomics: results are deterministic.
 *   d in {64, 128}.
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o,
                 const void* dout, const float* lse,
                 void* dq, void* dk, void* dv,
                 void* workspace, size_t workspace_bytes,
                 int B, int Hq, int Hkv, int Nq, int Nk, int d,
                 float scale, int causal, hipStream_t stream);

/*
 * Backward with a sliding window (the gradients of fa_fwd_window): same
 * arguments and workspace as fa_bwd plus the window; o and lse as written by
 * fa_fwd_window for the same inputs and window.  Requires Nq == Nk.
 */
fa_status fa_bwd_window(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse,
                        void* dq, void* dk, void* dv,
                        void* workspace, size_t workspace_bytes,
                        int B, int Hq, int Hkv, int Nq, int Nk, int d,
                        float scale, int causal, int window_left, int window_right,
                        hipStream_t stream);

/*
 * Backward of the block-sparse forward (the gradients of fa_fwd_block_sparse
 * for the same inputs and pattern; [CH18] §18.8.1 for the pattern, §18.4.4
 * for the gradients; skipped blocks have P = 0 and get no gradient).  Same
 * tensors as fa_bwd, pattern arguments as fa_fwd_block_sparse (the lists
 * must hold distinct blocks, as the forward requires).
 *   workspace: at least fa_bwd_block_sparse_workspace_size(B,Hq,Nq,Nk,d)
 *   bytes, 16-byte aligned: delta, then a byte map of the pattern (query
 *   tiles x key blocks) that the call rebuilds from the lists each time.
 * A row that sees no key gets dQ = 0; a key that no row sees dK = dV = 0.
 * Three launches on `stream` (the map, dQ with delta, dK/dV); deterministic.
 *   d in {64, 128}; ceil(Nq / FA_SPARSE_BLOCK_Q) <= 256 (FA_ERR_UNSUPPORTED
 *   above: a dK/dV work unit keeps the query tiles it visits in 256 slots).
 */
size_t fa_bwd_block_sparse_workspace_size(int B, int Hq, int Nq, int Nk, int d);
fa_status fa_bwd_block_sparse(const void* q, const void* k, const void* v, const void* o,
                              const void* dout, const float* lse,
                              void* dq, void* dk, void* dv,
                              void* workspace, size_t workspace_bytes,
                              int B, int Hq, int Hkv, int Nq, int Nk, int d,
                              float scale, int causal, const int* q_tile_ptr,
                              const int* kv_block_idx, int max_blocks_per_tile,
                              hipStream_t stream);

/*
 * Backward over a packed variable-length batch (the gradients of
 * fa_fwd_varlen, [CH18] §18.7.1 for the packing, §18.4.4 for the gradients):
 * q, o, dout, dq [total_q][Hq][d] and k, v, dk, dv [total_k][Hkv][d], bf16,
 * token-major; lse [Hq][total_q] as written by fa_fwd_varlen for the same
 * inputs; cu_seqlens_q / cu_seqlens_k and max_seqlen_q / max_seqlen_k as for
 * fa_fwd_varlen (device int32 offsets, not checked on the host).
 *   workspace: at least fa_bwd_workspace_size(1, Hq, total_q, d) bytes,
 *   16-byte aligned (delta, head-major like lse).
 * Gradients never cross a sequence boundary; a key with no visible query
 * (e.g. a sequence with keys but no queries) gets dK = dV = 0, a query with
 * no key dQ = 0.  Same two launches as fa_bwd; deterministic.
 *   d in {64, 128}; total_q * Hq * d * 2 and total_k * Hkv * d * 2 < 2^31.
 */
fa_status fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse,
                        void* dq, void* dk, void* dv,
                        void* workspace, size_t workspace_bytes,
                        const int* cu_seqlens_q, const int* cu_seqlens_k,
                        int batch, int Hq, int Hkv, int total_q, int total_k,
                        int max_seqlen_q, int max_seqlen_k, int d,
                        float scale, int causal, hipStream_t stream);

/*
 * The three stages of fa_bwd as separate calls, for callers that schedule or
 * time them individually.  Same arguments and workspace as fa_bwd; fa_bwd_pre
 * must precede the other two on the stream (or be ordered before them), which
 * are independent of each other.  fa_bwd_pre + fa_bwd_dkdv + fa_bwd_dq is
 * exactly fa_bwd.
 *   fa_bwd_pre:  delta_i = dO_i . O_i into the workspace ([CH18] §18.4.4: the
 *                row term of the softmax backward, rowsum(P * dP), equals
 *                dO_i . O_i).
 *   fa_bwd_dkdv: dk and dv written.
 *   fa_bwd_dq:   dq written.
 * fa_bwd itself runs the two-stage order fa_bwd_dq_delta + fa_bwd_dkdv: the
 * dQ kernel, which holds each row's dO, reads the row's O beside it and
 * writes delta itself, so no pre-pass is launched.
 *   fa_bwd_dq_delta: dq written, and delta into the workspace; fa_bwd_dkdv
 *                must follow it on the stream (or be ordered after it).
 */
fa_status fa_bwd_pre(const void* o, const void* dout, void* workspace, size_t workspace_bytes,
                     int B, int Hq, int Nq, int d, hipStream_t stream);
fa_status fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout,
                      const float* lse, void* dk, void* dv, const void* workspace,
                      size_t workspace_bytes, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                      float scale, int causal, hipStream_t stream);
fa_status fa_bwd_dq(const void* q, const void* k, const void* v, const void* dout,
                    const float* lse, void* dq, const void* workspace, size_t workspace_bytes,
                    int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                    hipStream_t stream);
fa_status fa_bwd_dq_delta(const void* q, const void* k, const void* v, const void* o,
                          const void* dout, const float* lse, void* dq, void* workspace,
                          size_t workspace_bytes, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                          float scale, int causal, hipStream_t stream);

/*
 * Backward, fp32 tensors, d == 64: the recompute backward of [CH18] §18.4.4
 * (P rebuilt from lse, delta = rowsum(dO * O), dS = P (dP - delta)), with the
 * same meaning and workspace as fa_bwd; deterministic.
 */
fa_status fa_bwd_f32(const float* q, const float* k, const float* v, const float* o,
                     const float* dout, const float* lse,
                     float* dq, float* dk, float* dv,
                     void* workspace, size_t workspace_bytes,
                     int B, int Hq, int Hkv, int Nq, int Nk, int d,
                     float scale, int causal, hipStream_t stream);

/*
 * Split-KV decode ([CH18] §18.8.2, Flash-Decoding; [L21] slides 57-60, GQA
 * packing).  One query position per (b, hq) attends all Nk keys, non-causal.
 * The key range is cut into num_splits equal chunks; each work unit handles
 * one chunk for one (b, KV head) and packs the Hq/Hkv query heads that share
 * the KV head into the rows of one tile, so K and V are read once per group.
 *   q [B][Hq][1][d] bf16; k,v [B][Hkv][Nk][d] bf16.
 *   o_part [B][Hq][num_splits][d] fp32: each chunk's softmax-normalised
 *   partial output.  lse_part [B][Hq][num_splits] fp32: each chunk's
 *   logsumexp.
 * Requirements: num_splits >= 1 divides Nk; d == 128 (and 64);
 * Hq/Hkv <= 32.
 */
fa_status fa_decode_splitkv(const void* q, const void* k, const void* v,
                            float* o_part, float* lse_part,
                            int B, int Hq, int Hkv, int Nk, int d,
                            float scale, int num_splits, hipStream_t stream);

/*
 * Split-KV decode with a few query tokens ([L21] slides 57-60: decode
 * queries are a few tokens against a long context, and GQA packing extends
 * from one query token to any number): the Hq/Hkv heads of a group times the
 * Nq tokens are packed into the columns of one tile, so K and V are still
 * read once per group.  The tokens are the newest Nq positions of each
 * sequence: with causal, token t (0-based) sees keys 0 .. Nk-Nq+t (a mask
 * aligned to the end of the keys; Nq == Nk gives the causal forward's mask);
 * without it every token sees all Nk keys.
 *   q [B][Hq][Nq][d] bf16; k,v [B][Hkv][Nk][d] bf16.
 *   o_part [B][Hq][Nq][num_splits][d] fp32, lse_part [B][Hq][Nq][num_splits]
 *   fp32 (as for fa_decode_splitkv, one row per (b, hq, token)); a chunk
 *   whose keys a token cannot see gets O_c = 0 and lse_c = -inf.
 * Combine with fa_decode_combine(o_part, lse_part, o, lse, B, Hq * Nq, d,
 * num_splits): o [B][Hq][Nq][d], lse [B][Hq][Nq].  fa_decode_workspace_size
 * (B, Hq * Nq, d, num_splits) sizes the partials.
 * Requirements: 1 <= Nq <= Nk; num_splits >= 1 divides Nk; d in {64, 128};
 * (Hq/Hkv) * Nq <= 32 (FA_ERR_UNSUPPORTED above).  Nq == 1 is exactly
 * fa_decode_splitkv.
 */
fa_status fa_decode_splitkv_q(const void* q, const void* k, const void* v,
                              float* o_part, float* lse_part,
                              int B, int Hq, int Hkv, int Nq, int Nk, int d,
                              float scale, int causal, int num_splits, hipStream_t stream);

/*
 * Split-KV decode over a paged KV cache ([CH18] §18.8.2 (3): Flash-Decoding
 * combined with a paged cache; §18.8.3 (1): the cache lives in fixed-size
 * physical pages and each request's page table maps its logical block j to a
 * physical page).  Same partial outputs as fa_decode_splitkv, merged by
 * fa_decode_combine.
 *   q [B][Hq][1][d] bf16.
 *   k_cache, v_cache [num_pages][page_size][Hkv][d] bf16: page p, row r holds
 *   one token's K (V) for every KV head.
 *   block_table: device int32 [B][max_pages]; logical key t of batch entry b
 *   is row t % page_size of page block_table[b][t / page_size].
 *   seqlens: device int32 [B], the number of keys of each entry (>= 1).
 *   o_part [B][Hq][num_splits][d], lse_part [B][Hq][num_splits] fp32 as for
 *   fa_decode_splitkv.  Chunk c covers logical keys [c*L, (c+1)*L) with
 *   L = ceil(max_seqlen / num_splits) rounded up to a multiple of 32; a chunk
 *   past an entry's length writes O_c = 0 and lse_c = -inf.
 * Requirements: page_size a power of two in [16, 4096]; max_seqlen >= every
 * seqlens[b] and <= max_pages * page_size; d in {64, 128}; Hq/Hkv <= 32.
 * The table and lengths are device data and are not checked on the host: a
 * page id outside [0, num_pages) or a length past max_pages * page_size is
 * clamped by the kernel (wrong rows are read, never memory out of bounds).
 * Both pointers must be 4-byte aligned.
 */
fa_status fa_decode_splitkv_paged(const void* q, const void* k_cache, const void* v_cache,
                                  const int* block_table, const int* seqlens,
                                  float* o_part, float* lse_part,
                                  int B, int Hq, int Hkv, int num_pages, int page_size,
                                  int max_pages, int max_seqlen, int d,
                                  float scale, int num_splits, hipStream_t stream);

/*
 * fa_decode_splitkv_paged with a few query tokens per head: q [B][Hq][Nq][d]
 * are the newest Nq positions of each entry, with the end-aligned causal mask
 * of fa_decode_splitkv_q (token t sees logical keys 0 .. seqlens[b]-Nq+t)
 * when causal is set.  Partials and the combine as for fa_decode_splitkv_q
 * (rows per (b, hq, token)).  Requires 1 <= Nq <= max_seqlen and
 * (Hq/Hkv) * Nq <= 32; an entry with seqlens[b] < Nq leaves its first tokens
 * without keys when causal (O = 0, LSE = -inf).  Nq == 1 is exactly
 * fa_decode_splitkv_paged.
 */
fa_status fa_decode_splitkv_paged_q(const void* q, const void* k_cache, const void* v_cache,
                                    const int* block_table, const int* seqlens,
                                    float* o_part, float* lse_part,
                                    int B, int Hq, int Hkv, int Nq, int num_pages, int page_size,
                                    int max_pages, int max_seqlen, int d,
                                    float scale, int causal, int num_splits, hipStream_t stream);

/*
 * Merge of the split partials ([CH18] §18.8.2 (2), reduction step):
 *   lse = M + ln sum_c exp(lse_c - M) with M = max_c lse_c,
 *   O   = sum_c exp(lse_c - lse) * O_c.
 *   o [B][Hq][1][d] bf16, lse [B][Hq][1] fp32.  d <= 256.
 */
fa_status fa_decode_combine(const float* o_part, const float* lse_part,
                            void* o, float* lse,
                            int B, int Hq, int d, int num_splits, hipStream_t stream);

/* Bytes the caller must provide for o_part and lse_part together (one
 * allocation: o_part first, lse_part at the next 256-byte boundary). */
size_t fa_decode_workspace_size(int B, int Hq, int d, int num_splits);

/*
 * Split-KV decode and its merge in one call that allocates nothing, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid it).  Same inputs, outputs and
 * requirements as fa_decode_splitkv followed by fa_decode_combine:
 *   q [B][Hq][1][d], k,v [B][Hkv][Nk][d] bf16 in; o [B][Hq][1][d] bf16 and
 *   lse [B][Hq][1] fp32 out.
 * The split partials go to a fixed scratch array in device memory that the
 * library holds for each GPU it runs on, until the process ends, instead of a
 * caller's workspace.  fa_decode_workspace_size(B, Hq, d, num_splits) must not
 * exceed FA_NOALLOC_SCRATCH_BYTES (16 MiB; e.g. B=8, Hq=32, d=128, 64 splits
 * needs 8.4 MB): a larger call returns FA_ERR_WORKSPACE and enqueues nothing.
 * Every call on one GPU shares that GPU's scratch, so calls that overlap on
 * one GPU (on different streams, or from different threads without ordering)
 * race and give undefined output; calls ordered on one stream are safe.  The
 * first call on a device looks up the scratch's address (no allocation).
 */
#define FA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
fa_status fa_decode_splitkv_noalloc(const void* q, const void* k, const void* v, void* o,
                                    float* lse, int B, int Hq, int Hkv, int Nk, int d,
                                    float scale, int num_splits, hipStream_t stream);

/*
 * FP8 quantisation pre-pass ([CH18] §18.6.2 (1)(2); [L21] slide 24).
 *   x [B][H][N][d] bf16 in; x8 [B][H][N][d] e4m3fn codes out (1 byte each);
 *   scales [B][H][ceil(N/128)] fp32 out.
 *   signs: device int8[d] of +-1, or NULL.  When given, every row is first
 *   rotated by J = diag(signs) * Hadamard(d) / sqrt(d) (incoherent
 *   processing: applied to Q and K with the same signs, (QJ)(KJ)^T = QK^T).
 *   Each (b, h, 128-row block) gets amax = max |x|, r = fp32(448 / amax),
 *   codes = e4m3(fp32(x * r)) rounded to nearest-even and saturated to +-448,
 *   scale = fp32(amax / 448) (1 for an all-zero block).
 *   d == 128.
 */
fa_status fa_quantize_fp8(const void* x, const int8_t* signs, uint8_t* x8, float* scales,
                          int B, int H, int N, int d, hipStream_t stream);

/*
 * FP8 forward ([CH18] §18.6.2 (1)-(2): e4m3 operands with per-block scales;
 * [L21] slide 24: incoherent processing by the quantiser): fa_fwd on e4m3
 * operands with per-128-row-block fp32 scales (from fa_quantize_fp8).  S = (Q8 K8^T) * s_q * s_k * scale; softmax in
 * fp32; P is rounded to e4m3 for the P V product; O is bf16, lse fp32.
 *   q8 [B][Hq][Nq][d], k8,v8 [B][Hkv][Nk][d]; q_scale [B][Hq][ceil(Nq/128)],
 *   k_scale, v_scale [B][Hkv][ceil(Nk/128)].  d == 128.
 * Every scale must be positive and finite, as fa_quantize_fp8 writes them
 * (1 for an all-zero block): the kernel folds each V block's scale into the
 * exponent as log2(s_v / max s_v), so a zero or negative scale gives
 * undefined output.  Scales live in device memory and are not checked.
 */
fa_status fa_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                     const float* q_scale, const float* k_scale, const float* v_scale,
                     void* o, float* lse,
                     int B, int Hq, int Hkv, int Nq, int Nk, int d,
                     float scale, int causal, hipStream_t stream);

/*
 * Power-of-two e4m3 quantisation for the fp8 gradient products ([CH18]
 * §18.6.2 (3); the operands of dQ = dS K and dK = dS^T Q).
 *   x [B][H][N][d] bf16 in; x8 [B][H][N][d] e4m3fn codes out;
 *   x_scale [B][H][ceil(N/32)] bytes out, one per block of 32 rows x d.
 *   Each block gets e = the smallest integer with max|x| <= 448 * 2^e (0 for
 *   an all-zero block), codes = e4m3(x * 2^-e) (the scaling is exact;
 *   rounding to nearest even) and x_scale = e + 127 (an e8m0 byte: the block
 *   holds code * 2^(x_scale - 127)).  e is kept >= -126: blocks whose maximum
 *   is below 448 * 2^-126 are scaled by 2^126 (their small values may round
 *   to zero).
 *   d == 128; x, x8 16-byte aligned.
 */
fa_status fa_quantize_pow2_e4m3(const void* x, uint8_t* x8, uint8_t* x_scale,
                                int B, int H, int N, int d, hipStream_t stream);

/*
 * Bytes of workspace fa_bwd_fp8 needs: delta [B][Hq][Nq] fp32, the e4m3
 * copies of K and Q with their 32-row scale codes (one 32-bit word each),
 * each part rounded up to 256 bytes.
 */
size_t fa_bwd_fp8_workspace_size(int B, int Hq, int Hkv, int Nq, int Nk, int d);

/*
 * Backward with fp8 dS products ([CH18] §18.6.2 (3)): S, P, dP and dS are
 * formed as in fa_bwd (bf16 products, fp32 softmax terms, delta = rowsum(dO *
 * O) from the given o); the two dS products then run on the scaled fp8
 * matrix cores with fp32 accumulation: dQ = scale * dS K with dS in e5m2, one
 * power-of-two scale per (query row, 32-key block), and dK = scale * dS^T Q
 * with dS in e5m2, one power-of-two scale per (key, 32-query block), against
 * K and Q in e4m3 (fa_quantize_pow2_e4m3 blocks, formed here into the
 * workspace).  dV = P^T dO stays bf16.
 *   Arguments as fa_bwd; workspace at least fa_bwd_fp8_workspace_size bytes,
 *   16-byte aligned (contents on entry do not matter).  d == 128.
 * Launches on `stream`: the K and Q quantisers, dQ (which also forms delta),
 * dK/dV.  Deterministic.
 */
fa_status fa_bwd_fp8(const void* q, const void* k, const void* v, const void* o,
                     const void* dout, const float* lse, void* dq, void* dk, void* dv,
                     void* workspace, size_t workspace_bytes,
                     int B, int Hq, int Hkv, int Nq, int Nk, int d,
                     float scale, int causal, hipStream_t stream);

/*
 * Host-side view of the forward's work order ([L21] slides 27-46: longest
 * processing time first).  Writes, for each of the n work units the forward
 * launches in dispatch order, its (b*Hq + h) index, its query-tile index and
 * its cost in KV tiles.  Returns the number of work units, or -1 on bad
 * arguments; with NULL outputs only the count is returned.  No GPU is needed.
 */
int fa_fwd_schedule(int B, int Hq, int Nq, int Nk, int d, int causal,
                    int* bh_out, int* qtile_out, int* cost_out, int capacity);

/*
 * Host-side view of the persistent grids ([L21] slide 26: a grid of as many
 * workgroups as compute units, each taking work units in turn; slides 27-46:
 * longest first).  The causal dense forward and dQ kernels launch
 * min(n_units, compute units) workgroups; workgroup w of G takes the
 * positions w, 2G-1-w, 2G+w, 4G-1-w, ... of the longest-first list (snake
 * order), so each round's longest units pair with the next round's shortest.
 * Writes, for each of the n_units list positions, the workgroup that takes
 * it.  Returns n_units, or -1 on bad arguments (n_units < 0, grid <= 0,
 * capacity < n_units with a non-NULL output).  No GPU is needed.
 */
int fa_persistent_schedule(int n_units, int grid, int* worker_out, int capacity);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */

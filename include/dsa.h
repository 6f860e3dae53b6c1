/*
 * dsa.h -- C ABI of the MI355X (gfx950) DeepSeek-Sparse-Attention
 * draft-and-verify library (libdsa.so).
 *
 * The path (pages: "Optimizing speculative decoding" and "GLM-5.2: Tuning MTP
 * speculative decoding to the limit", longformexplainers.com):
 *
 *   draft step 1   dsa_index_scores -> dsa_topk -> dsa_sparse_attn
 *   draft steps 2+ dsa_sparse_attn with the indices of step 1 (IndexShare)
 *   verify         spec_verify over the drafted chain (rejection sampling)
 *
 * Conventions shared by every entry point:
 *   - Tensor arguments are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or retains them.  Scratch memory is passed in
 *     as a caller-owned device workspace whose size the matching
 *     *_workspace_size() query returns (0 is valid when none is needed).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *     enqueue work on it and never synchronise; pointers must stay valid
 *     until that work completes.  Two calls sharing a workspace must be
 *     ordered on one stream.
 *   - Every shape/pointer check runs on the host before any HIP call; a
 *     failed check returns DSA_ERR_INVALID_ARG / DSA_ERR_UNSUPPORTED /
 *     DSA_ERR_WORKSPACE and enqueues nothing.  dsa_last_error() returns a
 *     message for the calling thread's last failure.  Launch failures return
 *     DSA_ERR_HIP.  Nothing aborts and no exception crosses the ABI.
 *   - Identical inputs (and seed/offset) give bitwise-identical outputs:
 *     reductions run in a fixed order and no float atomics are used.
 *   - bf16 tensors are IEEE bfloat16 bit patterns (uint16 storage).
 *   - Device-side preconditions (indices < row length, block-table entries
 *     naming allocated pages, no NaN scores) are not checked on the device;
 *     breaking them gives unspecified results.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_ABI_VERSION 1

/* Longest score row (ld) dsa_index_scores and dsa_topk accept: positions are
 * int32 inside the kernels, with headroom for whole tile steps past the end. */
#define DSA_MAX_LD (((int64_t)1 << 31) - 65536)

typedef enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = 1,   /* null pointer, non-positive size, bad stride */
  DSA_ERR_UNSUPPORTED = 2,   /* valid but not instantiated (e.g. head dim)   */
  DSA_ERR_WORKSPACE = 3,     /* workspace missing or smaller than required   */
  DSA_ERR_HIP = 4            /* a HIP launch/runtime call failed             */
} dsa_status;

/* Static description of a status code. */
const char* dsa_status_str(int status);
/* Message of the calling thread's last failed call ("" if none). */
const char* dsa_last_error(void);
/* DSA_ABI_VERSION of the loaded library. */
int dsa_abi_version(void);

/*
 * dsa_index_scores -- lightning-indexer scores (DSA glossary entry, section
 * "IndexShare and KVShare": a light indexer scores every past token with
 * cheap dot products).  For every sequence b, row r and visible position
 * t < row_len[b*R + r]:
 *
 *   scores[(b*R + r)*ld + t] = sum_h w[(b*R + r)*H_I + h]
 *                               * max(0, sum_d q[((b*R + r)*H_I + h)*D_I + d] * K(b, t, d))
 *
 * with K(b, t, d) = k_index[((block_table[b*max_pages + t/page]) * page
 *                             + t % page) * D_I + d]   (one key per position,
 * shared by all heads; paged in blocks of `page` positions).
 *
 *   q           bf16 [B, R, H_I, D_I]        w     fp32 [B, R, H_I]
 *   k_index     bf16 [num_pages, page, D_I]  block_table int32 [B, max_pages]
 *   row_len     int32 [B, R], 0 <= row_len <= min(ld, page*max_pages)
 *   scores      fp32 [B, R, ld]; entries at t >= row_len are left untouched.
 * Products are exact bf16*bf16 in fp32; dot products accumulate in fp32
 * (MFMA), the ReLU/weight/head sum runs in fp32.
 * Supported: D_I in {32, 64, 128}, 1 <= H_I <= 64, 1 <= R <= 8,
 * B <= 65535.  q and k_index 16-byte aligned.  A row_len beyond the bound
 * above is clamped to it (no access outside the score rows or the table).
 */
dsa_status dsa_index_scores(const void* q, const float* w, const void* k_index,
                            const int32_t* block_table, const int32_t* row_len,
                            float* scores, int B, int R, int H_I, int D_I,
                            int page, int max_pages, int64_t ld, void* stream);

/*
 * dsa_topk -- top-k selection per (sequence, row) (DSA glossary entry: a
 * top-k selection keeps the most relevant past positions).
 * Candidates are t in [0, row_len[row]).  Order: score descending, then
 * position ascending (equal scores keep the lower position; -0.0 == +0.0).
 * The kept min(k, row_len) positions are written to idx[row*k ...] in
 * ascending position order and the rest of the row is filled with -1.
 *
 *   scores  fp32 [B*R, ld] (NaN not allowed)   row_len int32 [B*R]
 *   idx     int32 [B*R, k]                      1 <= k <= 8192, B*R <= 65535
 * A row_len above ld is treated as ld.
 * workspace: dsa_topk_workspace_size() bytes (0 when ld <= 35840: one launch
 *   per call, the row's keys held in LDS); no initialisation required.
 */
size_t dsa_topk_workspace_size(int B, int R, int64_t ld, int k);
dsa_status dsa_topk(const float* scores, const int32_t* row_len, int B, int R,
                    int64_t ld, int k, int32_t* idx, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * dsa_sparse_attn -- attention over the selected positions only (DSA
 * glossary entry: full attention runs over only the top-k subset).  With
 * IndexShare the same `idx` from draft step 1 is passed unchanged to every
 * draft step, so each step reads only target-written KV (section
 * "IndexShare and KVShare").  For sequence b, query row s, head h with KV
 * head g = h / (H_q / H_kv) and S = { idx[b, *] >= 0 }:
 *
 *   out[b,s,h,:] = sum_{t in S} softmax_t(sm_scale * q[b,s,h,:] . Kt) * Vt
 *   lse[b,s,h]   = log sum_{t in S} exp(sm_scale * q[b,s,h,:] . Kt)
 *
 * where Kt / Vt are the first D_qk / D_v elements at
 *   cache + P*kv_page_stride + (t % page)*kv_row_stride + g*kv_head_stride,
 *   P = block_table[b*max_pages + t/page]   (strides in elements).
 * An empty S gives out = 0 and lse = -inf.
 *
 *   q        bf16 [B, S_q, H_q, D_qk]         out fp32 [B, S_q, H_q, D_v]
 *   k_cache, v_cache  bf16 paged; v_cache may equal k_cache (latent KV,
 *            V = the first D_v dims of the key row)
 *   idx      int32 [B, idx_rows, k], idx_rows = 1 (shared by every query
 *            row) or S_q (one set per row); -1 entries, and positions at or
 *            past page*max_pages, are ignored
 *   lse      fp32 [B, S_q, H_q] or NULL
 * workspace: dsa_sparse_attn_workspace_size() bytes (0: none needed) for
 *   split-k partial results; no initialisation required.
 * Supported: (H_q == H_kv or H_q/H_kv in {2, 4}) with D_qk == D_v in
 * {64, 128}; or H_kv == 1, H_q == 64, D_qk == 576, D_v == 512 with
 * v_cache == k_cache (latent MQA; QK^T and PV on bf16 MFMA, P rounded to
 * bf16).  k <= 131072 (latent: k <= 32768), B*S_q <= 65535.  Rows/heads/base
 * pointers of q, k_cache, v_cache and out 16-byte aligned (else
 * DSA_ERR_INVALID_ARG).
 */
size_t dsa_sparse_attn_workspace_size(int B, int S_q, int H_q, int H_kv,
                                      int D_qk, int D_v, int k);
dsa_status dsa_sparse_attn(const void* q, const void* k_cache, const void* v_cache,
                           int64_t kv_page_stride, int64_t kv_row_stride,
                           int64_t kv_head_stride, const int32_t* block_table,
                           const int32_t* idx, int idx_rows, int B, int S_q,
                           int H_q, int H_kv, int D_qk, int D_v, int page,
                           int max_pages, int k, float sm_scale, float* out,
                           float* lse, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * dsa_sparse_attn_noalloc -- dsa_sparse_attn without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, semantics, kernels and output bits as dsa_sparse_attn with
 * the same shapes; the split-k partials go to a file-scope device array of
 * DSA_NOALLOC_SCRATCH_BYTES bytes instead, one per GPU (the calling
 * thread's current device; `stream` must belong to it), held until the
 * process ends.  The call allocates and frees nothing.
 *   - A call whose split-k partials need more than DSA_NOALLOC_SCRATCH_BYTES
 *     (dsa_sparse_attn_workspace_size() of its shape) returns
 *     DSA_ERR_UNSUPPORTED and enqueues nothing.
 *   - Every call on a GPU shares that GPU's array: calls that may overlap
 *     on one GPU (different streams without ordering between them) race and
 *     give undefined results.  Nothing in the array needs to start at zero
 *     (every partial a call reads was written by that call).
 *   - The first call on a device looks up the array's device address
 *     (DSA_ERR_HIP if that fails).
 */
#define DSA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
dsa_status dsa_sparse_attn_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                   int64_t kv_page_stride, int64_t kv_row_stride,
                                   int64_t kv_head_stride, const int32_t* block_table,
                                   const int32_t* idx, int idx_rows, int B, int S_q,
                                   int H_q, int H_kv, int D_qk, int D_v, int page,
                                   int max_pages, int k, float sm_scale, float* out,
                                   float* lse, void* stream);

/*
 * spec_verify -- rejection-sampling verification of drafted chains
 * (section "Rejection sampling and a loss that optimizes acceptance
 * directly": drafts sampled from q are accepted or rejected against p, which
 * preserves p; section "Kimi K3": sum_x min(p, q) is the per-token acceptance
 * probability).  For each sequence b, with p_j = softmax(target row j) and
 * q_j = softmax(draft row j):
 *   for j = 0..G-1: accept d_j iff u_acc(b,j) * q_j(d_j) < p_j(d_j);
 *     on the first rejection emit icdf(norm(max(0, p_j - q_j)), u_smp(b,j))
 *     (p_j if that residual has no mass) and stop with accepted_len = j;
 *   if all G are accepted emit the bonus icdf(p_G, u_smp(b,G)), accepted_len = G.
 * icdf(w, u) = smallest i with sum_{t<=i} w_t > u * sum_t w_t (ascending i).
 *
 * Uniforms: if `uniforms` is non-NULL it is fp32 [B, G+1, 2] in [0,1):
 * [...,0] = u_acc (unused at j = G), [...,1] = u_smp.  Otherwise they are
 * generated in-kernel from Philox4x64-10 (Salmon et al., SC'11) with key
 * (seed, 0) and counter (offset, b, j, stream), stream 0 = u_acc, 1 = u_smp,
 * u = (first 64-bit output >> 40) * 2^-24.
 *
 *   target_logits fp32 [B, G+1, V]   draft_logits fp32 [B, G, V]
 *   draft_tokens  int32 [B, G] in [0, V) (a token outside is clamped into
 *                 the row for the read; its decision is then meaningless)
 *   accepted_len  int32 [B]          emitted int32 [B, G+1] (-1 after the
 *                                    accepted_len+1 emitted tokens)
 *   diag          fp32 [B, G+1, 4] or NULL: p_j(d_j), q_j(d_j), u_acc, u_smp
 *                 as used (NaN where not evaluated)
 * Supported: 1 <= G <= 32, 1 <= V <= 2^20, B*(2G+1) <= 65535.  Any V;
 * rows are read with 16-byte loads when V % 4 == 0 and the bases are aligned.
 * Schedule: batches with at least 1 GiB of logits stop reading a sequence's
 * rows after its first rejection (one launch per early position); smaller
 * ones read every row once.  The environment variable DSA_VERIFY_SCHEDULE
 * ("phased" or "onepass") overrides the choice, for tests and tuning; both
 * give the same decisions up to float32 rounding of the softmax statistics.
 * spec_verify_greedy follows the same rule over its target rows.
 */
size_t spec_verify_workspace_size(int B, int G, int V);
dsa_status spec_verify(const float* target_logits, const float* draft_logits,
                       const int32_t* draft_tokens, int B, int G, int V,
                       const float* uniforms, uint64_t seed, uint64_t offset,
                       int32_t* accepted_len, int32_t* emitted, float* diag,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * spec_verify_greedy -- greedy verification of drafted chains, the
 * alternative that section "Rejection sampling and a loss that optimizes
 * acceptance directly" contrasts with sampling (greedy drafts are brittle
 * when the target distribution is flat).  For each sequence b:
 *   for j = 0..G-1: accept d_j iff d_j == argmax_v target_logits[b, j, v];
 *     on the first mismatch emit that argmax and stop with accepted_len = j;
 *   if all G are accepted emit argmax of target row G, accepted_len = G.
 * argmax ties go to the lower token id (-0.0 == +0.0); NaN logits are
 * outside the domain; a row of -inf only yields token 0.  Only the target
 * rows are read, once.
 *
 *   target_logits fp32 [B, G+1, V]   draft_tokens int32 [B, G]
 *   accepted_len  int32 [B]          emitted int32 [B, G+1] (-1 padded)
 * workspace: spec_verify_greedy_workspace_size() bytes, no initialisation.
 * Supported: 1 <= G <= 32, 1 <= V <= 2^20, B*(G+1) <= 65535.
 */
size_t spec_verify_greedy_workspace_size(int B, int G, int V);
dsa_status spec_verify_greedy(const float* target_logits, const int32_t* draft_tokens,
                              int B, int G, int V, int32_t* accepted_len,
                              int32_t* emitted, void* workspace,
                              size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */

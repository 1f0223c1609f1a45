/*
 * focus.h - C ABI of the Focus inference path on AMD Instinct MI355X (gfx950).
 *
 * Focus ("Why Attend to Everything? Focus is the Key", arXiv 2604.03260) gates causal
 * attention with K learned centroids: hidden states are projected into a small group space,
 * scored against the centroids, balanced with Sinkhorn normalisation and given hard top-k
 * group membership; query i then attends key j <= i only if |i - j| < window or the two
 * tokens share at least one group, with an exact softmax over the allowed pairs.
 *
 * Pages cited below:
 *   (ZH)  "Why Attend to Everything? Focus is the Key", Chinese technical summary
 *         (gist.science/zh), sections 2.1.1 token grouping, 2.1.2 gated attention,
 *         2.1.3 top-k inference.
 *   (NL)  Same title, Dutch technical summary (gist.science/nl), "Kerncomponenten" 1-4,
 *         "Resultaten".
 *   (ABS) Same title, English abstract (arxivdaily.com).
 *
 * Conventions shared by every entry point
 *   - Pointers named as device buffers are device memory of the current HIP device, owned by
 *     the caller; the library never allocates, frees or retains them and keeps no state
 *     between calls. Scratch memory comes from the caller as `workspace`, sized by the
 *     matching *_workspace_size query (focus_decode_noalloc alone uses a fixed scratch array
 *     inside the library instead; see there).
 *   - bf16 tensors, the fp32 inputs of focus_assign and every workspace must be 16-byte
 *     aligned; int32 buffers and fp32 lse / col_potential outputs 4-byte aligned (else
 *     FOCUS_ERR_ALIGN). Tensors are dense and row-major in the shapes given. bf16 tensors are
 *     passed as uint16_t bit patterns.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and the call
 *     returns without waiting. Inputs are never written (focus_slots_append updates the
 *     membership rows it is given in place). Calls are re-entrant; two calls that share a
 *     workspace, or rows being appended to, must not overlap in time.
 *   - Arguments are validated on the host before anything is enqueued; an invalid call
 *     returns a negative status and enqueues nothing. A failed launch returns FOCUS_ERR_HIP.
 *     No C++ exception crosses this interface.
 *   - Index tensors are int32: n * top_k (tokens times memberships) must be below 2^31.
 */
#ifndef FOCUS_H
#define FOCUS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum focus_status {
  FOCUS_OK = 0,
  FOCUS_ERR_ARG = -1,          /* NULL pointer or out-of-range scalar argument          */
  FOCUS_ERR_SHAPE = -2,        /* sizes that overflow the int32 index space              */
  FOCUS_ERR_UNSUPPORTED = -3,  /* a valid shape this build has no kernel for             */
  FOCUS_ERR_ALIGN = -4,        /* a device pointer that is not 16-byte aligned           */
  FOCUS_ERR_WORKSPACE = -5,    /* workspace NULL or smaller than the size query returns  */
  FOCUS_ERR_HIP = -6,          /* the HIP runtime reported an error while enqueueing     */
  FOCUS_ERR_SCRATCH = -7       /* needs more scratch than focus_decode_noalloc holds     */
};

/* Human-readable name of a status code (static storage, never NULL). */
const char* focus_status_string(int status);

/* Library version as major * 10000 + minor * 100 + patch. */
int focus_version(void);

/* ------------------------------------------------------------------------------------
 * focus_assign - centroid group assignment (ZH 2.1.1 and 2.1.3; NL Kerncomponenten 1, 2, 4).
 *
 *   S = (hidden * w_g) * centroids^T                     scores, [n, K], fp32 arithmetic
 *       (products at fp32-level accuracy: fp32 operands split exactly into two fp16 parts,
 *       three part products on the matrix cores; a row holding a hidden value beyond fp16's
 *       largest finite value, 65504, has its scores recomputed with fp32 FMAs)
 *   repeat sinkhorn_iters times (log domain, unit temperature, u = v = 0 at the start):
 *     u_i = -logsumexp_c (S_ic + v_c)                    every token carries mass 1
 *     v_c = log(n / K) - logsumexp_i (S_ic + u_i)        every group receives mass n / K
 *   groups[i] = the top_k groups c with the largest S_ic + v_c (equal scores: lower c first),
 *               written in ascending group order.
 *
 *   hidden        device, [n, d] fp32, d % 4 == 0.
 *   w_g           device, [d, d_g] fp32 projection into group space, d_g % 4 == 0.
 *   centroids     device, [K, d_g] fp32.
 *   n             tokens, n >= 0 (n == 0: nothing is enqueued, outputs untouched).
 *   d, d_g        1 <= d, 1 <= d_g <= 1024.
 *   K             number of groups, 1 <= K <= 1024.
 *   top_k         memberships per token, 1 <= top_k <= min(K, 8).
 *   sinkhorn_iters  >= 0; 0 ranks the raw scores.
 *   groups        device, out [n, top_k] int32, distinct group ids in [0, K), ascending.
 *   col_potential device, out [K] fp32, the column potential v after the last iteration;
 *                 may be NULL.
 *   workspace     device scratch of at least focus_assign_workspace_size(n, d, d_g, K) bytes.
 * ------------------------------------------------------------------------------------ */
size_t focus_assign_workspace_size(int64_t n, int d, int d_g, int K);
int focus_assign(const float* hidden, const float* w_g, const float* centroids,
                 int64_t n, int d, int d_g, int K, int top_k, int sinkhorn_iters,
                 int32_t* groups, float* col_potential,
                 void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------
 * focus_bucket - stable counting sort of memberships into per-group segments
 * (the membership sets of ZH 2.1.3, laid out so each group's tokens are contiguous).
 *
 * For each of `batch` independent sequences of n tokens:
 *   offsets[b, c]  = number of memberships with a group id below c (offsets[b, K] = total),
 *   idx[b, s]      = token position of membership slot s; inside every segment
 *                    [offsets[b,c], offsets[b,c+1]) positions are strictly ascending,
 *   slot[b, i, r]  = the slot s holding membership (i, groups[b, i, r]).
 * A membership whose group id lies outside [0, K) is dropped: its slot is -1 and it appears
 * in no segment. Group ids of one token must be distinct.
 *
 *   groups   device, [batch, n, top_k] int32.
 *   batch    >= 1; n >= 0; 1 <= K <= 1024; 1 <= top_k <= 8.
 *   offsets  device, out [batch, K + 1] int32.
 *   idx      device, out [batch, n * top_k] int32 (entries past offsets[b, K] are -1).
 *   slot     device, out [batch, n, top_k] int32.
 *   workspace  at least focus_bucket_workspace_size(batch, n, K, top_k) bytes.
 * ------------------------------------------------------------------------------------ */
size_t focus_bucket_workspace_size(int batch, int64_t n, int K, int top_k);
int focus_bucket(const int32_t* groups, int batch, int64_t n, int K, int top_k,
                 int32_t* offsets, int32_t* idx, int32_t* slot,
                 void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------
 * focus_bucket_append - one decode step of membership maintenance: token p = cache_len[b] - 1
 * of every sequence joins the bucketed memberships of tokens 0 .. p - 1 (ZH 2.1.3: it joins
 * its top-k groups). Its position is the largest so far, so each of its memberships goes at the
 * end of its group's segment and every segment stays ascending. Given
 *   offsets_in, idx_in = focus_bucket of tokens 0 .. p - 1 (batch layout [B, K+1], [B, Lmax*top_k]),
 * it writes offsets_out, idx_out = focus_bucket of tokens 0 .. p, i.e. what focus_decode reads
 * as cache_offsets / cache_idx; entries of idx_out past offsets_out[b, K] are left unspecified.
 * Cost: one copy of the index lists (O(p * top_k) bytes per sequence), no sort.
 *
 *   new_groups  device, [B, top_k] int32: the new tokens' groups (ids outside [0, K) dropped).
 *   cache_len   device, [B] int32 in [0, Lmax]: lengths including the new token (0: nothing
 *               is appended for that sequence).
 *   B >= 1, Lmax >= 1, 1 <= K <= 1024, 1 <= top_k <= 8.
 *   offsets_in, idx_in     device, [B, K+1] and [B, Lmax*top_k] int32.
 *   offsets_out, idx_out   device, same shapes; must not alias the inputs.
 * Asynchronous on `stream`. The previous state's slot array (focus_bucket's third output) is not
 * maintained; focus_decode does not read it.
 * ------------------------------------------------------------------------------------ */
int focus_bucket_append(const int32_t* new_groups, const int32_t* cache_len, int batch,
                        int64_t Lmax, int K, int top_k, const int32_t* offsets_in,
                        const int32_t* idx_in, int32_t* offsets_out, int32_t* idx_out,
                        void* stream);

/* ------------------------------------------------------------------------------------
 * focus_attention - gated sparse causal attention for one sequence
 * (ZH 2.1.2 and 2.1.3; NL Kerncomponenten 3; ABS).
 *
 *   allowed(i, j) = j <= i and (i - j < window or groups[i] and groups[j] share a group)
 *   out[i, h]  = sum over allowed j of softmax_j(scale * q[i,h] . k[j,h/G]) * v[j,h/G]
 *   lse[i, h]  = natural log of sum over allowed j of exp(scale * q[i,h] . k[j,h/G])
 * with G = Hq / Hkv (query head h reads kv head h / G). Every allowed pair is counted once:
 * the kernels split the pairs into the window (i - j < window) and, for far pairs, the
 * lowest group the two tokens share, and merge the parts by their log-sum-exp.
 *
 *   q        device, [n, Hq, d_head] bf16;  k, v  device, [n, Hkv, d_head] bf16.
 *   n        >= 0 (0: nothing enqueued). Hq % Hkv == 0 and G in {1, 2, 4, 8, 16}.
 *   d_head   64 or 128.
 *   groups   device, [n, top_k] int32, ascending distinct ids in [0, K) (focus_assign output).
 *   offsets, idx, slot   device, focus_bucket output for these groups (batch 1).
 *   K        1 <= K <= 1024; top_k 1 <= top_k <= min(K, 4).
 *   window   >= 0 (0: only pairs that share a group, the diagonal included).
 *   scale    > 0, or <= 0 for 1 / sqrt(d_head).
 *   out      device, out [n, Hq, d_head] bf16.
 *   lse      device, out [n, Hq] fp32.
 *   workspace  at least focus_attention_workspace_size(n, Hq, Hkv, d_head, K, top_k) bytes.
 * Range: the group parts are kept in fp16 between the two passes. Each is a softmax-weighted
 * average of v rows, so its entries are bounded by max |v|; v entries must stay below 65504 in
 * magnitude (the largest fp16 value), else the merged output overflows.
 * ------------------------------------------------------------------------------------ */
size_t focus_attention_workspace_size(int64_t n, int Hq, int Hkv, int d_head, int K, int top_k);
int focus_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                    int64_t n, int Hq, int Hkv, int d_head,
                    const int32_t* groups, const int32_t* offsets, const int32_t* idx,
                    const int32_t* slot, int K, int top_k, int64_t window, float scale,
                    uint16_t* out, float* lse,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Same as focus_attention, and in addition records caller-created hipEvent_t handles on
 * `stream` around each of its four kernels, for benchmarks that time one stage:
 * stage_events[2 s] just before and stage_events[2 s + 1] just after stage s, with
 * s = 0 gather of K/V and per-membership key records into group segments, 1 tile prefix,
 * 2 group attention, 3 window attention (whose epilogue merges the group partials by
 * log-sum-exp and writes out/lse in token order). NULL entries are skipped; num_events is
 * the length of the array (0 to 8). Event-record failures return FOCUS_ERR_HIP. */
int focus_attention_ex(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       int64_t n, int Hq, int Hkv, int d_head,
                       const int32_t* groups, const int32_t* offsets, const int32_t* idx,
                       const int32_t* slot, int K, int top_k, int64_t window, float scale,
                       uint16_t* out, float* lse,
                       void* workspace, size_t workspace_bytes, void* stream,
                       void* const* stage_events, int num_events);

/* ------------------------------------------------------------------------------------
 * focus_attention_asym - the asymmetric top-k reading of top-k inference (Dutch summary,
 * Resultaten, "Inferentie": each token looks at 2 of the 4 groups for a 2x speed-up; Chinese
 * summary, section 4 table, top-k trade-off). Every token sits, as a key, in one group k_group
 * (its top-1: focus_assign with top_k 1) and looks, as a query, at its top_k groups q_groups
 * (focus_assign with top_k):
 *
 *   allowed(i, j) = j <= i and (i - j < window or k_group[j] is one of q_groups[i])
 *
 * and out / lse are as for focus_attention over that pair set. A far pair meets exactly one of
 * the query's memberships (the key has one group), so no ownership rule is needed; the window
 * pass merges the top_k group parts by log-sum-exp as in focus_attention.
 *
 *   q, k, v, n, Hq, Hkv, d_head, K, window, scale, out, lse   as for focus_attention
 *            (window 0 with k_group[i] not among q_groups[i] leaves row i with no pairs:
 *            lse -inf, out 0).
 *   q_offsets, q_idx, q_slot   device, focus_bucket output for q_groups [n, top_k] (batch 1).
 *   top_k    1 <= top_k <= min(K, 4), groups each query looks at.
 *   k_offsets, k_idx, k_slot   device, focus_bucket output for k_group [n, 1] (batch 1).
 *   workspace  at least focus_attention_asym_workspace_size(n, Hq, Hkv, d_head, K, top_k)
 *            bytes. Errors and the range of v as for focus_attention; asynchronous on `stream`.
 * ------------------------------------------------------------------------------------ */
size_t focus_attention_asym_workspace_size(int64_t n, int Hq, int Hkv, int d_head, int K,
                                           int top_k);
int focus_attention_asym(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         int64_t n, int Hq, int Hkv, int d_head,
                         const int32_t* q_offsets, const int32_t* q_idx, const int32_t* q_slot,
                         int top_k,
                         const int32_t* k_offsets, const int32_t* k_idx, const int32_t* k_slot,
                         int K, int64_t window, float scale, uint16_t* out, float* lse,
                         void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------
 * focus_soft_attention - the training-time soft gate (ZH 2.1.2 gate formula), forward only:
 * exact softmax over every causal pair, with far pairs' weights multiplied by the gate
 * sigmoid(lambda * a_ij):
 *
 *   a_ij       = [groups[i] and groups[j] share a group] - 1/2
 *   logit_ij   = scale * q[i,h] . k[j,h/G] + (i - j < window ? 0 : log sigmoid(lambda * a_ij))
 *   out[i, h]  = sum over j <= i of softmax_j(logit_ij) * v[j,h/G]
 *   lse[i, h]  = natural log of sum over j <= i of exp(logit_ij)
 *
 * (the printed form multiplies the logit itself by the gate, which does not approach the hard
 * mask as lambda grows; this reading does, and reduces to focus_attention's pair rule in the
 * limit). Dense causal cost: every pair j <= i is computed.
 *
 *   q, k, v, n, Hq, Hkv, d_head, scale, out, lse   as for focus_attention.
 *   groups   device, [n, top_k] int32; ids outside [0, K) never match.
 *   K        1 <= K <= 1024; top_k 1 <= top_k <= min(K, 4).
 *   window   >= 0.
 *   lambda   finite gate sharpness.
 * Needs no workspace. Asynchronous on `stream`.
 * ------------------------------------------------------------------------------------ */
int focus_soft_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         int64_t n, int Hq, int Hkv, int d_head,
                         const int32_t* groups, int K, int top_k, int64_t window, float lambda,
                         float scale, uint16_t* out, float* lse, void* stream);

/* ------------------------------------------------------------------------------------
 * Soft-gated training: the forward over every causal pair and the backward that trains only
 * the centroids and the projection (Dutch technical summary, Kerncomponenten 1, 2 and 4: the
 * soft assignment g_i, Sinkhorn balancing during training, soft gates on every pair; Chinese
 * technical summary, section 2.1.2 gate formula and section 2.2: only the centroids and the
 * projection are trained, the model stays frozen).
 *
 *   S = (hidden * w_g) * centroids^T; T = sinkhorn_iters log-domain Sinkhorn iterations as in
 *   focus_assign; g = exp(S + u + v) (the balanced plan, one row per token; T = 0: g = exp(S))
 *   a_ij       = g_i . g_j - 1/2                                  (group affinity)
 *   logit_ij   = scale * q[i,h] . k[j,h/G] + (i - j >= window ? log sigmoid(lambda * a_ij) : 0)
 *   out[i, h]  = sum over j <= i of softmax_j(logit_ij) * v[j,h/G];   lse as in focus_attention
 *
 * focus_soft_train_forward writes out and lse. focus_soft_train_backward takes them with the
 * upstream gradient dout = dL/dout and writes dL/dcentroids, dL/dw_g and, when d_hidden is not
 * NULL, dL/dhidden (q, k, v are inputs of the frozen model: no gradient). With one-hot rows g,
 * a_ij is the shared-group indicator minus 1/2 and the forward is focus_soft_attention's.
 *
 *   hidden, w_g, centroids, n, d, d_g, K, sinkhorn_iters   as for focus_assign, with
 *            K <= 128 (FOCUS_ERR_UNSUPPORTED above) and sinkhorn_iters <= 64.
 *   q, k, v, Hq, Hkv, d_head, scale, out, lse   as for focus_attention (out bf16 [n, Hq, d_head],
 *            lse fp32 [n, Hq]).
 *   window   >= 0: pairs with i - j < window carry no gate.
 *   lambda   finite gate sharpness.
 *   dout     device, [n, Hq, d_head] bf16.
 *   d_centroids  device, out [K, d_g] fp32;  d_w_g  device, out [d, d_g] fp32;
 *   d_hidden     device, out [n, d] fp32, or NULL.
 *   workspace    at least focus_soft_train_workspace_size(n, d, d_g, K, Hq, sinkhorn_iters)
 *            bytes (the same size serves both calls).
 * The gradients are accumulated with atomic adds, so their last bits may differ between runs.
 * Dense causal cost: every pair j <= i is computed (the backward visits only far pairs).
 * ------------------------------------------------------------------------------------ */
size_t focus_soft_train_workspace_size(int64_t n, int d, int d_g, int K, int Hq,
                                       int sinkhorn_iters);
int focus_soft_train_forward(const float* hidden, const float* w_g, const float* centroids,
                             int64_t n, int d, int d_g, int K, int sinkhorn_iters,
                             const uint16_t* q, const uint16_t* k, const uint16_t* v, int Hq,
                             int Hkv, int d_head, int64_t window, float lambda, float scale,
                             uint16_t* out, float* lse, void* workspace, size_t workspace_bytes,
                             void* stream);
int focus_soft_train_backward(const float* hidden, const float* w_g, const float* centroids,
                              int64_t n, int d, int d_g, int K, int sinkhorn_iters,
                              const uint16_t* q, const uint16_t* k, const uint16_t* v, int Hq,
                              int Hkv, int d_head, int64_t window, float lambda, float scale,
                              const uint16_t* out, const float* lse, const uint16_t* dout,
                              float* d_centroids, float* d_w_g, float* d_hidden, void* workspace,
                              size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------
 * focus_decode - one new token per sequence against its own cache (ZH 2.1.3 inference).
 *
 * Sequence b holds L_b = cache_len[b] tokens; its new token is the last one, at position
 * L_b - 1, whose K/V the caller has already written to the caches. The query carries the
 * groups q_groups[b] and attends key j <= L_b - 1 when L_b - 1 - j < window or when
 * cache_groups[b, j] shares a group with q_groups[b]; the new token always attends itself.
 * Results equal the last row of focus_attention over that sequence with groups[L_b - 1]
 * replaced by q_groups[b].
 *
 *   q            device, [B, Hq, d_head] bf16.
 *   q_groups     device, [B, top_k] int32; an id outside [0, K) matches no key and a repeated
 *                id counts once.
 *   k_cache, v_cache   device, [B, Lmax, Hkv, d_head] bf16.
 *   cache_len    device, [B] int32, 1 <= cache_len[b] <= Lmax (values outside are clamped).
 *   cache_groups device, [B, Lmax, top_k] int32.
 *   cache_offsets, cache_idx   device, focus_bucket output over cache_groups with
 *                batch = B and n = Lmax ([B, K + 1] and [B, Lmax * top_k]); tokens at
 *                positions >= cache_len[b] are ignored.
 *   B >= 0, Lmax >= 1, Lmax * top_k < 2^31; head, K and top_k limits as focus_attention.
 *   out          device, out [B, Hq, d_head] bf16;  lse  device, out [B, Hq] fp32.
 *   workspace    at least focus_decode_workspace_size(B, Lmax, Hq, Hkv, d_head, K, top_k).
 * ------------------------------------------------------------------------------------ */
size_t focus_decode_workspace_size(int B, int64_t Lmax, int Hq, int Hkv, int d_head, int K,
                                   int top_k);
int focus_decode(const uint16_t* q, const int32_t* q_groups,
                 const uint16_t* k_cache, const uint16_t* v_cache, const int32_t* cache_len,
                 const int32_t* cache_groups, const int32_t* cache_offsets,
                 const int32_t* cache_idx, int B, int64_t Lmax, int Hq, int Hkv, int d_head,
                 int K, int top_k, int64_t window, float scale,
                 uint16_t* out, float* lse,
                 void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------
 * focus_decode_noalloc - focus_decode for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, and harnesses that forbid hipMalloc.
 *
 * Same arguments, checks, results and kernels as focus_decode, without the workspace: the
 * scratch space lives in a fixed device array inside the library, one copy per GPU, of
 * focus_decode_noalloc_scratch_bytes() bytes (64 MiB), held until the process ends. The call
 * allocates and frees nothing. A call whose focus_decode_workspace_size(B, Lmax, Hq, Hkv,
 * d_head, K, top_k) exceeds that size returns FOCUS_ERR_SCRATCH and enqueues nothing (the
 * 64 x 65536-token decode with 32 query heads and d_head 128 needs about 8.5 MB; up to 2048
 * such sequences fit).
 * The first call on a device looks up that device's copy (FOCUS_ERR_HIP if the lookup fails).
 *
 * Every call on one GPU shares that GPU's scratch, and each call rewrites what it reads, so
 * calls need nothing cleared between them; but two calls that overlap in time on one GPU
 * (different streams, or host threads) race on the scratch and must be serialised by the
 * caller. Results are identical to focus_decode's on the same inputs.
 * ------------------------------------------------------------------------------------ */
size_t focus_decode_noalloc_scratch_bytes(void);
int focus_decode_noalloc(const uint16_t* q, const int32_t* q_groups,
                         const uint16_t* k_cache, const uint16_t* v_cache,
                         const int32_t* cache_len, const int32_t* cache_groups,
                         const int32_t* cache_offsets, const int32_t* cache_idx, int B,
                         int64_t Lmax, int Hq, int Hkv, int d_head, int K, int top_k,
                         int64_t window, float scale, uint16_t* out, float* lse, void* stream);

/* ------------------------------------------------------------------------------------
 * focus_decode_paged - focus_decode over a paged KV cache (the paged cache that goes with
 * incremental decode; Chinese summary, section 2.1.3 inference). The K/V rows of all
 * sequences live in one pool of fixed-size pages; each sequence lists its pages in order.
 * Position p of sequence b is pool row page_table[b, p / page_size] * page_size +
 * p % page_size. Results equal focus_decode on the caches the pages spell out (same keys,
 * same order, same arithmetic).
 *
 *   k_pages, v_pages  device, [num_pages, page_size, Hkv, d_head] bf16.
 *   num_pages >= 1, page_size >= 1, num_pages * page_size <= 2^31 (pool rows are int32).
 *   page_table   device, [B, pages_per_seq] int32 page ids. Only the pages that hold
 *                positions < cache_len[b] are read; keys on an entry outside
 *                [0, num_pages) are skipped (never read).
 *   pages_per_seq >= 1; Lmax = pages_per_seq * page_size is the logical capacity:
 *                cache_groups [B, Lmax, top_k], cache_offsets / cache_idx from focus_bucket
 *                over them (batch B, n = Lmax), cache_len[b] <= Lmax.
 *   Other arguments, limits, workspace (focus_decode_workspace_size(B, Lmax, ...)) and
 *   errors as for focus_decode.
 * ------------------------------------------------------------------------------------ */
int focus_decode_paged(const uint16_t* q, const int32_t* q_groups,
                       const uint16_t* k_pages, const uint16_t* v_pages,
                       int64_t num_pages, int page_size,
                       const int32_t* page_table, int64_t pages_per_seq,
                       const int32_t* cache_len, const int32_t* cache_groups,
                       const int32_t* cache_offsets, const int32_t* cache_idx,
                       int B, int Hq, int Hkv, int d_head, int K, int top_k,
                       int64_t window, float scale, uint16_t* out, float* lse,
                       void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------
 * Group-slotted cache memberships: an O(top_k) append per generated token (incremental
 * decode, Chinese summary, section 2.1.3 inference: a new token joins its groups and attends
 * their members). Each (sequence, group) owns a row of group_cap slots:
 *
 *   seg_len  device, [B, K] int32: members of group g of sequence b in use.
 *   seg_pos  device, [B, K, group_cap] int32: their positions, ascending, in
 *            seg_pos[b, g, 0 .. seg_len[b, g] - 1] (later slots unused).
 *   overflow device, one int32 the calls set to 1 (never clear) when a group would need more
 *            than group_cap slots; the members that do not fit are not stored, so the rows
 *            must then be rebuilt with a larger capacity. The caller zeroes it.
 *
 * group_cap >= 1 and K * group_cap < 2^31. Asynchronous on `stream`.
 *
 * focus_slots_from_bucket fills the rows from focus_bucket output over cache_groups
 * [B, Lmax, top_k] (offsets [B, K + 1], idx [B, Lmax * top_k]); batch <= 65535.
 *
 * focus_slots_append adds position cache_len[b] - 1 (the newest token of sequence b, larger
 * than every stored position) to the rows of its groups new_groups[b, 0 .. top_k - 1], in
 * place: one write per membership. Ids outside [0, K) are dropped and a repeated id joins
 * once; sequences with cache_len[b] < 1 are left alone.
 *
 * focus_decode_slots is focus_decode_paged with the cache memberships read from the rows
 * instead of a bucket; the results equal focus_decode_paged's on the same memberships.
 *   group_cap <= Lmax is not required; cache_groups [B, Lmax, top_k] is still read for the
 *   ownership rule. Other arguments, limits, workspace and errors as for focus_decode_paged.
 * ------------------------------------------------------------------------------------ */
int focus_slots_from_bucket(const int32_t* offsets, const int32_t* idx, int batch, int64_t Lmax,
                            int K, int top_k, int group_cap, int32_t* seg_len, int32_t* seg_pos,
                            int32_t* overflow, void* stream);
int focus_slots_append(const int32_t* new_groups, const int32_t* cache_len, int batch, int K,
                       int top_k, int group_cap, int32_t* seg_len, int32_t* seg_pos,
                       int32_t* overflow, void* stream);
int focus_decode_slots(const uint16_t* q, const int32_t* q_groups,
                       const uint16_t* k_pages, const uint16_t* v_pages,
                       int64_t num_pages, int page_size,
                       const int32_t* page_table, int64_t pages_per_seq,
                       const int32_t* cache_len, const int32_t* cache_groups,
                       const int32_t* seg_len, const int32_t* seg_pos, int group_cap,
                       int B, int Hq, int Hkv, int d_head, int K, int top_k,
                       int64_t window, float scale, uint16_t* out, float* lse,
                       void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FOCUS_H */

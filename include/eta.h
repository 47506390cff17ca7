/*
 * eta.h -- C ABI of the MI355X (gfx950) block-sparse decode library, libeta.so.
 *
 * The library implements the inference-time decode path of Elastic Threshold
 * Attention (paper: "Elastic Threshold Attention: Learned Contextual Sparsity
 * for Long-Context Decoding"; method as summarised on the picx.dev page,
 * Methodology sections 1-4).  One decode step for a batch of sequences is:
 *
 *   eta_append_kv        write the new token's k, v; statistics of a block
 *                        that this token completes                 (Meth. 4)
 *   eta_predict_tau      per-head threshold, linear in the query or frozen
 *                                                                   (Eq. 1)
 *   eta_screen           per-block upper bound vs. threshold, compacted list
 *                        of admitted blocks, admitted-token counter (Eq. 5)
 *   eta_decode           exact softmax attention over the admitted blocks only,
 *                        split over chunks of blocks, log-sum-exp combine
 *                                                        (Eq. 3, Fig. 6)
 *
 * plus eta_build_block_meta (statistics of many blocks, e.g. after prefill),
 * eta_dense_decode (the same kernels over every key: plain dense decode),
 * eta_calibrate_threshold (per-head constants for a target density) and the
 * grouped-query forms eta_screen_gqa / eta_decode_gqa / eta_dense_decode_gqa
 * (several query heads per KV head, one read of each union block), and
 * eta_gated_prefill (the gated causal attention forward over whole
 * sequences, with the density term of the sparsity loss).
 *
 * Conventions shared by every call
 *   - Every function returns eta_status; ETA_OK is 0.  All arguments are
 *     validated on the host before any HIP call; on error nothing is launched
 *     and eta_last_error() (thread-local) describes the first bad argument.
 *   - Ownership: the caller allocates, owns and frees every buffer.  Device
 *     pointers are hipMalloc'ed (or equivalent) device memory; the library
 *     allocates nothing, keeps no state between calls and never synchronises.
 *   - Streams: `stream` is a hipStream_t passed as void* (NULL: the null
 *     stream).  Every call only enqueues kernels on that stream; results are
 *     ready when the stream reaches them.  Two calls that write the same
 *     buffers must not run concurrently on different streams.
 *   - Types: q, tau, maxnorm and outputs are float32; the block statistics
 *     mu and var are stored as bfloat16 (see eta_cache).  The K/V cache is
 *     float32 (ETA_DT_F32) or bfloat16 (ETA_DT_BF16); bf16 is widened exactly
 *     to float32 and every accumulation is float32 (float64 for mu and var
 *     before their rounding).
 *   - Supported shapes: head_dim in {64, 128}; block in {4, 8, 16, 32, 64,
 *     128}.  Smaller head dimensions run zero-padded to 64 with `scale` given
 *     explicitly (zero coordinates change no dot product, norm or variance).
 *   - batch == 0 or heads == 0 is an empty problem: OK, nothing launched.
 */
#ifndef ETA_H_
#define ETA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ETA_ABI_VERSION 4

typedef int32_t eta_status;
enum {
  ETA_OK = 0,
  ETA_ERR_NULL_PTR = 1,  /* a required pointer is NULL                        */
  ETA_ERR_BAD_SHAPE = 2, /* unsupported head_dim/block, negative sizes, ...   */
  ETA_ERR_BAD_ARG = 3,   /* NaN or out-of-range scalar, unknown mode/dtype    */
  ETA_ERR_CAPACITY = 4,  /* a size exceeds the cache or index capacity        */
  ETA_ERR_WORKSPACE = 5, /* workspace NULL or smaller than the size query     */
  ETA_ERR_HIP = 6        /* a HIP launch or runtime call failed               */
};

enum { ETA_DT_F32 = 0, ETA_DT_BF16 = 1 };
enum { ETA_LOGIT_GATED = 0, ETA_LOGIT_RAW = 1 };

/*
 * The KV cache of one attention layer (Methodology 4: the cache is split into
 * contiguous blocks of `block` keys, and each complete block keeps its centroid
 * mu, per-coordinate population variance var and largest key norm maxnorm).
 *
 *   k, v      device, [batch][heads][cap_tokens][head_dim], kv_dtype elements
 *   mu, var   device, [batch][heads][cap_blocks][head_dim] bfloat16 (bit
 *             patterns): the block mean and population variance, computed in
 *             float64 and rounded to the nearest bfloat16 (ties to even), so
 *             the screen reads 4 bytes per coordinate instead of 8
 *   maxnorm   device, [batch][heads][cap_blocks] float32
 *   seq_len   device, [batch] int32: current length T_b of sequence b
 *             (ragged batches allowed, 0 <= T_b <= cap_tokens)
 *
 * cap_blocks = ceil(cap_tokens / block).  Statistics exist only for complete
 * blocks j < floor(T_b / block); the partial last block has none.  The
 * struct itself is read on the host during each call and may be a stack
 * object.
 */
typedef struct eta_cache {
  int32_t batch, heads, head_dim, block, cap_tokens, kv_dtype;
  void* k;
  void* v;
  uint16_t* mu;
  uint16_t* var;
  float* maxnorm;
  int32_t* seq_len;
} eta_cache;

int32_t eta_abi_version(void);
const char* eta_status_string(eta_status s);
const char* eta_last_error(void);
/* ceil(cap_tokens / block), the row count of the statistics arrays. */
int32_t eta_cache_blocks(const eta_cache* c);

/*
 * Append one token per sequence (decode step of the paper's Fig. 1 / Fig. 6
 * pipeline): for every (b, h), k_new[b][h][:] and v_new[b][h][:] (device,
 * [batch][heads][head_dim], kv_dtype) are written at position T_b, and when
 * T_b + 1 is a multiple of `block` the statistics of that now-complete block
 * are computed (Methodology 4).  Then T_b += 1.
 * `overflow` (device int32, required) reports the capacity error: T_b is
 * only known on the device, so it cannot be checked on the host.  A sequence
 * already at cap_tokens is left unchanged (its token is not written and T_b
 * keeps its value) and *overflow is set to 1; the flag is never cleared by
 * the library.  After a flagged append the caller must not screen or decode
 * that step: the query's own key (Eq. 3's never-gated diagonal) is missing.
 * overflow == NULL (for a non-empty cache) returns ETA_ERR_NULL_PTR.
 */
eta_status eta_append_kv(const eta_cache* c, const void* k_new, const void* v_new,
                         int32_t* overflow, void* stream);

/*
 * Statistics (mu, var, maxnorm) of blocks first_block .. first_block+n_blocks-1
 * of every (b, h) stream; blocks that are not complete for T_b are skipped.
 * n_blocks = -1 means every block from first_block to cap_blocks-1.  Used once
 * after prefill; the result equals what eta_append_kv computes block by block
 * (same kernel code, same summation order).  Methodology 4 (population
 * centroid, coordinate-wise variance over b keys, max norm).
 */
eta_status eta_build_block_meta(const eta_cache* c, int32_t first_block, int32_t n_blocks,
                                void* stream);

/*
 * Threshold (Methodology 1, Eq. 1).  q: device [batch][heads*head_dim] float32
 * (the concatenated per-head queries qbar).  Dynamic mode (W != NULL): W is
 * device [heads*head_dim][heads] float32, bias_or_c device [heads] and
 *     tau_gate[b][h] = sum_j q[b][j] W[j][h] + bias_or_c[h].
 * Frozen mode (W == NULL): tau_gate[b][h] = bias_or_c[h] (offline-calibrated
 * per-head constants).  Both modes: tau_screen = tau_gate - a (a is the
 * threshold adjustment; 0 leaves them equal).  Outputs device [batch][heads].
 * heads <= 256.  The sum over j runs in a fixed order (deterministic, and
 * shared with eta_fused_step): 256 partial sums, partial t over j = t,
 * t + 256, ... in turn, added by a fixed tree, then the bias.
 */
eta_status eta_predict_tau(int32_t batch, int32_t heads, int32_t head_dim, const float* q,
                           const float* W, const float* bias_or_c, float a, float* tau_gate,
                           float* tau_screen, void* stream);

/*
 * Screen (Methodology 4, Eq. 5).  For every complete block j of stream (b, h):
 *   s_j = scale * min(<q, mu_j> + z sqrt(sum_i q_i^2 var_j,i), ||q||_2 maxnorm_j)
 * (z = +inf: the geometric term alone).  Block j is admitted iff
 * s_j >= tau_screen[b][h]; the last block (the one holding position T_b - 1,
 * complete or not) is always admitted.  Outputs, all device:
 *   active_idx [batch][heads][cap_blocks] int32: admitted block indices of
 *              (b, h), ascending, in the first active_cnt[b][h] entries
 *              (the rest is left unspecified);
 *   active_cnt [batch][heads] int32;
 *   density_ctr (optional, one uint64): += number of admitted tokens summed
 *              over all (b, h) (integer atomics: exact and order-free).
 * q: device [batch][heads][head_dim]; tau_screen: device [batch][heads].
 * Workspace: eta_screen_workspace_bytes(); contents need no initialisation.
 */
size_t eta_screen_workspace_bytes(int32_t batch, int32_t heads, int32_t cap_blocks);
eta_status eta_screen(const eta_cache* c, const float* q, const float* tau_screen, float z,
                      float scale, int32_t* active_idx, int32_t* active_cnt,
                      uint64_t* density_ctr, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * Block-sparse decode (Theoretical Foundation: attention restricted to the
 * admitted set, normalised over it; Methodology 2, Eq. 3 for the logits;
 * Fig. 6: only admitted blocks are loaded, online softmax).  The admitted
 * lists of all streams, taken in (b, h) order, are cut into equal contiguous
 * ranges, min(waves on the device, ceil(N / blocks_per_split)) of them for N
 * admitted blocks, one per wavefront; every (range, stream) piece produces a
 * partial (max, sum, weighted V) and one combine pass merges each stream's
 * partials by log-sum-exp into out [batch][heads][head_dim] float32 (device).
 * Above 8191 streams a one-work-group scan kernel first writes the stream
 * offsets to the workspace.  batch * heads * cap_blocks must be below 2^31
 * (ETA_ERR_BAD_SHAPE).
 * Logits, with S_s = scale <q, k_s>:
 *   ETA_LOGIT_GATED  l_s = S_s sigmoid(beta (S_s - tau_gate[b][h])) for
 *                    s != T_b - 1, and l_{T_b-1} = S_{T_b-1} (the query's own
 *                    key is never gated);
 *   ETA_LOGIT_RAW    l_s = S_s   (tau_gate may be NULL).
 * A stream with T_b == 0 yields zeros.  active_idx/active_cnt are eta_screen's
 * outputs (any ascending list of distinct in-range blocks that contains the
 * last block is valid input).  1 <= blocks_per_split <= 4096.
 * Workspace: eta_decode_workspace_bytes(); contents need no initialisation.
 */
size_t eta_decode_workspace_bytes(int32_t batch, int32_t heads, int32_t head_dim,
                                  int32_t cap_blocks, int32_t blocks_per_split);
eta_status eta_decode(const eta_cache* c, const float* q, const float* tau_gate,
                      const int32_t* active_idx, const int32_t* active_cnt, int32_t logit_mode,
                      float beta, float scale, int32_t blocks_per_split, void* workspace,
                      size_t workspace_bytes, float* out, void* stream);

/*
 * eta_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): no
 * workspace argument, the same kernels and the same results as eta_decode.
 * Its scratch is a static device array of 8 MiB that every device the
 * library runs on holds until the process ends; that covers every call of up
 * to about 13000 streams at head_dim <= 128 (one partial slot per wave and
 * per stream).  A call that would need more returns ETA_ERR_CAPACITY and
 * launches nothing.  All such calls on
 * one device share that array, so calls that overlap in time on one device
 * (two streams, two host threads) race: the caller serialises them.  Nothing
 * in the array needs clearing between calls.
 */
eta_status eta_decode_noalloc(const eta_cache* c, const float* q, const float* tau_gate,
                              const int32_t* active_idx, const int32_t* active_cnt,
                              int32_t logit_mode, float beta, float scale,
                              int32_t blocks_per_split, float* out, void* stream);

/*
 * Dense decode over every key of every stream (Theoretical Foundation, dense
 * form): chunks of blocks_per_split consecutive blocks per stream, one
 * work-group each, with RAW logits and the same log-sum-exp combine.  The
 * in-house dense baseline.  Workspace as for eta_decode.
 */
eta_status eta_dense_decode(const eta_cache* c, const float* q, float scale,
                            int32_t blocks_per_split, void* workspace, size_t workspace_bytes,
                            float* out, void* stream);

/*
 * One decode step -- threshold (Methodology 1, Eq. 1), screen (Methodology
 * 4, Eq. 5) and block-sparse decode (Methodology 2, Eq. 3 logits; Fig. 6:
 * only admitted blocks are loaded, online softmax) -- in two launches, for
 * small steps where the separate calls' launches cost more than their work.
 * Every stream is cut into chunks of blocks_per_chunk consecutive blocks
 * (1 <= blocks_per_chunk <= 32), one work-group each, which computes its
 * stream's thresholds exactly as eta_predict_tau does (the same float32
 * operations in the same order, so the same bits), screens its chunk's blocks
 * exactly as eta_screen does (so the same admitted set, the last block always
 * in it) and attends over the blocks it admitted; a combine pass merges the
 * chunks of each stream by log-sum-exp in chunk order.
 * Inputs: q device [batch][heads][head_dim]; W, bias_or_c and a as for
 * eta_predict_tau (W NULL: frozen constants); z, scale as for eta_screen;
 * logit_mode, beta as for eta_decode.  heads <= 256.
 * Outputs: out [batch][heads][head_dim] float32 as eta_decode's (a stream with
 * T_b == 0 yields zeros); optional (NULL: not written):
 *   tau_gate, tau_screen  device [batch][heads], eta_predict_tau's outputs;
 *   chunk_bits  device [batch][heads][ceil(cap_blocks / blocks_per_chunk)]
 *               uint32: bit i of entry k set iff block k * blocks_per_chunk + i
 *               is admitted (entries of chunks past a stream's end are left
 *               unwritten);
 *   density_ctr one uint64, += admitted tokens as in eta_screen.
 * Workspace: eta_fused_step_workspace_bytes(); contents need no
 * initialisation.
 */
size_t eta_fused_step_workspace_bytes(int32_t batch, int32_t heads, int32_t head_dim,
                                      int32_t cap_blocks, int32_t blocks_per_chunk);
eta_status eta_fused_step(const eta_cache* c, const float* q, const float* W,
                          const float* bias_or_c, float a, float z, int32_t logit_mode,
                          float beta, float scale, int32_t blocks_per_chunk, float* tau_gate,
                          float* tau_screen, uint32_t* chunk_bits, uint64_t* density_ctr,
                          void* workspace, size_t workspace_bytes, float* out, void* stream);

/*
 * Offline calibration of frozen per-head constants (the pages' calibration
 * algorithm freezes per-(layer, head) thresholds; its steps are not given, so
 * this is the plain quantile reading).  For head h, pool over the n_sets
 * query sets q_sets[n] (device [n_sets][batch][heads][head_dim]) and the
 * sequences b the values x = s_j - tau0[n][b][h] of every complete block j
 * except the always-admitted last block (s_j as in eta_screen; tau0 device
 * [n_sets][batch][heads] or NULL for 0).  With F the tokens of the last
 * blocks and sum T the tokens of all streams, k = round((rho sum T - F) /
 * block) clamped to [0, N]; c_out[h] (device [heads] float32) is the midpoint
 * of the k-th and (k+1)-th largest pooled value (-inf when k = N, +inf when
 * k = 0).  Screening with tau_screen = tau0 + c_out then admits the top k.
 * Pooled values per head must not exceed 2^31 - 1.
 */
size_t eta_calibrate_workspace_bytes(int32_t n_sets, int32_t batch, int32_t heads,
                                     int32_t cap_blocks);
eta_status eta_calibrate_threshold(const eta_cache* c, int32_t n_sets, const float* q_sets,
                                   const float* tau0, float z, float scale,
                                   float target_density, void* workspace,
                                   size_t workspace_bytes, float* c_out, void* stream);

/*
 * Grouped-query attention (thelatestinai.com paper page: Table 5's benchmark
 * shape of 32 query heads on 4 KV heads, Fig. 9 union loading vs per-head
 * compute; picx.dev summary, Practical Implications: a block is read when any
 * head of the group admits it).  The cache holds KV heads: c->heads is the
 * KV head count H_kv, and query head h = kv * group + g (0 <= g < group)
 * reads KV head kv.  q is device [batch][H_kv * group][head_dim] float32;
 * thresholds are device [batch][H_kv * group].  1 <= group <= 16.
 *
 * eta_screen_gqa: every query head is screened exactly as eta_screen does
 * against the statistics of its KV head (Eq. 5, own query and own
 * tau_screen; the last block is admitted for every head).  Outputs, device:
 *   head_mask  [batch][H_kv][cap_blocks] uint32: bit g of entry j is set iff
 *              query head kv * group + g admits block j (entries j < n_b,
 *              the block count of sequence b; the rest unspecified);
 *   union_idx  [batch][H_kv][cap_blocks] int32: ascending list of the blocks
 *              admitted by at least one head of the group (the union), in
 *              the first union_cnt[b][kv] entries;
 *   union_cnt  [batch][H_kv] int32;
 *   density_ctr (optional, two uint64): [0] += admitted tokens summed over
 *              query heads (D_head numerator), [1] += union tokens summed
 *              over KV heads (D_union numerator).
 * Workspace: eta_screen_gqa_workspace_bytes(); no initialisation needed.
 */
size_t eta_screen_gqa_workspace_bytes(int32_t batch, int32_t kv_heads, int32_t cap_blocks);
eta_status eta_screen_gqa(const eta_cache* c, int32_t group, const float* q,
                          const float* tau_screen, float z, float scale, int32_t* union_idx,
                          uint32_t* head_mask, int32_t* union_cnt, uint64_t* density_ctr,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Grouped-query block-sparse decode.  Each block of the union list is read
 * once for its whole group; query head kv * group + g attends over the keys of
 * the blocks whose head_mask bit g is set, with the logits of eta_decode
 * (Eq. 3, its own tau_gate; the query's own key is never gated), normalised
 * over its own admitted set.  The union blocks of all streams, taken in
 * order, are cut into min(resident waves, ceil(N / blocks_per_split)) equal
 * ranges, one per wave (N = total union blocks); above 6143 KV streams a
 * one-work-group scan kernel first writes the stream offsets to the
 * workspace.  B * H_kv * cap_blocks must be below 2^31 (ETA_ERR_BAD_SHAPE).
 * Partial results per query head, log-sum-exp combine;
 * out is device
 * [batch][H_kv * group][head_dim] float32, zeros for T_b == 0.
 * Requires kv_dtype == ETA_DT_BF16: the scores and value sums run on the
 * matrix cores as bf16 products with float32 accumulation, the query and the
 * softmax weights each split into two bf16 terms (float32-level accuracy).
 * 1 <= blocks_per_split <= 2048.
 * Workspace: eta_decode_gqa_workspace_bytes(); no initialisation needed.
 */
size_t eta_decode_gqa_workspace_bytes(int32_t batch, int32_t kv_heads, int32_t group,
                                      int32_t head_dim, int32_t cap_blocks,
                                      int32_t blocks_per_split);
eta_status eta_decode_gqa(const eta_cache* c, int32_t group, const float* q,
                          const float* tau_gate, const int32_t* union_idx,
                          const uint32_t* head_mask, const int32_t* union_cnt,
                          int32_t logit_mode, float beta, float scale, int32_t blocks_per_split,
                          void* workspace, size_t workspace_bytes, float* out, void* stream);

/*
 * Grouped-query dense decode: every key of its KV head for every query head,
 * RAW logits, the same kernels as eta_decode_gqa (the dense GQA baseline).
 * Workspace as for eta_decode_gqa.
 */
eta_status eta_dense_decode_gqa(const eta_cache* c, int32_t group, const float* q, float scale,
                                int32_t blocks_per_split, void* workspace,
                                size_t workspace_bytes, float* out, void* stream);

/*
 * Gated causal attention forward over whole sequences: prefill, or the
 * forward pass of training (picx.dev summary, Methodology 2, Eqs. 2-3; and
 * Methodology 3, Eq. 4 for `dens`).  Query head h = kv * group + g reads KV
 * head kv.  For position t (0-based) and keys s <= t, with
 * S_ts = scale <q_t, k_s> and m_ts = sigmoid(beta (S_ts - tau_t)):
 *   out_t  = sum_s softmax_s(l_ts) v_s,  l_ts = S_ts m_ts (s < t), S_tt (s = t)
 *   dens_t = (1 / (t + 1)) sum_{s <= t} m_ts
 * (Eq. 4's term of the layer is lambda / (H T) sum_h sum_t dens_t.)
 *   q     device [batch][kv_heads*group][seq_len][head_dim] bf16
 *   k, v  device [batch][kv_heads][seq_len][head_dim] bf16
 *   tau   device [batch][kv_heads*group][seq_len] float32 (Eq. 1 per position)
 *   out   device [batch][kv_heads*group][seq_len][head_dim] float32
 *   dens  device [batch][kv_heads*group][seq_len] float32, or NULL
 * head_dim in {64, 128}; beta and scale finite and > 0; one K/V stream holds
 * fewer than 2^32 bytes (seq_len * head_dim * 2 < 2^32, else ETA_ERR_BAD_SHAPE).  Both products run
 * on the matrix cores with float32 accumulation; the softmax weights are
 * split into two bf16 terms.  No workspace.
 */
eta_status eta_gated_prefill(int32_t batch, int32_t kv_heads, int32_t group, int32_t seq_len,
                             int32_t head_dim, const void* q, const void* k, const void* v,
                             const float* tau, float beta, float scale, float* out, float* dens,
                             void* stream);

#ifdef __cplusplus
}
#endif
#endif /* ETA_H_ */

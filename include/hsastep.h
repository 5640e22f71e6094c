/*
 * hsastep.h - C ABI of the MI355X (gfx950) HSA denoise-iteration path.
 *
 * Heterogeneous Step Allocation (HSA) gives each token group its own number of
 * denoising steps.  One iteration i of the sampler is:
 *   hsa_active_set        which tokens run the model at iteration i
 *   hsa_select_groups     (once) which group each token belongs to
 *   hsastep_gather_rows   the active tokens' rows, in active order
 *   hsa_kv_update         fresh K/V rows of the active tokens into the per-layer cache
 *   hsa_attention_active  the active queries against all N cached keys/values
 *   hsa_euler_step        cached Euler update of all N latents
 * and, fusing the model's projection with the cache write:
 *   hsa_qkv_project       Q/K/V of the active rows; K/V straight into their cache slots
 * and one measurement utility:
 *   hsastep_mfma_probe    the sustained bf16 MFMA rate the attention kernel runs against
 *
 * Pages that define the operations (cited below by short name):
 *   [HSA-nl] "Technische Samenvatting: Heterogene Staptoewijzing (HSA) voor
 *            Efficiënte Videogeneratie", gist.science/nl/paper/2605.06892
 *            §2.1 Tokenpartitionering en Planning, §2.2 KV-cache Synchronisatie,
 *            §2.3 Gecachete Euler-update, §2.4 Fasebewuste Cachingvenster.
 *
 * Conventions shared by every call
 *   - Pointers are DEVICE pointers unless the name ends in _host.  bf16 data is
 *     passed as uint16_t bit patterns.  All arrays are dense row-major, in the
 *     shapes stated per call, with 16-byte aligned base pointers.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls enqueue work
 *     and return; none synchronises with the device.
 *   - The caller owns every buffer.  The library allocates nothing and keeps no
 *     state between calls (only a per-thread copy of the last error message),
 *     so calls on different streams may run concurrently on disjoint buffers.
 *   - Return value: HSASTEP_OK or a negative code.  Arguments are validated on
 *     the host before anything is enqueued; on a validation error nothing runs.
 *     HSASTEP_ERR_HIP reports a failed launch.  Faults inside a kernel surface
 *     at the caller's next synchronisation.  hsastep_last_error() describes the
 *     most recent failure on the calling thread.
 *   - Outputs must not alias inputs unless stated as in place.
 */
#ifndef HSASTEP_H
#define HSASTEP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HSASTEP_OK 0
#define HSASTEP_ERR_ARG -1         /* invalid argument (pointer, size, budget ...)    */
#define HSASTEP_ERR_UNSUPPORTED -2 /* valid in principle, not built (e.g. head_dim 96) */
#define HSASTEP_ERR_HIP -3         /* a HIP runtime call or kernel launch failed       */
#define HSASTEP_ERR_WORKSPACE -4   /* workspace missing or smaller than required       */

#define HSASTEP_MAX_GROUPS 16      /* K <= 16 token groups                              */
#define HSASTEP_MAX_CHANNELS 256   /* latent channels per token for the score kernel    */

/* Device workspace in bytes needed by hsa_select_groups and hsa_active_set for
 * n_tokens tokens and n_groups groups (either call accepts a workspace of this
 * size; the two calls may share one buffer if they run in stream order). */
size_t hsastep_workspace_bytes(int64_t n_tokens, int32_t n_groups);

/* Static text for a status code. */
const char* hsastep_error_string(int code);

/* Message of the last failure on the calling thread ("" if none). */
const char* hsastep_last_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int hsastep_version(void);

/* |A_i|, computed on the host from the group sizes alone ([HSA-nl] §2.1, §2.4):
 * N if i < m or i >= T - m, else the sum of group_sizes[k] over the groups with
 * i mod (T / budgets[k]) == 0.  Writes it to *n_active_host.  Same validation as
 * hsa_active_set.  No device work. */
int hsastep_n_active(int64_t n_tokens, const int32_t* budgets_host,
                     const int64_t* group_sizes_host, int32_t n_groups, int32_t T, int32_t m,
                     int32_t iter, int64_t* n_active_host);

/*
 * Dynamic Token Selection ([HSA-nl] §2.1; §2 introduction: slower tokens get
 * fewer steps, the baseline group keeps the full schedule).
 *
 * score r_n = ||v_cur[n] - v_prev[n]||_1 / ||v_prev[n]||_1 in fp32, each L1 norm
 * summed as a balanced pairwise tree over the channels (zero-padded to a power
 * of two), IEEE round-to-nearest division; 0/0 gives 0, x/0 gives +inf and a
 * NaN score becomes +inf.  Tokens are then ranked by r, largest first, ties by
 * ascending token index, and ranks [0, n_1) form group 0 (budget T), the next
 * n_2 ranks group 1, and so on.
 *
 *   v_prev, v_cur      [n_tokens, channels] fp32
 *   group_sizes_host   [n_groups] host int64, each >= 0, summing to n_tokens
 *   group_id           [n_tokens] int32 output, values in [0, n_groups)
 *   score_or_null      [n_tokens] fp32 output r, or NULL (r then stays in the workspace)
 *   workspace          device buffer, 16-byte aligned, of at least
 *                      hsastep_workspace_bytes(n_tokens, n_groups) bytes; always
 *                      required (it holds the grouping histograms); its contents
 *                      on entry do not matter and are overwritten
 * Limits: 1 <= n_tokens <= 2^31 - 1, 1 <= channels <= HSASTEP_MAX_CHANNELS,
 *         1 <= n_groups <= HSASTEP_MAX_GROUPS.
 */
int hsa_select_groups(const float* v_prev, const float* v_cur, int64_t n_tokens, int32_t channels,
                      const int64_t* group_sizes_host, int32_t n_groups, int32_t* group_id,
                      float* score_or_null, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * Active set A_i of iteration `iter` ([HSA-nl] §2.1, §2.4): token n is active
 * iff iter < m, or iter >= T - m, or iter mod (T / budgets[group_id[n]]) == 0.
 *
 *   group_id           [n_tokens] int32, values in [0, n_groups), with exactly
 *                      group_sizes_host[k] tokens in group k (as produced by
 *                      hsa_select_groups with the same sizes)
 *   budgets_host       [n_groups] host int32: budgets[0] == T, every budget
 *                      divides T, non-increasing
 *   group_sizes_host   [n_groups] host int64, summing to n_tokens
 *   active_idx         [n_tokens] int32 output: the first |A_i| entries are the
 *                      active token indices in ascending order (= cache slots)
 *   active_pos         [n_tokens] int32 output: position of n in active_idx, or -1
 *   n_active_host      host output |A_i| (closed form, see hsastep_n_active)
 * 0 <= iter < T, 0 <= m.  Tokens whose group_id is out of range are treated as
 * skipped.
 */
int hsa_active_set(const int32_t* group_id, int64_t n_tokens, const int32_t* budgets_host,
                   const int64_t* group_sizes_host, int32_t n_groups, int32_t T, int32_t m,
                   int32_t iter, int32_t* active_idx, int32_t* active_pos, int64_t* n_active_host,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * hsa_active_set fused with the gather of the active tokens' rows of one per-token array
 * ([HSA-nl] §2.2 item 1: only the active tokens enter the model; their latent rows are the
 * model's input), in the same two launches: same arguments, result, validation and errors
 * as hsa_active_set, plus
 *
 *   rows               [n_tokens, row_bytes] device array (e.g. the latent, fp32 [N, C])
 *   row_bytes          a positive multiple of 4 (16 and 16-byte aligned pointers take the
 *                      vector path)
 *   rows_out           [n_tokens, row_bytes] output: rows_out[a] = rows[active_idx[a]] for
 *                      a < |A_i|; rows past |A_i| are not written.  Must not alias rows.
 */
int hsa_active_set_gather(const int32_t* group_id, int64_t n_tokens, const int32_t* budgets_host,
                          const int64_t* group_sizes_host, int32_t n_groups, int32_t T, int32_t m,
                          int32_t iter, int32_t* active_idx, int32_t* active_pos,
                          int64_t* n_active_host, const void* rows, int64_t row_bytes,
                          void* rows_out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * hsa_active_set without a workspace, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, result, validation and errors as hsa_active_set, minus the workspace.  The
 * per-chunk counts live in the library's own device array (one word per 1024 tokens, 64 KB),
 * resident on every device the library runs on until the process ends; its address is looked
 * up on the first call on each device, so make that first call outside a graph capture.
 * Every call on one device shares that array: calls that overlap on one device (other streams,
 * other threads) race and must be ordered by the caller.  Calls allocate nothing and clear
 * nothing (each call writes every count it reads).
 * Limit: n_tokens <= HSASTEP_NOALLOC_MAX_TOKENS, else HSASTEP_ERR_UNSUPPORTED.
 */
#define HSASTEP_NOALLOC_MAX_TOKENS (1 << 24)
int hsa_active_set_noalloc(const int32_t* group_id, int64_t n_tokens,
                           const int32_t* budgets_host, const int64_t* group_sizes_host,
                           int32_t n_groups, int32_t T, int32_t m, int32_t iter,
                           int32_t* active_idx, int32_t* active_pos, int64_t* n_active_host,
                           void* stream);

/*
 * Row gather: dst[a] = src[index[a]] for a < n_rows, rows of row_bytes bytes.
 * Used for the model input of the active tokens (their latent rows) and any
 * per-token state ([HSA-nl] §2.2 item 1: only the active tokens enter the
 * projections).  row_bytes must be a multiple of 4; indices outside
 * [0, n_src_rows) produce a zero row.
 */
int hsastep_gather_rows(void* dst, const void* src, const int32_t* index, int64_t n_rows,
                        int64_t n_src_rows, int64_t row_bytes, void* stream);

/*
 * KV-cache synchronisation ([HSA-nl] §2.2 item 2): the fresh K and V rows of the
 * active tokens overwrite their slots (slot = token index) in one layer's cache;
 * every other slot keeps its stale-but-valid row.
 *
 *   k_cache, v_cache   [batch, n_tokens, heads, head_dim] bf16, in place
 *   k_new, v_new       [batch, n_active, heads, head_dim] bf16, active order
 *   active_idx         [n_active] int32, strictly increasing, in [0, n_tokens)
 * Entries outside [0, n_tokens) are skipped.  heads*head_dim must be a multiple
 * of 8.  n_active == 0 is a no-op.
 */
int hsa_kv_update(uint16_t* k_cache, uint16_t* v_cache, const uint16_t* k_new,
                  const uint16_t* v_new, const int32_t* active_idx, int64_t n_active,
                  int64_t n_tokens, int32_t batch, int32_t heads, int32_t head_dim, void* stream);

/*
 * Full-context attention of the active queries ([HSA-nl] §2.2 items 3-4): per
 * (b, h), O = softmax(Q_A K^T * softmax_scale) V over all n_tokens cache rows,
 * no mask, at O(|A_i| * N) cost.  bf16 inputs, fp32 accumulation and softmax,
 * bf16 output.
 *
 *   q_active           [batch, n_active, heads, head_dim] bf16
 *   k_cache, v_cache   [batch, n_tokens, heads, head_dim] bf16
 *   out                [batch, n_active, heads, head_dim] bf16 output
 * head_dim in {64, 128}; n_tokens >= 1; softmax_scale finite and > 0
 * (1/sqrt(head_dim) in the usual model).  n_active == 0 is a no-op.
 * Deterministic: repeated calls give the same bits, and a query's output does not depend on
 * the other queries of the launch (a launch of any subset of the rows gives the same rows).
 */
int hsa_attention_active(const uint16_t* q_active, const uint16_t* k_cache,
                         const uint16_t* v_cache, uint16_t* out, int64_t n_active,
                         int64_t n_tokens, int32_t batch, int32_t heads, int32_t head_dim,
                         float softmax_scale, void* stream);

/*
 * hsa_attention_active with a caller workspace, for small or ragged active sets ([HSA-nl]
 * §2.2 item 4: the cost is O(|A_i| * N), so iterations with few active tokens launch few
 * query tiles).  Same operation, arguments, layouts and errors as hsa_attention_active, plus:
 *
 *   workspace          device buffer (16-byte aligned) of workspace_bytes bytes, or NULL with
 *                      workspace_bytes == 0 (then it runs exactly as hsa_attention_active);
 *                      contents on entry do not matter; overwritten
 *   workspace_bytes    hsastep_attention_workspace_bytes(...) lets every plan run; a smaller
 *                      buffer limits the plan to what fits
 *
 * With head_dim 128 and n_tokens >= 512, when the query tiles of the launch do not fill the
 * last round of the device's compute units, the tiles of that round are split into up to 8
 * key ranges that run as separate workgroups, and a second kernel merges their partial
 * results (per query: unnormalised O, reference max and row sum of the rounded P, combined
 * in fp32).  The result equals the unsplit computation up to fp32 rounding and the final
 * bf16 rounding.  Calls on different streams need different workspaces.
 */
size_t hsastep_attention_workspace_bytes(int64_t n_active, int64_t n_tokens, int32_t batch,
                                         int32_t heads, int32_t head_dim);
/* The plan hsa_attention_active_ws follows for a launch on a device with compute_units
 * compute units and a workspace of workspace_bytes bytes (host only, no device work):
 * plan_host[4] = {whole tiles, split tiles, key ranges per split tile, keys per range}, tiles
 * of 256 queries of one (batch, head).  {0, 0, 0, 0} when the shape takes the kernel without
 * splits (head_dim 64 or fewer than 256 keys); {tiles, 0, 1, 0} when splitting would not
 * shorten the launch or nothing fits in the workspace. */
int hsastep_attention_plan(int64_t n_active, int64_t n_tokens, int32_t batch, int32_t heads,
                           int32_t head_dim, int32_t compute_units, size_t workspace_bytes,
                           int32_t* plan_host);
int hsa_attention_active_ws(const uint16_t* q_active, const uint16_t* k_cache,
                            const uint16_t* v_cache, uint16_t* out, int64_t n_active,
                            int64_t n_tokens, int32_t batch, int32_t heads, int32_t head_dim,
                            float softmax_scale, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * Fused QKV projection of the active tokens with the cache write as its epilogue
 * ([HSA-nl] §2.2 items 1-2: only the active tokens go through the model's projections,
 * and their fresh K and V rows overwrite their cache slots).  With HD = heads*head_dim,
 *   Y = x_active W^T (+ bias), fp32 accumulation, rounded to bf16 per element:
 *   Y[b*n_active + a, 0:HD)      -> q_out[b, a]
 *   Y[b*n_active + a, HD:2HD)    -> k_cache[b, active_idx[a]]
 *   Y[b*n_active + a, 2HD:3HD)   -> v_cache[b, active_idx[a]]
 * It replaces a projection into k_new/v_new followed by hsa_kv_update.
 *
 *   x_active           [batch, n_active, model_dim] bf16, active order (16-byte aligned)
 *   w_qkv              [3*HD, model_dim] bf16: the Q, K and V weights stacked by output
 *                      row (the usual [out_features, in_features] layout; 16-byte aligned)
 *   bias_or_null       [3*HD] bf16, or NULL
 *   q_out              [batch, n_active, heads, head_dim] bf16 output
 *   k_cache, v_cache   [batch, n_tokens, heads, head_dim] bf16, in place: only the rows of
 *                      the active slots are written
 *   active_idx         [n_active] int32, slots in [0, n_tokens) (others are skipped)
 * model_dim must be a positive multiple of 64 (else HSASTEP_ERR_UNSUPPORTED), and
 * x_active and w_qkv each below 4 GiB.  n_active == 0 is a no-op.  Outputs must not
 * alias inputs.
 */
int hsa_qkv_project(const uint16_t* x_active, const uint16_t* w_qkv, const uint16_t* bias_or_null,
                    uint16_t* q_out, uint16_t* k_cache, uint16_t* v_cache,
                    const int32_t* active_idx, int64_t n_active, int64_t n_tokens, int32_t batch,
                    int32_t heads, int32_t head_dim, int32_t model_dim, void* stream);

/*
 * Cached Euler update ([HSA-nl] §2.3), one branch-free pass over all N tokens:
 *   v_cache[n] <- v_fresh[active_pos[n]]     for active tokens (active_pos[n] >= 0)
 *   x[n]       <- x[n] + dt * v_cache[n]     for every token,
 * with dt = sigma_next - sigma_cur in fp32 and the product rounded before the
 * add (no fused multiply-add).
 *
 *   x, v_cache         [n_tokens, channels] fp32, in place
 *   v_fresh            [n_active, channels] fp32, active order
 *   active_pos         [n_tokens] int32 from hsa_active_set (-1 = skipped)
 * Positions >= n_active are treated as skipped.
 */
int hsa_euler_step(float* x, float* v_cache, const float* v_fresh, const int32_t* active_pos,
                   int64_t n_active, int64_t n_tokens, int32_t channels, float sigma_cur,
                   float sigma_next, void* stream);

/*
 * Measurement utility, not a step of the method: the sustained rate of the bf16
 * matrix instruction the attention kernel is built on (32x32x16, fp32
 * accumulate), on every compute unit.  The chip's quoted dense peak assumes its
 * full clock; under sustained matrix load it holds a lower one, so this rate is
 * the ceiling an MFMA-bound kernel such as hsa_attention_active can approach.
 * Each workgroup runs 4 wavefronts; each wavefront issues 64 * rounds
 * independent MFMAs (32*32*16*2 flops each), i.e. one launch performs
 * workgroups * 4 * 64 * rounds * 32768 flops.  Time it with events around the
 * call.  Zero operands draw less power and measure a higher, optimistic rate.
 *
 *   operands     [1024 * 8] bf16 bit patterns, read once per wavefront (the
 *                first 512 groups of 8 are the A operands, the rest B)
 *   sink         [workgroups * 256] fp32 out: per-lane sums of the
 *                accumulators, so no instruction can be dropped
 *   rounds       1 .. 2^24;  workgroups  1 .. 2^20
 */
int hsastep_mfma_probe(const uint16_t* operands, float* sink, int32_t rounds,
                       int32_t workgroups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HSASTEP_H */

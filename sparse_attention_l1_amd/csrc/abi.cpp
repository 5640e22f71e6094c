// C ABI of the HSA path (declared in include/hsastep.h): argument validation on
// the host, then kernel launches on the caller's stream.  Nothing here
// allocates device memory or synchronises.
#include "hsastep.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <string>

#include "host.hpp"
#include "kernels.hpp"

#define HSASTEP_API extern "C" __attribute__((visibility("default")))

static_assert(HSASTEP_NOALLOC_MAX_TOKENS == hsastep::kNoAllocMaxTokens,
              "the header's limit of hsa_active_set_noalloc must match its scratch size");

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

int ok() { return HSASTEP_OK; }

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(HSASTEP_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

HSASTEP_API int hsastep_version(void) { return 100; }

HSASTEP_API const char* hsastep_error_string(int code) {
  switch (code) {
    case HSASTEP_OK: return "ok";
    case HSASTEP_ERR_ARG: return "invalid argument";
    case HSASTEP_ERR_UNSUPPORTED: return "unsupported configuration";
    case HSASTEP_ERR_HIP: return "HIP error";
    case HSASTEP_ERR_WORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
  }
}

HSASTEP_API const char* hsastep_last_error(void) { return g_last_error.c_str(); }

HSASTEP_API size_t hsastep_workspace_bytes(int64_t n_tokens, int32_t n_groups) {
  return hsastep::workspace_layout(n_tokens, n_groups).total;
}

HSASTEP_API int hsastep_n_active(int64_t n_tokens, const int32_t* budgets_host,
                                 const int64_t* group_sizes_host, int32_t n_groups, int32_t T,
                                 int32_t m, int32_t iter, int64_t* n_active_host) {
  std::string msg;
  if (hsastep::check_schedule(n_tokens, budgets_host, group_sizes_host, n_groups, T, m, msg))
    return fail(HSASTEP_ERR_ARG, msg);
  if (iter < 0 || iter >= T) return fail(HSASTEP_ERR_ARG, "iter must be in [0, T)");
  if (n_active_host == nullptr) return fail(HSASTEP_ERR_ARG, "n_active_host is null");
  const uint32_t mask = hsastep::group_active_mask(budgets_host, n_groups, T, m, iter);
  *n_active_host = hsastep::n_active_from_mask(mask, group_sizes_host, n_groups);
  return ok();
}

HSASTEP_API int hsa_select_groups(const float* v_prev, const float* v_cur, int64_t n_tokens,
                                  int32_t channels, const int64_t* group_sizes_host,
                                  int32_t n_groups, int32_t* group_id, float* score_or_null,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  if (n_tokens < 1 || n_tokens > INT32_MAX)
    return fail(HSASTEP_ERR_ARG, "n_tokens must be in [1, 2^31-1]");
  if (channels < 1 || channels > HSASTEP_MAX_CHANNELS)
    return fail(HSASTEP_ERR_ARG, "channels must be in [1, 256]");
  if (n_groups < 1 || n_groups > HSASTEP_MAX_GROUPS)
    return fail(HSASTEP_ERR_ARG, "n_groups must be in [1, 16]");
  if (!v_prev || !v_cur || !group_id || !group_sizes_host)
    return fail(HSASTEP_ERR_ARG, "null pointer argument");
  if (!aligned16(v_prev) || !aligned16(v_cur))
    return fail(HSASTEP_ERR_ARG, "v_prev / v_cur must be 16-byte aligned");
  int64_t total = 0;
  for (int k = 0; k < n_groups; ++k) {
    if (group_sizes_host[k] < 0) return fail(HSASTEP_ERR_ARG, "group sizes must be >= 0");
    total += group_sizes_host[k];
  }
  if (total != n_tokens) return fail(HSASTEP_ERR_ARG, "group sizes must sum to n_tokens");
  const hsastep::WorkspaceLayout wl = hsastep::workspace_layout(n_tokens, n_groups);
  if (workspace == nullptr || workspace_bytes < wl.total)
    return fail(HSASTEP_ERR_WORKSPACE, "workspace smaller than hsastep_workspace_bytes()");
  if (!aligned16(workspace)) return fail(HSASTEP_ERR_ARG, "workspace must be 16-byte aligned");
  char* ws = static_cast<char*>(workspace);
  float* r = score_or_null ? score_or_null : reinterpret_cast<float*>(ws + wl.score_off);
  // first rank of each later group; ranks >= n_tokens never occur, so drop those targets
  int64_t targets[HSASTEP_MAX_GROUPS];
  int nt = 0;
  int64_t cum = 0;
  for (int k = 0; k + 1 < n_groups; ++k) {
    cum += group_sizes_host[k];
    if (cum < n_tokens) targets[nt++] = cum;
  }
  uint32_t* rank_ws = reinterpret_cast<uint32_t*>(ws + wl.rank_off);
  const int64_t zero_words = nt > 0 ? int64_t(hsastep::rank_workspace(n_tokens, nt).zero_words) : 0;
  hipStream_t s = as_stream(stream);
  if (int rc = hip_status(hsastep::launch_score(v_prev, v_cur, n_tokens, channels, r, rank_ws,
                                                zero_words, s), "score"))
    return rc;
  return hip_status(hsastep::launch_rank(r, n_tokens, targets, nt, rank_ws, group_id, s), "rank");
}

HSASTEP_API int hsa_active_set(const int32_t* group_id, int64_t n_tokens,
                               const int32_t* budgets_host, const int64_t* group_sizes_host,
                               int32_t n_groups, int32_t T, int32_t m, int32_t iter,
                               int32_t* active_idx, int32_t* active_pos, int64_t* n_active_host,
                               void* workspace, size_t workspace_bytes, void* stream) {
  std::string msg;
  if (hsastep::check_schedule(n_tokens, budgets_host, group_sizes_host, n_groups, T, m, msg))
    return fail(HSASTEP_ERR_ARG, msg);
  if (iter < 0 || iter >= T) return fail(HSASTEP_ERR_ARG, "iter must be in [0, T)");
  if (!group_id || !active_idx || !active_pos || !n_active_host)
    return fail(HSASTEP_ERR_ARG, "null pointer argument");
  const hsastep::WorkspaceLayout wl = hsastep::workspace_layout(n_tokens, n_groups);
  if (workspace == nullptr || workspace_bytes < wl.total)
    return fail(HSASTEP_ERR_WORKSPACE, "workspace smaller than hsastep_workspace_bytes()");
  const uint32_t mask = hsastep::group_active_mask(budgets_host, n_groups, T, m, iter);
  *n_active_host = hsastep::n_active_from_mask(mask, group_sizes_host, n_groups);
  int32_t* blockcnt =
      reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + wl.blockcnt_off);
  return hip_status(hsastep::launch_active(group_id, n_tokens, mask, n_groups, active_idx,
                                           active_pos, blockcnt, as_stream(stream)),
                    "active set");
}

HSASTEP_API int hsa_active_set_gather(const int32_t* group_id, int64_t n_tokens,
                                      const int32_t* budgets_host,
                                      const int64_t* group_sizes_host, int32_t n_groups,
                                      int32_t T, int32_t m, int32_t iter, int32_t* active_idx,
                                      int32_t* active_pos, int64_t* n_active_host,
                                      const void* rows, int64_t row_bytes, void* rows_out,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  std::string msg;
  if (hsastep::check_schedule(n_tokens, budgets_host, group_sizes_host, n_groups, T, m, msg))
    return fail(HSASTEP_ERR_ARG, msg);
  if (iter < 0 || iter >= T) return fail(HSASTEP_ERR_ARG, "iter must be in [0, T)");
  if (!group_id || !active_idx || !active_pos || !n_active_host || !rows || !rows_out)
    return fail(HSASTEP_ERR_ARG, "null pointer argument");
  if (row_bytes < 4 || row_bytes % 4 != 0)
    return fail(HSASTEP_ERR_ARG, "row_bytes must be a positive multiple of 4");
  if ((reinterpret_cast<uintptr_t>(rows) | reinterpret_cast<uintptr_t>(rows_out)) & 3u)
    return fail(HSASTEP_ERR_ARG, "rows / rows_out must be 4-byte aligned");
  const hsastep::WorkspaceLayout wl = hsastep::workspace_layout(n_tokens, n_groups);
  if (workspace == nullptr || workspace_bytes < wl.total)
    return fail(HSASTEP_ERR_WORKSPACE, "workspace smaller than hsastep_workspace_bytes()");
  const uint32_t mask = hsastep::group_active_mask(budgets_host, n_groups, T, m, iter);
  *n_active_host = hsastep::n_active_from_mask(mask, group_sizes_host, n_groups);
  int32_t* blockcnt =
      reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + wl.blockcnt_off);
  return hip_status(hsastep::launch_active(group_id, n_tokens, mask, n_groups, active_idx,
                                           active_pos, blockcnt, as_stream(stream), rows,
                                           row_bytes, rows_out),
                    "active set + gather");
}

HSASTEP_API int hsa_active_set_noalloc(const int32_t* group_id, int64_t n_tokens,
                                       const int32_t* budgets_host,
                                       const int64_t* group_sizes_host, int32_t n_groups,
                                       int32_t T, int32_t m, int32_t iter, int32_t* active_idx,
                                       int32_t* active_pos, int64_t* n_active_host,
                                       void* stream) {
  std::string msg;
  if (hsastep::check_schedule(n_tokens, budgets_host, group_sizes_host, n_groups, T, m, msg))
    return fail(HSASTEP_ERR_ARG, msg);
  if (n_tokens > HSASTEP_NOALLOC_MAX_TOKENS)
    return fail(HSASTEP_ERR_UNSUPPORTED,
                "hsa_active_set_noalloc: n_tokens above HSASTEP_NOALLOC_MAX_TOKENS (2^24); "
                "use hsa_active_set with a workspace");
  if (iter < 0 || iter >= T) return fail(HSASTEP_ERR_ARG, "iter must be in [0, T)");
  if (!group_id || !active_idx || !active_pos || !n_active_host)
    return fail(HSASTEP_ERR_ARG, "null pointer argument");
  int32_t* blockcnt = nullptr;
  if (int rc = hip_status(hsastep::active_scratch(&blockcnt), "active-set scratch address"))
    return rc;
  const uint32_t mask = hsastep::group_active_mask(budgets_host, n_groups, T, m, iter);
  *n_active_host = hsastep::n_active_from_mask(mask, group_sizes_host, n_groups);
  return hip_status(hsastep::launch_active(group_id, n_tokens, mask, n_groups, active_idx,
                                           active_pos, blockcnt, as_stream(stream)),
                    "active set");
}

HSASTEP_API int hsastep_gather_rows(void* dst, const void* src, const int32_t* index,
                                    int64_t n_rows, int64_t n_src_rows, int64_t row_bytes,
                                    void* stream) {
  if (n_rows < 0 || n_src_rows < 0 || row_bytes < 4 || (row_bytes & 3))
    return fail(HSASTEP_ERR_ARG, "n_rows/n_src_rows must be >= 0, row_bytes a multiple of 4");
  if (n_rows > INT32_MAX) return fail(HSASTEP_ERR_ARG, "n_rows must be < 2^31");
  if (n_rows == 0) return ok();
  if (!dst || !src || !index) return fail(HSASTEP_ERR_ARG, "null pointer argument");
  if ((reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(src)) & 3u)
    return fail(HSASTEP_ERR_ARG, "dst / src must be 4-byte aligned");
  return hip_status(
      hsastep::launch_gather(dst, src, index, n_rows, n_src_rows, row_bytes, as_stream(stream)),
      "gather");
}

HSASTEP_API int hsa_kv_update(uint16_t* k_cache, uint16_t* v_cache, const uint16_t* k_new,
                              const uint16_t* v_new, const int32_t* active_idx, int64_t n_active,
                              int64_t n_tokens, int32_t batch, int32_t heads, int32_t head_dim,
                              void* stream) {
  if (n_tokens < 1 || n_active < 0 || n_active > n_tokens || batch < 1 || heads < 1 ||
      head_dim < 1)
    return fail(HSASTEP_ERR_ARG, "need n_tokens >= 1, 0 <= n_active <= n_tokens, batch, heads, "
                                 "head_dim >= 1");
  if ((int64_t(heads) * head_dim) % 8 != 0)
    return fail(HSASTEP_ERR_ARG, "heads*head_dim must be a multiple of 8");
  if (n_active == 0) return ok();
  if (!k_cache || !v_cache || !k_new || !v_new || !active_idx)
    return fail(HSASTEP_ERR_ARG, "null pointer argument");
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new))
    return fail(HSASTEP_ERR_ARG, "cache and row buffers must be 16-byte aligned");
  return hip_status(hsastep::launch_kv_update(k_cache, v_cache, k_new, v_new, active_idx, n_active,
                                              n_tokens, batch, heads, head_dim, as_stream(stream)),
                    "kv update");
}

namespace {

int check_attention(const uint16_t* q_active, const uint16_t* k_cache, const uint16_t* v_cache,
                    uint16_t* out, int64_t n_active, int64_t n_tokens, int32_t batch,
                    int32_t heads, int32_t head_dim, float softmax_scale) {
  if (n_tokens < 1 || n_tokens > INT32_MAX || n_active < 0 || n_active > INT32_MAX ||
      batch < 1 || heads < 1)
    return fail(HSASTEP_ERR_ARG, "need 1 <= n_tokens < 2^31, 0 <= n_active < 2^31, batch, "
                                 "heads >= 1");
  if (head_dim != 64 && head_dim != 128)
    return fail(HSASTEP_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale))
    return fail(HSASTEP_ERR_ARG, "softmax_scale must be finite and > 0");
  if (n_active == 0) return ok();
  if (!q_active || !k_cache || !v_cache || !out)
    return fail(HSASTEP_ERR_ARG, "null pointer argument");
  if (!aligned16(q_active) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return fail(HSASTEP_ERR_ARG, "q/k/v/out must be 16-byte aligned");
  const int64_t qtiles = (n_active + 127) / 128;
  if (qtiles * heads * int64_t(batch) > INT32_MAX)
    return fail(HSASTEP_ERR_ARG, "grid too large");
  return ok();
}

}  // namespace

HSASTEP_API size_t hsastep_attention_workspace_bytes(int64_t n_active, int64_t n_tokens,
                                                     int32_t batch, int32_t heads,
                                                     int32_t head_dim) {
  if (n_active < 1 || n_tokens < 1 || batch < 1 || heads < 1) return 0;
  return hsastep::attention_split_workspace_bytes(n_active, n_tokens, batch, heads, head_dim);
}

HSASTEP_API int hsastep_attention_plan(int64_t n_active, int64_t n_tokens, int32_t batch,
                                       int32_t heads, int32_t head_dim, int32_t compute_units,
                                       size_t workspace_bytes, int32_t* plan_host) {
  if (plan_host == nullptr) return fail(HSASTEP_ERR_ARG, "plan_host is null");
  if (n_active < 1 || n_tokens < 1 || batch < 1 || heads < 1 || compute_units < 0)
    return fail(HSASTEP_ERR_ARG, "need n_active, n_tokens, batch, heads >= 1, compute_units >= 0");
  const int64_t tiles = (n_active + 255) / 256 * heads * int64_t(batch);
  if (!hsastep::attention_pipe_fits(n_tokens, heads, head_dim) || tiles > INT32_MAX) {
    plan_host[0] = plan_host[1] = plan_host[2] = plan_host[3] = 0;   // kernel without splits
    return ok();
  }
  const hsastep::AttentionPlan p = hsastep::attention_plan(n_active, n_tokens, batch, heads,
                                                           compute_units, workspace_bytes);
  plan_host[0] = p.full_tiles;
  plan_host[1] = p.splits > 1 ? p.tail_tiles : 0;
  plan_host[2] = p.splits;
  plan_host[3] = p.splits > 1 ? p.piece_keys : 0;
  return ok();
}

HSASTEP_API int hsa_attention_active_ws(const uint16_t* q_active, const uint16_t* k_cache,
                                        const uint16_t* v_cache, uint16_t* out, int64_t n_active,
                                        int64_t n_tokens, int32_t batch, int32_t heads,
                                        int32_t head_dim, float softmax_scale, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  if (int rc = check_attention(q_active, k_cache, v_cache, out, n_active, n_tokens, batch, heads,
                               head_dim, softmax_scale))
    return rc;
  if (n_active == 0) return ok();
  if (workspace_bytes > 0 && workspace == nullptr)
    return fail(HSASTEP_ERR_WORKSPACE, "workspace_bytes > 0 with a null workspace");
  if (workspace != nullptr && !aligned16(workspace))
    return fail(HSASTEP_ERR_ARG, "workspace must be 16-byte aligned");
  return hip_status(hsastep::launch_attention(q_active, k_cache, v_cache, out, n_active, n_tokens,
                                              batch, heads, head_dim, softmax_scale,
                                              workspace_bytes ? workspace : nullptr,
                                              workspace_bytes, as_stream(stream)),
                    "attention");
}

HSASTEP_API int hsa_attention_active(const uint16_t* q_active, const uint16_t* k_cache,
                                     const uint16_t* v_cache, uint16_t* out, int64_t n_active,
                                     int64_t n_tokens, int32_t batch, int32_t heads,
                                     int32_t head_dim, float softmax_scale, void* stream) {
  if (int rc = check_attention(q_active, k_cache, v_cache, out, n_active, n_tokens, batch, heads,
                               head_dim, softmax_scale))
    return rc;
  if (n_active == 0) return ok();
  return hip_status(hsastep::launch_attention(q_active, k_cache, v_cache, out, n_active, n_tokens,
                                              batch, heads, head_dim, softmax_scale, nullptr, 0,
                                              as_stream(stream)),
                    "attention");
}

HSASTEP_API int hsa_qkv_project(const uint16_t* x_active, const uint16_t* w_qkv,
                                const uint16_t* bias_or_null, uint16_t* q_out, uint16_t* k_cache,
                                uint16_t* v_cache, const int32_t* active_idx, int64_t n_active,
                                int64_t n_tokens, int32_t batch, int32_t heads, int32_t head_dim,
                                int32_t model_dim, void* stream) {
  if (n_tokens < 1 || n_tokens > INT32_MAX || n_active < 0 || n_active > n_tokens ||
      batch < 1 || heads < 1 || head_dim < 1)
    return fail(HSASTEP_ERR_ARG, "need 1 <= n_tokens < 2^31, 0 <= n_active <= n_tokens, "
                                 "batch, heads, head_dim >= 1");
  if (model_dim < 64 || model_dim % 64 != 0)
    return fail(HSASTEP_ERR_UNSUPPORTED, "model_dim must be a positive multiple of 64");
  const int64_t hd = int64_t(heads) * head_dim;
  const int64_t m_rows = int64_t(batch) * n_active;
  if (3 * hd > INT32_MAX / 2 || m_rows > INT32_MAX || int64_t(batch) * n_tokens > INT32_MAX)
    return fail(HSASTEP_ERR_UNSUPPORTED, "sizes too large");
  if (m_rows * model_dim * 2 >= (int64_t(1) << 32) || 3 * hd * model_dim * 2 >= (int64_t(1) << 32))
    return fail(HSASTEP_ERR_UNSUPPORTED, "x_active and w_qkv must each be below 4 GiB");
  if (((m_rows + 255) / 256) * ((3 * hd + 255) / 256) > INT32_MAX)
    return fail(HSASTEP_ERR_UNSUPPORTED, "grid too large");
  if (n_active == 0) return ok();
  if (!x_active || !w_qkv || !q_out || !k_cache || !v_cache || !active_idx)
    return fail(HSASTEP_ERR_ARG, "null pointer argument");
  if (!aligned16(x_active) || !aligned16(w_qkv))
    return fail(HSASTEP_ERR_ARG, "x_active / w_qkv must be 16-byte aligned");
  return hip_status(hsastep::launch_qkv_project(x_active, w_qkv, bias_or_null, q_out, k_cache,
                                                v_cache, active_idx, n_active, n_tokens, batch,
                                                heads, head_dim, model_dim, as_stream(stream)),
                    "qkv projection");
}

HSASTEP_API int hsastep_mfma_probe(const uint16_t* operands, float* sink, int32_t rounds,
                                   int32_t workgroups, void* stream) {
  if (!operands || !sink) return fail(HSASTEP_ERR_ARG, "null pointer argument");
  if (!aligned16(operands)) return fail(HSASTEP_ERR_ARG, "operands must be 16-byte aligned");
  if (rounds < 1 || rounds > (1 << 24) || workgroups < 1 || workgroups > (1 << 20))
    return fail(HSASTEP_ERR_ARG, "need 1 <= rounds <= 2^24 and 1 <= workgroups <= 2^20");
  return hip_status(hsastep::launch_mfma_probe(operands, sink, rounds, workgroups,
                                               as_stream(stream)),
                    "mfma probe");
}

HSASTEP_API int hsa_euler_step(float* x, float* v_cache, const float* v_fresh,
                               const int32_t* active_pos, int64_t n_active, int64_t n_tokens,
                               int32_t channels, float sigma_cur, float sigma_next, void* stream) {
  if (n_tokens < 1 || n_active < 0 || n_active > n_tokens || channels < 1)
    return fail(HSASTEP_ERR_ARG, "need n_tokens >= 1, 0 <= n_active <= n_tokens, channels >= 1");
  if (n_tokens * int64_t(channels) > (int64_t(1) << 40))
    return fail(HSASTEP_ERR_ARG, "latent too large");
  if (!x || !v_cache || !active_pos || (n_active > 0 && !v_fresh))
    return fail(HSASTEP_ERR_ARG, "null pointer argument");
  if (!aligned16(x) || !aligned16(v_cache) || (v_fresh && !aligned16(v_fresh)))
    return fail(HSASTEP_ERR_ARG, "x / v_cache / v_fresh must be 16-byte aligned");
  return hip_status(hsastep::launch_euler(x, v_cache, v_fresh, active_pos, n_active, n_tokens,
                                          channels, sigma_cur, sigma_next, as_stream(stream)),
                    "euler");
}

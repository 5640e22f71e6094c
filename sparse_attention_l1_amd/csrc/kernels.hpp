// Internal launchers of the HSA kernels (one per .hip file).  Each validates
// nothing: the C ABI layer (abi.cpp) checks arguments before calling them.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace hsastep {

// score.hip: r[n] = L1 relative change of token n (balanced-tree fp32 sums); the
// same launch also sets zero[0 .. zero_words) to 0 (the grouping histograms).
hipError_t launch_score(const float* v_prev, const float* v_cur, int64_t n_tokens, int channels,
                        float* r, uint32_t* zero, int64_t zero_words, hipStream_t stream);

// rank.hip: group id from the rank of r (largest first, ties by index).
// targets[t] = first rank of group t+1 (only targets < n_tokens are passed).
// rank_ws: the grouping workspace (RankWorkspace), its histograms already zero.
hipError_t launch_rank(const float* r, int64_t n_tokens, const int64_t* targets, int n_targets,
                       uint32_t* rank_ws, int32_t* group_id, hipStream_t stream);

// active.hip: ascending active index list + inverse map for one iteration; with rows, also
// rows_out[a] = rows[active_idx[a]] (rows of row_bytes, a multiple of 4) in the same launch.
hipError_t launch_active(const int32_t* group_id, int64_t n_tokens, uint32_t group_mask,
                         int n_groups, int32_t* active_idx, int32_t* active_pos, int32_t* blockcnt,
                         hipStream_t stream, const void* rows = nullptr, int64_t row_bytes = 0,
                         void* rows_out = nullptr);

// active.hip: device address of the library's own per-chunk count array on the current device
// (kNoAllocMaxTokens / 1024 + 1 words), looked up once per device; for callers that cannot
// allocate.  Calls that use it and overlap on one device race.
hipError_t active_scratch(int32_t** ptr);

// rows.hip: row gather and the KV-cache row scatter.
hipError_t launch_gather(void* dst, const void* src, const int32_t* index, int64_t n_rows,
                         int64_t n_src_rows, int64_t row_bytes, hipStream_t stream);
hipError_t launch_kv_update(uint16_t* k_cache, uint16_t* v_cache, const uint16_t* k_new,
                            const uint16_t* v_new, const int32_t* active_idx, int64_t n_active,
                            int64_t n_tokens, int batch, int heads, int head_dim,
                            hipStream_t stream);

// attn.hip: active-query full-context attention (bf16 MFMA, fp32 online softmax).
hipError_t launch_attention(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                            uint16_t* out, int64_t n_active, int64_t n_tokens, int batch, int heads,
                            int head_dim, float softmax_scale, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

// attn_pipe.hip: the head_dim 128 path of launch_attention (one wavefront per SIMD, 64
// queries each, hand-scheduled key loop); fits() says whether a shape can take it.
bool attention_pipe_fits(int64_t n_tokens, int heads, int head_dim);
// With a workspace, the tiles of a last round that would leave compute units idle are split
// into key ranges (pieces) whose partial results a merge kernel combines.
constexpr int kMaxSplits = 8;       // key ranges per split tile
constexpr int kMaxPieces = 512;     // pieces per launch (two rounds of 256 compute units)
struct AttentionPlan {
  int full_tiles, tail_tiles, splits, piece_keys;
};
AttentionPlan attention_plan(int64_t n_active, int64_t n_tokens, int batch, int heads, int cus,
                             size_t workspace_bytes);
size_t attention_piece_bytes();
size_t attention_split_workspace_bytes(int64_t n_active, int64_t n_tokens, int batch, int heads,
                                       int head_dim);
hipError_t launch_attention_pipe(const uint16_t* q, const uint16_t* k_cache,
                                 const uint16_t* v_cache, uint16_t* out, int64_t n_active,
                                 int64_t n_tokens, int batch, int heads, float softmax_scale,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

// proj.hip: fused QKV projection of the active rows; Q compacted, K/V into their cache slots.
hipError_t launch_qkv_project(const uint16_t* x, const uint16_t* w, const uint16_t* bias,
                              uint16_t* q_out, uint16_t* k_cache, uint16_t* v_cache,
                              const int32_t* active_idx, int64_t n_active, int64_t n_tokens,
                              int batch, int heads, int head_dim, int model_dim,
                              hipStream_t stream);

// euler.hip: cached Euler update over all tokens.
// sustained bf16 MFMA rate probe (measurement utility): 64 MFMAs per wavefront per round
hipError_t launch_mfma_probe(const uint16_t* operands, float* sink, int rounds, int workgroups,
                             hipStream_t stream);

hipError_t launch_euler(float* x, float* v_cache, const float* v_fresh, const int32_t* active_pos,
                        int64_t n_active, int64_t n_tokens, int channels, float sigma_cur,
                        float sigma_next, hipStream_t stream);

}  // namespace hsastep

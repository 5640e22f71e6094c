// Host-side helpers of the HSA path: argument checks and schedule arithmetic.
// HIP-free, so it can be compiled and tested with a plain host compiler.
//
// Schedule rule: "Technische Samenvatting: Heterogene Staptoewijzing (HSA) voor
// Efficiënte Videogeneratie" (gist.science/nl/paper/2605.06892), §2.1 (budgets
// divide T, the baseline group has s_1 = T, a reduced group is active iff
// i mod (T/s_k) = 0) and §2.4 (the first and last m iterations run all tokens).
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

namespace hsastep {

constexpr int kMaxGroups = 16;
constexpr int kMaxChannels = 256;
constexpr int kActiveBlockTokens = 1024;   // tokens per workgroup of the active-set kernels
constexpr int64_t kNoAllocMaxTokens = int64_t(1) << 24;   // limit of hsa_active_set_noalloc
constexpr int kRankThreads = 512;          // threads per workgroup of the grouping kernels
constexpr int kRankChunk = 512;            // tokens a grouping workgroup holds at once
constexpr int kRankMaxBlocks = 512;        // cap on grouping workgroups (bounds the workspace)

// Grouping kernels: tokens per workgroup (a multiple of kRankChunk) and workgroups.
int64_t rank_tokens_per_block(int64_t n_tokens);
int64_t rank_blocks(int64_t n_tokens);

// Grouping workspace, offsets in uint32 words from its start: the three global
// radix histograms (zeroed before each selection; they are contiguous, zero_words
// long) and every workgroup's own pass-2 counts.
struct RankWorkspace {
  size_t hist0_off, hist1_off, hist2_off, block2_off, zero_words, total_words;
};
RankWorkspace rank_workspace(int64_t n_tokens, int n_targets);

// Validates budgets / sizes / T / m for n_groups groups over n_tokens tokens.
// Returns 0 or -1 with a message.  Budgets must start with T, divide T and be
// non-increasing; sizes must be >= 0 and sum to n_tokens.
int check_schedule(int64_t n_tokens, const int32_t* budgets, const int64_t* sizes, int32_t n_groups,
                   int32_t T, int32_t m, std::string& msg);

// Bit k set iff group k is active at iteration iter (all bits inside a window).
uint32_t group_active_mask(const int32_t* budgets, int32_t n_groups, int32_t T, int32_t m,
                           int32_t iter);

// |A_i| = sum of sizes[k] over the groups whose bit is set.
int64_t n_active_from_mask(uint32_t mask, const int64_t* sizes, int32_t n_groups);

// Device workspace layout for the selection and active-set kernels.
struct WorkspaceLayout {
  size_t score_off, score_bytes;        // fp32 [N] scores when the caller passes none
  size_t blockcnt_off, blockcnt_bytes;  // int32 [ceil(N / 1024)] per-workgroup active counts
  size_t rank_off, rank_bytes;          // uint32 grouping histograms (RankWorkspace)
  size_t total;
};
WorkspaceLayout workspace_layout(int64_t n_tokens, int32_t n_groups);

}  // namespace hsastep

// Host-side argument checks and schedule arithmetic (see host.hpp).
#include "host.hpp"

namespace hsastep {

int check_schedule(int64_t n_tokens, const int32_t* budgets, const int64_t* sizes, int32_t n_groups,
                   int32_t T, int32_t m, std::string& msg) {
  if (n_tokens < 1 || n_tokens > INT32_MAX) {
    msg = "n_tokens must be in [1, 2^31-1]";
    return -1;
  }
  if (n_groups < 1 || n_groups > kMaxGroups) {
    msg = "n_groups must be in [1, 16]";
    return -1;
  }
  if (budgets == nullptr || sizes == nullptr) {
    msg = "budgets_host and group_sizes_host must be non-null";
    return -1;
  }
  if (T < 1) {
    msg = "T must be >= 1";
    return -1;
  }
  if (m < 0) {
    msg = "m must be >= 0";
    return -1;
  }
  if (budgets[0] != T) {
    msg = "the baseline group must have the full budget: budgets[0] == T";
    return -1;
  }
  int64_t total = 0;
  for (int k = 0; k < n_groups; ++k) {
    if (budgets[k] < 1 || T % budgets[k] != 0) {
      msg = "every budget must divide T (budget " + std::to_string(budgets[k]) + ", T " +
            std::to_string(T) + ")";
      return -1;
    }
    if (k > 0 && budgets[k] > budgets[k - 1]) {
      msg = "budgets must be non-increasing";
      return -1;
    }
    if (sizes[k] < 0) {
      msg = "group sizes must be >= 0";
      return -1;
    }
    total += sizes[k];
  }
  if (total != n_tokens) {
    msg = "group sizes must sum to n_tokens";
    return -1;
  }
  return 0;
}

uint32_t group_active_mask(const int32_t* budgets, int32_t n_groups, int32_t T, int32_t m,
                           int32_t iter) {
  const bool window = iter < m || iter >= T - m;
  uint32_t mask = 0;
  for (int k = 0; k < n_groups; ++k) {
    const int32_t period = T / budgets[k];
    if (window || iter % period == 0) mask |= 1u << k;
  }
  return mask;
}

int64_t n_active_from_mask(uint32_t mask, const int64_t* sizes, int32_t n_groups) {
  int64_t n = 0;
  for (int k = 0; k < n_groups; ++k)
    if (mask & (1u << k)) n += sizes[k];
  return n;
}

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int64_t rank_tokens_per_block(int64_t n_tokens) {
  const int64_t chunks = n_tokens > 0 ? (n_tokens + kRankChunk - 1) / kRankChunk : 1;
  const int64_t blocks = chunks < kRankMaxBlocks ? chunks : kRankMaxBlocks;
  return kRankChunk * ((chunks + blocks - 1) / blocks);
}

int64_t rank_blocks(int64_t n_tokens) {
  const int64_t per = rank_tokens_per_block(n_tokens);
  const int64_t b = n_tokens > 0 ? (n_tokens + per - 1) / per : 1;
  return b;
}

RankWorkspace rank_workspace(int64_t n_tokens, int n_targets) {
  RankWorkspace w{};
  const size_t nt = n_targets > 0 ? size_t(n_targets) : 0;
  w.hist0_off = 0;
  w.hist1_off = w.hist0_off + 2048;
  w.hist2_off = w.hist1_off + nt * 2048;
  w.block2_off = w.hist2_off + nt * 1024;
  w.zero_words = w.block2_off;
  w.total_words = w.block2_off + size_t(rank_blocks(n_tokens)) * nt * 1024;
  return w;
}

WorkspaceLayout workspace_layout(int64_t n_tokens, int32_t n_groups) {
  WorkspaceLayout w{};
  const size_t n = n_tokens > 0 ? size_t(n_tokens) : 0;
  w.score_off = 0;
  w.score_bytes = align256(n * sizeof(float));
  w.blockcnt_off = w.score_off + w.score_bytes;
  const size_t nblk = (n + kActiveBlockTokens - 1) / kActiveBlockTokens;
  w.blockcnt_bytes = align256((nblk + 1) * sizeof(int32_t));
  w.rank_off = w.blockcnt_off + w.blockcnt_bytes;
  const int nt = n_groups > 1 ? n_groups - 1 : 0;
  w.rank_bytes = align256(rank_workspace(n_tokens, nt).total_words * sizeof(uint32_t));
  w.total = w.rank_off + w.rank_bytes;
  return w;
}

}  // namespace hsastep

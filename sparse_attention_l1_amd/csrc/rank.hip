// Stable bucketing of tokens into groups by the rank of their score
// (Dynamic Token Selection, "Technische Samenvatting: Heterogene Staptoewijzing
// (HSA) voor Efficiënte Videogeneratie", §2.1 and the §2 introduction: the
// fastest-changing tokens keep the full budget, slower ones get fewer steps).
//
// rank(n) = #{j : r_j > r_n} + #{j < n : r_j == r_n}; group(n) = number of group
// boundaries P_k (first rank of group k+1) with rank(n) >= P_k.
//
// Only the K-1 boundary keys are needed, not a full sort.  Keys are the fp32 bit
// patterns (r >= +0, so they order like r), inverted so that ascending key =
// descending score.  A radix select over the whole grid, one launch per digit:
//   pass 0   bits 31..21  one 2048-bin histogram of all keys (shared by every boundary)
//   pass 1   bits 20..10  per boundary, 2048 bins over the keys that share its 11-bit prefix
//   pass 2   bits  9..0   per boundary, 1024 bins over the keys that share its 22-bit prefix
//   assign   group of every token, in token order
// Each workgroup counts its tokens in LDS (wavefront-aggregated atomics) and adds
// the non-zero bins to a global histogram.  Every later launch re-derives the digits
// chosen so far from those histograms (one wavefront per boundary scans the bins),
// so no state passes between workgroups except the counts.  Pass 2 also keeps each
// workgroup's own counts: the assignment needs, for boundary k with final key t_k,
// how many tokens equal to t_k lie in earlier workgroups, and that is the pass-2
// count of bin (t_k & 1023) summed over those workgroups.  A token equal to t_k
// joins the later group iff its index-order rank among the keys equal to t_k is at
// least e_k, the part of P_k that falls inside the run of equal keys.
// Integer-only after the keys are read, so the result is exact and deterministic.
// The global histograms must be zero at the first pass; the score kernel clears them.
#include <hip/hip_runtime.h>

#include "host.hpp"
#include "kernels.hpp"

namespace hsastep {
namespace {

constexpr int kThreads = kRankThreads;
constexpr int kWaves = kThreads / 64;
constexpr int kPerThread = kRankChunk / kThreads;   // keys a thread holds per chunk
constexpr int kMaxTargets = kMaxGroups - 1;
static_assert(kPerThread * kThreads == kRankChunk, "chunk must be a whole number of rounds");

struct RankArgs {
  const float* r;
  uint32_t n_tokens;
  uint32_t tokens_per_block;   // multiple of kRankChunk
  int nt;                      // boundaries
  uint32_t pos[kMaxTargets];   // P_k
  uint32_t* hist0;             // [2048]
  uint32_t* hist1;             // [nt][2048]
  uint32_t* hist2;             // [nt][1024]
  uint32_t* block2;            // [blocks][nt][1024]
};

__device__ __forceinline__ uint32_t sort_key(float r) { return ~__float_as_uint(r); }

// One wavefront: the digit d of `hist` (B bins) with cum(< d) <= remain < cum(<= d),
// and remain - cum(< d).  Requires remain < sum of the bins.
template <int B>
__device__ __forceinline__ void select_digit(const uint32_t* __restrict__ hist, uint32_t remain,
                                             uint32_t& digit, uint32_t& rest) {
  constexpr int kPer = B / 64;
  const int lane = threadIdx.x & 63;
  uint32_t c[kPer];
  const uint4* src = reinterpret_cast<const uint4*>(hist + lane * kPer);
#pragma unroll
  for (int j = 0; j < kPer / 4; ++j) {
    const uint4 q = src[j];
    c[4 * j] = q.x; c[4 * j + 1] = q.y; c[4 * j + 2] = q.z; c[4 * j + 3] = q.w;
  }
  uint32_t tot = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) tot += c[j];
  uint32_t incl = tot;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  uint32_t acc = incl - tot;
  const bool mine = remain >= acc && remain < incl;
  uint32_t d = 0, rr = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    if (remain >= acc && remain < acc + c[j]) {
      d = uint32_t(lane * kPer + j);
      rr = remain - acc;
    }
    acc += c[j];
  }
  const uint64_t owner = __ballot(mine);
  const int src_lane = owner ? __ffsll((unsigned long long)owner) - 1 : 0;
  digit = uint32_t(__shfl(int(d), src_lane));
  rest = uint32_t(__shfl(int(rr), src_lane));
}

// The digits of boundary k fixed by passes 0 .. levels-1: returns the key prefix
// (those digits concatenated) and the rank left inside it.  One wavefront.
__device__ __forceinline__ void boundary_prefix(const RankArgs& a, int k, int levels,
                                                uint32_t& prefix, uint32_t& remain,
                                                uint32_t& last_digit) {
  uint32_t d = 0, rem = a.pos[k];
  select_digit<2048>(a.hist0, rem, d, rem);
  prefix = d;
  if (levels >= 2) {
    select_digit<2048>(a.hist1 + size_t(k) * 2048, rem, d, rem);
    prefix = (prefix << 11) | d;
  }
  if (levels >= 3) {
    select_digit<1024>(a.hist2 + size_t(k) * 1024, rem, d, rem);
    prefix = (prefix << 10) | d;
  }
  remain = rem;
  last_digit = d;
}

// Adds one to h[digit] for every lane with `pending` set.  Lanes that share the
// first pending lane's digit add with one atomic; after a few rounds the rest
// add individually (scores cluster in few bins of the top digit).
__device__ __forceinline__ void add_aggregated(uint32_t* h, uint32_t digit, bool pending) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int round = 0; round < 4; ++round) {
    const uint64_t b = __ballot(pending);
    if (b == 0) return;
    const int leader = __ffsll((unsigned long long)b) - 1;
    const uint32_t ld = uint32_t(__builtin_amdgcn_readlane(int(digit), leader));
    const bool same = pending && digit == ld;
    const uint64_t sb = __ballot(same);
    if (lane == leader) atomicAdd(&h[ld], uint32_t(__popcll(sb)));
    pending = pending && !same;
  }
  if (pending) atomicAdd(&h[digit], 1u);
}

// Histogram pass PASS over this workgroup's tokens.
template <int PASS>
__global__ __launch_bounds__(kThreads) void rank_hist_kernel(RankArgs a) {
  constexpr int B = PASS == 2 ? 1024 : 2048;
  constexpr int kShift = PASS == 0 ? 21 : PASS == 1 ? 10 : 0;
  constexpr int kPrefixShift = PASS == 1 ? 21 : 10;
  constexpr int kHists = PASS == 0 ? 1 : kMaxTargets;
  __shared__ __attribute__((aligned(16))) uint32_t lh[kHists * B];
  __shared__ uint32_t s_prefix[kMaxTargets];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int nh = PASS == 0 ? 1 : a.nt;
  for (int i = tid; i < nh * B; i += kThreads) lh[i] = 0;
  if (PASS > 0) {
    for (int k = wave; k < a.nt; k += kWaves) {
      uint32_t prefix, remain, d;
      boundary_prefix(a, k, PASS, prefix, remain, d);
      if ((tid & 63) == 0) s_prefix[k] = prefix;
    }
  }
  __syncthreads();

  const uint32_t begin = blockIdx.x * a.tokens_per_block;
  const uint32_t end = min(a.n_tokens, begin + a.tokens_per_block);
  for (uint32_t base = begin; base < end; base += kRankChunk) {
    uint32_t key[kPerThread];
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const uint32_t n = base + uint32_t(j * kThreads + tid);
      key[j] = n < end ? sort_key(a.r[n]) : 0u;
    }
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const bool valid = base + uint32_t(j * kThreads + tid) < end;
      const uint32_t digit = (key[j] >> kShift) & uint32_t(B - 1);
      if (PASS == 0) {
        add_aggregated(lh, digit, valid);
      } else {
        const uint32_t hi = key[j] >> kPrefixShift;
        for (int k = 0; k < nh; ++k) add_aggregated(lh + k * B, digit, valid && hi == s_prefix[k]);
      }
    }
  }
  __syncthreads();

  uint32_t* g = PASS == 0 ? a.hist0 : PASS == 1 ? a.hist1 : a.hist2;
  uint32_t* own = a.block2 + size_t(blockIdx.x) * size_t(nh) * B;
  for (int i = tid; i < nh * B; i += kThreads) {
    const uint32_t v = lh[i];
    if (v) atomicAdd(&g[i], v);
    if (PASS == 2) own[i] = v;
  }
}

// Final keys t_k and tie offsets, then the group of every token in index order.
__global__ __launch_bounds__(kThreads) void rank_assign_kernel(RankArgs a,
                                                               int32_t* __restrict__ group_id) {
  __shared__ uint32_t s_t[kMaxTargets];
  __shared__ uint32_t s_e[kMaxTargets];
  __shared__ uint32_t s_run[kMaxTargets];   // keys equal to t_k in earlier tokens
  __shared__ uint32_t s_wcnt[kWaves];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nt = a.nt;
  for (int k = wave; k < nt; k += kWaves) {
    uint32_t t, e, d2;
    boundary_prefix(a, k, 3, t, e, d2);
    // equal keys in earlier workgroups: their pass-2 count in bin d2
    uint32_t before = 0;
    for (uint32_t b = lane; b < blockIdx.x; b += 64)
      before += a.block2[(size_t(b) * nt + k) * 1024 + d2];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) before += __shfl_xor(before, off);
    if (lane == 0) {
      s_t[k] = t;
      s_e[k] = e;
      s_run[k] = before;
    }
  }
  __syncthreads();

  const uint32_t begin = blockIdx.x * a.tokens_per_block;
  const uint32_t end = min(a.n_tokens, begin + a.tokens_per_block);
  for (uint32_t base = begin; base < end; base += kRankChunk) {
    uint32_t key[kPerThread];
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const uint32_t n = base + uint32_t(j * kThreads + tid);
      key[j] = n < end ? sort_key(a.r[n]) : 0u;
    }
    int g[kPerThread];
    uint32_t eq[kPerThread];
    uint32_t any_eq = 0;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const bool valid = base + uint32_t(j * kThreads + tid) < end;
      g[j] = 0;
      eq[j] = 0;
      for (int k = 0; k < nt; ++k) {
        const uint32_t t = s_t[k];
        g[j] += key[j] > t;
        eq[j] |= uint32_t(valid && key[j] == t) << k;
      }
      any_eq |= eq[j];
    }
    if (__syncthreads_or(any_eq != 0)) {
      // ties: rank the equal keys of each boundary in token order, 256 tokens a round
      for (int j = 0; j < kPerThread; ++j) {
        for (int k = 0; k < nt; ++k) {
          const bool f = (eq[j] >> k) & 1u;
          const uint64_t ballot = __ballot(f);
          const uint32_t below = __popcll(ballot & ((uint64_t(1) << lane) - 1));
          if (lane == 0) s_wcnt[wave] = __popcll(ballot);
          __syncthreads();
          uint32_t wave_off = 0, total = 0;
#pragma unroll
          for (int w = 0; w < kWaves; ++w) {
            const uint32_t c = s_wcnt[w];
            wave_off += w < wave ? c : 0u;
            total += c;
          }
          if (f && s_run[k] + wave_off + below >= s_e[k]) ++g[j];
          __syncthreads();
          if (tid == 0) s_run[k] += total;
          __syncthreads();
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const uint32_t n = base + uint32_t(j * kThreads + tid);
      if (n < end) group_id[n] = g[j];
    }
  }
}

}  // namespace

hipError_t launch_rank(const float* r, int64_t n_tokens, const int64_t* targets, int n_targets,
                       uint32_t* rank_ws, int32_t* group_id, hipStream_t stream) {
  RankArgs a{};
  a.r = r;
  a.n_tokens = uint32_t(n_tokens);
  a.tokens_per_block = uint32_t(rank_tokens_per_block(n_tokens));
  a.nt = n_targets;
  for (int k = 0; k < n_targets && k < kMaxTargets; ++k) a.pos[k] = uint32_t(targets[k]);
  const RankWorkspace w = rank_workspace(n_tokens, n_targets);
  a.hist0 = rank_ws + w.hist0_off;
  a.hist1 = rank_ws + w.hist1_off;
  a.hist2 = rank_ws + w.hist2_off;
  a.block2 = rank_ws + w.block2_off;
  const dim3 grid(unsigned(rank_blocks(n_tokens)));
  if (n_targets > 0) {
    rank_hist_kernel<0><<<grid, dim3(kThreads), 0, stream>>>(a);
    rank_hist_kernel<1><<<grid, dim3(kThreads), 0, stream>>>(a);
    rank_hist_kernel<2><<<grid, dim3(kThreads), 0, stream>>>(a);
  }
  rank_assign_kernel<<<grid, dim3(kThreads), 0, stream>>>(a, group_id);
  return hipGetLastError();
}

}  // namespace hsastep

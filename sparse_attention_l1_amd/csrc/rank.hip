// Stable bucketing of tokens into groups by the rank of their score
// (Dynamic Token Selection, "Technische Samenvatting: Heterogene Staptoewijzing
// (HSA) voor Efficiënte Videogeneratie", §2.1 and the §2 introduction: the
// fastest-changing tokens keep the full budget, slower ones get fewer steps).
//
// rank(n) = #{j : r_j > r_n} + #{j < n : r_j == r_n}; group(n) = number of group
// boundaries P_k (first rank of group k+1) with rank(n) >= P_k.
//
// Only the K-1 boundary keys are needed, not a full sort.  Keys are the fp32
// bit patterns (r >= +0, so they order like r), inverted so that ascending key
// = descending score.  One workgroup of 1024 threads:
//   1. radix select, 4 passes of 8-bit digits (MSB first): an LDS histogram per
//      boundary over the tokens that share the boundary's prefix so far; one
//      wavefront per boundary scans its 256 bins and fixes the next digit.
//      After the last pass each boundary has its exact key t_k and the number
//      e_k of tokens equal to t_k that rank before P_k.
//   2. assignment in index order, 1024 tokens at a time: group = #{k : key > t_k}
//      + #{k : key == t_k and (number of earlier tokens equal to t_k) >= e_k}.
//      The running count of equal keys uses wavefront ballots, and only runs in
//      the few chunks that hold a boundary key.
// Integer-only after the keys are read, so the result is exact and deterministic.
// The workload is O(N) integer work on 4N bytes (latency bound); for the sizes
// of video latents (N up to a few hundred thousand) one workgroup suffices.
#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace hsastep {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxTargets = 15;

struct Targets {
  int count;
  int64_t pos[kMaxTargets];
};

__device__ __forceinline__ uint32_t sort_key(float r) { return ~__float_as_uint(r); }

__global__ __launch_bounds__(kThreads) void rank_kernel(const float* __restrict__ r,
                                                        int64_t n_tokens, Targets tg,
                                                        int32_t* __restrict__ group_id) {
  __shared__ uint32_t hist[kMaxTargets][256];
  __shared__ uint32_t prefix[kMaxTargets];
  __shared__ int64_t remain[kMaxTargets];
  __shared__ int64_t tie_run[kMaxTargets];
  __shared__ uint32_t wave_cnt[kWaves];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nt = tg.count;

  if (tid < nt) {
    prefix[tid] = 0;
    remain[tid] = tg.pos[tid];
    tie_run[tid] = 0;
  }

  // ---- 1. radix select of every boundary key
  for (int pass = 0; pass < 4 && nt > 0; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < nt * 256; i += kThreads) (&hist[0][0])[i] = 0;
    __syncthreads();
    for (int64_t n = tid; n < n_tokens; n += kThreads) {
      const uint32_t key = sort_key(r[n]);
      const uint32_t hi = uint32_t(uint64_t(key) >> (shift + 8));   // prefix fixed so far
      const uint32_t digit = (key >> shift) & 255u;
      // scores cluster in few bins (the top byte is mostly sign + exponent), so lanes
      // that share the wavefront leader's digit add their count with one atomic
      const uint32_t lead = uint32_t(__builtin_amdgcn_readfirstlane(int(digit)));
      for (int k = 0; k < nt; ++k) {
        const bool match = pass == 0 || hi == prefix[k];
        const bool same = match && digit == lead;
        const uint64_t b = __ballot(same);
        if (same && lane == __ffsll((unsigned long long)b) - 1)
          atomicAdd(&hist[k][lead], uint32_t(__popcll(b)));
        if (match && !same) atomicAdd(&hist[k][digit], 1u);
      }
    }
    __syncthreads();
    if (wave < nt) {
      const int k = wave;
      uint32_t c[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j] = hist[k][lane * 4 + j];
      const uint32_t mine = c[0] + c[1] + c[2] + c[3];
      // inclusive scan of the per-lane totals across the wavefront
      uint32_t incl = mine;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t v = __shfl_up(incl, off);
        if (lane >= off) incl += v;
      }
      const int64_t rem = remain[k];
      int64_t before = int64_t(incl - mine);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (rem >= before && rem < before + int64_t(c[j])) {
          prefix[k] = (prefix[k] << 8) | uint32_t(lane * 4 + j);
          remain[k] = rem - before;
        }
        before += c[j];
      }
    }
    __syncthreads();
  }

  // ---- 2. assignment in token order
  for (int64_t base = 0; base < n_tokens; base += kThreads) {
    const int64_t n = base + tid;
    const bool valid = n < n_tokens;
    const uint32_t key = valid ? sort_key(r[n]) : 0u;
    int g = 0;
    uint32_t eq = 0;
    if (valid) {
      for (int k = 0; k < nt; ++k) {
        const uint32_t t = prefix[k];
        g += key > t;
        eq |= uint32_t(key == t) << k;
      }
    }
    if (__syncthreads_or(eq != 0)) {
      for (int k = 0; k < nt; ++k) {
        const bool f = (eq >> k) & 1u;
        const uint64_t ballot = __ballot(f);
        const uint32_t below = __popcll(ballot & ((uint64_t(1) << lane) - 1));
        if (lane == 0) wave_cnt[wave] = __popcll(ballot);
        __syncthreads();
        uint32_t wave_off = 0;
        uint32_t total = 0;
        for (int w = 0; w < kWaves; ++w) {
          const uint32_t c = wave_cnt[w];
          wave_off += (w < wave) ? c : 0u;
          total += c;
        }
        if (f && tie_run[k] + int64_t(wave_off + below) >= remain[k]) ++g;
        __syncthreads();
        if (tid == 0) tie_run[k] += total;
        __syncthreads();
      }
    }
    if (valid) group_id[n] = g;
  }
}

}  // namespace

hipError_t launch_rank(const float* r, int64_t n_tokens, const int64_t* targets, int n_targets,
                       int32_t* group_id, hipStream_t stream) {
  Targets tg{};
  tg.count = n_targets;
  for (int k = 0; k < n_targets && k < kMaxTargets; ++k) tg.pos[k] = targets[k];
  rank_kernel<<<dim3(1), dim3(kThreads), 0, stream>>>(r, n_tokens, tg, group_id);
  return hipGetLastError();
}

}  // namespace hsastep

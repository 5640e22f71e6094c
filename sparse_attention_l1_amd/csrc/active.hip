// Active set A_i of one iteration ("Technische Samenvatting: Heterogene
// Staptoewijzing (HSA) voor Efficiënte Videogeneratie", §2.1: a group with
// budget s_k is active iff i mod (T/s_k) = 0; §2.4: every token is active in
// the first and last m iterations).  The host folds the rule into a bit mask
// over the groups, so the device only tests bit group_id[n].
//
// Compaction keeps ascending token order (the cache slots of the active rows):
//   count kernel:   workgroup b counts the active tokens of its 1024-token chunk
//   compact kernel: workgroup b adds the counts of chunks < b, scans its own
//                   chunk with wavefront ballots, writes active_idx and active_pos.
// Two launches instead of one chained scan: no workgroup ever waits on another.
#include <hip/hip_runtime.h>

#include "host.hpp"
#include "kernels.hpp"

namespace hsastep {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = kActiveBlockTokens / kThreads;   // 4 consecutive tokens per thread
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ bool is_active(int32_t g, uint32_t mask, int n_groups) {
  return g >= 0 && g < n_groups && ((mask >> g) & 1u);
}

__device__ __forceinline__ int load_flags(const int32_t* __restrict__ gid, int64_t n_tokens,
                                          int64_t first, uint32_t mask, int n_groups) {
  int flags = 0;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const int64_t n = first + j;
    if (n < n_tokens && is_active(gid[n], mask, n_groups)) flags |= 1 << j;
  }
  return flags;
}

__global__ __launch_bounds__(kThreads) void active_count_kernel(const int32_t* __restrict__ gid,
                                                                int64_t n_tokens, uint32_t mask,
                                                                int n_groups,
                                                                int32_t* __restrict__ blockcnt) {
  __shared__ int wsum[kWaves];
  const int64_t first = int64_t(blockIdx.x) * kActiveBlockTokens + threadIdx.x * kPerThread;
  int c = __popc(load_flags(gid, n_tokens, first, mask, n_groups));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    int t = 0;
    for (int w = 0; w < kWaves; ++w) t += wsum[w];
    blockcnt[blockIdx.x] = t;
  }
}

__global__ __launch_bounds__(kThreads) void active_compact_kernel(
    const int32_t* __restrict__ gid, int64_t n_tokens, uint32_t mask, int n_groups,
    const int32_t* __restrict__ blockcnt, int32_t* __restrict__ active_idx,
    int32_t* __restrict__ active_pos) {
  __shared__ int64_t part[kWaves];
  __shared__ int wsum[kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // offset of this chunk = active tokens in all earlier chunks
  int64_t acc = 0;
  for (int b = tid; b < int(blockIdx.x); b += kThreads) acc += blockcnt[b];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) part[wave] = acc;

  const int64_t first = int64_t(blockIdx.x) * kActiveBlockTokens + tid * kPerThread;
  const int flags = load_flags(gid, n_tokens, first, mask, n_groups);
  const int mine = __popc(flags);
  // exclusive prefix of per-thread counts inside the wavefront
  int incl = mine;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int64_t base = 0;
  for (int w = 0; w < kWaves; ++w) {
    base += part[w];
    if (w < wave) base += wsum[w];
  }
  int64_t pos = base + (incl - mine);
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const int64_t n = first + j;
    if (n >= n_tokens) break;
    if ((flags >> j) & 1) {
      active_idx[pos] = int32_t(n);
      active_pos[n] = int32_t(pos);
      ++pos;
    } else {
      active_pos[n] = -1;
    }
  }
}

}  // namespace

hipError_t launch_active(const int32_t* group_id, int64_t n_tokens, uint32_t group_mask,
                         int n_groups, int32_t* active_idx, int32_t* active_pos, int32_t* blockcnt,
                         hipStream_t stream) {
  const int64_t nblk = (n_tokens + kActiveBlockTokens - 1) / kActiveBlockTokens;
  active_count_kernel<<<dim3(unsigned(nblk)), dim3(kThreads), 0, stream>>>(
      group_id, n_tokens, group_mask, n_groups, blockcnt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  active_compact_kernel<<<dim3(unsigned(nblk)), dim3(kThreads), 0, stream>>>(
      group_id, n_tokens, group_mask, n_groups, blockcnt, active_idx, active_pos);
  return hipGetLastError();
}

}  // namespace hsastep

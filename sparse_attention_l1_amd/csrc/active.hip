// Active set A_i of one iteration ("Technische Samenvatting: Heterogene
// Staptoewijzing (HSA) voor Efficiënte Videogeneratie", §2.1: a group with
// budget s_k is active iff i mod (T/s_k) = 0; §2.4: every token is active in
// the first and last m iterations).  The host folds the rule into a bit mask
// over the groups, so the device only tests bit group_id[n].
//
// Compaction keeps ascending token order (the cache slots of the active rows):
//   count kernel:   workgroup b counts the active tokens of its 1024-token chunk
//   compact kernel: workgroup b adds the counts of chunks < b, scans its own
//                   chunk with wavefront ballots, writes active_idx and active_pos, and
//                   (hsa_active_set_gather) copies the chunk's active rows of a per-token
//                   array into active order ([HSA-nl] §2.2 item 1: only the active tokens
//                   enter the model).
// Two launches instead of one chained scan: no workgroup ever waits on another.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

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

// Optional fused row gather: rows_out[a] = rows[active_idx[a]], rows of `words` units of Vec.
template <typename Vec>
struct RowGather {
  const Vec* rows;
  Vec* rows_out;
  int64_t words;
};

template <typename Vec, bool kGather>
__global__ __launch_bounds__(kThreads) void active_compact_kernel(
    const int32_t* __restrict__ gid, int64_t n_tokens, uint32_t mask, int n_groups,
    const int32_t* __restrict__ blockcnt, int32_t* __restrict__ active_idx,
    int32_t* __restrict__ active_pos, RowGather<Vec> rg) {
  __shared__ int64_t part[kWaves];
  __shared__ int wsum[kWaves];
  __shared__ int32_t s_tok[kGather ? kActiveBlockTokens : 1];   // this chunk's active tokens
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // with the row gather, gridDim.y workgroups share a chunk: each repeats the chunk's scan
  // (4 KB of group ids), the first writes the index lists, and each copies its share of the
  // chunk's rows, so that the copy runs on many more compute units than there are chunks
  const bool lists = blockIdx.y == 0;

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
  int64_t chunk_first = 0;                     // active tokens in all earlier chunks
  int count = 0;                               // active tokens in this chunk
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    chunk_first += part[w];
    count += wsum[w];
  }
  int64_t pos = base + (incl - mine);
  int local = int(pos - chunk_first);          // position inside the chunk
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const int64_t n = first + j;
    if (n >= n_tokens) break;
    if ((flags >> j) & 1) {
      if (lists) {
        active_idx[pos] = int32_t(n);
        active_pos[n] = int32_t(pos);
      }
      if (kGather) s_tok[local++] = int32_t(n);
      ++pos;
    } else if (lists) {
      active_pos[n] = -1;
    }
  }
  if (kGather) {
    // the chunk's active rows, in active order, from LDS: consecutive threads move
    // consecutive units of a row, so each row is one coalesced segment on both sides
    __syncthreads();
    const int r0 = int(int64_t(count) * blockIdx.y / gridDim.y);
    const int r1 = int(int64_t(count) * (blockIdx.y + 1) / gridDim.y);
    const int64_t total = int64_t(r1 - r0) * rg.words;
    for (int64_t t = tid; t < total; t += kThreads) {
      const int64_t r = r0 + t / rg.words, c = t % rg.words;
      rg.rows_out[(chunk_first + r) * rg.words + c] = rg.rows[int64_t(s_tok[r]) * rg.words + c];
    }
  }
}

// Per-chunk counts of hsa_active_set_noalloc, for callers that cannot allocate: one word per
// 1024-token chunk up to kNoAllocMaxTokens tokens (64 KB), resident on every device the
// library runs on until the process ends.  Host code never passes this name to a kernel (on
// the host it is only a stand-in); it uses the device address hipGetSymbolAddress returns.
constexpr int64_t kScratchWords = kNoAllocMaxTokens / kActiveBlockTokens + 1;
static __device__ __align__(256) int32_t scratch[kScratchWords];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t active_scratch(int32_t** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<int32_t*>(p);
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_active(const int32_t* group_id, int64_t n_tokens, uint32_t group_mask,
                         int n_groups, int32_t* active_idx, int32_t* active_pos, int32_t* blockcnt,
                         hipStream_t stream, const void* rows, int64_t row_bytes,
                         void* rows_out) {
  const int64_t nblk = (n_tokens + kActiveBlockTokens - 1) / kActiveBlockTokens;
  active_count_kernel<<<dim3(unsigned(nblk)), dim3(kThreads), 0, stream>>>(
      group_id, n_tokens, group_mask, n_groups, blockcnt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // gather: about 1024 workgroups in all (4 per compute unit), at most 16 per chunk
  const int64_t share = rows ? std::min<int64_t>(16, std::max<int64_t>(1, 1024 / nblk)) : 1;
  const dim3 grid{unsigned(nblk), unsigned(share)}, block{unsigned(kThreads)};
  const uintptr_t al = reinterpret_cast<uintptr_t>(rows) | reinterpret_cast<uintptr_t>(rows_out);
  if (rows == nullptr) {
    active_compact_kernel<uint32_t, false><<<grid, block, 0, stream>>>(
        group_id, n_tokens, group_mask, n_groups, blockcnt, active_idx, active_pos,
        RowGather<uint32_t>{nullptr, nullptr, 0});
  } else if (row_bytes % 16 == 0 && (al & 15u) == 0) {
    active_compact_kernel<uint4, true><<<grid, block, 0, stream>>>(
        group_id, n_tokens, group_mask, n_groups, blockcnt, active_idx, active_pos,
        RowGather<uint4>{static_cast<const uint4*>(rows), static_cast<uint4*>(rows_out),
                         row_bytes / 16});
  } else {
    active_compact_kernel<uint32_t, true><<<grid, block, 0, stream>>>(
        group_id, n_tokens, group_mask, n_groups, blockcnt, active_idx, active_pos,
        RowGather<uint32_t>{static_cast<const uint32_t*>(rows), static_cast<uint32_t*>(rows_out),
                            row_bytes / 4});
  }
  return hipGetLastError();
}

}  // namespace hsastep

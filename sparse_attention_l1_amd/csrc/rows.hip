// Row movement of the KV-cache synchronisation ("Technische Samenvatting:
// Heterogene Staptoewijzing (HSA) voor Efficiënte Videogeneratie", §2.2):
//   gather:   dst[a] = src[index[a]]                (the active tokens' rows)
//   kv scatter: cache[b, active_idx[a]] = new[b, a]  (fresh K/V overwrite stale slots)
//
// Pure copies, HBM bound: every byte is read once and written once.  One thread
// moves 16 bytes; consecutive threads cover consecutive 16-byte pieces of a row,
// so each row is one contiguous, fully coalesced segment on both sides.  The
// index is read once per piece (it is a broadcast within a row and stays in L1).
#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace hsastep {
namespace {

template <typename Vec>
__global__ __launch_bounds__(256) void gather_kernel(Vec* __restrict__ dst,
                                                     const Vec* __restrict__ src,
                                                     const int32_t* __restrict__ index,
                                                     int64_t n_rows, int64_t n_src_rows,
                                                     int64_t vecs_per_row) {
  const int64_t total = n_rows * vecs_per_row;
  for (int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; t < total;
       t += int64_t(gridDim.x) * blockDim.x) {
    const int64_t a = t / vecs_per_row;
    const int64_t c = t - a * vecs_per_row;
    const int32_t s = index[a];
    Vec v{};
    if (s >= 0 && s < n_src_rows) v = src[int64_t(s) * vecs_per_row + c];
    dst[t] = v;
  }
}

// grid.y = 0 moves K rows, 1 moves V rows
__global__ __launch_bounds__(256) void kv_scatter_kernel(uint4* __restrict__ k_cache,
                                                         uint4* __restrict__ v_cache,
                                                         const uint4* __restrict__ k_new,
                                                         const uint4* __restrict__ v_new,
                                                         const int32_t* __restrict__ active_idx,
                                                         int64_t n_active, int64_t n_tokens,
                                                         int batch, int64_t vecs_per_row) {
  uint4* __restrict__ cache = blockIdx.y == 0 ? k_cache : v_cache;
  const uint4* __restrict__ fresh = blockIdx.y == 0 ? k_new : v_new;
  const int64_t total = int64_t(batch) * n_active * vecs_per_row;
  for (int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; t < total;
       t += int64_t(gridDim.x) * blockDim.x) {
    const int64_t row = t / vecs_per_row;            // b * n_active + a
    const int64_t c = t - row * vecs_per_row;
    const int64_t b = row / n_active;
    const int64_t a = row - b * n_active;
    const int32_t slot = active_idx[a];
    if (slot < 0 || slot >= n_tokens) continue;
    cache[(b * n_tokens + slot) * vecs_per_row + c] = fresh[t];
  }
}

int64_t grid_for(int64_t work) {
  // enough workgroups to fill 256 CUs several times; the loops stride over the rest
  const int64_t blocks = (work + 255) / 256;
  return blocks < 65536 ? (blocks > 0 ? blocks : 1) : 65536;
}

}  // namespace

hipError_t launch_gather(void* dst, const void* src, const int32_t* index, int64_t n_rows,
                         int64_t n_src_rows, int64_t row_bytes, hipStream_t stream) {
  const uintptr_t al = reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(src);
  if (row_bytes % 16 == 0 && (al & 15u) == 0) {
    const int64_t vpr = row_bytes / 16;
    gather_kernel<uint4><<<dim3(unsigned(grid_for(n_rows * vpr))), dim3(256), 0, stream>>>(
        static_cast<uint4*>(dst), static_cast<const uint4*>(src), index, n_rows, n_src_rows, vpr);
  } else {
    const int64_t vpr = row_bytes / 4;
    gather_kernel<uint32_t><<<dim3(unsigned(grid_for(n_rows * vpr))), dim3(256), 0, stream>>>(
        static_cast<uint32_t*>(dst), static_cast<const uint32_t*>(src), index, n_rows, n_src_rows,
        vpr);
  }
  return hipGetLastError();
}

hipError_t launch_kv_update(uint16_t* k_cache, uint16_t* v_cache, const uint16_t* k_new,
                            const uint16_t* v_new, const int32_t* active_idx, int64_t n_active,
                            int64_t n_tokens, int batch, int heads, int head_dim,
                            hipStream_t stream) {
  const int64_t vpr = int64_t(heads) * head_dim / 8;   // 16-byte pieces per row
  const int64_t work = int64_t(batch) * n_active * vpr;
  kv_scatter_kernel<<<dim3(unsigned(grid_for(work)), 2), dim3(256), 0, stream>>>(
      reinterpret_cast<uint4*>(k_cache), reinterpret_cast<uint4*>(v_cache),
      reinterpret_cast<const uint4*>(k_new), reinterpret_cast<const uint4*>(v_new), active_idx,
      n_active, n_tokens, batch, vpr);
  return hipGetLastError();
}

}  // namespace hsastep

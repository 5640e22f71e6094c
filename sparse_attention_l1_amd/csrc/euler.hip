// Cached Euler update ("Technische Samenvatting: Heterogene Staptoewijzing
// (HSA) voor Efficiënte Videogeneratie", §2.3): every token stores the velocity
// of its latest active step; all N tokens advance by the same increment
// dt = sigma_{i+1} - sigma_i, active tokens with their fresh velocity, skipped
// ones with the cached one, in one pass without divergent control flow.
//
//   v   = active ? v_fresh[active_pos[n]] : v_cache[n]   (address select, not a branch)
//   v_cache[n] = v                                        (store predicated on active)
//   x[n] = fl(x[n] + fl(dt * v))                          (no fused multiply-add)
//
// HBM bound: reads x, one velocity row and active_pos, writes x and the fresh
// rows into the cache.  One thread handles 4 channels (16-byte accesses).
#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace hsastep {
namespace {

__global__ __launch_bounds__(256) void euler_vec4_kernel(float4* __restrict__ x,
                                                         float4* __restrict__ v_cache,
                                                         const float4* __restrict__ v_fresh,
                                                         const int32_t* __restrict__ active_pos,
                                                         int64_t n_active, int64_t n_tokens,
                                                         int vecs_per_row, float dt) {
#pragma clang fp contract(off)
  const int64_t total = n_tokens * vecs_per_row;
  for (int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; t < total;
       t += int64_t(gridDim.x) * blockDim.x) {
    const int64_t n = t / vecs_per_row;
    const int64_t c = t - n * vecs_per_row;
    const int32_t pos = active_pos[n];
    const bool act = pos >= 0 && pos < n_active;
    const float4* src = act ? v_fresh + int64_t(pos) * vecs_per_row + c : v_cache + t;
    const float4 v = *src;
    float4 xv = x[t];
    if (act) v_cache[t] = v;
    // contraction is off in this scope (and for the file): product, then sum
    xv.x = xv.x + dt * v.x;
    xv.y = xv.y + dt * v.y;
    xv.z = xv.z + dt * v.z;
    xv.w = xv.w + dt * v.w;
    x[t] = xv;
  }
}

__global__ __launch_bounds__(256) void euler_scalar_kernel(float* __restrict__ x,
                                                           float* __restrict__ v_cache,
                                                           const float* __restrict__ v_fresh,
                                                           const int32_t* __restrict__ active_pos,
                                                           int64_t n_active, int64_t n_tokens,
                                                           int channels, float dt) {
#pragma clang fp contract(off)
  const int64_t total = n_tokens * channels;
  for (int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; t < total;
       t += int64_t(gridDim.x) * blockDim.x) {
    const int64_t n = t / channels;
    const int64_t c = t - n * channels;
    const int32_t pos = active_pos[n];
    const bool act = pos >= 0 && pos < n_active;
    const float* src = act ? v_fresh + int64_t(pos) * channels + c : v_cache + t;
    const float v = *src;
    if (act) v_cache[t] = v;
    x[t] = x[t] + dt * v;   // no contraction: see the pragma
  }
}

}  // namespace

hipError_t launch_euler(float* x, float* v_cache, const float* v_fresh, const int32_t* active_pos,
                        int64_t n_active, int64_t n_tokens, int channels, float sigma_cur,
                        float sigma_next, hipStream_t stream) {
  const float dt = sigma_next - sigma_cur;   // one fp32 rounding
  const bool vec = channels % 4 == 0;
  const int64_t work = n_tokens * (vec ? channels / 4 : channels);
  int64_t blocks = (work + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (vec)
    euler_vec4_kernel<<<dim3(unsigned(blocks)), dim3(256), 0, stream>>>(
        reinterpret_cast<float4*>(x), reinterpret_cast<float4*>(v_cache),
        reinterpret_cast<const float4*>(v_fresh), active_pos, n_active, n_tokens, channels / 4,
        dt);
  else
    euler_scalar_kernel<<<dim3(unsigned(blocks)), dim3(256), 0, stream>>>(
        x, v_cache, v_fresh, active_pos, n_active, n_tokens, channels, dt);
  return hipGetLastError();
}

}  // namespace hsastep

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
// rows into the cache.  A thread handles kItems 16-byte pieces (4 channels each) and
// issues all their loads before using any.  The velocity row depends on active_pos, so
// the x loads go out with the active_pos loads and overlap that first latency.
#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace hsastep {
namespace {

constexpr int kItems = 4;   // 16-byte pieces per thread

// Every byte is touched once per call, so loads and stores carry the nontemporal hint
// (streamed through the caches instead of kept there); with inputs in HBM this moves
// about a fifth more bytes per second than plain accesses.
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load_stream(const float4* p) {
  return __builtin_bit_cast(float4, __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p)));
}
__device__ __forceinline__ void store_stream(float4* p, const float4& v) {
  __builtin_nontemporal_store(__builtin_bit_cast(f32x4, v), reinterpret_cast<f32x4*>(p));
}

// One group of kItems pieces per thread: piece k is base + k * 256, so consecutive threads
// stay on consecutive 16-byte pieces.  The active-position and x loads are issued together
// (x does not depend on the position), then the velocity loads that do; stores come last.
// kFull: every piece of the group is in range (block-uniform), so no piece is predicated.
template <typename Idx, bool kFull>
__device__ __forceinline__ void euler_group(float4* __restrict__ x, float4* __restrict__ v_cache,
                                            const float4* __restrict__ v_fresh,
                                            const int32_t* __restrict__ active_pos,
                                            int64_t n_active, Idx total, Idx vecs_per_row,
                                            float dt, Idx base) {
#pragma clang fp contract(off)
  int32_t pos[kItems];
  float4 xv[kItems], v[kItems];
#pragma unroll
  for (int k = 0; k < kItems; ++k) {
    const Idx t = base + Idx(k) * 256u;
    pos[k] = -1;
    if (kFull || t < total) {
      pos[k] = active_pos[t / vecs_per_row];
      xv[k] = load_stream(x + t);
    }
  }
#pragma unroll
  for (int k = 0; k < kItems; ++k) {
    const Idx t = base + Idx(k) * 256u;
    if (kFull || t < total) {
      const bool act = pos[k] >= 0 && pos[k] < n_active;
      const float4* src =
          act ? v_fresh + int64_t(pos[k]) * vecs_per_row + (t % vecs_per_row) : v_cache + t;
      v[k] = load_stream(src);
    }
  }
#pragma unroll
  for (int k = 0; k < kItems; ++k) {
    const Idx t = base + Idx(k) * 256u;
    if (kFull || t < total) {
      if (pos[k] >= 0 && pos[k] < n_active) store_stream(v_cache + t, v[k]);
      // contraction is off in this scope (and for the file): product, then sum
      xv[k].x = xv[k].x + dt * v[k].x;
      xv[k].y = xv[k].y + dt * v[k].y;
      xv[k].z = xv[k].z + dt * v[k].z;
      xv[k].w = xv[k].w + dt * v[k].w;
      store_stream(x + t, xv[k]);
    }
  }
}

// Idx: 32-bit piece indices when the latent has fewer than 2^31 pieces (cheap division)
template <typename Idx>
__global__ __launch_bounds__(256) void euler_vec4_kernel(float4* __restrict__ x,
                                                         float4* __restrict__ v_cache,
                                                         const float4* __restrict__ v_fresh,
                                                         const int32_t* __restrict__ active_pos,
                                                         int64_t n_active, Idx total,
                                                         Idx vecs_per_row, float dt) {
  constexpr Idx span = 256u * kItems;
  for (Idx first = Idx(blockIdx.x) * span; first < total; first += Idx(gridDim.x) * span) {
    const Idx base = first + threadIdx.x;
    if (total - first >= span)
      euler_group<Idx, true>(x, v_cache, v_fresh, active_pos, n_active, total, vecs_per_row, dt,
                             base);
    else
      euler_group<Idx, false>(x, v_cache, v_fresh, active_pos, n_active, total, vecs_per_row, dt,
                              base);
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
  const int64_t per_block = vec ? 256 * kItems : 256;
  int64_t blocks = (work + per_block - 1) / per_block;
  if (blocks > 65536) blocks = 65536;
  if (vec && work + 256 * kItems < (int64_t(1) << 31))
    euler_vec4_kernel<uint32_t><<<dim3(unsigned(blocks)), dim3(256), 0, stream>>>(
        reinterpret_cast<float4*>(x), reinterpret_cast<float4*>(v_cache),
        reinterpret_cast<const float4*>(v_fresh), active_pos, n_active, uint32_t(work),
        uint32_t(channels / 4), dt);
  else if (vec)
    euler_vec4_kernel<uint64_t><<<dim3(unsigned(blocks)), dim3(256), 0, stream>>>(
        reinterpret_cast<float4*>(x), reinterpret_cast<float4*>(v_cache),
        reinterpret_cast<const float4*>(v_fresh), active_pos, n_active, uint64_t(work),
        uint64_t(channels / 4), dt);
  else
    euler_scalar_kernel<<<dim3(unsigned(blocks)), dim3(256), 0, stream>>>(
        x, v_cache, v_fresh, active_pos, n_active, n_tokens, channels, dt);
  return hipGetLastError();
}

}  // namespace hsastep

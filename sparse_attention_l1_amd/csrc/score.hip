// Per-token L1 relative change of the velocity prediction (Dynamic Token
// Selection, "Technische Samenvatting: Heterogene Staptoewijzing (HSA) voor
// Efficiënte Videogeneratie", §2.1):
//     r_n = ||v_cur[n] - v_prev[n]||_1 / ||v_prev[n]||_1      (fp32)
//
// HBM-bound streaming kernel: 2*N*C*4 bytes read, 4*N written.  A token's C
// channels are spread over P lanes (4 consecutive channels per lane, one 16-byte
// load each, so a C = 64 row is one 256-byte coalesced segment).  Each sum is a
// balanced pairwise tree: a lane adds its 4 values as (a0+a1)+(a2+a3), then the
// P lanes combine with an xor butterfly over offsets 1, 2, 4, ...; because fp32
// addition is commutative, every lane ends with exactly the level-by-level tree
// over the zero-padded channels, so the score is bit-reproducible.
#include <hip/hip_runtime.h>

#include <cmath>

#include "kernels.hpp"

namespace hsastep {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int P, bool kVec4>
__global__ __launch_bounds__(256) void score_kernel(const float* __restrict__ v_prev,
                                                    const float* __restrict__ v_cur,
                                                    int64_t n_tokens, int channels,
                                                    float* __restrict__ r,
                                                    uint32_t* __restrict__ zero,
                                                    int64_t zero_words) {
#pragma clang fp contract(off)
  const int64_t tid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  for (int64_t i = tid; i < zero_words; i += int64_t(gridDim.x) * blockDim.x) zero[i] = 0u;
  const int64_t token = tid / P;
  const int lane = int(tid % P);
  // groups of P lanes are aligned inside a wavefront, so a whole group leaves together
  if (token >= n_tokens) return;
  const int c0 = lane * 4;
  const int64_t row = token * channels;
  float p[4], c[4];
  if (kVec4) {
    // channels % 4 == 0 here: c0 < channels or the whole lane is padding
    if (c0 < channels) {
      // read once per call: nontemporal loads stream the rows through the caches
      const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(v_prev + row + c0));
      const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(v_cur + row + c0));
      p[0] = a.x; p[1] = a.y; p[2] = a.z; p[3] = a.w;
      c[0] = b.x; c[1] = b.y; c[2] = b.z; c[3] = b.w;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) p[j] = c[j] = 0.0f;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool in = c0 + j < channels;
      p[j] = in ? v_prev[row + c0 + j] : 0.0f;
      c[j] = in ? v_cur[row + c0 + j] : 0.0f;
    }
  }
  float d[4], a[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    d[j] = fabsf(c[j] - p[j]);
    a[j] = fabsf(p[j]);
  }
  float num = (d[0] + d[1]) + (d[2] + d[3]);
  float den = (a[0] + a[1]) + (a[2] + a[3]);
#pragma unroll
  for (int off = 1; off < P; off <<= 1) {
    num = num + __shfl_xor(num, off);
    den = den + __shfl_xor(den, off);
  }
  if (lane == 0) {
    float q;
    if (den == 0.0f)
      q = (num == 0.0f) ? 0.0f : INFINITY;
    else
      q = num / den;   // IEEE round-to-nearest (correctly rounded divide is on)
    if (q != q) q = INFINITY;   // NaN -> +inf
    r[token] = q;
  }
}

template <int P>
hipError_t launch_p(const float* vp, const float* vc, int64_t n, int ch, float* r, uint32_t* z,
                    int64_t zw, hipStream_t s) {
  const int64_t threads = n * P;
  const int block = 256;
  const int64_t grid = (threads + block - 1) / block;
  if (ch % 4 == 0)
    score_kernel<P, true><<<dim3(unsigned(grid)), dim3(block), 0, s>>>(vp, vc, n, ch, r, z, zw);
  else
    score_kernel<P, false><<<dim3(unsigned(grid)), dim3(block), 0, s>>>(vp, vc, n, ch, r, z, zw);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_score(const float* v_prev, const float* v_cur, int64_t n_tokens, int channels,
                        float* r, uint32_t* zero, int64_t zero_words, hipStream_t stream) {
  // lanes per token: next power of two of ceil(C/4), at least 1, at most 64 (C <= 256)
  const int need = (channels + 3) / 4;
  int p = 1;
  while (p < need) p <<= 1;
  switch (p) {
    case 1: return launch_p<1>(v_prev, v_cur, n_tokens, channels, r, zero, zero_words, stream);
    case 2: return launch_p<2>(v_prev, v_cur, n_tokens, channels, r, zero, zero_words, stream);
    case 4: return launch_p<4>(v_prev, v_cur, n_tokens, channels, r, zero, zero_words, stream);
    case 8: return launch_p<8>(v_prev, v_cur, n_tokens, channels, r, zero, zero_words, stream);
    case 16: return launch_p<16>(v_prev, v_cur, n_tokens, channels, r, zero, zero_words, stream);
    case 32: return launch_p<32>(v_prev, v_cur, n_tokens, channels, r, zero, zero_words, stream);
    default: return launch_p<64>(v_prev, v_cur, n_tokens, channels, r, zero, zero_words, stream);
  }
}

}  // namespace hsastep

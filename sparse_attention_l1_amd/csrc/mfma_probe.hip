// Measurement utility, not a step of the method: the sustained rate of the bf16 MFMA that the
// attention kernel is built on (v_mfma_f32_32x32x16_bf16), on every compute unit, with finite
// non-zero operands that change from one MFMA to the next.  The dense peak quoted for the chip
// assumes the full clock; under sustained MFMA load the chip manages its power and holds a
// lower one, so this rate (and the clock it runs at) is the ceiling an MFMA-bound kernel can
// actually approach.  Zero operands draw less power and let the clock stay higher, so a caller
// that passes zeros measures an optimistic ceiling.
//
// A workgroup is 4 wavefronts (one per SIMD, as in the attention kernel).  Each wavefront keeps
// 8 independent 32x32x16 accumulators and cycles through 8 A and 8 B operand sets read once
// from the operand buffer, so no MFMA waits on the previous one's result.
#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace hsastep {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void mfma_probe_kernel(const bf16x8* __restrict__ operands,
                                                        float* __restrict__ sink, int rounds) {
  const int lane = threadIdx.x & 63;
  bf16x8 a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = operands[i * 64 + lane];
    b[i] = operands[512 + i * 64 + lane];
  }
  f32x16 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x16{};
  for (int r = 0; r < rounds; ++r) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int k = 0; k < 8; ++k)
        acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[k], b[(k + j) & 7], acc[k], 0, 0, 0);
  }
  // the accumulators reach memory, so no MFMA can be dropped
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += acc[i][j];
  sink[blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_mfma_probe(const uint16_t* operands, float* sink, int rounds, int workgroups,
                             hipStream_t stream) {
  mfma_probe_kernel<<<dim3(unsigned(workgroups)), dim3(256), 0, stream>>>(
      reinterpret_cast<const bf16x8*>(operands), sink, rounds);
  return hipGetLastError();
}

}  // namespace hsastep

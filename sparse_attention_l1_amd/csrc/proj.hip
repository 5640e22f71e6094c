// Fused QKV projection of the active tokens, with the KV-cache write as its epilogue
// ("Technische Samenvatting: Heterogene Staptoewijzing (HSA) voor Efficiënte
// Videogeneratie", §2.2 items 1-2: only the active tokens go through the projections, and
// their fresh K/V rows overwrite their slots in the per-layer cache):
//     Y = X_A W^T (+ bias)           X_A [B*|A|, Dm] bf16 (active order), W [3*H*D, Dm] bf16
//     Y[:, 0:HD)     -> q_out[b, a]                       (compacted, active order)
//     Y[:, HD:2HD)   -> k_cache[b, active_idx[a]]         (slot = token index)
//     Y[:, 2HD:3HD)  -> v_cache[b, active_idx[a]]
// so the K/V rows never make a round trip through a separate buffer and scatter.
//
// gfx950 design (bf16 MFMA bound: 2 * B*|A| * Dm * 3HD flops):
//   - A workgroup computes a 256 x 256 tile of Y with 8 wavefronts, two per SIMD (4 along
//     rows x 2 along columns, 64 x 128 each = 2 x 4 blocks of v_mfma_f32_32x32x16_bf16,
//     fp32 accumulate).  Four wavefronts of 128 x 128 (fewer LDS reads per MFMA, one wave
//     per SIMD) measured slower with compiler scheduling.
//   - Both operands are K-contiguous (X rows, W rows), so every fragment is one 16-byte
//     LDS read; the reduction dimension walks in 64-element stages.
//   - Stages travel global -> LDS with direct loads (global_load_lds, 16 bytes per lane),
//     double buffered, one barrier per stage; fragments are double buffered in registers
//     so the next k-step's LDS reads overlap the current MFMAs.  Rows are 128 bytes with a 16-byte-chunk XOR swizzle, chunk ^
//     ((row >> 1) & 7), which keeps the 16 rows a fragment read touches on distinct banks.
//   - Rows past the end of X or W are clamped to the last row (finite data, never stored).
//   - Workgroup order is XCD aware: each XCD walks a contiguous range of tiles, column
//     tiles fastest, so a row tile of X is fetched into one XCD's L2 once.
//   - The epilogue adds the bias in fp32, rounds to bf16 and stores each value straight to
//     its destination row: a wavefront's store covers two rows x 32 consecutive columns.
#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace hsastep {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(1))) void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

constexpr int kWaitVm0 = 0x0F70;   // s_waitcnt vmcnt(0) (expcnt and lgkmcnt unconstrained)
constexpr int kBM = 256, kBN = 256, kBK = 64;

struct ProjArgs {
  const uint16_t* x;
  const uint16_t* w;
  const uint16_t* bias;   // [3HD] bf16 or null
  uint16_t* q_out;
  uint16_t* k_cache;
  uint16_t* v_cache;
  const int32_t* active_idx;
  int m_rows;     // B * |A|
  int n_active;
  int n_tokens;
  int n_out;      // 3 * H * D
  int hd;         // H * D
  int dm;         // model dim, a multiple of kBK
  int n_ntiles;
  int total_blocks;
};

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(uint32_t(b) << 16);
}

// NWM x NWN wavefronts, each IM x JN blocks of 32 x 32 (NWM*IM*32 = NWN*JN*32 = 256)
template <int NWM, int NWN, int WPE>
__global__ __launch_bounds__(64 * NWM * NWN) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void proj_kernel(
    ProjArgs a) {
  constexpr int kThreads = 64 * NWM * NWN;
  constexpr int NW = NWM * NWN;
  constexpr int IM = kBM / 32 / NWM, JN = kBN / 32 / NWN;
  constexpr int kLoads = kBM * kBK / 8 / kThreads;   // 16-byte direct loads per operand per lane
  static_assert(kBM == kBN, "one load pattern serves both operands");
  __shared__ __attribute__((aligned(16))) uint16_t as[2][kBM * kBK];
  __shared__ __attribute__((aligned(16))) uint16_t bs[2][kBN * kBK];

  const int L = blockIdx.x;
  const int xcd = L & 7, per = a.total_blocks >> 3, rem = a.total_blocks & 7;
  const int Lp = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + (L >> 3);
  const int mt = Lp / a.n_ntiles, nt = Lp % a.n_ntiles;
  const int m0 = mt * kBM, n0 = nt * kBN;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / NWN, wn = wave % NWN;
  const int g = lane >> 5, lq = lane & 31;

  // direct loads: load i of this wavefront fills 16-byte slot s = (i*8 + wave)*64 + lane of
  // a stage, i.e. row s/8 at chunk s%8, which holds logical chunk (s%8) ^ swz(row)
  uint32_t aoff[kLoads], boff[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int s = (i * NW + wave) * 64 + lane;
    const int row = s >> 3;
    const int logical = (s & 7) ^ swz(row);
    const int arow = min(m0 + row, a.m_rows - 1);
    const int brow = min(n0 + row, a.n_out - 1);
    aoff[i] = (uint32_t(arow) * uint32_t(a.dm) + uint32_t(8 * logical)) * 2u;
    boff[i] = (uint32_t(brow) * uint32_t(a.dm) + uint32_t(8 * logical)) * 2u;
  }
  auto issue = [&](int kk, int dst) {
    const char* xs = reinterpret_cast<const char*>(a.x) + size_t(kk) * kBK * 2;
    const char* ws = reinterpret_cast<const char*>(a.w) + size_t(kk) * kBK * 2;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      __builtin_amdgcn_global_load_lds((gptr_t)(xs + aoff[i]), (lptr_t)&as[dst][(i * NW + wave) * 512],
                                       16, 0, 0);
      __builtin_amdgcn_global_load_lds((gptr_t)(ws + boff[i]), (lptr_t)&bs[dst][(i * NW + wave) * 512],
                                       16, 0, 0);
    }
  };

  f32x16 acc[IM][JN];
#pragma unroll
  for (int i = 0; i < IM; ++i)
#pragma unroll
    for (int j = 0; j < JN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // fragment rows of this lane and their swizzles
  int arow[IM], brow[JN];
#pragma unroll
  for (int i = 0; i < IM; ++i) arow[i] = wm * IM * 32 + i * 32 + lq;
#pragma unroll
  for (int j = 0; j < JN; ++j) brow[j] = wn * JN * 32 + j * 32 + lq;

  // fragments of k-step u of a stage, double buffered in registers: the reads of step u+1
  // (and, across the stage boundary, of the next stage's step 0) are in flight while the
  // MFMAs of step u run
  bf16x8 af[2][IM], bf[2][JN];
  auto read_frags = [&](int buf, int u, int slot) {
    const int chunk = 2 * u + g;
#pragma unroll
    for (int i = 0; i < IM; ++i)
      af[slot][i] =
          *reinterpret_cast<const bf16x8*>(&as[buf][arow[i] * kBK + 8 * (chunk ^ swz(arow[i]))]);
#pragma unroll
    for (int j = 0; j < JN; ++j)
      bf[slot][j] =
          *reinterpret_cast<const bf16x8*>(&bs[buf][brow[j] * kBK + 8 * (chunk ^ swz(brow[j]))]);
  };
  auto mfmas = [&](int slot) {
#pragma unroll
    for (int i = 0; i < IM; ++i)
#pragma unroll
      for (int j = 0; j < JN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[slot][i], bf[slot][j], acc[i][j],
                                                            0, 0, 0);
  };

  // one barrier per stage, before the last k-step's MFMAs: after it the next stage's loads
  // have landed for every wavefront and nobody reads this stage's buffer any more, so the
  // stage after next is issued into it
  const int nk = a.dm / kBK;
  issue(0, 0);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();
  if (nk > 1) issue(1, 1);
  read_frags(0, 0, 0);
  for (int kk = 0; kk < nk; ++kk) {
    const int buf = kk & 1;
#pragma unroll
    for (int u = 0; u < kBK / 16; ++u) {
      if (u + 1 < kBK / 16) {
        read_frags(buf, u + 1, (u + 1) & 1);
      } else if (kk + 1 < nk) {
        __builtin_amdgcn_s_waitcnt(kWaitVm0);   // the next stage's direct loads have landed
        __syncthreads();                        // ... for every wavefront; this buffer is free
        if (kk + 2 < nk) issue(kk + 2, buf);
        read_frags(buf ^ 1, 0, 0);
      }
      mfmas(u & 1);
    }
  }

  // ---- epilogue: register r of block (i, j) is row wm*IM*32 + 32i + 8(r/4) + 4g + r%4 and
  // column wn*JN*32 + 32j + lq of the tile.  Per row block i, the destination rows first:
  // the compacted row for Q, the cache row b*N + active_idx[a] for K and V (-1: past the
  // end, or a slot outside the cache).
  const int64_t HD = a.hd;
#pragma unroll
  for (int i = 0; i < IM; ++i) {
    int qrow[16], crow[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + wm * IM * 32 + i * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
      qrow[r] = -1;
      crow[r] = -1;
      if (m < a.m_rows) {
        const int b = m / a.n_active;
        const int slot = a.active_idx[m - b * a.n_active];
        qrow[r] = m;
        if (slot >= 0 && slot < a.n_tokens) crow[r] = b * a.n_tokens + slot;
      }
    }
#pragma unroll
    for (int j = 0; j < JN; ++j) {
      const int n = n0 + wn * JN * 32 + j * 32 + lq;
      if (n >= a.n_out) continue;
      const float bias = a.bias ? bf16_to_f32(a.bias[n]) : 0.0f;
      const int part = n / a.hd;
      const int c = n - part * a.hd;
      uint16_t* base = part == 0 ? a.q_out : (part == 1 ? a.k_cache : a.v_cache);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = part == 0 ? qrow[r] : crow[r];
        if (row < 0) continue;
        const __bf16 v = (__bf16)(acc[i][j][r] + bias);
        base[int64_t(row) * HD + c] = __builtin_bit_cast(uint16_t, v);
      }
    }
  }
}

}  // namespace

hipError_t launch_qkv_project(const uint16_t* x, const uint16_t* w, const uint16_t* bias,
                              uint16_t* q_out, uint16_t* k_cache, uint16_t* v_cache,
                              const int32_t* active_idx, int64_t n_active, int64_t n_tokens,
                              int batch, int heads, int head_dim, int model_dim,
                              hipStream_t stream) {
  ProjArgs a{};
  a.x = x;
  a.w = w;
  a.bias = bias;
  a.q_out = q_out;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.active_idx = active_idx;
  a.m_rows = int(int64_t(batch) * n_active);
  a.n_active = int(n_active);
  a.n_tokens = int(n_tokens);
  a.hd = heads * head_dim;
  a.n_out = 3 * a.hd;
  a.dm = model_dim;
  const int n_mtiles = (a.m_rows + kBM - 1) / kBM;
  a.n_ntiles = (a.n_out + kBN - 1) / kBN;
  a.total_blocks = n_mtiles * a.n_ntiles;
  proj_kernel<4, 2, 2><<<dim3(unsigned(a.total_blocks)), dim3(512), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace hsastep

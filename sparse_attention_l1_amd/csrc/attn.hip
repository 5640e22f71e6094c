// Active-query full-context attention ("Technische Samenvatting: Heterogene
// Staptoewijzing (HSA) voor Efficiënte Videogeneratie", §2.2 items 3-4): the
// |A_i| active queries attend to all N cached keys/values of their (b, h),
//     O = softmax(Q_A K^T * scale) V,        cost O(|A_i| * N),
// with no mask.  The queries arrive compacted (active order), so the tiles are
// dense even though the active set is scattered over the token grid.
//
// gfx950 design (bf16 MFMA bound: 4*|A|*N*D flops per (b, h)):
//   - workgroup = 4 wavefronts x 32 queries (128 queries of one (b, h));
//     the key loop walks all N keys in tiles of 64.
//   - Computed transposed: S^T = K Q^T and O^T = V^T P^T with
//     v_mfma_f32_32x32x16_bf16.  Q^T stays in registers as the B operand; K and
//     V^T tiles are the A operands, read from LDS.  In the 32x32 accumulator a
//     lane owns one column, i.e. one query, so the row max / row sum of the
//     online softmax are per-lane register reductions (the two lanes l, l^32
//     hold the two halves of a query's keys).
//   - K rows are fed to the MFMA in a permuted order (bits 2 and 3 of the row
//     swapped) so that each lane's accumulator registers hold 8 consecutive keys;
//     they are then exactly the B operand (P^T) of the P.V MFMA, with no
//     cross-lane shuffle.
//   - K tile in LDS row-major, V tile transposed (V^T: d-major), both with
//     16-byte-chunk XOR swizzles that make the MFMA operand reads and the tile
//     writes bank-conflict free.  Tiles are double buffered: the next tile's
//     global loads are in flight while the current one is multiplied.
//   - fp32 online softmax in base 2 (scale * log2 e folded into one FMA).  The
//     running max is only raised when a tile's max exceeds it by more than
//     2^8, so the O rescale is rare; the result is exact in real arithmetic for
//     any reference max, and the bound keeps P <= 2^8 in bf16/fp32 range.
//   - Workgroup order is XCD aware: consecutive workgroup ids go to different
//     XCDs, so ids are remapped so each XCD walks a contiguous range of query
//     tiles of the same head, whose K/V then stream through that XCD's L2 once.
#include <hip/hip_runtime.h>

#include <cmath>

#include "kernels.hpp"

namespace hsastep {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kBM = 128;      // queries per workgroup
constexpr int kBN = 64;       // keys per tile
constexpr float kTau = 8.0f;  // lazy-rescale threshold, log2 units

// 16-byte chunk swizzle of the K tile (row = key, D/8 chunks per row)
template <int D>
__device__ __forceinline__ int kswz(int r) {
  if constexpr (D == 128)
    return r & 15;
  else
    return (r & 3) | (((r >> 3) & 1) << 2);
}
// 16-byte chunk swizzle of the V^T tile (row = d, 8 chunks of 8 keys per row)
__device__ __forceinline__ int vswz(int d) { return (d & 7) ^ ((d >> 3) & 7); }
// MFMA A-row r reads key perm_row(r): bits 2 and 3 swapped
__device__ __forceinline__ int perm_row(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);   // (b.lo << 16) | a.lo
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);   // (b.hi << 16) | a.hi
}
__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, uint16_t* __restrict__ out, int n_active, int n_tokens,
    int heads, int n_qtiles, int total_blocks, float c_log2) {
  constexpr int CH = D / 8;                        // 16-byte chunks per K row
  constexpr int KL = kBN * CH / kThreads;          // K chunks loaded per thread (4 or 2)
  constexpr int NE = D / 32;                       // 32-row blocks of O^T
  constexpr int NU = D / 16;                       // MFMA k-steps over d
  __shared__ __attribute__((aligned(16))) uint16_t ks[2][kBN * D];
  __shared__ __attribute__((aligned(16))) uint16_t vt[2][D * kBN];

  // ---- XCD-aware tile order
  const int L = blockIdx.x;
  const int xcd = L & 7, per = total_blocks >> 3, rem = total_blocks & 7;
  const int Lp = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + (L >> 3);
  const int qt = Lp % n_qtiles;
  const int bh = Lp / n_qtiles;
  const int h = bh % heads;
  const int b = bh / heads;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, lq = lane & 31;
  const int64_t HD = int64_t(heads) * D;

  // ---- Q^T fragments (B operand): query lq of this wavefront, d = 16u + 8g .. +7
  const int qi = qt * kBM + wave * 32 + lq;
  const bool qvalid = qi < n_active;
  bf16x8 qf[NU];
  {
    const uint16_t* qrow = q + ((int64_t(b) * n_active + (qvalid ? qi : 0)) * heads + h) * D;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      bf16x8 z = {};
      qf[u] = qvalid ? *reinterpret_cast<const bf16x8*>(qrow + 16 * u + 8 * g) : z;
    }
  }

  const uint16_t* kbase = kc + (int64_t(b) * n_tokens * heads + h) * D;
  const uint16_t* vbase = vc + (int64_t(b) * n_tokens * heads + h) * D;

  // ---- tile loader mapping
  // K: thread covers chunk kc_c of rows kc_r + j * (kThreads / CH)
  const int kc_c = tid % CH;
  const int kc_r = tid / CH;
  // V: thread covers 4 keys (4*vg .. 4*vg+3) x 8 d (8*vcn .. +7); D = 64 uses 128 threads
  int vcn, vg;
  if constexpr (D == 128) {
    vcn = (tid & 7) + 8 * ((tid >> 4) & 1);
    vg = ((tid >> 3) & 1) + 2 * (tid >> 5);
  } else {
    vcn = tid & 7;
    vg = ((tid >> 3) & 1) + 2 * ((tid >> 4) & 7);
  }
  const bool vload = (D == 128) || tid < 128;

  uint4 kreg[KL], vreg[4];
  auto load_tile = [&](int kt) {
    const int k0 = kt * kBN;
#pragma unroll
    for (int j = 0; j < KL; ++j) {
      const int key = k0 + kc_r + j * (kThreads / CH);
      kreg[j] = key < n_tokens ? *reinterpret_cast<const uint4*>(kbase + int64_t(key) * HD + 8 * kc_c)
                               : make_uint4(0, 0, 0, 0);
    }
    if (vload) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = k0 + 4 * vg + j;
        vreg[j] = key < n_tokens
                      ? *reinterpret_cast<const uint4*>(vbase + int64_t(key) * HD + 8 * vcn)
                      : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int j = 0; j < KL; ++j) {
      const int r = kc_r + j * (kThreads / CH);
      *reinterpret_cast<uint4*>(&ks[buf][r * D + 8 * (kc_c ^ kswz<D>(r))]) = kreg[j];
    }
    if (vload) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = 8 * vcn + e;
        const int w = e >> 1;
        uint32_t w0, w1;
        if (e & 1) {
          w0 = pack_hi(word(vreg[0], w), word(vreg[1], w));
          w1 = pack_hi(word(vreg[2], w), word(vreg[3], w));
        } else {
          w0 = pack_lo(word(vreg[0], w), word(vreg[1], w));
          w1 = pack_lo(word(vreg[2], w), word(vreg[3], w));
        }
        const int phys = (vg >> 1) ^ vswz(d);
        *reinterpret_cast<uint2*>(&vt[buf][d * kBN + 8 * phys + 4 * (vg & 1)]) = make_uint2(w0, w1);
      }
    }
  };

  f32x16 oacc[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e)
#pragma unroll
    for (int j = 0; j < 16; ++j) oacc[e][j] = 0.0f;
  float m_run = -INFINITY;   // running max, log2 units, identical in lanes l and l^32
  float l_run = 0.0f;        // this lane's half of the row sum

  const int ntiles = (n_tokens + kBN - 1) / kBN;
  const bool ragged = (n_tokens % kBN) != 0;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int kt = 0; kt < ntiles; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < ntiles;
    if (more) load_tile(kt + 1);

    // ---- S^T = K Q^T for two 32-key blocks
    f32x16 sacc[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int j = 0; j < 16; ++j) sacc[s][j] = 0.0f;
      const int r = 32 * s + perm_row(lq);
      const uint16_t* krow = &ks[buf][r * D];
      const int sw = kswz<D>(r);
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(krow + 8 * ((2 * u + g) ^ sw));
        sacc[s] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[u], sacc[s], 0, 0, 0);
      }
    }
    // register j of block s holds key 32s + 16(j>>3) + 8g + (j&7) of this tile
    if (ragged && kt == ntiles - 1) {
      const int lim = n_tokens - kt * kBN;
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (32 * s + 16 * (j >> 3) + 8 * g + (j & 7) >= lim) sacc[s][j] = -INFINITY;
    }

    // ---- online softmax (base 2)
    float mx = sacc[0][0];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sacc[s][j]);
    const bool need = mx * c_log2 > m_run + kTau;
    if (__ballot(need)) {
      // the decision is per query (lanes l and l^32), never per wavefront, so a
      // query's result does not depend on which other queries share its tile
      const float mo = fmaxf(mx, __shfl_xor(mx, 32));
      const int other_need = __shfl_xor(int(need), 32);   // every lane takes part
      const bool pair_need = need || other_need != 0;
      const float m_new = pair_need ? fmaxf(m_run, mo * c_log2) : m_run;
      const float alpha = pair_need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
      l_run *= alpha;
#pragma unroll
      for (int e = 0; e < NE; ++e)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[e][j] *= alpha;
      m_run = m_new;
    }
    bf16x8 pf[4];
    float lsum = 0.0f;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[s][j], c_log2, -m_run));
        lsum += p;
        pf[2 * s + (j >> 3)][j & 7] = static_cast<__bf16>(p);
      }
    l_run += lsum;

    // ---- O^T += V^T P^T, four 16-key steps
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const int d = 32 * e + lq;
        const bf16x8 vf =
            *reinterpret_cast<const bf16x8*>(&vt[buf][d * kBN + 8 * ((2 * c + g) ^ vswz(d))]);
        oacc[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[c], oacc[e], 0, 0, 0);
      }
    }

    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- normalise and store O (lane holds d = 32e + 8a + 4g + 0..3 for a = 0..3)
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  if (qvalid) {
    uint16_t* orow = out + ((int64_t(b) * n_active + qi) * heads + h) * D;
#pragma unroll
    for (int e = 0; e < NE; ++e)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        __bf16 o0 = static_cast<__bf16>(oacc[e][4 * a + 0] * inv);
        __bf16 o1 = static_cast<__bf16>(oacc[e][4 * a + 1] * inv);
        __bf16 o2 = static_cast<__bf16>(oacc[e][4 * a + 2] * inv);
        __bf16 o3 = static_cast<__bf16>(oacc[e][4 * a + 3] * inv);
        const uint32_t lo = uint32_t(__builtin_bit_cast(uint16_t, o0)) |
                            (uint32_t(__builtin_bit_cast(uint16_t, o1)) << 16);
        const uint32_t hi = uint32_t(__builtin_bit_cast(uint16_t, o2)) |
                            (uint32_t(__builtin_bit_cast(uint16_t, o3)) << 16);
        *reinterpret_cast<uint2*>(orow + 32 * e + 8 * a + 4 * g) = make_uint2(lo, hi);
      }
  }
}

template <int D>
hipError_t launch_d(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                    int64_t n_active, int64_t n_tokens, int batch, int heads, float scale,
                    hipStream_t s) {
  const int n_qtiles = int((n_active + kBM - 1) / kBM);
  const int total = n_qtiles * heads * batch;
  const float c_log2 = float(double(scale) * 1.4426950408889634);
  attn_kernel<D><<<dim3(unsigned(total)), dim3(kThreads), 0, s>>>(
      q, k, v, o, int(n_active), int(n_tokens), heads, n_qtiles, total, c_log2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                            uint16_t* out, int64_t n_active, int64_t n_tokens, int batch, int heads,
                            int head_dim, float softmax_scale, hipStream_t stream) {
  if (head_dim == 128)
    return launch_d<128>(q, k_cache, v_cache, out, n_active, n_tokens, batch, heads, softmax_scale,
                         stream);
  return launch_d<64>(q, k_cache, v_cache, out, n_active, n_tokens, batch, heads, softmax_scale,
                      stream);
}

}  // namespace hsastep

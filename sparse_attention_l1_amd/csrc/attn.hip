// Active-query full-context attention ("Technische Samenvatting: Heterogene
// Staptoewijzing (HSA) voor Efficiënte Videogeneratie", §2.2 items 3-4): the
// |A_i| active queries attend to all N cached keys/values of their (b, h),
//     O = softmax(Q_A K^T * scale) V,        cost O(|A_i| * N),
// with no mask.  The queries arrive compacted (active order), so the tiles are
// dense even though the active set is scattered over the token grid.
//
// gfx950 design (bf16 MFMA bound: 4*|A|*N*D flops per (b, h)):
//   - A workgroup owns NW*32*QB queries of one (b, h): NW wavefronts, each with
//     QB blocks of 32 queries.  The key loop walks all N keys in tiles of BN.
//   - Computed transposed: S^T = K Q^T and O^T = V^T P^T with
//     v_mfma_f32_32x32x16_bf16.  Q^T stays in registers as the B operand; K and
//     V^T are the A operands, read from LDS, each fragment feeding QB MFMAs.  In
//     the 32x32 accumulator a lane owns one column, i.e. one query, so the
//     online-softmax reductions are per-lane (lanes l and l^32 hold the two
//     halves of a query's 32-key block).
//   - K and V tiles travel global -> LDS with direct loads (global_load_lds,
//     16 bytes per lane): no staging registers, no LDS write instructions.  Both
//     stay row-major ([key][d]) with a 16-byte-chunk XOR swizzle per row.  K
//     fragments are plain 16-byte reads; V^T fragments come from transposing
//     reads (ds_read_b64_tr_b16), which hand each lane 4 consecutive keys of one
//     d.  The 4-key runs follow the accumulator layout of S^T, so P^T goes from
//     the S^T registers straight into the P.V MFMA with no cross-lane shuffle.
//     The swizzle keeps both kinds of reads free of bank conflicts.
//   - Tiles are double buffered: the next tile's direct loads are in flight while
//     the current one is multiplied; the last (possibly ragged) tile is peeled
//     off so the steady-state loop has no masking branch.
//   - Softmax in base 2 with scale*log2(e) folded into one FMA, per 32-key
//     block.  Steady state needs no max: p = 2^(s*c - m) against a reference max
//     m, row sums by bf16 dot products of the rounded p (the values the MFMA
//     uses).  Only when a lane's block sum exceeds 2^8 or is not a number (the first
//     block, a new max far above m, or overflow) does the pair of lanes take the true max,
//     rescale O and recompute the block.  The decision is per query, so a query's
//     result never depends on its tile neighbours.
//   - Workgroup order is XCD aware: consecutive workgroup ids go to different
//     XCDs, so ids are remapped so that each XCD walks a contiguous range of
//     query tiles of the same head, whose K/V then stream through that XCD's L2.
#include <hip/hip_runtime.h>

#include <cmath>
#include <type_traits>

#include "kernels.hpp"

namespace hsastep {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaitVm0 = 0x0F70;      // s_waitcnt vmcnt(0) (expcnt and lgkmcnt unconstrained)
constexpr float kSumLimit = 256.0f;   // a lane's block sum above 2^8 asks for a new max
constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
// explicit address spaces for the direct global -> LDS load builtin
typedef __attribute__((address_space(1))) void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

// 16-byte chunk swizzle of a K or V tile row (row = key, D/8 chunks per row): a bijection
// on the chunks of each row.  LDS serves 16 lanes of a 16-byte read, or 32 lanes of an
// 8-byte read, per cycle; with this swizzle the 16 rows read together by a K fragment,
// and the 4-key runs read together by a V transpose, land on distinct banks.
template <int D>
__device__ __forceinline__ int tswz(int key) {
  if constexpr (D == 128) {
    return 4 * (key & 3) + ((key >> 2) & 3);
  } else {
    const int m = (key >> 1) & 7;   // 3-bit reversal of key/2
    return ((m & 1) << 2) | (m & 2) | ((m >> 2) & 1);
  }
}

// p_j = 2^(s_j * c - m) for the 16 accumulator values of one 32x32 block, packed to bf16 as
// the two B operands of the P.V MFMA (keys 8g..8g+7 and 16+8g..16+8g+7); returns the sum
// of the rounded p, accumulated with bf16 dot products against (1, 1).
__device__ __forceinline__ float softmax_block(const f32x16& s, float c, float m,
                                               bf16x8 (&pf)[2]) {
  float sum = 0.0f;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const f32x2 v = {__builtin_amdgcn_exp2f(fmaf(s[2 * t], c, -m)),
                     __builtin_amdgcn_exp2f(fmaf(s[2 * t + 1], c, -m))};
    const bf16x2 pr = __builtin_convertvector(v, bf16x2);
    pf[t >> 2][2 * (t & 3)] = pr[0];
    pf[t >> 2][2 * (t & 3) + 1] = pr[1];
    sum = __builtin_amdgcn_fdot2_f32_bf16(pr, kOnes2, sum, false);
  }
  return sum;
}

template <int D, int QB, int NW, int BN>
struct AttnCfg {
  static constexpr int kThreads = 64 * NW;
  static constexpr int kBM = NW * 32 * QB;            // queries per workgroup
  static constexpr int CH = D / 8;                    // 16-byte chunks per K row
  static constexpr int NL = BN * CH / kThreads;       // direct loads per tensor per lane
  static constexpr int NE = D / 32;                   // 32-row blocks of O^T
  static constexpr int NU = D / 16;                   // MFMA k-steps over d
  static constexpr int NS = BN / 32;                  // 32-key blocks per tile
  static_assert(NL >= 1 && BN * CH % kThreads == 0, "tiles must split evenly over lanes");
};

template <int D, int QB, int NW, int BN, int WPE>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, uint16_t* __restrict__ out, int n_active, int n_tokens,
    int heads, int n_qtiles, int total_blocks, float c_log2) {
  using C = AttnCfg<D, QB, NW, BN>;
  constexpr int CH = C::CH, NL = C::NL, NE = C::NE, NU = C::NU;
  __shared__ __attribute__((aligned(16))) uint16_t ks[2][BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t vs[2][BN * D];

  // ---- XCD-aware tile order
  const int L = blockIdx.x;
  const int xcd = L & 7, per = total_blocks >> 3, rem = total_blocks & 7;
  const int Lp = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + (L >> 3);
  const int qt = Lp % n_qtiles;
  const int bh = Lp / n_qtiles;
  const int h = bh % heads;
  const int b = bh / heads;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
  const int g = lane >> 5, lq = lane & 31;
  const int64_t HD = int64_t(heads) * D;

  // ---- Q^T fragments (B operands): block qb holds query qt*kBM + wave*32*QB + 32*qb + lq
  int qi[QB];
  bf16x8 qf[QB][NU];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    qi[qb] = qt * C::kBM + wave * (32 * QB) + 32 * qb + lq;
    const bool valid = qi[qb] < n_active;
    const uint16_t* qrow = q + ((int64_t(b) * n_active + (valid ? qi[qb] : 0)) * heads + h) * D;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const bf16x8 z = {};
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(qrow + 16 * u + 8 * g);
      qf[qb][u] = valid ? v : z;
    }
  }

  const uint16_t* kbase = kc + (int64_t(b) * n_tokens * heads + h) * D;
  const uint16_t* vbase = vc + (int64_t(b) * n_tokens * heads + h) * D;

  // ---- direct tile loads: instruction i of this wavefront fills the 16-byte LDS slots
  // (i*NW + wave)*64 + lane of the tile, i.e. tile row lrow[i], logical chunk lcol[i]/8.
  // Per-lane source pointers advance by one tile per step; only the last tile clamps rows
  // past the end (to the last row: finite data, masked in the softmax).
  int lrow[NL], lcol[NL];
  const uint16_t* kp[NL];
  const uint16_t* vp[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int lin = (i * NW + wave) * 64 + lane;
    lrow[i] = lin / CH;
    lcol[i] = 8 * ((lin % CH) ^ tswz<D>(lin / CH));
    kp[i] = kbase + int64_t(lrow[i]) * HD + lcol[i];
    vp[i] = vbase + int64_t(lrow[i]) * HD + lcol[i];
  }
  const int64_t tile_step = int64_t(BN) * HD;
  auto issue_loads = [&](int dst) {   // tile after the one the pointers were last advanced to
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      __builtin_amdgcn_global_load_lds((gptr_t)kp[i], (lptr_t)&ks[dst][(i * NW + wave) * 512], 16,
                                       0, 0);
      __builtin_amdgcn_global_load_lds((gptr_t)vp[i], (lptr_t)&vs[dst][(i * NW + wave) * 512], 16,
                                       0, 0);
      kp[i] += tile_step;
      vp[i] += tile_step;
    }
  };
  auto issue_last_loads = [&](int kt, int dst) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      int key = kt * BN + lrow[i];
      key = key < n_tokens ? key : n_tokens - 1;
      const int64_t off = int64_t(key) * HD + lcol[i];
      __builtin_amdgcn_global_load_lds((gptr_t)(kbase + off), (lptr_t)&ks[dst][(i * NW + wave) * 512],
                                       16, 0, 0);
      __builtin_amdgcn_global_load_lds((gptr_t)(vbase + off), (lptr_t)&vs[dst][(i * NW + wave) * 512],
                                       16, 0, 0);
    }
  };

  f32x16 oacc[QB][NE];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int e = 0; e < NE; ++e)
#pragma unroll
      for (int j = 0; j < 16; ++j) oacc[qb][e][j] = 0.0f;
  // reference max (log2 units, identical in lanes l and l^32) and this lane's half of the
  // row sum, per query block
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.0f;
  }

  // K fragment (block s, k-step u): row 32s + lq, d = 16u + 8g .. +7
  const int krow_off = lq * D;
  const int ksw = tswz<D>(lq);     // rows 32s + lq share the swizzle of lq
  // V transposing read (lane group G = lane/16, i = lane%16): row 8h + 4(G>>1) + (i>>2) of
  // the 16-key step, d = 32e + 16(G&1) + 4(i&3); the returned 4 values are keys
  // 16c + 8h + 4g .. +3 for d = 32e + (lane%32)
  const int G = lane >> 4, ti = lane & 15;
  int voff[2][NE];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      const int key = 8 * hh + 4 * (G >> 1) + (ti >> 2);
      const int d = 32 * e + 16 * (G & 1) + 4 * (ti & 3);
      voff[hh][e] = key * D + 8 * ((d >> 3) ^ tswz<D>(key)) + 4 * ((d >> 2) & 1);
    }

  const int ntiles = (n_tokens + BN - 1) / BN;
  const bool ragged = (n_tokens % BN) != 0;
  int buf = 0;
  int kt = 0;

  // S^T = K Q^T for keys 32s .. 32s+31 of the tile
  auto compute_s = [&](int s, f32x16 (&sacc)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int j = 0; j < 16; ++j) sacc[qb][j] = 0.0f;
    const uint16_t* krow = &ks[buf][32 * s * D + krow_off];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(krow + 8 * ((2 * u + g) ^ ksw));
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        sacc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][u], sacc[qb], 0, 0, 0);
    }
  };
  // online softmax of block s: P^T (bf16) into pf, running max / sum updated
  auto softmax_only = [&](int s, f32x16 (&sacc)[QB], bf16x8 (&pf)[QB][2], auto masked) {
    // register j holds key 32s + 16(j>>3) + 8((j>>2)&1) + 4g + (j&3) of this tile
    if constexpr (decltype(masked)::value) {
      const int lim = n_tokens - kt * BN - 32 * s;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (16 * (j >> 3) + 8 * ((j >> 2) & 1) + 4 * g + (j & 3) >= lim) sacc[qb][j] = -INFINITY;
    }
    float ls[QB];
    bool need = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      ls[qb] = softmax_block(sacc[qb], c_log2, m_run[qb], pf[qb]);
      need |= !(ls[qb] <= kSumLimit);
    }
    if (__builtin_expect(__ballot(need) != 0, 0)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const bool mine = !(ls[qb] <= kSumLimit);
        const int other = __shfl_xor(int(mine), 32);   // every lane takes part
        const bool pair_need = mine || other != 0;
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sacc[qb][j]);
        const float mo = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = pair_need ? fmaxf(m_run[qb], mo * c_log2) : m_run[qb];
        const float alpha = pair_need ? __builtin_amdgcn_exp2f(m_run[qb] - m_new) : 1.0f;
        l_run[qb] *= alpha;
#pragma unroll
        for (int e = 0; e < NE; ++e) {
          oacc[qb][e] *= alpha;
          __builtin_amdgcn_sched_barrier(0);   // rescale one block at a time
        }
        m_run[qb] = m_new;
        ls[qb] = softmax_block(sacc[qb], c_log2, m_new, pf[qb]);
      }
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) l_run[qb] += ls[qb];
  };
  // O^T += V^T P^T over the block's two 16-key steps; V^T fragments by transposing reads
  auto pv = [&](int s, const bf16x8 (&pf)[QB][2]) {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const uint16_t* vstep = &vs[buf][(32 * s + 16 * h2) * D];
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vstep + voff[0][e]));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vstep + voff[1][e]));
        const i16x4 w[2] = {lo, hi};
        const bf16x8 vf = __builtin_bit_cast(bf16x8, w);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          oacc[qb][e] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qb][h2], oacc[qb][e], 0, 0, 0);
      }
    }
  };
  auto softmax_pv = [&](int s, f32x16 (&sacc)[QB], auto masked) {
    bf16x8 pf[QB][2];
    softmax_only(s, sacc, pf, masked);
    pv(s, pf);
  };
  auto process_tile = [&](auto masked) {
#pragma unroll
    for (int s = 0; s < C::NS; ++s) {
      f32x16 sa[QB];
      compute_s(s, sa);
      softmax_pv(s, sa, masked);
    }
  };

  if (ntiles == 1)
    issue_last_loads(0, 0);
  else
    issue_loads(0);
  // the tile loop runs over full tiles; the last tile, which may be ragged, is peeled off
  // so that the steady-state body has no masking branch between MFMA and VALU work
  for (; kt < ntiles - 1; ++kt) {
    buf = kt & 1;
    __builtin_amdgcn_s_waitcnt(kWaitVm0);   // this tile's direct loads have landed
    __syncthreads();                        // ... for every wavefront; the other buffer is free
    if (kt + 1 < ntiles - 1)
      issue_loads(buf ^ 1);
    else
      issue_last_loads(kt + 1, buf ^ 1);
    process_tile(std::false_type{});
  }
  buf = kt & 1;
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();
  if (ragged)
    process_tile(std::true_type{});
  else
    process_tile(std::false_type{});

  // ---- normalise and store O (lane holds d = 32e + 8a + 4g + 0..3 for a = 0..3)
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 32);
    const float inv = 1.0f / l_tot;
    if (qi[qb] < n_active) {
      uint16_t* orow = out + ((int64_t(b) * n_active + qi[qb]) * heads + h) * D;
#pragma unroll
      for (int e = 0; e < NE; ++e)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const f32x2 lo2 = {oacc[qb][e][4 * a + 0] * inv, oacc[qb][e][4 * a + 1] * inv};
          const f32x2 hi2 = {oacc[qb][e][4 * a + 2] * inv, oacc[qb][e][4 * a + 3] * inv};
          const bf16x2 lo = __builtin_convertvector(lo2, bf16x2);
          const bf16x2 hi = __builtin_convertvector(hi2, bf16x2);
          *reinterpret_cast<uint2*>(orow + 32 * e + 8 * a + 4 * g) =
              make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
        }
    }
  }
}

template <int D, int QB, int NW, int BN, int WPE>
hipError_t launch_cfg(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                      int64_t n_active, int64_t n_tokens, int batch, int heads, float scale,
                      hipStream_t s) {
  using C = AttnCfg<D, QB, NW, BN>;
  const int n_qtiles = int((n_active + C::kBM - 1) / C::kBM);
  const int total = n_qtiles * heads * batch;
  const float c_log2 = float(double(scale) * 1.4426950408889634);
  attn_kernel<D, QB, NW, BN, WPE><<<dim3(unsigned(total)), dim3(C::kThreads), 0, s>>>(
      q, k, v, o, int(n_active), int(n_tokens), heads, n_qtiles, total, c_log2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                            uint16_t* out, int64_t n_active, int64_t n_tokens, int batch, int heads,
                            int head_dim, float softmax_scale, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  if (attention_pipe_fits(n_tokens, heads, head_dim))
    return launch_attention_pipe(q, k_cache, v_cache, out, n_active, n_tokens, batch, heads,
                                 softmax_scale, workspace, workspace_bytes, stream);
  if (head_dim == 128)
    return launch_cfg<128, 1, 8, 128, 2>(q, k_cache, v_cache, out, n_active, n_tokens, batch, heads,
                                      softmax_scale, stream);
  return launch_cfg<64, 1, 8, 128, 2>(q, k_cache, v_cache, out, n_active, n_tokens, batch, heads,
                                   softmax_scale, stream);
}

}  // namespace hsastep

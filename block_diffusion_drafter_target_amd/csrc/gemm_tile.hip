// LDS-tiled bf16 MFMA GEMM for many activation rows (M > 64), gfx950.
//
// Y[m][n] = sum_k A[m][k] * W[n][k] with W in the packed fragment layout and A
// row-major (optionally gathered rows). At M >= 128 every weight byte feeds
// 2*M flops, so the product leaves the HBM-bound regime of the streaming
// kernel; tiles are staged through LDS so that each operand element read from
// memory feeds 128 MFMA columns:
//   * workgroup (4 waves, 2 x 2) = 128 weight rows x 128 activation rows x
//     the split's k range; each wave owns a 64 x 64 corner (4 x 4 MFMA
//     16x16x32 tiles, 64 accumulators);
//   * k advances in 64-wide slabs, double buffered: the next slab's global
//     loads are in registers while the current slab's MFMAs run, then land in
//     the other LDS buffer (one barrier per slab);
//   * weight fragments are copied to LDS unchanged (1 KB operand blocks), so a
//     wave's operand read is 64 consecutive 16-byte words (no bank conflicts);
//     activation rows are stored with the 16-byte chunk index XOR (row & 7);
//   * weights are loaded non-temporally (read once);
//   * the same three epilogues as the streaming kernel: split partials,
//     SwiGLU (a tile holds the gate and up rows of 64 output columns) and
//     per-tile argmax keys.
#include "common.h"
#include "internal.h"

namespace dfl {

namespace {

constexpr int kBN = 128;  // weight rows per tile (8 fragment groups)
constexpr int kBM = 128;  // activation rows per tile
constexpr int kBK = 64;   // k per slab (2 fragments)
constexpr int kWFrag = kBN / 16 * (kBK / 32);  // weight fragments per slab (16)

template <int MODE>
__global__ __launch_bounds__(256) void gemm_tile_kernel(const GemmParams p) {
  __shared__ __align__(16) u32x4 sw[2][kWFrag * 64];   // 2 x 16 KB
  __shared__ __align__(16) u32x4 sx[2][kBM * kBK / 8];  // 2 x 16 KB
  __shared__ unsigned long long kbest[2][kBM];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int wn = wave & 1, wm = wave >> 1;
  const int z = blockIdx.z;
  const int m_tiles = (p.M + kBM - 1) / kBM;
  const int mt = blockIdx.y % m_tiles, s = blockIdx.y / m_tiles;
  const int m0 = mt * kBM;
  const int kbeg = s * p.k_per_split;
  const int kend = min(p.K, kbeg + p.k_per_split);
  const long long frag_row = (long long)(p.K / 32) * 512;

  // The 8 weight row groups of this tile (swiglu: 4 gate then 4 up groups of
  // the same 64 output columns).
  const bf16_t* wgrp[kBN / 16];
#pragma unroll
  for (int q = 0; q < kBN / 16; ++q) {
    const bf16_t* base;
    int grp;
    if (MODE == kGemmSwiglu) {
      const int col = min(blockIdx.x * 64 + (q & 3) * 16, p.N - 16);
      grp = col >> 4;
      base = q < 4 ? p.W0[z] : p.W1[z];
    } else {
      const int n = min(blockIdx.x * kBN + q * 16, p.N - 16);
      base = n < p.n_split ? p.W0[z] : p.W1[z];
      grp = (n < p.n_split ? n : n - p.n_split) >> 4;
    }
    wgrp[q] = base + grp * frag_row;
  }

  // global -> register staging: 4 weight and 4 activation 16-byte words per thread
  u32x4 rw[4], rx[4];
  int xrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = threadIdx.x + 256 * i;
    int m = min(m0 + e / 8, p.M - 1);
    if (p.a_idx) {
      m = p.a_idx[(long long)m * p.a_idx_stride];
      m = m < 0 ? 0 : (m >= p.a_idx_max ? p.a_idx_max - 1 : m);
    }
    xrow[i] = m;
  }
  auto load = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = threadIdx.x + 256 * i;  // weight word: group e/128, fragment (e/64)&1, lane e&63
      const int q = e >> 7, kc = (e >> 6) & 1, l = e & 63;
      rw[i] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(wgrp[q] + (long long)((k0 >> 5) + kc) * 512 + l * 8));
      const int ch = e & 7;  // activation word: row e/8, chunk e&7
      rx[i] = *reinterpret_cast<const u32x4*>(p.A + (long long)xrow[i] * p.lda + k0 + ch * 8);
    }
  };
  auto store = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = threadIdx.x + 256 * i;
      sw[buf][e] = rw[i];  // fragment-major, lane-minor: the packed order
      const int row = e >> 3, ch = e & 7;
      sx[buf][row * 8 + (ch ^ (row & 7))] = rx[i];
    }
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[f][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // wave's weight fragments inside the tile's 8 groups
  int wq[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) wq[f] = MODE == kGemmSwiglu ? (f < 2 ? wn * 2 + f : 4 + wn * 2 + f - 2) : wn * 4 + f;

  int buf = 0;
  if (kbeg < kend) {
    load(kbeg);
    store(0);
    __syncthreads();
  }
  for (int k0 = kbeg; k0 < kend; k0 += kBK) {
    const bool more = k0 + kBK < kend;
    if (more) load(k0 + kBK);
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      u32x4 a[4], b[4];
#pragma unroll
      for (int f = 0; f < 4; ++f) a[f] = sw[buf][(wq[f] * 2 + kc) * 64 + lane];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int row = wm * 64 + t * 16 + r;
        b[t] = sx[buf][row * 8 + ((kc * 4 + g) ^ (row & 7))];
      }
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[f][t] = mfma16x16x32(a[f], b[t], acc[f][t]);
    }
    if (more) {
      store(buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
  }

  if (MODE == kGemmPartial) {
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int m = m0 + wm * 64 + t * 16 + r;
        const int nb = blockIdx.x * kBN + (wn * 4 + f) * 16 + 4 * g;
        if (m < p.M && nb < p.N)
          *reinterpret_cast<f32x4_t*>(p.P + (long long)z * p.p_z_stride + (long long)s * p.p_s_stride +
                                      (long long)m * p.N + nb) = acc[f][t];
      }
  } else if (MODE == kGemmSwiglu) {
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int m = m0 + wm * 64 + t * 16 + r;
        const int nb = blockIdx.x * 64 + (wn * 2 + f) * 16 + 4 * g;
        if (m < p.M && nb < p.N) {
          const f32x4_t gv = acc[f][t], uv = acc[f + 2][t];
          float sv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) sv[i] = gv[i] / (1.0f + __expf(-gv[i])) * uv[i];
          *reinterpret_cast<u32x2*>(p.out + (long long)m * p.ld_out + nb) =
              u32x2{pack_bf2(sv[0], sv[1]), pack_bf2(sv[2], sv[3])};
        }
      }
  } else {
    if (p.dbg) {
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int m = m0 + wm * 64 + t * 16 + r;
          const int nb = blockIdx.x * kBN + (wn * 4 + f) * 16 + 4 * g;
          if (m < p.M && nb < p.N) *reinterpret_cast<f32x4_t*>(p.dbg + (long long)m * p.ld_dbg + nb) = acc[f][t];
        }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float bv = -__builtin_inff();
      int bn = 0x7FFFFFFF;
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int n = blockIdx.x * kBN + (wn * 4 + f) * 16 + 4 * g + i;
          if (n < p.N && acc[f][t][i] > bv) {
            bv = acc[f][t][i];
            bn = n;
          }
        }
#pragma unroll
      for (int o = 16; o <= 32; o <<= 1) {
        const float ov = __shfl_xor(bv, o);
        const int on = __shfl_xor(bn, o);
        if (ov > bv || (ov == bv && on < bn)) {
          bv = ov;
          bn = on;
        }
      }
      if (g == 0) kbest[wn][wm * 64 + t * 16 + r] = bn != 0x7FFFFFFF ? argmax_key(bv, bn) : 0ull;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kBM; i += 256) {
      const int m = m0 + i;
      if (m < p.M) p.keys[(long long)blockIdx.x * p.ld_keys + m] = max(kbest[0][i], kbest[1][i]);
    }
  }
}

}  // namespace

hipError_t launch_gemm_tile(const GemmParams& p, int mode, int nz, hipStream_t st) {
  const int m_tiles = (p.M + kBM - 1) / kBM;
  const int n_tiles = mode == kGemmSwiglu ? (p.N + 63) / 64 : (p.N + kBN - 1) / kBN;
  dim3 grid(n_tiles, m_tiles * p.splits, nz);
  if (p.K % kBK) return hipErrorInvalidValue;
  if (mode == kGemmArgmax)
    hipLaunchKernelGGL(gemm_tile_kernel<kGemmArgmax>, grid, dim3(256), 0, st, p);
  else if (mode == kGemmSwiglu)
    hipLaunchKernelGGL(gemm_tile_kernel<kGemmSwiglu>, grid, dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL(gemm_tile_kernel<kGemmPartial>, grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace dfl

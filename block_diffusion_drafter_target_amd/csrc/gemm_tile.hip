// Tiled bf16 MFMA GEMM for more activation rows (32 < M), gfx950.
//
// Y[m][n] = sum_k A[m][k] * W[n][k] with W in the packed fragment layout and A
// row-major (optionally gathered rows). Up to a few hundred rows the product is
// still bound by streaming W from HBM, so W takes the streaming kernel's path
// and only the activations are shared through LDS:
//   * workgroup (4 waves) = 64*NG weight rows (each wave NG fragment groups of
//     16 rows) x 16*MT activation rows (MT MFMA tiles per wave) x the split's k
//     range (NG = 1 halves the column tile, so fewer K splits, and their fp32
//     partials, fill the chip);
//   * each wave loads its weight fragments straight into MFMA operand
//     registers with non-temporal 16-byte loads (one fully used 1 KB line per
//     operand), 128 k per slab, one slab ahead of the MFMAs;
//   * the 16*MT x 128 activation slab is loaded by all threads, stored to LDS
//     with the 16-byte chunk index XOR (row & 15) (the 16 lanes of one LDS
//     cycle hit 16 different bank groups), double buffered; each wave
//     reads all MT activation tiles from it (MT MFMAs per weight load);
//   * the row tiles of one weight tile are consecutive workgroups of one XCD
//     (block ids go round-robin to the 8 XCDs), so they run together and
//     share the weights through that XCD's L2 and the Infinity Cache;
//   * epilogues as in the streaming kernel: split partials, SwiGLU (a wave's
//     two groups are the gate and up rows of 16 output columns) and one
//     argmax key per (column tile, row).
#include "common.h"
#include "internal.h"

namespace dfl {

namespace {

constexpr int kBK = 128;  // k per slab (4 MFMA steps)

// NG weight row groups (16 rows each) per wave, MT activation tiles (16 rows
// each) per workgroup: the workgroup covers 64*NG weight rows and 16*MT
// activation rows.
template <int NG, int MT>
struct TileShape {
  static constexpr int kBN = 64 * NG;
  static constexpr int kBM = 16 * MT;
  static constexpr int kXWords = kBM * kBK / 8;  // 16-byte words per activation slab
  static constexpr int kXPer = kXWords / 256;    // words each thread copies
  // waves per SIMD the registers and LDS allow
  static constexpr int kWaves = (NG == 4 || MT == 8) ? 2 : 3;
};

// SHARED: several row tiles read each weight tile, so weights take plain
// loads and stay in L2 for the sibling workgroups; otherwise they are read
// once and loaded non-temporally (both measured best in their case).
template <int NG, int MT, int MODE, bool SHARED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(TileShape<NG, MT>::kWaves,
                                                                      TileShape<NG, MT>::kWaves)))
void gemm_tile_kernel(const GemmParams p) {
  using T = TileShape<NG, MT>;
  constexpr int kBN = T::kBN, kBM = T::kBM, kXWords = T::kXWords, kXPer = T::kXPer;
  static_assert(MODE != kGemmSwiglu || NG % 2 == 0, "SwiGLU pairs gate and up groups");
  constexpr int kOut = MODE == kGemmSwiglu ? NG / 2 : NG;  // output groups per wave
  constexpr int kBNo = 64 * kOut;                           // output columns per workgroup
  __shared__ __align__(16) u32x4 sx[2][kXWords];
  __shared__ unsigned long long kbest[MODE == kGemmArgmax ? 4 : 1][kBM];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  // XCD-aware tile order: workgroup l runs on XCD l % 8, the XCD's own
  // sequence number is l / 8. The row tiles that share a weight tile (one
  // "column": column tile, split, matrix) are consecutive on one XCD, so they
  // run together and the weights come from HBM once.
  const int m_tiles = (p.M + kBM - 1) / kBM;
  const int n_tiles = (p.N + kBNo - 1) / kBNo;
  const int xseq = blockIdx.x >> 3;
  const int mt = xseq % m_tiles;
  const int col = (xseq / m_tiles) * 8 + (blockIdx.x & 7);
  if (col >= n_tiles * p.splits * p.n_mats) return;
  const int bx = col % n_tiles;
  const int s = (col / n_tiles) % p.splits, z = col / (n_tiles * p.splits);
  const int m0 = mt * kBM;
  const int kbeg = s * p.k_per_split;
  const int kend = min(p.K, kbeg + p.k_per_split);
  const long long frag_row = (long long)(p.K / 32) * 512;

  // this wave's weight row groups
  const bf16_t* wrow[NG];
#pragma unroll
  for (int f = 0; f < NG; ++f) {
    const bf16_t* base;
    int grp;
    if (MODE == kGemmSwiglu) {  // f < NG/2: gate rows, f >= NG/2: up rows of the same 16 columns
      const int fo = f < kOut ? f : f - kOut;
      grp = min(bx * kBNo + (wave * kOut + fo) * 16, p.N - 16) >> 4;
      base = f < kOut ? p.W0[z] : p.W1[z];
    } else {
      const int n = min(bx * kBN + (wave * NG + f) * 16, p.N - 16);
      base = n < p.n_split ? p.W0[z] : p.W1[z];
      grp = (n < p.n_split ? n : n - p.n_split) >> 4;
    }
    wrow[f] = base + grp * frag_row + lane * 8;
  }
  // activation rows this thread copies into LDS: words e = tid + 256*i,
  // row e / 16, chunk e % 16 (all threads share one chunk index)
  const bf16_t* xsrc[kXPer];
  const int xch = (threadIdx.x & 15) * 8;
#pragma unroll
  for (int i = 0; i < kXPer; ++i) {
    const int e = threadIdx.x + 256 * i;
    int m = min(m0 + (e >> 4), p.M - 1);
    if (p.a_idx) {
      m = p.a_idx[(long long)m * p.a_idx_stride];
      m = m < 0 ? 0 : (m >= p.a_idx_max ? p.a_idx_max - 1 : m);
    }
    xsrc[i] = p.A + (long long)m * p.lda;
  }

  const int klast = p.K - 32;
  u32x4 w[NG][4], xs[kXPer];
  auto load = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int kk = min(k0 + 32 * u, klast);
#pragma unroll
      for (int f = 0; f < NG; ++f)
        w[f][u] = SHARED ? *reinterpret_cast<const u32x4*>(wrow[f] + (long long)(kk >> 5) * 512)
                         : __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wrow[f] + (long long)(kk >> 5) * 512));
    }
    // k past the end (K % 128 == 64 on the last slab) re-reads the row's last
    // chunk; those values are zeroed before they reach LDS
    const int kx = min(k0 + xch, p.K - 8);
#pragma unroll
    for (int i = 0; i < kXPer; ++i) xs[i] = *reinterpret_cast<const u32x4*>(xsrc[i] + kx);
  };
  // chunks at k >= kend (the last slab when K % 128 == 64) are stored as
  // zeros, so the MFMAs need no mask
  auto store = [&](int buf, int k0) __attribute__((always_inline)) {
    if (k0 + kBK > kend) {  // uniform over the workgroup
      const bool zero = k0 + xch >= kend;
#pragma unroll
      for (int i = 0; i < kXPer; ++i)
        if (zero) xs[i] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < kXPer; ++i) {
      const int e = threadIdx.x + 256 * i;
      const int row = e >> 4, ch = e & 15;
      sx[buf][row * 16 + (ch ^ (row & 15))] = xs[i];
    }
  };

  f32x4_t acc[NG][MT];
#pragma unroll
  for (int f = 0; f < NG; ++f)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[f][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  int buf = 0;
  if (kbeg < kend) {
    load(kbeg);
    store(0, kbeg);
    __syncthreads();
  }
  for (int k0 = kbeg; k0 < kend; k0 += kBK) {
    u32x4 wc[NG][4];
#pragma unroll
    for (int f = 0; f < NG; ++f)
#pragma unroll
      for (int u = 0; u < 4; ++u) wc[f][u] = w[f][u];
    const bool more = k0 + kBK < kend;
    if (more) load(k0 + kBK);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int row = t * 16 + r;
        const u32x4 b = sx[buf][row * 16 + ((u * 4 + g) ^ (row & 15))];
#pragma unroll
        for (int f = 0; f < NG; ++f) acc[f][t] = mfma16x16x32(wc[f][u], b, acc[f][t]);
      }
    }
    if (more) {
      store(buf ^ 1, k0 + kBK);
      __syncthreads();
      buf ^= 1;
    }
  }

  if (MODE == kGemmPartial) {
#pragma unroll
    for (int f = 0; f < NG; ++f)
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int m = m0 + t * 16 + r;
        const int nb = bx * kBN + (wave * NG + f) * 16 + 4 * g;
        if (m < p.M && nb < p.N)
          *reinterpret_cast<f32x4_t*>(p.P + (long long)z * p.p_z_stride + (long long)s * p.p_s_stride +
                                      (long long)m * p.N + nb) = acc[f][t];
      }
  } else if (MODE == kGemmSwiglu) {
#pragma unroll
    for (int fo = 0; fo < kOut; ++fo)
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int m = m0 + t * 16 + r;
        const int nb = bx * kBNo + (wave * kOut + fo) * 16 + 4 * g;
        if (m < p.M && nb < p.N) {
          float sv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            sv[i] = acc[fo][t][i] / (1.0f + __expf(-acc[fo][t][i])) * acc[fo + kOut][t][i];
          *reinterpret_cast<u32x2*>(p.out + (long long)m * p.ld_out + nb) =
              u32x2{pack_bf2(sv[0], sv[1]), pack_bf2(sv[2], sv[3])};
        }
      }
  } else {
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int m = m0 + t * 16 + r;
      float bv = -__builtin_inff();
      int bn = 0x7FFFFFFF;
#pragma unroll
      for (int f = 0; f < NG; ++f) {
        const int nb = bx * kBN + (wave * NG + f) * 16 + 4 * g;
        if (p.dbg && m < p.M && nb < p.N) *reinterpret_cast<f32x4_t*>(p.dbg + (long long)m * p.ld_dbg + nb) = acc[f][t];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (nb + i < p.N && acc[f][t][i] > bv) {
            bv = acc[f][t][i];
            bn = nb + i;
          }
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
      if (g == 0) kbest[wave][t * 16 + r] = bn != 0x7FFFFFFF ? argmax_key(bv, bn) : 0ull;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kBM; i += 256) {
      const int m = m0 + i;
      if (m < p.M)
        p.keys[(long long)bx * p.ld_keys + m] =
            max(max(kbest[0][i], kbest[1][i]), max(kbest[2][i], kbest[3][i]));
    }
  }
}

template <int NG, int MT, bool SHARED>
hipError_t launch_kind(const GemmParams& p, int mode, dim3 grid, hipStream_t st) {
  if (mode == kGemmArgmax)
    hipLaunchKernelGGL((gemm_tile_kernel<NG, MT, kGemmArgmax, SHARED>), grid, dim3(256), 0, st, p);
  else if (mode == kGemmPartial)
    hipLaunchKernelGGL((gemm_tile_kernel<NG, MT, kGemmPartial, SHARED>), grid, dim3(256), 0, st, p);
  else if constexpr (NG % 2 == 0)
    hipLaunchKernelGGL((gemm_tile_kernel<NG, MT, kGemmSwiglu, SHARED>), grid, dim3(256), 0, st, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int NG, int MT>
hipError_t launch_shape(const GemmParams& p, int mode, int nz, hipStream_t st) {
  using T = TileShape<NG, MT>;
  const int m_tiles = (p.M + T::kBM - 1) / T::kBM;
  const int cols = mode == kGemmSwiglu ? 32 * NG : T::kBN;  // output columns per workgroup
  const int n_tiles = (p.N + cols - 1) / cols;
  if (p.n_mats != nz) return hipErrorInvalidValue;
  // columns rounded up to the 8 XCDs; the padding workgroups exit at once
  const long long cols8 = ((long long)n_tiles * p.splits * nz + 7) / 8 * 8;
  if (cols8 * m_tiles > 0x7FFFFFFFll) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(cols8 * m_tiles));
  return m_tiles > 1 ? launch_kind<NG, MT, true>(p, mode, grid, st) : launch_kind<NG, MT, false>(p, mode, grid, st);
}

}  // namespace

int gemm_tile_cols(int ng) { return 64 * ng; }
int gemm_tile_rows(int mt) { return 16 * mt; }

hipError_t launch_gemm_tile(const GemmParams& p, int ng, int mt, int mode, int nz, hipStream_t st) {
  if (p.K % 64 || p.K < kBK || p.k_per_split % kBK) return hipErrorInvalidValue;
  if (ng == 2 && mt == 8) return launch_shape<2, 8>(p, mode, nz, st);
  if (ng == 1 && mt == 8) return launch_shape<1, 8>(p, mode, nz, st);
  if (ng == 2 && mt == 4) return launch_shape<2, 4>(p, mode, nz, st);
  if (ng == 1 && mt == 4) return launch_shape<1, 4>(p, mode, nz, st);
  return hipErrorInvalidValue;
}

}  // namespace dfl

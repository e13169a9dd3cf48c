// Tiled bf16 MFMA GEMM with deep weight prefetch, for 33..255 activation rows
// (gfx950): the single-pass SwiGLU and partial-mode products over long K.
//
// Y[m][n] = sum_k A[m][k] * W[n][k], W in the packed fragment layout, A
// row-major (optionally gathered rows). At these row counts the product is
// still bound by streaming W from HBM. Loads complete in order, so when a wave
// waits for its own activation loads (to store them in LDS) it also waits for
// every weight load issued before them. The order of issue here keeps the
// weights three 128-k slabs ahead of the MFMAs anyway:
//   * workgroup (4 waves) = 64*NG weight rows (each wave NG groups of 16) x
//     16*MT activation rows x the split's k range, like the other tiled kernel;
//   * weights: a ring of three slabs of fragments in registers per wave
//     (non-temporal 16-byte loads, one fully used 1 KB line per operand);
//   * activations: each wave loads its quarter of slab j + 2 into registers
//     right after the weights of slab j + 2 were issued and stores it to LDS
//     one step later (a ring of two LDS buffers, chunk ch of row r at word
//     r*16 + (ch ^ (r & 15)): the 16 lanes of one LDS cycle hit 16 bank
//     groups); the wait for it then leaves the weights of slabs j + 2 and
//     j + 3 in flight; chunks past the end of K are stored as zeros, so the
//     MFMAs read LDS without a mask;
//   * the fragments of the next 32-k step are read from LDS while the MFMAs of
//     the current one run;
//   * whole groups of three slabs run as straight-line code, so the compiler
//     keeps exact wait counts across the loop's back edge (with the ring
//     index decided at run time it drained every load before the MFMAs);
//   * the row tiles of one weight tile are consecutive workgroups of one XCD
//     (block ids go round-robin to the 8 XCDs);
//   * epilogues: split partials, SwiGLU (a wave's two groups are the gate and
//     up rows of 16 output columns) and one argmax key per (column tile, row).
// Measured on MI355X against the other tiled kernel (Qwen3-8B-shaped drafter,
// batch 8): at 128 rows gate/up 67 -> 62 us, down 36 -> 34, fuse 51 -> 46
// per launch; at 64 rows gate/up 53 -> 47, down 30 -> 27. For qkv, o and the
// LM head, and for the gpt-oss-shaped 64-row products, it measured equal or
// slower, so the plan keeps the other kernel there. Single-launch floors for
// the same weights measured with a plain read kernel: 9 us for 33.5 MB, 12 us
// for 50 MB, 19 us for 100 MB, 35 us for 201 MB; the rest is the activation
// loads (about 5 us per launch at 128 rows) and the fp32 partials (4-6 us).
#include "common.h"
#include "internal.h"

namespace dfl {

namespace {

constexpr int kBK = 128;  // k per slab (4 MFMA steps)
constexpr int kRing = 2;  // activation slabs in LDS

template <int NG, int MT>
struct WsShape {
  static constexpr int kBN = 64 * NG;
  static constexpr int kBM = 16 * MT;
  static constexpr int kXWords = kBM * kBK / 8;  // 16-byte words per activation slab
  static constexpr int kXLoads = kXWords / 64;   // 16-byte activation loads per lane and slab
};

template <int NG, int MT, int D, int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(MT == 8 && NG == 2 ? 1 : 2, 2)))
void gemm_ws_kernel(const GemmParams p) {
  using T = WsShape<NG, MT>;
  constexpr int kBN = T::kBN, kBM = T::kBM, kXWords = T::kXWords;
  constexpr int kXW = T::kXLoads / 4;  // activation loads per lane and slab
  constexpr int kNW = NG * 4;          // weight loads per wave and slab
  static_assert(D == 3, "the wait counts below assume weights three slabs ahead");
  static_assert(MODE != kGemmSwiglu || NG % 2 == 0, "SwiGLU pairs gate and up groups");
  constexpr int kOut = MODE == kGemmSwiglu ? NG / 2 : NG;
  constexpr int kBNo = 64 * kOut;
  __shared__ __align__(1024) u32x4 sx[kRing][kXWords];
  __shared__ unsigned long long kbest[MODE == kGemmArgmax ? 4 : 1][kBM];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int m_tiles = (p.M + kBM - 1) / kBM;
  const int n_tiles = (p.N + kBNo - 1) / kBNo;
  const int xseq = blockIdx.x >> 3;
  const int mt = xseq % m_tiles;
  const int col = (xseq / m_tiles) * 8 + (blockIdx.x & 7);
  if (col >= n_tiles * p.splits * p.n_mats) return;  // uniform over the workgroup
  const int bx = col % n_tiles;
  const int s = (col / n_tiles) % p.splits, z = col / (n_tiles * p.splits);
  const int m0 = mt * kBM;
  const int kbeg = s * p.k_per_split;
  const int kend = min(p.K, kbeg + p.k_per_split);
  const int nslab = kend > kbeg ? (kend - kbeg + kBK - 1) / kBK : 0;

  // activation words of this wave: word e = wave*64*kXW + ii*64 + lane of a
  // slab, row e / 16, chunk e % 16 (stored at chunk position ch ^ (row & 15))
  const bf16_t* xsrc[kXW];
  int xdst[kXW];
  const int xch = (lane & 15) * 8;
#pragma unroll
  for (int ii = 0; ii < kXW; ++ii) {
    const int e = (wave * kXW + ii) * 64 + lane;
    const int row = e >> 4;
    int m = min(m0 + row, p.M - 1);
    if (p.a_idx) {
      m = p.a_idx[(long long)m * p.a_idx_stride];
      m = m < 0 ? 0 : (m >= p.a_idx_max ? p.a_idx_max - 1 : m);
    }
    xsrc[ii] = p.A + (long long)m * p.lda;
    xdst[ii] = row * 16 + ((lane & 15) ^ (row & 15));
  }
  u32x4 xr[kXW];
  // slabs past the end reload the last slab (never stored), so every step
  // issues the same loads
  auto load_x = [&](int j) __attribute__((always_inline)) {
    const int k0 = kbeg + min(j, max(nslab - 1, 0)) * kBK;
    // k past the end (K % 128 == 64 on the last slab) re-reads the row's last
    // chunk; those k are zeroed where the MFMAs read them
    const int kx = min(k0 + xch, p.K - 8);
#pragma unroll
    for (int ii = 0; ii < kXW; ++ii) xr[ii] = *reinterpret_cast<const u32x4*>(xsrc[ii] + kx);
  };
  // chunks at k >= kend (the last slab when K % 128 == 64) are stored as
  // zeros, so the MFMAs need no mask; slabs past the end are never read
  auto store_x = [&](int j) __attribute__((always_inline)) {
    u32x4* dst = &sx[j % kRing][0];
    const int k0 = kbeg + j * kBK;
    if (k0 + kBK > kend) {  // uniform over the workgroup
      const bool zero = k0 + xch >= kend;
#pragma unroll
      for (int ii = 0; ii < kXW; ++ii)
        if (zero) xr[ii] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int ii = 0; ii < kXW; ++ii) dst[xdst[ii]] = xr[ii];
  };

  const long long frag_row = (long long)(p.K / 32) * 512;
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
  const int klast = p.K - 32;
  // slabs past the end load the first fragment of the row group instead (an
  // L2 hit)
  u32x4 w[D][NG][4];
  auto load_w = [&](int d, int j) __attribute__((always_inline)) {
    const bool real = j < nslab;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int kk = real ? min(kbeg + j * kBK + 32 * u, klast) : 0;
#pragma unroll
      for (int f = 0; f < NG; ++f)
        w[d][f][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wrow[f] + (long long)(kk >> 5) * 512));
    }
  };

  f32x4_t acc[NG][MT];
#pragma unroll
  for (int f = 0; f < NG; ++f)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[f][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Issue order: X0, W0, W1, X1, W2, then per step j: X(j+2), W(j+3). A
  // slab's activations wait in registers for one step and are stored to LDS
  // at the end of the step before their use. Loads complete in order, so the
  // wait for X(j+1) leaves W(j+2) and W(j+3) in flight: the weights run three
  // slabs ahead of the MFMAs.
  load_x(0);
  load_w(0, 0);
  load_w(1, 1);
  wait_vm<2 * kNW>();  // X0 landed
  store_x(0);
  load_x(1);
  load_w(2, 2);
  __syncthreads();
  // one step: slab j from ring slot d (j % D == d) and LDS buffer j % kRing
  auto step = [&](int d, int j) __attribute__((always_inline)) {
    const u32x4* xs = &sx[j % kRing][0];
    // the MT activation fragments of k step u + 1 are read from LDS while the
    // MFMAs of step u run
    u32x4 b[2][MT];
    auto read_b = [&](int u, u32x4* dst) __attribute__((always_inline)) {
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int row = t * 16 + r;
        dst[t] = xs[row * 16 + ((u * 4 + g) ^ (row & 15))];
      }
    };
    read_b(0, b[0]);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (u < 3) read_b(u + 1, b[(u + 1) & 1]);
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int f = 0; f < NG; ++f) acc[f][t] = mfma16x16x32(w[d][f][u], b[u & 1][t], acc[f][t]);
    }
    // X(j+1) (only W(j+2) was issued after it) goes to the buffer of slab
    // j - 1, which every wave finished before the previous barrier
    wait_vm<kNW>();
    store_x(j + 1);
    load_x(j + 2);
    load_w(d, j + D);
    __syncthreads();
  };
  // whole groups of D steps as straight-line code (the compiler then keeps
  // exact wait counts across the loop's back edge), then the last 0..D-1 steps
  int j0 = 0;
  for (; j0 + D <= nslab; j0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) step(d, j0 + d);
  }
  if (j0 < nslab) step(0, j0);
  if (j0 + 1 < nslab) step(1, j0 + 1);

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
    } else if constexpr (MODE == kGemmArgmax) {
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int m = m0 + t * 16 + r;
        float bv = -__builtin_inff();
        int bn = 0x7FFFFFFF;
#pragma unroll
        for (int f = 0; f < NG; ++f) {
          const int nb = bx * kBN + (wave * NG + f) * 16 + 4 * g;
          if (p.dbg && m < p.M && nb < p.N)
            *reinterpret_cast<f32x4_t*>(p.dbg + (long long)m * p.ld_dbg + nb) = acc[f][t];
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
    }
  if constexpr (MODE == kGemmArgmax) {
    __syncthreads();
    for (int i = threadIdx.x; i < kBM; i += 256) {
      const int m = m0 + i;
      if (m < p.M)
        p.keys[(long long)bx * p.ld_keys + m] = max(max(kbest[0][i], kbest[1][i]), max(kbest[2][i], kbest[3][i]));
    }
  }
}

template <int NG, int MT, int D>
hipError_t launch_ws(const GemmParams& p, int mode, dim3 grid, hipStream_t st) {
  if (mode == kGemmArgmax)
    hipLaunchKernelGGL((gemm_ws_kernel<NG, MT, D, kGemmArgmax>), grid, dim3(256), 0, st, p);
  else if (mode == kGemmPartial)
    hipLaunchKernelGGL((gemm_ws_kernel<NG, MT, D, kGemmPartial>), grid, dim3(256), 0, st, p);
  else if constexpr (NG % 2 == 0)
    hipLaunchKernelGGL((gemm_ws_kernel<NG, MT, D, kGemmSwiglu>), grid, dim3(256), 0, st, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int NG, int MT, int D>
hipError_t launch_ws_shape(const GemmParams& p, int mode, int nz, hipStream_t st) {
  using T = WsShape<NG, MT>;
  const int m_tiles = (p.M + T::kBM - 1) / T::kBM;
  const int cols = mode == kGemmSwiglu ? 32 * NG : T::kBN;
  const int n_tiles = (p.N + cols - 1) / cols;
  if (p.n_mats != nz) return hipErrorInvalidValue;
  // activation rows are addressed with 32-bit element offsets from p.A
  const long long rows = p.a_idx ? p.a_idx_max : p.M;
  if ((rows - 1) * p.lda + p.K > 0x7FFFFFFFll) return hipErrorInvalidValue;
  const long long cols8 = ((long long)n_tiles * p.splits * nz + 7) / 8 * 8;
  if (cols8 * m_tiles > 0x7FFFFFFFll) return hipErrorInvalidValue;
  return launch_ws<NG, MT, D>(p, mode, dim3((unsigned)(cols8 * m_tiles)), st);
}

}  // namespace

hipError_t launch_gemm_ws(const GemmParams& p, int ng, int mt, int mode, int nz, hipStream_t st) {
  if (p.K % 64 || p.K < kBK || p.k_per_split % kBK || p.M < 1 || p.N < 16) return hipErrorInvalidValue;
  if (ng == 2 && mt == 8) return launch_ws_shape<2, 8, 3>(p, mode, nz, st);
  if (ng == 1 && mt == 8) return launch_ws_shape<1, 8, 3>(p, mode, nz, st);
  if (ng == 2 && mt == 4) return launch_ws_shape<2, 4, 3>(p, mode, nz, st);
  if (ng == 1 && mt == 4) return launch_ws_shape<1, 4, 3>(p, mode, nz, st);
  return hipErrorInvalidValue;
}

}  // namespace dfl

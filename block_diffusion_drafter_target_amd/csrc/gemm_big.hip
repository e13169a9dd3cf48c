// Large-tile bf16 MFMA GEMM for many activation rows (M >= 256), gfx950.
//
// Y[m][n] = sum_k A[m][k] * W[n][k], W in the packed fragment layout and A
// row-major (optionally gathered rows). With hundreds to thousands of rows the
// product is bound by the matrix cores, and the kernel is laid out for their
// operand traffic rather than for the weight stream:
//   * workgroup = 8 waves over a 256 (rows of A) x 256 (weight rows) tile;
//     wave w owns 128 rows (w & 1) x 64 weight rows (w >> 1), 32 MFMA tiles
//     of 16 x 16 and 128 accumulator registers;
//   * both operands go HBM/L2 -> LDS by gfx950's direct loads
//     (global_load_lds_dwordx4: lane l's 16 bytes land at offset 16*l of a
//     1 KB slot), so they take no registers on the way. A weight fragment is
//     one contiguous 1 KB block of the packed layout; an activation fragment
//     (16 rows x 32 k) is gathered so that it lands in MFMA operand order too.
//     Every LDS operand read is then one ds_read_b128 of 1 KB contiguous
//     bytes, free of bank conflicts, with no swizzle;
//   * a stage is 32 k (16 weight + 16 activation fragments, 32 KB), four
//     stages in LDS (128 KB, one workgroup per CU, two waves per SIMD), loads
//     issued three stages ahead; each wave waits for its own loads of a stage
//     with an explicit vmcnt (the compiler does not track direct LDS loads)
//     before the workgroup barrier that publishes the stage;
//   * the tile order keeps a compact block of tiles on each XCD (block ids go
//     round-robin to the 8 XCDs; each XCD takes one contiguous range of the
//     grouped tile order), so the panels of A and W that its workgroups share
//     are read from HBM about once per XCD;
//   * epilogues as in the other GEMM kernels: split-K fp32 partials, SwiGLU
//     (a wave's first two groups are gate rows, its last two the up rows of
//     the same 32 output columns) and one argmax key per (256-column tile, row).
#include "common.h"
#include "internal.h"

namespace dfl {

namespace {

constexpr int kBM = 256, kBN = 256;  // activation rows, weight rows per workgroup
constexpr int kStages = 4;
constexpr int kFrags = 32;           // per stage: 16 weight fragments, then 16 activation fragments
constexpr int kGroupM = 4;           // row tiles per group of the tile order

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt with vmcnt(N) only (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

template <int MODE>
__global__ __launch_bounds__(512) void gemm_big_kernel(const GemmParams p) {
  __shared__ __align__(1024) u32x4 lds[kStages][kFrags][kWave];
  static_assert(MODE != kGemmArgmax || sizeof(unsigned long long) * 4 * kBM <= sizeof(lds), "argmax staging fits");

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int wm = wave & 1, wn = wave >> 1;
  constexpr int kOutCols = MODE == kGemmSwiglu ? kBN / 2 : kBN;

  // tile order: workgroup l runs on XCD l % 8 and is that XCD's (l / 8)-th;
  // XCD x takes tiles [x * per, (x + 1) * per) of the grouped order, where
  // groups of kGroupM row tiles walk the columns with the row tile fastest
  const int m_tiles = (p.M + kBM - 1) / kBM;
  const int n_tiles = (p.N + kOutCols - 1) / kOutCols;
  const int cols = n_tiles * p.splits * p.n_mats;
  const int total = m_tiles * cols;
  const int per = (total + 7) >> 3;
  const int t = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (t >= total) return;
  const int grp = t / (kGroupM * cols), within = t - grp * kGroupM * cols;
  const int gm = min(kGroupM, m_tiles - grp * kGroupM);
  const int mt = grp * kGroupM + within % gm;
  const int col = within / gm;
  const int bx = col % n_tiles;
  const int s = (col / n_tiles) % p.splits, z = col / (n_tiles * p.splits);
  const int m0 = mt * kBM;
  const int kbeg = s * p.k_per_split;
  const int kend = min(p.K, kbeg + p.k_per_split);
  const int nk = (kend - kbeg) >> 5;  // 32-k stages of this split (K % 32 == 0)
  const long long frag_row = (long long)(p.K / 32) * 512;

  // this wave's two weight slots (2w, 2w + 1) and two activation slots
  const bf16_t* wsrc[2];
  const bf16_t* asrc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int slot = 2 * wave + i;  // weight slot: wave slot / 4 computes it, as its group slot % 4
    const bf16_t* base;
    int gi;
    if (MODE == kGemmSwiglu) {
      const int f = slot & 3, fo = f & 1;
      gi = min(bx * kOutCols + (slot >> 2) * 32 + fo * 16, p.N - 16) >> 4;
      base = f < 2 ? p.W0[z] : p.W1[z];
    } else {
      const int n = min(bx * kBN + slot * 16, p.N - 16);
      base = n < p.n_split ? p.W0[z] : p.W1[z];
      gi = (n < p.n_split ? n : n - p.n_split) >> 4;
    }
    wsrc[i] = base + gi * frag_row + (long long)(kbeg >> 5) * 512 + lane * 8;
    // activation slot: rows m0 + 16*slot .. +15, lane -> row r, k 8g .. 8g+7
    int m = min(m0 + slot * 16 + r, p.M - 1);
    if (p.a_idx) {
      m = p.a_idx[(long long)m * p.a_idx_stride];
      m = m < 0 ? 0 : (m >= p.a_idx_max ? p.a_idx_max - 1 : m);
    }
    asrc[i] = p.A + (long long)m * p.lda + kbeg + 8 * g;
  }

  auto issue = [&](int c) __attribute__((always_inline)) {
    const int b = c & (kStages - 1);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      __builtin_amdgcn_global_load_lds(wsrc[i] + (long long)c * 512, (lds_void*)&lds[b][2 * wave + i][0], 16, 0, 0);
      __builtin_amdgcn_global_load_lds(asrc[i] + c * 32, (lds_void*)&lds[b][16 + 2 * wave + i][0], 16, 0, 0);
    }
  };

  f32x4_t acc[4][8];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[f][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int c = 0; c < kStages - 1; ++c)
    if (c < nk) issue(c);

  for (int c = 0; c < nk; ++c) {
    // this wave's loads of stage c are done once at most the later stages'
    // (up to two, four loads each) are outstanding
    __builtin_amdgcn_sched_barrier(0);
    if (c + 2 < nk)
      wait_vm<8>();
    else if (c + 1 < nk)
      wait_vm<4>();
    else
      wait_vm<0>();
    // every wave's loads of stage c have landed, and every wave is done with
    // stage c - 1, whose buffer the next loads overwrite
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (c + kStages - 1 < nk) issue(c + kStages - 1);
    const u32x4(*st)[kWave] = lds[c & (kStages - 1)];
    u32x4 wf[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) wf[f] = st[4 * wn + f][lane];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x4 a = st[16 + 8 * wm + i][lane];
#pragma unroll
      for (int f = 0; f < 4; ++f) acc[f][i] = mfma16x16x32(wf[f], a, acc[f][i]);
    }
  }

  if (MODE == kGemmPartial) {
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int m = m0 + wm * 128 + i * 16 + r;
        const int nb = bx * kBN + (wn * 4 + f) * 16 + 4 * g;
        if (m < p.M && nb < p.N)
          *reinterpret_cast<f32x4_t*>(p.P + (long long)z * p.p_z_stride + (long long)s * p.p_s_stride +
                                      (long long)m * p.N + nb) = acc[f][i];
      }
  } else if (MODE == kGemmSwiglu) {
#pragma unroll
    for (int fo = 0; fo < 2; ++fo)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int m = m0 + wm * 128 + i * 16 + r;
        const int nb = bx * kOutCols + (wn * 2 + fo) * 16 + 4 * g;
        if (m < p.M && nb < p.N) {
          float sv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            sv[e] = acc[fo][i][e] / (1.0f + __expf(-acc[fo][i][e])) * acc[fo + 2][i][e];
          *reinterpret_cast<u32x2*>(p.out + (long long)m * p.ld_out + nb) =
              u32x2{pack_bf2(sv[0], sv[1]), pack_bf2(sv[2], sv[3])};
        }
      }
  } else {
    // per row: the best of the wave's 64 columns, then of the 4 column waves
    unsigned long long* kbest = reinterpret_cast<unsigned long long*>(&lds[0][0][0]);  // [4][kBM]
    __syncthreads();  // every wave is done reading the stages
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int m = m0 + wm * 128 + i * 16 + r;
      float bv = -__builtin_inff();
      int bn = 0x7FFFFFFF;
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int nb = bx * kBN + (wn * 4 + f) * 16 + 4 * g;
        if (p.dbg && m < p.M && nb < p.N) *reinterpret_cast<f32x4_t*>(p.dbg + (long long)m * p.ld_dbg + nb) = acc[f][i];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (nb + e < p.N && acc[f][i][e] > bv) {
            bv = acc[f][i][e];
            bn = nb + e;
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
      if (g == 0) kbest[wn * kBM + wm * 128 + i * 16 + r] = bn != 0x7FFFFFFF ? argmax_key(bv, bn) : 0ull;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kBM; i += 512) {
      const int m = m0 + i;
      if (m < p.M)
        p.keys[(long long)bx * p.ld_keys + m] =
            max(max(kbest[i], kbest[kBM + i]), max(kbest[2 * kBM + i], kbest[3 * kBM + i]));
    }
  }
}

}  // namespace

int gemm_big_cols(int mode) { return mode == kGemmSwiglu ? kBN / 2 : kBN; }
int gemm_big_rows() { return kBM; }

hipError_t launch_gemm_big(const GemmParams& p, int mode, int nz, hipStream_t st) {
  if (p.K % 32 || p.k_per_split % 32 || p.k_per_split < 32 || p.n_mats != nz || p.M < 1 || p.N < 16)
    return hipErrorInvalidValue;
  if (mode == kGemmSwiglu && p.splits != 1) return hipErrorInvalidValue;
  if (mode == kGemmArgmax && p.splits != 1) return hipErrorInvalidValue;
  const long long m_tiles = (p.M + kBM - 1) / kBM;
  const long long n_tiles = (p.N + gemm_big_cols(mode) - 1) / gemm_big_cols(mode);
  const long long total = m_tiles * n_tiles * p.splits * nz;
  const long long grid = (total + 7) / 8 * 8;
  if (grid > 0x7FFFFFFFll) return hipErrorInvalidValue;
  if (mode == kGemmPartial)
    hipLaunchKernelGGL(gemm_big_kernel<kGemmPartial>, dim3((unsigned)grid), dim3(512), 0, st, p);
  else if (mode == kGemmSwiglu)
    hipLaunchKernelGGL(gemm_big_kernel<kGemmSwiglu>, dim3((unsigned)grid), dim3(512), 0, st, p);
  else if (mode == kGemmArgmax)
    hipLaunchKernelGGL(gemm_big_kernel<kGemmArgmax>, dim3((unsigned)grid), dim3(512), 0, st, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dfl

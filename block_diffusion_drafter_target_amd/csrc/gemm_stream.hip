// Weight-streaming bf16 GEMM for few activation rows (M <= 64), gfx950.
//
// Y[m][n] = sum_k A[m][k] * W[n][k]. With M <= 64 the product is bound by
// reading W once from HBM (2 flop per weight byte per row of A), so the kernel
// is built around the weight stream:
//   * W is in the packed fragment layout (pack.hip): every 16-row x 32-k MFMA
//     operand is one contiguous 1 KB block, lane l's 16 bytes at offset 16*l,
//     and a 16-row group's blocks follow each other along k. One wave load of
//     an operand is one fully used 1 KB line, and a wave walking k reads
//     contiguous memory;
//   * weights are read once per step, so they are loaded non-temporally
//     (measured on MI355X with a cold Infinity Cache: the LM head reaches the
//     contiguous-read bandwidth this way, about 6.1 TB/s, against 5.5 without);
//   * a workgroup (4 waves) owns 16*NF weight rows and all 16*MT rows of A;
//     wave w takes every fourth 128-wide k block of the split's k range;
//     the four partial tiles are summed through LDS;
//   * A (activations, row-major) is tiny and re-read from L1/L2;
//   * grid y splits K (fp32 partials P[z][s][m][n], summed by the consumer),
//     grid z batches independent weight matrices;
//   * argmax mode (one split) reduces each row's logits over the workgroup's
//     columns to a packed (value, index) key and writes one key per row and
//     workgroup, keys[tile][row] (no atomics: 15 rows would serialize
//     thousands of atomics);
//     logits are never written unless a debug buffer is given;
//   * swiglu mode (one split) pairs gate rows (W0) and up rows (W1) of the same
//     output columns inside the workgroup and writes bf16 silu(g) * u;
//   * in swiglu mode an optional row scale applies the RMSNorm of A after the
//     product: A then holds x * gain, and each row's gate and up products are
//     multiplied by its 1/rms, formed from the per-chunk sums of squares of
//     the split row pass (loaded with the first weights, reduced after the k
//     loop). Partial products leave the scale to their consumer and an argmax
//     does not depend on it.
// MFMA: W rows are the A operand, activations the B operand, so a lane's four
// results are four consecutive n of one row m.
#include "common.h"
#include "internal.h"

namespace dfl {

namespace {

constexpr int kKB = 128;  // k per block = four 32-wide MFMA steps

// Waves per SIMD the register budget is tuned for (fewer activation tiles,
// more waves in flight). With one activation tile the argmax product (the LM
// head) runs five: Qwen3-8B-shaped LM head at batch 1 202 -> 196 us per launch
// against four, 199-200 at six or eight; five made the four-group SwiGLU
// slower (197 -> 252 us per step) and left the partial products unchanged,
// three slowed every mode (measured on MI355X).
template <int MT, int MODE>
struct Occ {
  static constexpr int kWaves = MT == 1 ? (MODE == kGemmArgmax ? 5 : 4) : (MT == 2 ? 3 : 2);
};

template <int MT, int NF, int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(Occ<MT, MODE>::kWaves, Occ<MT, MODE>::kWaves)))
void gemm_stream_kernel(const GemmParams p) {
  __shared__ f32x4_t red[4][NF * MT][kWave];
  __shared__ unsigned long long kbest[MODE == kGemmArgmax ? NF : 1][16 * MT];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int z = blockIdx.z;
  const int s = blockIdx.y;
  constexpr int kOutFrags = MODE == kGemmSwiglu ? NF / 2 : NF;  // output fragments
  const int n0 = blockIdx.x * 16 * kOutFrags;
  const int kbeg = s * p.k_per_split;
  const int kend = min(p.K, kbeg + p.k_per_split);
  const long long frag_row = (long long)(p.K / 32) * 512;  // elements per 16-row group

  const bf16_t* wrow[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const bf16_t* base;
    int grp;
    if (MODE == kGemmSwiglu) {
      const int fo = f < NF / 2 ? f : f - NF / 2;
      grp = min(n0 + 16 * fo, p.N - 16) >> 4;
      base = f < NF / 2 ? p.W0[z] : p.W1[z];
    } else {
      const int n = min(n0 + 16 * f, p.N - 16);
      base = n < p.n_split ? p.W0[z] : p.W1[z];
      grp = (n < p.n_split ? n : n - p.n_split) >> 4;
    }
    wrow[f] = base + grp * frag_row + lane * 8;
  }
  const bf16_t* arow[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int m = min(16 * t + r, p.M - 1);
    int row = m;
    if (p.a_idx) {  // gathered rows (commit rows of the KV injection)
      row = p.a_idx[(long long)m * p.a_idx_stride];
      row = row < 0 ? 0 : (row >= p.a_idx_max ? p.a_idx_max - 1 : row);
    }
    arow[t] = p.A + (long long)row * p.lda + g * 8;
  }

  // row-scale sums: lane group g holds chunks 4g .. 4g + 3 and 16 + 4g ..
  // 16 + 4g + 3 of its row (from A when there is no scale: valid memory,
  // values dropped, so no branch separates these loads from the weight
  // stream)
  static_assert(kMaxRowChunks == 32, "two float4 of chunk sums per lane");
  constexpr bool kRowScale = MODE == kGemmSwiglu;
  const bool has_rs = kRowScale && p.rs != nullptr;
  f32x4_t rsv[MT][2];
  if constexpr (kRowScale) {
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int m = min(16 * t + r, p.M - 1);
      const float* rsrow =
          has_rs ? p.rs + (long long)m * kMaxRowChunks + 4 * g : reinterpret_cast<const float*>(p.A);
#pragma unroll
      for (int i = 0; i < 2; ++i) rsv[t][i] = *reinterpret_cast<const f32x4_t*>(rsrow + (has_rs ? 16 * i : 0));
    }
  }

  f32x4_t acc[NF][MT];
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[f][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // One 128-wide k block per iteration: all of the block's loads are issued
  // before its MFMAs (the compiler overlaps the next iteration's loads with
  // these MFMAs by itself). Addresses are clamped to the row's last k chunk so
  // every load is unconditional; chunks past the split's end are zeroed on the
  // activation side with a uniform mask.
  const int klast = p.K - 32;
  for (int k = kbeg + wave * kKB; k < kend; k += 4 * kKB) {
    u32x4 w[NF][4], x[MT][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int kk = min(k + 32 * u, klast);
#pragma unroll
      for (int f = 0; f < NF; ++f)
        w[f][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wrow[f] + (long long)(kk >> 5) * 512));
#pragma unroll
      for (int t = 0; t < MT; ++t) x[t][u] = *reinterpret_cast<const u32x4*>(arow[t] + kk);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t keep = (k + 32 * u < kend) ? 0xFFFFFFFFu : 0u;
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const u32x4 xv = x[t][u] & keep;
#pragma unroll
        for (int f = 0; f < NF; ++f) acc[f][t] = mfma16x16x32(w[f][u], xv, acc[f][t]);
      }
    }
  }

#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int t = 0; t < MT; ++t) red[wave][f * MT + t][lane] = acc[f][t];
  // row scales of the lane's rows 16t + r (1 without one)
  float rsc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    rsc[t] = 1.f;
    if constexpr (!kRowScale) continue;
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (16 * i + 4 * g + e < p.rs_n) a += rsv[t][i][e];
    a += __shfl_xor(a, 16);
    a += __shfl_xor(a, 32);
    rsc[t] = has_rs ? 1.0f / sqrtf(a / (float)p.rs_len + p.rs_eps) : 1.f;
  }
  __syncthreads();

  // each wave finishes the output fragments idx = wave, wave + 4, ...
  for (int idx = wave; idx < kOutFrags * MT; idx += 4) {
    const int f = idx / MT, t = idx % MT;
    f32x4_t v = red[0][idx][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) v += red[w][idx][lane];
    const int m = 16 * t + r;
    const int nb = n0 + 16 * f + 4 * g;  // four consecutive n
    float sc = rsc[0];
#pragma unroll
    for (int tt = 1; tt < MT; ++tt)
      if (t == tt) sc = rsc[tt];
    if (MODE == kGemmSwiglu) v *= sc;
    if (MODE == kGemmPartial) {
      if (m < p.M && nb < p.N) {
        float* dst = p.P + (long long)z * p.p_z_stride + (long long)s * p.p_s_stride +
                     (long long)m * p.N + nb;
        *reinterpret_cast<f32x4_t*>(dst) = v;
      }
    } else if (MODE == kGemmSwiglu) {
      const int iu = (f + NF / 2) * MT + t;
      f32x4_t up = red[0][iu][lane];
#pragma unroll
      for (int w = 1; w < 4; ++w) up += red[w][iu][lane];
      up *= sc;
      if (m < p.M && nb < p.N) {
        float sv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[i] = v[i] / (1.0f + __expf(-v[i])) * up[i];
        const u32x2 o = u32x2{pack_bf2(sv[0], sv[1]), pack_bf2(sv[2], sv[3])};
        *reinterpret_cast<u32x2*>(p.out + (long long)m * p.ld_out + nb) = o;
      }
    } else {
      if (p.dbg != nullptr && m < p.M && nb < p.N)
        *reinterpret_cast<f32x4_t*>(p.dbg + (long long)m * p.ld_dbg + nb) = v;
      float bv = -__builtin_inff();
      int bn = 0x7FFFFFFF;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (nb + i < p.N && v[i] > bv) {
          bv = v[i];
          bn = nb + i;
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
      if (g == 0) kbest[f][m] = bn != 0x7FFFFFFF ? argmax_key(bv, bn) : 0ull;
    }
  }
  if (MODE == kGemmArgmax) {
    __syncthreads();
    for (int m = threadIdx.x; m < 16 * MT && m < p.M; m += 256) {
      unsigned long long best = kbest[0][m];
#pragma unroll
      for (int f = 1; f < kOutFrags; ++f) best = max(best, kbest[f][m]);
      p.keys[(long long)blockIdx.x * p.ld_keys + m] = best;
    }
  }
}

template <int MT, int NF>
hipError_t launch_mt_nf(const GemmParams& p, int mode, int nz, hipStream_t st) {
  const int out_frags = mode == kGemmSwiglu ? NF / 2 : NF;
  dim3 grid((p.N + 16 * out_frags - 1) / (16 * out_frags), p.splits, nz);
  if (mode == kGemmArgmax)
    hipLaunchKernelGGL((gemm_stream_kernel<MT, NF, kGemmArgmax>), grid, dim3(256), 0, st, p);
  else if (mode == kGemmSwiglu)
    hipLaunchKernelGGL((gemm_stream_kernel<MT, NF, kGemmSwiglu>), grid, dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((gemm_stream_kernel<MT, NF, kGemmPartial>), grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_stream(const GemmParams& p, int mt, int nf, int mode, int nz,
                              hipStream_t st) {
  // (MT, NF) pairs that fit the register file without spills
  if (mt == 1 && nf == 4) return launch_mt_nf<1, 4>(p, mode, nz, st);
  if (mt == 1 && nf == 2) return launch_mt_nf<1, 2>(p, mode, nz, st);
  if (mt == 2 && nf == 2) return launch_mt_nf<2, 2>(p, mode, nz, st);
  if (mt == 4 && nf == 2) return launch_mt_nf<4, 2>(p, mode, nz, st);
  return hipErrorInvalidValue;
}

}  // namespace dfl

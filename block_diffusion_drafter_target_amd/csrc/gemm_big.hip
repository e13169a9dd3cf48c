// Large-tile bf16 MFMA GEMM with both operands staged by direct loads, gfx950:
// for many activation rows (M >= 256) and for the split-K partials of one
// 65..128-row tile.
//
// Y[m][n] = sum_k A[m][k] * W[n][k], W in the packed fragment layout and A
// row-major (optionally gathered rows). With hundreds to thousands of rows the
// product is bound by the matrix cores, and the kernel is laid out for their
// operand traffic rather than for the weight stream:
//   * workgroup = 8 waves over a BM (rows of A) x BN (weight rows) tile:
//     256 x 256, 128 x 256, 128 x 192, 128 x 128 or 256 x 192. With WM = 2, wave w owns
//     BM / 2 rows (w & 1) x BN / 4 weight rows (w >> 1): at 256 x 256, 32 MFMA
//     tiles of 16 x 16 and 128 accumulator registers (two waves per SIMD; a
//     4-wave layout of 128 x 128 wave tiles, one wave per SIMD, measured
//     10-25% slower: nothing hides its LDS latency). BM = 128 reads more LDS
//     per MFMA but doubles the tiles, for products whose 256-row grid would
//     need split-K: half the splits, half the fp32 partials written here and
//     read by the next pass; 128 x 128 serves one tile of 65..128 rows, where
//     the product is still bound by the weight stream and the five stages of
//     direct loads keep 40 KB of weights in flight per workgroup; 128 x 192
//     (three 16-row weight groups per wave) fills the round where 128 x 256
//     partial tiles leave CUs idle (512 rows, QKV: 192 -> 256 workgroups,
//     the QKV phase 228 -> 209 us per step, measured on MI355X). The
//     256 x 192 SwiGLU tile (four waves of 64 rows
//     along A, two of 96 weight rows = 48 gate and 48 up rows) fills one
//     round of 256 CUs where 256 x 256 tiles leave a quarter of them idle;
//   * both operands go HBM/L2 -> LDS by gfx950's direct loads
//     (global_load_lds_dwordx4: lane l's 16 bytes land at offset 16*l of a
//     1 KB slot), so they take no registers on the way. A weight fragment is
//     one contiguous 1 KB block of the packed layout; an activation fragment
//     (16 rows x 32 k) is gathered so that it lands in MFMA operand order too.
//     Every LDS operand read is then one ds_read_b128 of 1 KB contiguous
//     bytes, free of bank conflicts, with no swizzle;
//   * a stage is 32 k (BN / 16 weight + BM / 16 activation fragments, at
//     most 32 KB); five stages take at most 160 KB of LDS (one workgroup per
//     CU). Every wave issues the same number of direct loads per stage; where
//     the weight fragments do not split evenly over the 8 waves, the waves
//     without a last one repeat a fragment into a spare slot. A stage's loads
//     are issued five stages ahead, at the end of the MFMAs of the stage
//     whose buffer they refill; each wave waits for its own direct loads of a
//     stage with an explicit vmcnt (the compiler does not track them) before
//     the workgroup barrier that publishes the stage. (Direct loads issued
//     among the LDS reads and MFMAs measured 13 times slower.)
//   * the fragments of stage c + 1 are read while the MFMAs of stage c run
//     (weights into a second register set, each activation fragment into the
//     register its stage-c twin frees), so the LDS reads after a barrier
//     overlap the matrix cores;
//   * the tile order keeps a compact block of tiles on each XCD (block ids go
//     round-robin to the 8 XCDs; each XCD takes one contiguous range of the
//     grouped tile order), so the panels of A and W that its workgroups share
//     are read from HBM about once per XCD;
//   * epilogues as in the other GEMM kernels: split-K fp32 partials, SwiGLU
//     (a wave's first two groups are gate rows, its last two the up rows of
//     the same 32 output columns) and one argmax key per (256-column tile, row).
// Measured on MI355X (cold weights): 4096 x 4096 x 20480 at 53% of the dense
// bf16 peak; the same loop without the direct loads reaches 73%.
#include "common.h"
#include "internal.h"

namespace dfl {

namespace {

constexpr int kStages = 5;    // 5 stages of at most 32 KB: one workgroup per CU
constexpr int kGroupM = 4;    // row tiles per group of the tile order

// Wave layout of an 8-wave workgroup over a BM (activation rows) x BN (weight
// rows) tile: WM waves along the rows (BM / WM each), 8 / WM along the weight
// rows.
template <int BM, int BN, int WM>
struct BigShape {
  static constexpr int kWaves = 8;
  static constexpr int kWavesN = kWaves / WM;  // waves along the weight rows
  static constexpr int kWF = BN / 16;          // weight fragments per stage
  static constexpr int kNF = kWF / kWavesN;    // weight fragments per wave
  static constexpr int kAF = BM / 16;          // activation fragments per stage
  static constexpr int kAFW = kAF / WM;        // activation fragments per wave
  static constexpr int kFrags = kWF + kAF;     // fragments per stage
  // direct loads per wave and stage: kWF / 8 weight and kAF / 8 activation
  // fragments, and where kWF % 8 != 0 one more weight fragment: a real one for
  // the first kWF % 8 waves, a repeated one into a spare LDS slot for the
  // others (so that every wave issues the same loads, with no branches)
  static constexpr int kLoads = (kWF + kWaves - 1) / kWaves + kAF / kWaves;
  static constexpr int kSpare = kWF % kWaves == 0 ? 0 : kWaves - kWF % kWaves;
  static constexpr int kThreads = 64 * kWaves;
  static_assert(kWF % kWavesN == 0 && kAF % WM == 0, "fragments split evenly over the waves");
};

template <int MODE, int BM, int BN, int WM>
__device__ __forceinline__ void gemm_big_body(const GemmParams& p) {
  using S = BigShape<BM, BN, WM>;
  constexpr int kNF = S::kNF, kWavesN = S::kWavesN, kWF = S::kWF;
  constexpr int kAFW = S::kAFW, kFrags = S::kFrags, kLoads = S::kLoads, kSpare = S::kSpare;
  constexpr int kBM = BM, kBN = BN, kWaves8 = S::kWaves;
  __shared__ __align__(1024) u32x4 lds[kStages][kFrags + kSpare][kWave];
  static_assert(MODE != kGemmArgmax || sizeof(unsigned long long) * kWavesN * kBM <= sizeof(lds),
                "argmax staging fits");
  static_assert(MODE != kGemmSwiglu || kNF % 2 == 0, "gate and up halves");

  // the wave index is uniform: kept in scalar registers, so are every
  // load's base address and LDS slot
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int wm = wave % WM, wn = wave / WM;
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

  // this wave's loads of every stage: kWL weight slots (and one more for the
  // first kWX waves; the other waves repeat slot kWF - 1 into a spare slot)
  // and kAL activation slots; weight slot q is computed by wave column
  // q / kNF as its group q % kNF. A weight load reads from a uniform fragment row (scalar
  // registers) plus the lane's 16 bytes, an activation load from the lane's
  // element offset in A.
  constexpr int kWL = kWF / kWaves8, kWX = kWF % kWaves8, kAL = S::kAF / kWaves8;
  static_assert(S::kAF % kWaves8 == 0, "activation fragments split evenly over the waves");
  // slots of this wave's loads: consecutive ones where the weight fragments
  // split evenly over the waves, else every eighth (the first kWX waves take
  // one more weight slot)
  auto wslot = [&](int j) __attribute__((always_inline)) {
    return kWX == 0 ? kWL * wave + j : min(wave + kWaves8 * j, kWF - 1);
  };
  auto aslot = [&](int j) __attribute__((always_inline)) { return kWX == 0 ? kAL * wave + j : wave + kWaves8 * j; };
  const bf16_t* wsrc[kWL + 1];  // uniform: the group's fragment row at the split's first stage
  int aoff[kAL];                // per lane: element offset of its row and k in A
#pragma unroll
  for (int j = 0; j <= kWL; ++j) {
    const int slot = wslot(j);
    const bf16_t* base;
    int gi;
    if (MODE == kGemmSwiglu) {  // a wave's first kNF/2 groups: gate rows, the rest: up rows of the same columns
      const int f = slot % kNF, fo = f % (kNF / 2);
      gi = min(bx * kOutCols + (slot / kNF) * (kNF / 2) * 16 + fo * 16, p.N - 16) >> 4;
      base = f < kNF / 2 ? p.W0[z] : p.W1[z];
    } else {
      const int n = min(bx * kBN + slot * 16, p.N - 16);
      base = n < p.n_split ? p.W0[z] : p.W1[z];
      gi = (n < p.n_split ? n : n - p.n_split) >> 4;
    }
    wsrc[j] = base + gi * frag_row + (long long)(kbeg >> 5) * 512;
  }
#pragma unroll
  for (int j = 0; j < kAL; ++j) {
    // activation slot a: rows m0 + 16a .. +15, lane -> row r, k 8g .. 8g+7
    int m = min(m0 + aslot(j) * 16 + r, p.M - 1);
    if (p.a_idx) {
      m = p.a_idx[(long long)m * p.a_idx_stride];
      m = m < 0 ? 0 : (m >= p.a_idx_max ? p.a_idx_max - 1 : m);
    }
    aoff[j] = (int)((long long)m * p.lda) + kbeg + 8 * g;
  }
  const int woff = lane * 8;  // per lane, shared by every weight fragment
  // LDS slot of the extra weight load (uniform)
  const int xslot = wave < kWX ? wave + kWaves8 * kWL : kFrags + wave - kWX;

  // this wave's direct loads of stage c into its LDS buffer (weight and
  // activation loads alternating while both remain, then the extra one)
  auto issue = [&](int c) __attribute__((always_inline)) {
    const int b = c % kStages;
#pragma unroll
    for (int j = 0; j < (kWL > kAL ? kWL : kAL); ++j) {
      if (j < kWL)
        __builtin_amdgcn_global_load_lds(wsrc[j] + (long long)c * 512 + woff, (lds_void*)&lds[b][wslot(j)][0], 16, 0, 0);
      if (j < kAL)
        __builtin_amdgcn_global_load_lds(p.A + (aoff[j] + c * 32), (lds_void*)&lds[b][kWF + aslot(j)][0], 16, 0, 0);
    }
    if (kWX != 0)
      __builtin_amdgcn_global_load_lds(wsrc[kWL] + (long long)c * 512 + woff, (lds_void*)&lds[b][xslot][0], 16, 0, 0);
  };

  f32x4_t acc[kNF][kAFW];
#pragma unroll
  for (int f = 0; f < kNF; ++f)
#pragma unroll
    for (int i = 0; i < kAFW; ++i) acc[f][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int c = 0; c < kStages; ++c)
    if (c < nk) issue(c);

  // Stage c + 1 is published, then its fragments are read while the MFMAs of
  // stage c run: the weight fragments into a second register set (the loop
  // is unrolled by two so that the sets keep fixed registers), each
  // activation fragment into the register its stage-c twin frees once its
  // MFMAs are issued. After those MFMAs the wave issues its direct loads of
  // stage c + kStages into the buffer of stage c.
  auto publish = [&](int c) __attribute__((always_inline)) {
    static_assert(kStages == 5, "wait counts below");
    __builtin_amdgcn_sched_barrier(0);
    // this wave's LDS reads of the stage just computed have landed (the
    // compiler then knows that no read is older than the ones issued next)
    wait_lgkm0();
    // this wave's direct loads of stage c have landed once at most those of
    // the stages issued after it (c + 1 .. c + 3, where they exist; before
    // stage 0 also c + 4, and the wait covers stage 1 too) remain
    if (c + 3 < nk)
      wait_vm<3 * kLoads>();
    else if (c + 2 < nk)
      wait_vm<2 * kLoads>();
    else if (c + 1 < nk)
      wait_vm<kLoads>();
    else
      wait_vm<0>();
    // every wave's loads of stage c have landed, and every wave's reads of
    // stage c - 1 have completed
    lds_barrier();
  };
  // The operand with fewer fragments per wave ("outer") is read for stage
  // c + 1 into a second register set while the MFMAs of stage c run; each
  // fragment of the other operand ("inner") is refilled with its stage c + 1
  // twin right after its MFMAs (2 x 128 rows x 64 weight rows: the weights are
  // outer; 4 x 64 rows x 96 weight rows: the activations).
  constexpr bool kWOuter = kNF <= kAFW;
  constexpr int kOuter = kWOuter ? kNF : kAFW, kInner = kWOuter ? kAFW : kNF;
  auto frag_w = [&](int c, int f) __attribute__((always_inline)) { return lds[c % kStages][kNF * wn + f][lane]; };
  auto frag_a = [&](int c, int i) __attribute__((always_inline)) {
    return lds[c % kStages][kWF + kAFW * wm + i][lane];
  };
  auto read_outer = [&](int c, u32x4(&of)[kOuter]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kOuter; ++j) of[j] = kWOuter ? frag_w(c, j) : frag_a(c, j);
  };
  // MFMAs of stage c_next - 1 with outer set of and inner fragments inf,
  // refilling inf with stage c_next; then the direct loads of stage
  // c_next - 1 + kStages into the buffer of stage c_next - 1, whose reads
  // every wave completed before the barrier that published stage c_next
  auto step = [&](const u32x4(&of)[kOuter], u32x4(&inf)[kInner], int c_next) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kInner; ++j) {
#pragma unroll
      for (int o = 0; o < kOuter; ++o) {
        if constexpr (kWOuter)
          acc[o][j] = mfma16x16x32(of[o], inf[j], acc[o][j]);
        else
          acc[j][o] = mfma16x16x32(inf[j], of[o], acc[j][o]);
      }
      inf[j] = kWOuter ? frag_a(c_next, j) : frag_w(c_next, j);
    }
    // order for the scheduler: the outer reads issued just before, then per
    // inner fragment its MFMAs and the read that refills it (hoisting the
    // reads would keep two operand sets live and spill)
    __builtin_amdgcn_sched_group_barrier(0x100, kOuter, 0);
#pragma unroll
    for (int j = 0; j < kInner; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, kOuter, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    const int cl = c_next - 1 + kStages;
    if (cl < nk) issue(cl);
  };
  u32x4 oa[kOuter], ob[kOuter], inf[kInner];
  publish(0);
  read_outer(0, oa);
#pragma unroll
  for (int j = 0; j < kInner; ++j) inf[j] = kWOuter ? frag_a(0, j) : frag_w(0, j);
  // one stage past the last is published (a plain barrier: its wait is
  // vmcnt(0)) and read too (its fragments come from a stale buffer and are
  // not used)
  if constexpr (WM == 2) {
    // unrolled by two, so that the outer sets keep fixed registers
    for (int c = 0; c < nk; c += 2) {
      publish(c + 1);
      read_outer(c + 1, ob);
      step(oa, inf, c + 1);
      if (c + 1 >= nk) break;
      publish(c + 2);
      read_outer(c + 2, oa);
      step(ob, inf, c + 2);
    }
  } else {
    // one stage per iteration and a register copy of the outer set: unrolled
    // by two, the compiler alternated the accumulators between two register
    // sets and spilled
    for (int c = 0; c < nk; ++c) {
      publish(c + 1);
      read_outer(c + 1, ob);
      step(oa, inf, c + 1);
#pragma unroll
      for (int j = 0; j < kOuter; ++j) oa[j] = ob[j];
    }
  }

  if (MODE == kGemmPartial) {
#pragma unroll
    for (int f = 0; f < kNF; ++f)
#pragma unroll
      for (int i = 0; i < kAFW; ++i) {
        const int m = m0 + wm * (kBM / WM) + i * 16 + r;
        const int nb = bx * kBN + (wn * kNF + f) * 16 + 4 * g;
        if (m < p.M && nb < p.N)
          *reinterpret_cast<f32x4_t*>(p.P + (long long)z * p.p_z_stride + (long long)s * p.p_s_stride +
                                      (long long)m * p.N + nb) = acc[f][i];
      }
  } else if (MODE == kGemmSwiglu) {
#pragma unroll
    for (int fo = 0; fo < kNF / 2; ++fo)
#pragma unroll
      for (int i = 0; i < kAFW; ++i) {
        const int m = m0 + wm * (kBM / WM) + i * 16 + r;
        const int nb = bx * kOutCols + (wn * (kNF / 2) + fo) * 16 + 4 * g;
        if (m < p.M && nb < p.N) {
          float sv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            sv[e] = acc[fo][i][e] / (1.0f + __expf(-acc[fo][i][e])) * acc[fo + kNF / 2][i][e];
          *reinterpret_cast<u32x2*>(p.out + (long long)m * p.ld_out + nb) =
              u32x2{pack_bf2(sv[0], sv[1]), pack_bf2(sv[2], sv[3])};
        }
      }
  } else {
    // per row: the best of the wave's columns, then of the column waves
    unsigned long long* kbest = reinterpret_cast<unsigned long long*>(&lds[0][0][0]);  // [kWavesN][kBM]
    __syncthreads();  // every wave is done reading the stages
#pragma unroll
    for (int i = 0; i < kAFW; ++i) {
      const int m = m0 + wm * (kBM / WM) + i * 16 + r;
      float bv = -__builtin_inff();
      int bn = 0x7FFFFFFF;
#pragma unroll
      for (int f = 0; f < kNF; ++f) {
        const int nb = bx * kBN + (wn * kNF + f) * 16 + 4 * g;
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
      if (g == 0) kbest[wn * kBM + wm * (kBM / WM) + i * 16 + r] = bn != 0x7FFFFFFF ? argmax_key(bv, bn) : 0ull;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kBM; i += S::kThreads) {
      const int m = m0 + i;
      if (m < p.M) {
        unsigned long long k = kbest[i];
#pragma unroll
        for (int w = 1; w < kWavesN; ++w) k = max(k, kbest[w * kBM + i]);
        p.keys[(long long)bx * p.ld_keys + m] = k;
      }
    }
  }
}

template <int MODE, int BM, int BN, int WM>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_big8_kernel(const GemmParams p) {
  gemm_big_body<MODE, BM, BN, WM>(p);
}

template <int MODE, int BM, int BN, int WM>
hipError_t launch_one(const GemmParams& p, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((gemm_big8_kernel<MODE, BM, BN, WM>), grid, dim3(512), 0, st, p);
  return hipGetLastError();
}

}  // namespace

int gemm_big_cols(int mode, int bn) { return mode == kGemmSwiglu ? bn / 2 : bn; }

hipError_t launch_gemm_big(const GemmParams& p, int mode, int nz, int bm, int bn, hipStream_t st) {
  // tile shapes: 256 x 256 for every mode, 128 x 256, 128 x 192 and 128 x
  // 128 for split-K partials, 256 x 192 (four waves along the rows) for the
  // SwiGLU
  const bool ok = (bm == 256 && bn == 256) ||
                  (mode == kGemmPartial && bm == 128 && (bn == 256 || bn == 192 || bn == 128)) ||
                  (mode == kGemmSwiglu && bm == 256 && bn == 192);
  if (!ok) return hipErrorInvalidValue;
  if (p.K % 32 || p.k_per_split % 32 || p.k_per_split < 32 || p.n_mats != nz || p.M < 1 || p.N < 16)
    return hipErrorInvalidValue;
  if (mode == kGemmSwiglu && p.splits != 1) return hipErrorInvalidValue;
  if (mode == kGemmArgmax && p.splits != 1) return hipErrorInvalidValue;
  // the kernel addresses activation rows with 32-bit element offsets from p.A
  const long long rows = p.a_idx ? p.a_idx_max : p.M;
  if ((rows - 1) * p.lda + p.K > 0x7FFFFFFFll) return hipErrorInvalidValue;
  const long long m_tiles = (p.M + bm - 1) / bm;
  const long long n_tiles = (p.N + gemm_big_cols(mode, bn) - 1) / gemm_big_cols(mode, bn);
  const long long total = m_tiles * n_tiles * p.splits * nz;
  const long long grid = (total + 7) / 8 * 8;
  if (grid > 0x7FFFFFFFll) return hipErrorInvalidValue;
  const dim3 g((unsigned)grid);
  if (mode == kGemmPartial) {
    if (bm == 256) return launch_one<kGemmPartial, 256, 256, 2>(p, g, st);
    if (bn == 256) return launch_one<kGemmPartial, 128, 256, 2>(p, g, st);
    return bn == 192 ? launch_one<kGemmPartial, 128, 192, 2>(p, g, st) : launch_one<kGemmPartial, 128, 128, 2>(p, g, st);
  }
  if (mode == kGemmSwiglu)
    return bn == 256 ? launch_one<kGemmSwiglu, 256, 256, 2>(p, g, st) : launch_one<kGemmSwiglu, 256, 192, 4>(p, g, st);
  if (mode == kGemmArgmax) return launch_one<kGemmArgmax, 256, 256, 2>(p, g, st);
  return hipErrorInvalidValue;
}

}  // namespace dfl

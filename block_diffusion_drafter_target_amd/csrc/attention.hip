// Block attention of the draft step on gfx950.
//
// For sequence b and kv head g, the G = Hq/Hkv query heads times B block rows
// (G*B query rows, padded to 16) attend over the cache slots [0, L_b + B): the
// context followed by the block's own K/V, with no mask (a draft block) or
// causally inside the block (a target pass: row j sees slots < L_b + j + 1). Every
// key costs 4*D bytes of K+V and 4*D*G*B flops, so at G*B = 64..128 the kernel
// is bound by streaming K/V from HBM; MFMA keeps the arithmetic far below that
// bound.
//
// Decomposition: workgroup (4 waves) = (chunk u, kv head g). Every sequence
// is cut into chunks of one batch-wide length from its own first key, and
// the chunks of all sequences are numbered in order (attn_split.h: the length
// is picked from the real lengths so that a ragged batch gives its long
// sequences more chunks and no workgroup more keys than the others); the
// first layer's q/k/v pass writes that split once per pass and every layer
// reads it. Workgroups past the last chunk exit at once. A chunk is walked
// in 64-key slices
// staged through LDS (K row-major with a 16-byte XOR swizzle over the row's
// chunks, V row-major in padded rows, read through gfx950's transposing LDS
// loads),
// the next slice's global loads issued before the current slice's math.
// Wave w owns query tiles w, w+4, ... (16 query rows each).
//   S^T = K Q^T    A = K slice rows (LDS), B = Q^T (registers for the chunk)
//   O^T += V^T P^T A = V^T (transposing LDS reads), B = P^T straight from the S^T
//                  accumulators, so each lane keeps one query's softmax state
// Online softmax in base 2 (the queries arrive multiplied by log2(e)/sqrt(D));
// the row max combines the four lanes that share a query with two xor
// shuffles; the row sum comes from the matrix cores (one more O^T tile) with
// up to two query tiles per wave, else from the same shuffles. Each
// workgroup writes (max, sum, unnormalised O) to its chunk's slot; the merge
// kernel combines the chunks of a sequence with the log-sum-exp rule.
#include "attn_split.h"
#include "common.h"
#include "internal.h"

namespace dfl {

namespace {

// SL keys per LDS slice (64: the only length the launcher takes).
template <int D, int SL>
struct Slice {
  static constexpr int DC = D / 8;  // 16-byte chunks per key row
  static constexpr int KL = SL * DC / 256;
  static constexpr int VL = (SL / 2) * DC / 256;
  // bf16 per V row in LDS: 32 bytes of padding put the eight rows that one
  // transposing read serves at a time on disjoint banks
  static constexpr int VP = D + 16;
};

// Global -> registers: the K and V rows of keys [k0, k0 + SL), clamped to the
// last valid key (clamped rows are masked out of the softmax). K/V are read
// once per step, so the loads are non-temporal.
template <int D, int SL>
__device__ __forceinline__ void load_slice(u32x4 (&kreg)[(Slice<D, SL>::KL)], u32x4 (&va)[(Slice<D, SL>::VL)],
                                           u32x4 (&vb)[(Slice<D, SL>::VL)], const bf16_t* kc,
                                           const bf16_t* vc, int k0, int k_end) {
  constexpr int DC = Slice<D, SL>::DC;
  // 32-bit byte offsets from the (uniform) head base: one sequence's and kv
  // head's cache slab is below 4 GB (checked at launch)
  const char* kb = reinterpret_cast<const char*>(kc);
  const char* vb_ = reinterpret_cast<const char*>(vc);
#pragma unroll
  for (int t = 0; t < Slice<D, SL>::KL; ++t) {
    const int e = threadIdx.x + t * 256;
    const int key = e / DC, ch = e % DC;
    const uint32_t kidx = (uint32_t)min(k0 + key, k_end - 1);
    kreg[t] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb + (kidx * (2u * D) + 16u * ch)));
  }
#pragma unroll
  for (int t = 0; t < Slice<D, SL>::VL; ++t) {
    const int e = threadIdx.x + t * 256;
    const int kp = e / DC, ch = e % DC;
    const uint32_t k0i = (uint32_t)min(k0 + 2 * kp, k_end - 1), k1i = (uint32_t)min(k0 + 2 * kp + 1, k_end - 1);
    va[t] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vb_ + (k0i * (2u * D) + 16u * ch)));
    vb[t] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vb_ + (k1i * (2u * D) + 16u * ch)));
  }
}

// Registers -> LDS: K row-major with the 16-byte chunk index XOR (key & (DC-1));
// V row-major too (padded rows): the O^T pass reads it transposed.
template <int D, int SL>
__device__ __forceinline__ void store_slice(u32x4* ks, bf16_t* vr, const u32x4 (&kreg)[(Slice<D, SL>::KL)],
                                            const u32x4 (&va)[(Slice<D, SL>::VL)],
                                            const u32x4 (&vb)[(Slice<D, SL>::VL)]) {
  constexpr int DC = Slice<D, SL>::DC;
  constexpr int VP = Slice<D, SL>::VP;
#pragma unroll
  for (int t = 0; t < Slice<D, SL>::KL; ++t) {
    const int e = threadIdx.x + t * 256;
    const int key = e / DC, ch = e % DC;
    ks[key * DC + (ch ^ (key & (DC - 1)))] = kreg[t];
  }
#pragma unroll
  for (int t = 0; t < Slice<D, SL>::VL; ++t) {
    const int e = threadIdx.x + t * 256;
    const int kp = e / DC, ch = e % DC;
    *reinterpret_cast<u32x4*>(vr + (2 * kp) * VP + ch * 8) = va[t];
    *reinterpret_cast<u32x4*>(vr + (2 * kp + 1) * VP + ch * 8) = vb[t];
  }
}

// gfx950's transposing LDS read of 16-bit data: within each group of 16
// lanes, lane i receives element i & 3 of the 8-byte chunks addressed by
// lanes 4e + (i >> 2), e = 0..3 (so lanes 4e..4e+3 address four consecutive
// chunks of one row, and lane i gets column i of four rows).
__device__ __forceinline__ u32x2 lds_read_tr16(const bf16_t* p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// Waves per SIMD the register budget targets: two where a wave's accumulators,
// queries and scores fit 256 registers, else one (QPW = 4, or D = 128 with two
// query tiles per wave).
template <int D, int QPW>
struct AttnOcc {
  static constexpr int kWaves = (QPW >= 4 || (D == 128 && QPW >= 2)) ? 1 : 2;
};

template <int D, int QPW, int SL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(AttnOcc<D, QPW>::kWaves, AttnOcc<D, QPW>::kWaves)))
void attn_kernel(const AttnParams p) {
  constexpr int DC = Slice<D, SL>::DC;
  constexpr int KL = Slice<D, SL>::KL;
  constexpr int VL = Slice<D, SL>::VL;
  constexpr int VP = Slice<D, SL>::VP;
  static_assert(KL >= 1 && VL >= 1, "slice too small");
  // D = 64: scores one slice ahead of the softmax, slices in two LDS buffers
  // (measured on MI355X: the gpt-oss-shaped attention 573 -> 544 us per step);
  // D = 128 keeps one buffer and one slice at a time (the pipelined loop
  // measured 1-2% slower there, and 12% slower for chunks of one slice)
  constexpr bool kPipe = D == 64;
  constexpr int NBUF = kPipe ? 2 : 1;
  // Lean softmax: the reference moves only when a score exceeds it by more
  // than 2^8 (a wave-uniform branch, so the rescale of O is skipped on almost
  // every slice; weights stay <= 256, exact in fp32 and in the bf16 operand),
  // and the row sums come out of the matrix cores as one more O^T tile
  // against an all-ones operand (measured with the D = 64 pipeline 546 -> 530
  // us per step; at D = 128 1-2% once the V store stopped transposing). Not
  // with four query tiles per wave (the extra accumulators would spill).
  constexpr bool kLean = QPW <= 2;
  __shared__ __align__(16) u32x4 ks[NBUF][SL * DC];
  __shared__ __align__(16) bf16_t vt[NBUF][SL * VP];

  const int u = blockIdx.x, g = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, gq = lane >> 4;
  const int G = p.Hq / p.Hkv;
  const int GB = G * p.B;
  const int QT = p.gb_pad / 16;
  // chunk u of the batch's split (read from the plan; uniform, so scalar)
  const int b_u = p.plan[1 + u];
  if (b_u < 0) return;
  const int C = p.plan[0];
  const int k0_u = p.plan[1 + p.n_ranges + u] * C;
  const int Lk_u = p.ctx_len[b_u] + p.B;

  // Chunk u: keys [k_start, k_end) of sequence b (Lk keys in all), its
  // (max, sum, O) partials to slot u.
  auto run_chunk = [&](int b, int Lk, int k_start, int k_end, int slot) __attribute__((always_inline)) {
    // queries of this wave, as MFMA B operands (column = query, k = d); jrow
    // is the block row of this lane's query column
    u32x4 qreg[QPW][D / 32];
    int jrow[QPW];
#pragma unroll
    for (int i = 0; i < QPW; ++i) {
      const int qt = wave + 4 * i;
      int rr = qt * 16 + r;
      rr = rr < GB ? rr : GB - 1;
      const int hl = rr / p.B, j = rr % p.B;
      jrow[i] = j;
      const bf16_t* qrow = p.q + ((long long)(b * p.B + j) * p.Hq + g * G + hl) * D + gq * 8;
      // rows past GB read the last row (valid memory); padded tiles are zeroed
      // by a select, not a guarded load
      const uint32_t keep = qt < QT ? 0xFFFFFFFFu : 0u;
#pragma unroll
      for (int ds = 0; ds < D / 32; ++ds) qreg[i][ds] = *reinterpret_cast<const u32x4*>(qrow + ds * 32) & keep;
    }

    // mrun: the lane's softmax reference (scaled base-2 units); o and the row
    // sums (lrun, or lsum: an O^T tile of the all-ones operand whose every
    // element is the row sum of the bf16 probabilities) hold sums of
    // exp2(s * c - mrun)
    float mrun[QPW], lrun[QPW];
    f32x4_t o[QPW][D / 16], lsum[QPW];
#pragma unroll
    for (int i = 0; i < QPW; ++i) {
      mrun[i] = -__builtin_inff();
      lrun[i] = 0.f;
      lsum[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) o[i][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    const u32x4 ones = u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    // lean path: the score MFMAs start from -mref (mref = mrun, or 0 before
    // the first visible key), so their results are already s * c - mref
    f32x4_t cref[QPW];
#pragma unroll
    for (int i = 0; i < QPW; ++i) cref[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const long long head_off = ((long long)b * p.Hkv + g) * p.max_ctx * D;
    const bf16_t* kc = p.k + head_off;
    const bf16_t* vc = p.v + head_off;

    u32x4 kreg[KL], va[VL], vb[VL];

    constexpr int KT = SL / 16;  // 16-key tiles per slice
    // S^T tiles of every query tile of the wave from the K slice in buffer
    // bi; each K fragment is read from LDS once and feeds all of them
    auto scores = [&](int bi, f32x4_t(&sacc)[QPW][KT]) __attribute__((always_inline)) {
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        const int key = kt * 16 + r;
#pragma unroll
        for (int ds = 0; ds < D / 32; ++ds) {
          const u32x4 a = ks[bi][key * DC + ((ds * 4 + gq) ^ (key & (DC - 1)))];
#pragma unroll
          for (int i = 0; i < QPW; ++i) {
            const f32x4_t c0 = kLean ? cref[i] : f32x4_t{0.f, 0.f, 0.f, 0.f};
            sacc[i][kt] = mfma16x16x32(a, qreg[i][ds], ds == 0 ? c0 : sacc[i][kt]);
          }
        }
      }
    };
    // keys past the end exist only in the chunk's last slice; in a causal
    // block, row j also drops the block keys after its own position
    const int lim0 = Lk - p.B + 1;  // key limit of block row 0
    auto mask = [&](int k0, f32x4_t(&sacc)[QPW][KT]) __attribute__((always_inline)) {
      if (k0 + SL > k_end || (p.causal && k0 + SL > lim0)) {
        int lim[QPW];
#pragma unroll
        for (int i = 0; i < QPW; ++i) lim[i] = p.causal ? min(k_end, lim0 + jrow[i]) : k_end;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int key = k0 + kt * 16 + 4 * gq + e;
#pragma unroll
            for (int i = 0; i < QPW; ++i)
              if (key >= lim[i]) sacc[i][kt][e] = -__builtin_inff();
          }
      }
    };
    // online softmax of one slice's scores (s * c, the running max in the same
    // scaled base-2 units), then O^T += V^T P^T from the V slice in buffer bi.
    // The lean path's scores arrive relative to the reference (s * c - mref):
    // when the reference moves by delta, this slice's scores and the next
    // slice's (nxt: already issued against the old reference) drop by delta.
    auto accumulate = [&](int bi, f32x4_t(&sacc)[QPW][KT], f32x4_t(&nxt)[QPW][KT]) __attribute__((always_inline)) {
      u32x4 pb[QPW][KT / 2];
#pragma unroll
      for (int i = 0; i < QPW; ++i) {
        float mx = -__builtin_inff();
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int e = 0; e < 4; ++e) mx = fmaxf(mx, sacc[i][kt][e]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        // a causal row may have no visible key yet: its reference is then 0,
        // and its weights exp2(-inf) = 0 instead of NaN
        if constexpr (kLean) {
          const float mref = mrun[i] == -__builtin_inff() ? 0.f : mrun[i];
          const float thr = mrun[i] == -__builtin_inff() ? -__builtin_inff() : 8.f;
          if (__builtin_amdgcn_ballot_w64(mx > thr) != 0) {
            const float mnew = fmaxf(mrun[i], mref + mx);
            const float alpha = mnew == -__builtin_inff() ? 1.f : fast_exp2(mrun[i] - mnew);
            mrun[i] = mnew;
            lsum[i] *= alpha;
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) o[i][dt] *= alpha;
            const float rnew = mnew == -__builtin_inff() ? 0.f : mnew;
            const float delta = rnew - mref;
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                sacc[i][kt][e] -= delta;
                if constexpr (kPipe) nxt[i][kt][e] -= delta;
              }
            cref[i] = f32x4_t{-rnew, -rnew, -rnew, -rnew};
          }
#pragma unroll
          for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int e = 0; e < 4; ++e) sacc[i][kt][e] = fast_exp2(sacc[i][kt][e]);
        } else {
          const float mnew = fmaxf(mrun[i], mx);
          const float alpha = mnew == -__builtin_inff() ? 1.f : fast_exp2(mrun[i] - mnew);
          mrun[i] = mnew;
          lrun[i] *= alpha;
#pragma unroll
          for (int dt = 0; dt < D / 16; ++dt) o[i][dt] *= alpha;
          const float mref = mnew == -__builtin_inff() ? 0.f : mnew;
#pragma unroll
          for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int e = 0; e < 4; ++e) sacc[i][kt][e] = fast_exp2(sacc[i][kt][e] - mref);
        }
        if constexpr (!kLean) {
          float rs = 0.f;
#pragma unroll
          for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int e = 0; e < 4; ++e) rs += sacc[i][kt][e];
          rs += __shfl_xor(rs, 16);
          rs += __shfl_xor(rs, 32);
          lrun[i] += rs;
        }
        // P^T as the B operand: keys 32h + 4gq.. and 32h + 16 + 4gq.. of lane
        // group gq, the same key order as the V^T operand below
#pragma unroll
        for (int h = 0; h < KT / 2; ++h)
          pb[i][h] = u32x4{pack_bf2(sacc[i][2 * h][0], sacc[i][2 * h][1]),
                           pack_bf2(sacc[i][2 * h][2], sacc[i][2 * h][3]),
                           pack_bf2(sacc[i][2 * h + 1][0], sacc[i][2 * h + 1][1]),
                           pack_bf2(sacc[i][2 * h + 1][2], sacc[i][2 * h + 1][3])};
      }
      // each V^T fragment is read once for all query tiles
#pragma unroll
      for (int h = 0; h < KT / 2; ++h) {
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          // lane (gq, r) gets V[keys 32h + 4gq + 0..3 (lo), + 16 (hi)][d = 16dt + r]
          const bf16_t* row = vt[bi] + (32 * h + 4 * gq + (r >> 2)) * VP + dt * 16 + 4 * (r & 3);
          const u32x2 lo = lds_read_tr16(row);
          const u32x2 hi = lds_read_tr16(row + 16 * VP);
          const u32x4 a = u32x4{lo.x, lo.y, hi.x, hi.y};
#pragma unroll
          for (int i = 0; i < QPW; ++i) o[i][dt] = mfma16x16x32(a, pb[i][h], o[i][dt]);
        }
        if constexpr (kLean) {
#pragma unroll
          for (int i = 0; i < QPW; ++i) lsum[i] = mfma16x16x32(ones, pb[i][h], lsum[i]);
        }
      }
    };
    // Pipelined (kPipe): slices in two LDS buffers, the scores one slice
    // ahead of the softmax. A step holds slice k in buffer bi with its scores
    // in cur: it stores slice k + 1 into the other buffer (whose last reader,
    // O^T of slice k - 1, finished before the previous step's closing
    // barrier), publishes it, issues slice k + 2's global loads, and then
    // computes the scores of k + 1 into nxt beside the softmax and O^T of
    // slice k (independent MFMA work the scheduler interleaves with the
    // VALU). Past the chunk's end the store, loads and scores still run (the
    // loads re-read the last key: valid memory) and are never used, which
    // keeps the step one block of straight-line code.
    f32x4_t sa[QPW][KT];
    load_slice<D, SL>(kreg, va, vb, kc, vc, k_start, k_end);
    if constexpr (kPipe) {
      auto step = [&](int bi, int k0, f32x4_t(&cur)[QPW][KT], f32x4_t(&nxt)[QPW][KT]) __attribute__((always_inline)) {
        store_slice<D, SL>(ks[bi ^ 1], vt[bi ^ 1], kreg, va, vb);
        __syncthreads();
        load_slice<D, SL>(kreg, va, vb, kc, vc, k0 + 2 * SL, k_end);
        mask(k0, cur);
        scores(bi ^ 1, nxt);
        accumulate(bi, cur, nxt);
        __syncthreads();
      };
      f32x4_t sb[QPW][KT];
      store_slice<D, SL>(ks[0], vt[0], kreg, va, vb);
      __syncthreads();
      load_slice<D, SL>(kreg, va, vb, kc, vc, k_start + SL, k_end);
      scores(0, sa);
      for (int k0 = k_start; k0 < k_end; k0 += 2 * SL) {
        step(0, k0, sa, sb);
        if (k0 + SL >= k_end) break;
        step(1, k0 + SL, sb, sa);
      }
    } else {
      // one buffer: store the slice, publish it, prefetch the next one (past
      // the end it re-reads the last key: valid memory, never used), then
      // scores, softmax and O^T of this slice
      for (int k0 = k_start; k0 < k_end; k0 += SL) {
        store_slice<D, SL>(ks[0], vt[0], kreg, va, vb);
        __syncthreads();
        load_slice<D, SL>(kreg, va, vb, kc, vc, k0 + SL, k_end);
        scores(0, sa);
        mask(k0, sa);
        accumulate(0, sa, sa);
        __syncthreads();
      }
    }

    const long long base = ((long long)g * p.slots + slot) * p.gb_pad;
#pragma unroll
    for (int i = 0; i < QPW; ++i) {
      const int qt = wave + 4 * i;
      if (qt >= QT) continue;
      const int rr = qt * 16 + r;
      if (gq == 0) {
        p.pm[base + rr] = mrun[i];
        p.pl[base + rr] = kLean ? lsum[i][0] : lrun[i];
      }
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
        *reinterpret_cast<f32x4_t*>(p.po + (base + rr) * D + dt * 16 + 4 * gq) = o[i][dt];
    }
  };

  run_chunk(b_u, Lk_u, k0_u, min(Lk_u, k0_u + C), u);
}

// o[m][h] = sum_c exp2(m_c - M) O_c / sum_c exp2(m_c - M) l_c over the
// chunks of the sequence. One wave per (row, head); lane c holds chunk c's
// statistics, lane i output elements E i .. E i + E - 1 (E = D / 64, one
// load of E floats per chunk). The statistics and the first NB chunks'
// partial outputs are loaded in one round trip (NB covers the typical chunk
// count up to 32; more take further rounds); the weights are applied once
// the wave's maximum is known.
template <int NB, int D>
__global__ __launch_bounds__(256) void merge_kernel(const MergeParams p) {
  constexpr int kMergeBatch = NB;
  constexpr int E = D / 64;
  static_assert(E == 1 || E == 2, "head size 64 or 128");
  typedef float fE __attribute__((ext_vector_type(E)));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = blockIdx.y;
  const int h = blockIdx.x * 4 + wave;
  if (h >= p.Hq) return;
  const int b = m / p.B, j = m % p.B;
  bf16_t* out = p.out + ((long long)m * p.Hq + h) * D;
  const int st = p.status[b];
  const int G = p.Hq / p.Hkv;
  const int g = h / G, rr = (h % G) * p.B + j;
  // the sequence's chunks: nch consecutive slots from its first (none for a
  // sequence with an error status; at most 64 by the chunk length's bound)
  const int32_t* first = p.plan + 1 + 2 * p.n_ranges;
  const int s0 = first[b], nch = first[p.batch + b];
  // (a sequence without chunks may have s0 == slots: its loads, never used,
  // stay in the buffer)
  const long long base = (long long)g * p.slots + min(s0, p.slots - 1);
  // Loads are unconditional at clamped chunk indexes: a guarded load becomes a
  // branch, and the compiler waits for every outstanding load where branches
  // join. Chunks past nch carry weight 0.
  const int clast = max(nch - 1, 0);
  const long long sl = (base + min(lane, clast)) * p.gb_pad + rr;
  float mc = p.pm[sl];
  float lc = p.pl[sl];
  fE a[kMergeBatch];
  auto load = [&](int c0) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < kMergeBatch; ++t) {
      const float* po = p.po + ((base + min(c0 + t, clast)) * p.gb_pad + rr) * D;
      a[t] = *reinterpret_cast<const fE*>(po + E * lane);
    }
  };
  load(0);
  // keep the whole batch of loads ahead of the reductions below
  __builtin_amdgcn_sched_barrier(0);
  if (lane >= nch) {
    mc = -__builtin_inff();
    lc = 0.f;
  }
  const float M = wave_max(mc);
  const float w = lane < nch ? fast_exp2(mc - M) : 0.f;
  const float l = wave_sum(w * lc);
  fE o = {};
  for (int c0 = 0; c0 < nch; c0 += kMergeBatch) {
    if (c0 > 0) load(c0);
#pragma unroll
    for (int t = 0; t < kMergeBatch; ++t) {
      const float wc = __shfl(w, (c0 + t) & 63);
      if (c0 + t < nch) o += wc * a[t];
    }
  }
  // a sequence with an error status gets zeros (selected, not multiplied:
  // its partials are never written)
  const float inv = 1.0f / l;
  if constexpr (E == 1) {
    out[lane] = f2bf(st != 0 ? 0.f : o[0] * inv);
  } else {
    *reinterpret_cast<uint32_t*>(out + 2 * lane) =
        pack_bf2(st != 0 ? 0.f : o[0] * inv, st != 0 ? 0.f : o[1] * inv);
  }
}

template <int D, int SL>
hipError_t launch_ds(const AttnParams& p, hipStream_t st) {
  dim3 grid(p.n_ranges, p.Hkv);
  const int qt = p.gb_pad / 16;
  if (qt <= 4)
    hipLaunchKernelGGL((attn_kernel<D, 1, SL>), grid, dim3(256), 0, st, p);
  else if (qt <= 8)
    hipLaunchKernelGGL((attn_kernel<D, 2, SL>), grid, dim3(256), 0, st, p);
  else if (qt <= 16) {
    hipLaunchKernelGGL((attn_kernel<D, 4, SL>), grid, dim3(256), 0, st, p);
  } else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnParams& p, hipStream_t st) {
  if (p.slice == 64) return launch_ds<D, 64>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_attention(const AttnParams& p, int D, hipStream_t st) {
  if (p.n_ranges < p.batch || p.batch < 1 || p.slots < p.n_ranges) return hipErrorInvalidValue;
  // the slice loads address one (sequence, kv head) slab with 32-bit byte offsets
  if (p.max_ctx < 1 || (long long)p.max_ctx * D * 2 > 0xFFFFFFFFll) return hipErrorInvalidValue;
  if (D == 128) return launch_d<128>(p, st);
  if (D == 64) return launch_d<64>(p, st);
  return hipErrorInvalidValue;
}

template <int D>
hipError_t launch_merge_d(const MergeParams& p, dim3 grid, hipStream_t st) {
  if (p.seg_hint <= 4)
    hipLaunchKernelGGL((merge_kernel<4, D>), grid, dim3(256), 0, st, p);
  else if (p.seg_hint <= 8)
    hipLaunchKernelGGL((merge_kernel<8, D>), grid, dim3(256), 0, st, p);
  else if (p.seg_hint <= 16)
    hipLaunchKernelGGL((merge_kernel<16, D>), grid, dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((merge_kernel<32, D>), grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_attn_merge(const MergeParams& p, hipStream_t st) {
  if (p.n_ranges < p.batch || p.batch < 1 || p.slots < p.n_ranges) return hipErrorInvalidValue;
  const dim3 grid((p.Hq + 3) / 4, p.batch * p.B);
  if (p.D == 64) return launch_merge_d<64>(p, grid, st);
  if (p.D == 128) return launch_merge_d<128>(p, grid, st);
  return hipErrorInvalidValue;
}

}  // namespace dfl

// Row-wise kernels of the draft step (gfx950): embedding + RMSNorm, split-K
// reduction + residual + RMSNorm, per-head q/k RMSNorm + RoPE + KV-cache
// append, the inject epilogue (k-norm + RoPE + cache scatter + commit
// of ctx_len), the final argmax over the LM-head tiles, the combine pass of a
// split SwiGLU, and the commit of rows whose K/V are already cached.
//
// All are bound by a few kilobytes per row; they exist to keep every fp32
// statistic (RMSNorm sums, residual stream, RoPE) on the device between the
// bf16 MFMA GEMMs.
#include "attn_split.h"
#include "common.h"
#include "internal.h"

namespace dfl {

namespace {

constexpr int kErrCapacity = -5;  // DFLASH_ERR_CAPACITY
constexpr int kErrShape = -2;     // DFLASH_ERR_SHAPE

constexpr int kRowThreads = 512;
// float4 columns per thread: rows of up to 8192. The row kernels are
// instantiated for 1, 2 and 4 of them and launched with the fewest that cover
// the row (at 4096 columns two, 112 registers and two workgroups per CU instead
// of 214 and one: Qwen3-8B-shaped drafter step at batch 1 813 -> 799 us,
// batch 32 2521 -> 2492, gpt-oss-shaped 1271 -> 1252, measured on MI355X)
constexpr int kMaxC4 = 4;
constexpr int kSplitBatch = 8;  // split partials loaded together

__device__ __forceinline__ float block_sum_512(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < kRowThreads / 64; ++w) t += red[w];
  return t;
}

// Adds the split partials of row m, columns 4*i4.., to v. All loads of a
// batch of splits are issued before any add, so the row costs one memory
// round trip per kSplitBatch splits. Loads are unconditional at clamped
// addresses (a guarded load becomes a branch, and the compiler waits for
// every outstanding load where branches join); out-of-range values are
// dropped by a select.
// SB splits per batch; add_splits picks the smallest batch that covers the
// split count (one split, a whole ingest chunk, would otherwise load eight
// copies of the same partial).
template <int SB, int C4>
__device__ __forceinline__ void add_splits_sb(f32x4_t (&v)[C4], const float* P, long long s_stride,
                                              int splits, long long row_off, int n4, float keep_v) {
  constexpr int kSplitBatch = SB;
  for (int s0 = 0; s0 < splits; s0 += kSplitBatch) {
    f32x4_t t[C4][kSplitBatch];
#pragma unroll
    for (int c = 0; c < C4; ++c) {
      const int i4 = min(threadIdx.x + c * kRowThreads, n4 - 1);
#pragma unroll
      for (int j = 0; j < kSplitBatch; ++j) {
        const int sj = min(s0 + j, splits - 1);
        t[c][j] = *reinterpret_cast<const f32x4_t*>(P + (long long)sj * s_stride + row_off + 4 * i4);
      }
    }
    if (s0 == 0) {
#pragma unroll
      for (int c = 0; c < C4; ++c) v[c] *= keep_v;
    }
#pragma unroll
    for (int c = 0; c < C4; ++c)
#pragma unroll
      for (int j = 0; j < kSplitBatch; ++j)
        if (threadIdx.x + c * kRowThreads < n4 && s0 + j < splits) v[c] += t[c][j];
  }
}

template <int C4>
__device__ __forceinline__ void add_splits(f32x4_t (&v)[C4], const float* P, long long s_stride,
                                           int splits, long long row_off, int n4, float keep_v) {
  if (splits == 1)
    add_splits_sb<1, C4>(v, P, s_stride, splits, row_off, n4, keep_v);
  else if (splits <= 2)
    add_splits_sb<2, C4>(v, P, s_stride, splits, row_off, n4, keep_v);
  else if (splits <= 4)
    add_splits_sb<4, C4>(v, P, s_stride, splits, row_off, n4, keep_v);
  else
    add_splits_sb<kSplitBatch, C4>(v, P, s_stride, splits, row_off, n4, keep_v);
}

// Unpacks four bf16 (two 32-bit words) to fp32.
__device__ __forceinline__ f32x4_t bf4_to_f32(u32x2 w) {
  return f32x4_t{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u), __uint_as_float(w.y << 16),
                 __uint_as_float(w.y & 0xFFFF0000u)};
}

// ---------------------------------------------------------------------------
// block row embedding: x = E[token], u = bf16(RMSNorm(x) * g_in of layer 0)
// Row j of sequence b holds the anchor (j = 0) or the mask id (a draft block),
// or the given token (a target pass). The j == 0 workgroup also records the
// sequence's capacity status.
template <int C4>
__global__ __launch_bounds__(kRowThreads) void embed_kernel(const EmbedParams p) {
  __shared__ float red[kRowThreads / 64];
  const int m = blockIdx.x;
  const int b = m / p.B, j = m % p.B;
  const int L = p.ctx_len[b];
  const bool cap_bad = L < 0 || L + p.B > p.max_ctx || L + p.B > p.rope_max;
  int tok = p.tokens ? p.tokens[(long long)b * p.B + j] : (j == 0 ? p.anchor[b] : p.mask_id);
  const bool tok_bad = tok < 0 || tok >= p.V;
  if (j == 0 && threadIdx.x == 0) p.status[b] = cap_bad ? kErrCapacity : (tok_bad ? kErrShape : 0);
  if (tok_bad) tok = 0;
  const bf16_t* e = p.embed + (long long)tok * p.H;
  const int n4 = p.H / 4;
  // unconditional loads at clamped columns (see add_splits)
  u32x2 ew[C4], gw[C4];
#pragma unroll
  for (int c = 0; c < C4; ++c) {
    const int i4 = min(threadIdx.x + c * kRowThreads, n4 - 1);
    ew[c] = *reinterpret_cast<const u32x2*>(e + 4 * i4);
    gw[c] = *reinterpret_cast<const u32x2*>(p.gain + 4 * i4);
  }
  f32x4_t v[C4];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < C4; ++c) {
    const int i4 = threadIdx.x + c * kRowThreads;
    v[c] = i4 < n4 ? bf4_to_f32(ew[c]) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (i4 < n4) {
      *reinterpret_cast<f32x4_t*>(p.x + (long long)m * p.H + 4 * i4) = v[c];
      if (p.dbg) *reinterpret_cast<f32x4_t*>(p.dbg + (long long)m * p.H + 4 * i4) = v[c];
    }
    ss += v[c][0] * v[c][0] + v[c][1] * v[c][1] + v[c][2] * v[c][2] + v[c][3] * v[c][3];
  }
  ss = block_sum_512(ss, red);
  const float inv = 1.0f / sqrtf(ss / (float)p.H + p.eps);
#pragma unroll
  for (int c = 0; c < C4; ++c) {
    const int i4 = threadIdx.x + c * kRowThreads;
    if (i4 < n4) {
      const f32x4_t g = bf4_to_f32(gw[c]);
      const u32x2 o = u32x2{pack_bf2(v[c][0] * inv * g[0], v[c][1] * inv * g[1]),
                            pack_bf2(v[c][2] * inv * g[2], v[c][3] * inv * g[3])};
      *reinterpret_cast<u32x2*>(p.u + (long long)m * p.H + 4 * i4) = o;
    }
  }
}

// The embedding pass in the split form of the RMSNorm (see row_split_kernel):
// one wave per (kRowChunkCols-column chunk, row); chunk 0 of a sequence's first
// row writes its status.
__global__ __launch_bounds__(64) void embed_split_kernel(const EmbedParams p) {
  const int m = blockIdx.y, c = blockIdx.x;
  const int b = m / p.B, j = m % p.B;
  const int L = p.ctx_len[b];
  const bool cap_bad = L < 0 || L + p.B > p.max_ctx || L + p.B > p.rope_max;
  int tok = p.tokens ? p.tokens[(long long)b * p.B + j] : (j == 0 ? p.anchor[b] : p.mask_id);
  const bool tok_bad = tok < 0 || tok >= p.V;
  if (j == 0 && c == 0 && threadIdx.x == 0) p.status[b] = cap_bad ? kErrCapacity : (tok_bad ? kErrShape : 0);
  if (tok_bad) tok = 0;
  const int n4 = p.H / 4;
  const int i4 = c * (kRowChunkCols / 4) + threadIdx.x;
  const int ci = min(i4, n4 - 1);
  const u32x2 gw = *reinterpret_cast<const u32x2*>(p.gain + 4 * ci);
  const u32x2 ew = *reinterpret_cast<const u32x2*>(p.embed + (long long)tok * p.H + 4 * ci);
  f32x4_t v = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if (i4 < n4) {
    v = bf4_to_f32(ew);
    *reinterpret_cast<f32x4_t*>(p.x + (long long)m * p.H + 4 * i4) = v;
    if (p.dbg) *reinterpret_cast<f32x4_t*>(p.dbg + (long long)m * p.H + 4 * i4) = v;
    const f32x4_t g = bf4_to_f32(gw);
    *reinterpret_cast<u32x2*>(p.u + (long long)m * p.H + 4 * i4) =
        u32x2{pack_bf2(v[0] * g[0], v[1] * g[1]), pack_bf2(v[2] * g[2], v[3] * g[3])};
  }
  const float ss = wave_sum(v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3]);
  if (threadIdx.x == 0) p.ssp[(long long)m * kMaxRowChunks + c] = ss;
}

// ---------------------------------------------------------------------------
// y = (x +=) sum of split partials (at least one split); out =
// bf16(RMSNorm(y) * gain)
template <int C4>
__global__ __launch_bounds__(kRowThreads) void row_norm_kernel(const RowNormParams p) {
  __shared__ float red[kRowThreads / 64];
  const int m = blockIdx.x;
  const int n = p.n, n4 = n / 4;
  const long long row_off = (long long)m * n;
  // the row, its split partials and the gains are independent loads, issued
  // unconditionally at clamped columns before the first use (see add_splits)
  f32x4_t v[C4];
  u32x2 gw[C4];
#pragma unroll
  for (int c = 0; c < C4; ++c) {
    const int i4 = min(threadIdx.x + c * kRowThreads, n4 - 1);
    gw[c] = *reinterpret_cast<const u32x2*>(p.gain + 4 * i4);
  }
  // without a residual the row loads read the first split instead (valid
  // memory, values dropped), so no branch separates them from the partials
  const float* xs = p.x ? p.x : p.P;
  const float keep_x = p.x ? 1.f : 0.f;
#pragma unroll
  for (int c = 0; c < C4; ++c) {
    const int i4 = min(threadIdx.x + c * kRowThreads, n4 - 1);
    v[c] = *reinterpret_cast<const f32x4_t*>(xs + row_off + 4 * i4);
  }
  add_splits(v, p.P, p.p_s_stride, p.splits, row_off, n4, keep_x);
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < C4; ++c) {
    const int i4 = threadIdx.x + c * kRowThreads;
    if (i4 >= n4) v[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (i4 < n4) {
      if (p.x) *reinterpret_cast<f32x4_t*>(p.x + row_off + 4 * i4) = v[c];
      if (p.dbg) *reinterpret_cast<f32x4_t*>(p.dbg + row_off + 4 * i4) = v[c];
      if (p.tap)
        *reinterpret_cast<u32x2*>(p.tap + (long long)m * p.tap_ld + 4 * i4) =
            u32x2{pack_bf2(v[c][0], v[c][1]), pack_bf2(v[c][2], v[c][3])};
    }
    ss += v[c][0] * v[c][0] + v[c][1] * v[c][1] + v[c][2] * v[c][2] + v[c][3] * v[c][3];
  }
  ss = block_sum_512(ss, red);
  const float inv = 1.0f / sqrtf(ss / (float)n + p.eps);
  bf16_t* out;
  if (p.final_mode) {
    const int b = m / p.B, j = m % p.B;
    if (j == 0) return;
    const int row = b * (p.B - 1) + j - 1;
    out = p.out + (long long)row * n;
  } else {
    out = p.out + row_off;
  }
#pragma unroll
  for (int c = 0; c < C4; ++c) {
    const int i4 = threadIdx.x + c * kRowThreads;
    if (i4 < n4) {
      const f32x4_t g = bf4_to_f32(gw[c]);
      const u32x2 o = u32x2{pack_bf2(v[c][0] * inv * g[0], v[c][1] * inv * g[1]),
                            pack_bf2(v[c][2] * inv * g[2], v[c][3] * inv * g[3])};
      *reinterpret_cast<u32x2*>(out + 4 * i4) = o;
    }
  }
}

// Split RMSNorm for few rows whose consumer is the weight-streaming GEMM: one
// wave per (kRowChunkCols-column chunk, row) sums the chunk's split partials
// into the residual (or takes them alone), writes x back (and the debug and
// tap copies), out = bf16(x * gain) and the chunk's sum of squares to ssp; the
// GEMM multiplies its products by the row's 1/rms. One workgroup per row put a
// 16-row pass on 16 CUs, each reading a whole row's partials (up to 144 KB);
// this grid spreads them over rows * n / 256 waves (measured on MI355X with
// the row scale left out: Qwen3-8B-shaped drafter step at batch 1, eleven
// row passes, 794 -> 777 us).
__global__ __launch_bounds__(64) void row_split_kernel(const RowNormParams p) {
  const int m = blockIdx.y, c = blockIdx.x;
  const int n4 = p.n / 4;
  const int i4 = c * (kRowChunkCols / 4) + threadIdx.x;
  const int ci = min(i4, n4 - 1);
  const long long row_off = (long long)m * p.n;
  // independent loads at clamped columns first (see add_splits); without a
  // residual the row load reads the first split (valid memory, dropped)
  const u32x2 gw = *reinterpret_cast<const u32x2*>(p.gain + 4 * ci);
  const float* xs = p.x ? p.x : p.P;
  const float keep_x = p.x ? 1.f : 0.f;
  f32x4_t v = *reinterpret_cast<const f32x4_t*>(xs + row_off + 4 * ci) * keep_x;
  for (int s0 = 0; s0 < p.splits; s0 += kSplitBatch) {
    f32x4_t a[kSplitBatch];
#pragma unroll
    for (int k = 0; k < kSplitBatch; ++k)
      a[k] = *reinterpret_cast<const f32x4_t*>(p.P + (long long)min(s0 + k, p.splits - 1) * p.p_s_stride + row_off +
                                               4 * ci);
#pragma unroll
    for (int k = 0; k < kSplitBatch; ++k)
      if (s0 + k < p.splits) v += a[k];
  }
  if (i4 >= n4) {
    v = f32x4_t{0.f, 0.f, 0.f, 0.f};
  } else {
    if (p.x) *reinterpret_cast<f32x4_t*>(p.x + row_off + 4 * i4) = v;
    if (p.dbg) *reinterpret_cast<f32x4_t*>(p.dbg + row_off + 4 * i4) = v;
    if (p.tap)
      *reinterpret_cast<u32x2*>(p.tap + (long long)m * p.tap_ld + 4 * i4) =
          u32x2{pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3])};
  }
  const float ss = wave_sum(v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3]);
  int orow = m;
  if (p.final_mode) {
    const int b = m / p.B, j = m % p.B;
    if (j == 0) return;
    orow = b * (p.B - 1) + j - 1;
  }
  if (i4 < n4) {
    const f32x4_t g = bf4_to_f32(gw);
    *reinterpret_cast<u32x2*>(p.out + (long long)orow * p.n + 4 * i4) =
        u32x2{pack_bf2(v[0] * g[0], v[1] * g[1]), pack_bf2(v[2] * g[2], v[3] * g[3])};
  }
  if (threadIdx.x == 0) p.ssp[(long long)orow * kMaxRowChunks + c] = ss;
}

// ---------------------------------------------------------------------------
// KV injection epilogue: for commit row i and layer l, k = RoPE(RMSNorm_head(
// W_k c)), v = W_v c, scattered to (seq, pos); ctx_len[seq] grows to pos + 1.
// One wave per (block of kInjectRows commit rows, layer, head), D/8 lanes per
// row: lane q of a row holds dimensions 4q..4q+3 and their RoPE partners
// 4q+D/2..4q+D/2+3, so the fp32 partials and the (cos, sin) row arrive in
// 16-byte loads and K/V leave in 8-byte stores; a wave covers 512/D rows per
// round, and the commit rows, partials and RoPE rows of every round are
// loaded before any arithmetic (one float per lane and a wave per head of 8
// rows ran the 4096-row ingest chunk's pass at 1.8 TB/s).
constexpr int kInjectRows = 16;

// x1/x2 += splits 1.. of the lane's two 4-dimension groups for every round
// (split 0 is already in x1/x2); SB splits per batch of loads, all issued
// before the adds (clamped split index: unconditional loads)
template <int NR, int SB>
__device__ __forceinline__ void inject_add_splits(f32x4_t (&x1)[NR], f32x4_t (&x2)[NR],
                                                  const float* const (&src)[NR], long long s_stride, int splits,
                                                  int half) {
  for (int s0 = 1; s0 < splits; s0 += SB) {
    f32x4_t a[SB][NR], b[SB][NR];
#pragma unroll
    for (int j = 0; j < SB; ++j)
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const float* q = src[r] + (long long)min(s0 + j, splits - 1) * s_stride;
        a[j][r] = *reinterpret_cast<const f32x4_t*>(q);
        b[j][r] = *reinterpret_cast<const f32x4_t*>(q + half);
      }
#pragma unroll
    for (int j = 0; j < SB; ++j)
      if (s0 + j < splits)
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          x1[r] += a[j][r];
          x2[r] += b[j][r];
        }
  }
}

template <int D>
__global__ __launch_bounds__(256) void inject_post_kernel(const InjectPostParams p) {
  constexpr int half = D / 2;
  constexpr int LPR = D / 8;               // lanes per row
  constexpr int RPR = 64 / LPR;            // rows per round
  constexpr int NR = kInjectRows / RPR;    // rounds
  static_assert(NR * RPR == kInjectRows, "rows per wave");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane % LPR, rs = lane / LPR;
  const int d0 = 4 * q;
  const int i0 = p.c0 + blockIdx.x * kInjectRows, l = blockIdx.y;
  const int head = blockIdx.z * 4 + wave;
  if (head >= 2 * p.Hkv) return;
  const int width = 2 * p.Hkv * D;
  int nc = *p.n_commit;
  nc = nc < 0 ? 0 : (nc > p.max_commit ? p.max_commit : nc);
  const int iend = min(nc, p.c1);
  const bool is_k = head < p.Hkv;
  // split 0 of the partials first (the bytes that matter), then the commit
  // rows, then the RoPE rows of K heads (they need the positions)
  const float* psrc[NR];
  f32x4_t x1[NR], x2[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {  // clamped rows: every load in bounds, results unused
    const int i = min(i0 + r * RPR + rs, p.c1 - 1);
    psrc[r] = p.P + (long long)l * p.p_z_stride + (long long)(i - p.c0) * width + head * D + d0;
    x1[r] = *reinterpret_cast<const f32x4_t*>(psrc[r]);
    x2[r] = *reinterpret_cast<const f32x4_t*>(psrc[r] + half);
  }
  int src[NR], seq[NR], pos[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int i = min(i0 + r * RPR + rs, p.c1 - 1);
    src[r] = p.commit_rows[3 * i];
    seq[r] = p.commit_rows[3 * i + 1];
    pos[r] = p.commit_rows[3 * i + 2];
  }
  // (cos, sin) of dimensions d0..d0+3 at the row's position: two 16-byte loads
  f32x4_t cs0[NR], cs1[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) cs0[r] = cs1[r] = f32x4_t{1.f, 0.f, 1.f, 0.f};
  if (is_k) {  // uniform over the wave
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int rpos = pos[r] < 0 ? 0 : (pos[r] >= p.rope_max ? p.rope_max - 1 : pos[r]);
      const f32x4_t* rp = reinterpret_cast<const f32x4_t*>(p.rope + ((long long)rpos * half + d0) * 2);
      cs0[r] = rp[0];
      cs1[r] = rp[1];
    }
  }
  // batches of at most two further splits hold the head size 128 kernel to
  // three waves per SIMD (four-split batches took 186 registers)
  if (p.splits > 1) inject_add_splits<NR, 2>(x1, x2, psrc, p.p_s_stride, p.splits, half);
  const u32x2 gw1 = *reinterpret_cast<const u32x2*>(p.gk[l] + d0);
  const u32x2 gw2 = *reinterpret_cast<const u32x2*>(p.gk[l] + d0 + half);
  const f32x4_t g1 = bf4_to_f32(gw1), g2 = bf4_to_f32(gw2);
  // one lane per row records the context length and capacity errors
  const bool first = l == 0 && blockIdx.z == 0 && wave == 0 && q == 0;
  const int g = head < p.Hkv ? head : head - p.Hkv;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    // the head's sum of squares over the row's LPR lanes (every lane takes
    // part in the shuffles, valid row or not)
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) ss += x1[r][e] * x1[r][e] + x2[r][e] * x2[r][e];
#pragma unroll
    for (int o = 1; o < LPR; o <<= 1) ss += __shfl_xor(ss, o);
    const int i = i0 + r * RPR + rs;
    if (i >= iend) continue;
    if (src[r] < 0 || src[r] >= p.n_ctx_rows || seq[r] < 0 || seq[r] >= p.batch) continue;
    if (pos[r] < 0 || pos[r] >= p.max_ctx || pos[r] >= p.rope_max) {
      if (first) p.status[seq[r]] = kErrCapacity;
      continue;
    }
    const long long off = ((((long long)l * p.batch + seq[r]) * p.Hkv + g) * p.max_ctx + pos[r]) * D + d0;
    u32x2 lo, hi;
    if (!is_k) {
      lo = u32x2{pack_bf2(x1[r][0], x1[r][1]), pack_bf2(x1[r][2], x1[r][3])};
      hi = u32x2{pack_bf2(x2[r][0], x2[r][1]), pack_bf2(x2[r][2], x2[r][3])};
      *reinterpret_cast<u32x2*>(p.vc + off) = lo;
      *reinterpret_cast<u32x2*>(p.vc + off + half) = hi;
    } else {
      const float inv = 1.0f / sqrtf(ss / (float)D + p.eps);
      const float c[4] = {cs0[r][0], cs0[r][2], cs1[r][0], cs1[r][2]};
      const float sn[4] = {cs0[r][1], cs0[r][3], cs1[r][1], cs1[r][3]};
      float k1[4], k2[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float y1 = x1[r][e] * inv * g1[e];
        const float y2 = x2[r][e] * inv * g2[e];
        k1[e] = y1 * c[e] - y2 * sn[e];
        k2[e] = y1 * sn[e] + y2 * c[e];
      }
      lo = u32x2{pack_bf2(k1[0], k1[1]), pack_bf2(k1[2], k1[3])};
      hi = u32x2{pack_bf2(k2[0], k2[1]), pack_bf2(k2[2], k2[3])};
      *reinterpret_cast<u32x2*>(p.kc + off) = lo;
      *reinterpret_cast<u32x2*>(p.kc + off + half) = hi;
    }
    if (first) atomicMax(p.ctx_len + seq[r], pos[r] + 1);
  }
}

// ---------------------------------------------------------------------------
// q/k/v of block rows: sum split partials per head; q and k get a per-head
// RMSNorm and rotate-half RoPE at position L_b + j; q goes to the query buffer
// (times q_scale), k and v to cache slot L_b + j (speculative append).
// Nothing is stored for a sequence with a nonzero status (the embedding pass
// has set it, capacity included). One wave per (block of 512/D rows, head),
// D/8 lanes per row as in inject_post_kernel (lane q: dimensions 4q..4q+3 and
// their RoPE partners 4q+D/2..): 16-byte loads of the partials and RoPE
// rows, 8-byte stores, every load of the wave issued before the arithmetic
// (one wave per (row, head) with a float per lane took 11-15 us per launch at
// 512 rows); one round of rows per wave keeps a 16-row block spread over
// many CUs. One more row of workgroups writes the attention chunk split.
template <int D>
constexpr int qkv_rows() { return 512 / D; }

template <int D>
__global__ __launch_bounds__(256) void qkv_post_kernel(const QkvPostParams p) {
  constexpr int half = D / 2;
  constexpr int LPR = D / 8;              // lanes per row
  constexpr int RPR = 64 / LPR;           // rows per round
  constexpr int kQkvRows = qkv_rows<D>();
  constexpr int NR = kQkvRows / RPR;      // rounds (one)
  static_assert(NR * RPR == kQkvRows, "rows per wave");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rows = p.batch * p.B;
  // the extra row of workgroups: the first one's first wave writes the
  // attention chunk split (the embedding pass has set every status)
  if ((int)blockIdx.y == (rows + kQkvRows - 1) / kQkvRows) {
    if (blockIdx.x == 0 && wave == 0)
      attn_plan_wave(p.ctx_len, p.status, p.batch, p.B, p.n_ranges, p.slice, p.plan);
    return;
  }
  const int head = blockIdx.x * 4 + wave;
  const int nh = p.Hq + 2 * p.Hkv;
  if (head >= nh) return;
  const int qd = lane % LPR, rs = lane / LPR;
  const int d0 = 4 * qd;
  const int width = nh * D;
  const int m0 = blockIdx.y * kQkvRows;
  const bool is_v = head >= p.Hq + p.Hkv;
  // split 0 of the partials first, then the rows' sequence state, then the
  // RoPE rows of q and k heads (they need the positions); clamped rows: every
  // load in bounds, results unused
  const float* psrc[NR];
  f32x4_t x1[NR], x2[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int m = min(m0 + r * RPR + rs, rows - 1);
    psrc[r] = p.P + (long long)m * width + head * D + d0;
    x1[r] = *reinterpret_cast<const f32x4_t*>(psrc[r]);
    x2[r] = *reinterpret_cast<const f32x4_t*>(psrc[r] + half);
  }
  // row scale of the split RMSNorm: the row's LPR lanes hold its chunk sums
  // (kMaxRowChunks / LPR each; from P when there is none: valid memory,
  // values dropped)
  constexpr int kRsLane = kMaxRowChunks / LPR;
  static_assert(kRsLane == 2 || kRsLane == 4, "chunk sums per lane");
  typedef float rsv_t __attribute__((ext_vector_type(kRsLane)));
  const bool has_rs = p.rs != nullptr;
  rsv_t rsv[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int m = min(m0 + r * RPR + rs, rows - 1);
    rsv[r] = *reinterpret_cast<const rsv_t*>(has_rs ? p.rs + (long long)m * kMaxRowChunks + kRsLane * qd : p.P);
  }
  int st[NR], pos[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int m = min(m0 + r * RPR + rs, rows - 1);
    const int b = m / p.B;
    st[r] = p.status[b];
    pos[r] = p.ctx_len[b] + m % p.B;
  }
  f32x4_t cs0[NR], cs1[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) cs0[r] = cs1[r] = f32x4_t{1.f, 0.f, 1.f, 0.f};
  if (!is_v) {  // uniform over the wave
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int rpos = pos[r] < 0 ? 0 : (pos[r] >= p.rope_max ? p.rope_max - 1 : pos[r]);
      const f32x4_t* rp = reinterpret_cast<const f32x4_t*>(p.rope + ((long long)rpos * half + d0) * 2);
      cs0[r] = rp[0];
      cs1[r] = rp[1];
    }
  }
  if (p.splits > 1) inject_add_splits<NR, 2>(x1, x2, psrc, p.p_s_stride, p.splits, half);
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    float a = 0.f;
#pragma unroll
    for (int e = 0; e < kRsLane; ++e)
      if (kRsLane * qd + e < p.rs_n) a += rsv[r][e];
#pragma unroll
    for (int o = 1; o < LPR; o <<= 1) a += __shfl_xor(a, o);
    const float sc = has_rs ? 1.0f / sqrtf(a / (float)p.rs_len + p.rs_eps) : 1.f;
    x1[r] *= sc;
    x2[r] *= sc;
  }
  const uint16_t* gain = head < p.Hq ? p.gq : p.gk;
  const f32x4_t g1 = bf4_to_f32(*reinterpret_cast<const u32x2*>(gain + d0));
  const f32x4_t g2 = bf4_to_f32(*reinterpret_cast<const u32x2*>(gain + d0 + half));
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    // the head's sum of squares over the row's LPR lanes (every lane takes
    // part in the shuffles, stored row or not)
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) ss += x1[r][e] * x1[r][e] + x2[r][e] * x2[r][e];
#pragma unroll
    for (int o = 1; o < LPR; o <<= 1) ss += __shfl_xor(ss, o);
    const int m = m0 + r * RPR + rs;
    if (m >= rows || st[r] != 0) continue;
    const int b = m / p.B;
    if (is_v) {
      const int g = head - p.Hq - p.Hkv;
      uint16_t* dst = p.vc + (((long long)b * p.Hkv + g) * p.max_ctx + pos[r]) * D + d0;
      *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf2(x1[r][0], x1[r][1]), pack_bf2(x1[r][2], x1[r][3])};
      *reinterpret_cast<u32x2*>(dst + half) = u32x2{pack_bf2(x2[r][0], x2[r][1]), pack_bf2(x2[r][2], x2[r][3])};
      continue;
    }
    const float inv = 1.0f / sqrtf(ss / (float)D + p.eps);
    // queries carry the softmax scale (one rounding to bf16)
    const float sc = head < p.Hq ? p.q_scale : 1.f;
    const float c[4] = {cs0[r][0], cs0[r][2], cs1[r][0], cs1[r][2]};
    const float sn[4] = {cs0[r][1], cs0[r][3], cs1[r][1], cs1[r][3]};
    float o1[4], o2[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float y1 = x1[r][e] * inv * g1[e];
      const float y2 = x2[r][e] * inv * g2[e];
      o1[e] = (y1 * c[e] - y2 * sn[e]) * sc;
      o2[e] = (y1 * sn[e] + y2 * c[e]) * sc;
    }
    uint16_t* dst = head < p.Hq ? p.q + ((long long)m * p.Hq + head) * D + d0
                                : p.kc + (((long long)b * p.Hkv + (head - p.Hq)) * p.max_ctx + pos[r]) * D + d0;
    *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf2(o1[0], o1[1]), pack_bf2(o1[2], o1[3])};
    *reinterpret_cast<u32x2*>(dst + half) = u32x2{pack_bf2(o2[0], o2[1]), pack_bf2(o2[2], o2[3])};
  }
}

// ---------------------------------------------------------------------------
// draft token of one LM row: the maximum key over the LM-head tiles (largest
// logit, lowest index on ties), unpacked to the index. keys[tile][row] (each
// GEMM workgroup writes its rows contiguously); 1024 threads with
// kFinishBatch loads in flight each cover 8192 tiles per round trip.
constexpr int kFinishThreads = 1024;
constexpr int kFinishBatch = 8;

__global__ __launch_bounds__(kFinishThreads) void argmax_finish_kernel(const unsigned long long* keys,
                                                                       int n_tiles, const int32_t* status,
                                                                       int batch, int rows_per_seq, int32_t* out) {
  __shared__ unsigned long long red[kFinishThreads / 64];
  const int row = blockIdx.x;
  const int rows = batch * rows_per_seq;
  unsigned long long best = 0ull;
  for (int t0 = threadIdx.x; t0 < n_tiles; t0 += kFinishThreads * kFinishBatch) {
    unsigned long long k[kFinishBatch];
#pragma unroll
    for (int u = 0; u < kFinishBatch; ++u) {
      const int t = t0 + u * kFinishThreads;
      k[u] = keys[(long long)min(t, n_tiles - 1) * rows + row];
    }
#pragma unroll
    for (int u = 0; u < kFinishBatch; ++u) best = max(best, k[u]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long other = __shfl_xor(best, o);
    best = max(best, other);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int w = 1; w < kFinishThreads / 64; ++w) best = max(best, red[w]);
    best = max(best, red[0]);
    const int b = row / rows_per_seq;
    out[row] = status[b] != 0 ? -1 : (int32_t)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFull));
  }
}

// ---------------------------------------------------------------------------
// commit without K/V writes (the rows' K/V are already in the cache): ctx_len
// of each committed row's sequence grows to pos + 1.
__global__ __launch_bounds__(256) void kv_commit_kernel(const int32_t* commit_rows, const int32_t* n_commit,
                                                        int max_commit, int batch, int max_ctx, int32_t* ctx_len) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= max_commit) return;
  int nc = *n_commit;
  nc = nc < 0 ? 0 : (nc > max_commit ? max_commit : nc);
  if (i >= nc) return;
  const int seq = commit_rows[3 * i + 1], pos = commit_rows[3 * i + 2];
  if (seq < 0 || seq >= batch || pos < 0 || pos >= max_ctx) return;
  atomicMax(ctx_len + seq, pos + 1);
}

// ---------------------------------------------------------------------------
// split SwiGLU: each thread sums the splits of four gate and four up columns
// of one row (loads of a batch of splits issued together, clamped), then
// writes bf16 silu(g) * u.
__global__ __launch_bounds__(256) void swiglu_combine_kernel(const SwigluCombineParams p) {
  const int m = blockIdx.y;
  const int n4 = p.n / 4;
  const int c4 = blockIdx.x * 256 + threadIdx.x;
  const int cc = min(c4, n4 - 1);
  const float* base = p.P + (long long)m * 2 * p.n + 4 * cc;
  f32x4_t gs = {0.f, 0.f, 0.f, 0.f}, us = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < p.splits; s0 += kSplitBatch) {
    f32x4_t tg[kSplitBatch], tu[kSplitBatch];
#pragma unroll
    for (int j = 0; j < kSplitBatch; ++j) {
      const float* src = base + (long long)min(s0 + j, p.splits - 1) * p.p_s_stride;
      tg[j] = *reinterpret_cast<const f32x4_t*>(src);
      tu[j] = *reinterpret_cast<const f32x4_t*>(src + p.n);
    }
#pragma unroll
    for (int j = 0; j < kSplitBatch; ++j)
      if (s0 + j < p.splits) {
        gs += tg[j];
        us += tu[j];
      }
  }
  if (c4 >= n4) return;
  float sv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) sv[i] = gs[i] / (1.0f + __expf(-gs[i])) * us[i];
  *reinterpret_cast<u32x2*>(p.out + (long long)m * p.ld_out + 4 * c4) =
      u32x2{pack_bf2(sv[0], sv[1]), pack_bf2(sv[2], sv[3])};
}

}  // namespace

hipError_t launch_swiglu_combine(const SwigluCombineParams& p, hipStream_t st) {
  if (p.n % 4 || p.splits < 1 || p.rows < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(swiglu_combine_kernel, dim3((p.n / 4 + 255) / 256, p.rows), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_embed(const EmbedParams& p, hipStream_t st) {
  if (p.ssp) {
    if (p.H % 4 != 0 || p.ss_chunks != (p.H + kRowChunkCols - 1) / kRowChunkCols || p.ss_chunks > kMaxRowChunks ||
        p.batch * p.B < 1)
      return hipErrorInvalidValue;
    hipLaunchKernelGGL(embed_split_kernel, dim3(p.ss_chunks, p.batch * p.B), dim3(64), 0, st, p);
    return hipGetLastError();
  }
  if (p.H > kRowThreads * 4 * kMaxC4 || p.H % 4) return hipErrorInvalidValue;
  const int c4 = (p.H / 4 + kRowThreads - 1) / kRowThreads;  // float4 columns per thread
  if (c4 <= 1)
    hipLaunchKernelGGL(embed_kernel<1>, dim3(p.batch * p.B), dim3(kRowThreads), 0, st, p);
  else if (c4 <= 2)
    hipLaunchKernelGGL(embed_kernel<2>, dim3(p.batch * p.B), dim3(kRowThreads), 0, st, p);
  else
    hipLaunchKernelGGL(embed_kernel<kMaxC4>, dim3(p.batch * p.B), dim3(kRowThreads), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_row_norm(const RowNormParams& p, hipStream_t st) {
  if (p.ssp) {
    if (p.n % 4 != 0 || p.ss_chunks != (p.n + kRowChunkCols - 1) / kRowChunkCols || p.ss_chunks > kMaxRowChunks ||
        !p.P || p.splits < 1 || p.rows < 1)
      return hipErrorInvalidValue;
    hipLaunchKernelGGL(row_split_kernel, dim3(p.ss_chunks, p.rows), dim3(64), 0, st, p);
    return hipGetLastError();
  }
  if (p.n > kRowThreads * 4 * kMaxC4 || p.n % 4 || !p.P || p.splits < 1) return hipErrorInvalidValue;
  const int c4 = (p.n / 4 + kRowThreads - 1) / kRowThreads;  // float4 columns per thread
  if (c4 <= 1)
    hipLaunchKernelGGL(row_norm_kernel<1>, dim3(p.rows), dim3(kRowThreads), 0, st, p);
  else if (c4 <= 2)
    hipLaunchKernelGGL(row_norm_kernel<2>, dim3(p.rows), dim3(kRowThreads), 0, st, p);
  else
    hipLaunchKernelGGL(row_norm_kernel<kMaxC4>, dim3(p.rows), dim3(kRowThreads), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_qkv_post(const QkvPostParams& p, hipStream_t st) {
  const int nh = p.Hq + 2 * p.Hkv;
  if (p.plan && (p.n_ranges < p.batch || p.slice < 1)) return hipErrorInvalidValue;
  const int rows = p.batch * p.B;
  if (p.D == 128)
    hipLaunchKernelGGL(qkv_post_kernel<128>, dim3((nh + 3) / 4, (rows + qkv_rows<128>() - 1) / qkv_rows<128>() + (p.plan ? 1 : 0)),
                       dim3(256), 0, st, p);
  else if (p.D == 64)
    hipLaunchKernelGGL(qkv_post_kernel<64>, dim3((nh + 3) / 4, (rows + qkv_rows<64>() - 1) / qkv_rows<64>() + (p.plan ? 1 : 0)),
                       dim3(256), 0, st, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_inject_post(const InjectPostParams& p, hipStream_t st) {
  if (p.c1 <= p.c0) return hipSuccess;
  const dim3 grid((p.c1 - p.c0 + kInjectRows - 1) / kInjectRows, p.n_layers, (2 * p.Hkv + 3) / 4);
  if (p.D == 128)
    hipLaunchKernelGGL(inject_post_kernel<128>, grid, dim3(256), 0, st, p);
  else if (p.D == 64)
    hipLaunchKernelGGL(inject_post_kernel<64>, grid, dim3(256), 0, st, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_argmax_finish(const unsigned long long* keys, int n_tiles, const int32_t* status,
                                int batch, int rows_per_seq, int32_t* out, hipStream_t st) {
  if (rows_per_seq < 1 || batch < 1 || n_tiles < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(argmax_finish_kernel, dim3(batch * rows_per_seq), dim3(kFinishThreads), 0, st, keys, n_tiles,
                     status, batch, rows_per_seq, out);
  return hipGetLastError();
}

hipError_t launch_kv_commit(const int32_t* commit_rows, const int32_t* n_commit, int max_commit, int batch,
                            int max_ctx, int32_t* ctx_len, hipStream_t st) {
  if (max_commit <= 0) return hipSuccess;
  hipLaunchKernelGGL(kv_commit_kernel, dim3((max_commit + 255) / 256), dim3(256), 0, st, commit_rows, n_commit,
                     max_commit, batch, max_ctx, ctx_len);
  return hipGetLastError();
}

}  // namespace dfl

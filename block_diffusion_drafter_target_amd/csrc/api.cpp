// C ABI of the draft-step library: argument checks, launch plans and the
// sequence of gfx950 kernels for each call. Every check that needs no GPU runs
// before the first HIP call, so failures are reported without a device.
#include <dflash.h>

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>
#include <vector>

#include "attn_split.h"
#include "internal.h"

struct dflash_model {
  dflash_config cfg;
  dflash_weights w;
  std::vector<dflash_layer_weights> layers;
  bool target = false;    // a target model (dflash_target_create): causal passes, taps
  std::vector<int> taps;  // target: tapped layers, increasing
};

namespace {

using dfl::GemmParams;

// ---------------------------------------------------------------------------
// optional per-phase event timing (benchmarks)
namespace prof {
struct Rec {
  int phase;
  hipEvent_t a, b;
};
uint32_t mask = 0;
std::vector<Rec> recs;  // events are created once and reused
size_t used = 0;
bool paused = false;                  // dflash_profile_pause: skip launches, keep the records
thread_local bool suspended = false;  // set while a call that must not allocate runs

struct Scope {
  Rec* r = nullptr;
  hipStream_t st;
  Scope(int phase, hipStream_t s) : st(s) {
    if (suspended || paused || !(mask >> phase & 1u)) return;
    if (used == recs.size()) {
      Rec n{phase, nullptr, nullptr};
      if (hipEventCreate(&n.a) != hipSuccess || hipEventCreate(&n.b) != hipSuccess) return;
      recs.push_back(n);
    }
    r = &recs[used++];
    r->phase = phase;
    if (hipEventRecord(r->a, st) != hipSuccess) r = nullptr;
  }
  ~Scope() {
    if (r) (void)hipEventRecord(r->b, st);
  }
};
}  // namespace prof

constexpr int kMaxBatch = 4096;
constexpr int kMaxTargetLayers = 256;
constexpr int kRowChunk = 4096;  // rows per fuse / inject GEMM pass
constexpr int kGemmRows = 64;    // rows per weight-streaming GEMM launch (at most)
constexpr int kTargetWGs = 768;  // workgroups a split-K GEMM launch aims for

inline long long cdiv(long long a, long long b) { return (a + b - 1) / b; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct GemmPlan {
  bool big;    // large-tile kernel (bm x 256 tiles) over all rows
  int bm = 256;  // large-tile kernel: activation rows per tile (256 or 128)
  int bn = 256;  // large-tile kernel: weight rows per tile (256, or 192 for the SwiGLU)
  bool tiled;  // LDS-tiled kernel over all rows, or the streaming kernel per kGemmRows rows
  int mt, nf;  // streaming: activation tiles and weight fragments per workgroup
  int ng;      // tiled: weight row groups per wave (64*ng columns per workgroup); mt: 16-row tiles
  int splits, k_per_split;
  bool swiglu_split;  // SwiGLU as split-K partials over [gate; up] plus a combine pass
  bool ws = false;    // tiled: the deep-prefetch kernel (gemm_ws.hip) instead of gemm_tile.hip
};

constexpr int kStreamMaxRows = 32;   // more rows take the tiled kernel
constexpr int kBigMinRows = 256;     // this many rows take the large-tile kernel
constexpr int kBigSlots = 256;       // large-tile workgroups resident at once (one per CU)
constexpr int kSwigluMinWGs = 256;   // fewer single-pass SwiGLU workgroups: split-K path
constexpr int kWsSlots = 256;        // deep-prefetch tiled workgroups per round (one per CU at 128 rows)
constexpr int kWsSwigluMinWGs = 128; // single-pass SwiGLU workgroups from which that kernel takes it
constexpr int kWsMinK = 8192;        // partial-mode K from which that kernel takes it

// Kernel, tile shape and split-K for Y = A W^T (every choice measured on
// MI355X against the alternatives).
// From kBigMinRows rows: the large-tile kernel (both operands staged through
// LDS; the product is bound by the matrix cores), 256 x 256 tiles, 128 x 256
// where those halve the split-K partials, 256 x 192 for a SwiGLU grid short
// of one round (see the branch below).
// Up to kStreamMaxRows rows (or K < 128): the weight-streaming kernel with
// NF = 2 weight fragments per workgroup (more waves in flight beat wider
// tiles with cold caches); split-K only in partial mode, to bring the grid to
// about kTargetWGs workgroups (1024 when there are at most 128 column tiles:
// longer splits per workgroup measured slower there).
// In between: partial-mode products of one 65..128-row tile with K below
// kWsMinK take the large-tile kernel's 128 x 128 tiles; the rest the tiled
// kernels (activations shared through LDS) with 64 or 128 activation rows
// per tile, the deep-prefetch one for the single-pass SwiGLU of at least
// kWsSwigluMinWGs workgroups and for partial products with K >= kWsMinK.
// Split-K partials cost 2*splits*M/K bytes per weight byte: with one row
// tile (HBM-bound) splits aim for 256 workgroups at 128 rows and 384 at 64
// rows (64-row tiles also use 64-column tiles), with several row tiles
// (MFMA-bound) for 512, two per CU. A SwiGLU whose single-pass grid would be
// smaller runs as a partial-mode GEMM over the concatenated gate and up rows
// and a combine pass.
GemmPlan plan_gemm(int M, int N, int K, int nz, int mode) {
  GemmPlan g;
  g.swiglu_split = false;
  g.big = false;
  if (M >= kBigMinRows && K >= 32) {
    // Large tiles (one 512-thread workgroup per CU). Split-K only in partial
    // mode and only while the grid still fits one round of kBigSlots
    // workgroups: a second, partly filled round costs more than the split
    // saves (512 rows: 6 splits of the QKV product, 288 workgroups, measured
    // 47% slower than 4). Where 256-row tiles need split-K, 128-row tiles
    // halve the splits and with them the fp32 partials that the GEMM writes
    // and the next pass reads; they are taken unless they cost more than a
    // quarter of the grid (512 rows of the Qwen3-8B-shaped drafter: o and
    // down 8 -> 4 splits at 256 workgroups, QKV 5 -> 2 at 240 -> 192; the
    // inject product over five layers keeps 256-row tiles, 240 workgroups
    // against 160; the step 2701 -> 2610 us, measured on MI355X).
    g.big = true;
    g.tiled = false;
    g.mt = g.nf = g.ng = 0;
    // A SwiGLU grid of 256 x 256 tiles short of one round of kBigSlots takes
    // 256 x 192 tiles where those fit one round (512 rows of the Qwen3-8B-
    // shaped drafter: 192 -> 256 workgroups)
    if (mode == dfl::kGemmSwiglu) {
      const long long m256 = cdiv(M, 256) * nz;
      if (m256 * cdiv(N, dfl::gemm_big_cols(mode, 256)) < kBigSlots &&
          m256 * cdiv(N, dfl::gemm_big_cols(mode, 192)) <= kBigSlots)
        g.bn = 192;
    }
    const long long cols = cdiv(N, dfl::gemm_big_cols(mode, g.bn)) * nz;
    const int chunks = K / 32;
    auto split = [&](int bm, int* per) {
      const long long base = cdiv(M, bm) * cols;
      int s = 1;
      if (mode == dfl::kGemmPartial && base < kBigSlots) {
        s = (int)(kBigSlots / base);
        s = std::min(s, std::max(1, chunks / 8));  // at least 256 k per split
      }
      *per = (int)cdiv(chunks, s);
      return (int)cdiv(chunks, *per);
    };
    int per = 0;
    g.splits = split(256, &per);
    if (g.splits > 1) {
      int per128 = 0;
      const int s128 = split(128, &per128);
      if (4 * cdiv(M, 128) * s128 >= 3 * cdiv(M, 256) * g.splits) {
        g.bm = 128;
        g.splits = s128;
        per = per128;
      }
    }
    // 128-row partial tiles whose 256-column grid leaves CUs idle take 192
    // columns where that fills more of the round (512 rows of the Qwen3-8B-
    // shaped drafter, QKV: 192 -> 256 workgroups at the same 2 splits)
    if (mode == dfl::kGemmPartial && g.bm == 128) {
      const long long grid256 = cdiv(M, 128) * cols * g.splits;
      const long long base = cdiv(M, 128) * cdiv(N, 192) * nz;
      if (grid256 < kBigSlots && base < kBigSlots) {
        int s = (int)(kBigSlots / base);
        s = std::min(s, std::max(1, chunks / 8));  // at least 256 k per split
        const int per192 = (int)cdiv(chunks, s);
        const int s192 = (int)cdiv(chunks, per192);
        if (base * s192 > grid256) {
          g.bn = 192;
          g.splits = s192;
          per = per192;
        }
      }
    }
    g.k_per_split = per * 32;
    return g;
  }
  if (mode == dfl::kGemmPartial && M > 64 && M <= 128 && K >= 256 && K < kWsMinK && K % 32 == 0) {
    // One row tile of 65..128 rows, split-K partials over K < kWsMinK: the
    // large-tile kernel's 128 x 128 tiles, splits for one round of kBigSlots
    // workgroups (batch 8 x block 16: QKV 25.9 -> 22.9 us, o 18.7 -> 17.8,
    // inject over five layers 36.3 -> 28.6 against the register-path tiled
    // kernel, measured on MI355X; the fuse and down products, K >= 8192, are
    // faster on the deep-prefetch tiled kernel)
    g.big = true;
    g.tiled = false;
    g.mt = g.nf = g.ng = 0;
    g.bm = 128;
    g.bn = 128;
    const long long base = cdiv(N, 128) * nz;
    const int chunks = K / 32;
    int s = (int)std::max<long long>(1, kBigSlots / base);
    s = std::min(s, std::max(1, chunks / 8));  // at least 256 k per split
    const int per = (int)cdiv(chunks, s);
    g.splits = (int)cdiv(chunks, per);
    g.k_per_split = per * 32;
    return g;
  }
  if (M > kStreamMaxRows && K >= 128) {
    g.tiled = true;
    g.nf = 0;
    g.mt = M <= 64 ? 4 : 8;
    const long long m_tiles = cdiv(M, 16 * g.mt);
    const int slabs = (int)cdiv(K, 128);
    // the deep-prefetch tiled kernel (gemm_ws.hip) for the single-pass SwiGLU
    // with at least kWsSwigluMinWGs workgroups and for partial-mode products
    // over long K: there it beats the other tiled kernel (Qwen3-8B-shaped
    // drafter, batch 8 x block 16: gate/up 67 -> 62 us, down 36 -> 34, fuse
    // 51 -> 46 per launch); elsewhere (qkv, o, the LM head, the gpt-oss-shaped
    // 64-row GEMMs) it measured equal or slower
    g.ws = (mode == dfl::kGemmSwiglu && cdiv(N, 64) * m_tiles * nz >= kWsSwigluMinWGs) ||
           (mode == dfl::kGemmPartial && K >= kWsMinK);
    if (g.ws) {
      g.ng = 2;
      const long long n_tiles = mode == dfl::kGemmSwiglu ? cdiv(N, 64) : cdiv(N, 128);
      const long long base = n_tiles * m_tiles * nz;
      int s = 1;
      if (mode == dfl::kGemmPartial) {  // at most one round of kWsSlots workgroups
        s = (int)std::max<long long>(1, kWsSlots / base);
        s = std::min(s, std::max(1, slabs / 2));  // at least two 128-k slabs per split
      }
      const int per = (int)cdiv(slabs, s);
      g.splits = (int)cdiv(slabs, per);
      g.k_per_split = per * 128;
      return g;
    }
    if (mode == dfl::kGemmSwiglu && cdiv(N, 64) * m_tiles * nz < kSwigluMinWGs) {
      GemmPlan p = plan_gemm(M, 2 * N, K, nz, dfl::kGemmPartial);
      p.swiglu_split = true;
      return p;
    }
    g.ng = (mode == dfl::kGemmPartial && g.mt == 4) ? 1 : 2;
    const long long n_tiles = mode == dfl::kGemmSwiglu ? cdiv(N, 64) : cdiv(N, 64 * g.ng);
    const long long base = n_tiles * m_tiles * nz;
    int s = 1;
    if (mode == dfl::kGemmPartial) {
      const int target = m_tiles > 1 ? 512 : (g.mt == 4 ? 384 : 256);  // see above
      s = (int)std::max<long long>(1, cdiv(target, base));
      s = std::min(s, std::max(1, slabs / 2));  // at least two 128-k slabs per split
    }
    const int per = (int)cdiv(slabs, s);
    g.splits = (int)cdiv(slabs, per);
    g.k_per_split = per * 128;
    return g;
  }
  g.tiled = false;
  g.ng = 0;
  const int rows = std::min(M, kGemmRows);
  g.mt = rows <= 16 ? 1 : (rows <= 32 ? 2 : 4);
  g.nf = 2;
  // Up to 16 rows the single-pass SwiGLU takes four weight groups per
  // workgroup (32 output columns) where that grid still fills kSwigluMinWGs:
  // each wave then reads a quarter as many activation bytes per weight byte
  // instead of half (Qwen3-8B-shaped drafter at batch 1: gate/up 41.5 -> 39.1
  // us per layer, step 827 -> 816 us, measured on MI355X). Partial and argmax
  // products keep two: with four, their capped split counts halve the grid
  // (step +34 and +26 us).
  if (mode == dfl::kGemmSwiglu && g.mt == 1 && cdiv(N, 32) * nz >= kSwigluMinWGs) g.nf = 4;
  if (mode == dfl::kGemmSwiglu && cdiv(N, 16) * nz < kSwigluMinWGs) {
    GemmPlan p = plan_gemm(M, 2 * N, K, nz, dfl::kGemmPartial);
    p.swiglu_split = true;
    return p;
  }
  const int out_frags = mode == dfl::kGemmSwiglu ? g.nf / 2 : g.nf;
  const long long tiles = cdiv(N, 16 * out_frags) * nz;
  const int kblocks = (int)cdiv(K, 128);
  int s = 1;
  if (mode == dfl::kGemmPartial) {
    s = (int)std::max<long long>(1, cdiv(tiles <= 128 ? 1024 : kTargetWGs, tiles));
    s = std::min(s, std::max(1, kblocks / 4));  // at least one 128-k block per wave
  }
  const int per = (int)cdiv(kblocks, s);
  g.splits = (int)cdiv(kblocks, per);
  g.k_per_split = per * 128;
  return g;
}

// Workgroup column tiles of the LM-head GEMM for M rows (one argmax key per
// tile and row).
int lm_tiles(const dflash_config& c, int M) {
  const GemmPlan g = plan_gemm(M, c.vocab, c.hidden, 1, dfl::kGemmArgmax);
  if (g.big) return (int)cdiv(c.vocab, dfl::gemm_big_cols(dfl::kGemmArgmax, g.bn));
  return (int)(g.tiled ? cdiv(c.vocab, 64 * g.ng) : cdiv(c.vocab, 16 * g.nf));
}

// Partial buffer (floats) that run_gemm needs for M rows in the given mode
// (a split SwiGLU keeps partials of its 2N gate and up columns).
size_t gemm_partial_floats(int M, int N, int K, int nz, int mode = dfl::kGemmPartial) {
  const GemmPlan g = plan_gemm(M, N, K, nz, mode);
  if (mode == dfl::kGemmSwiglu) return g.swiglu_split ? (size_t)nz * g.splits * M * 2 * N : 0;
  return (size_t)nz * g.splits * M * N;
}

struct GemmCall {
  const uint16_t* A = nullptr;
  long long lda = 0;
  const int32_t* a_idx = nullptr;
  int a_idx_stride = 0, a_idx_max = 0;
  const uint16_t* W0[dfl::kMaxZ] = {};
  const uint16_t* W1[dfl::kMaxZ] = {};
  long long ldw = 0;
  int n_split = 0;
  int M = 0, N = 0, K = 0, nz = 1;
  int mode = dfl::kGemmPartial;
  float* P = nullptr;                 // partial mode, and SwiGLU when split
  unsigned long long* keys = nullptr; // argmax mode: [tiles][ld_keys], one key per column tile and row
  long long ld_keys = 0;
  float* dbg = nullptr;
  long long ld_dbg = 0;
  uint16_t* out = nullptr;            // swiglu mode
  long long ld_out = 0;
  // row scale from the split RMSNorm (a single-pass SwiGLU on the weight-
  // streaming kernel only; see GemmParams::rs): sums of squares
  // [M][kMaxRowChunks], rs_n chunks of a row of rs_len columns
  const float* rs = nullptr;
  int rs_n = 0, rs_len = 0;
  float rs_eps = 0.f;
};

// Runs the weight-streaming GEMM over all M rows (kGemmRows per launch).
// Partial output P[z][s][M][N]; returns the split count through *splits.
hipError_t run_gemm(const GemmCall& c, hipStream_t st, int* splits) {
  const GemmPlan g = plan_gemm(c.M, c.N, c.K, c.nz, c.mode);
  if (splits) *splits = g.splits;
  if (g.swiglu_split) {
    // partials of [gate; up] (2N columns), then silu(gate) * up
    GemmCall pc = c;
    pc.mode = dfl::kGemmPartial;
    pc.N = 2 * c.N;
    pc.n_split = c.N;
    pc.out = nullptr;
    int sp = 0;
    hipError_t e = run_gemm(pc, st, &sp);
    if (e != hipSuccess) return e;
    dfl::SwigluCombineParams sc;
    sc.P = c.P;
    sc.p_s_stride = (long long)c.M * 2 * c.N;
    sc.splits = sp;
    sc.rows = c.M;
    sc.n = c.N;
    sc.out = c.out;
    sc.ld_out = c.ld_out;
    return dfl::launch_swiglu_combine(sc, st);
  }
  if (g.tiled || g.big) {
    if (c.rs) return hipErrorInvalidValue;  // only the weight-streaming SwiGLU applies a row scale
    GemmParams p;
    std::memset(&p, 0, sizeof(p));
    p.A = c.A;
    p.lda = c.lda;
    p.a_idx = c.a_idx;
    p.a_idx_stride = c.a_idx_stride;
    p.a_idx_max = c.a_idx_max;
    for (int z = 0; z < c.nz; ++z) {
      p.W0[z] = c.W0[z];
      p.W1[z] = c.W1[z] ? c.W1[z] : c.W0[z];
    }
    p.ldw = c.ldw;
    p.n_split = (c.W1[0] && c.mode != dfl::kGemmSwiglu) ? c.n_split : c.N;
    p.M = c.M;
    p.N = c.N;
    p.K = c.K;
    p.splits = g.splits;
    p.n_mats = c.nz;
    p.k_per_split = g.k_per_split;
    p.keys = c.keys;
    p.ld_keys = c.ld_keys;
    p.dbg = c.dbg;
    p.ld_dbg = c.ld_dbg;
    p.out = c.out;
    p.ld_out = c.ld_out;
    p.P = c.P;
    p.p_s_stride = (long long)c.M * c.N;
    p.p_z_stride = (long long)g.splits * c.M * c.N;
    if (g.big) return dfl::launch_gemm_big(p, c.mode, c.nz, g.bm, g.bn, st);
    return g.ws ? dfl::launch_gemm_ws(p, g.ng, g.mt, c.mode, c.nz, st)
                : dfl::launch_gemm_tile(p, g.ng, g.mt, c.mode, c.nz, st);
  }
  if (c.rs && c.mode != dfl::kGemmSwiglu) return hipErrorInvalidValue;
  for (int m0 = 0; m0 < c.M; m0 += kGemmRows) {
    GemmParams p;
    std::memset(&p, 0, sizeof(p));
    const int rows = std::min(kGemmRows, c.M - m0);
    const GemmPlan gl = plan_gemm(rows, c.N, c.K, c.nz, c.mode);
    // every chunk keeps the split layout of the full call
    p.A = c.a_idx ? c.A : c.A + (long long)m0 * c.lda;
    p.lda = c.lda;
    p.a_idx = c.a_idx ? c.a_idx + (long long)m0 * c.a_idx_stride : nullptr;
    p.a_idx_stride = c.a_idx_stride;
    p.a_idx_max = c.a_idx_max;
    for (int z = 0; z < c.nz; ++z) {
      p.W0[z] = c.W0[z];
      p.W1[z] = c.W1[z] ? c.W1[z] : c.W0[z];
    }
    p.ldw = c.ldw;
    p.n_split = (c.W1[0] && c.mode != dfl::kGemmSwiglu) ? c.n_split : c.N;
    p.M = rows;
    p.N = c.N;
    p.K = c.K;
    p.splits = g.splits;
    p.n_mats = c.nz;
    p.k_per_split = g.k_per_split;
    p.rs = c.rs ? c.rs + (long long)m0 * dfl::kMaxRowChunks : nullptr;
    p.rs_n = c.rs_n;
    p.rs_len = c.rs_len;
    p.rs_eps = c.rs_eps;
    if (c.mode == dfl::kGemmArgmax) {
      p.keys = c.keys + m0;
      p.ld_keys = c.ld_keys;
      p.dbg = c.dbg ? c.dbg + (long long)m0 * c.ld_dbg : nullptr;
      p.ld_dbg = c.ld_dbg;
    } else if (c.mode == dfl::kGemmSwiglu) {
      p.out = c.out + (long long)m0 * c.ld_out;
      p.ld_out = c.ld_out;
    } else {
      p.P = c.P + (long long)m0 * c.N;
      p.p_s_stride = (long long)c.M * c.N;
      p.p_z_stride = (long long)g.splits * c.M * c.N;
    }
    hipError_t e = dfl::launch_gemm_stream(p, gl.mt, gl.nf, c.mode, c.nz, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Whether run_gemm takes the weight-streaming kernel for this product in one
// pass (no split SwiGLU): the products that can consume the split RMSNorm.
bool gemm_streams(int M, int N, int K, int nz, int mode) {
  const GemmPlan g = plan_gemm(M, N, K, nz, mode);
  return !g.tiled && !g.big && !g.swiglu_split;
}

// Column chunks of the split RMSNorm over n columns, or 0 where the row
// passes keep the one-workgroup-per-row form (a consumer off the weight-
// streaming kernel, or rows too long for the chunk sums).
int split_norm_chunks(int n, bool consumer_streams) {
  const int ch = (n + dfl::kRowChunkCols - 1) / dfl::kRowChunkCols;
  return consumer_streams && n % 4 == 0 && ch <= dfl::kMaxRowChunks ? ch : 0;
}

struct AttnPlan {
  int n_chunks;  // key ranges per sequence at full length
  int n_ranges;  // attention workgroups (chunks at most) per kv head
  int slots;     // partial slots per kv head
  int slice, gb_pad;
};

// attention workgroups when every sequence is at full length, by head size
// (measured on MI355X with 256/384/512/768: D = 64 is fastest at 512, D = 128
// at 384 for the block-sweep batch, 261 against 272 us per step, the batch-32
// and batch-1 splits being the same at both)
constexpr int kAttnTargetWGsD64 = 512;
constexpr int kAttnTargetWGsD128 = 384;
// chunks per (sequence, kv head) at most: at batch 1 (context ~1050, so two
// 64-key slices per chunk) 16 measured 2-3 us per step faster than 32 (one
// slice per chunk: 17 chunks of partials to write and merge) and than 8 or 4
// (longer chunks in fewer workgroups), 64 slower still (measured on MI355X)
constexpr int kAttnMaxChunks = 16;

// Attention chunks: about the target number of workgroups over the batch,
// n_chunks per sequence and kv head at full length, without chunks shorter
// than 64 keys of the cache. The device picks one
// chunk length for the batch from the real lengths so that all chunks fit the
// n_chunks * batch workgroups per kv head: in a ragged batch the long
// sequences take more chunks than the short ones and no workgroup holds more
// keys than the chunk length (with equal lengths this is the per-sequence
// split). Measured on MI355X: 768, 1024 and 2048 workgroups were slower at
// every configuration, 256 too.
AttnPlan plan_attn(const dflash_config& c, int batch, int max_ctx, int B) {
  AttnPlan a;
  const int G = c.n_q_heads / c.n_kv_heads;
  a.gb_pad = (int)cdiv(G * B, 16) * 16;
  const long long units = (long long)batch * c.n_kv_heads;
  long long n = cdiv(c.head_dim == 64 ? kAttnTargetWGsD64 : kAttnTargetWGsD128, units);
  n = std::min<long long>(n, cdiv(max_ctx, 64));
  a.n_chunks = (int)std::max<long long>(1, std::min<long long>(n, kAttnMaxChunks));
  a.n_ranges = a.n_chunks * batch;
  a.slots = a.n_ranges;
  // 64-key slices at every shape: measured on MI355X against 128-key slices,
  // equal or faster everywhere (batch 8 at context 8192: 303 -> 274 us per
  // step, batch 32 at contexts 512..4096: 466 -> 444, the gpt-oss-shaped
  // batch 4 at context 32768: 538 -> 530), mostly because a chunk rounds up
  // to whole slices and the block's B keys push each chunk over a slice
  // boundary
  a.slice = 64;
  return a;
}

// Workspace of one pass of the layer stack over B rows per sequence, lm_rows
// of which reach the LM head (bytes, 256-aligned pieces): a draft block
// (B = block, lm_rows = B - 1) or a target pass (B = n, lm_rows = n).
struct StackWs {
  size_t x, u, q, ao, s, ulm, keys, pm, pl, po, plan, P, ss, total;
};

StackWs stack_ws(const dflash_config& c, int batch, int max_ctx, int B, int lm_rows) {
  StackWs w;
  const long long Mb = (long long)batch * B, Ml = (long long)batch * lm_rows;
  const int H = c.hidden, qw = c.n_q_heads * c.head_dim;
  const int qkvw = (c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim;
  const AttnPlan a = plan_attn(c, batch, max_ctx, B);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align256(bytes);
    return o;
  };
  w.x = take(Mb * H * 4);
  w.u = take(Mb * H * 2);
  w.q = take(Mb * qw * 2);
  w.ao = take(Mb * qw * 2);
  w.s = take(Mb * c.intermediate * 2);
  w.ulm = take(Ml * H * 2);
  w.keys = take((size_t)lm_tiles(c, (int)Ml) * Ml * 8);
  const long long att_rows = (long long)c.n_kv_heads * a.slots * a.gb_pad;
  w.pm = take(att_rows * 4);
  w.pl = take(att_rows * 4);
  w.po = take(att_rows * c.head_dim * 4);
  w.plan = take((size_t)dfl::attn_plan_ints(a.n_ranges, batch) * 4);
  size_t pf = 0;
  pf = std::max(pf, gemm_partial_floats((int)Mb, qkvw, H, 1));
  pf = std::max(pf, gemm_partial_floats((int)Mb, H, qw, 1));
  pf = std::max(pf, gemm_partial_floats((int)Mb, H, c.intermediate, 1));
  pf = std::max(pf, gemm_partial_floats((int)Mb, c.intermediate, H, 1, dfl::kGemmSwiglu));
  w.P = take(pf * 4);
  w.ss = take(Mb * dfl::kMaxRowChunks * 4);  // split RMSNorm sums of squares
  w.total = off;
  return w;
}

// Partial buffer of a fuse or inject call of up to `rows` rows, processed in
// chunks of kRowChunk rows. The split count depends on the chunk's row count
// and a shorter chunk can take more splits, so the buffer covers the largest
// need over every chunk size a call can produce (a full chunk, or any
// remainder below it).
size_t chunked_partial_bytes(int rows, int N, int K, int nz) {
  size_t worst = 0;
  const int top = std::min(std::max(rows, 1), kRowChunk);
  for (int r = 1; r <= top; ++r) worst = std::max(worst, gemm_partial_floats(r, N, K, nz));
  return align256(worst * 4);
}

size_t fuse_ws(const dflash_config& c, int rows) {
  return chunked_partial_bytes(rows, c.hidden, c.n_tap * c.hidden, 1);
}

size_t inject_ws(const dflash_config& c, int rows) {
  return chunked_partial_bytes(rows, 2 * c.n_kv_heads * c.head_dim, c.hidden, c.n_layers);
}

dflash_status hip_status(hipError_t e) { return e == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP; }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

dflash_status check_kv(const dflash_model* m, const dflash_kv* kv) {
  if (!kv || !kv->k || !kv->v || !kv->ctx_len || !kv->status) return DFLASH_ERR_NULL;
  if (kv->batch < 1 || kv->batch > kMaxBatch) return DFLASH_ERR_SHAPE;
  if (kv->max_ctx < m->cfg.block) return DFLASH_ERR_SHAPE;
  return DFLASH_OK;
}

}  // namespace

extern "C" {

const char* dflash_status_string(dflash_status s) {
  switch (s) {
    case DFLASH_OK: return "ok";
    case DFLASH_ERR_NULL: return "null pointer";
    case DFLASH_ERR_SHAPE: return "bad shape";
    case DFLASH_ERR_UNSUPPORTED: return "unsupported shape";
    case DFLASH_ERR_WORKSPACE: return "workspace too small";
    case DFLASH_ERR_CAPACITY: return "cache capacity exceeded";
    case DFLASH_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

namespace {

// Checks shared by drafter and target models.
dflash_status check_model(const dflash_config& c, const dflash_weights* w, int max_layers) {
  if (c.hidden <= 0 || c.n_layers <= 0 || c.n_q_heads <= 0 || c.n_kv_heads <= 0 ||
      c.head_dim <= 0 || c.intermediate <= 0 || c.vocab <= 1 || c.n_tap <= 0 || c.block <= 0)
    return DFLASH_ERR_SHAPE;
  if (c.mask_id < 0 || c.mask_id >= c.vocab) return DFLASH_ERR_SHAPE;
  if (c.n_q_heads % c.n_kv_heads != 0) return DFLASH_ERR_SHAPE;
  if (!(c.rms_eps > 0.f) || !(c.rope_theta > 0.f)) return DFLASH_ERR_SHAPE;
  if (c.n_layers > max_layers) return DFLASH_ERR_UNSUPPORTED;
  if (c.head_dim != 64 && c.head_dim != 128) return DFLASH_ERR_UNSUPPORTED;
  if (c.hidden % 64 || c.intermediate % 64 || (c.n_q_heads * c.head_dim) % 64 ||
      ((long long)c.n_tap * c.hidden) % 64 || c.vocab % 16)
    return DFLASH_ERR_UNSUPPORTED;
  if ((c.n_q_heads / c.n_kv_heads) * c.block > 256) return DFLASH_ERR_UNSUPPORTED;
  if (c.hidden > 8192) return DFLASH_ERR_UNSUPPORTED;  // row kernels hold a row in registers
  if (!w->embed || !w->lm_head || !w->g_final || !w->layers || !w->rope) return DFLASH_ERR_NULL;
  if (w->rope_max_pos < 1) return DFLASH_ERR_SHAPE;
  for (int l = 0; l < c.n_layers; ++l) {
    const dflash_layer_weights& L = w->layers[l];
    if (!L.g_in || !L.w_qkv || !L.g_q || !L.g_k || !L.w_o || !L.g_post || !L.w_gate || !L.w_up ||
        !L.w_down)
      return DFLASH_ERR_NULL;
  }
  return DFLASH_OK;
}

dflash_model* new_model(const dflash_config& c, const dflash_weights* w) {
  dflash_model* m = new (std::nothrow) dflash_model;
  if (!m) return nullptr;
  m->cfg = c;
  m->w = *w;
  m->layers.assign(w->layers, w->layers + c.n_layers);
  m->w.layers = m->layers.data();
  return m;
}

}  // namespace

dflash_status dflash_model_create(const dflash_config* cfg, const dflash_weights* w,
                                  dflash_model** out) {
  if (!cfg || !w || !out) return DFLASH_ERR_NULL;
  *out = nullptr;
  const dflash_config& c = *cfg;
  const dflash_status st = check_model(c, w, dfl::kMaxLayers);
  if (st != DFLASH_OK) return st;
  if (!w->w_fc || !w->g_fc) return DFLASH_ERR_NULL;
  if (c.block < 2 || c.block > 16) return DFLASH_ERR_UNSUPPORTED;
  dflash_model* m = new_model(c, w);
  if (!m) return DFLASH_ERR_SHAPE;
  *out = m;
  return DFLASH_OK;
}

dflash_status dflash_target_create(const dflash_config* cfg, const dflash_weights* w, const int32_t* tap_layers,
                                   dflash_model** out) {
  if (!cfg || !w || !out || !tap_layers) return DFLASH_ERR_NULL;
  *out = nullptr;
  const dflash_config& c = *cfg;
  const dflash_status st = check_model(c, w, kMaxTargetLayers);
  if (st != DFLASH_OK) return st;
  if (c.block > 64) return DFLASH_ERR_UNSUPPORTED;
  for (int t = 0; t < c.n_tap; ++t)
    if (tap_layers[t] < 0 || tap_layers[t] >= c.n_layers || (t > 0 && tap_layers[t] <= tap_layers[t - 1]))
      return DFLASH_ERR_SHAPE;
  dflash_model* m = new_model(c, w);
  if (!m) return DFLASH_ERR_SHAPE;
  m->target = true;
  m->taps.assign(tap_layers, tap_layers + c.n_tap);
  *out = m;
  return DFLASH_OK;
}

void dflash_model_destroy(dflash_model* m) { delete m; }

dflash_status dflash_rope_table(float* out, int32_t max_pos, int32_t head_dim, float theta) {
  if (!out) return DFLASH_ERR_NULL;
  if (max_pos < 1 || head_dim < 2 || head_dim % 2 || !(theta > 0.f)) return DFLASH_ERR_SHAPE;
  const int half = head_dim / 2;
  std::vector<double> freq(half);
  for (int i = 0; i < half; ++i) freq[i] = std::pow((double)theta, -2.0 * i / head_dim);
  for (long long p = 0; p < max_pos; ++p)
    for (int i = 0; i < half; ++i) {
      const double a = (double)p * freq[i];
      out[(p * half + i) * 2] = (float)std::cos(a);
      out[(p * half + i) * 2 + 1] = (float)std::sin(a);
    }
  return DFLASH_OK;
}

namespace {

// Workspace of sampling-mode verification (and of the Gumbel pass of a
// sampled draft block): log-sum-exps, the target-token row, per-sequence
// state and the chunk keys.
struct SampleWs {
  size_t pmax, psum, a, m, rej, keys, total;
};

SampleWs sample_ws(const dflash_config& c, int batch) {
  SampleWs w;
  const int B = c.block;
  const long long items = std::max<long long>(batch, (long long)batch * (B - 1));
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align256(bytes);
    return o;
  };
  const size_t pairs = (size_t)batch * (2 * B - 1) * dfl::sample_chunks(c.vocab);
  w.pmax = take(pairs * 4);
  w.psum = take(pairs * 4);
  w.a = take((size_t)batch * B * 4);
  w.m = take((size_t)batch * 4);
  w.rej = take((size_t)batch * 4);
  w.keys = take((size_t)dfl::gumbel_chunks(c.vocab) * items * 8);
  w.total = off;
  return w;
}

bool sample_temperature_ok(float t) { return t > 0.f && t < 3.0e38f; }

}  // namespace

size_t dflash_workspace_bytes(const dflash_model* m, int32_t max_batch, int32_t max_ctx,
                              int32_t max_rows) {
  if (!m || max_batch < 1 || max_ctx < 1 || max_rows < 0) return 0;
  const dflash_config& c = m->cfg;
  if (m->target) {
    // a target pass of any n <= block rows per sequence (split counts, and so
    // partial sizes, need not grow with n)
    size_t n = 0;
    for (int b = 1; b <= c.block; ++b) n = std::max(n, stack_ws(c, max_batch, max_ctx, b, b).total);
    return n;
  }
  size_t n = stack_ws(c, max_batch, max_ctx, c.block, c.block - 1).total;
  n = std::max(n, sample_ws(c, max_batch).total);
  n = std::max(n, fuse_ws(c, std::max(1, max_rows)));
  n = std::max(n, inject_ws(c, std::max(1, max_rows)));
  return n;
}

dflash_status dflash_fuse_ctx(const dflash_model* m, const void* taps, int32_t n_rows, void* ctx,
                              void* ws, size_t ws_bytes, void* stream) {
  if (!m) return DFLASH_ERR_NULL;
  if (n_rows < 0) return DFLASH_ERR_SHAPE;
  if (n_rows == 0) return DFLASH_OK;
  if (!taps || !ctx || !ws) return DFLASH_ERR_NULL;
  if (m->target) return DFLASH_ERR_UNSUPPORTED;
  const dflash_config& c = m->cfg;
  if (ws_bytes < fuse_ws(c, n_rows)) return DFLASH_ERR_WORKSPACE;
  const hipStream_t st = as_stream(stream);
  const int H = c.hidden, K = c.n_tap * c.hidden;
  float* P = static_cast<float*>(ws);
  for (int r0 = 0; r0 < n_rows; r0 += kRowChunk) {
    const int rows = std::min(kRowChunk, n_rows - r0);
    GemmCall g;
    g.A = static_cast<const uint16_t*>(taps) + (long long)r0 * K;
    g.lda = K;
    g.W0[0] = static_cast<const uint16_t*>(m->w.w_fc);
    g.ldw = K;
    g.M = rows;
    g.N = H;
    g.K = K;
    g.P = P;
    int splits = 1;
    hipError_t e;
    {
      prof::Scope ps(DFLASH_PHASE_FUSE, st);
      e = run_gemm(g, st, &splits);
    }
    if (e != hipSuccess) return DFLASH_ERR_HIP;
    dfl::RowNormParams rn;
    std::memset(&rn, 0, sizeof(rn));
    rn.P = P;
    rn.p_s_stride = (long long)rows * H;
    rn.splits = splits;
    rn.gain = static_cast<const uint16_t*>(m->w.g_fc);
    rn.eps = c.rms_eps;
    rn.rows = rows;
    rn.n = H;
    rn.out = static_cast<uint16_t*>(ctx) + (long long)r0 * H;
    e = dfl::launch_row_norm(rn, st);
    if (e != hipSuccess) return DFLASH_ERR_HIP;
  }
  return DFLASH_OK;
}

dflash_status dflash_inject_kv(const dflash_model* m, const void* ctx, int32_t n_ctx_rows,
                               const int32_t* commit_rows, const int32_t* n_commit,
                               int32_t max_commit, dflash_kv* kv, void* ws, size_t ws_bytes,
                               void* stream) {
  if (!m) return DFLASH_ERR_NULL;
  if (max_commit < 0 || n_ctx_rows < 0) return DFLASH_ERR_SHAPE;
  if (max_commit == 0) return DFLASH_OK;
  if (!ctx || !commit_rows || !n_commit || !ws) return DFLASH_ERR_NULL;
  if (n_ctx_rows == 0) return DFLASH_ERR_SHAPE;
  if (m->target) return DFLASH_ERR_UNSUPPORTED;
  // gathered context rows are addressed with 32-bit element offsets
  if ((long long)n_ctx_rows * m->cfg.hidden > 0x7FFFFFFFll) return DFLASH_ERR_UNSUPPORTED;
  dflash_status ks = check_kv(m, kv);
  if (ks != DFLASH_OK) return ks;
  const dflash_config& c = m->cfg;
  if (ws_bytes < inject_ws(c, max_commit)) return DFLASH_ERR_WORKSPACE;
  const hipStream_t st = as_stream(stream);
  const int H = c.hidden, D = c.head_dim, Hq = c.n_q_heads, Hkv = c.n_kv_heads;
  const int N = 2 * Hkv * D;
  float* P = static_cast<float*>(ws);
  for (int c0 = 0; c0 < max_commit; c0 += kRowChunk) {
    const int rows = std::min(kRowChunk, max_commit - c0);
    GemmCall g;
    g.A = static_cast<const uint16_t*>(ctx);
    g.lda = H;
    g.a_idx = commit_rows + 3ll * c0;
    g.a_idx_stride = 3;
    g.a_idx_max = n_ctx_rows;
    g.nz = c.n_layers;
    for (int l = 0; l < c.n_layers; ++l)  // k rows then v rows of each layer's (packed) W_qkv
      g.W0[l] = static_cast<const uint16_t*>(m->layers[l].w_qkv) + (long long)(Hq * D / 16) * (H / 32) * 512;
    g.ldw = H;
    g.M = rows;
    g.N = N;
    g.K = H;
    g.P = P;
    int splits = 1;
    hipError_t e;
    {
      prof::Scope ps(DFLASH_PHASE_INJECT, st);
      e = run_gemm(g, st, &splits);
    }
    if (e != hipSuccess) return DFLASH_ERR_HIP;
    dfl::InjectPostParams ip;
    std::memset(&ip, 0, sizeof(ip));
    ip.P = P;
    ip.p_s_stride = (long long)rows * N;
    ip.p_z_stride = (long long)splits * rows * N;
    ip.splits = splits;
    for (int l = 0; l < c.n_layers; ++l) ip.gk[l] = static_cast<const uint16_t*>(m->layers[l].g_k);
    ip.rope = m->w.rope;
    ip.rope_max = m->w.rope_max_pos;
    ip.commit_rows = commit_rows;
    ip.n_commit = n_commit;
    ip.max_commit = max_commit;
    ip.n_ctx_rows = n_ctx_rows;
    ip.c0 = c0;
    ip.c1 = c0 + rows;
    ip.n_layers = c.n_layers;
    ip.batch = kv->batch;
    ip.Hkv = Hkv;
    ip.D = D;
    ip.max_ctx = kv->max_ctx;
    ip.eps = c.rms_eps;
    ip.kc = static_cast<uint16_t*>(kv->k);
    ip.vc = static_cast<uint16_t*>(kv->v);
    ip.ctx_len = kv->ctx_len;
    ip.status = kv->status;
    e = dfl::launch_inject_post(ip, st);
    if (e != hipSuccess) return DFLASH_ERR_HIP;
  }
  return DFLASH_OK;
}

namespace {

// One pass of the layer stack over B rows per sequence (a draft block or a
// target pass); see dflash_draft_block and dflash_target_forward.
struct StackIO {
  const int32_t* anchor = nullptr;  // draft: row 0's token (rows 1..B-1: mask id)
  const int32_t* tokens = nullptr;  // target: every row's token [batch, B]
  int B = 0;                        // rows per sequence
  int lm_skip = 0;                  // 1: rows j >= 1 reach the LM head (draft), 0: all rows
  int causal = 0;                   // block attention causal inside the block
  uint16_t* taps = nullptr;         // target: bf16 [batch*B, n_tap*H] or NULL
  int32_t* out = nullptr;           // argmax of the LM rows, [batch, B - lm_skip]
  float* dbg_logits = nullptr;
  float* dbg_hidden = nullptr;
};

dflash_status run_stack(const dflash_model* m, dflash_kv* kv, const StackIO& io, void* ws, size_t ws_bytes,
                        void* stream) {
  const dflash_config& c = m->cfg;
  const int batch = kv->batch, B = io.B, H = c.hidden, D = c.head_dim;
  const int Hq = c.n_q_heads, Hkv = c.n_kv_heads, I = c.intermediate, NL = c.n_layers;
  const int lm_rows = B - io.lm_skip;
  const int Mb = batch * B, Ml = batch * lm_rows;
  const int qw = Hq * D, qkvw = (Hq + 2 * Hkv) * D;
  const StackWs w = stack_ws(c, batch, kv->max_ctx, B, lm_rows);
  if (ws_bytes < w.total) return DFLASH_ERR_WORKSPACE;
  const AttnPlan ap = plan_attn(c, batch, kv->max_ctx, B);
  float* dbg_hidden = io.dbg_hidden;
  float* dbg_logits = io.dbg_logits;
  const hipStream_t st = as_stream(stream);
  char* base = static_cast<char*>(ws);
  float* x = reinterpret_cast<float*>(base + w.x);
  uint16_t* u = reinterpret_cast<uint16_t*>(base + w.u);
  uint16_t* q = reinterpret_cast<uint16_t*>(base + w.q);
  uint16_t* ao = reinterpret_cast<uint16_t*>(base + w.ao);
  uint16_t* sb = reinterpret_cast<uint16_t*>(base + w.s);
  uint16_t* ulm = reinterpret_cast<uint16_t*>(base + w.ulm);
  unsigned long long* keys = reinterpret_cast<unsigned long long*>(base + w.keys);
  float* pm = reinterpret_cast<float*>(base + w.pm);
  float* pl = reinterpret_cast<float*>(base + w.pl);
  float* po = reinterpret_cast<float*>(base + w.po);
  int32_t* plan = reinterpret_cast<int32_t*>(base + w.plan);
  float* P = reinterpret_cast<float*>(base + w.P);
  float* ss = reinterpret_cast<float*>(base + w.ss);
  const long long layer_kv = (long long)batch * Hkv * kv->max_ctx * D;
  // Few rows (the weight-streaming GEMMs): the RMSNorms inside the stack take
  // the split form, u = x * gain with the row sums of squares in ss, and 1/rms
  // is applied after the next product, by the QKV post-pass or by the SwiGLU
  // epilogue. The final norm keeps the one-pass form, so that the LM head's
  // logits and argmax are the same numbers with or without logits requested.
  // u_chunks: chunks of the norm that wrote u (the embedding pass included),
  // 0 when u is normalised already.
  int u_chunks = 0;
  const long long hid = (long long)Mb * H;
  hipError_t e;

  dfl::EmbedParams ep;
  std::memset(&ep, 0, sizeof(ep));
  ep.anchor = io.anchor;
  ep.tokens = io.tokens;
  ep.embed = static_cast<const uint16_t*>(m->w.embed);
  ep.gain = static_cast<const uint16_t*>(m->layers[0].g_in);
  ep.ctx_len = kv->ctx_len;
  ep.status = kv->status;
  ep.batch = batch;
  ep.B = B;
  ep.H = H;
  ep.V = c.vocab;
  ep.mask_id = c.mask_id;
  ep.max_ctx = kv->max_ctx;
  ep.rope_max = m->w.rope_max_pos;
  ep.eps = c.rms_eps;
  ep.x = x;
  ep.u = u;
  ep.dbg = dbg_hidden;
  u_chunks = split_norm_chunks(H, gemm_streams(Mb, qkvw, H, 1, dfl::kGemmPartial));
  if (u_chunks) {
    ep.ssp = ss;
    ep.ss_chunks = u_chunks;
  }
  if ((e = dfl::launch_embed(ep, st)) != hipSuccess) return DFLASH_ERR_HIP;

  for (int l = 0; l < NL; ++l) {
    const dflash_layer_weights& L = m->layers[l];
    int splits = 1;
    // q, k, v
    GemmCall g;
    g.A = u;
    g.lda = H;
    g.W0[0] = static_cast<const uint16_t*>(L.w_qkv);
    g.ldw = H;
    g.M = Mb;
    g.N = qkvw;
    g.K = H;
    g.P = P;
    {
      prof::Scope ps(DFLASH_PHASE_QKV, st);
      e = run_gemm(g, st, &splits);
    }
    if (e != hipSuccess) return DFLASH_ERR_HIP;
    dfl::QkvPostParams qp;
    std::memset(&qp, 0, sizeof(qp));
    qp.P = P;
    qp.p_s_stride = (long long)Mb * qkvw;
    qp.splits = splits;
    qp.gq = static_cast<const uint16_t*>(L.g_q);
    qp.gk = static_cast<const uint16_t*>(L.g_k);
    qp.rope = m->w.rope;
    qp.rope_max = m->w.rope_max_pos;
    qp.ctx_len = kv->ctx_len;
    qp.status = kv->status;
    qp.batch = batch;
    qp.B = B;
    qp.Hq = Hq;
    qp.Hkv = Hkv;
    qp.D = D;
    qp.max_ctx = kv->max_ctx;
    qp.eps = c.rms_eps;
    qp.q = q;
    qp.q_scale = (float)(1.4426950408889634 / std::sqrt((double)D));
    qp.kc = static_cast<uint16_t*>(kv->k) + l * layer_kv;
    qp.vc = static_cast<uint16_t*>(kv->v) + l * layer_kv;
    // the attention chunk split holds for the whole pass (lengths and statuses
    // do not change in it): written once, by the first layer
    qp.plan = l == 0 ? plan : nullptr;
    qp.n_ranges = ap.n_ranges;
    qp.slice = ap.slice;
    if (u_chunks) {
      qp.rs = ss;
      qp.rs_n = u_chunks;
      qp.rs_len = H;
      qp.rs_eps = c.rms_eps;
    }
    if ((e = dfl::launch_qkv_post(qp, st)) != hipSuccess) return DFLASH_ERR_HIP;
    // attention over [context ; block]
    dfl::AttnParams at;
    std::memset(&at, 0, sizeof(at));
    at.q = q;
    at.k = qp.kc;
    at.v = qp.vc;
    at.ctx_len = kv->ctx_len;
    at.status = kv->status;
    at.batch = batch;
    at.Hq = Hq;
    at.Hkv = Hkv;
    at.B = B;
    at.max_ctx = kv->max_ctx;
    at.n_ranges = ap.n_ranges;
    at.slots = ap.slots;
    at.plan = plan;
    at.slice = ap.slice;
    at.gb_pad = ap.gb_pad;
    at.causal = io.causal;
    at.pm = pm;
    at.pl = pl;
    at.po = po;
    {
      prof::Scope ps(DFLASH_PHASE_ATTENTION, st);
      e = dfl::launch_attention(at, D, st);
    }
    if (e != hipSuccess) return DFLASH_ERR_HIP;
    dfl::MergeParams mp;
    std::memset(&mp, 0, sizeof(mp));
    mp.pm = pm;
    mp.pl = pl;
    mp.po = po;
    mp.ctx_len = kv->ctx_len;
    mp.status = kv->status;
    mp.batch = batch;
    mp.Hq = Hq;
    mp.Hkv = Hkv;
    mp.B = B;
    mp.D = D;
    mp.n_ranges = ap.n_ranges;
    mp.slots = ap.slots;
    mp.seg_hint = ap.n_chunks;
    mp.plan = plan;
    mp.gb_pad = ap.gb_pad;
    mp.out = ao;
    {
      prof::Scope ps(DFLASH_PHASE_MERGE, st);
      e = dfl::launch_attn_merge(mp, st);
    }
    if (e != hipSuccess) return DFLASH_ERR_HIP;
    // o projection, residual, post-attention norm
    GemmCall go;
    go.A = ao;
    go.lda = qw;
    go.W0[0] = static_cast<const uint16_t*>(L.w_o);
    go.ldw = qw;
    go.M = Mb;
    go.N = H;
    go.K = qw;
    go.P = P;
    {
      prof::Scope ps(DFLASH_PHASE_O, st);
      e = run_gemm(go, st, &splits);
    }
    if (e != hipSuccess) return DFLASH_ERR_HIP;
    dfl::RowNormParams rn;
    std::memset(&rn, 0, sizeof(rn));
    rn.x = x;
    rn.P = P;
    rn.p_s_stride = (long long)Mb * H;
    rn.splits = splits;
    rn.gain = static_cast<const uint16_t*>(L.g_post);
    rn.eps = c.rms_eps;
    rn.rows = Mb;
    rn.n = H;
    rn.out = u;
    const int gu_chunks = split_norm_chunks(H, gemm_streams(Mb, I, H, 1, dfl::kGemmSwiglu));
    if (gu_chunks) {
      rn.ssp = ss;
      rn.ss_chunks = gu_chunks;
    }
    if ((e = dfl::launch_row_norm(rn, st)) != hipSuccess) return DFLASH_ERR_HIP;
    // gate and up in one pass with SwiGLU in the epilogue
    GemmCall gg;
    gg.A = u;
    gg.lda = H;
    gg.W0[0] = static_cast<const uint16_t*>(L.w_gate);
    gg.W1[0] = static_cast<const uint16_t*>(L.w_up);
    gg.ldw = H;
    gg.M = Mb;
    gg.N = I;
    gg.K = H;
    gg.mode = dfl::kGemmSwiglu;
    gg.out = sb;
    gg.ld_out = I;
    gg.P = P;
    if (gu_chunks) {
      gg.rs = ss;
      gg.rs_n = gu_chunks;
      gg.rs_len = H;
      gg.rs_eps = c.rms_eps;
    }
    {
      prof::Scope ps(DFLASH_PHASE_GATE_UP, st);
      e = run_gemm(gg, st, nullptr);
    }
    if (e != hipSuccess) return DFLASH_ERR_HIP;
    // down projection, residual, next norm (or the final norm)
    GemmCall gd;
    gd.A = sb;
    gd.lda = I;
    gd.W0[0] = static_cast<const uint16_t*>(L.w_down);
    gd.ldw = I;
    gd.M = Mb;
    gd.N = H;
    gd.K = I;
    gd.P = P;
    {
      prof::Scope ps(DFLASH_PHASE_DOWN, st);
      e = run_gemm(gd, st, &splits);
    }
    if (e != hipSuccess) return DFLASH_ERR_HIP;
    std::memset(&rn, 0, sizeof(rn));
    rn.x = x;
    rn.P = P;
    rn.p_s_stride = (long long)Mb * H;
    rn.splits = splits;
    rn.eps = c.rms_eps;
    rn.rows = Mb;
    rn.n = H;
    rn.dbg = dbg_hidden ? dbg_hidden + (long long)(l + 1) * hid : nullptr;
    if (io.taps) {
      for (size_t t = 0; t < m->taps.size(); ++t)
        if (m->taps[t] == l) {
          rn.tap = io.taps + (long long)t * H;
          rn.tap_ld = (long long)m->taps.size() * H;
        }
    }
    if (l + 1 < NL) {
      rn.gain = static_cast<const uint16_t*>(m->layers[l + 1].g_in);
      rn.out = u;
      u_chunks = split_norm_chunks(H, gemm_streams(Mb, qkvw, H, 1, dfl::kGemmPartial));
    } else {
      rn.gain = static_cast<const uint16_t*>(m->w.g_final);
      rn.out = ulm;
      rn.final_mode = io.lm_skip;
      rn.B = B;
      u_chunks = 0;
    }
    if (u_chunks) {
      rn.ssp = ss;
      rn.ss_chunks = u_chunks;
    }
    if ((e = dfl::launch_row_norm(rn, st)) != hipSuccess) return DFLASH_ERR_HIP;
  }

  // LM head with the argmax fused; logits only for the debug buffer
  GemmCall gl;
  gl.A = ulm;
  gl.lda = H;
  gl.W0[0] = static_cast<const uint16_t*>(m->w.lm_head);
  gl.ldw = H;
  gl.M = Ml;
  gl.N = c.vocab;
  gl.K = H;
  gl.mode = dfl::kGemmArgmax;
  gl.keys = keys;
  gl.ld_keys = Ml;
  gl.dbg = dbg_logits;
  gl.ld_dbg = c.vocab;
  {
    prof::Scope ps(DFLASH_PHASE_LM_HEAD, st);
    e = run_gemm(gl, st, nullptr);
  }
  if (e != hipSuccess) return DFLASH_ERR_HIP;
  return hip_status(dfl::launch_argmax_finish(keys, lm_tiles(c, Ml), kv->status, batch, lm_rows, io.out, st));
}

}  // namespace

}  // extern "C"

dflash_status dfl::draft_block_check(const dflash_model* m, const dflash_kv* kv, const int32_t* anchor,
                                     const int32_t* draft, size_t* ws_need) {
  if (!m || !anchor || !draft) return DFLASH_ERR_NULL;
  if (m->target) return DFLASH_ERR_UNSUPPORTED;
  dflash_status ks = check_kv(m, kv);
  if (ks != DFLASH_OK) return ks;
  const int B = m->cfg.block;
  *ws_need = stack_ws(m->cfg, kv->batch, kv->max_ctx, B, B - 1).total;
  return DFLASH_OK;
}

dflash_status dfl::draft_block_run(const dflash_model* m, dflash_kv* kv, const int32_t* anchor, int32_t* draft,
                                   float* dbg_logits, float* dbg_hidden, void* ws, size_t ws_bytes, void* stream,
                                   bool no_events) {
  StackIO io;
  io.anchor = anchor;
  io.B = m->cfg.block;
  io.lm_skip = 1;
  io.out = draft;
  io.dbg_logits = dbg_logits;
  io.dbg_hidden = dbg_hidden;
  const bool was = prof::suspended;
  prof::suspended = was || no_events;
  const dflash_status s = run_stack(m, kv, io, ws, ws_bytes, stream);
  prof::suspended = was;
  return s;
}

extern "C" {

dflash_status dflash_draft_block(const dflash_model* m, dflash_kv* kv, const int32_t* anchor,
                                 int32_t* draft, float* dbg_logits, float* dbg_hidden, void* ws,
                                 size_t ws_bytes, void* stream) {
  size_t need = 0;
  const dflash_status s = dfl::draft_block_check(m, kv, anchor, draft, &need);
  if (s != DFLASH_OK) return s;
  if (!ws) return DFLASH_ERR_NULL;
  if (ws_bytes < need) return DFLASH_ERR_WORKSPACE;
  return dfl::draft_block_run(m, kv, anchor, draft, dbg_logits, dbg_hidden, ws, ws_bytes, stream, false);
}

dflash_status dflash_draft_block_sample(const dflash_model* m, dflash_kv* kv, const int32_t* anchor,
                                        int32_t* draft, float* logits, float temperature, uint64_t seed,
                                        int32_t step, const int32_t* step_dev, void* ws, size_t ws_bytes,
                                        void* stream) {
  if (!m || !anchor || !draft || !logits || !ws) return DFLASH_ERR_NULL;
  if (m->target) return DFLASH_ERR_UNSUPPORTED;
  if (!sample_temperature_ok(temperature)) return DFLASH_ERR_SHAPE;
  dflash_status ks = check_kv(m, kv);
  if (ks != DFLASH_OK) return ks;
  const dflash_config& c = m->cfg;
  const SampleWs sw = sample_ws(c, kv->batch);
  if (ws_bytes < sw.total) return DFLASH_ERR_WORKSPACE;
  // the greedy pass writes the raw logits; its argmax is then replaced by the
  // Gumbel-max samples (the stack's workspace is dead by then)
  StackIO io;
  io.anchor = anchor;
  io.B = c.block;
  io.lm_skip = 1;
  io.out = draft;
  io.dbg_logits = logits;
  const dflash_status s = run_stack(m, kv, io, ws, ws_bytes, stream);
  if (s != DFLASH_OK) return s;
  dfl::GumbelParams g{};
  std::memset(&g, 0, sizeof(g));
  g.z = logits;
  g.B = c.block;
  g.V = c.vocab;
  g.items = kv->batch * (c.block - 1);
  g.chunks = dfl::gumbel_chunks(c.vocab);
  g.inv_t = 1.0f / temperature;
  g.seed_lo = (uint32_t)seed;
  g.seed_hi = (uint32_t)(seed >> 32);
  g.step = (uint32_t)step;
  g.step_dev = step_dev;
  g.keys = reinterpret_cast<unsigned long long*>(static_cast<char*>(ws) + sw.keys);
  g.out = draft;
  g.status = kv->status;
  return hip_status(dfl::launch_gumbel(g, 0, as_stream(stream)));
}

dflash_status dflash_target_forward(const dflash_model* m, dflash_kv* kv, const int32_t* tokens, int32_t n,
                                    int32_t* argmax, void* taps, float* dbg_logits, void* ws, size_t ws_bytes,
                                    void* stream) {
  if (!m || !tokens || !argmax || !ws) return DFLASH_ERR_NULL;
  if (!m->target) return DFLASH_ERR_UNSUPPORTED;
  if (n < 1 || n > m->cfg.block) return DFLASH_ERR_SHAPE;
  dflash_status ks = check_kv(m, kv);
  if (ks != DFLASH_OK) return ks;
  StackIO io;
  io.tokens = tokens;
  io.B = n;
  io.lm_skip = 0;
  io.causal = 1;
  io.taps = static_cast<uint16_t*>(taps);
  io.out = argmax;
  io.dbg_logits = dbg_logits;
  return run_stack(m, kv, io, ws, ws_bytes, stream);
}

dflash_status dflash_kv_commit(const dflash_model* m, dflash_kv* kv, const int32_t* commit_rows,
                               const int32_t* n_commit, int32_t max_commit, void* stream) {
  if (!m) return DFLASH_ERR_NULL;
  if (max_commit < 0) return DFLASH_ERR_SHAPE;
  if (max_commit == 0) return DFLASH_OK;
  if (!commit_rows || !n_commit) return DFLASH_ERR_NULL;
  dflash_status ks = check_kv(m, kv);
  if (ks != DFLASH_OK) return ks;
  return hip_status(dfl::launch_kv_commit(commit_rows, n_commit, max_commit, kv->batch, kv->max_ctx, kv->ctx_len,
                                          as_stream(stream)));
}

dflash_status dflash_verify_accept(const dflash_model* m, const dflash_kv* kv,
                                   const int32_t* draft, const int32_t* target_argmax,
                                   const int32_t* stop_ids, int32_t n_stop, int32_t* budget,
                                   int32_t* accept_len, int32_t* anchor_out, int32_t* emitted,
                                   int32_t* n_emit, int32_t* done, int32_t* commit_rows,
                                   int32_t* n_commit, void* stream) {
  if (!m) return DFLASH_ERR_NULL;
  if (m->target) return DFLASH_ERR_UNSUPPORTED;
  dflash_status ks = check_kv(m, kv);
  if (ks != DFLASH_OK) return ks;
  if (!draft || !target_argmax || !accept_len || !anchor_out || !emitted || !n_emit || !done ||
      !commit_rows || !n_commit)
    return DFLASH_ERR_NULL;
  if (n_stop < 0) return DFLASH_ERR_SHAPE;
  if (n_stop > 0 && !stop_ids) return DFLASH_ERR_NULL;
  dfl::VerifyParams p;
  p.draft = draft;
  p.target = target_argmax;
  p.stop_ids = stop_ids;
  p.n_stop = n_stop;
  p.budget = budget;
  p.ctx_len = kv->ctx_len;
  p.status = kv->status;
  p.batch = kv->batch;
  p.B = m->cfg.block;
  p.accept_len = accept_len;
  p.anchor_out = anchor_out;
  p.emitted = emitted;
  p.n_emit = n_emit;
  p.done = done;
  p.commit_rows = commit_rows;
  p.n_commit = n_commit;
  prof::Scope ps(DFLASH_PHASE_VERIFY, as_stream(stream));
  return hip_status(dfl::launch_verify(p, as_stream(stream)));
}

dflash_status dflash_ingest_rows(const dflash_model* m, const dflash_kv* kv, int32_t seq, int32_t start, int32_t n,
                                 int32_t* commit_rows, int32_t* n_commit, void* stream) {
  if (!m || !commit_rows || !n_commit) return DFLASH_ERR_NULL;
  if (m->target) return DFLASH_ERR_UNSUPPORTED;
  const dflash_status ks = check_kv(m, kv);
  if (ks != DFLASH_OK) return ks;
  if (seq < 0 || seq >= kv->batch || start < 0 || n < 0 || (long long)start + n > kv->max_ctx) return DFLASH_ERR_SHAPE;
  return hip_status(dfl::launch_ingest_rows(commit_rows, n_commit, seq, start, n, as_stream(stream)));
}

dflash_status dflash_loop_tokens(const dflash_model* m, const dflash_kv* kv, const int32_t* anchor,
                                 const int32_t* draft, int32_t* tokens, void* stream) {
  if (!m || !anchor || !draft || !tokens) return DFLASH_ERR_NULL;
  if (m->target) return DFLASH_ERR_UNSUPPORTED;
  const dflash_status ks = check_kv(m, kv);
  if (ks != DFLASH_OK) return ks;
  return hip_status(dfl::launch_loop_tokens(anchor, draft, tokens, kv->batch, m->cfg.block, as_stream(stream)));
}

dflash_status dflash_loop_advance(const dflash_model* m, const dflash_kv* kv, const int32_t* anchor_out,
                                  const int32_t* emitted, const int32_t* n_emit, const int32_t* done, int32_t* out,
                                  int32_t ld_out, int32_t max_new, int32_t* cursor, int32_t* alive,
                                  int32_t* anchor, int32_t* step_dev, void* stream) {
  if (!m || !anchor_out || !emitted || !n_emit || !done || !out || !cursor || !alive || !anchor)
    return DFLASH_ERR_NULL;
  if (m->target) return DFLASH_ERR_UNSUPPORTED;
  const dflash_status ks = check_kv(m, kv);
  if (ks != DFLASH_OK) return ks;
  if (max_new < 0 || ld_out < max_new) return DFLASH_ERR_SHAPE;
  dfl::LoopAdvanceParams p;
  p.anchor_out = anchor_out;
  p.emitted = emitted;
  p.n_emit = n_emit;
  p.done = done;
  p.out = out;
  p.ld_out = ld_out;
  p.max_new = max_new;
  p.cursor = cursor;
  p.alive = alive;
  p.anchor = anchor;
  p.step_dev = step_dev;
  p.batch = kv->batch;
  p.B = m->cfg.block;
  return hip_status(dfl::launch_loop_advance(p, as_stream(stream)));
}

dflash_status dflash_sample_logits(const dflash_model* m, const float* logits, int32_t rows, float temperature,
                                   uint64_t seed, int32_t step, int32_t row0, int32_t* tokens, void* ws,
                                   size_t ws_bytes, void* stream) {
  if (!m) return DFLASH_ERR_NULL;
  if (rows < 0 || row0 < 0) return DFLASH_ERR_SHAPE;
  if (rows == 0) return DFLASH_OK;
  if (!logits || !tokens || !ws) return DFLASH_ERR_NULL;
  if (!sample_temperature_ok(temperature)) return DFLASH_ERR_SHAPE;
  const dflash_config& c = m->cfg;
  const size_t need = align256((size_t)dfl::gumbel_chunks(c.vocab) * rows * 8);
  if (ws_bytes < need) return DFLASH_ERR_WORKSPACE;
  dfl::GumbelParams g{};
  std::memset(&g, 0, sizeof(g));
  g.z = logits;
  g.row0 = row0;
  g.B = 2;
  g.V = c.vocab;
  g.items = rows;
  g.chunks = dfl::gumbel_chunks(c.vocab);
  g.inv_t = 1.0f / temperature;
  g.seed_lo = (uint32_t)seed;
  g.seed_hi = (uint32_t)(seed >> 32);
  g.step = (uint32_t)step;
  g.keys = static_cast<unsigned long long*>(ws);
  g.out = tokens;
  return hip_status(dfl::launch_gumbel(g, 0, as_stream(stream)));
}

dflash_status dflash_verify_sample(const dflash_model* m, const dflash_kv* kv, const int32_t* draft,
                                   const float* draft_logits, const float* target_logits, float temperature,
                                   uint64_t seed, int32_t step, const int32_t* step_dev, const int32_t* stop_ids,
                                   int32_t n_stop,
                                   int32_t* budget, int32_t* accept_len, int32_t* anchor_out, int32_t* emitted,
                                   int32_t* n_emit, int32_t* done, int32_t* commit_rows, int32_t* n_commit,
                                   void* ws, size_t ws_bytes, void* stream) {
  if (!m) return DFLASH_ERR_NULL;
  if (m->target) return DFLASH_ERR_UNSUPPORTED;
  dflash_status ks = check_kv(m, kv);
  if (ks != DFLASH_OK) return ks;
  if (!draft || !draft_logits || !target_logits || !accept_len || !anchor_out || !emitted || !n_emit || !done ||
      !commit_rows || !n_commit || !ws)
    return DFLASH_ERR_NULL;
  if (n_stop < 0) return DFLASH_ERR_SHAPE;
  if (n_stop > 0 && !stop_ids) return DFLASH_ERR_NULL;
  if (!sample_temperature_ok(temperature)) return DFLASH_ERR_SHAPE;
  const dflash_config& c = m->cfg;
  const int batch = kv->batch, B = c.block;
  const SampleWs sw = sample_ws(c, batch);
  if (ws_bytes < sw.total) return DFLASH_ERR_WORKSPACE;
  const hipStream_t st = as_stream(stream);
  char* base = static_cast<char*>(ws);
  float* pmax = reinterpret_cast<float*>(base + sw.pmax);
  float* psum = reinterpret_cast<float*>(base + sw.psum);
  const int chunks = dfl::sample_chunks(c.vocab);
  int32_t* a = reinterpret_cast<int32_t*>(base + sw.a);
  int32_t* mm = reinterpret_cast<int32_t*>(base + sw.m);
  int32_t* rej = reinterpret_cast<int32_t*>(base + sw.rej);
  prof::Scope ps(DFLASH_PHASE_VERIFY, st);
  dfl::LseParams lp{};
  lp.z0 = draft_logits;
  lp.z1 = target_logits;
  lp.rows0 = batch * (B - 1);
  lp.rows1 = batch * B;
  lp.V = c.vocab;
  lp.chunks = chunks;
  lp.inv_t = 1.0f / temperature;
  lp.pmax = pmax;
  lp.psum = psum;
  hipError_t e = dfl::launch_lse(lp, st);
  if (e != hipSuccess) return DFLASH_ERR_HIP;
  dfl::AcceptParams ap{};
  ap.draft = draft;
  ap.zd = draft_logits;
  ap.zt = target_logits;
  ap.pmax = pmax;
  ap.psum = psum;
  ap.rows_d = batch * (B - 1);
  ap.chunks = chunks;
  ap.batch = batch;
  ap.B = B;
  ap.V = c.vocab;
  ap.inv_t = lp.inv_t;
  ap.seed_lo = (uint32_t)seed;
  ap.seed_hi = (uint32_t)(seed >> 32);
  ap.step = (uint32_t)step;
  ap.step_dev = step_dev;
  ap.a = a;
  ap.m = mm;
  ap.rejected = rej;
  if ((e = dfl::launch_accept(ap, st)) != hipSuccess) return DFLASH_ERR_HIP;
  dfl::GumbelParams g{};
  std::memset(&g, 0, sizeof(g));
  g.zd = draft_logits;
  g.zt = target_logits;
  g.pmax = pmax;
  g.psum = psum;
  g.rows_d = ap.rows_d;
  g.lse_chunks = chunks;
  g.m = mm;
  g.rejected = rej;
  g.B = B;
  g.V = c.vocab;
  g.items = batch;
  g.chunks = dfl::gumbel_chunks(c.vocab);
  g.inv_t = lp.inv_t;
  g.seed_lo = ap.seed_lo;
  g.seed_hi = ap.seed_hi;
  g.step = ap.step;
  g.step_dev = step_dev;
  g.keys = reinterpret_cast<unsigned long long*>(base + sw.keys);
  g.a = a;
  if ((e = dfl::launch_gumbel(g, 1, st)) != hipSuccess) return DFLASH_ERR_HIP;
  // the greedy rule on (draft, a) yields the sampled outcome: a holds the
  // accepted drafts and then the new token, which never equals the rejected
  // draft (the residual is zero there)
  dfl::VerifyParams p;
  p.draft = draft;
  p.target = a;
  p.stop_ids = stop_ids;
  p.n_stop = n_stop;
  p.budget = budget;
  p.ctx_len = kv->ctx_len;
  p.status = kv->status;
  p.batch = batch;
  p.B = B;
  p.accept_len = accept_len;
  p.anchor_out = anchor_out;
  p.emitted = emitted;
  p.n_emit = n_emit;
  p.done = done;
  p.commit_rows = commit_rows;
  p.n_commit = n_commit;
  return hip_status(dfl::launch_verify(p, st));
}

dflash_status dflash_pack_matrix(const void* src, void* dst, int32_t rows, int32_t cols, void* stream) {
  if (!src || !dst) return DFLASH_ERR_NULL;
  if (rows <= 0 || cols <= 0 || rows % 16 || cols % 32) return DFLASH_ERR_SHAPE;
  if (src == dst) return DFLASH_ERR_SHAPE;
  return hip_status(dfl::launch_pack(static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst), rows,
                                     cols, as_stream(stream)));
}

dflash_status dflash_profile_enable(uint32_t phase_mask) {
  prof::mask = phase_mask;
  prof::paused = false;
  if (phase_mask) prof::used = 0;
  return DFLASH_OK;
}

dflash_status dflash_profile_pause(int32_t paused) {
  prof::paused = paused != 0;
  return DFLASH_OK;
}

dflash_status dflash_profile_read(int32_t phase, double* total_ms, int32_t* launches) {
  if (!total_ms || !launches) return DFLASH_ERR_NULL;
  if (phase < 0 || phase >= DFLASH_N_PHASES) return DFLASH_ERR_SHAPE;
  double t = 0.0;
  int n = 0;
  for (size_t i = 0; i < prof::used; ++i) {
    const prof::Rec& r = prof::recs[i];
    if (r.phase != phase) continue;
    if (hipEventSynchronize(r.b) != hipSuccess) return DFLASH_ERR_HIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return DFLASH_ERR_HIP;
    t += ms;
    ++n;
  }
  *total_ms = t;
  *launches = n;
  return DFLASH_OK;
}

}  // extern "C"

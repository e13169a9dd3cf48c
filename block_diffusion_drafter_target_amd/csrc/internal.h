// Host-visible launch parameters and launchers of the gfx950 kernels. Used by
// the C ABI implementation (api.cpp); not part of the public interface.
#pragma once

#include <dflash.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dfl {

// The draft-block pass of dflash_draft_block (api.cpp), shared with the
// allocation-free entry point. draft_block_check runs every host-side check
// and returns the workspace the pass needs through *ws_need; draft_block_run
// enqueues the pass on a workspace of ws_bytes (no event timing when
// no_events is set).
dflash_status draft_block_check(const dflash_model* m, const dflash_kv* kv, const int32_t* anchor,
                                const int32_t* draft, size_t* ws_need);
dflash_status draft_block_run(const dflash_model* m, dflash_kv* kv, const int32_t* anchor, int32_t* draft,
                              float* dbg_logits, float* dbg_hidden, void* ws, size_t ws_bytes, void* stream,
                              bool no_events);

constexpr int kMaxZ = 16;       // weight matrices batched in one GEMM launch
constexpr int kMaxLayers = 16;  // draft layers supported

// Y = A * W^T, bf16 in, fp32 accumulate. W matrices are in the packed
// fragment layout (pack.hip). Rows n < n_split of the logical W come from
// W0[z] (row n), rows n >= n_split from W1[z] (row n - n_split); in swiglu
// mode W0 holds the gate rows and W1 the up rows of the N output columns.
struct GemmParams {
  const uint16_t* A;  // [M, K] activations, row stride lda
  long long lda;
  // optional row gather: GEMM row m reads A row a_idx[m * a_idx_stride],
  // clamped to [0, a_idx_max)
  const int32_t* a_idx;
  int a_idx_stride, a_idx_max;
  const uint16_t* W0[kMaxZ];
  const uint16_t* W1[kMaxZ];
  long long ldw;
  int n_split;
  int M, N, K;
  int k_per_split;  // k range of one split (multiple of 128)
  int splits;
  int n_mats;       // weight matrices batched in one launch (W0[z], W1[z], z < n_mats)
  // partial-sum output: P[z][s][m][n], fp32
  float* P;
  long long p_z_stride, p_s_stride;
  // argmax output (splits == 1): keys[tile * ld_keys + m] = max over the
  // column tile's n of argmax_key(y[m][n], n)
  unsigned long long* keys;
  long long ld_keys;
  float* dbg;  // optional logits [M, ld_dbg]
  long long ld_dbg;
  // swiglu output (splits == 1): out[m][n] = bf16(silu(gate) * up)
  uint16_t* out;
  long long ld_out;
  // optional row scale (the RMSNorm of A applied after the product; the
  // weight-streaming kernel in SwiGLU mode only): gate and up products of row
  // m are multiplied by 1 / sqrt(sum_{c < rs_n} rs[m * kMaxRowChunks + c] /
  // rs_len + rs_eps) before the SwiGLU; rs_n <= kMaxRowChunks
  const float* rs;
  int rs_n, rs_len;
  float rs_eps;
};

// Column chunks of the split RMSNorm (row_norm with ssp set): kRowChunkCols
// columns each, rows of up to kMaxRowChunks chunks.
constexpr int kRowChunkCols = 256;
constexpr int kMaxRowChunks = 32;

enum GemmMode { kGemmPartial = 0, kGemmArgmax = 1, kGemmSwiglu = 2 };

// Packs a row-major bf16 matrix [rows, cols] (rows % 16 == 0, cols % 32 == 0)
// into the fragment layout used by the weight-streaming GEMM.
hipError_t launch_pack(const uint16_t* src, uint16_t* dst, int rows, int cols, hipStream_t st);

hipError_t launch_gemm_stream(const GemmParams& p, int mt, int nf, int mode, int nz,
                              hipStream_t st);

// Tiled variant for M > 64 (128 x 128 tiles, one launch over all rows;
// K >= 128, k_per_split a multiple of 128). Argmax keys: one per 128-column
// tile.
// Tiled kernel: ng weight row groups per wave (64*ng columns per workgroup),
// mt 16-row activation tiles per workgroup; (ng, mt) in {1, 2} x {4, 8}.
hipError_t launch_gemm_tile(const GemmParams& p, int ng, int mt, int mode, int nz, hipStream_t st);

// The same tiles with weights three slabs ahead of the MFMAs and activations
// through registers into an LDS ring (gemm_ws.hip). (ng, mt) in {1, 2} x {4, 8}.
hipError_t launch_gemm_ws(const GemmParams& p, int ng, int mt, int mode, int nz, hipStream_t st);

// Large-tile variant (bm x bn tiles of 8 waves: 256 x 256 in every mode,
// 128 x 256 and 128 x 128 for split-K partials, 256 x 192 for the SwiGLU; both
// operands staged through LDS by direct loads; K and k_per_split multiples of
// 32). Argmax keys: one per gemm_big_cols(mode, bn) columns; SwiGLU and argmax
// take one split.
hipError_t launch_gemm_big(const GemmParams& p, int mode, int nz, int bm, int bn, hipStream_t st);
int gemm_big_cols(int mode, int bn);

// out[m][c] = bf16(silu(g) * u), g and u the split sums of P[s][m][c] and
// P[s][m][n + c] (gate and up partials of a split SwiGLU GEMM).
struct SwigluCombineParams {
  const float* P;
  long long p_s_stride;
  int splits, rows, n;
  uint16_t* out;
  long long ld_out;
};
hipError_t launch_swiglu_combine(const SwigluCombineParams& p, hipStream_t st);

struct AttnParams {
  const uint16_t* q;  // [batch*B, Hq, D]
  const uint16_t* k;  // layer base: [batch][Hkv][max_ctx][D]
  const uint16_t* v;
  const int32_t* ctx_len;
  const int32_t* status;
  int batch, Hq, Hkv, B, max_ctx;
  int n_ranges;  // chunk workgroups per kv head (grid x, >= batch)
  int slots;     // partial slots per kv head (>= n_ranges; slot = chunk number)
  const int32_t* plan;  // the batch's chunk split (attn_split.h), written earlier in the pass
  int causal;    // 0: every block row sees all L_b + B keys; 1: block row j sees keys < L_b + j + 1
  int slice;     // keys per LDS slice (64)
  int gb_pad;    // query rows per (b, g), padded to 16
                 // (q carries the softmax scale in base 2, log2(e) / sqrt(D): the
                 // scores come out of the MFMAs as s * c)
  float* pm;   // [Hkv][slots][gb_pad]
  float* pl;
  float* po;   // [Hkv][slots][gb_pad][D]
};

hipError_t launch_attention(const AttnParams& p, int D, hipStream_t st);

struct MergeParams {
  const float* pm;
  const float* pl;
  const float* po;
  const int32_t* ctx_len;
  const int32_t* status;
  int batch, Hq, Hkv, B, D, n_ranges, slots, gb_pad;
  int seg_hint;   // typical chunks per sequence (picks how many partials one load batch reads)
  const int32_t* plan;  // the batch's chunk split (attn_split.h)
  uint16_t* out;  // [batch*B, Hq*D]
};

hipError_t launch_attn_merge(const MergeParams& p, hipStream_t st);

// Row-wise RMSNorm with optional residual add of split partials.
//   x[m] (fp32, [rows, n]) += sum_s P[s][m] when residual; else y = sum_s P[s][m]
//   out[m] = bf16(rmsnorm(x or y) * gain)
// Final mode: rows j >= 1 of each block go to out[b*(B-1)+j-1]; row j == 0
// writes nothing.
struct RowNormParams {
  float* x;            // residual stream or NULL
  const float* P;      // partials [splits][rows][n] or NULL
  long long p_s_stride;
  int splits;
  const uint16_t* gain;
  float eps;
  int rows, n;
  uint16_t* out;       // bf16 [rows, n] (or [batch*(B-1), n] in final mode)
  float* dbg;          // optional fp32 copy of x after the add, [rows, n]
  uint16_t* tap;       // optional bf16 copy of x after the add, row stride tap_ld
  long long tap_ld;
  int final_mode, B;   // final_mode 1: out holds rows j >= 1 of every B-row sequence only
  // Split form (few rows whose consumer is the weight-streaming GEMM): when
  // set, out[row] = bf16(x * gain) without the 1/rms factor, and
  // ssp[row * ss_chunks + c] = the sum of squares of x over column chunk c
  // (kRowChunkCols columns; ss_chunks = ceil(n / kRowChunkCols)); the GEMM
  // applies the factor through its row scale. Row stride kMaxRowChunks
  // floats; row = the output row.
  float* ssp;
  int ss_chunks;
};

hipError_t launch_row_norm(const RowNormParams& p, hipStream_t st);

struct EmbedParams {
  const int32_t* anchor;  // row 0 of every sequence (rows 1..B-1: mask_id), or
  const int32_t* tokens;  // every row's token [batch, B] when not NULL
  const uint16_t* embed;
  const uint16_t* gain;
  int32_t* ctx_len;
  int32_t* status;
  int batch, B, H, V, mask_id, max_ctx, rope_max;
  float eps;
  float* x;        // [batch*B, H]
  uint16_t* u;     // [batch*B, H]
  float* dbg;      // optional [batch*B, H]
  // split form (as RowNormParams::ssp): u = bf16(x * gain), the chunk sums of
  // squares in ssp [batch*B][kMaxRowChunks]
  float* ssp;
  int ss_chunks;
};

hipError_t launch_embed(const EmbedParams& p, hipStream_t st);

struct QkvPostParams {
  const float* P;  // [splits][rows][(Hq+2Hkv)*D]
  long long p_s_stride;
  int splits;
  const uint16_t* gq;
  const uint16_t* gk;
  const float* rope;  // [rope_max][D/2][2]
  int rope_max;
  const int32_t* ctx_len;
  const int32_t* status;
  int batch, B, Hq, Hkv, D, max_ctx;
  float eps;
  uint16_t* q;        // [rows, Hq, D], multiplied by q_scale before rounding
  float q_scale;      // log2(e) / sqrt(D): the attention scores in base 2
  uint16_t* kc;       // layer base [batch][Hkv][max_ctx][D]
  uint16_t* vc;
  int32_t* plan;      // if not NULL, one more workgroup writes the attention chunk split
  int n_ranges, slice;  // of the batch (attn_split.h) with n_ranges chunks per kv head
  // optional row scale of the split RMSNorm that wrote the GEMM's input: the
  // split sums of row m are multiplied by 1 / sqrt(sum_{c < rs_n}
  // rs[m * kMaxRowChunks + c] / rs_len + rs_eps) (as in GemmParams)
  const float* rs;
  int rs_n, rs_len;
  float rs_eps;
};

hipError_t launch_qkv_post(const QkvPostParams& p, hipStream_t st);

struct InjectPostParams {
  const float* P;  // [layer][split][c1 - c0][2*Hkv*D], row = commit index - c0
  long long p_z_stride, p_s_stride;
  int splits;
  const uint16_t* gk[kMaxLayers];
  const float* rope;
  int rope_max;
  const int32_t* commit_rows;
  const int32_t* n_commit;
  int max_commit, n_ctx_rows;
  int c0, c1;  // commit indices handled by this launch
  int n_layers, batch, Hkv, D, max_ctx;
  float eps;
  uint16_t* kc;  // [NL][batch][Hkv][max_ctx][D]
  uint16_t* vc;
  int32_t* ctx_len;
  int32_t* status;
};

hipError_t launch_inject_post(const InjectPostParams& p, hipStream_t st);

// draft[b][j-1] = index of max over tiles of keys[tile * (batch*(B-1)) + row],
// row = b*(B-1) + j-1; -1 for a sequence whose status is nonzero.
hipError_t launch_argmax_finish(const unsigned long long* keys, int n_tiles, const int32_t* status,
                                int batch, int rows_per_seq, int32_t* out, hipStream_t st);

// ctx_len[seq] = max(ctx_len[seq], pos + 1) for the first min(n_commit, max_commit)
// commit rows (src, seq, pos) with a valid seq and 0 <= pos < max_ctx.
hipError_t launch_kv_commit(const int32_t* commit_rows, const int32_t* n_commit, int max_commit, int batch,
                            int max_ctx, int32_t* ctx_len, hipStream_t st);

// On-device loop (loop.hip). tokens[b] = [anchor[b], draft[b][0..B-2]].
// commit_rows[i] = (i, seq, start + i) for i < n, *n_commit = n (loop.hip).
hipError_t launch_ingest_rows(int32_t* commit_rows, int32_t* n_commit, int seq, int start, int n, hipStream_t st);
hipError_t launch_loop_tokens(const int32_t* anchor, const int32_t* draft, int32_t* tokens, int batch, int B,
                              hipStream_t st);

// End of a loop step, per sequence b: while alive[b], the first n_emit[b]
// emitted tokens go to out[b][cursor[b] + i] (positions below max_new only)
// and cursor[b] += n_emit[b]; alive[b] drops once done[b] is set; anchor[b] =
// anchor_out[b]; *step_dev += 1 when step_dev is not NULL.
struct LoopAdvanceParams {
  const int32_t* anchor_out;
  const int32_t* emitted;  // [batch, B]
  const int32_t* n_emit;
  const int32_t* done;
  int32_t* out;            // [batch, ld_out]
  long long ld_out;
  int max_new;
  int32_t* cursor;
  int32_t* alive;
  int32_t* anchor;
  int32_t* step_dev;
  int batch, B;
};
hipError_t launch_loop_advance(const LoopAdvanceParams& p, hipStream_t st);

struct VerifyParams {
  const int32_t* draft;
  const int32_t* target;
  const int32_t* stop_ids;
  int n_stop;
  int32_t* budget;
  const int32_t* ctx_len;
  const int32_t* status;
  int batch, B;
  int32_t* accept_len;
  int32_t* anchor_out;
  int32_t* emitted;
  int32_t* n_emit;
  int32_t* done;
  int32_t* commit_rows;
  int32_t* n_commit;
};

hipError_t launch_verify(const VerifyParams& p, hipStream_t st);

// Sampling mode (sample.hip). Per-chunk log-sum-exp pairs of z * inv_t for the
// rows0 rows of z0 followed by the rows1 rows of z1 (each row V floats):
// pmax[row][chunk] and psum[row][chunk] (sample_chunks(V) chunks per row).
struct LseParams {
  const float* z0;
  const float* z1;
  int rows0, rows1, V, chunks;
  float inv_t;
  float* pmax;
  float* psum;
};
hipError_t launch_lse(const LseParams& p, hipStream_t st);

// Acceptance walk per sequence: accepted drafts into a[b][j-1], the count m[b]
// and rejected[b] (0: every draft passed).
struct AcceptParams {
  const int32_t* draft;  // [batch, B-1]
  const float* zd;       // draft logits [batch*(B-1), V]
  const float* zt;       // target logits [batch*B, V]
  const float* pmax;     // log-sum-exp pairs: draft rows, then target rows from rows_d
  const float* psum;
  int rows_d, chunks;
  int batch, B, V;
  float inv_t;
  uint32_t seed_lo, seed_hi, step;
  const int32_t* step_dev;  // or NULL: the draws' step is step + *step_dev
  int32_t* a;  // [batch, B]
  int32_t* m;
  int32_t* rejected;
};
hipError_t launch_accept(const AcceptParams& p, hipStream_t st);

// Gumbel-max sampling over the vocabulary in sample_chunks(V) chunks per item.
// mode 0: items = LM rows of z, RNG rows row0 + item, out[item] = token (-1
// where status of the item's sequence, item / (B-1), is nonzero);
// mode 1: items = sequences, the residual (rejected) or bonus sample written to
// a[item][m[item]].
struct GumbelParams {
  const float* z;
  int row0;
  const float* zd;
  const float* zt;
  const float* pmax;  // log-sum-exp pairs as in AcceptParams
  const float* psum;
  int rows_d, lse_chunks;
  const int32_t* m;
  const int32_t* rejected;
  int B, V, items, chunks;
  float inv_t;
  uint32_t seed_lo, seed_hi, step;
  const int32_t* step_dev;  // or NULL: the draws' step is step + *step_dev
  unsigned long long* keys;  // [chunks, items], chunks = gumbel_chunks(V)
  int32_t* out;
  const int32_t* status;
  int32_t* a;
};
int sample_chunks(int V);  // log-sum-exp chunks per row
int gumbel_chunks(int V);  // Gumbel-argmax chunks per item (keys)
hipError_t launch_gumbel(const GumbelParams& p, int mode, hipStream_t st);

}  // namespace dfl

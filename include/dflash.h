/*
 * dflash.h — C ABI of the MI355X (gfx950) library for one DFlash-style draft
 * step: fuse target taps into a context feature, inject it into every draft
 * layer's KV cache, denoise a masked block in one forward pass, and accept the
 * longest verified prefix with KV commit / rollback.
 *
 * Sources (prose only; none gives equations):
 *   [P1] "DFlash: slik kan spekulativ dekoding gi opptil 6x raskere
 *        AI-inferens", jansverre.net/?p=12023
 *   [P2] DFlash news article, news.bpdata.com (address slug
 *        "dflash-block-diffuzios-spekulativ-dekodolassal-akar-15")
 *   [P3] "DFlash Crea Blocchi Interi di Token Contemporaneamente, Aumentando
 *        Fino a 15x la Velocità su NVIDIA Blackwell", theaistack.guide
 *   [P4] DFlash news article, 7minutos.es, 2026-06-26
 *
 * Conventions for every call
 *   - bf16 tensors are 16-bit brain-float bit patterns, row-major, densely
 *     packed unless a leading dimension is given. Matrices are [out, in].
 *   - "device" pointers are GPU memory owned by the caller (for example torch
 *     tensors); "host" pointers are CPU memory. The library never allocates,
 *     frees or retains device memory, and never synchronises the stream.
 *   - stream is a hipStream_t passed as void*; NULL means the null stream.
 *     Work is enqueued asynchronously on it; all calls that share a dflash_kv
 *     must use one stream (or be ordered by the caller).
 *   - Argument checks that need no GPU run first and return an error before
 *     any HIP call. Errors of kernel launch return DFLASH_ERR_HIP. Conditions
 *     only visible on the device (a context that would overflow the cache) are
 *     reported per sequence in dflash_kv.status, and that sequence is skipped.
 *   - No C++ exception crosses this boundary.
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dflash_status {
  DFLASH_OK = 0,
  DFLASH_ERR_NULL = -1,        /* a required pointer is NULL */
  DFLASH_ERR_SHAPE = -2,       /* a size is out of range or inconsistent */
  DFLASH_ERR_UNSUPPORTED = -3, /* a shape the kernels do not implement */
  DFLASH_ERR_WORKSPACE = -4,   /* workspace too small */
  DFLASH_ERR_CAPACITY = -5,    /* per-sequence: positions beyond max_ctx or the RoPE table */
  DFLASH_ERR_HIP = -6          /* a HIP launch failed */
} dflash_status;

/* Drafter shape. Requirements checked at create: hidden, intermediate,
 * n_q_heads*head_dim and n_tap*hidden multiples of 64; head_dim 64 or 128;
 * n_q_heads a multiple of n_kv_heads; 2 <= block <= 16; 1 <= n_layers <= 16;
 * 0 <= mask_id < vocab. */
typedef struct dflash_config {
  int32_t hidden;       /* H */
  int32_t n_layers;     /* NL */
  int32_t n_q_heads;    /* Hq */
  int32_t n_kv_heads;   /* Hkv */
  int32_t head_dim;     /* D */
  int32_t intermediate; /* I (SwiGLU) */
  int32_t vocab;        /* V */
  int32_t n_tap;        /* number of tapped target layers */
  int32_t block;        /* B: block rows per sequence (anchor + B-1 masks) */
  int32_t mask_id;      /* token id that fills block rows 1..B-1 */
  float rope_theta;
  float rms_eps;
} dflash_config;

/* One draft layer; all device bf16. Matrices are [out, in] in the packed
 * fragment layout written by dflash_pack_matrix; gains are plain vectors.
 *   g_in [H], g_post [H], g_q [D], g_k [D]     RMSNorm gains
 *   w_qkv [(Hq+2Hkv)*D, H]  rows: q heads, then k heads, then v heads
 *   w_o   [H, Hq*D]
 *   w_gate, w_up [I, H]
 *   w_down [H, I] */
typedef struct dflash_layer_weights {
  const void* g_in;
  const void* w_qkv;
  const void* g_q;
  const void* g_k;
  const void* w_o;
  const void* g_post;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
} dflash_layer_weights;

/* Whole drafter; device pointers unless noted.
 *   embed [V, H] bf16 row-major; lm_head [V, H] bf16 packed (the target's
 *         embedding and head, shared)
 *   w_fc [H, n_tap*H] bf16 packed, columns tap-major; g_fc [H], g_final [H]
 *   layers: HOST array of n_layers entries (copied at create)
 *   rope: device fp32 [rope_max_pos, D/2, 2] = (cos, sin) of pos*theta^(-2i/D),
 *         as written by dflash_rope_table. */
typedef struct dflash_weights {
  const void* embed;
  const void* lm_head;
  const void* w_fc;
  const void* g_fc;
  const void* g_final;
  const dflash_layer_weights* layers;
  const float* rope;
  int32_t rope_max_pos;
} dflash_weights;

/* Draft KV cache of a batch of sequences; device memory.
 *   k, v   bf16 [NL][batch][Hkv][max_ctx][D]
 *   ctx_len int32 [batch]: committed context length L_b. Only inject_kv
 *          advances it, so block slots written speculatively by draft_block
 *          are dead until a commit overwrites them (rollback by construction).
 *   status  int32 [batch]: 0, or DFLASH_ERR_CAPACITY set by the device. */
typedef struct dflash_kv {
  void* k;
  void* v;
  int32_t batch;
  int32_t max_ctx;
  int32_t* ctx_len;
  int32_t* status;
} dflash_kv;

typedef struct dflash_model dflash_model;

/* Check the shape, copy the layer table, and keep the (borrowed) weight
 * pointers; they must outlive the model. Host only: no HIP call. */
dflash_status dflash_model_create(const dflash_config* cfg, const dflash_weights* w,
                                  dflash_model** out);
void dflash_model_destroy(dflash_model* m);

/* Host helper: cos/sin table for RoPE, computed in double and rounded to
 * float. out: host float[max_pos * head_dim/2 * 2]. */
dflash_status dflash_rope_table(float* out, int32_t max_pos, int32_t head_dim, float theta);

/* Packed fragment layout of a weight matrix. src: device bf16 row-major
 * [rows, cols]; dst: device bf16, same size, not overlapping src. rows must be
 * a multiple of 16 and cols of 32. The 16-row x 32-column block (rg, kc) of W
 * is stored contiguously (1 KB) at block index rg*(cols/32) + kc, element
 *   dst[((rg*(cols/32) + kc)*64 + 16*g + r)*8 + e] = W[16*rg + r][32*kc + 8*g + e]
 * for r < 16, g < 4, e < 8: the operand order of the 16x16x32 bf16 MFMA, so a
 * wavefront reads one block with one fully used 1 KB load. Enqueued on
 * stream. */
dflash_status dflash_pack_matrix(const void* src, void* dst, int32_t rows, int32_t cols,
                                 void* stream);

/* Workspace (device scratch, caller-allocated) needed by calls that handle up
 * to max_batch sequences, a cache of max_ctx slots and up to max_rows context
 * rows per fuse/inject call; for a target model, by a dflash_target_forward of
 * any n <= block (max_rows unused). */
size_t dflash_workspace_bytes(const dflash_model* m, int32_t max_batch, int32_t max_ctx,
                              int32_t max_rows);

/* S1 — context-feature fusion. [P3 "L'idea chiave: Il target sa meglio";
 * P4 "La idea de que 'el objetivo sabe más'"]: the hidden states of several
 * target layers are merged into one compact context feature.
 *   taps  device bf16 [n_rows, n_tap*H], taps of one row layer-major
 *   ctx   device bf16 [n_rows, H] out: RMSNorm(W_fc taps_r; g_fc)
 * n_rows >= 0 (0 is a no-op). */
dflash_status dflash_fuse_ctx(const dflash_model* m, const void* taps, int32_t n_rows, void* ctx,
                              void* ws, size_t ws_bytes, void* stream);

/* S2 — KV injection. [P3 "L'idea chiave: Il target sa meglio"; P4 "La idea
 * de que 'el objetivo sabe más'"; P1 "Hva gjør DFlash annerledes enn vanlig
 * spekulativ dekoding?"]: the context feature enters the key and value
 * projections of every draft layer and stays in the draft KV cache.
 * For every layer l and commit row i < *n_commit (device count):
 *   (src, seq, pos) = commit_rows[i]
 *   K^l[seq][g][pos] = RoPE(RMSNorm_head(W_k^l ctx[src]; g_k^l), pos)
 *   V^l[seq][g][pos] = W_v^l ctx[src]
 *   ctx_len[seq] = max(ctx_len[seq], pos + 1)
 *   ctx          device bf16 [n_ctx_rows, H]
 *   commit_rows  device int32 [max_commit, 3]
 *   n_commit     device int32 [1], clamped to [0, max_commit]
 * A row with src, seq or pos out of range is skipped; out-of-range pos also
 * sets status[seq] = DFLASH_ERR_CAPACITY. n_ctx_rows * H above 2^31 - 1
 * returns DFLASH_ERR_UNSUPPORTED (rows are addressed with 32-bit offsets). */
dflash_status dflash_inject_kv(const dflash_model* m, const void* ctx, int32_t n_ctx_rows,
                               const int32_t* commit_rows, const int32_t* n_commit,
                               int32_t max_commit, dflash_kv* kv, void* ws, size_t ws_bytes,
                               void* stream);

/* S3–S10 — one denoising pass over the masked block. [P1 "Hva gjør DFlash
 * annerledes enn vanlig spekulativ dekoding?"; P3 "Come funziona il drafting a
 * blocchi"; P2 "Hogyan működik a DFlash spekulatív dekódolás?"]
 * Row j of sequence b sits at position L_b + j and holds anchor[b] (j = 0) or
 * mask_id (j >= 1). Each layer appends the block's K/V at slots
 * [L_b, L_b + B) and attends, unmasked, over slots [0, L_b + B).
 *   anchor     device int32 [batch]
 *   draft      device int32 [batch, B-1] out: argmax of rows 1..B-1,
 *              lowest index on ties
 *   dbg_logits device fp32 [batch*(B-1), V] or NULL
 *   dbg_hidden device fp32 [NL+1, batch*B, H] or NULL: residual stream after
 *              the embedding and after each layer
 * status[b] is set to DFLASH_ERR_CAPACITY when L_b + B exceeds max_ctx or the
 * RoPE table; that sequence's draft is then filled with -1. */
dflash_status dflash_draft_block(const dflash_model* m, dflash_kv* kv, const int32_t* anchor,
                                 int32_t* draft, float* dbg_logits, float* dbg_hidden, void* ws,
                                 size_t ws_bytes, void* stream);

/* Allocation-free draft block, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Same pass, arguments (without ws), outputs, cache effects and
 * status rules as dflash_draft_block; the workspace is a static device array
 * of DFLASH_NOALLOC_SCRATCH_BYTES inside the library, one copy per GPU that
 * the library runs on, held until the process ends. The call uses the current
 * device's copy (stream must belong to that device) and calls nothing that
 * allocates (phase timing is skipped in it).
 *   Returns DFLASH_ERR_WORKSPACE, before any HIP call, when the pass needs more
 *   than DFLASH_NOALLOC_SCRATCH_BYTES (the draft-block part of
 *   dflash_workspace_bytes for kv->batch and kv->max_ctx; for example a
 *   Qwen3-8B-shaped drafter at batch 32 needs about 118 MiB).
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (the pass reads only what it wrote in the same call, so nothing
 * needs clearing). Calls that overlap on one GPU, from different streams or
 * threads, race on the array: the caller must order them. */
#define DFLASH_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
dflash_status dflash_draft_block_noalloc(const dflash_model* m, dflash_kv* kv, const int32_t* anchor,
                                         int32_t* draft, float* dbg_logits, float* dbg_hidden, void* stream);

/* Sampling mode, draft side (temperature > 0). [P4 "Ejecutando DFlash": the
 * user call takes a temperature; P2 results: speed-ups are quoted under
 * sampling too] The pages give no sampling rule; the plain reading is standard
 * speculative sampling, whose draft side samples every block token from the
 * drafter's own distribution at its position, q_j = softmax(z_j / T).
 * Runs the pass of dflash_draft_block (same inputs, cache effects and status
 * rules), writes the raw logits of rows 1..B-1 and replaces each greedy token
 * by a Gumbel-max sample: draft[b][j-1] = argmax_v z_v / T + g_v with
 * g_v = -log(-log u_v), u_v the Philox4x32-10 uniform of the draw
 * (seed, tag 0, step, row b*(B-1)+j-1, v) (see dflash_verify_sample).
 *   logits      device fp32 [batch*(B-1), V] out, required (the verify reads
 *               them)
 *   temperature > 0, finite (else DFLASH_ERR_SHAPE)
 *   seed, step  the draws' key and step counter (a new step per block keeps
 *               the draws of different steps independent)
 *   step_dev    device int32 [1] or NULL: the draws' step is step + *step_dev
 *               (a loop captured in a graph advances it on the device)
 * ws: dflash_workspace_bytes covers it. */
dflash_status dflash_draft_block_sample(const dflash_model* m, dflash_kv* kv, const int32_t* anchor,
                                        int32_t* draft, float* logits, float temperature, uint64_t seed,
                                        int32_t step, const int32_t* step_dev, void* ws, size_t ws_bytes,
                                        void* stream);

/* Sampling mode: Gumbel-max samples of softmax(logits / T) for `rows` rows of
 * the model's vocabulary width, the draw of row r being (seed, tag 0, step,
 * row0 + r) (see dflash_verify_sample), e.g. the first token after a prompt,
 * which comes from the target's last prompt row. [P4 "Ejecutando DFlash":
 * the call's temperature]
 *   logits  device fp32 [rows, V]; tokens device int32 [rows] out
 *   ws      at least 8 * ceil(V / 2048) * rows bytes (dflash_workspace_bytes
 *           covers rows <= batch * (block - 1)) */
dflash_status dflash_sample_logits(const dflash_model* m, const float* logits, int32_t rows, float temperature,
                                   uint64_t seed, int32_t step, int32_t row0, int32_t* tokens, void* ws,
                                   size_t ws_bytes, void* stream);

/* Sampling mode, verify side: standard speculative-sampling acceptance (the
 * plain reading; see dflash_draft_block_sample). With p_i = softmax(zt_i / T)
 * the target's distribution after block row i and q_j = softmax(zd_j / T):
 * draft d_j is accepted when u_j <= p_{j-1}(d_j) / q_j(d_j), for j = 1, 2, ...
 * until the first rejection; the first rejected position takes a token
 * sampled from the normalised max(0, p_{j-1} - q_j), and when all B-1 drafts
 * pass a bonus token is sampled from p_{B-1}. The emitted tokens are the
 * accepted drafts and the new token, cut by stop ids and budget, and rows
 * 0..m are committed, exactly as in dflash_verify_accept (same outputs).
 * Random numbers: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11), key =
 * (seed low word, high word), counter = (v / 4, row, step, tag), output word
 * v % 4, uniform ((word >> 9) + 0.5) * 2^-23. u_j: tag 1, row b*B + j, v 0;
 * the residual or bonus sample: Gumbel-max with tag 2, row b.
 *   draft_logits  device fp32 [batch*(B-1), V]: the drafter's rows 1..B-1
 *   target_logits device fp32 [batch*B, V]: the target's logits after rows
 *                 0..B-1 of [anchor, d_1..d_{B-1}]
 *   temperature   > 0, finite (else DFLASH_ERR_SHAPE)
 *   step_dev      device int32 [1] or NULL: the draws' step is step + *step_dev
 * ws: dflash_workspace_bytes covers it. ctx_len is read, never written. */
dflash_status dflash_verify_sample(const dflash_model* m, const dflash_kv* kv, const int32_t* draft,
                                   const float* draft_logits, const float* target_logits, float temperature,
                                   uint64_t seed, int32_t step, const int32_t* step_dev, const int32_t* stop_ids,
                                   int32_t n_stop,
                                   int32_t* budget, int32_t* accept_len, int32_t* anchor_out, int32_t* emitted,
                                   int32_t* n_emit, int32_t* done, int32_t* commit_rows, int32_t* n_commit,
                                   void* ws, size_t ws_bytes, void* stream);

/* S11 — greedy acceptance of the longest valid prefix. [P2 introduction: the
 * target checks the block in parallel and keeps the longest valid prefix;
 * P4 "Ejecutando DFlash" for stop tokens and the token budget]
 *   draft          device int32 [batch, B-1]  d_1..d_{B-1}
 *   target_argmax  device int32 [batch, B]    a_0..a_{B-1}
 *   stop_ids       device int32 [n_stop] (may be NULL if n_stop == 0)
 *   budget         device int32 [batch] in/out remaining tokens, or NULL
 * Outputs (device int32):
 *   accept_len [batch]  m_b = max k <= B-1 with d_j == a_{j-1} for all j <= k
 *   anchor_out [batch]  a_m
 *   emitted [batch, B]  a_0..a_m cut after the first stop id and to budget,
 *                       -1 padded; n_emit [batch]; done [batch] (0/1)
 *   commit_rows [batch*B, 3], n_commit [1]: (b*B + i, b, L_b + i) for
 *                       i = 0..m_b, sequences in order
 * ctx_len is read, never written (inject_kv commits). A sequence whose status
 * is nonzero emits and commits nothing and is reported done. */
dflash_status dflash_verify_accept(const dflash_model* m, const dflash_kv* kv,
                                   const int32_t* draft, const int32_t* target_argmax,
                                   const int32_t* stop_ids, int32_t n_stop, int32_t* budget,
                                   int32_t* accept_len, int32_t* anchor_out, int32_t* emitted,
                                   int32_t* n_emit, int32_t* done, int32_t* commit_rows,
                                   int32_t* n_commit, void* stream);

/* Target side of the step: a causal pass of the target model over n new
 * tokens per sequence. [P2 introduction and P3 introduction: the target
 * checks the whole drafted block in one parallel pass and keeps the longest
 * valid prefix; P3 "L'idea chiave: Il target sa meglio" and P4 "La idea de que
 * 'el objetivo sabe más'": the drafter is conditioned on hidden states of
 * several target layers, which this pass emits as taps]
 *
 * dflash_target_create builds a target model from the same config and weight
 * structs as the drafter: n_layers decoder layers of the drafter's layer shape
 * (up to 256), the shared embedding and LM head and g_final; w_fc and g_fc are
 * not used (may be NULL); block = the largest n per call (1..64, and
 * Hq/Hkv * block <= 256); n_tap tapped layers tap_layers[n_tap] (host array,
 * strictly increasing, in [0, n_layers)). Host only: no HIP call. The model
 * works with dflash_target_forward, dflash_kv_commit and
 * dflash_workspace_bytes only (the drafter entry points return
 * DFLASH_ERR_UNSUPPORTED for it), and is released with dflash_model_destroy. */
dflash_status dflash_target_create(const dflash_config* cfg, const dflash_weights* w,
                                   const int32_t* tap_layers, dflash_model** out);

/* One target pass over tokens[b][0..n) at positions L_b .. L_b+n-1 (L_b =
 * ctx_len[b]): token j attends to the cached slots [0, L_b) and to tokens
 * 0..j of the pass (causal), and its K/V are written to cache slots L_b + j of
 * every layer. ctx_len is not advanced: dflash_kv_commit keeps the accepted
 * prefix; the rest is rolled back by construction.
 *   tokens      device int32 [batch, n], 1 <= n <= block
 *   argmax      device int32 [batch, n]: greedy next token after each input
 *               token (lowest index on ties); -1 for a sequence whose status
 *               is nonzero
 *   taps        device bf16 [batch*n, n_tap*H] or NULL: the residual stream
 *               after each tapped layer, layer-major within a row (the layout
 *               dflash_fuse_ctx reads)
 *   dbg_logits  device fp32 [batch*n, V] or NULL
 * kv is the target's own cache ([NL][batch][Hkv][max_ctx][D] per dflash_kv).
 * Capacity (L_b + n > max_ctx) is reported per sequence in kv->status.
 * Workspace as in dflash_workspace_bytes of this model. */
dflash_status dflash_target_forward(const dflash_model* m, dflash_kv* kv, const int32_t* tokens,
                                    int32_t n, int32_t* argmax, void* taps, float* dbg_logits,
                                    void* ws, size_t ws_bytes, void* stream);

/* Commit rows whose K/V are already in the cache (a target pass wrote them):
 * for the first min(n_commit, max_commit) rows (src, seq, pos) of commit_rows
 * (device int32 [max_commit, 3], the layout dflash_verify_accept writes) with
 * 0 <= seq < batch and 0 <= pos < max_ctx, ctx_len[seq] grows to pos + 1.
 * [P2 introduction: the longest valid prefix is kept] */
dflash_status dflash_kv_commit(const dflash_model* m, dflash_kv* kv, const int32_t* commit_rows,
                               const int32_t* n_commit, int32_t max_commit, void* stream);

/* Commit rows of a context ingest: commit_rows[i] = (i, seq, start + i) for
 * i < n and *n_commit = n, the rows dflash_inject_kv takes to inject n fused
 * context rows of sequence seq at positions start .. start + n - 1 (the
 * context is injected as the target writes it, [P3 "L'idea chiave: Il
 * target sa meglio"]).
 *   commit_rows  device int32 [n, 3] out; n_commit device int32 [1] out
 * 0 <= seq < batch, start >= 0, n >= 0 and start + n <= max_ctx, else
 * DFLASH_ERR_SHAPE before any launch. */
dflash_status dflash_ingest_rows(const dflash_model* m, const dflash_kv* kv, int32_t seq, int32_t start, int32_t n,
                                 int32_t* commit_rows, int32_t* n_commit, void* stream);

/* On-device speculative loop: the two steps of the greedy loop that are
 * neither drafting, verification nor commit, so that a whole step (draft
 * block, target pass, verify, commits, fuse, inject, advance) runs without
 * host synchronisation and can be captured in a graph. [P4 "Ejecutando
 * DFlash": the user call generates up to a token budget with stop ids; P2
 * introduction: the target checks the drafted block and the longest valid
 * prefix is kept]
 *
 * dflash_loop_tokens: the target's input row of the step,
 *   tokens[b][0] = anchor[b], tokens[b][j] = draft[b][j-1] for 1 <= j < B
 *   anchor device int32 [batch]; draft device int32 [batch, B-1];
 *   tokens device int32 [batch, B] out. */
dflash_status dflash_loop_tokens(const dflash_model* m, const dflash_kv* kv, const int32_t* anchor,
                                 const int32_t* draft, int32_t* tokens, void* stream);

/* dflash_loop_advance: the end of a step, from dflash_verify_accept's (or
 * dflash_verify_sample's) outputs. For each sequence b with alive[b] != 0:
 *   out[b][cursor[b] + i] = emitted[b][i] for i < n_emit[b] and
 *   cursor[b] + i < max_new; cursor[b] += n_emit[b]; alive[b] = 0 once done[b];
 * for every sequence anchor[b] = anchor_out[b]; and *step_dev += 1 when
 * step_dev is not NULL (the step counter of the sampling mode's draws).
 *   out     device int32 [batch, ld_out], ld_out >= max_new >= 0
 *   cursor, alive, anchor  device int32 [batch], in/out
 * A sequence that is not alive is left as it is (cursor, output, flag). */
dflash_status dflash_loop_advance(const dflash_model* m, const dflash_kv* kv, const int32_t* anchor_out,
                                  const int32_t* emitted, const int32_t* n_emit, const int32_t* done, int32_t* out,
                                  int32_t ld_out, int32_t max_new, int32_t* cursor, int32_t* alive,
                                  int32_t* anchor, int32_t* step_dev, void* stream);

/* Kernel timing for benchmarks. dflash_profile_enable(mask) times the phases
 * whose bit (1 << phase) is set in mask (0 switches timing off): every launch
 * of such a phase is bracketed by two HIP events recorded on the call's
 * stream (hipEventCreate objects owned by the library; no device memory).
 * Process-wide, off by default, not thread-safe; enabling clears earlier
 * records.
 * dflash_profile_read waits for the recorded events and returns the summed
 * duration (ms) and the number of launches of one phase. */
typedef enum dflash_phase {
  DFLASH_PHASE_LM_HEAD = 0,   /* LM-head GEMM with fused argmax (S10) */
  DFLASH_PHASE_ATTENTION = 1, /* block attention kernel (S6, without the merge) */
  DFLASH_PHASE_QKV = 2,       /* q/k/v projection GEMM (S4) */
  DFLASH_PHASE_O = 3,         /* o projection GEMM (S7) */
  DFLASH_PHASE_GATE_UP = 4,   /* gate/up GEMM (S8) */
  DFLASH_PHASE_DOWN = 5,      /* down projection GEMM (S9) */
  DFLASH_PHASE_FUSE = 6,      /* fusion GEMM (S1) */
  DFLASH_PHASE_INJECT = 7,    /* injection GEMM (S2) */
  DFLASH_PHASE_VERIFY = 8,    /* verify kernel (S11) */
  DFLASH_PHASE_MERGE = 9,     /* log-sum-exp merge of the attention chunks (S6) */
  DFLASH_N_PHASES = 10
} dflash_phase;

dflash_status dflash_profile_enable(uint32_t phase_mask);
dflash_status dflash_profile_read(int32_t phase, double* total_ms, int32_t* launches);
/* dflash_profile_pause(1) stops recording events without clearing the records
 * or the mask, dflash_profile_pause(0) resumes: a benchmark times a sample of
 * the launches (every event pair recorded on the stream costs the stream a few
 * microseconds). Process-wide, not thread-safe; always DFLASH_OK. */
dflash_status dflash_profile_pause(int32_t paused);

const char* dflash_status_string(dflash_status s);

#ifdef __cplusplus
}
#endif
#endif /* DFLASH_H */

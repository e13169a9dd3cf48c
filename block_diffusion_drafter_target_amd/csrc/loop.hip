// Bookkeeping kernels of the on-device speculative loop (gfx950), integer
// only: the target's input row per sequence, the end-of-step update that
// appends the emitted tokens to the output and moves the cursor, the running
// flags, the anchors and the step counter (one wave per sequence), and the
// commit rows of a context ingest.
#include "common.h"
#include "internal.h"

namespace dfl {

namespace {

// tokens[b][0] = anchor[b], tokens[b][j] = draft[b][j - 1] for 1 <= j < B
__global__ __launch_bounds__(256) void loop_tokens_kernel(const int32_t* anchor, const int32_t* draft,
                                                          int32_t* tokens, int batch, int B) {
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6), j = threadIdx.x & 63;
  if (b >= batch || j >= B) return;
  tokens[b * B + j] = j == 0 ? anchor[b] : draft[b * (B - 1) + j - 1];
}

__global__ __launch_bounds__(256) void loop_advance_kernel(const LoopAdvanceParams p) {
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6), j = threadIdx.x & 63;
  if (blockIdx.x == 0 && threadIdx.x == 0 && p.step_dev) p.step_dev[0] += 1;
  if (b >= p.batch) return;
  const int alive = p.alive[b];
  const int n = alive ? p.n_emit[b] : 0;
  const int cur = p.cursor[b];
  if (j < p.B && j < n && cur + j < p.max_new) p.out[(long long)b * p.ld_out + cur + j] = p.emitted[b * p.B + j];
  if (j == 0) {
    // every lane of the wave has read cursor[b] above (the loads have
    // returned before the stores they feed are issued)
    p.cursor[b] = cur + n;
    p.alive[b] = alive && !p.done[b] ? 1 : 0;
    p.anchor[b] = p.anchor_out[b];
  }
}

// commit_rows[i] = (i, seq, start + i) for i < n, *n_commit = n
__global__ __launch_bounds__(256) void ingest_rows_kernel(int32_t* commit_rows, int32_t* n_commit, int seq, int start,
                                                          int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i == 0) n_commit[0] = n;
  if (i >= n) return;
  commit_rows[3 * i] = i;
  commit_rows[3 * i + 1] = seq;
  commit_rows[3 * i + 2] = start + i;
}

}  // namespace

hipError_t launch_ingest_rows(int32_t* commit_rows, int32_t* n_commit, int seq, int start, int n, hipStream_t st) {
  hipLaunchKernelGGL(ingest_rows_kernel, dim3(n > 0 ? (n + 255) / 256 : 1), dim3(256), 0, st, commit_rows, n_commit, seq,
                     start, n);
  return hipGetLastError();
}

hipError_t launch_loop_tokens(const int32_t* anchor, const int32_t* draft, int32_t* tokens, int batch, int B,
                              hipStream_t st) {
  if (batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(loop_tokens_kernel, dim3((batch + 3) / 4), dim3(256), 0, st, anchor, draft, tokens, batch, B);
  return hipGetLastError();
}

hipError_t launch_loop_advance(const LoopAdvanceParams& p, hipStream_t st) {
  if (p.batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(loop_advance_kernel, dim3((p.batch + 3) / 4), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace dfl

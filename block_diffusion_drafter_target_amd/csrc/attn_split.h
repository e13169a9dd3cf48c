// Split of a batch's attention keys into chunks, shared by the kernel that
// computes it once per pass of the layer stack (the first layer's q/k/v
// post-processing) and by the attention and merge kernels that read it.
//
// Every sequence is cut into chunks of C keys from its own first key (its
// last chunk shorter), the chunks of all sequences numbered in order, sequence
// after sequence; C is one length for the batch, the shortest whole number of
// slices for which the batch has no more chunks than attention workgroups per
// kv head, so in a ragged batch the long sequences take more chunks than the
// short ones and no workgroup holds more than C keys. A sequence has
// Lk = L + B keys, or none if it carries an error status.
//
// Plan layout (int32, attn_plan_ints() of them):
//   [0]                          C
//   [1 + u], u < n_ranges        sequence of chunk u, or -1 past the last chunk
//   [1 + n_ranges + u]           index of chunk u within its sequence
//   [1 + 2 n_ranges + b]         first chunk (partial slot) of sequence b
//   [1 + 2 n_ranges + batch + b] chunk count of sequence b
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace dfl {

inline long long attn_plan_ints(int n_ranges, int batch) { return 1 + 2ll * n_ranges + 2ll * batch; }

// Inclusive prefix sum over the 64 lanes of a wave.
template <typename T>
__device__ __forceinline__ T split_wave_scan(T v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const T t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

__device__ __forceinline__ int split_wave_sum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Keys of sequence i: L_i + B, or 0 with an error status (or past the batch);
// the loads stay at a clamped index.
__device__ __forceinline__ int split_seq_keys(const int32_t* ctx_len, const int32_t* status, int batch, int B, int i) {
  const int ic = min(i, batch - 1);
  const int lk = status[ic] == 0 ? ctx_len[ic] + B : 0;
  return i < batch ? lk : 0;
}

// C for the batch (the same in every lane), at least ceil(max Lk / 64) so
// that no sequence has more than 64 chunks (the merge holds one chunk's
// statistics per lane). With T keys over nb sequences the answer lies in
// [T / n_ranges, T / (n_ranges - nb)] (sum ceil(Lk / C) <= T / C + nb), and
// C >= max Lk always qualifies (one chunk each, n_ranges >= batch): a binary
// search of a few probes. lk0 holds the keys of sequence lane.
__device__ __forceinline__ int split_chunk_keys(const int32_t* ctx_len, const int32_t* status, int batch, int B,
                                                int n_ranges, int slice, int lk0) {
  const int lane = threadIdx.x & 63;
  long long t = lk0;
  int mx = lk0, nb = lk0 > 0;
  for (int i = lane + 64; i < batch; i += 64) {
    const int lk = split_seq_keys(ctx_len, status, batch, B, i);
    t += lk;
    mx = max(mx, lk);
    nb += lk > 0;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    t += __shfl_xor(t, o);
    mx = max(mx, __shfl_xor(mx, o));
    nb += __shfl_xor(nb, o);
  }
  const long long sl = slice;
  int lo = (int)max(max(1ll, ((mx + 63) / 64 + sl - 1) / sl), (t + n_ranges * sl - 1) / (n_ranges * sl));
  int hi = max(lo, (int)((mx + sl - 1) / sl));
  if (n_ranges > nb) {
    const long long c = (t + (n_ranges - nb) - 1) / (n_ranges - nb);
    hi = min(hi, max(lo, (int)((c + sl - 1) / sl)));
  }
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    const int c = mid * slice;
    int n = (lk0 + c - 1) / c;
    for (int i = lane + 64; i < batch; i += 64) n += (split_seq_keys(ctx_len, status, batch, B, i) + c - 1) / c;
    if (split_wave_sum(n) <= n_ranges)
      hi = mid;
    else
      lo = mid + 1;
  }
  return lo * slice;
}

// One wave writes the plan of the batch (layout above). n_ranges >= batch.
__device__ __forceinline__ void attn_plan_wave(const int32_t* ctx_len, const int32_t* status, int batch, int B,
                                               int n_ranges, int slice, int32_t* plan) {
  const int lane = threadIdx.x & 63;
  const int lk0 = split_seq_keys(ctx_len, status, batch, B, lane);
  const int C = split_chunk_keys(ctx_len, status, batch, B, n_ranges, slice, lk0);
  if (lane == 0) plan[0] = C;
  int32_t* seq_of = plan + 1;
  int32_t* idx_of = plan + 1 + n_ranges;
  int32_t* first = plan + 1 + 2 * n_ranges;
  int32_t* count = first + batch;
  int total = 0;
  for (int sb = 0; sb < batch; sb += 64) {
    const int b = sb + lane;
    const int lk = sb == 0 ? lk0 : split_seq_keys(ctx_len, status, batch, B, b);
    const int nseg = (lk + C - 1) / C;
    const int incl = split_wave_scan<int>(nseg);
    const int s0 = total + incl - nseg;
    if (b < batch) {
      first[b] = s0;
      count[b] = nseg;
      for (int j = 0; j < nseg; ++j) {
        seq_of[s0 + j] = b;
        idx_of[s0 + j] = j;
      }
    }
    total += __shfl(incl, 63);
  }
  for (int u = total + lane; u < n_ranges; u += 64) seq_of[u] = -1;
}

}  // namespace dfl

// Sampling mode (temperature > 0): Gumbel-max draft sampling and
// speculative-sampling verification, gfx950.
//
// The acceptance rule is the standard speculative-sampling one: draft token
// d_j (sampled from the drafter's q_j = softmax(z^d_j / T)) is accepted when
// u_j <= p_{j-1}(d_j) / q_j(d_j), p_i = softmax(z^t_i / T) the target's
// distribution after block row i; the first rejected position takes a token
// sampled from the normalised max(0, p_{j-1} - q_j), and when every draft
// passes a bonus token is sampled from p_{B-1}. Sampling from a distribution
// is the argmax of its log-probabilities plus Gumbel noise -log(-log u).
//
// Uniforms come from Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11: ten
// rounds of two 32x32-bit multiplications by 0xD2511F53 and 0xCD9E8D57, Weyl
// key increments 0x9E3779B9 and 0xBB67AE85). A draw (seed, tag, step, row, v)
// uses key (seed low word, seed high word), counter (v / 4, row, step, tag) and
// output word v % 4, mapped to ((word >> 9) + 0.5) * 2^-23 (exact in fp32).
// Tags: 0 draft sampling (row = LM row), 1 acceptance (row = b*B + j, v = 0),
// 2 residual or bonus sample (row = b).
//
// Work layout: every vocabulary pass runs in chunks of kChunk values per
// 256-thread workgroup, a thread taking eight groups of four consecutive
// values (one Philox call each) with all eight 16-byte loads issued before any
// arithmetic. The log-sum-exp of a row is kept as per-chunk (max, sum) pairs
// that its readers combine (19 pairs at V = 151936). The Gumbel argmax runs in
// chunks of kGChunk values (two groups per thread) and leaves one packed
// (score, index) key per chunk, reduced by a finishing kernel with one wave
// per item (no atomics): at batch 1 the residual pass over one row had 19
// workgroups with the 8192-value chunks (Qwen3-8B-shaped drafter at batch 1:
// sampling verify 37.5 -> 28.1 us, sampled step 844 -> 829 us, measured on
// MI355X, with the residual pass's log-sum-exps formed by one wave each).
#include "common.h"
#include "internal.h"

namespace dfl {

namespace {

constexpr int kChunk = 8192;   // vocabulary values per log-sum-exp workgroup
constexpr int kGChunk = 2048;  // vocabulary values per Gumbel-argmax workgroup
constexpr int kTagDraft = 0, kTagAccept = 1, kTagResidual = 2;

__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                               uint32_t k1) {
  constexpr uint32_t kM0 = 0xD2511F53u, kM1 = 0xCD9E8D57u, kW0 = 0x9E3779B9u, kW1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += kW0;
      k1 += kW1;
    }
    const uint32_t hi0 = __umulhi(kM0, c0), lo0 = kM0 * c0;
    const uint32_t hi1 = __umulhi(kM1, c2), lo1 = kM1 * c2;
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  return u32x4{c0, c1, c2, c3};
}

__device__ __forceinline__ float u01(uint32_t w) { return ((float)(w >> 9) + 0.5f) * 0x1p-23f; }

__device__ __forceinline__ float gumbel(float u) { return -logf(-logf(u)); }

constexpr int kGroups = kChunk / 1024;    // float4 groups per thread and chunk
constexpr int kGGroups = kGChunk / 1024;  // the same for the Gumbel argmax

// Partial log-sum-exp of z * inv_t over one chunk of one row: pmax[row][chunk]
// and psum[row][chunk] = sum over the chunk of exp(z * inv_t - pmax).
__global__ __launch_bounds__(256) void lse_partial_kernel(const LseParams p) {
  __shared__ float red[2][4];
  const int row = blockIdx.y, chunk = blockIdx.x;
  const float* z = row < p.rows0 ? p.z0 + (long long)row * p.V : p.z1 + (long long)(row - p.rows0) * p.V;
  const int v0 = chunk * kChunk;
  f32x4_t x[kGroups];
#pragma unroll
  for (int k = 0; k < kGroups; ++k) {
    const int v = min(v0 + (k * 256 + (int)threadIdx.x) * 4, p.V - 4);  // clamped: loads stay in the row
    x[k] = *reinterpret_cast<const f32x4_t*>(z + v);
  }
  float mx = -__builtin_inff();
#pragma unroll
  for (int k = 0; k < kGroups; ++k) {
    const bool in = v0 + (k * 256 + (int)threadIdx.x) * 4 < p.V;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (in) mx = fmaxf(mx, x[k][i] * p.inv_t);
  }
  float sum = 0.f;
#pragma unroll
  for (int k = 0; k < kGroups; ++k) {
    const bool in = v0 + (k * 256 + (int)threadIdx.x) * 4 < p.V;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (in) sum += __expf(x[k][i] * p.inv_t - mx);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float om = __shfl_xor(mx, o), os = __shfl_xor(sum, o);
    const float nm = fmaxf(mx, om);
    sum = (mx == -__builtin_inff() ? 0.f : sum * __expf(mx - nm)) + (om == -__builtin_inff() ? 0.f : os * __expf(om - nm));
    mx = nm;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    red[0][wave] = mx;
    red[1][wave] = sum;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = red[0][0];
    for (int w = 1; w < 4; ++w) m = fmaxf(m, red[0][w]);
    float t = 0.f;
    for (int w = 0; w < 4; ++w) t += red[0][w] == -__builtin_inff() ? 0.f : red[1][w] * __expf(red[0][w] - m);
    p.pmax[(long long)row * p.chunks + chunk] = m;
    p.psum[(long long)row * p.chunks + chunk] = t;
  }
}

// log-sum-exp of one row from its per-chunk pairs: up to kLseBatch pairs are
// loaded together (clamped indexes, no branch between the loads) and folded
// into a running (max, sum), so a row of up to kLseBatch chunks costs one
// round trip instead of one per unrolled step of two serial loops
constexpr int kLseBatch = 32;
__device__ __forceinline__ float lse_of(const float* pmax, const float* psum, int row, int chunks) {
  const float* pm = pmax + (long long)row * chunks;
  const float* ps = psum + (long long)row * chunks;
  float m = -__builtin_inff(), t = 0.f;
  for (int c0 = 0; c0 < chunks; c0 += kLseBatch) {
    float a[kLseBatch], b[kLseBatch];
#pragma unroll
    for (int j = 0; j < kLseBatch; ++j) {
      const int c = min(c0 + j, chunks - 1);
      a[j] = pm[c];
      b[j] = ps[c];
    }
    float bm = m;
#pragma unroll
    for (int j = 0; j < kLseBatch; ++j)
      if (c0 + j < chunks) bm = fmaxf(bm, a[j]);
    t = m == -__builtin_inff() ? 0.f : t * __expf(m - bm);
#pragma unroll
    for (int j = 0; j < kLseBatch; ++j)
      if (c0 + j < chunks) t += b[j] * __expf(a[j] - bm);
    m = bm;
  }
  return m + logf(t);
}

// The same, formed by one wave (every lane calls it and gets the result): lane
// c combines chunks c, c + 64, ..., then the wave's maximum and sum.
__device__ __forceinline__ float lse_of_wave(const float* pmax, const float* psum, int row, int chunks) {
  const int lane = threadIdx.x & 63;
  const float* pm = pmax + (long long)row * chunks;
  const float* ps = psum + (long long)row * chunks;
  float m = -__builtin_inff();
  for (int c = lane; c < chunks; c += 64) m = fmaxf(m, pm[c]);
  m = wave_max(m);
  float t = 0.f;
  for (int c = lane; c < chunks; c += 64) t += ps[c] * __expf(pm[c] - m);
  return m + logf(wave_sum(t));
}

// Acceptance of one sequence per wave: lane j (1 <= j <= B-1) tests draft j
// (the tests are independent given the drafts), the first failing lane ends
// the accepted prefix (ballot). Writes the accepted drafts into the
// target-token row a, the count m[b] and rejected[b] (0: every draft passed).
__global__ __launch_bounds__(64) void accept_kernel(const AcceptParams p) {
  const int b = blockIdx.x, j = threadIdx.x;
  const int B = p.B;
  bool ok = true;
  int d = 0;
  if (j >= 1 && j < B) {
    d = p.draft[b * (B - 1) + j - 1];
    const int dc = d < 0 ? 0 : (d >= p.V ? p.V - 1 : d);
    const float lp = p.zt[(long long)(b * B + j - 1) * p.V + dc] * p.inv_t -
                     lse_of(p.pmax, p.psum, p.rows_d + b * B + j - 1, p.chunks);
    const float lq = p.zd[(long long)(b * (B - 1) + j - 1) * p.V + dc] * p.inv_t -
                     lse_of(p.pmax, p.psum, b * (B - 1) + j - 1, p.chunks);
    const uint32_t step = p.step + (p.step_dev ? (uint32_t)*p.step_dev : 0u);
    const u32x4 w = philox4x32_10(0u, (uint32_t)(b * B + j), step, kTagAccept, p.seed_lo, p.seed_hi);
    ok = d == dc && logf(u01(w[0])) <= lp - lq;
  }
  const unsigned long long fail = __ballot(!ok);  // lanes 1..B-1 only can fail
  const int first = fail ? __ffsll((long long)fail) - 1 : B;  // first rejected position, or B
  const int m = first - 1;
  if (j >= 1 && j <= m) p.a[b * B + j - 1] = d;
  if (j == 0) {
    p.m[b] = m;
    p.rejected[b] = first < B ? 1 : 0;
  }
}

// One chunk of the Gumbel argmax of one item: MODE 0 draft sampling (item =
// LM row; score z * inv_t + g), MODE 1 the new token of sequence `item`
// (score log(max(0, p - q)) + g after a rejection, log p + g for the bonus).
template <int MODE>
__global__ __launch_bounds__(256) void gumbel_argmax_kernel(const GumbelParams p) {
  __shared__ unsigned long long red[4];
  const int item = blockIdx.y, chunk = blockIdx.x;
  const int v0 = chunk * kGChunk;
  const float* zp;  // MODE 0: the row's logits; MODE 1: the target row p is taken from
  const float* zq = nullptr;
  float lse_p = 0.f, lse_q = 0.f;
  uint32_t row_id, tag;
  if (MODE == 0) {
    zp = p.z + (long long)item * p.V;
    row_id = (uint32_t)(p.row0 + item);
    tag = kTagDraft;
  } else {
    const int B = p.B, m = p.m[item];
    const int tr = item * B + m;
    zp = p.zt + (long long)tr * p.V;
    lse_p = lse_of_wave(p.pmax, p.psum, p.rows_d + tr, p.lse_chunks);
    if (p.rejected[item]) {
      const int dr = item * (B - 1) + m;
      zq = p.zd + (long long)dr * p.V;
      lse_q = lse_of_wave(p.pmax, p.psum, dr, p.lse_chunks);
    }
    row_id = (uint32_t)item;
    tag = kTagResidual;
  }
  const uint32_t step = p.step + (p.step_dev ? (uint32_t)*p.step_dev : 0u);
  f32x4_t x[kGGroups], y[kGGroups];
#pragma unroll
  for (int k = 0; k < kGGroups; ++k) {
    const int v = min(v0 + (k * 256 + (int)threadIdx.x) * 4, p.V - 4);  // clamped: loads stay in the row
    x[k] = *reinterpret_cast<const f32x4_t*>(zp + v);
    if (MODE == 1) y[k] = zq ? *reinterpret_cast<const f32x4_t*>(zq + v) : f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  float bv = -__builtin_inff();
  int bn = 0x7FFFFFFF;
#pragma unroll
  for (int k = 0; k < kGGroups; ++k) {  // ascending v within the thread: lowest index on ties
    const int v = v0 + (k * 256 + (int)threadIdx.x) * 4;
    if (v >= p.V) continue;
    const u32x4 w = philox4x32_10((uint32_t)(v >> 2), row_id, step, tag, p.seed_lo, p.seed_hi);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float s;
      if (MODE == 0) {
        s = x[k][i] * p.inv_t;
      } else if (zq) {
        const float r = __expf(x[k][i] * p.inv_t - lse_p) - __expf(y[k][i] * p.inv_t - lse_q);
        s = r > 0.f ? logf(r) : -__builtin_inff();
      } else {
        s = x[k][i] * p.inv_t - lse_p;
      }
      if (s != -__builtin_inff()) {
        s += gumbel(u01(w[i]));
        if (s > bv) {
          bv = s;
          bn = v + i;
        }
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o);
    const int on = __shfl_xor(bn, o);
    if (ov > bv || (ov == bv && on < bn)) {
      bv = ov;
      bn = on;
    }
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = bn != 0x7FFFFFFF ? argmax_key(bv, bn) : 0ull;
  __syncthreads();
  if (threadIdx.x == 0)
    p.keys[(long long)chunk * p.items + item] = max(max(red[0], red[1]), max(red[2], red[3]));
}

// Best key over the chunks of every item: MODE 0 writes the sampled draft
// token (-1 for a sequence whose status is nonzero, as the greedy path does),
// MODE 1 writes the new token into the target-token row at position m.
template <int MODE>
__global__ __launch_bounds__(256) void gumbel_finish_kernel(const GumbelParams p) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);  // one wave per item
  if (item >= p.items) return;
  unsigned long long best = 0ull;
  for (int c = lane; c < p.chunks; c += 64) best = max(best, p.keys[(long long)c * p.items + item]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) best = max(best, (unsigned long long)__shfl_xor(best, o));
  if (lane != 0) return;
  const int tok = best ? (int)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFull)) : 0;
  if (MODE == 0) {
    const int seq = item / (p.B - 1);
    p.out[item] = (p.status && p.status[seq] != 0) ? -1 : tok;
  } else {
    p.a[item * p.B + p.m[item]] = tok;
  }
}

}  // namespace

int sample_chunks(int V) { return (V + kChunk - 1) / kChunk; }
int gumbel_chunks(int V) { return (V + kGChunk - 1) / kGChunk; }

hipError_t launch_lse(const LseParams& p, hipStream_t st) {
  if (p.V % 4 || p.V < 4 || p.rows0 < 0 || p.rows0 + p.rows1 < 1 || p.chunks != sample_chunks(p.V))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(lse_partial_kernel, dim3(p.chunks, p.rows0 + p.rows1), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_accept(const AcceptParams& p, hipStream_t st) {
  if (p.batch < 1 || p.B < 2 || p.B > 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(accept_kernel, dim3(p.batch), dim3(64), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_gumbel(const GumbelParams& p, int mode, hipStream_t st) {
  if (p.V % 4 || p.V < 4 || p.items < 1 || p.chunks != gumbel_chunks(p.V) ||
      (mode == 1 && p.lse_chunks != sample_chunks(p.V)))
    return hipErrorInvalidValue;
  const dim3 grid(p.chunks, p.items);
  if (mode == 0) {
    hipLaunchKernelGGL(gumbel_argmax_kernel<0>, grid, dim3(256), 0, st, p);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    hipLaunchKernelGGL(gumbel_finish_kernel<0>, dim3((p.items + 3) / 4), dim3(256), 0, st, p);
  } else {
    hipLaunchKernelGGL(gumbel_argmax_kernel<1>, grid, dim3(256), 0, st, p);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    hipLaunchKernelGGL(gumbel_finish_kernel<1>, dim3((p.items + 3) / 4), dim3(256), 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace dfl

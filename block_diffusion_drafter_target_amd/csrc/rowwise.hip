// Row-wise kernels of the draft step (gfx950): embedding + RMSNorm, split-K
// reduction + residual + RMSNorm, per-head q/k RMSNorm + RoPE + KV-cache
// append, SwiGLU, the inject epilogue (k-norm + RoPE + cache scatter + commit
// of ctx_len), and the unpacking of argmax keys into draft tokens.
//
// All are bound by a few kilobytes per row; they exist to keep every fp32
// statistic (RMSNorm sums, residual stream, RoPE) on the device between the
// bf16 MFMA GEMMs.
#include "common.h"
#include "internal.h"

namespace dfl {

namespace {

constexpr int kErrCapacity = -5;  // DFLASH_ERR_CAPACITY
constexpr int kErrShape = -2;     // DFLASH_ERR_SHAPE

// ---------------------------------------------------------------------------
// block row embedding: x = E[token], u = bf16(RMSNorm(x) * g_in of layer 0)
// Row j of sequence b holds the anchor (j = 0) or the mask id. The j == 0
// workgroup also records the sequence's capacity status.
__global__ __launch_bounds__(256) void embed_kernel(const EmbedParams p) {
  __shared__ float red[4];
  const int m = blockIdx.x;
  const int b = m / p.B, j = m % p.B;
  const int L = p.ctx_len[b];
  const bool cap_bad = L < 0 || L + p.B > p.max_ctx || L + p.B > p.rope_max;
  int tok = j == 0 ? p.anchor[b] : p.mask_id;
  const bool tok_bad = tok < 0 || tok >= p.V;
  if (j == 0 && threadIdx.x == 0) p.status[b] = cap_bad ? kErrCapacity : (tok_bad ? kErrShape : 0);
  if (tok_bad) tok = 0;
  const bf16_t* e = p.embed + (long long)tok * p.H;
  float* x = p.x + (long long)m * p.H;
  float ss = 0.f;
  for (int i = threadIdx.x; i < p.H; i += 256) {
    const float v = bf2f(e[i]);
    x[i] = v;
    if (p.dbg) p.dbg[(long long)m * p.H + i] = v;
    ss += v * v;
  }
  ss = block_sum_256(ss, red);
  const float inv = 1.0f / sqrtf(ss / (float)p.H + p.eps);
  bf16_t* u = p.u + (long long)m * p.H;
  for (int i = threadIdx.x; i < p.H; i += 256) u[i] = f2bf(x[i] * inv * bf2f(p.gain[i]));
}

// ---------------------------------------------------------------------------
// y = (x +=) sum of split partials; out = bf16(RMSNorm(y) * gain)
__global__ __launch_bounds__(256) void row_norm_kernel(const RowNormParams p) {
  __shared__ float red[4];
  const int m = blockIdx.x;
  const int n = p.n;
  constexpr int kPer = 16;  // the first 16*256 columns stay in registers
  auto load = [&](int i) {
    float v = 0.f;
    if (p.P) {
      const float* src = p.P + (long long)m * n + i;
      for (int s = 0; s < p.splits; ++s) v += src[(long long)s * p.p_s_stride];
    }
    if (p.x) {
      float* xp = p.x + (long long)m * n + i;
      v += *xp;
      *xp = v;
    }
    if (p.dbg) p.dbg[(long long)m * n + i] = v;
    return v;
  };
  float vals[kPer];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < kPer; ++c) {
    const int i = threadIdx.x + c * 256;
    vals[c] = i < n ? load(i) : 0.f;
    ss += vals[c] * vals[c];
  }
  for (int i = threadIdx.x + kPer * 256; i < n; i += 256) {
    const float v = load(i);
    ss += v * v;
  }
  ss = block_sum_256(ss, red);
  const float inv = 1.0f / sqrtf(ss / (float)n + p.eps);
  bf16_t* out = nullptr;
  if (p.final_mode) {
    const int b = m / p.B, j = m % p.B;
    if (j == 0) return;
    const int row = b * (p.B - 1) + j - 1;
    out = p.out + (long long)row * n;
    if (threadIdx.x == 0) p.keys[row] = 0ull;
  } else {
    out = p.out + (long long)m * n;
  }
#pragma unroll
  for (int c = 0; c < kPer; ++c) {
    const int i = threadIdx.x + c * 256;
    if (i < n) out[i] = f2bf(vals[c] * inv * bf2f(p.gain[i]));
  }
  for (int i = threadIdx.x + kPer * 256; i < n; i += 256) {
    float v;
    if (p.x) {
      v = p.x[(long long)m * n + i];
    } else {
      v = 0.f;
      const float* src = p.P + (long long)m * n + i;
      for (int s = 0; s < p.splits; ++s) v += src[(long long)s * p.p_s_stride];
    }
    out[i] = f2bf(v * inv * bf2f(p.gain[i]));
  }
}

// ---------------------------------------------------------------------------
// q/k/v of block rows: sum split partials per head; q and k get a per-head
// RMSNorm and rotate-half RoPE at position L_b + j; q goes to the query buffer,
// k and v to cache slot L_b + j (speculative append). One wave per head;
// lane i < D/2 holds the pair (i, i + D/2).
__global__ __launch_bounds__(256) void qkv_post_kernel(const QkvPostParams p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = blockIdx.y;
  const int head = blockIdx.x * 4 + wave;
  const int nh = p.Hq + 2 * p.Hkv;
  if (head >= nh) return;
  const int b = m / p.B, j = m % p.B;
  if (p.status[b] != 0) return;
  const int pos = p.ctx_len[b] + j;
  const int D = p.D, half = D >> 1;
  const int width = nh * D;
  const bool active = lane < half;
  float x1 = 0.f, x2 = 0.f;
  if (active) {
    const float* src = p.P + (long long)m * width + head * D + lane;
    for (int s = 0; s < p.splits; ++s) {
      x1 += src[(long long)s * p.p_s_stride];
      x2 += src[(long long)s * p.p_s_stride + half];
    }
  }
  if (head >= p.Hq + p.Hkv) {  // v
    if (active) {
      const int g = head - p.Hq - p.Hkv;
      bf16_t* dst = p.vc + (((long long)b * p.Hkv + g) * p.max_ctx + pos) * D;
      dst[lane] = f2bf(x1);
      dst[lane + half] = f2bf(x2);
    }
    return;
  }
  const float ss = wave_sum(x1 * x1 + x2 * x2);
  const float inv = 1.0f / sqrtf(ss / (float)D + p.eps);
  if (!active) return;
  const bf16_t* gain = head < p.Hq ? p.gq : p.gk;
  const float y1 = x1 * inv * bf2f(gain[lane]);
  const float y2 = x2 * inv * bf2f(gain[lane + half]);
  const float2 cs = reinterpret_cast<const float2*>(p.rope)[(long long)pos * half + lane];
  const float o1 = y1 * cs.x - y2 * cs.y;
  const float o2 = y1 * cs.y + y2 * cs.x;
  bf16_t* dst;
  if (head < p.Hq) {
    dst = p.q + ((long long)m * p.Hq + head) * D;
  } else {
    const int g = head - p.Hq;
    dst = p.kc + (((long long)b * p.Hkv + g) * p.max_ctx + pos) * D;
  }
  dst[lane] = f2bf(o1);
  dst[lane + half] = f2bf(o2);
}

// ---------------------------------------------------------------------------
// s = silu(gate) * up from split partials; silu(z) = z / (1 + e^-z)
__global__ __launch_bounds__(256) void swiglu_kernel(const SwigluParams p) {
  const long long total = (long long)p.rows * p.I;
  for (long long e = blockIdx.x * 256ll + threadIdx.x; e < total; e += (long long)gridDim.x * 256) {
    const int m = (int)(e / p.I), i = (int)(e % p.I);
    const float* src = p.P + (long long)m * 2 * p.I + i;
    float gsum = 0.f, usum = 0.f;
    for (int s = 0; s < p.splits; ++s) {
      gsum += src[(long long)s * p.p_s_stride];
      usum += src[(long long)s * p.p_s_stride + p.I];
    }
    const float silu = gsum / (1.0f + __expf(-gsum));
    p.out[e] = f2bf(silu * usum);
  }
}

// ---------------------------------------------------------------------------
// KV injection epilogue: for commit row i and layer l, k = RoPE(RMSNorm_head(
// W_k c)), v = W_v c, scattered to (seq, pos); ctx_len[seq] grows to pos + 1.
__global__ __launch_bounds__(256) void inject_post_kernel(const InjectPostParams p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = p.c0 + blockIdx.x, l = blockIdx.y;
  int nc = *p.n_commit;
  nc = nc < 0 ? 0 : (nc > p.max_commit ? p.max_commit : nc);
  if (i >= nc || i >= p.c1) return;
  const int src = p.commit_rows[3 * i], seq = p.commit_rows[3 * i + 1], pos = p.commit_rows[3 * i + 2];
  if (src < 0 || src >= p.n_ctx_rows || seq < 0 || seq >= p.batch) return;
  if (pos < 0 || pos >= p.max_ctx || pos >= p.rope_max) {
    if (l == 0 && threadIdx.x == 0) p.status[seq] = kErrCapacity;
    return;
  }
  const int D = p.D, half = D >> 1;
  const int width = 2 * p.Hkv * D;
  const bool active = lane < half;
  for (int head = wave; head < 2 * p.Hkv; head += 4) {
    float x1 = 0.f, x2 = 0.f;
    if (active) {
      const float* s0 = p.P + (long long)l * p.p_z_stride + (long long)(i - p.c0) * width + head * D + lane;
      for (int s = 0; s < p.splits; ++s) {
        x1 += s0[(long long)s * p.p_s_stride];
        x2 += s0[(long long)s * p.p_s_stride + half];
      }
    }
    const int g = head < p.Hkv ? head : head - p.Hkv;
    const long long off = ((((long long)l * p.batch + seq) * p.Hkv + g) * p.max_ctx + pos) * D;
    if (head >= p.Hkv) {
      if (active) {
        p.vc[off + lane] = f2bf(x1);
        p.vc[off + lane + half] = f2bf(x2);
      }
      continue;
    }
    const float ss = wave_sum(x1 * x1 + x2 * x2);
    const float inv = 1.0f / sqrtf(ss / (float)D + p.eps);
    if (active) {
      const float y1 = x1 * inv * bf2f(p.gk[l][lane]);
      const float y2 = x2 * inv * bf2f(p.gk[l][lane + half]);
      const float2 cs = reinterpret_cast<const float2*>(p.rope)[(long long)pos * half + lane];
      p.kc[off + lane] = f2bf(y1 * cs.x - y2 * cs.y);
      p.kc[off + lane + half] = f2bf(y1 * cs.y + y2 * cs.x);
    }
  }
  if (l == 0 && threadIdx.x == 0) atomicMax(p.ctx_len + seq, pos + 1);
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void unpack_draft_kernel(const unsigned long long* keys,
                                                           const int32_t* status, int batch, int B,
                                                           int32_t* draft) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= batch * (B - 1)) return;
  const int b = e / (B - 1);
  draft[e] = status[b] != 0 ? -1 : (int32_t)(0xFFFFFFFFu - (uint32_t)(keys[e] & 0xFFFFFFFFull));
}

}  // namespace

hipError_t launch_embed(const EmbedParams& p, hipStream_t st) {
  hipLaunchKernelGGL(embed_kernel, dim3(p.batch * p.B), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_row_norm(const RowNormParams& p, hipStream_t st) {
  hipLaunchKernelGGL(row_norm_kernel, dim3(p.rows), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_qkv_post(const QkvPostParams& p, hipStream_t st) {
  const int nh = p.Hq + 2 * p.Hkv;
  hipLaunchKernelGGL(qkv_post_kernel, dim3((nh + 3) / 4, p.batch * p.B), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_swiglu(const SwigluParams& p, hipStream_t st) {
  const long long total = (long long)p.rows * p.I;
  long long blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(swiglu_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_inject_post(const InjectPostParams& p, hipStream_t st) {
  if (p.c1 <= p.c0) return hipSuccess;
  hipLaunchKernelGGL(inject_post_kernel, dim3(p.c1 - p.c0, p.n_layers), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_unpack_draft(const unsigned long long* keys, const int32_t* status, int batch,
                               int B, int32_t* draft, hipStream_t st) {
  const int n = batch * (B - 1);
  hipLaunchKernelGGL(unpack_draft_kernel, dim3((n + 255) / 256), dim3(256), 0, st, keys, status,
                     batch, B, draft);
  return hipGetLastError();
}

}  // namespace dfl

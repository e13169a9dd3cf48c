// Packed fragment layout of GEMM weights (gfx950).
//
// A row-major bf16 matrix W[rows][cols] is cut into 16-row x 32-column
// fragments, one MFMA 16x16x32 operand each. Fragment (rg, kc) holds rows
// 16*rg .. 16*rg+15 and columns 32*kc .. 32*kc+31 and is stored as 1 KB at
// fragment index rg * (cols/32) + kc. Inside it, the 16 bytes read by lane
// l = 16*g + r are row 16*rg + r, columns 32*kc + 8*g .. 32*kc + 8*g + 7:
//   packed[((rg * (cols/32) + kc) * 64 + 16*g + r) * 8 + e]
//     = W[16*rg + r][32*kc + 8*g + e]
// A 16-row group is therefore one contiguous run along k.
#include "common.h"
#include "internal.h"

namespace dfl {

namespace {

__global__ __launch_bounds__(256) void pack_kernel(const bf16_t* __restrict__ src, bf16_t* __restrict__ dst,
                                                   int rows, int cols) {
  const long long slot = blockIdx.x * 256ll + threadIdx.x;  // one 16-byte lane slot
  const int kcs = cols / 32;
  const long long nslots = (long long)(rows / 16) * kcs * 64;
  if (slot >= nslots) return;
  const int lane = (int)(slot & 63);
  const long long frag = slot >> 6;
  const int kc = (int)(frag % kcs);
  const long long rg = frag / kcs;
  const int r = lane & 15, g = lane >> 4;
  const long long row = rg * 16 + r;
  const u32x4 v = *reinterpret_cast<const u32x4*>(src + row * cols + kc * 32 + g * 8);
  *reinterpret_cast<u32x4*>(dst + slot * 8) = v;
}

}  // namespace

hipError_t launch_pack(const uint16_t* src, uint16_t* dst, int rows, int cols, hipStream_t st) {
  const long long nslots = (long long)(rows / 16) * (cols / 32) * 64;
  if (nslots == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)((nslots + 255) / 256)), dim3(256), 0, st, src, dst,
                     rows, cols);
  return hipGetLastError();
}

}  // namespace dfl

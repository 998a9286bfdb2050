// Weight repacking at handle creation: the projection matrices of kernels 1
// and 3 are stored in the order their lanes hold them in registers, so that
// every weight load of a wave reads 1 KB of contiguous memory.
//
// Register order ("fragments"): a row-major matrix of 16-row blocks, [R][D]
// with R = 16 * nblocks. In both kernels lane l = 16 g + r of the wave that
// owns block b holds row 16 b + r, elements [g D/4, g D/4 + D/4) (the matrix
// cores contract the four lane groups' K ranges side by side), loaded as
// D*es/64 pieces of 16 bytes. Fragment order puts, for each block b and each
// piece v, the 64 lanes' 16-byte pieces one after another:
//   frags[((b * (D*es/64) + v) * 64 + l) * 16 bytes]
//     = row 16 b + r, bytes [(g D/4) es + 16 v, +16).
#include "device_common.h"
#include "tri_attn_internal.h"

namespace tpa {

__global__ __launch_bounds__(256) void pack_weight_frags(const char *rows, char *frags, int D, int es, int nblocks) {
  const int nvw = D * es / 64;
  const long total = (long)nblocks * nvw * 64;
  const long o = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (o >= total) return;
  const int lane = (int)(o % 64);
  const long bv = o / 64;
  const int v = (int)(bv % nvw), b = (int)(bv / nvw);
  const int g = lane >> 4, r = lane & 15;
  const size_t src = ((size_t)(b * 16 + r) * D + (size_t)g * (D / 4)) * es + (size_t)v * 16;
  *reinterpret_cast<uint4 *>(frags + o * 16) = *reinterpret_cast<const uint4 *>(rows + src);
}

// Float32 rows [16 * nblocks][D] into three bf16 planes (the split3 parts),
// each in the bf16 fragment order above (D*2/64 pieces of 8 elements per lane
// and block); plane p starts at frags + p * plane_bytes.
__global__ __launch_bounds__(256) void pack_weight_frags_split3(const float *rows, char *frags, size_t plane_bytes,
                                                                int D, int nblocks) {
  const int nvw = D / 32;
  const long total = (long)nblocks * nvw * 64;
  const long o = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (o >= total) return;
  const int lane = (int)(o % 64);
  const long bv = o / 64;
  const int v = (int)(bv % nvw), b = (int)(bv / nvw);
  const int g = lane >> 4, r = lane & 15;
  const float *src = rows + (size_t)(b * 16 + r) * D + (size_t)g * (D / 4) + (size_t)v * 8;
  uint32_t p1[4], p2[4], p3[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) split3(src[2 * u], src[2 * u + 1], p1[u], p2[u], p3[u]);
  *reinterpret_cast<uint4 *>(frags + o * 16) = make_uint4(p1[0], p1[1], p1[2], p1[3]);
  *reinterpret_cast<uint4 *>(frags + plane_bytes + o * 16) = make_uint4(p2[0], p2[1], p2[2], p2[3]);
  *reinterpret_cast<uint4 *>(frags + 2 * plane_bytes + o * 16) = make_uint4(p3[0], p3[1], p3[2], p3[3]);
}

hipError_t launch_pack_frags_split3(int D, const void *rows, void *frags, size_t plane_bytes, int nblocks,
                                    hipStream_t s) {
  if (D % 32 != 0 || nblocks <= 0) return hipErrorInvalidValue;
  const long total = (long)nblocks * (D / 32) * 64;
  hipLaunchKernelGGL(pack_weight_frags_split3, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                     static_cast<const float *>(rows), static_cast<char *>(frags), plane_bytes, D, nblocks);
  return hipGetLastError();
}

hipError_t launch_pack_frags(int elem_bytes, int D, const void *rows, void *frags, int nblocks, hipStream_t s) {
  if ((D * elem_bytes) % 64 != 0 || nblocks <= 0) return hipErrorInvalidValue;
  const long total = (long)nblocks * (D * elem_bytes / 64) * 64;
  hipLaunchKernelGGL(pack_weight_frags, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                     static_cast<const char *>(rows), static_cast<char *>(frags), D, elem_bytes, nblocks);
  return hipGetLastError();
}

}  // namespace tpa

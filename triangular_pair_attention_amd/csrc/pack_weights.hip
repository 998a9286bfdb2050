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

hipError_t launch_pack_frags(int elem_bytes, int D, const void *rows, void *frags, int nblocks, hipStream_t s) {
  if ((D * elem_bytes) % 64 != 0 || nblocks <= 0) return hipErrorInvalidValue;
  const long total = (long)nblocks * (D * elem_bytes / 64) * 64;
  hipLaunchKernelGGL(pack_weight_frags, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                     static_cast<const char *>(rows), static_cast<char *>(frags), D, elem_bytes, nblocks);
  return hipGetLastError();
}

}  // namespace tpa

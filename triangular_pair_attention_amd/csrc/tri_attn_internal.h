// Internal declarations shared by the host library and the kernels.
// Not part of the public ABI (include/tri_attn.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tri_attn.h"

namespace tpa {

constexpr int kChunk = 64;  // key chunk of the per-chunk maxima; also K1's position tile

// Workspace regions (byte offsets); see tri_attn_workspace_layout in the header.
struct Layout {
  size_t q, k, vt, g, zm, zmax, kmax, vsum, rflag, total;
  int Np;      // N rounded up to kChunk
  int nchunk;  // Np / kChunk
  int items;   // attention work items (one recovery flag byte each)
};

Layout make_layout(int B, int N, int D, int h, int elem_bytes);

// Kernel 1: LayerNorm + one fused projection GEMM.
struct K1Args {
  const void *P;          // [B][N][N][D]
  const uint8_t *mask;    // [B][N][N]
  const void *W;          // packed [(4D + 16)][D]: Wq; Wk; Wv; Wg; Wz; zero rows
  const void *Wf;         // Wq; Wk; Wv; Wg in fragment order (pack_weights.hip)
  const void *Ws;         // float32 handles: Wq; Wk; Wv; Wg; Wo as three bf16 planes in fragment order
  size_t ws_plane;        // bytes from one plane of Ws to the next
  const void *gamma, *beta, *bg;  // [D]
  void *q, *k, *vt, *g;
  float *zm, *zmax, *kmax, *vsum;
  float eps;
  float qscale;  // log2(e) / sqrt(d)
  int B, N, Np, nchunk, tiles;
  int transposed;  // ending-node: position (b, i, j) reads pair_repr[b][j][i] and mask[b][j][i]
};

// Kernel 2: attention core + gate, per head; writes g * o over the gate.
struct K2Args {
  const void *q, *k, *vt;
  void *g;
  const float *zm, *zmax, *kmax, *vsum;
  float mask_fill;  // finite (uniform rule on fully masked columns) or -inf (NaN there)
  float shift_slack;
  uint8_t *rflag;   // [items]: 1 where the item took the exact-maximum recovery, else 0 (null: not recorded)
  int B, N, Np, nchunk, items;
};

// Training-mode attention (k2_train.hip): dropout and the saved log-sum-exp.
struct K2TrainArgs {
  float *lse;        // [B][N][h][N] float32 or null
  uint32_t thr;      // keep iff the generator's word >= thr
  float scale;       // 2^32 / (2^32 - thr)
  uint32_t seed_lo, seed_hi, offset;
  int h;
};

// Kernel 3: output projection of g * o (left by kernel 2 in the gate region).
struct K3Args {
  const void *go;  // [B][N][D/16][Np][16]
  const void *Wof;  // Wo in fragment order (pack_weights.hip); float32 handles: its first split plane
  size_t wo_plane;  // float32 handles: bytes from one split plane of Wo to the next
  const void *bo;
  void *out;       // [B][N][N][D]
  int B, N, Np, nchunk, tiles;
  int transposed;  // ending-node: position (b, i, j) is written to out[b][j][i]
};

hipError_t launch_k2_train(int dtype, int dh, const K2Args &a, const K2TrainArgs &tr, hipStream_t s);

// Launchers: return the launch status. `dtype` is TRI_ATTN_F32 / TRI_ATTN_BF16.
hipError_t launch_k1(int dtype, int D, int dh, const K1Args &a, int grid, hipStream_t s);
// grid: persistent workgroups (a multiple of 8 when smaller than a.items)
hipError_t launch_k2(int dtype, int D, int dh, const K2Args &a, int grid, hipStream_t s);
hipError_t launch_k3(int dtype, int D, const K3Args &a, int grid, hipStream_t s);
// Copies the row-major [16 * nblocks][D] matrix `rows` into fragment order.
hipError_t launch_pack_frags(int elem_bytes, int D, const void *rows, void *frags, int nblocks, hipStream_t s);
// Splits the float32 rows into three bf16 planes (plane_bytes apart), each in bf16 fragment order.
hipError_t launch_pack_frags_split3(int D, const void *rows, void *frags, size_t plane_bytes, int nblocks,
                                    hipStream_t s);
int k2_items(int dtype, int D, int dh, int B, int N);
int k2_blocks_per_cu(int dtype, int D, int dh);  // resident workgroups of kernel 2 per CU
int k3_blocks_per_cu(int dtype, int D);  // resident workgroups of kernel 3 per CU
int k1_blocks_per_cu(int dtype, int D, int dh);  // resident workgroups of kernel 1 per CU
// Float32 kernel 1 (split products): grid = 2 x workgroups per half (each
// workgroup computes one half of the projections).
hipError_t launch_k1_split(int D, int dh, const K1Args &a, int grid, hipStream_t s);
int k1_split_blocks_per_cu(int D, int dh);
bool supported(int D, int dh);

// Training-mode backward (bwd_train.hip): every argument of the C ABI call
// plus the handle's packed weights.
struct BwdRunArgs {
  const void *P;          // [B][N][N][D] config dtype
  const uint8_t *mask;    // [B][N][N]
  const void *dy;         // [B][N][N][D] config dtype
  const void *wpack;      // [(4D + 16)][D]: Wq; Wk; Wv; Wg; Wz; zero rows (config dtype)
  const void *vecs;       // gamma, beta, bg, bo ([D] each), then Wo [D][D] (config dtype)
  tri_attn_grads g;       // outputs, float32
  void *ws;
  float eps, fill, scale;
  uint32_t thr, seed_lo, seed_hi, offset;
  int B, N;
  int transposed;  // ending-node handle: the starting-node backward of the transposed problem
  int dz_ranges;   // row ranges of the pair-bias gradient step (0: chosen from the sizes)
  // a second stream for the dropout keep bits, forked from and joined to the
  // caller's stream by the two events (null: everything on the caller's stream)
  hipStream_t side;
  hipEvent_t fork, join;
};
hipError_t launch_bwd(int dtype, int D, int dh, const BwdRunArgs &r, hipStream_t s);
size_t bwd_workspace_bytes(int B, int N, int D, int h, int elem_bytes, int transposed, int dz_ranges);
// One-pass variant (onepass.hip): the pre-pass writes zm, the fused row
// kernel does everything else.
struct OnePassArgs {
  const void *P;         // pair_repr [B][N][N][D], config dtype
  const uint8_t *mask;   // [B][N][N]
  const void *W;         // [(4D + 16)][D]: Wq; Wk; Wv; Wg; Wz; zero rows (config dtype)
  const void *vecs;      // gamma, beta, bg, bo ([D] each), then Wo [D][D] (config dtype)
  float *zm;             // [B][h][N][Np] float32: z * log2(e), -inf where masked and for k >= N
  void *out;             // y [B][N][N][D], config dtype
  float eps, fill, qscale;  // qscale = log2(e) / sqrt(d)
  int B, N, Np, h;
  int transposed;        // ending-node: position (b, i, j) reads and writes (b, j, i)
};
constexpr int kOnePassMaxN = 512;
hipError_t launch_onepass(int dtype, int D, int dh, const OnePassArgs &a, hipStream_t s);

// Device address of this GPU's static workspace array (noalloc.hip), looked up
// once per device; `device` must be current. Returns a TRI_ATTN_* code.
int scratch_address(int device, void **ptr);

}  // namespace tpa

// Kernel 3 of the triangular self-attention forward: the output projection
// y = Wo (g * o) + bo per pair position (Kimi-K2.6 / l2_p6 transcript: the
// last step of its forward listing and its finalize kernel; FW-GLM-5-1 /
// l2_p6: the output kernel).
//
// g * o comes from kernel 2, written over the gate in the workspace as
// [b][i][c/16][j][16]. Work unit: 64 consecutive positions (b, i, j0..j0+63);
// persistent grid. Each wave holds the 16 rows of Wo of one output channel
// block in registers (read from a copy in fragment order); the tile goes through LDS once, is multiplied on the
// matrix cores (bias as the accumulator's start), and the bf16 result goes
// back through LDS so that every output row is written as whole 16-byte
// chunks (float32 results are 16 contiguous bytes per lane already and are
// stored straight from the accumulators).
// The next tile is prefetched into registers while the current one computes.
//
// Float32 tensors use the bf16 matrix cores with three-way split operands
// (six exact bf16 products per float32 product, float32 accumulation; see
// kernel 1's split products): Wo comes from its three-plane copy, and the
// tile is split once, by the thread that loads it, into three bf16 planes in
// LDS.
#include "device_common.h"
#include "tri_attn_internal.h"

#include <type_traits>

#include "tri_attn.h"

namespace tpa {

template <typename T, int D>
__global__ __launch_bounds__(D / 16 * 64) void k3_out_proj(K3Args a) {
  constexpr bool BF = is_bf16<T>::value;
  constexpr int ES = BF ? 2 : 4;
  constexpr int NB = D / 16;  // output channel blocks = waves
  constexpr int NT = NB * 64;
  constexpr int KQ = D / 4;
  constexpr int KS = D / 32;                   // MFMA steps over K = D
  constexpr int PARTS = BF ? 1 : 3;            // bf16 parts per operand
  constexpr int PITCH = D + 16 / ES;           // output staging row pitch (elements of T)
  constexpr int XPITCH = D + 8;                // operand row pitch (bf16 elements)
  constexpr int TILE = kChunk;
  constexpr int NV = 16 * ES / 16;             // 16-byte chunks of one position's channel block
  constexpr int ROWV = D * ES / 16;            // 16-byte chunks per output row
  constexpr int CPT = TILE * ROWV / NT;        // output chunks per thread

  __shared__ __align__(16) uint16_t xs[PARTS][TILE * XPITCH];
  __shared__ __align__(16) T ys[BF ? TILE * PITCH : 1];  // bf16: output staging

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int N = a.N, Np = a.Np, nch = a.nchunk;
  const T *GO = reinterpret_cast<const T *>(a.go);

  // Wo rows of this wave's block, stored in fragment order (each load of the
  // wave reads 1 KB contiguously): lane (g, r16) holds row wave*16 + r16,
  // K-range [g*KQ, g*KQ+KQ), in PARTS bf16 planes
  bf16x8 wo[KS][PARTS];
  {
    const char *wsrc = reinterpret_cast<const char *>(a.Wof) + ((size_t)wave * KS * 64 + lane) * 16;
#pragma unroll
    for (int v = 0; v < KS; ++v)
#pragma unroll
      for (int q = 0; q < PARTS; ++q) wo[v][q] = as_bf16x8(ldg<uint4>(wsrc + q * a.wo_plane + (size_t)v * 1024));
  }
  f32x4 bias;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int c = wave * 16 + 4 * g + r;
    bias[r] = BF ? bf2f(reinterpret_cast<const uint16_t *>(a.bo)[c]) : reinterpret_cast<const float *>(a.bo)[c];
  }

  // thread (wave, lane) loads channel block `wave` of position `lane` of a tile
  auto load_tile = [&](int tile, uint4 (&pre)[NV]) {
    const int bi_row = tile / nch, chunk = tile - bi_row * nch;
    const int j = chunk * TILE + lane;
    const T *src = GO + (((size_t)bi_row * NB + wave) * Np + j) * 16;
#pragma unroll
    for (int v = 0; v < NV; ++v) pre[v] = (j < N) ? ldg<uint4>(src + v * (16 / ES)) : make_uint4(0, 0, 0, 0);
  };

  // output element (b, i, j); ending-node writes (b, j, i)
  auto out_at = [&](int bi_row, int j) -> size_t {
    const int bb = bi_row / N;
    return a.transposed ? ((size_t)bb * N + j) * N + (bi_row - bb * N) : (size_t)bi_row * N + j;
  };

  int tile = blockIdx.x;
  if (tile >= a.tiles) return;
  uint4 pre[NV];
  load_tile(tile, pre);
#pragma unroll 1
  for (; tile < a.tiles; tile += gridDim.x) {
    const int bi_row = tile / nch, chunk = tile - bi_row * nch;
    const int j0 = chunk * TILE;
    if constexpr (BF) {
#pragma unroll
      for (int v = 0; v < NV; ++v) *reinterpret_cast<uint4 *>(&xs[0][lane * XPITCH + wave * 16 + v * 8]) = pre[v];
    } else {
      // this position's 16 channels, split into three bf16 parts
      const float *f = reinterpret_cast<const float *>(pre);
#pragma unroll
      for (int h8 = 0; h8 < 2; ++h8) {
        uint32_t p1[4], p2[4], p3[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) split3(f[8 * h8 + 2 * u], f[8 * h8 + 2 * u + 1], p1[u], p2[u], p3[u]);
        const int o = lane * XPITCH + wave * 16 + 8 * h8;
        *reinterpret_cast<uint4 *>(&xs[0][o]) = make_uint4(p1[0], p1[1], p1[2], p1[3]);
        *reinterpret_cast<uint4 *>(&xs[PARTS - 2][o]) = make_uint4(p2[0], p2[1], p2[2], p2[3]);
        *reinterpret_cast<uint4 *>(&xs[PARTS - 1][o]) = make_uint4(p3[0], p3[1], p3[2], p3[3]);
      }
    }
    lds_barrier();
    if (tile + (int)gridDim.x < a.tiles) load_tile(tile + gridDim.x, pre);

#pragma unroll
    for (int pb = 0; pb < TILE / 16; ++pb) {
      const int xo = (pb * 16 + r16) * XPITCH + g * KQ;
      auto xf = [&](int q, int s) { return as_bf16x8(*reinterpret_cast<const uint4 *>(&xs[q][xo + 8 * s])); };
      f32x4 acc = bias;
      if constexpr (BF) {
#pragma unroll
        for (int s = 0; s < KS; ++s) acc = mfma(wo[s][0], xf(0, s), acc);
      } else {
        // (weight part, tile part): small terms (3,1) (2,2) (1,3) into acc1,
        // large terms (2,1) (1,2) (1,1) into acc
        f32x4 acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const bf16x8 x1 = xf(0, s), x2 = xf(PARTS - 2, s), x3 = xf(PARTS - 1, s);
          acc1 = mfma(wo[s][PARTS - 1], x1, acc1);
          acc = mfma(wo[s][PARTS - 2], x1, acc);
          acc1 = mfma(wo[s][PARTS - 2], x2, acc1);
          acc = mfma(wo[s][0], x2, acc);
          acc1 = mfma(wo[s][0], x3, acc1);
          acc = mfma(wo[s][0], x1, acc);
        }
        acc += acc1;
      }
      // y^T tile: lane (g, r16) holds channels wave*16 + 4g..4g+3 of position pb*16 + r16
      if constexpr (BF) {
        T *dst = &ys[(pb * 16 + r16) * PITCH + wave * 16 + 4 * g];
        *reinterpret_cast<uint2 *>(dst) = make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
      } else {
        // float32: 16 contiguous bytes per lane, stored at once, so the
        // stores of block pb overlap the products of block pb + 1
        const int j = j0 + pb * 16 + r16;
        if (j < N)
          stg<float4>(reinterpret_cast<float *>(a.out) + out_at(bi_row, j) * D + wave * 16 + 4 * g,
                      make_float4(acc[0], acc[1], acc[2], acc[3]));
      }
    }
    // every wave is done with xs before the next tile overwrites it (and, for
    // bf16, the staged output tile is complete)
    lds_barrier();
    if constexpr (BF) {
      // whole 16-byte chunks of each output row
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        const int c = tid + NT * k;
        const int pos = c / ROWV, off = c - pos * ROWV;
        if (j0 + pos < N) {
          const uint4 v = *reinterpret_cast<const uint4 *>(&ys[pos * PITCH + off * (16 / ES)]);
          stg<uint4>(reinterpret_cast<T *>(a.out) + out_at(bi_row, j0 + pos) * D + off * (16 / ES), v);
        }
      }
    }
  }
}

template <typename T, int D>
static hipError_t launch_k3_t(const K3Args &a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((k3_out_proj<T, D>), dim3(grid), dim3(D / 16 * 64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_k3(int dtype, int D, const K3Args &a, int grid, hipStream_t s) {
  if (dtype == TRI_ATTN_BF16) {
    if (D == 128) return launch_k3_t<bf16_t, 128>(a, grid, s);
    if (D == 64) return launch_k3_t<bf16_t, 64>(a, grid, s);
  } else {
    if (D == 128) return launch_k3_t<float, 128>(a, grid, s);
    if (D == 64) return launch_k3_t<float, 64>(a, grid, s);
  }
  return hipErrorInvalidValue;
}

int k3_blocks_per_cu(int dtype, int D) {
  int n = 0;
  hipError_t e = hipErrorInvalidValue;
  if (dtype == TRI_ATTN_BF16)
    e = D == 128 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k3_out_proj<bf16_t, 128>, 512, 0)
                 : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k3_out_proj<bf16_t, 64>, 256, 0);
  else
    e = D == 128 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k3_out_proj<float, 128>, 512, 0)
                 : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k3_out_proj<float, 64>, 256, 0);
  return (e == hipSuccess && n > 0) ? n : 1;
}

}  // namespace tpa

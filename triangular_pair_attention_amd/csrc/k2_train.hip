// Training-mode attention core: kernel 2's step with dropout on the attention
// weights and the row log-sum-exp saved (FW-GLM-5-1 / l2_p6 transcript, the
// forward as restated: dropout right after the softmax over keys, before the
// product with v; Kimi-K2.6 / l2_p6: the module's dropout layer).
//
// Dropout decision of key k for query column j, head t, row (b, i): word
// k mod 4 of Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC 2011) at counter (k / 4, j,
// (b*N + i)*h + t, offset) and key (seed low word, seed high word); the
// weight is kept iff that word >= thr and kept weights are scaled by
// 2^32 / (2^32 - thr), which keeps the expectation exact. The row sums that
// normalise the softmax use the undropped weights.
//
// Reads kernel 1's workspace (q pre-scaled by log2(e)/sqrt(d), the bias+mask
// tile in the log2 domain), writes g * o over the gate like kernel 2 (kernel 3
// then projects it), and lse[b][i][t][j] = ln sum_k exp(s), s the masked
// scores. A fully masked column (finite fill) has uniform weights 1/N over
// all N keys before dropout and lse = fill + ln N; with fill = -inf it gets
// NaN, as the definition does.
//
// One workgroup per (b, i, t, 256 query columns), one lane per column, a
// running maximum over the keys in float32, updated once per four keys.
// Tiles of 64 keys of k and v go through LDS (every lane reads the same key:
// broadcasts); each lane forms its own scores with FMAs and draws its own
// numbers (one generator call per four keys). A column with no valid key is known from kernel 1's per-chunk
// bias maxima, so its uniform-weight sum runs in the same loop.
#include "device_common.h"
#include "tri_attn.h"
#include "tri_attn_internal.h"

namespace tpa {


template <typename T, int DH>
__global__ __launch_bounds__(256) void k2_train(K2Args a, K2TrainArgs tr) {
  constexpr bool BF = is_bf16<T>::value;
  constexpr bool KSPLIT = !BF && DH == 32;  // k stored as three bf16 parts (kernel 1)
  constexpr int KT = 64;                    // keys per LDS tile
  constexpr int QW = 256;                   // query columns per workgroup
  __shared__ float ks[KT][DH];              // k of the tile's keys (read as broadcasts)
  __shared__ float vs[KT][DH];              // v of the tile's keys (key-major, like ks)
  const int N = a.N, Np = a.Np, nch = a.nchunk;
  const int H = tr.h, NB = tr.h * DH / 16;
  const int nq = (N + QW - 1) / QW;
  int blk = blockIdx.x;
  const int qc = blk % nq;
  blk /= nq;
  const int t = blk % H;
  const int row = blk / H;  // b * N + i
  const int b = row / N;
  const int tid = threadIdx.x;
  const int j = qc * QW + tid;
  const bool active = j < N;  // every thread stays for the barriers
  const int jc = active ? j : N - 1;

  float q[DH];
#pragma unroll
  for (int u = 0; u < DH; ++u)
    q[u] = ld_elem<T>(a.q, (((size_t)row * NB + t * (DH / 16) + u / 16) * Np + jc) * 16 + u % 16);
  const float *zrow = a.zm + ((size_t)(b * H + t) * N + jc) * Np;
  // a column with no valid key (finite fill): uniform weights over all N keys
  bool dead = true;
  for (int c = 0; c < nch; ++c) dead = dead && a.zmax[((size_t)(b * H + t) * nch + c) * N + jc] == -INFINITY;
  const size_t vbase = ((size_t)row * H + t) * DH * Np;  // v^T [b][i][t][u][k]
  const uint32_t ctr2 = (uint32_t)(row * H + t);

  float m = -INFINITY, l = 0.f, o[DH];
#pragma unroll
  for (int u = 0; u < DH; ++u) o[u] = 0.f;
  uint4 w = make_uint4(0, 0, 0, 0);
  float4 z4;  // bias of the current four keys (rows run to Np)
  for (int k0 = 0; k0 < N; k0 += KT) {
    // stage the tile (keys past N as zeros)
    for (int e = tid; e < KT * DH; e += QW) {
      const int kk = e / DH, u = e - kk * DH, k = k0 + kk;
      float kv = 0.f;
      if (k < N) {
        if constexpr (KSPLIT) {
          const uint16_t *kp = reinterpret_cast<const uint16_t *>(a.k) + ((size_t)row * H + t) * 3 * Np * 32 +
                               (size_t)(k >> 4) * 512 + (k & 15) * 8 + (size_t)(u >> 3) * 128 + (u & 7);
          kv = bf2f(kp[0]) + bf2f(kp[(size_t)Np * 32]) + bf2f(kp[(size_t)Np * 64]);
        } else {
          kv = ld_elem<T>(a.k, (((size_t)row * NB + t * (DH / 16) + u / 16) * Np + k) * 16 + u % 16);
        }
      }
      ks[kk][u] = kv;
    }
    for (int e = tid; e < KT * DH; e += QW) {
      const int u = e / KT, kk = e - u * KT, k = k0 + kk;
      vs[kk][u] = k < N ? ld_elem<T>(a.vt, vbase + (size_t)u * Np + k) : 0.f;
    }
    __syncthreads();
    const int kn = min(KT, N - k0);  // keys past N in the tile: zero k and v, bias -inf
    if (active) {
      for (int kk = 0; kk < kn; kk += 4) {
        const int k = k0 + kk;
        w = philox4x32_10(make_uint4((uint32_t)(k >> 2), (uint32_t)j, ctr2, tr.offset), tr.seed_lo, tr.seed_hi);
        const bool keep[4] = {w.x >= tr.thr, w.y >= tr.thr, w.z >= tr.thr, w.w >= tr.thr};
        if (dead) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (keep[e]) {
#pragma unroll
              for (int u = 0; u < DH; ++u) o[u] += vs[kk + e][u];
            }
          continue;
        }
        z4 = *reinterpret_cast<const float4 *>(zrow + k);
        float s4[4] = {z4.x, z4.y, z4.z, z4.w};  // -inf for masked keys stays -inf
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int u = 0; u < DH; ++u) s4[e] = fmaf(q[u], ks[kk + e][u], s4[e]);
        const float mx = fmaxf(fmaxf(s4[0], s4[1]), fmaxf(s4[2], s4[3]));
        if (mx > m) {
          const float c = exp2f(m - mx);  // 0 for the first live keys
          l *= c;
#pragma unroll
          for (int u = 0; u < DH; ++u) o[u] *= c;
          m = mx;
        }
        if (m == -INFINITY) continue;  // no live key yet
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = exp2f(s4[e] - m);  // masked: 0
          l += p;
          const float pk = keep[e] ? p : 0.f;
#pragma unroll
          for (int u = 0; u < DH; ++u) o[u] = fmaf(pk, vs[kk + e][u], o[u]);
        }
      }
    }
    __syncthreads();  // every lane is done with the tile before it is refilled
  }
  if (!active) return;  // past the last barrier
  float inv, lse;
  if (dead) {
    if (a.mask_fill == -INFINITY) {
      inv = NAN;
      lse = NAN;
    } else {
      inv = tr.scale / (float)N;
      lse = a.mask_fill + logf((float)N);
    }
  } else {
    inv = tr.scale / l;
    lse = (m + log2f(l)) * 0.69314718055994531f;
  }
  if (tr.lse) tr.lse[((size_t)row * H + t) * N + j] = lse;
  // g * o over the gate: [b][i][c/16][j][16]
#pragma unroll
  for (int u = 0; u < DH; ++u) {
    const size_t gi = (((size_t)row * NB + t * (DH / 16) + u / 16) * Np + j) * 16 + u % 16;
    const float val = ld_elem<T>(a.g, gi) * (o[u] * inv);
    if constexpr (BF)
      reinterpret_cast<uint16_t *>(a.g)[gi] = (uint16_t)(pack_bf16x2(val, 0.f) & 0xFFFFu);
    else
      reinterpret_cast<float *>(a.g)[gi] = val;
  }
}

template <typename T, int DH>
static hipError_t launch_t(const K2Args &a, const K2TrainArgs &tr, hipStream_t s) {
  const long long blocks = (long long)a.B * a.N * tr.h * ((a.N + 255) / 256);
  if (blocks <= 0 || blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k2_train<T, DH>), dim3((unsigned)blocks), dim3(256), 0, s, a, tr);
  return hipGetLastError();
}

hipError_t launch_k2_train(int dtype, int dh, const K2Args &a, const K2TrainArgs &tr, hipStream_t s) {
  if (dtype == TRI_ATTN_BF16) {
    if (dh == 16) return launch_t<bf16_t, 16>(a, tr, s);
    if (dh == 32) return launch_t<bf16_t, 32>(a, tr, s);
  } else {
    if (dh == 16) return launch_t<float, 16>(a, tr, s);
    if (dh == 32) return launch_t<float, 32>(a, tr, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tpa

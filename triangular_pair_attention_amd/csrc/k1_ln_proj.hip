// Kernel 1 of the triangular self-attention forward: LayerNorm of the pair
// representation and ONE fused projection GEMM producing q | k | v | gate |
// pair bias (Kimi-K2.6 / l2_p6 transcript: steps 1-7 of its forward listing
// and its layer list; FW-GLM-5-1 / l2_p6: the LayerNorm and linear kernels).
//
// Work unit: a tile of 64 consecutive pair positions (b, i, j0..j0+63) of one
// row. A persistent grid walks the tiles; each workgroup (8 waves) keeps its
// slice of the packed weight [Wq; Wk; Wv; Wg; Wz] in registers for its whole
// life, so the weight is read from L2 once per workgroup, not once per tile.
//
//  1. LayerNorm (fp32 statistics, two-pass in registers): 8 lanes per
//     position, the normalised row goes to LDS in the operand type. The next
//     tile's pair_repr is prefetched into registers meanwhile.
//  2. Each wave owns D/32 16-channel blocks of one projection (waves 0-1: q,
//     2-3: k, 4-5: v, 6-7: gate; wave 0 also the pair-bias block) and runs
//     the 16x16 MFMA tiles against the LDS activations.
//  3. Epilogues write directly in the layouts kernel 2 reads:
//     q (pre-scaled by log2(e)/sqrt(d)), k, gate (sigmoid(+bias)) as
//     [b][i][c/16][j][16] (one 512-byte burst per tile); v transposed per
//     head [b][i][t][u][j]; the pair bias z*log2(e) with the mask folded in
//     (-inf where masked) as [b][t][i][j]; plus per-64-key-chunk maxima of
//     zm and of |k|^2, used by kernel 2 to bound the softmax shift and skip
//     fully masked key chunks.
#include "device_common.h"
#include "tri_attn_internal.h"

#include <type_traits>

#include "tri_attn.h"

namespace tpa {

// Waves per projection: 2 (8 waves per workgroup), or 4 (16 waves) where the
// per-wave weight slice would not fit the register file (fp32, D = 128).
template <typename T, int D>
struct K1Shape {
  static constexpr int WPP = (!is_bf16<T>::value && D == 128) ? 4 : 2;
  static constexpr int THREADS = 4 * WPP * 64;
};

template <typename T, int D, int DH>
__global__ __launch_bounds__((K1Shape<T, D>::THREADS)) void k1_ln_proj(K1Args a) {
  constexpr bool BF = is_bf16<T>::value;
  constexpr int WPP = K1Shape<T, D>::WPP;
  constexpr int NT = K1Shape<T, D>::THREADS;
  constexpr int ES = BF ? 2 : 4;        // element bytes
  constexpr int H = D / DH;             // heads
  constexpr int NB = D / 16;            // 16-channel blocks per projection
  constexpr int BPW = NB / WPP;         // blocks per wave
  constexpr int HPW = BPW * 16 / DH;    // k heads per k wave
  constexpr int KQ = D / 4;             // K-dim elements per lane (lane group g owns [g*KQ, g*KQ+KQ))
  constexpr int KS = BF ? D / 32 : D / 4;  // MFMA steps over K = D
  constexpr int PITCH = D + 16 / ES;    // LDS row pitch (elements), 16-byte pad against bank conflicts
  constexpr int TPP = NT / 64;          // LayerNorm threads per position
  constexpr int EPT = D / TPP;          // LayerNorm elements per thread
  constexpr int NV = EPT * ES / 16;     // 16-byte loads per thread per tile
  constexpr int TILE = kChunk;
  using Frag = typename std::conditional<BF, bf16x8, float>::type;
  static_assert(BPW >= 1 && (DH == 16 || BPW % 2 == 0), "a k head must not straddle two waves");

  __shared__ __align__(16) T xs[2][TILE * PITCH];
  __shared__ uint8_t mask_s[2][TILE];  // the tile's mask bytes (0 also for j >= N)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int ptype = wave / WPP;          // 0 q, 1 k, 2 v, 3 gate
  const int cb0 = (wave % WPP) * BPW;  // first block of this wave inside its projection
  const int N = a.N, Np = a.Np, nch = a.nchunk;

  // ---- weights into registers: lane (g, r16) holds row r16 of each block, K-range [g*KQ, g*KQ+KQ)
  Frag wf[BPW][KS];
  const T *W = reinterpret_cast<const T *>(a.W);
#pragma unroll
  for (int bi = 0; bi < BPW; ++bi) {
    const T *wrow = W + (size_t)((ptype * NB + cb0 + bi) * 16 + r16) * D + g * KQ;
    if constexpr (BF) {
#pragma unroll
      for (int s = 0; s < KS; ++s) wf[bi][s] = as_bf16x8(ldg<uint4>(wrow + 8 * s));
    } else {
#pragma unroll
      for (int s = 0; s < KS; s += 4) {
        float4 v = ldg<float4>(wrow + s);
        wf[bi][s] = v.x, wf[bi][s + 1] = v.y, wf[bi][s + 2] = v.z, wf[bi][s + 3] = v.w;
      }
    }
  }
  __shared__ float vec_s[3][D];  // gamma, beta, gate bias (fp32)
  __shared__ __align__(16) T wz_s[16 * PITCH];  // pair-bias weight block (rows >= h are zero)
  for (int e = tid; e < 16 * D; e += NT) wz_s[(e / D) * PITCH + e % D] = W[(size_t)4 * D * D + e];
  for (int c = tid; c < 3 * D; c += NT) {
    const int which = c / D, cc = c - which * D;
    const void *src = which == 0 ? a.gamma : (which == 1 ? a.beta : a.bg);
    vec_s[which][cc] = BF ? bf2f(reinterpret_cast<const uint16_t *>(src)[cc]) : reinterpret_cast<const float *>(src)[cc];
  }
  __syncthreads();

  // ---- LayerNorm thread mapping: TPP threads per position, EPT channels each
  const int lpos = tid / TPP, lpart = tid % TPP;

  auto load_tile = [&](int tile, uint4 (&pre)[NV], uint32_t &mpre) {
    const int bi_row = tile / nch, chunk = tile - bi_row * nch;
    const int j = chunk * TILE + lpos;
    mpre = (j < N && lpart == 0) ? a.mask[(size_t)bi_row * N + j] : 0u;
    if (j < N) {
      const char *src = reinterpret_cast<const char *>(a.P) + ((size_t)bi_row * N + j) * D * ES + lpart * EPT * ES;
#pragma unroll
      for (int v = 0; v < NV; ++v) pre[v] = ldg<uint4>(src + 16 * v);
    } else {
#pragma unroll
      for (int v = 0; v < NV; ++v) pre[v] = make_uint4(0, 0, 0, 0);
    }
  };

  auto layer_norm_to_lds = [&](int tile, const uint4 (&pre)[NV], uint32_t mpre, int buf) {
    const int bi_row = tile / nch, chunk = tile - bi_row * nch;
    const int j = chunk * TILE + lpos;
    if (lpart == 0) mask_s[buf][lpos] = (uint8_t)mpre;
    float v[EPT];
    const uint32_t *w32 = reinterpret_cast<const uint32_t *>(pre);
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      if constexpr (BF)
        v[e] = (e & 1) ? bfhi(w32[e >> 1]) : bflo(w32[e >> 1]);
      else
        v[e] = __uint_as_float(w32[e]);
    }
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < EPT; ++e) s += v[e];
#pragma unroll
    for (int m = 1; m < TPP; m <<= 1) s = xor_sum(s, m);
    const float mean = s * (1.0f / D);
    float q = 0.f;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const float dv = v[e] - mean;
      q += dv * dv;
    }
#pragma unroll
    for (int m = 1; m < TPP; m <<= 1) q = xor_sum(q, m);
    const float rstd = rsqrtf(q * (1.0f / D) + a.eps);
    const bool valid = j < N;
    const float *gam = &vec_s[0][lpart * EPT];
    const float *bet = &vec_s[1][lpart * EPT];
    T *dst = &xs[buf][lpos * PITCH + lpart * EPT];
    if constexpr (BF) {
      uint32_t packed[EPT / 2];
#pragma unroll
      for (int e = 0; e < EPT; e += 2) {
        const float x0 = valid ? (v[e] - mean) * rstd * gam[e] + bet[e] : 0.f;
        const float x1 = valid ? (v[e + 1] - mean) * rstd * gam[e + 1] + bet[e + 1] : 0.f;
        packed[e / 2] = pack_bf16x2(x0, x1);
      }
#pragma unroll
      for (int e = 0; e < EPT / 2; e += 4)
        *reinterpret_cast<uint4 *>(dst + 2 * e) = make_uint4(packed[e], packed[e + 1], packed[e + 2], packed[e + 3]);
    } else {
#pragma unroll
      for (int e = 0; e < EPT; e += 4) {
        float4 o;
        o.x = valid ? (v[e] - mean) * rstd * gam[e] + bet[e] : 0.f;
        o.y = valid ? (v[e + 1] - mean) * rstd * gam[e + 1] + bet[e + 1] : 0.f;
        o.z = valid ? (v[e + 2] - mean) * rstd * gam[e + 2] + bet[e + 2] : 0.f;
        o.w = valid ? (v[e + 3] - mean) * rstd * gam[e + 3] + bet[e + 3] : 0.f;
        *reinterpret_cast<float4 *>(dst + e) = o;
      }
    }
  };

  auto store4 = [&](T *dst, float v0, float v1, float v2, float v3) {
    if constexpr (BF)
      stg<uint2>(dst, make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)));
    else
      stg<float4>(dst, make_float4(v0, v1, v2, v3));
  };

  // acc[bi] = block bi of this wave's projection for one 16-position block
  auto gemm = [&](auto is_v, const T *xrow, f32x4 (&acc)[BPW]) {
#pragma unroll
    for (int bi = 0; bi < BPW; ++bi) acc[bi] = f32x4{0.f, 0.f, 0.f, 0.f};
    constexpr int KC = BF ? 1 : 4;
#pragma unroll
    for (int s0 = 0; s0 < KS; s0 += KC) {
      Frag xf[KC];
      if constexpr (BF) {
        xf[0] = as_bf16x8(*reinterpret_cast<const uint4 *>(xrow + 8 * s0));
      } else {
        const float4 v = *reinterpret_cast<const float4 *>(xrow + s0);
        xf[0] = v.x, xf[1] = v.y, xf[2] = v.z, xf[3] = v.w;
      }
#pragma unroll
      for (int s = 0; s < KC; ++s)
#pragma unroll
        for (int bi = 0; bi < BPW; ++bi) {
          if constexpr (decltype(is_v)::value)
            acc[bi] = mfma(xf[s], wf[bi][s0 + s], acc[bi]);  // rows = positions
          else
            acc[bi] = mfma(wf[bi][s0 + s], xf[s], acc[bi]);  // rows = channels
        }
    }
  };
  // pair-bias block (weights in LDS): rows = positions, column = head
  auto gemm_z = [&](const T *xrow) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const T *zrow = &wz_s[r16 * PITCH + g * KQ];
    constexpr int KC = BF ? 1 : 4;
#pragma unroll
    for (int s0 = 0; s0 < KS; s0 += KC) {
      if constexpr (BF) {
        acc = mfma(as_bf16x8(*reinterpret_cast<const uint4 *>(xrow + 8 * s0)),
                   as_bf16x8(*reinterpret_cast<const uint4 *>(zrow + 8 * s0)), acc);
      } else {
        const float4 v = *reinterpret_cast<const float4 *>(xrow + s0);
        const float4 u = *reinterpret_cast<const float4 *>(zrow + s0);
        acc = mfma(v.x, u.x, acc);
        acc = mfma(v.y, u.y, acc);
        acc = mfma(v.z, u.z, acc);
        acc = mfma(v.w, u.w, acc);
      }
    }
    return acc;
  };

  auto compute_tile = [&](int tile, int buf) {
    const int bi_row = tile / nch, chunk = tile - bi_row * nch;
    const int b = bi_row / N, i = bi_row - b * N;
    const int j0 = chunk * TILE;
    float kn_run[HPW];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) kn_run[hh] = 0.f;
    float z_run = -INFINITY;

#pragma unroll 1
    for (int pb = 0; pb < TILE / 16; ++pb) {
      // GEMM over K = D; lane (g, r16) reads position pb*16+r16, K-range
      // [g*KQ, g*KQ+KQ) of the LDS activations. v tiles swap the operand roles
      // so that their rows are positions (transposed store per head).
      f32x4 acc[BPW];
      const T *xrow = &xs[buf][(pb * 16 + r16) * PITCH + g * KQ];
      if (ptype == 2)
        gemm(std::true_type{}, xrow, acc);
      else
        gemm(std::false_type{}, xrow, acc);
      const int jcol = j0 + pb * 16 + r16;  // position of this lane's column (q/k/gate tiles)
      float ksq = 0.f;
#pragma unroll
      for (int bi = 0; bi < BPW; ++bi) {
        const int cb = cb0 + bi;
        if (ptype == 2) {
          // v^T per head: lane (g, r16) holds channel r16 of positions 4g..4g+3
          const int c = cb * 16 + r16, th = c / DH, uu = c - th * DH;
          T *dst = reinterpret_cast<T *>(a.vt) + ((((size_t)bi_row * H + th) * DH + uu) * Np + j0 + pb * 16 + 4 * g);
          store4(dst, acc[bi][0], acc[bi][1], acc[bi][2], acc[bi][3]);
        } else {
          float v0 = acc[bi][0], v1 = acc[bi][1], v2 = acc[bi][2], v3 = acc[bi][3];
          T *base;
          if (ptype == 0) {
            v0 *= a.qscale, v1 *= a.qscale, v2 *= a.qscale, v3 *= a.qscale;
            base = reinterpret_cast<T *>(a.q);
          } else if (ptype == 1) {
            base = reinterpret_cast<T *>(a.k);
            ksq += v0 * v0 + v1 * v1 + v2 * v2 + v3 * v3;
            if (DH == 16 || (bi & 1)) {
              const float n2 = group4_sum(ksq);
              const int hh = (DH == 16) ? bi : (bi >> 1);
              kn_run[hh] = fmaxf(kn_run[hh], n2);
              ksq = 0.f;
            }
          } else {
            const float4 bgv = *reinterpret_cast<const float4 *>(&vec_s[2][cb * 16 + 4 * g]);
            v0 = fast_rcp(1.f + fast_exp2(-(v0 + bgv.x) * kLog2e));
            v1 = fast_rcp(1.f + fast_exp2(-(v1 + bgv.y) * kLog2e));
            v2 = fast_rcp(1.f + fast_exp2(-(v2 + bgv.z) * kLog2e));
            v3 = fast_rcp(1.f + fast_exp2(-(v3 + bgv.w) * kLog2e));
            base = reinterpret_cast<T *>(a.g);
          }
          T *dst = base + ((((size_t)bi_row * NB + cb) * Np + jcol) * 16 + 4 * g);
          store4(dst, v0, v1, v2, v3);
        }
      }
      if (wave == 0) {
        const f32x4 accz = gemm_z(xrow);
        if (r16 < H) {
        const int jb = j0 + pb * 16 + 4 * g;
        float z[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool keep = mask_s[buf][pb * 16 + 4 * g + r] != 0;
          z[r] = keep ? accz[r] * kLog2e : -INFINITY;
          z_run = fmaxf(z_run, z[r]);
        }
        float *dst = a.zm + (((size_t)(b * H + r16) * N + i) * Np + jb);
        stg<float4>(dst, make_float4(z[0], z[1], z[2], z[3]));
        }
      }
    }
    // per-chunk maxima
    if (ptype == 1) {
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) {
        const float m = row16_max(kn_run[hh]);
        const int th = (cb0 * 16) / DH + hh;
        if (lane == 0) a.kmax[((size_t)bi_row * H + th) * nch + chunk] = m;
      }
    }
    if (wave == 0) {
      const float m = group4_max(z_run);
      if (g == 0 && r16 < H) a.zmax[((size_t)(b * H + r16) * N + i) * nch + chunk] = m;
    }
  };

  int tile = blockIdx.x;
  if (tile >= a.tiles) return;
  uint4 pre[NV];
  uint32_t mpre;
  int buf = 0;
  if constexpr (BF) {
    // bf16 is HBM-bound: prefetch the next tile's pair_repr and mask while this one computes
    load_tile(tile, pre, mpre);
#pragma unroll 1
    for (; tile < a.tiles; tile += gridDim.x) {
      layer_norm_to_lds(tile, pre, mpre, buf);
      __syncthreads();
      if (tile + (int)gridDim.x < a.tiles) load_tile(tile + gridDim.x, pre, mpre);
      compute_tile(tile, buf);
      buf ^= 1;
    }
  } else {
    // fp32 is matrix-core-bound and short of registers: no cross-tile prefetch
#pragma unroll 1
    for (; tile < a.tiles; tile += gridDim.x) {
      load_tile(tile, pre, mpre);
      layer_norm_to_lds(tile, pre, mpre, buf);
      __syncthreads();
      compute_tile(tile, buf);
      buf ^= 1;
    }
  }
}

template <typename T, int D, int DH>
static hipError_t launch_k1_t(const K1Args &a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((k1_ln_proj<T, D, DH>), dim3(grid), dim3(K1Shape<T, D>::THREADS), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_k1(int dtype, int D, int dh, const K1Args &a, int grid, hipStream_t s) {
#define TRI_K1_CASE(TT, DD, HH) \
  if (D == DD && dh == HH) return launch_k1_t<TT, DD, HH>(a, grid, s);
  if (dtype == TRI_ATTN_BF16) {
    TRI_K1_CASE(bf16_t, 128, 16)
    TRI_K1_CASE(bf16_t, 128, 32)
    TRI_K1_CASE(bf16_t, 64, 16)
    TRI_K1_CASE(bf16_t, 64, 32)
  } else {
    TRI_K1_CASE(float, 128, 16)
    TRI_K1_CASE(float, 128, 32)
    TRI_K1_CASE(float, 64, 16)
    TRI_K1_CASE(float, 64, 32)
  }
#undef TRI_K1_CASE
  return hipErrorInvalidValue;
}

bool supported(int D, int dh) { return (D == 64 || D == 128) && (dh == 16 || dh == 32); }

}  // namespace tpa

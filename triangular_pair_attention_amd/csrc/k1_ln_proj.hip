// Kernel 1 of the triangular self-attention forward for bf16 tensors
// (float32 tensors use k1_split.hip): LayerNorm of the pair
// representation and ONE fused projection GEMM producing q | k | v | gate |
// pair bias (Kimi-K2.6 / l2_p6 transcript: the LayerNorm and projection steps
// of its forward listing and its layer list; FW-GLM-5-1 / l2_p6: the
// LayerNorm and linear kernels).
//
// Work unit: a tile of 64 consecutive pair positions (b, i, j0..j0+63) of one
// row. A persistent grid walks the tiles; each workgroup keeps the packed
// weight [Wq; Wk; Wv; Wg] in registers for its whole life (each wave holds
// one 16-channel block of TPW projections), so the weight is read from L2
// once per workgroup, not once per tile, and is stored in fragment order
// (one contiguous kilobyte per wave load).
//
//  1. LayerNorm (fp32 statistics, two-pass in registers), TPP lanes per
//     position; the normalised rows go to LDS in the operand type. bf16 tiles
//     prefetch pair_repr and the mask two tiles ahead.
//  2. Wave w owns channel block w % NB of its TPW projections, so every wave
//     has the same MFMA and epilogue work; the pair-bias block (its weight
//     sits in LDS) is the only extra, one 16-position block on each of the
//     first four waves (one per SIMD). The four 16-position blocks
//     of a tile run as a software pipeline (the products of block pb + 1
//     are issued before the epilogue of block pb). A grid with one tile per
//     workgroup uses its own instantiation without a tile loop, whose first
//     products wait only for their own weights.
//  3. Epilogues write directly in the layouts kernel 2 reads:
//     q (pre-scaled by log2(e)/sqrt(d)), k, gate (sigmoid(+bias)) as
//     [b][i][c/16][j][16] (one 512-byte burst per 16x16 tile); v transposed
//     per head [b][i][t][u][j]; the pair bias z*log2(e) with the mask folded
//     in (-inf where masked) as [b][t][i][j]; per-64-key-chunk maxima of that
//     tile and of the squared norm of k over each 16-channel block, which
//     kernel 2 uses to bound the softmax shift and to skip masked key chunks;
//     per-chunk sums of v, for the uniform weights of fully masked columns.
#include "device_common.h"
#include "tri_attn_internal.h"

#include <type_traits>

#include "tri_attn.h"

namespace tpa {

// TPW projections per wave; NW = 4 * NB / TPW waves per workgroup.
template <int D>
struct K1Shape {
  static constexpr int NB = D / 16;
  static constexpr int TPW = 4;
  static constexpr int NW = 4 * NB / TPW;
  static constexpr int THREADS = NW * 64;
};

// ONE: the grid has one tile per workgroup (a straight path with no prefetch
// and no tile loop); otherwise a persistent loop over tiles.
template <int D, int DH, bool ONE>
__global__ __launch_bounds__((K1Shape<D>::THREADS)) void k1_ln_proj(K1Args a) {
  using T = bf16_t;
  constexpr int ES = 2;                    // element bytes
  constexpr int H = D / DH;                // heads
  constexpr int NB = K1Shape<D>::NB;       // 16-channel blocks per projection
  constexpr int TPW = K1Shape<D>::TPW;     // projections per wave
  constexpr int NW = K1Shape<D>::NW;
  constexpr int NT = K1Shape<D>::THREADS;
  constexpr int KQ = D / 4;                // K-dim elements per lane (lane group g owns [g*KQ, g*KQ+KQ))
  constexpr int KS = D / 32;               // MFMA steps over K = D
  constexpr int PITCH = D + 16 / ES;       // LDS row pitch (elements), 16-byte pad against bank conflicts
  constexpr int TPP = NT / 64;             // LayerNorm threads per position
  constexpr int EPT = D / TPP;             // LayerNorm elements per thread
  constexpr int NV = EPT * ES / 16;        // 16-byte loads per thread per tile
  constexpr int TILE = kChunk;
  using Frag = bf16x8;
  static_assert(NV >= 1 && EPT % 8 == 0, "");

  __shared__ __align__(16) T xs[2][TILE * PITCH];
  __shared__ uint8_t mask_s[2][TILE];           // the tile's mask bytes (0 also for j >= N)
  __shared__ float vec_s[3][D];                 // gamma, beta, gate bias (fp32)
  __shared__ __align__(16) T wz_s[16 * PITCH];  // pair-bias weight block (rows >= h are zero)
  __shared__ float zpart_s[TILE / 16][16];      // per-block maxima of the pair bias of a tile
  // this wave's v^T block of a tile (16 channels x 64 positions), written out
  // as whole 128-byte channel rows instead of 16 pieces of 32 bytes per block
  constexpr int VPITCH = TILE + 8;
  __shared__ __align__(16) uint16_t vst_s[NW][16 * VPITCH];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar block and base arithmetic
  const int g = lane >> 4, r16 = lane & 15;
  const int cb = wave % NB;             // this wave's channel block in each of its projections
  const int type0 = (wave / NB) * TPW;  // first projection of this wave (0 q, 1 k, 2 v, 3 gate)
  const int N = a.N, Np = a.Np, nch = a.nchunk;
  const T *W = reinterpret_cast<const T *>(a.W);

  // ---- weights into registers: lane (g, r16) holds row r16 of the block, K-range [g*KQ, g*KQ+KQ).
  // Loaded after the first tile's pair_repr loads are issued, so that the
  // LayerNorm of the first tile waits on its own data only. The weights are
  // stored in fragment order: each load of a wave reads 1 KB contiguously.
  constexpr int NVW = D * ES / 64;  // 16-byte pieces per lane per block
  static_assert(NVW == KS, "");
  Frag wf[TPW][KS];
  auto load_weights = [&]() {
    const char *wsrc = reinterpret_cast<const char *>(a.Wf) + (size_t)lane * 16;
    auto piece = [&](int p, int v) {
      return ldg<uint4>(wsrc + ((size_t)((type0 + p) * NB + cb) * NVW + v) * 1024);
    };
    // issued in the order the MFMAs consume them (contraction step outer), so
    // the first products start while later weights are still arriving
#pragma unroll
    for (int v = 0; v < NVW; ++v)
#pragma unroll
      for (int p = 0; p < TPW; ++p) {
        wf[p][v] = as_bf16x8(piece(p, v));
      }
  };
  // LayerNorm affine parameters, gate bias and the pair-bias weight block,
  // staged through LDS: one element of the three vectors and one 16-byte
  // vector of the block per thread. issue_params() starts the loads (their
  // pointer is chosen per wave, so no load waits on another), and
  // commit_params() writes them to LDS once they have arrived.
  constexpr int WZV = 16 * D * ES / 16;  // 16-byte vectors of the pair-bias block
  static_assert(3 * D <= NT && WZV <= NT, "one parameter load per thread");
  const int pwhich = __builtin_amdgcn_readfirstlane(tid / D);  // 0 gamma, 1 beta, 2 gate bias (D % 64 == 0)
  float pv = 0.f;
  uint4 wzv = make_uint4(0, 0, 0, 0);
  auto issue_params = [&]() {
    if (pwhich < 3) {
      const void *src = pwhich == 0 ? a.gamma : (pwhich == 1 ? a.beta : a.bg);
      pv = bf2f(reinterpret_cast<const uint16_t *>(src)[tid - pwhich * D]);
    }
    if (tid < WZV) wzv = ldg<uint4>(reinterpret_cast<const char *>(W + (size_t)4 * D * D) + 16 * tid);
  };
  auto commit_params = [&]() {
    if (pwhich < 3) vec_s[pwhich][tid - pwhich * D] = pv;
    if (tid < WZV) {
      const int e = tid * (16 / ES);  // first element of this vector; rows are whole vectors
      *reinterpret_cast<uint4 *>(&wz_s[(e / D) * PITCH + e % D]) = wzv;
    }
  };

  // ---- LayerNorm thread mapping: TPP threads per position, EPT channels each
  const int lpos = tid / TPP, lpart = tid % TPP;

  auto load_tile = [&](int tile, uint4 (&pre)[NV], uint32_t &mpre) {
    const int bi_row = tile / nch, chunk = tile - bi_row * nch;
    const int j = chunk * TILE + lpos;
    // element (b, i, j) of pair_repr and the mask; ending-node reads (b, j, i)
    const int bb = bi_row / N;
    const size_t at = a.transposed ? ((size_t)bb * N + j) * N + (bi_row - bb * N) : (size_t)bi_row * N + j;
    mpre = (j < N && lpart == 0) ? a.mask[at] : 0u;
    if (j < N) {
      const char *src = reinterpret_cast<const char *>(a.P) + at * D * ES + lpart * EPT * ES;
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
    for (int e = 0; e < EPT; ++e) v[e] = (e & 1) ? bfhi(w32[e >> 1]) : bflo(w32[e >> 1]);
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < EPT; ++e) s += v[e];
    s = group_sum<TPP>(s);
    const float mean = s * (1.0f / D);
    float q = 0.f;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const float dv = v[e] - mean;
      q += dv * dv;
    }
    q = group_sum<TPP>(q);
    const float rstd = rsqrtf(q * (1.0f / D) + a.eps);
    const float scale = (j < N) ? rstd : 0.f;  // padding positions (j >= N) become zero rows
    const float bmul = (j < N) ? 1.f : 0.f;
    const float *gam = &vec_s[0][lpart * EPT];
    const float *bet = &vec_s[1][lpart * EPT];
    T *dst = &xs[buf][lpos * PITCH + lpart * EPT];
#pragma unroll
    for (int e = 0; e < EPT; e += 8) {
      uint32_t p4[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = e + 2 * u;
        p4[u] = pack_bf16x2((v[c] - mean) * scale * gam[c] + bet[c] * bmul,
                            (v[c + 1] - mean) * scale * gam[c + 1] + bet[c + 1] * bmul);
      }
      *reinterpret_cast<uint4 *>(dst + e) = make_uint4(p4[0], p4[1], p4[2], p4[3]);
    }
  };

  // four consecutive elements at element offset `off` from a uniform base: the
  // offset stays a 32-bit byte offset, so the store adds it to the scalar base
  auto store4 = [&](T *base, uint32_t off, float v0, float v1, float v2, float v3) {
    char *dst = reinterpret_cast<char *>(base) + off * (uint32_t)ES;
    stg<uint2>(dst, make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)));
  };

  // One tile with this wave's projections starting at TYPE0 (compile time).
  // Straight-line code throughout, so on a workgroup's first tile each
  // product waits only for its own weight registers while later ones are
  // still arriving (inside a loop the compiler waits for all outstanding loads
  // before entering it).
  auto compute_tile = [&](auto type0_c, int tile, int buf) __attribute__((always_inline)) {
    constexpr int TYPE0 = decltype(type0_c)::value;
    const int bi_row = tile / nch, chunk = tile - bi_row * nch;
    const int b = bi_row / N, i = bi_row - b * N;
    const int j0 = chunk * TILE;
    float kn_run = 0.f;  // running max over positions of |k|^2 over this channel block
    float v_run = 0.f;   // running sum of v over this lane's positions
    float z_run = -INFINITY;
    static_assert(NW >= TILE / 16, "");

    // gate bias of this lane's four channels (cb*16 + 4g .. +3): the gate
    // accumulators start from it
    f32x4 bg4 = {0.f, 0.f, 0.f, 0.f};
    if constexpr (TYPE0 <= 3 && TYPE0 + TPW > 3) {
      const float4 v = *reinterpret_cast<const float4 *>(&vec_s[2][cb * 16 + 4 * g]);
      bg4 = f32x4{v.x, v.y, v.z, v.w};
    }
    // store bases of this tile (uniform); lanes add 32-bit offsets
    T *const qbase = reinterpret_cast<T *>(a.q) + ((size_t)bi_row * NB + cb) * Np * 16;
    T *const kbase = reinterpret_cast<T *>(a.k) + ((size_t)bi_row * NB + cb) * Np * 16;
    T *const gbase = reinterpret_cast<T *>(a.g) + ((size_t)bi_row * NB + cb) * Np * 16;
    T *const vbase = reinterpret_cast<T *>(a.vt) + (size_t)bi_row * D * Np;

    auto products = [&](int pb, f32x4 (&acc)[TPW]) __attribute__((always_inline)) {
      // x fragments: lane (g, r16) = position pb*16 + r16, K-range [g*KQ, g*KQ+KQ)
      const T *xrow = &xs[buf][(pb * 16 + r16) * PITCH + g * KQ];
#pragma unroll
      for (int p = 0; p < TPW; ++p) acc[p] = (TYPE0 + p == 3) ? bg4 : f32x4{0.f, 0.f, 0.f, 0.f};  // gate: + bg
#pragma unroll
      for (int s0 = 0; s0 < KS; ++s0) {
        const Frag xf = as_bf16x8(*reinterpret_cast<const uint4 *>(xrow + 8 * s0));
#pragma unroll
        for (int p = 0; p < TPW; ++p) {
          if (TYPE0 + p == 2)
            acc[p] = mfma(xf, wf[p][s0], acc[p]);  // v: rows = positions
          else
            acc[p] = mfma(wf[p][s0], xf, acc[p]);  // q, k, gate: rows = channels
        }
      }
    };
    auto epilogue = [&](int pb, const f32x4 (&acc)[TPW]) __attribute__((always_inline)) {
      const T *xrow = &xs[buf][(pb * 16 + r16) * PITCH + g * KQ];  // for the pair-bias block
      const int jcol = j0 + pb * 16 + r16;  // position of this lane's column (q/k/gate tiles)
#pragma unroll
      for (int p = 0; p < TPW; ++p) {
        const int type = TYPE0 + p;
        const f32x4 c = acc[p];
        const uint32_t toff = (uint32_t)(jcol * 16 + 4 * g);  // q/k/gate tiles: [b][i][c/16][j][16]
        if (type == 2) {
          // v^T per head, [b][i][t][u][j] (t * DH + u = channel): lane (g, r16)
          // holds channel cb*16 + r16 of positions 4g..4g+3; staged in LDS
          // and stored after the tile's four blocks
          *reinterpret_cast<uint2 *>(&vst_s[wave][r16 * VPITCH + pb * 16 + 4 * g]) =
              make_uint2(pack_bf16x2(c[0], c[1]), pack_bf16x2(c[2], c[3]));
          v_run += (c[0] + c[1]) + (c[2] + c[3]);  // positions j >= N hold v = 0
        } else if (type == 0) {
          store4(qbase, toff, c[0] * a.qscale, c[1] * a.qscale, c[2] * a.qscale, c[3] * a.qscale);
        } else if (type == 1) {
          store4(kbase, toff, c[0], c[1], c[2], c[3]);
          kn_run = fmaxf(kn_run, group4_sum(c[0] * c[0] + c[1] * c[1] + c[2] * c[2] + c[3] * c[3]));
        } else {
          // sigmoid of (Wg x + bg): the bias is already in the accumulator
          store4(gbase, toff, fast_rcp(1.f + fast_exp2(-c[0] * kLog2e)), fast_rcp(1.f + fast_exp2(-c[1] * kLog2e)),
                 fast_rcp(1.f + fast_exp2(-c[2] * kLog2e)), fast_rcp(1.f + fast_exp2(-c[3] * kLog2e)));
        }
      }
      if (wave == pb) {
        // pair bias of this 16-position block, on wave pb (spread over the
        // SIMDs): rows = positions, column r16 = head
        const T *zrow = &wz_s[r16 * PITCH + g * KQ];
        f32x4 accz = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s0 = 0; s0 < KS; ++s0)
          accz = mfma(as_bf16x8(*reinterpret_cast<const uint4 *>(xrow + 8 * s0)),
                      as_bf16x8(*reinterpret_cast<const uint4 *>(zrow + 8 * s0)), accz);
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
    };
    static_assert(TILE / 16 == 4, "four 16-position blocks per tile");
    // software pipeline over the four blocks: the products of block pb + 1
    // go to the matrix cores before the epilogue of block pb, which then
    // finds its results ready
    f32x4 accA[TPW], accB[TPW];
    products(0, accA);
    products(1, accB);
    epilogue(0, accA);
    products(2, accA);
    epilogue(1, accB);
    products(3, accB);
    epilogue(2, accA);
    epilogue(3, accB);

    if constexpr (TYPE0 <= 2 && TYPE0 + TPW > 2) {
      // v^T rows of this wave's channel block: 128 contiguous bytes per
      // channel, 16 per lane (each wave reads back only what it wrote)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int piece = lane + 64 * hh, row = piece >> 3, col = (piece & 7) * 8;
        const uint4 v = *reinterpret_cast<const uint4 *>(&vst_s[wave][row * VPITCH + col]);
        stg<uint4>(reinterpret_cast<char *>(vbase) + ((size_t)(cb * 16 + row) * Np + j0 + col) * ES, v);
      }
    }
    // per-chunk sums of v (a fixed summation order: deterministic)
    if (TYPE0 <= 2 && TYPE0 + TPW > 2) {
      const float sv = group4_sum(v_run);
      if (g == 0) a.vsum[((size_t)bi_row * nch + chunk) * D + cb * 16 + r16] = sv;
    }
    // per-chunk maxima
    if (TYPE0 <= 1 && TYPE0 + TPW > 1) {
      const float m = row16_max(kn_run);
      if (lane == 0) a.kmax[((size_t)bi_row * NB + cb) * nch + chunk] = m;
    }
    // the chunk maximum of the bias combines the blocks of waves 0..3 through LDS
    if (wave < TILE / 16) {
      const float m = group4_max(z_run);
      if (g == 0) zpart_s[wave][r16] = m;
    }
    lds_barrier();
    if (wave == 0 && lane < H) {
      float m = zpart_s[0][lane];
#pragma unroll
      for (int q = 1; q < TILE / 16; ++q) m = fmaxf(m, zpart_s[q][lane]);
      a.zmax[((size_t)(b * H + lane) * nch + chunk) * N + i] = m;
    }
  };

  auto compute = [&](int tile, int buf) __attribute__((always_inline)) {
    if constexpr (TPW == 4) {
      compute_tile(std::integral_constant<int, 0>{}, tile, buf);
    } else {
      if (type0 == 0)
        compute_tile(std::integral_constant<int, 0>{}, tile, buf);
      else
        compute_tile(std::integral_constant<int, 2>{}, tile, buf);
    }
  };

  int tile = blockIdx.x;
  if (tile >= a.tiles) return;
  const int G = gridDim.x;
  if constexpr (ONE) {
    // the weight loads go out between the parameter loads and their LDS
    // writes: products start as their own weights arrive
    uint4 pre[NV];
    uint32_t mpre;
    load_tile(tile, pre, mpre);
    issue_params();
    load_weights();
    commit_params();
    lds_barrier();
    layer_norm_to_lds(tile, pre, mpre, 0);
    lds_barrier();
    compute(tile, 0);
  } else {
    // HBM-bound: pair_repr and the mask are prefetched two tiles ahead,
    // alternately into A and B
    uint4 preA[NV], preB[NV];
    uint32_t mA, mB = 0;
    load_tile(tile, preA, mA);
    if (tile + G < a.tiles) load_tile(tile + G, preB, mB);
    issue_params();
    commit_params();
    load_weights();
    lds_barrier();
    layer_norm_to_lds(tile, preA, mA, 0);
    lds_barrier();
    if (tile + 2 * G < a.tiles) load_tile(tile + 2 * G, preA, mA);
    compute(tile, 0);
#pragma unroll 1
    for (tile += G; tile < a.tiles; tile += 2 * G) {
      layer_norm_to_lds(tile, preB, mB, 1);
      lds_barrier();
      if (tile + 2 * G < a.tiles) load_tile(tile + 2 * G, preB, mB);
      compute(tile, 1);
      if (tile + G >= a.tiles) break;
      layer_norm_to_lds(tile + G, preA, mA, 0);
      lds_barrier();
      if (tile + 3 * G < a.tiles) load_tile(tile + 3 * G, preA, mA);
      compute(tile + G, 0);
    }
  }
}

template <int D, int DH>
static hipError_t launch_k1_t(const K1Args &a, int grid, hipStream_t s) {
  if (a.tiles <= grid)
    hipLaunchKernelGGL((k1_ln_proj<D, DH, true>), dim3(a.tiles), dim3(K1Shape<D>::THREADS), 0, s, a);
  else
    hipLaunchKernelGGL((k1_ln_proj<D, DH, false>), dim3(grid), dim3(K1Shape<D>::THREADS), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_k1(int dtype, int D, int dh, const K1Args &a, int grid, hipStream_t s) {
  if (dtype != TRI_ATTN_BF16) return hipErrorInvalidValue;  // float32: launch_k1_split
#define TRI_K1_CASE(DD, HH) \
  if (D == DD && dh == HH) return launch_k1_t<DD, HH>(a, grid, s);
  TRI_K1_CASE(128, 16)
  TRI_K1_CASE(128, 32)
  TRI_K1_CASE(64, 16)
  TRI_K1_CASE(64, 32)
#undef TRI_K1_CASE
  return hipErrorInvalidValue;
}

int k1_blocks_per_cu(int dtype, int D, int dh) {
  int n = 0;
  if (dtype != TRI_ATTN_BF16) return 1;
#define TRI_K1_OCC(DD, HH)                                                                                    \
  if (D == DD && dh == HH &&                                                                                  \
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k1_ln_proj<DD, HH, false>, K1Shape<DD>::THREADS, 0) != \
          hipSuccess)                                                                                         \
    n = 1;
  TRI_K1_OCC(128, 16)
  TRI_K1_OCC(128, 32)
  TRI_K1_OCC(64, 16)
  TRI_K1_OCC(64, 32)
#undef TRI_K1_OCC
  return n > 0 ? n : 1;
}

bool supported(int D, int dh) { return (D == 64 || D == 128) && (dh == 16 || dh == 32); }

}  // namespace tpa

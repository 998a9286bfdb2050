// Kernel 1 for float32 tensors: LayerNorm of the pair representation and the
// fused q | k | v | gate | pair-bias projection (Kimi-K2.6 / l2_p6 transcript:
// the LayerNorm and projection steps of its forward listing and its layer
// list; FW-GLM-5-1 / l2_p6: the LayerNorm and linear kernels), with every
// float32 product formed on the bf16 matrix cores.
//
// Split products. Each float32 operand is written as three bf16 numbers,
// a = a1 + a2 + a3 exactly (split3 in device_common.h). The product a*b is
// summed as the six terms a_i*b_j with i + j <= 4; the three dropped terms are
// at most 2^-24 |a b| each, and every kept term is an exact bf16 x bf16
// product accumulated in float32 by the matrix cores, so the result is as
// accurate as a float32 GEMM (the six-product scheme of Henry, Tang and
// Heinecke, "Leveraging the bfloat16 Artificial Intelligence Datatype For
// Higher-Precision Computations", ARITH 2019). A 16x16x32 block of work takes
// six bf16 16x16x32 MFMAs instead of eight float32 16x16x4 ones: about 2.4x
// fewer matrix-core cycles at the rates gfx950 runs them.
//
// Work item: a tile of 64 consecutive positions (b, i, j0..j0+63) of one row
// and one half of the projections: half 0 computes q, k and the pair bias,
// half 1 v and the gate. A workgroup keeps its half for its whole life, so
// the half's weights (three bf16 planes, fragment order) stay in registers:
// wave w owns channel block w % NB of TPW projections. Each workgroup walks
// the tiles of its half; the two workgroups of a tile sit on the same XCD when
// the grid allows it, so the second read of the tile's pair_repr hits L2.
//
//  1. LayerNorm (fp32 statistics, two-pass in registers), 8 lanes per
//     position; the normalised row goes to LDS as its three bf16 parts. A
//     workgroup's first two tiles are normalised together before their
//     products; later tiles' pair_repr and mask are prefetched one ahead.
//  2. Products: six MFMAs per step into two accumulators per projection (the
//     three small terms, then the three large), so consecutive MFMAs are
//     independent; the four 16-position blocks run as a software pipeline.
//  3. Epilogues as in the bf16 kernel: q pre-scaled by log2(e)/sqrt(d), k,
//     gate = sigmoid(+bias) as [b][i][c/16][j][16] (with d = 32, k instead
//     as its three bf16 parts in kernel 2's fragment order, so that kernel 2
//     does not split every key it loads); v transposed per head
//     [b][i][t][u][j]; the pair bias z*log2(e) with the mask folded in as
//     [b][t][i][j]; per-64-key-chunk maxima of the bias and of |k|^2 per
//     16-channel block, and per-chunk sums of v.
#include <type_traits>

#include "device_common.h"
#include "tri_attn.h"
#include "tri_attn_internal.h"

namespace tpa {

template <int D>
struct K1SplitShape {
  static constexpr int NB = D / 16;      // 16-channel blocks per projection
  static constexpr int TPW = NB / 4;     // projections per wave (of the half's two)
  static constexpr int NW = 2 * NB / TPW;
  static constexpr int THREADS = NW * 64;
  static_assert(NW == 8, "eight waves");
};

template <int D, int DH>
__global__ __launch_bounds__(512) void k1_ln_proj_split(K1Args a) {
  constexpr int H = D / DH;
  constexpr bool KSPLIT = DH == 32;  // k is stored pre-split for kernel 2's split score products
  constexpr int NB = K1SplitShape<D>::NB;
  constexpr int TPW = K1SplitShape<D>::TPW;
  constexpr int NT = K1SplitShape<D>::THREADS;
  constexpr int KQ = D / 4;          // K elements per lane group (lane group g owns [g*KQ, g*KQ+KQ))
  constexpr int KS = D / 32;         // MFMA steps over K = D
  constexpr int PITCH = D + 8;       // LDS row pitch (bf16 elements), 16-byte pad against bank conflicts
  constexpr int TPP = NT / 64;       // LayerNorm threads per position
  constexpr int EPT = D / TPP;       // LayerNorm elements per thread
  constexpr int NV = EPT / 4;        // 16-byte loads per thread per tile
  constexpr int TILE = kChunk;
  constexpr int PLANE = TILE * PITCH;
  static_assert(EPT % 8 == 0, "");

  __shared__ __align__(16) uint16_t xs[2][3][PLANE];  // LayerNorm output, three bf16 parts
  __shared__ uint8_t mask_s[2][TILE];                 // the tile's mask bytes (0 also for j >= N)
  __shared__ float vec_s[3][D];                       // gamma, beta, gate bias
  __shared__ __align__(16) uint16_t wz_s[3][16 * PITCH];  // pair-bias weight block, three parts (rows >= h zero)
  __shared__ float zpart_s[2][TILE / 16][16];         // per-block maxima of the pair bias of a tile (per buffer:
                                                      // a workgroup's first two tiles have no barrier between them)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int N = a.N, Np = a.Np, nch = a.nchunk;

  // workgroup -> (half, slot): with a multiple of 8 workgroups per half, the
  // two halves of a slot are 8 apart and so on the same XCD
  const int GH = gridDim.x >> 1;
  const int wg = blockIdx.x;
  const bool paired = (GH & 7) == 0;
  const int half = paired ? ((wg >> 3) & 1) : (wg & 1);
  const int slot = paired ? ((wg & 7) | ((wg >> 4) << 3)) : (wg >> 1);
  const int cb = wave % NB;
  const int type0 = half * 2 + (wave / NB) * TPW;  // first projection of this wave (0 q, 1 k, 2 v, 3 gate)

  // ---- weights: lane (g, r16) holds row r16 of the block, K-range [g*KQ, g*KQ+KQ), three parts
  bf16x8 wf[TPW][KS][3];
  auto load_weights = [&]() {
    const char *wsrc = reinterpret_cast<const char *>(a.Ws) + (size_t)lane * 16;
    // contraction step outer, in the order the MFMAs consume them
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int p = 0; p < TPW; ++p)
#pragma unroll
        for (int q = 0; q < 3; ++q)
          wf[p][s][q] = as_bf16x8(ldg<uint4>(wsrc + q * a.ws_plane + ((size_t)((type0 + p) * NB + cb) * KS + s) * 1024));
  };
  // LayerNorm parameters and gate bias (one element per thread) and the
  // pair-bias weight block (one 16-byte vector of four floats per thread,
  // split into its parts), staged through LDS
  constexpr int WZV = 16 * D / 4;
  static_assert(3 * D <= NT && WZV <= NT, "one parameter load per thread");
  const int pwhich = __builtin_amdgcn_readfirstlane(tid / D);  // 0 gamma, 1 beta, 2 gate bias
  float pv = 0.f;
  float4 wzv = make_float4(0.f, 0.f, 0.f, 0.f);
  auto issue_params = [&]() {
    if (pwhich < 3) {
      const float *src = reinterpret_cast<const float *>(pwhich == 0 ? a.gamma : (pwhich == 1 ? a.beta : a.bg));
      pv = src[tid - pwhich * D];
    }
    if (tid < WZV) wzv = ldg<float4>(reinterpret_cast<const float *>(a.W) + (size_t)4 * D * D + 4 * tid);
  };
  auto commit_params = [&]() {
    if (pwhich < 3) vec_s[pwhich][tid - pwhich * D] = pv;
    if (tid < WZV) {
      const int e = tid * 4, row = e / D, col = e % D;
      uint32_t p1[2], p2[2], p3[2];
      split3(wzv.x, wzv.y, p1[0], p2[0], p3[0]);
      split3(wzv.z, wzv.w, p1[1], p2[1], p3[1]);
      *reinterpret_cast<uint2 *>(&wz_s[0][row * PITCH + col]) = make_uint2(p1[0], p1[1]);
      *reinterpret_cast<uint2 *>(&wz_s[1][row * PITCH + col]) = make_uint2(p2[0], p2[1]);
      *reinterpret_cast<uint2 *>(&wz_s[2][row * PITCH + col]) = make_uint2(p3[0], p3[1]);
    }
  };

  // ---- LayerNorm thread mapping: TPP threads per position, EPT channels each
  const int lpos = tid / TPP, lpart = tid % TPP;

  auto load_tile = [&](int tile, float4 (&pre)[NV], uint32_t &mpre) {
    const int bi_row = tile / nch, chunk = tile - bi_row * nch;
    const int j = chunk * TILE + lpos;
    // element (b, i, j) of pair_repr and the mask; ending-node reads (b, j, i)
    const int bb = bi_row / N;
    const size_t at = a.transposed ? ((size_t)bb * N + j) * N + (bi_row - bb * N) : (size_t)bi_row * N + j;
    mpre = (j < N && lpart == 0) ? a.mask[at] : 0u;
    if (j < N) {
      const float *src = reinterpret_cast<const float *>(a.P) + at * D + lpart * EPT;
#pragma unroll
      for (int v = 0; v < NV; ++v) pre[v] = ldg<float4>(src + 4 * v);
    } else {
#pragma unroll
      for (int v = 0; v < NV; ++v) pre[v] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };

  auto layer_norm_to_lds = [&](int tile, const float4 (&pre)[NV], uint32_t mpre, int buf) {
    const int bi_row = tile / nch, chunk = tile - bi_row * nch;
    const int j = chunk * TILE + lpos;
    if (lpart == 0) mask_s[buf][lpos] = (uint8_t)mpre;
    const float *v = reinterpret_cast<const float *>(pre);
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
    const int off = lpos * PITCH + lpart * EPT;
#pragma unroll
    for (int e = 0; e < EPT; e += 8) {
      uint32_t p1[4], p2[4], p3[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = e + 2 * u;
        split3((v[c] - mean) * scale * gam[c] + bet[c] * bmul, (v[c + 1] - mean) * scale * gam[c + 1] + bet[c + 1] * bmul,
               p1[u], p2[u], p3[u]);
      }
      *reinterpret_cast<uint4 *>(&xs[buf][0][off + e]) = make_uint4(p1[0], p1[1], p1[2], p1[3]);
      *reinterpret_cast<uint4 *>(&xs[buf][1][off + e]) = make_uint4(p2[0], p2[1], p2[2], p2[3]);
      *reinterpret_cast<uint4 *>(&xs[buf][2][off + e]) = make_uint4(p3[0], p3[1], p3[2], p3[3]);
    }
  };

  // four consecutive floats at element offset `off` from a uniform base
  auto store4 = [&](float *base, uint32_t off, float v0, float v1, float v2, float v3) {
    stg<float4>(reinterpret_cast<char *>(base) + off * 4u, make_float4(v0, v1, v2, v3));
  };
  auto lds16 = [&](const uint16_t *p) { return as_bf16x8(*reinterpret_cast<const uint4 *>(p)); };

  // One tile with this wave's projections starting at TYPE0 (compile time).
  auto compute_tile = [&](auto type0_c, int tile, int buf) __attribute__((always_inline)) {
    constexpr int TYPE0 = decltype(type0_c)::value;
    constexpr bool HALF0 = TYPE0 < 2;
    const int bi_row = tile / nch, chunk = tile - bi_row * nch;
    const int b = bi_row / N, i = bi_row - b * N;
    const int j0 = chunk * TILE;
    float kn_run = 0.f;  // running max over positions of |k|^2 over this channel block
    float v_run = 0.f;   // running sum of v over this lane's positions
    float z_run = -INFINITY;

    f32x4 bg4 = {0.f, 0.f, 0.f, 0.f};  // gate bias of this lane's four channels: the gate accumulators start there
    if constexpr (TYPE0 <= 3 && TYPE0 + TPW > 3) {
      const float4 v = *reinterpret_cast<const float4 *>(&vec_s[2][cb * 16 + 4 * g]);
      bg4 = f32x4{v.x, v.y, v.z, v.w};
    }
    float *const qbase = reinterpret_cast<float *>(a.q) + ((size_t)bi_row * NB + cb) * Np * 16;
    float *const kbase = reinterpret_cast<float *>(a.k) + ((size_t)bi_row * NB + cb) * Np * 16;
    char *const ksp = reinterpret_cast<char *>(a.k) + ((size_t)bi_row * H + (cb >> 1)) * 3 * Np * 64;
    float *const gbase = reinterpret_cast<float *>(a.g) + ((size_t)bi_row * NB + cb) * Np * 16;
    float *const vbase = reinterpret_cast<float *>(a.vt) + (size_t)bi_row * D * Np;

    // acc[p][0] takes the three large terms, acc[p][1] the three small ones
    auto products = [&](int pb, f32x4 (&acc)[TPW][2]) __attribute__((always_inline)) {
      const int xo = (pb * 16 + r16) * PITCH + g * KQ;
#pragma unroll
      for (int p = 0; p < TPW; ++p) {
        acc[p][0] = (TYPE0 + p == 3) ? bg4 : f32x4{0.f, 0.f, 0.f, 0.f};
        acc[p][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 x1 = lds16(&xs[buf][0][xo + 8 * s]);
        const bf16x8 x2 = lds16(&xs[buf][1][xo + 8 * s]);
        const bf16x8 x3 = lds16(&xs[buf][2][xo + 8 * s]);
        // (weight part, x part) pairs: small terms (3,1) (2,2) (1,3), large (2,1) (1,2) (1,1)
        auto mm = [&](int p, const bf16x8 &w, const bf16x8 &x, f32x4 &c) __attribute__((always_inline)) {
          if (TYPE0 + p == 2)
            c = mfma(x, w, c);  // v: rows = positions
          else
            c = mfma(w, x, c);  // q, k, gate: rows = channels
        };
#pragma unroll
        for (int p = 0; p < TPW; ++p) mm(p, wf[p][s][2], x1, acc[p][1]);
#pragma unroll
        for (int p = 0; p < TPW; ++p) mm(p, wf[p][s][1], x1, acc[p][0]);
#pragma unroll
        for (int p = 0; p < TPW; ++p) mm(p, wf[p][s][1], x2, acc[p][1]);
#pragma unroll
        for (int p = 0; p < TPW; ++p) mm(p, wf[p][s][0], x2, acc[p][0]);
#pragma unroll
        for (int p = 0; p < TPW; ++p) mm(p, wf[p][s][0], x3, acc[p][1]);
#pragma unroll
        for (int p = 0; p < TPW; ++p) mm(p, wf[p][s][0], x1, acc[p][0]);
      }
    };
    auto epilogue = [&](int pb, const f32x4 (&acc)[TPW][2]) __attribute__((always_inline)) {
      const int jcol = j0 + pb * 16 + r16;  // position of this lane's column (q/k/gate tiles)
#pragma unroll
      for (int p = 0; p < TPW; ++p) {
        const int type = TYPE0 + p;
        const f32x4 c = acc[p][1] + acc[p][0];
        const uint32_t toff = (uint32_t)(jcol * 16 + 4 * g);  // q/k/gate tiles: [b][i][c/16][j][16]
        if (type == 2) {
          // v^T per head: lane (g, r16) holds channel cb*16 + r16 of positions 4g..4g+3
          store4(vbase, (uint32_t)((cb * 16 + r16) * Np + j0 + pb * 16 + 4 * g), c[0], c[1], c[2], c[3]);
          v_run += (c[0] + c[1]) + (c[2] + c[3]);  // positions j >= N hold v = 0
        } else if (type == 0) {
          store4(qbase, toff, c[0] * a.qscale, c[1] * a.qscale, c[2] * a.qscale, c[3] * a.qscale);
        } else if (type == 1) {
          if constexpr (KSPLIT) {
            // k as three bf16 parts, 1 KB per (row, head, part, 16 keys):
            // lane (G, r) of that block holds channels 8G..8G+7 of key r of
            // the head; this lane's four channels are half of one such slot,
            // and the wave's 64 lanes fill 512 contiguous bytes
            uint32_t p1[2], p2[2], p3[2];
            split3(c[0], c[1], p1[0], p2[0], p3[0]);
            split3(c[2], c[3], p1[1], p2[1], p3[1]);
            char *dst = ksp + (size_t)(jcol >> 4) * 1024 + ((2 * (cb & 1) + (g >> 1)) * 16 + r16) * 16 + (g & 1) * 8;
            stg<uint2>(dst, make_uint2(p1[0], p1[1]));
            stg<uint2>(dst + (size_t)Np * 64, make_uint2(p2[0], p2[1]));
            stg<uint2>(dst + (size_t)Np * 128, make_uint2(p3[0], p3[1]));
          } else {
            store4(kbase, toff, c[0], c[1], c[2], c[3]);
          }
          kn_run = fmaxf(kn_run, group4_sum(c[0] * c[0] + c[1] * c[1] + c[2] * c[2] + c[3] * c[3]));
        } else {
          // sigmoid of (Wg x + bg): the bias is already in the accumulator
          store4(gbase, toff, fast_rcp(1.f + fast_exp2(-c[0] * kLog2e)), fast_rcp(1.f + fast_exp2(-c[1] * kLog2e)),
                 fast_rcp(1.f + fast_exp2(-c[2] * kLog2e)), fast_rcp(1.f + fast_exp2(-c[3] * kLog2e)));
        }
      }
      if constexpr (HALF0) {
        if (wave == pb) {
          // pair bias of this 16-position block, on wave pb: rows = positions,
          // column r16 = head
          const int xo = (pb * 16 + r16) * PITCH + g * KQ;
          const int zo = r16 * PITCH + g * KQ;
          f32x4 az0 = {0.f, 0.f, 0.f, 0.f}, az1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            const bf16x8 x1 = lds16(&xs[buf][0][xo + 8 * s]), x2 = lds16(&xs[buf][1][xo + 8 * s]),
                         x3 = lds16(&xs[buf][2][xo + 8 * s]);
            const bf16x8 z1 = lds16(&wz_s[0][zo + 8 * s]), z2 = lds16(&wz_s[1][zo + 8 * s]),
                         z3 = lds16(&wz_s[2][zo + 8 * s]);
            az1 = mfma(x1, z3, az1);
            az0 = mfma(x1, z2, az0);
            az1 = mfma(x2, z2, az1);
            az0 = mfma(x2, z1, az0);
            az1 = mfma(x3, z1, az1);
            az0 = mfma(x1, z1, az0);
          }
          const f32x4 az = az1 + az0;
          if (r16 < H) {
            const int jb = j0 + pb * 16 + 4 * g;
            float z[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const bool keep = mask_s[buf][pb * 16 + 4 * g + r] != 0;
              z[r] = keep ? az[r] * kLog2e : -INFINITY;
              z_run = fmaxf(z_run, z[r]);
            }
            float *dst = a.zm + (((size_t)(b * H + r16) * N + i) * Np + jb);
            stg<float4>(dst, make_float4(z[0], z[1], z[2], z[3]));
          }
        }
      }
    };
    static_assert(TILE / 16 == 4, "four 16-position blocks per tile");
    // software pipeline over the four blocks: the products of block pb + 1
    // go to the matrix cores before the epilogue of block pb
    f32x4 accA[TPW][2], accB[TPW][2];
    products(0, accA);
    products(1, accB);
    epilogue(0, accA);
    products(2, accA);
    epilogue(1, accB);
    products(3, accB);
    epilogue(2, accA);
    epilogue(3, accB);

    // per-chunk sums of v (a fixed summation order: deterministic)
    if constexpr (TYPE0 <= 2 && TYPE0 + TPW > 2) {
      const float sv = group4_sum(v_run);
      if (g == 0) a.vsum[((size_t)bi_row * nch + chunk) * D + cb * 16 + r16] = sv;
    }
    if constexpr (TYPE0 <= 1 && TYPE0 + TPW > 1) {
      const float m = row16_max(kn_run);
      if (lane == 0) a.kmax[((size_t)bi_row * NB + cb) * nch + chunk] = m;
    }
    // the chunk maximum of the bias combines the blocks of waves 0..3 through
    // LDS (half 0: every wave of the workgroup takes this branch)
    if constexpr (HALF0) {
      if (wave < TILE / 16) {
        const float m = group4_max(z_run);
        if (g == 0) zpart_s[buf][wave][r16] = m;
      }
      lds_barrier();
      if (wave == 0 && lane < H) {
        float m = zpart_s[buf][0][lane];
#pragma unroll
        for (int q = 1; q < TILE / 16; ++q) m = fmaxf(m, zpart_s[buf][q][lane]);
        a.zmax[((size_t)(b * H + lane) * nch + chunk) * N + i] = m;
      }
    }
  };

  auto compute = [&](int tile, int buf) __attribute__((always_inline)) {
    if constexpr (TPW == 2) {
      if (type0 == 0)
        compute_tile(std::integral_constant<int, 0>{}, tile, buf);
      else
        compute_tile(std::integral_constant<int, 2>{}, tile, buf);
    } else {
      if (type0 == 0)
        compute_tile(std::integral_constant<int, 0>{}, tile, buf);
      else if (type0 == 1)
        compute_tile(std::integral_constant<int, 1>{}, tile, buf);
      else if (type0 == 2)
        compute_tile(std::integral_constant<int, 2>{}, tile, buf);
      else
        compute_tile(std::integral_constant<int, 3>{}, tile, buf);
    }
  };

  int tile = slot;
  if (tile >= a.tiles) return;  // uniform over the workgroup
  const bool two = tile + GH < a.tiles;
  float4 pre[NV], pre2[NV];
  uint32_t mpre, mpre2 = 0;
  // the first two tiles' pair_repr go out first, then the small parameters,
  // then the weights: LayerNorm waits only for its own data
  load_tile(tile, pre, mpre);
  if (two) load_tile(tile + GH, pre2, mpre2);
  issue_params();
  load_weights();
  commit_params();
  lds_barrier();
  // the first two tiles in straight-line code, both normalised before any
  // product: their eight 16-position blocks run with no barrier between the
  // tiles (one wave's late finish of the first tile holds no one up), and the
  // products wait only for their own weights (a loop would wait for every
  // outstanding load first)
  layer_norm_to_lds(tile, pre, mpre, 0);
  if (two) layer_norm_to_lds(tile + GH, pre2, mpre2, 1);
  lds_barrier();
  if (tile + 2 * GH < a.tiles) load_tile(tile + 2 * GH, pre, mpre);
  compute(tile, 0);
  if (!two) return;
  compute(tile + GH, 1);
  if (tile + 2 * GH >= a.tiles) return;
  // both buffers were read by the two tiles above: every wave must be done
  // with them before the loop overwrites buffer 0
  lds_barrier();
  int buf = 0;
#pragma unroll 1
  for (tile += 2 * GH; tile < a.tiles; tile += GH) {
    layer_norm_to_lds(tile, pre, mpre, buf);
    lds_barrier();
    if (tile + GH < a.tiles) load_tile(tile + GH, pre, mpre);
    compute(tile, buf);
    buf ^= 1;
  }
}

hipError_t launch_k1_split(int D, int dh, const K1Args &a, int grid, hipStream_t s) {
#define TRI_K1S_CASE(DD, HH)                                                                            \
  if (D == DD && dh == HH) {                                                                            \
    hipLaunchKernelGGL((k1_ln_proj_split<DD, HH>), dim3(grid), dim3(K1SplitShape<DD>::THREADS), 0, s, a); \
    return hipGetLastError();                                                                           \
  }
  TRI_K1S_CASE(128, 16)
  TRI_K1S_CASE(128, 32)
  TRI_K1S_CASE(64, 16)
  TRI_K1S_CASE(64, 32)
#undef TRI_K1S_CASE
  return hipErrorInvalidValue;
}

int k1_split_blocks_per_cu(int D, int dh) {
  int n = 0;
#define TRI_K1S_OCC(DD, HH)                                                                             \
  if (D == DD && dh == HH &&                                                                            \
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k1_ln_proj_split<DD, HH>, K1SplitShape<DD>::THREADS, \
                                                   0) != hipSuccess)                                    \
    n = 1;
  TRI_K1S_OCC(128, 16)
  TRI_K1S_OCC(128, 32)
  TRI_K1S_OCC(64, 16)
  TRI_K1S_OCC(64, 32)
#undef TRI_K1S_OCC
  return n > 0 ? n : 1;
}

}  // namespace tpa

// Backward of the training-mode forward: the gradients of L = sum(dy * y)
// with respect to pair_repr and every parameter, for the same dropout
// decisions as tri_attn_forward_train (FW-GLM-5-1 / l2_p6 transcript: the
// forward as restated, dropout on the attention weights after the softmax;
// Kimi-K2.6 / l2_p6: the module's layer list). Back-propagation runs through
// the forward's steps in reverse:
//
//   (8) y = Wo (g*o) + bo      dWo = sum dy (g*o)^T, dbo = sum dy, d(g*o) = Wo^T dy
//   gate                       dg = d(g*o) * o, do = d(g*o) * g
//   (2) g = sigmoid(.)          dgp = dg * g (1 - g): dWg, dbg, dx += Wg^T dgp
//   (7) o = sum_k a' v          da'[j,k] = do_j . v_k, dv_k = sum_j a'[j,k] do_j
//   dropout a' = a keep scale   da = da' keep scale
//   (6) softmax                 ds = a (da - sum_k a da), and sum_k a da = do_j . o_j
//   (5) masked scores           dsm = ds where the mask is set; dq = dsm k / sqrt(d),
//                               dk = dsm^T q / sqrt(d); dz[b,t,j,k] = sum_i dsm
//   (3), (4) projections        dW = d^T x, dx += W^T d for q, k, v, the gate, z
//   (1) LayerNorm               dgamma, dbeta, dP from x-hat and 1/std
//
// Everything is recomputed from the inputs in float32 (LayerNorm, the five
// projections, the attention weights with their row maximum and sum, the
// dropout decisions from the same Philox4x32-10 counters), so the backward
// needs nothing saved by the forward. Every sum over positions is split into
// fixed chunks whose partial results are added in a fixed order by a second
// pass: no atomics, the same bits on every call.
//
// All arithmetic is float32, the products (the projection GEMMs and the
// attention's score, value and gradient tiles) as split bf16 products (two
// bf16 parts per float32 operand, three 16x16x16 matrix-core products per
// float32 product, ~2^-16 relative error). The dropout decisions are
// computed once into a bit array (one generator call per four keys) that
// every attention step reads; the backward's copy of the pair bias carries
// the mask (FILL where masked), and query columns without a valid key are
// flagged once, so no attention step reads the mask itself.
#include "device_common.h"
#include "tri_attn.h"
#include "tri_attn_internal.h"

#include <algorithm>
#include <type_traits>

namespace tpa {

// Float32 products as split bf16 products: a = ah + al with ah = bf16(a) and
// al = bf16(a - ah) (a - ah is exact in float32), and a b ~ ah bh + ah bl +
// al bh, three bf16 16x16x16 products (each ~0.6 of a float32 16x16x4
// product's cost here, for 4x the contraction); the dropped al bl and the
// remainders a - ah - al are ~2^-16 relative. The lane layout is the float32
// product's: lane group g holds contraction elements 4g..4g+3.
struct Split4 {
  bf16x4 h, l;
};
__device__ __forceinline__ Split4 split4(float a, float b, float c, float d) {
  const uint32_t h0 = pack_bf16x2(a, b), h1 = pack_bf16x2(c, d);
  const uint32_t l0 = pack_bf16x2(a - bflo(h0), b - bfhi(h0)), l1 = pack_bf16x2(c - bflo(h1), d - bfhi(h1));
  return {__builtin_bit_cast(bf16x4, make_uint2(h0, h1)), __builtin_bit_cast(bf16x4, make_uint2(l0, l1))};
}
__device__ __forceinline__ f32x4 mma_split(const Split4 &a, const Split4 &b, f32x4 c) {
  c = mfma(a.h, b.h, c);
  c = mfma(a.h, b.l, c);
  return mfma(a.l, b.h, c);
}
// four consecutive bf16 of a hi plane and of its lo plane
__device__ __forceinline__ Split4 lds_split4(const uint16_t *hi, const uint16_t *lo) {
  return {__builtin_bit_cast(bf16x4, *reinterpret_cast<const uint2 *>(hi)),
          __builtin_bit_cast(bf16x4, *reinterpret_cast<const uint2 *>(lo))};
}

// ------------------------------------------------------------------ products
// C[z][m][n] = sum over k in chunk z of A[m, k] B[k, n]; A(m, k) at
// A[m*sam + k*sak], B(k, n) at B[k*sbk + n*sbn], C(z, m, n) at
// C[z*scz + m*scm + n]. 64x64 tile per workgroup as split products, K in
// steps of 16 through LDS, loads laid out along the contiguous index.
struct GemmArgs {
  const void *A, *B;
  float *C;
  long long M, N, K, kchunk;
  long long sam, sak, sbk, sbn, scz, scm;
  long long nz;  // K chunks
};

// four consecutive elements (the first one's index a multiple of 4), as floats
template <typename T>
__device__ __forceinline__ float4 ld4(const void *p, size_t i) {
  if constexpr (is_bf16<T>::value) {
    const uint2 u = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(p) + i);
    return make_float4(bflo(u.x), bfhi(u.x), bflo(u.y), bfhi(u.y));
  } else {
    return *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(p) + i);
  }
}

template <typename TA, typename TB>
__global__ __launch_bounds__(256) void bwd_gemm(GemmArgs g) {
  // A and B tiles of one 16-deep K slice as split bf16 planes ([0] hi, [1]
  // lo), each row a tile row (m, or n) with its 16 k contiguous, so a lane
  // reads its four contraction elements 4g..4g+3 as one 8-byte load per plane
  constexpr int PK = 16 + 4;  // row pitch (elements)
  __shared__ __align__(16) uint16_t As[2][64 * PK];
  __shared__ __align__(16) uint16_t Bs[2][64 * PK];
  const int tid = threadIdx.x;
  // one-dimensional grid over tiles (K chunk, row block, column block),
  // column block fastest, mapped XCD-aware: workgroup v runs on XCD v % 8,
  // and each XCD takes a contiguous range of that order, so the workgroups
  // sharing a row block of A (or, split over K, one chunk's A and B) run on
  // one XCD and read them from memory into its L2 once
  const long long ncb = (g.N + 63) / 64, ntile = ((g.M + 63) / 64) * ncb;
  const long long total = ntile * g.nz, v = blockIdx.x;
  const long long w8 = (total / 8) * 8;
  const long long lin = v < w8 ? (v & 7) * (w8 / 8) + (v >> 3) : v;
  const long long zc = lin / ntile, tile = lin - zc * ntile;
  const long long m0 = (tile / ncb) * 64, n0 = (tile % ncb) * 64;
  const long long kb = zc * g.kchunk;
  const long long ke = min(kb + g.kchunk, g.K);
  // wave w computes the 32 x 32 quadrant (w / 2, w % 2) as 2 x 2 tiles of
  // split products (three bf16 16x16x16 products per float32 product)
  const int lane = tid & 63, wave = tid >> 6, g4 = lane >> 4, r16 = lane & 15;
  const int wm = wave >> 1, wn = wave & 1;
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const bool a_m_contig = g.sam == 1, b_n_contig = g.sbn == 1;
  // one operand's 64 x 16 slice: each thread loads four elements (load) and
  // writes their two bf16 parts to the planes (put). Contiguous along k: the
  // four threads of a tile row read its 16 k as one 64-byte piece (one 16-
  // or 8-byte load each) and each writes its four k as one 8-byte store per
  // plane. Contiguous along the row index, float32: thread (row, k quad) reads
  // its four k as four 4-byte loads, which the wave's 64 consecutive rows make
  // coalesced, and writes them the same way. Contiguous along the row index,
  // bf16 (2-byte loads would be too narrow): four consecutive rows of one k
  // in one load, written to the planes as scattered 2-byte stores.
  auto load = [&](auto ta, const void *X, long long s_t, long long s_k, long long T, long long t0, bool t_contig,
                  long long k0) {
    using TX = decltype(ta);
    if (t_contig && is_bf16<TX>::value) {
      const int lin = (tid & 15) * 4, oth = tid >> 4;  // four rows, one k
      const long long tt = t0 + lin, kk = k0 + oth;
      if (tt + 3 < T && kk < ke) return ld4<TX>(X, (size_t)(tt * s_t + kk * s_k));
      float t4[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) t4[c] = (tt + c < T && kk < ke) ? ld_elem<TX>(X, (size_t)((tt + c) * s_t + kk * s_k)) : 0.f;
      return make_float4(t4[0], t4[1], t4[2], t4[3]);
    }
    const int r = t_contig ? (tid & 63) : (tid >> 2), kq = t_contig ? (tid >> 6) : (tid & 3);
    const long long tt = t0 + r, kk = k0 + 4 * kq;
    if (!t_contig && tt < T && kk + 3 < ke) return ld4<TX>(X, (size_t)(tt * s_t + kk * s_k));
    float t4[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
      t4[c] = (tt < T && kk + c < ke) ? ld_elem<TX>(X, (size_t)(tt * s_t + (kk + c) * s_k)) : 0.f;
    return make_float4(t4[0], t4[1], t4[2], t4[3]);
  };
  auto put = [&](auto ta, float4 v, bool t_contig, uint16_t (*pl)[64 * PK]) {
    using TX = decltype(ta);
    const Split4 sp = split4(v.x, v.y, v.z, v.w);
    const uint2 hv = __builtin_bit_cast(uint2, sp.h), lv = __builtin_bit_cast(uint2, sp.l);
    if (t_contig && is_bf16<TX>::value) {
      const int lin = (tid & 15) * 4, oth = tid >> 4;
      const uint32_t hw[2] = {hv.x, hv.y}, lw[2] = {lv.x, lv.y};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        pl[0][(lin + c) * PK + oth] = (uint16_t)(hw[c >> 1] >> (16 * (c & 1)));
        pl[1][(lin + c) * PK + oth] = (uint16_t)(lw[c >> 1] >> (16 * (c & 1)));
      }
      return;
    }
    const int r = t_contig ? (tid & 63) : (tid >> 2), kq = t_contig ? (tid >> 6) : (tid & 3);
    *reinterpret_cast<uint2 *>(&pl[0][r * PK + 4 * kq]) = hv;
    *reinterpret_cast<uint2 *>(&pl[1][r * PK + 4 * kq]) = lv;
  };
  // the next slice's elements are loaded into registers while the current
  // one is multiplied; the barriers wait for LDS traffic only, so those
  // loads stay in flight across them
  float4 va = load(TA{}, g.A, g.sam, g.sak, g.M, m0, a_m_contig, kb);
  float4 vb = load(TB{}, g.B, g.sbn, g.sbk, g.N, n0, b_n_contig, kb);
  for (long long k0 = kb; k0 < ke; k0 += 16) {
    put(TA{}, va, a_m_contig, As);
    put(TB{}, vb, b_n_contig, Bs);
    lds_barrier();
    if (k0 + 16 < ke) {
      va = load(TA{}, g.A, g.sam, g.sak, g.M, m0, a_m_contig, k0 + 16);
      vb = load(TB{}, g.B, g.sbn, g.sbk, g.N, n0, b_n_contig, k0 + 16);
    }
    Split4 av[2], bv[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int o = (32 * wm + 16 * i + r16) * PK + 4 * g4;
      av[i] = lds_split4(&As[0][o], &As[1][o]);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int o = (32 * wn + 16 * j + r16) * PK + 4 * g4;
      bv[j] = lds_split4(&Bs[0][o], &Bs[1][o]);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mma_split(av[i], bv[j], acc[i][j]);
    lds_barrier();
  }
  // lane: rows 4 g4 + r, column r16 of each tile
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const long long n = n0 + 32 * wn + 16 * j + r16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const long long m = m0 + 32 * wm + 16 * i + 4 * g4 + r;
        if (m < g.M && n < g.N) g.C[(size_t)(zc * g.scz + m * g.scm + n)] = acc[i][j][r];
      }
    }
}

// out[e] = sum over z of part[z*stride + e], z = 0..nz-1 in order
// (sixteen loads in flight at a time, added in the same order z = 0, 1, ...)
__global__ __launch_bounds__(256) void bwd_reduce(const float *part, long long n, int nz, long long stride,
                                                   float *out) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  float s = 0.f;
  int z = 0;
  for (; z + 16 <= nz; z += 16) {
    float v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = part[(size_t)((z + u) * stride + e)];
#pragma unroll
    for (int u = 0; u < 16; ++u) s += v[u];
  }
  for (; z < nz; ++z) s += part[(size_t)(z * stride + e)];
  out[e] = s;
}

// part[blk][c] = sum over positions p of block blk of X[p*ldx + c] (c < ncol):
// the block's 1024 threads cover 1024 / ncol groups of positions (each thread
// one column), eight independent partial sums per thread, then the groups
// are added in a fixed order through LDS
template <typename T>
__global__ __launch_bounds__(1024) void bwd_colsum(const void *X, long long P, int ncol, long long ldx,
                                                    long long per_blk, float *part) {
  __shared__ float red[1024];
  const long long p0 = (long long)blockIdx.x * per_blk, p1 = min(p0 + per_blk, P);
  const int ng = 1024 / ncol, grp = threadIdx.x / ncol, c = threadIdx.x - grp * ncol;
  float s = 0.f;
  if (grp < ng) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    long long p = p0 + grp;
    for (; p + 7 * ng < p1; p += 8 * ng) {
#pragma unroll
      for (int u = 0; u < 8; ++u) acc[u] += ld_elem<T>(X, (size_t)((p + u * ng) * ldx + c));
    }
    for (; p < p1; p += ng) acc[0] += ld_elem<T>(X, (size_t)(p * ldx + c));
    s = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
  }
  red[threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x < ncol) {
    float t = 0.f;
    for (int q = 0; q < ng; ++q) t += red[q * ncol + threadIdx.x];
    part[(size_t)blockIdx.x * ncol + threadIdx.x] = t;
  }
}

// ------------------------------------------------------------------ LayerNorm
// One wave per position: x-hat, 1/std and x = x-hat * gamma + beta.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_ln(const void *P, const void *gamma, const void *beta, float eps,
                                               long long npos, float *x, float *xhat, float *rstd) {
  constexpr int PER = D / 64;
  const long long p = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (p >= npos) return;
  float v[PER], s = 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    v[e] = ld_elem<T>(P, (size_t)(p * D + lane + 64 * e));
    s += v[e];
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) s += __shfl_xor(s, m, 64);
  const float mean = s / D;
  float q = 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) q += (v[e] - mean) * (v[e] - mean);
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) q += __shfl_xor(q, m, 64);
  const float r = 1.0f / sqrtf(q / D + eps);
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int c = lane + 64 * e;
    const float xh = (v[e] - mean) * r;
    xhat[p * D + c] = xh;
    x[p * D + c] = xh * ld_elem<T>(gamma, c) + ld_elem<T>(beta, c);
  }
  if (lane == 0) rstd[p] = r;
}

// Sum over each row of 16 lanes, every lane getting its row's sum: DPP lane
// moves on the VALU (swap neighbours, swap pairs, mirror within 8, mirror
// within 16).
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_mov<0xB1>(v);
  v += dpp_mov<0x4E>(v);
  v += dpp_mov<0x141>(v);
  return v + dpp_mov<0x140>(v);
}

// LayerNorm backward per position: 16 lanes per position (four channels per
// lane and 16-byte access), four positions per wave and step, the two sums
// over channels reduced within each row of 16 lanes; per-block partial sums
// of dx * x-hat (for dgamma) and dx (for dbeta): block blk (16 waves) covers
// positions blk*per .. ; the 64 (wave, row) partials are added in a fixed
// order.
template <typename T, int D>
__global__ __launch_bounds__(1024) void bwd_ln_back(const float *dx, const float *xhat, const float *rstd,
                                                    const void *gamma, long long npos, long long per_blk, float *dP,
                                                    float *part_g, float *part_b) {
  constexpr int PER = D / 64;  // 16-byte pieces per lane and position
  constexpr int NW = 16;
  __shared__ __align__(16) float red[2][NW * 4][D];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, pr = lane >> 4, c16 = lane & 15;
  float4 gm[PER], sg[PER], sb[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int c = 4 * c16 + 64 * e;
    gm[e] = make_float4(ld_elem<T>(gamma, c), ld_elem<T>(gamma, c + 1), ld_elem<T>(gamma, c + 2),
                        ld_elem<T>(gamma, c + 3));
    sg[e] = sb[e] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const long long p0 = (long long)blockIdx.x * per_blk, p1 = min(p0 + per_blk, npos);
  for (long long pb = p0 + 4 * wave; pb < p1; pb += 4 * NW) {
    const long long p = pb + pr;
    const bool ok = p < p1;
    float4 d[PER], xh[PER];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const size_t off = (size_t)p * D + 4 * c16 + 64 * e;
      d[e] = ok ? ldg<float4>(dx + off) : make_float4(0.f, 0.f, 0.f, 0.f);
      xh[e] = ok ? ldg<float4>(xhat + off) : make_float4(0.f, 0.f, 0.f, 0.f);
      sg[e].x += d[e].x * xh[e].x, sg[e].y += d[e].y * xh[e].y, sg[e].z += d[e].z * xh[e].z,
          sg[e].w += d[e].w * xh[e].w;
      sb[e].x += d[e].x, sb[e].y += d[e].y, sb[e].z += d[e].z, sb[e].w += d[e].w;
      const float4 dh = make_float4(d[e].x * gm[e].x, d[e].y * gm[e].y, d[e].z * gm[e].z, d[e].w * gm[e].w);
      s1 += (dh.x + dh.y) + (dh.z + dh.w);
      s2 += (dh.x * xh[e].x + dh.y * xh[e].y) + (dh.z * xh[e].z + dh.w * xh[e].w);
    }
    s1 = row16_sum(s1);
    s2 = row16_sum(s2);
    if (ok) {
      const float r = rstd[p], m1 = s1 / D, m2 = s2 / D;
#pragma unroll
      for (int e = 0; e < PER; ++e)
        stg<float4>(dP + (size_t)p * D + 4 * c16 + 64 * e,
                    make_float4((d[e].x * gm[e].x - m1 - xh[e].x * m2) * r, (d[e].y * gm[e].y - m1 - xh[e].y * m2) * r,
                                (d[e].z * gm[e].z - m1 - xh[e].z * m2) * r,
                                (d[e].w * gm[e].w - m1 - xh[e].w * m2) * r));
    }
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    *reinterpret_cast<float4 *>(&red[0][wave * 4 + pr][4 * c16 + 64 * e]) = sg[e];
    *reinterpret_cast<float4 *>(&red[1][wave * 4 + pr][4 * c16 + 64 * e]) = sb[e];
  }
  __syncthreads();
  for (int c = threadIdx.x; c < 2 * D; c += NW * 64) {
    const int w = c / D, ch = c - w * D;
    float acc = 0.f;
#pragma unroll 8
    for (int q = 0; q < NW * 4; ++q) acc += red[w][q][ch];
    (w == 0 ? part_g : part_b)[(size_t)blockIdx.x * D + ch] = acc;
  }
}

// ------------------------------------------------------------------ attention
// Scores in the log2 domain: sl = (q.k / sqrt(d) + z) * log2(e), FILL * log2(e)
// where masked, -inf for keys past N; m2 and l are a column's maximum and sum
// of exp2(sl - m2) over the keys (undropped), so a = exp2(sl - m2) / l.
struct BwdAttnArgs {
  const float *proj;     // [P][C]: q | k | v | gate (before the sigmoid and its bias) | z
  const float *zt;       // [B][h][N][N]: z[b,t,j,k] * log2(e), FILL * log2(e) where masked
  const uint8_t *mask;   // [B][N][N]
  const uint32_t *bits;  // [B][N][h][N][NW]: bit k%32 of word k/32 set where key k is kept
  float *m, *l, *Dj;     // [B][N][h][N]: m2, l, sum_k a da (= do . o)
  float *dob;            // [P][D]: d o (written by the forward-and-dq step)
  float *dcat;           // [P][C]: dq | dk | dv | dgp | dz
  float fill2, scale, qs;  // fill * log2(e); keep scale; log2(e) / sqrt(d)
  float rsd;             // 1 / sqrt(d)
  uint32_t thr, seed_lo, seed_hi, offset;
  int B, N, D, h, C, NW;
  const uint8_t *dead;  // [B][N]: 1 where query column j has no valid key (every M[b, j, k] is 0)
  float *zpart;      // [zsplit][B*h][N][N]: dz partial sums over row ranges (zsplit > 1)
  int zsplit, zrows;  // row ranges of the dz step and rows per range
};

// The dropout decisions, one bit per (b, i, t, j, key), from the forward's
// generator words: thread n computes word n (32 keys, eight calls of four).
__global__ __launch_bounds__(256) void bwd_keep_bits(BwdAttnArgs a, uint32_t *bits, long long nwords) {
  const long long n = (long long)blockIdx.x * 256 + threadIdx.x;
  if (n >= nwords) return;
  const long long rowj = n / a.NW;  // ((b*N + i)*h + t)*N + j
  const int kw = (int)(n - rowj * a.NW);
  const int j = (int)(rowj % a.N);
  const uint32_t ctr2 = (uint32_t)(rowj / a.N);  // (b*N + i)*h + t
  uint32_t word = 0;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int k = kw * 32 + 4 * c;
    if (k < a.N) {
      const uint4 r = philox4x32_10(make_uint4((uint32_t)(k >> 2), (uint32_t)j, ctr2, a.offset), a.seed_lo, a.seed_hi);
      word |= ((uint32_t)(r.x >= a.thr) | (uint32_t)(r.y >= a.thr) << 1 | (uint32_t)(r.z >= a.thr) << 2 |
               (uint32_t)(r.w >= a.thr) << 3)
              << (4 * c);
    }
  }
  bits[n] = word;
}

__device__ __forceinline__ const uint32_t *keep_row(const BwdAttnArgs &a, int bi, int t, int j) {
  return a.bits + (((size_t)bi * a.h + t) * a.N + j) * a.NW;
}

// The attention steps run as split bf16 products (above), with the score
// tile transposed, S^T = k q^T (keys in rows), in the forward and dq kernels:
// lane l = 16 g + r16 holds keys 4g + r of query column r16, which is the
// k-slice of the P^T / dS^T operand of o^T = v^T P^T and dq^T = k^T dS^T.
// In a 16-slice, lane group g takes channels (or keys) 4g..4g+3 of both
// operands. Staged operands are held in LDS as their hi and lo bf16 planes. Work item: (b, i, t, 128 query columns), 8 waves of 16 columns;
// keys through LDS in chunks of 64.
template <int DH>
struct BwdTile {
  static constexpr int NW = 8, QB = NW * 16, KT = 64, CB = DH / 16;
  static constexpr int KP = DH + 4;   // [key][c] row pitch (elements)
  static constexpr int TP = KT + 4;   // [c][key] row pitch (elements)
};

template <int DH>
constexpr int S_KP = BwdTile<DH>::KP;  // [key][c] row pitch
constexpr int S_TP = BwdTile<16>::TP;  // [c][key] row pitch (independent of the head size)

// stage the chunk's k (or v) rows of head t as split bf16 planes ([0] hi,
// [1] lo), [key][c] and/or [c][key]
template <int DH>
__device__ __forceinline__ void stage_rows(const BwdAttnArgs &a, size_t rowp, int col0, int k0,
                                           uint16_t (*rows)[S_KP<DH> * 64], uint16_t (*cols)[DH * S_TP]) {
  using S = BwdTile<DH>;
  constexpr int V4 = S::KT * DH / 4;  // float4 pieces
  for (int e = threadIdx.x; e < V4; e += S::NW * 64) {
    const int kk = e / (DH / 4), u4 = (e - kk * (DH / 4)) * 4, k = k0 + kk;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (k < a.N) v = ldg<float4>(a.proj + (rowp + k) * a.C + col0 + u4);
    const Split4 sp = split4(v.x, v.y, v.z, v.w);
    const uint2 hv = __builtin_bit_cast(uint2, sp.h), lv = __builtin_bit_cast(uint2, sp.l);
    if (rows) {
      *reinterpret_cast<uint2 *>(rows[0] + kk * S::KP + u4) = hv;
      *reinterpret_cast<uint2 *>(rows[1] + kk * S::KP + u4) = lv;
    }
    if (cols) {
      const uint32_t hw[2] = {hv.x, hv.y}, lw[2] = {lv.x, lv.y};
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        cols[0][(u4 + cc) * S::TP + kk] = (uint16_t)(hw[cc >> 1] >> (16 * (cc & 1)));
        cols[1][(u4 + cc) * S::TP + kk] = (uint16_t)(lw[cc >> 1] >> (16 * (cc & 1)));
      }
    }
  }
}

// S^T tile of 16 keys (kb) x the lane's query: bias + q.k, -inf for keys past
// N. A masked key's bias is FILL, so its score FILL + q.k has weight exactly 0
// beside any valid key; a query column without a valid key has q = 0 (and do
// = 0, D = 0) wherever it is staged, so its scores are FILL exactly (uniform
// weights, the rule of a finite fill) and its dS is exactly 0, as the masked
// entries' must be. No per-score mask test is needed.
template <int DH>
__device__ __forceinline__ f32x4 score_tile_t(const BwdAttnArgs &a, const uint16_t (*kbuf)[S_KP<DH> * 64],
                                              const Split4 (&qf)[DH / 16], const float *zq, int k0, int kb, int g,
                                              int r16) {
  using S = BwdTile<DH>;
  const int kq = k0 + kb * 16 + 4 * g;  // first of the lane's four keys
  const bool full = kq + 3 < a.N;
  f32x4 st;
  if (full && (a.N & 3) == 0) {  // rows of z are 16-byte aligned when N % 4 == 0
    const float4 z4 = ldg<float4>(zq + kq);
    st = (f32x4){z4.x, z4.y, z4.z, z4.w};
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) st[r] = kq + r < a.N ? zq[kq + r] : 0.f;
  }
#pragma unroll
  for (int cb = 0; cb < S::CB; ++cb) {
    const int o = (kb * 16 + r16) * S::KP + 16 * cb + 4 * g;
    st = mma_split(lds_split4(kbuf[0] + o, kbuf[1] + o), qf[cb], st);
  }
  if (!full) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (kq + r >= a.N) st[r] = -INFINITY;
  }
  return st;
}

// Attention forward again, with the output and gate step, per work item
// (b, i, t, 128 query columns): m2, l and o = scale * sum_k keep * a v (kept
// in registers, never stored); then, per query column and channel of head t,
// g = sigmoid(gate pre-activation + bg) and, from d(g*o) = Wo^T dy,
// dgp = d(g*o) o g (1 - g) (into dcat), do = d(g*o) g (for the dq, dk/dv and
// dz steps), g*o (for dWo) and D = sum_k a da = do . o.
template <typename T, int DH>
__global__ __launch_bounds__(512) void bwd_attn_fwd(BwdAttnArgs a, const float *dgo, const void *bg, float *go) {
  using S = BwdTile<DH>;
  constexpr int CB = S::CB, KT = S::KT;
  __shared__ __align__(16) uint16_t kbuf[2][KT * S::KP];
  __shared__ __align__(16) uint16_t cT[2][DH * S::TP];  // v transposed
  const int N = a.N, D = a.D, h = a.h, C = a.C;
  const int nq = (N + S::QB - 1) / S::QB;
  const int item = blockIdx.x, qc = item % nq, bt = item / nq, bi = bt / h, t = bt - bi * h, b = bi / N;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, r16 = lane & 15;
  const int j = qc * S::QB + wave * 16 + r16, jc = min(j, N - 1);
  const size_t rowp = (size_t)bi * N;
  // no valid key: q = 0 (its scores are FILL exactly), and D = 0 (the dS
  // path's do is zeroed where staged), so its dS is exactly 0
  const float live = a.dead[(size_t)b * N + jc] ? 0.f : 1.f;
  Split4 qf[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const float4 q4 = ldg<float4>(a.proj + (rowp + jc) * C + t * DH + 16 * cb + 4 * g);
    const float qsc = a.qs * live;
    qf[cb] = split4(q4.x * qsc, q4.y * qsc, q4.z * qsc, q4.w * qsc);
  }
  const float *zq = a.zt + ((size_t)(b * h + t) * N + jc) * N;
  const uint32_t *kr = keep_row(a, bi, t, jc);
  // running maximum, row sum and o^T (lane: channels 16 cb + 4g + r of query j)
  float mrun = -INFINITY, lsum = 0.f;
  f32x4 ot[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) ot[cb] = (f32x4){0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < N; k0 += KT) {
    stage_rows<DH>(a, rowp, D + t * DH, k0, kbuf, nullptr);
    stage_rows<DH>(a, rowp, 2 * D + t * DH, k0, nullptr, cT);
    __syncthreads();
    f32x4 st[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) st[kb] = score_tile_t<DH>(a, kbuf, qf, zq, k0, kb, g, r16);
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, st[kb][r]);
    mx = group4_max(mx);
    const float mnew = fmaxf(mrun, mx);
    const float msh = mnew == -INFINITY ? 0.f : mnew;  // every lane stays in the step
    const float alpha = fast_exp2(mrun - msh);
    mrun = mnew;
    lsum *= alpha;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) ot[cb] *= alpha;
    const uint32_t w32[2] = {k0 < N ? kr[k0 >> 5] : 0u, k0 + 32 < N ? kr[(k0 >> 5) + 1] : 0u};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const uint32_t nib = w32[kb >> 1] >> (16 * (kb & 1) + 4 * g);
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = fast_exp2(st[kb][r] - msh);
        lsum += e;
        p[r] = (nib >> r) & 1u ? e : 0.f;
      }
      const Split4 ps = split4(p[0], p[1], p[2], p[3]);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int o = (16 * cb + r16) * S::TP + kb * 16 + 4 * g;
        ot[cb] = mma_split(lds_split4(cT[0] + o, cT[1] + o), ps, ot[cb]);
      }
    }
    __syncthreads();
  }
  const float lt = group4_sum(lsum);
  const size_t st_ = ((size_t)bi * h + t) * N + jc;
  if (j < N && g == 0) {
    a.m[st_] = mrun;
    a.l[st_] = lt;
  }
  // ---- the output and gate step, and D
  const float inv = a.scale / lt;
  float dsum = 0.f;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int c0 = t * DH + 16 * cb + 4 * g;  // the lane's first channel
    const size_t pc = (rowp + jc) * D + c0;
    const float4 d4 = ldg<float4>(dgo + pc);
    const float4 gp4 = ldg<float4>(a.proj + (rowp + jc) * C + 3 * D + c0);
    const float dgv[4] = {d4.x, d4.y, d4.z, d4.w}, gpv[4] = {gp4.x, gp4.y, gp4.z, gp4.w};
    float ov[4], dov[4], dgp[4], gov[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      ov[r] = ot[cb][r] * inv;
      const float gg = 1.0f / (1.0f + expf(-(gpv[r] + ld_elem<T>(bg, c0 + r))));
      dov[r] = dgv[r] * gg;
      dgp[r] = dgv[r] * ov[r] * gg * (1.0f - gg);
      gov[r] = gg * ov[r];
    }
    if (j < N) {
      stg<float4>(a.dcat + (rowp + j) * C + 3 * D + c0, make_float4(dgp[0], dgp[1], dgp[2], dgp[3]));
      stg<float4>(a.dob + pc, make_float4(dov[0], dov[1], dov[2], dov[3]));
      stg<float4>(go + pc, make_float4(gov[0], gov[1], gov[2], gov[3]));
    }
    dsum += live * ((dov[0] * ov[0] + dov[1] * ov[1]) + (dov[2] * ov[2] + dov[3] * ov[3]));
  }
  const float Dv = group4_sum(dsum);
  if (j < N && g == 0) a.Dj[st_] = Dv;
}

// dq per work item (b, i, t, 128 query columns), with the statistics, do and
// D of the forward-and-gate step.
template <int DH>
__global__ __launch_bounds__(512) void bwd_attn_dq(BwdAttnArgs a) {
  using S = BwdTile<DH>;
  constexpr int CB = S::CB, KT = S::KT;
  __shared__ __align__(16) uint16_t kbuf[2][KT * S::KP];
  __shared__ __align__(16) uint16_t kT[2][DH * S::TP];
  __shared__ __align__(16) uint16_t vbuf[2][KT * S::KP];
  const int N = a.N, D = a.D, h = a.h, C = a.C;
  const int nq = (N + S::QB - 1) / S::QB;
  const int item = blockIdx.x, qc = item % nq, bt = item / nq, bi = bt / h, t = bt - bi * h, b = bi / N;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, r16 = lane & 15;
  const int j = qc * S::QB + wave * 16 + r16, jc = min(j, N - 1);
  const size_t rowp = (size_t)bi * N;
  // no valid key: q, do = 0 (and D = 0 from the forward step), so the
  // column's dS is exactly 0
  const float live = a.dead[(size_t)b * N + jc] ? 0.f : 1.f;
  Split4 qf[CB], df[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const float4 q4 = ldg<float4>(a.proj + (rowp + jc) * C + t * DH + 16 * cb + 4 * g);
    const float qsc = a.qs * live;
    qf[cb] = split4(q4.x * qsc, q4.y * qsc, q4.z * qsc, q4.w * qsc);
    const float4 d4 = ldg<float4>(a.dob + (rowp + jc) * D + t * DH + 16 * cb + 4 * g);
    df[cb] = split4(d4.x * live, d4.y * live, d4.z * live, d4.w * live);
  }
  const size_t st_ = ((size_t)bi * h + t) * N + jc;
  const float Dv = a.Dj[st_];
  // every score -inf (-inf fill, no valid key): weights 0 (not 0 * inf)
  const float m2r = a.m[st_], m2 = m2r == -INFINITY ? 0.f : m2r, linv = m2r == -INFINITY ? 0.f : 1.f / a.l[st_];
  const float *zq = a.zt + ((size_t)(b * h + t) * N + jc) * N;
  const uint32_t *kr = keep_row(a, bi, t, jc);
  f32x4 dq[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) dq[cb] = (f32x4){0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < N; k0 += KT) {
    stage_rows<DH>(a, rowp, D + t * DH, k0, kbuf, kT);
    stage_rows<DH>(a, rowp, 2 * D + t * DH, k0, vbuf, nullptr);
    __syncthreads();
    const uint32_t w32[2] = {k0 < N ? kr[k0 >> 5] : 0u, k0 + 32 < N ? kr[(k0 >> 5) + 1] : 0u};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const f32x4 st = score_tile_t<DH>(a, kbuf, qf, zq, k0, kb, g, r16);
      // dP^T = v do^T (keys x the lane's query)
      f32x4 dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int o = (kb * 16 + r16) * S::KP + 16 * cb + 4 * g;
        dp = mma_split(lds_split4(vbuf[0] + o, vbuf[1] + o), df[cb], dp);
      }
      const uint32_t nib = w32[kb >> 1] >> (16 * (kb & 1) + 4 * g);
      float ds[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = fast_exp2(st[r] - m2) * linv;
        const float da = (nib >> r) & 1u ? dp[r] : 0.f;  // the keep scale enters below
        ds[r] = p * fmaf(da, a.scale, -Dv);
      }
      // dq^T += k^T dS^T
      const Split4 dss = split4(ds[0], ds[1], ds[2], ds[3]);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int o = (16 * cb + r16) * S::TP + kb * 16 + 4 * g;
        dq[cb] = mma_split(lds_split4(kT[0] + o, kT[1] + o), dss, dq[cb]);
      }
    }
    __syncthreads();
  }
  if (j >= N) return;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
    stg<float4>(a.dcat + (rowp + j) * C + t * DH + 16 * cb + 4 * g,
                make_float4(dq[cb][0] * a.rsd, dq[cb][1] * a.rsd, dq[cb][2] * a.rsd, dq[cb][3] * a.rsd));
}

// dk and dv per (b, i, t, 128 key columns), 8 waves of 16 keys, queries in
// chunks of 64 through LDS. Here the score tile is S = q k^T (queries in
// rows): lane l holds queries 4g + r of key r16, the k-slice of the P and dS
// operands of dv^T = do^T P' and dk^T = q^T dS.
template <int DH>
__global__ __launch_bounds__(512) void bwd_attn_dkv(BwdAttnArgs a) {
  using S = BwdTile<DH>;
  constexpr int CB = S::CB, QT = S::KT;
  // q and do of the chunk as split bf16 planes (hi, lo): rows [query][c]
  // and transposed [c][query]
  __shared__ __align__(16) uint16_t qbuf[2][QT * S::KP];
  __shared__ __align__(16) uint16_t qT[2][DH * S::TP];
  __shared__ __align__(16) uint16_t dbuf[2][QT * S::KP];
  __shared__ __align__(16) uint16_t dT[2][DH * S::TP];
  __shared__ __align__(16) float ms[QT], ls[QT], Ds[QT];
  // the chunk's bias, mask and keep bits for the workgroup's 128 keys
  __shared__ __align__(16) float zs[QT][S::QB + 4];
  __shared__ uint32_t kbits[QT][S::QB / 32];
  const int N = a.N, D = a.D, h = a.h, C = a.C;
  const int nk = (N + S::QB - 1) / S::QB;
  const int item = blockIdx.x, kc = item % nk, bt = item / nk, bi = bt / h, t = bt - bi * h, b = bi / N;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, r16 = lane & 15;
  const int k = kc * S::QB + wave * 16 + r16, kcl = min(k, N - 1);
  const size_t rowp = (size_t)bi * N;
  Split4 kf[CB], vf[CB];  // lane: key r16, channels 16 cb + 4g .. +3 (k pre-scaled)
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const float4 k4 = ldg<float4>(a.proj + (rowp + kcl) * C + D + t * DH + 16 * cb + 4 * g);
    const float4 v4 = ldg<float4>(a.proj + (rowp + kcl) * C + 2 * D + t * DH + 16 * cb + 4 * g);
    kf[cb] = split4(k4.x * a.qs, k4.y * a.qs, k4.z * a.qs, k4.w * a.qs);
    vf[cb] = split4(v4.x, v4.y, v4.z, v4.w);
  }
  f32x4 dk[CB], dv[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) dk[cb] = dv[cb] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const float *zb = a.zt + (size_t)(b * h + t) * N * N;
  // A query chunk's q and do rows of head t ([query][c] and [c][query]),
  // statistics, bias tile and keep bits pass through LDS. With d = 16 each
  // thread loads its share of chunk c + 1 into registers while chunk c is
  // computed (load_chunk), and writes it to LDS after chunk c's products
  // (store_chunk): the loads' round trip overlaps the products. Shares: at
  // most one q/do piece, one statistic, ZP bias pieces and one keep word.
  constexpr int V4 = QT * DH / 4, ZP = QT * S::QB / 4 / (S::NW * 64), KW = QT * (S::QB / 32);
  static_assert(V4 <= S::NW * 64 && KW <= S::NW * 64 && ZP * S::NW * 64 == QT * S::QB / 4, "chunk shares");
  const int kw0 = (kc * S::QB) >> 5;
  struct Chunk {
    float4 q, d, z[ZP];
    float m, il, Dq, live;  // live = 0: the query column has no valid key
    uint32_t kw;
  };
  auto load_chunk = [&](int j0) {
    Chunk c;
    const int e = threadIdx.x;
    c.q = c.d = make_float4(0.f, 0.f, 0.f, 0.f);
    c.live = 0.f;
    if (e < V4) {
      const int jj = e / (DH / 4), u4 = (e - jj * (DH / 4)) * 4, jq = j0 + jj;
      if (jq < N) {
        c.q = ldg<float4>(a.proj + (rowp + jq) * C + t * DH + u4);
        c.d = ldg<float4>(a.dob + (rowp + jq) * D + t * DH + u4);
        c.live = a.dead[(size_t)b * N + jq] ? 0.f : 1.f;
      }
    }
    // m and 1 / l (one division per query, not per score); a column past N,
    // or one whose every score is -inf (-inf fill, all keys masked), gets
    // m = 0 and 1 / l = 0, so that its weights below come out 0 without a
    // test per score
    c.m = 0.f, c.il = 0.f, c.Dq = 0.f;
    if (e < QT) {
      const int jq = j0 + e;
      const size_t st_ = ((size_t)bi * h + t) * N + jq;
      const float mj = jq < N ? a.m[st_] : -INFINITY;
      if (mj != -INFINITY) c.m = mj, c.il = 1.f / a.l[st_];
      if (jq < N) c.Dq = a.Dj[st_];
    }
#pragma unroll
    for (int u = 0; u < ZP; ++u) {
      const int x = e + u * S::NW * 64;
      const int jj = x / (S::QB / 4), kk = (x - jj * (S::QB / 4)) * 4, jq = j0 + jj, kq = kc * S::QB + kk;
      // -inf past N (query or key): such a score is -inf whatever q.k is
      float4 z4 = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      if (jq < N && kq + 3 < N && (N & 3) == 0) {  // rows of z are 16-byte aligned when N % 4 == 0
        z4 = ldg<float4>(zb + (size_t)jq * N + kq);
      } else if (jq < N) {
        float t4[4];
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) t4[cc] = kq + cc < N ? zb[(size_t)jq * N + kq + cc] : -INFINITY;
        z4 = make_float4(t4[0], t4[1], t4[2], t4[3]);
      }
      c.z[u] = z4;
    }
    c.kw = 0u;
    if (e < KW) {
      const int jj = e / (S::QB / 32), w = e - jj * (S::QB / 32), jq = j0 + jj;
      if (jq < N && kw0 + w < a.NW) c.kw = keep_row(a, bi, t, jq)[kw0 + w];
    }
    return c;
  };
  auto store_chunk = [&](const Chunk &c) {
    const int e = threadIdx.x;
    if (e < V4) {
      const int jj = e / (DH / 4), u4 = (e - jj * (DH / 4)) * 4;
      // a query column without a valid key: q = 0 (its scores are FILL
      // exactly) and do = 0 in the dP operand (its dS is exactly 0); its do
      // stays in the transposed planes, for dv
      const float lv = c.live;
      const Split4 qs4 = split4(c.q.x * lv, c.q.y * lv, c.q.z * lv, c.q.w * lv),
                   ds4 = split4(c.d.x, c.d.y, c.d.z, c.d.w),
                   dz4 = split4(c.d.x * lv, c.d.y * lv, c.d.z * lv, c.d.w * lv);
      const uint2 qh = __builtin_bit_cast(uint2, qs4.h), ql = __builtin_bit_cast(uint2, qs4.l);
      const uint2 dh = __builtin_bit_cast(uint2, ds4.h), dl = __builtin_bit_cast(uint2, ds4.l);
      *reinterpret_cast<uint2 *>(qbuf[0] + jj * S::KP + u4) = qh;
      *reinterpret_cast<uint2 *>(qbuf[1] + jj * S::KP + u4) = ql;
      *reinterpret_cast<uint2 *>(dbuf[0] + jj * S::KP + u4) = __builtin_bit_cast(uint2, dz4.h);
      *reinterpret_cast<uint2 *>(dbuf[1] + jj * S::KP + u4) = __builtin_bit_cast(uint2, dz4.l);
      const uint32_t w[4][2] = {{qh.x, qh.y}, {ql.x, ql.y}, {dh.x, dh.y}, {dl.x, dl.y}};
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const int sh = 16 * (cc & 1);
        qT[0][(u4 + cc) * S::TP + jj] = (uint16_t)(w[0][cc >> 1] >> sh);
        qT[1][(u4 + cc) * S::TP + jj] = (uint16_t)(w[1][cc >> 1] >> sh);
        dT[0][(u4 + cc) * S::TP + jj] = (uint16_t)(w[2][cc >> 1] >> sh);
        dT[1][(u4 + cc) * S::TP + jj] = (uint16_t)(w[3][cc >> 1] >> sh);
      }
    }
    if (e < QT) ms[e] = c.m, ls[e] = c.il, Ds[e] = c.Dq;
#pragma unroll
    for (int u = 0; u < ZP; ++u) {
      const int x = e + u * S::NW * 64;
      const int jj = x / (S::QB / 4), kk = (x - jj * (S::QB / 4)) * 4;
      *reinterpret_cast<float4 *>(&zs[jj][kk]) = c.z[u];
    }
    if (e < KW) kbits[e / (S::QB / 32)][e % (S::QB / 32)] = c.kw;
  };
  // d = 32 loads each chunk just before it is used: the prefetch registers
  // would take it past the budget that two workgroups per CU leave a wave
  constexpr bool PIPE = DH == 16;
  Chunk nxt;
  if constexpr (PIPE) nxt = load_chunk(0);
  for (int j0 = 0; j0 < N; j0 += QT) {
    if constexpr (PIPE)
      store_chunk(nxt);
    else
      store_chunk(load_chunk(j0));
    __syncthreads();
    if constexpr (PIPE)
      if (j0 + QT < N) nxt = load_chunk(j0 + QT);
#pragma unroll 1
    for (int qb = 0; qb < 4; ++qb) {
      // S = q k^T (queries x keys): bias (FILL where masked, -inf past N) +
      // product, with no per-score mask test (see score_tile_t)
      const int kk = wave * 16 + r16;  // the lane's key within the workgroup's 128
      f32x4 s;
#pragma unroll
      for (int r = 0; r < 4; ++r) s[r] = zs[qb * 16 + 4 * g + r][kk];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int o = (qb * 16 + r16) * S::KP + 16 * cb + 4 * g;
        s = mma_split(lds_split4(qbuf[0] + o, qbuf[1] + o), kf[cb], s);
      }
      // dP = do v^T
      f32x4 dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int o = (qb * 16 + r16) * S::KP + 16 * cb + 4 * g;
        dp = mma_split(lds_split4(dbuf[0] + o, dbuf[1] + o), vf[cb], dp);
      }
      float pk[4], ds[4];
      // statistics of the lane's four queries (16-byte LDS reads; l as 1 / l)
      const float4 m4 = *reinterpret_cast<const float4 *>(&ms[qb * 16 + 4 * g]);
      const float4 l4 = *reinterpret_cast<const float4 *>(&ls[qb * 16 + 4 * g]);
      const float4 d4 = *reinterpret_cast<const float4 *>(&Ds[qb * 16 + 4 * g]);
      const float mq[4] = {m4.x, m4.y, m4.z, m4.w}, lq[4] = {l4.x, l4.y, l4.z, l4.w};
      const float dq4[4] = {d4.x, d4.y, d4.z, d4.w};
      // A score past N (query or key) is -inf (its bias is), so its weight
      // p is 0, and so are its terms below (a keep bit past N may be set: the
      // generator draws keys in fours). A masked score is FILL + q.k: weight
      // 0 beside any valid key; in a column without one, q, do (in the dP
      // operand) and D are 0, so its weights are uniform and its dS is 0.
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int jj = qb * 16 + 4 * g + r;
        const float p = fast_exp2(s[r] - mq[r]) * lq[r];
        const bool kp = ((kbits[jj][kk >> 5] >> (kk & 31)) & 1u) != 0u;
        const float da = kp ? dp[r] : 0.f;  // the keep scale enters below
        pk[r] = kp ? p : 0.f;               // and in dv's store
        ds[r] = p * fmaf(da, a.scale, -dq4[r]);
      }
      // dv^T += do^T P', dk^T += q^T dS
      const Split4 pks = split4(pk[0], pk[1], pk[2], pk[3]), dss = split4(ds[0], ds[1], ds[2], ds[3]);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int o = (16 * cb + r16) * S::TP + qb * 16 + 4 * g;
        dv[cb] = mma_split(lds_split4(dT[0] + o, dT[1] + o), pks, dv[cb]);
        dk[cb] = mma_split(lds_split4(qT[0] + o, qT[1] + o), dss, dk[cb]);
      }
    }
    __syncthreads();
  }
  if (k >= N) return;
  // lane: channels 16 cb + 4g + r of key r16
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    stg<float4>(a.dcat + (rowp + k) * C + D + t * DH + 16 * cb + 4 * g,
                make_float4(dk[cb][0] * a.rsd, dk[cb][1] * a.rsd, dk[cb][2] * a.rsd, dk[cb][3] * a.rsd));
    stg<float4>(a.dcat + (rowp + k) * C + 2 * D + t * DH + 16 * cb + 4 * g,
                make_float4(dv[cb][0] * a.scale, dv[cb][1] * a.scale, dv[cb][2] * a.scale, dv[cb][3] * a.scale));
  }
}

// dz[b,t,j,k] = sum over rows i of ds, masked, per (b, t, 64 query columns j,
// 64 key columns k) and range of zrows rows i (blockIdx.z), 4 waves: wave w
// owns query columns j0 + 16w .. +15 and all 64 keys. With one range the sum
// goes straight to dcat; with several (small N, where the (j, k) tiles alone
// would leave most CUs idle) each range writes its partial sum, and
// bwd_dz_reduce adds the ranges in order. Per row i the rows' q, do, k and v and the queries' m2, l,
// sum a da and keep bits pass through LDS; S = q k^T and dP = do v^T come
// from split bf16 products (lane: queries 4g + r, key r16), and ds is
// summed over i in registers. The bias and the mask of (j, k) are the same
// for every row i and stay in registers.
template <int DH>
__global__ __launch_bounds__(256) void bwd_attn_dz(BwdAttnArgs a) {
  constexpr int JT = 64, KT = 64, RP = DH + 4, CB = DH / 16;
  // the row's k, v, q and do as split bf16 planes ([0] hi, [1] lo)
  __shared__ __align__(16) uint16_t ks[2][KT][RP], vs[2][KT][RP], qs[2][JT][RP], dos[2][JT][RP];
  __shared__ float ms[JT], ls[JT], Ds[JT];
  __shared__ uint32_t kb[JT][2];
  const int N = a.N, D = a.D, h = a.h, C = a.C;
  const int nkt = (N + KT - 1) / KT;
  const int bt = blockIdx.y, b = bt / h, t = bt - b * h;
  const int j0 = (blockIdx.x / nkt) * JT, k0 = (blockIdx.x % nkt) * KT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, r16 = lane & 15;
  // the bias of the valid (j, k) (masked ones and those past N add nothing:
  // bit 4 kb + r of valid)
  float zl[4][4], dz[4][4];  // [key block][r]: query j0 + 16 wave + 4g + r, key k0 + 16 kb + r16
  uint32_t valid = 0;
#pragma unroll
  for (int kbk = 0; kbk < 4; ++kbk)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = j0 + 16 * wave + 4 * g + r, k = k0 + 16 * kbk + r16;
      const float z = (j < N && k < N) ? a.zt[((size_t)(b * h + t) * N + j) * N + k] : a.fill2;
      const bool v = j < N && k < N && z != a.fill2;
      valid |= (uint32_t)v << (4 * kbk + r);
      zl[kbk][r] = v ? z : 0.f;
      dz[kbk][r] = 0.f;
    }
  const int i_begin = blockIdx.z * a.zrows, i_end = min(N, i_begin + a.zrows);
  for (int i = i_begin; i < i_end; ++i) {
    const size_t rowp = ((size_t)b * N + i) * N;
    for (int e = threadIdx.x; e < KT * DH / 4; e += 256) {
      const int r = e / (DH / 4), u4 = (e - r * (DH / 4)) * 4;
      const int k = k0 + r, j = j0 + r;
      float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv, qv = kv, dv = kv;
      if (k < N) {
        kv = ldg<float4>(a.proj + (rowp + k) * C + D + t * DH + u4);
        vv = ldg<float4>(a.proj + (rowp + k) * C + 2 * D + t * DH + u4);
      }
      if (j < N) {
        qv = ldg<float4>(a.proj + (rowp + j) * C + t * DH + u4);
        dv = ldg<float4>(a.dob + (rowp + j) * D + t * DH + u4);
      }
      auto put = [&](uint16_t (*pl)[KT][RP], const Split4 &sp) {
        *reinterpret_cast<uint2 *>(&pl[0][r][u4]) = __builtin_bit_cast(uint2, sp.h);
        *reinterpret_cast<uint2 *>(&pl[1][r][u4]) = __builtin_bit_cast(uint2, sp.l);
      };
      put(ks, split4(kv.x * a.qs, kv.y * a.qs, kv.z * a.qs, kv.w * a.qs));
      put(vs, split4(vv.x, vv.y, vv.z, vv.w));
      put(qs, split4(qv.x, qv.y, qv.z, qv.w));
      put(dos, split4(dv.x, dv.y, dv.z, dv.w));
    }
    if (threadIdx.x < JT) {
      const int jq = j0 + threadIdx.x;
      const size_t st = (((size_t)b * N + i) * h + t) * N + jq;
      ms[threadIdx.x] = jq < N ? a.m[st] : 0.f;
      ls[threadIdx.x] = jq < N ? 1.f / a.l[st] : 1.f;  // 1 / l: one division per query and row
      Ds[threadIdx.x] = jq < N ? a.Dj[st] : 0.f;
      const uint32_t *kr = keep_row(a, b * N + i, t, jq < N ? jq : 0);
      const int w0 = k0 >> 5;
      kb[threadIdx.x][0] = jq < N ? kr[w0] : 0u;
      kb[threadIdx.x][1] = (jq < N && w0 + 1 < a.NW) ? kr[w0 + 1] : 0u;
    }
    __syncthreads();
    float m2[4], linv[4], Dv[4];
    uint32_t w2[4][2];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int jj = 16 * wave + 4 * g + r;
      m2[r] = ms[jj], linv[r] = ls[jj], Dv[r] = Ds[jj];
      w2[r][0] = kb[jj][0], w2[r][1] = kb[jj][1];
    }
#pragma unroll
    for (int kbk = 0; kbk < 4; ++kbk) {
      f32x4 sc = {0.f, 0.f, 0.f, 0.f}, dp = sc;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int cq = 16 * cb + 4 * g, jr = 16 * wave + r16, kr = 16 * kbk + r16;
        sc = mma_split(lds_split4(&qs[0][jr][cq], &qs[1][jr][cq]), lds_split4(&ks[0][kr][cq], &ks[1][kr][cq]), sc);
        dp = mma_split(lds_split4(&dos[0][jr][cq], &dos[1][jr][cq]), lds_split4(&vs[0][kr][cq], &vs[1][kr][cq]),
                       dp);
      }
      const int kk = 16 * kbk + r16;  // the lane's key within the tile
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = fast_exp2(zl[kbk][r] + sc[r] - m2[r]) * linv[r];
        const float dav = (w2[r][kk >> 5] >> (kk & 31)) & 1u ? dp[r] : 0.f;  // the keep scale enters below
        if ((valid >> (4 * kbk + r)) & 1u) dz[kbk][r] += p * fmaf(dav, a.scale, -Dv[r]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int kbk = 0; kbk < 4; ++kbk)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = j0 + 16 * wave + 4 * g + r, k = k0 + 16 * kbk + r16;
      if (j < N && k < N) {
        if (a.zsplit == 1)
          a.dcat[(((size_t)b * N + j) * N + k) * C + 4 * D + t] = dz[kbk][r];
        else
          a.zpart[(((size_t)blockIdx.z * a.B * h + bt) * N + j) * N + k] = dz[kbk][r];
      }
    }
}

// dz = the row ranges' partial sums added in range order, into dcat
__global__ __launch_bounds__(256) void bwd_dz_reduce(BwdAttnArgs a) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;  // (b, t, j, k)
  const int N = a.N, h = a.h;
  const long long nz = (long long)a.B * h * N * N;
  if (e >= nz) return;
  float sum = 0.f;
  for (int z = 0; z < a.zsplit; ++z) sum += a.zpart[z * nz + e];
  const long long jk = e % ((long long)N * N), bt = e / ((long long)N * N);
  const int b = (int)(bt / h), t = (int)(bt - (long long)b * h);
  a.dcat[((size_t)b * N * N + jk) * a.C + 4 * a.D + t] = sum;
}

// dead[b][j] = 1 where query column j of batch b has no valid key (every
// mask entry M[b, j, k] is 0): one wave per column
__global__ __launch_bounds__(256) void bwd_dead_columns(const uint8_t *mask, long long ncol, int N, uint8_t *dead) {
  const long long col = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (col >= ncol) return;  // the whole wave
  const int lane = threadIdx.x & 63;
  const uint8_t *row = mask + col * N;
  bool any = false;
  for (int k = lane; k < N; k += 64) any |= row[k] != 0;
  const bool any_w = __ballot(any) != 0;
  if (lane == 0) dead[col] = any_w ? 0 : 1;
}

// z[b,t,j,k] * log2(e) from the projection columns, FILL * log2(e) where the
// mask is 0, into a [B][h][N][N] copy: the attention kernels tell a masked
// key by that exact value and read no mask
__global__ __launch_bounds__(256) void bwd_ztrans(const float *proj, const uint8_t *mask, float fill2, int B, int N,
                                                   int D, int h, int C, float *zt) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long total = (long long)B * h * N * N;
  if (e >= total) return;
  const long long jk = e % ((long long)N * N), bt = e / ((long long)N * N);
  const int b = (int)(bt / h), t = (int)(bt - (long long)b * h);
  zt[e] = mask[(size_t)b * N * N + jk] ? proj[((size_t)b * N * N + jk) * C + 4 * D + t] * kLog2e : fill2;
}

// ------------------------------------------------------------------ host side
struct BwdLayout {
  size_t x, xhat, rstd, proj, zt, dead, m, l, Dj, dgo, dob, go, dcat, dx, part, vpart, bits, zpart, pt, mt, dyt, dpt, total;
  long long S, kchunk, nvblk, vper;
  int zsplit, zrows;
};

static size_t al256(size_t v) { return (v + 255) & ~size_t(255); }

static BwdLayout bwd_layout(int B, int N, int D, int h, int elem, int transposed, int dz_ranges) {
  BwdLayout L{};
  const long long P = (long long)B * N * N, C = 4LL * D + h;
  // split-K chunks of the weight gradients (sums over all positions): at most
  // 256, each a multiple of 16 positions
  L.kchunk = ((P + 255) / 256 + 15) / 16 * 16;
  if (L.kchunk < 16) L.kchunk = 16;
  L.S = (P + L.kchunk - 1) / L.kchunk;
  // column sums (bias gradients, dgamma, dbeta): at most 256 blocks of 16
  // waves, so the ordered sum of their partials stays short
  L.vper = (P + 255) / 256;
  L.nvblk = (P + L.vper - 1) / L.vper;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = al256(off + bytes);
    return o;
  };
  L.x = take((size_t)P * D * 4);
  L.xhat = take((size_t)P * D * 4);
  L.rstd = take((size_t)P * 4);
  L.proj = take((size_t)P * C * 4);
  L.zt = take((size_t)B * h * N * N * 4);
  L.dead = take((size_t)B * N);
  L.m = take((size_t)B * N * h * N * 4);
  L.l = take((size_t)B * N * h * N * 4);
  L.Dj = take((size_t)B * N * h * N * 4);
  L.dgo = take((size_t)P * D * 4);
  L.dob = take((size_t)P * D * 4);
  L.go = take((size_t)P * D * 4);
  L.dcat = take((size_t)P * C * 4);
  L.dx = take((size_t)P * D * 4);
  L.part = take((size_t)L.S * C * D * 4);
  L.vpart = take((size_t)2 * L.nvblk * D * 4);
  L.bits = take((size_t)B * N * h * N * ((N + 31) / 32) * 4);
  // dz row ranges: enough workgroups to fill the CUs several times over
  // (2048), at least 8 rows per range; or the number the handle was given
  {
    const long long tiles = (long long)((N + 63) / 64) * ((N + 63) / 64) * B * h;
    long long zs = tiles >= 2048 ? 1 : (2048 + tiles - 1) / tiles;
    zs = std::min(zs, (long long)std::max(1, (N + 7) / 8));
    if (dz_ranges > 0) zs = std::min(dz_ranges, std::max(N, 1));
    zs = std::min(zs, 65535LL);  // the grid's z dimension
    L.zrows = (int)((N + zs - 1) / zs);
    L.zsplit = (N + L.zrows - 1) / L.zrows;
    if (L.zsplit < 1) L.zsplit = 1;
  }
  L.zpart = L.zsplit > 1 ? take((size_t)L.zsplit * B * h * N * N * 4) : 0;
  if (transposed) {  // ending-node: pair_repr, mask and dy with both residue axes swapped, and dP before swapping back
    L.pt = take((size_t)P * D * elem);
    L.mt = take((size_t)P);
    L.dyt = take((size_t)P * D * elem);
    L.dpt = take((size_t)P * D * 4);
  }
  L.total = off;
  return L;
}

size_t bwd_workspace_bytes(int B, int N, int D, int h, int elem, int transposed, int dz_ranges) {
  return bwd_layout(B, N, D, h, elem, transposed, dz_ranges).total;
}

// dst[b][i][j][:] = src[b][j][i][:] (W elements per position): the two
// residue axes swapped
template <typename E>
__global__ __launch_bounds__(256) void bwd_swap_axes(const E *src, E *dst, int B, int N, int W) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long total = (long long)B * N * N * W;
  if (e >= total) return;
  const long long pos = e / W, w = e - pos * W;
  const long long bi = pos / N, j = pos - bi * N, b = bi / N, i = bi - b * N;
  dst[e] = src[((b * N + j) * N + i) * W + w];
}

template <typename E>
static hipError_t swap_axes(const void *src, void *dst, int B, int N, int W, hipStream_t s) {
  const long long total = (long long)B * N * N * W;
  hipLaunchKernelGGL((bwd_swap_axes<E>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                     static_cast<const E *>(src), static_cast<E *>(dst), B, N, W);
  return hipGetLastError();
}

template <typename TA, typename TB>
static hipError_t gemm(const void *A, long long sam, long long sak, const void *Bm, long long sbk, long long sbn,
                       float *C, long long scz, long long scm, long long M, long long N, long long K,
                       long long kchunk, int nz, hipStream_t s) {
  GemmArgs g{A, Bm, C, M, N, K, kchunk, sam, sak, sbk, sbn, scz, scm, nz};
  const long long blocks = ((M + 63) / 64) * ((N + 63) / 64) * nz;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks);
  hipLaunchKernelGGL((bwd_gemm<TA, TB>), grid, dim3(256), 0, s, g);
  return hipGetLastError();
}

static hipError_t reduce(const float *part, long long n, int nz, long long stride, float *out, hipStream_t s) {
  hipLaunchKernelGGL(bwd_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, part, n, nz, stride, out);
  return hipGetLastError();
}

template <typename T, int D, int DH>
static hipError_t run_bwd_t(const BwdRunArgs &r, hipStream_t s) {
  const int B = r.B, N = r.N, h = D / DH;
  const long long P = (long long)B * N * N, C = 4LL * D + h;
  const BwdLayout L = bwd_layout(B, N, D, h, (int)sizeof(T) == 2 ? 2 : 4, r.transposed, r.dz_ranges);
  char *w = static_cast<char *>(r.ws);
  float *x = reinterpret_cast<float *>(w + L.x), *xhat = reinterpret_cast<float *>(w + L.xhat);
  float *rstd = reinterpret_cast<float *>(w + L.rstd), *proj = reinterpret_cast<float *>(w + L.proj);
  float *zt = reinterpret_cast<float *>(w + L.zt);
  float *dgo = reinterpret_cast<float *>(w + L.dgo), *dob = reinterpret_cast<float *>(w + L.dob);
  float *go = reinterpret_cast<float *>(w + L.go), *dcat = reinterpret_cast<float *>(w + L.dcat);
  float *dx = reinterpret_cast<float *>(w + L.dx), *part = reinterpret_cast<float *>(w + L.part);
  float *vpart = reinterpret_cast<float *>(w + L.vpart);
  const char *vp = static_cast<const char *>(r.vecs);
  const size_t es = sizeof(T) == 2 ? 2 : 4, vec = (size_t)D * es;
  const void *gamma = vp, *beta = vp + vec, *bg = vp + 2 * vec, *Wo = vp + 4 * vec;
  hipError_t e;
#define TPA_CHECK(x)                     \
  do {                                   \
    if ((e = (x)) != hipSuccess) return e; \
  } while (0)
  // whatever path this function leaves by, this stream ends up ordered after
  // the second stream's work once the join event is recorded
  struct JoinGuard {
    hipStream_t s;
    hipEvent_t ev;
    bool armed;
    ~JoinGuard() {
      if (armed) (void)hipStreamWaitEvent(s, ev, 0);
    }
  } join{s, r.join, false};
  BwdAttnArgs aa{};
  aa.proj = proj, aa.zt = zt;
  aa.m = reinterpret_cast<float *>(w + L.m), aa.l = reinterpret_cast<float *>(w + L.l);
  aa.Dj = reinterpret_cast<float *>(w + L.Dj);
  aa.dob = dob, aa.dcat = dcat;
  aa.fill2 = r.fill * kLog2e, aa.scale = r.scale, aa.rsd = 1.0f / sqrtf((float)DH);
  aa.qs = kLog2e * aa.rsd;
  aa.thr = r.thr, aa.seed_lo = r.seed_lo, aa.seed_hi = r.seed_hi, aa.offset = r.offset;
  aa.B = B, aa.N = N, aa.D = D, aa.h = h, aa.C = (int)C;
  aa.NW = (N + 31) / 32;
  uint32_t *bits = reinterpret_cast<uint32_t *>(w + L.bits);
  aa.bits = bits;
  {
    // the keep bits need only the generator's key, counter offset and the
    // sizes: on the handle's second stream they are made while the
    // LayerNorm, the projection GEMM, the bias copy and the d(g*o) GEMM run
    // on this one (latency-bound tiles that leave VALU issue slots free); the
    // fork orders them after everything earlier on this stream (a previous
    // call may still read the workspace), the join before the first
    // attention step reads them
    const long long nwords = (long long)B * N * h * N * aa.NW;
    hipStream_t ks = s;
    if (r.side) {
      TPA_CHECK(hipEventRecord(r.fork, s));
      TPA_CHECK(hipStreamWaitEvent(r.side, r.fork, 0));
      ks = r.side;
    }
    hipLaunchKernelGGL(bwd_keep_bits, dim3((unsigned)((nwords + 255) / 256)), dim3(256), 0, ks, aa, bits, nwords);
    const hipError_t le = hipGetLastError();
    if (r.side) {
      TPA_CHECK(hipEventRecord(r.join, r.side));
      join.armed = true;
    }
    TPA_CHECK(le);
  }
  // ending-node: the starting-node backward of the transposed problem
  using E = typename std::conditional<sizeof(T) == 2, uint16_t, float>::type;
  const void *Pin = r.P, *dyin = r.dy;
  const uint8_t *Min = r.mask;
  float *dPout = r.g.d_pair_repr;
  if (r.transposed) {
    TPA_CHECK(swap_axes<E>(r.P, w + L.pt, B, N, D, s));
    TPA_CHECK(swap_axes<uint8_t>(r.mask, w + L.mt, B, N, 1, s));
    TPA_CHECK(swap_axes<E>(r.dy, w + L.dyt, B, N, D, s));
    Pin = w + L.pt, Min = reinterpret_cast<const uint8_t *>(w + L.mt), dyin = w + L.dyt;
    dPout = reinterpret_cast<float *>(w + L.dpt);
  }
  // LayerNorm and the five projections, in float32
  hipLaunchKernelGGL((bwd_ln<T, D>), dim3((unsigned)((P + 3) / 4)), dim3(256), 0, s, Pin, gamma, beta, r.eps, P, x,
                     xhat, rstd);
  TPA_CHECK(hipGetLastError());
  TPA_CHECK((gemm<float, T>(x, D, 1, r.wpack, 1, D, proj, 0, C, P, C, D, D, 1, s)));
  hipLaunchKernelGGL(bwd_ztrans, dim3((unsigned)(((long long)B * h * N * N + 255) / 256)), dim3(256), 0, s, proj,
                     Min, r.fill * kLog2e, B, N, D, h, (int)C, zt);
  TPA_CHECK(hipGetLastError());
  aa.mask = Min;
  {
    uint8_t *dead = reinterpret_cast<uint8_t *>(w + L.dead);
    const long long ncol = (long long)B * N;
    hipLaunchKernelGGL(bwd_dead_columns, dim3((unsigned)((ncol + 3) / 4)), dim3(256), 0, s, Min, ncol, N, dead);
    TPA_CHECK(hipGetLastError());
    aa.dead = dead;
  }
  // work items (b, i, t, 128 columns): x only, so no grid limit applies
  const long long items = (long long)B * N * h * ((N + BwdTile<DH>::QB - 1) / BwdTile<DH>::QB);
  if (items > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 ga((unsigned)items);
  // d(g*o) = Wo^T dy, then the attention forward again with the output and
  // gate step, dq, dk/dv and the pair bias
  TPA_CHECK((gemm<T, T>(dyin, D, 1, Wo, D, 1, dgo, 0, D, P, D, D, D, 1, s)));
  if (join.armed) {
    TPA_CHECK(hipStreamWaitEvent(s, r.join, 0));
    join.armed = false;
  }
  hipLaunchKernelGGL((bwd_attn_fwd<T, DH>), ga, dim3(512), 0, s, aa, dgo, bg, go);
  TPA_CHECK(hipGetLastError());
  hipLaunchKernelGGL((bwd_attn_dq<DH>), ga, dim3(512), 0, s, aa);
  TPA_CHECK(hipGetLastError());
  hipLaunchKernelGGL((bwd_attn_dkv<DH>), ga, dim3(512), 0, s, aa);
  TPA_CHECK(hipGetLastError());
  const int nkt = (N + 63) / 64, njt = (N + 63) / 64;
  aa.zsplit = L.zsplit, aa.zrows = L.zrows;
  aa.zpart = reinterpret_cast<float *>(w + L.zpart);
  hipLaunchKernelGGL((bwd_attn_dz<DH>), dim3((unsigned)(njt * nkt), (unsigned)(B * h), (unsigned)L.zsplit), dim3(256),
                     0, s, aa);
  TPA_CHECK(hipGetLastError());
  if (L.zsplit > 1) {
    const long long nz = (long long)B * h * N * N;
    hipLaunchKernelGGL(bwd_dz_reduce, dim3((unsigned)((nz + 255) / 256)), dim3(256), 0, s, aa);
    TPA_CHECK(hipGetLastError());
  }
  // projections and LayerNorm
  TPA_CHECK((gemm<float, T>(dcat, C, 1, r.wpack, D, 1, dx, 0, D, P, D, C, C, 1, s)));
  hipLaunchKernelGGL((bwd_ln_back<T, D>), dim3((unsigned)L.nvblk), dim3(1024), 0, s, dx, xhat, rstd, gamma, P, L.vper,
                     dPout, vpart, vpart + (size_t)L.nvblk * D);
  TPA_CHECK(hipGetLastError());
  TPA_CHECK(reduce(vpart, D, (int)L.nvblk, D, r.g.d_ln_weight, s));
  TPA_CHECK(reduce(vpart + (size_t)L.nvblk * D, D, (int)L.nvblk, D, r.g.d_ln_bias, s));
  // weight gradients: split-K partial products over positions, then ordered sums
  TPA_CHECK((gemm<float, float>(dcat, 1, C, x, D, 1, part, C * D, D, C, D, P, L.kchunk, (int)L.S, s)));
  float *dst[5] = {r.g.d_w_query, r.g.d_w_key, r.g.d_w_value, r.g.d_w_gate, r.g.d_w_bias_proj};
  for (int q = 0; q < 5; ++q)
    TPA_CHECK(reduce(part + (size_t)q * D * D, (q < 4 ? D : h) * (long long)D, (int)L.S, C * D, dst[q], s));
  TPA_CHECK((gemm<T, float>(dyin, 1, D, go, D, 1, part, (long long)D * D, D, D, D, P, L.kchunk, (int)L.S, s)));
  TPA_CHECK(reduce(part, (long long)D * D, (int)L.S, (long long)D * D, r.g.d_w_out, s));
  // bias gradients: column sums over positions
  hipLaunchKernelGGL((bwd_colsum<T>), dim3((unsigned)L.nvblk), dim3(1024), 0, s, dyin, P, D, (long long)D, L.vper,
                     vpart);
  TPA_CHECK(hipGetLastError());
  TPA_CHECK(reduce(vpart, D, (int)L.nvblk, D, r.g.d_b_out, s));
  hipLaunchKernelGGL((bwd_colsum<float>), dim3((unsigned)L.nvblk), dim3(1024), 0, s, dcat + 3 * D, P, D, C, L.vper,
                     vpart);
  TPA_CHECK(hipGetLastError());
  TPA_CHECK(reduce(vpart, D, (int)L.nvblk, D, r.g.d_b_gate, s));
  if (r.transposed) TPA_CHECK(swap_axes<float>(dPout, r.g.d_pair_repr, B, N, D, s));
#undef TPA_CHECK
  return hipSuccess;
}

hipError_t launch_bwd(int dtype, int D, int dh, const BwdRunArgs &r, hipStream_t s) {
  if (dtype == TRI_ATTN_BF16) {
    if (D == 128 && dh == 16) return run_bwd_t<bf16_t, 128, 16>(r, s);
    if (D == 128 && dh == 32) return run_bwd_t<bf16_t, 128, 32>(r, s);
    if (D == 64 && dh == 16) return run_bwd_t<bf16_t, 64, 16>(r, s);
    if (D == 64 && dh == 32) return run_bwd_t<bf16_t, 64, 32>(r, s);
  } else {
    if (D == 128 && dh == 16) return run_bwd_t<float, 128, 16>(r, s);
    if (D == 128 && dh == 32) return run_bwd_t<float, 128, 32>(r, s);
    if (D == 64 && dh == 16) return run_bwd_t<float, 64, 16>(r, s);
    if (D == 64 && dh == 32) return run_bwd_t<float, 64, 32>(r, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tpa

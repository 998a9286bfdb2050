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
// The kernels are plain float32 code (tiled FMAs for the products): the
// backward is checked against the oracle's gradients, not tuned.
#include "device_common.h"
#include "tri_attn.h"
#include "tri_attn_internal.h"

namespace tpa {

// ------------------------------------------------------------------ products
// C[z][m][n] = sum over k in chunk z of A[m, k] B[k, n]; A(m, k) at
// A[m*sam + k*sak], B(k, n) at B[k*sbk + n*sbn], C(z, m, n) at
// C[z*scz + m*scm + n]. 64x64 tile per workgroup, 4x4 outputs per thread, K
// in steps of 16 through LDS, loads laid out along the contiguous index.
struct GemmArgs {
  const void *A, *B;
  float *C;
  long long M, N, K, kchunk;
  long long sam, sak, sbk, sbn, scz, scm;
};

template <typename TA, typename TB>
__global__ __launch_bounds__(256) void bwd_gemm(GemmArgs g) {
  __shared__ float As[16][68];
  __shared__ float Bs[16][68];
  const int tid = threadIdx.x;
  // grid x: row blocks (M can be large), y: column blocks, z: K chunks
  const long long m0 = (long long)blockIdx.x * 64, n0 = (long long)blockIdx.y * 64;
  const long long kb = (long long)blockIdx.z * g.kchunk;
  const long long ke = min(kb + g.kchunk, g.K);
  const int tm = tid >> 4, tn = tid & 15;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  const bool a_m_contig = g.sam == 1, b_n_contig = g.sbn == 1;
  for (long long k0 = kb; k0 < ke; k0 += 16) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = tid + 256 * e;
      const int mm = a_m_contig ? (idx & 63) : (idx >> 4), ka = a_m_contig ? (idx >> 6) : (idx & 15);
      const long long am = m0 + mm, ak = k0 + ka;
      As[ka][mm] = (am < g.M && ak < ke) ? ld_elem<TA>(g.A, (size_t)(am * g.sam + ak * g.sak)) : 0.f;
      const int nn = b_n_contig ? (idx & 63) : (idx >> 4), kbk = b_n_contig ? (idx >> 6) : (idx & 15);
      const long long bn = n0 + nn, bk = k0 + kbk;
      Bs[kbk][nn] = (bn < g.N && bk < ke) ? ld_elem<TB>(g.B, (size_t)(bk * g.sbk + bn * g.sbn)) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[kk][tm * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = Bs[kk][tn * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += av[i] * bv[j];
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const long long m = m0 + tm * 4 + i;
    if (m >= g.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const long long n = n0 + tn * 4 + j;
      if (n < g.N) g.C[(size_t)(blockIdx.z * g.scz + m * g.scm + n)] = acc[i][j];
    }
  }
}

// out[e] = sum over z of part[z*stride + e], z = 0..nz-1 in order
__global__ __launch_bounds__(256) void bwd_reduce(const float *part, long long n, int nz, long long stride,
                                                   float *out) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  float s = 0.f;
  for (int z = 0; z < nz; ++z) s += part[(size_t)(z * stride + e)];
  out[e] = s;
}

// part[blk][c] = sum over positions p of block blk of X[p*ldx + c] (c < ncol)
template <typename T>
__global__ __launch_bounds__(256) void bwd_colsum(const void *X, long long P, int ncol, long long ldx,
                                                   long long per_blk, float *part) {
  const long long p0 = (long long)blockIdx.x * per_blk, p1 = min(p0 + per_blk, P);
  for (int c = threadIdx.x; c < ncol; c += 256) {
    float s = 0.f;
    for (long long p = p0; p < p1; ++p) s += ld_elem<T>(X, (size_t)(p * ldx + c));
    part[(size_t)blockIdx.x * ncol + c] = s;
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

// LayerNorm backward per position, and per-block partial sums of dx * x-hat
// (for dgamma) and dx (for dbeta): block blk covers positions blk*per .. .
template <typename T, int D>
__global__ __launch_bounds__(D) void bwd_ln_back(const float *dx, const float *xhat, const float *rstd,
                                                  const void *gamma, long long npos, long long per_blk, float *dP,
                                                  float *part_g, float *part_b) {
  __shared__ float red[2][D / 64];
  const int c = threadIdx.x, lane = c & 63, wave = c >> 6;
  const float gm = ld_elem<T>(gamma, c);
  const long long p0 = (long long)blockIdx.x * per_blk, p1 = min(p0 + per_blk, npos);
  float sg = 0.f, sb = 0.f;
  for (long long p = p0; p < p1; ++p) {
    const float d = dx[p * D + c], xh = xhat[p * D + c];
    sg += d * xh;
    sb += d;
    const float dxh = d * gm;
    float s1 = dxh, s2 = dxh * xh;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      s1 += __shfl_xor(s1, m, 64);
      s2 += __shfl_xor(s2, m, 64);
    }
    if (lane == 0) red[0][wave] = s1, red[1][wave] = s2;
    __syncthreads();
    float t1 = 0.f, t2 = 0.f;
#pragma unroll
    for (int w = 0; w < D / 64; ++w) t1 += red[0][w], t2 += red[1][w];
    __syncthreads();
    dP[p * D + c] = (dxh - t1 / D - xh * (t2 / D)) * rstd[p];
  }
  part_g[(size_t)blockIdx.x * D + c] = sg;
  part_b[(size_t)blockIdx.x * D + c] = sb;
}

// ------------------------------------------------------------------ attention
struct BwdAttnArgs {
  const float *proj;   // [P][C]: q | k | v | gate (before the sigmoid and its bias) | z
  const float *zt;     // [B][h][N][N]: z[b,t,j,k]
  const uint8_t *mask; // [B][N][N]
  float *m, *l, *Dj;   // [B][N][h][N]: row maximum, row sum, sum_k a da
  float *o;            // [P][D]: o after dropout
  const float *dob;    // [P][D]: d o
  float *dcat;         // [P][C]: dq | dk | dv | dgp | dz
  float fill, scale, rsd;
  uint32_t thr, seed_lo, seed_hi, offset;
  int B, N, D, h, C;
};

__device__ __forceinline__ uint32_t keep_word(const BwdAttnArgs &a, int b, int i, int t, int j, int k) {
  const uint4 r = philox4x32_10(make_uint4((uint32_t)(k >> 2), (uint32_t)j, (uint32_t)((b * a.N + i) * a.h + t),
                                           a.offset),
                                a.seed_lo, a.seed_hi);
  const int w = k & 3;
  return w == 0 ? r.x : w == 1 ? r.y : w == 2 ? r.z : r.w;
}

// Attention forward again, per (b, i, t), one thread per query column j:
// running maximum m and sum l over the keys (undropped weights), and
// o = scale * sum_k keep * exp(s - m) v_k / l.
template <int DH>
__global__ __launch_bounds__(256) void bwd_attn_fwd(BwdAttnArgs a) {
  constexpr int KT = 64;
  __shared__ float ks[KT][DH], vs[KT][DH];
  const int N = a.N, D = a.D, h = a.h, C = a.C;
  const int bi = blockIdx.x / h, t = blockIdx.x - bi * h, b = bi / N, i = bi - b * N;
  const int j = blockIdx.y * 256 + threadIdx.x;
  const bool live = j < N;
  const size_t rowp = (size_t)bi * N;  // position of (b, i, 0)
  float q[DH];
#pragma unroll
  for (int u = 0; u < DH; ++u) q[u] = live ? a.proj[(rowp + j) * C + t * DH + u] * a.rsd : 0.f;
  float m = -INFINITY, l = 0.f, o[DH];
#pragma unroll
  for (int u = 0; u < DH; ++u) o[u] = 0.f;
  const float *zrow = a.zt + ((size_t)(b * h + t) * N + (live ? j : 0)) * N;
  const uint8_t *mrow = a.mask + ((size_t)b * N + (live ? j : 0)) * N;
  for (int k0 = 0; k0 < N; k0 += KT) {
    for (int e = threadIdx.x; e < KT * DH; e += 256) {
      const int kk = e / DH, u = e - kk * DH, k = k0 + kk;
      ks[kk][u] = k < N ? a.proj[(rowp + k) * C + D + t * DH + u] : 0.f;
      vs[kk][u] = k < N ? a.proj[(rowp + k) * C + 2 * D + t * DH + u] : 0.f;
    }
    __syncthreads();
    const int kn = min(KT, N - k0);
    if (live) {
      for (int kk = 0; kk < kn; ++kk) {
        const int k = k0 + kk;
        float s = zrow[k];
#pragma unroll
        for (int u = 0; u < DH; ++u) s += q[u] * ks[kk][u];
        if (!mrow[k]) s = a.fill;
        if (s > m) {
          const float f = (m == -INFINITY) ? 0.f : expf(m - s);
          l *= f;
#pragma unroll
          for (int u = 0; u < DH; ++u) o[u] *= f;
          m = s;
        }
        const float p = (s == -INFINITY) ? 0.f : expf(s - m);
        l += p;
        if (keep_word(a, b, i, t, j, k) >= a.thr) {
#pragma unroll
          for (int u = 0; u < DH; ++u) o[u] += p * vs[kk][u];
        }
      }
    }
    __syncthreads();
  }
  if (!live) return;
  const size_t st = ((size_t)bi * h + t) * N + j;
  a.m[st] = m;
  a.l[st] = l;
  const float inv = a.scale / l;
#pragma unroll
  for (int u = 0; u < DH; ++u) a.o[(rowp + j) * D + t * DH + u] = o[u] * inv;
}

// dq, and sum_k a da = do_j . o_j, per (b, i, t), one thread per query column j.
template <int DH>
__global__ __launch_bounds__(256) void bwd_attn_dq(BwdAttnArgs a) {
  constexpr int KT = 64;
  __shared__ float ks[KT][DH], vs[KT][DH];
  const int N = a.N, D = a.D, h = a.h, C = a.C;
  const int bi = blockIdx.x / h, t = blockIdx.x - bi * h, b = bi / N, i = bi - b * N;
  const int j = blockIdx.y * 256 + threadIdx.x;
  const bool live = j < N;
  const size_t rowp = (size_t)bi * N;
  float q[DH], dov[DH], dq[DH];
  float Dv = 0.f;
#pragma unroll
  for (int u = 0; u < DH; ++u) {
    q[u] = live ? a.proj[(rowp + j) * C + t * DH + u] * a.rsd : 0.f;
    dov[u] = live ? a.dob[(rowp + j) * D + t * DH + u] : 0.f;
    Dv += live ? dov[u] * a.o[(rowp + j) * D + t * DH + u] : 0.f;
    dq[u] = 0.f;
  }
  const size_t st = ((size_t)bi * h + t) * N + (live ? j : 0);
  const float m = a.m[st], l = a.l[st];
  if (live) a.Dj[st] = Dv;
  const float *zrow = a.zt + ((size_t)(b * h + t) * N + (live ? j : 0)) * N;
  const uint8_t *mrow = a.mask + ((size_t)b * N + (live ? j : 0)) * N;
  for (int k0 = 0; k0 < N; k0 += KT) {
    for (int e = threadIdx.x; e < KT * DH; e += 256) {
      const int kk = e / DH, u = e - kk * DH, k = k0 + kk;
      ks[kk][u] = k < N ? a.proj[(rowp + k) * C + D + t * DH + u] : 0.f;
      vs[kk][u] = k < N ? a.proj[(rowp + k) * C + 2 * D + t * DH + u] : 0.f;
    }
    __syncthreads();
    const int kn = min(KT, N - k0);
    if (live) {
      for (int kk = 0; kk < kn; ++kk) {
        const int k = k0 + kk;
        if (!mrow[k]) continue;  // masked: no gradient reaches q
        float s = zrow[k];
#pragma unroll
        for (int u = 0; u < DH; ++u) s += q[u] * ks[kk][u];
        const float p = expf(s - m) / l;
        float da = 0.f;
        if (keep_word(a, b, i, t, j, k) >= a.thr) {
#pragma unroll
          for (int u = 0; u < DH; ++u) da += dov[u] * vs[kk][u];
          da *= a.scale;
        }
        const float ds = p * (da - Dv);
#pragma unroll
        for (int u = 0; u < DH; ++u) dq[u] += ds * ks[kk][u];
      }
    }
    __syncthreads();
  }
  if (!live) return;
#pragma unroll
  for (int u = 0; u < DH; ++u) a.dcat[(rowp + j) * C + t * DH + u] = dq[u] * a.rsd;
}

// dk and dv per (b, i, t), one thread per key column k; the queries' q, do,
// m, l and sum_k a da pass through LDS in tiles.
template <int DH>
__global__ __launch_bounds__(256) void bwd_attn_dkv(BwdAttnArgs a) {
  constexpr int QT = 64;
  __shared__ float qs[QT][DH], dos[QT][DH], ms[QT], ls[QT], Ds[QT];
  const int N = a.N, D = a.D, h = a.h, C = a.C;
  const int bi = blockIdx.x / h, t = blockIdx.x - bi * h, b = bi / N, i = bi - b * N;
  const int k = blockIdx.y * 256 + threadIdx.x;
  const bool live = k < N;
  const size_t rowp = (size_t)bi * N;
  float kv[DH], vv[DH], dk[DH], dv[DH];
#pragma unroll
  for (int u = 0; u < DH; ++u) {
    kv[u] = live ? a.proj[(rowp + k) * C + D + t * DH + u] : 0.f;
    vv[u] = live ? a.proj[(rowp + k) * C + 2 * D + t * DH + u] : 0.f;
    dk[u] = dv[u] = 0.f;
  }
  const size_t st0 = ((size_t)bi * h + t) * N;
  for (int j0 = 0; j0 < N; j0 += QT) {
    for (int e = threadIdx.x; e < QT * DH; e += 256) {
      const int jj = e / DH, u = e - jj * DH, j = j0 + jj;
      qs[jj][u] = j < N ? a.proj[(rowp + j) * C + t * DH + u] * a.rsd : 0.f;
      dos[jj][u] = j < N ? a.dob[(rowp + j) * D + t * DH + u] : 0.f;
    }
    for (int jj = threadIdx.x; jj < QT; jj += 256) {
      const int j = j0 + jj;
      ms[jj] = j < N ? a.m[st0 + j] : 0.f;
      ls[jj] = j < N ? a.l[st0 + j] : 1.f;
      Ds[jj] = j < N ? a.Dj[st0 + j] : 0.f;
    }
    __syncthreads();
    const int jn = min(QT, N - j0);
    if (live) {
      for (int jj = 0; jj < jn; ++jj) {
        const int j = j0 + jj;
        const bool valid = a.mask[((size_t)b * N + j) * N + k] != 0;
        float s = a.zt[((size_t)(b * h + t) * N + j) * N + k];
#pragma unroll
        for (int u = 0; u < DH; ++u) s += qs[jj][u] * kv[u];
        if (!valid) s = a.fill;
        const float p = (s == -INFINITY) ? 0.f : expf(s - ms[jj]) / ls[jj];
        const bool kept = keep_word(a, b, i, t, j, k) >= a.thr;
        float da = 0.f;
        if (kept) {
          const float pw = p * a.scale;
#pragma unroll
          for (int u = 0; u < DH; ++u) {
            dv[u] += pw * dos[jj][u];
            da += dos[jj][u] * vv[u];
          }
          da *= a.scale;
        }
        if (valid) {
          const float ds = p * (da - Ds[jj]);
#pragma unroll
          for (int u = 0; u < DH; ++u) dk[u] += ds * qs[jj][u];
        }
      }
    }
    __syncthreads();
  }
  if (!live) return;
#pragma unroll
  for (int u = 0; u < DH; ++u) {
    a.dcat[(rowp + k) * C + D + t * DH + u] = dk[u];
    a.dcat[(rowp + k) * C + 2 * D + t * DH + u] = dv[u];
  }
}

// dz[b,t,j,k] = sum over rows i of ds, masked, per (b, t, 16 query columns j,
// 64 key columns k): each thread owns one query and four keys; per row i the
// keys' k and v and the queries' q, do, m, l and sum a da pass through LDS.
template <int DH>
__global__ __launch_bounds__(256) void bwd_attn_dz(BwdAttnArgs a) {
  constexpr int JT = 16, KT = 64;
  __shared__ float ks[KT][DH + 1], vs[KT][DH + 1], qs[JT][DH], dos[JT][DH], ms[JT], ls[JT], Ds[JT];
  const int N = a.N, D = a.D, h = a.h, C = a.C;
  const int nkt = (N + KT - 1) / KT;
  const int bt = blockIdx.y, b = bt / h, t = bt - b * h;
  const int j0 = (blockIdx.x / nkt) * JT, k0 = (blockIdx.x % nkt) * KT;
  const int jj = threadIdx.x >> 4, j = j0 + jj;
  float dz[4] = {0.f, 0.f, 0.f, 0.f};
  // the bias and the mask of (j, k) are the same for every row i
  float zr[4];
  bool valid[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int k = k0 + (threadIdx.x & 15) + 16 * r;
    valid[r] = j < N && k < N && a.mask[((size_t)b * N + j) * N + k] != 0;
    zr[r] = valid[r] ? a.zt[((size_t)(b * h + t) * N + j) * N + k] : 0.f;
  }
  for (int i = 0; i < N; ++i) {
    const size_t rowp = ((size_t)b * N + i) * N;
    for (int e = threadIdx.x; e < KT * DH; e += 256) {
      const int kk = e / DH, u = e - kk * DH, k = k0 + kk;
      ks[kk][u] = k < N ? a.proj[(rowp + k) * C + D + t * DH + u] : 0.f;
      vs[kk][u] = k < N ? a.proj[(rowp + k) * C + 2 * D + t * DH + u] : 0.f;
    }
    for (int e = threadIdx.x; e < JT * DH; e += 256) {
      const int q = e / DH, u = e - q * DH, jq = j0 + q;
      qs[q][u] = jq < N ? a.proj[(rowp + jq) * C + t * DH + u] * a.rsd : 0.f;
      dos[q][u] = jq < N ? a.dob[(rowp + jq) * D + t * DH + u] : 0.f;
    }
    if (threadIdx.x < JT) {
      const int jq = j0 + threadIdx.x;
      const size_t st = (((size_t)b * N + i) * h + t) * N + jq;
      ms[threadIdx.x] = jq < N ? a.m[st] : 0.f;
      ls[threadIdx.x] = jq < N ? a.l[st] : 1.f;
      Ds[threadIdx.x] = jq < N ? a.Dj[st] : 0.f;
    }
    __syncthreads();
    if (j < N) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kk = (threadIdx.x & 15) + 16 * r, k = k0 + kk;
        if (!valid[r]) continue;
        float s = zr[r];
#pragma unroll
        for (int u = 0; u < DH; ++u) s += qs[jj][u] * ks[kk][u];
        const float p = expf(s - ms[jj]) / ls[jj];
        float da = 0.f;
        if (keep_word(a, b, i, t, j, k) >= a.thr) {
#pragma unroll
          for (int u = 0; u < DH; ++u) da += dos[jj][u] * vs[kk][u];
          da *= a.scale;
        }
        dz[r] += p * (da - Ds[jj]);
      }
    }
    __syncthreads();
  }
  if (j >= N) return;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int k = k0 + (threadIdx.x & 15) + 16 * r;
    if (k < N) a.dcat[(((size_t)b * N + j) * N + k) * C + 4 * D + t] = dz[r];
  }
}

// z[b,t,j,k] from the projection columns, into a [B][h][N][N] copy
__global__ __launch_bounds__(256) void bwd_ztrans(const float *proj, int B, int N, int D, int h, int C, float *zt) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long total = (long long)B * h * N * N;
  if (e >= total) return;
  const long long jk = e % ((long long)N * N), bt = e / ((long long)N * N);
  const int b = (int)(bt / h), t = (int)(bt - (long long)b * h);
  zt[e] = proj[((size_t)b * N * N + jk) * C + 4 * D + t];
}

// Output and gate step per (position, head): dg, dgp (into dcat), do, g * o.
template <typename T>
__global__ __launch_bounds__(256) void bwd_gate(const float *dgo, const float *proj, const float *o,
                                                 const void *bg, long long npos, int D, int C, float *dcat,
                                                 float *dob, float *go) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e >= npos * D) return;
  const long long p = e / D;
  const int c = (int)(e - p * D);
  const float gp = proj[p * C + 3 * D + c] + ld_elem<T>(bg, c);
  const float g = 1.0f / (1.0f + expf(-gp));
  const float ov = o[e], dv = dgo[e];
  dcat[p * C + 3 * D + c] = dv * ov * g * (1.0f - g);
  dob[e] = dv * g;
  go[e] = g * ov;
}

// ------------------------------------------------------------------ host side
struct BwdLayout {
  size_t x, xhat, rstd, proj, zt, m, l, Dj, o, dgo, dob, go, dcat, dx, part, vpart, total;
  long long S, kchunk, nvblk, vper;
};

static size_t al256(size_t v) { return (v + 255) & ~size_t(255); }

static BwdLayout bwd_layout(int B, int N, int D, int h) {
  BwdLayout L{};
  const long long P = (long long)B * N * N, C = 4LL * D + h;
  // split-K chunks of the weight gradients (sums over all positions): at most
  // 256, each a multiple of 16 positions
  L.kchunk = ((P + 255) / 256 + 15) / 16 * 16;
  if (L.kchunk < 16) L.kchunk = 16;
  L.S = (P + L.kchunk - 1) / L.kchunk;
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
  L.m = take((size_t)B * N * h * N * 4);
  L.l = take((size_t)B * N * h * N * 4);
  L.Dj = take((size_t)B * N * h * N * 4);
  L.o = take((size_t)P * D * 4);
  L.dgo = take((size_t)P * D * 4);
  L.dob = take((size_t)P * D * 4);
  L.go = take((size_t)P * D * 4);
  L.dcat = take((size_t)P * C * 4);
  L.dx = take((size_t)P * D * 4);
  L.part = take((size_t)L.S * C * D * 4);
  L.vpart = take((size_t)2 * L.nvblk * D * 4);
  L.total = off;
  return L;
}

size_t bwd_workspace_bytes(int B, int N, int D, int h) { return bwd_layout(B, N, D, h).total; }

template <typename TA, typename TB>
static hipError_t gemm(const void *A, long long sam, long long sak, const void *Bm, long long sbk, long long sbn,
                       float *C, long long scz, long long scm, long long M, long long N, long long K,
                       long long kchunk, int nz, hipStream_t s) {
  GemmArgs g{A, Bm, C, M, N, K, kchunk, sam, sak, sbk, sbn, scz, scm};
  const dim3 grid((unsigned)((M + 63) / 64), (unsigned)((N + 63) / 64), (unsigned)nz);
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
  const BwdLayout L = bwd_layout(B, N, D, h);
  char *w = static_cast<char *>(r.ws);
  float *x = reinterpret_cast<float *>(w + L.x), *xhat = reinterpret_cast<float *>(w + L.xhat);
  float *rstd = reinterpret_cast<float *>(w + L.rstd), *proj = reinterpret_cast<float *>(w + L.proj);
  float *zt = reinterpret_cast<float *>(w + L.zt), *o = reinterpret_cast<float *>(w + L.o);
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
  // LayerNorm and the five projections, in float32
  hipLaunchKernelGGL((bwd_ln<T, D>), dim3((unsigned)((P + 3) / 4)), dim3(256), 0, s, r.P, gamma, beta, r.eps, P, x,
                     xhat, rstd);
  TPA_CHECK(hipGetLastError());
  TPA_CHECK((gemm<float, T>(x, D, 1, r.wpack, 1, D, proj, 0, C, P, C, D, D, 1, s)));
  hipLaunchKernelGGL(bwd_ztrans, dim3((unsigned)(((long long)B * h * N * N + 255) / 256)), dim3(256), 0, s, proj, B,
                     N, D, h, (int)C, zt);
  TPA_CHECK(hipGetLastError());
  BwdAttnArgs aa{};
  aa.proj = proj, aa.zt = zt, aa.mask = r.mask;
  aa.m = reinterpret_cast<float *>(w + L.m), aa.l = reinterpret_cast<float *>(w + L.l);
  aa.Dj = reinterpret_cast<float *>(w + L.Dj);
  aa.o = o, aa.dob = dob, aa.dcat = dcat;
  aa.fill = r.fill, aa.scale = r.scale, aa.rsd = 1.0f / sqrtf((float)DH);
  aa.thr = r.thr, aa.seed_lo = r.seed_lo, aa.seed_hi = r.seed_hi, aa.offset = r.offset;
  aa.B = B, aa.N = N, aa.D = D, aa.h = h, aa.C = (int)C;
  const dim3 ga((unsigned)(B * N * h), (unsigned)((N + 255) / 256));  // x: (b, i, t), y: column block
  hipLaunchKernelGGL((bwd_attn_fwd<DH>), ga, dim3(256), 0, s, aa);
  TPA_CHECK(hipGetLastError());
  // output projection and gate
  TPA_CHECK((gemm<T, T>(r.dy, D, 1, Wo, D, 1, dgo, 0, D, P, D, D, D, 1, s)));
  hipLaunchKernelGGL((bwd_gate<T>), dim3((unsigned)((P * D + 255) / 256)), dim3(256), 0, s, dgo, proj, o, bg, P, D,
                     (int)C, dcat, dob, go);
  TPA_CHECK(hipGetLastError());
  // attention
  hipLaunchKernelGGL((bwd_attn_dq<DH>), ga, dim3(256), 0, s, aa);
  TPA_CHECK(hipGetLastError());
  hipLaunchKernelGGL((bwd_attn_dkv<DH>), ga, dim3(256), 0, s, aa);
  TPA_CHECK(hipGetLastError());
  const int nkt = (N + 63) / 64, njt = (N + 15) / 16;
  hipLaunchKernelGGL((bwd_attn_dz<DH>), dim3((unsigned)(njt * nkt), (unsigned)(B * h)), dim3(256), 0, s, aa);
  TPA_CHECK(hipGetLastError());
  // projections and LayerNorm
  TPA_CHECK((gemm<float, T>(dcat, C, 1, r.wpack, D, 1, dx, 0, D, P, D, C, C, 1, s)));
  hipLaunchKernelGGL((bwd_ln_back<T, D>), dim3((unsigned)L.nvblk), dim3(D), 0, s, dx, xhat, rstd, gamma, P, L.vper,
                     r.g.d_pair_repr, vpart, vpart + (size_t)L.nvblk * D);
  TPA_CHECK(hipGetLastError());
  TPA_CHECK(reduce(vpart, D, (int)L.nvblk, D, r.g.d_ln_weight, s));
  TPA_CHECK(reduce(vpart + (size_t)L.nvblk * D, D, (int)L.nvblk, D, r.g.d_ln_bias, s));
  // weight gradients: split-K partial products over positions, then ordered sums
  TPA_CHECK((gemm<float, float>(dcat, 1, C, x, D, 1, part, C * D, D, C, D, P, L.kchunk, (int)L.S, s)));
  float *dst[5] = {r.g.d_w_query, r.g.d_w_key, r.g.d_w_value, r.g.d_w_gate, r.g.d_w_bias_proj};
  for (int q = 0; q < 5; ++q)
    TPA_CHECK(reduce(part + (size_t)q * D * D, (q < 4 ? D : h) * (long long)D, (int)L.S, C * D, dst[q], s));
  TPA_CHECK((gemm<T, float>(r.dy, 1, D, go, D, 1, part, (long long)D * D, D, D, D, P, L.kchunk, (int)L.S, s)));
  TPA_CHECK(reduce(part, (long long)D * D, (int)L.S, (long long)D * D, r.g.d_w_out, s));
  // bias gradients: column sums over positions
  hipLaunchKernelGGL((bwd_colsum<T>), dim3((unsigned)L.nvblk), dim3(256), 0, s, r.dy, P, D, (long long)D, L.vper,
                     vpart);
  TPA_CHECK(hipGetLastError());
  TPA_CHECK(reduce(vpart, D, (int)L.nvblk, D, r.g.d_b_out, s));
  hipLaunchKernelGGL((bwd_colsum<float>), dim3((unsigned)L.nvblk), dim3(256), 0, s, dcat + 3 * D, P, D, C, L.vper,
                     vpart);
  TPA_CHECK(hipGetLastError());
  TPA_CHECK(reduce(vpart, D, (int)L.nvblk, D, r.g.d_b_gate, s));
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

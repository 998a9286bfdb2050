// Kernel 2 of the triangular self-attention forward: per pair row (b, i),
// attention of the query columns j over the key columns k with the shared
// pair bias and mask, softmax over k, the value sum, the gate multiply and
// the output projection (Kimi-K2.6 / l2_p6 transcript: steps 8-18 of its
// forward listing, its attention and finalize kernels; FW-GLM-5-1 / l2_p6:
// the fused attention and output kernels).
//
// Workgroup = (b, IG rows i, JW*16 query columns j), one wave per head. The
// (B, N, h, N, N) scores are never stored: each wave streams key tiles.
//
// Softmax without a running maximum. Per (row i, query j) the kernel fixes
// the shift m = |q'_j| * max_k |k_k| + max_k zm[j, k] before the key loop
// (Cauchy-Schwarz: m >= every score of the row, so exp2(s - m) <= 1 and
// nothing overflows). Softmax is invariant to the shift, so the result is
// exact up to rounding; the loop then needs no max, no rescaling and no
// cross-lane traffic. The shift enters the MFMA itself (an extra K-slot with
// q' = -m, k = 1), and the score tile's accumulator starts from the bias+mask
// tile zm, so the only VALU work per score is exp2 and the bf16 conversion.
// The row sum comes out of the MFMA too (a row of ones next to V). If the
// bound is so loose that a column's sum falls below 2^-64 (only with
// pathological inputs or the shift_slack test knob), the wave recomputes that
// column block with the exact maximum (a max pass, then the loop again).
//
// Mask: zm = -inf where masked, so masked keys get weight exactly 0. A query
// column whose keys are all masked (max zm = -inf) gets the rule of the
// finite fill value: uniform weights over all N keys, i.e. the mean of v; or
// NaN when the fill is -inf. Key chunks of 64 that are masked for every query
// of the wave are skipped.
//
// Epilogue: o / l, times the gate, into LDS as one [positions][D] tile for
// all heads; then (gate*o) Wo^T + bo on MFMA with Wo fragments in registers.
#include "device_common.h"
#include "tri_attn_internal.h"

#include <type_traits>

#include "tri_attn.h"

namespace tpa {

// Rows i per workgroup (IG) and 16-column query blocks per wave (JW). The bias
// tile is reused across the IG rows in registers; k and v across the JW*16
// columns. Workgroups with 4 waves (h = 4) take 2 rows to keep 2 waves per SIMD.
template <int D, int DH>
struct K2Shape {
  static constexpr int IG = (D / DH >= 8) ? 4 : 2;
  static constexpr int JW = 2;
};

template <typename T, int D, int DH>
__global__ __launch_bounds__(64 * (D / DH)) void k2_attention(K2Args a) {
  constexpr bool BF = is_bf16<T>::value;
  constexpr int ES = BF ? 2 : 4;
  constexpr int H = D / DH;
  constexpr int NB = D / 16;
  constexpr int MB = DH / 16;  // 16-row blocks of one head's channels
  constexpr int IG = K2Shape<D, DH>::IG;
  constexpr int JW = K2Shape<D, DH>::JW;
  constexpr int NJ = JW * 16;
  constexpr int NPOS = IG * NJ;
  constexpr int PITCH = D + 16 / ES;
  constexpr int KQ = D / 4;
  constexpr int KSO = BF ? D / 32 : D / 4;  // output-projection MFMA steps
  constexpr int NBO = NB / H;               // output channel blocks per wave
  constexpr int KSTEP = BF ? 32 : 16;       // keys per loop step
  constexpr int QS = DH / 4;                // fp32: q/k elements per lane
  using Frag = typename std::conditional<BF, bf16x8, float>::type;
  static_assert(NBO >= 1, "");

  __shared__ __align__(16) T go[NPOS * PITCH];

  const int lane = threadIdx.x & 63, t = threadIdx.x >> 6;  // wave = head
  const int g = lane >> 4, r16 = lane & 15;
  const int N = a.N, Np = a.Np, nch = a.nchunk;

  // ---- work item, XCD-aware. Workgroup w runs on XCD w % 8; each XCD takes a
  // contiguous range of the linear order below, in which consecutive items form
  // super-tiles of SI row groups x SJ query ranges (about one item per CU of an
  // XCD), so the concurrently running workgroups of an XCD share k, v (same
  // rows) and the bias tile (same query columns) through its L2.
  const int nJR = (N + NJ - 1) / NJ, nIG = (N + IG - 1) / IG;
  int lin = blockIdx.x;
  {
    const int w8 = (a.items / 8) * 8;
    if (lin < w8) lin = (lin & 7) * (w8 / 8) + (lin >> 3);
  }
  const int per_b = nIG * nJR;
  const int b = lin / per_b;
  int ig, jr;
  {
    const int SJ = nJR < 8 ? nJR : 8;
    const int SI = 32 / SJ;
    const int rem = lin - b * per_b;
    const int igs = (rem / (SI * nJR)) * SI;
    const int si = min(SI, nIG - igs);
    const int r2 = rem - igs * nJR;
    const int jrs = (r2 / (si * SJ)) * SJ;
    const int sj = min(SJ, nJR - jrs);
    const int r3 = r2 - jrs * si;
    ig = igs + r3 / sj;
    jr = jrs + r3 % sj;
  }
  const int i0 = ig * IG, j0 = jr * NJ;

  const T *Q = reinterpret_cast<const T *>(a.q);
  const T *K = reinterpret_cast<const T *>(a.k);
  const T *VT = reinterpret_cast<const T *>(a.vt);
  const T *G = reinterpret_cast<const T *>(a.g);

  int rows[IG];
  float kn2[IG];
#pragma unroll
  for (int i = 0; i < IG; ++i) {
    rows[i] = min(i0 + i, N - 1);
    // |k|^2 <= sum over the head's 16-channel blocks of each block's chunk maxima
    float m2 = 0.f;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const float *kp = a.kmax + ((size_t)(b * N + rows[i]) * NB + t * MB + mb) * nch;
      float m = 0.f;
      for (int c = 0; c < nch; ++c) m = fmaxf(m, kp[c]);
      m2 += m;
    }
    kn2[i] = m2;
  }

  // ---- per query column: bias+mask maximum, last live key chunk
  float zmx[JW];
  int jrow[JW];
  int kend = 0;
#pragma unroll
  for (int jb = 0; jb < JW; ++jb) {
    const int j = j0 + jb * 16 + r16;
    jrow[jb] = min(j, N - 1);
    float zx = -INFINITY;
    if (j < N) {
      const float *zp = a.zmax + ((size_t)(b * H + t) * N + j) * nch;
      for (int c = 0; c < nch; ++c) {
        const float v = zp[c];
        zx = fmaxf(zx, v);
        if (v > -INFINITY) kend = c + 1;
      }
    }
    zmx[jb] = zx;
  }
  for (int m = 1; m < 64; m <<= 1) kend = max(kend, __shfl_xor(kend, m, 64));
  const int kend_keys = __builtin_amdgcn_readfirstlane(kend) * kChunk;

  // ---- query fragments and their norms; the shift
  // bf16: lane (g, r16) holds q'[j = r16][8g..8g+7] (d = 16: groups 0-1 real, group 2 slot 0 = -m);
  // fp32: lane (g, r16) holds q'[j][g*d/4 .. +d/4).
  Frag qf[IG][JW][BF ? 1 : QS];
  bf16x4 qsh[IG][JW];  // bf16, d = 32: B operand of the 16x16x16 shift MFMA
  float msh[IG][JW];
#pragma unroll
  for (int i = 0; i < IG; ++i)
#pragma unroll
    for (int jb = 0; jb < JW; ++jb) {
      const int j = j0 + jb * 16 + r16;  // < Np
      const size_t rowbase = (size_t)(b * N + rows[i]) * NB;
      float n2 = 0.f;
      if constexpr (BF) {
        const int cb = (DH == 16) ? t : 2 * t + (g >> 1);
        const int off = (DH == 16) ? 8 * (g & 1) : 8 * (g & 1);
        uint4 raw = ldg<uint4>(Q + ((rowbase + cb) * Np + j) * 16 + off);
        if (DH == 16 && g >= 2) raw = make_uint4(0, 0, 0, 0);
        qf[i][jb][0] = as_bf16x8(raw);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = (float)qf[i][jb][0][e];
          n2 += x * x;
        }
      } else {
        const int cb = (DH == 16) ? t : 2 * t + (g >> 1);
        const int off = (DH == 16) ? 4 * g : 8 * (g & 1);
        const float *src = reinterpret_cast<const float *>(Q) + ((rowbase + cb) * Np + j) * 16 + off;
#pragma unroll
        for (int s = 0; s < QS; s += 4) {
          float4 v = ldg<float4>(src + s);
          qf[i][jb][s] = v.x, qf[i][jb][s + 1] = v.y, qf[i][jb][s + 2] = v.z, qf[i][jb][s + 3] = v.w;
        }
#pragma unroll
        for (int s = 0; s < QS; ++s) n2 += qf[i][jb][s] * qf[i][jb][s];
      }
      n2 = group4_sum(n2);
      msh[i][jb] = (zmx[jb] == -INFINITY) ? 0.f : sqrtf(n2 * kn2[i]) + zmx[jb] + a.shift_slack;
    }

  auto set_shift = [&](const float (&m)[IG][JW]) {
    if constexpr (BF) {
#pragma unroll
      for (int i = 0; i < IG; ++i)
#pragma unroll
        for (int jb = 0; jb < JW; ++jb) {
          const __bf16 nm = (__bf16)(-m[i][jb]);
          const __bf16 z = (__bf16)0.f;
          if (DH == 16) {
            if (g == 2) qf[i][jb][0] = bf16x8{nm, z, z, z, z, z, z, z};
          } else {
            qsh[i][jb] = (g == 0) ? bf16x4{nm, z, z, z} : bf16x4{z, z, z, z};
          }
        }
    }
  };
  set_shift(msh);

  // ---- accumulators
  f32x4 o[IG][JW][MB];
  f32x4 ol[IG][JW];     // bf16: row 0 = sum of p (ones row)
  float lacc[IG][JW];   // fp32: per-lane partial sums
  auto zero_acc = [&]() {
#pragma unroll
    for (int i = 0; i < IG; ++i)
#pragma unroll
      for (int jb = 0; jb < JW; ++jb) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) o[i][jb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
        ol[i][jb] = f32x4{0.f, 0.f, 0.f, 0.f};
        lacc[i][jb] = 0.f;
      }
  };

  const float *ZM = a.zm + (size_t)(b * H + t) * N * Np;
  const __bf16 one = (__bf16)1.f, zero = (__bf16)0.f;
  // constant operands: ones row for the sum, unit key slot for the shift
  const bf16x8 ones8 = (r16 == 0) ? bf16x8{one, one, one, one, one, one, one, one}
                                  : bf16x8{zero, zero, zero, zero, zero, zero, zero, zero};
  const bf16x8 kunit = (g == 2) ? bf16x8{one, zero, zero, zero, zero, zero, zero, zero}
                                : bf16x8{zero, zero, zero, zero, zero, zero, zero, zero};
  const bf16x4 kunit4 = (g == 0) ? bf16x4{one, zero, zero, zero} : bf16x4{zero, zero, zero, zero};

  // Score tiles of one (row, key step): bf16 -> sA (keys k0+8g+0..3), sB (k0+8g+4..7);
  // fp32 -> s (keys k0+4g+0..3). Shared by the main loop and the max pass.
  // The bias+mask tile of the next key step is loaded one step ahead (it is
  // the operand least likely to be in L2).
  auto main_loop = [&](bool max_pass, float (&mx)[IG][JW]) {
    if (kend_keys == 0) return;
    f32x4 zA[JW], zB[JW];  // bf16: keys k0+8g+0..3 and k0+8g+4..7; fp32: zA = keys k0+4g+0..3
    auto load_z = [&](int k0, f32x4 (&za)[JW], f32x4 (&zb)[JW]) {
#pragma unroll
      for (int jb = 0; jb < JW; ++jb) {
        if constexpr (BF) {
          const float *zp = ZM + (size_t)jrow[jb] * Np + k0 + 8 * g;
          za[jb] = ldg<f32x4>(zp);
          zb[jb] = ldg<f32x4>(zp + 4);
        } else {
          za[jb] = ldg<f32x4>(ZM + (size_t)jrow[jb] * Np + k0 + 4 * g);
        }
      }
    };
    load_z(0, zA, zB);
#pragma unroll 1
    for (int k0 = 0; k0 < kend_keys; k0 += KSTEP) {
      f32x4 nA[JW], nB[JW];
      load_z(k0 + KSTEP < kend_keys ? k0 + KSTEP : k0, nA, nB);
      if constexpr (BF) {
        const int keyA = k0 + 8 * (r16 >> 2) + (r16 & 3);  // S^T row r16 of tile A
#pragma unroll
        for (int i = 0; i < IG; ++i) {
          const size_t rowbase = (size_t)(b * N + rows[i]) * NB;
          bf16x8 kA, kB;
          {
            const int cb = (DH == 16) ? t : 2 * t + (g >> 1);
            const T *kp = K + ((rowbase + cb) * Np + keyA) * 16 + 8 * (g & 1);
            kA = as_bf16x8(ldg<uint4>(kp));
            kB = as_bf16x8(ldg<uint4>(kp + 4 * 16));
            if (DH == 16 && g >= 2) kA = kunit, kB = kunit;
          }
          bf16x8 vf[MB];
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            vf[mb] = as_bf16x8(
                ldg<uint4>(VT + (((size_t)(b * N + rows[i]) * H + t) * DH + mb * 16 + r16) * Np + k0 + 8 * g));
#pragma unroll
          for (int jb = 0; jb < JW; ++jb) {
            f32x4 sA = mfma(kA, qf[i][jb][0], zA[jb]);
            f32x4 sB = mfma(kB, qf[i][jb][0], zB[jb]);
            if (DH == 32 && !max_pass) {
              sA = mfma(kunit4, qsh[i][jb], sA);
              sB = mfma(kunit4, qsh[i][jb], sB);
            }
            if (max_pass) {
              float m = mx[i][jb];
#pragma unroll
              for (int e = 0; e < 4; ++e) m = fmaxf(m, fmaxf(sA[e], sB[e]));
              mx[i][jb] = m;
            } else {
              bf16x8 p;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                p[e] = (__bf16)fast_exp2(sA[e]);
                p[4 + e] = (__bf16)fast_exp2(sB[e]);
              }
#pragma unroll
              for (int mb = 0; mb < MB; ++mb) o[i][jb][mb] = mfma(vf[mb], p, o[i][jb][mb]);
              ol[i][jb] = mfma(ones8, p, ol[i][jb]);
            }
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < IG; ++i) {
          const size_t rowbase = (size_t)(b * N + rows[i]) * NB;
          float kf[QS];
          {
            const int cb = (DH == 16) ? t : 2 * t + (g >> 1);
            const int off = (DH == 16) ? 4 * g : 8 * (g & 1);
            const float *kp = reinterpret_cast<const float *>(K) + ((rowbase + cb) * Np + k0 + r16) * 16 + off;
#pragma unroll
            for (int s = 0; s < QS; s += 4) {
              float4 v = ldg<float4>(kp + s);
              kf[s] = v.x, kf[s + 1] = v.y, kf[s + 2] = v.z, kf[s + 3] = v.w;
            }
          }
          f32x4 vf[MB];
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            vf[mb] = ldg<f32x4>(reinterpret_cast<const float *>(VT) +
                                (((size_t)(b * N + rows[i]) * H + t) * DH + mb * 16 + r16) * Np + k0 + 4 * g);
#pragma unroll
          for (int jb = 0; jb < JW; ++jb) {
            f32x4 s = zA[jb];
#pragma unroll
            for (int ss = 0; ss < QS; ++ss) s = mfma(kf[ss], qf[i][jb][ss], s);
            if (max_pass) {
              float m = mx[i][jb];
#pragma unroll
              for (int e = 0; e < 4; ++e) m = fmaxf(m, s[e]);
              mx[i][jb] = m;
            } else {
              float p[4];
              const float sh = msh[i][jb];
#pragma unroll
              for (int e = 0; e < 4; ++e) p[e] = fast_exp2(s[e] - sh);
              lacc[i][jb] += (p[0] + p[1]) + (p[2] + p[3]);
#pragma unroll
              for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) o[i][jb][mb] = mfma(vf[mb][e], p[e], o[i][jb][mb]);
            }
          }
        }
      }
#pragma unroll
      for (int jb = 0; jb < JW; ++jb) {
        zA[jb] = nA[jb];
        if constexpr (BF) zB[jb] = nB[jb];
      }
    }
  };

  float lsum[IG][JW];
  auto row_sums = [&]() {
#pragma unroll
    for (int i = 0; i < IG; ++i)
#pragma unroll
      for (int jb = 0; jb < JW; ++jb) {
        if constexpr (BF)
          lsum[i][jb] = __shfl(ol[i][jb][0], r16, 64);  // row 0 lives in lane group 0
        else
          lsum[i][jb] = group4_sum(lacc[i][jb]);
      }
  };

  float dummy[IG][JW];
  zero_acc();
  main_loop(false, dummy);
  row_sums();

  // ---- recovery: exact maximum where the bound was too loose
  bool need = false;
#pragma unroll
  for (int i = 0; i < IG; ++i)
#pragma unroll
    for (int jb = 0; jb < JW; ++jb)
      if (zmx[jb] > -INFINITY && !(lsum[i][jb] >= 0x1p-64f)) need = true;
  if (__ballot(need) != 0) {
    float mx[IG][JW];
#pragma unroll
    for (int i = 0; i < IG; ++i)
#pragma unroll
      for (int jb = 0; jb < JW; ++jb) {
        mx[i][jb] = -INFINITY;
        msh[i][jb] = 0.f;
      }
    set_shift(msh);  // no shift during the max pass
    main_loop(true, mx);
#pragma unroll
    for (int i = 0; i < IG; ++i)
#pragma unroll
      for (int jb = 0; jb < JW; ++jb) {
        const float m = group4_max(mx[i][jb]);
        msh[i][jb] = (zmx[jb] == -INFINITY) ? 0.f : m;
      }
    set_shift(msh);
    zero_acc();
    main_loop(false, dummy);
    row_sums();
  }

  // ---- normalise, fully masked columns, gate -> LDS tile [NPOS][D]
  const bool fill_nan = (a.mask_fill == -INFINITY);
  const float inv_n = 1.0f / (float)N;
#pragma unroll
  for (int i = 0; i < IG; ++i) {
    bool masked_any = false;
#pragma unroll
    for (int jb = 0; jb < JW; ++jb) masked_any |= (zmx[jb] == -INFINITY);
    float vmean[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) vmean[mb][r] = 0.f;
    if (__ballot(masked_any) != 0 && !fill_nan) {
      // mean of v over all N keys (padding keys hold zeros), lane (g, u) partial over its key slots
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const T *vrow = VT + (((size_t)(b * N + rows[i]) * H + t) * DH + mb * 16 + r16) * Np;
        float s = 0.f;
        for (int k0 = 4 * g; k0 < Np; k0 += 16) {
          if constexpr (BF) {
            const uint2 w = ldg<uint2>(vrow + k0);
            s += (bflo(w.x) + bfhi(w.x)) + (bflo(w.y) + bfhi(w.y));
          } else {
            const float4 w = ldg<float4>(vrow + k0);
            s += (w.x + w.y) + (w.z + w.w);
          }
        }
        s = group4_sum(s) * inv_n;  // lanes (*, u) hold mean v[u]
#pragma unroll
        for (int r = 0; r < 4; ++r) vmean[mb][r] = __shfl(s, 4 * g + r, 64);
      }
    }
#pragma unroll
    for (int jb = 0; jb < JW; ++jb) {
      const int j = j0 + jb * 16 + r16;
      const int pos = i * NJ + jb * 16 + r16;
      const bool masked = (zmx[jb] == -INFINITY);
      const float inv_l = masked ? 0.f : 1.0f / lsum[i][jb];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int cb = t * MB + mb;
        const T *gp = G + (((size_t)(b * N + rows[i]) * NB + cb) * Np + j) * 16 + 4 * g;
        float gv[4];
        if constexpr (BF) {
          const uint2 w = ldg<uint2>(gp);
          gv[0] = bflo(w.x), gv[1] = bfhi(w.x), gv[2] = bflo(w.y), gv[3] = bfhi(w.y);
        } else {
          const float4 w = ldg<float4>(gp);
          gv[0] = w.x, gv[1] = w.y, gv[2] = w.z, gv[3] = w.w;
        }
        float ov[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float oo = masked ? (fill_nan ? __builtin_nanf("") : vmean[mb][r]) : o[i][jb][mb][r] * inv_l;
          ov[r] = oo * gv[r];
        }
        T *dst = &go[pos * PITCH + t * DH + mb * 16 + 4 * g];
        if constexpr (BF)
          *reinterpret_cast<uint2 *>(dst) = make_uint2(pack_bf16x2(ov[0], ov[1]), pack_bf16x2(ov[2], ov[3]));
        else
          *reinterpret_cast<float4 *>(dst) = make_float4(ov[0], ov[1], ov[2], ov[3]);
      }
    }
  }
  lds_barrier();

  // ---- output projection: y^T[c][pos] = Wo[c] . go[pos] + bo[c]
  const T *Wo = reinterpret_cast<const T *>(a.Wo);
#pragma unroll
  for (int ob = 0; ob < NBO; ++ob) {
    const int cbo = t * NBO + ob;
    Frag wo[KSO];
    const T *wrow = Wo + (size_t)(cbo * 16 + r16) * D + g * KQ;
    if constexpr (BF) {
#pragma unroll
      for (int s = 0; s < KSO; ++s) wo[s] = as_bf16x8(ldg<uint4>(wrow + 8 * s));
    } else {
#pragma unroll
      for (int s = 0; s < KSO; s += 4) {
        float4 v = ldg<float4>(wrow + s);
        wo[s] = v.x, wo[s + 1] = v.y, wo[s + 2] = v.z, wo[s + 3] = v.w;
      }
    }
    f32x4 bias;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = cbo * 16 + 4 * g + r;
      bias[r] = BF ? bf2f(reinterpret_cast<const uint16_t *>(a.bo)[c]) : reinterpret_cast<const float *>(a.bo)[c];
    }
#pragma unroll 1
    for (int pb = 0; pb < IG * JW; ++pb) {
      const int i = pb / JW, jb = pb - i * JW;
      const T *grow = &go[(pb * 16 + r16) * PITCH + g * KQ];
      f32x4 acc = bias;
      if constexpr (BF) {
#pragma unroll
        for (int s = 0; s < KSO; ++s) acc = mfma(wo[s], as_bf16x8(*reinterpret_cast<const uint4 *>(grow + 8 * s)), acc);
      } else {
#pragma unroll
        for (int s = 0; s < KSO; s += 4) {
          const float4 v = *reinterpret_cast<const float4 *>(grow + s);
          acc = mfma(wo[s], v.x, acc);
          acc = mfma(wo[s + 1], v.y, acc);
          acc = mfma(wo[s + 2], v.z, acc);
          acc = mfma(wo[s + 3], v.w, acc);
        }
      }
      const int row = i0 + i, j = j0 + jb * 16 + r16;
      if (row < N && j < N) {
        T *dst = reinterpret_cast<T *>(a.out) + ((size_t)(b * N + row) * N + j) * D + cbo * 16 + 4 * g;
        if constexpr (BF)
          stg<uint2>(dst, make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])));
        else
          stg<float4>(dst, make_float4(acc[0], acc[1], acc[2], acc[3]));
      }
    }
  }
}

template <typename T, int D, int DH>
static hipError_t launch_k2_t(const K2Args &a, hipStream_t s) {
  hipLaunchKernelGGL((k2_attention<T, D, DH>), dim3(a.items), dim3(64 * (D / DH)), 0, s, a);
  return hipGetLastError();
}

int k2_items(int D, int dh, int B, int N) {
  int IG = 4, NJ = 32;
#define TRI_K2_SHAPE(DD, HH)                 \
  if (D == DD && dh == HH) {                 \
    IG = K2Shape<DD, HH>::IG;                \
    NJ = K2Shape<DD, HH>::JW * 16;           \
  }
  TRI_K2_SHAPE(128, 16)
  TRI_K2_SHAPE(128, 32)
  TRI_K2_SHAPE(64, 16)
  TRI_K2_SHAPE(64, 32)
#undef TRI_K2_SHAPE
  return B * ((N + IG - 1) / IG) * ((N + NJ - 1) / NJ);
}

hipError_t launch_k2(int dtype, int D, int dh, const K2Args &a, hipStream_t s) {
#define TRI_K2_CASE(TT, DD, HH) \
  if (D == DD && dh == HH) return launch_k2_t<TT, DD, HH>(a, s);
  if (dtype == TRI_ATTN_BF16) {
    TRI_K2_CASE(bf16_t, 128, 16)
    TRI_K2_CASE(bf16_t, 128, 32)
    TRI_K2_CASE(bf16_t, 64, 16)
    TRI_K2_CASE(bf16_t, 64, 32)
  } else {
    TRI_K2_CASE(float, 128, 16)
    TRI_K2_CASE(float, 128, 32)
    TRI_K2_CASE(float, 64, 16)
    TRI_K2_CASE(float, 64, 32)
  }
#undef TRI_K2_CASE
  return hipErrorInvalidValue;
}

}  // namespace tpa

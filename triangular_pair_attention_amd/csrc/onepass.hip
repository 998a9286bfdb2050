// One-pass variant of the triangular self-attention forward: the projections
// q, k, v and the gate never leave the chip (Kimi-K2.6 / l2_p6 transcript:
// the single fused kernel approach, one block per (b, i) row doing LayerNorm,
// the projections and the attention of that row, and its Option A / Option B
// comparison, which notes that the pair bias depends on every position of
// the batch element and so needs a pass of its own first).
//
// Two kernels:
//
//   op_bias   the pre-pass: LayerNorm of every position and the pair-bias
//             projection only, z[b,t,j,k] * log2(e) with the mask folded in
//             (-inf where masked and for the key padding), [b][t][j][Np].
//
//   op_fused  one workgroup per pair row (b, i), 8 waves; wave w owns the
//             16-position blocks w, w + 8, ... of the row. For each head t:
//               A. every wave recomputes LayerNorm of its positions (row
//                  statistics kept in registers), projects k_t and v_t on the
//                  matrix cores and stores them in LDS (k as [key][c], v
//                  transposed as [c][key]) for the whole row;
//               B. every wave recomputes q_t and the gate for its own query
//                  positions, runs the attention over all keys with a running
//                  maximum (online softmax, no bound needed), multiplies by
//                  the gate and adds this head's share of the output
//                  projection Wo[:, t] (g*o)_t to float32 accumulators that
//                  stay in registers for the whole row.
//             At the end the row's y (+ bo) is written once.
//
// Matrix-core layouts (lane l = 16 g + r16): the score tile is built
// transposed, S^T = k q^T (keys in rows, queries in columns), so each lane
// owns one query column and four keys, and its result registers are exactly
// the operand registers of the next products: S^T's four keys per lane are
// the k-slice of the P^T operand of o^T = v^T P^T, and o^T's four channels
// per lane are the k-slice of the (g*o)^T operand of y^T = Wo (g*o)^T.
// The softmax column maximum needs only a reduction over the four lane
// groups. bf16 uses 16x16x16 products for the attention and the output and
// 16x16x32 for the projections; float32 uses 16x16x4 float32 products
// throughout (the channel or key assigned to lane group g in step e is
// 4g + e of each 16-slice, the same for both operands).
//
// Rows of one batch element go to the same XCD (blockIdx -> row remap), so
// the bias slices z[b, t] that every row of the element reads head after
// head are shared in that XCD's L2.
//
// Limits: N <= 512 (a wave holds the output accumulators of up to four
// position blocks), head size 16 or 32, D = 64 or 128.
#include "device_common.h"
#include "tri_attn.h"
#include "tri_attn_internal.h"

#include <type_traits>

namespace tpa {

// ------------------------------------------------------------------ pre-pass
// 16 lanes per position, 16 positions per workgroup. Position (b, r, c) of
// the output's own indexing: query column r, key column c; the ending-node
// variant reads pair_repr and the mask at (b, c, r).
template <typename T, int D>
__global__ __launch_bounds__(256) void op_bias(OnePassArgs a) {
  constexpr int CPL = D / 16;  // channels per lane
  const int H = a.h, N = a.N, Np = a.Np;
  const int l16 = threadIdx.x & 15;
  const long long P = (long long)a.B * N * N;
  const long long pos = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const bool live = pos < P;
  const long long pc = live ? pos : P - 1;
  const long long bn = pc / N;
  const int c = (int)(pc - bn * N);
  const int b = (int)(bn / N), r = (int)(bn - (long long)b * N);
  const size_t at = a.transposed ? ((size_t)b * N + c) * N + r : (size_t)pc;
  float x[CPL];
#pragma unroll
  for (int e = 0; e < CPL; ++e) x[e] = ld_elem<T>(a.P, at * D + l16 * CPL + e);
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < CPL; ++e) s += x[e];
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) s = xor_sum(s, m);
  const float mean = s * (1.0f / D);
  float q = 0.f;
#pragma unroll
  for (int e = 0; e < CPL; ++e) q += (x[e] - mean) * (x[e] - mean);
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) q = xor_sum(q, m);
  const float rstd = 1.0f / sqrtf(q * (1.0f / D) + a.eps);
#pragma unroll
  for (int e = 0; e < CPL; ++e) {
    const int ch = l16 * CPL + e;
    x[e] = (x[e] - mean) * rstd * ld_elem<T>(a.vecs, ch) + ld_elem<T>(a.vecs, (size_t)D + ch);
  }
  const bool keep = a.mask[at] != 0;
  const size_t wz = (size_t)4 * D * D;  // Wz rows in the packed weights
  for (int t = 0; t < H; ++t) {
    float z = 0.f;
#pragma unroll
    for (int e = 0; e < CPL; ++e) z = fmaf(x[e], ld_elem<T>(a.W, wz + (size_t)t * D + l16 * CPL + e), z);
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) z = xor_sum(z, m);
    if (live && l16 == t) a.zm[((size_t)(b * H + t) * N + r) * Np + c] = keep ? z * kLog2e : -INFINITY;
  }
  // key padding of the row: -inf
  if (live && c == N - 1 && l16 < H)
    for (int k = N; k < Np; ++k) a.zm[((size_t)(b * H + l16) * N + r) * Np + k] = -INFINITY;
}

// ------------------------------------------------------------------ fused row kernel
template <typename T, int D, int DH>
struct OpShape {
  static constexpr bool BF = is_bf16<T>::value;
  static constexpr int NW = 8;     // waves
  static constexpr int MAXB = 4;   // 16-position blocks per wave: N <= 512
  static constexpr int NPMAX = NW * MAXB * 16;
  static constexpr int KP = DH + 4;           // k row pitch (elements)
  static constexpr int VP = NPMAX + (BF ? 16 : 8);  // v^T row pitch (elements): rows 32 bytes apart mod 256
  using L = typename std::conditional<BF, uint16_t, float>::type;
  static constexpr size_t LDS = (size_t)(NPMAX * KP + DH * VP) * sizeof(L) + NW * DH * 4;
};

template <typename T, int D, int DH>
__global__ __launch_bounds__(512) void op_fused(OnePassArgs a) {
  using S = OpShape<T, D, DH>;
  using L = typename S::L;
  constexpr bool BF = S::BF;
  constexpr int NW = S::NW, MAXB = S::MAXB, KP = S::KP, VP = S::VP;
  constexpr int H = D / DH, CB = DH / 16, OB = D / 16;
  constexpr int KS = BF ? D / 32 : D / 16;  // x slices per lane: 8 bf16 (bf16) or 4 floats (float32)
  // 16-key blocks per softmax step (one column-maximum reduction each); two
  // where the wider head or float32 operands leave fewer registers
  constexpr int KSB = (BF && DH == 16) ? 4 : 2;
  static_assert(S::LDS <= 160 * 1024, "LDS budget");
  __shared__ __align__(16) L kbuf[S::NPMAX * KP];
  __shared__ __align__(16) L vtb[DH * VP];
  __shared__ float vpart[NW][DH];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int g = lane >> 4;
  const int r16 = lane & 15;
  const int N = a.N, Np = a.Np;
  const int nblk = (N + 15) / 16, nkb = Np / 16;
  // row of this workgroup: consecutive rows on one XCD (workgroups are
  // dealt to the 8 XCDs round robin)
  const int rows = a.B * N;
  int item = blockIdx.x;
  if (rows % 8 == 0) item = (blockIdx.x % 8) * (rows / 8) + blockIdx.x / 8;
  const int b = item / N, i = item - b * N;
  const char *W = static_cast<const char *>(a.W);
  const char *V = static_cast<const char *>(a.vecs);
  constexpr int ES = BF ? 2 : 4;
  const T *gamma = reinterpret_cast<const T *>(V), *beta = reinterpret_cast<const T *>(V + D * ES);
  const T *bg = reinterpret_cast<const T *>(V + 2 * D * ES), *bo = reinterpret_cast<const T *>(V + 3 * D * ES);
  const T *Wo = reinterpret_cast<const T *>(V + 4 * D * ES);
  auto pos_at = [&](int j) -> size_t {  // element (b, i, j); ending-node (b, j, i)
    return a.transposed ? ((size_t)b * N + j) * N + i : ((size_t)b * N + i) * N + j;
  };

  // channels of this lane in slice s: bf16 8(g) + 32 s .. +7; float32 4 g + 16 s .. +3
  auto chan = [&](int s) { return BF ? 32 * s + 8 * g : 16 * s + 4 * g; };
  constexpr int CPS = BF ? 8 : 4;  // channels per slice

  // raw channels of position j (zeros past N)
  auto load_raw = [&](int j, float (&x)[KS][CPS]) {
    const bool ok = j < N;
    const char *src = static_cast<const char *>(a.P) + pos_at(ok ? j : 0) * D * ES;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if constexpr (BF) {
        uint4 u = ldg<uint4>(src + chan(s) * 2);
        if (!ok) u = make_uint4(0, 0, 0, 0);
        const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) x[s][2 * e] = bflo(w4[e]), x[s][2 * e + 1] = bfhi(w4[e]);
      } else {
        float4 f = ldg<float4>(src + chan(s) * 4);
        if (!ok) f = make_float4(0.f, 0.f, 0.f, 0.f);
        x[s][0] = f.x, x[s][1] = f.y, x[s][2] = f.z, x[s][3] = f.w;
      }
    }
  };

  // LayerNorm statistics of the wave's positions (lane r16 of block m)
  float mean[MAXB], rstd[MAXB];
#pragma unroll
  for (int m = 0; m < MAXB; ++m) {
    const int blk = wave + NW * m;
    float x[KS][CPS];
    load_raw(blk * 16 + r16, x);
    float s = 0.f;
#pragma unroll
    for (int u = 0; u < KS; ++u)
#pragma unroll
      for (int e = 0; e < CPS; ++e) s += x[u][e];
    s = group4_sum(s);
    const float mu = s * (1.0f / D);
    float q = 0.f;
#pragma unroll
    for (int u = 0; u < KS; ++u)
#pragma unroll
      for (int e = 0; e < CPS; ++e) q += (x[u][e] - mu) * (x[u][e] - mu);
    q = group4_sum(q);
    mean[m] = mu;
    rstd[m] = 1.0f / sqrtf(q * (1.0f / D) + a.eps);
  }

  // keeps the scheduler from hoisting the weight loads of every slice (or
  // output block) ahead of the products: with the output accumulators
  // resident, that would run out of registers
  auto sched_fence = [] { __builtin_amdgcn_sched_barrier(0); };

  // slice s of the normalised x of block m as a matrix-core operand (zeros past N)
  using XF = typename std::conditional<BF, bf16x8, float4>::type;
  auto x_slice = [&](int m, int s) -> XF {
    const int j = (wave + NW * m) * 16 + r16;
    const bool ok = j < N;
    // positions past N read position 0 (always in bounds) and are zeroed below
    const char *src = static_cast<const char *>(a.P) + pos_at(ok ? j : 0) * D * ES;
    float x[CPS];
    if constexpr (BF) {
      const uint4 u = ldg<uint4>(src + chan(s) * 2);
      const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) x[2 * e] = bflo(w4[e]), x[2 * e + 1] = bfhi(w4[e]);
    } else {
      const float4 f = ldg<float4>(src + chan(s) * 4);
      x[0] = f.x, x[1] = f.y, x[2] = f.z, x[3] = f.w;
    }
#pragma unroll
    for (int e = 0; e < CPS; ++e) {
      const int ch = chan(s) + e;
      x[e] = ok ? (x[e] - mean[m]) * rstd[m] * ld_elem<T>(gamma, ch) + ld_elem<T>(beta, ch) : 0.f;
    }
    if constexpr (BF)
      return as_bf16x8(make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                                  pack_bf16x2(x[6], x[7])));
    else
      return make_float4(x[0], x[1], x[2], x[3]);
  };

  // acc += rows row0 + r16 of a packed weight matrix [rows][D] times slice s
  // of x: W x^T (lane: row 4g + r, position r16), or with x_first x W^T
  // (lane: position 4g + r, row r16)
  auto proj_step = [&](f32x4 &acc, const T *Wm, int row0, int s, const XF &xs, bool x_first) {
    const char *wrow = reinterpret_cast<const char *>(Wm) + ((size_t)(row0 + r16) * D) * ES;
    if constexpr (BF) {
      const bf16x8 w = as_bf16x8(ldg<uint4>(wrow + chan(s) * 2));
      acc = x_first ? mfma(xs, w, acc) : mfma(w, xs, acc);
    } else {
      const float4 w = ldg<float4>(wrow + chan(s) * 4);
      const float wv[4] = {w.x, w.y, w.z, w.w}, xv[4] = {xs.x, xs.y, xs.z, xs.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = x_first ? mfma(xv[e], wv[e], acc) : mfma(wv[e], xv[e], acc);
    }
  };
  const T *Wq = reinterpret_cast<const T *>(W);
  const T *Wk = Wq + (size_t)D * D, *Wv = Wq + (size_t)2 * D * D, *Wg = Wq + (size_t)3 * D * D;

  f32x4 yacc[MAXB][OB];
#pragma unroll
  for (int m = 0; m < MAXB; ++m)
#pragma unroll
    for (int o = 0; o < OB; ++o) yacc[m][o] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const float *zbase = a.zm + (size_t)b * H * N * Np;
#pragma unroll 1
  for (int t = 0; t < H; ++t) {
    // g is re-declared opaque for every head, so the per-channel loads (LayerNorm
    // weights, projection rows) are not hoisted out of the head loop and held
    // in registers across it
    asm volatile("" : "+v"(g));
    // A. k_t and v_t of every key of the row into LDS; per-wave sums of v
    float vs[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) vs[cb] = 0.f;
#pragma unroll
    for (int m = 0; m < MAXB; ++m) {
      const int blk = wave + NW * m;
      if (blk < nkb) {
        f32x4 kts[CB], vvs[CB];  // k^T (lane: channel 4g + r, key r16), v (lane: key 4g + r, channel r16)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) kts[cb] = vvs[cb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const XF xs = x_slice(m, s);
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
            proj_step(kts[cb], Wk, t * DH + 16 * cb, s, xs, false);
            proj_step(vvs[cb], Wv, t * DH + 16 * cb, s, xs, true);
          }
          sched_fence();
        }
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const f32x4 kt = kts[cb], v = vvs[cb];
          L *kd = &kbuf[(blk * 16 + r16) * KP + 16 * cb + 4 * g];
          L *vd = &vtb[(16 * cb + r16) * VP + blk * 16 + 4 * g];
          if constexpr (BF) {
            *reinterpret_cast<uint2 *>(kd) = make_uint2(pack_bf16x2(kt[0], kt[1]), pack_bf16x2(kt[2], kt[3]));
            *reinterpret_cast<uint2 *>(vd) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
          } else {
            *reinterpret_cast<float4 *>(kd) = make_float4(kt[0], kt[1], kt[2], kt[3]);
            *reinterpret_cast<float4 *>(vd) = make_float4(v[0], v[1], v[2], v[3]);
          }
          vs[cb] += v[0] + v[1] + v[2] + v[3];  // positions past N hold zeros
        }
      }
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const float s = group4_sum(vs[cb]);
      if (g == 0) vpart[wave][16 * cb + r16] = s;
    }
    __syncthreads();

    // B. attention of the wave's query blocks over every key
    const float *zt = zbase + (size_t)t * N * Np;
#pragma unroll
    for (int m = 0; m < MAXB; ++m) {
      const int blk = wave + NW * m;
      if (blk >= nblk) continue;
      const int jq = min(blk * 16 + r16, N - 1);  // query column of this lane (clamped past N)
      f32x4 qt[CB], gt[CB];
      {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) qt[cb] = gt[cb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const XF xs = x_slice(m, s);
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
            proj_step(qt[cb], Wq, t * DH + 16 * cb, s, xs, false);
            proj_step(gt[cb], Wg, t * DH + 16 * cb, s, xs, false);
          }
          sched_fence();
        }
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          qt[cb] *= a.qscale;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float gp = gt[cb][r] + ld_elem<T>(bg, t * DH + 16 * cb + 4 * g + r);
            gt[cb][r] = 1.0f / (1.0f + __expf(-gp));
          }
        }
      }
      bf16x4 qb[CB];
      if constexpr (BF) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          qb[cb] = __builtin_bit_cast(bf16x4, make_uint2(pack_bf16x2(qt[cb][0], qt[cb][1]),
                                                          pack_bf16x2(qt[cb][2], qt[cb][3])));
      }
      float mrun = -INFINITY, lsum = 0.f;
      f32x4 ot[CB];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) ot[cb] = (f32x4){0.f, 0.f, 0.f, 0.f};
      const float *zq = zt + (size_t)jq * Np;
#pragma unroll 1
      for (int k0 = 0; k0 < Np; k0 += 16 * KSB) {
        f32x4 st[KSB];
#pragma unroll
        for (int kk = 0; kk < KSB; ++kk) {
          const int kb = k0 / 16 + kk;
          const float4 z4 = ldg<float4>(zq + kb * 16 + 4 * g);  // lane: keys 4g + r, query r16
          st[kk] = (f32x4){z4.x, z4.y, z4.z, z4.w};
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
            const L *kp = &kbuf[(kb * 16 + r16) * KP + 16 * cb + 4 * g];
            if constexpr (BF) {
              st[kk] = mfma(__builtin_bit_cast(bf16x4, *reinterpret_cast<const uint2 *>(kp)), qb[cb], st[kk]);
            } else {
              const float4 kv = *reinterpret_cast<const float4 *>(kp);
              st[kk] = mfma(kv.x, qt[cb][0], st[kk]);
              st[kk] = mfma(kv.y, qt[cb][1], st[kk]);
              st[kk] = mfma(kv.z, qt[cb][2], st[kk]);
              st[kk] = mfma(kv.w, qt[cb][3], st[kk]);
            }
          }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kk = 0; kk < KSB; ++kk)
#pragma unroll
          for (int r = 0; r < 4; ++r) mx = fmaxf(mx, st[kk][r]);
        mx = group4_max(mx);
        // every lane stays in the step: the value products take their v^T rows
        // from all lanes, so a column with no live key yet shifts by 0 and
        // adds zeros (exp2(-inf) = 0) instead of skipping the step
        const float mnew = fmaxf(mrun, mx);
        const float msh = mnew == -INFINITY ? 0.f : mnew;
        const float alpha = fast_exp2(mrun - msh);  // 0 while mrun = -inf
        mrun = mnew;
        lsum *= alpha;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) ot[cb] *= alpha;
#pragma unroll
        for (int kk = 0; kk < KSB; ++kk) {
          const int kb = k0 / 16 + kk;
          float p[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            p[r] = fast_exp2(st[kk][r] - msh);  // masked and padded keys: 0
            lsum += p[r];
          }
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
            const L *vp = &vtb[(16 * cb + r16) * VP + kb * 16 + 4 * g];
            if constexpr (BF) {
              const bf16x4 pb = __builtin_bit_cast(bf16x4, make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])));
              ot[cb] = mfma(__builtin_bit_cast(bf16x4, *reinterpret_cast<const uint2 *>(vp)), pb, ot[cb]);
            } else {
              const float4 vv = *reinterpret_cast<const float4 *>(vp);
              ot[cb] = mfma(vv.x, p[0], ot[cb]);
              ot[cb] = mfma(vv.y, p[1], ot[cb]);
              ot[cb] = mfma(vv.z, p[2], ot[cb]);
              ot[cb] = mfma(vv.w, p[3], ot[cb]);
            }
          }
        }
      }
      // o / l (a column without a live key: uniform weights over the N keys
      // for a finite fill, NaN for -inf), times the gate
      const float ltot = group4_sum(lsum);
      const bool dead = mrun == -INFINITY;
      const float inv = dead ? 0.f : 1.0f / ltot;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float o = ot[cb][r] * inv;
          if (dead) {
            const int ch = 16 * cb + 4 * g + r;
            float vsum = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) vsum += vpart[w][ch];
            o = a.fill == -INFINITY ? NAN : vsum / (float)N;
          }
          ot[cb][r] = o * gt[cb][r];
        }
      // this head's share of the output projection: y^T += Wo[:, t] (g*o)_t^T
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        bf16x4 gob;
        if constexpr (BF)
          gob = __builtin_bit_cast(bf16x4, make_uint2(pack_bf16x2(ot[cb][0], ot[cb][1]),
                                                      pack_bf16x2(ot[cb][2], ot[cb][3])));
#pragma unroll
        for (int o = 0; o < OB; ++o) {
          const char *wp = reinterpret_cast<const char *>(Wo) +
                           ((size_t)(16 * o + r16) * D + t * DH + 16 * cb + 4 * g) * ES;
          if constexpr (BF) {
            yacc[m][o] = mfma(__builtin_bit_cast(bf16x4, ldg<uint2>(wp)), gob, yacc[m][o]);
          } else {
            const float4 w = ldg<float4>(wp);
            yacc[m][o] = mfma(w.x, ot[cb][0], yacc[m][o]);
            yacc[m][o] = mfma(w.y, ot[cb][1], yacc[m][o]);
            yacc[m][o] = mfma(w.z, ot[cb][2], yacc[m][o]);
            yacc[m][o] = mfma(w.w, ot[cb][3], yacc[m][o]);
          }
          if ((o & 3) == 3) sched_fence();
        }
      }
    }
    __syncthreads();  // every wave is done with this head's k, v and sums
  }

  // y = Wo (g*o) + bo; lane: channels 16 o + 4g + r of position r16
#pragma unroll
  for (int m = 0; m < MAXB; ++m) {
    const int j = (wave + NW * m) * 16 + r16;
    if (j >= N) continue;
    char *dst = static_cast<char *>(a.out) + pos_at(j) * D * ES;
#pragma unroll
    for (int o = 0; o < OB; ++o) {
      float y[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) y[r] = yacc[m][o][r] + ld_elem<T>(bo, 16 * o + 4 * g + r);
      if constexpr (BF)
        stg<uint2>(dst + (16 * o + 4 * g) * 2, make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])));
      else
        stg<float4>(dst + (16 * o + 4 * g) * 4, make_float4(y[0], y[1], y[2], y[3]));
    }
  }
}

template <typename T, int D, int DH>
static hipError_t launch_op_t(const OnePassArgs &a, hipStream_t s) {
  const long long P = (long long)a.B * a.N * a.N;
  hipLaunchKernelGGL((op_bias<T, D>), dim3((unsigned)((P + 15) / 16)), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((op_fused<T, D, DH>), dim3((unsigned)(a.B * a.N)), dim3(512), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_onepass(int dtype, int D, int dh, const OnePassArgs &a, hipStream_t s) {
  static_assert(OpShape<float, 128, 32>::NPMAX == kOnePassMaxN, "row limit");
  if (a.N <= 0 || a.N > kOnePassMaxN || a.Np > kOnePassMaxN || a.Np % 64 || a.Np < a.N || a.B <= 0)
    return hipErrorInvalidValue;
  if ((long long)a.B * a.N > 0x7FFFFFFF || ((long long)a.B * a.N * a.N + 15) / 16 > 0x7FFFFFFF)
    return hipErrorInvalidValue;
  if (dtype == TRI_ATTN_BF16) {
    if (D == 128 && dh == 16) return launch_op_t<bf16_t, 128, 16>(a, s);
    if (D == 128 && dh == 32) return launch_op_t<bf16_t, 128, 32>(a, s);
    if (D == 64 && dh == 16) return launch_op_t<bf16_t, 64, 16>(a, s);
    if (D == 64 && dh == 32) return launch_op_t<bf16_t, 64, 32>(a, s);
  } else {
    if (D == 128 && dh == 16) return launch_op_t<float, 128, 16>(a, s);
    if (D == 128 && dh == 32) return launch_op_t<float, 128, 32>(a, s);
    if (D == 64 && dh == 16) return launch_op_t<float, 64, 16>(a, s);
    if (D == 64 && dh == 32) return launch_op_t<float, 64, 32>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tpa

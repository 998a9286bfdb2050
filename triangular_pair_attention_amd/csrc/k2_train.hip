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
// Work item = (b, i, head t, 256 query columns); 8 waves, each owning two
// 16-column query blocks. Keys go through LDS in chunks of 64 (k as
// [key][c], v transposed as [c][key]), double-buffered: the next chunk's
// loads are in flight while the current one is computed. The scores are
// built transposed on the matrix cores, S^T = k q^T, so each lane holds four
// consecutive keys of one query column: exactly the four words of one
// generator call, and exactly the k-slice of the P^T operand of
// o^T = v^T P^T. The softmax keeps a running maximum per column (one
// reduction over the four lane groups per chunk), which also gives the
// log-sum-exp. bf16 uses 16x16x16 bf16 products, float32 16x16x4 float32
// products (channel or key 4g + e of each 16-slice in step e, for both
// operands).
#include "device_common.h"
#include "tri_attn.h"
#include "tri_attn_internal.h"

#include <type_traits>

namespace tpa {

template <typename T, int DH>
struct K2TShape {
  static constexpr bool BF = is_bf16<T>::value;
  static constexpr int NW = 8, QPW = 2;       // waves; 16-column query blocks per wave
  static constexpr int QB = NW * QPW * 16;    // query columns per work item
  static constexpr int KT = 64;               // keys per chunk
  static constexpr int KP = DH + 4;           // k row pitch (elements)
  static constexpr int VP = KT + (BF ? 16 : 8);  // v^T row pitch (elements)
  static constexpr int EPT = KT * DH / (NW * 64);  // k (and v) elements per thread per chunk
  using L = typename std::conditional<BF, uint16_t, float>::type;
};

template <typename T, int DH>
__global__ __launch_bounds__(512) void k2_train(K2Args a, K2TrainArgs tr) {
  using S = K2TShape<T, DH>;
  using L = typename S::L;
  constexpr bool BF = S::BF;
  constexpr bool KSPLIT = !BF && DH == 32;  // k stored as three bf16 parts (kernel 1)
  constexpr int NW = S::NW, QPW = S::QPW, QB = S::QB, KT = S::KT, KP = S::KP, VP = S::VP, EPT = S::EPT;
  constexpr int CB = DH / 16;
  static_assert(EPT >= 1 && KT * DH == EPT * NW * 64, "staging split");
  __shared__ __align__(16) L kbuf[2][KT * KP];
  __shared__ __align__(16) L vtb[2][DH * VP];

  const int N = a.N, Np = a.Np, nch = a.nchunk;
  const int H = tr.h, NB = H * CB;
  const int nq = (N + QB - 1) / QB;
  int blk = blockIdx.x;
  const int qc = blk % nq;
  blk /= nq;
  const int t = blk % H;
  const int row = blk / H;  // b * N + i
  const int b = row / N;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;

  // ---- staging of one key chunk: thread tid holds elements tid + 512 e of
  // the chunk's k (key-major) and v^T (channel-major), zeros past N
  const size_t vbase = ((size_t)row * H + t) * DH * Np;  // v^T [b][i][t][u][k]
  auto load_chunk = [&](int c, float (&kr)[EPT], float (&vr)[EPT]) {
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int idx = tid + NW * 64 * e;
      {
        const int kk = idx / DH, u = idx - kk * DH, k = c * KT + kk;
        float kv = 0.f;
        if (k < N) {
          if constexpr (KSPLIT) {
            const uint16_t *kp = reinterpret_cast<const uint16_t *>(a.k) + ((size_t)row * H + t) * 3 * Np * 32 +
                                 (size_t)(k >> 4) * 512 + (k & 15) * 8 + (size_t)(u >> 3) * 128 + (u & 7);
            kv = bf2f(kp[0]) + bf2f(kp[(size_t)Np * 32]) + bf2f(kp[(size_t)Np * 64]);
          } else {
            kv = ld_elem<T>(a.k, (((size_t)row * NB + t * CB + u / 16) * Np + k) * 16 + u % 16);
          }
        }
        kr[e] = kv;
      }
      {
        const int u = idx / KT, kk = idx - u * KT, k = c * KT + kk;
        vr[e] = k < N ? ld_elem<T>(a.vt, vbase + (size_t)u * Np + k) : 0.f;
      }
    }
  };
  auto store_chunk = [&](int buf, const float (&kr)[EPT], const float (&vr)[EPT]) {
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int idx = tid + NW * 64 * e;
      const int kk = idx / DH, u = idx - kk * DH;
      const int vu = idx / KT, vk = idx - vu * KT;
      if constexpr (BF) {
        kbuf[buf][kk * KP + u] = f2bf(kr[e]);  // exact: the values are bf16
        vtb[buf][vu * VP + vk] = f2bf(vr[e]);
      } else {
        kbuf[buf][kk * KP + u] = kr[e];
        vtb[buf][vu * VP + vk] = vr[e];
      }
    }
  };

  // ---- the wave's query columns: q^T operands, dead-column flags
  const float *zrow_base = a.zm + (size_t)(b * H + t) * N * Np;
  int jq[QPW];
  bool dead[QPW];
  f32x4 qf[QPW][CB];  // lane: channels 16 cb + 4g + r of column jq
#pragma unroll
  for (int m = 0; m < QPW; ++m) {
    const int j = qc * QB + (wave * QPW + m) * 16 + r16;
    jq[m] = j;
    const int jc = min(j, N - 1);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const size_t qi = (((size_t)row * NB + t * CB + cb) * Np + jc) * 16 + 4 * g;
      if constexpr (BF) {
        const uint2 u = ldg<uint2>(reinterpret_cast<const uint16_t *>(a.q) + qi);
        qf[m][cb] = (f32x4){bflo(u.x), bfhi(u.x), bflo(u.y), bfhi(u.y)};
      } else {
        const float4 f = ldg<float4>(reinterpret_cast<const float *>(a.q) + qi);
        qf[m][cb] = (f32x4){f.x, f.y, f.z, f.w};
      }
    }
    bool d = true;
    for (int c = 0; c < nch; ++c) d = d && a.zmax[((size_t)(b * H + t) * nch + c) * N + jc] == -INFINITY;
    dead[m] = d;
  }
  bf16x4 qb[QPW][CB];
  if constexpr (BF) {
#pragma unroll
    for (int m = 0; m < QPW; ++m)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
        qb[m][cb] = __builtin_bit_cast(bf16x4, make_uint2(pack_bf16x2(qf[m][cb][0], qf[m][cb][1]),
                                                          pack_bf16x2(qf[m][cb][2], qf[m][cb][3])));
  }

  float mrun[QPW], lsum[QPW];
  f32x4 ot[QPW][CB];  // o^T: lane holds channels 16 cb + 4g + r of column jq
#pragma unroll
  for (int m = 0; m < QPW; ++m) {
    mrun[m] = -INFINITY;
    lsum[m] = 0.f;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) ot[m][cb] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }
  const uint32_t ctr2 = (uint32_t)(row * H + t);

  float kr[EPT], vr[EPT];
  load_chunk(0, kr, vr);
  store_chunk(0, kr, vr);
  __syncthreads();
#pragma unroll 1
  for (int c = 0; c < nch; ++c) {
    const int buf = c & 1;
    const bool more = c + 1 < nch;
    if (more) load_chunk(c + 1, kr, vr);  // in flight during this chunk
    const L *kb_ = kbuf[buf];
    const L *vb_ = vtb[buf];
    const int k0 = c * KT;
    // the chunk's dropout words, all calls first: independent chains the
    // scheduler can interleave (one call's rounds are a serial chain)
    uint4 wd[QPW][4];
#pragma unroll
    for (int m = 0; m < QPW; ++m)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        wd[m][kb] = philox4x32_10(make_uint4((uint32_t)((k0 >> 2) + kb * 4 + g), (uint32_t)jq[m], ctr2, tr.offset),
                                  tr.seed_lo, tr.seed_hi);
#pragma unroll
    for (int m = 0; m < QPW; ++m) {
      const int jc = min(jq[m], N - 1);
      const float *zq = zrow_base + (size_t)jc * Np + k0;
      f32x4 st[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const float4 z4 = ldg<float4>(zq + kb * 16 + 4 * g);  // lane: keys 4g + r, column jq
        st[kb] = (f32x4){z4.x, z4.y, z4.z, z4.w};
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const L *kp = &kb_[(kb * 16 + r16) * KP + 16 * cb + 4 * g];
          if constexpr (BF) {
            st[kb] = mfma(__builtin_bit_cast(bf16x4, *reinterpret_cast<const uint2 *>(kp)), qb[m][cb], st[kb]);
          } else {
            const float4 kv = *reinterpret_cast<const float4 *>(kp);
            st[kb] = mfma(kv.x, qf[m][cb][0], st[kb]);
            st[kb] = mfma(kv.y, qf[m][cb][1], st[kb]);
            st[kb] = mfma(kv.z, qf[m][cb][2], st[kb]);
            st[kb] = mfma(kv.w, qf[m][cb][3], st[kb]);
          }
        }
        if (dead[m]) {
          // no valid key: every one of the N keys has the same score (the
          // fill); 0 in place of it, past N still -inf
#pragma unroll
          for (int r = 0; r < 4; ++r) st[kb][r] = (k0 + kb * 16 + 4 * g + r < N) ? 0.f : -INFINITY;
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, st[kb][r]);
      mx = group4_max(mx);
      // every lane stays in the step (the value products take their v^T rows
      // from all lanes): no live key yet shifts by 0 and adds zeros
      const float mnew = fmaxf(mrun[m], mx);
      const float msh = mnew == -INFINITY ? 0.f : mnew;
      const float alpha = fast_exp2(mrun[m] - msh);
      mrun[m] = mnew;
      lsum[m] *= alpha;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) ot[m][cb] *= alpha;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const uint4 w = wd[m][kb];
        const uint32_t wv[4] = {w.x, w.y, w.z, w.w};  // keys k0 + 16 kb + 4g + r
        float p[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = fast_exp2(st[kb][r] - msh);
          lsum[m] += e;
          p[r] = wv[r] >= tr.thr ? e : 0.f;
        }
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const L *vp = &vb_[(16 * cb + r16) * VP + kb * 16 + 4 * g];
          if constexpr (BF) {
            const bf16x4 pb = __builtin_bit_cast(bf16x4, make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])));
            ot[m][cb] = mfma(__builtin_bit_cast(bf16x4, *reinterpret_cast<const uint2 *>(vp)), pb, ot[m][cb]);
          } else {
            const float4 vv = *reinterpret_cast<const float4 *>(vp);
            ot[m][cb] = mfma(vv.x, p[0], ot[m][cb]);
            ot[m][cb] = mfma(vv.y, p[1], ot[m][cb]);
            ot[m][cb] = mfma(vv.z, p[2], ot[m][cb]);
            ot[m][cb] = mfma(vv.w, p[3], ot[m][cb]);
          }
        }
      }
    }
    if (more) store_chunk(buf ^ 1, kr, vr);  // the other buffer: last read before the previous barrier
    __syncthreads();
  }

  // ---- normalise, log-sum-exp, gate
#pragma unroll
  for (int m = 0; m < QPW; ++m) {
    const int j = jq[m];
    const float lt = group4_sum(lsum[m]);
    float inv, lse;
    if (dead[m]) {
      if (a.mask_fill == -INFINITY) {
        inv = NAN;
        lse = NAN;
      } else {
        inv = tr.scale / (float)N;
        lse = a.mask_fill + logf((float)N);
      }
    } else {
      inv = tr.scale / lt;
      lse = (mrun[m] + log2f(lt)) * 0.69314718055994531f;
    }
    if (j >= N) continue;
    if (tr.lse && g == 0) tr.lse[((size_t)row * H + t) * N + j] = lse;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const size_t gi = (((size_t)row * NB + t * CB + cb) * Np + j) * 16 + 4 * g;
      if constexpr (BF) {
        uint16_t *gp = reinterpret_cast<uint16_t *>(a.g) + gi;
        const uint2 gv = *reinterpret_cast<const uint2 *>(gp);
        const float o0 = bflo(gv.x) * (ot[m][cb][0] * inv), o1 = bfhi(gv.x) * (ot[m][cb][1] * inv);
        const float o2 = bflo(gv.y) * (ot[m][cb][2] * inv), o3 = bfhi(gv.y) * (ot[m][cb][3] * inv);
        *reinterpret_cast<uint2 *>(gp) = make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
      } else {
        float *gp = reinterpret_cast<float *>(a.g) + gi;
        const float4 gv = *reinterpret_cast<const float4 *>(gp);
        *reinterpret_cast<float4 *>(gp) = make_float4(gv.x * (ot[m][cb][0] * inv), gv.y * (ot[m][cb][1] * inv),
                                                      gv.z * (ot[m][cb][2] * inv), gv.w * (ot[m][cb][3] * inv));
      }
    }
  }
}

template <typename T, int DH>
static hipError_t launch_t(const K2Args &a, const K2TrainArgs &tr, hipStream_t s) {
  constexpr int QB = K2TShape<T, DH>::QB;
  const long long blocks = (long long)a.B * a.N * tr.h * ((a.N + QB - 1) / QB);
  if (blocks <= 0 || blocks > 0x7FFFFFFF || a.Np % K2TShape<T, DH>::KT) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k2_train<T, DH>), dim3((unsigned)blocks), dim3(512), 0, s, a, tr);
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

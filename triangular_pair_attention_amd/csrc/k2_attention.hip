// Kernel 2 of the triangular self-attention forward: for one head, rows i of
// a row block attend over the key columns k of their own row, query columns j
// of a query block, with the shared pair bias and mask; softmax over k; the
// value sum; the gate multiply (Kimi-K2.6 / l2_p6 transcript: the score,
// softmax, value and gate steps of its forward listing and its attention
// kernel; FW-GLM-5-1 / l2_p6: the fused attention kernel). The output
// projection is kernel 3.
//
// Work item = (b, head t, RB rows i, QB query columns j); wave (wr, wq) takes
// IG rows x JW*16 queries. The (B, N, h, N, N) scores are never stored.
// Workgroups are persistent (as many as are resident) and loop over items:
// after an item's key loop, the next item's setup loads, query fragments and
// first key steps go out together with this item's gate, and the next item's
// setup runs while they arrive, followed by this item's epilogue, so the CU
// is not left idle on the round trips at the start and end of an item.
//
// Key tiles through LDS. Per key step (KT keys) the workgroup needs k and v
// of its RB rows and the bias+mask tile zm of its QB query columns. Every
// piece is a 1 KB block laid out exactly as the consuming lanes read their
// MFMA fragments (lane l's 16 bytes at 16*l), filled by direct global->LDS
// loads (each loader lane supplies its own global address). A three-stage
// ring keeps two steps in flight, with one LDS barrier per step. Each k/v
// block is read by all WQ waves of its rows and each zm block by all WR waves
// of its columns, so the L2 traffic per score is shared WQ (WR) ways.
//
// Softmax without a running maximum. Per (row i, query j) the kernel fixes
// the shift m = |q'_j| * max_k |k_k| + max_k zm[j, k] - H before the key
// loop. Cauchy-Schwarz makes m + H >= every score of the row, so exp2(s - m)
// <= 2^H; with the headroom H = 96 nothing overflows (a column sum stays
// below N * 2^96) while a bound up to 64 + 96 above the column's true maximum
// still leaves its sum above 2^-64 (peaked inputs, with large query norms and
// bias, make the Cauchy-Schwarz bound loose by much more than 64). Softmax is
// invariant to the shift, so the result is exact up to rounding; the loop
// needs no max, no rescaling and no cross-lane traffic. For bf16 the shift rides in the MFMA (d = 16: a spare contraction
// slot holds q' = -m against k = 1; d = 32: one more MFMA), the score
// accumulator starts from the zm tile and the row sum comes from a row of
// ones in the PV MFMA: the VALU work per score is one exp2 and half a bf16
// conversion. If a column's sum falls below 2^-64 (only with a pathological
// bound, or the shift_slack test knob) the workgroup recomputes that item
// with the exact maximum (a max pass, then the loop again).
//
// Mask: zm = -inf where masked, so masked keys get weight exactly 0. A query
// column whose keys are all masked (max zm = -inf) gets the rule of the
// finite fill value: uniform weights over all N keys, i.e. the mean of v
// (from kernel 1's per-chunk sums of v); or NaN when the fill is -inf. Key
// chunks of 64 beyond the last live chunk of the workgroup's columns are
// skipped.
//
// Float32: the scores of head size 32 are six bf16 products of three-way
// split operands (float32 accuracy at fewer matrix-core cycles); the
// probability-value products are float32 MFMAs.
//
// Output: o / l times the gate, written over the gate in the workspace
// ([b][i][c/16][j][16]); kernel 3 reads it from there.
#include "device_common.h"
#include "tri_attn_internal.h"

#include <type_traits>

#include "tri_attn.h"

namespace tpa {

// Headroom of the softmax shift below its Cauchy-Schwarz bound (log2 units):
// exp2 of a score is at most 2^96, so column sums (N keys) and the value sums
// stay far inside the float32 range.
constexpr float kShiftHeadroom = 96.f;

// IG rows x JW 16-query blocks per wave; WR x WQ waves per workgroup.
template <typename T, int D, int DH>
struct K2Shape {
  static constexpr bool BF = is_bf16<T>::value;
  // fp32 runs at sizes where one workgroup per CU would leave the CUs idle
  // on latency: one row per wave and small blocks, so two fit on a CU.
  // bf16, d = 32: one row per wave and four query blocks, so a row's k and v
  // serve 128 query columns (the feed per score is what limits this shape).
  static constexpr int IG = BF ? ((DH == 16) ? 4 : 1) : 1;
  static constexpr int JW = BF ? ((DH == 16) ? 2 : 4) : ((DH == 16) ? 1 : 2);
  static constexpr int WR = (BF && DH == 32) ? 4 : 2;
  static constexpr int WQ = BF ? ((DH == 16) ? 4 : 2) : 2;
  static constexpr int NW = WR * WQ;
  static constexpr int RB = WR * IG;       // rows per workgroup
  static constexpr int QB = WQ * JW * 16;  // query columns per workgroup
  // k blocks per row and key step (float32, d = 32: the three bf16 parts)
  static constexpr int KBR = (DH == 16) ? 1 : (BF ? 2 : 3);
  static constexpr int VBR = DH / 16;             // v blocks per row and key step
  static constexpr int ZBJ = BF ? 2 : 1;          // zm blocks per 16 queries and key step
  static constexpr int NBLK = RB * (KBR + VBR) + (QB / 16) * ZBJ;
  static constexpr int LPW = (NBLK + NW - 1) / NW;  // loads per wave per step
  static constexpr int NBLKP = LPW * NW;            // blocks per stage (the last ones pad)
  // ring stages: NS - 1 key steps in flight (a fourth stage measured no faster)
  static constexpr int NS = 3;
  // k blocks come first in a stage. bf16, d = 16: each k block has a third
  // half-KB of constants (the unit key slot of the lanes that carry no
  // channels), so that every lane reads its fragment from a fixed offset.
  static constexpr int NK = RB * KBR;
  static constexpr int KSTR = (BF && DH == 16) ? 1536 : 1024;
  static constexpr int STAGE = NK * KSTR + (NBLKP - NK) * 1024;  // bytes
  static constexpr size_t LDS = (size_t)NS * STAGE;
};

template <typename T, int D, int DH>
__global__ __launch_bounds__((K2Shape<T, D, DH>::NW * 64)) void k2_attention(K2Args a) {
  using S = K2Shape<T, D, DH>;
  constexpr bool BF = is_bf16<T>::value;
  constexpr int ES = BF ? 2 : 4;
  constexpr int H = D / DH;
  constexpr int NB = D / 16;
  constexpr int MB = DH / 16;  // 16-row blocks of one head's channels
  constexpr int IG = S::IG, JW = S::JW, WQ = S::WQ, NW = S::NW, RB = S::RB, QB = S::QB;
  constexpr int KT = BF ? 32 : 16;  // keys per step
  constexpr int KBR = S::KBR, VBR = S::VBR, ZBJ = S::ZBJ, NBLK = S::NBLK, LPW = S::LPW, NBLKP = S::NBLKP;
  constexpr int NS = S::NS, NK = S::NK, KSTR = S::KSTR, STAGE = S::STAGE;
  constexpr int QS = DH / 4;  // fp32: q/k elements per lane
  using Frag = typename std::conditional<BF, bf16x8, float>::type;
  static_assert(S::LDS <= 150 * 1024, "stage ring exceeds LDS");

  __shared__ __align__(16) uint4 ring[NS * STAGE / 16];  // NS stages of STAGE bytes
  static_assert(S::LDS + RB * DH * 4 <= 150 * 1024, "LDS budget");

  // lane, g and r16 are re-declared opaque to the compiler after every item's
  // key loop (see below), so address arithmetic of the next item is not
  // hoisted out of the item loop and kept live across the key loop
  int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int g = lane >> 4, r16 = lane & 15;
  const int wr = wave / WQ, wq = wave - wr * WQ;
  const int N = a.N, Np = a.Np, nch = a.nchunk;

  // ---- persistent workgroups. Virtual workgroup v (this workgroup's index,
  // then + G, + 2G, ...) maps to a work item XCD-aware: v runs on XCD v % 8
  // (G is a multiple of 8); each XCD takes a contiguous range of the linear
  // order below, in which consecutive items of one (b, t) form super-tiles of
  // SI row blocks x SJ query blocks, so the concurrently running workgroups
  // of an XCD share k/v (same rows) and zm (same query columns) through its L2.
  const int nRB = (N + RB - 1) / RB, nQB = (N + QB - 1) / QB;
  const int per_bt = nRB * nQB;
  const int G8 = gridDim.x;
  struct Item {
    int b, t, i0, j0;
  };
  auto coords = [&](int v) {
    int lin = v;
    const int w8 = (a.items / 8) * 8;
    if (lin < w8) lin = (lin & 7) * (w8 / 8) + (lin >> 3);
    const int bt = lin / per_bt;
    Item it;
    it.b = bt / H;
    it.t = bt - it.b * H;
    const int SJ = nQB < 8 ? nQB : 8;
    const int SI = 32 / SJ;
    const int rem = lin - bt * per_bt;
    const int igs = (rem / (SI * nQB)) * SI;
    const int si = min(SI, nRB - igs);
    const int r2 = rem - igs * nQB;
    const int jrs = (r2 / (si * SJ)) * SJ;
    const int sj = min(SJ, nQB - jrs);
    const int r3 = r2 - jrs * si;
    it.i0 = (igs + r3 / sj) * RB;
    it.j0 = (jrs + r3 % sj) * QB;
    return it;
  };

  const T *Q = reinterpret_cast<const T *>(a.q);
  const T *K = reinterpret_cast<const T *>(a.k);
  const T *VT = reinterpret_cast<const T *>(a.vt);
  T *G = reinterpret_cast<T *>(a.g);

  // ---- the item in flight: coordinates and everything derived from them
  int b = 0, t = 0, i0 = 0, j0 = 0;
  const float *ZM = a.zm;
  int rows[IG];
  auto set_item = [&](const Item &it) {
    b = it.b, t = it.t, i0 = it.i0, j0 = it.j0;
    ZM = a.zm + (size_t)(b * H + t) * N * Np;
#pragma unroll
    for (int i = 0; i < IG; ++i) rows[i] = min(i0 + wr * IG + i, N - 1);
  };

  // query fragments
  // bf16: lane (g, r16) holds q'[j = r16][8g..8g+7] (d = 16: groups 0-1 real, group 2 slot 0 = -m);
  // fp32: lane (g, r16) holds q'[j][g*d/4 .. +d/4).
  Frag qf[IG][JW][BF ? 1 : QS];
  // fp32, d = 32: the scores run as six bf16 products of three-way split
  // operands (float32 accuracy; kernel 1's split products): each lane
  // already holds channels 8g..8g+7 of one query and of one key, the bf16
  // 16x16x32 fragment layout. The queries are split once per item (below,
  // in setup); kernel 1 stores the keys already split.
  constexpr bool SPLITQK = !BF && DH == 32;
  bf16x8 qsp[IG][JW][SPLITQK ? 3 : 1];
  auto load_q = [&]() {
#pragma unroll
    for (int i = 0; i < IG; ++i)
#pragma unroll
      for (int jb = 0; jb < JW; ++jb) {
        const int j = min(j0 + (wq * JW + jb) * 16 + r16, Np - 1);
        const size_t rowbase = (size_t)(b * N + rows[i]) * NB;
        const int cb = (DH == 16) ? t : 2 * t + (g >> 1);
        if constexpr (BF) {
          uint4 raw = ldg<uint4>(Q + ((rowbase + cb) * Np + j) * 16 + 8 * (g & 1));
          if (DH == 16 && g >= 2) raw = make_uint4(0, 0, 0, 0);
          qf[i][jb][0] = as_bf16x8(raw);
        } else {
          const int off = (DH == 16) ? 4 * g : 8 * (g & 1);
          const float *src = reinterpret_cast<const float *>(Q) + ((rowbase + cb) * Np + j) * 16 + off;
#pragma unroll
          for (int s = 0; s < QS; s += 4) {
            const float4 v = ldg<float4>(src + s);
            qf[i][jb][s] = v.x, qf[i][jb][s + 1] = v.y, qf[i][jb][s + 2] = v.z, qf[i][jb][s + 3] = v.w;
          }
        }
      }
  };

  // the gate of this wave's outputs (addresses clamped into the tensor; values
  // of rows or columns past N are not used)
  using GVec = typename std::conditional<BF, uint2, float4>::type;
  GVec gate[IG][JW][MB];
  auto load_gate = [&]() {
#pragma unroll
    for (int i = 0; i < IG; ++i)
#pragma unroll
      for (int jb = 0; jb < JW; ++jb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int jc = min(j0 + (wq * JW + jb) * 16 + r16, N - 1);
          gate[i][jb][mb] = ldg<GVec>(G + (((size_t)(b * N + rows[i]) * NB + t * MB + mb) * Np + jc) * 16 + 4 * g);
        }
  };

  // ---- loader: this wave fills blocks wave + NW*l of each stage; each lane
  // keeps the byte address of its 16 bytes at key step 0 and the per-step stride.
  const char *src_ptr[LPW];
  int src_step[LPW];
  auto set_loader = [&]() {
#pragma unroll
    for (int l = 0; l < LPW; ++l) {
      int blk = wave + NW * l;
      if (blk >= NBLK) blk = 0;  // padding block: a harmless duplicate of block 0
      const char *p;
      int step;
      if (blk < RB * KBR) {
        const int r = blk / KBR, kp = blk - r * KBR;
        const int row = min(i0 + r, N - 1);
        const size_t rowbase = (size_t)(b * N + row) * NB;
        if constexpr (BF) {
          if (DH == 16) {
            // lanes 0-31: key tile A (keys 8(rho/4)+rho%4), lanes 32-63: tile B (+4); 16 channels in two halves
            const int half = lane >> 5, gg = (lane >> 4) & 1, rho = lane & 15;
            const int key = 4 * half + 8 * (rho >> 2) + (rho & 3);
            p = reinterpret_cast<const char *>(K + ((rowbase + t) * Np + key) * 16 + 8 * gg);
          } else {
            const int key = 4 * kp + 8 * (r16 >> 2) + (r16 & 3);
            p = reinterpret_cast<const char *>(K + ((rowbase + 2 * t + (g >> 1)) * Np + key) * 16 + 8 * (g & 1));
          }
        } else {
          if (DH == 16)
            p = reinterpret_cast<const char *>(K + ((rowbase + t) * Np + r16) * 16 + 4 * g);
          else  // part kp of k, as kernel 1 stores it: 1 KB per 16 keys in fragment order
            p = reinterpret_cast<const char *>(K) + ((((size_t)(b * N + row) * H + t) * 3 + kp) * (Np / 16)) * 1024 +
                lane * 16;
        }
        step = KT * 16 * ES;
      } else if (blk < RB * (KBR + VBR)) {
        const int v = blk - RB * KBR;
        const int r = v / VBR, mb = v - r * VBR;
        const int row = min(i0 + r, N - 1);
        p = reinterpret_cast<const char *>(VT + (((size_t)(b * N + row) * H + t) * DH + mb * 16 + r16) * Np +
                                           (BF ? 8 : 4) * g);
        step = KT * ES;
      } else {
        const int z = blk - RB * (KBR + VBR);
        const int jb = z / ZBJ, zp = z - jb * ZBJ;
        const int jrow = min(j0 + jb * 16 + r16, N - 1);
        p = reinterpret_cast<const char *>(ZM + (size_t)jrow * Np + (BF ? 8 : 4) * g + 4 * zp);
        step = KT * 4;
      }
      src_ptr[l] = p;
      src_step[l] = step;
    }
  };
  const uint32_t ring_base = lds_addr(ring);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  uint32_t blk_lds[LPW];  // byte offset of this wave's block l within a stage
#pragma unroll
  for (int l = 0; l < LPW; ++l) {
    const int blk = wave_u + NW * l;
    blk_lds[l] = __builtin_amdgcn_readfirstlane(blk < NK ? blk * KSTR : NK * KSTR + (blk - NK) * 1024);
  }
  auto issue = [&](int s) {  // global -> LDS: key step s into stage s % NS
    const uint32_t stage = ring_base + (uint32_t)((s % NS) * STAGE);
#pragma unroll
    for (int l = 0; l < LPW; ++l) dma16_to_lds(src_ptr[l] + (size_t)s * src_step[l], stage + blk_lds[l]);
  };
  // An item's first LA key steps go out before its setup is done: every key
  // step below Np / KT (>= LA) addresses padded, in-bounds rows, so they are
  // issued before the number of live steps is known; steps past that number
  // are waited for and ignored.
  constexpr int LA = NS - 1;  // steps in flight
  static_assert(LA >= 1 && LA <= 3, "");

  // ---- setup loads. The per-chunk maxima and sums are spread over the
  // lanes and reduced across lanes; the first round of every one of these
  // loads is issued before any of them is used (one round trip); rows longer
  // than that first round (more than 64 / IG key chunks for |k|, 16 for the
  // bias, 8 for the v sums) continue in loops.
  // |k|^2 <= sum over the head's 16-channel blocks of each block's chunk
  // maxima: the wave's lanes form IG groups of KL, group kr takes the wave's
  // row kr, its lanes chunks kc, kc + KL, ...
  // Bias+mask maximum and last live key chunk of this wave's query columns:
  // lane (g, r16) takes chunks g, g + 4, ... of column r16.
  // Sum of v over all keys of each (row, channel) of the workgroup, from
  // kernel 1's per-chunk sums (the uniform weights of a fully masked column,
  // finite fill): VQ adjacent threads per (row, channel), each taking VS of
  // its eight partial-sum slots. bf16 with d = 16 spreads them over every
  // thread of the workgroup (measured faster at B = 4, N = 512, h = 8); the
  // other shapes keep one thread per (row, channel) (measured faster there).
  constexpr int ZR = 4;
  constexpr int KL = 64 / IG;
  static_assert(64 % IG == 0, "");
  constexpr int VQ = (BF && DH == 16) ? (NW * 64) / (RB * DH) : 1;
  static_assert(VQ * RB * DH <= NW * 64 && (VQ == 1 || VQ == 2 || VQ == 4 || VQ == 8), "v-sum threads");
  constexpr int VS = 8 / VQ;
  const bool vthread = VQ * RB * DH == NW * 64 || threadIdx.x < VQ * RB * DH;
  float kmx[MB], zfirst[JW][ZR], sv[VS];
  auto kmax_row = [&](int mb) {  // this lane's row of the |k| chunk maxima, block mb of head t
    const int kr = lane / KL;
    const int row = min(i0 + wr * IG + kr, N - 1);
    return a.kmax + ((size_t)(b * N + row) * NB + t * MB + mb) * nch;
  };
  auto vsum_row = [&]() {  // this thread's (row, channel) of the per-chunk v sums
    const int rc = threadIdx.x / VQ, r = rc / DH, ch = rc - r * DH;
    // [b][i][chunk][channel]
    return a.vsum + (size_t)(b * N + min(i0 + r, N - 1)) * nch * D + t * DH + ch;
  };
  auto load_setup = [&]() {
    {
      const int kc = lane % KL;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) kmx[mb] = kc < nch ? kmax_row(mb)[kc] : 0.f;
    }
#pragma unroll
    for (int jb = 0; jb < JW; ++jb) {
      const int j = j0 + (wq * JW + jb) * 16 + r16;
      // [b][t][chunk][j]: the 16 lanes of a lane group read 16 consecutive columns
      const float *zp = a.zmax + (size_t)(b * H + t) * nch * N + min(j, N - 1);
#pragma unroll
      for (int u = 0; u < ZR; ++u) zfirst[jb][u] = (j < N && g + 4 * u < nch) ? zp[(size_t)(g + 4 * u) * N] : -INFINITY;
    }
    if (vthread) {
      const float *p = vsum_row();
      const int q = threadIdx.x % VQ;
#pragma unroll
      for (int k = 0; k < VS; ++k) sv[k] = q * VS + k < nch ? p[(size_t)(q * VS + k) * D] : 0.f;
    }
  };

  // ---- setup: per-item LDS state is double-buffered by item parity, so the
  // next item's setup can run before the current item's epilogue
  __shared__ __align__(16) float vsum_s[2][RB * DH];
  __shared__ int kend_s[NW];
  __shared__ int need_s[2];
  float kn2[IG], zmx[JW];
  bool colmask[JW];  // a real column whose keys are all masked
  float msh[IG][JW];
  int nsteps = 0;
  bool shift_on = true;
  auto set_shift = [&](const float (&m)[IG][JW]) {
    if constexpr (BF) {
#pragma unroll
      for (int i = 0; i < IG; ++i)
#pragma unroll
        for (int jb = 0; jb < JW; ++jb) {
          const __bf16 nm = (__bf16)(-m[i][jb]);
          const __bf16 z = (__bf16)0.f;
          if (DH == 16 && g == 2) qf[i][jb][0] = bf16x8{nm, z, z, z, z, z, z, z};
        }
    }
  };
  auto setup = [&](int buf) {
    if (vthread) {
      // slot u of a (row, channel) sums chunks u, u + 8, ...; the eight slots
      // are added in one fixed tree, ((s0 + s1) + (s2 + s3)) + ((s4 + s5) +
      // (s6 + s7)), its lower levels inside a thread and its upper levels
      // across the VQ lanes: deterministic
      const float *p = vsum_row();
      const int q = threadIdx.x % VQ;
      float sk[VS];
#pragma unroll
      for (int k = 0; k < VS; ++k) sk[k] = sv[k];
      for (int c = 8; c < nch; c += 8) {
#pragma unroll
        for (int k = 0; k < VS; ++k) sk[k] += c + q * VS + k < nch ? p[(size_t)(c + q * VS + k) * D] : 0.f;
      }
#pragma unroll
      for (int w = 1; w < VS; w <<= 1)
#pragma unroll
        for (int k = 0; k < VS; k += 2 * w) sk[k] += sk[k + w];
      float part = sk[0];
#pragma unroll
      for (int m = 1; m < VQ; m <<= 1) part += __shfl_xor(part, m, 64);
      if (q == 0) vsum_s[buf][threadIdx.x / VQ] = part;
    }
    {
      const int kc = lane % KL;
      float m2 = 0.f;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const float *kp = kmax_row(mb);
        float m = kmx[mb];
        for (int c = kc + KL; c < nch; c += KL) m = fmaxf(m, kp[c]);
#pragma unroll
        for (int x = 1; x < KL; x <<= 1) m = xor_max(m, x);
        m2 += m;
      }
      // lane group i holds row i's bound
#pragma unroll
      for (int i = 0; i < IG; ++i) kn2[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m2), i * KL));
    }
    int kend = 0;
#pragma unroll
    for (int jb = 0; jb < JW; ++jb) {
      const int j = j0 + (wq * JW + jb) * 16 + r16;
      float zx = -INFINITY;
#pragma unroll
      for (int u = 0; u < ZR; ++u) {
        zx = fmaxf(zx, zfirst[jb][u]);
        if (zfirst[jb][u] > -INFINITY) kend = max(kend, g + 4 * u + 1);
      }
      if (j < N) {
        const float *zp = a.zmax + (size_t)(b * H + t) * nch * N + j;
        for (int c = g + 4 * ZR; c < nch; c += 4) {
          const float v = zp[(size_t)c * N];
          zx = fmaxf(zx, v);
          if (v > -INFINITY) kend = max(kend, c + 1);
        }
      }
      zx = group4_max(zx);
      zmx[jb] = zx;
      colmask[jb] = (j < N) && zx == -INFINITY;
    }
    // the workgroup steps through the keys together: its end is the max over all waves
    for (int m = 1; m < 64; m <<= 1) kend = max(kend, __shfl_xor(kend, m, 64));
    if (lane == 0) kend_s[wave] = kend;
    if (threadIdx.x == 0) need_s[buf] = 0;
    lds_barrier();
    {
      int k = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) k = max(k, kend_s[w]);
      nsteps = __builtin_amdgcn_readfirstlane(k) * kChunk / KT;
    }
    // query norms and the shift
#pragma unroll
    for (int i = 0; i < IG; ++i)
#pragma unroll
      for (int jb = 0; jb < JW; ++jb) {
        float n2 = 0.f;
        if constexpr (BF) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float x = (float)qf[i][jb][0][e];
            n2 += x * x;
          }
        } else {
#pragma unroll
          for (int s = 0; s < QS; ++s) n2 += qf[i][jb][s] * qf[i][jb][s];
        }
        n2 = group4_sum(n2);
        msh[i][jb] = (zmx[jb] == -INFINITY) ? 0.f : sqrtf(n2 * kn2[i]) + zmx[jb] + a.shift_slack - kShiftHeadroom;
      }
    set_shift(msh);
    if constexpr (SPLITQK) {
#pragma unroll
      for (int i = 0; i < IG; ++i)
#pragma unroll
        for (int jb = 0; jb < JW; ++jb) {
          uint32_t p1[4], p2[4], p3[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) split3(qf[i][jb][2 * u], qf[i][jb][2 * u + 1], p1[u], p2[u], p3[u]);
          qsp[i][jb][0] = as_bf16x8(make_uint4(p1[0], p1[1], p1[2], p1[3]));
          qsp[i][jb][1] = as_bf16x8(make_uint4(p2[0], p2[1], p2[2], p2[3]));
          qsp[i][jb][2] = as_bf16x8(make_uint4(p3[0], p3[1], p3[2], p3[3]));
        }
    }
    // bf16, d = 32: the shift costs two more MFMAs per score tile. Where every
    // shift of the wave is at most 0 (bound at most H), exp2 of a score cannot
    // overflow without it (at most 2^H per key) and the wave goes without it;
    // scores far below their bound only risk a tiny sum, which the recovery
    // below catches either way.
    shift_on = true;
    if constexpr (BF && DH == 32) {
      bool big = false;
#pragma unroll
      for (int i = 0; i < IG; ++i)
#pragma unroll
        for (int jb = 0; jb < JW; ++jb) big |= !(msh[i][jb] <= 0.f);
      shift_on = __ballot(big) != 0;
    }
  };

  if constexpr (BF && DH == 16) {
    // the constant half of every k block: lanes 32-47 read (1, 0, ..., 0), lanes 48-63 zeros
    for (int x = threadIdx.x; x < NS * NK * 32; x += NW * 64) {
      const int stg = x / (NK * 32), rem = x - stg * (NK * 32), r = rem >> 5, u = rem & 31;
      ring[(stg * STAGE + r * KSTR + 1024) / 16 + u] = make_uint4(u < 16 ? 0x3f80u : 0u, 0u, 0u, 0u);
    }
  }

  // ---- accumulators
  f32x4 o[IG][JW][MB];
  f32x4 ol[IG][JW];    // bf16: row 0 = sum of p (ones row)
  float lacc[IG][JW];  // fp32: per-lane partial sums
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

  const __bf16 one = (__bf16)1.f, zero = (__bf16)0.f;
  // constant operands: ones row for the sum, unit key slot for the shift
  const bf16x8 ones8 = (r16 == 0) ? bf16x8{one, one, one, one, one, one, one, one}
                                  : bf16x8{zero, zero, zero, zero, zero, zero, zero, zero};
  const bf16x8 kunit0 = (g == 0) ? bf16x8{one, zero, zero, zero, zero, zero, zero, zero}
                                 : bf16x8{zero, zero, zero, zero, zero, zero, zero, zero};

  // One key step from a stage of the ring (max_pass: only the running maxima).
  auto step_compute = [&](const uint4 *st, bool max_pass, float (&mx)[IG][JW]) {
    const uint4 *kblk = st;
    const uint4 *vblk = st + NK * KSTR / 16;
    const uint4 *zblk = vblk + RB * VBR * 64;
    if constexpr (BF) {
      // all fragments of the step first, then the (row, query block) pairs in
      // a software pipeline: the scores of pair n + 1 go to the matrix cores
      // before the exponentials of pair n, so the two overlap.
      constexpr int NP = IG * JW;
      f32x4 zA[JW], zB[JW];
#pragma unroll
      for (int jb = 0; jb < JW; ++jb) {
        const int q = wq * JW + jb;
        zA[jb] = __builtin_bit_cast(f32x4, zblk[(q * ZBJ) * 64 + lane]);
        zB[jb] = __builtin_bit_cast(f32x4, zblk[(q * ZBJ + 1) * 64 + lane]);
      }
      bf16x8 kA[IG], kB[IG], vf[IG][MB];
      auto load_row = [&](int i) {
        const int r = wr * IG + i;
        if (DH == 16) {
          const uint4 *kb = kblk + r * (KSTR / 16);
          kA[i] = as_bf16x8(kb[lane + (lane & 32)]);
          kB[i] = as_bf16x8(kb[32 + lane]);
        } else {
          kA[i] = as_bf16x8(kblk[(2 * r) * 64 + lane]);
          kB[i] = as_bf16x8(kblk[(2 * r + 1) * 64 + lane]);
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) vf[i][mb] = as_bf16x8(vblk[(r * VBR + mb) * 64 + lane]);
      };
      load_row(0);
      f32x4 sA[NP], sB[NP];
      auto scores = [&](int n) {
        const int i = n / JW, jb = n % JW;
        sA[n] = mfma(kA[i], qf[i][jb][0], zA[jb]);
        sB[n] = mfma(kB[i], qf[i][jb][0], zB[jb]);
        // The shift MFMA has the same shape as the score MFMA on purpose: a
        // 16x16x16 MFMA reading, as its accumulator, the result that the
        // 16x16x32 one wrote a few instructions before gave wrong sums on
        // gfx950 (only where the two were closest), so only one opcode ever
        // feeds an accumulator chain here.
        if (DH == 32 && !max_pass && shift_on) {
          // B operand: -m in row 0 of lane group 0 (built here: it is rarely needed)
          const __bf16 nm = (__bf16)(-msh[i][jb]), z = (__bf16)0.f;
          const bf16x8 qsh = (g == 0) ? bf16x8{nm, z, z, z, z, z, z, z} : bf16x8{z, z, z, z, z, z, z, z};
          sA[n] = mfma(kunit0, qsh, sA[n]);
          sB[n] = mfma(kunit0, qsh, sB[n]);
        }
      };
      scores(0);
#pragma unroll
      for (int n = 0; n < NP; ++n) {
        const int i = n / JW, jb = n % JW;
        if (jb == 0 && i + 1 < IG) load_row(i + 1);
        if (n + 1 < NP) scores(n + 1);
        if (max_pass) {
          float m = mx[i][jb];
#pragma unroll
          for (int e = 0; e < 4; ++e) m = fmaxf(m, fmaxf(sA[n][e], sB[n][e]));
          mx[i][jb] = m;
        } else {
          bf16x8 p;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            p[e] = (__bf16)fast_exp2(sA[n][e]);
            p[4 + e] = (__bf16)fast_exp2(sB[n][e]);
          }
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) o[i][jb][mb] = mfma(vf[i][mb], p, o[i][jb][mb]);
          ol[i][jb] = mfma(ones8, p, ol[i][jb]);
        }
      }
    } else {
      f32x4 zA[JW];
#pragma unroll
      for (int jb = 0; jb < JW; ++jb) {
        zA[jb] = __builtin_bit_cast(f32x4, zblk[(wq * JW + jb) * 64 + lane]);
      }
#pragma unroll
      for (int i = 0; i < IG; ++i) {
        const int r = wr * IG + i;
        float kf[SPLITQK ? 1 : QS];
        bf16x8 ks[SPLITQK ? 3 : 1];
        if constexpr (SPLITQK) {
          // the key's three bf16 parts, split by kernel 1
#pragma unroll
          for (int kp = 0; kp < 3; ++kp) ks[kp] = as_bf16x8(kblk[(r * KBR + kp) * 64 + lane]);
        } else {
#pragma unroll
          for (int kp = 0; kp < KBR; ++kp) {
            const float4 v = __builtin_bit_cast(float4, kblk[(r * KBR + kp) * 64 + lane]);
            kf[4 * kp] = v.x, kf[4 * kp + 1] = v.y, kf[4 * kp + 2] = v.z, kf[4 * kp + 3] = v.w;
          }
        }
        f32x4 vf[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) vf[mb] = __builtin_bit_cast(f32x4, vblk[(r * VBR + mb) * 64 + lane]);
#pragma unroll
        for (int jb = 0; jb < JW; ++jb) {
          f32x4 s = zA[jb];
          if constexpr (SPLITQK) {
            // (key part, query part): small terms (3,1) (2,2) (1,3), then large (2,1) (1,2) (1,1)
            f32x4 s1 = {0.f, 0.f, 0.f, 0.f};
            s1 = mfma(ks[2], qsp[i][jb][0], s1);
            s = mfma(ks[1], qsp[i][jb][0], s);
            s1 = mfma(ks[1], qsp[i][jb][1], s1);
            s = mfma(ks[0], qsp[i][jb][1], s);
            s1 = mfma(ks[0], qsp[i][jb][2], s1);
            s = mfma(ks[0], qsp[i][jb][0], s);
            s += s1;
          } else {
#pragma unroll
            for (int ss = 0; ss < QS; ++ss) s = mfma(kf[ss], qf[i][jb][ss], s);
          }
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
  };

  // The key loop over the ring: stage s is waited for (this wave's own loads
  // via vmcnt, everyone's via the barrier, which also retires every wave's
  // reads of the stage that the next issue overwrites), then step s + 2 is
  // issued and step s computed. `issued`: the first LA steps are already out.
  auto key_loop = [&](bool max_pass, float (&mx)[IG][JW], bool issued) {
    if (!issued) {
#pragma unroll
      for (int s = 0; s < LA; ++s)
        if (s < nsteps) issue(s);
    }
#pragma unroll 1
    for (int s = 0; s < nsteps; ++s) {
      // step s is complete once at most (steps issued after it) * LPW loads are outstanding
      const int after = min(LA - 1, nsteps - 1 - s);
      if (after >= 2)
        vmcnt_wait<2 * LPW>();
      else if (after == 1)
        vmcnt_wait<LPW>();
      else
        vmcnt_wait<0>();
      lds_barrier();
      if (s + LA < nsteps) issue(s + LA);
      step_compute(ring + (size_t)(s % NS) * (STAGE / 16), max_pass, mx);
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


  // ---- normalise, fully masked columns, gate; write over the gate. `it`,
  // `cm` and vsum_s[buf] belong to the finished item (the next item's setup
  // may have run already).
  const bool fill_nan = (a.mask_fill == -INFINITY);
  const float inv_n = 1.0f / (float)N;
  auto epilogue = [&](const Item &it, const bool (&cm)[JW], int buf) {
#pragma unroll
    for (int i = 0; i < IG; ++i) {
      const int row = it.i0 + wr * IG + i;
      // Uniform weights of a fully masked column (finite fill): the mean of v
      // over all N keys (padding keys are zero). Lane (g, r16) needs channels
      // 4g..4g+3 of each of the head's 16-channel blocks.
      float vmean[MB][4];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const float4 m4 = *reinterpret_cast<const float4 *>(&vsum_s[buf][(wr * IG + i) * DH + mb * 16 + 4 * g]);
        vmean[mb][0] = m4.x * inv_n, vmean[mb][1] = m4.y * inv_n, vmean[mb][2] = m4.z * inv_n, vmean[mb][3] = m4.w * inv_n;
      }
#pragma unroll
      for (int jb = 0; jb < JW; ++jb) {
        const int j = it.j0 + (wq * JW + jb) * 16 + r16;
        const bool masked = cm[jb];
        const float inv_l = masked ? 0.f : 1.0f / lsum[i][jb];
        if (row < N && j < N) {
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            T *gp = G + (((size_t)(it.b * N + row) * NB + it.t * MB + mb) * Np + j) * 16 + 4 * g;
            const GVec w = gate[i][jb][mb];
            float gv[4];
            if constexpr (BF)
              gv[0] = bflo(w.x), gv[1] = bfhi(w.x), gv[2] = bflo(w.y), gv[3] = bfhi(w.y);
            else
              gv[0] = w.x, gv[1] = w.y, gv[2] = w.z, gv[3] = w.w;
            float ov[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float oo = masked ? (fill_nan ? __builtin_nanf("") : vmean[mb][r]) : o[i][jb][mb][r] * inv_l;
              ov[r] = oo * gv[r];
            }
            if constexpr (BF)
              stg<uint2>(gp, make_uint2(pack_bf16x2(ov[0], ov[1]), pack_bf16x2(ov[2], ov[3])));
            else
              stg<float4>(gp, make_float4(ov[0], ov[1], ov[2], ov[3]));
          }
        }
      }
    }
  };

  // ---- the first item
  int v = blockIdx.x;
  if (v >= a.items) return;
  Item cur = coords(v);
  set_item(cur);
  load_setup();
  load_q();
  set_loader();
#pragma unroll
  for (int s = 0; s < LA; ++s) issue(s);
  int buf = 0;
  setup(buf);

  float dummy[IG][JW];
#pragma unroll 1
  for (;;) {
    zero_acc();
    key_loop(false, dummy, true);
    vmcnt_wait<0>();  // early steps past the live ones, if any, have landed
    row_sums();

    // ---- recovery: exact maximum where the bound was too loose. The
    // decision is workgroup-wide: every wave runs the key loop and its
    // barriers together.
    bool need = false;
#pragma unroll
    for (int i = 0; i < IG; ++i)
#pragma unroll
      for (int jb = 0; jb < JW; ++jb)
        if (zmx[jb] > -INFINITY && !(lsum[i][jb] >= 0x1p-64f)) need = true;
    if (__ballot(need) != 0 && lane == 0) need_s[buf] = 1;
    lds_barrier();  // also: every wave is done with the ring
    if (a.rflag && threadIdx.x == 0) a.rflag[v] = (uint8_t)need_s[buf];
    if (need_s[buf]) {
      float mx[IG][JW];
#pragma unroll
      for (int i = 0; i < IG; ++i)
#pragma unroll
        for (int jb = 0; jb < JW; ++jb) {
          mx[i][jb] = -INFINITY;
          msh[i][jb] = 0.f;
        }
      set_shift(msh);  // no shift during the max pass
      key_loop(true, mx, false);
#pragma unroll
      for (int i = 0; i < IG; ++i)
#pragma unroll
        for (int jb = 0; jb < JW; ++jb) {
          const float m = group4_max(mx[i][jb]);
          msh[i][jb] = (zmx[jb] == -INFINITY) ? 0.f : m;
        }
      set_shift(msh);
      shift_on = true;
      zero_acc();
      lds_barrier();  // every wave is done with the ring before it is refilled
      key_loop(false, dummy, false);
      row_sums();
      vmcnt_wait<0>();
      lds_barrier();  // every wave is done with the ring
    }

    // ---- this item's gate, then the next item's setup loads, query
    // fragments and first key steps (the ring is free): their round trips
    // overlap the next item's setup and this item's epilogue
    asm volatile("" : "+v"(lane), "+v"(g), "+v"(r16));
    load_gate();
    bool cm[JW];
#pragma unroll
    for (int jb = 0; jb < JW; ++jb) cm[jb] = colmask[jb];
    const Item done = cur;
    v += G8;
    const bool more = v < a.items;
    if (more) {
      cur = coords(v);
      set_item(cur);
      load_setup();
      load_q();
      set_loader();
#pragma unroll
      for (int s = 0; s < LA; ++s) issue(s);
      setup(buf ^ 1);
    }
    epilogue(done, cm, buf);
    if (!more) break;
    buf ^= 1;
  }
}

template <typename T, int D, int DH>
static hipError_t launch_k2_t(const K2Args &a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((k2_attention<T, D, DH>), dim3(grid), dim3(K2Shape<T, D, DH>::NW * 64), 0, s, a);
  return hipGetLastError();
}

// bf16 with head size 16 is compiled in a unit of its own (this source with
// TPA_K2_BF16_D16 defined), built with LLVM's max-memory-clause instruction
// scheduler: its key loop measured 3% faster that way, the other shapes
// slower. Each kernel instantiation lives in exactly one unit.
hipError_t launch_k2_bf16_d16(int D, const K2Args &a, int grid, hipStream_t s);
int k2_blocks_per_cu_bf16_d16(int D);

#ifdef TPA_K2_BF16_D16
hipError_t launch_k2_bf16_d16(int D, const K2Args &a, int grid, hipStream_t s) {
  if (D == 128) return launch_k2_t<bf16_t, 128, 16>(a, grid, s);
  if (D == 64) return launch_k2_t<bf16_t, 64, 16>(a, grid, s);
  return hipErrorInvalidValue;
}

int k2_blocks_per_cu_bf16_d16(int D) {
  int n = 0;
  hipError_t e = hipErrorInvalidValue;
  if (D == 128)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k2_attention<bf16_t, 128, 16>,
                                                     K2Shape<bf16_t, 128, 16>::NW * 64, 0);
  else if (D == 64)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k2_attention<bf16_t, 64, 16>,
                                                     K2Shape<bf16_t, 64, 16>::NW * 64, 0);
  return (e == hipSuccess && n > 0) ? n : 1;
}
#else
int k2_items(int dtype, int D, int dh, int B, int N) {
  int RB = 8, QB = 64;
#define TRI_K2_SHAPE(TT, DD, HH)  \
  if (D == DD && dh == HH) {      \
    RB = K2Shape<TT, DD, HH>::RB; \
    QB = K2Shape<TT, DD, HH>::QB; \
  }
  if (dtype == TRI_ATTN_BF16) {
    TRI_K2_SHAPE(bf16_t, 128, 16)
    TRI_K2_SHAPE(bf16_t, 128, 32)
    TRI_K2_SHAPE(bf16_t, 64, 16)
    TRI_K2_SHAPE(bf16_t, 64, 32)
  } else {
    TRI_K2_SHAPE(float, 128, 16)
    TRI_K2_SHAPE(float, 128, 32)
    TRI_K2_SHAPE(float, 64, 16)
    TRI_K2_SHAPE(float, 64, 32)
  }
#undef TRI_K2_SHAPE
  return B * (D / dh) * ((N + RB - 1) / RB) * ((N + QB - 1) / QB);
}

hipError_t launch_k2(int dtype, int D, int dh, const K2Args &a, int grid, hipStream_t s) {
#define TRI_K2_CASE(TT, DD, HH) \
  if (D == DD && dh == HH) return launch_k2_t<TT, DD, HH>(a, grid, s);
  if (dtype == TRI_ATTN_BF16) {
    if (dh == 16) return launch_k2_bf16_d16(D, a, grid, s);
    TRI_K2_CASE(bf16_t, 128, 32)
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

int k2_blocks_per_cu(int dtype, int D, int dh) {
  if (dtype == TRI_ATTN_BF16 && dh == 16) return k2_blocks_per_cu_bf16_d16(D);
  int n = 0;
#define TRI_K2_OCC(TT, DD, HH)                                                                                   \
  if (D == DD && dh == HH &&                                                                                     \
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k2_attention<TT, DD, HH>, K2Shape<TT, DD, HH>::NW * 64, 0) != \
          hipSuccess)                                                                                            \
    n = 1;
  if (dtype == TRI_ATTN_BF16) {
    TRI_K2_OCC(bf16_t, 128, 32)
    TRI_K2_OCC(bf16_t, 64, 32)
  } else {
    TRI_K2_OCC(float, 128, 16)
    TRI_K2_OCC(float, 128, 32)
    TRI_K2_OCC(float, 64, 16)
    TRI_K2_OCC(float, 64, 32)
  }
#undef TRI_K2_OCC
  return n > 0 ? n : 1;
}
#endif

}  // namespace tpa

// Host side of the C ABI declared in include/tri_attn.h: argument checks,
// weight packing, workspace layout and the two kernel launches.
#include "tri_attn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <new>

#include "tri_attn_internal.h"

struct tri_attn {
  tri_attn_config cfg;
  float shift_slack;  // testing aid (tri_attn_set_shift_slack), 0 in normal use
  int bwd_dz_ranges;  // testing aid (tri_attn_set_backward_dz_ranges), 0 in normal use
  int D, h, dh, elem;
  int device;
  int k1_grid;     // persistent grid of kernel 1 (resident workgroups)
  int k2_grid;     // persistent grid of kernel 2
  int k3_grid;     // persistent grid of kernel 3
  void *wpack;     // [(4D + 16)][D] Wq; Wk; Wv; Wg; Wz; zero rows
  void *vecs;      // gamma, beta, bg, bo ([D] each), then Wo [D][D]
  void *wfrag;     // Wq; Wk; Wv; Wg, then Wo, in fragment order
  void *wsplit;    // float32 handles: the same five matrices as three bf16 planes in fragment order
  size_t wpack_bytes, vecs_bytes, wfrag_bytes, wsplit_plane;
  void *scratch;   // this device's static workspace array (tri_attn_forward_noalloc)
  int scratch_rc;  // status of its address lookup at creation
  // the backward's second stream (default priority) and its fork/join events
  hipStream_t bwd_side;
  hipEvent_t bwd_fork, bwd_join;
};

namespace tpa {

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

Layout make_layout(int B, int N, int D, int h, int elem) {
  Layout L{};
  L.Np = ((N + kChunk - 1) / kChunk) * kChunk;
  L.nchunk = L.Np / kChunk;
  const size_t proj = (size_t)B * N * D * L.Np * elem;  // [B][N][D/16][Np][16] (and v^T)
  size_t off = 0;
  L.q = off, off = align256(off + proj);
  // float32 with d = 32: k as three bf16 parts (6 bytes per element)
  L.k = off, off = align256(off + ((elem == 4 && D / h == 32) ? proj / 4 * 6 : proj));
  L.vt = off, off = align256(off + proj);
  L.g = off, off = align256(off + proj);
  L.zm = off, off = align256(off + (size_t)B * h * N * L.Np * 4);
  L.zmax = off, off = align256(off + (size_t)B * h * N * L.nchunk * 4);
  L.kmax = off, off = align256(off + (size_t)B * N * (D / 16) * L.nchunk * 4);
  L.vsum = off, off = align256(off + (size_t)B * N * D * L.nchunk * 4);
  L.items = k2_items(elem == 2 ? TRI_ATTN_BF16 : TRI_ATTN_F32, D, D / h, B, N);
  L.rflag = off, off = align256(off + (size_t)L.items);
  L.total = off;
  return L;
}

}  // namespace tpa

using namespace tpa;

extern "C" {

const char *tri_attn_strerror(int code) {
  switch (code) {
    case TRI_ATTN_OK: return "ok";
    case TRI_ATTN_ERR_INVALID_ARG: return "invalid argument";
    case TRI_ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case TRI_ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case TRI_ATTN_ERR_HIP: return "HIP runtime error";
    case TRI_ATTN_ERR_OOM: return "device allocation failed";
    default: return "unknown error code";
  }
}

static int check_config(const tri_attn_config *cfg) {
  if (!cfg) return TRI_ATTN_ERR_INVALID_ARG;
  if (cfg->pair_dim <= 0 || cfg->num_heads <= 0 || cfg->pair_dim % cfg->num_heads != 0)
    return TRI_ATTN_ERR_INVALID_ARG;
  if (cfg->dtype != TRI_ATTN_F32 && cfg->dtype != TRI_ATTN_BF16) return TRI_ATTN_ERR_INVALID_ARG;
  if (!(cfg->ln_eps > 0.f) || !std::isfinite(cfg->ln_eps)) return TRI_ATTN_ERR_INVALID_ARG;
  const float f = cfg->mask_fill;
  if (std::isnan(f) || !(f == -INFINITY || (std::isfinite(f) && f <= -1e4f))) return TRI_ATTN_ERR_INVALID_ARG;
  if (cfg->ending_node != 0 && cfg->ending_node != 1) return TRI_ATTN_ERR_INVALID_ARG;
  if (!supported(cfg->pair_dim, cfg->pair_dim / cfg->num_heads)) return TRI_ATTN_ERR_UNSUPPORTED;
  return TRI_ATTN_OK;
}

// fault injection for tests: the armed create call fails its nth device allocation
static std::atomic<int> g_alloc_fault{0};

int tri_attn_set_alloc_fault(int nth) {
  if (nth < 0) return TRI_ATTN_ERR_INVALID_ARG;
  g_alloc_fault.store(nth);
  return TRI_ATTN_OK;
}

int tri_attn_create(const tri_attn_config *cfg, const tri_attn_weights *w, void *stream, tri_attn_t *out) {
  if (!out) return TRI_ATTN_ERR_INVALID_ARG;
  *out = nullptr;
  int rc = check_config(cfg);
  if (rc) return rc;
  const int fault = g_alloc_fault.exchange(0);
  int nalloc = 0;
  auto device_alloc = [&](void **p, size_t bytes) -> hipError_t {
    if (++nalloc == fault) return hipErrorOutOfMemory;
    return hipMalloc(p, bytes);
  };
  if (!w || !w->ln_weight || !w->ln_bias || !w->w_query || !w->w_key || !w->w_value || !w->w_gate ||
      !w->b_gate || !w->w_bias_proj || !w->w_out || !w->b_out)
    return TRI_ATTN_ERR_INVALID_ARG;

  tri_attn *t = new (std::nothrow) tri_attn();
  if (!t) return TRI_ATTN_ERR_OOM;
  t->cfg = *cfg;
  t->shift_slack = 0.f;
  t->bwd_dz_ranges = 0;
  t->D = cfg->pair_dim;
  t->h = cfg->num_heads;
  t->dh = t->D / t->h;
  t->elem = cfg->dtype == TRI_ATTN_BF16 ? 2 : 4;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int D = t->D, h = t->h, e = t->elem;

  if (hipGetDevice(&t->device) != hipSuccess) {
    delete t;
    return TRI_ATTN_ERR_HIP;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, t->device) != hipSuccess || cus <= 0) {
    delete t;
    return TRI_ATTN_ERR_HIP;
  }
  t->k1_grid = cus * (cfg->dtype == TRI_ATTN_F32 ? k1_split_blocks_per_cu(t->D, t->dh)
                                                 : k1_blocks_per_cu(cfg->dtype, t->D, t->dh));
  t->k2_grid = cus * k2_blocks_per_cu(cfg->dtype, t->D, t->dh);
  t->k3_grid = cus * k3_blocks_per_cu(cfg->dtype, t->D);
  // the static workspace array's address on this device, looked up once per device
  t->scratch_rc = scratch_address(t->device, &t->scratch);

  t->wpack_bytes = (size_t)(4 * D + 16) * D * e;
  t->vecs_bytes = (size_t)4 * D * e + (size_t)D * D * e;
  if (device_alloc(&t->wpack, t->wpack_bytes) != hipSuccess) {
    delete t;
    return TRI_ATTN_ERR_OOM;
  }
  if (device_alloc(&t->vecs, t->vecs_bytes) != hipSuccess) {
    (void)hipFree(t->wpack);
    delete t;
    return TRI_ATTN_ERR_OOM;
  }
  t->wfrag_bytes = (size_t)5 * D * D * e;
  if (device_alloc(&t->wfrag, t->wfrag_bytes) != hipSuccess) {
    (void)hipFree(t->wpack);
    (void)hipFree(t->vecs);
    delete t;
    return TRI_ATTN_ERR_OOM;
  }
  t->wsplit_plane = (size_t)5 * D * D * 2;
  if (cfg->dtype == TRI_ATTN_F32 && device_alloc(&t->wsplit, 3 * t->wsplit_plane) != hipSuccess) {
    (void)hipFree(t->wpack);
    (void)hipFree(t->vecs);
    (void)hipFree(t->wfrag);
    delete t;
    return TRI_ATTN_ERR_OOM;
  }
  char *wp = static_cast<char *>(t->wpack);
  char *vp = static_cast<char *>(t->vecs);
  const size_t mat = (size_t)D * D * e, vec = (size_t)D * e;
  bool ok = hipMemsetAsync(t->wpack, 0, t->wpack_bytes, s) == hipSuccess;
  ok = ok && hipMemcpyAsync(wp + 0 * mat, w->w_query, mat, hipMemcpyDefault, s) == hipSuccess;
  ok = ok && hipMemcpyAsync(wp + 1 * mat, w->w_key, mat, hipMemcpyDefault, s) == hipSuccess;
  ok = ok && hipMemcpyAsync(wp + 2 * mat, w->w_value, mat, hipMemcpyDefault, s) == hipSuccess;
  ok = ok && hipMemcpyAsync(wp + 3 * mat, w->w_gate, mat, hipMemcpyDefault, s) == hipSuccess;
  ok = ok && hipMemcpyAsync(wp + 4 * mat, w->w_bias_proj, (size_t)h * D * e, hipMemcpyDefault, s) == hipSuccess;
  ok = ok && hipMemcpyAsync(vp + 0 * vec, w->ln_weight, vec, hipMemcpyDefault, s) == hipSuccess;
  ok = ok && hipMemcpyAsync(vp + 1 * vec, w->ln_bias, vec, hipMemcpyDefault, s) == hipSuccess;
  ok = ok && hipMemcpyAsync(vp + 2 * vec, w->b_gate, vec, hipMemcpyDefault, s) == hipSuccess;
  ok = ok && hipMemcpyAsync(vp + 3 * vec, w->b_out, vec, hipMemcpyDefault, s) == hipSuccess;
  ok = ok && hipMemcpyAsync(vp + 4 * vec, w->w_out, mat, hipMemcpyDefault, s) == hipSuccess;
  ok = ok && launch_pack_frags(e, D, wp, t->wfrag, 4 * D / 16, s) == hipSuccess;
  ok = ok && launch_pack_frags(e, D, vp + 4 * vec, static_cast<char *>(t->wfrag) + 4 * mat, D / 16, s) == hipSuccess;
  if (t->wsplit) {
    ok = ok && launch_pack_frags_split3(D, wp, t->wsplit, t->wsplit_plane, 4 * D / 16, s) == hipSuccess;
    ok = ok && launch_pack_frags_split3(D, vp + 4 * vec, static_cast<char *>(t->wsplit) + (size_t)4 * D * D * 2,
                                        t->wsplit_plane, D / 16, s) == hipSuccess;
  }
  ok = ok && hipStreamSynchronize(s) == hipSuccess;
  t->bwd_side = nullptr, t->bwd_fork = nullptr, t->bwd_join = nullptr;
  ok = ok && hipStreamCreateWithFlags(&t->bwd_side, hipStreamNonBlocking) == hipSuccess;
  ok = ok && hipEventCreateWithFlags(&t->bwd_fork, hipEventDisableTiming) == hipSuccess;
  ok = ok && hipEventCreateWithFlags(&t->bwd_join, hipEventDisableTiming) == hipSuccess;
  if (!ok) {
    if (t->bwd_side) (void)hipStreamDestroy(t->bwd_side);
    if (t->bwd_fork) (void)hipEventDestroy(t->bwd_fork);
    if (t->bwd_join) (void)hipEventDestroy(t->bwd_join);
    (void)hipGetLastError();
    (void)hipFree(t->wpack);
    (void)hipFree(t->vecs);
    (void)hipFree(t->wfrag);
    if (t->wsplit) (void)hipFree(t->wsplit);
    delete t;
    return TRI_ATTN_ERR_HIP;
  }
  *out = t;
  return TRI_ATTN_OK;
}

static int check_sizes(tri_attn_t t, int B, int N) {
  if (!t) return TRI_ATTN_ERR_INVALID_ARG;
  if (B < 0 || N < 0) return TRI_ATTN_ERR_INVALID_ARG;
  if (B == 0 || N == 0) return TRI_ATTN_OK;
  // kernels index elements of one tensor with 64-bit bases but 32-bit item counts
  const Layout L = make_layout(B, N, t->D, t->h, t->elem);
  if ((double)B * N * ((N + 15) / 16) > 2.0e9 || (double)B * N * L.nchunk > 2.0e9) return TRI_ATTN_ERR_UNSUPPORTED;
  return TRI_ATTN_OK;
}

int tri_attn_workspace_size(tri_attn_t t, int B, int N, size_t *bytes) {
  if (!bytes) return TRI_ATTN_ERR_INVALID_ARG;
  int rc = check_sizes(t, B, N);
  if (rc) return rc;
  *bytes = (B == 0 || N == 0) ? 0 : make_layout(B, N, t->D, t->h, t->elem).total;
  return TRI_ATTN_OK;
}

int tri_attn_get_workspace_layout(tri_attn_t t, int B, int N, tri_attn_workspace_layout *out) {
  if (!out) return TRI_ATTN_ERR_INVALID_ARG;
  int rc = check_sizes(t, B, N);
  if (rc) return rc;
  std::memset(out, 0, sizeof(*out));
  if (B == 0 || N == 0) return TRI_ATTN_OK;
  const Layout L = make_layout(B, N, t->D, t->h, t->elem);
  out->q = L.q, out->k = L.k, out->vt = L.vt, out->g = L.g;
  out->zm = L.zm, out->zmax = L.zmax, out->kmax = L.kmax, out->vsum = L.vsum;
  out->recover_flags = L.rflag;
  out->attention_items = L.items;
  out->total = L.total;
  out->padded_n = L.Np;
  return TRI_ATTN_OK;
}

// stages: bit 0 = projection kernel, bit 1 = attention kernel, bit 2 = output projection
static int run(tri_attn_t t, const void *pair_repr, const uint8_t *pair_mask, void *out, int B, int N,
               void *ws, size_t ws_bytes, void *stream, int stages, const K2TrainArgs *train = nullptr) {
  int rc = check_sizes(t, B, N);
  if (rc) return rc;
  if (B == 0 || N == 0) return TRI_ATTN_OK;
  if (((stages & 1) && (!pair_repr || !pair_mask)) || ((stages & 4) && !out)) return TRI_ATTN_ERR_INVALID_ARG;
  const Layout L = make_layout(B, N, t->D, t->h, t->elem);
  if (!ws || ws_bytes < L.total || (reinterpret_cast<uintptr_t>(ws) & 255)) return TRI_ATTN_ERR_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char *w = static_cast<char *>(ws);
  const int D = t->D, e = t->elem;
  const char *vp = static_cast<const char *>(t->vecs);

  K1Args a1{};
  a1.P = pair_repr;
  a1.mask = pair_mask;
  a1.W = t->wpack;
  a1.Wf = t->wfrag;
  a1.Ws = t->wsplit;
  a1.ws_plane = t->wsplit_plane;
  a1.gamma = vp;
  a1.beta = vp + (size_t)D * e;
  a1.bg = vp + (size_t)2 * D * e;
  a1.q = w + L.q, a1.k = w + L.k, a1.vt = w + L.vt, a1.g = w + L.g;
  a1.zm = reinterpret_cast<float *>(w + L.zm);
  a1.zmax = reinterpret_cast<float *>(w + L.zmax);
  a1.kmax = reinterpret_cast<float *>(w + L.kmax);
  a1.vsum = reinterpret_cast<float *>(w + L.vsum);
  a1.eps = t->cfg.ln_eps;
  a1.qscale = (float)(1.4426950408889634 / std::sqrt((double)t->dh));
  a1.B = B, a1.N = N, a1.Np = L.Np, a1.nchunk = L.nchunk;
  a1.transposed = t->cfg.ending_node;
  a1.tiles = B * N * L.nchunk;
  if (stages & 1) {
    hipError_t e1;
    if (t->cfg.dtype == TRI_ATTN_F32) {
      // two workgroups per tile (one per half of the projections); a multiple
      // of 8 per half when the tiles fill the device, so a tile's two halves
      // share an XCD
      int half = t->k1_grid / 2;
      if (half >= 8) half = half / 8 * 8;
      if (half < 1) half = 1;
      e1 = launch_k1_split(D, t->dh, a1, 2 * (a1.tiles < half ? a1.tiles : half), s);
    } else {
      e1 = launch_k1(t->cfg.dtype, D, t->dh, a1, a1.tiles < t->k1_grid ? a1.tiles : t->k1_grid, s);
    }
    if (e1 != hipSuccess) return TRI_ATTN_ERR_HIP;
  }

  K2Args a2{};
  a2.q = a1.q, a2.k = a1.k, a2.vt = a1.vt, a2.g = a1.g;
  a2.zm = a1.zm, a2.zmax = a1.zmax, a2.kmax = a1.kmax, a2.vsum = a1.vsum;
  a2.mask_fill = t->cfg.mask_fill;
  a2.shift_slack = t->shift_slack;
  a2.B = B, a2.N = N, a2.Np = L.Np, a2.nchunk = L.nchunk;
  a2.items = L.items;
  a2.rflag = reinterpret_cast<uint8_t *>(w + L.rflag);
  // persistent workgroups; with more items than that, a multiple of 8 so that
  // each keeps its XCD from item to item
  int grid2 = a2.items;
  if (grid2 > t->k2_grid) grid2 = t->k2_grid >= 8 ? t->k2_grid / 8 * 8 : t->k2_grid;
  if (stages & 2) {
    const hipError_t e2 = train ? launch_k2_train(t->cfg.dtype, t->dh, a2, *train, s)
                                : launch_k2(t->cfg.dtype, D, t->dh, a2, grid2, s);
    if (e2 != hipSuccess) return TRI_ATTN_ERR_HIP;
  }

  K3Args a3{};
  a3.go = a1.g;
  if (t->wsplit) {
    a3.Wof = static_cast<const char *>(t->wsplit) + (size_t)4 * D * D * 2;
    a3.wo_plane = t->wsplit_plane;
  } else {
    a3.Wof = static_cast<const char *>(t->wfrag) + (size_t)4 * D * D * e;
  }
  a3.bo = vp + (size_t)3 * D * e;
  a3.out = out;
  a3.B = B, a3.N = N, a3.Np = L.Np, a3.nchunk = L.nchunk;
  a3.transposed = t->cfg.ending_node;
  a3.tiles = a1.tiles;
  const int grid3 = a3.tiles < t->k3_grid ? a3.tiles : t->k3_grid;
  if ((stages & 4) && launch_k3(t->cfg.dtype, D, a3, grid3, s) != hipSuccess) return TRI_ATTN_ERR_HIP;
  return TRI_ATTN_OK;
}

int tri_attn_forward(tri_attn_t t, const void *pair_repr, const uint8_t *pair_mask, void *out, int B, int N,
                     void *workspace, size_t ws_bytes, void *stream) {
  return run(t, pair_repr, pair_mask, out, B, N, workspace, ws_bytes, stream, 7);
}

int tri_attn_forward_noalloc(tri_attn_t t, const void *pair_repr, const uint8_t *pair_mask, void *out, int B, int N,
                             void *stream) {
  size_t need = 0;
  const int rc = tri_attn_workspace_size(t, B, N, &need);
  if (rc) return rc;
  if (need > TRI_ATTN_NOALLOC_MAX_BYTES) return TRI_ATTN_ERR_WORKSPACE;
  if (t->scratch_rc || !t->scratch) return TRI_ATTN_ERR_HIP;
  return run(t, pair_repr, pair_mask, out, B, N, t->scratch, TRI_ATTN_NOALLOC_MAX_BYTES, stream, 7);
}

int tri_attn_forward_train(tri_attn_t t, const void *pair_repr, const uint8_t *pair_mask, void *out, float *lse,
                           int B, int N, double dropout_rate, uint64_t seed, uint32_t offset, void *workspace,
                           size_t ws_bytes, void *stream) {
  if (!t) return TRI_ATTN_ERR_INVALID_ARG;
  if (!(dropout_rate >= 0.0 && dropout_rate < 1.0)) return TRI_ATTN_ERR_INVALID_ARG;
  K2TrainArgs tr{};
  const double thr = std::min(std::nearbyint(dropout_rate * 4294967296.0), 4294967295.0);
  tr.thr = (uint32_t)thr;
  tr.scale = (float)(4294967296.0 / (4294967296.0 - thr));
  tr.seed_lo = (uint32_t)(seed & 0xFFFFFFFFu);
  tr.seed_hi = (uint32_t)(seed >> 32);
  tr.offset = offset;
  tr.lse = lse;
  tr.h = t->h;
  return run(t, pair_repr, pair_mask, out, B, N, workspace, ws_bytes, stream, 7, &tr);
}

int tri_attn_backward_workspace_size(tri_attn_t t, int B, int N, size_t *bytes) {
  if (!bytes) return TRI_ATTN_ERR_INVALID_ARG;
  const int rc = check_sizes(t, B, N);
  if (rc) return rc;
  *bytes = (B == 0 || N == 0) ? 0 : bwd_workspace_bytes(B, N, t->D, t->h, t->elem, t->cfg.ending_node, t->bwd_dz_ranges);
  return TRI_ATTN_OK;
}

int tri_attn_backward_train(tri_attn_t t, const void *pair_repr, const uint8_t *pair_mask, const void *dy, int B,
                            int N, double dropout_rate, uint64_t seed, uint32_t offset, const tri_attn_grads *grads,
                            void *workspace, size_t ws_bytes, void *stream) {
  if (!t) return TRI_ATTN_ERR_INVALID_ARG;
  if (!(dropout_rate >= 0.0 && dropout_rate < 1.0)) return TRI_ATTN_ERR_INVALID_ARG;
  int rc = check_sizes(t, B, N);
  if (rc) return rc;
  if (B == 0 || N == 0) return TRI_ATTN_OK;
  if (!pair_repr || !pair_mask || !dy || !grads) return TRI_ATTN_ERR_INVALID_ARG;
  const tri_attn_grads &g = *grads;
  if (!g.d_pair_repr || !g.d_ln_weight || !g.d_ln_bias || !g.d_w_query || !g.d_w_key || !g.d_w_value ||
      !g.d_w_gate || !g.d_b_gate || !g.d_w_bias_proj || !g.d_w_out || !g.d_b_out)
    return TRI_ATTN_ERR_INVALID_ARG;
  const size_t need = bwd_workspace_bytes(B, N, t->D, t->h, t->elem, t->cfg.ending_node, t->bwd_dz_ranges);
  if (!workspace || ws_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255)) return TRI_ATTN_ERR_WORKSPACE;
  BwdRunArgs r{};
  r.P = pair_repr, r.mask = pair_mask, r.dy = dy, r.wpack = t->wpack, r.vecs = t->vecs, r.g = g, r.ws = workspace;
  r.eps = t->cfg.ln_eps, r.fill = t->cfg.mask_fill;
  const double thr = std::min(std::nearbyint(dropout_rate * 4294967296.0), 4294967295.0);
  r.thr = (uint32_t)thr;
  r.scale = (float)(4294967296.0 / (4294967296.0 - thr));
  r.seed_lo = (uint32_t)(seed & 0xFFFFFFFFu), r.seed_hi = (uint32_t)(seed >> 32), r.offset = offset;
  r.B = B, r.N = N;
  r.transposed = t->cfg.ending_node;
  r.dz_ranges = t->bwd_dz_ranges;
  r.side = t->bwd_side, r.fork = t->bwd_fork, r.join = t->bwd_join;
  if (launch_bwd(t->cfg.dtype, t->D, t->dh, r, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return TRI_ATTN_ERR_HIP;
  return TRI_ATTN_OK;
}

int tri_attn_onepass_workspace_size(tri_attn_t t, int B, int N, size_t *bytes) {
  if (!bytes) return TRI_ATTN_ERR_INVALID_ARG;
  const int rc = check_sizes(t, B, N);
  if (rc) return rc;
  if (N > kOnePassMaxN) return TRI_ATTN_ERR_UNSUPPORTED;
  const size_t Np = ((size_t)N + 63) / 64 * 64;
  *bytes = (B == 0 || N == 0) ? 0 : (size_t)B * t->h * N * Np * sizeof(float);
  return TRI_ATTN_OK;
}

int tri_attn_forward_onepass(tri_attn_t t, const void *pair_repr, const uint8_t *pair_mask, void *out, int B, int N,
                             void *workspace, size_t ws_bytes, void *stream) {
  size_t need = 0;
  const int rc = tri_attn_onepass_workspace_size(t, B, N, &need);
  if (rc) return rc;
  if (B == 0 || N == 0) return TRI_ATTN_OK;
  if (!pair_repr || !pair_mask || !out) return TRI_ATTN_ERR_INVALID_ARG;
  if (!workspace || ws_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255)) return TRI_ATTN_ERR_WORKSPACE;
  OnePassArgs a{};
  a.P = pair_repr, a.mask = pair_mask, a.W = t->wpack, a.vecs = t->vecs;
  a.zm = static_cast<float *>(workspace), a.out = out;
  a.eps = t->cfg.ln_eps, a.fill = t->cfg.mask_fill;
  a.qscale = (float)(1.4426950408889634 / std::sqrt((double)t->dh));
  a.B = B, a.N = N, a.Np = (N + 63) / 64 * 64, a.h = t->h, a.transposed = t->cfg.ending_node;
  if (launch_onepass(t->cfg.dtype, t->D, t->dh, a, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return TRI_ATTN_ERR_HIP;
  return TRI_ATTN_OK;
}

int tri_attn_project(tri_attn_t t, const void *pair_repr, const uint8_t *pair_mask, int B, int N, void *workspace,
                     size_t ws_bytes, void *stream) {
  return run(t, pair_repr, pair_mask, nullptr, B, N, workspace, ws_bytes, stream, 1);
}

int tri_attn_attend(tri_attn_t t, int B, int N, void *workspace, size_t ws_bytes, void *stream) {
  return run(t, nullptr, nullptr, nullptr, B, N, workspace, ws_bytes, stream, 2);
}

int tri_attn_output(tri_attn_t t, void *out, int B, int N, void *workspace, size_t ws_bytes, void *stream) {
  return run(t, nullptr, nullptr, out, B, N, workspace, ws_bytes, stream, 4);
}

int tri_attn_set_shift_slack(tri_attn_t t, float slack) {
  if (!t || !std::isfinite(slack) || slack < 0.f) return TRI_ATTN_ERR_INVALID_ARG;
  t->shift_slack = slack;
  return TRI_ATTN_OK;
}

int tri_attn_set_backward_dz_ranges(tri_attn_t t, int ranges) {
  if (!t || ranges < 0) return TRI_ATTN_ERR_INVALID_ARG;
  t->bwd_dz_ranges = ranges;
  return TRI_ATTN_OK;
}

int tri_attn_destroy(tri_attn_t t) {
  if (!t) return TRI_ATTN_OK;
  int rc = TRI_ATTN_OK;
  if (hipDeviceSynchronize() != hipSuccess) rc = TRI_ATTN_ERR_HIP;
  if (hipFree(t->wpack) != hipSuccess) rc = TRI_ATTN_ERR_HIP;
  if (hipFree(t->vecs) != hipSuccess) rc = TRI_ATTN_ERR_HIP;
  if (hipFree(t->wfrag) != hipSuccess) rc = TRI_ATTN_ERR_HIP;
  if (t->wsplit && hipFree(t->wsplit) != hipSuccess) rc = TRI_ATTN_ERR_HIP;
  if (hipStreamDestroy(t->bwd_side) != hipSuccess) rc = TRI_ATTN_ERR_HIP;
  if (hipEventDestroy(t->bwd_fork) != hipSuccess) rc = TRI_ATTN_ERR_HIP;
  if (hipEventDestroy(t->bwd_join) != hipSuccess) rc = TRI_ATTN_ERR_HIP;
  delete t;
  return rc;
}

}  // extern "C"

/*
 * tri_attn.h — C ABI of the MI355X (gfx950) starting-node triangular
 * self-attention forward.
 *
 * The operation is the one the POPCORNBENCH l2_p6 transcripts work on
 * ("Kimi-K2.6 / l2_p6": its forward listing and its layer list;
 * "FW-GLM-5-1 / l2_p6": the module's forward as restated while debugging).
 * For a pair representation P of shape (B, N, N, D), a pair mask M of shape
 * (B, N, N), h heads of size d = D / h:
 *
 *   x = LayerNorm_D(P)                          (biased variance, eps, affine)
 *   g = sigmoid(x Wg^T + bg)
 *   z[b,t,j,k] = x[b,j,k] . Wz[t]               (pair bias, shared by all rows i)
 *   q, k, v = x Wq^T, x Wk^T, x Wv^T            (channel t*d+u is head t)
 *   s[b,i,t,j,k] = q[b,i,j,t] . k[b,i,k,t] / sqrt(d) + z[b,t,j,k],
 *                  replaced by mask_fill where M[b,j,k] == 0
 *   a = softmax over k (dropout off: inference)
 *   o[b,i,j,t*d+u] = sum_k a[b,i,t,j,k] v[b,i,k,t*d+u]
 *   y = (g * o) Wo^T + bo                       -> output (B, N, N, D)
 *
 * All functions return 0 on success or a negative TRI_ATTN_ERR_* code; none
 * prints, aborts or lets an exception out. Streams are hipStream_t values
 * passed as void* (NULL = the default stream).
 */
#ifndef TRI_ATTN_H
#define TRI_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct tri_attn *tri_attn_t; /* opaque handle */

/* Element type of pair_repr, the weights and the output. TRI_ATTN_F32:
 * float32 accuracy throughout; the projections (LayerNorm output times the
 * q/k/v/gate/bias weights, and the output projection) run on the bf16 matrix
 * cores with each float32 operand split exactly into three bf16 parts and
 * six of the nine part products summed in float32 (relative error per
 * product at most about 2^-23, float32 level); so do the attention scores
 * q.k for head size 32, while the probability-value products (and head size
 * 16's scores) are float32 matrix-core products. TRI_ATTN_BF16: the
 * matrix-core operands are
 * bf16 and every statistic and accumulator is float32. */
enum { TRI_ATTN_F32 = 0, TRI_ATTN_BF16 = 1 };

enum {
  TRI_ATTN_OK = 0,
  TRI_ATTN_ERR_INVALID_ARG = -1,  /* NULL pointer, negative size, D % h != 0, bad dtype */
  TRI_ATTN_ERR_UNSUPPORTED = -2,  /* valid but not built: see tri_attn_create */
  TRI_ATTN_ERR_WORKSPACE = -3,    /* workspace NULL or smaller than tri_attn_workspace_size */
  TRI_ATTN_ERR_HIP = -4,          /* a HIP runtime call or kernel launch failed */
  TRI_ATTN_ERR_OOM = -5           /* device allocation failed in tri_attn_create */
};

typedef struct {
  int pair_dim;   /* D */
  int num_heads;  /* h; head_dim d = D / h (integer division, as the module does) */
  int dtype;      /* TRI_ATTN_F32 or TRI_ATTN_BF16 */
  float ln_eps;   /* LayerNorm epsilon; nn.LayerNorm's default is 1e-5 */
  /* Score written where M == 0. A finite value must be <= -1e4: masked keys
   * then get weight exactly 0 on every query column with a valid key, and a
   * column whose keys are all masked gets uniform weights over all N keys
   * (the transcripts' kernels use -1e9). -INFINITY reproduces the module's
   * masked_fill(-inf): such columns give NaN. */
  float mask_fill;
  /* 0: starting-node attention, the variant the transcripts work through
   * (each pair row i attends along its columns: scores q[i,j].k[i,k] plus the
   * bias z[j,k], mask M[j,k]). 1: ending-node attention, the counterpart
   * along the other residue axis: the starting-node computation applied to
   * the transposed pair representation and mask, transposed back, i.e.
   * y[i,j] from scores q[i,j].k[k,j] plus the bias z[k,i] (from the
   * LayerNorm output at position (k,i)), mask M[k,i], values v[k,j]. The
   * transcripts name only the starting-node variant; this reading of its
   * counterpart swaps the two residue axes throughout. Same workspace, same
   * cost. Any other value: TRI_ATTN_ERR_INVALID_ARG. */
  int ending_node;
} tri_attn_config;

/* Parameters in nn.LayerNorm / nn.Linear layouts (weight = (out, in)),
 * row-major, element type = config dtype. Pointers may be device or host
 * memory (they are copied with hipMemcpyDefault). */
typedef struct {
  const void *ln_weight, *ln_bias;        /* [D]                      */
  const void *w_query, *w_key, *w_value;  /* [D, D], no bias          */
  const void *w_gate, *b_gate;            /* [D, D], [D]              */
  const void *w_bias_proj;                /* [h, D], no bias          */
  const void *w_out, *b_out;              /* [D, D], [D]              */
} tri_attn_weights;

/* Build a handle: the module's construction from (pair_dim, num_heads) and
 * its parameters ("Kimi-K2.6 / l2_p6" transcript: the layer list, with
 * head_dim = pair_dim // num_heads, and the harness that builds the module
 * once and then calls its forward). Validates cfg, copies and packs the
 * weights into handle-owned device memory on the current device (the caller
 * may free its copies when this returns; the call synchronises `stream`),
 * and creates the handle's second stream (default priority, non-blocking)
 * and two events for tri_attn_backward_train.
 * Supported: D in {64, 128} with d in {16, 32}; other shapes with D % h == 0
 * return TRI_ATTN_ERR_UNSUPPORTED (each supported shape is its own set of
 * kernel instantiations with a register and LDS budget of its own; d = 64 and
 * D = 256 are not built). On error *out is set to NULL. */
int tri_attn_create(const tri_attn_config *cfg, const tri_attn_weights *w, void *stream, tri_attn_t *out);

/* Bytes of device workspace tri_attn_forward needs for (B, N): the
 * projections of steps (2)-(4) of the forward listing ("Kimi-K2.6 / l2_p6")
 * kept between the kernels, never the (B, N, h, N, N) scores. B == 0 or
 * N == 0 needs 0 bytes. Errors: INVALID_ARG (NULL handle or bytes, negative
 * sizes), UNSUPPORTED (sizes past the kernels' 32-bit item counts). */
int tri_attn_workspace_size(tri_attn_t h, int B, int N, size_t *bytes);

/* y = forward(pair_repr, pair_mask): the module's inference forward
 * ("Kimi-K2.6 / l2_p6" transcript: the forward listing from LayerNorm to the
 * output projection, dropout the identity in eval mode; "FW-GLM-5-1 / l2_p6":
 * the restated forward with the bias and mask broadcast over rows i), enqueued
 * on `stream`, asynchronous.
 *   pair_repr [B, N, N, D] contiguous, config dtype, device memory
 *   pair_mask [B, N, N] uint8, 0 = masked, device memory
 *   out       [B, N, N, D] contiguous, config dtype, device memory
 *   workspace device memory of at least tri_attn_workspace_size bytes, 256-byte aligned
 * All pointers are borrowed until the stream work completes; out must not
 * alias the inputs. B == 0 or N == 0 is a no-op. Kernel faults surface at
 * the caller's next synchronisation. One handle is used by one stream at a
 * time. Deterministic: no atomics, same bits on every call. */
int tri_attn_forward(tri_attn_t h, const void *pair_repr, const uint8_t *pair_mask, void *out, int B, int N,
                     void *workspace, size_t ws_bytes, void *stream);

/* Training-mode forward (arguments as tri_attn_forward, same workspace):
 * dropout on the attention weights after the softmax over keys and before
 * their product with v (FW-GLM-5-1 / l2_p6 transcript, the restated forward;
 * Kimi-K2.6 / l2_p6, the module's dropout layer). Key k of query column j,
 * head t, row (b, i) is kept iff word (k mod 4) of Philox4x32-10 (Salmon,
 * Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3",
 * SC 2011) at counter (k / 4, j, (b*N + i)*h + t, offset) and key
 * (seed & 0xFFFFFFFF, seed >> 32) is >= thr = min(round(dropout_rate * 2^32),
 * 2^32 - 1); kept weights are scaled by 2^32 / (2^32 - thr). The softmax is
 * normalised over the undropped weights.
 *   lse : DEVICE pointer, [B][N][h][N] float32, written with
 *         ln sum_k exp(s[b,i,t,j,k]) over the masked scores (fill included:
 *         a fully masked column has fill + ln N); may be NULL.
 * dropout_rate in [0, 1), else TRI_ATTN_ERR_INVALID_ARG; rate 0 gives the
 * inference output. Ending-node handles run the starting-node computation of
 * the transposed pair representation and mask: the dropout counters and lse
 * use its indices, so lse[b][j][t][i] belongs to output position (b, i, j). The
 * attention step runs on the matrix cores with a running-maximum softmax (no
 * bound on the scores is needed) and draws the dropout words inside the key
 * loop; generating them makes it several times slower than the inference
 * attention step. */
int tri_attn_forward_train(tri_attn_t h, const void *pair_repr, const uint8_t *pair_mask, void *out, float *lse,
                           int B, int N, double dropout_rate, uint64_t seed, uint32_t offset, void *workspace,
                           size_t ws_bytes, void *stream);

/* Gradients of the training-mode forward, float32 DEVICE pointers in the
 * shapes of the inputs they belong to (every one must be given). */
typedef struct {
  float *d_pair_repr;                      /* [B, N, N, D]  */
  float *d_ln_weight, *d_ln_bias;          /* [D]           */
  float *d_w_query, *d_w_key, *d_w_value;  /* [D, D]        */
  float *d_w_gate, *d_b_gate;              /* [D, D], [D]   */
  float *d_w_bias_proj;                    /* [h, D]        */
  float *d_w_out, *d_b_out;                /* [D, D], [D]   */
} tri_attn_grads;

/* Bytes of device workspace tri_attn_backward_train needs for (B, N): the
 * forward's intermediates in float32 (LayerNorm output and x-hat, the five
 * projections, the pair bias, the attention's row statistics, d(g*o), do and
 * g*o), their gradients and the partial sums of the weight gradients, and the
 * dropout decisions (one bit per score); about 8(7D + 3h) * B * N^2 +
 * B * h * N^3 / 8 bytes, plus
 * transposed copies of the inputs for ending-node handles and, when N is
 * small, partial sums of the pair-bias gradient over ranges of rows (below
 * 64 MiB). B == 0 or N == 0 needs 0 bytes. */
int tri_attn_backward_workspace_size(tri_attn_t h, int B, int N, size_t *bytes);

/* Backward of tri_attn_forward_train: with dy = dL/dy [B, N, N, D] (config
 * dtype, device), writes dL/d(pair_repr) and dL/d(every parameter) for the
 * same pair_repr, pair_mask, dropout_rate, seed and offset (hence the same
 * dropout decisions) into `grads`. It follows the forward's steps in reverse
 * (the forward listing of "Kimi-K2.6 / l2_p6"; dropout after the softmax as
 * restated in "FW-GLM-5-1 / l2_p6"): the output projection and the gate, the
 * value sum, dropout, the softmax (whose row sum of a * da is do . o), the
 * masked scores (masked entries pass no gradient: the fill is a constant),
 * the pair bias (summed over the rows i that share it), the projections and
 * the LayerNorm. Everything is recomputed from the inputs in float32 arithmetic,
 * whatever the config dtype, so nothing from the forward call is needed; the
 * products run on the matrix cores with each float32 operand split into two
 * bf16 parts (three bf16 products per float32 product, about 2^-16 relative
 * error).
 * Sums over positions are split into fixed chunks and added in a fixed order:
 * deterministic, no atomics. Asynchronous on `stream`; pointers borrowed until
 * the stream work completes. The dropout keep bits are made on the handle's
 * own second stream, forked from `stream` by an event at the call's start
 * and joined back by another before the attention steps read them, so the
 * call stays ordered on `stream`; it enqueues kernels and events only and may
 * be captured into a HIP graph from `stream`.
 * Ending-node handles: the starting-node backward
 * of the problem with both residue axes of pair_repr, pair_mask and dy
 * swapped, dL/d(pair_repr) swapped back (the ending-node training forward is
 * the starting-node one of that transposed problem, dropout counters
 * included). Errors: INVALID_ARG (NULL pointers, sizes, rate outside
 * [0, 1)), WORKSPACE, HIP. B == 0 or N == 0 is a no-op. */
int tri_attn_backward_train(tri_attn_t h, const void *pair_repr, const uint8_t *pair_mask, const void *dy, int B,
                            int N, double dropout_rate, uint64_t seed, uint32_t offset,
                            const tri_attn_grads *grads, void *workspace, size_t ws_bytes, void *stream);

/* Bytes of device workspace tri_attn_forward_onepass needs for (B, N): the
 * pair bias with the mask folded in, float32 [B][h][N][Np], Np = N rounded up
 * to 64. UNSUPPORTED for N > 512. B == 0 or N == 0 needs 0 bytes. */
int tri_attn_onepass_workspace_size(tri_attn_t h, int B, int N, size_t *bytes);

/* One-pass variant of tri_attn_forward (same arguments and result, to
 * rounding; the single fused kernel approach of "Kimi-K2.6 / l2_p6", one
 * workgroup per (b, i) row, with the pre-pass for the pair bias that its
 * Option A / Option B comparison says the bias needs): a pre-pass computes
 * LayerNorm and the pair bias of every position; then one kernel per pair row
 * recomputes LayerNorm and the q, k, v and gate projections of that row on
 * chip, attends with a running-maximum softmax, gates, and applies the output
 * projection, writing y once. q, k, v and the gate never go to device memory.
 * Starting- and ending-node handles, both dtypes, N <= 512 (UNSUPPORTED
 * above). Errors as tri_attn_forward. Asynchronous on `stream`; pointers
 * borrowed until the stream work completes. */
int tri_attn_forward_onepass(tri_attn_t h, const void *pair_repr, const uint8_t *pair_mask, void *out, int B, int N,
                             void *workspace, size_t ws_bytes, void *stream);

/* Testing hook (fault injection for tests of the error paths, not for use
 * in production): arms the next tri_attn_create call, on any thread, so that
 * its nth device allocation (1-based) fails as if the device were out of
 * memory; that create then returns TRI_ATTN_ERR_OOM after freeing what it had
 * allocated. The next create call disarms the hook whether or not it reaches
 * the nth allocation (a create makes three allocations, four for float32
 * handles); nth = 0 disarms it. Returns TRI_ATTN_OK, or INVALID_ARG for nth < 0. */
int tri_attn_set_alloc_fault(int nth);

/* Largest workspace tri_attn_forward_noalloc can use: the size of the static
 * device array that holds it (256 MiB per GPU). */
#define TRI_ATTN_NOALLOC_MAX_BYTES ((size_t)256 << 20)

/* For callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid allocation): tri_attn_forward
 * with its workspace in a static device array of TRI_ATTN_NOALLOC_MAX_BYTES
 * that the library holds, one copy per GPU, until the process ends. Arguments
 * as tri_attn_forward without the workspace; same kernels, same result bit for
 * bit. Allocates nothing: no hipMalloc, hipFree or allocating library call.
 * Errors as tri_attn_forward, and TRI_ATTN_ERR_WORKSPACE when
 * tri_attn_workspace_size(h, B, N) exceeds TRI_ATTN_NOALLOC_MAX_BYTES (B = 4,
 * N = 512, D = 128 in bf16 needs about 1.1 GB: use tri_attn_forward there),
 * TRI_ATTN_ERR_HIP if the array's device address could not be found when the
 * handle was created. Every call on one GPU shares that GPU's array: calls
 * that overlap in time on one GPU (from other streams, handles or threads)
 * race and corrupt each other's results; order them on one stream or
 * synchronise between them. The forward writes every workspace byte before
 * it reads it, so nothing is cleared between calls. */
int tri_attn_forward_noalloc(tri_attn_t h, const void *pair_repr, const uint8_t *pair_mask, void *out, int B,
                             int N, void *stream);

/* Free everything the handle owns (synchronises the device). NULL is a no-op.
 * Returns TRI_ATTN_ERR_HIP if a runtime call fails (everything is still freed). */
int tri_attn_destroy(tri_attn_t h);

/* Static message for an error code (never NULL; unknown codes get a generic text). */
const char *tri_attn_strerror(int code);

/* ---------------------------------------------------------------------------
 * Stage access (tests and tools): each of the three kernels alone, and
 * where it leaves its results in the workspace.
 * ------------------------------------------------------------------------ */

/* Offsets are in bytes from the workspace start; Np = N rounded up to 64.
 *   q, k, g : [B][N][D/16][Np][16] config dtype. Channel c of query column j
 *             of row (b, i) is at [b][i][c/16][j][c%16]. q is pre-scaled by
 *             log2(e)/sqrt(d); g is after the sigmoid (the attention stage
 *             overwrites it with g * o). Columns j >= N hold q = k = 0.
 *             Exception: float32 handles with d = 32 store k as its three
 *             bf16 parts, k = k1 + k2 + k3 exactly (round to nearest even
 *             at each step), [B][N][h][3][Np/16][4][16][8] bf16: channel
 *             8G + e of head t, key column 16s + r, part p is at
 *             [b][i][t][p][s][G][r][e].
 *   vt      : [B][N][h][d][Np] config dtype (value, transposed per head),
 *             zero for j >= N.
 *   zm      : [B][h][N][Np] float32: z[b,t,j,k] * log2(e) where M[b,j,k] != 0
 *             and k < N, -inf elsewhere.
 *   zmax    : [B][h][Np/64][N] float32: max of zm[b,t,j,:] over each 64-key
 *             chunk (chunk-major: consecutive j are adjacent).
 *   kmax    : [B][N][D/16][Np/64] float32: max over each 64-column chunk of
 *             the squared norm of k over one 16-channel block.
 *   vsum    : [B][N][Np/64][D] float32: sum of v over each 64-column chunk
 *             (for the uniform weights of fully masked query columns;
 *             chunk-major: consecutive channels are adjacent).
 *   recover_flags : [attention_items] uint8, written by every inference
 *             forward (tri_attn_forward, tri_attn_attend): 1 where the
 *             attention work item found its softmax bound too loose (a column
 *             sum below 2^-64) and recomputed with the exact maximum, else 0.
 *             A work item is one head of a block of rows and query columns;
 *             the fraction of ones is the share of the attention work done
 *             twice. */
typedef struct {
  size_t q, k, vt, g, zm, zmax, kmax, vsum, recover_flags;
  size_t total;
  int padded_n;
  int attention_items;
} tri_attn_workspace_layout;

int tri_attn_get_workspace_layout(tri_attn_t h, int B, int N, tri_attn_workspace_layout *out);

/* Testing aid: add `slack` (finite, >= 0; default 0) to every per-column
 * softmax shift of later calls on this handle. Softmax does not depend on
 * the shift, so results are unchanged. The shift normally sits 96 (log2
 * units) below the columns' Cauchy-Schwarz bound; once slack lifts it more
 * than 64 above a column's true maximum (a slack of a few hundred on ordinary
 * inputs), that column's sum falls below 2^-64 and its work item takes the
 * attention kernel's exact-maximum recovery path, which tests use to exercise
 * it. Errors: INVALID_ARG. */
int tri_attn_set_shift_slack(tri_attn_t h, float slack);

/* Testing aid: the number of row ranges (1 .. N; more are clamped to N)
 * that later tri_attn_backward_train calls on this handle split the
 * pair-bias gradient step into, each range's partial sum added in range order
 * afterwards; 0 (the default) chooses it from the sizes (one range once the
 * (query, key) tiles alone fill the GPU, more below that). Results agree to
 * float32 rounding whatever the count; tri_attn_backward_workspace_size
 * depends on it, so query the size after setting it. Errors: INVALID_ARG
 * (NULL handle, ranges < 0). */
int tri_attn_set_backward_dz_ranges(tri_attn_t h, int ranges);

/* Run only the LayerNorm + projection kernel (arguments as tri_attn_forward). */
int tri_attn_project(tri_attn_t h, const void *pair_repr, const uint8_t *pair_mask, int B, int N,
                     void *workspace, size_t ws_bytes, void *stream);

/* Run only the attention kernel on a workspace that tri_attn_project filled
 * for the same handle, B and N: it writes g * o over the gate region. The
 * gate is consumed, so run tri_attn_project again before another
 * tri_attn_attend. */
int tri_attn_attend(tri_attn_t h, int B, int N, void *workspace, size_t ws_bytes, void *stream);

/* Run only the output-projection kernel: out [B, N, N, D] = Wo (g * o) + bo
 * from the gate region left by tri_attn_attend. tri_attn_project,
 * tri_attn_attend, tri_attn_output in turn equal tri_attn_forward. */
int tri_attn_output(tri_attn_t h, void *out, int B, int N, void *workspace, size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TRI_ATTN_H */

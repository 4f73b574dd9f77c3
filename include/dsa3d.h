/*
 * dsa3d.h -- C ABI of libdsa3d: 3D Deformable Slide Attention (3D-DSA) on
 * AMD MI355X (gfx950).
 *
 * The operator. 3D-DSA is deformable attention carried over to video tokens:
 * each token (t,h,w) of a [B,T,H,W] token grid attends, per head, to the P
 * points of its k_t x k_h x k_w spatiotemporal neighbourhood, each displaced by
 * a learned offset (dt,dh,dw) [MegaSlide-DiT, §5.1 Rationale; Dutch and French
 * summaries, "3D Deformable Slide Attention", Mechanism]. Keys and values are
 * read at the displaced points by trilinear interpolation -- the pages use
 * grid_sample in bilinear mode on 5-D tensors [MegaSlide-DiT, §5.3
 * Implementation considerations] -- with zero padding outside the grid. Each
 * head takes a softmax over the P scaled dot products q.k_p/sqrt(d) and
 * returns the weighted sum of the sampled values. There is no causal mask
 * [same section]. With every offset zero this is fixed-window local attention
 * [MegaSlide-DiT, §9.1 Effect of local offsets]. The offsets come from a
 * pointwise (linear) projection of the query [§5.3; Dutch summary,
 * Implementation].
 *
 * Exact definition (the formula section §5.2 is empty in the page text; this
 * is the plain reading of the statements above):
 *   point p = (i_t,i_h,i_w), row-major over the window (w fastest);
 *   ref = (t,h,w) + dil * (i - (k-1)/2)                       (integers)
 *   pos = (float)ref + offset[p]                               (one fp32 add per axis)
 *   x0 = floorf(pos), f = pos - x0                             (fp32)
 *   k_p = sum_{c in {0,1}^3} prod_axis(c ? f : 1-f) * K[x0 + c]  (0 outside the grid)
 *   s_p = scale * <q, k_p>, a = softmax_p(s), o = sum_p a_p v_p, lse = log sum_p exp(s_p)
 * A position that is NaN, infinite or |pos| >= 2^30 makes its sample read
 * zeros. Samples outside the grid stay in the softmax with logit 0.
 *
 * Conventions for every call:
 *  - Tensors are dense, row-major, on the device, owned by the caller:
 *      q, k, v, out, dout, dq, dk, dv:  [B,T,H,W,heads,head_dim]
 *      offsets, doffsets:               [B,T,H,W,heads,P,3], last axis (dt,dh,dw)
 *      lse:                             [B,T,H,W,heads] float32
 *    Element type: desc->dtype (DSA3D_F32 = float32, DSA3D_BF16 = bfloat16 bits),
 *    except lse, dW and dbias, which are always float32.
 *  - Base pointers must be 16-byte aligned (DSA3D_ERR_MISALIGNED otherwise).
 *  - Calls only enqueue work on `stream` (a hipStream_t; NULL = the null
 *    stream) and return; they never synchronise and never allocate device
 *    memory. Scratch memory is the caller's workspace, sized by
 *    dsa3d_workspace_size() (dsa3d_backward_noalloc uses a fixed array of the
 *    library instead).
 *  - Errors: a negative dsa3d_status. Argument errors are found before any
 *    work is enqueued. A HIP launch error gives DSA3D_ERR_HIP. No C++
 *    exception crosses this boundary.
 *  - Calls on distinct streams may run concurrently if they share no output
 *    or workspace. The only mutable state is the opt-in, per-thread launch
 *    log (dsa3d_set_launch_log) and the per-GPU scratch array of
 *    dsa3d_backward_noalloc.
 */
#ifndef DSA3D_H
#define DSA3D_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DSA3D_OK = 0,
    DSA3D_ERR_INVALID_ARG = -1,  /* bad shape, window, P, dilation, null pointer */
    DSA3D_ERR_UNSUPPORTED = -2,  /* valid but not built: head_dim, P, dtype */
    DSA3D_ERR_MISALIGNED = -3,   /* a base pointer is not 16-byte aligned */
    DSA3D_ERR_WORKSPACE = -4,    /* workspace missing or too small */
    DSA3D_ERR_HIP = -5           /* the HIP runtime reported an error */
} dsa3d_status;

typedef enum { DSA3D_F32 = 0, DSA3D_BF16 = 1 } dsa3d_dtype;

typedef struct dsa3d_desc {
    int64_t B, T, H, W;           /* token grid; each >= 1; B*T*H*W < 2^31 */
    int32_t heads, head_dim;      /* C = heads * head_dim; head_dim a power of two in [8, 256] */
    int32_t kt, kh, kw;           /* window shape; each odd, >= 1 */
    int32_t P;                    /* sampling points; must equal kt*kh*kw, <= 1024 */
    int32_t dil_t, dil_h, dil_w;  /* window dilation, each >= 1 (it spaces the
                                     reference grid; offsets are not scaled) */
    int32_t dtype;                /* dsa3d_dtype of every tensor except lse/dW/dbias */
    float scale;                  /* logit scale; 0 means 1/sqrt(head_dim) */
    int32_t deterministic;        /* backward: 1 = bitwise-reproducible dk/dv */
} dsa3d_desc;

/* Which call a workspace is for. */
typedef enum {
    DSA3D_WS_FORWARD = 0,
    DSA3D_WS_BACKWARD = 1,
    DSA3D_WS_PROJ_BACKWARD = 2,
    DSA3D_WS_DWCONV_BACKWARD = 3,
    DSA3D_WS_BACKWARD_FIXED = 4    /* dsa3d_backward with offsets == NULL */
} dsa3d_ws_kind;

/* Library version (major*10000 + minor*100 + patch). */
int dsa3d_version(void);

/* Human-readable name of a status code (static storage). */
const char* dsa3d_status_string(int status);

/* Check a descriptor on the host; no GPU is touched. Returns DSA3D_OK or the
 * error that every compute call would return for it. */
int dsa3d_validate(const dsa3d_desc* desc);

/* Recommended workspace bytes for `kind` (0 if none is needed; 0 also for an
 * invalid descriptor). The backward accepts any workspace of at least its
 * one-head minimum (dsa3d_workspace_min) and runs fewer passes over the heads
 * the more it gets; the recommended size caps one pass at 16 GiB. */
size_t dsa3d_workspace_size(const dsa3d_desc* desc, int kind);
size_t dsa3d_workspace_min(const dsa3d_desc* desc, int kind);

/* Offset projection: offsets[n, f] = sum_c q[n, c] * w[f, c] + bias[f], with n
 * over the B*T*H*W tokens, c over C = heads*head_dim and f = (head*P + p)*3 +
 * axis over F = heads*P*3 -- a Linear layer (weight [F, C], row-major) applied
 * to each token's full query row [MegaSlide-DiT, §5.3: pointwise convolution;
 * Dutch summary, Implementation: a linear layer]. bias may be NULL. The
 * result is accumulated in float32 and rounded once to the output dtype. */
int dsa3d_offset_proj_forward(const dsa3d_desc* desc, const void* q, const void* w,
                              const void* bias, void* offsets, void* stream);

/* Forward. Writes out and lse (log of the softmax denominator, float32, used
 * by the backward). No workspace is needed.
 * offsets == NULL selects the fixed window: every offset is zero, so each
 * sample is the reference token itself and the operator is fixed local
 * attention over the dilated window [MegaSlide-DiT, §9.1: offsets frozen at
 * zero, a fixed (3,7,7) window]; the result equals the general path with a
 * zero offsets tensor (bf16 rows of 32-256 channels with k_w <= 17 and no
 * dilation along w are summed on the matrix cores, in another order, so they
 * agree to rounding), without reading offsets or interpolating. */
int dsa3d_forward(const dsa3d_desc* desc, const void* q, const void* k, const void* v,
                  const void* offsets, void* out, float* lse, void* stream);

/* Backward for a loss L given dout = dL/dout: the gradients the pages' own
 * implementation takes by autograd through grid_sample, softmax and the
 * weighted sum [MegaSlide-DiT, §5.3 Implementation considerations], i.e. of
 * the definition above with the derivative of the trilinear weights taken
 * inside the sample's cell (from the right at an exact integer position).
 * Writes dq (the attention path's
 * share), dk, dv and doffsets (dL/doffsets); every element of the four
 * outputs is overwritten. `out` and `lse` are the forward's outputs for the
 * same inputs. No atomic operation touches a gradient: each query's dq and
 * doffsets are summed by the thread group that owns the query, and each key's
 * dk/dv row by the group that owns the key, which streams the records of the
 * samples whose trilinear cell has that key as a corner (the samples are
 * filed by base cell in the workspace) and sums their contributions in
 * float32 before one rounding to the output dtype. With deterministic = 1 the
 * records of every cell are sorted by sample, so every sum runs in a fixed
 * order and all outputs are bitwise identical from run to run and for any
 * workspace size; with deterministic = 0 the order of dk/dv terms, and so
 * their last bits, may vary.
 * The workspace (at least dsa3d_workspace_min(desc, DSA3D_WS_BACKWARD), the
 * size of a pass over one head) holds the index; a larger one lets one pass
 * cover more heads. A single head whose B*T*H*W*P samples, or whose
 * B*(T+1)*(H+1)*(W+1) cells, reach 2^32 gives DSA3D_ERR_UNSUPPORTED.
 * offsets == NULL (and doffsets == NULL; one without the other is
 * DSA3D_ERR_INVALID_ARG) is the fixed window of dsa3d_forward: no offset
 * gradient; each key walks the queries whose window contains it, so dk and dv
 * are summed in a fixed order for either value of `deterministic` (bf16 rows
 * of 32-128 channels with k_w <= 17 and no dilation along w run these sums on
 * the matrix cores, also in a fixed order); the workspace
 * (DSA3D_WS_BACKWARD_FIXED) holds two floats per (token, head). */
int dsa3d_backward(const dsa3d_desc* desc, const void* q, const void* k, const void* v,
                   const void* offsets, const void* out, const float* lse, const void* dout,
                   void* dq, void* dk, void* dv, void* doffsets,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Size of the fixed scratch array of dsa3d_backward_noalloc, per GPU, in bytes. */
#define DSA3D_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation: the
 * backward of dsa3d_backward (same arguments, outputs, errors and
 * determinism) without a workspace argument. Its scratch memory is a fixed
 * array of DSA3D_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, which
 * that GPU holds from the library's load until the process ends; the call
 * itself allocates nothing (no hipMalloc, hipFree or allocating library
 * routine). A problem whose one-head pass needs more than the array
 * (dsa3d_workspace_min with DSA3D_WS_BACKWARD, or DSA3D_WS_BACKWARD_FIXED
 * when offsets is NULL, above the limit) returns DSA3D_ERR_WORKSPACE before
 * any work is enqueued; otherwise the heads are processed in as many passes
 * as the array requires. `stream` must belong to the current device. Every
 * call on a GPU shares that GPU's array and leaves its contents there: calls
 * that overlap in time on one GPU (on different streams, or from different
 * host threads) race on it and give wrong results, so serialise them. */
int dsa3d_backward_noalloc(const dsa3d_desc* desc, const void* q, const void* k, const void* v,
                           const void* offsets, const void* out, const float* lse, const void* dout,
                           void* dq, void* dk, void* dv, void* doffsets, void* stream);

/* Backward of the offset projection for doffsets [N, F]:
 *   dq_accum[n, c] += sum_f doffsets[n, f] * w[f, c]   (added to the dtype tensor,
 *                                                      one rounding per element)
 *   dw[f, c]  = sum_n doffsets[n, f] * q[n, c]          (float32, overwritten)
 *   dbias[f]  = sum_n doffsets[n, f]                    (float32, overwritten; may be NULL)
 * dw and dbias are summed in a fixed order (bitwise reproducible). The
 * workspace (DSA3D_WS_PROJ_BACKWARD) holds split-sum partials and, for bf16,
 * a transposed copy of w. */
int dsa3d_offset_proj_backward(const dsa3d_desc* desc, const void* q, const void* w,
                               const void* doffsets, void* dq_accum, float* dw, float* dbias,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Depthwise 3-D convolution of the offset network, before its pointwise layer
 * [MegaSlide-DiT, §5.3 Implementation considerations: nn.Conv3d with groups
 * equal to the hidden size; Dutch and French summaries, Implementation: a
 * lightweight depthwise 3-D convolution]. The pages give no kernel size; this
 * is 3x3x3, stride 1, zero padding 1, per channel c of q [B,T,H,W,C]
 * (C = heads*head_dim), as a cross-correlation:
 *   y[b,t,h,w,c] = bias[c] + sum_{i,j,k in 0..2} wt[c,i,j,k] * q[b,t+i-1,h+j-1,w+k-1,c]
 * with q read as zero outside the grid. wt is [C,3,3,3] (torch's [C,1,3,3,3])
 * in the run dtype, bias [C] in the run dtype or NULL; y [B,T,H,W,C] in the run
 * dtype, accumulated in float32 and rounded once. All device pointers, 16-byte
 * aligned; asynchronous on `stream`. */
int dsa3d_dwconv_forward(const dsa3d_desc* desc, const void* q, const void* wt, const void* bias,
                         void* y, void* stream);

/* Backward of dsa3d_dwconv_forward for dy = dL/dy [B,T,H,W,C]:
 *   dq_accum[b,t,h,w,c] += sum_{i,j,k} wt[c,i,j,k] * dy[b,t-i+1,h-j+1,w-k+1,c]  (one rounding)
 *   dwt[c,i,j,k] = sum over all tokens of dy[tok,c] * q[tok + (i-1,j-1,k-1), c]  (float32, overwritten)
 *   dbias[c]     = sum over all tokens of dy[tok,c]                            (float32, overwritten; may be NULL)
 * dwt and dbias are summed in a fixed order (bitwise reproducible); the
 * workspace (DSA3D_WS_DWCONV_BACKWARD) holds their split partials. */
int dsa3d_dwconv_backward(const dsa3d_desc* desc, const void* q, const void* wt, const void* dy,
                          void* dq_accum, float* dwt, float* dbias,
                          void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Hybrid attention: G global tokens combined with the local 3D-DSA samples
 * [MegaSlide-DiT, §11 Limitations and Discussion, future work (i): sparse
 * global tokens with local 3D-DSA]. The pages only name the idea; the reading
 * here: every query of a (batch item, head) attends in ONE softmax to its P
 * samples and to the G global rows gk[b, g, head, :], gv[b, g, head, :]
 * (shared by all queries of that batch item and head; the caller decides what
 * they are: learned tokens, pooled summaries, a strided subset of the grid):
 *   s_g = scale * <q, gk_g>;  a = softmax over the P + G logits;
 *   o = sum_p a_p v_p + sum_g a_g gv_g;  lse = log of the joint denominator.
 * gk, gv, dgk, dgv: [B, G, heads, head_dim] in the run dtype; 1 <= G <= 1024.
 * offsets == NULL: the fixed window as for dsa3d_forward/dsa3d_backward.
 * ------------------------------------------------------------------------- */

/* Forward: writes out and lse of the joint softmax (lse float32). */
int dsa3d_forward_hybrid(const dsa3d_desc* desc, const void* q, const void* k, const void* v, const void* offsets,
                         int32_t G, const void* gk, const void* gv, void* out, float* lse, void* stream);

/* Workspace bytes of dsa3d_backward_hybrid: the backward's own (the recommended
 * size, for `kind` DSA3D_WS_BACKWARD or DSA3D_WS_BACKWARD_FIXED) or the global
 * rows' partial sums, whichever is larger; the _min variant uses the
 * backward's one-head minimum. 0 for an invalid descriptor or G. */
size_t dsa3d_hybrid_workspace_size(const dsa3d_desc* desc, int32_t G, int kind);
size_t dsa3d_hybrid_workspace_min(const dsa3d_desc* desc, int32_t G, int kind);

/* Backward of dsa3d_forward_hybrid for dout: dq, dk, dv, doffsets as for
 * dsa3d_backward (of the joint softmax), plus dgk = scale * sum over the
 * queries of ds_g q and dgv = sum over the queries of a_g dout (each summed in
 * float32 in a fixed order and rounded once). `out` and `lse` are the hybrid
 * forward's. Deterministic mode as for dsa3d_backward; dq, dgk and dgv are
 * reproducible in both modes. */
int dsa3d_backward_hybrid(const dsa3d_desc* desc, const void* q, const void* k, const void* v, const void* offsets,
                          const void* out, const float* lse, const void* dout, int32_t G, const void* gk,
                          const void* gv, void* dq, void* dk, void* dv, void* doffsets, void* dgk, void* dgv,
                          void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * The transformer block around the operator. The pages wrap their attention in
 * layer normalisation and residual connections as usual, and its queries, keys
 * and values come from (and its output goes through) dense projections
 * [MegaSlide-DiT, §5.3 Implementation considerations]. These calls give that
 * block without leaving the library: per token,
 *   h = LayerNorm(x); q|k|v = h.W_qkv^T + b_qkv; o = 3D-DSA(q, k, v, offsets);
 *   y = x + o.W_out^T + b_out
 * (each of q, k, v is one dsa3d_linear_forward with its [C, C] slice of W_qkv;
 * the residual add is the output projection's epilogue). They take plain
 * sizes instead of a descriptor: rows M (tokens), widths N and K; tensors are
 * dense row-major device tensors of `dtype` (DSA3D_F32 or DSA3D_BF16) unless
 * stated, 16-byte aligned, owned by the caller; calls are asynchronous on
 * `stream` and allocate nothing; errors as for every call.
 * ------------------------------------------------------------------------- */

/* Layer normalisation over the last axis of x [M, N]:
 *   mean = sum(x)/N, var = sum((x - mean)^2)/N, rstd = 1/sqrt(var + eps),
 *   y = (x - mean) * rstd * gamma + beta
 * gamma/beta [N] (NULL: 1 and 0). stats [M, 2] float32 receives (mean, rstd)
 * per row for the backward. Float32 arithmetic, one rounding per element of y.
 * Needs N % 8 == 0, N <= 4096, eps > 0 (DSA3D_ERR_UNSUPPORTED /
 * DSA3D_ERR_INVALID_ARG otherwise). y may not alias x. */
int dsa3d_layernorm_forward(int dtype, int64_t M, int64_t N, float eps, const void* x, const void* gamma,
                            const void* beta, void* y, float* stats, void* stream);

/* Workspace bytes of dsa3d_layernorm_backward (split partials of dgamma/dbeta). */
size_t dsa3d_layernorm_workspace_size(int64_t M, int64_t N);

/* Backward of dsa3d_layernorm_forward for dy = dL/dy [M, N], with the forward's
 * stats: xh = (x - mean)*rstd, g = dy*gamma,
 *   dx = dres + rstd * (g - mean(g) - xh * mean(g*xh))   (one rounding)
 *   dgamma = sum over rows of dy*xh, dbeta = sum over rows of dy
 *   (float32 [N], overwritten, either may be NULL; summed in a fixed order).
 * dres [M, N] is the gradient reaching x by another path (the block's residual
 * connection), NULL for none; it may be dx itself (add in place). */
int dsa3d_layernorm_backward(int dtype, int64_t M, int64_t N, const void* x, const void* gamma, const float* stats,
                             const void* dy, const void* dres, void* dx, float* dgamma, float* dbeta,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Linear layer y[M, N] = x[M, K] . w[N, K]^T + bias[N] (+ residual[M, N]), on
 * the matrix cores for bf16, accumulated in float32 and rounded once. bias and
 * residual may be NULL; residual may be y itself (an in-place add). Sizes each
 * in [1, 2^31). */
int dsa3d_linear_forward(int dtype, int64_t M, int64_t N, int64_t K, const void* x, const void* w,
                         const void* bias, const void* residual, void* y, void* stream);

/* Workspace bytes of dsa3d_linear_backward (split partials of dw and dbias
 * and, for bf16, w transposed). */
size_t dsa3d_linear_workspace_size(int dtype, int64_t M, int64_t N, int64_t K);

/* Backward of dsa3d_linear_forward for dy = dL/dy [M, N]:
 *   dx[M, K] = dres + dy . w   (one rounding; dres [M, K] NULL for none, or dx
 *                               itself to add in place)
 *   dw[N, K] = dy^T . x (float32, overwritten), dbias[N] = column sums of dy
 *   (float32, overwritten, may be NULL); dw and dbias summed in a fixed order. */
int dsa3d_linear_backward(int dtype, int64_t M, int64_t N, int64_t K, const void* x, const void* w, const void* dy,
                          const void* dres, void* dx, float* dw, float* dbias, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Test hook: the integer base corner floor(pos) and the float32 fraction f of
 * every sample, both [B,T,H,W,heads,P,3] (int32, float32). A sample whose
 * position is NaN, infinite or |pos| >= 2^30 reports base INT32_MIN and f 0. */
int dsa3d_debug_geometry(const dsa3d_desc* desc, const void* offsets, int32_t* base,
                         float* frac, void* stream);

/* Profiling aid: per-launch HIP events.
 *
 * Kernels of libdsa3d, as reported in dsa3d_launch_log.kernel[]: */
typedef enum {
    DSA3D_K_PROJ_FORWARD = 1,   /* projection GEMM */
    DSA3D_K_FORWARD = 2,        /* fused sample + softmax + aggregate */
    DSA3D_K_BWD_QUERY = 3,      /* backward per query: dq, doffsets, sample records by cell */
    DSA3D_K_BWD_KEY = 4,        /* backward per key: dk, dv */
    DSA3D_K_FILL = 5,           /* workspace clearing */
    DSA3D_K_PROJ_BWD_DQ = 6,    /* dq += doffsets . W */
    DSA3D_K_PROJ_BWD_DW = 7,    /* split dW = doffsets^T . q */
    DSA3D_K_SPLIT_SUM = 8,      /* fixed-order sum of split partials */
    DSA3D_K_COLSUM = 9,         /* split column sums for dbias */
    DSA3D_K_GEOMETRY = 10,      /* test hook */
    DSA3D_K_BWD_SCAN = 11,      /* backward: bucket starts (3 small kernels, one entry) */
    DSA3D_K_BWD_COUNT = 12,     /* backward: samples per base cell */
    DSA3D_K_BWD_SORT = 13,      /* backward, deterministic: bucket sort (2 kernels, one entry) */
    DSA3D_K_TRANSPOSE = 14,     /* projection backward: W transposed for the dq product */
    DSA3D_K_DWCONV = 15,        /* depthwise convolution forward */
    DSA3D_K_DWCONV_WGRAD = 16,  /* depthwise convolution backward: split weight and bias sums */
    DSA3D_K_DWCONV_DQ = 17,     /* depthwise convolution backward: dq += conv with the mirrored kernel */
    DSA3D_K_LAYERNORM = 18,     /* layer normalisation forward */
    DSA3D_K_LAYERNORM_BWD = 19, /* layer normalisation backward: dx and partial dgamma/dbeta */
    DSA3D_K_LINEAR_FORWARD = 20,/* linear layer y = x.w^T + bias (+ residual) */
    DSA3D_K_LINEAR_BWD_DX = 21, /* linear layer backward: dx (+)= dy.w */
    DSA3D_K_LINEAR_BWD_DW = 22, /* linear layer backward: split dw = dy^T.x */
    DSA3D_K_HYBRID_FORWARD = 23,   /* hybrid attention: global rows merged into the local softmax */
    DSA3D_K_HYBRID_BWD_QUERY = 24, /* hybrid backward: the global rows' share of dq */
    DSA3D_K_HYBRID_BWD_ROWS = 25   /* hybrid backward: partial dGK/dGV per slab of queries */
} dsa3d_kernel;

typedef struct dsa3d_launch_log {
    int32_t capacity;  /* entries available in kernel[], start[] and stop[] */
    int32_t count;     /* entries used; the library increments it */
    int32_t* kernel;   /* dsa3d_kernel of each entry */
    void** start;      /* hipEvent_t handles created by the caller with timing */
    void** stop;       /* enabled; recorded on the launch's stream */
} dsa3d_launch_log;

/* While `log` is set on the calling host thread, every kernel that a libdsa3d
 * call made on this thread launches is bracketed by hipEventRecord(start[i])
 * and hipEventRecord(stop[i]) on the call's stream, for i = count, count+1, ...
 * up to capacity (launches beyond it are not logged). NULL stops logging.
 * The log is only read and written by calls on the same thread; it must stay
 * valid while set. Returns DSA3D_OK, or DSA3D_ERR_INVALID_ARG for a log with
 * capacity > 0 and a NULL array. */
int dsa3d_set_launch_log(dsa3d_launch_log* log);

#ifdef __cplusplus
}
#endif

#endif /* DSA3D_H */

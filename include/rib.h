/*
 * rib.h -- C ABI of the MI355X (gfx950) library for RIB window attention with
 * the CLA output gate.
 *
 * Source of the method: "Rank-Factorized Implicit Neural Bias: Scaling
 * Super-Resolution Transformer with FlashAttention" (arXiv 2603.06738), as
 * summarised on gist.science (French and Italian pages, methodology part A
 * "Rank-factorized Implicit Neural Bias" and part B "Convolutional Local
 * Attention") and on the omica.com.cn explainer (section 2.2 "RIB core
 * design", section 2.3 "CLA", section 5.2 "caching the positional factors").
 *
 * Conventions shared by every entry point:
 *   - All pointers are device pointers (memory from hipMalloc or a framework
 *     allocator on the current device) unless stated otherwise.  The caller
 *     owns every buffer; the library allocates no device or host memory and
 *     keeps no state apart from a thread-local error message and the fixed
 *     per-device array of rib_encode_backward_noalloc (with its looked-up
 *     address per device); the number of compute units, which sizes some
 *     grids, is queried on every call.
 *   - Calls are asynchronous: work is enqueued on `stream` (a hipStream_t
 *     passed as void*, NULL = the null stream) and the call returns.  RIB_OK
 *     means "validated and enqueued"; a fault inside a kernel surfaces at the
 *     caller's next synchronisation.
 *   - Arguments are validated before anything is launched.  On any error no
 *     work is enqueued, outputs are untouched, and rib_last_error() describes
 *     the problem.  Validation makes no HIP call, so it also works on a host
 *     without a GPU.
 *   - Feature maps are flat NHWC: element (b, y, x, c) of a [B][H][W][C] array
 *     sits at ((b*H + y)*W + x)*C + c with C = heads*dh; head h owns channels
 *     [h*dh, (h+1)*dh).
 */
#ifndef RIB_H
#define RIB_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RIB_OK = 0,
  RIB_ERR_INVALID_ARG = 1, /* null pointer, size < 1, window < 2, misalignment, aliasing */
  RIB_ERR_UNSUPPORTED = 2, /* valid request outside the compiled variants (never a slow fallback) */
  RIB_ERR_HIP = 3          /* the HIP runtime refused a launch; see rib_last_error() */
} rib_status;

typedef enum { RIB_F32 = 0, RIB_BF16 = 1 } rib_dtype;

/*
 * rib_encode -- positional factors of one window size (explainer section 2.2:
 * coordinate encoding layer, implicit neural field; gist.science part A,
 * mechanism steps 1-2).
 *
 * For every in-window position n = iy*window + ix (0 <= n < window^2):
 *   c   = (u(iy), u(ix)),  u(k) = float32((2k - (window-1)) / (window-1)),
 *         i.e. coordinates in [-1, 1] with both ends included;
 *   r   = [c_y, c_x, then for i = 0..L-1: sin(2^i c_y), sin(2^i c_x),
 *          cos(2^i c_y), cos(2^i c_x)]                    (2 + 4L features);
 *   h   = ReLU(r W_h + b_h)                                (hidden values);
 *   qp[n] = h Wp_q,  kp[n] = h Wp_k                        (R values each).
 *
 * weights : device, float32, packed row-major, y = x W convention:
 *           W_h[2+4L][hidden] | b_h[hidden] | Wp_q[hidden][R] | Wp_k[hidden][R].
 * qp, kp  : device, float32, [window*window][R] row-major, written.
 *           Compute once per window size and reuse them for every window,
 *           head and image (explainer section 5.2 caches them).
 * Limits  : 2 <= window <= 128, 0 <= L <= 16, 1 <= hidden <= 256, 1 <= R <= 64;
 *           all pointers 4-byte aligned; qp and kp must not overlap weights
 *           or each other.  Arithmetic is float32 (sinf/cosf, fp32 sums).
 */
rib_status rib_encode(int window, int L, int hidden, int R, const float* weights, float* qp,
                      float* kp, void* stream);

/*
 * rib_window_attn -- RIB window attention with the CLA gate (gist.science
 * part A mechanism steps 3-4 and part B; explainer section 2.2 "attention
 * rewrite" and section 2.3):
 *
 *   per image b, window (wy, wx) of window x window tokens, head h:
 *     S = Qc Kc^T / sqrt(dh) + Qp Kp^T / sqrt(R)
 *       = [Qc/sqrt(dh), Qp/sqrt(R)] [Kc, Kp]^T        (one contraction)
 *     O = (softmax(S) V) * sigmoid(G)                 (element-wise gate)
 *
 * The window grid is anchored at (0,0).  A window holds only the real tokens
 * (y < H, x < W): when H or W is not a multiple of `window`, the missing
 * positions are masked out of the softmax and produce no output.  Qp/Kp are
 * indexed by in-window position n = (y mod window)*window + (x mod window)
 * and are shared by all heads.
 *
 * qc, kc, v, g : device, [B][H][W][heads*dh] of `dtype` (read).
 * o            : device, same shape and dtype (written); must not overlap any
 *                input.
 * qp, kp       : device, float32 [window*window][R] from rib_encode (read).
 * dtype        : RIB_F32 -- fp32 in, fp32 arithmetic, fp32 out;
 *                RIB_BF16 -- bf16 in and out, bf16 matrix-core products with
 *                fp32 accumulation and fp32 softmax.
 * Limits       : 2 <= window <= 128; B*H*W*heads*dh < 2^31;
 *                RIB_F32: dh <= 64, R <= 64;
 *                RIB_BF16: (dh, R) in {(8,8), (16,16), (30,16), (32,16),
 *                (16,32), (30,32)} (others return RIB_ERR_UNSUPPORTED).
 *                qc, kc, v, g, o 4-byte aligned (dword accesses); qp, kp
 *                8-byte aligned (float pairs).
 */
rib_status rib_window_attn(const void* qc, const void* kc, const void* v, const void* g,
                           const float* qp, const float* kp, void* o, int B, int H, int W,
                           int heads, int dh, int R, int window, rib_dtype dtype, void* stream);

/*
 * rib_window_attn_heads -- rib_window_attn with one positional pair per head
 * instead of one shared pair: qp and kp are float32 [heads][window*window][R]
 * (for example, rib_encode run once per head with that head's weights).  The
 * pages give Qp, Kp without a head index (explainer section 2.2 attention
 * rewrite), which rib_window_attn reads as one shared pair; this entry point
 * is the per-head alternative.  Everything else (layouts, dtypes, limits,
 * errors) is as for rib_window_attn.
 */
rib_status rib_window_attn_heads(const void* qc, const void* kc, const void* v, const void* g,
                                 const float* qp, const float* kp, void* o, int B, int H, int W,
                                 int heads, int dh, int R, int window, rib_dtype dtype, void* stream);

/*
 * rib_window_attn_multi -- several independent rib_window_attn calls in as
 * few kernel launches as possible.  The window size of the SST blocks cycles
 * through 16, 32 and 64 (explainer section 3.2 "cyclic window strategy"); a
 * caller holding independent work at several points of that cycle (other
 * images, other streams of a batch, or the three window sizes of one shape)
 * passes the calls together, and the library runs them side by side:
 * RIB_BF16 calls that share (dh, R) take one launch per workgroup size and
 * per 8 calls, largest windows first: calls on the 256-thread kernels share
 * one launch; only the (dh, R) shapes (32, 16), (16, 32) and (30, 32) run
 * windows of more than 2,048 tokens (4,096 when the call's 256-query
 * workgroups number more than three per compute unit) on the 512-thread
 * tiled kernel, in a launch of their own.  The 16/32/64 cycle is one launch
 * for (dh, R) = (16, 16) and (30, 16).
 * RIB_F32 calls run one after another.  Each call's output is bit-identical to
 * that of rib_window_attn with the same arguments.
 *
 * calls : host array of n call descriptions (read; not kept after return);
 *         each field as the argument of the same name of rib_window_attn
 *         (one shared (qp, kp) pair per call, window sizes may differ).
 * n     : 1 <= n <= RIB_MAX_CALLS.
 * Errors: every call is validated as rib_window_attn validates its arguments,
 *         and no call's output may overlap an argument of another call;
 *         on any error nothing is launched.
 */
#define RIB_MAX_CALLS 16
typedef struct {
  const void* qc;
  const void* kc;
  const void* v;
  const void* g;
  const float* qp;
  const float* kp;
  void* o;
  int B, H, W, heads, dh, R, window;
} rib_attn_call;
rib_status rib_window_attn_multi(int n, const rib_attn_call* calls, rib_dtype dtype, void* stream);

/*
 * rib_window_attn_train -- rib_window_attn that also writes the row
 * log-sum-exp the backward needs (the training iteration of explainer
 * section 4.1: forward, then rib_window_attn_backward):
 *   lse[b][y][x][h] = log sum_j exp(s_ij)   (natural log, over the real keys j
 *                                           of the query's window, head h)
 * lse : device, float32 [B][H][W][heads] (written); must not overlap any other
 *       argument.  Every other argument, limit and error as rib_window_attn
 *       (one shared (qp, kp) pair).
 */
rib_status rib_window_attn_train(const void* qc, const void* kc, const void* v, const void* g,
                                 const float* qp, const float* kp, void* o, float* lse, int B, int H, int W,
                                 int heads, int dh, int R, int window, rib_dtype dtype, void* stream);

/*
 * rib_attn_supported -- RIB_OK if rib_window_attn has a compiled variant for
 * (dh, R, window, dtype), RIB_ERR_UNSUPPORTED if not, RIB_ERR_INVALID_ARG for
 * nonsensical values.  Launches nothing.
 */
rib_status rib_attn_supported(int dh, int R, int window, rib_dtype dtype);

/*
 * rib_cla_gate -- the gating map of Convolutional Local Attention (explainer
 * section 2.3: G = PWConv(DWConv3x3(X)), a depth-wise separable convolution of
 * the block input; gist.science summaries part B: depth-wise 3x3, then
 * point-wise 1x1):
 *   D[b,y,x,c] = dw_b[c] + sum_{dy,dx in {-1,0,1}} X[b,y+dy,x+dx,c] dw_w[c][dy+1][dx+1]
 *                (positions outside the map are zero: same-size output)
 *   G[b,y,x,o] = pw_b[o] + sum_c D[b,y,x,c] pw_w[c][o]
 * G is the `g` argument of rib_window_attn.
 *
 * x      : device, [B][H][W][C] of `dtype` (read).
 * g      : device, same shape and dtype (written); must not overlap x or the
 *          weights.
 * dw_w   : device, float32 [C][3][3]; dw_b: device, float32 [C].
 * pw_w   : device, float32 [C][C], row = input channel (y = x W); pw_b: [C].
 * dtype  : RIB_F32 -- fp32 throughout; RIB_BF16 -- bf16 maps; the depth-wise
 *          stencil on bf16 dot products (taps rounded to bf16, exact products,
 *          fp32 sums starting from the fp32 bias), D rounded to bf16; the
 *          point-wise product on bf16 matrix cores (weights rounded to bf16)
 *          with fp32 accumulation from the bias; G rounded to bf16.
 * Limits : C even, 2 <= C <= 256; B*H*W*C < 2^31; pointers 4-byte aligned.
 */
rib_status rib_cla_gate(const void* x, const float* dw_w, const float* dw_b, const float* pw_w,
                        const float* pw_b, void* g, int B, int H, int W, int C, rib_dtype dtype,
                        void* stream);

/*
 * rib_window_attn_backward -- gradients of rib_window_attn for an upstream
 * gradient dO: the backward half of the training iteration the explainer
 * times (section 4.1), by the chain rule of the forward above (explainer
 * sections 2.2 and 2.3).  With sg = sigmoid(G), A = softmax(S) V, O = A * sg:
 *   dG = dO * O * (1 - sg)            dA = dO * sg
 *   D_i = dO_i . O_i                  dS_ij = P_ij (dA_i . V_j - D_i)
 *   dQc = dS Kc / sqrt(dh)            dKc = dS^T Qc / sqrt(dh)
 *   dV  = P^T dA
 *   dqp[n] = sum over images, windows, heads of the row of dS Kp / sqrt(R)
 *            at in-window index n; dkp[n] likewise from dS^T Qp / sqrt(R).
 * P = exp(S - lse) is recomputed from the inputs and the forward's row
 * log-sum-exp; O is the forward's output, used only for D and dG.
 *
 * qc, kc, v, g, o, dout : device, [B][H][W][heads*dh] of `dtype` (read);
 *                         o and lse from rib_window_attn_train on the same
 *                         inputs.
 * lse                   : device, float32 [B][H][W][heads] (read).
 * qp, kp                : device, float32 [window*window][R] (one shared pair).
 * dqc, dkc, dv, dg      : device, like qc (written).
 * dqp, dkp              : device, float32 [window*window][R] (written, not
 *                         accumulated into).
 * workspace             : device, at least
 *                         rib_window_attn_backward_workspace(...) bytes,
 *                         16-byte aligned; the library keeps nothing in it
 *                         between calls.
 * dtype                 : RIB_F32 or RIB_BF16 (bf16 storage, fp32 arithmetic).
 * Every output and the workspace must be disjoint from every other buffer.
 * Limits : window <= 128, dh <= 64, R <= 64; B*H*W*heads*max(dh, R) < 2^31.
 * Alignment: maps, lse, dqp, dkp 4 bytes (dword accesses); qp, kp 8 bytes
 *          (float pairs); the workspace 16 bytes (its packed operand images
 *          are copied into LDS and read in 16-byte pieces).
 */
size_t rib_window_attn_backward_workspace(int B, int H, int W, int heads, int dh, int R, int window,
                                          rib_dtype dtype);
rib_status rib_window_attn_backward(const void* qc, const void* kc, const void* v, const void* g,
                                    const float* qp, const float* kp, const void* o, const float* lse,
                                    const void* dout, void* dqc, void* dkc, void* dv, void* dg, float* dqp,
                                    float* dkp, void* workspace, size_t workspace_bytes, int B, int H, int W,
                                    int heads, int dh, int R, int window, rib_dtype dtype, void* stream);

/*
 * rib_window_attn_heads_train / rib_window_attn_heads_backward -- the training
 * forward and the backward with one positional pair per head (the per-head
 * reading of the explainer's section 2.2 attention rewrite, as in
 * rib_window_attn_heads): qp and kp are float32 [heads][window*window][R], and
 * so are dqp and dkp, whose head h sums over the images and windows of that
 * head only.  Every other argument, layout, limit, workspace size
 * (rib_window_attn_backward_workspace) and error as rib_window_attn_train and
 * rib_window_attn_backward.  The encoder gradient of head h's tables is
 * rib_encode_backward on dqp[h], dkp[h] with that head's weights.
 */
rib_status rib_window_attn_heads_train(const void* qc, const void* kc, const void* v, const void* g,
                                       const float* qp, const float* kp, void* o, float* lse, int B, int H, int W,
                                       int heads, int dh, int R, int window, rib_dtype dtype, void* stream);
rib_status rib_window_attn_heads_backward(const void* qc, const void* kc, const void* v, const void* g,
                                          const float* qp, const float* kp, const void* o, const float* lse,
                                          const void* dout, void* dqc, void* dkc, void* dv, void* dg,
                                          float* dqp, float* dkp, void* workspace, size_t workspace_bytes, int B,
                                          int H, int W, int heads, int dh, int R, int window, rib_dtype dtype,
                                          void* stream);

/*
 * rib_encode_backward -- gradient of the packed encoder weights (layout of
 * rib_encode) for upstream dqp, dkp (explainer section 2.2, the coordinate
 * encoder and the two rank heads; the ReLU derivative at 0 is 0):
 *   dWp_q = sum_n h_n (x) dqp_n     dWp_k = sum_n h_n (x) dkp_n
 *   dpre_n = (dqp_n Wp_q^T + dkp_n Wp_k^T) * [pre_n > 0]
 *   dW_h = sum_n r_n (x) dpre_n     db_h = sum_n dpre_n
 * weights, dqp, dkp : device float32 (read); dweights: device float32, same
 * length as weights (written).  workspace: device, at least
 * rib_encode_backward_workspace(...) bytes.  Limits as rib_encode.
 */
size_t rib_encode_backward_workspace(int window, int L, int hidden, int R);
rib_status rib_encode_backward(int window, int L, int hidden, int R, const float* weights, const float* dqp,
                               const float* dkp, float* dweights, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * rib_encode_backward_noalloc -- rib_encode_backward for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving or
 * training loops, harnesses that forbid hipMalloc.  Same arguments, layouts,
 * limits and errors as rib_encode_backward, without the workspace: the
 * partial gradients go to a fixed 4 MiB array that the library holds on each
 * device it runs on until the process ends.  It calls no hipMalloc, hipFree
 * or allocating library routine; the first call on a device looks up that
 * device's array once.  The workspace holds min(ceil(window^2 / 16),
 * 2^20 / weights) partial rows, so every size rib_encode_backward takes fits
 * (at most 49,920 weights); a weight count beyond 2^20 floats would be
 * refused with RIB_ERR_UNSUPPORTED.  When the row count equals
 * ceil(window^2 / 16) (window <= 59 for the 4,800-weight encoder) the result
 * is bit-identical to rib_encode_backward's; otherwise a workgroup sums
 * several 16-position chunks and the summation order differs.  Calls on one
 * device share the array: two calls whose executions overlap on one device
 * (different streams, or host threads without ordering) race and give wrong
 * gradients; calls ordered on one stream are safe.
 */
rib_status rib_encode_backward_noalloc(int window, int L, int hidden, int R, const float* weights,
                                       const float* dqp, const float* dkp, float* dweights, void* stream);

/*
 * rib_ln_qkv -- the attention's input projection in an SST block (explainer
 * section 3.1: each block runs LayerNorm, then the RIB attention), per token:
 *   mu = mean_c x_c,  var = mean_c (x_c - mu)^2         (biased variance)
 *   xn_c = (x_c - mu) / sqrt(var + eps) * gamma_c + beta_c
 *   [q | k | v] = xn W + bias                           (y = x W, W [C][3C])
 * x, q, k, v : device, [B][H][W][C] of `dtype` (x read; q, k, v written) --
 *              q, k, v are the qc, kc, v arguments of rib_window_attn.
 * xn         : device, like x, or NULL; receives LN(X) (the gate producer's
 *              input in this reading of the block).
 * gamma, beta: device float32 [C]; w: device float32 [C][3C], columns Q | K | V;
 *              bias: device float32 [3C].
 * dtype      : RIB_F32 -- fp32 throughout.  RIB_BF16 -- LayerNorm in fp32,
 *              xn and W rounded to bf16, the product on bf16 matrix cores
 *              with fp32 accumulation, outputs rounded to bf16.
 * q may be NULL: Q is then not written (for rib_window_attn_lnq, which
 * computes it inside the attention).
 * Outputs must not overlap each other or any input.
 * Limits : C <= 256 (even for bf16); B*H*W*C < 2^30; pointers 16-byte
 *          aligned; 0 <= eps <= 1.
 */
rib_status rib_ln_qkv(const void* x, const float* gamma, const float* beta, const float* w, const float* bias,
                      void* q, void* k, void* v, void* xn, int B, int H, int W, int C, float eps, rib_dtype dtype,
                      void* stream);

/*
 * rib_window_attn_lnq -- rib_window_attn with the Q side of the block's input
 * projection fused into the attention (explainer section 3.1: LayerNorm, then
 * the RIB attention): Qc = LN(x) W_q + b_q is computed inside the kernel for
 * each query block and never stored; K and V come from rib_ln_qkv (whose q
 * may then be NULL).  The LayerNorm and the Q columns of w and bias are those
 * of rib_ln_qkv; the arithmetic folds the affine part into the weights:
 *   q_d = bf16( inv (sum_c x_c W'_cd - mu sum_c W'_cd) + b'_d ),
 *   W'_cd = bf16(gamma_c W_cd),  b'_d = bias_d + sum_c beta_c W_cd,
 * inv = 1/sqrt(var + eps); the statistics are fp32 sums of x and x^2 (the
 * bf16 products are exact), var = E[x^2] - mu^2; the product runs on bf16
 * matrix cores with fp32 accumulation.  q can therefore differ from rib_ln_qkv's
 * (which rounds LN(x) to bf16 before its product) by about one bf16 unit.
 * The attention is rib_window_attn's.
 * x          : device bf16 [B][H][W][heads*dh], the block input (read).
 * gamma, beta: device float32 [C]; w: device float32 [C][3C], columns
 *              Q | K | V; bias: device float32 [3C] (only Q's are read).
 * kc, v, g, qp, kp, o, B, H, W, heads, dh, R, window: as rib_window_attn.
 * Limits : RIB_BF16 only; (dh, R) in {(30, 16), (16, 16)}; heads*dh <= 192;
 *          0 <= eps <= 1; alignment and aliasing as rib_window_attn (x in
 *          place of qc), parameters 4-byte aligned and not overlapping o.
 * Always runs the 512-query tiled kernel, whatever the window size.
 */
rib_status rib_window_attn_lnq(const void* x, const float* gamma, const float* beta, const float* w,
                               const float* bias, const void* kc, const void* v, const void* g, const float* qp,
                               const float* kp, void* o, int B, int H, int W, int heads, int dh, int R, int window,
                               float eps, rib_dtype dtype, void* stream);

/*
 * Space-time windows for video (explainer section 6: the coordinate MLP takes
 * spatio-temporal coordinates and the attention windows become 3-D).
 *
 * rib_encode3d -- Qp, Kp float32 [frames*window*window][R] for windows of
 * `frames` frames x window x window.  Position n = (it*window + iy)*window + ix
 * has coordinates (c_t, c_y, c_x) on the float32 grid -1 + 2k/(n-1) of each
 * axis (c_t = 0 when frames == 1); features [c_t, c_y, c_x], then for each
 * frequency 2^i, i < L: sin t, sin y, sin x, cos t, cos y, cos x (3 + 6L).
 * weights: W_h[(3+6L)][hidden] | b_h | Wp_q[hidden][R] | Wp_k[hidden][R].
 * Limits: frames*window^2 <= 16384, window <= 128, L <= 16, hidden <= 256,
 * R <= 64.
 *
 * rib_window_attn3d -- rib_window_attn over [B][T][H][W][heads*dh] video maps
 * with windows of `frames` frames x window x window anchored at (0, 0, 0);
 * edge windows hold only their real tokens.  qp, kp from rib_encode3d.
 * Limits as rib_window_attn, with frames*window^2 <= 16384 and
 * B*T*H*W*heads*dh < 2^31.
 */
rib_status rib_encode3d(int frames, int window, int L, int hidden, int R, const float* weights, float* qp,
                        float* kp, void* stream);
rib_status rib_window_attn3d(const void* qc, const void* kc, const void* v, const void* g, const float* qp,
                             const float* kp, void* o, int B, int T, int H, int W, int heads, int dh, int R,
                             int frames, int window, rib_dtype dtype, void* stream);

/* Text describing the last non-OK status returned on this thread ("" if none).
 * The pointer stays valid until the next library call on the same thread. */
const char* rib_last_error(void);

/* ABI version of this header (incremented on any incompatible change). */
int rib_abi_version(void);

#define RIB_ABI_VERSION 11

#ifdef __cplusplus
}
#endif

#endif /* RIB_H */

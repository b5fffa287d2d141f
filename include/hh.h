/*
 * hh.h -- C ABI of libhh: Hedgehog-style linear attention on AMD MI355X (gfx950).
 *
 * The method ("The Hedgehog & the Porcupine: Expressive Linear Attentions with
 * Softmax Mimicry", arXiv 2402.04347) replaces softmax attention by a kernel
 * phi(q)^T phi(k) with a learned feature map phi and evaluates Eq. 2
 *     y_i = phi(q_i)^T S_i / phi(q_i)^T z_i,
 *     S_i = sum_{j<=i} phi(k_j) v_j^T,   z_i = sum_{j<=i} phi(k_j)
 * with running sums (paper-graph-ui walkthrough, section 2 and section 3.4
 * "Complexity Analysis").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  Layout   q, k, v, y: [B][H][N][d] row-major.  W: [H][d][d], row l is the
 *           direction w_l (u = W x + b, "the l-th row of W", section 3.4,
 *           Choice 1).  b: [H][d].  phi: [B][H][N][d'].  State S: [B][H][d'][d]
 *           fp32, z: [B][H][d'] fp32.  d' = 2d (Hedgehog) or 1 + d + d*d (Taylor and
 *           the generalised quadratic map, whose W is instead fp32 [H][3]: the
 *           coefficients a, b, c of each head, in every dtype).
 *  Dtype    `dtype` selects the element type of q, k, v, W, b, y and phi
 *           (HH_F32 or HH_BF16).  The state S, z is always fp32.  Products are
 *           accumulated in fp32 on the GPU.
 *  Memory   Every tensor pointer is a device pointer owned by the caller and
 *           16-byte aligned.  The library allocates no device memory and keeps
 *           no state between calls; scratch space comes from the caller's
 *           `workspace`.
 *  Streams  `stream` is a hipStream_t passed as void* (NULL = the default
 *           stream).  Every call is asynchronous on that stream; the library
 *           never synchronizes.  Faults inside kernels surface at the caller's
 *           next synchronization.
 *  Errors   Arguments are checked on the host before anything is enqueued; on a
 *           failed check the call returns HH_EINVAL / HH_EUNSUPPORTED /
 *           HH_EWORKSPACE and launches nothing.  A failed launch returns HH_EHIP.
 *           hh_last_error() gives a thread-local message for the last failure.
 *  Threads  Calls are thread-safe (no global mutable state).
 *  Sizes    B, H >= 1; N >= 0 (N == 0 is a no-op apart from the state outputs);
 *           N * d < 2^31 and B * H < 2^24.
 *  Supported head dims: d in {16, 32, 64, 128} for the maps with a W; the Taylor and the
 *  generalised quadratic map d == 16.
 *  Maps 2-4 run the attention over features that a feature-map kernel writes into the
 *  workspace first (bf16), so their forward needs a workspace even with one segment; the
 *  exception is map 2 in the causal bf16 forward at d == 64 and 128, whose kernels form and normalise
 *  the features themselves (its workspace then holds only segment slots, as for map 0).
 */
#ifndef HH_H
#define HH_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    HH_OK = 0,           /* success, work enqueued                                  */
    HH_EINVAL = 1,       /* bad argument: null/misaligned pointer, bad size, aliasing */
    HH_EUNSUPPORTED = 2, /* valid request outside what the library implements       */
    HH_EWORKSPACE = 3,   /* workspace missing or smaller than the size query says   */
    HH_EHIP = 4          /* a HIP launch or runtime call failed                     */
} hh_status_t;

typedef enum { HH_F32 = 0, HH_BF16 = 1 } hh_dtype_t;

typedef enum {
    /* phi(x) = [exp(W x + b), exp(-(W x + b))], d' = 2d: the Hedgehog map of
     * section 3.4, "The Hedgehog MLP Feature Map", Choice 1 (element-wise exp
     * after one linear layer, shared by q and k of a head) with the negation
     * mapping of Choice 3 (paperlayer.ai summary, A.1). */
    HH_MAP_HEDGEHOG = 0,
    /* phi(x) = [1, x_0..x_{d-1}, x_a x_c / sqrt(2) for a, c in [d] (row-major)],
     * d' = 1 + d + d^2, so phi(q)^T phi(k) = 1 + q.k + (q.k)^2 / 2: the degree-2
     * Taylor map of section 3.4, "The Taylor Exponential as a Bridge Result". */
    HH_MAP_TAYLOR2 = 1,
    /* phi(x) = [softmax(W x), softmax(-W x)], d' = 2d, no bias (b must be NULL): the softmax
     * over the feature directions of Choice 4 (section 3.4), with the negation mapping of
     * Choice 3, one softmax per half (each half sums to 1). */
    HH_MAP_HEDGEHOG_SOFTMAX = 2,
    /* phi(x) = exp(W x + b), d' = d: the single-sided map of Choice 1 with the default d' = d of
     * the same section ("The Hedgehog MLP Feature Map"). */
    HH_MAP_EXP = 3,
    /* phi(x) = softmax(W x), d' = d, no bias (b must be NULL): Choice 4 as printed. */
    HH_MAP_SOFTMAX = 4,
    /* phi(x) = [sqrt(a), sqrt(b) x_0..x_{d-1}, sqrt(c) x_a x_c for a, c in [d] (row-major)],
     * d' = 1 + d + d^2, so phi(q)^T phi(k) = a + b q.k + c (q.k)^2: the learned global quadratic
     * kernel of the paperlayer.ai summary of arXiv 2610.13674 (section 2, and App. D "Global
     * Reference and HD Realization"); (a, b, c) = (1, 1, 1/2) is HH_MAP_TAYLOR2.  W points to
     * the coefficients, fp32 [H][3] = (a, b, c) per head whatever the dtype, each >= 0 (a
     * negative coefficient gives NaN features); b must be NULL.  Positive weights need
     * b^2 < 4 a c.  The backward and the distillation loss do not take this map. */
    HH_MAP_QUADRATIC = 5
} hh_map_t;

/* ABI revision of this header; bumped on any incompatible change. */
int hh_abi_version(void);

/* Feature dimension d' for (map, d): 2d, 1 + d + d^2 or d; -1 if (map, d) is invalid. */
int hh_feature_dim(int map, int d);

/* Feature map alone (section 3.4, "The Hedgehog MLP Feature Map" / "The Taylor
 * Exponential as a Bridge Result").
 *   x   [B][H][N][d]  queries or keys (dtype)
 *   W   [H][d][d], b [H][d]  map parameters (dtype); b may be NULL (zero bias) for the
 *       maps with a bias and must be NULL for the softmax maps; both ignored and may be NULL
 *       for the Taylor map
 *   phi [B][H][N][d'] output (dtype), features in the order documented above.
 * phi must not overlap x. */
hh_status_t hh_featuremap(int map, int dtype, int B, int H, int N, int d,
                          const void *x, const void *W, const void *b,
                          void *phi, void *stream);

/* Bytes of workspace hh_linattn_fwd needs for this problem (0 = none).  Returns
 * 0 as well for invalid arguments; the forward call reports those. */
size_t hh_linattn_fwd_workspace(int map, int dtype, int causal, int B, int H, int N, int d);

/* Linear-attention forward, feature map included (Eq. 2).
 *   causal = 1: y_i uses keys j <= i (inclusive), as in Eq. 2 (section 2).
 *   causal = 0: y_i uses every key (bidirectional encoders, paperlayer.ai
 *               summary, section 1).
 *   q, k, v [B][H][N][d], W [H][d][d], b [H][d] or NULL   (dtype)
 *   S0 [B][H][d'][d], z0 [B][H][d'] (fp32): optional initial state, both NULL
 *       or both set; causal only.  The sums start from them, which resumes a
 *       sequence that an earlier call ended.
 *   y  [B][H][N][d] output (dtype); must not overlap q, k, v.
 *   S_out, z_out (fp32): optional final inclusive state (both NULL or both
 *       set); causal only.  May alias S0, z0.
 *   workspace: device scratch of at least hh_linattn_fwd_workspace() bytes
 *       (may be NULL when that is 0). */
hh_status_t hh_linattn_fwd(int map, int dtype, int causal, int B, int H, int N, int d,
                           const void *q, const void *k, const void *v,
                           const void *W, const void *b,
                           const float *S0, const float *z0,
                           void *y, float *S_out, float *z_out,
                           void *workspace, size_t workspace_bytes, void *stream);

/* hh_linattn_fwd without a caller workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).
 * Arguments and results are those of hh_linattn_fwd.  The segment slots live in a scratch
 * array that the library owns: 64 MiB per device, allocated when the library is loaded and held
 * until the process ends.  A problem whose hh_linattn_fwd_workspace() exceeds that returns
 * HH_EWORKSPACE with nothing enqueued.  This call allocates nothing.  Every call on one device
 * shares that device's array: calls that overlap in time on one device (other streams, other
 * threads) race on it and must be serialised by the caller; the array needs no clearing (each
 * call writes every slot it later reads). */
hh_status_t hh_linattn_fwd_noalloc(int map, int dtype, int causal, int B, int H, int N, int d,
                                   const void *q, const void *k, const void *v,
                                   const void *W, const void *b,
                                   const float *S0, const float *z0,
                                   void *y, float *S_out, float *z_out, void *stream);

/* Bytes of workspace hh_linattn_bwd needs (0 for invalid or unsupported arguments, or N == 0). */
size_t hh_linattn_bwd_workspace(int map, int dtype, int causal, int B, int H, int N, int d);

/* Backward of hh_linattn_fwd: the gradients of a loss L given dL/dy, for training end to end
 * with the task loss (section 3.4, "Training Protocols for the Three Regimes").  With
 * den_i = sum_j phi(q_i).phi(k_j) over the keys query i sees, g_i = dy_i / den_i and
 * c_i = -(dy_i . y_i) / den_i:  dL/dphi(q_i) = sum_j phi(k_j) (v_j . g_i + c_i),
 * dL/dphi(k_j) = sum_i phi(q_i) (v_j . g_i + c_i), dL/dv_j = sum_i phi(q_i).phi(k_j) g_i, then
 * the chain rule through the feature map to dq, dk, dW, db.  The sequence starts from a zero
 * state (no S0).
 *   map: every map with a W (the Taylor map returns HH_EUNSUPPORTED); dtype: HH_BF16 only.
 *   q, k, v, W, b as in hh_linattn_fwd; y [B][H][N][d] the forward's output; dy = dL/dy.
 *   dq, dk, dv [B][H][N][d] (bf16) outputs; dW [H][d][d] and db [H][d] fp32 outputs, summed
 *   over the batch, the tokens and both q and k (db NULL exactly when the map has no bias or b
 *   is NULL).  No output may overlap an input or another output.
 *   workspace: at least hh_linattn_bwd_workspace() bytes.
 * Features, the products' operands (g, the intra-chunk weights) and dq, dk, dv are rounded to
 * bf16; sums run in fp32. */
hh_status_t hh_linattn_bwd(int map, int dtype, int causal, int B, int H, int N, int d,
                           const void *q, const void *k, const void *v,
                           const void *W, const void *b, const void *y, const void *dy,
                           void *dq, void *dk, void *dv, float *dW, float *db,
                           void *workspace, size_t workspace_bytes, void *stream);

/* One recurrent decode step (running-sum update of section 3.4, "Complexity
 * Analysis"): for each (b, h), with f = phi(k), g = phi(q):
 *     S += f v^T;  z += f;  y = g^T S / g^T z     (update, then read: j <= i)
 *   q, k, v, y [B][H][d] (dtype, one token per sequence)
 *   S [B][H][d'][d], z [B][H][d'] fp32, read and written in place.
 *   W, b as in hh_linattn_fwd.  y must not overlap q, k, v, S, z. */
hh_status_t hh_linattn_decode_step(int map, int dtype, int B, int H, int d,
                                   const void *q, const void *k, const void *v,
                                   const void *W, const void *b,
                                   float *S, float *z, void *y, void *stream);

/* Bytes of workspace hh_distill_loss needs (the features of k for the Hedgehog map, 0 for the
 * Taylor map).  Returns 0 as well for invalid arguments. */
size_t hh_distill_loss_workspace(int map, int dtype, int B, int H, int N, int d);

/* Attention-weight distillation loss of Eq. 4 (paper-graph-ui walkthrough, section 3.4, "The
 * Attention Weight Distillation Loss"), per query: for each (b, h) and i,
 *     p_ij = exp(q_i.k_j / sqrt(d)) / sum_{m<=i} exp(q_i.k_m / sqrt(d))      (j <= i)
 *     a_ij = phi(q_i).phi(k_j)
 *     loss_i = -sum_{j<=i} p_ij log(a_ij / sum_{m<=i} a_im)
 * the cross-entropy between the causal softmax weights of the raw q, k and the linear-attention
 * weights of their features.  The total loss of the pages is the sum of loss over b, h, i.
 *   q, k [B][H][N][d] (bf16; fp32 inputs return HH_EUNSUPPORTED), W [H][d][d], b [H][d] or
 *       NULL as in hh_linattn_fwd (Taylor map: ignored, d = 16).
 *   loss [B][H][N] fp32 output; must not overlap q or k.
 *   workspace: device scratch of at least hh_distill_loss_workspace() bytes (may be NULL when
 *       that is 0); must not overlap the other arguments.
 * The features enter the weights rounded to bf16, as in the forward pass. */
hh_status_t hh_distill_loss(int map, int dtype, int B, int H, int N, int d,
                            const void *q, const void *k, const void *W, const void *b,
                            float *loss, void *workspace, size_t workspace_bytes, void *stream);

/* Static description of a status code. */
const char *hh_status_str(int status);

/* Thread-local message describing the last failure on this thread ("" if none). */
const char *hh_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* HH_H */

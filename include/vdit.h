/*
 * vdit.h — C ABI of the spacetime-attention library (libvdit.so), gfx950.
 *
 * The operations of a video diffusion transformer's self-attention input
 * path, each enqueued on a caller-supplied HIP stream:
 *
 *   vdit_patchify       Conv3d with stride = kernel, as a GEMM, to token-major
 *                       tokens;
 *   vdit_rope3d         3D factorised rotary position embedding on Q or K;
 *   vdit_attn_full      softmax attention over all T*Hp*Wp tokens of a clip;
 *   vdit_attn_spatial   the same, with keys limited to the query's own latent
 *                       frame;
 *   vdit_attn_full_rope, vdit_attn_spatial_rope, vdit_attn_temporal_rope
 *                       full, spatial and temporal attention with 3D RoPE
 *                       applied to q and k inside the attention kernel (no
 *                       separate RoPE pass);
 *   vdit_attn_temporal  the same, with keys limited to the query's own patch
 *                       position across frames;
 *   vdit_attn_cross     attention from the video tokens to another token set
 *                       (the text prompt);
 *   vdit_attn_window    the same, with keys limited to the query's own
 *                       non-overlapping wt x wh x ww spacetime window;
 *   vdit_qkv_proj       the attention input: tokens projected to Q, K, V,
 *                       with per-head RMSNorm and 3D RoPE on Q and K.
 *
 * Conventions shared by every call
 * --------------------------------
 * Token order. A clip of T latent frames of Hp x Wp patches has N = T*Hp*Wp
 * tokens; token (t, h, w) has index n = (t*Hp + h)*Wp + w, time slowest. This
 * is the flattening of "How AI Generates Video: Inside Sora and Wan2.1 on a
 * Real GPU", section 7 (query (2, 18, 26) of a (5, 30, 52) grid is token 4082).
 *
 * Q/K/V/O layout. Token-major, contiguous: element (b, n, head, d) sits at
 * ((b*N + n)*heads + head)*head_dim + d. This is the [B, N, heads*head_dim]
 * token tensor viewed per head; the time<->space permutes of divided
 * attention are never materialised.
 *
 * Types. VDIT_BF16: every tensor argument is bfloat16, arithmetic in fp32
 * (bf16 matrix cores for products, fp32 softmax and accumulation, as the
 * "Failure modes" of "Video Diffusion Models, in depth" require), results
 * rounded to bf16 to nearest even. VDIT_F32: every tensor is fp32 and all
 * arithmetic is fp32.
 *
 * Pointers are device pointers owned by the caller. The library allocates
 * no device memory, keeps no pointer after a call returns and has no mutable
 * global state, so calls on different streams may run concurrently. Every
 * call only enqueues work on `stream` (a hipStream_t; NULL means the default
 * stream) and returns without synchronising; inputs must stay valid until the
 * work completes in stream order.
 *
 * Errors. All checks run before anything is enqueued, so a call that returns
 * an error has enqueued nothing. NaN and Inf in the data are not errors; they
 * propagate to the outputs.
 */
#ifndef VDIT_H
#define VDIT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    VDIT_BF16 = 0,
    VDIT_F32 = 1
} vdit_dtype_t;

typedef enum {
    VDIT_OK = 0,
    VDIT_E_NULL = 1,       /* a required pointer is NULL                         */
    VDIT_E_SHAPE = 2,      /* a size is <= 0, the grid does not match the latent,
                              or an element count overflows                       */
    VDIT_E_HEAD_DIM = 3,   /* head_dim is not one the kernels support             */
    VDIT_E_ROPE_SPLIT = 4, /* d_t + d_h + d_w != head_dim, or a part is odd       */
    VDIT_E_ALIGN = 5,      /* a pointer is not 16-byte aligned                   */
    VDIT_E_ALIAS = 6,      /* an output overlaps an input it may not overlap      */
    VDIT_E_DTYPE = 7,      /* unknown dtype                                       */
    VDIT_E_LAUNCH = 8      /* the kernel launch failed (hipGetLastError)          */
} vdit_status_t;

/* Human-readable name of a status code (a static string). */
const char *vdit_status_str(vdit_status_t status);

/*
 * vdit_patchify — spacetime tube patchify.
 *
 * Defined by the "Video and 3D Generation" cheatsheet, "Tiny video DiT"
 * (a Conv3d whose stride equals its kernel turns a (N, C, T, H, W) clip into
 * a grid of tokens), and "How AI Generates Video ...", section 4 (16-channel
 * 1x2x2 bricks, 64 numbers each, projected to 1,536-wide tokens):
 *
 *   tokens[b][n][o] = bias[o] + sum_{c,i,j,k} weight[o][c][i][j][k] *
 *                     latent[b][c][t*pt+i][h*ph+j][w*pw+k],   n = (t*Hp+h)*Wp+w
 *
 * latent : [B, C, Tl, Hl, Wl] (NCTHW), contiguous.
 * weight : [heads*head_dim, C, pt, ph, pw] (the Conv3d weight layout).
 * bias   : [heads*head_dim] or NULL (no bias).
 * tokens : [B, T*Hp*Wp, heads*head_dim], token-major output; may not overlap
 *          latent, weight or bias (VDIT_E_ALIAS).
 * The grid must be the strided convolution's: T = Tl/pt, Hp = Hl/ph,
 * Wp = Wl/pw with floor division (a remainder is dropped, as a Conv3d without
 * padding does); otherwise VDIT_E_SHAPE. For VDIT_BF16 the patch length
 * C*pt*ph*pw, rounded up to a multiple of 16, must be <= 512 (else
 * VDIT_E_SHAPE). head_dim: any positive value with heads*head_dim a multiple
 * of 8.
 */
vdit_status_t vdit_patchify(const void *latent, const void *weight, const void *bias,
                            void *tokens, int B, int C, int pt, int ph, int pw,
                            int Tl, int Hl, int Wl, int heads, int T, int Hp, int Wp,
                            int head_dim, vdit_dtype_t dtype, void *stream);

/*
 * vdit_rope3d — 3D factorised rotary position embedding.
 *
 * Defined by "How AI Generates Video ...", section 4 ("How 3D Factorized RoPE
 * Encodes (t', h, w)"): every head vector is cut into three consecutive
 * segments of widths (d_t, d_h, d_w), (44, 42, 42) for head_dim 128. In
 * segment a, the pair (x[2j], x[2j+1]) is rotated by the angle p_a * f_{a,j},
 * with p_a the token's t, h or w index (from 0) and f_{a,j} = theta^(-2j/d_a)
 * (theta = 10,000 in the pages):
 *   y[2j]   = x[2j] cos - x[2j+1] sin
 *   y[2j+1] = x[2j] sin + x[2j+1] cos
 * The "Video and 3D Generation" cheatsheet ("Troubleshooting") makes a split
 * that does not add up to the head width an error: VDIT_E_ROPE_SPLIT, also
 * for an odd part.
 *
 * x, y : [B, N, heads, head_dim]. y may equal x (in place); partial overlap is
 *        VDIT_E_ALIAS. Each angle is formed and reduced to [-pi, pi] in fp64,
 *        then its sin/cos are taken in fp32.
 * head_dim: a multiple of 8, <= 256 (else VDIT_E_HEAD_DIM); theta > 0.
 */
vdit_status_t vdit_rope3d(const void *x, void *y, int B, int heads, int T, int Hp, int Wp,
                          int head_dim, int d_t, int d_h, int d_w, float theta,
                          vdit_dtype_t dtype, void *stream);

/*
 * vdit_attn_full — full 3D spacetime self-attention.
 *
 * Every token attends to every token of its clip ("Video Diffusion Models, in
 * depth", Step 3; "How AI Generates Video ...", section 5, attn1):
 *   o[b][n][h] = sum_m softmax_m(scale * <q[b][n][h], k[b][m][h]>) v[b][m][h],
 * m over all N tokens, no mask. The work is 4*N^2*head_dim FLOP per
 * (b, head), the count of "Video Diffusion Models, in depth", Step 2.
 *
 * q, k, v, o : [B, N, heads, head_dim], N = T*Hp*Wp. o may not overlap q, k
 *              or v (VDIT_E_ALIAS).
 * scale      : softmax scale; <= 0 selects 1/sqrt(head_dim).
 * head_dim   : 32, 64 or 128 (VDIT_BF16 and VDIT_F32)
 *              (else VDIT_E_HEAD_DIM).
 * Size limit : VDIT_BF16 needs one batch's tensor, N*heads*head_dim*2 bytes,
 *              below 2 GiB (else VDIT_E_SHAPE); 720p at 40 heads is 774 MB.
 */
vdit_status_t vdit_attn_full(const void *q, const void *k, const void *v, void *o,
                             int B, int heads, int T, int Hp, int Wp, int head_dim,
                             float scale, vdit_dtype_t dtype, void *stream);

/*
 * vdit_attn_spatial — the spatial pass of divided attention.
 *
 * Attention within each latent frame: the keys of query (t, h, w) are the
 * Hp*Wp tokens of frame t ("Video as a 3D signal", "Patches and attention";
 * the T*(HW)^2 term of the divided cost in the "Video and 3D Generation"
 * cheatsheet, "Formulas and numbers"). Arguments as vdit_attn_full.
 */
vdit_status_t vdit_attn_spatial(const void *q, const void *k, const void *v, void *o,
                                int B, int heads, int T, int Hp, int Wp, int head_dim,
                                float scale, vdit_dtype_t dtype, void *stream);

/*
 * vdit_attn_full_rope, vdit_attn_spatial_rope, vdit_attn_temporal_rope —
 * full, spatial or temporal attention of the rotated queries and keys: the
 * result equals vdit_rope3d on q and on k (same d_t, d_h, d_w, theta)
 * followed by vdit_attn_full, vdit_attn_spatial or vdit_attn_temporal,
 * without the rotated copies ever reaching memory. In Wan 2.1's attn1 ("How
 * AI Generates Video ...", section 5) the rotation is the step right before
 * the attention product. The full and spatial kernels apply it to the
 * queries once after reading them and to every K tile as it arrives in
 * on-chip memory, so it is repeated once per query block that reads the
 * tile; the temporal kernel rotates each sequence's Q and K rows once, in
 * on-chip memory. q and k in memory are not modified. T as
 * vdit_attn_temporal for the temporal call (<= 64).
 *
 * Speed: the temporal call takes about half the time of vdit_rope3d on q and
 * k followed by vdit_attn_temporal (that pass is bound by memory traffic,
 * and the rotation saves two tensor round trips). The full and spatial
 * calls are SLOWER than vdit_rope3d followed by the plain call (1.2-1.4x
 * measured at 480p): every workgroup re-rotates each K tile it reads, which
 * adds half again to the vector work that already bounds those kernels.
 * They exist for callers that cannot hold rotated copies of q and k (two
 * extra tensors, 1.5 GB at the 720p shape); no default path uses them.
 *
 * Arguments, layouts, limits and errors as vdit_attn_full, plus d_t, d_h,
 * d_w and theta as vdit_rope3d (VDIT_E_ROPE_SPLIT for a bad split,
 * VDIT_E_SHAPE for theta <= 0 or not finite). The angle of each pair is
 * formed in fp32 in revolutions and its sin/cos taken by the hardware's
 * v_sin_f32/v_cos_f32; the rotated q and k are rounded to bf16, as
 * vdit_rope3d's output is. dtype: VDIT_BF16 only (VDIT_F32 gives
 * VDIT_E_DTYPE: the fp32 parity path is vdit_rope3d then the plain call).
 */
vdit_status_t vdit_attn_full_rope(const void *q, const void *k, const void *v, void *o,
                                  int B, int heads, int T, int Hp, int Wp, int head_dim,
                                  int d_t, int d_h, int d_w, float theta, float scale,
                                  vdit_dtype_t dtype, void *stream);
vdit_status_t vdit_attn_spatial_rope(const void *q, const void *k, const void *v, void *o,
                                     int B, int heads, int T, int Hp, int Wp, int head_dim,
                                     int d_t, int d_h, int d_w, float theta, float scale,
                                     vdit_dtype_t dtype, void *stream);
vdit_status_t vdit_attn_temporal_rope(const void *q, const void *k, const void *v, void *o,
                                      int B, int heads, int T, int Hp, int Wp, int head_dim,
                                      int d_t, int d_h, int d_w, float theta, float scale,
                                      vdit_dtype_t dtype, void *stream);

/*
 * vdit_attn_temporal — the temporal pass of divided attention.
 *
 * Attention across frames at one patch position: the keys of query (t, h, w)
 * are the T tokens (t', h, w), t' = 0..T-1 (same passages; the (HW)*T^2
 * term). Consecutive keys of a sequence are Hp*Wp tokens apart in the
 * token-major layout; the kernel reads them in place. Arguments as
 * vdit_attn_full; head_dim 32, 64 or 128.
 * T <= 64 for VDIT_BF16 and T <= 256 for VDIT_F32 (else VDIT_E_SHAPE).
 */
vdit_status_t vdit_attn_temporal(const void *q, const void *k, const void *v, void *o,
                                 int B, int heads, int T, int Hp, int Wp, int head_dim,
                                 float scale, vdit_dtype_t dtype, void *stream);

/*
 * vdit_attn_cross — cross-attention from the video tokens to another token
 * set (the text prompt).
 *
 * "How AI Generates Video ...", section 5 (attn2: the video bricks supply the
 * queries, the 512 UMT5 text embeddings, projected to the model width, the
 * keys and values); "Video Diffusion Models, in depth", Step 3 (the video
 * tokens read the text embeddings):
 *   o[b][n][h] = sum_m softmax_m(scale * <q[b][n][h], k[b][m][h]>) v[b][m][h],
 * m over all Nk keys of batch b, no mask. 4*Nq*Nk*head_dim FLOP per (b, head).
 *
 * q, o : [B, Nq, heads, head_dim]; k, v : [B, Nk, heads, head_dim], token-
 *        major. o may not overlap q, k or v (VDIT_E_ALIAS).
 * scale, head_dim, dtype and the 2 GiB-per-batch bf16 limit (on both token
 * sets) as vdit_attn_full.
 */
vdit_status_t vdit_attn_cross(const void *q, const void *k, const void *v, void *o,
                              int B, int heads, int Nq, int Nk, int head_dim,
                              float scale, vdit_dtype_t dtype, void *stream);

/*
 * vdit_attn_window — attention within local spacetime windows.
 *
 * "Video Diffusion Models, in depth", "Inference: where the time goes":
 * limiting attention to local windows of space and time is the direct
 * attack on the quadratic term. Reading taken here: the grid is cut into
 * non-overlapping windows of wt x wh x ww tokens, the last window along an
 * axis cut short by the grid, and the keys of query (t, h, w) are the tokens
 * (t', h', w') with t'/wt = t/wt, h'/wh = h/wh and w'/ww = w/ww (integer
 * division):
 *   o[b][n][h] = sum_{m in window(n)} softmax_m(scale * <q_n, k_m>) v_m.
 * Window (1, Hp, Wp) is the spatial pass, (T, 1, 1) the temporal pass and
 * (T, Hp, Wp) full attention. 4*|window|^2*head_dim FLOP per window and head.
 *
 * wt, wh, ww : window extents in tokens, >= 1 (else VDIT_E_SHAPE); extents
 *              larger than the grid are clipped to it.
 * Other arguments, layouts, limits and errors as vdit_attn_full.
 */
vdit_status_t vdit_attn_window(const void *q, const void *k, const void *v, void *o,
                               int B, int heads, int T, int Hp, int Wp, int head_dim,
                               int wt, int wh, int ww, float scale, vdit_dtype_t dtype,
                               void *stream);

/*
 * vdit_qkv_proj — the projection in front of a block's self-attention.
 *
 * "How AI Generates Video ...", section 5 (attn1): the tokens are projected
 * into heads of Queries, Keys and Values, RMSNorm is applied to Q and K, and
 * Q and K are rotated with the 3D factorised RoPE of section 4. Readings
 * taken here: one fused weight W [3*dim][dim] (nn.Linear layout [out][in];
 * rows 0..dim-1 produce Q, dim..2*dim-1 K, 2*dim..3*dim-1 V), dim =
 * heads*head_dim; the RMSNorm statistic is taken over each head's head_dim
 * values (the same vectors RoPE then rotates), with a per-channel gain:
 *   y[m][c]   = bias[c] + sum_j W[c][j] * x[m][j]
 *   Q[m][h][d] = RoPE_m( y_q[m][h][d] / sqrt(mean_d' y_q[m][h][d']^2 + eps)
 *                        * gamma_q[h*head_dim + d] )           (K alike)
 *   V[m][h][d] = y_v[m][h][d]
 * with RoPE as vdit_rope3d at token m's grid position (t, h, w).
 * 2*M*3*dim*dim FLOP, M = B*T*Hp*Wp.
 *
 * x        : [B, N, dim] tokens (vdit_patchify's output), N = T*Hp*Wp.
 * w        : [3*dim, dim]; bias: [3*dim] or NULL.
 * gamma_q, gamma_k : [dim] gains, or NULL to leave that tensor unnormalised.
 * q, k, v  : [B, N, heads, head_dim] outputs; they may not overlap the inputs
 *            or each other (VDIT_E_ALIAS).
 * d_t, d_h, d_w, theta : RoPE split and base as vdit_rope3d; all three zero
 *            disables the rotation.
 * eps      : RMSNorm epsilon (>= 0).
 * Limits   : VDIT_BF16: head_dim 128, dim a multiple of 128, x and w each
 *            below 2 GiB (else VDIT_E_HEAD_DIM / VDIT_E_SHAPE); VDIT_F32:
 *            head_dim <= 256, for small workloads. Pointers 16-byte aligned.
 */
vdit_status_t vdit_qkv_proj(const void *x, const void *w, const void *bias, const void *gamma_q,
                            const void *gamma_k, void *q, void *k, void *v, int B, int T, int Hp,
                            int Wp, int heads, int head_dim, int d_t, int d_h, int d_w, float theta,
                            float eps, vdit_dtype_t dtype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* VDIT_H */

/*
 * moga.h - C ABI of libmoga.so: the Mixture-of-Groups Attention (MoGA) forward
 * path with static spatial-temporal group attention (STGA), for AMD MI355X
 * (gfx950).
 *
 * Sources (cited by site and section):
 *   papernotes.org ICLR 2026 note "MoGA: Mixture-of-Groups Attention for
 *     End-to-End Long Video Generation", 方法详解 / 关键设计 1-4 ("design 1" ...
 *     "design 4" below);
 *   jxzklqfsx.com Chinese translation of the paper, section 方法;
 *   xugj520.cn MoGA blog, §2.2-2.3 (router), §3.2 and §9 (STGA boundary frames).
 *
 * Conventions for every entry point
 *   - Tensor pointers are DEVICE pointers owned by the caller, unless a comment
 *     says HOST.  The library never allocates, frees or synchronises.
 *   - Attention tensors are bf16, row-major [H][rows][head_dim] (head-major: one
 *     contiguous [rows][head_dim] block per head).
 *   - `stream` is a hipStream_t (NULL: the legacy default stream).  Each call
 *     validates its arguments, enqueues kernels on `stream` and returns; results
 *     are valid once the stream has reached that point.
 *   - Validation happens before any launch: a call that returns an error has
 *     enqueued nothing.  Faults during kernel execution surface at the
 *     caller's next synchronisation, not as a return code.
 *   - `ws` is caller-owned device scratch of at least the size the matching
 *     *_workspace_bytes function returns; calls that share a workspace must be
 *     ordered on one stream.  Its contents need not be initialised.
 *   - All outputs are bitwise reproducible from run to run (no floating-point
 *     atomics, fixed reduction orders).
 *   - moga_last_error() returns a thread-local description of the last
 *     non-OK status on the calling thread.
 */
#ifndef MOGA_H
#define MOGA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOGA_OK = 0,
    MOGA_ERR_ARG = 1,          /* a NULL required pointer, a size out of range, bad geometry */
    MOGA_ERR_UNSUPPORTED = 2,  /* the current device is not gfx950, or a shape it does not cover */
    MOGA_ERR_WORKSPACE = 3,    /* ws is NULL or ws_bytes is below the required size */
    MOGA_ERR_HIP = 4           /* a HIP runtime call or launch failed; text in moga_last_error() */
} moga_status;

typedef enum { MOGA_F32 = 0, MOGA_BF16 = 1 } moga_dtype;

/* Problem sizes shared by the calls.
 *   n_tokens      N, 1 <= N < 2^31
 *   d_model       router input width d, 1 <= d <= 2^20 (a multiple of 8 for bf16 x, of 4
 *                 for f32 x)
 *   n_heads       H >= 1, with H * (ceil(N/128) + M) < 2^31 (the attention work list;
 *                 with a STGA layout M is replaced by the larger of its group and frame counts)
 *   head_dim      64 or 128
 *   n_groups      M, 1 <= M <= 64
 *   softmax_scale attention scale; <= 0 selects 1/sqrt(head_dim)
 *   alpha         weight of the group-balancing loss (0.1 on the pages) */
typedef struct {
    int64_t n_tokens;
    int32_t d_model;
    int32_t n_heads;
    int32_t head_dim;
    int32_t n_groups;
    float softmax_scale;
    double alpha;
} moga_dims;

/* STGA geometry (design 4).  Tokens are frame-major: token = (f*height + y)*width + x,
 * so N == frames*height*width.  shot_start is a HOST array of n_shots+1 strictly
 * increasing frame indices, shot_start[0] == 0 and shot_start[n_shots] == frames;
 * 1 <= n_shots <= 256.  Spatial windows are win_h x win_w and must tile the frame;
 * temporal groups are t_group consecutive frames of one shot, starting at the
 * shot's first frame (a shorter last chunk is its own group).  The keys and
 * values of the first chunk of shot s > 0 also hold the last aug_frames frames
 * of shot s-1, and those of the last chunk of shot s < n_shots-1 the first
 * aug_frames frames of shot s+1 (same window; clipped to the neighbour shot's
 * length).  Per-frame groups are whole frames. */
typedef struct {
    int32_t frames, height, width;
    int32_t n_shots;
    const int32_t *shot_start; /* HOST, n_shots + 1 entries */
    int32_t win_h, win_w;
    int32_t t_group;
    int32_t aug_frames;
} stga_layout;

/* Inputs and outputs of moga_forward. */
typedef struct {
    const void *x;        /* [N][d_model], x_dtype */
    moga_dtype x_dtype;
    const float *w;       /* router weight [d_model][M] fp32, no bias */
    const void *q, *k, *v;/* bf16 [H][N][head_dim], token order */
    const int32_t *pin;   /* NULL or [N]: -1 = free, else the forced group of the token */
} moga_inputs;

typedef struct {
    void *out;            /* required, bf16 [H][N][head_dim], token order */
    double *loss;         /* required, one fp64 scalar: L_gb */
    int32_t *group_id;    /* optional [N] */
    float *p_sel;         /* optional [N]: p(g(x)|x) */
    int32_t *cu_seqlens;  /* optional [M+1] */
    int32_t *perm;        /* optional [N]: grouped row -> token */
    int32_t *counts;      /* optional [M] */
    double *prob_sum;     /* optional [M]: sum over tokens of p(i|x) */
    float *lse;           /* optional [H][N] fp32, token order: natural log of the softmax
                             normaliser of the token's MoGA attention row,
                             log sum_u exp(scale q.k_u) over its group's keys; the state
                             moga_backward needs besides out.  With a STGA layout: [3][H][N],
                             the MoGA, temporal and per-frame normalisers (planes in that
                             order), allowed only together with o_branches (else the call
                             returns MOGA_ERR_UNSUPPORTED) */
    void *o_branches;     /* optional, STGA layout only: bf16 [3][H][N][head_dim], token order:
                             each branch's row before the mean (the MoGA row scaled by
                             p(g|x), the temporal row, the per-frame row), each rounded to
                             bf16 once; with lse, the state moga_hybrid_backward needs */
} moga_outputs;

const char *moga_last_error(void);

/* Workspace bytes needed by moga_forward, moga_route and moga_permute for these
 * sizes (stga NULL: MoGA only; non-NULL also covers stga_group_attn).  Returns 0
 * if the sizes are invalid. */
size_t moga_workspace_bytes(const moga_dims *dims, const stga_layout *stga);

/* Workspace bytes needed by moga_group_attn with n_seg segments and len_q query rows.
 * With head_dim 128 this includes room for the key-range split of a launch's last items
 * (fp32 partial rows: at most 256 parts of 256 rows, and no more rows than H * len_q). */
size_t moga_group_attn_workspace_bytes(const moga_dims *dims, int32_t n_seg, int64_t len_q);

/* Router (design 1; blog §2.3): r = x W in fp32 (no bias), p = softmax(r),
 * g = argmax r with the lowest index winning exact ties; pin[t] >= 0 overrides g.
 * Writes group_id [N] (int32), p_sel [N] = p(g|x) (fp32), counts [M] (int32) and
 * prob_sum [M] = sum over tokens of p(i|x) accumulated in fp64 in a fixed order.
 * pin may be NULL.  ws: moga_workspace_bytes(dims, NULL). */
moga_status moga_route(const void *x, moga_dtype x_dtype, const float *w, const int32_t *pin,
                       const moga_dims *dims, int32_t *group_id, float *p_sel, int32_t *counts,
                       double *prob_sum, void *ws, size_t ws_bytes, void *stream);

/* Stable permute into contiguous groups, and its inverse (design 2).
 *   inverse == 0: from group_id [N] (values in [0, M)) compute cu_seqlens [M+1]
 *     (cu[0] = 0, cu[i+1] = cu[i] + n_i) and perm [N] (grouped row j -> token;
 *     groups in ascending id, tokens in ascending order within a group), then
 *     dst[i][h][j] = src[i][h][perm[j]] for each of the n_tensors bf16 tensors
 *     [H][N][head_dim], and p_perm[j] = p_sel[perm[j]] if both are non-NULL.
 *   inverse == 1: perm is an input (group_id and cu_seqlens may be NULL) and
 *     dst[i][h][perm[j]] = src[i][h][j]; p_sel/p_perm are ignored.
 * src and dst are HOST arrays of n_tensors device pointers, 0 <= n_tensors <= 4;
 * dst must not overlap src.  Group ids outside [0, M) are an error the library
 * cannot see: the results are then undefined (no out-of-bounds access occurs).
 * ws: moga_workspace_bytes(dims, NULL). */
moga_status moga_permute(int inverse, const int32_t *group_id, const moga_dims *dims,
                         int32_t *cu_seqlens, int32_t *perm, const void *const *src,
                         void *const *dst, int n_tensors, const float *p_sel, float *p_perm,
                         void *ws, size_t ws_bytes, void *stream);

/* Variable-length group attention (design 1 and 2): for every head h and segment
 * s, the query rows [cu_q[s], cu_q[s+1]) attend to the key rows [cu_k[s],
 * cu_k[s+1]):  o = softmax(scale q K^T) V, computed with bf16 MFMA, fp32
 * accumulation and an fp32 online softmax, then multiplied by row_scale[row]
 * (if non-NULL) and rounded to bf16.  cu_q and cu_k are DEVICE arrays of
 * n_seg+1 non-decreasing int32 with cu_q[n_seg] <= len_q and cu_k[n_seg] <= len_k
 * (rows outside every segment are left untouched; a segment with no keys
 * writes zeros).  q, o: [H][len_q][head_dim]; k, v: [H][len_k][head_dim];
 * row_scale: NULL or fp32 [len_q].  ws: moga_group_attn_workspace_bytes. */
moga_status moga_group_attn(const void *q, const void *k, const void *v, int64_t len_q,
                            int64_t len_k, int32_t n_seg, const int32_t *cu_q,
                            const int32_t *cu_k, const float *row_scale, const moga_dims *dims,
                            void *o, void *ws, size_t ws_bytes, void *stream);

/* moga_group_attn without a workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The arguments and results are those of moga_group_attn (bitwise the same outputs); the
 * attention plan lives in a static array of 40 MiB that the library holds on every device it
 * runs on until the process ends.  Sizes whose plan exceeds it (moga_group_attn_workspace_bytes
 * above 40 MiB: H * len_q beyond about 60 M query rows) return MOGA_ERR_WORKSPACE before any
 * launch.  Every call on one device shares that device's array: calls that overlap in time on
 * one device (different streams, or several host threads without ordering) race and must not
 * be issued.  The call allocates nothing and needs no initialised memory (the planning kernel
 * writes every counter the attention kernels read). */
moga_status moga_group_attn_noalloc(const void *q, const void *k, const void *v, int64_t len_q,
                                    int64_t len_k, int32_t n_seg, const int32_t *cu_q,
                                    const int32_t *cu_k, const float *row_scale,
                                    const moga_dims *dims, void *o, void *stream);

/* STGA (design 4): temporal-window groups with boundary-frame K/V augmentation,
 * written to o_temporal, and per-frame groups, written to o_frame, both bf16
 * [H][N][head_dim] in token order and unscaled.  Either output may be NULL to
 * skip that branch.  q, k, v: bf16 [H][N][head_dim], token order.
 * ws: moga_workspace_bytes(dims, stga). */
moga_status stga_group_attn(const void *q, const void *k, const void *v, const moga_dims *dims,
                            const stga_layout *stga, void *o_temporal, void *o_frame, void *ws,
                            size_t ws_bytes, void *stream);

/* Group-balancing loss (design 3): F_i = counts_i / N, P_i = prob_sum_i / N,
 * loss = alpha * M * sum_i F_i P_i, all fp64.  P_i is the mean of p(i|x) over
 * all N tokens.  counts, prob_sum: [M] device inputs; loss: one device fp64;
 * F, P: NULL or [M] device fp64. */
moga_status moga_balance_loss(const int32_t *counts, const double *prob_sum,
                              const moga_dims *dims, double *loss, double *F, double *P,
                              void *stream);

/* The whole forward: route -> permute -> group attention scaled by p(g|x), whose epilogue
 * writes every row straight back to its token (the inverse permute), plus the balance loss.
 * With stga non-NULL the two STGA branches run first (each rounded to bf16 as it is stored in
 * the workspace) and out is the mean of the three rows, taken in fp32 in the MoGA epilogue
 * from the unrounded MoGA row and rounded to bf16 once.  ws: moga_workspace_bytes(dims, stga). */
moga_status moga_forward(const moga_inputs *in, const moga_dims *dims, const stga_layout *stga,
                         const moga_outputs *out, void *ws, size_t ws_bytes, void *stream);

/* Permute-free variant of moga_forward, for the same inputs and outputs: the attention
 * kernel reads the query, key and value rows of each group through perm and writes every
 * output row straight back to its token (as moga_forward's epilogue does too), so the
 * permuted copies of Q, K and V and their gather are skipped.  Keys are visited in the same order, so every output is
 * bitwise identical to moga_forward's.  perm and cu_seqlens are still computed (and
 * returned if requested).  ws: moga_workspace_bytes(dims, stga). */
moga_status moga_forward_fused(const moga_inputs *in, const moga_dims *dims,
                               const stga_layout *stga, const moga_outputs *out, void *ws,
                               size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------ backward
 * Gradients of the MoGA forward (design 1: the router learns through the factor
 * p(g(x)|x) of the output; design 3: L_gb), with the routing held fixed: g(x), the
 * counts and the permutation are piecewise constant in x and W, so only p(g|x), the
 * attention and P_i carry gradient.  Given G = d objective / d out and d_loss =
 * d objective / d L_gb:
 *   D[h][t]  = <G[h][t], out[h][t]>,  dp_t = sum_h D[h][t] / p_t  (gradient w.r.t. p(g_t|x_t))
 *   attention backward of each group with dO' = p_t G (dQ, dK, dV; softmax recomputed from lse)
 *   a_ti = [i = g_t] dp_t + d_loss alpha M F_i / N,  dr_t = p_t (a_t - <a_t, p_t>)  (p_t: all M
 *   probabilities, recomputed from x W in fp32),  dx = dr W^T,  dW = x^T dr.
 * moga_hybrid_backward below covers the mean with the two STGA branches. */

/* What moga_backward reads from the forward; all DEVICE, as written by moga_forward or
 * moga_forward_fused called with stga NULL on the same inputs. */
typedef struct {
    const int32_t *group_id;   /* [N] */
    const float *p_sel;        /* [N] */
    const int32_t *counts;     /* [M] */
    const int32_t *cu_seqlens; /* [M+1] */
    const int32_t *perm;       /* [N] */
    const void *out;           /* bf16 [H][N][head_dim], token order */
    const float *lse;          /* [H][N], token order */
} moga_saved;

typedef struct {
    void *dq, *dk, *dv;  /* required, bf16 [H][N][head_dim], token order */
    float *dx;           /* optional [N][d_model] fp32 (for bf16 x too), 16-byte aligned */
    float *dw;           /* optional [d_model][M] fp32, 16-byte aligned */
    float *dp;           /* optional [N] fp32: dp_t above */
} moga_grads;

/* Workspace bytes needed by moga_backward (0 if the sizes are invalid). */
size_t moga_backward_workspace_bytes(const moga_dims *dims);

/* The backward above.  in: the forward's x, x_dtype, w, q, k, v (pin is not read: the
 * saved group_id already holds it).  d_out: bf16 [H][N][head_dim], token order.  head_dim 64
 * or 128 (the attention backward kernels work on 128-channel rows: head_dim 64 rows are copied
 * into them with the upper half zero, which adds nothing to any score or product, and the
 * results copied back).  dq, dk, dv, dx, dw, dp are fully overwritten.  dQ and dK/dV are computed by
 * two kernels so that every output row has one writer (no atomics), and all sums run in a
 * fixed order.  ws: moga_backward_workspace_bytes(dims). */
moga_status moga_backward(const moga_inputs *in, const moga_saved *saved, const void *d_out,
                          double d_loss, const moga_dims *dims, const moga_grads *grads,
                          void *ws, size_t ws_bytes, void *stream);

/* Gradients of the hybrid forward out = (O_m + O_t + O_f) / 3 (design 4 beside design 1:
 * every token takes the mean of its MoGA row O_m = p O, its temporal-window row O_t and its
 * per-frame row O_f), with the routing held fixed as above.  Each branch receives G / 3:
 *   MoGA: as moga_backward with G / 3 (dp_t = sum_h <G, O_m> / (3 p_t)); the loss term as is;
 *   per-frame: attention backward of each frame with dO = G / 3;
 *   temporal: attention backward of each temporal group with dO = G / 3; a key row that a
 *   group borrows from the adjacent shot passes its dK, dV back to the token it was taken
 *   from, so a token's dK and dV sum over every group whose key set holds it.
 * The three branches' dQ, dK, dV are added per token in fp32 and rounded to bf16 once.
 * saved: as moga_forward wrote it with this stga layout, with out = o_branches
 * ([3][H][N][head_dim]) and lse = the [3][H][N] normalisers; the other fields as for
 * moga_backward.  head_dim 64 or 128, as for moga_backward.
 * ws: moga_hybrid_backward_workspace_bytes. */
size_t moga_hybrid_backward_workspace_bytes(const moga_dims *dims, const stga_layout *stga);
moga_status moga_hybrid_backward(const moga_inputs *in, const moga_saved *saved,
                                 const stga_layout *stga, const void *d_out, double d_loss,
                                 const moga_dims *dims, const moga_grads *grads, void *ws,
                                 size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOGA_H */

// Host side of the C ABI declared in include/moga.h: argument validation (always before
// any launch), the gfx950 check, workspace carving and the launch sequences.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "moga.h"
#include "moga_internal.h"

using namespace moga;

namespace {

thread_local std::string g_err;

moga_status fail(moga_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

moga_status hip_fail(hipError_t e, const char *what) {
    return fail(MOGA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIP_TRY(expr, what)                          \
    do {                                             \
        hipError_t _e = (expr);                      \
        if (_e != hipSuccess) return hip_fail(_e, what); \
    } while (0)

// ---------------------------------------------------------------- device check
std::mutex g_dev_mu;
int g_dev_state[64];  // 0 unknown, 1 gfx950, 2 other

moga_status check_device() {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(MOGA_ERR_UNSUPPORTED, "no HIP device: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= 64) return fail(MOGA_ERR_UNSUPPORTED, "device index %d out of range", dev);
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (g_dev_state[dev] == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
        g_dev_state[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    }
    if (g_dev_state[dev] != 1) return fail(MOGA_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
    return MOGA_OK;
}

// ---------------------------------------------------------------- validation
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

moga_status check_dims(const moga_dims *d) {
    if (!d) return fail(MOGA_ERR_ARG, "dims is NULL");
    if (d->n_tokens < 1 || d->n_tokens >= (int64_t(1) << 31))
        return fail(MOGA_ERR_ARG, "n_tokens %lld outside [1, 2^31)", (long long)d->n_tokens);
    if (d->d_model < 1 || d->d_model > kMaxDModel)
        return fail(MOGA_ERR_ARG, "d_model %d outside [1, %d]", d->d_model, kMaxDModel);
    if (d->n_heads < 1) return fail(MOGA_ERR_ARG, "n_heads %d < 1", d->n_heads);
    if (d->head_dim != 64 && d->head_dim != 128)
        return fail(MOGA_ERR_ARG, "head_dim %d is not 64 or 128", d->head_dim);
    if (d->n_groups < 1 || d->n_groups > kMaxGroups)
        return fail(MOGA_ERR_ARG, "n_groups %d outside [1, %d]", d->n_groups, kMaxGroups);
    if (!std::isfinite(d->softmax_scale)) return fail(MOGA_ERR_ARG, "softmax_scale is not finite");
    if (!std::isfinite(d->alpha)) return fail(MOGA_ERR_ARG, "alpha is not finite");
    // the attention work list is indexed with 32-bit integers on the device
    if (attn_max_items(d->n_heads, d->n_tokens, d->n_groups) >= (int64_t(1) << 31))
        return fail(MOGA_ERR_ARG, "n_heads x query tiles reaches 2^31 attention work items");
    return MOGA_OK;
}

float scale_of(const moga_dims *d) {
    return d->softmax_scale > 0.0f ? d->softmax_scale : 1.0f / std::sqrt((float)d->head_dim);
}

moga_status check_stga(const moga_dims *d, const stga_layout *s, StgaGeom *g) {
    if (!s) return fail(MOGA_ERR_ARG, "stga layout is NULL");
    if (s->frames < 1 || s->height < 1 || s->width < 1)
        return fail(MOGA_ERR_ARG, "stga grid %dx%dx%d has an empty side", s->frames, s->height, s->width);
    if ((int64_t)s->frames * s->height * s->width != d->n_tokens)
        return fail(MOGA_ERR_ARG, "frames*height*width = %lld != n_tokens %lld",
                    (long long)((int64_t)s->frames * s->height * s->width), (long long)d->n_tokens);
    if (s->n_shots < 1 || s->n_shots > kMaxShots)
        return fail(MOGA_ERR_ARG, "n_shots %d outside [1, %d]", s->n_shots, kMaxShots);
    if (!s->shot_start) return fail(MOGA_ERR_ARG, "shot_start is NULL");
    if (s->shot_start[0] != 0 || s->shot_start[s->n_shots] != s->frames)
        return fail(MOGA_ERR_ARG, "shot_start must begin at 0 and end at frames");
    for (int i = 0; i < s->n_shots; ++i)
        if (s->shot_start[i + 1] <= s->shot_start[i])
            return fail(MOGA_ERR_ARG, "shot_start is not strictly increasing at %d", i);
    if (s->win_h < 1 || s->win_w < 1 || s->height % s->win_h || s->width % s->win_w)
        return fail(MOGA_ERR_ARG, "window %dx%d does not tile the %dx%d frame", s->win_h, s->win_w,
                    s->height, s->width);
    if (s->t_group < 1) return fail(MOGA_ERR_ARG, "t_group %d < 1", s->t_group);
    if (s->aug_frames < 0) return fail(MOGA_ERR_ARG, "aug_frames %d < 0", s->aug_frames);
    std::memset(g, 0, sizeof *g);
    g->frames = s->frames; g->height = s->height; g->width = s->width; g->n_shots = s->n_shots;
    g->win_h = s->win_h; g->win_w = s->win_w; g->t_group = s->t_group; g->aug = s->aug_frames;
    for (int i = 0; i <= s->n_shots; ++i) g->shot_start[i] = s->shot_start[i];
    if (d->n_tokens + stga_extra_rows(*g) >= (int64_t(1) << 31))
        return fail(MOGA_ERR_ARG, "n_tokens plus borrowed key rows reaches 2^31");
    const int32_t segs = std::max(stga_n_groups(*g), g->frames);
    if (attn_max_items(d->n_heads, d->n_tokens, segs) >= (int64_t(1) << 31))
        return fail(MOGA_ERR_ARG, "n_heads x stga query tiles reaches 2^31 attention work items");
    return MOGA_OK;
}

// ---------------------------------------------------------------- workspace
size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

// query rows of an attention launch whose kernel may split key ranges (head_dim 128)
int64_t split_rows(const moga_dims *d, int64_t len_q) {
    return d->head_dim == 128 ? (int64_t)d->n_heads * len_q : 0;
}

struct Carver {
    size_t off = 0;
    size_t take(size_t bytes) {
        const size_t o = off;
        off += align256(bytes);
        return o;
    }
};

struct Layout {
    // MoGA
    size_t part_p, part_c, wsplit, gid, psel, counts, probsum, cu, perm, table, base_rel, totals, pperm;
    size_t qp, kp, vp, plan;
    // STGA
    size_t shot_info, cu_tq, cu_tk, cu_f, q_idx, kv_idx, ot, of;
    int32_t plan_seg;
    int64_t plan_items;
    size_t total;
};

Layout make_layout(const moga_dims *d, const StgaGeom *g) {
    Layout L{};
    Carver c;
    const int64_t n = d->n_tokens;
    const int m = d->n_groups;
    const int64_t nbr = route_partials(n), nbp = permute_blocks(n);
    const size_t tensor = (size_t)d->n_heads * n * d->head_dim * sizeof(uint16_t);
    L.part_p = c.take(sizeof(double) * nbr * kMaxGroups);
    L.part_c = c.take(sizeof(int32_t) * nbr * kMaxGroups);
    L.wsplit = c.take(route_split_bytes(d->d_model, m));
    L.gid = c.take(sizeof(int32_t) * n);
    L.psel = c.take(sizeof(float) * n);
    L.counts = c.take(sizeof(int32_t) * m);
    L.probsum = c.take(sizeof(double) * m);
    L.cu = c.take(sizeof(int32_t) * (m + 1));
    L.perm = c.take(sizeof(int32_t) * n);
    L.table = c.take(sizeof(int32_t) * nbp * m);
    L.base_rel = c.take(sizeof(int32_t) * nbp * m);
    L.totals = c.take(sizeof(int32_t) * m);
    L.pperm = c.take(sizeof(float) * n);
    L.qp = c.take(tensor);
    L.kp = c.take(tensor);
    L.vp = c.take(tensor);
    int32_t seg = m;
    int64_t items = attn_max_items(d->n_heads, n, m);
    if (g) {
        const int32_t ng = stga_n_groups(*g);
        const int64_t extra = stga_extra_rows(*g);
        L.shot_info = c.take(sizeof(int32_t) * 6 * g->n_shots);
        L.cu_tq = c.take(sizeof(int32_t) * (ng + 1));
        L.cu_tk = c.take(sizeof(int32_t) * (ng + 1));
        L.cu_f = c.take(sizeof(int32_t) * (g->frames + 1));
        L.q_idx = c.take(sizeof(int32_t) * n);
        L.kv_idx = c.take(sizeof(int32_t) * (n + extra));
        L.ot = c.take(tensor);
        L.of = c.take(tensor);
        seg = std::max(seg, std::max(ng, g->frames));
        items = std::max(items, std::max(attn_max_items(d->n_heads, n, ng),
                                         attn_max_items(d->n_heads, n, g->frames)));
    }
    L.plan_seg = seg;
    L.plan_items = items;
    L.plan = c.take(attn_plan_bytes(seg, items, split_rows(d, n)));
    L.total = c.off;
    return L;
}

// backward: token-order D and dp, group-order copies of everything the attention backward
// reads and writes, the router's dr and dW partials, and the attention plan.  With a STGA
// layout (hybrid backward) the copies of K and V also hold the borrowed key rows of the
// temporal groups, and the temporal branch's dQ, dK, dV (position order), its index maps and
// each token's positions in them come on top; the per-frame branch reuses the MoGA copies.
struct BwdLayout {
    size_t D, dp, Dp, lse2p, qp, kp, vp, dov, dqp, dkp, dvp, dr, dw_part;
    size_t shot_info, cu_tq, cu_tk, cu_f, q_idx, kv_idx, tpos, dqt, dkt, dvt, plan;
    int32_t plan_seg;
    int64_t plan_items;
    size_t total;
};

BwdLayout make_bwd_layout(const moga_dims *d, const StgaGeom *g = nullptr) {
    BwdLayout B{};
    Carver c;
    const int64_t n = d->n_tokens;
    const int64_t nk = g ? n + stga_extra_rows(*g) : n;  // key rows of the widest launch
    const size_t rows = sizeof(float) * d->n_heads * n;
    // the backward kernels work on 128-channel rows (head_dim 64 is widened with zeros)
    const size_t row_bytes = (size_t)d->n_heads * 128 * sizeof(uint16_t);
    const size_t tensor = row_bytes * n, ktensor = row_bytes * nk;
    B.D = c.take(rows);
    B.dp = c.take(sizeof(float) * n);
    B.Dp = c.take(rows);
    B.lse2p = c.take(rows);
    B.qp = c.take(tensor);
    B.kp = c.take(ktensor);
    B.vp = c.take(ktensor);
    B.dov = c.take(tensor);
    B.dqp = c.take(tensor);
    B.dkp = c.take(tensor);
    B.dvp = c.take(tensor);
    B.dr = c.take(sizeof(float) * n * d->n_groups);
    B.dw_part = c.take(sizeof(float) * bwd_dw_chunks(n) * d->d_model * d->n_groups);
    B.plan_seg = d->n_groups;
    if (g) {
        const int32_t ng = stga_n_groups(*g);
        B.shot_info = c.take(sizeof(int32_t) * 6 * g->n_shots);
        B.cu_tq = c.take(sizeof(int32_t) * (ng + 1));
        B.cu_tk = c.take(sizeof(int32_t) * (ng + 1));
        B.cu_f = c.take(sizeof(int32_t) * (g->frames + 1));
        B.q_idx = c.take(sizeof(int32_t) * n);
        B.kv_idx = c.take(sizeof(int32_t) * nk);
        B.tpos = c.take(sizeof(int32_t) * 4 * n);
        B.dqt = c.take(tensor);
        B.dkt = c.take(ktensor);
        B.dvt = c.take(ktensor);
        B.plan_seg = std::max(B.plan_seg, std::max(ng, g->frames));
    }
    // the dK/dV kernel's items run over key tiles, of which the temporal groups have more
    B.plan_items = attn_max_items(d->n_heads, nk, B.plan_seg);
    B.plan = c.take(attn_plan_bytes(B.plan_seg, B.plan_items, 0));
    B.total = c.off;
    return B;
}

template <typename T>
T *at(void *ws, size_t off) {
    return reinterpret_cast<T *>(static_cast<char *>(ws) + off);
}

moga_status check_ws(void *ws, size_t have, size_t need) {
    if (!ws) return fail(MOGA_ERR_WORKSPACE, "workspace is NULL");
    if (have < need)
        return fail(MOGA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", have, need);
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
        return fail(MOGA_ERR_WORKSPACE, "workspace is not 256-byte aligned");
    return MOGA_OK;
}

moga_status check_route_args(const void *x, moga_dtype xt, const float *w, const moga_dims *d) {
    if (!x || !w) return fail(MOGA_ERR_ARG, "x or w is NULL");
    if (xt != MOGA_F32 && xt != MOGA_BF16) return fail(MOGA_ERR_ARG, "x_dtype %d unknown", (int)xt);
    const int vec = xt == MOGA_BF16 ? 8 : 4;
    if (d->d_model % vec)
        return fail(MOGA_ERR_UNSUPPORTED, "d_model %d is not a multiple of %d", d->d_model, vec);
    if (!aligned16(x)) return fail(MOGA_ERR_ARG, "x is not 16-byte aligned");
    return MOGA_OK;
}

moga_status run_route(const void *x, moga_dtype xt, const float *w, const int32_t *pin,
                      const moga_dims *d, int32_t *gid, float *psel, int32_t *counts,
                      double *prob_sum, void *ws, const Layout &L, hipStream_t s) {
    RouteLaunch r{};
    r.x = x; r.x_is_bf16 = xt == MOGA_BF16; r.w = w; r.pin = pin; r.n = d->n_tokens;
    r.d = d->d_model; r.m = d->n_groups; r.group_id = gid; r.p_sel = psel;
    r.part_p = at<double>(ws, L.part_p); r.part_c = at<int32_t>(ws, L.part_c);
    r.counts = counts; r.prob_sum = prob_sum; r.wsplit = at<void>(ws, L.wsplit);
    HIP_TRY(launch_route(r, s), "route launch");
    return MOGA_OK;
}

moga_status run_perm_index(const int32_t *gid, const moga_dims *d, int32_t *cu, int32_t *perm,
                           void *ws, const Layout &L, hipStream_t s) {
    PermuteLaunch p{};
    p.group_id = gid; p.n = d->n_tokens; p.m = d->n_groups;
    p.table = at<int32_t>(ws, L.table); p.base_rel = at<int32_t>(ws, L.base_rel);
    p.totals = at<int32_t>(ws, L.totals); p.cu = cu; p.perm = perm;
    HIP_TRY(launch_perm_index(p, s), "permute index launch");
    return MOGA_OK;
}

moga_status run_gather(int inverse, const int32_t *perm, const moga_dims *d,
                       const void *const *src, void *const *dst, int nt, const float *p_sel,
                       float *p_perm, hipStream_t s) {
    GatherLaunch g{};
    for (int i = 0; i < nt; ++i) { g.src[i] = src[i]; g.dst[i] = dst[i]; }
    g.n_tensors = nt; g.perm = perm; g.n = d->n_tokens; g.n_heads = d->n_heads;
    g.head_dim = d->head_dim; g.inverse = inverse; g.p_sel = p_sel; g.p_perm = p_perm;
    HIP_TRY(launch_gather(g, s), "gather launch");
    return MOGA_OK;
}

// Optional parts of an attention launch's epilogue: output rows through a map, the log-sum-exp,
// and the mean with two other branches' rows (and the row before the mean).
struct AttnEpilogue {
    const int32_t *o_idx = nullptr;
    float *lse = nullptr;
    const void *mean_a = nullptr, *mean_b = nullptr;
    void *o_raw = nullptr;
};

moga_status run_attn(const void *q, const void *k, const void *v, void *o, const int32_t *cu_q,
                     const int32_t *cu_k, int32_t n_seg, const int32_t *q_idx,
                     const int32_t *kv_idx, const float *row_scale, int64_t len_q, int64_t len_k,
                     int64_t q_rows, int64_t kv_rows, int64_t o_rows, const moga_dims *d,
                     void *plan_mem, int32_t plan_seg, int64_t plan_items, int waves,
                     hipStream_t s, const AttnEpilogue &ep = AttnEpilogue()) {
    AttnLaunch a{};
    a.q = static_cast<const bf16 *>(q); a.k = static_cast<const bf16 *>(k);
    a.v = static_cast<const bf16 *>(v); a.o = static_cast<bf16 *>(o);
    a.cu_q = cu_q; a.cu_k = cu_k; a.n_seg = n_seg; a.q_idx = q_idx; a.kv_idx = kv_idx;
    a.row_scale = row_scale; a.len_q = len_q; a.len_k = len_k;
    a.q_rows = q_rows; a.kv_rows = kv_rows; a.o_rows = o_rows;
    a.n_heads = d->n_heads; a.head_dim = d->head_dim; a.scale = scale_of(d);
    a.max_items = attn_max_items(d->n_heads, len_q, n_seg);
    a.waves = waves;
    a.lse = ep.lse;
    a.o_idx = ep.o_idx;
    a.mean_a = static_cast<const bf16 *>(ep.mean_a);
    a.mean_b = static_cast<const bf16 *>(ep.mean_b);
    a.o_raw = static_cast<bf16 *>(ep.o_raw);
    if (a.max_items > plan_items || n_seg > plan_seg)
        return fail(MOGA_ERR_WORKSPACE, "attention plan larger than its workspace region");
    attn_plan_carve(a.plan, plan_mem, n_seg, a.max_items, split_rows(d, len_q));
    HIP_TRY(launch_attention(a, s), "attention launch");
    return MOGA_OK;
}

// The two STGA branches (token order); lse_t, lse_f: NULL or [H][N] normalisers of each.
moga_status run_stga(const void *q, const void *k, const void *v, const moga_dims *d,
                     const StgaGeom &g, void *o_t, void *o_f, void *ws, const Layout &L,
                     hipStream_t s, float *lse_t = nullptr, float *lse_f = nullptr) {
    StgaBuffers b{};
    b.shot_info = at<int32_t>(ws, L.shot_info); b.cu_tq = at<int32_t>(ws, L.cu_tq);
    b.cu_tk = at<int32_t>(ws, L.cu_tk); b.cu_f = at<int32_t>(ws, L.cu_f);
    b.q_idx = at<int32_t>(ws, L.q_idx); b.kv_idx = at<int32_t>(ws, L.kv_idx);
    HIP_TRY(launch_stga_index(g, b, s), "stga index launch");
    const int64_t n = d->n_tokens;
    void *plan = at<char>(ws, L.plan);
    if (o_t) {
        const int32_t ng = stga_n_groups(g);
        AttnEpilogue ep;
        ep.lse = lse_t;
        moga_status st = run_attn(q, k, v, o_t, b.cu_tq, b.cu_tk, ng, b.q_idx, b.kv_idx, nullptr, n,
                                  n + stga_extra_rows(g), n, n, n, d, plan, L.plan_seg,
                                  L.plan_items, 4, s, ep);
        if (st != MOGA_OK) return st;
    }
    if (o_f) {
        AttnEpilogue ep;
        ep.lse = lse_f;
        moga_status st = run_attn(q, k, v, o_f, b.cu_f, b.cu_f, g.frames, nullptr, nullptr, nullptr,
                                  n, n, n, n, n, d, plan, L.plan_seg, L.plan_items, 4, s, ep);
        if (st != MOGA_OK) return st;
    }
    return MOGA_OK;
}

moga_status check_group_attn(const void *q, const void *k, const void *v, int64_t len_q,
                             int64_t len_k, int32_t n_seg, const int32_t *cu_q,
                             const int32_t *cu_k, const moga_dims *dims, const void *o,
                             size_t *need) {
    moga_status st = check_dims(dims);
    if (st != MOGA_OK) return st;
    if (!q || !k || !v || !o || !cu_q || !cu_k) return fail(MOGA_ERR_ARG, "a required pointer is NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return fail(MOGA_ERR_ARG, "q, k, v and o must be 16-byte aligned");
    if (len_q < 0 || len_q >= (int64_t(1) << 31) || len_k < 0 || len_k >= (int64_t(1) << 31))
        return fail(MOGA_ERR_ARG, "len_q/len_k outside [0, 2^31)");
    if (n_seg < 1) return fail(MOGA_ERR_ARG, "n_seg %d < 1", n_seg);
    const int64_t items = attn_max_items(dims->n_heads, len_q, n_seg);
    if (items >= (int64_t(1) << 31)) return fail(MOGA_ERR_ARG, "too many work items");
    *need = attn_plan_bytes(n_seg, items, split_rows(dims, len_q));
    return MOGA_OK;
}

// The launch of moga_group_attn on a validated call; plan_mem holds attn_plan_bytes of room.
moga_status run_group_attn(const void *q, const void *k, const void *v, int64_t len_q,
                           int64_t len_k, int32_t n_seg, const int32_t *cu_q, const int32_t *cu_k,
                           const float *row_scale, const moga_dims *dims, void *o,
                           void *plan_mem, hipStream_t s) {
    const int64_t items = attn_max_items(dims->n_heads, len_q, n_seg);
    // long segments on average: 256-row query tiles; short ones: 128
    const int waves = len_q / n_seg >= 1024 ? 8 : 4;
    return run_attn(q, k, v, o, cu_q, cu_k, n_seg, nullptr, nullptr, row_scale, len_q, len_k, len_q,
                    len_k, len_q, dims, plan_mem, n_seg, items, waves, s);
}

moga_status check_bwd_args(const moga_inputs *in, const moga_saved *saved, const void *d_out,
                           double d_loss, const moga_dims *dims, const moga_grads *grads) {
    moga_status st = check_dims(dims);
    if (st != MOGA_OK) return st;
    if (!in || !saved || !grads) return fail(MOGA_ERR_ARG, "inputs, saved or grads is NULL");
    if ((st = check_route_args(in->x, in->x_dtype, in->w, dims)) != MOGA_OK) return st;
    if (!in->q || !in->k || !in->v || !d_out) return fail(MOGA_ERR_ARG, "q, k, v or d_out is NULL");
    if (!saved->group_id || !saved->p_sel || !saved->counts || !saved->cu_seqlens ||
        !saved->perm || !saved->out || !saved->lse)
        return fail(MOGA_ERR_ARG, "a saved forward tensor is NULL");
    if (!grads->dq || !grads->dk || !grads->dv) return fail(MOGA_ERR_ARG, "dq, dk or dv is NULL");
    const void *vec[8] = {in->q, in->k, in->v, d_out, saved->out, grads->dq, grads->dk, grads->dv};
    for (const void *p : vec)
        if (!aligned16(p)) return fail(MOGA_ERR_ARG, "q, k, v, d_out, out, dq, dk, dv must be 16-byte aligned");
    if ((grads->dx && !aligned16(grads->dx)) || (grads->dw && !aligned16(grads->dw)))
        return fail(MOGA_ERR_ARG, "dx and dw must be 16-byte aligned");
    if (!std::isfinite(d_loss)) return fail(MOGA_ERR_ARG, "d_loss is not finite");
    return MOGA_OK;
}

// The MoGA backward on a validated call: out_m and lse_m are the MoGA branch's rows (p-scaled)
// and normalisers, dp_scale the factor of the branch in the objective's output (1, or 1/3 under
// the hybrid mean), applied to dp only: dQ, dK, dV come out for the unscaled G.
moga_status run_moga_bwd(const moga_inputs *in, const moga_saved *saved, const void *out_m,
                         const float *lse_m, const void *d_out, double d_loss, float dp_scale,
                         const moga_dims *dims, const moga_grads *grads, void *ws,
                         const BwdLayout &B, hipStream_t s) {
    moga_status st;
    const int64_t n = dims->n_tokens;
    const int nh = dims->n_heads, m = dims->n_groups, hd = dims->head_dim;
    const int32_t *perm = saved->perm;

    // D = <G, out> per (head, token) row; dp = dp_scale * sum over heads of D / p
    float *D = at<float>(ws, B.D);
    float *dp = grads->dp ? grads->dp : at<float>(ws, B.dp);
    HIP_TRY(launch_bwd_rowdot(static_cast<const bf16 *>(d_out), static_cast<const bf16 *>(out_m),
                              (int64_t)nh * n, hd, D, s),
            "row dot launch");
    HIP_TRY(launch_bwd_dp(D, saved->p_sel, n, nh, dp_scale, dp, s), "dp launch");
    // group order: Q, K, V; dO' = p * G; D; lse in base 2 (head_dim 64: rows widened to 128)
    void *qp = at<char>(ws, B.qp), *kp = at<char>(ws, B.kp), *vp = at<char>(ws, B.vp);
    void *dov = at<char>(ws, B.dov);
    if (hd == 128) {
        const void *src[3] = {in->q, in->k, in->v};
        void *dst[3] = {qp, kp, vp};
        if ((st = run_gather(0, perm, dims, src, dst, 3, nullptr, nullptr, s)) != MOGA_OK) return st;
        GatherLaunch g{};
        g.src[0] = d_out; g.dst[0] = dov; g.n_tensors = 1; g.perm = perm; g.n = n;
        g.n_heads = nh; g.head_dim = hd; g.inverse = 0; g.src_scale = saved->p_sel;
        HIP_TRY(launch_gather(g, s), "scaled gather launch");
    } else {
        const void *src[4] = {in->q, in->k, in->v, d_out};
        void *dst[4] = {qp, kp, vp, dov};
        for (int i = 0; i < 4; ++i)
            HIP_TRY(launch_pad_rows(static_cast<const bf16 *>(src[i]), n, perm,
                                    i == 3 ? saved->p_sel : nullptr, n, nh,
                                    static_cast<bf16 *>(dst[i]), s),
                    "widening gather launch");
    }
    float *Dp = at<float>(ws, B.Dp), *lse2p = at<float>(ws, B.lse2p);
    HIP_TRY(launch_bwd_gather_f32(D, perm, n, nh, 1.0f, 0, Dp, s), "D gather launch");
    HIP_TRY(launch_bwd_gather_f32(lse_m, perm, n, nh, 1.4426950408889634f, 0, lse2p, s),
            "lse gather launch");
    // attention backward per group
    void *dqp = at<char>(ws, B.dqp), *dkp = at<char>(ws, B.dkp), *dvp = at<char>(ws, B.dvp);
    {
        AttnBwdLaunch a{};
        a.q = static_cast<const bf16 *>(qp); a.k = static_cast<const bf16 *>(kp);
        a.v = static_cast<const bf16 *>(vp); a.dov = static_cast<const bf16 *>(dov);
        a.lse2 = lse2p; a.D = Dp;
        a.dq = static_cast<bf16 *>(dqp); a.dk = static_cast<bf16 *>(dkp);
        a.dv = static_cast<bf16 *>(dvp);
        a.cu_q = a.cu_k = saved->cu_seqlens; a.n_seg = m; a.len_q = a.len_k = n; a.n_heads = nh;
        a.scale = scale_of(dims);
        a.max_items = B.plan_items;
        attn_plan_carve(a.plan, at<char>(ws, B.plan), B.plan_seg, B.plan_items, 0);
        HIP_TRY(launch_attention_bwd(a, s), "attention backward launch");
    }
    // back to token order
    {
        const void *gsrc[3] = {dqp, dkp, dvp};
        void *gdst[3] = {grads->dq, grads->dk, grads->dv};
        if (hd == 128) {
            if ((st = run_gather(1, perm, dims, gsrc, gdst, 3, nullptr, nullptr, s)) != MOGA_OK)
                return st;
        } else {
            for (int i = 0; i < 3; ++i)
                HIP_TRY(launch_unpad_rows(static_cast<const bf16 *>(gsrc[i]), perm, n, n, nh,
                                          static_cast<bf16 *>(gdst[i]), s),
                        "narrowing scatter launch");
        }
    }
    // router: softmax backward, dx, dW
    if (grads->dx || grads->dw) {
        BwdRouterLaunch r{};
        r.x = in->x; r.x_is_bf16 = in->x_dtype == MOGA_BF16; r.w = in->w; r.n = n;
        r.d = dims->d_model; r.m = m; r.group_id = saved->group_id; r.counts = saved->counts;
        r.dp = dp;
        r.loss_coef = (float)(d_loss * dims->alpha * m / ((double)n * (double)n));
        r.dr = at<float>(ws, B.dr); r.dx = grads->dx; r.dw = grads->dw;
        r.dw_part = at<float>(ws, B.dw_part);
        HIP_TRY(launch_router_bwd(r, s), "router backward launch");
    }
    return MOGA_OK;
}

// ---------------------------------------------------------------- library-owned scratch
// moga_group_attn_noalloc keeps its attention plan (segment tables, work list, dispatch
// counters and the split parts' rows) in this array instead of a caller workspace.  Every
// device the library runs on holds its own copy until the process ends, and every call on a
// device shares it.  On the host the array's name denotes a host-side stand-in, so host code
// only ever uses the device address hipGetSymbolAddress returns for the current device.
constexpr size_t kNoAllocScratchBytes = size_t(40) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

struct ScratchSlot {
    std::once_flag once;
    void *ptr = nullptr;
    hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[64];

// Device address of the current device's copy of `scratch`, looked up once per device with
// that device current.
moga_status scratch_address(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= 64) return fail(MOGA_ERR_UNSUPPORTED, "device index %d out of range", dev);
    ScratchSlot &slot = g_scratch[dev];
    std::call_once(slot.once, [&slot] {
        void *p = nullptr;
        slot.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (slot.err == hipSuccess) slot.ptr = p;
    });
    if (slot.err != hipSuccess) return hip_fail(slot.err, "hipGetSymbolAddress(scratch)");
    if (!slot.ptr || (reinterpret_cast<uintptr_t>(slot.ptr) & 255u) != 0)
        return fail(MOGA_ERR_HIP, "static scratch has no 256-byte aligned device address");
    *out = slot.ptr;
    return MOGA_OK;
}

}  // namespace

extern "C" {

const char *moga_last_error(void) { return g_err.c_str(); }

size_t moga_workspace_bytes(const moga_dims *dims, const stga_layout *stga) {
    if (check_dims(dims) != MOGA_OK) return 0;
    StgaGeom g;
    if (stga && check_stga(dims, stga, &g) != MOGA_OK) return 0;
    return make_layout(dims, stga ? &g : nullptr).total;
}

size_t moga_group_attn_workspace_bytes(const moga_dims *dims, int32_t n_seg, int64_t len_q) {
    if (check_dims(dims) != MOGA_OK || n_seg < 1 || len_q < 0) return 0;
    return attn_plan_bytes(n_seg, attn_max_items(dims->n_heads, len_q, n_seg), split_rows(dims, len_q));
}

moga_status moga_route(const void *x, moga_dtype x_dtype, const float *w, const int32_t *pin,
                       const moga_dims *dims, int32_t *group_id, float *p_sel, int32_t *counts,
                       double *prob_sum, void *ws, size_t ws_bytes, void *stream) {
    moga_status st = check_dims(dims);
    if (st != MOGA_OK) return st;
    if ((st = check_route_args(x, x_dtype, w, dims)) != MOGA_OK) return st;
    if (!group_id || !p_sel || !counts || !prob_sum)
        return fail(MOGA_ERR_ARG, "an output pointer is NULL");
    const Layout L = make_layout(dims, nullptr);
    if ((st = check_ws(ws, ws_bytes, L.gid)) != MOGA_OK) return st;  // the router partials only
    if ((st = check_device()) != MOGA_OK) return st;
    return run_route(x, x_dtype, w, pin, dims, group_id, p_sel, counts, prob_sum, ws, L,
                     static_cast<hipStream_t>(stream));
}

moga_status moga_permute(int inverse, const int32_t *group_id, const moga_dims *dims,
                         int32_t *cu_seqlens, int32_t *perm, const void *const *src,
                         void *const *dst, int n_tensors, const float *p_sel, float *p_perm,
                         void *ws, size_t ws_bytes, void *stream) {
    moga_status st = check_dims(dims);
    if (st != MOGA_OK) return st;
    if (inverse != 0 && inverse != 1) return fail(MOGA_ERR_ARG, "inverse must be 0 or 1");
    if (!perm) return fail(MOGA_ERR_ARG, "perm is NULL");
    if (!inverse && (!group_id || !cu_seqlens))
        return fail(MOGA_ERR_ARG, "group_id or cu_seqlens is NULL");
    if (n_tensors < 0 || n_tensors > 4) return fail(MOGA_ERR_ARG, "n_tensors %d outside [0, 4]", n_tensors);
    if (n_tensors > 0 && (!src || !dst)) return fail(MOGA_ERR_ARG, "src or dst is NULL");
    for (int i = 0; i < n_tensors; ++i) {
        if (!src[i] || !dst[i]) return fail(MOGA_ERR_ARG, "tensor %d pointer is NULL", i);
        if (!aligned16(src[i]) || !aligned16(dst[i]))
            return fail(MOGA_ERR_ARG, "tensor %d is not 16-byte aligned", i);
        if (src[i] == dst[i]) return fail(MOGA_ERR_ARG, "tensor %d: dst aliases src", i);
    }
    const Layout L = make_layout(dims, nullptr);
    if ((st = check_ws(ws, ws_bytes, L.pperm)) != MOGA_OK) return st;  // up to the scan tables
    if ((st = check_device()) != MOGA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!inverse && (st = run_perm_index(group_id, dims, cu_seqlens, perm, ws, L, s)) != MOGA_OK)
        return st;
    return run_gather(inverse, perm, dims, src, dst, n_tensors, inverse ? nullptr : p_sel,
                      inverse ? nullptr : p_perm, s);
}

moga_status moga_group_attn(const void *q, const void *k, const void *v, int64_t len_q,
                            int64_t len_k, int32_t n_seg, const int32_t *cu_q,
                            const int32_t *cu_k, const float *row_scale, const moga_dims *dims,
                            void *o, void *ws, size_t ws_bytes, void *stream) {
    size_t need = 0;
    moga_status st = check_group_attn(q, k, v, len_q, len_k, n_seg, cu_q, cu_k, dims, o, &need);
    if (st != MOGA_OK) return st;
    if ((st = check_ws(ws, ws_bytes, need)) != MOGA_OK) return st;
    if ((st = check_device()) != MOGA_OK) return st;
    return run_group_attn(q, k, v, len_q, len_k, n_seg, cu_q, cu_k, row_scale, dims, o, ws,
                          static_cast<hipStream_t>(stream));
}

moga_status moga_group_attn_noalloc(const void *q, const void *k, const void *v, int64_t len_q,
                                    int64_t len_k, int32_t n_seg, const int32_t *cu_q,
                                    const int32_t *cu_k, const float *row_scale,
                                    const moga_dims *dims, void *o, void *stream) {
    size_t need = 0;
    moga_status st = check_group_attn(q, k, v, len_q, len_k, n_seg, cu_q, cu_k, dims, o, &need);
    if (st != MOGA_OK) return st;
    if (need > kNoAllocScratchBytes)
        return fail(MOGA_ERR_WORKSPACE,
                    "moga_group_attn_noalloc: the attention plan needs %zu bytes and the "
                    "library's static scratch holds %zu (use moga_group_attn with a workspace)",
                    need, kNoAllocScratchBytes);
    if ((st = check_device()) != MOGA_OK) return st;
    void *scratch_dev = nullptr;
    if ((st = scratch_address(&scratch_dev)) != MOGA_OK) return st;
    return run_group_attn(q, k, v, len_q, len_k, n_seg, cu_q, cu_k, row_scale, dims, o,
                          scratch_dev, static_cast<hipStream_t>(stream));
}

moga_status stga_group_attn(const void *q, const void *k, const void *v, const moga_dims *dims,
                            const stga_layout *stga, void *o_temporal, void *o_frame, void *ws,
                            size_t ws_bytes, void *stream) {
    moga_status st = check_dims(dims);
    if (st != MOGA_OK) return st;
    StgaGeom g;
    if ((st = check_stga(dims, stga, &g)) != MOGA_OK) return st;
    if (!q || !k || !v) return fail(MOGA_ERR_ARG, "q, k or v is NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o_temporal) ||
        !aligned16(o_frame))
        return fail(MOGA_ERR_ARG, "tensors must be 16-byte aligned");
    const Layout L = make_layout(dims, &g);
    if ((st = check_ws(ws, ws_bytes, L.total)) != MOGA_OK) return st;
    if ((st = check_device()) != MOGA_OK) return st;
    return run_stga(q, k, v, dims, g, o_temporal, o_frame, ws, L, static_cast<hipStream_t>(stream));
}

moga_status moga_balance_loss(const int32_t *counts, const double *prob_sum,
                              const moga_dims *dims, double *loss, double *F, double *P,
                              void *stream) {
    moga_status st = check_dims(dims);
    if (st != MOGA_OK) return st;
    if (!counts || !prob_sum || !loss) return fail(MOGA_ERR_ARG, "counts, prob_sum or loss is NULL");
    if ((st = check_device()) != MOGA_OK) return st;
    HIP_TRY(launch_balance_loss(counts, prob_sum, dims->n_tokens, dims->n_groups, dims->alpha, loss,
                                F, P, static_cast<hipStream_t>(stream)),
            "loss launch");
    return MOGA_OK;
}

static moga_status forward_impl(const moga_inputs *in, const moga_dims *dims, const stga_layout *stga,
                         const moga_outputs *out, void *ws, size_t ws_bytes, void *stream,
                         bool fused) {
    moga_status st = check_dims(dims);
    if (st != MOGA_OK) return st;
    if (!in || !out) return fail(MOGA_ERR_ARG, "inputs or outputs is NULL");
    if ((st = check_route_args(in->x, in->x_dtype, in->w, dims)) != MOGA_OK) return st;
    if (!in->q || !in->k || !in->v) return fail(MOGA_ERR_ARG, "q, k or v is NULL");
    if (!out->out || !out->loss) return fail(MOGA_ERR_ARG, "out or loss is NULL");
    if (!aligned16(in->q) || !aligned16(in->k) || !aligned16(in->v) || !aligned16(out->out))
        return fail(MOGA_ERR_ARG, "q, k, v and out must be 16-byte aligned");
    StgaGeom g;
    if (stga && (st = check_stga(dims, stga, &g)) != MOGA_OK) return st;
    if (out->o_branches && !stga) return fail(MOGA_ERR_ARG, "o_branches needs a STGA layout");
    if (out->o_branches && !aligned16(out->o_branches))
        return fail(MOGA_ERR_ARG, "o_branches is not 16-byte aligned");
    if (stga && out->lse && !out->o_branches)
        return fail(MOGA_ERR_UNSUPPORTED,
                    "with a STGA layout lse holds the three branches' normalisers, which are "
                    "returned only together with o_branches (the rows the backward pairs them with)");
    const Layout L = make_layout(dims, stga ? &g : nullptr);
    if ((st = check_ws(ws, ws_bytes, L.total)) != MOGA_OK) return st;
    if ((st = check_device()) != MOGA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t n = dims->n_tokens;

    int32_t *gid = out->group_id ? out->group_id : at<int32_t>(ws, L.gid);
    float *psel = out->p_sel ? out->p_sel : at<float>(ws, L.psel);
    int32_t *counts = out->counts ? out->counts : at<int32_t>(ws, L.counts);
    double *probsum = out->prob_sum ? out->prob_sum : at<double>(ws, L.probsum);
    int32_t *cu = out->cu_seqlens ? out->cu_seqlens : at<int32_t>(ws, L.cu);
    int32_t *perm = out->perm ? out->perm : at<int32_t>(ws, L.perm);
    void *plan = at<char>(ws, L.plan);

    // 1 route  2 histogram/scan/stable permutation
    if ((st = run_route(in->x, in->x_dtype, in->w, in->pin, dims, gid, psel, counts, probsum, ws,
                        L, s)) != MOGA_OK)
        return st;
    if ((st = run_perm_index(gid, dims, cu, perm, ws, L, s)) != MOGA_OK) return st;
    // 3 group-balancing loss
    HIP_TRY(launch_balance_loss(counts, probsum, n, dims->n_groups, dims->alpha, out->loss, nullptr,
                                nullptr, s),
            "loss launch");
    // 4 with a STGA layout: the two static branches first, in token order; the MoGA epilogue
    // then stores the mean of the three rows (in fp32, one rounding)
    AttnEpilogue ep;
    ep.lse = out->lse;
    if (stga) {
        // o_branches given: the branch rows are stored there (MoGA row, temporal, per-frame),
        // and lse holds the three normalisers in the same plane order
        const size_t plane = (size_t)dims->n_heads * n * dims->head_dim * sizeof(uint16_t);
        char *ob = static_cast<char *>(out->o_branches);
        void *ot = ob ? ob + plane : at<char>(ws, L.ot), *of = ob ? ob + 2 * plane : at<char>(ws, L.of);
        float *lse_t = out->lse ? out->lse + (size_t)dims->n_heads * n : nullptr;
        float *lse_f = out->lse ? out->lse + 2 * (size_t)dims->n_heads * n : nullptr;
        if ((st = run_stga(in->q, in->k, in->v, dims, g, ot, of, ws, L, s, lse_t, lse_f)) != MOGA_OK)
            return st;
        ep.mean_a = ot;
        ep.mean_b = of;
        ep.o_raw = ob;
    }
    if (fused) {
        // 5 rows are read through perm and written back in token order
        if ((st = run_attn(in->q, in->k, in->v, out->out, cu, cu, dims->n_groups, perm, perm, psel,
                           n, n, n, n, n, dims, plan, L.plan_seg, L.plan_items, 8, s, ep)) !=
            MOGA_OK)
            return st;
    } else {
        // 5 gather Q, K, V and p by perm, then the varlen group attention scaled by p(g|x),
        // whose epilogue writes each row straight to its token (no separate inverse permute)
        float *pperm = at<float>(ws, L.pperm);
        void *qp = at<char>(ws, L.qp), *kp = at<char>(ws, L.kp), *vp = at<char>(ws, L.vp);
        const void *src[3] = {in->q, in->k, in->v};
        void *dst[3] = {qp, kp, vp};
        if ((st = run_gather(0, perm, dims, src, dst, 3, psel, pperm, s)) != MOGA_OK) return st;
        ep.o_idx = perm;
        if ((st = run_attn(qp, kp, vp, out->out, cu, cu, dims->n_groups, nullptr, nullptr, pperm, n,
                           n, n, n, n, dims, plan, L.plan_seg, L.plan_items, 8, s, ep)) != MOGA_OK)
            return st;
    }
    return MOGA_OK;
}

moga_status moga_forward(const moga_inputs *in, const moga_dims *dims, const stga_layout *stga,
                         const moga_outputs *out, void *ws, size_t ws_bytes, void *stream) {
    return forward_impl(in, dims, stga, out, ws, ws_bytes, stream, false);
}

moga_status moga_forward_fused(const moga_inputs *in, const moga_dims *dims,
                               const stga_layout *stga, const moga_outputs *out, void *ws,
                               size_t ws_bytes, void *stream) {
    return forward_impl(in, dims, stga, out, ws, ws_bytes, stream, true);
}

size_t moga_backward_workspace_bytes(const moga_dims *dims) {
    if (check_dims(dims) != MOGA_OK) return 0;
    return make_bwd_layout(dims).total;
}

size_t moga_hybrid_backward_workspace_bytes(const moga_dims *dims, const stga_layout *stga) {
    if (check_dims(dims) != MOGA_OK) return 0;
    StgaGeom g;
    if (check_stga(dims, stga, &g) != MOGA_OK) return 0;
    return make_bwd_layout(dims, &g).total;
}

moga_status moga_backward(const moga_inputs *in, const moga_saved *saved, const void *d_out,
                          double d_loss, const moga_dims *dims, const moga_grads *grads,
                          void *ws, size_t ws_bytes, void *stream) {
    moga_status st = check_bwd_args(in, saved, d_out, d_loss, dims, grads);
    if (st != MOGA_OK) return st;
    const BwdLayout B = make_bwd_layout(dims);
    if ((st = check_ws(ws, ws_bytes, B.total)) != MOGA_OK) return st;
    if ((st = check_device()) != MOGA_OK) return st;
    return run_moga_bwd(in, saved, saved->out, saved->lse, d_out, d_loss, 1.0f, dims, grads, ws, B,
                        static_cast<hipStream_t>(stream));
}

moga_status moga_hybrid_backward(const moga_inputs *in, const moga_saved *saved,
                                 const stga_layout *stga, const void *d_out, double d_loss,
                                 const moga_dims *dims, const moga_grads *grads, void *ws,
                                 size_t ws_bytes, void *stream) {
    moga_status st = check_bwd_args(in, saved, d_out, d_loss, dims, grads);
    if (st != MOGA_OK) return st;
    StgaGeom g;
    if ((st = check_stga(dims, stga, &g)) != MOGA_OK) return st;
    const BwdLayout B = make_bwd_layout(dims, &g);
    if ((st = check_ws(ws, ws_bytes, B.total)) != MOGA_OK) return st;
    if ((st = check_device()) != MOGA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t n = dims->n_tokens, nk = n + stga_extra_rows(g);
    const int nh = dims->n_heads, hd = dims->head_dim;
    const size_t plane = (size_t)nh * n * hd;  // elements of one branch's rows
    const bf16 *o_br = static_cast<const bf16 *>(saved->out);
    const float *lse_br = saved->lse;
    const float third = 1.0f / 3.0f;
    const float log2e = 1.4426950408889634f;

    // 1 the MoGA branch with G (dQ, dK, dV unscaled, to token order in grads); the router sees
    //   dp with the 1/3 of the mean and the loss term as is
    if ((st = run_moga_bwd(in, saved, o_br, lse_br, d_out, d_loss, third, dims, grads, ws, B, s)) !=
        MOGA_OK)
        return st;
    // 2 the STGA index maps and each token's positions in them
    StgaBuffers sb{};
    sb.shot_info = at<int32_t>(ws, B.shot_info); sb.cu_tq = at<int32_t>(ws, B.cu_tq);
    sb.cu_tk = at<int32_t>(ws, B.cu_tk); sb.cu_f = at<int32_t>(ws, B.cu_f);
    sb.q_idx = at<int32_t>(ws, B.q_idx); sb.kv_idx = at<int32_t>(ws, B.kv_idx);
    sb.tpos = at<int32_t>(ws, B.tpos);
    HIP_TRY(launch_stga_index(g, sb, s), "stga index launch");
    const bf16 *G = static_cast<const bf16 *>(d_out);
    float *D = at<float>(ws, B.D), *Dp = at<float>(ws, B.Dp), *lse2p = at<float>(ws, B.lse2p);
    AttnBwdLaunch a{};
    a.n_heads = nh;
    a.scale = scale_of(dims);
    a.max_items = B.plan_items;
    attn_plan_carve(a.plan, at<char>(ws, B.plan), B.plan_seg, B.plan_items, 0);
    // 3 per-frame branch, in token order (segments cu_f), with G: in place at head_dim 128,
    //   on rows widened to 128 channels in the MoGA copies' Q, K, V, dO' regions at 64; results
    //   in the MoGA copies' dQ, dK, dV regions
    bf16 *qt = at<bf16>(ws, B.qp), *kt = at<bf16>(ws, B.kp), *vt = at<bf16>(ws, B.vp);
    bf16 *dot = at<bf16>(ws, B.dov);
    bf16 *dqf = at<bf16>(ws, B.dqp), *dkf = at<bf16>(ws, B.dkp), *dvf = at<bf16>(ws, B.dvp);
    HIP_TRY(launch_bwd_rowdot(G, o_br + 2 * plane, (int64_t)nh * n, hd, D, s), "row dot launch");
    HIP_TRY(launch_bwd_gather_f32(lse_br + 2 * (size_t)nh * n, nullptr, n, nh, log2e, 0, lse2p, s),
            "lse scale launch");
    if (hd == 128) {
        a.q = static_cast<const bf16 *>(in->q); a.k = static_cast<const bf16 *>(in->k);
        a.v = static_cast<const bf16 *>(in->v); a.dov = G;
    } else {
        const void *src[4] = {in->q, in->k, in->v, d_out};
        bf16 *dst[4] = {qt, kt, vt, dot};
        for (int i = 0; i < 4; ++i)
            HIP_TRY(launch_pad_rows(static_cast<const bf16 *>(src[i]), n, nullptr, nullptr, n, nh,
                                    dst[i], s),
                    "widening copy launch");
        a.q = qt; a.k = kt; a.v = vt; a.dov = dot;
    }
    a.lse2 = lse2p; a.D = D;
    a.dq = dqf; a.dk = dkf; a.dv = dvf;
    a.cu_q = a.cu_k = sb.cu_f; a.n_seg = g.frames; a.len_q = a.len_k = n;
    HIP_TRY(launch_attention_bwd(a, s), "per-frame attention backward launch");
    // 4 temporal branch: Q, dO, D, lse to query positions, K and V to key positions (own rows
    //   and borrowed frames), the backward over the groups, results in position order
    if (hd == 128) {
        GatherLaunch gq{};
        gq.src[0] = in->q; gq.dst[0] = qt; gq.src[1] = d_out; gq.dst[1] = dot; gq.n_tensors = 2;
        gq.perm = sb.q_idx; gq.n = n; gq.n_heads = nh; gq.head_dim = dims->head_dim;
        HIP_TRY(launch_gather(gq, s), "temporal query gather launch");
        GatherLaunch gk{};
        gk.src[0] = in->k; gk.dst[0] = kt; gk.src[1] = in->v; gk.dst[1] = vt; gk.n_tensors = 2;
        gk.perm = sb.kv_idx; gk.n = nk; gk.src_rows = n; gk.n_heads = nh;
        gk.head_dim = dims->head_dim;
        HIP_TRY(launch_gather(gk, s), "temporal key gather launch");
    } else {
        HIP_TRY(launch_pad_rows(static_cast<const bf16 *>(in->q), n, sb.q_idx, nullptr, n, nh, qt,
                                s), "temporal query gather launch");
        HIP_TRY(launch_pad_rows(G, n, sb.q_idx, nullptr, n, nh, dot, s),
                "temporal query gather launch");
        HIP_TRY(launch_pad_rows(static_cast<const bf16 *>(in->k), n, sb.kv_idx, nullptr, nk, nh, kt,
                                s), "temporal key gather launch");
        HIP_TRY(launch_pad_rows(static_cast<const bf16 *>(in->v), n, sb.kv_idx, nullptr, nk, nh, vt,
                                s), "temporal key gather launch");
    }
    HIP_TRY(launch_bwd_rowdot(G, o_br + plane, (int64_t)nh * n, hd, D, s), "row dot launch");
    HIP_TRY(launch_bwd_gather_f32(D, sb.q_idx, n, nh, 1.0f, 0, Dp, s), "D gather launch");
    HIP_TRY(launch_bwd_gather_f32(lse_br + (size_t)nh * n, sb.q_idx, n, nh, log2e, 0, lse2p, s),
            "lse gather launch");
    bf16 *dqt = at<bf16>(ws, B.dqt), *dkt = at<bf16>(ws, B.dkt), *dvt = at<bf16>(ws, B.dvt);
    a.q = qt; a.k = kt; a.v = vt; a.dov = dot; a.lse2 = lse2p; a.D = Dp;
    a.dq = dqt; a.dk = dkt; a.dv = dvt;
    a.cu_q = sb.cu_tq; a.cu_k = sb.cu_tk; a.n_seg = stga_n_groups(g); a.len_q = n; a.len_k = nk;
    HIP_TRY(launch_attention_bwd(a, s), "temporal attention backward launch");
    // 5 the mean: grad = (MoGA + per-frame + temporal at the token's positions) / 3
    bf16 *dq = static_cast<bf16 *>(grads->dq), *dk = static_cast<bf16 *>(grads->dk),
         *dv = static_cast<bf16 *>(grads->dv);
    HIP_TRY(launch_grad_sum(dq, dqf, dqt, hd, 128, n, sb.tpos, 0, 1, n, nh, third, dq, s),
            "dQ sum launch");
    HIP_TRY(launch_grad_sum(dk, dkf, dkt, hd, 128, nk, sb.tpos, 1, 3, n, nh, third, dk, s),
            "dK sum launch");
    HIP_TRY(launch_grad_sum(dv, dvf, dvt, hd, 128, nk, sb.tpos, 1, 3, n, nh, third, dv, s),
            "dV sum launch");
    return MOGA_OK;
}

}  // extern "C"

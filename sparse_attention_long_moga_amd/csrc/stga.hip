// Spatial-temporal group attention (STGA) index maps and the group-balancing loss.
//
// STGA (papernotes.org MoGA note, 关键设计 4; jxzklqfsx.com translation, 時空分組注意力;
// xugj520.cn MoGA blog §3.2 and §9): the latent video is cut into fixed spatial windows,
// frames are grouped along time inside each shot, and the keys/values (not the queries)
// of a group that touches a shot boundary also take two latent frames of the adjacent
// shot.  A second static grouping is the whole frame.  Each token receives one dynamic
// (MoGA) and two static outputs and takes their mean (formed in the MoGA attention's
// epilogue).
//
// Temporal groups are enumerated (shot, chunk, window) and every offset has a closed
// form, so instead of gathering Q/K/V the attention kernel reads rows through two index
// maps built here:
//   q_idx[cu_tq[g] + r]  = token of query row r of group g (r in (frame, y, x) order)
//   kv_idx[cu_tk[g] + r] = token of key row r: the group's own rows, then the rows of
//                          the previous shot's last frames (first chunk of a shot), then
//                          the rows of the next shot's first frames (last chunk).
// The per-frame grouping is contiguous in frame-major token order: cu_f[f] = f*H*W.
// For the backward the same pass can also record, per token, the inverse of these maps: its
// query position and the (up to three) key positions that hold it.
#include "moga_internal.h"

namespace moga {
namespace {

// shot_info row: start, len, chunk_base, aug_base, aug_prev, aug_next
enum { SI_START = 0, SI_LEN, SI_CB, SI_AB, SI_AP, SI_AN, SI_W };

__global__ __launch_bounds__(256) void stga_prep_kernel(StgaGeom g, StgaBuffers b, int n_groups) {
    __shared__ int s_info[kMaxShots + 1][SI_W];
    const int S = g.n_shots;
    if (threadIdx.x == 0) {
        int cb = 0, ab = 0;
        for (int s = 0; s < S; ++s) {
            const int start = g.shot_start[s], len = g.shot_start[s + 1] - start;
            const int lp = s > 0 ? g.shot_start[s] - g.shot_start[s - 1] : 0;
            const int ln = s + 1 < S ? g.shot_start[s + 2] - g.shot_start[s + 1] : 0;
            const int ap = s > 0 ? (g.aug < lp ? g.aug : lp) : 0;
            const int an = s + 1 < S ? (g.aug < ln ? g.aug : ln) : 0;
            int *r = s_info[s];
            r[SI_START] = start; r[SI_LEN] = len; r[SI_CB] = cb; r[SI_AB] = ab;
            r[SI_AP] = ap; r[SI_AN] = an;
            cb += (len + g.t_group - 1) / g.t_group;
            ab += ap + an;
        }
        s_info[S][SI_CB] = cb;
        s_info[S][SI_AB] = ab;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < S * SI_W; i += 256) b.shot_info[i] = s_info[i / SI_W][i % SI_W];
    const int nwx = g.width / g.win_w, nwin = (g.height / g.win_h) * nwx;
    const int wt = g.win_h * g.win_w;
    const int64_t hw = (int64_t)g.height * g.width;
    for (int grp = threadIdx.x; grp < n_groups; grp += 256) {
        const int gc = grp / nwin, w = grp % nwin;
        int lo = 0, hi = S;  // chunk_base[lo] <= gc < chunk_base[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_info[mid][SI_CB] <= gc) lo = mid; else hi = mid;
        }
        const int *r = s_info[lo];
        const int c = gc - r[SI_CB];
        const int nch = s_info[lo + 1][SI_CB] - r[SI_CB];
        const int tf = r[SI_LEN] - c * g.t_group < g.t_group ? r[SI_LEN] - c * g.t_group : g.t_group;
        const int64_t qoff = (int64_t)(r[SI_START] + c * g.t_group) * hw + (int64_t)w * tf * wt;
        const int augf = (c == 0 ? r[SI_AP] : 0) + (c == nch - 1 ? r[SI_AN] : 0);
        const int aug_before = r[SI_AB] + (c > 0 ? r[SI_AP] : 0);
        const int64_t kaug = ((int64_t)aug_before * nwin + (int64_t)w * augf) * wt;
        b.cu_tq[grp] = (int32_t)qoff;
        b.cu_tk[grp] = (int32_t)(qoff + kaug);
    }
    if (threadIdx.x == 0) {
        b.cu_tq[n_groups] = (int32_t)(g.frames * hw);
        b.cu_tk[n_groups] = (int32_t)(g.frames * hw + (int64_t)s_info[S][SI_AB] * hw);
    }
    for (int f = threadIdx.x; f <= g.frames; f += 256) b.cu_f[f] = (int32_t)(f * hw);
}

__global__ __launch_bounds__(256) void stga_index_kernel(StgaGeom g, StgaBuffers b) {
    const int64_t hw = (int64_t)g.height * g.width;
    const int64_t n = g.frames * hw;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= n) return;
    const int S = g.n_shots;
    const int f = (int)(t / hw);
    const int rem = (int)(t % hw);
    const int y = rem / g.width, x = rem % g.width;
    int lo = 0, hi = S;  // start[lo] <= f < start[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (b.shot_info[mid * SI_W + SI_START] <= f) lo = mid; else hi = mid;
    }
    const int s = lo;
    const int *r = b.shot_info + s * SI_W;
    const int start = r[SI_START], len = r[SI_LEN];
    const int T = g.t_group;
    const int c = (f - start) / T;
    const int nwx = g.width / g.win_w, nwin = (g.height / g.win_h) * nwx;
    const int wy = y / g.win_h, wx = x / g.win_w, w = wy * nwx + wx;
    const int ly = y - wy * g.win_h, lx = x - wx * g.win_w;
    const int wt = g.win_h * g.win_w;
    const int grp = (r[SI_CB] + c) * nwin + w;
    const int row = ((f - (start + c * T)) * g.win_h + ly) * g.win_w + lx;
    const int32_t qpos = b.cu_tq[grp] + row, kpos = b.cu_tk[grp] + row;
    int32_t next_pos = -1, prev_pos = -1;
    b.q_idx[qpos] = (int32_t)t;
    b.kv_idx[kpos] = (int32_t)t;
    if (s + 1 < S) {  // borrowed by the first chunk of shot s+1
        const int *rn = b.shot_info + (s + 1) * SI_W;
        const int apn = rn[SI_AP];
        const int f0 = start + len - apn;
        if (f >= f0) {
            const int g2 = rn[SI_CB] * nwin + w;
            const int tf2 = rn[SI_LEN] < T ? rn[SI_LEN] : T;
            const int r2 = ((f - f0) * g.win_h + ly) * g.win_w + lx;
            next_pos = b.cu_tk[g2] + tf2 * wt + r2;
            b.kv_idx[next_pos] = (int32_t)t;
        }
    }
    if (s > 0) {  // borrowed by the last chunk of shot s-1
        const int *rp = b.shot_info + (s - 1) * SI_W;
        const int anp = rp[SI_AN];
        if (f < start + anp) {
            const int lastc = (rp[SI_LEN] + T - 1) / T - 1;
            const int g3 = (r[SI_CB] - 1) * nwin + w;
            const int tf3 = rp[SI_LEN] - lastc * T;
            const int prev_rows = (lastc == 0 ? rp[SI_AP] : 0) * wt;
            const int r3 = ((f - start) * g.win_h + ly) * g.win_w + lx;
            prev_pos = b.cu_tk[g3] + tf3 * wt + prev_rows + r3;
            b.kv_idx[prev_pos] = (int32_t)t;
        }
    }
    if (b.tpos)
        *reinterpret_cast<int4 *>(b.tpos + 4 * t) = make_int4(qpos, kpos, next_pos, prev_pos);
}

// Group-balancing loss (papernotes.org MoGA note, 关键设计 3): F_i = n_i / N,
// P_i = (sum over tokens of p(i|x)) / N, L = alpha * M * sum_i F_i P_i, in fp64.
__global__ void balance_loss_kernel(const int32_t *counts, const double *prob_sum, int64_t n,
                                    int m, double alpha, double *loss, double *F, double *P) {
    if (threadIdx.x != 0) return;
    double acc = 0.0;
    for (int i = 0; i < m; ++i) {
        const double f = (double)counts[i] / (double)n;
        const double p = prob_sum[i] / (double)n;
        if (F) F[i] = f;
        if (P) P[i] = p;
        acc += f * p;
    }
    *loss = alpha * (double)m * acc;
}

}  // namespace

int32_t stga_n_groups(const StgaGeom &g) {
    const int nwin = (g.height / g.win_h) * (g.width / g.win_w);
    int64_t chunks = 0;
    for (int s = 0; s < g.n_shots; ++s) {
        const int len = g.shot_start[s + 1] - g.shot_start[s];
        chunks += (len + g.t_group - 1) / g.t_group;
    }
    return (int32_t)(chunks * nwin);
}

int64_t stga_extra_rows(const StgaGeom &g) {
    int64_t frames = 0;
    for (int s = 0; s < g.n_shots; ++s) {
        const int lp = s > 0 ? g.shot_start[s] - g.shot_start[s - 1] : 0;
        const int ln = s + 1 < g.n_shots ? g.shot_start[s + 2] - g.shot_start[s + 1] : 0;
        frames += (s > 0 ? (g.aug < lp ? g.aug : lp) : 0) + (s + 1 < g.n_shots ? (g.aug < ln ? g.aug : ln) : 0);
    }
    return frames * g.height * g.width;
}

hipError_t launch_stga_index(const StgaGeom &g, const StgaBuffers &b, hipStream_t s) {
    const int ng = stga_n_groups(g);
    hipLaunchKernelGGL(stga_prep_kernel, dim3(1), dim3(256), 0, s, g, b, ng);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n = (int64_t)g.frames * g.height * g.width;
    hipLaunchKernelGGL(stga_index_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, g, b);
    return hipGetLastError();
}

hipError_t launch_balance_loss(const int32_t *counts, const double *prob_sum, int64_t n, int m,
                               double alpha, double *loss, double *F, double *P, hipStream_t s) {
    hipLaunchKernelGGL(balance_loss_kernel, dim3(1), dim3(64), 0, s, counts, prob_sum, n, m, alpha,
                       loss, F, P);
    return hipGetLastError();
}

}  // namespace moga

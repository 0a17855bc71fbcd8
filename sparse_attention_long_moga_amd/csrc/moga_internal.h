// Internal declarations shared by the HIP translation units of libmoga.so.
// Not part of the public ABI (that is include/moga.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

namespace moga {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxGroups = 64;    // M <= 64
constexpr int kMaxDModel = 1 << 20;  // router width d; keeps 32-bit buffer offsets in range
constexpr int kMaxShots = 256;    // STGA shots passed by value
constexpr int kAttnBQMin = 128;   // smallest query rows per attention work item (4 waves x 32)
constexpr int kAttnThreads = 256;
constexpr int kPermTokensPerBlock = 2048;
constexpr int64_t kFusedScanReads = int64_t(1) << 24;  // nblk^2 x m bound of the in-scatter scan
constexpr int kRouteTokensPerBlock = 256;
constexpr int kPlanSortMax = 4096; // segments sorted by key length up to this count

constexpr float kLog2e = 1.4426950408889634f;

constexpr int kMaxDevices = 64;

// Compute units of the current device (cached per device; thread-safe).
hipError_t device_cus(int *n);

// A set-up step run once per device, with that device current, the first time any thread asks
// for it there; later calls return the first call's status.  Thread-safe.
class DeviceOnce {
  public:
    template <typename F>
    hipError_t run(F &&f) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
        std::call_once(flag_[dev], [&] { status_[dev] = f(); });
        return status_[dev];
    }

  private:
    std::once_flag flag_[kMaxDevices];
    hipError_t status_[kMaxDevices] = {};
};

// ---------------------------------------------------------------- router
struct RouteLaunch {
    const void *x;
    int x_is_bf16;
    const float *w;
    const int32_t *pin;
    int64_t n;
    int d, m;
    int32_t *group_id;
    float *p_sel;
    double *part_p;   // [nblk][kMaxGroups]
    int32_t *part_c;  // [nblk][kMaxGroups]
    int32_t *counts;  // [m]
    double *prob_sum; // [m]
    void *wsplit;     // route_split_bytes(d, m): W split into bf16 MFMA fragments (bf16 x)
};
int64_t route_blocks(int64_t n);
int64_t route_partials(int64_t n);  // part_p / part_c hold route_partials(n) * kMaxGroups entries
size_t route_split_bytes(int d, int m);  // wsplit: fragments plus a work-queue counter
hipError_t launch_route(const RouteLaunch &a, hipStream_t s);

// ---------------------------------------------------------------- permute
struct PermuteLaunch {
    const int32_t *group_id;
    int64_t n;
    int m;
    int32_t *table;     // [nblk][m] per-block counts
    int32_t *base_rel;  // [nblk][m] exclusive prefix over blocks (large inputs: scan launch)
    int32_t *totals;    // [m]
    int32_t *cu;        // [m+1]
    int32_t *perm;      // [n]
};
int64_t permute_blocks(int64_t n);
hipError_t launch_perm_index(const PermuteLaunch &a, hipStream_t s);

// dst[i][h][j] = src[i][h][perm[j]] (inverse == 0) or dst[i][h][perm[j]] = src[i][h][j]
struct GatherLaunch {
    const void *src[4];
    void *dst[4];
    int n_tensors;
    const int32_t *perm;
    int64_t n;
    int n_heads, head_dim;
    int inverse;
    const float *p_sel;  // optional gather of one fp32 value per row (inverse == 0 only)
    float *p_perm;
    const float *src_scale;  // NULL, or (inverse == 0, one tensor) dst row j = src_scale[perm[j]] * src row
    int64_t src_rows;        // (inverse == 0) rows per head of src when != 0 (else n); perm < it
};
hipError_t launch_gather(const GatherLaunch &a, hipStream_t s);

// ---------------------------------------------------------------- attention
struct AttnPlan {
    int32_t *seg_klen;   // [n_seg]
    int32_t *seg_ntile;  // [n_seg]
    int32_t *order;      // [n_seg] segments by descending key length
    int32_t *item_base;  // [n_seg + 1]
    int4 *items;         // [max_items + split_cap] (segment, head, q tile, split part + 1 or 0)
    int4 *spans;         // [max_items + split_cap] the entry's segment: (qb, qe, kb, ke), clamped
    int32_t *chain_off;  // [max_items] XCD-local queues: offset of chain (segment, head) in its queue
    // [0..5]: dispatch counter, dispatch count, first split item, parts per split item, dispatch
    // counter and count of the split parts; [6]: 1 if the whole items sit in XCD-local queues;
    // [8..15]: the queues' dispatch counters; [16..24]: queue x holds entries [q[x], q[x+1])
    int32_t *counter;
    // Key-range split of the last items (forward, head_dim 128): part u of the split items
    // leaves its unnormalised rows in split_o [u][kSplitRows][128] and (row max, row sum) in
    // split_ml [u][kSplitRows][2]; split_cap parts fit (0: no splitting).
    float *split_o, *split_ml;
    int32_t split_cap;
};
constexpr int kSplitRows = 256;     // rows per split part (the largest query tile)
constexpr int kSplitMaxParts = 8;   // key ranges per split item
// split parts held in the workspace: the planner uses at most one part per block of the
// persistent grid (one 8-wave block per CU, 256 on gfx950), so more room would never be used
constexpr int kSplitMaxCap = 256;
constexpr int kSplitMinKeys = 2048; // shortest key range of an item worth splitting
// split_rows: heads x query rows of the launches that use the plan when their kernel can split
// key ranges (head_dim 128), else 0; the room for split parts is about their fp32 size
size_t attn_plan_bytes(int32_t n_seg, int64_t max_items, int64_t split_rows);
int64_t attn_max_items(int n_heads, int64_t len_q, int32_t n_seg);
void attn_plan_carve(AttnPlan &p, void *base, int32_t n_seg, int64_t max_items,
                     int64_t split_rows);

struct AttnLaunch {
    const bf16 *q, *k, *v;
    bf16 *o;
    const int32_t *cu_q, *cu_k;
    int32_t n_seg;
    const int32_t *q_idx;    // NULL or logical q row -> physical row of q, o and row_scale
    const int32_t *kv_idx;   // NULL or logical kv row -> physical row of k, v
    const float *row_scale;  // NULL or [physical q rows]
    const int32_t *o_idx;    // NULL: output rows are the physical q rows; else logical q row ->
                             // physical output row (of o, lse and the mean rows)
    const bf16 *mean_a, *mean_b;  // NULL, or [H][o_rows][hd] rows stored as (o + a + b) / 3
    bf16 *o_raw;             // NULL, or [H][o_rows][hd]: the rows before the mean, stored too
    int64_t len_q, len_k;    // logical rows
    int64_t q_rows, kv_rows, o_rows;  // physical rows per head
    int n_heads, head_dim;
    float scale;
    AttnPlan plan;
    int64_t max_items;
    int waves;               // 8: long segments (MoGA groups), 4: short ones (STGA)
    float *lse;              // NULL or [H][o_rows]: natural-log softmax normaliser per row
};
hipError_t launch_attention(const AttnLaunch &a, hipStream_t s);
// Builds the item list of a launch: items (segment, head, tile of bq rows of cu_q), segments
// ordered by decreasing cu_k length.
hipError_t launch_attn_plan(const int32_t *cu_q, const int32_t *cu_k, int32_t n_seg,
                            int64_t len_q, int64_t len_k, int n_heads, int bq, int64_t max_items,
                            const AttnPlan &plan, hipStream_t s);

// ---------------------------------------------------------------- attention backward
struct AttnBwdLaunch {
    const bf16 *q, *k, *v;   // segment order: q [H][len_q][hd], k and v [H][len_k][hd]
    const bf16 *dov;         // dO' (the upstream gradient of each row's output), [H][len_q][hd]
    const float *lse2;       // [H][len_q]: log2(sum_u exp2(c q.k_u)), c = scale * log2(e)
    const float *D;          // [H][len_q]: <dO', O'>
    bf16 *dq;                // [H][len_q][hd]
    bf16 *dk, *dv;           // [H][len_k][hd]
    const int32_t *cu_q;     // [n_seg + 1]: segment u's query rows are [cu_q[u], cu_q[u+1])
    const int32_t *cu_k;     // [n_seg + 1]: and its key rows [cu_k[u], cu_k[u+1])
    int32_t n_seg;
    int64_t len_q, len_k;    // rows per head
    int n_heads;
    float scale;
    AttnPlan plan;           // rebuilt for each of the two kernels
    int64_t max_items;
};
hipError_t launch_attention_bwd(const AttnBwdLaunch &a, hipStream_t s);

// ---------------------------------------------------------------- backward support
struct BwdRouterLaunch {
    const void *x;
    int x_is_bf16;
    const float *w;          // [d][m]
    int64_t n;
    int d, m;
    const int32_t *group_id; // [n]
    const int32_t *counts;   // [m]
    const float *dp;         // [n]
    float loss_coef;         // d_loss * alpha * m / n^2  (times counts_i = the L_gb term)
    float *dr;               // [n][m]
    float *dx;               // NULL or [n][d]
    float *dw;               // NULL or [d][m]
    float *dw_part;          // [bwd_dw_chunks(n)][d][m]
};
int64_t bwd_dw_chunks(int64_t n);
hipError_t launch_bwd_rowdot(const bf16 *d_out, const bf16 *out, int64_t rows, int hd, float *D,
                             hipStream_t s);
hipError_t launch_bwd_dp(const float *D, const float *p_sel, int64_t n, int n_heads, float scale, float *dp,
                         hipStream_t s);
hipError_t launch_bwd_gather_f32(const float *src, const int32_t *perm, int64_t n, int n_heads,
                                 float mult, int inverse, float *dst, hipStream_t s);
hipError_t launch_router_bwd(const BwdRouterLaunch &a, hipStream_t s);

// ---------------------------------------------------------------- STGA
struct StgaGeom {
    int32_t frames, height, width, n_shots, win_h, win_w, t_group, aug;
    int32_t shot_start[kMaxShots + 1];
};
struct StgaBuffers {
    int32_t *shot_info;  // [n_shots][6]: start, len, chunk_base, aug_base, aug_prev, aug_next
    int32_t *cu_tq;      // [n_groups + 1]
    int32_t *cu_tk;      // [n_groups + 1]
    int32_t *cu_f;       // [frames + 1]
    int32_t *q_idx;      // [N]
    int32_t *kv_idx;     // [N + extra]
    int32_t *tpos;       // NULL or [N][4]: the token's query position and its key positions (its
                         // own, then as borrowed by the next and the previous shot, -1 if none)
};
// out[h][t] = w * (a[h][t] + b[h][t] + sum of c[h][p] over the positions p in pos[4t + first ..
// 4t + first + npos) that are >= 0), in fp32, rounded to bf16 once (a, b and out token order,
// out may be a; a and out rows of hd channels, b and c rows of bc_hd >= hd, of which the first
// hd are used; c with c_rows rows per head)
hipError_t launch_grad_sum(const bf16 *a, const bf16 *b, const bf16 *c, int hd, int bc_hd,
                           int64_t c_rows, const int32_t *pos, int first, int npos, int64_t n,
                           int n_heads, float w, bf16 *out, hipStream_t s);
// head_dim-64 rows widened to 128 channels (upper half zero): dst[h][j] = f * src[h][r], r =
// perm[j] (perm NULL: j), f = row_scale[r] (NULL: 1); r outside [0, src_rows) gives a zero row
hipError_t launch_pad_rows(const bf16 *src, int64_t src_rows, const int32_t *perm,
                           const float *row_scale, int64_t n, int n_heads, bf16 *dst,
                           hipStream_t s);
// back to 64 channels: dst[h][perm[j]] = src[h][j][0:64] (perm NULL: j; src rows of 128)
hipError_t launch_unpad_rows(const bf16 *src, const int32_t *perm, int64_t n, int64_t dst_rows,
                             int n_heads, bf16 *dst, hipStream_t s);
int32_t stga_n_groups(const StgaGeom &g);
int64_t stga_extra_rows(const StgaGeom &g);
hipError_t launch_stga_index(const StgaGeom &g, const StgaBuffers &b, hipStream_t s);


// ---------------------------------------------------------------- loss
hipError_t launch_balance_loss(const int32_t *counts, const double *prob_sum, int64_t n, int m,
                               double alpha, double *loss, double *F, double *P, hipStream_t s);

}  // namespace moga

// Variable-length group attention on bf16 MFMA (papernotes.org MoGA note, 关键设计 1:
// full self-attention inside each group, output scaled by p(g(x)|x); 关键设计 2: groups are
// described by per-segment offsets; 关键设计 4: STGA groups use separate query and key
// lengths because keys/values carry extra boundary frames).
//
// One work item = (segment, head, 128 query rows).  A block of 4 waves owns an item; each
// wave owns 32 query rows.  Per 64-key tile:
//   S^T = K Q^T       v_mfma_f32_32x32x16_bf16, K from LDS as the A operand, Q^T held in
//                     registers as the B operand, so every lane holds one query column and
//                     16 of the 32 keys of each sub-block: the row max and row sum need
//                     one exchange with lane^32 only.
//   online softmax    fp32, exp2 with the scale folded into one FMA per score.
//   O^T += V^T P^T    the probabilities are already laid out as the B operand (the output
//                     layout of the first product groups keys in runs of 4); V is written to
//                     LDS transposed in 4x4 blocks, so the A operand is two 8-byte reads.
// K and V tiles are double-buffered in LDS and prefetched into registers one tile ahead.
// A persistent grid pulls items from an atomic counter in an order sorted by decreasing
// key length (a small planning kernel builds it on the device from cu_q/cu_k), so skewed
// group sizes keep every CU busy and the host never reads the offsets.  Consecutive items
// share (segment, head), so the blocks running at one time stream the same K/V through L2.
#include <math.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "attn_common.h"

namespace moga {
namespace {

// ---------------------------------------------------------------------------- planning
// slots: blocks of the persistent grid that will run the items (0: no key-range split).
// xcd: lay the whole items out in eight XCD-local queues (chains of one segment and head kept
// whole, chain c in longest-first order going to queue c mod 8) instead of one list.
__global__ __launch_bounds__(1024) void plan_kernel(const int32_t *cu_q, const int32_t *cu_k,
                                                     int n_seg, int64_t len_q, int64_t len_k,
                                                     int n_heads, int bq, int64_t max_items,
                                                     int slots, int xcd, AttnPlan p) {
    __shared__ int s_klen[kPlanSortMax];
    __shared__ int s_order[kPlanSortMax];
    __shared__ int s_scan[1024];
    const int tid = threadIdx.x;
    const bool sorted = n_seg <= kPlanSortMax;
    for (int s = tid; s < n_seg; s += 1024) {
        const int64_t qb = clamp64(cu_q[s], 0, len_q), qe = clamp64(cu_q[s + 1], qb, len_q);
        const int64_t kb = clamp64(cu_k[s], 0, len_k), ke = clamp64(cu_k[s + 1], kb, len_k);
        const int klen = (int)(ke - kb);
        p.seg_klen[s] = klen;
        p.seg_ntile[s] = (int)((qe - qb + bq - 1) / bq);
        if (sorted) s_klen[s] = klen;
    }
    __syncthreads();
    if (sorted) {
        // rank sort: longest key range first, ties by segment index
        for (int s = tid; s < n_seg; s += 1024) {
            const int k = s_klen[s];
            int rank = 0;
            for (int s2 = 0; s2 < n_seg; ++s2) {
                const int k2 = s_klen[s2];
                rank += (k2 > k || (k2 == k && s2 < s)) ? 1 : 0;
            }
            s_order[rank] = s;
            p.order[rank] = s;
        }
    } else {
        for (int s = tid; s < n_seg; s += 1024) p.order[s] = s;
    }
    __syncthreads();
    int carry = 0;
    for (int r0 = 0; r0 < n_seg; r0 += 1024) {
        const int r = r0 + tid;
        int v = 0;
        if (r < n_seg) {
            const int s = sorted ? s_order[r] : r;
            const int64_t qb = clamp64(cu_q[s], 0, len_q), qe = clamp64(cu_q[s + 1], qb, len_q);
            v = n_heads * (int)((qe - qb + bq - 1) / bq);
        }
        s_scan[tid] = v;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {
            const int add = tid >= off ? s_scan[tid - off] : 0;
            __syncthreads();
            s_scan[tid] += add;
            __syncthreads();
        }
        if (r < n_seg) p.item_base[r] = carry + s_scan[tid] - v;
        carry += s_scan[1023];
        __syncthreads();
    }
    if (tid == 0) {
        p.item_base[n_seg] = carry;
        p.counter[0] = 0;
        // overlapping (non-monotone) offsets could ask for more items than the list holds
        const int n_items = carry < max_items ? carry : (int)max_items;
        // Items of one launch cost about the same when its segments do (and the list runs
        // longest first), so the last n_items mod slots of them would occupy a few blocks for a
        // whole item's time while the rest of the grid idles.  When that remainder is at most
        // half the grid and its longest item has at least kSplitMinKeys keys (shorter items
        // finish sooner than the extra launches take), each of those items is cut into `parts`
        // key ranges that a second launch runs side by side, and attn_split_combine merges them.
        int first = n_items, parts = 1;
        const int cap = slots < p.split_cap ? slots : p.split_cap;
        const int r = slots > 0 ? n_items % slots : 0;
        if (r > 0 && 2 * r <= cap) {
            const int t = n_items - r;
            int lo = 0, hi = n_seg;  // item_base[lo] <= t < item_base[hi]
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (p.item_base[mid] <= t) lo = mid; else hi = mid;
            }
            if (p.seg_klen[p.order[lo]] >= kSplitMinKeys) {
                parts = min(kSplitMaxParts, cap / r);
                first = t;
            }
        }
        p.counter[1] = first;                       // whole items
        p.counter[2] = first;
        p.counter[3] = parts;
        p.counter[4] = 0;                           // dispatch counter of the split parts
        p.counter[5] = (n_items - first) * parts;   // split parts
        // one queue unless the XCD-local layout below applies (it needs every item listed)
        p.counter[6] = 0;
        for (int x = 0; x < 8; ++x) p.counter[8 + x] = 0;
        p.counter[16] = 0;
        for (int x = 1; x <= 8; ++x) p.counter[16 + x] = first;
    }
    if (!xcd) return;
    __syncthreads();
    const int n_items = p.counter[1];
    if (n_items != p.item_base[n_seg] || p.counter[5] != 0) return;  // clamped or split: one queue
    // Chains c = r * n_heads + h (segment rank r in longest-first order, head h) of seg_ntile
    // items each go to queue c mod 8: chain_off[c] = the items of the earlier chains of its queue
    // (a scan with stride 8 over the chains, 1024 at a time, one carry per queue).
    __shared__ int s_carry[8];
    if (tid < 8) s_carry[tid] = 0;
    __syncthreads();
    const int64_t n_chains = (int64_t)n_seg * n_heads;
    for (int64_t c0 = 0; c0 < n_chains; c0 += 1024) {
        const int64_t c = c0 + tid;
        int v = 0;
        if (c < n_chains) {
            const int r = (int)(c / n_heads);
            v = p.seg_ntile[sorted ? s_order[r] : r];
        }
        s_scan[tid] = v;
        __syncthreads();
        for (int off = 8; off < 1024; off <<= 1) {
            const int add = tid >= off ? s_scan[tid - off] : 0;
            __syncthreads();
            s_scan[tid] += add;
            __syncthreads();
        }
        if (c < n_chains) p.chain_off[c] = s_carry[tid & 7] + s_scan[tid] - v;
        __syncthreads();
        if (tid < 8) s_carry[tid] += s_scan[1016 + tid];
        __syncthreads();
    }
    if (tid == 0) {
        int base = 0;
        for (int x = 0; x < 8; ++x) {
            p.counter[16 + x] = base;
            base += s_carry[x];
        }
        p.counter[24] = base;  // == n_items
        p.counter[6] = 1;
    }
}

// Dispatch entry i: item i before the first split item; from there, part u of split item b
// (entry first + b parts + u) carries the item's (segment, head, q tile) and w = u + 1.
__global__ __launch_bounds__(256) void fill_items_kernel(AttnPlan p, int n_seg, int n_heads,
                                                          const int32_t *cu_q, const int32_t *cu_k,
                                                          int64_t len_q, int64_t len_k) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= p.counter[1] + p.counter[5]) return;
    const int first = p.counter[2], parts = p.counter[3];
    int seg, head, qt, part;
    if (p.counter[6]) {
        // entry i of the XCD-major layout: queue x, then the chain of x that holds it
        int x = 0;
        while (x < 7 && p.counter[17 + x] <= i) ++x;
        const int pos = i - p.counter[16 + x];
        const int64_t n_chains = (int64_t)n_seg * n_heads;
        int64_t lo = 0, hi = (n_chains - x + 7) / 8;  // chain_off[x + 8 lo] <= pos, last such
        while (hi - lo > 1) {
            const int64_t mid = (lo + hi) >> 1;
            if (p.chain_off[x + 8 * mid] <= pos) lo = mid; else hi = mid;
        }
        const int64_t c = x + 8 * lo;
        seg = p.order[(int)(c / n_heads)];
        head = (int)(c % n_heads);
        qt = pos - p.chain_off[c];
        part = 0;
    } else {
        const int src = i < first ? i : first + (i - first) / parts;
        part = i < first ? 0 : 1 + (i - first) % parts;
        int lo = 0, hi = n_seg;  // item_base[lo] <= src < item_base[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (p.item_base[mid] <= src) lo = mid; else hi = mid;
        }
        seg = p.order[lo];
        const int local = src - p.item_base[lo];
        const int nt = p.seg_ntile[seg];
        head = local / nt;
        qt = local % nt;
    }
    p.items[i] = make_int4(seg, head, qt, part);
    // the segment's rows, clamped as the kernels use them (one load decodes an item)
    const int64_t qb = clamp64(cu_q[seg], 0, len_q), qe = clamp64(cu_q[seg + 1], qb, len_q);
    const int64_t kb = clamp64(cu_k[seg], 0, len_k), ke = clamp64(cu_k[seg + 1], kb, len_k);
    p.spans[i] = make_int4((int)qb, (int)qe, (int)kb, (int)ke);
}

// ---------------------------------------------------------------------------- attention
template <int HD, int WAVES>
struct Tile {
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int KP = HD + 8;       // K tile row pitch (bf16): rows shift 4 banks
    static constexpr int VP = KT + 4;       // V^T tile row pitch (bf16): 34 dwords
    static constexpr int NS = HD / 16;      // MFMA k-steps of S^T = K Q^T
    static constexpr int NT = HD / 32;      // 32-row tiles of O^T
    static constexpr int KLOADS = KT * HD / 8 / THREADS;   // 16-byte K chunks per thread
    static constexpr int XN = HD / 32;      // groups of 8 d-quads
    static constexpr int VCOMBOS = 4 * XN;  // 4x4 V blocks per tile, in units of 32 lanes
    static constexpr int VUNITS = (VCOMBOS + 2 * WAVES - 1) / (2 * WAVES);
};

// Rescale the running output only when the row maximum has grown by more than 2^8 in
// exp2 units; until then probabilities are formed against the stale maximum (they stay
// <= 256), which changes no result beyond rounding because numerator and denominator
// use the same reference.
constexpr float kRescaleLog2 = 8.0f;
constexpr float kLn2 = 0.69314718055994531f;

// WAVES waves per block, 32 query rows each; every K/V tile brought into LDS serves all of
// them, so 8 waves (256 rows, one block per CU, two waves per SIMD) halve the K/V traffic
// from L2 and the per-wave load work relative to 4.
template <int HD, bool IDX, int WAVES>
__global__ __launch_bounds__(64 * WAVES, 8 / WAVES) void attn_kernel(AttnLaunch a) {
    using T = Tile<HD, WAVES>;
    constexpr int BQ = 32 * WAVES;
    __shared__ __attribute__((aligned(16))) bf16 ks[2][KT * T::KP];
    __shared__ __attribute__((aligned(16))) bf16 vt[2][HD * T::VP];
    __shared__ int s_item;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int j = lane & 31, hh = lane >> 5;
    const int total = uniform(a.plan.counter[1]);
    const float c = a.scale * kLog2e;
    const float thr = kRescaleLog2 / c;

    // per-thread constant parts of the tile loads
    int k_row[T::KLOADS], k_col[T::KLOADS];
#pragma unroll
    for (int i = 0; i < T::KLOADS; ++i) {
        const int cidx = tid + T::THREADS * i;
        k_row[i] = cidx / (HD / 8);
        k_col[i] = cidx % (HD / 8);
    }
    // V: a "combo" is 32 lanes moving 4x4 blocks; lanes of one combo cover 8 d-quads x
    // 4 key-quads, which keeps the transposed LDS writes bank-conflict free
    int v_ax[T::VUNITS], v_bx[T::VUNITS];
    bool v_on[T::VUNITS];
#pragma unroll
    for (int u = 0; u < T::VUNITS; ++u) {
        const int combo = u * 2 * WAVES + wave * 2 + hh;
        v_on[u] = combo < T::VCOMBOS;
        const int cb = v_on[u] ? combo : 0;
        v_ax[u] = (lane & 7) + 8 * (cb % T::XN);
        v_bx[u] = ((lane >> 3) & 3) + 4 * (cb / T::XN);
    }

    for (;;) {
        if (tid == 0) s_item = atomicAdd(a.plan.counter, 1);
        __syncthreads();
        const int item = uniform(s_item);
        __syncthreads();
        if (item >= total) break;
        const int4 itm = a.plan.items[item];
        const int seg = uniform(itm.x), h = uniform(itm.y), qt = uniform(itm.z);
        const int qb = uniform((int)clamp64(a.cu_q[seg], 0, a.len_q));
        const int qe = uniform((int)clamp64(a.cu_q[seg + 1], qb, a.len_q));
        const int kb = uniform((int)clamp64(a.cu_k[seg], 0, a.len_k));
        const int ke = uniform((int)clamp64(a.cu_k[seg + 1], kb, a.len_k));
        const int klen = ke - kb;

        // ---- Q^T fragments (B operand): lane (query j, half hh) holds q[16s + 8hh .. +8)
        const int qrow = qb + qt * BQ + wave * 32 + j;
        const bool qvalid = qrow < qe;
        const int qrow_c = qvalid ? qrow : qe - 1;   // qe > qb for every item
        // indexed rows are clamped to the head so a bad map cannot address outside it
        const int64_t qphys = IDX ? min(max((int64_t)a.q_idx[qrow_c], (int64_t)0), a.q_rows - 1)
                                  : (int64_t)qrow_c;
        bf16x8 qf[T::NS];
        {
            const bf16 *qp = a.q + (int64_t)h * a.q_rows * HD + qphys * HD + 8 * hh;
#pragma unroll
            for (int s = 0; s < T::NS; ++s) qf[s] = *reinterpret_cast<const bf16x8 *>(qp + 16 * s);
        }

        const bf16 *kbase = a.k + (int64_t)h * a.kv_rows * HD;
        const bf16 *vbase = a.v + (int64_t)h * a.kv_rows * HD;
        const int ntiles = (klen + KT - 1) / KT;

        // two register sets: tile t+2 is requested while tile t is computed, so every load
        // has two tiles of compute to arrive
        uint4 kreg[2][T::KLOADS];
        uint2 vreg[2][T::VUNITS][4];
        auto load_tile = [&](auto rc, int t) {
            constexpr int R = decltype(rc)::value;
            const int key0 = t * KT;
            if constexpr (!IDX) {
                // rows [kb + key0, ke) of this head; rows past ke read as zeros
                // one tile at most; readfirstlane keeps the count (and so the descriptor) in scalar
                // registers: the compiler clamps with a vector instruction, and a descriptor in
                // vector registers costs a waterfall loop around every load
                const uint32_t bytes = (uint32_t)uniform(min(max(klen - key0, 0), KT)) * HD * 2;
                const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + (int64_t)(kb + key0) * HD, bytes);
                const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + (int64_t)(kb + key0) * HD, bytes);
#pragma unroll
                for (int i = 0; i < T::KLOADS; ++i) {
                    const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(
                        rk, (k_row[i] * HD + k_col[i] * 8) * 2, 0, 0);
                    kreg[R][i] = make_uint4(w[0], w[1], w[2], w[3]);
                }
#pragma unroll
                for (int u = 0; u < T::VUNITS; ++u)
                    if (v_on[u])
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(
                            rv, ((4 * v_bx[u] + r) * HD + 4 * v_ax[u]) * 2, 0, 0);
                        vreg[R][u][r] = make_uint2(w[0], w[1]);
                    }
            } else {
                // gathered rows; rows past the segment are clamped to its last row (finite
                // data: their scores are masked and their probabilities are zero)
                const int last = klen - 1;
#pragma unroll
                for (int i = 0; i < T::KLOADS; ++i) {
                    const int key = min(key0 + k_row[i], last);
                    const int64_t row = a.kv_idx[kb + key];
                    kreg[R][i] = *reinterpret_cast<const uint4 *>(kbase + row * HD + k_col[i] * 8);
                }
#pragma unroll
                for (int u = 0; u < T::VUNITS; ++u)
                    if (v_on[u])
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int key = min(key0 + 4 * v_bx[u] + r, last);
                        const int64_t row = a.kv_idx[kb + key];
                        vreg[R][u][r] = *reinterpret_cast<const uint2 *>(vbase + row * HD + 4 * v_ax[u]);
                    }
            }
        };
        auto store_tile = [&](int buf) {
#pragma unroll
            for (int i = 0; i < T::KLOADS; ++i)
                *reinterpret_cast<uint4 *>(&ks[buf][k_row[i] * T::KP + k_col[i] * 8]) = kreg[buf][i];
#pragma unroll
            for (int u = 0; u < T::VUNITS; ++u) {
                if (!v_on[u]) continue;
                const uint2 v0 = vreg[buf][u][0], v1 = vreg[buf][u][1], v2 = vreg[buf][u][2],
                            v3 = vreg[buf][u][3];
                // column cc of the 4 rows -> one 8-byte run of V^T row (4*ax + cc)
                uint2 w[4];
                w[0] = make_uint2(__builtin_amdgcn_perm(v1.x, v0.x, 0x05040100u),
                                  __builtin_amdgcn_perm(v3.x, v2.x, 0x05040100u));
                w[1] = make_uint2(__builtin_amdgcn_perm(v1.x, v0.x, 0x07060302u),
                                  __builtin_amdgcn_perm(v3.x, v2.x, 0x07060302u));
                w[2] = make_uint2(__builtin_amdgcn_perm(v1.y, v0.y, 0x05040100u),
                                  __builtin_amdgcn_perm(v3.y, v2.y, 0x05040100u));
                w[3] = make_uint2(__builtin_amdgcn_perm(v1.y, v0.y, 0x07060302u),
                                  __builtin_amdgcn_perm(v3.y, v2.y, 0x07060302u));
#pragma unroll
                for (int cc = 0; cc < 4; ++cc)
                    *reinterpret_cast<uint2 *>(&vt[buf][(4 * v_ax[u] + cc) * T::VP + 4 * v_bx[u]]) = w[cc];
            }
        };

        float m_run = -INFINITY, l_run = 0.0f;
        f32x16 o[T::NT];
#pragma unroll
        for (int ti = 0; ti < T::NT; ++ti) o[ti] = f32x16{};

        // one tile: publish the prefetched registers into LDS buffer BUF, prefetch the next
        // tile, then S^T, softmax and O^T += V^T P^T.  BUF is a compile-time constant so all
        // LDS addresses fold into immediate offsets.
        auto tile = [&](auto bufc, auto maskc, int t) {
            constexpr int buf = decltype(bufc)::value;
            constexpr bool MASK = decltype(maskc)::value;  // only the last, partial tile
            store_tile(buf);
            __syncthreads();
            if (t + 2 < ntiles) load_tile(bufc, t + 2);

            // S^T for two 32-key sub-blocks
            f32x16 sacc[2];
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) sacc[sb] = f32x16{};
#pragma unroll
            for (int s = 0; s < T::NS; ++s)
#pragma unroll
                for (int sb = 0; sb < 2; ++sb) {
                    const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(
                        &ks[buf][(sb * 32 + j) * T::KP + 8 * hh + 16 * s]);
                    sacc[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc[sb], 0, 0, 0);
                }
            const int key0 = t * KT;
            if constexpr (MASK) {
#pragma unroll
                for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int key = key0 + sb * 32 + 8 * (v >> 2) + 4 * hh + (v & 3);
                        if (key >= klen) sacc[sb][v] = -INFINITY;
                    }
            }
            float tmax = -INFINITY;
#pragma unroll
            for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                for (int v = 0; v < 16; v += 2) tmax = fmaxf(tmax, fmaxf(sacc[sb][v], sacc[sb][v + 1]));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
            const bool up = tmax > m_run + thr;
            if (__ballot(up)) {
                const float m_new = up ? tmax : m_run;
                const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
                m_run = m_new;
                l_run *= alpha;
#pragma unroll
                for (int ti = 0; ti < T::NT; ++ti)
#pragma unroll
                    for (int v = 0; v < 16; ++v) o[ti][v] *= alpha;
            }
            const float mc = m_run * c;

            bf16x8 pf[4];
#pragma unroll
            for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    float pv[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[sb][half * 8 + e], c, -mc));
                        l_run += pv[e];
                    }
                    const uint4 packed = make_uint4(pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                                                    pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7]));
                    pf[sb * 2 + half] = __builtin_bit_cast(bf16x8, packed);
                }
#pragma unroll
            for (int ch = 0; ch < 4; ++ch)
#pragma unroll
                for (int ti = 0; ti < T::NT; ++ti) {
                    const bf16 *vrow = &vt[buf][(32 * ti + j) * T::VP + 4 * hh + 16 * ch];
                    const uint2 lo = *reinterpret_cast<const uint2 *>(vrow);
                    const uint2 hi = *reinterpret_cast<const uint2 *>(vrow + 8);
                    const bf16x8 vf = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
                    o[ti] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ch], o[ti], 0, 0, 0);
                }
        };

        if (ntiles > 0) load_tile(std::integral_constant<int, 0>{}, 0);
        if (ntiles > 1) load_tile(std::integral_constant<int, 1>{}, 1);
        // full tiles without any masking code, then the partial last tile (if any) masked
        const int nfull = klen / KT;
        using B0 = std::integral_constant<int, 0>;
        using B1 = std::integral_constant<int, 1>;
        using NoMask = std::integral_constant<bool, false>;
        using Mask = std::integral_constant<bool, true>;
        int t = 0;
        for (; t + 1 < nfull; t += 2) {
            tile(B0{}, NoMask{}, t);
            tile(B1{}, NoMask{}, t + 1);
        }
        if (t < nfull) {  // odd number of full tiles: t is even, buffer 0
            tile(B0{}, NoMask{}, t);
            ++t;
        }
        if (t < ntiles) {  // the partial tile; its buffer is t & 1
            if (t & 1) tile(B1{}, Mask{}, t);
            else tile(B0{}, Mask{}, t);
        }

        // ---- epilogue: 1/l, optional per-row scale, bf16, 8-byte stores of 4 head channels
        const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
        if (qvalid) {
            const int64_t orow = out_row(a, qrow, qphys);
            if (a.lse && hh == 0)  // log(sum exp(scale q.k)) = scale*m + ln(l)
                a.lse[(int64_t)h * a.o_rows + orow] =
                    l_tot > 0.0f ? (m_run * c + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
            float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
            if (a.row_scale) inv *= a.row_scale[qphys];
            const int64_t off = (int64_t)h * a.o_rows * HD + orow * HD + 4 * hh;
#pragma unroll
            for (int ti = 0; ti < T::NT; ++ti) {
#pragma unroll
                for (int kq = 0; kq < 4; ++kq)
                    store4(a, off + 32 * ti + 8 * kq, o[ti][kq * 4 + 0] * inv,
                           o[ti][kq * 4 + 1] * inv, o[ti][kq * 4 + 2] * inv,
                           o[ti][kq * 4 + 3] * inv);
                // one block of 32 columns at a time: the mean rows' loads are not all hoisted
                asm volatile("" ::: "memory");
            }
        }
    }
}

// ---------------------------------------------------------------------------- attention,
// head_dim 128: K and V tiles go from HBM straight into LDS, K in the A layout (S^T = K Q^T
// reads it as the A operand) and V in the T layout (O^T += V^T P^T reads it transposed);
// see attn_common.h.

// IDX: rows are read through the index maps (STGA groups, or the permutation itself for
// the permute-free MoGA variant); each lane then fetches its chunk's row index first.
// SPLIT: the launch that runs the parts of split items (entries first + u of the item list,
// dispatched from their own counter); otherwise the whole items.
template <int WAVES, bool IDX, bool SPLIT>
__global__ __launch_bounds__(64 * WAVES, 8 / WAVES) void attn_kernel_direct(AttnLaunch a) {
    constexpr int HD = 128;
    constexpr int NS = HD / 16, NT = HD / 32;
    constexpr int THREADS = 64 * WAVES;
    constexpr int BQ = 32 * WAVES;
    constexpr int ROWB = HD * 2;                 // bytes per K or V row
    constexpr int TILEB = KT * ROWB;             // bytes per K or V tile (16 KB)
    constexpr int LOADS = TILEB / 16 / THREADS;  // direct 16-byte loads per thread per tile
    static_assert(LOADS * THREADS * 16 == TILEB, "tile must split into whole wave loads");
    __shared__ __attribute__((aligned(1024))) unsigned char lds[2][2][TILEB];  // [buf][K, V]
    __shared__ int s_item[2];
    __shared__ int s_qbase[9];  // queue x holds entries [s_qbase[x], s_qbase[x + 1])
    __shared__ __attribute__((aligned(16))) int4 s_desc[2][2];  // [slot]: items and spans entries

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int j = lane & 31, hh = lane >> 5;
    const int total = uniform(a.plan.counter[SPLIT ? 5 : 1]);
    [[maybe_unused]] const int split_first = SPLIT ? uniform(a.plan.counter[2]) : 0;
    [[maybe_unused]] const int split_parts = SPLIT ? uniform(a.plan.counter[3]) : 1;
    const float c = a.scale * kLog2e;
    const float thr = kRescaleLog2 / c;

    // per-lane LDS byte offsets of the MFMA operands within a tile
    static_assert(ROWB == ROWB128, "direct-load layouts are for head_dim 128");
    static_assert(BQ <= kSplitRows, "a split part holds one query tile");
    int koff[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) koff[s] = a_frag_off(j, hh, s);
    const int s16 = lane & 15;
    int voff[NT];
#pragma unroll
    for (int ti = 0; ti < NT; ++ti) voff[ti] = t_read_off(lane, ti);
    // per-lane global byte offsets of the direct loads within a tile
    int kgo[LOADS], vgo[LOADS], lrow[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        const int r = (i * WAVES + wave) * 4 + (lane >> 4);
        lrow[i] = r;
        kgo[i] = a_dma_chunk(r, s16) + (IDX ? 0 : r * ROWB);
        vgo[i] = t_dma_chunk(r, s16) + (IDX ? 0 : r * ROWB);
    }

    // Work items come from an atomic counter.  Each block reserves its next item as soon as it
    // starts one and hands the index to every wave after the item's first two tiles, where
    // the next item's descriptor (head, query tile, segment rows: one entry of the plan) is
    // loaded too; a new item then waits only for its own query rows and first key tiles.
    // Whole items come from the plan's queues: one, or eight XCD-local ones (blocks run on XCD
    // blockIdx.x mod 8) of which a block drains its own first and then the others in turn.  The
    // split parts have a queue of their own.  Only thread 0 tracks the queue it draws from.
    int *const queue = a.plan.counter + (SPLIT ? 4 : 8);
    int qcur = SPLIT ? 0 : (int)(blockIdx.x & 7) * uniform(a.plan.counter[6]);
    if (!SPLIT && tid < 9) s_qbase[tid] = a.plan.counter[16 + tid];  // read before the first grab
    auto request = [&]() { return atomicAdd(queue + qcur, 1); };
    // entry index of a drawn position (total once every queue is empty)
    auto grab = [&](int raw) {
        if constexpr (SPLIT) {
            return raw;
        } else {
            for (int tries = 1;; ++tries) {
                const int lo = s_qbase[qcur], hi = s_qbase[qcur + 1];
                if (raw < hi - lo) return lo + raw;
                if (tries == 8) return total;
                qcur = (qcur + 1) & 7;
                raw = request();
            }
        }
    };
    // The descriptor of entry e (its items and spans records, which the plan lays out one
    // after the other) is fetched by two lanes of wave 0 straight into LDS slot `sl`: no
    // registers are held for it, and the tile loop's own wait and barrier publish it.
    const uint32_t span_off = (uint32_t)(reinterpret_cast<const char *>(a.plan.spans) -
                                         reinterpret_cast<const char *>(a.plan.items));
    const __amdgpu_buffer_rsrc_t rdesc = make_rsrc(
        a.plan.items, span_off + (uint32_t)((SPLIT ? split_first + total : total) * 16));
    auto fetch_desc = [&](int it, int sl) {
        const uint32_t e = (uint32_t)(SPLIT ? split_first + it : it);
        if (wave == 0 && lane < 2)
            load_lds16(rdesc, reinterpret_cast<unsigned char *>(&s_desc[sl][0]),
                       (int)((lane ? span_off : 0u) + 16u * e));
    };
    __syncthreads();  // s_qbase
    if (tid == 0) s_item[0] = grab(request());
    __syncthreads();
    int item = uniform(s_item[0]);
    int slot = 0;  // s_item[slot] and s_desc[slot] describe the current item
    if (item < total) fetch_desc(item, 0);
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    __syncthreads();
    while (item < total) {
        int next_raw = 0;
        if (tid == 0) next_raw = request();
        // a split part (entry split_first + item, w = part + 1) takes its share of the
        // segment's key tiles and leaves its rows in split slot `item`
        const int4 itm = s_desc[slot][0], spn = s_desc[slot][1];
        const int h = uniform(itm.y), qt = uniform(itm.z);
        const int qb = uniform(spn.x), qe = uniform(spn.y);
        int kb = uniform(spn.z);
        const int ke = uniform(spn.w);
        int klen = ke - kb;
        if constexpr (SPLIT) {
            const int part = uniform(itm.w) - 1, nt = (klen + KT - 1) / KT;
            const int t_lo = part * nt / split_parts, t_hi = (part + 1) * nt / split_parts;
            kb = uniform(kb + t_lo * KT);
            klen = uniform(max(min(t_hi * KT, klen) - t_lo * KT, 0));
        }

        const int qrow = qb + qt * BQ + wave * 32 + j;
        const bool qvalid = qrow < qe;
        const int qrow_c = qvalid ? qrow : qe - 1;  // qe > qb for every item
        // indexed rows are clamped to the head so a bad map cannot address outside it
        const int64_t qphys = IDX ? min(max((int64_t)a.q_idx[qrow_c], (int64_t)0), a.q_rows - 1)
                                  : (int64_t)qrow_c;
        bf16x8 qf[NS];
        {
            const bf16 *qp = a.q + (int64_t)h * a.q_rows * HD + qphys * HD + 8 * hh;
#pragma unroll
            for (int s = 0; s < NS; ++s) qf[s] = *reinterpret_cast<const bf16x8 *>(qp + 16 * s);
        }
        const bf16 *kbase = a.k + (int64_t)h * a.kv_rows * HD;
        const bf16 *vbase = a.v + (int64_t)h * a.kv_rows * HD;
        const int ntiles = (klen + KT - 1) / KT;

        // whole-head descriptors for gathered rows (every index is a row of this head)
        const __amdgpu_buffer_rsrc_t rk_head = make_rsrc(kbase, (uint32_t)(a.kv_rows * ROWB));
        const __amdgpu_buffer_rsrc_t rv_head = make_rsrc(vbase, (uint32_t)(a.kv_rows * ROWB));

        // Gathered rows: the row indices of the next tile to issue, fetched while the tile
        // before it is computed, so issuing a tile never waits for its indices.  Rows past the
        // segment are clamped to its last row (finite data whose scores are masked and whose
        // probabilities are zero), which also keeps the fetch past the last tile in bounds.
        int nrow[LOADS];
        auto load_rows = [&](int t) {
            if constexpr (IDX) {
                const int last = klen - 1;
#pragma unroll
                for (int i = 0; i < LOADS; ++i) nrow[i] = a.kv_idx[kb + min(t * KT + lrow[i], last)];
            }
        };

        // tile t -> LDS buffer BUF.  Contiguous rows: rows past the segment read as zeros.
        auto issue = [&](auto bufc, int t) {
            constexpr int buf = decltype(bufc)::value;
            const int key0 = t * KT;
            if constexpr (!IDX) {
                // one tile at most, kept scalar (see the generic kernel)
                const uint32_t bytes = (uint32_t)uniform(min(max(klen - key0, 0), KT)) * ROWB;
                const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + (int64_t)(kb + key0) * HD, bytes);
                const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + (int64_t)(kb + key0) * HD, bytes);
#pragma unroll
                for (int i = 0; i < LOADS; ++i) {
                    const int slot = (i * WAVES + wave) * 1024;
                    load_lds16(rk, &lds[buf][0][slot], kgo[i]);
                    load_lds16(rv, &lds[buf][1][slot], vgo[i]);
                }
            } else {
                // the rows were fetched a tile earlier (load_rows)
#pragma unroll
                for (int i = 0; i < LOADS; ++i) {
                    const int slot = (i * WAVES + wave) * 1024;
                    load_lds16(rk_head, &lds[buf][0][slot], nrow[i] * ROWB + kgo[i]);
                    load_lds16(rv_head, &lds[buf][1][slot], nrow[i] * ROWB + vgo[i]);
                }
            }
        };

        float m_run = -INFINITY, l_run = 0.0f;
        f32x16 o[NT];
#pragma unroll
        for (int ti = 0; ti < NT; ++ti) o[ti] = f32x16{};

        uint4 pf_u[4];  // the tile's probabilities, bf16, in the B-operand layout
        // MODE 0: a whole tile; 1: the last, partial tile (masked); 2: a last tile of at most 32
        // keys, whose second 32-key sub-block is all masked: its products and exponentials are
        // skipped (they would add exact zeros)
        auto tile = [&](auto bufc, auto modec, int t) {
            constexpr int buf = decltype(bufc)::value;
            constexpr int MODE = decltype(modec)::value;
            constexpr bool MASK = MODE >= 1, HALF = MODE == 2;
            if (t + 1 < ntiles) {
                issue(std::integral_constant<int, buf ^ 1>{}, t + 1);
                load_rows(t + 2);
            }
            const unsigned char *kt = lds[buf][0];
            const unsigned char *vt_ = lds[buf][1];

            // S^T for the two 32-key sub-blocks, one accumulation chain each, sub-block 0 first
            // so that its probabilities can be formed while sub-block 1's products run
            f32x16 sacc[2];
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
                sacc[sb] = f32x16{};
                if (HALF && sb == 1) continue;
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(kt + sb * 32 * ROWB + koff[s]);
                    sacc[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc[sb], 0, 0, 0);
                }
            }
            if constexpr (MASK) {
                // score v of sub-block sb is key t*KT + sb*32 + 8*(v/4) + 4*hh + v%4: compare the
                // constant part against one per-lane limit (no per-lane key table to keep)
                const int lim = klen - t * KT - 4 * hh;
#pragma unroll
                for (int sb = 0; sb < (HALF ? 1 : 2); ++sb)
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        if (sb * 32 + 8 * (v >> 2) + (v & 3) >= lim) sacc[sb][v] = -INFINITY;
            }
            // this lane's largest score of each sub-block (16 keys each)
            float pm[2] = {-INFINITY, -INFINITY};
#pragma unroll
            for (int sb = 0; sb < (HALF ? 1 : 2); ++sb) {
                const f32x16 &sv = sacc[sb];
                float m0 = fmaxf(fmaxf(sv[0], sv[1]), sv[2]);
                m0 = fmaxf(fmaxf(m0, sv[3]), sv[4]);
                m0 = fmaxf(fmaxf(m0, sv[5]), sv[6]);
                float m1 = fmaxf(fmaxf(sv[8], sv[9]), sv[10]);
                m1 = fmaxf(fmaxf(m1, sv[11]), sv[12]);
                m1 = fmaxf(fmaxf(m1, sv[13]), sv[14]);
                pm[sb] = fmaxf(fmaxf(m0, sv[7]), fmaxf(m1, sv[15]));
            }
            // probabilities of sub-block sb against the running maximum
            auto probs = [&](int sb, float mc) {
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    float pv[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[sb][half * 8 + e], c, -mc));
                    const uint4 packed = make_uint4(pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                                                    pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7]));
                    pf_u[sb * 2 + half] = packed;
                }
            };
            // Speculatively, sub-block 0's probabilities are formed against the running maximum
            // before sub-block 1's scores are known.  They stand unless some score of the tile
            // exceeds the running maximum by more than the lazy threshold; only then (the first
            // tile of an item, or a large jump) is the row maximum over the whole tile taken, the
            // running output rescaled and the probabilities formed again, exactly as a kernel
            // that always took the maximum first would have done.
            float mc = m_run * c;
            probs(0, mc);
            // keep them here: without this the compiler moves them below the branch, after
            // sub-block 1's products, which is the serialisation this order avoids
            asm volatile("" ::"v"(__builtin_bit_cast(u32x4, pf_u[0])),
                         "v"(__builtin_bit_cast(u32x4, pf_u[1])));
            const bool up_lane = fmaxf(pm[0], pm[1]) > m_run + thr;
            // order for the scheduler: sub-block 0's eight K reads, each of its products followed
            // by one of sub-block 1's reads, then sub-block 1's products each followed by vector
            // work (sub-block 0's probabilities), so the products never wait on a read just issued
            // and the exponentials run while the matrix core is busy
            if constexpr (!HALF) {
                __builtin_amdgcn_sched_group_barrier(0x100, NS, 0);  // LDS reads
#pragma unroll
                for (int i = 0; i < NS; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
                }
#pragma unroll
                for (int i = 0; i < NS; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // VALU
                }
            }
            if (__ballot(up_lane)) {
                float tmax = max_across_halves(fmaxf(pm[0], pm[1]));
                const bool up = tmax > m_run + thr;
                const float m_new = up ? tmax : m_run;
                const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
                m_run = m_new;
                l_run *= alpha;
#pragma unroll
                for (int ti = 0; ti < NT; ++ti)
#pragma unroll
                    for (int v = 0; v < 16; ++v) o[ti][v] *= alpha;
                mc = m_run * c;
                probs(0, mc);
            }
            if constexpr (HALF) {
                pf_u[2] = make_uint4(0u, 0u, 0u, 0u);
                pf_u[3] = make_uint4(0u, 0u, 0u, 0u);
            } else {
                probs(1, mc);
            }
            // the row sum adds the bf16 probabilities the MFMA multiplies V with, two per dot2
#pragma unroll
            for (int ch = 0; ch < (HALF ? 2 : 4); ++ch) {
                l_run = sum_bf16x2(pf_u[ch].x, l_run);
                l_run = sum_bf16x2(pf_u[ch].y, l_run);
                l_run = sum_bf16x2(pf_u[ch].z, l_run);
                l_run = sum_bf16x2(pf_u[ch].w, l_run);
            }
#pragma unroll
            for (int ch = 0; ch < (HALF ? 2 : 4); ++ch) {
                const bf16x8 pfc = __builtin_bit_cast(bf16x8, pf_u[ch]);
#pragma unroll
                for (int ti = 0; ti < NT; ++ti) {
                    const unsigned char *vp = vt_ + ch * 16 * ROWB + voff[ti];
                    const uint2 ulo = lds_read_tr16(vp), uhi = lds_read_tr16(vp + 8 * ROWB);
                    const bf16x8 vf = __builtin_bit_cast(bf16x8, make_uint4(ulo.x, ulo.y, uhi.x, uhi.y));
                    o[ti] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pfc, o[ti], 0, 0, 0);
                }
            }
            // the next tile's direct loads must have landed before anyone reads them
            __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
            __syncthreads();
        };

        if (ntiles > 0) {
            load_rows(0);
            issue(std::integral_constant<int, 0>{}, 0);
            load_rows(1);
            __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
            __syncthreads();
        }
        const int nfull = klen / KT;
        using B0 = std::integral_constant<int, 0>;
        using B1 = std::integral_constant<int, 1>;
        using NoMask = std::integral_constant<int, 0>;
        using Mask = std::integral_constant<int, 1>;
        using Half = std::integral_constant<int, 2>;
        // the next item's index to every wave, and its descriptor requested into the other slot
        int next = total;
        auto handoff = [&]() {
            if (tid == 0) s_item[slot ^ 1] = grab(next_raw);
            __syncthreads();
            next = uniform(s_item[slot ^ 1]);
            if (next < total) fetch_desc(next, slot ^ 1);
        };
        int t = 0;
        // Short-segment (4-wave) items hand off early, two tiles in, when at least two more
        // tiles follow to hide the descriptor load; the long MoGA items keep their tile loop
        // free of it and hand off at the end.
        constexpr bool EARLY = WAVES == 4;
        const bool handed = EARLY && nfull >= 4;
        // A wave of a 4-wave item without any query row (the last item of a short segment)
        // computes nothing: it only issues its share of each tile's loads and meets the same
        // barriers in the same order, so the other block's waves on its SIMD run alone.
        bool idle = false;
        if constexpr (WAVES == 4 && !SPLIT) idle = uniform(qb + qt * BQ + wave * 32) >= qe;
        if (idle) {
            auto idle_tile = [&](auto bufc, int tt) {
                constexpr int buf = decltype(bufc)::value;
                if (tt + 1 < ntiles) {
                    issue(std::integral_constant<int, buf ^ 1>{}, tt + 1);
                    load_rows(tt + 2);
                }
                __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
                __syncthreads();
            };
            for (; t + 1 < nfull; t += 2) {
                if (EARLY && t == 2) handoff();
                idle_tile(B0{}, t);
                idle_tile(B1{}, t + 1);
            }
            if (t < nfull) {
                idle_tile(B0{}, t);
                ++t;
            }
            if (t < ntiles) {
                if (t & 1) idle_tile(B1{}, t);
                else idle_tile(B0{}, t);
            }
            t = ntiles;
        }
        for (; t + 1 < nfull; t += 2) {
            if (EARLY && t == 2) handoff();
            tile(B0{}, NoMask{}, t);
            tile(B1{}, NoMask{}, t + 1);
        }
        if (t < nfull) {
            tile(B0{}, NoMask{}, t);
            ++t;
        }
        if (t < ntiles) {
            // short-segment (4-wave) items end on a tile of at most 32 keys often enough for the
            // half tile to pay; the long MoGA items keep their code as it was
            if constexpr (WAVES == 4) {
                const bool half = klen - t * KT <= 32;
                if (t & 1) {
                    if (half) tile(B1{}, Half{}, t);
                    else tile(B1{}, Mask{}, t);
                } else {
                    if (half) tile(B0{}, Half{}, t);
                    else tile(B0{}, Mask{}, t);
                }
            } else {
                if (t & 1) tile(B1{}, Mask{}, t);
                else tile(B0{}, Mask{}, t);
            }
        }
        if (!handed) {
            handoff();
            __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the descriptor has landed
            __syncthreads();
        }
        slot ^= 1;

        const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
        if constexpr (SPLIT) {
            // a part of a split item: its rows unnormalised, with their maximum and sum
            const int64_t row = (int64_t)item * kSplitRows + wave * 32 + j;
            float *po = a.plan.split_o + row * HD + 4 * hh;
#pragma unroll
            for (int ti = 0; ti < NT; ++ti)
#pragma unroll
                for (int kq = 0; kq < 4; ++kq)
                    *reinterpret_cast<float4 *>(po + 32 * ti + 8 * kq) =
                        make_float4(o[ti][kq * 4 + 0], o[ti][kq * 4 + 1], o[ti][kq * 4 + 2],
                                    o[ti][kq * 4 + 3]);
            if (hh == 0)
                *reinterpret_cast<float2 *>(a.plan.split_ml + 2 * row) = make_float2(m_run, l_tot);
            item = next;
            continue;
        }
        if (qvalid) {
            // the 8-wave (MoGA) launches may write through an output map and store the mean of
            // three branches; the 4-wave (short-segment) launches store their rows plainly
            constexpr bool FULL_EPI = WAVES == 8;
            const int64_t orow = FULL_EPI ? out_row(a, qrow, qphys) : qphys;
            if (a.lse && hh == 0)  // log(sum exp(scale q.k)) = scale*m + ln(l)
                a.lse[(int64_t)h * a.o_rows + orow] =
                    l_tot > 0.0f ? (m_run * c + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
            float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
            if (a.row_scale) inv *= a.row_scale[qphys];
            const int64_t off = (int64_t)h * a.o_rows * HD + orow * HD + 4 * hh;
#pragma unroll
            for (int ti = 0; ti < NT; ++ti) {
#pragma unroll
                for (int kq = 0; kq < 4; ++kq) {
                    const float v0 = o[ti][kq * 4 + 0] * inv, v1 = o[ti][kq * 4 + 1] * inv,
                                v2 = o[ti][kq * 4 + 2] * inv, v3 = o[ti][kq * 4 + 3] * inv;
                    if constexpr (FULL_EPI)
                        store4(a, off + 32 * ti + 8 * kq, v0, v1, v2, v3);
                    else
                        *reinterpret_cast<uint2 *>(a.o + off + 32 * ti + 8 * kq) =
                            make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
                }
                // one block of 32 columns at a time: the mean rows' loads are not all hoisted
                if constexpr (FULL_EPI) asm volatile("" ::: "memory");
            }
        }
        item = next;
    }
}

// Merges the key-range parts of the split items.  Per row: with part u's maximum m_u and
// sum l_u (probabilities formed as 2^(c (s - m_u))), the row's maximum is m = max m_u, its sum
// l = sum_u l_u 2^(c (m_u - m)) and its output sum_u O_u 2^(c (m_u - m)) / l, scaled by the
// row's factor and stored as the unsplit epilogue stores it (with its log-sum-exp when asked
// for).  Half a wave per row, four columns per lane, eight rows per block and bq / 8 blocks per
// split item; each lane issues all its parts' loads before it uses any of them.
__global__ __launch_bounds__(256) void attn_split_combine(AttnLaunch a, int bq) {
    constexpr int HD = 128;
    const int first = a.plan.counter[2], parts = a.plan.counter[3];
    const int n_split = a.plan.counter[5] / parts;
    const int per_item = bq / 8;
    const int b = blockIdx.x / per_item;
    if (b >= n_split) return;
    const int4 itm = a.plan.items[first + b * parts];
    const int seg = itm.x, h = itm.y, qt = itm.z;
    const int r = (blockIdx.x % per_item) * 8 + (threadIdx.x >> 5);
    const int64_t qb = clamp64(a.cu_q[seg], 0, a.len_q);
    const int64_t qe = clamp64(a.cu_q[seg + 1], qb, a.len_q);
    const int64_t qrow = qb + (int64_t)qt * bq + r;
    if (qrow >= qe) return;
    const int col = 4 * (threadIdx.x & 31);
    const int64_t row0 = (int64_t)b * parts * kSplitRows + r;  // part u: row0 + u kSplitRows
    float2 ml[kSplitMaxParts];
    float4 ou[kSplitMaxParts];
#pragma unroll
    for (int u = 0; u < kSplitMaxParts; ++u) {
        if (u < parts) {
            const int64_t ru = row0 + (int64_t)u * kSplitRows;
            ml[u] = *reinterpret_cast<const float2 *>(a.plan.split_ml + 2 * ru);
            ou[u] = *reinterpret_cast<const float4 *>(a.plan.split_o + ru * HD + col);
        }
    }
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < kSplitMaxParts; ++u)
        if (u < parts) m = fmaxf(m, ml[u].x);
    const float c = a.scale * kLog2e;
    float l = 0.0f;
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (m > -INFINITY) {
#pragma unroll
        for (int u = 0; u < kSplitMaxParts; ++u) {
            if (u < parts) {
                const float w = __builtin_amdgcn_exp2f((ml[u].x - m) * c);  // 0: an empty part
                l += ml[u].y * w;
                acc.x += ou[u].x * w; acc.y += ou[u].y * w;
                acc.z += ou[u].z * w; acc.w += ou[u].w * w;
            }
        }
    }
    const int64_t qphys =
        a.q_idx ? min(max((int64_t)a.q_idx[qrow], (int64_t)0), a.q_rows - 1) : qrow;
    const int64_t orow = out_row(a, qrow, qphys);
    if (a.lse && col == 0)
        a.lse[(int64_t)h * a.o_rows + orow] =
            l > 0.0f ? (m * c + __builtin_amdgcn_logf(l)) * kLn2 : -INFINITY;
    float inv = l > 0.0f ? 1.0f / l : 0.0f;
    if (a.row_scale) inv *= a.row_scale[qphys];
    store4(a, (int64_t)h * a.o_rows * HD + orow * HD + col, acc.x * inv, acc.y * inv,
           acc.z * inv, acc.w * inv);
}

std::atomic<int> g_num_cus[kMaxDevices];  // per device; 0 until first queried

}  // namespace

hipError_t device_cus(int *out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    int n = g_num_cus[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        // concurrent first calls may both query; they store the same value
        if ((e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev)) !=
            hipSuccess)
            return e;
        g_num_cus[dev].store(n, std::memory_order_relaxed);
    }
    *out = n;
    return hipSuccess;
}

int64_t attn_max_items(int n_heads, int64_t len_q, int32_t n_seg) {
    // sized for the smallest query tile any launch uses (128 rows)
    return (int64_t)n_heads * ((len_q + kAttnBQMin - 1) / kAttnBQMin + n_seg);
}

static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// split parts the workspace holds: no more rows than the launch's queries, at most kSplitMaxCap
static int64_t split_cap(int64_t split_rows) {
    return std::min<int64_t>(kSplitMaxCap, std::max<int64_t>(split_rows, 0) / kSplitRows);
}

size_t attn_plan_bytes(int32_t n_seg, int64_t max_items, int64_t split_rows) {
    const size_t seg = align256(sizeof(int32_t) * (size_t)(n_seg + 1));
    const size_t cap = (size_t)split_cap(split_rows);
    return 4 * seg + 2 * align256(sizeof(int4) * (size_t)(max_items + cap)) +
           align256(sizeof(int32_t) * (size_t)max_items) + 256 +
           cap * kSplitRows * (128 + 2) * sizeof(float);
}

void attn_plan_carve(AttnPlan &p, void *base, int32_t n_seg, int64_t max_items,
                     int64_t split_rows) {
    char *b = static_cast<char *>(base);
    const size_t seg = align256(sizeof(int32_t) * (size_t)(n_seg + 1));
    p.seg_klen = reinterpret_cast<int32_t *>(b); b += seg;
    p.seg_ntile = reinterpret_cast<int32_t *>(b); b += seg;
    p.order = reinterpret_cast<int32_t *>(b); b += seg;
    p.item_base = reinterpret_cast<int32_t *>(b); b += seg;
    p.split_cap = (int32_t)split_cap(split_rows);
    p.items = reinterpret_cast<int4 *>(b);
    b += align256(sizeof(int4) * (size_t)(max_items + p.split_cap));
    p.spans = reinterpret_cast<int4 *>(b);
    b += align256(sizeof(int4) * (size_t)(max_items + p.split_cap));
    p.chain_off = reinterpret_cast<int32_t *>(b);
    b += align256(sizeof(int32_t) * (size_t)max_items);
    p.counter = reinterpret_cast<int32_t *>(b); b += 256;
    p.split_o = reinterpret_cast<float *>(b); b += (size_t)p.split_cap * kSplitRows * 128 * sizeof(float);
    p.split_ml = reinterpret_cast<float *>(b);
}

hipError_t launch_attn_plan(const int32_t *cu_q, const int32_t *cu_k, int32_t n_seg,
                            int64_t len_q, int64_t len_k, int n_heads, int bq, int64_t max_items,
                            const AttnPlan &plan, hipStream_t s) {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, s, cu_q, cu_k, n_seg, len_q, len_k,
                       n_heads, bq, max_items, 0, 0, plan);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fill_items_kernel, dim3((unsigned)((max_items + plan.split_cap + 255) / 256)), dim3(256), 0,
                       s, plan, n_seg, n_heads, cu_q, cu_k, len_q, len_k);
    return hipGetLastError();
}

hipError_t launch_attention(const AttnLaunch &a, hipStream_t s) {
    if (a.n_seg <= 0) return hipSuccess;
    // MoGA groups are long: 8 waves (256 query rows) share every K/V tile.  STGA segments are
    // short (195-1560 rows): 4 waves (128 rows) keep the padded tail small.  Heads whose K/V
    // exceed the 32-bit buffer offset range take the generic kernel.
    const bool indexed = a.kv_idx || a.q_idx;
    const bool direct = a.head_dim == 128 && a.kv_rows * 256 < (int64_t(1) << 31);
    const int waves = a.waves == 4 ? 4 : 8;
    // an output map and the three-branch mean are epilogue features of the 8-wave launches only
    if (direct && waves == 4 && (a.o_idx || a.mean_a || a.o_raw)) return hipErrorInvalidValue;
    const int bq = direct ? 32 * waves : (indexed ? 128 : 256);
    int cus = 0;
    hipError_t e = device_cus(&cus);
    if (e != hipSuccess) return e;
    // persistent grids: two waves per SIMD in every configuration; the head_dim 128 kernel
    // with 256-row items (long segments) may split the last items' key ranges over the grid
    const int slots = cus * (8 / waves);
    const bool splits = direct && waves == 8;
    // long segments (8-wave launches) share one queue, whose tail may split; the items of short
    // segments (4-wave launches) go to XCD-local queues, so the few items of a segment and head
    // stream its keys and values through one L2
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, s, a.cu_q, a.cu_k, a.n_seg, a.len_q,
                       a.len_k, a.n_heads, bq, a.max_items, splits ? slots : 0,
                       direct && !splits ? 1 : 0, a.plan);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t fill_blocks = (a.max_items + a.plan.split_cap + 255) / 256;
    hipLaunchKernelGGL(fill_items_kernel, dim3((unsigned)fill_blocks), dim3(256), 0, s, a.plan,
                       a.n_seg, a.n_heads, a.cu_q, a.cu_k, a.len_q, a.len_k);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const dim3 grid((unsigned)slots), blk((unsigned)(64 * waves));
    const dim3 grid4((unsigned)(cus * 2)), blk4(256u);
    const dim3 grid8((unsigned)cus), blk8(512u);
    if (direct) {
        if (indexed) {
            if (waves == 8) hipLaunchKernelGGL((attn_kernel_direct<8, true, false>), grid, blk, 0, s, a);
            else hipLaunchKernelGGL((attn_kernel_direct<4, true, false>), grid, blk, 0, s, a);
        } else {
            if (waves == 8) hipLaunchKernelGGL((attn_kernel_direct<8, false, false>), grid, blk, 0, s, a);
            else hipLaunchKernelGGL((attn_kernel_direct<4, false, false>), grid, blk, 0, s, a);
        }
        // the split parts, at most min(slots, split_cap) of them (one per block), then their
        // merge: split items number at most half of that (the planner's rule)
        const int room = splits ? std::min(slots, (int)a.plan.split_cap) : 0;
        if (room >= 2) {
            if ((e = hipGetLastError()) != hipSuccess) return e;
            const dim3 gsplit((unsigned)room);
            if (indexed) {
                if (waves == 8) hipLaunchKernelGGL((attn_kernel_direct<8, true, true>), gsplit, blk, 0, s, a);
                else hipLaunchKernelGGL((attn_kernel_direct<4, true, true>), gsplit, blk, 0, s, a);
            } else {
                if (waves == 8) hipLaunchKernelGGL((attn_kernel_direct<8, false, true>), gsplit, blk, 0, s, a);
                else hipLaunchKernelGGL((attn_kernel_direct<4, false, true>), gsplit, blk, 0, s, a);
            }
            if ((e = hipGetLastError()) != hipSuccess) return e;
            hipLaunchKernelGGL(attn_split_combine, dim3((unsigned)(room / 2 * (bq / 8))), dim3(256),
                               0, s, a, bq);
        }
    } else if (a.head_dim == 128) {
        if (indexed) hipLaunchKernelGGL((attn_kernel<128, true, 4>), grid4, blk4, 0, s, a);
        else hipLaunchKernelGGL((attn_kernel<128, false, 8>), grid8, blk8, 0, s, a);
    } else {
        if (indexed) hipLaunchKernelGGL((attn_kernel<64, true, 4>), grid4, blk4, 0, s, a);
        else hipLaunchKernelGGL((attn_kernel<64, false, 8>), grid8, blk8, 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace moga

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

#include "moga_internal.h"

namespace moga {
namespace {

constexpr int KT = 64;  // keys per LDS tile

__device__ __forceinline__ int64_t clamp64(int64_t v, int64_t lo, int64_t hi) {
    return v < lo ? lo : (v > hi ? hi : v);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 r = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, r);
}

// ---------------------------------------------------------------------------- planning
__global__ __launch_bounds__(1024) void plan_kernel(const int32_t *cu_q, const int32_t *cu_k,
                                                     int n_seg, int64_t len_q, int64_t len_k,
                                                     int n_heads, AttnPlan p) {
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
        p.seg_ntile[s] = (int)((qe - qb + kAttnBQ - 1) / kAttnBQ);
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
            v = n_heads * (int)((qe - qb + kAttnBQ - 1) / kAttnBQ);
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
        p.counter[1] = carry;
    }
}

__global__ __launch_bounds__(256) void fill_items_kernel(AttnPlan p, int n_seg) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    const int total = p.counter[1];
    if (i >= total) return;
    int lo = 0, hi = n_seg;  // item_base[lo] <= i < item_base[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (p.item_base[mid] <= i) lo = mid; else hi = mid;
    }
    const int seg = p.order[lo];
    const int local = i - p.item_base[lo];
    const int nt = p.seg_ntile[seg];
    p.items[i] = make_int4(seg, local / nt, local % nt, 0);
}

// ---------------------------------------------------------------------------- attention
template <int HD>
struct Tile {
    static constexpr int KP = HD + 8;       // K tile row pitch (bf16): rows shift 4 banks
    static constexpr int VP = KT + 4;       // V^T tile row pitch (bf16): 34 dwords
    static constexpr int NS = HD / 16;      // MFMA k-steps of S^T = K Q^T
    static constexpr int NT = HD / 32;      // 32-row tiles of O^T
    static constexpr int KLOADS = KT * HD / 8 / kAttnThreads;   // 16-byte K chunks per thread
    static constexpr int XN = HD / 32;      // groups of 8 d-quads
    static constexpr int VUNITS = XN / 2;   // 4x4 V blocks per thread
};

template <int HD>
__global__ __launch_bounds__(256, 2) void attn_kernel(AttnLaunch a) {
    using T = Tile<HD>;
    __shared__ __attribute__((aligned(16))) bf16 ks[2][KT * T::KP];
    __shared__ __attribute__((aligned(16))) bf16 vt[2][HD * T::VP];
    __shared__ int s_item;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int j = lane & 31, hh = lane >> 5;
    const int total = a.plan.counter[1];
    const float c = a.scale * kLog2e;

    for (;;) {
        if (tid == 0) s_item = atomicAdd(a.plan.counter, 1);
        __syncthreads();
        const int item = s_item;
        __syncthreads();
        if (item >= total) break;
        const int4 itm = a.plan.items[item];
        const int seg = itm.x, h = itm.y, qt = itm.z;
        const int64_t qb = clamp64(a.cu_q[seg], 0, a.len_q);
        const int64_t qe = clamp64(a.cu_q[seg + 1], qb, a.len_q);
        const int64_t kb = clamp64(a.cu_k[seg], 0, a.len_k);
        const int64_t ke = clamp64(a.cu_k[seg + 1], kb, a.len_k);
        const int klen = (int)(ke - kb);

        // ---- Q^T fragments (B operand): lane (query j, half hh) holds q[16s + 8hh .. +8)
        const int64_t qrow = qb + (int64_t)qt * kAttnBQ + wave * 32 + j;
        const bool qvalid = qrow < qe;
        int64_t qphys = 0;
        if (qvalid) qphys = a.q_idx ? (int64_t)a.q_idx[qrow] : qrow;
        bf16x8 qf[T::NS];
        {
            const bf16 *qp = a.q + (int64_t)h * a.q_rows * HD + qphys * HD + 8 * hh;
#pragma unroll
            for (int s = 0; s < T::NS; ++s) {
                if (qvalid) qf[s] = *reinterpret_cast<const bf16x8 *>(qp + 16 * s);
                else qf[s] = bf16x8{};
            }
        }

        const bf16 *kbase = a.k + (int64_t)h * a.kv_rows * HD;
        const bf16 *vbase = a.v + (int64_t)h * a.kv_rows * HD;
        const int ntiles = (klen + KT - 1) / KT;

        uint4 kreg[T::KLOADS];
        uint2 vreg[T::VUNITS][4];
        auto phys_row = [&](int key) -> int64_t {
            return a.kv_idx ? (int64_t)a.kv_idx[kb + key] : kb + key;
        };
        auto load_tile = [&](int t) {
            const int key0 = t * KT;
#pragma unroll
            for (int i = 0; i < T::KLOADS; ++i) {
                const int cidx = tid + kAttnThreads * i;
                const int row = cidx / (HD / 8), col = cidx % (HD / 8);
                const int key = key0 + row;
                if (key < klen)
                    kreg[i] = *reinterpret_cast<const uint4 *>(kbase + phys_row(key) * HD + col * 8);
                else
                    kreg[i] = make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < T::VUNITS; ++u) {
                const int combo = u * 8 + wave * 2 + hh;
                const int ax = (lane & 7) + 8 * (combo % T::XN);
                const int bx = ((lane >> 3) & 3) + 4 * (combo / T::XN);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int key = key0 + 4 * bx + r;
                    if (key < klen)
                        vreg[u][r] =
                            *reinterpret_cast<const uint2 *>(vbase + phys_row(key) * HD + 4 * ax);
                    else
                        vreg[u][r] = make_uint2(0, 0);
                }
            }
        };
        auto store_tile = [&](int buf) {
#pragma unroll
            for (int i = 0; i < T::KLOADS; ++i) {
                const int cidx = tid + kAttnThreads * i;
                const int row = cidx / (HD / 8), col = cidx % (HD / 8);
                *reinterpret_cast<uint4 *>(&ks[buf][row * T::KP + col * 8]) = kreg[i];
            }
#pragma unroll
            for (int u = 0; u < T::VUNITS; ++u) {
                const int combo = u * 8 + wave * 2 + hh;
                const int ax = (lane & 7) + 8 * (combo % T::XN);
                const int bx = ((lane >> 3) & 3) + 4 * (combo / T::XN);
                const uint2 v0 = vreg[u][0], v1 = vreg[u][1], v2 = vreg[u][2], v3 = vreg[u][3];
                // column cc of the 4 rows -> one 8-byte run of V^T row (4*ax + cc)
                uint2 w[4];
                w[0] = make_uint2((v0.x & 0xffffu) | (v1.x << 16), (v2.x & 0xffffu) | (v3.x << 16));
                w[1] = make_uint2((v0.x >> 16) | (v1.x & 0xffff0000u),
                                  (v2.x >> 16) | (v3.x & 0xffff0000u));
                w[2] = make_uint2((v0.y & 0xffffu) | (v1.y << 16), (v2.y & 0xffffu) | (v3.y << 16));
                w[3] = make_uint2((v0.y >> 16) | (v1.y & 0xffff0000u),
                                  (v2.y >> 16) | (v3.y & 0xffff0000u));
#pragma unroll
                for (int cc = 0; cc < 4; ++cc)
                    *reinterpret_cast<uint2 *>(&vt[buf][(4 * ax + cc) * T::VP + 4 * bx]) = w[cc];
            }
        };

        float m_run = -INFINITY, l_run = 0.0f;
        f32x16 o[T::NT];
#pragma unroll
        for (int ti = 0; ti < T::NT; ++ti) o[ti] = f32x16{};

        if (ntiles > 0) load_tile(0);
        for (int t = 0; t < ntiles; ++t) {
            const int buf = t & 1;
            store_tile(buf);
            __syncthreads();
            if (t + 1 < ntiles) load_tile(t + 1);

            // S^T for two 32-key sub-blocks
            f32x16 sacc[2];
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
                sacc[sb] = f32x16{};
                const bf16 *krow = &ks[buf][(sb * 32 + j) * T::KP + 8 * hh];
#pragma unroll
                for (int s = 0; s < T::NS; ++s) {
                    const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(krow + 16 * s);
                    sacc[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc[sb], 0, 0, 0);
                }
            }
            const int key0 = t * KT;
            if (key0 + KT > klen) {
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
                for (int v = 0; v < 16; ++v) tmax = fmaxf(tmax, sacc[sb][v]);
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
            const float m_new = fmaxf(m_run, tmax);
            const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
            m_run = m_new;
            const float mc = m_new * c;
            l_run *= alpha;
#pragma unroll
            for (int ti = 0; ti < T::NT; ++ti)
#pragma unroll
                for (int v = 0; v < 16; ++v) o[ti][v] *= alpha;

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
            for (int ti = 0; ti < T::NT; ++ti) {
                const bf16 *vrow = &vt[buf][(32 * ti + j) * T::VP + 4 * hh];
#pragma unroll
                for (int ch = 0; ch < 4; ++ch) {
                    const uint2 lo = *reinterpret_cast<const uint2 *>(vrow + 16 * ch);
                    const uint2 hi = *reinterpret_cast<const uint2 *>(vrow + 16 * ch + 8);
                    const bf16x8 vf = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
                    o[ti] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ch], o[ti], 0, 0, 0);
                }
            }
        }

        // ---- epilogue: 1/l, optional per-row scale, bf16, 8-byte stores of 4 head channels
        const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
        if (qvalid) {
            float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
            if (a.row_scale) inv *= a.row_scale[qphys];
            bf16 *op = a.o + (int64_t)h * a.o_rows * HD + qphys * HD + 4 * hh;
#pragma unroll
            for (int ti = 0; ti < T::NT; ++ti)
#pragma unroll
                for (int kq = 0; kq < 4; ++kq) {
                    const uint2 w = make_uint2(
                        pack_bf16x2(o[ti][kq * 4 + 0] * inv, o[ti][kq * 4 + 1] * inv),
                        pack_bf16x2(o[ti][kq * 4 + 2] * inv, o[ti][kq * 4 + 3] * inv));
                    *reinterpret_cast<uint2 *>(op + 32 * ti + 8 * kq) = w;
                }
        }
    }
}

int g_num_cus = 0;

}  // namespace

int64_t attn_max_items(int n_heads, int64_t len_q, int32_t n_seg) {
    return (int64_t)n_heads * ((len_q + kAttnBQ - 1) / kAttnBQ + n_seg);
}

static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t attn_plan_bytes(int32_t n_seg, int64_t max_items) {
    const size_t seg = align256(sizeof(int32_t) * (size_t)(n_seg + 1));
    return 4 * seg + align256(sizeof(int4) * (size_t)max_items) + 256;
}

void attn_plan_carve(AttnPlan &p, void *base, int32_t n_seg, int64_t max_items) {
    char *b = static_cast<char *>(base);
    const size_t seg = align256(sizeof(int32_t) * (size_t)(n_seg + 1));
    p.seg_klen = reinterpret_cast<int32_t *>(b); b += seg;
    p.seg_ntile = reinterpret_cast<int32_t *>(b); b += seg;
    p.order = reinterpret_cast<int32_t *>(b); b += seg;
    p.item_base = reinterpret_cast<int32_t *>(b); b += seg;
    p.items = reinterpret_cast<int4 *>(b); b += align256(sizeof(int4) * (size_t)max_items);
    p.counter = reinterpret_cast<int32_t *>(b);
}

hipError_t launch_attention(const AttnLaunch &a, hipStream_t s) {
    if (a.n_seg <= 0) return hipSuccess;
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, s, a.cu_q, a.cu_k, a.n_seg, a.len_q,
                       a.len_k, a.n_heads, a.plan);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t fill_blocks = (a.max_items + 255) / 256;
    hipLaunchKernelGGL(fill_items_kernel, dim3((unsigned)fill_blocks), dim3(256), 0, s, a.plan,
                       a.n_seg);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (g_num_cus == 0) {
        int dev = 0, n = 0;
        if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
        if ((e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev)) !=
            hipSuccess)
            return e;
        g_num_cus = n;
    }
    const unsigned grid = (unsigned)(g_num_cus * 2);
    if (a.head_dim == 128)
        hipLaunchKernelGGL(attn_kernel<128>, dim3(grid), dim3(kAttnThreads), 0, s, a);
    else
        hipLaunchKernelGGL(attn_kernel<64>, dim3(grid), dim3(kAttnThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace moga

// Backward of the group attention (head_dim 128, segments as contiguous row ranges, with
// separate query and key ranges per segment), given the
// forward's softmax normaliser per row (lse, natural log) and D = <dO', O'> per row:
//   P = exp(scale Q K^T - lse),  dP = dO' V^T,  dS = P * (dP - D),
//   dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO'
// (dO' = p(g|x) * d_out: the factor of the MoGA output, papernotes.org MoGA note 关键设计 1).
// Two kernels, so that each output row is written by one wave and no floating-point atomics
// are needed (outputs are reproducible): one walks the keys of each query tile (dQ), the other
// the queries of each key tile (dK, dV); both recompute P and dP from lse.
// Tiles come from HBM straight into LDS in the two layouts described in attn_common.h.
#include "attn_common.h"

namespace moga {
namespace {

constexpr float kLog2eB = 1.4426950408889634f;



// ------------------------------------------------------------------------------------- dQ
// Item = (group, head, 128 query rows); wave w owns query rows 32w .. 32w+31 of the item.
// Per 64-key tile: K in the A layout (S^T = K Q^T), K in the T layout (dQ^T += K^T dS^T) and
// V in the A layout (dP^T = V dO'^T).  Q^T and dO'^T stay in registers as B operands; each
// lane holds one query (a column of the 32x32 accumulators), so lse and D are one value per
// lane, and the scores of a lane are 16 keys in runs of 4, the order dS^T is fed back in.
// Eight waves (two per SIMD) share each K/V tile: a wave's Q^T, dO'^T, dQ^T and one block's
// score accumulators fit the 256 registers it gets, so the products accumulate in ordinary
// vector registers that the softmax reads directly, and one wave computes while the other
// waits on LDS.
template <int WAVES>
__global__ __launch_bounds__(64 * WAVES, 1) void attn_bwd_dq_kernel(AttnBwdLaunch a) {
    constexpr int HD = 128, NS = HD / 16, NT = HD / 32, THREADS = 64 * WAVES;
    constexpr int BQ = 32 * WAVES;
    constexpr int ROWB = ROWB128, TILEB = KT * ROWB;
    constexpr int LOADS = TILEB / 16 / THREADS;
    static_assert(LOADS * THREADS * 16 == TILEB, "tile must split into whole wave loads");
    __shared__ __attribute__((aligned(1024))) unsigned char lds[2][3][TILEB];  // K_A, K_T, V_A
    __shared__ int s_item;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int j = lane & 31, hh = lane >> 5, s16 = lane & 15;
    const int total = uniform(a.plan.counter[1]);
    const float c = a.scale * kLog2eB;
    int koff[NS], voff[NT];
#pragma unroll
    for (int s = 0; s < NS; ++s) koff[s] = a_frag_off(j, hh, s);
#pragma unroll
    for (int ti = 0; ti < NT; ++ti) voff[ti] = t_read_off(lane, ti);
    int ago[LOADS], tgo[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        const int r = (i * WAVES + wave) * 4 + (lane >> 4);
        ago[i] = a_dma_chunk(r, s16) + r * ROWB;
        tgo[i] = t_dma_chunk(r, s16) + r * ROWB;
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
        const int rb = uniform((int)clamp64(a.cu_k[seg], 0, a.len_k));
        const int re = uniform((int)clamp64(a.cu_k[seg + 1], rb, a.len_k));
        const int klen = re - rb;
        const int qrow = qb + qt * BQ + wave * 32 + j;
        const bool qvalid = qrow < qe;
        const int qrow_c = qvalid ? qrow : qe - 1;  // qe > qb for every item
        const int64_t hrow = (int64_t)h * a.len_q, hrow_k = (int64_t)h * a.len_k;
        bf16x8 qf[NS], gf[NS];
        {
            const bf16 *qp = a.q + (hrow + qrow_c) * HD + 8 * hh;
            const bf16 *gp = a.dov + (hrow + qrow_c) * HD + 8 * hh;
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                qf[s] = *reinterpret_cast<const bf16x8 *>(qp + 16 * s);
                gf[s] = *reinterpret_cast<const bf16x8 *>(gp + 16 * s);
            }
        }
        const float lse2 = a.lse2[hrow + qrow_c], dd = a.D[hrow + qrow_c];
        const bf16 *kbase = a.k + hrow_k * HD, *vbase = a.v + hrow_k * HD;
        const int ntiles = (klen + KT - 1) / KT;

        // key tile t -> buffer BUF; rows past the group read as zeros
        auto issue = [&](auto bufc, int t) {
            constexpr int buf = decltype(bufc)::value;
            const int key0 = t * KT;
            // one tile at most; readfirstlane keeps the count (and so the descriptor) scalar
            const uint32_t bytes = (uint32_t)uniform(min(max(klen - key0, 0), KT)) * ROWB;
            const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + (int64_t)(rb + key0) * HD, bytes);
            const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + (int64_t)(rb + key0) * HD, bytes);
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                const int slot = (i * WAVES + wave) * 1024;
                load_lds16(rk, &lds[buf][0][slot], ago[i]);
                load_lds16(rk, &lds[buf][1][slot], tgo[i]);
                load_lds16(rv, &lds[buf][2][slot], ago[i]);
            }
        };

        f32x16 dq[NT];
#pragma unroll
        for (int ti = 0; ti < NT; ++ti) dq[ti] = f32x16{};

        auto tile = [&](auto bufc, auto maskc, int t) {
            constexpr int buf = decltype(bufc)::value;
            constexpr bool MASK = decltype(maskc)::value;  // only the last, partial tile
            if (t + 1 < ntiles) issue(std::integral_constant<int, buf ^ 1>{}, t + 1);
            lds_cu8 *ka = lds_ptr(lds[buf][0]), *kt_ = lds_ptr(lds[buf][1]), *va = lds_ptr(lds[buf][2]);
            // S^T and dP^T of 32-key block sb (16 products; operands read from LDS)
            auto sdp = [&](int sb, f32x16 &sacc, f32x16 &pacc) {
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    const bf16x8 kf = lds_read_b128(ka + sb * 32 * ROWB + koff[s]);
                    sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], s ? sacc : f32x16{}, 0, 0, 0);
                    const bf16x8 vf = lds_read_b128(va + sb * 32 * ROWB + koff[s]);
                    pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, gf[s], s ? pacc : f32x16{}, 0, 0, 0);
                }
            };
            // dS^T = P^T * (dP^T - D), packed to bf16 as the B operand of dQ^T += K^T dS^T
            auto softmax = [&](int sb, const f32x16 &sacc, const f32x16 &pacc, bf16x8 (&dsf)[2]) {
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    float ds[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int v = half * 8 + e;
                        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[v], c, -lse2));
                        // key t*KT + sb*32 + 8*(v/4) + 4*hh + v%4: the constant part against one
                        // per-lane limit (no per-lane table to keep)
                        if constexpr (MASK)
                            if (sb * 32 + 8 * (v >> 2) + (v & 3) >= klen - t * KT - 4 * hh) p = 0.0f;
                        ds[e] = p * (pacc[v] - dd);
                    }
                    const uint4 packed = make_uint4(pack_bf16x2(ds[0], ds[1]), pack_bf16x2(ds[2], ds[3]),
                                                    pack_bf16x2(ds[4], ds[5]), pack_bf16x2(ds[6], ds[7]));
                    dsf[half] = __builtin_bit_cast(bf16x8, packed);
                }
            };
            auto dqmm = [&](int sb, const bf16x8 (&dsf)[2]) {
#pragma unroll
                for (int half = 0; half < 2; ++half)
#pragma unroll
                    for (int ti = 0; ti < NT; ++ti) {
                        lds_cu8 *kp = kt_ + (sb * 2 + half) * 16 * ROWB + voff[ti];
                        const uint2 ulo = lds_read_tr16(kp), uhi = lds_read_tr16(kp + 8 * ROWB);
                        const bf16x8 kf = __builtin_bit_cast(bf16x8, make_uint4(ulo.x, ulo.y, uhi.x, uhi.y));
                        dq[ti] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, dsf[half], dq[ti], 0, 0, 0);
                    }
            };
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
                f32x16 sacc, pacc;
                bf16x8 dsf[2];
                sdp(sb, sacc, pacc);
                softmax(sb, sacc, pacc, dsf);
                dqmm(sb, dsf);
            }
            __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the next tile has landed
            __syncthreads();
        };

        if (ntiles > 0) {
            issue(std::integral_constant<int, 0>{}, 0);
            __builtin_amdgcn_s_waitcnt(0x0f70);
            __syncthreads();
        }
        const int nfull = klen / KT;
        // buffer indices are compile-time constants so that the compiler can tell the LDS reads
        // of one buffer from the direct loads into the other and adds no waits between them
        using B0 = std::integral_constant<int, 0>;
        using B1 = std::integral_constant<int, 1>;
        using NoMask = std::integral_constant<bool, false>;
        using Mask = std::integral_constant<bool, true>;
        int t = 0;
        for (; t + 1 < nfull; t += 2) {
            tile(B0{}, NoMask{}, t);
            tile(B1{}, NoMask{}, t + 1);
        }
        if (t < nfull) {
            tile(B0{}, NoMask{}, t);
            ++t;
        }
        if (t < ntiles) {
            if (t & 1) tile(B1{}, Mask{}, t);
            else tile(B0{}, Mask{}, t);
        }
        if (qvalid) {
            bf16 *op = a.dq + (hrow + qrow) * HD + 4 * hh;
#pragma unroll
            for (int ti = 0; ti < NT; ++ti)
#pragma unroll
                for (int kq = 0; kq < 4; ++kq) {
                    const uint2 w = make_uint2(
                        pack_bf16x2(dq[ti][kq * 4 + 0] * a.scale, dq[ti][kq * 4 + 1] * a.scale),
                        pack_bf16x2(dq[ti][kq * 4 + 2] * a.scale, dq[ti][kq * 4 + 3] * a.scale));
                    *reinterpret_cast<uint2 *>(op + 32 * ti + 8 * kq) = w;
                }
        }
    }
}

// ---------------------------------------------------------------------------------- dK, dV
// Item = (group, head, 128 key rows).  Eight waves; waves w and w + 4 share a SIMD and own the
// same 32 key rows (32 (w & 3) .. + 31).  Per 32-query block, wave w computes S = Q K^T and
// P, hands P (bf16, in the B-operand layout) to wave w + 4 through LDS and accumulates
// dV^T += dO'^T P; wave w + 4 computes dP = dO' V^T and, half a tile later, once P is
// visible, accumulates dK^T += Q^T dS with dS = P (dP - D).  Each wave issues 16 products per block
// (the same total as one wave doing both) and holds one 64-register accumulator, so two fit
// a SIMD.  Per 64-query tile: Q and dO' each in the A layout (read as A operands) and in the
// T layout (read transposed), plus lse2 and D of the tile's queries.  K^T (dV waves) or V^T
// (dK waves) stays in registers as the B operand; each lane holds one key (a column of the
// 32x32 accumulators) and 16 query rows in runs of 4, the order P and dS are fed back in.
__global__ __launch_bounds__(512, 1) void attn_bwd_dkdv_kernel(AttnBwdLaunch a) {
    constexpr int HD = 128, NS = HD / 16, NT = HD / 32, WAVES = 8, THREADS = 64 * WAVES;
    constexpr int BK = 128;
    constexpr int ROWB = ROWB128, TILEB = KT * ROWB;
    constexpr int LOADS = TILEB / 16 / THREADS;
    static_assert(LOADS * THREADS * 16 == TILEB, "tile must split into whole wave loads");
    __shared__ __attribute__((aligned(1024))) unsigned char lds[2][4][TILEB];  // Q_A Q_T G_A G_T
    __shared__ __attribute__((aligned(16))) float rowv[2][2][256];              // lse2, D
    __shared__ __attribute__((aligned(16))) uint4 pbuf[2][4][2][64];            // P: [block][pair][half][lane]
    __shared__ int s_item;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // the role test reads a scalar copy (a scalar branch); addresses use `wave` itself, whose
    // range the compiler knows, so it can tell this buffer's reads from the other's loads
    const bool dk_role = uniform(wave) >= 4;
    const int kw = wave & 3;
    const int j = lane & 31, hh = lane >> 5, s16 = lane & 15;
    const int total = uniform(a.plan.counter[1]);
    const float c = a.scale * kLog2eB;
    int koff[NS], voff[NT];
#pragma unroll
    for (int s = 0; s < NS; ++s) koff[s] = a_frag_off(j, hh, s);
#pragma unroll
    for (int ti = 0; ti < NT; ++ti) voff[ti] = t_read_off(lane, ti);
    int ago[LOADS], tgo[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        const int r = (i * WAVES + wave) * 4 + (lane >> 4);
        ago[i] = a_dma_chunk(r, s16) + r * ROWB;
        tgo[i] = t_dma_chunk(r, s16) + r * ROWB;
    }

    for (;;) {
        if (tid == 0) s_item = atomicAdd(a.plan.counter, 1);
        __syncthreads();
        const int item = uniform(s_item);
        __syncthreads();
        if (item >= total) break;
        const int4 itm = a.plan.items[item];
        const int seg = uniform(itm.x), h = uniform(itm.y), kt = uniform(itm.z);
        const int kb = uniform((int)clamp64(a.cu_k[seg], 0, a.len_k));
        const int ke = uniform((int)clamp64(a.cu_k[seg + 1], kb, a.len_k));
        const int rb = uniform((int)clamp64(a.cu_q[seg], 0, a.len_q));
        const int re = uniform((int)clamp64(a.cu_q[seg + 1], rb, a.len_q));
        const int qlen = re - rb;
        const int krow = kb + kt * BK + kw * 32 + j;
        const bool kvalid = krow < ke;
        const int krow_c = kvalid ? krow : ke - 1;  // ke > kb for every item
        const int64_t hrow = (int64_t)h * a.len_q, hrow_k = (int64_t)h * a.len_k;
        // B operand: K^T in dV waves, V^T in dK waves
        bf16x8 bf[NS];
        {
            const bf16 *bp = (dk_role ? a.v : a.k) + (hrow_k + krow_c) * HD + 8 * hh;
#pragma unroll
            for (int s = 0; s < NS; ++s) bf[s] = *reinterpret_cast<const bf16x8 *>(bp + 16 * s);
        }
        const bf16 *qbase = a.q + hrow * HD, *gbase = a.dov + hrow * HD;
        const int ntiles = (qlen + KT - 1) / KT;

        // Query tile t -> buffer BUF (rows past the group read as zeros), in two groups.  The
        // first (Q and dO' in the A layout, dO' in the T layout, lse2) is issued at the start of
        // tile t - 1: the buffer's previous tile, t - 2, was last read by those roles before tile
        // t - 2 ended.  The second (Q in the T layout, D) is read by the dK waves one tile later
        // than the rest, so it is issued after the middle barrier of tile t - 1, once those
        // waves are done with tile t - 2.
        auto tile_rsrc = [&](int t, bool g) {
            const int q0 = t * KT;
            // one tile at most; readfirstlane keeps the count (and so the descriptor) scalar
            const uint32_t bytes = (uint32_t)uniform(min(max(qlen - q0, 0), KT)) * ROWB;
            return make_rsrc((g ? gbase : qbase) + (int64_t)(rb + q0) * HD, bytes);
        };
        // lse2 or D of the tile's queries (256 entries; 64 are used), by wave 0
        auto issue_row = [&](unsigned char *dst, const float *src, int t) {
            if (wave == 0) {
                const int q0 = t * KT;
                // what one load reads, kept scalar
                const uint32_t rbytes = (uint32_t)uniform(min(max(qlen - q0, 0), 256)) * 4;
                load_lds16(make_rsrc(src + hrow + rb + q0, rbytes), dst, 16 * lane);
            }
        };
        auto issue_first = [&](auto bufc, int t) {
            constexpr int buf = decltype(bufc)::value;
            const __amdgpu_buffer_rsrc_t rq = tile_rsrc(t, false), rg = tile_rsrc(t, true);
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                const int slot = (i * WAVES + wave) * 1024;
                load_lds16(rq, &lds[buf][0][slot], ago[i]);
                load_lds16(rg, &lds[buf][2][slot], ago[i]);
                load_lds16(rg, &lds[buf][3][slot], tgo[i]);
            }
            issue_row(reinterpret_cast<unsigned char *>(&rowv[buf][0][0]), a.lse2, t);
        };
        // LOADS loads per thread (one more in wave 0, issued first): the count the end-of-tile
        // wait leaves in flight
        auto issue_second = [&](auto bufc, int t) {
            constexpr int buf = decltype(bufc)::value;
            issue_row(reinterpret_cast<unsigned char *>(&rowv[buf][1][0]), a.D, t);
            const __amdgpu_buffer_rsrc_t rq = tile_rsrc(t, false);
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                const int slot = (i * WAVES + wave) * 1024;
                load_lds16(rq, &lds[buf][1][slot], tgo[i]);
            }
        };
        static_assert(LOADS == 2, "the end-of-tile wait below leaves two loads in flight");

        f32x16 acc[NT];  // dV^T or dK^T of the wave's 32 keys
#pragma unroll
        for (int ti = 0; ti < NT; ++ti) acc[ti] = f32x16{};
        f32x16 pacc[2];  // dK waves: dP of the tile before, until its dS is formed

        // acc^T += X^T B for the 16-query chunk ch of a tile, X in the T layout at xt
        auto accumulate = [&](lds_cu8 *xt, int ch, const bf16x8 &bop) {
#pragma unroll
            for (int ti = 0; ti < NT; ++ti) {
                lds_cu8 *xp = xt + ch * 16 * ROWB + voff[ti];
                const uint2 lo = lds_read_tr16(xp), hi = lds_read_tr16(xp + 8 * ROWB);
                const bf16x8 xf = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
                acc[ti] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xf, bop, acc[ti], 0, 0, 0);
            }
        };
        auto pack8 = [](const float (&x)[8]) {
            return __builtin_bit_cast(
                bf16x8, make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                                   pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])));
        };
        // dK waves: dS = P (dP - D) of the tile in buffer PB (P from the dV waves, dP from this
        // wave's products one tile earlier) and dK^T += Q^T dS
        auto dk_products = [&](auto pbc) {
            constexpr int pb = decltype(pbc)::value;
            lds_cu8 *qt_ = lds_ptr(lds[pb][1]);
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const uint4 pw = pbuf[qb][kw][half][lane];
                    const uint32_t w4[4] = {pw.x, pw.y, pw.z, pw.w};
                    float4 d4[2];
#pragma unroll
                    for (int k2 = 0; k2 < 2; ++k2)
                        d4[k2] = *reinterpret_cast<const float4 *>(
                            &rowv[pb][1][qb * 32 + 8 * (2 * half + k2) + 4 * hh]);
                    float ds[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float p = __uint_as_float(e & 1 ? (w4[e >> 1] & 0xffff0000u) : (w4[e >> 1] << 16));
                        ds[e] = p * (pacc[qb][half * 8 + e] - (&d4[e >> 2].x)[e & 3]);
                    }
                    accumulate(qt_, qb * 2 + half, pack8(ds));
                }
        };

        // Tile t in buffer BUF.  First half: the dV waves form S and P of tile t (kept in
        // registers); the dK waves form dS of tile t - 1 and its dK products.  Middle barrier
        // (LDS only): tile t - 1's P, D and Q^T are no longer read, so the second group of tile
        // t + 1's loads may go into that buffer.  Second half: the dV waves store P and form the
        // dV products; the dK waves form dP of tile t.  End barrier: P of tile t is visible and
        // tile t + 1's first group (and tile t's second) has landed.  Each role's products are
        // issued in the same order as by a kernel that finishes every tile before the next.
        auto tile = [&](auto rolec, auto bufc, auto maskc, int t) {
            constexpr bool DK = decltype(rolec)::value;
            constexpr int buf = decltype(bufc)::value;
            constexpr bool MASK = decltype(maskc)::value;  // only the last, partial tile
            if (t + 1 < ntiles) issue_first(std::integral_constant<int, buf ^ 1>{}, t + 1);
            bf16x8 pf[2][2];
            if constexpr (!DK) {
                lds_cu8 *qa = lds_ptr(lds[buf][0]);
                // P of the 16 query rows of this lane in block qb: rows qb*32 + 8*kq + 4*hh + e,
                // kq < 4, e < 4; the 8 values of half `half` are kq = 2*half, 2*half + 1
                f32x16 sacc[2];
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int s = 0; s < NS; ++s) {
                        const bf16x8 qf = lds_read_b128(qa + qb * 32 * ROWB + koff[s]);
                        sacc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf, bf[s], s ? sacc[qb] : f32x16{}, 0, 0, 0);
                    }
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int half = 0; half < 2; ++half) {
                        float4 l4[2];
#pragma unroll
                        for (int k2 = 0; k2 < 2; ++k2)
                            l4[k2] = *reinterpret_cast<const float4 *>(
                                &rowv[buf][0][qb * 32 + 8 * (2 * half + k2) + 4 * hh]);
                        float pv[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const int v = half * 8 + e;
                            float p = __builtin_amdgcn_exp2f(
                                __builtin_fmaf(sacc[qb][v], c, -(&l4[e >> 2].x)[v & 3]));
                            // query t*KT + qb*32 + 8*(v/4) + 4*hh + v%4: the constant part
                            // against one per-lane limit (no per-lane table to keep)
                            if constexpr (MASK)
                                if (qb * 32 + 8 * (v >> 2) + (v & 3) >= qlen - t * KT - 4 * hh) p = 0.0f;
                            pv[e] = p;
                        }
                        pf[qb][half] = pack8(pv);
                    }
            } else {
                if (t > 0) dk_products(std::integral_constant<int, buf ^ 1>{});
            }
            lds_handoff_barrier();  // middle: tile t - 1 is no longer read
            if (t + 1 < ntiles) issue_second(std::integral_constant<int, buf ^ 1>{}, t + 1);
            if constexpr (!DK) {
                lds_cu8 *gt_ = lds_ptr(lds[buf][3]);
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int half = 0; half < 2; ++half)
                        pbuf[qb][kw][half][lane] = __builtin_bit_cast(uint4, pf[qb][half]);
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int half = 0; half < 2; ++half) accumulate(gt_, qb * 2 + half, pf[qb][half]);
            } else {
                lds_cu8 *ga = lds_ptr(lds[buf][2]);
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int s = 0; s < NS; ++s) {
                        const bf16x8 gf = lds_read_b128(ga + qb * 32 * ROWB + koff[s]);
                        pacc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(gf, bf[s], s ? pacc[qb] : f32x16{}, 0, 0, 0);
                    }
            }
            // end: everything but the two newest loads (tile t + 1's second group, LOADS per
            // thread; in wave 0 the row load before them is waited for too) has landed
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_waitcnt(0x0f72);  // vmcnt(2), lgkmcnt and expcnt at their maximum
            lds_handoff_barrier();
        };

        if (ntiles > 0) {
            issue_first(std::integral_constant<int, 0>{}, 0);
            issue_second(std::integral_constant<int, 0>{}, 0);
            __builtin_amdgcn_s_waitcnt(0x0f70);
            __syncthreads();
        }
        const int nfull = qlen / KT;
        // buffer indices are compile-time constants so that the compiler can tell the LDS reads
        // of one buffer from the direct loads into the other and adds no waits between them
        using B0 = std::integral_constant<int, 0>;
        using B1 = std::integral_constant<int, 1>;
        using NoMask = std::integral_constant<bool, false>;
        using Mask = std::integral_constant<bool, true>;
        // one copy of the tile loop per role, so that the compiler's tracking of outstanding
        // loads never merges the two roles' paths (merged, it adds waits for loads in flight)
        auto run = [&](auto rolec) {
            constexpr bool DK = decltype(rolec)::value;
            int t = 0;
            for (; t + 1 < nfull; t += 2) {
                tile(rolec, B0{}, NoMask{}, t);
                tile(rolec, B1{}, NoMask{}, t + 1);
            }
            if (t < nfull) {
                tile(rolec, B0{}, NoMask{}, t);
                ++t;
            }
            if (t < ntiles) {
                if (t & 1) tile(rolec, B1{}, Mask{}, t);
                else tile(rolec, B0{}, Mask{}, t);
            }
            // the last tile's dK products (its second group of loads is the one left in flight)
            if (ntiles > 0) {
                __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
                __syncthreads();
                if constexpr (DK) {
                    if ((ntiles - 1) & 1) dk_products(B1{});
                    else dk_products(B0{});
                }
            }
        };
        if (dk_role) run(std::true_type{});
        else run(std::false_type{});
        if (kvalid) {
            bf16 *op = (dk_role ? a.dk : a.dv) + (hrow_k + krow) * HD + 4 * hh;
            const float mul = dk_role ? a.scale : 1.0f;
#pragma unroll
            for (int ti = 0; ti < NT; ++ti)
#pragma unroll
                for (int kq = 0; kq < 4; ++kq) {
                    const uint2 w = make_uint2(
                        pack_bf16x2(acc[ti][kq * 4 + 0] * mul, acc[ti][kq * 4 + 1] * mul),
                        pack_bf16x2(acc[ti][kq * 4 + 2] * mul, acc[ti][kq * 4 + 3] * mul));
                    *reinterpret_cast<uint2 *>(op + 32 * ti + 8 * kq) = w;
                }
        }
    }
}

}  // namespace

hipError_t launch_attention_bwd(const AttnBwdLaunch &a, hipStream_t s) {
    if (a.n_seg <= 0) return hipSuccess;
    int cus = 0;
    hipError_t e = device_cus(&cus);
    if (e != hipSuccess) return e;
    // dQ: items of 256 query rows, inner loop over the group's keys
    constexpr int kDqWaves = 8;
    if ((e = launch_attn_plan(a.cu_q, a.cu_k, a.n_seg, a.len_q, a.len_k, a.n_heads,
                              32 * kDqWaves, a.max_items, a.plan, s)) != hipSuccess)
        return e;
    hipLaunchKernelGGL(attn_bwd_dq_kernel<kDqWaves>, dim3((unsigned)cus), dim3(64 * kDqWaves), 0, s,
                       a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // dK, dV: items of 128 key rows, inner loop over the group's queries (the plan is rebuilt
    // in place once the dQ kernel, earlier on the stream, is done with it)
    if ((e = launch_attn_plan(a.cu_k, a.cu_q, a.n_seg, a.len_k, a.len_q, a.n_heads, 128,
                              a.max_items, a.plan, s)) != hipSuccess)
        return e;
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel, dim3((unsigned)cus), dim3(512), 0, s, a);
    return hipGetLastError();
}

}  // namespace moga

// Token router: r = x W (fp32, no bias), p = softmax(r), g = argmax r, p_sel = p[g],
// plus per-group counts and fp64 sums of p (papernotes.org MoGA note, 关键设计 1 and 3;
// xugj520.cn MoGA blog §2.3 for the linear, bias-free form and the argmax).
//
// bf16 x (the model's activations): x W on the matrix cores.  W is fp32, so it is split
// exactly into three bf16 terms, w = w1 + w2 + w3 (w1 = bf16(w), w2 = bf16(w - w1),
// w3 = w - w1 - w2, which needs at most 8 significant bits): every product x*w_j is exact
// in fp32 and the MFMA accumulates in fp32, so the logits carry fp32 accuracy.  One
// 16x16x32 MFMA takes 16 groups (A, from the split W) against 16 tokens (B), so each logit's
// reduction over d happens inside the matrix core and only the softmax needs two cross-lane
// steps.  route_stage_kernel (m <= 16, W image within 64 KiB) reads x rows in whole-row
// pieces and transposes them through LDS; route_chunk_kernel (a larger image, m <= 30) reads
// rows the same way and streams the image through LDS in chunks of 256 columns;
// route_mfma_kernel (more groups) loads the B operand straight from memory and streams W
// fragments from L2.  Each of the three takes the k-steps in order and the three terms
// smallest first, so all give the same logits.  Group statistics are written per wave, block
// or work item and summed in a fixed order, so they are bitwise reproducible.
//
// fp32 x: VALU pass.  Each wave streams TPW token rows at a time with 16-byte coalesced
// loads (lane l holds columns [VEC*l, VEC*l+VEC) of every 64*VEC-wide stripe), multiplies
// them by W^T staged once per block in LDS, and reduces the per-lane partial logits across
// the wave.  Group statistics are kept per lane (lane i owns group i).
#include <algorithm>
#include <atomic>

#include "moga_internal.h"

namespace moga {
namespace {

// dynamic LDS of the vector router (W^T, or a chunk of its columns): with the kernel's 3 KiB of
// static reduction arrays the block stays within 64 KiB
constexpr int kRouteLdsBytes = 60 * 1024;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

template <bool XBF16>
__device__ __forceinline__ void load_x(const void *x, int64_t off, float *out) {
    if constexpr (XBF16) {
        const uint4 raw = *reinterpret_cast<const uint4 *>(static_cast<const bf16 *>(x) + off);
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = __uint_as_float(w[i] << 16);
            out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    } else {
        const float4 raw = *reinterpret_cast<const float4 *>(static_cast<const float *>(x) + off);
        out[0] = raw.x; out[1] = raw.y; out[2] = raw.z; out[3] = raw.w;
    }
}

// wt[mm][c] = W[c0 + c][mm] for mm < m, 0 for m <= mm < MM.
template <int MM>
__device__ void stage_w(float *wt, const float *w, int c0, int cl, int m, int dc) {
    for (int idx = threadIdx.x; idx < cl * MM; idx += blockDim.x) {
        const int c = idx / MM, mm = idx % MM;
        wt[mm * dc + c] = mm < m ? w[(int64_t)(c0 + c) * m + mm] : 0.0f;
    }
}

template <int MM, int TPW, bool XBF16>
__global__ __launch_bounds__(256) void route_kernel(RouteLaunch a, int dc) {
    extern __shared__ float wt[];  // [MM][dc]
    __shared__ double red_p[4][64];
    __shared__ int red_c[4][64];
    constexpr int VEC = XBF16 ? 8 : 4;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int d = a.d, m = a.m;
    const int64_t tb0 = (int64_t)blockIdx.x * kRouteTokensPerBlock;
    const int64_t tb1 = tb0 + kRouteTokensPerBlock < a.n ? tb0 + kRouteTokensPerBlock : a.n;
    const bool single = dc >= d;
    double psum = 0.0;
    int cnt = 0;
    if (single) {
        stage_w<MM>(wt, a.w, 0, d, m, dc);
        __syncthreads();
    }
    for (int64_t base = tb0; base < tb1; base += 4 * TPW) {
        const int64_t t0 = base + wave * TPW;
        float acc[TPW][MM];
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
            for (int mm = 0; mm < MM; ++mm) acc[tt][mm] = 0.0f;
        for (int c0 = 0; c0 < d; c0 += dc) {
            const int cl = d - c0 < dc ? d - c0 : dc;
            if (!single) {
                __syncthreads();
                stage_w<MM>(wt, a.w, c0, cl, m, dc);
                __syncthreads();
            }
            for (int c = lane * VEC; c < cl; c += 64 * VEC) {
                float xv[TPW][VEC];
#pragma unroll
                for (int tt = 0; tt < TPW; ++tt) {
                    if (t0 + tt < tb1) {
                        load_x<XBF16>(a.x, (t0 + tt) * (int64_t)d + c0 + c, xv[tt]);
                    } else {
#pragma unroll
                        for (int e = 0; e < VEC; ++e) xv[tt][e] = 0.0f;
                    }
                }
#pragma unroll
                for (int mm = 0; mm < MM; ++mm) {
                    float wv[VEC];
#pragma unroll
                    for (int e4 = 0; e4 < VEC; e4 += 4) {
                        const float4 q = *reinterpret_cast<const float4 *>(&wt[mm * dc + c + e4]);
                        wv[e4] = q.x; wv[e4 + 1] = q.y; wv[e4 + 2] = q.z; wv[e4 + 3] = q.w;
                    }
#pragma unroll
                    for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
                        for (int e = 0; e < VEC; ++e)
                            acc[tt][mm] = __builtin_fmaf(xv[tt][e], wv[e], acc[tt][mm]);
                }
            }
        }
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
            for (int mm = 0; mm < MM; ++mm) acc[tt][mm] = wave_sum(acc[tt][mm]);
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
            const int64_t t = t0 + tt;
            if (t >= tb1) continue;
            // every lane holds the full logits of token t
            float rmax = acc[tt][0];
            int best = 0;
#pragma unroll
            for (int mm = 1; mm < MM; ++mm)
                if (mm < m && acc[tt][mm] > rmax) { rmax = acc[tt][mm]; best = mm; }
            float z = 0.0f, e_own = 0.0f;
            int g = best;
            if (a.pin) {
                const int pv = a.pin[t];
                if (pv >= 0 && pv < m) g = pv;
            }
            float e_g = 0.0f;
#pragma unroll
            for (int mm = 0; mm < MM; ++mm) {
                if (mm < m) {
                    const float e = __builtin_amdgcn_exp2f((acc[tt][mm] - rmax) * kLog2e);
                    z += e;
                    if (mm == lane) e_own = e;
                    if (mm == g) e_g = e;
                }
            }
            if (lane == 0) {
                a.group_id[t] = g;
                a.p_sel[t] = e_g / z;
            }
            if (lane < m) {
                psum += (double)(e_own / z);
                cnt += (g == lane) ? 1 : 0;
            }
        }
    }
    red_p[wave][lane] = psum;
    red_c[wave][lane] = cnt;
    __syncthreads();
    if ((int)threadIdx.x < m) {
        double s = 0.0;
        int c = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) { s += red_p[w][threadIdx.x]; c += red_c[w][threadIdx.x]; }
        a.part_p[(int64_t)blockIdx.x * kMaxGroups + threadIdx.x] = s;
        a.part_c[(int64_t)blockIdx.x * kMaxGroups + threadIdx.x] = c;
    }
}

// ---------------------------------------------------------------- bf16 x: matrix cores
constexpr int kNoGroup = 1 << 30;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// cache policy of the loads of x: every row is read once, so the loads are non-temporal (the nt
// bit), which streams them past the caches rather than keeping them there (30 s router 161 ->
// 142 us, 60 s 1.00 -> 0.93 ms)
constexpr int kStreamed = 2;

// a value the caller knows to be the same in every lane, made visibly so to the compiler
__device__ __forceinline__ int uniform_int(int v) { return __builtin_amdgcn_readfirstlane(v); }

// wf[j][mt][s][lane] = 8 bf16: term j of W[32s + 8(lane/16) + i][16mt + lane%16], i < 8
// (zero outside d x m): the A operand of a 16x16x32 MFMA for group tile mt, k-step s.
// Also resets the work-queue counter that follows the fragments.
__global__ __launch_bounds__(256) void route_split_kernel(const float *w, int d, int m, int mt_n,
                                                          int steps, bf16x8 *wf, int *queue) {
    const int64_t frags = (int64_t)mt_n * steps * 64;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx == 0) *queue = 0;
    if (idx >= frags) return;
    const int lane = (int)(idx & 63);
    const int64_t rest = idx >> 6;
    const int s = (int)(rest % steps), mt = (int)(rest / steps);
    const int g = 16 * mt + (lane & 15), k0 = 32 * s + 8 * (lane >> 4);
    bf16x8 t0, t1, t2;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int k = k0 + i;
        const float v = (g < m && k < d) ? w[(int64_t)k * m + g] : 0.0f;
        const bf16 h = (bf16)v;
        const float r1 = v - (float)h;  // exact
        const bf16 md = (bf16)r1;
        const float r2 = r1 - (float)md;  // exact, at most 8 significant bits
        t0[i] = h;
        t1[i] = md;
        t2[i] = (bf16)r2;
    }
    wf[idx] = t0;
    wf[frags + idx] = t1;
    wf[2 * frags + idx] = t2;
}

// Operands of one k-step: x for T token tiles and the three W terms for MT group tiles.
template <int MT, int T>
struct RouteFrag {
    bf16x8 x[T];
    bf16x8 w[3][MT];
};

// x rows of the work item through rx (row r of the item at byte r*d*2; rows past the item's
// end read as zeros), W fragments through rw.  Byte offsets of k-step s are scalar.
template <int MT, int T>
__device__ __forceinline__ void route_load(RouteFrag<MT, T> &f, __amdgpu_buffer_rsrc_t rx,
                                           const uint32_t (&xoff)[T], __amdgpu_buffer_rsrc_t rw,
                                           uint32_t woff, int frags, int steps, int s) {
#pragma unroll
    for (int i = 0; i < T; ++i)
        f.x[i] = as_bf16x8(__builtin_amdgcn_raw_buffer_load_b128(rx, xoff[i], 64 * s, kStreamed));
#pragma unroll
    for (int j = 0; j < 3; ++j)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            f.w[j][mt] = as_bf16x8(__builtin_amdgcn_raw_buffer_load_b128(
                rw, woff, (j * frags + (mt * steps + s) * 64) * 16, 0));
}

// acc[i][mt] += W-tile mt (three terms, smallest first) x x-tile i.
template <int MT, int T>
__device__ __forceinline__ void route_mma(f32x4 (&acc)[T][MT], const RouteFrag<MT, T> &f) {
#pragma unroll
    for (int j = 2; j >= 0; --j)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < T; ++i)
                acc[i][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.w[j][mt], f.x[i], acc[i][mt],
                                                                     0, 0, 0);
}

// Argmax (lowest group index on equal logits), pin, softmax and outputs of one token whose
// logits lane l holds as acc[mt][v] for groups 16mt + 4kq + v (the four lanes l, l ^ 16, l ^ 32,
// l ^ 48 hold its other groups); p and the chosen group added to this lane's statistics.
// pin: the token's pinned group, or anything outside [0, m) for none.
template <int MT>
__device__ __forceinline__ void route_token(const RouteLaunch &a, const f32x4 (&acc)[MT], int64_t t,
                                            bool valid, int pin, int kq, double (&psum)[MT][4],
                                            int (&cnt)[MT][4]) {
    const int m = a.m;
    float best = 0.0f;
    int bi = kNoGroup;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int g = 16 * mt + 4 * kq + v;
            if (g < m && (bi == kNoGroup || acc[mt][v] > best)) {
                best = acc[mt][v];
                bi = g;
            }
        }
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
        const float ob = __shfl_xor(best, off, 64);
        const int oi = __shfl_xor(bi, off, 64);
        if (oi != kNoGroup && (bi == kNoGroup || ob > best || (ob == best && oi < bi))) {
            best = ob;
            bi = oi;
        }
    }
    const int g = (valid && pin >= 0 && pin < m) ? pin : bi;
    float e[MT][4];
    float z = 0.0f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int gg = 16 * mt + 4 * kq + v;
            e[mt][v] = gg < m ? __builtin_amdgcn_exp2f((acc[mt][v] - best) * kLog2e) : 0.0f;
            z += e[mt][v];
        }
    // the four lanes of a token add the same pairs, so all get the same z
    z += __shfl_xor(z, 16, 64);
    z += __shfl_xor(z, 32, 64);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int gg = 16 * mt + 4 * kq + v;
            if (gg < m && valid) {
                const float p = e[mt][v] / z;
                psum[mt][v] += (double)p;
                if (gg == g) {
                    cnt[mt][v] += 1;
                    a.group_id[t] = g;
                    a.p_sel[t] = p;
                }
            }
        }
}

// Sum of one wave's statistics over the 16 lanes of each k-quarter (they hold the same groups).
template <int MT>
__device__ __forceinline__ void route_wave_stats(double (&psum)[MT][4], int (&cnt)[MT][4]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) {
                psum[mt][v] += __shfl_xor(psum[mt][v], off, 64);
                cnt[mt][v] += __shfl_xor(cnt[mt][v], off, 64);
            }
}

// Softmax, argmax, pins, outputs and the statistics of one work item of T*16 tokens starting
// at t0.  Lane l holds the logits acc[i][mt][v] of groups 16mt + 4kq + v of token
// t0 + 16i + tok; the item's statistics go to row `item` of part_p / part_c (stride m).
template <int MT, int T>
__device__ __forceinline__ void route_finish(const RouteLaunch &a, const f32x4 (&acc)[T][MT],
                                             int64_t t0, int item, int tok, int kq) {
    const int m = a.m;
    const int64_t n = a.n;
    double psum[MT][4];
    int cnt[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) { psum[mt][v] = 0.0; cnt[mt][v] = 0; }
#pragma unroll
    for (int i = 0; i < T; ++i) {
        const int64_t t = t0 + 16 * i + tok;
        const bool valid = t < n;
        const int pin = (a.pin && valid) ? a.pin[t] : -1;
        route_token<MT>(a, acc[i], t, valid, pin, kq, psum, cnt);
    }
    route_wave_stats<MT>(psum, cnt);
    if (tok == 0) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int g = 16 * mt + 4 * kq + v;
                if (g < m) {
                    a.part_p[(int64_t)item * m + g] = psum[mt][v];
                    a.part_c[(int64_t)item * m + g] = cnt[mt][v];
                }
            }
    }
}

// Persistent waves take work items of T*16 tokens from a queue.  Lane l: token l%16 of each
// 16-token tile, k-quarter kq = l/16 of each 32-wide k-step; after the MFMAs it holds the
// logits of groups 16mt + 4kq + v (v < 4) of its token.  The k-steps run in a two-buffer
// pipeline of U steps per buffer: the loads of the next U steps are in flight while the
// current U are multiplied (past the last step the loads repeat it and their products are
// skipped).  Group statistics are written per work item, so their fixed-order sum does not
// depend on which wave took which item.
template <int MT, int T, int U>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(MT == 1 ? 3 : 2)))
void route_mfma_kernel(RouteLaunch a, const bf16x8 *wf,
                                                         int *queue, int steps) {
    const int lane = threadIdx.x & 63, tok = lane & 15, kq = lane >> 4;
    const int d = a.d;
    const int64_t n = a.n;
    const int frags = MT * steps * 64;
    const int full = d / 32;  // k-steps whose 32 columns all lie inside the row
    const int64_t n_items = (n + 16 * T - 1) / (16 * T);
    const bf16 *x = static_cast<const bf16 *>(a.x);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(wf, (uint32_t)(3 * frags * 16));
    const uint32_t woff = 16 * lane;
    uint32_t xoff[T];
#pragma unroll
    for (int i = 0; i < T; ++i) xoff[i] = (uint32_t)(((16 * i + tok) * d + 8 * kq) * 2);

    int next = 0;
    if (lane == 0) next = atomicAdd(queue, 1);
    for (;;) {
        const int item = __builtin_amdgcn_readfirstlane(next);
        if (item >= n_items) break;
        if (lane == 0) next = atomicAdd(queue, 1);  // the following item, fetched early
        const int64_t t0 = (int64_t)item * (16 * T);
        const int64_t rows = min((int64_t)(16 * T), n - t0);
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + t0 * d, (uint32_t)(rows * d * 2));
        f32x4 acc[T][MT];
#pragma unroll
        for (int i = 0; i < T; ++i)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[i][mt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if (full > 0) {
            RouteFrag<MT, T> fa[U], fb[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                route_load(fa[u], rx, xoff, rw, woff, frags, steps, min(u, full - 1));
                __builtin_amdgcn_sched_barrier(0);  // issue order = consumption order
            }
            // whole groups of 2U steps without branches (a branch inside the loop makes the
            // compiler wait for every load in flight), then the rest
            const int whole = full / (2 * U);
            for (int gi = 0; gi < whole; ++gi) {
                const int s = gi * 2 * U;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    route_load(fb[u], rx, xoff, rw, woff, frags, steps, min(s + U + u, full - 1));
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int u = 0; u < U; ++u) route_mma(acc, fa[u]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    route_load(fa[u], rx, xoff, rw, woff, frags, steps, min(s + 2 * U + u, full - 1));
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int u = 0; u < U; ++u) route_mma(acc, fb[u]);
                __builtin_amdgcn_sched_barrier(0);
            }
            // fa holds steps whole*2U .. +U-1 (clamped); fb is loaded here for the rest
            const int s = whole * 2 * U;
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (s + u < full) route_mma(acc, fa[u]);
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (s + U + u < full) {
                    route_load(fb[u], rx, xoff, rw, woff, frags, steps, s + U + u);
                    route_mma(acc, fb[u]);
                }
        }
        if (full < steps) {  // last k-step: columns past d are zero (W is zero there too)
            RouteFrag<MT, T> f;
            route_load(f, rx, xoff, rw, woff, frags, steps, full);
            if (32 * full + 8 * kq >= d)
#pragma unroll
                for (int i = 0; i < T; ++i) f.x[i] = bf16x8{};
            route_mma(acc, f);
        }
        route_finish<MT, T>(a, acc, t0, item, tok, kq);
    }
}

// The three-term W image held in LDS by route_stage_kernel: at most kRouteLdsW bytes.
constexpr int kRouteLdsW = 64 * 1024;

// Row stride of the W image: whole k-steps plus 16 bytes, an odd number of 16-byte chunks,
// so the 16 group rows that one k-slice read touches start in 16 different LDS bank groups.
__host__ __device__ inline int route_stage_row_bytes(int d) { return ((d + 31) / 32) * 64 + 16; }

// Row-contiguous reads for the matrix cores (bf16 x, m <= 16, the three-term W image of at
// most kRouteLdsW bytes).  A load instruction in the MFMA operand layout covers 16 rows x 64
// bytes, which streams from HBM at about half the rate of whole-row reads; here each wave
// instead reads UB contiguous bytes of a token row per 64/(UB/16) lanes (one instruction
// covers 64*16/UB rows), writes them into its own LDS tile of 16 rows x UB bytes (16-byte
// chunk c of row r at chunk position c ^ (r & 15)), and reads the B fragments of the
// 16x16x32 MFMAs from there: the 16 lanes that read one k-slice of 16 rows hit 16 different
// bank groups.  A unit of work is UB/2 columns of a 16-token tile; the rows of the next NH
// units are in flight (a ring of registers) while a unit is written to LDS and multiplied.
// A wave reads only what it wrote itself, so no barrier is needed after the W image is
// built.  Each wave owns a contiguous, balanced range of tiles; its group statistics go to
// row `wave` of part_p / part_c.
template <int NW, int NH, int UB>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void route_stage_kernel(RouteLaunch a, int n_waves) {
    static_assert(NH == 1 || NH == 2, "the unit loop below handles one or two ring parts");
    static_assert(NW % 4 == 0, "whole waves per SIMD");
    constexpr int LPR = UB / 16;      // lanes per row in a load
    constexpr int RPI = 64 / LPR;     // rows per load instruction
    constexpr int NL = 16 / RPI;      // load instructions per unit
    constexpr int KS = UB / 64;       // k-steps per unit
    constexpr int UC = UB / 2;        // columns per unit
    extern __shared__ __attribute__((aligned(16))) char smem[];  // W image, then NW x 16 UB
    const int d = a.d, m = a.m;
    const int64_t n = a.n;
    const int steps = (d + 31) / 32, units_per_tile = (d + UC - 1) / UC;
    const int rs = route_stage_row_bytes(d);  // bytes per image row: whole k-steps + 16
    const int img_bytes = (3 * m + 1) * rs;
    const int img_pad = (img_bytes + 1023) & ~1023;
    const int lane = threadIdx.x & 63, tok = lane & 15, kq = lane >> 4;
    const int lrow = lane / LPR, lchunk = lane % LPR;  // the row and chunk this lane loads
    const int wave_in_block = threadIdx.x >> 6;
    const int wave = uniform_int(blockIdx.x * NW + wave_in_block);
    const int64_t n_tiles = (n + 15) / 16;
    const int64_t t0 = wave < n_waves ? (int64_t)wave * n_tiles / n_waves : 0;
    const int64_t t1 = wave < n_waves ? (int64_t)(wave + 1) * n_tiles / n_waves : 0;
    const bf16 *x = static_cast<const bf16 *>(a.x);
    const uint32_t rowb = (uint32_t)d * 2;
    // this lane's byte offset within the tile for unit j's load i, or an offset past any
    // descriptor (columns at or past d)
    auto xoff = [&](int j) -> uint32_t {
        return UC * j + 8 * lchunk < d ? (uint32_t)lrow * rowb + (uint32_t)UB * j + 16u * lchunk
                                       : 0x80000000u;
    };
    // rows of one tile (none past this wave's range: those loads read zeros, touching nothing)
    auto tile_rsrc = [&](int64_t tile) {
        const int64_t rows = tile < t1 ? min((int64_t)16, n - 16 * tile) : 0;
        return make_rsrc(x + (tile < t1 ? 16 * tile : 0) * (int64_t)d, (uint32_t)rows * rowb);
    };
    // units in order: (tile, column range), column ranges fastest
    auto advance = [&](int64_t &tile, int &j) {
        if (++j == units_per_tile) { j = 0; ++tile; }
    };
    // The W image, built from W by the block: term t of W[k][g] at byte (t m + g) rs + 2k
    // (w = t0 + t1 + t2 exactly, each term bf16), zeros for k >= d, then one zero row.  Thread
    // i takes the (pair of k, g) entries i, i + 64 NW, ... (at most kImgPairs of them) and
    // writes one dword per term.  Its loads of W are issued first, then the first NH units'
    // rows: loads complete in order, so the image is built while the rows are in flight
    // (entries past the end read zeros and are not written).
    // each entry writes 12 bytes of the image, which holds at most kRouteLdsW bytes
    constexpr int kImgPairs = (kRouteLdsW / 12 + 64 * NW - 1) / (64 * NW);
    const int pairs = steps * 16 * m;  // (pair of k over whole k-steps, g)
    float wv[kImgPairs][2];
    {
        const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w, (uint32_t)d * m * 4);
#pragma unroll
        for (int i = 0; i < kImgPairs; ++i) {
            const int idx = threadIdx.x + i * 64 * NW;
            const int k2 = idx / m, g = idx - k2 * m;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int k = 2 * k2 + h;
                wv[i][h] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                    rw, (idx < pairs && k < d) ? (uint32_t)(k * m + g) * 4 : 0x80000000u, 0, 0));
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    u32x4 ring[NH][NL];
    int64_t tp = t0;
    int jp = 0;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        const __amdgpu_buffer_rsrc_t r0 = tile_rsrc(tp);
        const uint32_t o = xoff(jp);
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            ring[h][i] = __builtin_amdgcn_raw_buffer_load_b128(r0, o + i * RPI * rowb, 0, kStreamed);
            __builtin_amdgcn_sched_barrier(0);  // the order the loop consumes them in
        }
        advance(tp, jp);
    }
    {
#pragma unroll
        for (int i = 0; i < kImgPairs; ++i) {
            const int idx = threadIdx.x + i * 64 * NW;
            if (idx < pairs) {
                const int k2 = idx / m, g = idx - k2 * m;
                uint32_t packed[3] = {0u, 0u, 0u};
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const float v = wv[i][h];
                    const bf16 b0 = (bf16)v;
                    const float r1 = v - (float)b0;  // exact
                    const bf16 b1 = (bf16)r1;
                    const bf16 b2 = (bf16)(r1 - (float)b1);  // exact, at most 8 significant bits
                    packed[0] |= (uint32_t)__builtin_bit_cast(uint16_t, b0) << (16 * h);
                    packed[1] |= (uint32_t)__builtin_bit_cast(uint16_t, b1) << (16 * h);
                    packed[2] |= (uint32_t)__builtin_bit_cast(uint16_t, b2) << (16 * h);
                }
#pragma unroll
                for (int t = 0; t < 3; ++t)
                    *reinterpret_cast<uint32_t *>(smem + (t * m + g) * rs + 4 * k2) = packed[t];
            }
        }
        for (int b = 4 * threadIdx.x; b < rs; b += 4 * 64 * NW)
            *reinterpret_cast<uint32_t *>(smem + 3 * m * rs + b) = 0u;
    }
    __syncthreads();
    // A fragments: lane (g = tok, kq) reads term t of W[32 st + 8 kq .. +8][g]; lanes of padding
    // groups (g >= m) read the zero row, so the k-step loop has no branch
    const bool wact = tok < m;
    const char *wl0 = smem + (wact ? tok * rs : 3 * m * rs) + 16 * kq;
    const int wterm = wact ? m * rs : 0;
    char *xs = smem + img_pad + wave_in_block * (16 * UB);
    const char *xr = xs + tok * UB;

    double psum[4];
    int cnt[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) { psum[v] = 0.0; cnt[v] = 0; }
    f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    int pin_raw = -1;

    // one unit: write ring part H (unit (tc, jc)) into the LDS tile and refill it with unit
    // (tp, jp), NH units ahead; multiply; finish the tile after its last unit
    auto unit = [&](auto hc, int64_t tc, int jc) {
        constexpr int H = decltype(hc)::value;
        // the pin of this row's token, read in every unit of the tile (none: zero records);
        // issued before the refills, so waiting for it waits for nothing newer
        const __amdgpu_buffer_rsrc_t rp = make_rsrc(
            a.pin ? a.pin + (tc < t1 ? 16 * tc : 0) : nullptr,
            (a.pin && tc < t1) ? (uint32_t)min((int64_t)16, n - 16 * tc) * 4 : 0u);
        pin_raw = (int)__builtin_amdgcn_raw_buffer_load_b32(rp, 4u * tok, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (jc == 0) acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        const __amdgpu_buffer_rsrc_t rn = tile_rsrc(tp);
        const uint32_t on = xoff(jp);
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int r = RPI * i + lrow;
            *reinterpret_cast<u32x4 *>(xs + r * UB + ((lchunk ^ (r & 15)) << 4)) = ring[H][i];
            __builtin_amdgcn_sched_barrier(0);
            ring[H][i] = __builtin_amdgcn_raw_buffer_load_b128(rn, on + i * RPI * rowb, 0, kStreamed);
            __builtin_amdgcn_sched_barrier(0);
        }
        // operands of k-step s of this unit: the three W terms and the x tile's k-slice
        auto frag_read = [&](bf16x8 (&f)[4], int s) {
            const int st = KS * jc + s;
#pragma unroll
            for (int t = 0; t < 3; ++t)
                f[t] = *reinterpret_cast<const bf16x8 *>(wl0 + t * wterm + 64 * st);
            f[3] = *reinterpret_cast<const bf16x8 *>(xr + (((4 * s + kq) ^ tok) << 4));
        };
        auto frag_mma = [&](const bf16x8 (&f)[4]) {
#pragma unroll
            for (int t = 2; t >= 0; --t)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f[t], f[3], acc, 0, 0, 0);
        };
        const int ks = min(KS, steps - KS * jc);
        if (ks == KS) {
            // reads two k-steps ahead of the products (a ring of three operand sets), so the
            // LDS latency is covered by the products of the two steps in between
            bf16x8 fr[3][4];
            frag_read(fr[0], 0);
            frag_read(fr[1], 1);
#pragma unroll
            for (int s2 = 0; s2 < KS; ++s2) {
                if (s2 + 2 < KS) frag_read(fr[(s2 + 2) % 3], s2 + 2);
                __builtin_amdgcn_sched_barrier(0);
                frag_mma(fr[s2 % 3]);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            for (int s2 = 0; s2 < ks; ++s2) {
                bf16x8 f[4];
                frag_read(f, s2);
                frag_mma(f);
            }
        }
        if (jc + 1 == units_per_tile && tc < t1) {
            // lane (tok, kq) holds the logits of groups 4 kq + v (v < 4) of token 16 tc + tok
            const int64_t tt = 16 * tc + tok;
            const bool valid = tt < n;
            float best = 0.0f;
            int bi = kNoGroup;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int g = 4 * kq + v;
                if (g < m && (bi == kNoGroup || acc[v] > best)) { best = acc[v]; bi = g; }
            }
#pragma unroll
            for (int off = 16; off <= 32; off <<= 1) {
                const float ob = __shfl_xor(best, off, 64);
                const int oi = __shfl_xor(bi, off, 64);
                if (oi != kNoGroup && (bi == kNoGroup || ob > best || (ob == best && oi < bi))) {
                    best = ob;
                    bi = oi;
                }
            }
            const int gs = (a.pin && valid && pin_raw >= 0 && pin_raw < m) ? pin_raw : bi;
            float e[4];
            float z = 0.0f;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int g = 4 * kq + v;
                e[v] = g < m ? __builtin_amdgcn_exp2f((acc[v] - best) * kLog2e) : 0.0f;
                z += e[v];
            }
            z += __shfl_xor(z, 16, 64);
            z += __shfl_xor(z, 32, 64);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int g = 4 * kq + v;
                if (g < m && valid) {
                    const float p = e[v] / z;
                    psum[v] += (double)p;
                    if (g == gs) {
                        cnt[v] += 1;
                        a.group_id[tt] = gs;
                        a.p_sel[tt] = p;
                    }
                }
            }
        }
        advance(tp, jp);
    };

    // NH units per iteration (one per ring part); a count that is not a multiple of NH ends
    // with units past the range, whose loads read nothing and whose tiles are not finished
    const int64_t n_units = (t1 - t0) * units_per_tile;
    int64_t tc = t0;
    int jc = 0;
    for (int64_t u = 0; u < n_units; u += NH) {
        unit(std::integral_constant<int, 0>{}, tc, jc);
        advance(tc, jc);
        if constexpr (NH == 2) {
            unit(std::integral_constant<int, 1>{}, tc, jc);
            advance(tc, jc);
        }
    }
    if (wave < n_waves) {
        // statistics of the wave: the 16 lanes of one k-quarter hold the same groups
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) {
                psum[v] += __shfl_xor(psum[v], off, 64);
                cnt[v] += __shfl_xor(cnt[v], off, 64);
            }
        if (tok == 0) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int g = 4 * kq + v;
                if (g < m) {
                    a.part_p[(int64_t)wave * m + g] = psum[v];
                    a.part_c[(int64_t)wave * m + g] = cnt[v];
                }
            }
        }
    }
}

// Columns of W per chunk of route_chunk_kernel, and the bytes of one image row in LDS: the
// chunk's 512 bytes plus 16, an odd number (33) of 16-byte pieces, so the 16 group rows that
// one k-slice read touches start in 16 different bank groups.
constexpr int kChunkCols = 256;
constexpr int kChunkRow = 2 * kChunkCols + 16;
constexpr size_t kLdsBytes = 160 * 1024;  // LDS of one workgroup

// Workgroup barrier for data written into LDS with ordinary stores, leaving vector-memory loads
// in flight: any fence would wait for them, so the wave's LDS stores are waited for explicitly
// (lgkmcnt(0)) and the empty asm statements keep the compiler from moving memory accesses
// across.
__device__ __forceinline__ void lds_store_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt left at their maximum
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// LDS of one image buffer of route_chunk_kernel: 3m rows of terms and one zero row.
__host__ __device__ inline int route_chunk_wbuf(int m) {
    return ((3 * m + 1) * kChunkRow + 255) & ~255;
}

// The image route_chunk_kernel streams, chunk-major: chunk c, row t m + g, column j holds term t
// of W[256 c + j][g] (w = t0 + t1 + t2 exactly, each term bf16; zero for k >= d).  Thread i
// takes the column pair (2 j2, 2 j2 + 1) of one (chunk, group) and writes one dword per term.
__global__ __launch_bounds__(256) void route_image_kernel(const float *w, int d, int m,
                                                          int n_chunks, uint32_t *img) {
    constexpr int kPairs = kChunkCols / 2;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)n_chunks * m * kPairs) return;
    const int j2 = (int)(idx % kPairs);
    const int64_t rest = idx / kPairs;
    const int g = (int)(rest % m), c = (int)(rest / m);
    uint32_t packed[3] = {0u, 0u, 0u};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int k = c * kChunkCols + 2 * j2 + h;
        const float v = k < d ? w[(int64_t)k * m + g] : 0.0f;
        const bf16 b0 = (bf16)v;
        const float r1 = v - (float)b0;  // exact
        const bf16 b1 = (bf16)r1;
        const bf16 b2 = (bf16)(r1 - (float)b1);  // exact, at most 8 significant bits
        packed[0] |= (uint32_t)__builtin_bit_cast(uint16_t, b0) << (16 * h);
        packed[1] |= (uint32_t)__builtin_bit_cast(uint16_t, b1) << (16 * h);
        packed[2] |= (uint32_t)__builtin_bit_cast(uint16_t, b2) << (16 * h);
    }
#pragma unroll
    for (int t = 0; t < 3; ++t)
        img[((int64_t)c * 3 * m + t * m + g) * kPairs + j2] = packed[t];
}

// LDS of route_chunk_kernel<NW, T>: two image buffers and one tile of T x 16 rows per wave.
template <int NW, int T>
constexpr size_t route_chunk_smem(int m) {
    return 2 * (size_t)route_chunk_wbuf(m) + (size_t)NW * 16 * T * 2 * kChunkCols;
}

// Row-contiguous reads for the matrix cores with W streamed through LDS (bf16 x, m <= 16 MT,
// a three-term W image too large for route_stage_kernel's LDS budget, as at width 5120).  A
// block of NW waves owns a contiguous, balanced range of 16-token tiles and takes them NW*T at
// a time (T consecutive tiles per wave), running through W in chunks of 256 columns.  A unit
// of work is one chunk of the block's current tiles: each wave writes its tiles' rows (T x 16
// rows x 512 bytes, 16-byte piece c of row r at position c ^ (r & 15)) from its ring of
// registers into its own LDS tile, refills the ring with the unit NH ahead, and multiplies the
// rows by the block's LDS copy of the chunk (16x16x32 MFMAs, A = W terms, B = x).  Meanwhile
// the block loads the next chunk of the image (from L2) into registers and writes it into the
// other of two LDS buffers, handed over behind a barrier that waits for LDS stores only, so the
// rows' loads stay in flight across it.  The waves' statistics are summed in a fixed order
// into row blockIdx.x of part_p / part_c.
template <int NW, int T, int MT, int NH>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void route_chunk_kernel(RouteLaunch a, const void *img, int n_chunks, int n_blocks) {
    static_assert(NH == 1 || NH == 2, "the unit loop below handles one or two ring parts");
    static_assert(NW % 4 == 0, "whole waves per SIMD");
    constexpr int UB = 2 * kChunkCols;   // bytes of a row per chunk
    constexpr int LPR = UB / 16;         // lanes per row in a load
    constexpr int RPI = 64 / LPR;        // rows per load instruction
    constexpr int NL = 16 * T / RPI;     // load instructions per unit
    constexpr int KS = kChunkCols / 32;  // k-steps per chunk
    constexpr int PPR = UB / 16;         // 16-byte pieces per image row
    constexpr int NWL = (3 * 16 * MT * PPR + 64 * NW - 1) / (64 * NW);  // image loads per thread
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int d = a.d, m = a.m;
    const int64_t n = a.n;
    const int wbuf = route_chunk_wbuf(m);
    const int lane = threadIdx.x & 63, tok = lane & 15, kq = lane >> 4;
    const int lrow = lane / LPR, lchunk = lane % LPR;  // the row and piece this lane loads
    const int wv = uniform_int(threadIdx.x >> 6);
    const int64_t n_tiles = (n + 15) / 16;
    const int64_t bt0 = (int64_t)blockIdx.x * n_tiles / n_blocks;
    const int64_t bt1 = (int64_t)(blockIdx.x + 1) * n_tiles / n_blocks;
    const int n_units = (int)((bt1 - bt0 + NW * T - 1) / (NW * T)) * n_chunks;
    const int64_t row_end = min(n, 16 * bt1);  // rows of this block end here
    const bf16 *x = static_cast<const bf16 *>(a.x);
    const uint32_t rowb = (uint32_t)d * 2;
    // this wave's first tile in tile group k
    auto wave_tile = [&](int k) { return bt0 + (int64_t)k * (NW * T) + wv * T; };
    // this wave's rows in tile group k (none past the block's range: those loads read zeros)
    auto rows_rsrc = [&](int k) {
        const int64_t r0 = 16 * wave_tile(k);
        const int64_t rows = r0 < row_end ? min((int64_t)(16 * T), row_end - r0) : 0;
        return make_rsrc(x + (rows > 0 ? r0 : 0) * (int64_t)d, (uint32_t)rows * rowb);
    };
    // this lane's byte offset in its rows for chunk c, or one past any descriptor (columns at
    // or past d)
    auto xoff = [&](int c) -> uint32_t {
        return kChunkCols * c + 8 * lchunk < d
                   ? (uint32_t)lrow * rowb + (uint32_t)UB * c + 16u * lchunk
                   : 0x80000000u;
    };
    const int pieces = 3 * m * PPR;  // of one chunk of the image
    const __amdgpu_buffer_rsrc_t rimg = make_rsrc(img, (uint32_t)n_chunks * pieces * 16);
    auto load_image = [&](u32x4 (&wr)[NWL], int c, bool live) {
#pragma unroll
        for (int i = 0; i < NWL; ++i) {
            const int pc = threadIdx.x + i * 64 * NW;
            wr[i] = __builtin_amdgcn_raw_buffer_load_b128(
                rimg, (live && pc < pieces) ? (uint32_t)(c * pieces + pc) * 16 : 0x80000000u, 0, 0);
        }
    };
    auto store_image = [&](const u32x4 (&wr)[NWL], int b) {
#pragma unroll
        for (int i = 0; i < NWL; ++i) {
            const int pc = threadIdx.x + i * 64 * NW;
            if (pc < pieces)
                *reinterpret_cast<u32x4 *>(smem + b * wbuf + (pc / PPR) * kChunkRow +
                                           (pc % PPR) * 16) = wr[i];
        }
    };
    // units in order: (tile group, chunk), chunks fastest
    auto advance = [&](int &k, int &c) {
        if (++c == n_chunks) { c = 0; ++k; }
    };

    // zero rows of both buffers (read by the lanes of padding groups), the first chunk, and the
    // rows of the first NH units
    if ((int)threadIdx.x < kChunkRow / 4) {
        *reinterpret_cast<uint32_t *>(smem + 3 * m * kChunkRow + 4 * threadIdx.x) = 0u;
        *reinterpret_cast<uint32_t *>(smem + wbuf + 3 * m * kChunkRow + 4 * threadIdx.x) = 0u;
    }
    u32x4 wr[NWL];
    load_image(wr, 0, true);
    __builtin_amdgcn_sched_barrier(0);
    u32x4 ring[NH][NL];
    int kp = 0, cp = 0;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        const __amdgpu_buffer_rsrc_t r0 = rows_rsrc(kp);
        const uint32_t o = xoff(cp);
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            ring[h][i] = __builtin_amdgcn_raw_buffer_load_b128(r0, o + i * RPI * rowb, 0, kStreamed);
            __builtin_amdgcn_sched_barrier(0);  // the order the loop consumes them in
        }
        advance(kp, cp);
    }
    store_image(wr, 0);
    lds_store_barrier();

    // A fragments: lane (g = tok, kq) of group tile mt reads term t of W[32 s + 8 kq .. +8]
    // [16 mt + g]; lanes of padding groups read the zero row, so the k-step loop has no branch
    int wl[MT], wterm[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const bool act = 16 * mt + tok < m;
        wl[mt] = (act ? (16 * mt + tok) : 3 * m) * kChunkRow + 16 * kq;
        wterm[mt] = act ? m * kChunkRow : 0;
    }
    char *xs = smem + 2 * wbuf + wv * (16 * T * UB);

    double psum[MT][4];
    int cnt[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) { psum[mt][v] = 0.0; cnt[mt][v] = 0; }
    f32x4 acc[T][MT];
    int pin_raw[T];

    // one unit u = (k, c): write ring part H into the LDS tile and refill it with unit (kp, cp),
    // NH units ahead; multiply; finish the tiles after the last chunk; hand over the next chunk
    auto unit = [&](auto hc, int u, int k, int c) {
        constexpr int H = decltype(hc)::value;
        const int64_t tile0 = wave_tile(k);
        // the pins of this lane's tokens, read in every unit (none: zero records); issued before
        // the refills, so waiting for them waits for nothing newer
        {
            const int64_t r0 = 16 * tile0;
            const int64_t rows = (a.pin && r0 < row_end) ? min((int64_t)(16 * T), row_end - r0) : 0;
            const __amdgpu_buffer_rsrc_t rp = make_rsrc(a.pin + (rows > 0 ? r0 : 0),
                                                        (uint32_t)rows * 4);
#pragma unroll
            for (int i = 0; i < T; ++i)
                pin_raw[i] = (int)__builtin_amdgcn_raw_buffer_load_b32(rp, 4u * (16 * i + tok), 0, 0);
        }
        const bool wnext = u + 1 < n_units;
        load_image(wr, c + 1 == n_chunks ? 0 : c + 1, wnext);
        __builtin_amdgcn_sched_barrier(0);
        const __amdgpu_buffer_rsrc_t rn = rows_rsrc(kp);
        const uint32_t on = xoff(cp);
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int r = RPI * i + lrow;
            *reinterpret_cast<u32x4 *>(xs + r * UB + ((lchunk ^ (r & 15)) << 4)) = ring[H][i];
            __builtin_amdgcn_sched_barrier(0);
            ring[H][i] = __builtin_amdgcn_raw_buffer_load_b128(rn, on + i * RPI * rowb, 0, kStreamed);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (c == 0) {
#pragma unroll
            for (int i = 0; i < T; ++i)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) acc[i][mt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
        const char *wb = smem + (u & 1) * wbuf;
        // operands of k-step s: the three W terms of each group tile and the x k-slice of each
        // tile
        struct Ops {
            bf16x8 w[3][MT];
            bf16x8 x[T];
        };
        auto read_ops = [&](Ops &f, int s) {
#pragma unroll
            for (int t = 0; t < 3; ++t)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    f.w[t][mt] = *reinterpret_cast<const bf16x8 *>(wb + wl[mt] + t * wterm[mt] + 64 * s);
#pragma unroll
            for (int i = 0; i < T; ++i)
                f.x[i] = *reinterpret_cast<const bf16x8 *>(xs + (16 * i + tok) * UB +
                                                           (((4 * s + kq) ^ tok) << 4));
        };
        auto mma = [&](const Ops &f) {
#pragma unroll
            for (int t = 2; t >= 0; --t)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int i = 0; i < T; ++i)
                        acc[i][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.w[t][mt], f.x[i],
                                                                             acc[i][mt], 0, 0, 0);
        };
        // reads one k-step ahead of the products
        Ops fr[2];
        read_ops(fr[0], 0);
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) {
            if (s2 + 1 < KS) read_ops(fr[(s2 + 1) & 1], s2 + 1);
            __builtin_amdgcn_sched_barrier(0);
            mma(fr[s2 & 1]);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (c + 1 == n_chunks) {
#pragma unroll
            for (int i = 0; i < T; ++i) {
                const int64_t t = 16 * (tile0 + i) + tok;
                if (16 * (tile0 + i) < row_end)  // the same for the whole wave
                    route_token<MT>(a, acc[i], t, t < row_end, a.pin ? pin_raw[i] : -1, kq, psum,
                                    cnt);
            }
        }
        if (wnext) store_image(wr, (u + 1) & 1);
        lds_store_barrier();
        advance(kp, cp);
    };

    // NH units per iteration (one per ring part); a count that is not a multiple of NH ends
    // with a unit past the range, whose loads read nothing and whose tiles are not finished
    int kc = 0, cc = 0;
    for (int u = 0; u < n_units; u += NH) {
        unit(std::integral_constant<int, 0>{}, u, kc, cc);
        advance(kc, cc);
        if constexpr (NH == 2) {
            unit(std::integral_constant<int, 1>{}, u + 1, kc, cc);
            advance(kc, cc);
        }
    }
    // the block's statistics: each wave's, then the waves' in order (through LDS)
    route_wave_stats<MT>(psum, cnt);
    __syncthreads();
    double *sp = reinterpret_cast<double *>(smem);                 // [NW][16 MT]
    int *sc = reinterpret_cast<int *>(smem + NW * 16 * MT * 8);    // [NW][16 MT]
    if (tok == 0) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                sp[wv * 16 * MT + 16 * mt + 4 * kq + v] = psum[mt][v];
                sc[wv * 16 * MT + 16 * mt + 4 * kq + v] = cnt[mt][v];
            }
    }
    __syncthreads();
    if ((int)threadIdx.x < m) {
        double p = 0.0;
        int c = 0;
        for (int w = 0; w < NW; ++w) {
            p += sp[w * 16 * MT + threadIdx.x];
            c += sc[w * 16 * MT + threadIdx.x];
        }
        a.part_p[(int64_t)blockIdx.x * m + threadIdx.x] = p;
        a.part_c[(int64_t)blockIdx.x * m + threadIdx.x] = c;
    }
}

// One block per group: fixed-order sum of the per-block partials.
__global__ __launch_bounds__(256) void route_finalize(const double *part_p, const int32_t *part_c,
                                                       int64_t nblk, int stride, double *prob_sum,
                                                       int32_t *counts) {
    __shared__ double sp[256];
    __shared__ int sc[256];
    const int g = blockIdx.x;
    double s = 0.0;
    int c = 0;
    // rows tid, tid + 256, ... added in that order; eight loads in flight at a time (clamped
    // rows, whose values are not used, keep them unconditional)
    for (int64_t b0 = threadIdx.x; b0 < nblk; b0 += 256 * 8) {
        double vp[8];
        int vc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t b = min(b0 + 256 * i, nblk - 1);
            vp[i] = part_p[b * stride + g];
            vc[i] = part_c[b * stride + g];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (b0 + 256 * i < nblk) { s += vp[i]; c += vc[i]; }
    }
    sp[threadIdx.x] = s;
    sc[threadIdx.x] = c;
    __syncthreads();
    for (int w = 128; w >= 1; w >>= 1) {
        if ((int)threadIdx.x < w) {
            sp[threadIdx.x] += sp[threadIdx.x + w];
            sc[threadIdx.x] += sc[threadIdx.x + w];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        prob_sum[g] = sp[0];
        counts[g] = sc[0];
    }
}

template <int MM, int TPW>
hipError_t launch_mm(const RouteLaunch &a, hipStream_t s) {
    const int vec = a.x_is_bf16 ? 8 : 4;
    int dc = a.d;
    if ((size_t)MM * a.d * sizeof(float) > (size_t)kRouteLdsBytes) {
        dc = kRouteLdsBytes / (MM * (int)sizeof(float));
        dc -= dc % vec;  // stripes of a chunk may be partial; chunks stay VEC-aligned
    }
    const size_t lds = (size_t)MM * dc * sizeof(float);
    const int64_t nblk = route_blocks(a.n);
    if (a.x_is_bf16)
        hipLaunchKernelGGL((route_kernel<MM, TPW, true>), dim3((unsigned)nblk), dim3(256), lds, s,
                           a, dc);
    else
        hipLaunchKernelGGL((route_kernel<MM, TPW, false>), dim3((unsigned)nblk), dim3(256), lds, s,
                           a, dc);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(route_finalize, dim3(a.m), dim3(256), 0, s, a.part_p, a.part_c, nblk,
                       kMaxGroups, a.prob_sum, a.counts);
    return hipGetLastError();
}

template <int NW, int NH, int UB>
hipError_t launch_stage(const RouteLaunch &a, size_t lds, hipStream_t s) {
    int cus = 0;
    hipError_t e = device_cus(&cus);
    if (e != hipSuccess) return e;
    const size_t smem = ((lds + 1023) & ~(size_t)1023) + (size_t)NW * 16 * UB;
    // once per device (and thread-safe): allow the largest image, kRouteLdsW + NW x 16 UB
    static DeviceOnce attr;
    if ((e = attr.run([] {
             return hipFuncSetAttribute(
                 reinterpret_cast<const void *>(&route_stage_kernel<NW, NH, UB>),
                 hipFuncAttributeMaxDynamicSharedMemorySize, kRouteLdsW + NW * 16 * UB);
         })) != hipSuccess)
        return e;
    // one block of NW waves per CU, at least one tile (16 tokens) per wave (short inputs still
    // spread over every CU), and no more waves than rows of partial statistics
    const int64_t n_tiles = (a.n + 15) / 16;
    const int64_t n_waves = std::max<int64_t>(
        1, std::min<int64_t>({(int64_t)cus * NW, n_tiles, route_partials(a.n)}));
    hipLaunchKernelGGL((route_stage_kernel<NW, NH, UB>), dim3((unsigned)((n_waves + NW - 1) / NW)),
                       dim3(64 * NW), smem, s, a, (int)n_waves);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(route_finalize, dim3(a.m), dim3(256), 0, s, a.part_p, a.part_c, n_waves,
                       a.m, a.prob_sum, a.counts);
    return hipGetLastError();
}

template <int NW, int T, int MT, int NH>
hipError_t launch_chunk(const RouteLaunch &a, hipStream_t s) {
    int cus = 0;
    hipError_t e = device_cus(&cus);
    if (e != hipSuccess) return e;
    // once per device (and thread-safe): allow the largest LDS of this instantiation
    static DeviceOnce attr;
    if ((e = attr.run([] {
             return hipFuncSetAttribute(
                 reinterpret_cast<const void *>(&route_chunk_kernel<NW, T, MT, NH>),
                 hipFuncAttributeMaxDynamicSharedMemorySize,
                 (int)std::min(route_chunk_smem<NW, T>(16 * MT), kLdsBytes));
         })) != hipSuccess)
        return e;
    const int n_chunks = (a.d + kChunkCols - 1) / kChunkCols;
    uint32_t *img = reinterpret_cast<uint32_t *>(static_cast<char *>(a.wsplit) + 256);
    const int64_t pairs = (int64_t)n_chunks * a.m * (kChunkCols / 2);
    hipLaunchKernelGGL(route_image_kernel, dim3((unsigned)((pairs + 255) / 256)), dim3(256), 0, s,
                       a.w, a.d, a.m, n_chunks, img);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // at most one block per CU, each with the same whole number of tile groups (NW*T tiles) as
    // nearly as the count allows, so that no block ends on a mostly empty group (60 s router:
    // 256 blocks of 17.2 groups 1.012 ms, 245 blocks of 17.96 0.988 ms)
    const int64_t n_tiles = (a.n + 15) / 16;
    const int64_t groups = (n_tiles + NW * T - 1) / (NW * T);
    const int64_t iters = (groups + cus - 1) / cus;
    const int n_blocks = (int)std::max<int64_t>(1, (groups + iters - 1) / iters);
    const size_t smem = route_chunk_smem<NW, T>(a.m);
    hipLaunchKernelGGL((route_chunk_kernel<NW, T, MT, NH>), dim3((unsigned)n_blocks),
                       dim3(64 * NW), smem, s, a,
                       static_cast<const void *>(img), n_chunks, n_blocks);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(route_finalize, dim3(a.m), dim3(256), 0, s, a.part_p, a.part_c, n_blocks,
                       a.m, a.prob_sum, a.counts);
    return hipGetLastError();
}

template <int MT, int T, int U>
hipError_t launch_mfma(const RouteLaunch &a, hipStream_t s) {
    // occupancy of this instantiation, queried once per device (thread-safe)
    static DeviceOnce occ;
    static std::atomic<int> occ_blocks[kMaxDevices];
    int cus = 0;
    hipError_t e = device_cus(&cus);
    if (e != hipSuccess) return e;
    int dev = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    if ((e = occ.run([dev] {
             int b = 0;
             const hipError_t r = hipOccupancyMaxActiveBlocksPerMultiprocessor(
                 &b, reinterpret_cast<const void *>(&route_mfma_kernel<MT, T, U>), 256, 0);
             occ_blocks[dev].store(b > 0 ? b : 1);
             return r;
         })) != hipSuccess)
        return e;
    const int blocks_per_cu = occ_blocks[dev].load();
    const int steps = (a.d + 31) / 32;
    const int64_t frags = (int64_t)MT * steps * 64;
    int *queue = reinterpret_cast<int *>(a.wsplit);
    bf16x8 *wf = reinterpret_cast<bf16x8 *>(static_cast<char *>(a.wsplit) + 256);
    hipLaunchKernelGGL(route_split_kernel, dim3((unsigned)((frags + 255) / 256)), dim3(256), 0, s,
                       a.w, a.d, a.m, MT, steps, wf, queue);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t n_items = (a.n + 16 * T - 1) / (16 * T);
    const int64_t grid = std::min<int64_t>((int64_t)cus * blocks_per_cu, (n_items + 3) / 4);
    hipLaunchKernelGGL((route_mfma_kernel<MT, T, U>), dim3((unsigned)grid), dim3(256), 0, s, a,
                       wf, queue, steps);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(route_finalize, dim3(a.m), dim3(256), 0, s, a.part_p, a.part_c, n_items,
                       a.m, a.prob_sum, a.counts);
    return hipGetLastError();
}

}  // namespace

int64_t route_blocks(int64_t n) { return (n + kRouteTokensPerBlock - 1) / kRouteTokensPerBlock; }

int64_t route_partials(int64_t n) {
    // per-block rows of kMaxGroups (fp32 x) or per-wave / per-block / per-item rows of
    // m <= kMaxGroups (bf16 x: waves and blocks of at least one 16-token tile, items of 64 tokens)
    return std::max<int64_t>(route_blocks(n), (n + 15) / 16);
}

size_t route_split_bytes(int d, int m) {
    const size_t frags = (size_t)3 * ((m + 15) / 16) * ((d + 31) / 32) * 64 * sizeof(bf16x8);
    const size_t image = (size_t)3 * m * ((d + kChunkCols - 1) / kChunkCols) * kChunkCols * 2;
    return 256 + std::max(frags, image);
}

hipError_t launch_route(const RouteLaunch &a, hipStream_t s) {
    if (a.x_is_bf16) {
        const size_t lds_img = (size_t)(3 * a.m + 1) * route_stage_row_bytes(a.d);
        if (a.m <= 16 && lds_img <= (size_t)kRouteLdsW) return launch_stage<8, 1, 512>(a, lds_img, s);
        // a larger image streamed through LDS in chunks of columns, as long as two chunk buffers
        // and the row tiles fit
        if (a.m <= 16) return launch_chunk<8, 1, 1, 2>(a, s);
        if (route_chunk_smem<8, 1>(a.m) <= kLdsBytes) return launch_chunk<8, 1, 2, 2>(a, s);
        // W fragments streamed from L2 into registers, many 16-token tiles per item, so that
        // each fragment serves as many tokens as the registers allow
        if (a.m <= 32) return launch_mfma<2, 10, 1>(a, s);
        if (a.m <= 48) return launch_mfma<3, 2, 1>(a, s);
        return launch_mfma<4, 2, 1>(a, s);
    }
    if (a.m <= 4) return launch_mm<4, 4>(a, s);
    if (a.m <= 5) return launch_mm<5, 4>(a, s);
    if (a.m <= 8) return launch_mm<8, 4>(a, s);
    if (a.m <= 16) return launch_mm<16, 2>(a, s);
    if (a.m <= 20) return launch_mm<20, 2>(a, s);
    if (a.m <= 32) return launch_mm<32, 1>(a, s);
    return launch_mm<64, 1>(a, s);
}

}  // namespace moga

// Token router: r = x W (fp32, no bias), p = softmax(r), g = argmax r, p_sel = p[g],
// plus per-group counts and fp64 sums of p (papernotes.org MoGA note, 关键设计 1 and 3;
// xugj520.cn MoGA blog §2.3 for the linear, bias-free form and the argmax).
//
// bf16 x (the model's activations): x W on the matrix cores.  W is fp32, so it is split
// exactly into three bf16 terms, w = w1 + w2 + w3 (w1 = bf16(w), w2 = bf16(w - w1),
// w3 = w - w1 - w2, which needs at most 8 significant bits): every product x*w_j is exact
// in fp32 and the MFMA accumulates in fp32, so the logits carry fp32 accuracy.  One
// 16x16x32 MFMA takes 16 groups (A, from the split W) against 16 tokens (B, one 16-byte
// load of x per lane), so each logit's reduction over d happens inside the matrix core and
// only the softmax needs two cross-lane steps.  Each wave owns a contiguous run of token
// tiles (a balanced static split), so the group statistics are summed in a fixed order.
//
// fp32 x: VALU pass.  Each wave streams TPW token rows at a time with 16-byte coalesced
// loads (lane l holds columns [VEC*l, VEC*l+VEC) of every 64*VEC-wide stripe), multiplies
// them by W^T staged once per block in LDS, and reduces the per-lane partial logits across
// the wave.  Group statistics are kept per lane (lane i owns group i).
#include <algorithm>

#include "moga_internal.h"

namespace moga {
namespace {

constexpr int kRouteLdsBytes = 64 * 1024;

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
    if (threadIdx.x < m) {
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
        f.x[i] = as_bf16x8(__builtin_amdgcn_raw_buffer_load_b128(rx, xoff[i], 64 * s, 0));
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

// Softmax, argmax (lowest group index on equal logits), pins, outputs and the statistics of
// one work item of T*16 tokens starting at t0.  Lane l holds the logits acc[i][mt][v] of
// groups 16mt + 4kq + v of token t0 + 16i + tok; the item's statistics go to row `item` of
// part_p / part_c (stride m).
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
        // argmax, lowest group index on equal logits
        float best = 0.0f;
        int bi = kNoGroup;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int g = 16 * mt + 4 * kq + v;
                if (g < m && (bi == kNoGroup || acc[i][mt][v] > best)) {
                    best = acc[i][mt][v];
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
        int g = bi;
        if (a.pin && valid) {
            const int pv = a.pin[t];
            if (pv >= 0 && pv < m) g = pv;
        }
        float e[MT][4];
        float z = 0.0f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int gg = 16 * mt + 4 * kq + v;
                e[mt][v] = gg < m ? __builtin_amdgcn_exp2f((acc[i][mt][v] - best) * kLog2e)
                                  : 0.0f;
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
    // item statistics: the 16 lanes of one k-quarter hold the same groups
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) {
                psum[mt][v] += __shfl_xor(psum[mt][v], off, 64);
                cnt[mt][v] += __shfl_xor(cnt[mt][v], off, 64);
            }
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
    const int d = a.d, m = a.m;
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
            // whole groups of 2U steps without branches (see route_lds_kernel), then the rest
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

// W resident in LDS.  When the three bf16 terms of W fit (3 * m * row bytes <= kRouteLdsW),
// every persistent block splits W once into LDS, [term][group][k] with rows padded to whole
// k-steps (zeros past d).  The A fragments then come from LDS just before their MFMAs, on
// the LDS counter, so the x loads can run DX k-steps ahead in a ring of registers without
// W loads queued behind them (global loads complete in issue order).  m <= 16.
constexpr int kRouteLdsW = 64 * 1024;

inline int route_lds_row_bytes(int d) { return ((d + 31) / 32) * 64 + 64; }

// The LDS image of W, built once per call: term j of W[k][g] at byte (j*m + g)*rs + 2k, zeros
// for k >= d, then one zero row.  One thread per (k, g) pair and one per zero-row chunk.
__global__ __launch_bounds__(256) void route_image_kernel(const float *w, int d, int m, int kp,
                                                          int rs, char *img) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t pairs = (int64_t)kp * m;
    if (idx < pairs) {
        const int k = (int)(idx / m), g = (int)(idx - (int64_t)k * m);
        const float v = k < d ? w[idx] : 0.0f;  // w[k*m + g]
        const bf16 h = (bf16)v;
        const float r1 = v - (float)h;  // exact
        const bf16 md = (bf16)r1;
        const float r2 = r1 - (float)md;  // exact, at most 8 significant bits
        *reinterpret_cast<bf16 *>(img + (int64_t)g * rs + 2 * k) = h;
        *reinterpret_cast<bf16 *>(img + (int64_t)(m + g) * rs + 2 * k) = md;
        *reinterpret_cast<bf16 *>(img + (int64_t)(2 * m + g) * rs + 2 * k) = (bf16)r2;
    } else if (idx < pairs + rs / 16) {
        *reinterpret_cast<u32x4 *>(img + (int64_t)3 * m * rs + 16 * (idx - pairs)) =
            u32x4{0u, 0u, 0u, 0u};
    }
}

template <int T, int DX, int NT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(NT == 512 ? 4 : 3)))
void route_lds_kernel(RouteLaunch a, const char *img, int lds_bytes, int *queue) {
    extern __shared__ __attribute__((aligned(16))) char wsm[];  // [3][m][rs] bf16, zero row
    const int d = a.d, m = a.m;
    const int64_t n = a.n;
    const int steps = (d + 31) / 32, full = d / 32;
    const int rs = steps * 64 + 64;
    {
        // copy the image in batches of 16 loads per thread (<= 64 KiB each), all in flight
        const __amdgpu_buffer_rsrc_t ri = make_rsrc(img, (uint32_t)lds_bytes);
        constexpr int STRIDE = 16 * NT;
        for (int b0 = 0; b0 < lds_bytes; b0 += 16 * STRIDE) {
            u32x4 v[16];
#pragma unroll
            for (int i = 0; i < 16; ++i)
                v[i] = __builtin_amdgcn_raw_buffer_load_b128(ri, b0 + STRIDE * i + 16 * threadIdx.x, 0, 0);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int b = b0 + STRIDE * i + 16 * threadIdx.x;
                if (b < lds_bytes) *reinterpret_cast<u32x4 *>(wsm + b) = v[i];
            }
        }
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, tok = lane & 15, kq = lane >> 4;
    // lanes of padding groups (>= m) read the zero row for every term: no branch in the loop
    const bool wact = (lane & 15) < m;
    const char *wl0 = wsm + (wact ? (lane & 15) * rs : 3 * m * rs) + 16 * kq;
    const int wterm = wact ? m * rs : 0;
    const int64_t n_items = (n + 16 * T - 1) / (16 * T);
    const bf16 *x = static_cast<const bf16 *>(a.x);
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
        f32x4 acc[T][1];
#pragma unroll
        for (int i = 0; i < T; ++i) acc[i][0] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        auto mma = [&](const bf16x8 (&xv)[T], int st) {
            bf16x8 wv[3];
#pragma unroll
            for (int j = 0; j < 3; ++j)
                wv[j] = *reinterpret_cast<const bf16x8 *>(wl0 + j * wterm + 64 * st);
#pragma unroll
            for (int j = 2; j >= 0; --j)
#pragma unroll
                for (int i = 0; i < T; ++i)
                    acc[i][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wv[j], xv[i], acc[i][0], 0,
                                                                        0, 0);
        };
        auto xload = [&](bf16x8 (&xv)[T], int st) {
#pragma unroll
            for (int i = 0; i < T; ++i)
                xv[i] = as_bf16x8(__builtin_amdgcn_raw_buffer_load_b128(rx, xoff[i], 64 * st, 0));
        };
        if (full > 0) {
            // whole groups of DX steps in a loop without branches (a branch inside it would
            // make the compiler wait for every load in flight), then the remaining steps,
            // whose operands the last group has already loaded
            bf16x8 ring[DX][T];
#pragma unroll
            for (int u = 0; u < DX; ++u) {
                xload(ring[u], min(u, full - 1));
                __builtin_amdgcn_sched_barrier(0);  // slots in order, as the loop refills them
            }
            const int whole = full / DX;
            for (int gi = 0; gi < whole; ++gi) {
#pragma unroll
                for (int u = 0; u < DX; ++u) {
                    mma(ring[u], gi * DX + u);
                    xload(ring[u], min(gi * DX + u + DX, full - 1));  // past the end: repeats
                    // keep the refill here: the scheduler would otherwise sink it to the end
                    // of the group and the next group would wait for loads just issued
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
#pragma unroll
            for (int u = 0; u < DX - 1; ++u)
                if (whole * DX + u < full) mma(ring[u], whole * DX + u);
        }
        if (full < steps) {  // last k-step: columns past d are zero (W is zero there too)
            bf16x8 xv[T];
            xload(xv, full);
            if (32 * full + 8 * kq >= d)
#pragma unroll
                for (int i = 0; i < T; ++i) xv[i] = bf16x8{};
            mma(xv, full);
        }
        route_finish<1, T>(a, acc, t0, item, tok, kq);
    }
}

__global__ void route_queue_reset(int *queue) {
    if (threadIdx.x == 0) *queue = 0;
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
    for (int64_t b = threadIdx.x; b < nblk; b += 256) {
        s += part_p[b * stride + g];
        c += part_c[b * stride + g];
    }
    sp[threadIdx.x] = s;
    sc[threadIdx.x] = c;
    __syncthreads();
    for (int w = 128; w >= 1; w >>= 1) {
        if (threadIdx.x < w) {
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

template <int T, int DX, int NT>
hipError_t launch_lds(const RouteLaunch &a, size_t lds, hipStream_t s) {
    static int vgpr_blocks = 0;  // blocks per CU allowed by registers (same on every gfx950)
    int cus = 0;
    hipError_t e = device_cus(&cus);
    if (e != hipSuccess) return e;
    if (vgpr_blocks == 0) {
        int b = 0;
        if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
                 &b, reinterpret_cast<const void *>(&route_lds_kernel<T, DX, NT>), NT, 0)) !=
            hipSuccess)
            return e;
        vgpr_blocks = b > 0 ? b : 1;
    }
    const int bpc = std::max(1, std::min(vgpr_blocks, (int)(160 * 1024 / lds)));
    int *queue = reinterpret_cast<int *>(a.wsplit);
    char *img = static_cast<char *>(a.wsplit) + 256;
    const int kp = (a.d + 31) / 32 * 32, rs = route_lds_row_bytes(a.d);
    const int64_t threads = (int64_t)kp * a.m + rs / 16;
    hipLaunchKernelGGL(route_image_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                       a.w, a.d, a.m, kp, rs, img);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(route_queue_reset, dim3(1), dim3(64), 0, s, queue);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t n_items = (a.n + 16 * T - 1) / (16 * T);
    const int64_t wpb = NT / 64;
    const int64_t grid = std::min<int64_t>((int64_t)cus * bpc, (n_items + wpb - 1) / wpb);
    hipLaunchKernelGGL((route_lds_kernel<T, DX, NT>), dim3((unsigned)grid), dim3(NT), lds, s, a,
                       img, (int)lds, queue);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(route_finalize, dim3(a.m), dim3(256), 0, s, a.part_p, a.part_c, n_items,
                       a.m, a.prob_sum, a.counts);
    return hipGetLastError();
}

template <int MT, int T, int U>
hipError_t launch_mfma(const RouteLaunch &a, hipStream_t s) {
    static int blocks_per_cu = 0;  // occupancy of this instantiation (same on every gfx950)
    int cus = 0;
    hipError_t e = device_cus(&cus);
    if (e != hipSuccess) return e;
    if (blocks_per_cu == 0) {
        int b = 0;
        if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
                 &b, reinterpret_cast<const void *>(&route_mfma_kernel<MT, T, U>), 256, 0)) !=
            hipSuccess)
            return e;
        blocks_per_cu = b > 0 ? b : 1;
    }
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
    // per-block rows of kMaxGroups (fp32 x) or per-item rows of m <= kMaxGroups (bf16 x, items of
    // at least 32 tokens)
    return std::max<int64_t>(route_blocks(n), (n + 31) / 32);
}

size_t route_split_bytes(int d, int m) {
    const size_t frags = (size_t)3 * ((m + 15) / 16) * ((d + 31) / 32) * 64 * sizeof(bf16x8);
    const size_t image = (size_t)(3 * m + 1) * route_lds_row_bytes(d);
    return 256 + std::max(frags, image);
}

hipError_t launch_route(const RouteLaunch &a, hipStream_t s) {
    if (a.x_is_bf16) {
        const size_t lds = (size_t)(3 * a.m + 1) * route_lds_row_bytes(a.d);
        if (a.m <= 16 && lds <= (size_t)kRouteLdsW) return launch_lds<4, 4, 256>(a, lds, s);
        if (a.m <= 16) return launch_mfma<1, 4, 2>(a, s);
        if (a.m <= 32) return launch_mfma<2, 4, 1>(a, s);
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

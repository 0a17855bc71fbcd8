// Token router: r = x W (fp32, no bias), p = softmax(r), g = argmax r, p_sel = p[g],
// plus per-group counts and fp64 sums of p (papernotes.org MoGA note, 关键设计 1 and 3;
// xugj520.cn MoGA blog §2.3 for the linear, bias-free form and the argmax).
//
// HBM-bound GEMV-like pass over x.  Each wave streams TPW token rows at a time with
// 16-byte coalesced loads (lane l holds columns [VEC*l, VEC*l+VEC) of every 64*VEC-wide
// stripe), multiplies them by W^T staged once per block in LDS, and reduces the per-lane
// partial logits across the wave.  Group statistics are kept per lane (lane i owns group
// i) and combined in a fixed order, so counts and sums are bitwise reproducible.
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

// One block per group: fixed-order sum of the per-block partials.
__global__ __launch_bounds__(256) void route_finalize(const double *part_p, const int32_t *part_c,
                                                       int64_t nblk, double *prob_sum,
                                                       int32_t *counts) {
    __shared__ double sp[256];
    __shared__ int sc[256];
    const int g = blockIdx.x;
    double s = 0.0;
    int c = 0;
    for (int64_t b = threadIdx.x; b < nblk; b += 256) {
        s += part_p[b * kMaxGroups + g];
        c += part_c[b * kMaxGroups + g];
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
                       a.prob_sum, a.counts);
    return hipGetLastError();
}

}  // namespace

int64_t route_blocks(int64_t n) { return (n + kRouteTokensPerBlock - 1) / kRouteTokensPerBlock; }

hipError_t launch_route(const RouteLaunch &a, hipStream_t s) {
    if (a.m <= 4) return launch_mm<4, 4>(a, s);
    if (a.m <= 5) return launch_mm<5, 4>(a, s);
    if (a.m <= 8) return launch_mm<8, 4>(a, s);
    if (a.m <= 16) return launch_mm<16, 2>(a, s);
    if (a.m <= 20) return launch_mm<20, 2>(a, s);
    if (a.m <= 32) return launch_mm<32, 1>(a, s);
    return launch_mm<64, 1>(a, s);
}

}  // namespace moga

// Backward of the MoGA forward, everything but the attention kernels (papernotes.org MoGA
// note, 关键设计 1: the router is trained through the p(g(x)|x) factor; 关键设计 3: L_gb).
// With the routing held fixed (the argmax and the counts are piecewise constant in x):
//   D[h][t]  = <d_out[h][t], out[h][t]>   (= <dO', O'> with dO' = p d_out, O' = out / p)
//   dp_t     = sum_h D[h][t] / p_t         (gradient with respect to p(g_t|x_t))
//   a_ti     = [i = g_t] dp_t + d_loss * alpha * M * F_i / N
//   dr_ti    = p_ti (a_ti - sum_j a_tj p_tj)    (softmax backward; p recomputed from x W)
//   dx_t     = sum_i dr_ti W[:, i],   dW = x^T dr
// Sums run in a fixed order (no floating-point atomics), so every output is reproducible.
#include <algorithm>

#include "moga_internal.h"

namespace moga {
namespace {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// D[h][t] for hd 128 rows: 16 lanes per row, 16 bytes each, then a sum over the 16 lanes.
__global__ __launch_bounds__(256) void bwd_rowdot_kernel(const bf16 *d_out, const bf16 *out,
                                                          int64_t rows, float *D) {
    const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int ch = threadIdx.x & 15;
    float acc = 0.0f;
    if (row < rows) {
        const uint4 g = *reinterpret_cast<const uint4 *>(d_out + row * 128 + ch * 8);
        const uint4 o = *reinterpret_cast<const uint4 *>(out + row * 128 + ch * 8);
        const uint32_t gw[4] = {g.x, g.y, g.z, g.w}, ow[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc = __builtin_fmaf(bf16_lo(gw[i]), bf16_lo(ow[i]), acc);
            acc = __builtin_fmaf(bf16_hi(gw[i]), bf16_hi(ow[i]), acc);
        }
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) acc += __shfl_xor(acc, off, 64);
    if (row < rows && ch == 0) D[row] = acc;
}

// dp_t = sum over heads (in head order) of D[h][t], divided by p_t.
__global__ __launch_bounds__(256) void bwd_dp_kernel(const float *D, const float *p_sel,
                                                      int64_t n, int n_heads, float *dp) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= n) return;
    float s = 0.0f;
    for (int h = 0; h < n_heads; ++h) s += D[(int64_t)h * n + t];
    dp[t] = s / p_sel[t];
}

// fp32 [H][N] rows by perm: dst[h][j] = mult * src[h][perm[j]], or with inverse set
// dst[h][perm[j]] = mult * src[h][j].  perm entries outside [0, n) are skipped.
__global__ __launch_bounds__(256) void bwd_gather_f32_kernel(const float *src, const int32_t *perm,
                                                              int64_t n, float mult, int inverse,
                                                              float *dst) {
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (j >= n) return;
    const int64_t h = blockIdx.y;
    const int32_t pj = perm[j];
    if (inverse) {
        if (pj >= 0 && pj < n) dst[h * n + pj] = mult * src[h * n + j];
    } else {
        dst[h * n + j] = (pj >= 0 && pj < n) ? mult * src[h * n + pj] : 0.0f;
    }
}

// One wave per token: logits x_t W (fp32), softmax, dr_t, dx_t.  Lanes stride over d.
template <int MM>
__global__ __launch_bounds__(256) void bwd_router_rows_kernel(BwdRouterLaunch a) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= a.n) return;
    const int d = a.d, m = a.m;
    float r[MM];
#pragma unroll
    for (int i = 0; i < MM; ++i) r[i] = 0.0f;
    for (int c = lane; c < d; c += 64) {
        const float xv = a.x_is_bf16 ? (float)static_cast<const bf16 *>(a.x)[t * d + c]
                                     : static_cast<const float *>(a.x)[t * d + c];
#pragma unroll
        for (int i = 0; i < MM; ++i)
            if (i < m) r[i] = __builtin_fmaf(xv, a.w[(int64_t)c * m + i], r[i]);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < MM; ++i) {
        if (i < m) {
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) r[i] += __shfl_xor(r[i], off, 64);
            mx = fmaxf(mx, r[i]);
        }
    }
    float z = 0.0f;
#pragma unroll
    for (int i = 0; i < MM; ++i)
        if (i < m) { r[i] = __expf(r[i] - mx); z += r[i]; }
    const int g = a.group_id[t];
    const float dp = a.dp[t];
    float dot = 0.0f;
#pragma unroll
    for (int i = 0; i < MM; ++i)
        if (i < m) {
            r[i] /= z;  // p_ti
            const float ai = (i == g ? dp : 0.0f) + a.loss_coef * (float)a.counts[i];
            dot += ai * r[i];
        }
#pragma unroll
    for (int i = 0; i < MM; ++i)
        if (i < m) {
            const float ai = (i == g ? dp : 0.0f) + a.loss_coef * (float)a.counts[i];
            r[i] = r[i] * (ai - dot);  // dr_ti
            if (lane == 0) a.dr[t * m + i] = r[i];
        }
    if (!a.dx) return;
    for (int c = lane; c < d; c += 64) {
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < MM; ++i)
            if (i < m) acc = __builtin_fmaf(r[i], a.w[(int64_t)c * m + i], acc);
        a.dx[t * d + c] = acc;
    }
}

// dW partials: block (chunk of tokens, 256 columns); thread c sums x[t][c] dr[t][i] over the
// chunk's tokens in token order for all i < m.
constexpr int kDwChunk = 1024;

template <int MM>
__global__ __launch_bounds__(256) void bwd_router_dw_kernel(BwdRouterLaunch a) {
    const int c = blockIdx.y * 256 + threadIdx.x;
    const int64_t t0 = (int64_t)blockIdx.x * kDwChunk;
    const int64_t t1 = std::min<int64_t>(t0 + kDwChunk, a.n);
    const int d = a.d, m = a.m;
    float acc[MM];
#pragma unroll
    for (int i = 0; i < MM; ++i) acc[i] = 0.0f;
    if (c < d) {
        for (int64_t t = t0; t < t1; ++t) {
            const float xv = a.x_is_bf16 ? (float)static_cast<const bf16 *>(a.x)[t * d + c]
                                         : static_cast<const float *>(a.x)[t * d + c];
#pragma unroll
            for (int i = 0; i < MM; ++i)
                if (i < m) acc[i] = __builtin_fmaf(xv, a.dr[t * m + i], acc[i]);
        }
#pragma unroll
        for (int i = 0; i < MM; ++i)
            if (i < m) a.dw_part[((int64_t)blockIdx.x * d + c) * m + i] = acc[i];
    }
}

__global__ __launch_bounds__(256) void bwd_router_dw_sum_kernel(const float *part, int64_t nchunk,
                                                                 int64_t dm, float *dw) {
    const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (k >= dm) return;
    float s = 0.0f;
    for (int64_t b = 0; b < nchunk; ++b) s += part[b * dm + k];
    dw[k] = s;
}

template <int MM>
hipError_t launch_router_bwd_mm(const BwdRouterLaunch &a, hipStream_t s) {
    hipLaunchKernelGGL((bwd_router_rows_kernel<MM>), dim3((unsigned)((a.n + 3) / 4)), dim3(256), 0,
                       s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !a.dw) return e;
    const int64_t nchunk = bwd_dw_chunks(a.n);
    hipLaunchKernelGGL((bwd_router_dw_kernel<MM>), dim3((unsigned)nchunk, (unsigned)((a.d + 255) / 256)),
                       dim3(256), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t dm = (int64_t)a.d * a.m;
    hipLaunchKernelGGL(bwd_router_dw_sum_kernel, dim3((unsigned)((dm + 255) / 256)), dim3(256), 0, s,
                       a.dw_part, nchunk, dm, a.dw);
    return hipGetLastError();
}

}  // namespace

int64_t bwd_dw_chunks(int64_t n) { return (n + kDwChunk - 1) / kDwChunk; }

hipError_t launch_bwd_rowdot(const bf16 *d_out, const bf16 *out, int64_t rows, float *D,
                             hipStream_t s) {
    hipLaunchKernelGGL(bwd_rowdot_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, s, d_out,
                       out, rows, D);
    return hipGetLastError();
}

hipError_t launch_bwd_dp(const float *D, const float *p_sel, int64_t n, int n_heads, float *dp,
                         hipStream_t s) {
    hipLaunchKernelGGL(bwd_dp_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, D, p_sel,
                       n, n_heads, dp);
    return hipGetLastError();
}

hipError_t launch_bwd_gather_f32(const float *src, const int32_t *perm, int64_t n, int n_heads,
                                 float mult, int inverse, float *dst, hipStream_t s) {
    hipLaunchKernelGGL(bwd_gather_f32_kernel, dim3((unsigned)((n + 255) / 256), (unsigned)n_heads),
                       dim3(256), 0, s, src, perm, n, mult, inverse, dst);
    return hipGetLastError();
}

hipError_t launch_router_bwd(const BwdRouterLaunch &a, hipStream_t s) {
    if (a.m <= 4) return launch_router_bwd_mm<4>(a, s);
    if (a.m <= 8) return launch_router_bwd_mm<8>(a, s);
    if (a.m <= 16) return launch_router_bwd_mm<16>(a, s);
    if (a.m <= 32) return launch_router_bwd_mm<32>(a, s);
    return launch_router_bwd_mm<64>(a, s);
}

}  // namespace moga

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

// D[h][t] for rows of HD channels: HD/8 lanes per row, 16 bytes each, then a sum over them.
template <int HD>
__global__ __launch_bounds__(256) void bwd_rowdot_kernel(const bf16 *d_out, const bf16 *out,
                                                          int64_t rows, float *D) {
    constexpr int LPR = HD / 8, RPB = 256 / LPR;
    const int64_t row = (int64_t)blockIdx.x * RPB + (threadIdx.x / LPR);
    const int ch = threadIdx.x % LPR;
    float acc = 0.0f;
    if (row < rows) {
        const uint4 g = *reinterpret_cast<const uint4 *>(d_out + row * HD + ch * 8);
        const uint4 o = *reinterpret_cast<const uint4 *>(out + row * HD + ch * 8);
        const uint32_t gw[4] = {g.x, g.y, g.z, g.w}, ow[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc = __builtin_fmaf(bf16_lo(gw[i]), bf16_lo(ow[i]), acc);
            acc = __builtin_fmaf(bf16_hi(gw[i]), bf16_hi(ow[i]), acc);
        }
    }
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1) acc += __shfl_xor(acc, off, 64);
    if (row < rows && ch == 0) D[row] = acc;
}

// head_dim-64 rows widened to the 128 channels of the backward kernels, the upper half zero:
// dst[h][j] = (f * src[h][r], 0) with r = perm[j] (perm NULL: j) and f = row_scale[r] (NULL: 1);
// a row index outside [0, src_rows) gives a zero row.  One thread per 16 bytes of dst.
__global__ __launch_bounds__(256) void pad_rows_kernel(const bf16 *src, int64_t src_rows,
                                                        const int32_t *perm, const float *row_scale,
                                                        int64_t n, bf16 *dst) {
    const int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t j = gi >> 4;
    if (j >= n) return;
    const int ch = (int)(gi & 15);
    const int h = blockIdx.y;
    const int64_t r = perm ? (int64_t)perm[j] : j;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (ch < 8 && r >= 0 && r < src_rows) {
        v = *reinterpret_cast<const uint4 *>(src + ((int64_t)h * src_rows + r) * 64 + ch * 8);
        if (row_scale) {
            const float f = row_scale[r];
            uint32_t w[4] = {v.x, v.y, v.z, v.w};
            typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bf16x2 b = {(__bf16)(f * bf16_lo(w[i])), (__bf16)(f * bf16_hi(w[i]))};
                w[i] = __builtin_bit_cast(uint32_t, b);
            }
            v = make_uint4(w[0], w[1], w[2], w[3]);
        }
    }
    *reinterpret_cast<uint4 *>(dst + ((int64_t)h * n + j) * 128 + ch * 8) = v;
}

// The first 64 channels of 128-channel rows: dst[h][perm[j]] = src[h][j][0:64] (perm NULL: j;
// entries outside [0, dst_rows) are skipped).  One thread per 16 bytes of dst.
__global__ __launch_bounds__(256) void unpad_rows_kernel(const bf16 *src, const int32_t *perm,
                                                          int64_t n, int64_t dst_rows, bf16 *dst) {
    const int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t j = gi >> 3;
    if (j >= n) return;
    const int ch = (int)(gi & 7);
    const int h = blockIdx.y;
    const int64_t r = perm ? (int64_t)perm[j] : j;
    if (r < 0 || r >= dst_rows) return;
    *reinterpret_cast<uint4 *>(dst + ((int64_t)h * dst_rows + r) * 64 + ch * 8) =
        *reinterpret_cast<const uint4 *>(src + ((int64_t)h * n + j) * 128 + ch * 8);
}

// dp_t = scale * (sum over heads (in head order) of D[h][t]) / p_t.
__global__ __launch_bounds__(256) void bwd_dp_kernel(const float *D, const float *p_sel,
                                                      int64_t n, int n_heads, float scale,
                                                      float *dp) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= n) return;
    float s = 0.0f;
    for (int h = 0; h < n_heads; ++h) s += D[(int64_t)h * n + t];
    dp[t] = scale * s / p_sel[t];
}

// fp32 [H][N] rows by perm: dst[h][j] = mult * src[h][perm[j]], or with inverse set
// dst[h][perm[j]] = mult * src[h][j].  perm entries outside [0, n) are skipped; perm NULL is
// the identity.
__global__ __launch_bounds__(256) void bwd_gather_f32_kernel(const float *src, const int32_t *perm,
                                                              int64_t n, float mult, int inverse,
                                                              float *dst) {
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (j >= n) return;
    const int64_t h = blockIdx.y;
    const int32_t pj = perm ? perm[j] : (int32_t)j;
    if (inverse) {
        if (pj >= 0 && pj < n) dst[h * n + pj] = mult * src[h * n + j];
    } else {
        dst[h * n + j] = (pj >= 0 && pj < n) ? mult * src[h * n + pj] : 0.0f;
    }
}

// Gradient of a token under the mean of the three branches (hybrid backward): the two
// token-order gradients a and b and the position-order rows c of the token (its query position
// for dQ; for dK and dV every key position that holds it, i.e. its own group's and those of
// the groups that borrow its frame), summed in fp32 in that order and scaled by w.  a and out
// have rows of HD channels, b and c rows of bc_hd >= HD channels (the 128-channel rows of the
// backward kernels), of which the first HD are summed.  One thread per 8 channels; every row of
// out has exactly this one writer.
template <int HD>
__global__ __launch_bounds__(256) void grad_sum_kernel(const bf16 *a, const bf16 *b, const bf16 *c,
                                                        int bc_hd, int64_t c_rows,
                                                        const int32_t *pos, int first, int npos,
                                                        int64_t n, float w, bf16 *out) {
    constexpr int CPR = HD / 8;  // 16-byte chunks per row of a and out
    const int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x;  // chunk of row h*n + t
    const int64_t row = gi / CPR;
    const int h = blockIdx.y;
    if (row >= n) return;
    const int ch = (int)(gi % CPR);
    const int64_t off = ((int64_t)h * n + row) * HD + ch * 8;
    const uint4 ua = *reinterpret_cast<const uint4 *>(a + off);
    const uint4 ub = *reinterpret_cast<const uint4 *>(b + ((int64_t)h * n + row) * bc_hd + ch * 8);
    const uint32_t aw[4] = {ua.x, ua.y, ua.z, ua.w}, bw[4] = {ub.x, ub.y, ub.z, ub.w};
    float acc[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        acc[2 * i] = bf16_lo(aw[i]) + bf16_lo(bw[i]);
        acc[2 * i + 1] = bf16_hi(aw[i]) + bf16_hi(bw[i]);
    }
    for (int k = 0; k < npos; ++k) {
        const int32_t p = pos[4 * row + first + k];
        if (p < 0 || p >= c_rows) continue;
        const uint4 uc = *reinterpret_cast<const uint4 *>(c + ((int64_t)h * c_rows + p) * bc_hd + ch * 8);
        const uint32_t cw[4] = {uc.x, uc.y, uc.z, uc.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[2 * i] += bf16_lo(cw[i]);
            acc[2 * i + 1] += bf16_hi(cw[i]);
        }
    }
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    uint32_t r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bf16x2 v = {(__bf16)(w * acc[2 * i]), (__bf16)(w * acc[2 * i + 1])};
        r[i] = __builtin_bit_cast(uint32_t, v);
    }
    *reinterpret_cast<uint4 *>(out + off) = make_uint4(r[0], r[1], r[2], r[3]);
}

// Router backward for the tokens of one wave: logits x_t W (fp32), softmax, dr_t, dx_t.  A wave
// takes TPW tokens at once so that each weight it loads serves all of them; lane l handles the
// CPL consecutive columns CPL*l, CPL*l + 64*CPL, ... (16-byte loads of x, 16-byte stores of dx);
// the column sums are reduced over the wave with butterfly shuffles in a fixed order.
template <int MM, bool XB, bool WL>
__global__ __launch_bounds__(256) void bwd_router_rows_kernel(BwdRouterLaunch a) {
    // WL: the block first copies W ([d][m] fp32) into LDS and reads it from there
    extern __shared__ __attribute__((aligned(16))) float wsh[];
    constexpr int TPW = MM <= 16 ? 4 : 1;
    constexpr int CPL = XB ? 8 : 4, STRIDE = 64 * CPL;
    const int lane = threadIdx.x & 63;
    const int d = a.d, m = a.m;
    const float *w = a.w;
    if constexpr (WL) {
        const int nw = d * m;  // w carries no alignment promise: element-wise copy
        for (int k = threadIdx.x; k < nw; k += 256) wsh[k] = a.w[k];
        __syncthreads();
        w = wsh;
    }
    const int64_t t0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * TPW;
    if (t0 >= a.n) return;
    const int nt = (int)min((int64_t)TPW, a.n - t0);
    float r[TPW][MM];
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
        for (int i = 0; i < MM; ++i) r[tt][i] = 0.0f;
    for (int c0 = CPL * lane; c0 < d; c0 += STRIDE) {  // d is a multiple of CPL
        float xv[TPW][CPL];
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
            const int64_t row = t0 + min(tt, nt - 1);  // rows past the end repeat the last one
            if constexpr (XB) {
                const uint4 u = *reinterpret_cast<const uint4 *>(static_cast<const bf16 *>(a.x) + row * d + c0);
                const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    xv[tt][2 * q] = bf16_lo(w4[q]);
                    xv[tt][2 * q + 1] = bf16_hi(w4[q]);
                }
            } else {
                const float4 f = *reinterpret_cast<const float4 *>(static_cast<const float *>(a.x) + row * d + c0);
                xv[tt][0] = f.x; xv[tt][1] = f.y; xv[tt][2] = f.z; xv[tt][3] = f.w;
            }
        }
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
            const float *wr = w + (c0 + cc) * m;
#pragma unroll
            for (int i = 0; i < MM; ++i)
                if (i < m) {
                    const float wv = wr[i];
#pragma unroll
                    for (int tt = 0; tt < TPW; ++tt) r[tt][i] = __builtin_fmaf(xv[tt][cc], wv, r[tt][i]);
                }
        }
    }
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
        for (int i = 0; i < MM; ++i)
            if (i < m) {
#pragma unroll
                for (int off = 32; off >= 1; off >>= 1) r[tt][i] += __shfl_xor(r[tt][i], off, 64);
            }
    // softmax and its backward, per token (every lane holds every logit)
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
        if (tt >= nt) break;
        const int64_t t = t0 + tt;
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < MM; ++i)
            if (i < m) mx = fmaxf(mx, r[tt][i]);
        float z = 0.0f;
#pragma unroll
        for (int i = 0; i < MM; ++i)
            if (i < m) { r[tt][i] = __expf(r[tt][i] - mx); z += r[tt][i]; }
        const int g = a.group_id[t];
        const float dp = a.dp[t];
        float dot = 0.0f;
#pragma unroll
        for (int i = 0; i < MM; ++i)
            if (i < m) {
                r[tt][i] /= z;  // p_ti
                const float ai = (i == g ? dp : 0.0f) + a.loss_coef * (float)a.counts[i];
                dot += ai * r[tt][i];
            }
#pragma unroll
        for (int i = 0; i < MM; ++i)
            if (i < m) {
                const float ai = (i == g ? dp : 0.0f) + a.loss_coef * (float)a.counts[i];
                r[tt][i] = r[tt][i] * (ai - dot);  // dr_ti
                if (lane == 0) a.dr[t * m + i] = r[tt][i];
            }
    }
    if (!a.dx) return;
    for (int c0 = CPL * lane; c0 < d; c0 += STRIDE) {
        float acc[TPW][CPL];
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) acc[tt][cc] = 0.0f;
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
            const float *wr = w + (c0 + cc) * m;
#pragma unroll
            for (int i = 0; i < MM; ++i)
                if (i < m) {
                    const float wv = wr[i];
#pragma unroll
                    for (int tt = 0; tt < TPW; ++tt) acc[tt][cc] = __builtin_fmaf(r[tt][i], wv, acc[tt][cc]);
                }
        }
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt)
            if (tt < nt) {
                float *dst = a.dx + (t0 + tt) * d + c0;
#pragma unroll
                for (int q = 0; q < CPL / 4; ++q)
                    *reinterpret_cast<float4 *>(dst + 4 * q) =
                        make_float4(acc[tt][4 * q], acc[tt][4 * q + 1], acc[tt][4 * q + 2], acc[tt][4 * q + 3]);
            }
    }
}

// dW partials: block (chunk of tokens, 256 * CPT columns); thread k sums x[t][c] dr[t][i] over
// the chunk's tokens in token order for its CPT consecutive columns c and all i < m.  The dr
// values of a token are the same for every thread of the block.
constexpr int kDwChunk = 256;

template <int MM, bool XB>
__global__ __launch_bounds__(256) void bwd_router_dw_kernel(BwdRouterLaunch a) {
    constexpr int CPT = MM <= 8 ? (XB ? 8 : 4) : (MM <= 16 ? 4 : (MM <= 32 ? 2 : 1));
    const int c0 = (blockIdx.y * 256 + threadIdx.x) * CPT;
    const int64_t t0 = (int64_t)blockIdx.x * kDwChunk;
    const int64_t t1 = std::min<int64_t>(t0 + kDwChunk, a.n);
    const int d = a.d, m = a.m;
    float acc[CPT][MM];
#pragma unroll
    for (int cc = 0; cc < CPT; ++cc)
#pragma unroll
        for (int i = 0; i < MM; ++i) acc[cc][i] = 0.0f;
    if (c0 < d) {  // d is a multiple of CPT (of 8 for bf16 x, of 4 for fp32 x)
        for (int64_t t = t0; t < t1; ++t) {
            float xv[CPT];
            if constexpr (XB) {
                const bf16 *xp = static_cast<const bf16 *>(a.x) + t * d + c0;
                if constexpr (CPT == 8) {
                    const uint4 u = *reinterpret_cast<const uint4 *>(xp);
                    const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                    for (int q = 0; q < 4; ++q) { xv[2 * q] = bf16_lo(w4[q]); xv[2 * q + 1] = bf16_hi(w4[q]); }
                } else {
#pragma unroll
                    for (int cc = 0; cc < CPT; ++cc) xv[cc] = (float)xp[cc];
                }
            } else {
                const float *xp = static_cast<const float *>(a.x) + t * d + c0;
#pragma unroll
                for (int cc = 0; cc < CPT; ++cc) xv[cc] = xp[cc];
            }
            const float *drt = a.dr + t * m;
#pragma unroll
            for (int i = 0; i < MM; ++i)
                if (i < m) {
                    const float dv = drt[i];
#pragma unroll
                    for (int cc = 0; cc < CPT; ++cc) acc[cc][i] = __builtin_fmaf(xv[cc], dv, acc[cc][i]);
                }
        }
#pragma unroll
        for (int cc = 0; cc < CPT; ++cc)
#pragma unroll
            for (int i = 0; i < MM; ++i)
                if (i < m) a.dw_part[((int64_t)blockIdx.x * d + c0 + cc) * m + i] = acc[cc][i];
    }
}

// dW = sum of the chunk partials: eight running sums over chunks b = 8q + u, added in a fixed
// order at the end (the result is reproducible; eight loads are in flight per thread)
__global__ __launch_bounds__(64) void bwd_router_dw_sum_kernel(const float *part, int64_t nchunk,
                                                                int64_t dm, float *dw) {
    const int64_t k = (int64_t)blockIdx.x * 64 + threadIdx.x;
    if (k >= dm) return;
    float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    int64_t b = 0;
    for (; b + 8 <= nchunk; b += 8)
#pragma unroll
        for (int u = 0; u < 8; ++u) acc[u] += part[(b + u) * dm + k];
    for (int u = 0; b + u < nchunk; ++u) acc[u] += part[(b + u) * dm + k];
    dw[k] = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
}

template <int MM, bool XB>
hipError_t launch_router_bwd_mm(const BwdRouterLaunch &a, hipStream_t s) {
    constexpr int TPW = MM <= 16 ? 4 : 1;
    const int64_t waves = (a.n + TPW - 1) / TPW;
    const size_t wbytes = sizeof(float) * (size_t)a.d * a.m;
    if (wbytes <= 48 * 1024)
        hipLaunchKernelGGL((bwd_router_rows_kernel<MM, XB, true>), dim3((unsigned)((waves + 3) / 4)),
                           dim3(256), wbytes, s, a);
    else
        hipLaunchKernelGGL((bwd_router_rows_kernel<MM, XB, false>), dim3((unsigned)((waves + 3) / 4)),
                           dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !a.dw) return e;
    constexpr int CPT = MM <= 8 ? (XB ? 8 : 4) : (MM <= 16 ? 4 : (MM <= 32 ? 2 : 1));
    const int64_t nchunk = bwd_dw_chunks(a.n);
    const int cols_per_block = 256 * CPT;
    hipLaunchKernelGGL((bwd_router_dw_kernel<MM, XB>),
                       dim3((unsigned)nchunk, (unsigned)((a.d + cols_per_block - 1) / cols_per_block)),
                       dim3(256), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t dm = (int64_t)a.d * a.m;
    hipLaunchKernelGGL(bwd_router_dw_sum_kernel, dim3((unsigned)((dm + 63) / 64)), dim3(64), 0, s,
                       a.dw_part, nchunk, dm, a.dw);
    return hipGetLastError();
}

template <int MM>
hipError_t launch_router_bwd_x(const BwdRouterLaunch &a, hipStream_t s) {
    return a.x_is_bf16 ? launch_router_bwd_mm<MM, true>(a, s) : launch_router_bwd_mm<MM, false>(a, s);
}

}  // namespace

int64_t bwd_dw_chunks(int64_t n) { return (n + kDwChunk - 1) / kDwChunk; }

hipError_t launch_bwd_rowdot(const bf16 *d_out, const bf16 *out, int64_t rows, int hd, float *D,
                             hipStream_t s) {
    if (hd == 64)
        hipLaunchKernelGGL(bwd_rowdot_kernel<64>, dim3((unsigned)((rows + 31) / 32)), dim3(256), 0,
                           s, d_out, out, rows, D);
    else
        hipLaunchKernelGGL(bwd_rowdot_kernel<128>, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0,
                           s, d_out, out, rows, D);
    return hipGetLastError();
}

hipError_t launch_pad_rows(const bf16 *src, int64_t src_rows, const int32_t *perm,
                           const float *row_scale, int64_t n, int n_heads, bf16 *dst,
                           hipStream_t s) {
    hipLaunchKernelGGL(pad_rows_kernel, dim3((unsigned)((n * 16 + 255) / 256), (unsigned)n_heads),
                       dim3(256), 0, s, src, src_rows, perm, row_scale, n, dst);
    return hipGetLastError();
}

hipError_t launch_unpad_rows(const bf16 *src, const int32_t *perm, int64_t n, int64_t dst_rows,
                             int n_heads, bf16 *dst, hipStream_t s) {
    hipLaunchKernelGGL(unpad_rows_kernel, dim3((unsigned)((n * 8 + 255) / 256), (unsigned)n_heads),
                       dim3(256), 0, s, src, perm, n, dst_rows, dst);
    return hipGetLastError();
}

hipError_t launch_bwd_dp(const float *D, const float *p_sel, int64_t n, int n_heads, float scale,
                         float *dp, hipStream_t s) {
    hipLaunchKernelGGL(bwd_dp_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, D, p_sel,
                       n, n_heads, scale, dp);
    return hipGetLastError();
}

hipError_t launch_bwd_gather_f32(const float *src, const int32_t *perm, int64_t n, int n_heads,
                                 float mult, int inverse, float *dst, hipStream_t s) {
    hipLaunchKernelGGL(bwd_gather_f32_kernel, dim3((unsigned)((n + 255) / 256), (unsigned)n_heads),
                       dim3(256), 0, s, src, perm, n, mult, inverse, dst);
    return hipGetLastError();
}

hipError_t launch_grad_sum(const bf16 *a, const bf16 *b, const bf16 *c, int hd, int bc_hd,
                           int64_t c_rows, const int32_t *pos, int first, int npos, int64_t n,
                           int n_heads, float w, bf16 *out, hipStream_t s) {
    const int64_t chunks = n * (hd / 8);
    const dim3 grid((unsigned)((chunks + 255) / 256), (unsigned)n_heads);
    if (hd == 64)
        hipLaunchKernelGGL(grad_sum_kernel<64>, grid, dim3(256), 0, s, a, b, c, bc_hd, c_rows, pos,
                           first, npos, n, w, out);
    else
        hipLaunchKernelGGL(grad_sum_kernel<128>, grid, dim3(256), 0, s, a, b, c, bc_hd, c_rows, pos,
                           first, npos, n, w, out);
    return hipGetLastError();
}

hipError_t launch_router_bwd(const BwdRouterLaunch &a, hipStream_t s) {
    if (a.m <= 4) return launch_router_bwd_x<4>(a, s);
    if (a.m <= 8) return launch_router_bwd_x<8>(a, s);
    if (a.m <= 16) return launch_router_bwd_x<16>(a, s);
    if (a.m <= 32) return launch_router_bwd_x<32>(a, s);
    return launch_router_bwd_x<64>(a, s);
}

}  // namespace moga

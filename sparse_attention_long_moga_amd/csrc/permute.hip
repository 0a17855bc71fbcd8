// Group histogram, scan and stable permutation (papernotes.org MoGA note, 关键设计 2:
// tokens of one group are made contiguous before a varlen attention call described by
// per-group offsets, and put back in token order afterwards).
//
// A counting sort with no atomics deciding positions:
//   hist    - block b counts the group ids of its kPermTokensPerBlock tokens with wave
//             ballots (lane i accumulates group i) -> table[b][i];
//   scatter - each block takes its own exclusive prefix of table[.][i] over the blocks before
//             it and the group totals; cu = prefix of group totals; every token's position is
//             cu[g] + (tokens of g in earlier blocks) + (earlier in this block), the
//             in-block part from ballots and popcounts, so equal ids keep token order.
// The row gathers then move whole head_dim rows (128 or 256 bytes) with 16-byte lanes.
#include "moga_internal.h"

namespace moga {
namespace {

__device__ __forceinline__ uint64_t lanemask_lt(int lane) {
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

__global__ __launch_bounds__(256) void hist_kernel(const int32_t *gid, int64_t n, int m,
                                                    int32_t *table) {
    __shared__ int wc[4][kMaxGroups];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t b0 = (int64_t)blockIdx.x * kPermTokensPerBlock;
    // every id of the block is loaded first: one memory round trip, not one per pass
    constexpr int R = kPermTokensPerBlock / 256;
    int gv[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t t = b0 + r * 256 + threadIdx.x;
        gv[r] = t < n ? gid[t] : -1;
    }
    int cnt = 0;  // lane i counts group i
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int g = gv[r];
        for (int i = 0; i < m; ++i) {
            const uint64_t bal = __ballot(g == i);
            if (lane == i) cnt += __popcll(bal);
        }
    }
    wc[wave][lane] = cnt;
    __syncthreads();
    if ((int)threadIdx.x < m)
        table[(int64_t)blockIdx.x * m + threadIdx.x] =
            wc[0][threadIdx.x] + wc[1][threadIdx.x] + wc[2][threadIdx.x] + wc[3][threadIdx.x];
}

// Block i (large inputs only): base_rel[b][i] = sum_{b' < b} table[b'][i]; totals[i] = the sum
// over all blocks.  One block per group, a Hillis-Steele scan over 256 entries at a time.
__global__ __launch_bounds__(256) void scan_kernel(const int32_t *table, int64_t nblk, int m,
                                                    int32_t *base_rel, int32_t *totals) {
    __shared__ int s[256];
    const int g = blockIdx.x;
    int carry = 0;
    for (int64_t c0 = 0; c0 < nblk; c0 += 256) {
        const int64_t b = c0 + threadIdx.x;
        const int v = b < nblk ? table[b * m + g] : 0;
        s[threadIdx.x] = v;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            const int add = (int)threadIdx.x >= off ? s[threadIdx.x - off] : 0;
            __syncthreads();
            s[threadIdx.x] += add;
            __syncthreads();
        }
        if (b < nblk) base_rel[b * m + g] = carry + s[threadIdx.x] - v;
        carry += s[255];
        __syncthreads();
    }
    if (threadIdx.x == 0) totals[g] = carry;
}

// Block b: its tokens' positions.  The exclusive prefix of table[.][i] over blocks b' < b and
// the group totals come from scan_kernel (base_rel, totals) or, when base_rel is NULL, are taken
// here from the whole table (nblk x m integers, read from L2 by every block, so only for inputs
// where nblk^2 x m stays small; integer sums, so the order of the LDS atomics does not matter),
// then
// cu = prefix of group totals and every token's position is cu[g] + (tokens of g in earlier
// blocks) + (earlier in this block), the in-block part from ballots and popcounts.
__global__ __launch_bounds__(256) void scatter_kernel(const int32_t *gid, int64_t n, int m,
                                                       const int32_t *table, int nblk,
                                                       const int32_t *base_rel,
                                                       const int32_t *totals, int32_t *cu,
                                                       int32_t *perm) {
    __shared__ int before[kMaxGroups], total[kMaxGroups];
    __shared__ int base[kMaxGroups];
    __shared__ int wc[4][kMaxGroups];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // the block's ids are requested before the table is read, so both loads overlap
    constexpr int R = kPermTokensPerBlock / 256;
    int gv[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t t = (int64_t)blockIdx.x * kPermTokensPerBlock + r * 256 + threadIdx.x;
        gv[r] = t < n ? gid[t] : -1;
    }
    if (base_rel) {
        if ((int)threadIdx.x < m) {
            before[threadIdx.x] = base_rel[(int64_t)blockIdx.x * m + threadIdx.x];
            total[threadIdx.x] = totals[threadIdx.x];
        }
    } else {
        if ((int)threadIdx.x < m) before[threadIdx.x] = total[threadIdx.x] = 0;
        __syncthreads();
        const int ne = nblk * m, mine = (int)blockIdx.x * m;
        for (int e = threadIdx.x; e < ne; e += 256) {
            const int v = table[e], g = e % m;
            atomicAdd(&total[g], v);
            if (e < mine) atomicAdd(&before[g], v);
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int acc = 0;
        for (int i = 0; i < m; ++i) {
            base[i] = acc + before[i];
            if (blockIdx.x == 0) cu[i] = acc;
            acc += total[i];
        }
        if (blockIdx.x == 0) cu[m] = acc;
    }
    __syncthreads();
    const int64_t b0 = (int64_t)blockIdx.x * kPermTokensPerBlock;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t t = b0 + r * 256 + threadIdx.x;
        const int g = gv[r];
        int rank = 0;
        for (int i = 0; i < m; ++i) {
            const uint64_t bal = __ballot(g == i);
            if (g == i) rank = __popcll(bal & lanemask_lt(lane));
            if (lane == i) wc[wave][i] = __popcll(bal);
        }
        __syncthreads();
        if (g >= 0 && g < m) {
            int pos = base[g] + rank;
            for (int w = 0; w < wave; ++w) pos += wc[w][g];
            perm[pos] = (int32_t)t;
        }
        __syncthreads();
        if ((int)threadIdx.x < m)
            base[threadIdx.x] += wc[0][threadIdx.x] + wc[1][threadIdx.x] + wc[2][threadIdx.x] +
                                 wc[3][threadIdx.x];
        __syncthreads();
    }
}

// Row gather/scatter.  grid = (row blocks, heads, tensors); each thread moves 16 bytes.  Every
// byte is read once and written once, so the accesses are non-temporal (streamed past the
// caches rather than kept in them: about 10% faster than ordinary loads and stores here).
// SCALED: dst row j = bf16(src_scale[perm[j]] * src row perm[j]) (forward direction only).  In
// the forward direction src may hold another number of rows per head than dst (src_rows).
template <int HD, bool SCALED>
__global__ __launch_bounds__(256) void gather_kernel(GatherLaunch a) {
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    constexpr int CH = HD * 2 / 16;         // 16-byte chunks per row
    constexpr int ROWS = 256 / CH;          // rows per block pass
    constexpr int PASSES = 8;
    const int tensor = blockIdx.z, h = blockIdx.y;
    const int64_t n = a.n;
    const int64_t srows = (!a.inverse && a.src_rows > 0) ? a.src_rows : n;  // rows perm may name
    const int64_t head_off = (int64_t)h * n * HD;
    // select by comparisons: indexing the by-value pointer arrays with a runtime value
    // would place the whole argument struct in per-lane scratch memory
    const void *sv = a.src[0];
    void *dv = a.dst[0];
    if (tensor == 1) { sv = a.src[1]; dv = a.dst[1]; }
    if (tensor == 2) { sv = a.src[2]; dv = a.dst[2]; }
    if (tensor == 3) { sv = a.src[3]; dv = a.dst[3]; }
    const bf16 *src = static_cast<const bf16 *>(sv) + (a.inverse ? head_off : (int64_t)h * srows * HD);
    bf16 *dst = static_cast<bf16 *>(dv) + head_off;
    const int r_in = threadIdx.x / CH, ch = threadIdx.x % CH;
    const int64_t j0 = (int64_t)blockIdx.x * ROWS * PASSES + r_in;
    // every load is unconditional (clamped indices), so all of them are in flight together;
    // perm entries are range-checked, since with ids outside [0, m) part of perm is never
    // written and stale workspace values must not become addresses
    int32_t pj[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) pj[p] = a.perm[min(j0 + p * ROWS, n - 1)];
    i32x4 buf[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int64_t j = j0 + p * ROWS;
        const bool ok = j < n && pj[p] >= 0 && pj[p] < srows;
        const int64_t s_row = ok ? (a.inverse ? j : (int64_t)pj[p]) : 0;
        buf[p] = __builtin_nontemporal_load(reinterpret_cast<const i32x4 *>(src + s_row * HD + ch * 8));
    }
    if constexpr (SCALED) {
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const int64_t j = j0 + p * ROWS;
            const bool ok = j < n && pj[p] >= 0 && pj[p] < srows;
            const float f = a.src_scale[ok ? pj[p] : 0];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t w = (uint32_t)buf[p][q];
                const float lo = __uint_as_float(w << 16) * f, hi = __uint_as_float(w & 0xffff0000u) * f;
                typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
                const bf16x2 r = {(__bf16)lo, (__bf16)hi};
                buf[p][q] = (int)__builtin_bit_cast(uint32_t, r);
            }
        }
    }
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int64_t j = j0 + p * ROWS;
        if (j < n && pj[p] >= 0 && pj[p] < srows) {
            const int64_t d_row = a.inverse ? (int64_t)pj[p] : j;
            __builtin_nontemporal_store(buf[p], reinterpret_cast<i32x4 *>(dst + d_row * HD + ch * 8));
        }
    }
}

__global__ __launch_bounds__(256) void gather_scalar_kernel(const float *src, const int32_t *perm,
                                                             int64_t n, float *dst) {
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (j < n) {
        const int32_t pj = perm[j];
        dst[j] = (pj >= 0 && pj < n) ? src[pj] : 0.0f;
    }
}

}  // namespace

int64_t permute_blocks(int64_t n) {
    return (n + kPermTokensPerBlock - 1) / kPermTokensPerBlock;
}

hipError_t launch_perm_index(const PermuteLaunch &a, hipStream_t s) {
    const int64_t nblk = permute_blocks(a.n);
    hipLaunchKernelGGL(hist_kernel, dim3((unsigned)nblk), dim3(256), 0, s, a.group_id, a.n, a.m,
                       a.table);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // the scan inside the scatter costs nblk^2 x m table reads: up to 2^24 (1.5 M at 563,160
    // tokens and 20 groups) it saves a launch; above, the linear scan runs as its own launch
    const bool fused = nblk * nblk * a.m <= kFusedScanReads;
    if (!fused) {
        hipLaunchKernelGGL(scan_kernel, dim3(a.m), dim3(256), 0, s, a.table, nblk, a.m, a.base_rel,
                           a.totals);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)nblk), dim3(256), 0, s, a.group_id, a.n, a.m,
                       a.table, (int)nblk, fused ? nullptr : a.base_rel,
                       fused ? nullptr : a.totals, a.cu, a.perm);
    return hipGetLastError();
}

hipError_t launch_gather(const GatherLaunch &a, hipStream_t s) {
    if (a.n_tensors > 0) {
        const int ch = a.head_dim * 2 / 16;
        const int64_t rows_per_block = (256 / ch) * 8;
        dim3 grid((unsigned)((a.n + rows_per_block - 1) / rows_per_block), a.n_heads, a.n_tensors);
        const bool scaled = a.src_scale && !a.inverse;
        if (a.head_dim == 128) {
            if (scaled) hipLaunchKernelGGL((gather_kernel<128, true>), grid, dim3(256), 0, s, a);
            else hipLaunchKernelGGL((gather_kernel<128, false>), grid, dim3(256), 0, s, a);
        } else {
            if (scaled) hipLaunchKernelGGL((gather_kernel<64, true>), grid, dim3(256), 0, s, a);
            else hipLaunchKernelGGL((gather_kernel<64, false>), grid, dim3(256), 0, s, a);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (!a.inverse && a.p_sel && a.p_perm) {
        hipLaunchKernelGGL(gather_scalar_kernel, dim3((unsigned)((a.n + 255) / 256)), dim3(256), 0,
                           s, a.p_sel, a.perm, a.n, a.p_perm);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace moga

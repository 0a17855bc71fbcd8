// Device helpers shared by the forward and backward attention kernels of libmoga.so
// (internal; not part of the public ABI).
//
// Direct-to-LDS tiles (head_dim 128): a buffer load that writes LDS places lane l's 16 bytes
// at base + 16*l, so the row layout is chosen on the global side: LDS chunk c of row r holds
// global chunk c ^ sw(r).  Two layouts:
//   "A" layout, sw(r) = r & 15: an MFMA A operand (32 rows x 16 columns) is read with one
//      ds_read_b128 per lane (row j, 16-byte chunk 2s + hh); 16 consecutive rows hit 16
//      different chunk positions, so the read is bank-conflict free.
//   "T" layout, natural [row][d] order, sw(r) = 4 * (r & 3): the transposed A operand
//      (32 columns of d x 16 rows) is read with two ds_read_b64_tr_b16; within a group of 16
//      lanes, output lane 4a+b receives element b of the 8-byte pieces addressed by lanes a,
//      a+4, a+8, a+12.  Lane s of group g points at row kc + 4*(g/2) + s/4 (+8 for the second
//      read), columns 32*ti + 16*(g%2) + 4*(s%4); lane d of the MFMA layout then holds
//      X[4 rows][d] in the same row order as a 32x32 accumulator's rows (runs of 4), which is
//      the order a B operand built from such an accumulator uses.  The four rows a half-wave
//      reads fall on four different 64-byte column ranges, so these reads are conflict free.
#pragma once

#include "moga_internal.h"

namespace moga {
namespace {

constexpr int KT = 64;       // rows per LDS tile
constexpr int ROWB128 = 256; // bytes per bf16 row at head_dim 128

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int64_t clamp64(int64_t v, int64_t lo, int64_t hi) {
    return v < lo ? lo : (v > hi ? hi : v);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 r = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, r);
}

// Buffer descriptor over [base, base + bytes): loads past the end return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// LDS-side helpers (kept out of lambdas: the host compilation pass must not see the
// address-space-3 builtins)
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, unsigned char *lds_base,
                                           int voffset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void *)lds_base, 16, voffset, 0, 0, 0);
}
__device__ __forceinline__ uint2 lds_read_tr16(const unsigned char *p) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)(p));
    return __builtin_bit_cast(uint2, v);
}

// LDS reads through pointers that are in the LDS address space from the start (a cast of the
// __shared__ array's own address, which the compiler resolves to the array): offsets added to
// them keep their value ranges visible, and no generic-to-LDS conversion is left to emit.
typedef __attribute__((address_space(3))) const unsigned char lds_cu8;
__device__ __forceinline__ lds_cu8 *lds_ptr(const unsigned char *shared_array) {
    return (lds_cu8 *)shared_array;
}
__device__ __forceinline__ bf16x8 lds_read_b128(lds_cu8 *p) {
    return *(__attribute__((address_space(3))) const bf16x8 *)p;
}
__device__ __forceinline__ uint2 lds_read_tr16(lds_cu8 *p) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)(p));
    return __builtin_bit_cast(uint2, v);
}

// Workgroup barrier for handing data between waves through LDS with ordinary LDS stores,
// while direct-to-LDS loads of another buffer stay in flight.  Any fence would wait for those
// loads too (they write LDS and share the vector-memory counter), so there is none: the wave's
// own LDS stores are waited for explicitly (lgkmcnt(0)), LDS is coherent within the workgroup,
// and the empty asm statements keep the compiler from moving memory accesses across.  Only
// for data written with ds_write by the waves of this workgroup.
__device__ __forceinline__ void lds_handoff_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt left at their maximum
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// max(v, value of the lane 32 apart): v_permlane32_swap exchanges the upper half of one
// operand with the lower half of the other, so with both operands v each lane sees both
__device__ __forceinline__ float max_across_halves(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// acc + lo + hi of a packed pair of bf16 values (v_dot2 against (1, 1))
__device__ __forceinline__ float sum_bf16x2(uint32_t packed, float acc) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed), one, acc, false);
}

// LDS byte offset, within a tile in the A layout, of the 16 bytes lane (row j, half hh) reads
// for MFMA k-step s (columns 16s .. 16s+15 of head_dim 128)
__device__ __forceinline__ int a_frag_off(int j, int hh, int s) {
    return j * ROWB128 + (((2 * s + hh) ^ (j & 15)) << 4);
}
// LDS byte offset, within a tile in the T layout, of lane's first transposed 8-byte read for
// d block ti (the second read is 8 rows further); add 16 * ROWB128 per 16-row chunk
__device__ __forceinline__ int t_read_off(int lane, int ti) {
    const int s16 = lane & 15, g = lane >> 4;
    return (4 * (g >> 1) + (s16 >> 2)) * ROWB128 +
           ((((ti ^ (s16 >> 2)) << 2) + 2 * (g & 1) + ((s16 & 3) >> 1)) << 4) + (s16 & 1) * 8;
}
// byte offset within a global row of the 16-byte chunk that lands in LDS chunk s16 of row r
__device__ __forceinline__ int a_dma_chunk(int r, int s16) { return (s16 ^ (r & 15)) << 4; }
__device__ __forceinline__ int t_dma_chunk(int r, int s16) { return (s16 ^ (4 * (r & 3))) << 4; }

// Physical output row of logical query row qrow whose query is physical row qphys: the query
// row itself unless an output map is given (clamped to the head so a bad map cannot address
// outside it).
__device__ __forceinline__ int64_t out_row(const AttnLaunch &a, int64_t qrow, int64_t qphys) {
    return a.o_idx ? min(max((int64_t)a.o_idx[qrow], (int64_t)0), a.o_rows - 1) : qphys;
}

// Stores four consecutive output channels of one row from their fp32 values: rounded to bf16
// once, after the mean with the two other branches' rows when the launch asks for it
// (out = (v + a + b) / 3 in fp32), and the row itself to o_raw when given (the state the
// backward of the mean needs).  off: element offset of the first of the four in o.
__device__ __forceinline__ void store4(const AttnLaunch &a, int64_t off, float v0, float v1,
                                       float v2, float v3) {
    if (a.o_raw)
        *reinterpret_cast<uint2 *>(a.o_raw + off) =
            make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
    if (a.mean_a) {
        const uint2 ua = *reinterpret_cast<const uint2 *>(a.mean_a + off);
        const uint2 ub = *reinterpret_cast<const uint2 *>(a.mean_b + off);
        constexpr float third = 1.0f / 3.0f;
        v0 = (v0 + __uint_as_float(ua.x << 16) + __uint_as_float(ub.x << 16)) * third;
        v1 = (v1 + __uint_as_float(ua.x & 0xffff0000u) + __uint_as_float(ub.x & 0xffff0000u)) * third;
        v2 = (v2 + __uint_as_float(ua.y << 16) + __uint_as_float(ub.y << 16)) * third;
        v3 = (v3 + __uint_as_float(ua.y & 0xffff0000u) + __uint_as_float(ub.y & 0xffff0000u)) * third;
    }
    *reinterpret_cast<uint2 *>(a.o + off) = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
}

}  // namespace
}  // namespace moga

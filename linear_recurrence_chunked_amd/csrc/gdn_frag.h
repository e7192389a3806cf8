// Matrix-core fragments, conversions and masks shared by the Gated DeltaNet
// kernels on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16).
//
// Lane layout of a 16x16x32 product: the A operand of lane l is row l%16 with
// 8 k-values, the B operand column l%16 with the same 8 k-values, and the
// accumulator holds column l%16, rows 4(l/16) .. +3.  A wave's own [rows x 16]
// accumulators serve directly as B operands when the k-values of lane group g
// are taken as rows {4g .. 4g+3} of one 16-row tile and {16+4g .. 16+4g+3} of
// the next (acc_frag); the A operand then needs the same two 4-element runs
// of its row, which the k-permuted row layout below keeps in one 16-byte run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lrc_device.h"

namespace lrc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// Row stride (bf16) of 64-column operands where LDS is short (the chunk-parallel
// prep kernel); 16-byte reads by 16 such rows meet some bank conflicts, which
// a stride of 80 avoids where the room allows.
constexpr int L64 = 64 + 8;
constexpr int CG = 2;        // 16-column groups of a state wave: its even and its odd columns
__device__ __forceinline__ floatx4 mfma(bf16x8 a, bf16x8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 frag(const __bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
// A k-permuted layout of a row: within each block of 32 k-values, positions
// 8g .. 8g+3 hold k = 4g .. 4g+3 and positions 8g+4 .. 8g+7 hold
// k = 16+4g .. 16+4g+3 (g = 0 .. 3).  Rows stored this way give the A operand
// of lane group g as one contiguous 16-byte read at position 8g (a single
// ds_read_b128 instead of two 8-byte reads 32 bytes apart).  A run of
// 4 k-values starting at a multiple of 4 stays contiguous.  Products whose two
// operands are both stored this way (K K^T, Q K^T) are unchanged by it.
__device__ __forceinline__ int kperm(int k) {
    const int x = k & 31;
    return (k & ~31) + ((x & 15) >> 2) * 8 + (x >> 4) * 4 + (x & 3);
}
__device__ __forceinline__ int kperm_inv(int pos) {
    const int x = pos & 31;
    return (pos & ~31) + ((x >> 2) & 1) * 16 + (x >> 3) * 4 + (x & 3);
}
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// Two FP32 values as packed bf16 hi = bf16(x) and lo = bf16(x - hi) (round to
// nearest even both times): one conversion for each pair, the hi parts
// unpacked with a shift and a mask.
__device__ __forceinline__ void split_pair(float a, float b, uint32_t& hi, uint32_t& lo) {
    hi = __builtin_bit_cast(uint32_t, bf16x2{static_cast<__bf16>(a), static_cast<__bf16>(b)});
    const float ra = a - __uint_as_float(hi << 16);
    const float rb = b - __uint_as_float(hi & 0xffff0000u);
    lo = __builtin_bit_cast(uint32_t, bf16x2{static_cast<__bf16>(ra), static_cast<__bf16>(rb)});
}
__device__ __forceinline__ uint32_t pack_pair(float a, float b) {
    return __builtin_bit_cast(uint32_t, bf16x2{static_cast<__bf16>(a), static_cast<__bf16>(b)});
}
// B fragment from two accumulator tiles (rows 16t.. and 16t+16..): the bf16
// values, and with SPLIT also the lo parts.
template <bool SPLIT>
__device__ __forceinline__ void acc_frag(const floatx4& t0, const floatx4& t1, bf16x8& hi, bf16x8& lo) {
    uint4 h, l;
    if constexpr (SPLIT) {
        split_pair(t0[0], t0[1], h.x, l.x);
        split_pair(t0[2], t0[3], h.y, l.y);
        split_pair(t1[0], t1[1], h.z, l.z);
        split_pair(t1[2], t1[3], h.w, l.w);
        lo = __builtin_bit_cast(bf16x8, l);
    } else {
        h = uint4{pack_pair(t0[0], t0[1]), pack_pair(t0[2], t0[3]), pack_pair(t1[0], t1[1]), pack_pair(t1[2], t1[3])};
    }
    hi = __builtin_bit_cast(bf16x8, h);
}
__device__ __forceinline__ void split4(const floatx4& x, bf16x4& hi, bf16x4& lo) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        hi[r] = static_cast<__bf16>(x[r]);
        lo[r] = static_cast<__bf16>(x[r] - static_cast<float>(hi[r]));
    }
}

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Scheduling hint for an unrolled run of N steps that each read R fragments
// from LDS and issue M products: the reads run AHEAD steps ahead of the
// products, so that the waits before the products are partial.
template <int N, int R, int M, int AHEAD>
__device__ __forceinline__ void read_ahead() {
    __builtin_amdgcn_sched_group_barrier(0x100, R * AHEAD, 0);
#pragma unroll
    for (int i = 0; i < N - AHEAD; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, M, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, M * AHEAD, 0);
}

// Lower-triangular 16x16 tile pair pr = 0 .. 9 (query tile ti, key tile tj) of
// the 64x64 masks, row by row: (0,0), (1,0), (1,1), (2,0), ...  Formed with
// scalar arithmetic: a table in memory would be read with scalar loads, whose
// waits also wait for every LDS read in flight.
__device__ __forceinline__ void tile_pair(int pr, int& ti, int& tj) {
    ti = (pr >= 1) + (pr >= 3) + (pr >= 6);
    tj = pr - ti * (ti + 1) / 2;
}

// Decays e^{gamma_i - gamma_j} for query i = 16 ti + lr and keys
// j = 16 tj + lq .. +3; zero above the diagonal.
__device__ __forceinline__ floatx4 tile_decay(const float* gam, int ti, int tj, int lr, int lq) {
    const int i = 16 * ti + lr;
    const float gi = gam[i];
    const floatx4 gj = *reinterpret_cast<const floatx4*>(&gam[16 * tj + lq]);
    floatx4 dec;
    if (ti > tj) {
        const float gc = gam[16 * ti];
        const float rowf = fast_exp(gi - gc);
#pragma unroll
        for (int r = 0; r < 4; ++r) dec[r] = rowf * fast_exp(gc - gj[r]);
    } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) dec[r] = i >= 16 * tj + lq + r ? fast_exp(gi - gj[r]) : 0.f;
    }
    return dec;
}

}  // namespace
}  // namespace lrc

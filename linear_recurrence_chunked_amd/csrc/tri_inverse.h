// Unit lower-triangular inverse on a 64-row padding, FP32, in LDS, on the
// FP32 matrix cores of CDNA4 (v_mfma_f32_16x16x4f32), for one workgroup of NW
// waves.
//
// Source: "perf(qwen3_5): prefill text prompts in multi-token chunks",
// Implementation -- the chunk is padded to 64 rows with identity rows; the
// eight 8x8 diagonal blocks are inverted by a truncated Neumann series, and
// the result is assembled by merging neighbouring blocks two at a time, all
// blocks of one size together.
//
//  * Diagonal 8x8 blocks: with N the block's strictly lower part, N^8 = 0, so
//        (I + N)^-1 = (I - N)(I + N^2)(I + N^4).
//  * Levels s = 8, 16, 32: each 2s x 2s diagonal block is
//        [[T11, 0], [L21, T22]]  ->  T21 = -T22 (L21 T11),
//    where T11, T22 are the inverted s x s blocks of the previous level and
//    L21 is the untouched block of A below T11.
//
// Mapping.  Everything is a product of 16x16 tiles.  A wave inverts one
// diagonal 16x16 tile alone: N holds the strictly lower parts of its two 8x8
// diagonal blocks, D = (I - N)(I + N^2)(I + N^4) inverts both at once, and the
// level-8 step is T = D - D (L D) with L the tile's lower-left 8x8 block of A.
// The level-16 and level-32 steps follow with workgroup barriers between
// them (five barriers in all); the phases are also available one by one, for
// callers that interleave other work between the barriers.  Products run in FP32 with FP32 accumulation.
//
// Tile product Z = X Y: lane l holds, for X, the row segment
// X[l%16][4g .. 4g+3] (g = l/16) and, for Y, the accumulator-layout column
// slice Y[4g .. 4g+3][l%16]; the four 16x16x4 steps pair k = 4g + kk on both
// sides, so Y can be a previous product's accumulator as it is.
//
// Two ways to form a tile product, chosen by the caller:
//  * MmF32: four v_mfma_f32_16x16x4f32, FP32 operands (32 cycles each).
//  * MmBf16Split: each FP32 operand is split as hi = bf16(x), lo = bf16(x - hi)
//    and the product is hi.hi + lo.hi + hi.lo on the bf16 matrix cores, two
//    v_mfma_f32_16x16x32_bf16 (16 cycles each): the lane's 8 k-slots carry
//    (hi, lo) of X against (hi, hi) of Y, then (hi, lo) against (lo, 0).  The
//    dropped lo.lo term and the roundings leave about 2^-17 of each product's
//    operands, against 2^-24 for MmF32, at a quarter of the matrix-core time.
#pragma once

#include <hip/hip_runtime.h>

namespace lrc {

constexpr int kTriLd = 68;            // row stride of the 64x64 matrix in LDS (floats), 16-byte aligned rows
constexpr int kTriScratch = 32 * 36;  // floats: the 32x36 level-32 product

typedef float tri_f4 __attribute__((ext_vector_type(4)));

namespace tri {

typedef __bf16 tri_bf8 __attribute__((ext_vector_type(8)));

struct MmF32 {
    static __device__ __forceinline__ tri_f4 mm(tri_f4 z, tri_f4 xrow, tri_f4 yc) {
        z = __builtin_amdgcn_mfma_f32_16x16x4f32(xrow[0], yc[0], z, 0, 0, 0);
        z = __builtin_amdgcn_mfma_f32_16x16x4f32(xrow[1], yc[1], z, 0, 0, 0);
        z = __builtin_amdgcn_mfma_f32_16x16x4f32(xrow[2], yc[2], z, 0, 0, 0);
        z = __builtin_amdgcn_mfma_f32_16x16x4f32(xrow[3], yc[3], z, 0, 0, 0);
        return z;
    }
};

struct MmBf16Split {
    static __device__ __forceinline__ tri_f4 mm(tri_f4 z, tri_f4 xrow, tri_f4 yc) {
        tri_bf8 a, b1, b2;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const __bf16 xh = static_cast<__bf16>(xrow[r]);
            const __bf16 yh = static_cast<__bf16>(yc[r]);
            a[r] = xh;
            a[4 + r] = static_cast<__bf16>(xrow[r] - static_cast<float>(xh));
            b1[r] = yh;
            b1[4 + r] = yh;
            b2[r] = static_cast<__bf16>(yc[r] - static_cast<float>(yh));
            b2[4 + r] = static_cast<__bf16>(0.f);
        }
        z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b1, z, 0, 0, 0);
        z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b2, z, 0, 0, 0);
        return z;
    }
};

__device__ __forceinline__ tri_f4 mm(tri_f4 z, tri_f4 xrow, tri_f4 yc) { return MmF32::mm(z, xrow, yc); }
// Row segment X[lr][4g .. 4g+3] of a row-major tile.
__device__ __forceinline__ tri_f4 ld_row(const float* t, int ld, int lr, int g) {
    return *reinterpret_cast<const tri_f4*>(t + lr * ld + 4 * g);
}
// Accumulator-layout slice Y[4g .. 4g+3][lr] of a row-major tile.
__device__ __forceinline__ tri_f4 ld_acc(const float* t, int ld, int lr, int g) {
    return tri_f4{t[(4 * g) * ld + lr], t[(4 * g + 1) * ld + lr], t[(4 * g + 2) * ld + lr], t[(4 * g + 3) * ld + lr]};
}
__device__ __forceinline__ void st_acc(float* t, int ld, int lr, int g, tri_f4 v) {
#pragma unroll
    for (int r = 0; r < 4; ++r) t[(4 * g + r) * ld + lr] = v[r];
}
// Order this wave's LDS writes before its later LDS reads of other lanes'
// data.  A wave's LDS operations execute in order, so fences at wavefront
// scope only keep the compiler from moving the accesses across this point;
// no wait is needed.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace tri

// The inverse in four phases, each run by NW waves numbered w = 0 .. NW-1
// and separated by workgroup barriers that the caller provides:
//   diag    each diagonal 16x16 tile: Neumann on its 8x8 blocks, level 8
//   lvl16   T21 of the two 32x32 diagonal blocks
//   lvl32a  Y = L21 T11 of the 64x64 matrix, into scratch
//   lvl32b  T21 = -T22 Y
// In:  M[i * kTriLd + j] holds A_ij for j < i; entries above the diagonal
//      must be zero; diagonal entries are ignored.
// Out: M holds T = (I + A)^-1 (ones on the diagonal, zeros above).
namespace tri {

__device__ __forceinline__ void lanes(int& lr, int& g) {
    // lane index through an empty asm: addresses are formed per call, not
    // kept in registers by a caller that calls this in a loop
    int tl = threadIdx.x;
    asm volatile("" : "+v"(tl));
    const int lane = tl & 63;
    lr = lane & 15;
    g = lane >> 4;
}

template <int NW, class MM = MmF32>
__device__ inline void diag(float* M, float* /*scratch*/, int w) {
    constexpr int ld = kTriLd;
    int lr, g;
    lanes(lr, g);
    const tri_f4 zero = {0.f, 0.f, 0.f, 0.f};
    for (int t = w; t < 4; t += NW) {
        float* Mt = M + 16 * t * ld + 16 * t;
        tri_f4 nrow = ld_row(Mt, ld, lr, g), nacc = ld_acc(Mt, ld, lr, g);
        tri_f4 lorow = nrow;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int jr = 4 * g + k;  // column of the row segment
            const int ia = 4 * g + k;  // row of the accumulator slice
            const bool in_row = jr < lr && (jr >> 3) == (lr >> 3);
            const bool in_acc = lr < ia && (lr >> 3) == (ia >> 3);
            lorow[k] = (lr >= 8 && jr < 8) ? nrow[k] : 0.f;
            nrow[k] = in_row ? nrow[k] : 0.f;
            nacc[k] = in_acc ? nacc[k] : 0.f;
        }
        // Every product that is needed again as a row operand is also formed
        // in row layout, as the transposed product: MM::mm(Y_acc, X_row) is
        // (X Y)^T in accumulator layout, i.e. X Y in row layout.  That trades
        // the LDS round trips of a layout change for three more products.
        const tri_f4 n2 = MM::mm(zero, nrow, nacc);     // N^2
        const tri_f4 n2r = MM::mm(zero, nacc, nrow);    // N^2, row layout
        const tri_f4 nn2 = MM::mm(zero, nrow, n2);      // N N^2
        const tri_f4 nn2r = MM::mm(zero, n2, nrow);     // N N^2, row layout
        const tri_f4 n4 = MM::mm(zero, n2r, n2);        // N^4
        tri_f4 x, xr;                               // (I - N)(I + N^2), both layouts
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float id = 4 * g + k == lr ? 1.f : 0.f;
            x[k] = id - nacc[k] + n2[k] - nn2[k];
            xr[k] = id - nrow[k] + n2r[k] - nn2r[k];
        }
        const tri_f4 d = x + MM::mm(zero, xr, n4);     // D = X (I + N^4)
        const tri_f4 dr = xr + MM::mm(zero, n4, xr);   // D, row layout
        const tri_f4 y = MM::mm(zero, lorow, d);       // L D
        const tri_f4 z = MM::mm(zero, dr, y);          // D L D
        st_acc(Mt, ld, lr, g, d - z);
    }
}

// The diagonal phase on the vector ALUs in FP32, one 16x16 tile per wave, for
// callers with kDiagScratch floats of LDS per wave: the 8x8 Neumann products
// and the level-8 step as 8x8 products.  Lane l holds entries (i, j), (i, j+1)
// of block b = l/32 of the tile's two 8x8 diagonal blocks, i = (l/4) % 8,
// j = 2 (l%4), so the four lanes of a quad hold one row.  An 8x8 product is
// 16 FMAs per lane over a row of the left operand and two columns of the
// right one.  The left operand's row comes from LDS once (N, and L for level
// 8) and otherwise from the quad's own results through DPP quad broadcasts;
// each right operand is written to LDS transposed, so its two columns read
// back as four 16-byte rows.  Per wave that is six products in five
// dependent steps, against the nine 16x16 tile products of diag():
//   N2 = N N;  N3 = N N2, N4 = N2 N2;  X = I - N + N2 - N3;  D = X + X N4;
//   level 8:  T21 = -D1 (L D0).
constexpr int kDiagScratch = 6 * 64;  // N2, N4 (two blocks each), D0, L D0: 8x8 blocks, transposed

// Row i of a row-major 8x8 block with row stride ld (16-byte aligned rows).
__device__ __forceinline__ void row8(const float* m, int ld, int i, float (&r)[8]) {
    const tri_f4 a = *reinterpret_cast<const tri_f4*>(m + i * ld);
    const tri_f4 b = *reinterpret_cast<const tri_f4*>(m + i * ld + 4);
    r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
    r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
}
// Columns j, j+1 of a row-major 8x8 block.
__device__ __forceinline__ void cols8(const float* m, int ld, int j, float (&c0)[8], float (&c1)[8]) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const float2 x = *reinterpret_cast<const float2*>(m + k * ld + j);
        c0[k] = x.x;
        c1[k] = x.y;
    }
}
__device__ __forceinline__ float2 dot8(const float (&r)[8], const float (&c0)[8], const float (&c1)[8]) {
    float2 z = make_float2(0.f, 0.f);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        z.x = fmaf(r[k], c0[k], z.x);
        z.y = fmaf(r[k], c1[k], z.y);
    }
    return z;
}

// Lane Q of this lane's quad, through a DPP quad broadcast.
template <int Q>
__device__ __forceinline__ float quad_lane(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), Q * 0x55, 0xf, 0xf, false));
}
// Row i of an 8x8 block whose entries (i, 2q), (i, 2q+1) sit in lane q of the quad.
__device__ __forceinline__ void quad_row(float2 c, float (&r)[8]) {
    r[0] = quad_lane<0>(c.x);
    r[1] = quad_lane<0>(c.y);
    r[2] = quad_lane<1>(c.x);
    r[3] = quad_lane<1>(c.y);
    r[4] = quad_lane<2>(c.x);
    r[5] = quad_lane<2>(c.y);
    r[6] = quad_lane<3>(c.x);
    r[7] = quad_lane<3>(c.y);
}
// Entries (i, j), (i, j+1) into the transposed copy bt (row stride 8).
__device__ __forceinline__ void put_t(float* bt, int i, int j, float2 v) {
    bt[j * 8 + i] = v.x;
    bt[(j + 1) * 8 + i] = v.y;
}

//   With ZERO_UPPER the caller guarantees that each diagonal tile of M is zero
//   on and above its diagonal (A as the masked products write it), so N is
//   the 8x8 block as it stands and the masking is skipped.
template <int NW, bool ZERO_UPPER = false>
__device__ inline void diag_valu(float* M, float* scratch, int w) {
    constexpr int ld = kTriLd;
    int tl = threadIdx.x;
    asm volatile("" : "+v"(tl));
    const int lane = tl & 63, b = lane >> 5, i = (lane >> 2) & 7, j = 2 * (lane & 3);
    float* S = scratch + w * kDiagScratch;
    float* N2t = S + 64 * b;        // this lane's block of N2 and N4, transposed
    float* N4t = S + 128 + 64 * b;
    float* D0t = S + 256;           // D0, transposed
    float* Yt = S + 320;            // L D0, transposed
    for (int t = w; t < 4; t += NW) {
        float* Mt = M + 16 * t * ld + 16 * t;
        const float* Mb = Mt + 8 * b * ld + 8 * b;  // block b of the tile in A
        float n[8], c0[8], c1[8], l[8];
        row8(Mb, ld, i, n);
        cols8(Mb, ld, j, c0, c1);
        row8(Mt + 8 * ld, ld, i, l);  // row i of the tile's lower-left block
        if constexpr (!ZERO_UPPER)
#pragma unroll
            for (int k = 0; k < 8; ++k) {  // N: the block's strictly lower part
                n[k] = k < i ? n[k] : 0.f;
                c0[k] = j < k ? c0[k] : 0.f;
                c1[k] = j + 1 < k ? c1[k] : 0.f;
            }
        // N_ij, N_i,j+1 as one read (indexing c0, c1 by the lane's i would be a chain of selects)
        float2 nown = *reinterpret_cast<const float2*>(Mb + i * ld + j);
        if constexpr (!ZERO_UPPER) {
            nown.x = j < i ? nown.x : 0.f;
            nown.y = j + 1 < i ? nown.y : 0.f;
        }
        const float2 n2 = dot8(n, c0, c1);
        put_t(N2t, i, j, n2);
        wave_sync();
        float r2[8];
        quad_row(n2, r2);
        row8(N2t, 8, j, c0);
        row8(N2t, 8, j + 1, c1);
        const float2 n3 = dot8(n, c0, c1);
        const float2 n4 = dot8(r2, c0, c1);
        put_t(N4t, i, j, n4);
        wave_sync();
        float r3[8], x[8];
        quad_row(n3, r3);
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = ((k == i ? 1.f : 0.f) - n[k]) + (r2[k] - r3[k]);
        row8(N4t, 8, j, c0);
        row8(N4t, 8, j + 1, c1);
        const float2 xn4 = dot8(x, c0, c1);
        const float2 d = make_float2((((i == j ? 1.f : 0.f) - nown.x) + (n2.x - n3.x)) + xn4.x,
                                     (((i == j + 1 ? 1.f : 0.f) - nown.y) + (n2.y - n3.y)) + xn4.y);
        *reinterpret_cast<float2*>(&Mt[(8 * b + i) * ld + 8 * b + j]) = d;
        if (!b) put_t(D0t, i, j, d);
        wave_sync();
        row8(D0t, 8, j, c0);
        row8(D0t, 8, j + 1, c1);
        const float2 y = dot8(l, c0, c1);  // L D0 (both halves; block 1's lanes keep it)
        if (b) put_t(Yt, i, j, y);
        wave_sync();
        float dr[8];
        quad_row(d, dr);                   // row i of D1 on block 1's lanes
        row8(Yt, 8, j, c0);
        row8(Yt, 8, j + 1, c1);
        const float2 z = dot8(dr, c0, c1);
        if (b) *reinterpret_cast<float2*>(&Mt[(8 + i) * ld + j]) = make_float2(-z.x, -z.y);
        if constexpr (NW < 4) wave_sync();  // the scratch is reused by the next tile
    }
}

// level 16: blocks b = 0, 1 (rows 32b+16 .., columns 32b ..)
template <int NW, class MM = MmF32>
__device__ inline void lvl16(float* M, int w) {
    constexpr int ld = kTriLd;
    int lr, g;
    lanes(lr, g);
    const tri_f4 zero = {0.f, 0.f, 0.f, 0.f};
    for (int b = w; b < 2; b += NW) {
        float* L21 = M + (32 * b + 16) * ld + 32 * b;
        const tri_f4 y = MM::mm(zero, ld_row(L21, ld, lr, g), ld_acc(M + 32 * b * ld + 32 * b, ld, lr, g));
        const tri_f4 z = MM::mm(zero, ld_row(M + (32 * b + 16) * ld + 32 * b + 16, ld, lr, g), y);
        st_acc(L21, ld, lr, g, -z);
    }
}

// level 32, first half: Y = L21 T11 by 16x16 output tiles (ta, tb), into scratch (32 x 36)
template <int NW, class MM = MmF32>
__device__ inline void lvl32a(float* M, float* scratch, int w) {
    constexpr int ld = kTriLd;
    int lr, g;
    lanes(lr, g);
    const tri_f4 zero = {0.f, 0.f, 0.f, 0.f};
    for (int q = w; q < 4; q += NW) {
        const int ta = q >> 1, tb = q & 1;
        tri_f4 acc = zero;
        for (int c = tb; c < 2; ++c)  // T11 is block lower triangular
            acc = MM::mm(acc, ld_row(M + (32 + 16 * ta) * ld + 16 * c, ld, lr, g),
                     ld_acc(M + 16 * c * ld + 16 * tb, ld, lr, g));
        st_acc(scratch + 16 * ta * 36 + 16 * tb, 36, lr, g, acc);
    }
}

// level 32, second half: T21 = -T22 Y
template <int NW, class MM = MmF32>
__device__ inline void lvl32b(float* M, const float* scratch, int w) {
    constexpr int ld = kTriLd;
    int lr, g;
    lanes(lr, g);
    const tri_f4 zero = {0.f, 0.f, 0.f, 0.f};
    for (int q = w; q < 4; q += NW) {
        const int ta = q >> 1, tb = q & 1;
        tri_f4 acc = zero;
        for (int c = 0; c <= ta; ++c)  // T22 is block lower triangular
            acc = MM::mm(acc, ld_row(M + (32 + 16 * ta) * ld + 32 + 16 * c, ld, lr, g),
                     ld_acc(scratch + 16 * c * 36 + 16 * tb, 36, lr, g));
        st_acc(M + (32 + 16 * ta) * ld + 16 * tb, ld, lr, g, -acc);
    }
}

}  // namespace tri

// The whole inverse for a workgroup of NW waves.  All NW waves of the block
// must call it; it begins and ends with a barrier.
template <int NW>
__device__ inline void tri_inverse64(float* M, float* scratch) {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    __syncthreads();
    tri::diag<NW>(M, scratch, w);
    __syncthreads();
    tri::lvl16<NW>(M, w);
    __syncthreads();
    tri::lvl32a<NW>(M, scratch, w);
    __syncthreads();
    tri::lvl32b<NW>(M, scratch, w);
    __syncthreads();
}

}  // namespace lrc

// Unit lower-triangular inverse on a 64-row padding, for one workgroup of
// 256 threads, in LDS, FP32.
//
// Source: "perf(qwen3_5): prefill text prompts in multi-token chunks",
// Implementation -- I + A is inverted on a fixed 64-row padding (padded rows
// are identity): 8x8 diagonal blocks by a Neumann product, then 2x2 block
// inversion level by level, batched over the blocks of each level.
//
//  * Diagonal 8x8 blocks: with N the block's strictly lower part, N^8 = 0, so
//        (I + N)^-1 = (I - N)(I + N^2)(I + N^4).
//  * Levels s = 8, 16, 32: each 2s x 2s diagonal block is
//        [[T11, 0], [L21, T22]]  ->  T21 = -T22 (L21 T11),
//    where T11, T22 are the inverted s x s blocks of the previous level and
//    L21 is the untouched block of A below T11.
// All loops have compile-time trip counts and read 16-byte row segments, so
// the loads of a level issue together instead of one dependent load at a
// time.
#pragma once

#include <hip/hip_runtime.h>

namespace lrc {

constexpr int kTriLd = 68;  // row stride of the 64x64 matrix in LDS (floats), 16-byte aligned rows

// Scratch: 3 x 8 x 64 floats for the Neumann stage, up to 32 x 32 for the levels.
constexpr int kTriScratch = 3 * 8 * 64;

template <int s>
__device__ __forceinline__ void tri_level(float* M, float* Y) {
    constexpr int quads = 8 * s;            // (64 / 2s) blocks x s*s/4 output quads
    constexpr int per = s * s / 4;          // quads per block
    const int tid = threadIdx.x;
    int b = 0, r = 0, c = 0, base = 0;
    if (tid < quads) {
        b = tid / per;
        r = (tid % per) / (s / 4);
        c = (tid % (s / 4)) * 4;
        base = b * 2 * s;
        // Y_b = L21_b T11_b (entries of T11 above its diagonal are zero)
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        const float* l21 = M + (base + s + r) * kTriLd + base;
#pragma unroll
        for (int m = 0; m < s; ++m) {
            const float l = l21[m];
            const float4 t = *reinterpret_cast<const float4*>(M + (base + m) * kTriLd + base + c);
            acc.x = fmaf(l, t.x, acc.x);
            acc.y = fmaf(l, t.y, acc.y);
            acc.z = fmaf(l, t.z, acc.z);
            acc.w = fmaf(l, t.w, acc.w);
        }
        *reinterpret_cast<float4*>(Y + b * s * s + r * s + c) = acc;
    }
    __syncthreads();
    if (tid < quads) {
        // T21_b = -T22_b Y_b, written over L21_b (entries of T22 above its diagonal are zero)
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        const float* t22 = M + (base + s + r) * kTriLd + base + s;
#pragma unroll
        for (int m = 0; m < s; ++m) {
            const float t = t22[m];
            const float4 y = *reinterpret_cast<const float4*>(Y + b * s * s + m * s + c);
            acc.x = fmaf(t, y.x, acc.x);
            acc.y = fmaf(t, y.y, acc.y);
            acc.z = fmaf(t, y.z, acc.z);
            acc.w = fmaf(t, y.w, acc.w);
        }
        *reinterpret_cast<float4*>(M + (base + s + r) * kTriLd + base + c) =
            make_float4(-acc.x, -acc.y, -acc.z, -acc.w);
    }
    __syncthreads();
}

// In:  M[i * kTriLd + j] holds A_ij for j < i; entries above the diagonal
//      must be zero; diagonal entries are ignored.
// Out: M holds T = (I + A)^-1 (ones on the diagonal, zeros above).
// All 256 threads of the block must call it; it begins and ends with a
// barrier.
__device__ inline void tri_inverse64(float* M, float* scratch) {
    const int tid = threadIdx.x;
    __syncthreads();
    // ---- Neumann stage: 8 blocks x 64 entries, 2 entries per thread.
    float* N2 = scratch;
    float* N4 = scratch + 512;
    float* X = scratch + 1024;
    auto Nb = [&](int blk, int r, int c) -> float {  // strictly lower part of a diagonal block
        return c < r ? M[(blk * 8 + r) * kTriLd + blk * 8 + c] : 0.f;
    };
#pragma unroll
    for (int e2 = 0; e2 < 2; ++e2) {
        const int e = tid * 2 + e2, blk = e >> 6, r = (e >> 3) & 7, c = e & 7;
        float s = 0.f;
#pragma unroll
        for (int m = 0; m < 8; ++m) s = fmaf(Nb(blk, r, m), Nb(blk, m, c), s);
        N2[e] = s;
    }
    __syncthreads();
#pragma unroll
    for (int e2 = 0; e2 < 2; ++e2) {
        const int e = tid * 2 + e2, blk = e >> 6, r = (e >> 3) & 7, c = e & 7;
        const float* n2 = N2 + blk * 64;
        float s4 = 0.f, sx = 0.f;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            s4 = fmaf(n2[r * 8 + m], n2[m * 8 + c], s4);
            sx = fmaf(Nb(blk, r, m), n2[m * 8 + c], sx);  // N N^2
        }
        N4[e] = s4;
        // X = (I - N)(I + N^2) = I - N + N^2 - N N^2
        X[e] = (r == c ? 1.f : 0.f) - Nb(blk, r, c) + n2[r * 8 + c] - sx;
    }
    __syncthreads();
    float tnew[2];
#pragma unroll
    for (int e2 = 0; e2 < 2; ++e2) {
        const int e = tid * 2 + e2, blk = e >> 6, r = (e >> 3) & 7, c = e & 7;
        const float* x = X + blk * 64;
        const float* n4 = N4 + blk * 64;
        float s = x[r * 8 + c];  // X (I + N^4) = X + X N^4
#pragma unroll
        for (int m = 0; m < 8; ++m) s = fmaf(x[r * 8 + m], n4[m * 8 + c], s);
        tnew[e2] = s;
    }
    __syncthreads();  // every read of the diagonal blocks of A is done
#pragma unroll
    for (int e2 = 0; e2 < 2; ++e2) {
        const int e = tid * 2 + e2, blk = e >> 6, r = (e >> 3) & 7, c = e & 7;
        M[(blk * 8 + r) * kTriLd + blk * 8 + c] = tnew[e2];
    }
    __syncthreads();
    // ---- Levels s = 8, 16, 32 (two barriers each, the last one closes the routine).
    tri_level<8>(M, scratch);
    tri_level<16>(M, scratch);
    tri_level<32>(M, scratch);
}

}  // namespace lrc

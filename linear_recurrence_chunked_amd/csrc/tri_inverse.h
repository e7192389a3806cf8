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
#pragma once

#include <hip/hip_runtime.h>

namespace lrc {

constexpr int kTriLd = 65;  // row stride of the 64x64 matrix in LDS (floats)

// Scratch: 3 x 8 x 64 floats for the Neumann stage, 32 x 32 for the levels.
constexpr int kTriScratch = 3 * 8 * 64;

// In:  M[i * kTriLd + j] holds A_ij for j < i (the strictly lower part);
//      entries on and above the diagonal are ignored.
// Out: M holds T = (I + A)^-1 in full (ones on the diagonal, zeros above).
// All 256 threads of the block must call it; it begins and ends with a
// barrier.
__device__ inline void tri_inverse64(float* M, float* scratch) {
    const int tid = threadIdx.x;
    __syncthreads();
    // ---- Neumann stage: 8 blocks x 64 entries, 2 entries per thread.
    float* N2 = scratch;
    float* N4 = scratch + 512;
    float* X = scratch + 1024;
    auto Nb = [&](int blk, int r, int c) -> float {  // strictly lower part of diagonal block
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
    // ---- Levels: s = 8, 16, 32.
    float* Y = scratch;  // holds L21 T11 for every block of the level (64 * s / 2 <= 1024 floats)
#pragma unroll
    for (int s = 8; s <= 32; s *= 2) {
        const int nblk = 64 / (2 * s);
        const int per = s * s;  // entries per block
        __syncthreads();
        // Y_b = L21_b T11_b
        for (int e = tid; e < nblk * per; e += 256) {
            const int b = e / per, r = (e % per) / s, c = e % s;
            const int base = b * 2 * s;
            const float* l21 = M + (base + s + r) * kTriLd + base;
            float acc = 0.f;
            for (int m = c; m < s; ++m) acc = fmaf(l21[m], M[(base + m) * kTriLd + base + c], acc);  // T11 lower
            Y[e] = acc;
        }
        __syncthreads();
        // T21_b = -T22_b Y_b, written over L21_b
        for (int e = tid; e < nblk * per; e += 256) {
            const int b = e / per, r = (e % per) / s, c = e % s;
            const int base = b * 2 * s;
            const float* t22 = M + (base + s + r) * kTriLd + base + s;
            const float* y = Y + b * per;
            float acc = 0.f;
            for (int m = 0; m <= r; ++m) acc = fmaf(t22[m], y[m * s + c], acc);  // T22 lower
            M[(base + s + r) * kTriLd + base + c] = -acc;
        }
    }
    __syncthreads();
    // Upper triangle to zero (the diagonal already holds ones).
    for (int e = tid; e < 64 * 64; e += 256) {
        const int r = e >> 6, c = e & 63;
        if (c > r) M[r * kTriLd + c] = 0.f;
    }
    __syncthreads();
}

}  // namespace lrc

// RWKV-4 time shift over rows, FP32, on gfx950.
//
// Source: "perf(rwkv): prefill text prompts in multi-token chunks",
// Implementation -- each mixed input blends row t with row t-1, and row 0 with
// the incoming shift state; the shift state kept for the next chunk is the
// chunk's last row.  RWKV-4 blends per channel, mu x_t + (1 - mu) x_{t-1},
// once per mixed input (key, value, receptance): M mixing vectors applied to
// the same rows.
//
// Mapping on CDNA4: a thread owns 4 adjacent channels (one 16-byte run) of a
// tile of kTile rows and walks it row by row, keeping the previous row in
// registers, so every row of x is read once and all M mixed rows are written
// from it (the M outputs of the input path in one pass).  A tile's first row
// takes its predecessor from x, or from the incoming state for the prompt's
// first row.  Only the tile-0 thread of a (prompt, channel group) reads the
// incoming state, and it reads it before writing the new one, so the state
// may be updated in place.  The blend is computed as mu * x + (1 - mu) * prev
// so that mu = 1 and mu = 0 give the row and the previous row exactly.
#include "lrc_device.h"
#include "lrc_internal.h"

namespace lrc {
namespace {

// One wave per workgroup: at C = 2560 a row is 640 threads of 4 channels, ten
// whole workgroups of 64 where workgroups of 256 left half of the third idle,
// and the tiles of short and long prompts spread more evenly (0.263 -> 0.251 ms
// on the mixed prefill lengths).
constexpr int kThreads = 64;
constexpr int kTile = 16;
constexpr int kUnroll = 8;

// The 16-byte accesses are nontemporal: each row is read, and each output row
// written, once.
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int VEC>
__device__ __forceinline__ void ld(const float* p, int nc, float* v) {
    if (VEC == 4) {
        const f32x4 q = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
        v[0] = q[0]; v[1] = q[1]; v[2] = q[2]; v[3] = q[3];
    } else {
#pragma unroll
        for (int i = 0; i < VEC; ++i) v[i] = i < nc ? p[i] : 0.f;
    }
}

template <int VEC>
__device__ __forceinline__ void st(float* p, int nc, const float* v) {
    if (VEC == 4) {
        __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4*>(p));
    } else {
#pragma unroll
        for (int i = 0; i < VEC; ++i)
            if (i < nc) p[i] = v[i];
    }
}

template <int VEC>
__global__ __launch_bounds__(kThreads) void time_shift_kernel(const float* __restrict__ x, float* __restrict__ out,
                                                             const float* state_in, float* state_out,
                                                             const float* __restrict__ mix, Batch bt, int C, int M,
                                                             long plane) {
    const int c0 = (blockIdx.x * kThreads + threadIdx.x) * VEC;
    if (c0 >= C) return;
    const int nc = min(VEC, C - c0);
    const int p = batch_prompt(bt, blockIdx.y);
    const long row0 = batch_row0(bt, p);
    const int L = batch_len(bt, p);
    float mu[LRC_MAX_MIX][VEC], om[LRC_MAX_MIX][VEC];
#pragma unroll
    for (int j = 0; j < LRC_MAX_MIX; ++j) {
        if (j < M) {
            ld<VEC>(mix + (long)j * C + c0, nc, mu[j]);
        } else {
#pragma unroll
            for (int i = 0; i < VEC; ++i) mu[j][i] = 0.f;
        }
#pragma unroll
        for (int i = 0; i < VEC; ++i) om[j][i] = 1.f - mu[j][i];
    }
    const int ntiles = max(1, (L + kTile - 1) / kTile);
    for (int tile = blockIdx.z; tile < ntiles; tile += gridDim.z) {
        const int t0 = tile * kTile;
        float prev[VEC];
        if (t0 == 0)
            ld<VEC>(state_in + (long)p * C + c0, nc, prev);
        else
            ld<VEC>(x + (row0 + t0 - 1) * C + c0, nc, prev);
        const int n = min(kTile, L - t0);
        auto emit = [&](long r, const float* cur) {
#pragma unroll
            for (int j = 0; j < LRC_MAX_MIX; ++j) {
                if (j >= M) break;
                float o[VEC];
#pragma unroll
                for (int e = 0; e < VEC; ++e) o[e] = fmaf(mu[j][e], cur[e], om[j][e] * prev[e]);
                st<VEC>(out + j * plane + r * C + c0, nc, o);
            }
#pragma unroll
            for (int e = 0; e < VEC; ++e) prev[e] = cur[e];
        };
        int i = 0;
        // groups of kUnroll rows: all loads first, so they are in flight together
        for (; i + kUnroll <= n; i += kUnroll) {
            float cur[kUnroll][VEC];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) ld<VEC>(x + (row0 + t0 + i + u) * C + c0, nc, cur[u]);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) emit(row0 + t0 + i + u, cur[u]);
        }
        for (; i < n; ++i) {
            float cur[VEC];
            ld<VEC>(x + (row0 + t0 + i) * C + c0, nc, cur);
            emit(row0 + t0 + i, cur);
        }
        if (tile == 0) {
            float ns[VEC];
            if (L > 0)
                ld<VEC>(x + (row0 + L - 1) * C + c0, nc, ns);
            else
#pragma unroll
                for (int e = 0; e < VEC; ++e) ns[e] = prev[e];
            st<VEC>(state_out + (long)p * C + c0, nc, ns);
        }
    }
}

}  // namespace

hipError_t launch_time_shift(const float* x, float* out, const float* state_in, float* state_out, const float* mix,
                             const Batch& bt, int C, int M, long plane, hipStream_t st) {
    int maxL = 0;
    for (int i = 0; i < bt.P; ++i) maxL = max(maxL, batch_len(bt, batch_prompt(bt, i)));
    const int tiles = max(1, min(65535, (maxL + kTile - 1) / kTile));
    if (C % 4 == 0) {
        const dim3 grid((unsigned)((C / 4 + kThreads - 1) / kThreads), (unsigned)bt.P, (unsigned)tiles);
        hipLaunchKernelGGL(time_shift_kernel<4>, grid, dim3(kThreads), 0, st, x, out, state_in, state_out, mix, bt,
                           C, M, plane);
    } else {
        const dim3 grid((unsigned)((C + kThreads - 1) / kThreads), (unsigned)bt.P, (unsigned)tiles);
        hipLaunchKernelGGL(time_shift_kernel<1>, grid, dim3(kThreads), 0, st, x, out, state_in, state_out, mix, bt,
                           C, M, plane);
    }
    return hipGetLastError();
}

}  // namespace lrc

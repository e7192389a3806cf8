// Mamba mixer rows with the discretisation and the readout fused around the
// selective scan, FP32, on gfx950.
//
// Source: "perf(mamba): prefill text prompts in multi-token chunks",
// Implementation -- the mixer rows run the scan h_t = a_t h_{t-1} + b_t
// between forming a, b and reading h out.  Here those steps are the
// selective state-space step of Mamba:
//   a_t[d][n] = exp(dt[t][d] A[d][n]),  b_t[d][n] = dt[t][d] B[t][n] x[t][d],
//   h_t = a_t h_{t-1} + b_t,            y[t][d] = sum_n C[t][n] h_t[d][n] + D[d] x[t][d].
// a, b and h never reach HBM: per row the kernel reads x, dt (per channel)
// and B, C (per row, shared by all channels) and writes y, instead of
// reading a, b and writing h for every (d, n).
//
// Mapping on CDNA4.  LPD consecutive lanes (4 for d_state >= 16, else 2) own
// one channel d: lane (d, part) keeps the N/LPD states h[d][part*N/LPD ..] in
// registers for the whole prompt and walks the prompt's rows; the parts of
// C.h are added across the lanes by DPP quad permutes.  More lanes per channel
// shorten the per-row chain of the longest prompts, whose waves also get
// issue priority.  Each lane's N/2 recurrences are independent, so one
// row's exps and FMAs overlap.  a = exp(dt A) is the hardware base-2
// exponential of dt (A log2 e), with A log2 e formed once per lane.
//   * B and C of a 64-row chunk are staged in LDS by the workgroup (the next
//     chunk's rows load into registers while the current chunk computes);
//     every lane of a part reads the same LDS address (a broadcast).
//   * x and dt move through a register ring of two 16-row groups, loaded one
//     group ahead; loads past the prompt re-read its last row and those rows
//     are never computed, so the state stops at the prompt's last row.
#include "lrc_device.h"
#include "lrc_internal.h"

namespace lrc {
namespace {

#ifndef LRC_MIXER_LANES
#define LRC_MIXER_LANES 4
#endif
constexpr int kThreads = 256;
constexpr int kLanes = LRC_MIXER_LANES;  // lanes per channel when d_state allows (2 or 4)
constexpr int kChunk = 64;             // rows of B and C staged per chunk
// Rows of x and dt per register group; a full group is straight-line code,
// so the longer it is, the more rows' reads and exponentials are in flight
// while the state chain runs (two groups per chunk at most: the ring
// alternates within a chunk).
constexpr int kGroup = 16;
constexpr float kLog2e = 1.4426950408889634f;

// Sum over the LPD lanes (1, 2 or 4 consecutive lanes of a quad) that share a channel.
template <int LPD>
__device__ __forceinline__ float lanes_sum(float v) {
    if (LPD >= 2) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xb1, 0xf, 0xf, false));
    if (LPD >= 4) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4e, 0xf, 0xf, false));
    return v;
}

template <int NP, int LPD>
__global__ __launch_bounds__(kThreads) void mamba_mixer_kernel(const float* __restrict__ x,
                                                              const float* __restrict__ dt,
                                                              const float* __restrict__ A,
                                                              const float* __restrict__ Bm,
                                                              const float* __restrict__ Cm,
                                                              const float* __restrict__ Dp, float* __restrict__ y,
                                                              const float* h_in, float* h_out, Batch bt, int Dm) {
    constexpr int N = LPD * NP;
    constexpr int PER_ROW = 2 * N;                   // floats of B and C per row
    constexpr int STAGE = kChunk * PER_ROW;          // floats staged per chunk
    constexpr int LOADS = (STAGE + kThreads - 1) / kThreads;
    __shared__ __align__(16) float bc[2][kChunk][PER_ROW];  // [buffer][row][B | C]

    const int tid = threadIdx.x;
    const int part = tid % LPD;  // which part of the channel's states this lane owns
    const int d = blockIdx.x * (kThreads / LPD) + tid / LPD;
    const bool valid = d < Dm;
    const int dl = valid ? d : Dm - 1;  // lanes past Dm compute a copy of the last channel and store nothing
    const int p = batch_prompt(bt, blockIdx.y);
    const long row0 = batch_row0(bt, p);
    const int L = batch_len(bt, p);
    {   // the longest prompts come first in the grid; their waves get issue priority
        const int q4 = (4 * blockIdx.y) / gridDim.y;
        if (q4 == 0) __builtin_amdgcn_s_setprio(3);
        else if (q4 == 1) __builtin_amdgcn_s_setprio(2);
        else if (q4 == 2) __builtin_amdgcn_s_setprio(1);
    }

    float a2[NP], h[NP];
    const long sbase = ((long)p * Dm + dl) * N + part * NP;
#pragma unroll
    for (int n = 0; n < NP; ++n) {
        a2[n] = A[(long)dl * N + part * NP + n] * kLog2e;
        h[n] = h_in[sbase + n];
    }
    const float dd = Dp[dl];

    // B and C rows of a chunk, cooperatively: element e of the stage is row e / PER_ROW,
    // entry e % PER_ROW (B for the first N, C for the rest).
    float pre[LOADS];
    auto fetch_bc = [&](int c0) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int e = tid + i * kThreads;
            const int r = e / PER_ROW, k = e % PER_ROW;
            const long row = row0 + min(c0 + r, L - 1);
            pre[i] = e < STAGE ? (k < N ? Bm[row * N + k] : Cm[row * N + k - N]) : 0.f;
        }
    };
    auto stage_bc = [&](int buf) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int e = tid + i * kThreads;
            if (e < STAGE) (&bc[buf][0][0])[e] = pre[i];
        }
    };
    float xg[2][kGroup], tg[2][kGroup];
    auto fetch_x = [&](int g0, float (&xs)[kGroup], float (&ts)[kGroup]) {
        const float* xp = x + (row0 + min(g0, L - 1)) * Dm + dl;
        const float* tp = dt + (row0 + min(g0, L - 1)) * Dm + dl;
        const int last = L - 1 - min(g0, L - 1);
#pragma unroll
        for (int i = 0; i < kGroup; ++i) {
            const int off = min(i, last) * Dm;
            xs[i] = xp[off];
            ts[i] = tp[off];
        }
    };
    // Row i of a group (its B, C at row rb + i of LDS buffer buf): advances the
    // lane's states and returns the channel's output y (complete on part 0).
    auto row = [&](int i, int buf, int rb, const float (&xs)[kGroup], const float (&ts)[kGroup]) {
        const float* bcr = &bc[buf][rb + i][0];
        float bv[NP], cv[NP];
#pragma unroll
        for (int n4 = 0; n4 < NP; n4 += (NP >= 4 ? 4 : NP)) {
            if (NP >= 4) {
                const float4 b4 = *reinterpret_cast<const float4*>(bcr + part * NP + n4);
                const float4 c4 = *reinterpret_cast<const float4*>(bcr + N + part * NP + n4);
                bv[n4] = b4.x; bv[n4 + 1] = b4.y; bv[n4 + 2] = b4.z; bv[n4 + 3] = b4.w;
                cv[n4] = c4.x; cv[n4 + 1] = c4.y; cv[n4 + 2] = c4.z; cv[n4 + 3] = c4.w;
            } else {
#pragma unroll
                for (int q = 0; q < NP; ++q) {
                    bv[q] = bcr[part * NP + q];
                    cv[q] = bcr[N + part * NP + q];
                }
            }
        }
        const float dtv = ts[i], xv = xs[i];
        const float dtx = dtv * xv;
        float acc = 0.f;
#pragma unroll
        for (int q = 0; q < NP; ++q) {
            const float a = __builtin_amdgcn_exp2f(dtv * a2[q]);
            h[q] = fmaf(a, h[q], dtx * bv[q]);
            acc = fmaf(cv[q], h[q], acc);
        }
        acc = lanes_sum<LPD>(acc);
        return fmaf(dd, xv, acc);
    };
    // Rows g0 .. g0+n-1 of the prompt.  A full group is straight-line code with
    // its stores at the end, so the reads and exponentials of later rows can be
    // issued while the earlier rows' chains run; only a prompt's last group can
    // be partial.
    auto rows = [&](int g0, int n, int buf, int rb, const float (&xs)[kGroup], const float (&ts)[kGroup]) {
        float* yp = y + (row0 + g0) * Dm + d;
        if (n == kGroup) {
            float out[kGroup];
#pragma unroll
            for (int i = 0; i < kGroup; ++i) out[i] = row(i, buf, rb, xs, ts);
            if (part == 0 && valid)
#pragma unroll
                for (int i = 0; i < kGroup; ++i) yp[(long)i * Dm] = out[i];
        } else {
#pragma unroll
            for (int i = 0; i < kGroup; ++i) {
                if (i >= n) break;
                const float o = row(i, buf, rb, xs, ts);
                if (part == 0 && valid) yp[(long)i * Dm] = o;
            }
        }
    };

    if (L > 0) {
        fetch_bc(0);
        fetch_x(0, xg[0], tg[0]);
    }
    int buf = 0;
    for (int c0 = 0; c0 < L; c0 += kChunk) {
        __syncthreads();  // every wave is done with the buffer about to be written
        stage_bc(buf);
        fetch_bc(c0 + kChunk);
        __syncthreads();
        const int S = min(kChunk, L - c0);
#pragma unroll
        for (int gi = 0; gi < kChunk / kGroup; gi += 2) {
            const int g0 = c0 + gi * kGroup;
            if (gi * kGroup >= S) break;
            fetch_x(g0 + kGroup, xg[1], tg[1]);
            rows(g0, min(kGroup, S - gi * kGroup), buf, gi * kGroup, xg[0], tg[0]);
            if ((gi + 1) * kGroup >= S) break;  // only in a prompt's last chunk
            fetch_x(g0 + 2 * kGroup, xg[0], tg[0]);
            rows(g0 + kGroup, min(kGroup, S - (gi + 1) * kGroup), buf, (gi + 1) * kGroup, xg[1], tg[1]);
        }
        buf ^= 1;
    }
#pragma unroll
    for (int n = 0; n < NP; ++n)
        if (valid) h_out[sbase + n] = h[n];
}

template <int N>
hipError_t launch_np(const float* x, const float* dt, const float* A, const float* Bm, const float* Cm,
                     const float* Dp, float* y, const float* h_in, float* h_out, const Batch& bt, int Dm,
                     hipStream_t st) {
    constexpr int LPD = N >= 16 ? kLanes : 2;
    const int per = kThreads / LPD;
    const dim3 grid((unsigned)((Dm + per - 1) / per), (unsigned)bt.P);
    hipLaunchKernelGGL((mamba_mixer_kernel<N / LPD, LPD>), grid, dim3(kThreads), 0, st, x, dt, A, Bm, Cm, Dp, y,
                       h_in, h_out, bt, Dm);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mamba_mixer(const float* x, const float* dt, const float* A, const float* Bm, const float* Cm,
                              const float* Dp, float* y, const float* h_in, float* h_out, const Batch& bt, int Dm,
                              int N, hipStream_t st) {
    switch (N) {
        case 2: return launch_np<2>(x, dt, A, Bm, Cm, Dp, y, h_in, h_out, bt, Dm, st);
        case 4: return launch_np<4>(x, dt, A, Bm, Cm, Dp, y, h_in, h_out, bt, Dm, st);
        case 8: return launch_np<8>(x, dt, A, Bm, Cm, Dp, y, h_in, h_out, bt, Dm, st);
        case 16: return launch_np<16>(x, dt, A, Bm, Cm, Dp, y, h_in, h_out, bt, Dm, st);
        case 32: return launch_np<32>(x, dt, A, Bm, Cm, Dp, y, h_in, h_out, bt, Dm, st);
        case 64: return launch_np<64>(x, dt, A, Bm, Cm, Dp, y, h_in, h_out, bt, Dm, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace lrc

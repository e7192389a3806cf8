// K2: RWKV-4 WKV over rows, FP32, on gfx950.
//
// Source: "perf(rwkv): prefill text prompts in multi-token chunks",
// Implementation.  Per channel the state keeps A = num e^max and
// B = den e^max.  Row t of a chunk sums, relative to the incoming state,
// three kinds of exponent -- max_0 + t w (the state), k_i + (t-1-i) w for the
// chunk's earlier rows, and the bonus u + k_t -- and shifts by its largest
// exponent before exp; row S, without the bonus, is the outgoing
// (num, den, max).
//
// Mapping on CDNA4: one lane owns one channel of one prompt and walks the
// prompt's 64-row chunks row by row, so every row's loads and stores are
// contiguous across the wave (channels innermost).  Because w does not depend
// on the row, the largest exponent over the state and the earlier rows obeys
//     m_t = max(m_{t-1} + w, k_{t-1}),   m_0 = max_0,
// so each row needs one running maximum instead of a max over t terms, and
// the sums over earlier rows are carried as (num, den) scaled by e^{-m_t}.
// Row t's largest exponent is p_t = max(m_t, u + k_t); exactly one of the two
// exp factors is 1, so a row costs one exp for the output and one for the
// state update (instead of t + 2 per row for the materialised [S+1, S] form).
// After the chunk's last row the carried triple is the page's row-S state.
#include "lrc_device.h"
#include "lrc_internal.h"

namespace lrc {
namespace {

constexpr int kThreads = 256;
constexpr int kGroup = 16;  // rows loaded ahead of the arithmetic

__global__ __launch_bounds__(kThreads) void wkv4_kernel(const float* __restrict__ k, const float* __restrict__ v,
                                                       const float* __restrict__ w, const float* __restrict__ u,
                                                       float* __restrict__ wkv, float* num, float* den, float* mx,
                                                       Batch bt, int C) {
    const int c = blockIdx.x * kThreads + threadIdx.x;
    if (c >= C) return;
    const int p = batch_prompt(bt, blockIdx.y);
    const long row0 = batch_row0(bt, p);
    const int L = batch_len(bt, p);
    const long sidx = (long)p * C + c;
    float aa = num[sidx], bb = den[sidx], pp = mx[sidx];
    const float wc = w[c], uc = u[c];
    const float* kp = k + row0 * C + c;
    const float* vp = v + row0 * C + c;
    float* op = wkv + row0 * C + c;

    for (int t0 = 0; t0 < L; t0 += kGroup) {
        const int n = min(kGroup, L - t0);
        float kb[kGroup], vb[kGroup];
#pragma unroll
        for (int i = 0; i < kGroup; ++i) {
            if (i < n) {
                kb[i] = kp[(long)(t0 + i) * C];
                vb[i] = vp[(long)(t0 + i) * C];
            }
        }
#pragma unroll
        for (int i = 0; i < kGroup; ++i) {
            if (i < n) {
                const float kt = kb[i], vt = vb[i];
                // output: largest exponent of the state and the bonus
                const float eb = uc + kt;
                const float d = pp - eb;
                const float e = fast_exp(-fabsf(d));
                const float fs = d >= 0.f ? 1.f : e;
                const float fb = d >= 0.f ? e : 1.f;
                const float nt = fmaf(fs, aa, fb * vt);
                const float dt = fmaf(fs, bb, fb);
                op[(long)(t0 + i) * C] = nt * __builtin_amdgcn_rcpf(dt);
                // state: decay by e^w, then add row t with its own exponent
                const float ed = pp + wc;
                const float d2 = ed - kt;
                const float e2 = fast_exp(-fabsf(d2));
                const bool keep = d2 >= 0.f;
                const float gs = keep ? 1.f : e2;
                const float gk = keep ? e2 : 1.f;
                aa = fmaf(gs, aa, gk * vt);
                bb = fmaf(gs, bb, gk);
                pp = keep ? ed : kt;
            }
        }
    }
    num[sidx] = aa;
    den[sidx] = bb;
    mx[sidx] = pp;
}

}  // namespace

hipError_t launch_wkv4(const float* k, const float* v, const float* w, const float* u, float* wkv, float* num,
                       float* den, float* mx, const Batch& bt, int C, hipStream_t st) {
    const dim3 grid((unsigned)((C + kThreads - 1) / kThreads), (unsigned)bt.P);
    hipLaunchKernelGGL(wkv4_kernel, grid, dim3(kThreads), 0, st, k, v, w, u, wkv, num, den, mx, bt, C);
    return hipGetLastError();
}

}  // namespace lrc

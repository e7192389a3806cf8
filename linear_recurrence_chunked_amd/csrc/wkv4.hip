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
// on the row, the largest exponent among the state and the rows before row t
// is always of the form  m + n w : m is the incoming max_0 or the key k_i that
// last took the lead, and n the number of rows since (t for the state, t-1-i
// for row i).  The kernel carries (m, n) and forms every exponent directly as
// fma(n, w, m), exactly the page's max_0 + t w and k_i + (t-1-i) w, so no
// rounding accumulates in the running maximum.  The sums over earlier rows
// are carried as (num, den) scaled by e^{-(m + n w)}.  Row t's largest
// exponent is max(m + n w, u + k_t) and exactly one of its two exp factors
// is 1, so a row costs one exp for the output and one for the state update
// (against t + 2 for the materialised [S+1, S] form).
//
// Rows are fetched kGroup at a time, one group ahead of the arithmetic, so
// the HBM latency of the next rows overlaps the current rows' exps.
#include "lrc_device.h"
#include "lrc_internal.h"

namespace lrc {
namespace {

constexpr int kThreads = 256;
constexpr int kGroup = 16;

struct WkvState {
    float aa, bb;  // num, den scaled by e^{-(m + n w)}
    float m, n;    // current largest exponent is m + n w
};

__device__ __forceinline__ void wkv_row(WkvState& s, float wc, float uc, float kt, float vt, float* out) {
    const float pp = fmaf(s.n, wc, s.m);
    // output: largest exponent of (state, earlier rows) against the bonus
    const float eb = uc + kt;
    const float d = pp - eb;
    const float e = fast_exp(-fabsf(d));
    const float fs = d >= 0.f ? 1.f : e;
    const float fb = d >= 0.f ? e : 1.f;
    const float nt = fmaf(fs, s.aa, fb * vt);
    const float dt = fmaf(fs, s.bb, fb);
    *out = nt * __builtin_amdgcn_rcpf(dt);
    // state: one more decay, then row t with its own exponent
    const float ed = fmaf(s.n + 1.f, wc, s.m);
    const float d2 = ed - kt;
    const float e2 = fast_exp(-fabsf(d2));
    if (d2 >= 0.f) {  // the decayed maximum stays in the lead
        s.aa = fmaf(e2, vt, s.aa);
        s.bb = s.bb + e2;
        s.n = s.n + 1.f;
    } else {          // row t's key takes the lead
        s.aa = fmaf(e2, s.aa, vt);
        s.bb = fmaf(e2, s.bb, 1.f);
        s.m = kt;
        s.n = 0.f;
    }
}

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
    WkvState s{num[sidx], den[sidx], mx[sidx], 0.f};
    const float wc = w[c], uc = u[c];
    const float* kp = k + row0 * C + c;
    const float* vp = v + row0 * C + c;
    float* op = wkv + row0 * C + c;

    float k0[kGroup], v0[kGroup], k1[kGroup], v1[kGroup];
    auto fetch = [&](int t0, float (&kb)[kGroup], float (&vb)[kGroup]) {
#pragma unroll
        for (int i = 0; i < kGroup; ++i)
            if (t0 + i < L) {
                kb[i] = kp[(long)(t0 + i) * C];
                vb[i] = vp[(long)(t0 + i) * C];
            }
    };
    auto consume = [&](int t0, const float (&kb)[kGroup], const float (&vb)[kGroup]) {
#pragma unroll
        for (int i = 0; i < kGroup; ++i)
            if (t0 + i < L) wkv_row(s, wc, uc, kb[i], vb[i], op + (long)(t0 + i) * C);
    };

    if (L > 0) fetch(0, k0, v0);
    for (int t0 = 0; t0 < L; t0 += 2 * kGroup) {
        if (t0 + kGroup < L) fetch(t0 + kGroup, k1, v1);
        consume(t0, k0, v0);
        if (t0 + kGroup >= L) break;
        if (t0 + 2 * kGroup < L) fetch(t0 + 2 * kGroup, k0, v0);
        consume(t0 + kGroup, k1, v1);
    }
    num[sidx] = s.aa;
    den[sidx] = s.bb;
    mx[sidx] = fmaf(s.n, wc, s.m);
}

}  // namespace

hipError_t launch_wkv4(const float* k, const float* v, const float* w, const float* u, float* wkv, float* num,
                       float* den, float* mx, const Batch& bt, int C, hipStream_t st) {
    const dim3 grid((unsigned)((C + kThreads - 1) / kThreads), (unsigned)bt.P);
    hipLaunchKernelGGL(wkv4_kernel, grid, dim3(kThreads), 0, st, k, v, w, u, wkv, num, den, mx, bt, C);
    return hipGetLastError();
}

}  // namespace lrc

// WKV with a token-dependent decay, FP32 sums with FP64 exponents, on gfx950.
//
// Source: "perf(rwkv): prefill text prompts in multi-token chunks", Notes For
// Future Readers -- RWKV versions whose decay depends on the token need
// another chunk form than the RWKV-4 one.  The pages give no formula for those
// versions; this kernel computes the RWKV-4 recurrence with the channel decay
// w replaced by a decay w_t of each row:
//   A_t = e^{w_t} A_{t-1} + e^{k_t} v_t,   B_t = e^{w_t} B_{t-1} + e^{k_t},
//   wkv_t = (A_{t-1} + e^{u+k_t} v_t) / (B_{t-1} + e^{u+k_t}).
// Row t of a chunk then combines the exponents max_0 + W_t (the incoming
// state, W_t = w_0 + .. + w_{t-1}), k_i + W_t - W_{i+1} for earlier rows i, and
// the bonus u + k_t: the RWKV-4 chunk form with sums of the rows' decays in
// place of multiples of one decay.
//
// Exponent bookkeeping.  With a constant decay the running maximum is
// m + n w, formed exactly; here the decays of different rows add up, so the
// running maximum and every sum of decays are kept in FP64, where rounding
// stays far below what the FP32 sums can see.  The sums over rows are FP32,
// scaled by e^{-m}; each exponent difference is formed in FP64 and then
// rounded to FP32 for the exp.
//
// Mapping on CDNA4: as for the RWKV-4 kernel.  A workgroup owns 64 channels
// (one per lane) of one prompt and walks its 64-row chunks; its NW waves split
// a chunk into NW blocks.  Each wave reduces its block from a zero state to
// (sums, largest exponent relative to the block's end, total decay of the
// block); the block states meet in LDS, each wave folds the carried state and
// the blocks before its own into its start state, the last wave hands the
// state after the chunk to the next one, and each wave replays its rows.  The
// next chunk's k, v and w are loaded while the current one computes.
#include "lrc_device.h"
#include "lrc_internal.h"

namespace lrc {
namespace {

constexpr int kTdWaves = 8;
constexpr int kTdDepth = 2;  // chunks whose rows are in flight ahead of the one computing

struct TdState {
    float aa, bb;  // num, den scaled by e^{-m}
    double m;      // current largest exponent
};

// Scale factors that line up a sum at exponent x with one at exponent y:
// exactly one of them is 1.
__device__ __forceinline__ void line_up(double x, double y, float& fx, float& fy) {
    const float d = (float)(x - y);
    const float e = fast_exp(-fabsf(d));
    fx = d >= 0.f ? 1.f : e;
    fy = d >= 0.f ? e : 1.f;
}

// One more row: decay the state by e^{w_t}, then add row (k_t, v_t).
__device__ __forceinline__ void push_row(TdState& s, float wt, float kt, float vt) {
    const double dec = s.m + (double)wt;
    float fs, fb;
    line_up(dec, (double)kt, fs, fb);
    s.aa = fmaf(fs, s.aa, fb * vt);
    s.bb = fmaf(fs, s.bb, fb);
    s.m = dec >= (double)kt ? dec : (double)kt;
}

// Output of row t from the state before it and the bonus exponent u + k_t.
__device__ __forceinline__ float out_row(const TdState& s, float uc, float kt, float vt) {
    float fs, fb;
    line_up(s.m, (double)(uc + kt), fs, fb);
    return fmaf(fs, s.aa, fb * vt) * __builtin_amdgcn_rcpf(fmaf(fs, s.bb, fb));
}

// A block of rows reduced from a zero state: sums scaled by e^{-zm}, zm the
// largest exponent at the block's end, zd the block's total decay.
struct TdBlock {
    float aa, bb;
    double zm, zd;
};

// s <- (s decayed by the block) + z.
__device__ __forceinline__ void absorb(TdState& s, const TdBlock& z) {
    const double dec = s.m + z.zd;
    float fs, fz;
    line_up(dec, z.zm, fs, fz);
    s.aa = fmaf(fs, s.aa, fz * z.aa);
    s.bb = fmaf(fs, s.bb, fz * z.bb);
    s.m = dec >= z.zm ? dec : z.zm;
}

// Rows 0 .. nb-1 of a block from a zero state.  Row i's exponent at the
// block's end is k_i plus the decays of rows i+1 .. nb-1.
template <int R>
__device__ __forceinline__ TdBlock reduce_block(const float (&kb)[R], const float (&vb)[R], const float (&wb)[R],
                                                int nb) {
    double ex[R];
    double tail = 0.0;  // decays of the rows after row i within the block
    double best = -1e300;
#pragma unroll
    for (int i = R - 1; i >= 0; --i) {
        ex[i] = (double)kb[i] + tail;
        if (i < nb) {
            best = ex[i] > best ? ex[i] : best;
            tail += (double)wb[i];
        }
    }
    float aa = 0.f, bb = 0.f;
#pragma unroll
    for (int i = 0; i < R; ++i)
        if (i < nb) {
            const float e = fast_exp((float)(ex[i] - best));
            aa = fmaf(e, vb[i], aa);
            bb = bb + e;
        }
    return TdBlock{aa, bb, best, tail};
}

template <int NW, int DEPTH, bool FULL>
__global__ __launch_bounds__(NW * 64) void wkv_tdecay_kernel(const float* __restrict__ k, const float* __restrict__ v,
                                                            const float* __restrict__ w, const float* __restrict__ u,
                                                            float* __restrict__ wkv, float* num, float* den, float* mx,
                                                            Batch bt, int C) {
    constexpr int R = 64 / NW;  // rows per wave and chunk
    __shared__ float2 zs[2][NW][64];   // block sums of a chunk
    __shared__ double2 zx[2][NW][64];  // block (largest exponent, decay)
    __shared__ float2 cs[2][64];       // state after a chunk, from the last wave
    __shared__ double cm[2][64];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = blockIdx.x * 64 + lane;
    const bool valid = FULL || c < C;
    const int cl = valid ? c : C - 1;  // lanes past C compute a copy of the last channel and store nothing
    {   // the longest prompts come first in the grid; their waves get issue priority
        const int q4 = (4 * blockIdx.y) / gridDim.y;
        if (q4 == 0) __builtin_amdgcn_s_setprio(3);
        else if (q4 == 1) __builtin_amdgcn_s_setprio(2);
        else if (q4 == 2) __builtin_amdgcn_s_setprio(1);
    }
    const int p = batch_prompt(bt, blockIdx.y);
    const long row0 = batch_row0(bt, p);
    const int L = batch_len(bt, p);
    const long sidx = (long)p * C + cl;
    const float uc = u[cl];
    TdState carry{num[sidx], den[sidx], (double)mx[sidx]};
    // Rows go through buffer resources based at the workgroup's first channel
    // and the wave's first row: row offsets are uniform (scalar offset), the
    // channel offset is the same for every row, so no address is formed per
    // access.  R rows x C channels of a resource stay below 2^31 bytes.
    const uint32_t lane_off = (uint32_t)(cl - blockIdx.x * 64) * 4;
    const float* k0 = k + row0 * C + blockIdx.x * 64;
    const float* v0 = v + row0 * C + blockIdx.x * 64;
    const float* w0 = w + row0 * C + blockIdx.x * 64;

    float kb_[DEPTH + 1][R], vb_[DEPTH + 1][R], wb_[DEPTH + 1][R];  // ring of row buffers
    // Loads are issued unconditionally (rows past the prompt re-read its last
    // row), so that only the chunk about to be used is waited for; k, v, w and
    // the output are touched once, so their accesses are nontemporal.
    auto fetch = [&](int c0, float (&kb)[R], float (&vb)[R], float (&wb)[R]) {
        const int r0 = min(c0 + R * wv, L - 1);
        const auto krs = buffer_rsrc(k0 + (long)r0 * C, (uint32_t)R * C * 4);
        const auto vrs = buffer_rsrc(v0 + (long)r0 * C, (uint32_t)R * C * 4);
        const auto wrs = buffer_rsrc(w0 + (long)r0 * C, (uint32_t)R * C * 4);
        const int last = L - 1 - r0;
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int soff = min(i, last) * C * 4;
            kb[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(krs, lane_off, soff, kNontemporal));
            vb[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(vrs, lane_off, soff, kNontemporal));
            wb[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(wrs, lane_off, soff, kNontemporal));
        }
    };
    int buf = 0;
    auto chunk = [&](int c0, const float (&kb)[R], const float (&vb)[R], const float (&wb)[R]) {
        const int S = min(64, L - c0);
        const int nb = min(R, max(0, S - R * wv));  // rows of this wave's block
        if (nb > 0) {
            const TdBlock z = nb == R ? reduce_block<R>(kb, vb, wb, R) : reduce_block<R>(kb, vb, wb, nb);
            zs[buf][wv][lane] = make_float2(z.aa, z.bb);
            zx[buf][wv][lane] = make_double2(z.zm, z.zd);
        }
        __syncthreads();
        if (c0 > 0) {
            const float2 s2 = cs[buf ^ 1][lane];
            carry = TdState{s2.x, s2.y, cm[buf ^ 1][lane]};
        }
        TdState s = carry;
        const int jn = min(wv, (S + R - 1) / R);  // non-empty blocks before this wave's
#pragma unroll
        for (int j = 0; j < NW - 1; ++j)
            if (j < jn) {
                const float2 a = zs[buf][j][lane];
                const double2 x = zx[buf][j][lane];
                absorb(s, TdBlock{a.x, a.y, x.x, x.y});
            }
        if (wv == NW - 1) {
            TdState e = s;
            if (nb > 0) {
                const float2 a = zs[buf][NW - 1][lane];
                const double2 x = zx[buf][NW - 1][lane];
                absorb(e, TdBlock{a.x, a.y, x.x, x.y});
            }
            cs[buf][lane] = make_float2(e.aa, e.bb);
            cm[buf][lane] = e.m;
            carry = e;
        }
        buf ^= 1;
        // lanes past C store at an offset past the resource's end: dropped
        const auto ors = buffer_rsrc(wkv + (row0 + c0 + R * wv) * C + blockIdx.x * 64, (uint32_t)R * C * 4);
        const uint32_t st_off = valid ? lane_off : 0x80000000u;
#pragma unroll
        for (int i = 0; i < R; ++i)
            if (i < nb) {
                const float o = out_row(s, uc, kb[i], vb[i]);
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o), ors, st_off, i * C * 4, kNontemporal);
                if (i + 1 < nb) push_row(s, wb[i], kb[i], vb[i]);
            }
    };

    if (L > 0) {
#pragma unroll
        for (int s = 0; s < DEPTH; ++s) fetch(64 * s, kb_[s], vb_[s], wb_[s]);
    }
    for (int c0 = 0; c0 < L; c0 += 64 * (DEPTH + 1)) {
#pragma unroll
        for (int s = 0; s <= DEPTH; ++s) {
            const int cc = c0 + 64 * s;
            if (cc >= L) break;
            const int nx = (s + DEPTH) % (DEPTH + 1);
            fetch(cc + 64 * DEPTH, kb_[nx], vb_[nx], wb_[nx]);
            chunk(cc, kb_[s], vb_[s], wb_[s]);
        }
    }
    // the last wave holds the state after the prompt (or the incoming one);
    // the sums are rescaled to the FP32 maximum that is stored with them
    if (wv == NW - 1 && valid) {
        const float mf = (float)carry.m;
        const float f = carry.m > -1e30 ? fast_exp((float)(carry.m - (double)mf)) : 1.f;
        num[sidx] = carry.aa * f;
        den[sidx] = carry.bb * f;
        mx[sidx] = mf;
    }
}

}  // namespace

hipError_t launch_wkv_tdecay(const float* k, const float* v, const float* w, const float* u, float* wkv, float* num,
                             float* den, float* mx, const Batch& bt, int C, hipStream_t st) {
    const dim3 grid((unsigned)((C + 63) / 64), (unsigned)bt.P);
    if (C % 64 == 0)
        hipLaunchKernelGGL((wkv_tdecay_kernel<kTdWaves, kTdDepth, true>), grid, dim3(kTdWaves * 64), 0, st, k, v, w,
                           u, wkv, num, den, mx, bt, C);
    else
        hipLaunchKernelGGL((wkv_tdecay_kernel<kTdWaves, kTdDepth, false>), grid, dim3(kTdWaves * 64), 0, st, k, v, w,
                           u, wkv, num, den, mx, bt, C);
    return hipGetLastError();
}

}  // namespace lrc

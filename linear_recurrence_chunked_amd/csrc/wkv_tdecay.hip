// WKV with a token-dependent decay, FP32 sums with FP64 exponents, on gfx950.
//
// Source: "perf(rwkv): prefill text prompts in multi-token chunks", Notes For
// Future Readers -- RWKV generations with a per-token decay call for a
// different chunk form from the RWKV-4 one.  The pages give no formula for those
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
// (one per lane) of one prompt and walks its 64-row chunks with NW row waves,
// which split a chunk into NW blocks, and one fold wave.  In the step of
// chunk n each row wave reduces its block of chunk n+1 from a zero state to
// (sums, largest exponent relative to the block's end, total decay of the
// block) and signals it, then waits for its start state of chunk n and
// replays its rows.  The fold wave waits for a chunk's block states, folds
// them in row order into the carried state, writing each block's start state
// to LDS, and publishes.  The waves meet through LDS counters, not workgroup
// barriers, so the chain from chunk to chunk runs through the fold alone.
// Block and start states are double-buffered by chunk parity; a row wave
// cannot reduce chunk n+2 before chunk n is folded, which makes a count of
// reductions per parity exact.  k, v and w are fetched two chunks ahead.
#include "lrc_device.h"
#include "lrc_internal.h"

namespace lrc {
namespace {

constexpr int kTdWaves = 8;  // row waves per workgroup (blocks of 8 rows)

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

// NW row waves (a block of R = 64/NW rows each) and one fold wave.
template <int NW, bool FULL>
__global__ __launch_bounds__((NW + 1) * 64) void wkv_tdecay_kernel(const float* __restrict__ k,
                                                                  const float* __restrict__ v,
                                                                  const float* __restrict__ w,
                                                                  const float* __restrict__ u,
                                                                  float* __restrict__ wkv, float* num, float* den,
                                                                  float* mx, Batch bt, int C, unsigned* timeouts) {
    constexpr int R = 64 / NW;         // rows per row wave and chunk
    __shared__ float2 zs[2][NW][64];   // block sums of a chunk, by chunk parity
    __shared__ double2 zx[2][NW][64];  // block (largest exponent, decay)
    __shared__ float2 ps[2][NW][64];   // start state of every block, by chunk parity
    __shared__ double pm[2][NW][64];
    __shared__ int red_cnt[2];         // block reductions done, of even and of odd chunks
    __shared__ int ps_seq;             // chunks whose start states are published
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = blockIdx.x * 64 + lane;
    const bool valid = FULL || c < C;
    const int cl = valid ? c : C - 1;  // lanes past C compute a copy of the last channel and store nothing
    if (threadIdx.x == 0) {
        red_cnt[0] = red_cnt[1] = 0;
        ps_seq = 0;
    }
    __syncthreads();
    const int p = batch_prompt(bt, blockIdx.y);
    const long row0 = batch_row0(bt, p);
    const int L = batch_len(bt, p);
    if (L == 0) return;  // the state stays as it is
    const int nc = (L + 63) / 64;
    const long sidx = (long)p * C + cl;
    const float uc = u[cl];

    if (wv == NW) {
        // ---- fold wave: the chain from chunk to chunk.  Waits for the NW block
        // states of chunk n, folds them in row order into the carried state,
        // publishing each block's start state, and keeps the state after it.
        __builtin_amdgcn_s_setprio(3);
        TdState s{num[sidx], den[sidx], (double)mx[sidx]};
        for (int n = 0; n < nc; ++n) {
            const int S = min(64, L - 64 * n), nblk = (S + R - 1) / R, b = n & 1;
            // No row wave reduces chunk n+2 before chunk n's start states are
            // out, so the count of this parity covers chunks up to n only.
            lds_wait_at_least(&red_cnt[b], NW * (n / 2 + 1), timeouts);
#pragma unroll
            for (int j = 0; j < NW; ++j) {
                ps[b][j][lane] = make_float2(s.aa, s.bb);
                pm[b][j][lane] = s.m;
                if (j < nblk) {
                    const float2 a = zs[b][j][lane];
                    const double2 x = zx[b][j][lane];
                    absorb(s, TdBlock{a.x, a.y, x.x, x.y});
                }
            }
            if (lane == 0) __hip_atomic_store(&ps_seq, n + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        // the sums are rescaled to the FP32 maximum that is stored with them
        if (valid) {
            const float mf = (float)s.m;
            const float f = s.m > -1e30 ? fast_exp((float)(s.m - (double)mf)) : 1.f;
            num[sidx] = s.aa * f;
            den[sidx] = s.bb * f;
            mx[sidx] = mf;
        }
        return;
    }

    // ---- row waves.  In the step of chunk n a row wave reduces its block of
    // chunk n+1, then waits for its start state of chunk n and replays its
    // rows.  The longest prompts come first in the grid; their row waves get
    // issue priority.
    {
        const int q4 = (4 * blockIdx.y) / gridDim.y;
        if (q4 == 0) __builtin_amdgcn_s_setprio(2);
        else if (q4 == 1) __builtin_amdgcn_s_setprio(1);
    }
    // Rows go through buffer resources based at the workgroup's first channel
    // and the wave's first row: row offsets are uniform (scalar offset), the
    // channel offset is the same for every row, so no address is formed per
    // access.  R rows x C channels of a resource stay below 2^31 bytes.  Loads
    // are issued unconditionally (rows past the prompt re-read its last row),
    // so that only the chunk about to be used is waited for; k, v, w and the
    // output are touched once, so their accesses are nontemporal.
    const uint32_t lane_off = (uint32_t)(cl - blockIdx.x * 64) * 4;
    const float* k0 = k + row0 * C + blockIdx.x * 64;
    const float* v0 = v + row0 * C + blockIdx.x * 64;
    const float* w0 = w + row0 * C + blockIdx.x * 64;
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
    auto reduce = [&](int n, const float (&kb)[R], const float (&vb)[R], const float (&wb)[R]) {
        const int S = min(64, L - 64 * n);
        const int nb = min(R, max(0, S - R * wv));
        if (nb > 0) {
            const TdBlock z = nb == R ? reduce_block<R>(kb, vb, wb, R) : reduce_block<R>(kb, vb, wb, nb);
            zs[n & 1][wv][lane] = make_float2(z.aa, z.bb);
            zx[n & 1][wv][lane] = make_double2(z.zm, z.zd);
        }
        if (lane == 0) __hip_atomic_fetch_add(&red_cnt[n & 1], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    auto replay = [&](int n, const float (&kb)[R], const float (&vb)[R], const float (&wb)[R]) {
        const int c0 = 64 * n, S = min(64, L - c0);
        const int nb = min(R, max(0, S - R * wv));
        lds_wait_at_least(&ps_seq, n + 1, timeouts);
        const float2 st = ps[n & 1][wv][lane];
        TdState s{st.x, st.y, pm[n & 1][wv][lane]};
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

    // A ring of three row buffers: chunk n (replayed), n+1 (reduced), n+2 (in flight).
    float kb0[R], vb0[R], wb0[R], kb1[R], vb1[R], wb1[R], kb2[R], vb2[R], wb2[R];
    fetch(0, kb0, vb0, wb0);
    fetch(64, kb1, vb1, wb1);
    reduce(0, kb0, vb0, wb0);
    for (int n = 0; n < nc; n += 3) {
        fetch(64 * (n + 2), kb2, vb2, wb2);
        if (n + 1 < nc) reduce(n + 1, kb1, vb1, wb1);
        replay(n, kb0, vb0, wb0);
        if (n + 1 >= nc) break;
        fetch(64 * (n + 3), kb0, vb0, wb0);
        if (n + 2 < nc) reduce(n + 2, kb2, vb2, wb2);
        replay(n + 1, kb1, vb1, wb1);
        if (n + 2 >= nc) break;
        fetch(64 * (n + 4), kb1, vb1, wb1);
        if (n + 3 < nc) reduce(n + 3, kb0, vb0, wb0);
        replay(n + 2, kb2, vb2, wb2);
    }
}

}  // namespace

hipError_t launch_wkv_tdecay(const float* k, const float* v, const float* w, const float* u, float* wkv, float* num,
                             float* den, float* mx, const Batch& bt, int C, hipStream_t st) {
    unsigned* timeouts = wait_timeouts_counter();
    if (!timeouts) return hipErrorInvalidSymbol;
    const dim3 grid((unsigned)((C + 63) / 64), (unsigned)bt.P);
    if (C % 64 == 0)
        hipLaunchKernelGGL((wkv_tdecay_kernel<kTdWaves, true>), grid, dim3((kTdWaves + 1) * 64), 0, st, k, v, w, u,
                           wkv, num, den, mx, bt, C, timeouts);
    else
        hipLaunchKernelGGL((wkv_tdecay_kernel<kTdWaves, false>), grid, dim3((kTdWaves + 1) * 64), 0, st, k, v, w,
                           u, wkv, num, den, mx, bt, C, timeouts);
    return hipGetLastError();
}

}  // namespace lrc

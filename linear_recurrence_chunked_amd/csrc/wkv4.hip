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
// Exponent bookkeeping.  Because w does not depend on the row, the largest
// exponent among the state and the rows before row t is always of the form
// m + n w: m is the incoming max_0 or the key k_i that last took the lead,
// and n the number of rows since (t for the state, t-1-i for row i).  A
// running state carries (m, n) and forms every exponent directly as
// fma(n, w, m), exactly the page's max_0 + t w and k_i + (t-1-i) w, so no
// rounding accumulates in the running maximum; the sums over earlier rows are
// carried as (num, den) scaled by e^{-(m + n w)}.  Of the two exp factors
// that line up two such sums, exactly one is 1, so each step costs one exp.
//
// Mapping on CDNA4.  The recurrence is linear in (num, den) with the constant
// factor e^w per row, so a block of rows reduces, from a zero state, to one
// state of the same form, and "decay a state by n rows, then add a block" is
// again one exp.  A workgroup owns 64 channels (one per lane, so every row's
// loads and stores are one contiguous 256-byte run) of one prompt and walks
// the prompt's 64-row chunks with NW row waves (blocks of 64/NW rows) and one
// fold wave:
//   1. in the step of chunk n, each row wave reduces its block of chunk n+1
//      from a zero state (the block's exponents k_i + (n-1-i) w are
//      independent of each other, so their maximum and the sums relative to
//      it are plain reductions over registers) and signals it;
//   2. the fold wave waits for the NW block states of chunk n, folds them in
//      row order into the carried state, writes each block's start state to
//      LDS as it goes, keeps the state after the chunk, and publishes;
//   3. each row wave waits for its start state of chunk n and replays its
//      rows (the larger of the running maximum and the bonus u + k_t, then the
//      push of the row into the state: two exps and one reciprocal per row;
//      the push exponent is the output's plus w + u).
// The waves meet through LDS counters, not workgroup barriers, so the chain
// from one chunk to the next runs through the fold alone: a row wave's
// replay of chunk n and reduction of chunk n+2 are off it.  Block states and
// start states are double-buffered by chunk parity; a row wave cannot reduce
// chunk n+2 before chunk n is folded, which is what makes a count of
// reductions per parity exact.  Rows are fetched two chunks ahead.
// Exponents are kept in base 2 (k, w, u and the maximum scaled by log2 e,
// the maximum scaled back on the way out), so each exponential is a bare
// v_exp_f32.
#include "lrc_device.h"
#include "lrc_internal.h"

namespace lrc {
namespace {

constexpr int kWkvWaves = 8;  // row waves per workgroup (blocks of 8 rows)

// Exponents are held in base 2 (k, w, u and the running maximum scaled by
// log2 e once), so that every exponential is one v_exp_f32 with no scaling.
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
__device__ __forceinline__ float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }

struct WkvState {
    float aa, bb;  // num, den scaled by 2^{-(m + n w)}
    float m, n;    // current largest exponent (base 2) is m + n w
};

// Output of row t from the state before it and the bonus exponent u + k_t;
// then, if PUSH, the state after row t (decayed by one row, row t added).  The
// push exponent (m + (n+1) w) - k_t is the output's (m + n w) - (u + k_t)
// plus w + u (wu).
template <bool PUSH>
__device__ __forceinline__ float step_row(WkvState& s, float wc, float uc, float wu, float kt, float vt) {
    const float d = fmaf(s.n, wc, s.m) - (uc + kt);
    const float e = exp2_(-fabsf(d));
    const float fs = d >= 0.f ? 1.f : e;
    const float fb = d >= 0.f ? e : 1.f;
    const float o = fmaf(fs, s.aa, fb * vt) * __builtin_amdgcn_rcpf(fmaf(fs, s.bb, fb));
    if (PUSH) {
        const float dp = d + wu;
        const float ep = exp2_(-fabsf(dp));
        const bool lead = dp >= 0.f;  // the decayed maximum stays in the lead
        const float ps = lead ? 1.f : ep, pb = lead ? ep : 1.f;
        s.aa = fmaf(ps, s.aa, pb * vt);
        s.bb = fmaf(ps, s.bb, pb);
        s.n = lead ? s.n + 1.f : 0.f;
        s.m = lead ? s.m : kt;
    }
    return o;
}

// s <- (s decayed by len rows) + z, where z is a block reduced from a zero state.
__device__ __forceinline__ void absorb(WkvState& s, const float4& z, float len, float wc) {
    const float nl = s.n + len;
    const float d = fmaf(nl, wc, s.m) - fmaf(z.w, wc, z.z);
    const float e = exp2_(-fabsf(d));
    const bool lead = d >= 0.f;
    s.aa = fmaf(e, lead ? z.x : s.aa, lead ? s.aa : z.x);
    s.bb = fmaf(e, lead ? z.y : s.bb, lead ? s.bb : z.y);
    s.n = lead ? nl : z.w;
    s.m = lead ? s.m : z.z;
}

// Rows 0 .. nb-1 of a block reduced from a zero state, as (aa, bb, m, n).
template <int R>
__device__ __forceinline__ float4 reduce_block(const float (&kb)[R], const float (&vb)[R], int nb, float wc) {
    float ex[R];
    float best = fmaf((float)(nb - 1), wc, kb[0]), zm = kb[0], zn = (float)(nb - 1);
#pragma unroll
    for (int i = 1; i < R; ++i) {
        ex[i] = fmaf((float)(nb - 1 - i), wc, kb[i]);
        const bool gt = i < nb && ex[i] > best;
        best = gt ? ex[i] : best;
        zm = gt ? kb[i] : zm;
        zn = gt ? (float)(nb - 1 - i) : zn;
    }
    ex[0] = fmaf((float)(nb - 1), wc, kb[0]);
    float aa = 0.f, bb = 0.f;
#pragma unroll
    for (int i = 0; i < R; ++i)
        if (i < nb) {
            const float e = exp2_(ex[i] - best);
            aa = fmaf(e, vb[i], aa);
            bb = bb + e;
        }
    return make_float4(aa, bb, zm, zn);
}

// NW row waves (a block of R = 64/NW rows each) and one fold wave.
template <int NW, bool FULL>
__global__ __launch_bounds__((NW + 1) * 64) void wkv4_kernel(const float* __restrict__ k, const float* __restrict__ v,
                                                            const float* __restrict__ w, const float* __restrict__ u,
                                                            float* __restrict__ wkv, float* num, float* den, float* mx,
                                                            Batch bt, int C, unsigned* timeouts) {
    constexpr int R = 64 / NW;        // rows per row wave and chunk
    __shared__ float4 zs[2][NW][64];  // block states of a chunk, by chunk parity
    __shared__ float4 ps[2][NW][64];  // start state of every block, by chunk parity
    __shared__ int red_cnt[2];        // block reductions done, of even and of odd chunks
    __shared__ int ps_seq;            // chunks whose start states are published
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
    const float wc = w[cl] * kLog2e, uc = u[cl] * kLog2e, wu = wc + uc;

    if (wv == NW) {
        // ---- fold wave: the chain from chunk to chunk.  Waits for the NW block
        // states of chunk n, folds them in row order into the carried state,
        // publishing each block's start state, and keeps the state after it.
        __builtin_amdgcn_s_setprio(3);
        WkvState s{num[sidx], den[sidx], mx[sidx] * kLog2e, 0.f};
        for (int n = 0; n < nc; ++n) {
            const int S = min(64, L - 64 * n), nblk = (S + R - 1) / R, b = n & 1;
            // No row wave reduces chunk n+2 before chunk n's start states are
            // out, so the count of this parity covers chunks up to n only.
            lds_wait_at_least(&red_cnt[b], NW * (n / 2 + 1), timeouts);
#pragma unroll
            for (int j = 0; j < NW; ++j) {
                ps[b][j][lane] = make_float4(s.aa, s.bb, s.m, s.n);
                float4 z = zs[b][j][lane];
                asm volatile("" : "+v"(z.x), "+v"(z.y), "+v"(z.z), "+v"(z.w));
                if (j < nblk) absorb(s, z, (float)min(R, S - R * j), wc);
            }
            if (lane == 0) __hip_atomic_store(&ps_seq, n + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        if (valid) {
            num[sidx] = s.aa;
            den[sidx] = s.bb;
            mx[sidx] = fmaf(s.n, wc, s.m) * kLn2;
        }
        return;
    }

    // ---- row waves.  In the step of chunk n a row wave reduces its block of
    // chunk n+1 (so the fold wave never waits on a replay), then waits for its
    // start state of chunk n and replays its rows.  The longest prompts come
    // first in the grid; their row waves get issue priority.
    {
        const int q4 = (4 * blockIdx.y) / gridDim.y;
        if (q4 == 0) __builtin_amdgcn_s_setprio(2);
        else if (q4 == 1) __builtin_amdgcn_s_setprio(1);
    }
    // Rows through buffer resources based at the wave's first row (uniform
    // row offsets in the scalar offset, a fixed channel offset per lane).
    // Loads are issued unconditionally (rows past the prompt re-read its last
    // row) so that the compiler can count them.  R rows x C channels of a
    // resource stay below 2^31 bytes.
    const uint32_t lane_off = (uint32_t)(cl - blockIdx.x * 64) * 4;
    const float* k0 = k + row0 * C + blockIdx.x * 64;
    const float* v0 = v + row0 * C + blockIdx.x * 64;
    auto fetch = [&](int c0, float (&kb)[R], float (&vb)[R]) {
        const int r0 = min(c0 + R * wv, L - 1);
        const auto krs = buffer_rsrc(k0 + (long)r0 * C, (uint32_t)R * C * 4);
        const auto vrs = buffer_rsrc(v0 + (long)r0 * C, (uint32_t)R * C * 4);
        const int last = L - 1 - r0;
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int soff = min(i, last) * C * 4;
            kb[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(krs, lane_off, soff, kNontemporal));
            vb[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(vrs, lane_off, soff, kNontemporal));
        }
    };
    auto reduce = [&](int n, const float (&kr)[R], const float (&vb)[R]) {
        float kb[R];  // keys in base 2
#pragma unroll
        for (int i = 0; i < R; ++i) kb[i] = kr[i] * kLog2e;
        const int S = min(64, L - 64 * n);
        const int nb = min(R, max(0, S - R * wv));
        if (nb == R)
            zs[n & 1][wv][lane] = reduce_block<R>(kb, vb, R, wc);  // constant row count: no per-row checks
        else if (nb > 0)
            zs[n & 1][wv][lane] = reduce_block<R>(kb, vb, nb, wc);
        if (lane == 0) __hip_atomic_fetch_add(&red_cnt[n & 1], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    auto replay = [&](int n, const float (&kr)[R], const float (&vb)[R]) {
        float kb[R];  // keys in base 2
#pragma unroll
        for (int i = 0; i < R; ++i) kb[i] = kr[i] * kLog2e;
        const int c0 = 64 * n, S = min(64, L - c0);
        const int nb = min(R, max(0, S - R * wv));
        lds_wait_at_least(&ps_seq, n + 1, timeouts);
        const float4 st = ps[n & 1][wv][lane];
        WkvState s{st.x, st.y, st.z, st.w};
        // lanes past C store at an offset past the resource's end: dropped
        const auto ors = buffer_rsrc(wkv + (row0 + c0 + R * wv) * C + blockIdx.x * 64, (uint32_t)R * C * 4);
        const uint32_t st_off = valid ? lane_off : 0x80000000u;
        if (nb == R) {  // full block: straight-line code
#pragma unroll
            for (int i = 0; i < R; ++i) {
                const float o = i + 1 < R ? step_row<true>(s, wc, uc, wu, kb[i], vb[i])
                                          : step_row<false>(s, wc, uc, wu, kb[i], vb[i]);
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o), ors, st_off, i * C * 4, kNontemporal);
            }
        } else if (nb > 0) {
#pragma unroll
            for (int i = 0; i < R; ++i)
                if (i < nb) {
                    const float o = step_row<true>(s, wc, uc, wu, kb[i], vb[i]);
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o), ors, st_off, i * C * 4, kNontemporal);
                }
        }
    };

    // A ring of three row buffers: chunk n (replayed), n+1 (reduced), n+2 (in flight).
    float kb0[R], vb0[R], kb1[R], vb1[R], kb2[R], vb2[R];
    fetch(0, kb0, vb0);
    fetch(64, kb1, vb1);
    reduce(0, kb0, vb0);
    for (int n = 0; n < nc; n += 3) {
        fetch(64 * (n + 2), kb2, vb2);
        if (n + 1 < nc) reduce(n + 1, kb1, vb1);
        replay(n, kb0, vb0);
        if (n + 1 >= nc) break;
        fetch(64 * (n + 3), kb0, vb0);
        if (n + 2 < nc) reduce(n + 2, kb2, vb2);
        replay(n + 1, kb1, vb1);
        if (n + 2 >= nc) break;
        fetch(64 * (n + 4), kb1, vb1);
        if (n + 3 < nc) reduce(n + 3, kb0, vb0);
        replay(n + 2, kb2, vb2);
    }
}

}  // namespace

hipError_t launch_wkv4(const float* k, const float* v, const float* w, const float* u, float* wkv, float* num,
                       float* den, float* mx, const Batch& bt, int C, hipStream_t st) {
    unsigned* timeouts = wait_timeouts_counter();
    if (!timeouts) return hipErrorInvalidSymbol;
    const dim3 grid((unsigned)((C + 63) / 64), (unsigned)bt.P);
    if (C % 64 == 0)
        hipLaunchKernelGGL((wkv4_kernel<kWkvWaves, true>), grid, dim3((kWkvWaves + 1) * 64), 0, st, k, v, w, u, wkv,
                           num, den, mx, bt, C, timeouts);
    else
        hipLaunchKernelGGL((wkv4_kernel<kWkvWaves, false>), grid, dim3((kWkvWaves + 1) * 64), 0, st, k, v, w, u, wkv,
                           num, den, mx, bt, C, timeouts);
    return hipGetLastError();
}

}  // namespace lrc

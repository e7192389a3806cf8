// K3, bf16-input path, chunk-parallel form: Gated DeltaNet for launches with
// few prompts, where one workgroup per (prompt, value head) walking the
// chunks one after the other would leave most compute units idle.
//
// Source: "perf(qwen3_5): prefill text prompts in multi-token chunks",
// Implementation.  For a chunk of S <= 64 rows with gamma the chunk-local
// inclusive cumulative sum of g, Gamma = e^gamma and T = (I + A)^-1,
//   U   = T (diag(beta) V - diag(beta Gamma) K S_0)
//   O   = diag(Gamma) Q S_0 + (e^{gamma_t - gamma_i} q_t.k_i)_{i <= t} U
//   S_S = e^{gamma_S} S_0 + (K * e^{min(gamma_S - gamma, 0)})^T U.
// Everything but S_0 can be formed for every chunk at once: U splits as
//   U = U' - W S_0,  U' = T diag(beta) V,  W = T diag(beta Gamma) K,
// the same product regrouped.  Two kernels therefore run one after the other
// on the stream:
//  * prep (grid: every chunk x every value head): stages the chunk's K, Q, V,
//    forms A = beta_i e^{gamma_i - gamma_j} k_i.k_j (j < i) and inverts I + A
//    on the 64-row padding (8x8 Neumann blocks, then 2x2 block levels, as in
//    tri_inverse.h), then W, U', the masked decayed Q K^T (P), K^T and the
//    per-row Gamma and state-update decay, into one block of the caller's
//    workspace per (chunk, value head);
//  * state (grid: value heads x column slices x prompts): walks a prompt's
//    chunks with its 32-column slices of the [dk x dv] state in matrix-core
//    accumulators and runs only what needs the state: W S_0, Q S_0,
//    U = U' - W S_0, O = diag(Gamma) Q S_0 + P U and the state update.  Loader
//    waves copy the next chunk's W, Q, K^T and P into LDS while the state
//    waves work on the current one; one workgroup barrier per chunk.
// Precision: as the fused path, FP32 accumulation with each FP32 operand of
// a product rounded to bf16 once: T diag(beta Gamma) and T diag(beta) (T in
// FP32 from the inverse, whose tile products run as hi/lo bf16 pairs), W and
// P as stored, S_0 and U on their way into the matrix cores.  U' stays FP32.
#include <algorithm>
#include <cstddef>

#include "gdn_frag.h"
#include "lrc_device.h"
#include "lrc_internal.h"
#include "tri_inverse.h"

namespace lrc {

namespace {

constexpr int kCpPrepWaves = 4;
constexpr int kCpLoaders = 2;  // loader waves of the state kernel

// One (chunk, value head) block of the workspace: W [64][DK] bf16, K^T [DK][64]
// bf16, P [64][64] bf16, U' [64][DV] f32, Gamma [64] f32, decay [64] f32.  The
// rows of W, K^T and P are stored k-permuted along their contraction index
// (kperm), so that the state kernel reads each operand fragment as one
// 16-byte run.
template <int DK, int DV>
struct CpBlock {
    static constexpr size_t W = 0;
    static constexpr size_t KT = W + 64 * DK * 2;
    static constexpr size_t P = KT + DK * 64 * 2;
    static constexpr size_t U = P + 64 * 64 * 2;
    static constexpr size_t GAM = U + 64 * DV * 4;
    static constexpr size_t DEC = GAM + 64 * 4;
    static constexpr size_t BYTES = (DEC + 64 * 4 + 255) / 256 * 256;
};

// Chunk numbering of a launch: prompt p (batch index) owns the chunks
// [off[p], off[p + 1]).
struct CpChunks {
    int total;
    int off[LRC_MAX_PROMPTS + 1];
};

// About 78 KiB at dk = dv = 128, so that two workgroups share a compute unit.
// Q never enters LDS (its fragments are read from memory); V is staged
// transposed; T diag(beta Gamma) and T diag(beta) take the space of the K rows,
// which are dead once A and K^T are formed.
template <int DK, int DV>
struct CpPrepSmem {
    static constexpr int LDK = DK + 16;  // K rows: 16-byte fragment reads free of bank conflicts
    static constexpr int R1 = 64 * LDK > 2 * 64 * L64 ? 64 * LDK : 2 * 64 * L64;
    __bf16 KT_[R1];       // K rows, then T diag(beta Gamma) and T diag(beta)
    __bf16 KT[DK * L64];  // K^T
    __bf16 VT[DV * L64];  // V^T
    float M[64 * kTriLd];  // A, then T
    float scratch[kTriScratch];
    float gam[64], Gam[64], beta[64];
    __device__ __bf16* K() { return KT_; }
    __device__ __bf16* Tg() { return KT_; }             // T diag(beta Gamma)
    __device__ __bf16* Tb() { return KT_ + 64 * L64; }  // T diag(beta)
};

// Rows r = 0 .. 63 of a [64][D] bf16 tile in LDS (row stride ld) into its
// transpose [D][L64]: blocks of 4 rows x 8 columns, by byte permutes.
// The destination's columns (rows of the source) are stored k-permuted (kperm).
__device__ __forceinline__ void transpose64(const __bf16* src, int ld, __bf16* dst, int D, int t0, int nt) {
    for (int b = t0; b < 2 * D; b += nt) {
        const int nn = b & 15, m = b >> 4;  // rows 4nn .. 4nn+3, columns 8m .. 8m+7
        uint4 rw[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) rw[a] = *reinterpret_cast<const uint4*>(&src[(4 * nn + a) * ld + 8 * m]);
        const uint32_t d0[4] = {rw[0].x, rw[0].y, rw[0].z, rw[0].w};
        const uint32_t d1[4] = {rw[1].x, rw[1].y, rw[1].z, rw[1].w};
        const uint32_t d2[4] = {rw[2].x, rw[2].y, rw[2].z, rw[2].w};
        const uint32_t d3[4] = {rw[3].x, rw[3].y, rw[3].z, rw[3].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;  // high or low halves of two dwords
            uint2 out;
            out.x = __builtin_amdgcn_perm(d1[e >> 1], d0[e >> 1], sel);
            out.y = __builtin_amdgcn_perm(d3[e >> 1], d2[e >> 1], sel);
            *reinterpret_cast<uint2*>(&dst[(8 * m + e) * L64 + kperm(4 * nn)]) = out;
        }
    }
}

// The prompt (batch index) and chunk within it of global chunk c.
__device__ __forceinline__ void cp_locate(const CpChunks& cm, int P, int c, int& p, int& j) {
    int lo = 0, hi = P;  // off[lo] <= c < off[lo + 1]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cm.off[mid] <= c) lo = mid;
        else hi = mid;
    }
    p = lo;
    j = c - cm.off[lo];
}

// ------------------------------------------------------------------ prep
template <int DK, int DV>
__global__ __launch_bounds__(64 * kCpPrepWaves, 2) void gdn_cp_prep_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ beta, const float* __restrict__ g, Batch bt, CpChunks cm, int Hk, int Hv,
    unsigned char* __restrict__ ws) {
    using Sm = CpPrepSmem<DK, DV>;
    using Blk = CpBlock<DK, DV>;
    constexpr int LDK = Sm::LDK;
    constexpr int NT = 64 * kCpPrepWaves;
    constexpr int KS = DK / 32;
    constexpr int NP = 3;  // tile pairs w, w + 4, w + 8 of the 10 below the diagonal
    extern __shared__ __align__(16) unsigned char smem_raw[];
    Sm& sm = *reinterpret_cast<Sm*>(smem_raw);

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // grid.x is the chunk count rounded up to a multiple of 8: workgroups go to the 8 XCDs
    // in launch order, so the value heads of one key head, which read the same K and Q
    // rows, run on one XCD and share its L2
    const int c = blockIdx.x, h = blockIdx.y, kh = h / (Hv / Hk);
    if (c >= cm.total) return;
    int tid_c = tid;
    asm volatile("" : "+v"(tid_c));
    const int lr = tid_c & 15, lg = (tid_c >> 4) & 3, lk = lg * 8, lq = lg * 4;
    int p, j;
    cp_locate(cm, bt.P, c, p, j);
    const long r0 = batch_row0(bt, p) + 64l * j;
    const int S = min(64, batch_len(bt, p) - 64 * j);
    unsigned char* blk = ws + ((long)c * Hv + h) * Blk::BYTES;

    // ---- stage K rows and V^T (rows past the chunk read as zero), g and beta; the Q
    //      fragments of this wave's tile pairs go to registers
    bf16x8 qf[KS][NP];
    {
        const uint32_t rowK = Hk * DK * 2, rowV = Hv * DV * 2;
        const auto krs = buffer_rsrc(k + (r0 * Hk + kh) * DK, (uint32_t)S * rowK);
        const auto qrs = buffer_rsrc(q + (r0 * Hk + kh) * DK, (uint32_t)S * rowK);
        const auto vrs = buffer_rsrc(v + (r0 * Hv + h) * DV, (uint32_t)S * rowV);
        // every load first, then the LDS stores: the loads are in flight together
        constexpr int NK = 8 * DK / NT, NV = 8 * DV / NT;
        static_assert(8 * DK % NT == 0 && 8 * DV % NT == 0, "whole 16-byte pieces per thread");
        u32x4 ka[NK], va[NV];
#pragma unroll
        for (int x = 0; x < NK; ++x) {
            const int e = tid + x * NT, r = e / (DK / 8), c8 = (e % (DK / 8)) * 8;
            ka[x] = __builtin_amdgcn_raw_buffer_load_b128(krs, (uint32_t)r * rowK + c8 * 2, 0, 0);
        }
#pragma unroll
        for (int x = 0; x < NV; ++x) {
            const int e = tid + x * NT, r = e / (DV / 8), c8 = (e % (DV / 8)) * 8;
            va[x] = __builtin_amdgcn_raw_buffer_load_b128(vrs, (uint32_t)r * rowV + c8 * 2, 0, 0);
        }
#pragma unroll
        for (int s8 = 0; s8 < KS; ++s8)
#pragma unroll
            for (int x = 0; x < NP; ++x) {
                int ti, tj;
                tile_pair(min(w + 4 * x, 9), ti, tj);
                qf[s8][x] = __builtin_bit_cast(
                    bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qrs, (uint32_t)(16 * ti + lr) * rowK + (32 * s8 + lk) * 2,
                                                                  0, 0));
            }
#pragma unroll
        for (int x = 0; x < NK; ++x) {
            const int e = tid + x * NT, r = e / (DK / 8), c8 = (e % (DK / 8)) * 8;
            *reinterpret_cast<u32x4*>(&sm.K()[r * LDK + c8]) = ka[x];
        }
#pragma unroll
        for (int x = 0; x < NV; ++x) {
            const int e = tid + x * NT, r = e / (DV / 8), c8 = (e % (DV / 8)) * 8;
            const bf16x8 vv = __builtin_bit_cast(bf16x8, va[x]);
#pragma unroll
            for (int z = 0; z < 8; ++z) sm.VT[(c8 + z) * L64 + kperm(r)] = vv[z];
        }
        if (w == kCpPrepWaves - 1) {
            const auto grs = buffer_rsrc(g + r0 * Hv + h, (uint32_t)S * Hv * 4);
            const auto brs = buffer_rsrc(beta + r0 * Hv + h, (uint32_t)S * Hv * 4);
            const float pg = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(grs, lane * Hv * 4, 0, 0));
            const float pb = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(brs, lane * Hv * 4, 0, 0));
            const float x = wave_prefix_sum(pg);  // gamma, inclusive; flat past the chunk
            const float Gx = fast_exp(x);
            const float gS = readlane_f(x, S - 1);  // the last cumulative sum
            const float dS = lane < S ? fast_exp(fminf(gS - x, 0.f)) : 0.f;
            sm.gam[lane] = x;
            sm.Gam[lane] = Gx;
            sm.beta[lane] = pb;
            reinterpret_cast<float*>(blk + Blk::GAM)[lane] = Gx;
            reinterpret_cast<float*>(blk + Blk::DEC)[lane] = dS;
        }
        for (int e = tid; e < 64 * kTriLd; e += NT) sm.M[e] = 0.f;  // above the diagonal stays zero
    }
    __syncthreads();

    // ---- A (FP32, into M); P (bf16, into the block); K^T
    {
        floatx4 kk[NP], qk[NP];
#pragma unroll
        for (int x = 0; x < NP; ++x) kk[x] = qk[x] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s8 = 0; s8 < KS; ++s8)
#pragma unroll
            for (int x = 0; x < NP; ++x) {
                int ti, tj;
                tile_pair(min(w + 4 * x, 9), ti, tj);
                const bf16x8 kj = frag(&sm.K()[(16 * tj + lr) * LDK + 32 * s8 + lk]);
                kk[x] = mfma(kj, frag(&sm.K()[(16 * ti + lr) * LDK + 32 * s8 + lk]), kk[x]);
                qk[x] = mfma(kj, qf[s8][x], qk[x]);
            }
        __bf16* P = reinterpret_cast<__bf16*>(blk + Blk::P);
#pragma unroll
        for (int x = 0; x < NP; ++x)
            if (w + 4 * x < 10) {
                int ti, tj;
                tile_pair(w + 4 * x, ti, tj);
                const floatx4 dec = tile_decay(sm.gam, ti, tj, lr, lq);
                const int i = 16 * ti + lr;
                const float bi = sm.beta[i];
                floatx4 av;
#pragma unroll
                for (int r = 0; r < 4; ++r) av[r] = i > 16 * tj + lq + r ? bi * dec[r] * kk[x][r] : 0.f;
                *reinterpret_cast<floatx4*>(&sm.M[i * kTriLd + 16 * tj + lq]) = av;
                const floatx4 pv = dec * qk[x];
                bf16x4 ph;
#pragma unroll
                for (int r = 0; r < 4; ++r) ph[r] = static_cast<__bf16>(pv[r]);
                *reinterpret_cast<bf16x4*>(&P[i * 64 + kperm(16 * tj + lq)]) = ph;
            }
        // the 6 tiles of P above the diagonal: zeros, 16 rows x 4 runs of 4 keys each
        for (int e = tid; e < 6 * 16 * 4; e += NT) {
            const int t = e >> 6, r = (e >> 2) & 15, run = e & 3;
            const int ti = t < 3 ? 0 : (t < 5 ? 1 : 2), tj = t < 3 ? t + 1 : (t < 5 ? t - 1 : 3);
            *reinterpret_cast<uint2*>(&P[(16 * ti + r) * 64 + kperm(16 * tj + 4 * run)]) = make_uint2(0u, 0u);
        }
        transpose64(sm.K(), LDK, sm.KT, DK, tid, NT);
    }

    // ---- T = (I + A)^-1
    __syncthreads();
    tri::diag<kCpPrepWaves, tri::MmBf16Split>(sm.M, sm.scratch, w);
    __syncthreads();
    tri::lvl16<kCpPrepWaves, tri::MmBf16Split>(sm.M, w);
    __syncthreads();
    tri::lvl32a<kCpPrepWaves, tri::MmBf16Split>(sm.M, sm.scratch, w);
    __syncthreads();
    tri::lvl32b<kCpPrepWaves, tri::MmBf16Split>(sm.M, sm.scratch, w);
    __syncthreads();

    // ---- T diag(beta Gamma) and T diag(beta) in bf16; K^T into the block
    {
        const int i = tid >> 2, c0 = 16 * (tid & 3);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int cc = c0 + 4 * q4;
            const floatx4 t4 = *reinterpret_cast<const floatx4*>(&sm.M[i * kTriLd + cc]);
            const floatx4 b4 = *reinterpret_cast<const floatx4*>(&sm.beta[cc]);
            const floatx4 G4 = *reinterpret_cast<const floatx4*>(&sm.Gam[cc]);
            bf16x4 tg, tb;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                tb[r] = static_cast<__bf16>(t4[r] * b4[r]);
                tg[r] = static_cast<__bf16>(t4[r] * (b4[r] * G4[r]));
            }
            *reinterpret_cast<bf16x4*>(&sm.Tg()[i * L64 + kperm(cc)]) = tg;
            *reinterpret_cast<bf16x4*>(&sm.Tb()[i * L64 + kperm(cc)]) = tb;
        }
        __bf16* KT = reinterpret_cast<__bf16*>(blk + Blk::KT);
        for (int e = tid; e < DK * 8; e += NT) {
            const int d = e >> 3, c8 = (e & 7) * 8;
            *reinterpret_cast<uint4*>(&KT[d * 64 + c8]) = *reinterpret_cast<const uint4*>(&sm.KT[d * L64 + c8]);
        }
    }
    __syncthreads();

    // ---- W^T = K^T (T diag(beta Gamma))^T and U'^T = V^T (T diag(beta))^T: lane (column i, rows
    //      d = 16 td + 4 lg .. +3) writes 4 consecutive entries of row i of W and U'
    {
        __bf16* W = reinterpret_cast<__bf16*>(blk + Blk::W);
        float* Up = reinterpret_cast<float*>(blk + Blk::U);
        for (int tile = w; tile < (DK / 16) * 4; tile += kCpPrepWaves) {
            const int td = tile >> 2, ti = tile & 3;
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mfma(frag(&sm.KT[(16 * td + lr) * L64 + lk]), frag(&sm.Tg()[(16 * ti + lr) * L64 + lk]), acc);
            if (ti >= 2)
                acc = mfma(frag(&sm.KT[(16 * td + lr) * L64 + 32 + lk]), frag(&sm.Tg()[(16 * ti + lr) * L64 + 32 + lk]),
                           acc);
            bf16x4 wv;
#pragma unroll
            for (int r = 0; r < 4; ++r) wv[r] = static_cast<__bf16>(acc[r]);
            *reinterpret_cast<bf16x4*>(&W[(16 * ti + lr) * DK + kperm(16 * td + lq)]) = wv;
        }
        for (int tile = w; tile < (DV / 16) * 4; tile += kCpPrepWaves) {
            const int tc = tile >> 2, ti = tile & 3;
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mfma(frag(&sm.VT[(16 * tc + lr) * L64 + lk]), frag(&sm.Tb()[(16 * ti + lr) * L64 + lk]), acc);
            if (ti >= 2)
                acc = mfma(frag(&sm.VT[(16 * tc + lr) * L64 + 32 + lk]), frag(&sm.Tb()[(16 * ti + lr) * L64 + 32 + lk]),
                           acc);
            *reinterpret_cast<floatx4*>(&Up[(16 * ti + lr) * DV + 16 * tc + lq]) = acc;
        }
    }
}

// ------------------------------------------------------------------ state
// LDS of the state kernel: W and K^T (with the state-update decay) of two
// chunks, Q and P (with Gamma) of two chunks, and the bf16 fragments of S_0
// and U that each state wave hands to its output wave, by chunk parity.
template <int DK, int NSW>
struct CpStateSmem {
    // Row strides (bf16) at which 16-byte fragment reads by 16 rows are free of
    // LDS bank conflicts (rows start 32 bytes apart modulo 128).
    static constexpr int LDK = DK + 16;  // W, Q rows
    static constexpr int LT = 80;        // K^T, P rows (64 columns)
    static constexpr int KS = DK / 32;
    __bf16 W[2][64 * LDK];
    __bf16 KT[2][DK * LT];
    __bf16 Q[2][64 * LDK];
    __bf16 P[2][64 * LT];
    float dec[2][64];  // with W, K^T: e^{min(gamma_S - gamma_r, 0)}, 0 past the chunk
    float Gam[2][64];  // with Q, P: e^{gamma_r}
    float GS[2];       // with W, K^T: e^{gamma_S}
    alignas(16) bf16x8 xs[2][NSW][KS][64];  // S_0 as B fragments, per lane
    alignas(16) bf16x8 xu[2][NSW][2][64];   // U as B fragments, per lane
};

// Grid (value heads x column slices, prompts).  Waves: NSW state waves of 16
// columns each, then NSW output waves (one per state wave, same columns),
// then kCpLoaders loader waves.  In iteration n the state waves run the chain
// that chunk n + 1 depends on (W S_0, U = U' - W S_0, the state update) and
// hand S_0 and U of chunk n to the output waves, which form O of chunk n - 1
// (diag(Gamma) Q S_0 + P U) at the same time; the loaders stage W, K^T of
// chunk n + 1 and Q, P of chunk n.  One workgroup barrier per iteration.
template <int DK, int DV, int NSW>
__global__ __launch_bounds__(64 * (2 * NSW + kCpLoaders), 1) void gdn_cp_state_kernel(
    const uint16_t* __restrict__ q, float* __restrict__ o, float* state, Batch bt, CpChunks cm, int Hk, int Hv,
    const unsigned char* __restrict__ ws) {
    using Sm = CpStateSmem<DK, NSW>;
    using Blk = CpBlock<DK, DV>;
    constexpr int LDK = Sm::LDK;
    constexpr int KS = DK / 32;  // k-steps over dk
    constexpr int RT = DK / 16;  // state row tiles
    constexpr int NCW = DV / (16 * NSW);
    extern __shared__ __align__(16) unsigned char smem_raw[];
    Sm& sm = *reinterpret_cast<Sm*>(smem_raw);

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // The NCW column slices of a head read the same W, K^T, Q and P: with Hv a multiple
    // of 8 they are placed 8 workgroups apart, on one XCD, so that they share its L2.
    int h, slice;
    if (NCW > 1 && Hv % 8 == 0) {
        const int grp = blockIdx.x / (8 * NCW), r = blockIdx.x % (8 * NCW);
        h = 8 * grp + r % 8;
        slice = r / 8;
    } else {
        h = blockIdx.x / NCW;
        slice = blockIdx.x % NCW;
    }
    const int kh = h / (Hv / Hk);
    const int p = batch_prompt(bt, blockIdx.y);
    const int L = batch_len(bt, p);
    const int nc = (L + 63) >> 6;
    if (nc == 0) return;  // the state stays as it is
    const long row0 = batch_row0(bt, p);
    const int c0 = cm.off[p];
    const uint32_t rowV = Hv * DV;
    auto block = [&](int n) { return ws + ((long)(c0 + n) * Hv + h) * Blk::BYTES; };
    int tid_c = tid;
    asm volatile("" : "+v"(tid_c));
    const int lr = tid_c & 15, lg = (tid_c >> 4) & 3, lq = lg * 4;

    if (w >= 2 * NSW) {
        // ================= loader waves
        const int lt = tid - 128 * NSW;
        constexpr int NT = 64 * kCpLoaders;
        const uint32_t rowK = Hk * DK * 2;
        constexpr int NP8 = 8 * DK / NT;  // 16-byte pieces of W, Q and K^T per loader thread
        static_assert(8 * DK % NT == 0 && 512 % NT == 0, "whole 16-byte pieces per loader thread");
        u32x4 rw[NP8], rk[NP8], rq[NP8], rp[512 / NT];
        float rdec = 0.f, rgam = 0.f, rgs = 0.f;
        // loads into registers (all in flight together), LDS stores one iteration later
        auto issue_wk = [&](int n) __attribute__((always_inline)) {
            const auto brs = buffer_rsrc(block(n), (uint32_t)Blk::BYTES);
#pragma unroll
            for (int x = 0; x < NP8; ++x) {
                const int e = lt + x * NT, r = e / (DK / 8), c8 = (e % (DK / 8)) * 8;
                rw[x] = __builtin_amdgcn_raw_buffer_load_b128(brs, (uint32_t)(Blk::W + (r * DK + c8) * 2), 0, 0);
                rk[x] = __builtin_amdgcn_raw_buffer_load_b128(brs, (uint32_t)(Blk::KT + e * 16), 0, 0);  // [DK][64]
            }
            rdec = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(brs, (uint32_t)(Blk::DEC + lt * 4), 0, 0));
            // e^{gamma_S} of chunk n: the Gamma of its last row
            const int S = min(64, L - 64 * n);
            rgs = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(brs, (uint32_t)(Blk::GAM + (S - 1) * 4), 0, 0));
        };
        auto commit_wk = [&](int n) __attribute__((always_inline)) {
            const int b = n & 1;
#pragma unroll
            for (int x = 0; x < NP8; ++x) {
                const int e = lt + x * NT, r = e / (DK / 8), c8 = (e % (DK / 8)) * 8;
                *reinterpret_cast<u32x4*>(&sm.W[b][r * LDK + c8]) = rw[x];
                *reinterpret_cast<u32x4*>(&sm.KT[b][(e >> 3) * Sm::LT + (e & 7) * 8]) = rk[x];
            }
            if (lt < 64) sm.dec[b][lt] = rdec;
            if (lt == 0) sm.GS[b] = rgs;
        };
        auto issue_qp = [&](int n) __attribute__((always_inline)) {
            const int S = min(64, L - 64 * n);
            const auto brs = buffer_rsrc(block(n), (uint32_t)Blk::BYTES);
            const auto qrs = buffer_rsrc(q + ((row0 + 64l * n) * Hk + kh) * DK, (uint32_t)S * rowK);
#pragma unroll
            for (int x = 0; x < NP8; ++x) {
                const int e = lt + x * NT, r = e / (DK / 8), c8 = (e % (DK / 8)) * 8;
                rq[x] = __builtin_amdgcn_raw_buffer_load_b128(qrs, (uint32_t)r * rowK + c8 * 2, 0, 0);
            }
#pragma unroll
            for (int x = 0; x < 512 / NT; ++x)
                rp[x] = __builtin_amdgcn_raw_buffer_load_b128(brs, (uint32_t)(Blk::P + (lt + x * NT) * 16), 0, 0);
            rgam = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(brs, (uint32_t)(Blk::GAM + lt * 4), 0, 0));
        };
        auto commit_qp = [&](int n) __attribute__((always_inline)) {
            const int b = n & 1;
#pragma unroll
            for (int x = 0; x < NP8; ++x) {
                const int e = lt + x * NT, r = e / (DK / 8), c8 = (e % (DK / 8)) * 8;
                *reinterpret_cast<u32x2*>(&sm.Q[b][r * LDK + kperm(c8)]) = u32x2{rq[x][0], rq[x][1]};
                *reinterpret_cast<u32x2*>(&sm.Q[b][r * LDK + kperm(c8 + 4)]) = u32x2{rq[x][2], rq[x][3]};
            }
#pragma unroll
            for (int x = 0; x < 512 / NT; ++x) {
                const int e = lt + x * NT;
                *reinterpret_cast<u32x4*>(&sm.P[b][(e >> 3) * Sm::LT + (e & 7) * 8]) = rp[x];
            }
            if (lt < 64) sm.Gam[b][lt] = rgam;
        };
        issue_wk(0);
        commit_wk(0);
        if (nc > 1) issue_wk(1);
        issue_qp(0);
        __syncthreads();
        for (int n = 0; n <= nc; ++n) {
            if (n + 1 < nc) commit_wk(n + 1);
            if (n < nc) commit_qp(n);
            if (n + 2 < nc) issue_wk(n + 2);
            if (n + 1 < nc) issue_qp(n + 1);
            __syncthreads();
        }
        return;
    }

    const int pair = w % NSW;  // the state wave and its output wave share 16 columns
    const int col0 = 16 * (slice * NSW + pair);
    if (w >= NSW) {
        // ================= output waves: O of chunk n - 1 in iteration n
        __syncthreads();
        for (int n = 0; n <= nc; ++n) {
            if (n >= 1) {
                const int m = n - 1, b = m & 1;
                const int S = min(64, L - 64 * m);
                floatx4 qs0[4], pu[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) qs0[t] = pu[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    const bf16x8 bs = sm.xs[b][pair][s][lane];
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        qs0[t] = mfma(frag(&sm.Q[b][(16 * t + lr) * LDK + 32 * s + 8 * lg]), bs, qs0[t]);
                }
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const bf16x8 bu = sm.xu[b][pair][s][lane];
#pragma unroll
                    for (int t = 2 * s; t < 4; ++t)
                        pu[t] = mfma(frag(&sm.P[b][(16 * t + lr) * Sm::LT + 32 * s + 8 * lg]), bu, pu[t]);
                }
                const auto orsrc = buffer_rsrc(o + (row0 + 64l * m) * (long)rowV + (long)h * DV + col0,
                                              (uint32_t)S * rowV * 4);
                uint32_t o_lane = (__umul24(lq, rowV) + lr) * 4;
                asm volatile("" : "+v"(o_lane));
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const floatx4 G4 = *reinterpret_cast<const floatx4*>(&sm.Gam[b][16 * t + lq]);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(fmaf(G4[r], qs0[t][r], pu[t][r])), orsrc,
                                                              o_lane + (16 * t + r) * rowV * 4, 0, 0);
                }
            }
            __syncthreads();
        }
        return;
    }

    // ================= state waves: 16 columns each
    int s_lane = (lane >> 4) * 4 * DV + lr;
    asm volatile("" : "+v"(s_lane));
    floatx4 sacc[RT];
    const auto srs = buffer_rsrc(state + ((long)p * Hv + h) * DK * DV + col0, (uint32_t)(DK * DV * 4));
    {
        int sl = s_lane * 4, dv4 = DV * 4;
        asm volatile("" : "+v"(sl), "+s"(dv4));
#pragma unroll
        for (int tr = 0; tr < RT; ++tr)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sacc[tr][r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(srs, sl, (16 * tr + r) * dv4, 0));
    }
    // U' of a chunk in accumulator layout: rows 16t + 4(l/16) + r, the lane's column
    float up[16];
    auto load_up = [&](int n) __attribute__((always_inline)) {
        const auto urs = buffer_rsrc(block(n) + Blk::U, (uint32_t)(64 * DV * 4));
        uint32_t u_lane = ((lane >> 4) * 4 * DV + col0 + lr) * 4;
        asm volatile("" : "+v"(u_lane));
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                up[4 * t + r] =
                    __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(urs, u_lane + (16 * t + r) * DV * 4, 0, 0));
    };
    load_up(0);
    __syncthreads();  // chunk 0's W and K^T in LDS

    for (int n = 0; n <= nc; ++n) {
        if (n < nc) {
            const int b = n & 1;
            // All fragments of W and K^T of chunk n, and its decays, are in LDS since
            // the last barrier: one wave per SIMD has the registers to read them all
            // at once, W's first, so that the chain below waits for LDS only once.
            bf16x8 wf[KS][4], kt[2][RT];
#pragma unroll
            for (int s = 0; s < KS; ++s)
#pragma unroll
                for (int t = 0; t < 4; ++t) wf[s][t] = frag(&sm.W[b][(16 * t + lr) * LDK + 32 * s + 8 * lg]);
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int tr = 0; tr < RT; ++tr) kt[s][tr] = frag(&sm.KT[b][(16 * tr + lr) * Sm::LT + 32 * s + 8 * lg]);
            floatx4 dec4[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) dec4[t] = *reinterpret_cast<const floatx4*>(&sm.dec[b][16 * t + lq]);
            const float GS = sm.GS[b];
            // ---- W S_0, with S_0 handed to the output wave as B fragments
            floatx4 ws0[4], u[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) ws0[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                bf16x8 bh, bl;
                acc_frag<false>(sacc[2 * s], sacc[2 * s + 1], bh, bl);
                sm.xs[b][pair][s][lane] = bh;
#pragma unroll
                for (int t = 0; t < 4; ++t) ws0[t] = mfma(wf[s][t], bh, ws0[t]);
            }
            // ---- U = U' - W S_0 (zero past the chunk: W and U' rows are zero there)
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) u[t][r] = up[4 * t + r] - ws0[t][r];
            if (n + 1 < nc) load_up(n + 1);
            // ---- U to the output wave; S_S = e^{gamma_S} S_0 + K^T (decay U)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                bf16x8 bh, bl;
                acc_frag<false>(u[2 * s], u[2 * s + 1], bh, bl);
                sm.xu[b][pair][s][lane] = bh;
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) u[t] *= dec4[t];
#pragma unroll
            for (int tr = 0; tr < RT; ++tr) sacc[tr] = sacc[tr] * GS;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                bf16x8 bh, bl;
                acc_frag<false>(u[2 * s], u[2 * s + 1], bh, bl);
#pragma unroll
                for (int tr = 0; tr < RT; ++tr) sacc[tr] = mfma(kt[s][tr], bh, sacc[tr]);
            }
        }
        __syncthreads();
    }
    {
        int sl = s_lane * 4, dv4 = DV * 4;
        asm volatile("" : "+v"(sl), "+s"(dv4));
#pragma unroll
        for (int tr = 0; tr < RT; ++tr)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sacc[tr][r]), srs, sl, (16 * tr + r) * dv4, 0);
    }
}

CpChunks cp_chunks(const Batch& bt) {
    CpChunks cm;
    int c = 0;
    for (int p = 0; p < bt.P; ++p) {
        cm.off[p] = c;
        c += (batch_len(bt, p) + 63) / 64;
    }
    cm.off[bt.P] = c;
    cm.total = c;
    return cm;
}

template <class K>
hipError_t opt_in_lds(K kern, size_t bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)bytes);
}

template <int DK, int DV, int NSW>
hipError_t launch_state(const void* q, float* o, float* state, const Batch& bt, const CpChunks& cm, int Hk, int Hv,
                        void* ws, hipStream_t st) {
    constexpr int NCW = DV / (16 * NSW);
    auto stk = gdn_cp_state_kernel<DK, DV, NSW>;
    static const hipError_t e = opt_in_lds(stk, sizeof(CpStateSmem<DK, NSW>));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(stk, dim3((unsigned)(Hv * NCW), (unsigned)bt.P), dim3(64 * (2 * NSW + kCpLoaders)),
                       sizeof(CpStateSmem<DK, NSW>), st, static_cast<const uint16_t*>(q), o, state, bt, cm, Hk, Hv,
                       static_cast<const unsigned char*>(ws));
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_cp(const void* q, const void* k, const void* v, const float* beta, const float* g, float* o,
                     float* state, const Batch& bt, int Hk, int Hv, void* ws, hipStream_t st) {
    const CpChunks cm = cp_chunks(bt);
    if (cm.total == 0) return hipSuccess;
    auto prep = gdn_cp_prep_kernel<DK, DV>;
    static const hipError_t e1 = opt_in_lds(prep, sizeof(CpPrepSmem<DK, DV>));
    if (e1 != hipSuccess) return e1;
    hipLaunchKernelGGL(prep, dim3((unsigned)((cm.total + 7) / 8 * 8), (unsigned)Hv), dim3(64 * kCpPrepWaves),
                       sizeof(CpPrepSmem<DK, DV>), st, static_cast<const uint16_t*>(q),
                       static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), beta, g, bt, cm, Hk, Hv,
                       static_cast<unsigned char*>(ws));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // A workgroup per 16 columns of a head when that fills no more than the compute units
    // (fewer waves read the same fragments from one CU's LDS); per 32 columns otherwise.
    int nonempty = 0;
    for (int p = 0; p < bt.P; ++p) nonempty += batch_len(bt, p) > 0;
    if ((long)nonempty * Hv * (DV / 16) <= compute_units())
        return launch_state<DK, DV, 1>(q, o, state, bt, cm, Hk, Hv, ws, st);
    return launch_state<DK, DV, 2>(q, o, state, bt, cm, Hk, Hv, ws, st);
}

template <int DK>
hipError_t launch_cp_dv(const void* q, const void* k, const void* v, const float* beta, const float* g, float* o,
                        float* state, const Batch& bt, int Hk, int Hv, int dv, void* ws, hipStream_t st) {
    switch (dv) {
        case 32: return launch_cp<DK, 32>(q, k, v, beta, g, o, state, bt, Hk, Hv, ws, st);
        case 64: return launch_cp<DK, 64>(q, k, v, beta, g, o, state, bt, Hk, Hv, ws, st);
        case 128: return launch_cp<DK, 128>(q, k, v, beta, g, o, state, bt, Hk, Hv, ws, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

size_t gdn_cp_block_bytes(int dk, int dv) {
    return (size_t)((256l * dk + 8192 + 256l * dv + 512 + 255) / 256 * 256);
}

hipError_t launch_gdn_chunk_parallel(const void* q, const void* k, const void* v, const float* beta, const float* g,
                                     float* o, float* state, const Batch& bt, int Hk, int Hv, int dk, int dv,
                                     void* ws, hipStream_t st) {
    switch (dk) {
        case 32: return launch_cp_dv<32>(q, k, v, beta, g, o, state, bt, Hk, Hv, dv, ws, st);
        case 64: return launch_cp_dv<64>(q, k, v, beta, g, o, state, bt, Hk, Hv, dv, ws, st);
        case 128: return launch_cp_dv<128>(q, k, v, beta, g, o, state, bt, Hk, Hv, dv, ws, st);
    }
    return hipErrorInvalidValue;
}

static_assert(CpBlock<128, 128>::BYTES == (256 * 128 + 8192 + 256 * 128 + 512 + 255) / 256 * 256,
              "the block size formula of the host matches the layout");

}  // namespace lrc

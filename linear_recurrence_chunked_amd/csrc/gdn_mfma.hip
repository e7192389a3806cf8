// K3, bf16-input path: Gated DeltaNet chunked delta rule on CDNA4 matrix cores.
//
// Source: "perf(qwen3_5): prefill text prompts in multi-token chunks",
// Implementation.  For a chunk of S <= 64 rows of value head h (key head
// h / (Hv/Hk)), with gamma the chunk-local inclusive cumulative sum of g and
// Gamma = e^gamma:
//   A_ij = beta_i e^{gamma_i - gamma_j} k_i.k_j  (j < i)
//   U    = (I + A)^-1 (diag(beta) V - diag(beta Gamma) K S_0)
//   O    = diag(Gamma) Q S_0 + (e^{gamma_t - gamma_i} q_t.k_i)_{i <= t} U
//   S_S  = e^{gamma_S} S_0 + (K * e^{min(gamma_S - gamma, 0)})^T U
// gamma_S is the last entry of the same cumulative sum.
//
// Work split.  A workgroup owns a DVT-wide slice (the whole head for dv = 128,
// else min(dv, 64)) of one value head of one prompt and walks the prompt's
// chunks; it has DVT/16 waves and wave w owns state columns 16w .. 16w+15 of
// the slice.  A wave's [dk x 16] state slice, and its columns of V, RHS, U and
// Q S_0, stay in registers (MFMA accumulator layout) for the whole prompt.
// Only operands every wave needs sit in LDS: the chunk's K and Q, K^T, the
// FP32 matrix A -> T of the inverse, T and P as hi/lo bf16, and the per-row
// gamma, Gamma, beta and state-update decay.  The waves share the per-chunk
// work that does not depend on the column (the masked products, the inverse,
// K^T).
//
// Matrix cores: v_mfma_f32_16x16x32_bf16, FP32 accumulation.  The A operand
// of lane l is row l%16 with 8 k-values, the B operand column l%16 with the
// same 8 k-values, and the accumulator holds column l%16, rows 4(l/16) .. +3.
// A wave's own [rows x 16] accumulators serve directly as B operands when
// the k-values of lane group g are taken as rows {4g .. 4g+3} of one 16-row
// tile and {16+4g .. 16+4g+3} of the next; the A operand then reads the same
// two 4-element runs of its row from LDS.  The masked products are computed
// transposed (keys as rows), so each lane holds 4 consecutive keys of one
// query and writes them as one packed store.
// FP32 operands enter as a hi + lo pair of bf16 (hi = bf16(x),
// lo = bf16(x - hi)), about 16 mantissa bits:
//   K K^T, Q K^T        bf16 x bf16 (exact products)            1 pass
//   K S_0, Q S_0        bf16 x (S_0 hi, lo)                     2 passes
//   K^T (d U)           bf16 x (decayed U hi, lo)               2 passes
//   T RHS, P U          (hi, lo) x (hi, lo) without lo x lo     3 passes
// Decay factors: on the diagonal 16x16 tiles e^{gamma_i - gamma_j} is formed
// per element; below them it is the product e^{gamma_i - gamma_c}
// e^{gamma_c - gamma_j} through the tile's first row c, both factors <= 1.
// The 64-row inverse (8x8 Neumann blocks, then 2x2 block levels) runs in
// FP32 on the FP32 matrix cores.  The next chunk's K, Q, V, beta and g are loaded
// into registers once the inverse is done, while U, O and the state update
// compute.
#include "lrc_device.h"
#include "lrc_internal.h"
#include "tri_inverse.h"

namespace lrc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int L64 = 64 + 8;  // row stride (bf16) of 64-column operands

__device__ __forceinline__ floatx4 mfma(bf16x8 a, bf16x8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// Contiguous fragment: 8 k-values from one 16-byte run.
__device__ __forceinline__ bf16x8 frag(const __bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
// Permuted fragment: k-values {4g..4g+3} and {16+4g..16+4g+3} of a 32-wide k-step.
__device__ __forceinline__ bf16x8 frag_perm(const __bf16* row_ks, int g) {
    const bf16x4 a = *reinterpret_cast<const bf16x4*>(row_ks + 4 * g);
    const bf16x4 b = *reinterpret_cast<const bf16x4*>(row_ks + 16 + 4 * g);
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
// B fragment from two accumulator tiles (rows 16t.. and 16t+16..): hi and lo parts.
__device__ __forceinline__ void acc_frag(const floatx4& t0, const floatx4& t1, bf16x8& hi, bf16x8& lo) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const __bf16 h0 = static_cast<__bf16>(t0[r]);
        const __bf16 h1 = static_cast<__bf16>(t1[r]);
        hi[r] = h0;
        hi[4 + r] = h1;
        lo[r] = static_cast<__bf16>(t0[r] - static_cast<float>(h0));
        lo[4 + r] = static_cast<__bf16>(t1[r] - static_cast<float>(h1));
    }
}
__device__ __forceinline__ void split4(const floatx4& x, bf16x4& hi, bf16x4& lo) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        hi[r] = static_cast<__bf16>(x[r]);
        lo[r] = static_cast<__bf16>(x[r] - static_cast<float>(hi[r]));
    }
}

// LDS of one workgroup, kept under 80 KiB so that two workgroups share a CU.
// One buffer holds, in turn, Q (staging .. masked products), T as hi/lo
// (after the inverse .. U) and K^T (after U .. state update).
template <int DK, int DVT>
struct MfmaSmem {
    static constexpr int LDK = DK + 8;
    __bf16 K[64 * LDK];
    union {
        __bf16 Q[64 * LDK];
        struct {
            __bf16 hi[64 * L64];  // (I + A)^-1
            __bf16 lo[64 * L64];
        } T;
        __bf16 KT[DK * L64];     // K^T, exact
    } u;
    __bf16 P_hi[64 * L64];  // masked decayed Q K^T
    __bf16 P_lo[64 * L64];
    float M[64 * kTriLd];   // A, then T, in FP32
    float scratch[kTriScratch];
    float gam[64];
    float Gam[64];          // e^gamma
    float beta[64];
    float decS[64];         // e^{min(gamma_S - gamma_r, 0)}, 0 past the chunk
};

// Lower-triangular 16x16 tile pairs (query tile, key tile) of the 64x64 masks.
__constant__ int kPairs[10][2] = {{0, 0}, {1, 0}, {1, 1}, {2, 0}, {2, 1}, {2, 2}, {3, 0}, {3, 1}, {3, 2}, {3, 3}};

template <int DK, int DVT>
__global__ __launch_bounds__(DVT * 4, DVT >= 64 ? 2 : 1) void gdn_mfma_kernel(const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ k,
                                                          const uint16_t* __restrict__ v,
                                                          const float* __restrict__ beta,
                                                          const float* __restrict__ g, float* __restrict__ o,
                                                          const float* S_in, float* S_out, Batch bt, int Hk, int Hv,
                                                          int dv) {
    using Sm = MfmaSmem<DK, DVT>;
    constexpr int NW = DVT / 16;           // waves: one per 16 state columns
    constexpr int NT = NW * 64;
    constexpr int LDK = Sm::LDK;
    constexpr int KS = DK / 32;            // k-steps over dk
    constexpr int RT = DK / 16;            // state row tiles
    constexpr int PK = 64 * DK / 8;        // 16-byte pieces of a K (or Q) chunk
    constexpr int NK = (PK + NT - 1) / NT;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    Sm& sm = *reinterpret_cast<Sm*>(smem_raw);

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15;        // fragment row / column within a tile
    const int lg = lane >> 4;        // lane group
    const int lk = lg * 8;           // contiguous fragment k offset
    const int lq = lg * 4;           // accumulator row offset
    const int ntile = dv / DVT;
    const int h = blockIdx.x / ntile;
    const int c0v = (blockIdx.x % ntile) * DVT;  // first column of the slice
    const int kh = h / (Hv / Hk);
    const int p = batch_prompt(bt, blockIdx.y);
    const long row0 = batch_row0(bt, p);
    const int L = batch_len(bt, p);
    const long sbase = ((long)p * Hv + h) * DK * dv + c0v + 16 * w;

    // Per-lane address offsets pass through an empty asm wherever they are
    // used, so that the compiler recomputes addresses (a few adds) instead of
    // keeping dozens of 64-bit addresses alive across the chunk loop.
    int s_lane = lq * dv + lr;
    asm volatile("" : "+v"(s_lane));
    floatx4 sacc[RT];
#pragma unroll
    for (int tr = 0; tr < RT; ++tr)
#pragma unroll
        for (int r = 0; r < 4; ++r) sacc[tr][r] = S_in[sbase + s_lane + (long)(16 * tr + r) * dv];
    // The masks' tiles above the diagonal stay zero for the whole prompt.
    for (int e = tid; e < 64 * kTriLd; e += NT) sm.M[e] = 0.f;
    for (int e = tid; e < 64 * L64; e += NT) sm.P_hi[e] = sm.P_lo[e] = static_cast<__bf16>(0.f);

    uint4 pk[NK], pq[NK];
    uint16_t pv[16];  // next chunk's V in accumulator layout: rows 16t + 4(l/16) + r, column l%16 of this wave's slice
    u16x2 vc2[8];     // this chunk's V, two rows a word
    float pg = 0.f, pb = 0.f;
    // Addresses: a 64-bit base per chunk (scalar) plus 32-bit lane offsets
    // formed with 24-bit multiplies (heads x head size stays below 2^24).
    const uint32_t rowK = Hk * DK, rowV = Hv * dv;
    auto fetch = [&](int c0) {
        const int S = min(64, L - c0);
        const uint16_t* kc = k + ((row0 + c0) * Hk + kh) * (long)DK;
        const uint16_t* qc = q + ((row0 + c0) * Hk + kh) * (long)DK;
#pragma unroll
        for (int x = 0; x < NK; ++x) {
            const int e = tid + x * NT, r = e / (DK / 8), c8 = (e % (DK / 8)) * 8;
            pk[x] = pq[x] = make_uint4(0, 0, 0, 0);
            if (e < PK && r < S) {
                const uint32_t off = __umul24(r, rowK) + c8;
                pk[x] = *reinterpret_cast<const uint4*>(kc + off);
                pq[x] = *reinterpret_cast<const uint4*>(qc + off);
            }
        }
        const uint16_t* vc = v + (row0 + c0) * (long)rowV + (long)h * dv + c0v + 16 * w;
        int v_lane = lr;
        asm volatile("" : "+v"(v_lane));
        // Rows past the chunk re-read its last row and are zeroed where V is
        // used; the values are packed only at staging, so nothing waits here.
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) pv[4 * t + r] = vc[__umul24(min(16 * t + lq + r, S - 1), rowV) + v_lane];
        pg = pb = 0.f;
        if (tid < S) {
            const long gi = (row0 + c0) * Hv + h + __umul24(tid, Hv);
            pg = g[gi];
            pb = beta[gi];
        }
    };

    if (L > 0) fetch(0);
    for (int c0 = 0; c0 < L; c0 += 64) {
        const int S = min(64, L - c0);
        // The lane indices pass through an empty asm once per chunk, so that
        // the LDS addresses derived from them are recomputed here instead of
        // being held in registers across the whole prompt.
        int tid_c = tid;
        asm volatile("" : "+v"(tid_c));
        const int lr = tid_c & 15, lg = (tid_c >> 4) & 3, lk = lg * 8, lq = lg * 4;
        __syncthreads();  // previous chunk done with every LDS buffer
        // ---- stage the prefetched chunk: K, Q, V, beta, gamma, Gamma, decay of the state update
#pragma unroll
        for (int x = 0; x < NK; ++x) {
            const int e = tid + x * NT, r = e / (DK / 8), c8 = (e % (DK / 8)) * 8;
            if (e < PK) {
                *reinterpret_cast<uint4*>(&sm.K[r * LDK + c8]) = pk[x];
                *reinterpret_cast<uint4*>(&sm.u.Q[r * LDK + c8]) = pq[x];
            }
        }
#pragma unroll
        for (int x = 0; x < 8; ++x) vc2[x] = u16x2{pv[2 * x], pv[2 * x + 1]};
        if (tid < 64) {
            sm.beta[tid] = pb;
            const float x = wave_prefix_sum(pg);  // gamma, inclusive over the chunk rows
            sm.gam[tid] = x;
            sm.Gam[tid] = fast_exp(x);
            const float gS = readlane_f(x, S - 1);  // the last cumulative sum
            sm.decS[tid] = tid < S ? fast_exp(fminf(gS - x, 0.f)) : 0.f;
        }
        __syncthreads();

        // ---- private: K S_0 and Q S_0 for this wave's columns (B from the state accumulators)
        floatx4 ks0[4], qs0[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) ks0[t] = qs0[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            bf16x8 bh, bl;
            acc_frag(sacc[2 * s], sacc[2 * s + 1], bh, bl);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const bf16x8 ak = frag_perm(&sm.K[(16 * t + lr) * LDK + 32 * s], lg);
                const bf16x8 aq = frag_perm(&sm.u.Q[(16 * t + lr) * LDK + 32 * s], lg);
                ks0[t] = mfma(ak, bh, ks0[t]);
                ks0[t] = mfma(ak, bl, ks0[t]);
                qs0[t] = mfma(aq, bh, qs0[t]);
                qs0[t] = mfma(aq, bl, qs0[t]);
            }
        }
        // ---- shared: masked products, transposed (keys as rows) -> A (FP32) and P (hi/lo)
        {
            constexpr int PPW = (10 + NW - 1) / NW;  // tile pairs per wave
            floatx4 kk[PPW], qk[PPW];
            int ti[PPW], tj[PPW];
#pragma unroll
            for (int q = 0; q < PPW; ++q) {
                const int pr = min(w + q * NW, 9);
                ti[q] = kPairs[pr][0];
                tj[q] = kPairs[pr][1];
                kk[q] = qk[q] = floatx4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int s = 0; s < KS; ++s)
#pragma unroll
                for (int q = 0; q < PPW; ++q) {
                    const bf16x8 ak = frag(&sm.K[(16 * tj[q] + lr) * LDK + 32 * s + lk]);
                    kk[q] = mfma(ak, frag(&sm.K[(16 * ti[q] + lr) * LDK + 32 * s + lk]), kk[q]);
                    qk[q] = mfma(ak, frag(&sm.u.Q[(16 * ti[q] + lr) * LDK + 32 * s + lk]), qk[q]);
                }
#pragma unroll
            for (int q = 0; q < PPW; ++q) {
                if (w + q * NW >= 10) break;
                const int i = 16 * ti[q] + lr;
                const float gi = sm.gam[i];
                const floatx4 gj = *reinterpret_cast<const floatx4*>(&sm.gam[16 * tj[q] + lq]);
                floatx4 dec;
                if (ti[q] > tj[q]) {
                    const float gc = sm.gam[16 * ti[q]];
                    const float rowf = fast_exp(gi - gc);
#pragma unroll
                    for (int r = 0; r < 4; ++r) dec[r] = rowf * fast_exp(gc - gj[r]);
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = 16 * tj[q] + lq + r;
                        dec[r] = i >= j ? fast_exp(gi - gj[r]) : 0.f;
                    }
                }
                const float bi = sm.beta[i];
                floatx4 av, pv4;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = 16 * tj[q] + lq + r;
                    av[r] = i > j ? bi * dec[r] * kk[q][r] : 0.f;
                    pv4[r] = dec[r] * qk[q][r];
                }
                *reinterpret_cast<floatx4*>(&sm.M[i * kTriLd + 16 * tj[q] + lq]) = av;
                bf16x4 ph, pl;
                split4(pv4, ph, pl);
                *reinterpret_cast<bf16x4*>(&sm.P_hi[i * L64 + 16 * tj[q] + lq]) = ph;
                *reinterpret_cast<bf16x4*>(&sm.P_lo[i * L64 + 16 * tj[q] + lq]) = pl;
            }
        }
        // ---- private: RHS = diag(beta) V - diag(beta Gamma) K S_0, in registers
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const floatx4 b4 = *reinterpret_cast<const floatx4*>(&sm.beta[16 * t + lq]);
            const floatx4 G4 = *reinterpret_cast<const floatx4*>(&sm.Gam[16 * t + lq]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint16_t raw = (r & 1) ? vc2[2 * t + r / 2].y : vc2[2 * t + r / 2].x;
                const float vv = 16 * t + lq + r < S ? bf16_to_f32(raw) : 0.f;
                ks0[t][r] = b4[r] * (vv - G4[r] * ks0[t][r]);
            }
        }
        // ---- shared: T = (I + A)^-1 in FP32 (barriers inside), then T as hi/lo bf16
        tri_inverse64<NW>(sm.M, sm.scratch);
        if (c0 + 64 < L) fetch(c0 + 64);  // next chunk's rows, in flight during U, O and the state update
#pragma unroll
        for (int xi = 0; xi < 512 / NT; ++xi) {
            const int x = tid + xi * NT;
            const int r = x >> 3, c = (x & 7) * 8;
            const floatx4 a = *reinterpret_cast<const floatx4*>(&sm.M[r * kTriLd + c]);
            const floatx4 b = *reinterpret_cast<const floatx4*>(&sm.M[r * kTriLd + c + 4]);
            bf16x4 ah, al, bh, bl;
            split4(a, ah, al);
            split4(b, bh, bl);
            *reinterpret_cast<bf16x8*>(&sm.u.T.hi[r * L64 + c]) = bf16x8{ah[0], ah[1], ah[2], ah[3], bh[0], bh[1], bh[2], bh[3]};
            *reinterpret_cast<bf16x8*>(&sm.u.T.lo[r * L64 + c]) = bf16x8{al[0], al[1], al[2], al[3], bl[0], bl[1], bl[2], bl[3]};
        }
        __syncthreads();

        // ---- private: U = T RHS (T lower triangular: k-steps up to the row tile's diagonal)
        floatx4 u[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) u[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            bf16x8 bh, bl;
            acc_frag(ks0[2 * s], ks0[2 * s + 1], bh, bl);
#pragma unroll
            for (int t = 2 * s; t < 4; ++t) {
                const bf16x8 ah = frag_perm(&sm.u.T.hi[(16 * t + lr) * L64 + 32 * s], lg);
                const bf16x8 al = frag_perm(&sm.u.T.lo[(16 * t + lr) * L64 + 32 * s], lg);
                u[t] = mfma(ah, bh, u[t]);
                u[t] = mfma(ah, bl, u[t]);
                u[t] = mfma(al, bh, u[t]);
            }
        }
        __syncthreads();  // every wave is done reading T
        // ---- shared: K^T by 4-row x 8-column blocks, into the buffer T occupied
        for (int b = tid; b < 2 * DK; b += NT) {
            const int n = b & 15, m = b >> 4;  // rows 4n .. 4n+3, columns 8m .. 8m+7
            uint4 rw[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) rw[a] = *reinterpret_cast<const uint4*>(&sm.K[(4 * n + a) * LDK + 8 * m]);
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
                *reinterpret_cast<uint2*>(&sm.u.KT[(8 * m + e) * L64 + 4 * n]) = out;
            }
        }
        // ---- private: O = diag(Gamma) Q S_0 + P U for this wave's columns
        {
            floatx4 pu[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) pu[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                bf16x8 bh, bl;
                acc_frag(u[2 * s], u[2 * s + 1], bh, bl);
#pragma unroll
                for (int t = 2 * s; t < 4; ++t) {
                    const bf16x8 ah = frag_perm(&sm.P_hi[(16 * t + lr) * L64 + 32 * s], lg);
                    const bf16x8 al = frag_perm(&sm.P_lo[(16 * t + lr) * L64 + 32 * s], lg);
                    pu[t] = mfma(ah, bh, pu[t]);
                    pu[t] = mfma(ah, bl, pu[t]);
                    pu[t] = mfma(al, bh, pu[t]);
                }
            }
            float* oc = o + (row0 + c0) * (long)rowV + (long)h * dv + c0v + 16 * w;
            uint32_t o_lane = __umul24(lq, rowV) + lr;
            asm volatile("" : "+v"(o_lane));
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const floatx4 G4 = *reinterpret_cast<const floatx4*>(&sm.Gam[16 * t + lq]);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (16 * t + lq + r < S) oc[o_lane + (16 * t + r) * rowV] = fmaf(G4[r], qs0[t][r], pu[t][r]);
            }
        }
        __syncthreads();  // K^T complete
        // ---- private: S_S = e^{gamma_S} S_0 + K^T (decS * U), in the state accumulators
        {
            const float GS = sm.Gam[S - 1];
#pragma unroll
            for (int t = 0; t < 4; ++t) u[t] *= *reinterpret_cast<const floatx4*>(&sm.decS[16 * t + lq]);
#pragma unroll
            for (int tr = 0; tr < RT; ++tr) sacc[tr] = sacc[tr] * GS;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                bf16x8 bh, bl;
                acc_frag(u[2 * s], u[2 * s + 1], bh, bl);
#pragma unroll
                for (int tr = 0; tr < RT; ++tr) {
                    const bf16x8 a = frag_perm(&sm.u.KT[(16 * tr + lr) * L64 + 32 * s], lg);
                    sacc[tr] = mfma(a, bh, sacc[tr]);
                    sacc[tr] = mfma(a, bl, sacc[tr]);
                }
            }
        }
    }
    asm volatile("" : "+v"(s_lane));
#pragma unroll
    for (int tr = 0; tr < RT; ++tr)
#pragma unroll
        for (int r = 0; r < 4; ++r) S_out[sbase + s_lane + (long)(16 * tr + r) * dv] = sacc[tr][r];
}

template <int DK, int DVT>
hipError_t launch_mfma(const void* q, const void* k, const void* v, const float* beta, const float* g, float* o,
                       const float* S_in, float* S_out, const Batch& bt, int Hk, int Hv, int dv, hipStream_t st) {
    auto kern = gdn_mfma_kernel<DK, DVT>;
    const size_t smem = sizeof(MfmaSmem<DK, DVT>);
    static bool configured = false;
    if (!configured) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
        configured = true;
    }
    const dim3 grid((unsigned)(Hv * (dv / DVT)), (unsigned)bt.P);
    hipLaunchKernelGGL(kern, grid, dim3(DVT * 4), smem, st, static_cast<const uint16_t*>(q),
                       static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), beta, g, o, S_in, S_out, bt,
                       Hk, Hv, dv);
    return hipGetLastError();
}

template <int DVT>
hipError_t launch_dk(const void* q, const void* k, const void* v, const float* beta, const float* g, float* o,
                     const float* S_in, float* S_out, const Batch& bt, int Hk, int Hv, int dk, int dv,
                     hipStream_t st) {
    switch (dk) {
        case 32: return launch_mfma<32, DVT>(q, k, v, beta, g, o, S_in, S_out, bt, Hk, Hv, dv, st);
        case 64: return launch_mfma<64, DVT>(q, k, v, beta, g, o, S_in, S_out, bt, Hk, Hv, dv, st);
        case 128: return launch_mfma<128, DVT>(q, k, v, beta, g, o, S_in, S_out, bt, Hk, Hv, dv, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gdn_bf16_mfma(const void* q, const void* k, const void* v, const float* beta, const float* g,
                                float* o, const float* S_in, float* S_out, const Batch& bt, int Hk, int Hv, int dk,
                                int dv, hipStream_t st) {
    if (dv == 32) return launch_dk<32>(q, k, v, beta, g, o, S_in, S_out, bt, Hk, Hv, dk, dv, st);
    if (dv == 128) return launch_dk<128>(q, k, v, beta, g, o, S_in, S_out, bt, Hk, Hv, dk, dv, st);
    return launch_dk<64>(q, k, v, beta, g, o, S_in, S_out, bt, Hk, Hv, dk, dv, st);
}

}  // namespace lrc

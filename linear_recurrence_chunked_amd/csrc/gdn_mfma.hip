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
// gamma_S is the last entry of the same cumulative sum; the decay factors
// are formed element by element from differences of gamma.
//
// Work split.  A workgroup (4 waves) owns value head h and a DVT-wide slice
// of dv for one prompt and walks the prompt's chunks.  Wave w owns 16 state
// columns; its [dk x 16] state slice, and its columns of RHS, U and Q S_0,
// stay in MFMA accumulators in registers for the whole prompt.  Only the
// operands every wave needs sit in LDS: the chunk's K, Q, V, K^T, the FP32
// matrix A -> T for the inverse, T and P.  After the inverse no barrier is
// needed until the next chunk.
//
// Matrix cores: v_mfma_f32_16x16x32_bf16, FP32 accumulation.  The A operand
// of lane l is row l%16 with 8 k-values, the B operand column l%16 with the
// same 8 k-values, and the accumulator holds column l%16, rows 4(l/16) .. +3.
// A wave's own [rows x 16] accumulators therefore serve directly as B
// operands when the k-values of lane group g are taken as rows
// {4g .. 4g+3} of one 16-row tile and {16+4g .. 16+4g+3} of the next; the A
// operand then reads the same two 4-element runs of its row from LDS.
// FP32 operands enter as a hi + lo pair of bf16 (hi = bf16(x),
// lo = bf16(x - hi)), about 16 mantissa bits:
//   K K^T, Q K^T        bf16 x bf16 (exact products)            1 pass
//   K S_0, Q S_0        bf16 x (S_0 hi, lo)                     2 passes
//   K^T (d U)           bf16 x (decayed U hi, lo)               2 passes
//   T RHS, P U          (hi, lo) x (hi, lo) without lo x lo     3 passes
// The decay e^{min(gamma_S - gamma_r, 0)} of the state update is applied to
// the rows of U, so K^T enters exact.  The 64-row inverse (8x8 Neumann
// blocks, then 2x2 block levels) runs in FP32 on the vector units.  The next
// chunk's K, Q, V, beta and g are loaded into registers while the current
// chunk computes.
#include "lrc_device.h"
#include "lrc_internal.h"
#include "tri_inverse.h"

namespace lrc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
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
__device__ __forceinline__ void split(float x, __bf16& hi, __bf16& lo) {
    hi = static_cast<__bf16>(x);
    lo = static_cast<__bf16>(x - static_cast<float>(hi));
}

template <int DK, int DVT>
struct MfmaSmem {
    static constexpr int LDK = DK + 8;
    static constexpr int LDV = DVT + 8;
    __bf16 K[64 * LDK];
    __bf16 Q[64 * LDK];
    __bf16 KT[DK * L64];   // K^T, exact
    __bf16 V[64 * LDV];
    __bf16 P_hi[64 * L64];  // masked decayed Q K^T
    __bf16 P_lo[64 * L64];
    __bf16 T_hi[64 * L64];  // (I + A)^-1
    __bf16 T_lo[64 * L64];
    float M[64 * kTriLd];   // A, then T, in FP32
    float scratch[kTriScratch];
    float gam[64];
    float beta[64];
    float decS[64];         // e^{min(gamma_S - gamma_r, 0)}, 0 past the chunk
};

template <int DK, int DVT>
struct Prefetch {
    static constexpr int NK = 64 * DK / 8 / kThreads;    // 16-byte pieces of K (and of Q) per thread
    static constexpr int NV = (64 * DVT / 8 + kThreads - 1) / kThreads;
    uint4 k[NK], q[NK], v[NV];
    float g, beta;
};

template <int DK, int DVT>
__global__ __launch_bounds__(kThreads) void gdn_mfma_kernel(const uint16_t* __restrict__ q,
                                                           const uint16_t* __restrict__ k,
                                                           const uint16_t* __restrict__ v,
                                                           const float* __restrict__ beta,
                                                           const float* __restrict__ g, float* __restrict__ o,
                                                           const float* S_in, float* S_out, Batch bt, int Hk, int Hv,
                                                           int dv) {
    using Sm = MfmaSmem<DK, DVT>;
    using Pf = Prefetch<DK, DVT>;
    constexpr int LDK = Sm::LDK, LDV = Sm::LDV;
    constexpr int KS = DK / 32;   // k-steps over dk
    constexpr int RT = DK / 16;   // state row tiles
    extern __shared__ __align__(16) unsigned char smem_raw[];
    Sm& sm = *reinterpret_cast<Sm*>(smem_raw);

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15;        // fragment row / column within a tile
    const int lg = lane >> 4;        // lane group
    const int lk = lg * 8;           // contiguous fragment k offset
    const int lq = lg * 4;           // accumulator row offset
    const bool owner = 16 * w < DVT; // this wave owns state columns 16w .. 16w+15 of the slice
    const int ntile = dv / DVT;
    const int h = blockIdx.x / ntile;
    const int vt = blockIdx.x % ntile;
    const int kh = h / (Hv / Hk);
    const int p = batch_prompt(bt, blockIdx.y);
    const long row0 = batch_row0(bt, p);
    const int L = batch_len(bt, p);
    const long sbase = ((long)p * Hv + h) * DK * dv + vt * DVT + 16 * w;

    floatx4 sacc[RT];
#pragma unroll
    for (int tr = 0; tr < RT; ++tr)
#pragma unroll
        for (int r = 0; r < 4; ++r) sacc[tr][r] = owner ? S_in[sbase + (long)(16 * tr + lq + r) * dv + lr] : 0.f;

    Pf pf;
    auto fetch = [&](int c0) {
        const int S = min(64, L - c0);
#pragma unroll
        for (int x = 0; x < Pf::NK; ++x) {
            const int e = tid + x * kThreads, r = e / (DK / 8), c8 = (e % (DK / 8)) * 8;
            pf.k[x] = pf.q[x] = make_uint4(0, 0, 0, 0);
            if (r < S) {
                const long off = ((row0 + c0 + r) * Hk + kh) * DK + c8;
                pf.k[x] = *reinterpret_cast<const uint4*>(k + off);
                pf.q[x] = *reinterpret_cast<const uint4*>(q + off);
            }
        }
#pragma unroll
        for (int x = 0; x < Pf::NV; ++x) {
            const int e = tid + x * kThreads, r = e / (DVT / 8), c8 = (e % (DVT / 8)) * 8;
            pf.v[x] = make_uint4(0, 0, 0, 0);
            if (e < 64 * DVT / 8 && r < S)
                pf.v[x] = *reinterpret_cast<const uint4*>(v + ((row0 + c0 + r) * Hv + h) * (long)dv + vt * DVT + c8);
        }
        pf.g = 0.f;
        pf.beta = 0.f;
        if (tid < S) {
            pf.g = g[(row0 + c0 + tid) * Hv + h];
            pf.beta = beta[(row0 + c0 + tid) * Hv + h];
        }
    };

    if (L > 0) fetch(0);
    for (int c0 = 0; c0 < L; c0 += 64) {
        const int S = min(64, L - c0);
        __syncthreads();  // previous chunk done with every LDS buffer
        // ---- stage the prefetched chunk: K, K^T, Q, V, beta, gamma
#pragma unroll
        for (int x = 0; x < Pf::NK; ++x) {
            const int e = tid + x * kThreads, r = e / (DK / 8), c8 = (e % (DK / 8)) * 8;
            *reinterpret_cast<uint4*>(&sm.K[r * LDK + c8]) = pf.k[x];
            *reinterpret_cast<uint4*>(&sm.Q[r * LDK + c8]) = pf.q[x];
            const uint32_t wd[4] = {pf.k[x].x, pf.k[x].y, pf.k[x].z, pf.k[x].w};
            uint16_t* kt = reinterpret_cast<uint16_t*>(sm.KT);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                kt[(c8 + 2 * i) * L64 + r] = uint16_t(wd[i] & 0xffffu);
                kt[(c8 + 2 * i + 1) * L64 + r] = uint16_t(wd[i] >> 16);
            }
        }
#pragma unroll
        for (int x = 0; x < Pf::NV; ++x) {
            const int e = tid + x * kThreads, r = e / (DVT / 8), c8 = (e % (DVT / 8)) * 8;
            if (e < 64 * DVT / 8) *reinterpret_cast<uint4*>(&sm.V[r * LDV + c8]) = pf.v[x];
        }
        if (tid < 64) {
            sm.beta[tid] = pf.beta;
            float x = pf.g;  // inclusive prefix sum over the wave
#pragma unroll
            for (int s = 1; s < 64; s <<= 1) {
                const float y = __shfl_up(x, s, 64);
                if (tid >= s) x += y;
            }
            sm.gam[tid] = x;
            const float gS = __shfl(x, S - 1, 64);
            sm.decS[tid] = tid < S ? fast_exp(fminf(gS - x, 0.f)) : 0.f;
        }
        if (c0 + 64 < L) fetch(c0 + 64);
        __syncthreads();

        // ---- private: K S_0 and Q S_0 for this wave's columns (B from the state accumulators)
        floatx4 ks0[4], qs0[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) ks0[t] = qs0[t] = floatx4{0.f, 0.f, 0.f, 0.f};
        if (owner) {
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                bf16x8 bh, bl;
                acc_frag(sacc[2 * s], sacc[2 * s + 1], bh, bl);
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const bf16x8 ak = frag_perm(&sm.K[(16 * t + lr) * LDK + 32 * s], lg);
                    const bf16x8 aq = frag_perm(&sm.Q[(16 * t + lr) * LDK + 32 * s], lg);
                    ks0[t] = mfma(ak, bh, ks0[t]);
                    ks0[t] = mfma(ak, bl, ks0[t]);
                    qs0[t] = mfma(aq, bh, qs0[t]);
                    qs0[t] = mfma(aq, bl, qs0[t]);
                }
            }
        }
        // ---- shared: K K^T and Q K^T for row tile w -> A (FP32, strictly lower) and P (hi/lo)
#pragma unroll
        for (int tc = 0; tc < 4; ++tc) {
            floatx4 kk = {0.f, 0.f, 0.f, 0.f}, qk = {0.f, 0.f, 0.f, 0.f};
            if (tc <= w) {
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    const bf16x8 bk = frag(&sm.K[(16 * tc + lr) * LDK + 32 * s + lk]);
                    kk = mfma(frag(&sm.K[(16 * w + lr) * LDK + 32 * s + lk]), bk, kk);
                    qk = mfma(frag(&sm.Q[(16 * w + lr) * LDK + 32 * s + lk]), bk, qk);
                }
            }
            const int j = 16 * tc + lr;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * w + lq + r;
                const float dec = i >= j ? fast_exp(sm.gam[i] - sm.gam[j]) : 0.f;
                sm.M[i * kTriLd + j] = i > j ? sm.beta[i] * dec * kk[r] : 0.f;
                split(i >= j ? dec * qk[r] : 0.f, sm.P_hi[i * L64 + j], sm.P_lo[i * L64 + j]);
            }
        }
        // ---- RHS = diag(beta) V - diag(beta Gamma) K S_0 (private, in registers)
        if (owner) {
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * t + lq + r;
                    const float bi = sm.beta[i];
                    ks0[t][r] = bi * static_cast<float>(sm.V[i * LDV + 16 * w + lr]) -
                                bi * fast_exp(sm.gam[i]) * ks0[t][r];
                }
        }
        // ---- T = (I + A)^-1 in FP32 (barriers inside), then T as hi/lo bf16
        tri_inverse64(sm.M, sm.scratch);
        for (int e = tid; e < 64 * 64; e += kThreads) {
            const int r = e >> 6, c = e & 63;
            split(sm.M[r * kTriLd + c], sm.T_hi[r * L64 + c], sm.T_lo[r * L64 + c]);
        }
        __syncthreads();
        if (!owner) continue;

        // ---- U = T RHS (T lower triangular: k-steps up to the row tile's diagonal)
        floatx4 u[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) u[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            bf16x8 bh, bl;
            acc_frag(ks0[2 * s], ks0[2 * s + 1], bh, bl);
#pragma unroll
            for (int t = 2 * s; t < 4; ++t) {
                const bf16x8 ah = frag_perm(&sm.T_hi[(16 * t + lr) * L64 + 32 * s], lg);
                const bf16x8 al = frag_perm(&sm.T_lo[(16 * t + lr) * L64 + 32 * s], lg);
                u[t] = mfma(ah, bh, u[t]);
                u[t] = mfma(ah, bl, u[t]);
                u[t] = mfma(al, bh, u[t]);
            }
        }
        // ---- O = diag(Gamma) Q S_0 + P U for this wave's columns
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
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * t + lq + r;
                    if (i < S)
                        o[((row0 + c0 + i) * Hv + h) * (long)dv + vt * DVT + 16 * w + lr] =
                            fmaf(fast_exp(sm.gam[i]), qs0[t][r], pu[t][r]);
                }
        }
        // ---- S_S = e^{gamma_S} S_0 + K^T (decS * U), in the state accumulators
        {
            const float GS = fast_exp(sm.gam[S - 1]);
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) u[t][r] *= sm.decS[16 * t + lq + r];
#pragma unroll
            for (int tr = 0; tr < RT; ++tr) sacc[tr] = sacc[tr] * GS;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                bf16x8 bh, bl;
                acc_frag(u[2 * s], u[2 * s + 1], bh, bl);
#pragma unroll
                for (int tr = 0; tr < RT; ++tr) {
                    const bf16x8 a = frag_perm(&sm.KT[(16 * tr + lr) * L64 + 32 * s], lg);
                    sacc[tr] = mfma(a, bh, sacc[tr]);
                    sacc[tr] = mfma(a, bl, sacc[tr]);
                }
            }
        }
    }
    if (owner) {
#pragma unroll
        for (int tr = 0; tr < RT; ++tr)
#pragma unroll
            for (int r = 0; r < 4; ++r) S_out[sbase + (long)(16 * tr + lq + r) * dv + lr] = sacc[tr][r];
    }
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
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), smem, st, static_cast<const uint16_t*>(q),
                       static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), beta, g, o, S_in, S_out, bt,
                       Hk, Hv, dv);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gdn_bf16_mfma(const void* q, const void* k, const void* v, const float* beta, const float* g,
                                float* o, const float* S_in, float* S_out, const Batch& bt, int Hk, int Hv, int dk,
                                int dv, hipStream_t st) {
    if (dv >= 64) {
        switch (dk) {
            case 32: return launch_mfma<32, 64>(q, k, v, beta, g, o, S_in, S_out, bt, Hk, Hv, dv, st);
            case 64: return launch_mfma<64, 64>(q, k, v, beta, g, o, S_in, S_out, bt, Hk, Hv, dv, st);
            case 128: return launch_mfma<128, 64>(q, k, v, beta, g, o, S_in, S_out, bt, Hk, Hv, dv, st);
        }
    } else {
        switch (dk) {
            case 32: return launch_mfma<32, 32>(q, k, v, beta, g, o, S_in, S_out, bt, Hk, Hv, dv, st);
            case 64: return launch_mfma<64, 32>(q, k, v, beta, g, o, S_in, S_out, bt, Hk, Hv, dv, st);
            case 128: return launch_mfma<128, 32>(q, k, v, beta, g, o, S_in, S_out, bt, Hk, Hv, dv, st);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace lrc

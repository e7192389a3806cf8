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
// A workgroup (4 waves) owns value head h and a DVT-wide slice of dv for one
// prompt and walks the prompt's chunks.  Its state slice [dk x DVT] lives in
// the accumulators of the state-update product for the whole prompt, and is
// written to HBM once at the end.  Every dense contraction runs on
// v_mfma_f32_16x16x32_bf16 with FP32 accumulation:
//   K K^T, Q K^T         bf16 x bf16 (exact products)
//   K S_0, Q S_0         bf16 x (S_0 as hi + lo bf16 pair)          2 passes
//   T RHS, P U, Kd^T U   (hi + lo) x (hi + lo), dropping lo x lo     3 passes
// where x = hi + lo with hi = bf16(x) and lo = bf16(x - hi) carries about 16
// mantissa bits, so FP32 quantities (state, U, T, P, decayed K) keep near-FP32
// accuracy through bf16 matrix cores.  The 64-row inverse (8x8 Neumann
// blocks, then 2x2 block levels) runs in FP32 on the vector units.
//
// Tiling: 16x16 output tiles.  Operand fragments are 16-byte LDS reads: the
// A operand of lane l is row l%16, k = 8*(l/16) .. +7; the B operand is
// column l%16, the same k; the accumulator holds column l%16, rows
// 4*(l/16) .. +3.  Operands needed as B are kept transposed in LDS (S^T,
// RHS^T / U^T) and the decayed K as Kd^T, so every fragment is contiguous.
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
__device__ __forceinline__ bf16x8 frag(const __bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
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
    __bf16 V[64 * LDV];
    __bf16 ST_hi[DVT * LDK];  // S_0^T
    __bf16 ST_lo[DVT * LDK];
    __bf16 P_hi[64 * L64];    // masked decayed Q K^T
    __bf16 P_lo[64 * L64];
    __bf16 RU_hi[DVT * L64];  // RHS^T, then U^T
    __bf16 RU_lo[DVT * L64];
    union {
        struct {
            float M[64 * kTriLd];  // A, then T, in FP32
            float scratch[kTriScratch];
            __bf16 T_hi[64 * L64];
            __bf16 T_lo[64 * L64];
        } inv;
        struct {
            __bf16 KT_hi[DK * L64];  // (K * decay)^T
            __bf16 KT_lo[DK * L64];
        } st;
    } u;
    float gam[64];
    float beta[64];
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
    constexpr int LDK = Sm::LDK, LDV = Sm::LDV;
    constexpr int NT = DVT / 16;            // column tiles of a [64 x DVT] output
    constexpr int KS = DK / 32;             // k-steps over dk
    constexpr int TS = (DK / 16) * NT;      // state tiles
    constexpr int TPW = TS / 4;             // state tiles per wave
    extern __shared__ __align__(16) unsigned char smem_raw[];
    Sm& sm = *reinterpret_cast<Sm*>(smem_raw);

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15;        // fragment row / column within a tile
    const int lk = (lane >> 4) * 8;  // fragment k offset
    const int lq = (lane >> 4) * 4;  // accumulator row offset
    const int ntile = dv / DVT;
    const int h = blockIdx.x / ntile;
    const int vt = blockIdx.x % ntile;
    const int kh = h / (Hv / Hk);
    const int p = batch_prompt(bt, blockIdx.y);
    const long row0 = batch_row0(bt, p);
    const int L = batch_len(bt, p);
    const long sbase = ((long)p * Hv + h) * DK * dv + vt * DVT;

    // ---- state slice into the accumulators: tile t -> (tr, tc)
    floatx4 sacc[TPW];
#pragma unroll
    for (int x = 0; x < TPW; ++x) {
        const int t = w * TPW + x, tr = t / NT, tc = t % NT;
#pragma unroll
        for (int r = 0; r < 4; ++r) sacc[x][r] = S_in[sbase + (long)(16 * tr + lq + r) * dv + 16 * tc + lr];
    }
    auto export_state = [&]() {
#pragma unroll
        for (int x = 0; x < TPW; ++x) {
            const int t = w * TPW + x, tr = t / NT, tc = t % NT;
            bf16x4 hi, lo;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                __bf16 a, b;
                split(sacc[x][r], a, b);
                hi[r] = a;
                lo[r] = b;
            }
            const int off = (16 * tc + lr) * LDK + 16 * tr + lq;
            *reinterpret_cast<bf16x4*>(&sm.ST_hi[off]) = hi;
            *reinterpret_cast<bf16x4*>(&sm.ST_lo[off]) = lo;
        }
    };
    export_state();

    for (int c0 = 0; c0 < L; c0 += 64) {
        const int S = min(64, L - c0);
        __syncthreads();  // previous chunk done with every buffer
        // ---- stage K, Q [64 x DK], V slice [64 x DVT] (bf16, zero rows past S), beta, gamma
        for (int e = tid; e < 64 * (DK / 8); e += kThreads) {
            const int r = e / (DK / 8), c8 = (e % (DK / 8)) * 8;
            uint4 kv = make_uint4(0, 0, 0, 0), qv = make_uint4(0, 0, 0, 0);
            if (r < S) {
                const long off = ((row0 + c0 + r) * Hk + kh) * DK + c8;
                kv = *reinterpret_cast<const uint4*>(k + off);
                qv = *reinterpret_cast<const uint4*>(q + off);
            }
            *reinterpret_cast<uint4*>(&sm.K[r * LDK + c8]) = kv;
            *reinterpret_cast<uint4*>(&sm.Q[r * LDK + c8]) = qv;
        }
        for (int e = tid; e < 64 * (DVT / 8); e += kThreads) {
            const int r = e / (DVT / 8), c8 = (e % (DVT / 8)) * 8;
            uint4 vv = make_uint4(0, 0, 0, 0);
            if (r < S) vv = *reinterpret_cast<const uint4*>(v + ((row0 + c0 + r) * Hv + h) * (long)dv + vt * DVT + c8);
            *reinterpret_cast<uint4*>(&sm.V[r * LDV + c8]) = vv;
        }
        if (tid < 64) {
            const bool ok = tid < S;
            const float gv = ok ? g[(row0 + c0 + tid) * Hv + h] : 0.f;
            sm.beta[tid] = ok ? beta[(row0 + c0 + tid) * Hv + h] : 0.f;
            float x = gv;  // inclusive prefix sum over the wave
#pragma unroll
            for (int s = 1; s < 64; s <<= 1) {
                const float y = __shfl_up(x, s, 64);
                if (tid >= s) x += y;
            }
            sm.gam[tid] = x;
        }
        __syncthreads();

        // ---- K K^T and Q K^T for row tile w: A (FP32, strictly lower) and P (hi/lo, lower with diagonal)
        for (int tc = 0; tc < 4; ++tc) {
            floatx4 kk = {0.f, 0.f, 0.f, 0.f}, qk = {0.f, 0.f, 0.f, 0.f};
            if (tc <= w) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const bf16x8 bk = frag(&sm.K[(16 * tc + lr) * LDK + 32 * ks + lk]);
                    kk = mfma(frag(&sm.K[(16 * w + lr) * LDK + 32 * ks + lk]), bk, kk);
                    qk = mfma(frag(&sm.Q[(16 * w + lr) * LDK + 32 * ks + lk]), bk, qk);
                }
            }
            const int j = 16 * tc + lr;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * w + lq + r;
                const float dec = i >= j ? fast_exp(sm.gam[i] - sm.gam[j]) : 0.f;
                sm.u.inv.M[i * kTriLd + j] = i > j ? sm.beta[i] * dec * kk[r] : 0.f;
                __bf16 hi, lo;
                split(i >= j ? dec * qk[r] : 0.f, hi, lo);
                sm.P_hi[i * L64 + j] = hi;
                sm.P_lo[i * L64 + j] = lo;
            }
        }
        // ---- T = (I + A)^-1 in FP32 (barriers inside), then T as hi/lo bf16
        tri_inverse64(sm.u.inv.M, sm.u.inv.scratch);
        for (int e = tid; e < 64 * 64; e += kThreads) {
            const int r = e >> 6, c = e & 63;
            split(sm.u.inv.M[r * kTriLd + c], sm.u.inv.T_hi[r * L64 + c], sm.u.inv.T_lo[r * L64 + c]);
        }
        // ---- RHS = diag(beta) V - diag(beta Gamma) K S_0, stored as RHS^T (hi/lo)
        {
            floatx4 acc[NT];
#pragma unroll
            for (int tc = 0; tc < NT; ++tc) {
                acc[tc] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const bf16x8 a = frag(&sm.K[(16 * w + lr) * LDK + 32 * ks + lk]);
                    acc[tc] = mfma(a, frag(&sm.ST_hi[(16 * tc + lr) * LDK + 32 * ks + lk]), acc[tc]);
                    acc[tc] = mfma(a, frag(&sm.ST_lo[(16 * tc + lr) * LDK + 32 * ks + lk]), acc[tc]);
                }
            }
#pragma unroll
            for (int tc = 0; tc < NT; ++tc) {
                const int j = 16 * tc + lr;
                bf16x4 hi, lo;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * w + lq + r;
                    const float bi = sm.beta[i];
                    const float rhs = bi * static_cast<float>(sm.V[i * LDV + j]) - bi * fast_exp(sm.gam[i]) * acc[tc][r];
                    __bf16 a, b;
                    split(rhs, a, b);
                    hi[r] = a;
                    lo[r] = b;
                }
                *reinterpret_cast<bf16x4*>(&sm.RU_hi[j * L64 + 16 * w + lq]) = hi;
                *reinterpret_cast<bf16x4*>(&sm.RU_lo[j * L64 + 16 * w + lq]) = lo;
            }
        }
        __syncthreads();  // T and RHS^T complete
        // ---- U = T RHS (T lower triangular: k-steps up to the diagonal), then U^T over RHS^T
        {
            const int nks = (16 * w + 16 + 31) / 32;
            floatx4 acc[NT];
#pragma unroll
            for (int tc = 0; tc < NT; ++tc) acc[tc] = floatx4{0.f, 0.f, 0.f, 0.f};
            for (int ks = 0; ks < nks; ++ks) {
                const bf16x8 ah = frag(&sm.u.inv.T_hi[(16 * w + lr) * L64 + 32 * ks + lk]);
                const bf16x8 al = frag(&sm.u.inv.T_lo[(16 * w + lr) * L64 + 32 * ks + lk]);
#pragma unroll
                for (int tc = 0; tc < NT; ++tc) {
                    const bf16x8 bh = frag(&sm.RU_hi[(16 * tc + lr) * L64 + 32 * ks + lk]);
                    const bf16x8 bl = frag(&sm.RU_lo[(16 * tc + lr) * L64 + 32 * ks + lk]);
                    acc[tc] = mfma(ah, bh, acc[tc]);
                    acc[tc] = mfma(ah, bl, acc[tc]);
                    acc[tc] = mfma(al, bh, acc[tc]);
                }
            }
            __syncthreads();  // every read of RHS^T and T is done
#pragma unroll
            for (int tc = 0; tc < NT; ++tc) {
                const int j = 16 * tc + lr;
                bf16x4 hi, lo;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    __bf16 a, b;
                    split(acc[tc][r], a, b);
                    hi[r] = a;
                    lo[r] = b;
                }
                *reinterpret_cast<bf16x4*>(&sm.RU_hi[j * L64 + 16 * w + lq]) = hi;
                *reinterpret_cast<bf16x4*>(&sm.RU_lo[j * L64 + 16 * w + lq]) = lo;
            }
        }
        // ---- (K * e^{min(gamma_S - gamma, 0)})^T as hi/lo, over the inverse's buffers
        {
            const float gS = sm.gam[S - 1];
            for (int e = tid; e < DK * 64; e += kThreads) {
                const int i = e >> 6, r = e & 63;  // KT[i][r] = K[r][i] * dec_r
                const float dec = r < S ? fast_exp(fminf(gS - sm.gam[r], 0.f)) : 0.f;
                split(static_cast<float>(sm.K[r * LDK + i]) * dec, sm.u.st.KT_hi[i * L64 + r], sm.u.st.KT_lo[i * L64 + r]);
            }
        }
        __syncthreads();  // U^T and Kd^T complete
        // ---- O = diag(Gamma) Q S_0 + P U for row tile w
        {
            const int nks = (16 * w + 16 + 31) / 32;
            floatx4 qs[NT], pu[NT];
#pragma unroll
            for (int tc = 0; tc < NT; ++tc) {
                qs[tc] = floatx4{0.f, 0.f, 0.f, 0.f};
                pu[tc] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const bf16x8 a = frag(&sm.Q[(16 * w + lr) * LDK + 32 * ks + lk]);
                    qs[tc] = mfma(a, frag(&sm.ST_hi[(16 * tc + lr) * LDK + 32 * ks + lk]), qs[tc]);
                    qs[tc] = mfma(a, frag(&sm.ST_lo[(16 * tc + lr) * LDK + 32 * ks + lk]), qs[tc]);
                }
            }
            for (int ks = 0; ks < nks; ++ks) {
                const bf16x8 ah = frag(&sm.P_hi[(16 * w + lr) * L64 + 32 * ks + lk]);
                const bf16x8 al = frag(&sm.P_lo[(16 * w + lr) * L64 + 32 * ks + lk]);
#pragma unroll
                for (int tc = 0; tc < NT; ++tc) {
                    const bf16x8 bh = frag(&sm.RU_hi[(16 * tc + lr) * L64 + 32 * ks + lk]);
                    const bf16x8 bl = frag(&sm.RU_lo[(16 * tc + lr) * L64 + 32 * ks + lk]);
                    pu[tc] = mfma(ah, bh, pu[tc]);
                    pu[tc] = mfma(ah, bl, pu[tc]);
                    pu[tc] = mfma(al, bh, pu[tc]);
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * w + lq + r;
                if (i < S) {
                    const float G = fast_exp(sm.gam[i]);
                    float* orow = o + ((row0 + c0 + i) * Hv + h) * (long)dv + vt * DVT + lr;
#pragma unroll
                    for (int tc = 0; tc < NT; ++tc) orow[16 * tc] = fmaf(G, qs[tc][r], pu[tc][r]);
                }
            }
        }
        // ---- S_S = e^{gamma_S} S_0 + Kd^T U in the accumulators; export S^T for the next chunk
        {
            const float GS = fast_exp(sm.gam[S - 1]);
#pragma unroll
            for (int x = 0; x < TPW; ++x) {
                const int t = w * TPW + x, tr = t / NT, tc = t % NT;
                floatx4 acc = sacc[x] * GS;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const bf16x8 ah = frag(&sm.u.st.KT_hi[(16 * tr + lr) * L64 + 32 * ks + lk]);
                    const bf16x8 al = frag(&sm.u.st.KT_lo[(16 * tr + lr) * L64 + 32 * ks + lk]);
                    const bf16x8 bh = frag(&sm.RU_hi[(16 * tc + lr) * L64 + 32 * ks + lk]);
                    const bf16x8 bl = frag(&sm.RU_lo[(16 * tc + lr) * L64 + 32 * ks + lk]);
                    acc = mfma(ah, bh, acc);
                    acc = mfma(ah, bl, acc);
                    acc = mfma(al, bh, acc);
                }
                sacc[x] = acc;
            }
            __syncthreads();  // every read of S_0^T (Q S_0 above) is done
            export_state();
        }
    }
#pragma unroll
    for (int x = 0; x < TPW; ++x) {
        const int t = w * TPW + x, tr = t / NT, tc = t % NT;
#pragma unroll
        for (int r = 0; r < 4; ++r) S_out[sbase + (long)(16 * tr + lq + r) * dv + 16 * tc + lr] = sacc[x][r];
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

// K3: Gated DeltaNet chunked delta rule, on gfx950.
//
// Source: "perf(qwen3_5): prefill text prompts in multi-token chunks",
// Implementation.  For a chunk of S <= 64 rows of value head h (key head
// h / (Hv/Hk)), with gamma the chunk-local inclusive cumulative sum of g and
// Gamma = e^gamma:
//   A_ij = beta_i e^{gamma_i - gamma_j} k_i.k_j  (j < i)
//   U    = (I + A)^-1 (diag(beta) V - diag(beta Gamma) K S_0)
//   O    = diag(Gamma) Q S_0 + (e^{gamma_t - gamma_i} q_t.k_i)_{i <= t} U
//   S_S  = e^{gamma_S} S_0 + (K * e^{min(gamma_S - gamma, 0)})^T U
// gamma_S is the last entry of the same cumulative sum; decay factors are
// formed element by element from differences of gamma (never as ratios of
// Gamma, which under- and overflow at large decays).
//
// This file holds the FP32-input path (bf16 inputs run on the matrix cores,
// in gdn_mfma.hip): every contraction is an FP32 FMA loop over tiles staged
// in LDS.  A workgroup owns one value head and a DVT-wide slice
// of dv for one prompt, keeps that slice of the state resident in LDS while
// it walks the prompt's chunks, and writes the state back once at the end.
#include "lrc_device.h"
#include "lrc_internal.h"
#include "tri_inverse.h"

namespace lrc {
namespace {

constexpr int kThreads = 256;

template <typename T>
__device__ __forceinline__ float to_f32(T x);
template <>
__device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ float to_f32<uint16_t>(uint16_t x) { return bf16_to_f32(x); }

// Inclusive prefix sum over the 64 lanes of one wave.
__device__ __forceinline__ float wave_inclusive_sum(float x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int k = 1; k < 64; k <<= 1) {
        const float y = __shfl_up(x, k, 64);
        if (lane >= k) x += y;
    }
    return x;
}

template <int DK, int DVT>
struct GdnSmem {
    static constexpr int LDK = DK + 4;    // row stride of K and Q tiles
    static constexpr int LDV = DVT + 4;   // row stride of V / U tiles and of the state slice
    float K[64 * LDK];
    float Q[64 * LDK];
    float U[64 * LDV];
    float S[DK * LDV];
    float M[64 * kTriLd];   // A, then T
    float P[64 * kTriLd];   // masked, decayed Q K^T
    float scratch[kTriScratch];
    float gam[64];
    float beta[64];
};

template <typename TIN, int DK, int DVT>
__global__ __launch_bounds__(kThreads) void gdn_f32_kernel(const TIN* __restrict__ q, const TIN* __restrict__ k,
                                                          const TIN* __restrict__ v, const float* __restrict__ beta,
                                                          const float* __restrict__ g, float* __restrict__ o,
                                                          const float* S_in, float* S_out, Batch bt, int Hk, int Hv,
                                                          int dv) {
    using Sm = GdnSmem<DK, DVT>;
    constexpr int LDK = Sm::LDK, LDV = Sm::LDV;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    Sm& sm = *reinterpret_cast<Sm*>(smem_raw);

    const int tid = threadIdx.x;
    const int ntile = dv / DVT;
    const int h = blockIdx.x / ntile;
    const int vt = blockIdx.x % ntile;
    const int kh = h / (Hv / Hk);
    const int p = batch_prompt(bt, blockIdx.y);
    const long row0 = batch_row0(bt, p);
    const int L = batch_len(bt, p);

    // State slice S[:, vt*DVT : (vt+1)*DVT] of (prompt p, head h).
    const long sbase = ((long)p * Hv + h) * DK * dv + vt * DVT;
    for (int e = tid; e < DK * DVT; e += kThreads) {
        const int r = e / DVT, c = e % DVT;
        sm.S[r * LDV + c] = S_in[sbase + (long)r * dv + c];
    }

    // Thread tiles: rows 4*ti .. 4*ti+3 of a 64-row operand, CPT columns.
    const int ti = tid >> 4, tj = tid & 15;
    constexpr int CPT = DVT / 16;   // columns of a [64 x DVT] output per thread
    constexpr int RPS = DK / 16;    // state rows per thread

    for (int c0 = 0; c0 < L; c0 += 64) {
        const int S = min(64, L - c0);
        __syncthreads();  // previous chunk finished with every tile
        // ---- stage the chunk: K, Q [64 x DK], V slice [64 x DVT], beta, g
        for (int e = tid; e < 64 * DK; e += kThreads) {
            const int r = e / DK, d = e % DK;
            float kv = 0.f, qv = 0.f;
            if (r < S) {
                const long off = ((row0 + c0 + r) * Hk + kh) * DK + d;
                kv = to_f32(k[off]);
                qv = to_f32(q[off]);
            }
            sm.K[r * LDK + d] = kv;
            sm.Q[r * LDK + d] = qv;
        }
        for (int e = tid; e < 64 * DVT; e += kThreads) {
            const int r = e / DVT, c = e % DVT;
            sm.U[r * LDV + c] = r < S ? to_f32(v[((row0 + c0 + r) * Hv + h) * (long)dv + vt * DVT + c]) : 0.f;
        }
        if (tid < 64) {
            const bool ok = tid < S;
            const float gv = ok ? g[(row0 + c0 + tid) * Hv + h] : 0.f;
            sm.beta[tid] = ok ? beta[(row0 + c0 + tid) * Hv + h] : 0.f;
            sm.gam[tid] = wave_inclusive_sum(gv);
        }
        __syncthreads();

        // ---- A (strictly lower) and P (lower with diagonal) from K K^T and Q K^T
        {
            float kk[4][4] = {}, qk[4][4] = {};
            if (tj <= ti) {
                for (int d = 0; d < DK; d += 4) {
                    float4 ki[4], qi[4], kj[4];
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        ki[a] = *reinterpret_cast<const float4*>(&sm.K[(4 * ti + a) * LDK + d]);
                        qi[a] = *reinterpret_cast<const float4*>(&sm.Q[(4 * ti + a) * LDK + d]);
                        kj[a] = *reinterpret_cast<const float4*>(&sm.K[(4 * tj + a) * LDK + d]);
                    }
#pragma unroll
                    for (int a = 0; a < 4; ++a)
#pragma unroll
                        for (int b = 0; b < 4; ++b) {
                            kk[a][b] = fmaf(ki[a].x, kj[b].x, kk[a][b]);
                            kk[a][b] = fmaf(ki[a].y, kj[b].y, kk[a][b]);
                            kk[a][b] = fmaf(ki[a].z, kj[b].z, kk[a][b]);
                            kk[a][b] = fmaf(ki[a].w, kj[b].w, kk[a][b]);
                            qk[a][b] = fmaf(qi[a].x, kj[b].x, qk[a][b]);
                            qk[a][b] = fmaf(qi[a].y, kj[b].y, qk[a][b]);
                            qk[a][b] = fmaf(qi[a].z, kj[b].z, qk[a][b]);
                            qk[a][b] = fmaf(qi[a].w, kj[b].w, qk[a][b]);
                        }
                }
            }
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int i = 4 * ti + a, j = 4 * tj + b;
                    const float dec = i >= j ? fast_exp(sm.gam[i] - sm.gam[j]) : 0.f;
                    sm.M[i * kTriLd + j] = i > j ? sm.beta[i] * dec * kk[a][b] : 0.f;
                    sm.P[i * kTriLd + j] = i >= j ? dec * qk[a][b] : 0.f;
                }
        }
        // ---- T = (I + A)^-1 (barriers inside)
        tri_inverse64<kThreads / 64>(sm.M, sm.scratch);

        // ---- RHS = diag(beta) V - diag(beta Gamma) K S_0, in registers
        float rhs[4][CPT];
        {
            float ks[4][CPT] = {};
            for (int d = 0; d < DK; ++d) {
                float sv[CPT];
#pragma unroll
                for (int c = 0; c < CPT; ++c) sv[c] = sm.S[d * LDV + tj * CPT + c];
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const float kv = sm.K[(4 * ti + a) * LDK + d];
#pragma unroll
                    for (int c = 0; c < CPT; ++c) ks[a][c] = fmaf(kv, sv[c], ks[a][c]);
                }
            }
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int i = 4 * ti + a;
                const float bi = sm.beta[i];
                const float bg = bi * fast_exp(sm.gam[i]);
#pragma unroll
                for (int c = 0; c < CPT; ++c) rhs[a][c] = bi * sm.U[i * LDV + tj * CPT + c] - bg * ks[a][c];
            }
        }
        __syncthreads();  // every read of V is done
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int c = 0; c < CPT; ++c) sm.U[(4 * ti + a) * LDV + tj * CPT + c] = rhs[a][c];
        __syncthreads();
        // ---- U = T RHS (T lower triangular with unit diagonal)
        {
            float u[4][CPT] = {};
            for (int m = 0; m < 4 * ti + 4; ++m) {
                float rv[CPT];
#pragma unroll
                for (int c = 0; c < CPT; ++c) rv[c] = sm.U[m * LDV + tj * CPT + c];
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const float t = sm.M[(4 * ti + a) * kTriLd + m];
#pragma unroll
                    for (int c = 0; c < CPT; ++c) u[a][c] = fmaf(t, rv[c], u[a][c]);
                }
            }
            __syncthreads();  // every read of RHS is done
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int c = 0; c < CPT; ++c) sm.U[(4 * ti + a) * LDV + tj * CPT + c] = u[a][c];
        }
        __syncthreads();
        // ---- O = diag(Gamma) Q S_0 + P U
        {
            float qs[4][CPT] = {}, pu[4][CPT] = {};
            for (int d = 0; d < DK; ++d) {
                float sv[CPT];
#pragma unroll
                for (int c = 0; c < CPT; ++c) sv[c] = sm.S[d * LDV + tj * CPT + c];
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const float qv = sm.Q[(4 * ti + a) * LDK + d];
#pragma unroll
                    for (int c = 0; c < CPT; ++c) qs[a][c] = fmaf(qv, sv[c], qs[a][c]);
                }
            }
            for (int m = 0; m < 4 * ti + 4; ++m) {
                float uv[CPT];
#pragma unroll
                for (int c = 0; c < CPT; ++c) uv[c] = sm.U[m * LDV + tj * CPT + c];
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const float pv = sm.P[(4 * ti + a) * kTriLd + m];
#pragma unroll
                    for (int c = 0; c < CPT; ++c) pu[a][c] = fmaf(pv, uv[c], pu[a][c]);
                }
            }
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int i = 4 * ti + a;
                if (i < S) {
                    const float G = fast_exp(sm.gam[i]);
                    float* orow = o + ((row0 + c0 + i) * Hv + h) * (long)dv + vt * DVT + tj * CPT;
#pragma unroll
                    for (int c = 0; c < CPT; ++c) orow[c] = fmaf(G, qs[a][c], pu[a][c]);
                }
            }
        }
        // ---- S_S = e^{gamma_S} S_0 + (K * e^{min(gamma_S - gamma, 0)})^T U
        {
            const float gS = sm.gam[S - 1];
            const float GS = fast_exp(gS);
            float acc[RPS][CPT];
#pragma unroll
            for (int r = 0; r < RPS; ++r)
#pragma unroll
                for (int c = 0; c < CPT; ++c) acc[r][c] = GS * sm.S[(ti * RPS + r) * LDV + tj * CPT + c];
            for (int m = 0; m < S; ++m) {
                const float dec = fast_exp(fminf(gS - sm.gam[m], 0.f));
                float uv[CPT];
#pragma unroll
                for (int c = 0; c < CPT; ++c) uv[c] = sm.U[m * LDV + tj * CPT + c];
#pragma unroll
                for (int r = 0; r < RPS; ++r) {
                    const float kd = sm.K[m * LDK + ti * RPS + r] * dec;
#pragma unroll
                    for (int c = 0; c < CPT; ++c) acc[r][c] = fmaf(kd, uv[c], acc[r][c]);
                }
            }
            __syncthreads();  // every read of S_0 is done
#pragma unroll
            for (int r = 0; r < RPS; ++r)
#pragma unroll
                for (int c = 0; c < CPT; ++c) sm.S[(ti * RPS + r) * LDV + tj * CPT + c] = acc[r][c];
        }
    }
    __syncthreads();
    for (int e = tid; e < DK * DVT; e += kThreads) {
        const int r = e / DVT, c = e % DVT;
        S_out[sbase + (long)r * dv + c] = sm.S[r * LDV + c];
    }
}

template <typename TIN, int DK, int DVT>
hipError_t launch_f32_path(const void* q, const void* k, const void* v, const float* beta, const float* g, float* o,
                           const float* S_in, float* S_out, const Batch& bt, int Hk, int Hv, int dv, hipStream_t st) {
    auto kern = gdn_f32_kernel<TIN, DK, DVT>;
    const size_t smem = sizeof(GdnSmem<DK, DVT>);
    // Opt in to more than 64 KiB of LDS once per process (a thread-safe static).
    static const hipError_t configured = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (configured != hipSuccess) return configured;
    const dim3 grid((unsigned)(Hv * (dv / DVT)), (unsigned)bt.P);
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), smem, st, static_cast<const TIN*>(q), static_cast<const TIN*>(k),
                       static_cast<const TIN*>(v), beta, g, o, S_in, S_out, bt, Hk, Hv, dv);
    return hipGetLastError();
}

template <typename TIN>
hipError_t dispatch_dk(const void* q, const void* k, const void* v, const float* beta, const float* g, float* o,
                       const float* S_in, float* S_out, const Batch& bt, int Hk, int Hv, int dk, int dv,
                       hipStream_t st) {
    // DVT = 64 when dv allows, else 32.
    if (dv >= 64) {
        switch (dk) {
            case 32: return launch_f32_path<TIN, 32, 64>(q, k, v, beta, g, o, S_in, S_out, bt, Hk, Hv, dv, st);
            case 64: return launch_f32_path<TIN, 64, 64>(q, k, v, beta, g, o, S_in, S_out, bt, Hk, Hv, dv, st);
            case 128: return launch_f32_path<TIN, 128, 64>(q, k, v, beta, g, o, S_in, S_out, bt, Hk, Hv, dv, st);
        }
    } else {
        switch (dk) {
            case 32: return launch_f32_path<TIN, 32, 32>(q, k, v, beta, g, o, S_in, S_out, bt, Hk, Hv, dv, st);
            case 64: return launch_f32_path<TIN, 64, 32>(q, k, v, beta, g, o, S_in, S_out, bt, Hk, Hv, dv, st);
            case 128: return launch_f32_path<TIN, 128, 32>(q, k, v, beta, g, o, S_in, S_out, bt, Hk, Hv, dv, st);
        }
    }
    return hipErrorInvalidValue;
}

// Standalone inverse: one workgroup per matrix.
__global__ __launch_bounds__(kThreads) void tri_inverse_kernel(const float* __restrict__ A, float* __restrict__ T,
                                                              int n) {
    __shared__ __align__(16) float M[64 * kTriLd];
    __shared__ __align__(16) float scratch[kTriScratch];
    const long base = (long)blockIdx.x * n * n;
    for (int e = threadIdx.x; e < 64 * 64; e += kThreads) {
        const int r = e >> 6, c = e & 63;
        M[r * kTriLd + c] = (r < n && c < r) ? A[base + (long)r * n + c] : 0.f;
    }
    tri_inverse64<kThreads / 64>(M, scratch);
    for (int e = threadIdx.x; e < n * n; e += kThreads) {
        const int r = e / n, c = e % n;
        T[base + e] = M[r * kTriLd + c];
    }
}

}  // namespace

hipError_t launch_gdn(const void* q, const void* k, const void* v, const float* beta, const float* g, float* o,
                      const float* S_in, float* S_out, const Batch& bt, int Hk, int Hv, int dk, int dv, lrc_dtype dt,
                      hipStream_t st) {
    if (dt == LRC_BF16 || dt == LRC_BF16_SPLIT)
        return launch_gdn_bf16_mfma(q, k, v, beta, g, o, S_in, S_out, bt, Hk, Hv, dk, dv, dt == LRC_BF16_SPLIT, st);
    return dispatch_dk<float>(q, k, v, beta, g, o, S_in, S_out, bt, Hk, Hv, dk, dv, st);
}

hipError_t launch_unit_lower_inverse(const float* A, float* T, int batch, int n, hipStream_t st) {
    hipLaunchKernelGGL(tri_inverse_kernel, dim3((unsigned)batch), dim3(kThreads), 0, st, A, T, n);
    return hipGetLastError();
}

}  // namespace lrc

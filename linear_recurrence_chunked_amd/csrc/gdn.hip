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
// This file holds the FP32-input path (bf16 inputs run on the bf16 matrix
// cores, in gdn_mfma.hip): every contraction is a product of 16x16 tiles
// staged in LDS, on the FP32 matrix cores (v_mfma_f32_16x16x4f32) with FP32
// accumulation.  A workgroup owns one value head and a DVT-wide slice
// of dv for one prompt, keeps that slice of the state resident in LDS while
// it walks the prompt's chunks, and writes the state back once at the end.
#include "lrc_device.h"
#include "lrc_internal.h"
#include "tri_inverse.h"

namespace lrc {
namespace {

constexpr int kThreads = 256;       // the standalone inverse
constexpr int kChunkThreads = 1024;  // the chunk kernel: four waves per SIMD

template <typename T>
__device__ __forceinline__ float to_f32(T x);
template <>
__device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ float to_f32<uint16_t>(uint16_t x) { return bf16_to_f32(x); }

// Lower-triangular 16x16 tile pair pr = 0 .. 9 (row tile ti, column tile tj)
// of a 64x64 matrix, row by row: (0,0), (1,0), (1,1), (2,0), ...
__device__ __forceinline__ void tile_pair(int pr, int& ti, int& tj) {
    ti = (pr >= 1) + (pr >= 3) + (pr >= 6);
    tj = pr - ti * (ti + 1) / 2;
}

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
    alignas(16) float decS[64];  // e^{min(gamma_S - gamma_r, 0)}
};

template <typename TIN, int DK, int DVT>
__global__ __launch_bounds__(kChunkThreads) void gdn_f32_kernel(const TIN* __restrict__ q, const TIN* __restrict__ k,
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
    for (int e = tid; e < DK * DVT; e += kChunkThreads) {
        const int r = e / DVT, c = e % DVT;
        sm.S[r * LDV + c] = S_in[sbase + (long)r * dv + c];
    }

    // Products run as 16x16 tiles on the FP32 matrix cores, dealt to the waves.
    constexpr int kWaves = kChunkThreads / 64;
    constexpr int NCT = DVT / 16;                      // column tiles of a [64 x DVT] operand
    constexpr int NT = 4 * NCT, NS = (DK / 16) * NCT;  // [64 x DVT] tiles, state tiles
    constexpr int TPW = (NT + kWaves - 1) / kWaves;    // per wave, the last ones maybe idle
    constexpr int SPW = (NS + kWaves - 1) / kWaves;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    int lr, lg;
    tri::lanes(lr, lg);
    const tri_f4 zero4 = {0.f, 0.f, 0.f, 0.f};
    // Tiles above the diagonal of A (then T) and P stay zero for the whole prompt.
    for (int e = tid; e < 64 * kTriLd; e += kChunkThreads) sm.M[e] = sm.P[e] = 0.f;

    for (int c0 = 0; c0 < L; c0 += 64) {
        const int S = min(64, L - c0);
        __syncthreads();  // previous chunk finished with every tile
        // ---- stage the chunk: K, Q [64 x DK], V slice [64 x DVT], beta, g
        for (int e = tid; e < 64 * DK; e += kChunkThreads) {
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
        for (int e = tid; e < 64 * DVT; e += kChunkThreads) {
            const int r = e / DVT, c = e % DVT;
            sm.U[r * LDV + c] = r < S ? to_f32(v[((row0 + c0 + r) * Hv + h) * (long)dv + vt * DVT + c]) : 0.f;
        }
        if (tid < 64) {
            const bool ok = tid < S;
            const float gv = ok ? g[(row0 + c0 + tid) * Hv + h] : 0.f;
            sm.beta[tid] = ok ? beta[(row0 + c0 + tid) * Hv + h] : 0.f;
            const float x = wave_inclusive_sum(gv);
            sm.gam[tid] = x;
            sm.decS[tid] = fast_exp(fminf(__shfl(x, S - 1, 64) - x, 0.f));  // 1 past the chunk
        }
        __syncthreads();

        // ---- A (strictly lower) and P (lower with diagonal) from K K^T and Q K^T:
        //      the 10 lower 16x16 tiles of each, over the waves
        for (int x = w; x < 20; x += kWaves) {
            const bool isq = x >= 10;
            int ti, tj;
            tile_pair(isq ? x - 10 : x, ti, tj);
            const float* X = (isq ? sm.Q : sm.K) + 16 * ti * LDK;
            const float* Y = sm.K + 16 * tj * LDK;
            tri_f4 acc = zero4;
#pragma unroll 4
            for (int kc = 0; kc < DK; kc += 16)
                acc = tri::mm(acc, tri::ld_row(X + kc, LDK, lr, lg), tri::ld_row(Y + kc, LDK, lr, lg));
            const int j = 16 * tj + lr;
#pragma unroll
            for (int r = 0; r < 4; ++r) {  // acc[r] is row 16 ti + 4 g + r, column j
                const int i = 16 * ti + 4 * lg + r;
                const float dec = i >= j ? fast_exp(sm.gam[i] - sm.gam[j]) : 0.f;
                if (isq)
                    sm.P[i * kTriLd + j] = dec * acc[r];
                else
                    sm.M[i * kTriLd + j] = i > j ? sm.beta[i] * dec * acc[r] : 0.f;
            }
        }
        // ---- T = (I + A)^-1 (barriers inside)
        tri_inverse64<kChunkThreads / 64>(sm.M, sm.scratch);

        // ---- RHS = diag(beta) V - diag(beta Gamma) K S_0 by [16 x 16] tiles, in registers
        tri_f4 rhs[TPW];
#pragma unroll
        for (int y = 0; y < TPW; ++y) {
            const int x = w + kWaves * y, ti = x / NCT, tc = x % NCT;
            if (x >= NT) continue;
            tri_f4 acc = zero4;
#pragma unroll 4
            for (int kc = 0; kc < DK; kc += 16)
                acc = tri::mm(acc, tri::ld_row(sm.K + 16 * ti * LDK + kc, LDK, lr, lg),
                              tri::ld_acc(sm.S + kc * LDV + 16 * tc, LDV, lr, lg));
            const int c = 16 * tc + lr;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * ti + 4 * lg + r;
                const float bi = sm.beta[i];
                rhs[y][r] = bi * sm.U[i * LDV + c] - bi * fast_exp(sm.gam[i]) * acc[r];
            }
        }
        __syncthreads();  // every read of V is done
#pragma unroll
        for (int y = 0; y < TPW; ++y) {
            const int x = w + kWaves * y, ti = x / NCT, tc = x % NCT;
            if (x >= NT) continue;
            tri::st_acc(sm.U + 16 * ti * LDV + 16 * tc, LDV, lr, lg, rhs[y]);
        }
        __syncthreads();
        // ---- U = T RHS (T lower triangular: tiles up to the diagonal)
        {
            tri_f4 u[TPW];
#pragma unroll
            for (int y = 0; y < TPW; ++y) {
                const int x = w + kWaves * y, ti = x / NCT, tc = x % NCT;
                if (x >= NT) continue;
                tri_f4 acc = zero4;
                for (int tk = 0; tk <= ti; ++tk)
                    acc = tri::mm(acc, tri::ld_row(sm.M + 16 * ti * kTriLd + 16 * tk, kTriLd, lr, lg),
                                  tri::ld_acc(sm.U + 16 * tk * LDV + 16 * tc, LDV, lr, lg));
                u[y] = acc;
            }
            __syncthreads();  // every read of RHS is done
#pragma unroll
            for (int y = 0; y < TPW; ++y) {
                const int x = w + kWaves * y, ti = x / NCT, tc = x % NCT;
                if (x >= NT) continue;
                tri::st_acc(sm.U + 16 * ti * LDV + 16 * tc, LDV, lr, lg, u[y]);
            }
        }
        __syncthreads();
        // ---- O = diag(Gamma) Q S_0 + P U
#pragma unroll
        for (int y = 0; y < TPW; ++y) {
            const int x = w + kWaves * y, ti = x / NCT, tc = x % NCT;
            if (x >= NT) continue;
            tri_f4 qs = zero4, pu = zero4;
#pragma unroll 4
            for (int kc = 0; kc < DK; kc += 16)
                qs = tri::mm(qs, tri::ld_row(sm.Q + 16 * ti * LDK + kc, LDK, lr, lg),
                             tri::ld_acc(sm.S + kc * LDV + 16 * tc, LDV, lr, lg));
            for (int tk = 0; tk <= ti; ++tk)
                pu = tri::mm(pu, tri::ld_row(sm.P + 16 * ti * kTriLd + 16 * tk, kTriLd, lr, lg),
                             tri::ld_acc(sm.U + 16 * tk * LDV + 16 * tc, LDV, lr, lg));
            const int c = vt * DVT + 16 * tc + lr;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * ti + 4 * lg + r;
                if (i < S) o[((row0 + c0 + i) * Hv + h) * (long)dv + c] = fmaf(fast_exp(sm.gam[i]), qs[r], pu[r]);
            }
        }
        // ---- S_S = e^{gamma_S} S_0 + (K * e^{min(gamma_S - gamma, 0)})^T U; rows past the chunk
        //      add nothing (their K and U rows are zero)
        {
            const float GS = fast_exp(sm.gam[S - 1]);
            tri_f4 acc[SPW];
#pragma unroll
            for (int y = 0; y < SPW; ++y) {
                const int x = w + kWaves * y, td = x / NCT, tc = x % NCT;
                if (x >= NS) continue;
                acc[y] = GS * tri::ld_acc(sm.S + 16 * td * LDV + 16 * tc, LDV, lr, lg);
#pragma unroll
                for (int mc = 0; mc < 64; mc += 16) {
                    const tri_f4 d4 = *reinterpret_cast<const tri_f4*>(&sm.decS[mc + 4 * lg]);
                    acc[y] = tri::mm(acc[y], d4 * tri::ld_acc(sm.K + mc * LDK + 16 * td, LDK, lr, lg),
                                     tri::ld_acc(sm.U + mc * LDV + 16 * tc, LDV, lr, lg));
                }
            }
            __syncthreads();  // every read of S_0 is done
#pragma unroll
            for (int y = 0; y < SPW; ++y) {
                const int x = w + kWaves * y, td = x / NCT, tc = x % NCT;
                if (x >= NS) continue;
                tri::st_acc(sm.S + 16 * td * LDV + 16 * tc, LDV, lr, lg, acc[y]);
            }
        }
    }
    __syncthreads();
    for (int e = tid; e < DK * DVT; e += kChunkThreads) {
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
    hipLaunchKernelGGL(kern, grid, dim3(kChunkThreads), smem, st, static_cast<const TIN*>(q), static_cast<const TIN*>(k),
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

// Standalone inverse: one workgroup per matrix, the phases of the bf16 chunk
// kernel (diagonal tiles on the vector ALUs) with the level products on the
// FP32 matrix cores.
__global__ __launch_bounds__(kThreads) void tri_inverse_kernel(const float* __restrict__ A, float* __restrict__ T,
                                                              int n) {
    constexpr int NW = kThreads / 64;
    __shared__ __align__(16) float M[64 * kTriLd];
    __shared__ __align__(16) float scratch[kTriScratch];
    __shared__ __align__(16) float dscratch[NW * tri::kDiagScratch];
    const long base = (long)blockIdx.x * n * n;
    for (int e = threadIdx.x; e < 64 * 64; e += kThreads) {
        const int r = e >> 6, c = e & 63;
        M[r * kTriLd + c] = (r < n && c < r) ? A[base + (long)r * n + c] : 0.f;
    }
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    __syncthreads();
    tri::diag_valu<NW>(M, dscratch, w);
    __syncthreads();
    tri::lvl16<NW>(M, w);
    __syncthreads();
    tri::lvl32a<NW>(M, scratch, w);
    __syncthreads();
    tri::lvl32b<NW>(M, scratch, w);
    __syncthreads();
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

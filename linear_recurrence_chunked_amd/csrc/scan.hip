// K1: selective scan h_t = a_t h_{t-1} + b_t over rows, FP32, on gfx950.
//
// Source: "perf(mamba): prefill text prompts in multi-token chunks",
// Implementation -- the scan over a chunk of at most 64 rows is a doubling
// (Hillis-Steele) scan of the pairs (a, b)_t under
//     (a, b)_t <- (a_t a_{t-k}, a_t b_{t-k} + b_t),  k = 1, 2, 4, ...
// followed by h_t = a_t h_0 + b_t for the incoming state.  Every factor is a
// decay in (0, 1], so the products stay finite.
//
// Mapping on CDNA4: one wave64 owns 16 consecutive state elements of one
// prompt and walks that prompt's 64-row chunks; lane t holds row t of the
// chunk, so the whole chunk is one wave-wide scan.  Each lane reads and
// writes its row's 16 elements as four 16-byte vectors (a 64-byte run per
// row; the four waves of a block cover 256 contiguous bytes of every row).
// The six doubling rounds run on DPP: rounds k = 1, 2, 4, 8 shift within each
// 16-lane row (row_shr), then two row-broadcast rounds carry each row's
// running pair into the rows after it (row_bcast:15, row_bcast:31), which is
// the wave64 form of the k = 16, 32 rounds.  Lanes past the chunk's last row
// and lanes without a source take the identity pair (1, 0).  The carried
// state of each element stays in registers from chunk to chunk and is read
// back from lane S-1 of the chunk.
#include "lrc_device.h"
#include "lrc_internal.h"

namespace lrc {
namespace {

constexpr int kCols = 16;
constexpr int kWavesPerBlock = 4;

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void scan_round(float& a, float& b) {
    const float ap = dpp_move<CTRL, ROW_MASK>(1.0f, a);
    const float bp = dpp_move<CTRL, ROW_MASK>(0.0f, b);
    b = fmaf(a, bp, b);
    a = a * ap;
}

// Inclusive scan of the pairs held by the 64 lanes (lane = row).
__device__ __forceinline__ void wave_scan(float& a, float& b) {
    scan_round<kRowShr1, 0xf>(a, b);
    scan_round<kRowShr2, 0xf>(a, b);
    scan_round<kRowShr4, 0xf>(a, b);
    scan_round<kRowShr8, 0xf>(a, b);
    scan_round<kRowBcast15, 0xa>(a, b);
    scan_round<kRowBcast31, 0xc>(a, b);
}

template <bool VEC4>
__global__ __launch_bounds__(256) void scan_rows_kernel(const float* __restrict__ a, const float* __restrict__ b,
                                                        float* __restrict__ h, const float* h0, float* hS, Batch bt,
                                                        long E) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const long col0 = ((long)blockIdx.x * kWavesPerBlock + wave) * kCols;
    if (col0 >= E) return;
    const int ncol = (int)min((long)kCols, E - col0);
    const int p = batch_prompt(bt, blockIdx.y);
    const long row0 = batch_row0(bt, p);
    const int L = batch_len(bt, p);

    float carry[kCols];
    const float* h0p = h0 + (long)p * E + col0;
#pragma unroll
    for (int j = 0; j < kCols; ++j) carry[j] = j < ncol ? h0p[j] : 0.0f;

    float A[kCols], B[kCols];
    for (int c0 = 0; c0 < L; c0 += kWave) {
        const int S = min(kWave, L - c0);
        const bool valid = lane < S;
        const long base = (row0 + c0 + lane) * E + col0;
        if (VEC4) {
#pragma unroll
            for (int q = 0; q < kCols / 4; ++q) {
                float4 va = make_float4(1.f, 1.f, 1.f, 1.f), vb = make_float4(0.f, 0.f, 0.f, 0.f);
                if (valid && 4 * q < ncol) {
                    va = *reinterpret_cast<const float4*>(a + base + 4 * q);
                    vb = *reinterpret_cast<const float4*>(b + base + 4 * q);
                }
                A[4 * q] = va.x; A[4 * q + 1] = va.y; A[4 * q + 2] = va.z; A[4 * q + 3] = va.w;
                B[4 * q] = vb.x; B[4 * q + 1] = vb.y; B[4 * q + 2] = vb.z; B[4 * q + 3] = vb.w;
            }
        } else {
#pragma unroll
            for (int j = 0; j < kCols; ++j) {
                const bool ok = valid && j < ncol;
                A[j] = ok ? a[base + j] : 1.0f;
                B[j] = ok ? b[base + j] : 0.0f;
            }
        }
#pragma unroll
        for (int j = 0; j < kCols; ++j) {
            wave_scan(A[j], B[j]);
            const float hv = fmaf(A[j], carry[j], B[j]);
            carry[j] = readlane_f(hv, S - 1);
            A[j] = hv;
        }
        if (VEC4) {
#pragma unroll
            for (int q = 0; q < kCols / 4; ++q)
                if (valid && 4 * q < ncol)
                    *reinterpret_cast<float4*>(h + base + 4 * q) =
                        make_float4(A[4 * q], A[4 * q + 1], A[4 * q + 2], A[4 * q + 3]);
        } else {
#pragma unroll
            for (int j = 0; j < kCols; ++j)
                if (valid && j < ncol) h[base + j] = A[j];
        }
    }
    if (lane == 0) {
        float* hSp = hS + (long)p * E + col0;
#pragma unroll
        for (int j = 0; j < kCols; ++j)
            if (j < ncol) hSp[j] = carry[j];
    }
}

}  // namespace

hipError_t launch_scan(const float* a, const float* b, float* h, const float* h0, float* hS, const Batch& bt, long E,
                       hipStream_t st) {
    const long per_block = (long)kCols * kWavesPerBlock;
    const dim3 grid((unsigned)((E + per_block - 1) / per_block), (unsigned)bt.P);
    const bool vec4 = (E % 4) == 0;
    if (vec4)
        hipLaunchKernelGGL(scan_rows_kernel<true>, grid, dim3(256), 0, st, a, b, h, h0, hS, bt, E);
    else
        hipLaunchKernelGGL(scan_rows_kernel<false>, grid, dim3(256), 0, st, a, b, h, h0, hS, bt, E);
    return hipGetLastError();
}

}  // namespace lrc

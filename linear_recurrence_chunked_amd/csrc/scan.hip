// K1: selective scan h_t = a_t h_{t-1} + b_t over rows, FP32, on gfx950.
//
// Source: "perf(mamba): prefill text prompts in multi-token chunks",
// Implementation -- within a chunk of at most 64 rows the recurrence is
// evaluated as a doubling (Hillis-Steele) scan: in round k = 1, 2, 4, ... each
// row t combines its pair with the pair k rows earlier,
//     (a, b)_t <- (a_t a_{t-k}, a_t b_{t-k} + b_t),
// and the carried state enters last, h_t = A_t h_0 + B_t.  The a_t are decay
// factors no larger than one, so the running products cannot overflow.
//
// Mapping on CDNA4.  A workgroup (one wave per 16 elements) owns COLS
// consecutive state elements of one prompt and walks that prompt's 64-row
// chunks, keeping the carried state of its elements in registers:
//  1. The chunk's a and b tiles [64 rows x COLS elements] are read with
//     row-contiguous 16-byte loads (4*COLS bytes per row, whole cache lines)
//     and written to LDS; the next chunk's loads are issued before this
//     chunk is scanned, so their latency hides behind the arithmetic.
//  2. Each wave reads 16 element columns out of LDS with lane t = row t and
//     scans each column across the wave in six rounds.  Rounds k = 1, 2, 4, 8
//     shift within each 16-lane row of the wave (DPP row_shr); the last two
//     rounds carry each 16-lane row's running pair into the rows after it
//     (DPP row_bcast:15, row_bcast:31), the wave64 form of rounds k = 16, 32.
//     The DPP reads are folded into the arithmetic (v_fmac_f32_dpp,
//     v_mul_f32_dpp); a lane whose source is out of range keeps its pair,
//     which is the identity (1, 0) step.  Lanes past the chunk's last row
//     hold the identity pair.  Four columns are interleaved so that no DPP
//     read follows the write of its source too closely.
//  3. h_t = A_t h0 + B_t; the new carried state is read from lane S-1; the
//     h column goes back to LDS and leaves as row-contiguous 16-byte stores.
//  The row loads and stores are nontemporal: every byte is used once.
#include "lrc_device.h"
#include "lrc_internal.h"

namespace lrc {
namespace {

// State elements per workgroup.  Wider tiles read longer runs of every row
// (1 KiB at 256 columns), which keeps more DRAM-page locality between the 64
// rows a chunk touches; 256 measured fastest of 64 / 128 / 256 on the mixed
// prefill shape.  LDS: 2 x 64 x 257 floats per workgroup.
constexpr int kScanCols = 256;

constexpr int kColsPerWave = 16;

// a, b and h are touched once each: the 16-byte accesses are marked
// nontemporal (streaming), which measured 5% faster than plain accesses on
// the mixed prefill shape (plain stores with nontemporal loads were slower).
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define LRC_SCAN_ROUND(CTRL)                                   \
    "v_fmac_f32_dpp %0, %0, %4 " CTRL "\n"                    \
    "v_fmac_f32_dpp %1, %1, %5 " CTRL "\n"                    \
    "v_fmac_f32_dpp %2, %2, %6 " CTRL "\n"                    \
    "v_fmac_f32_dpp %3, %3, %7 " CTRL "\n"                    \
    "v_mul_f32_dpp %4, %4, %4 " CTRL "\n"                     \
    "v_mul_f32_dpp %5, %5, %5 " CTRL "\n"                     \
    "v_mul_f32_dpp %6, %6, %6 " CTRL "\n"                     \
    "v_mul_f32_dpp %7, %7, %7 " CTRL "\n"

// Inclusive wave scan of four independent columns of (a, b) pairs (lane = row).
// Each round computes b <- b + a * b_src and then a <- a * a_src, where
// (a_src, b_src) is the pair the DPP pattern routes to the lane.
__device__ __forceinline__ void wave_scan4(float (&a)[4], float (&b)[4]) {
    asm volatile(
        "s_nop 1\n"
        LRC_SCAN_ROUND("row_shr:1 row_mask:0xf bank_mask:0xf")
        LRC_SCAN_ROUND("row_shr:2 row_mask:0xf bank_mask:0xf")
        LRC_SCAN_ROUND("row_shr:4 row_mask:0xf bank_mask:0xf")
        LRC_SCAN_ROUND("row_shr:8 row_mask:0xf bank_mask:0xf")
        LRC_SCAN_ROUND("row_bcast:15 row_mask:0xa bank_mask:0xf")
        LRC_SCAN_ROUND("row_bcast:31 row_mask:0xc bank_mask:0xf")
        : "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]), "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]));
}
#undef LRC_SCAN_ROUND

// COLS state elements per workgroup, one wave per 16 of them.
template <int COLS, bool VEC4>
__global__ __launch_bounds__(COLS * 4) void scan_rows_kernel(const float* __restrict__ a, const float* __restrict__ b,
                                                            float* __restrict__ h, const float* h0, float* hS,
                                                            Batch bt, long E) {
    constexpr int kTileCols = COLS;
    constexpr int kLd = COLS + 1;  // LDS row stride (floats): column reads hit distinct banks
    constexpr int kLoadThreadsPerRow = COLS / 4;
    __shared__ float As[kWave * kLd];
    __shared__ float Bs[kWave * kLd];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const long tile0 = (long)blockIdx.x * kTileCols;
    const int p = batch_prompt(bt, blockIdx.y);
    const long row0 = batch_row0(bt, p);
    const int L = batch_len(bt, p);

    // Load-phase mapping: thread -> (row lr + 16 r, 4 columns at lc).
    const int lr = tid / kLoadThreadsPerRow;
    const int lc = (tid % kLoadThreadsPerRow) * 4;
    const bool lcol_ok = tile0 + lc < E;

    // Column-phase mapping: this wave's 16 columns start at cw.
    const int cw = wave * kColsPerWave;
    float carry[kColsPerWave];
#pragma unroll
    for (int j = 0; j < kColsPerWave; ++j) {
        const long col = tile0 + cw + j;
        carry[j] = col < E ? h0[(long)p * E + col] : 0.f;
    }

    float ra[4][4], rb[4][4];  // [row group][column] of the chunk in flight
    auto issue_loads = [&](int c0) {
        const int S = min(kWave, L - c0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = lr + 16 * r;
            const long off = (row0 + c0 + row) * E + tile0 + lc;
            if (VEC4) {
                float4 va = make_float4(1.f, 1.f, 1.f, 1.f), vb = make_float4(0.f, 0.f, 0.f, 0.f);
                if (row < S && lcol_ok) {
                    const f32x4 xa = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a + off));
                    const f32x4 xb = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(b + off));
                    va = make_float4(xa[0], xa[1], xa[2], xa[3]);
                    vb = make_float4(xb[0], xb[1], xb[2], xb[3]);
                }
                ra[r][0] = va.x; ra[r][1] = va.y; ra[r][2] = va.z; ra[r][3] = va.w;
                rb[r][0] = vb.x; rb[r][1] = vb.y; rb[r][2] = vb.z; rb[r][3] = vb.w;
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool ok = row < S && tile0 + lc + i < E;
                    ra[r][i] = ok ? a[off + i] : 1.f;
                    rb[r][i] = ok ? b[off + i] : 0.f;
                }
            }
        }
    };

    if (L > 0) issue_loads(0);
    for (int c0 = 0; c0 < L; c0 += kWave) {
        const int S = min(kWave, L - c0);
        __syncthreads();  // the previous chunk's h rows have left LDS
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                As[(lr + 16 * r) * kLd + lc + i] = ra[r][i];
                Bs[(lr + 16 * r) * kLd + lc + i] = rb[r][i];
            }
        if (c0 + kWave < L) issue_loads(c0 + kWave);
        __syncthreads();

        // Column phase: lane = row.
#pragma unroll
        for (int g = 0; g < kColsPerWave; g += 4) {
            float A[4], B[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                A[i] = As[lane * kLd + cw + g + i];
                B[i] = Bs[lane * kLd + cw + g + i];
            }
            wave_scan4(A, B);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float hv = fmaf(A[i], carry[g + i], B[i]);
                carry[g + i] = readlane_f(hv, S - 1);
                As[lane * kLd + cw + g + i] = hv;
            }
        }
        __syncthreads();

        // Row phase: h rows leave as 16-byte stores.
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = lr + 16 * r;
            if (row < S) {
                const long off = (row0 + c0 + row) * E + tile0 + lc;
                const float* src = &As[row * kLd + lc];
                if (VEC4) {
                    if (lcol_ok)
                        __builtin_nontemporal_store(f32x4{src[0], src[1], src[2], src[3]}, reinterpret_cast<f32x4*>(h + off));
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (tile0 + lc + i < E) h[off + i] = src[i];
                }
            }
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int j = 0; j < kColsPerWave; ++j) {
            const long col = tile0 + cw + j;
            if (col < E) hS[(long)p * E + col] = carry[j];
        }
    }
}

}  // namespace

template <int COLS>
hipError_t launch_cols(const float* a, const float* b, float* h, const float* h0, float* hS, const Batch& bt, long E,
                       hipStream_t st) {
    const dim3 grid((unsigned)((E + COLS - 1) / COLS), (unsigned)bt.P);
    if (E % 4 == 0)
        hipLaunchKernelGGL((scan_rows_kernel<COLS, true>), grid, dim3(COLS * 4), 0, st, a, b, h, h0, hS, bt, E);
    else
        hipLaunchKernelGGL((scan_rows_kernel<COLS, false>), grid, dim3(COLS * 4), 0, st, a, b, h, h0, hS, bt, E);
    return hipGetLastError();
}

hipError_t launch_scan(const float* a, const float* b, float* h, const float* h0, float* hS, const Batch& bt, long E,
                       hipStream_t st) {
    return launch_cols<kScanCols>(a, b, h, h0, hS, bt, E, st);
}

}  // namespace lrc

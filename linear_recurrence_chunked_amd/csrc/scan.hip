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
#include <algorithm>
#include <atomic>
#include <mutex>

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

// State elements per workgroup of the tiled form: a tile's LDS (2 x 64 x 129
// floats at 128) lets two workgroups share a CU, so that one loads or stores
// while the other scans.
#ifndef LRC_SCAN_TILE_COLS
#define LRC_SCAN_TILE_COLS 128
#endif
constexpr int kScanTileCols = LRC_SCAN_TILE_COLS;
// Persistent workgroups per CU of the tiled form (as many as the tile's LDS lets share a CU).
constexpr int kScanTileBlocksPerCU = (160 * 1024) / (2 * kWave * (kScanTileCols + 1) * 4 + 64);

// Polls of a chunk's hand-over flag before the tiled form gives up and
// records an error (a poll is a load from memory, about a microsecond, and a
// 128-cycle sleep: about 0.2 s in all).
constexpr int kScanWaitLimit = 1 << 17;

// Cache policy of a device-coherent buffer access on this target (sc1).
constexpr int kCoherent = 16;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Tiles of the tiled form: chunk_off[s] is the first chunk of batch slot s
// in the tiled launch (slots in batch order), chunk_off[P] the total.
struct ScanTiles {
    int ncb;
    int chunk_off[LRC_MAX_PROMPTS + 1];
};

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

// ---------------------------------------------------------------- tiled form
// The same chunk arithmetic over tiles of (chunk, COLS-element block).  Tiles
// are numbered prompt by prompt, chunk by chunk, block-fastest within a chunk,
// and handed out in that order from a ticket counter to persistent
// workgroups, so the tiles in flight at any moment cover whole rows of the
// same chunks (the long-lived form lets the blocks of a prompt drift apart,
// and rows are then read in pieces at different times, which loses
// DRAM-page locality).  A workgroup prefetches its next tile's rows while it
// scans the current one.  A tile is scanned from a zero carry first; only then
// does it wait for the previous chunk of its block, whose last h row is the
// carry, and finish h_t = A_t h0 + B_t.
//
// Hand-over: the last h row of a chunk is written with device-coherent
// stores; the writing wave waits for them, the workgroup meets at a barrier,
// and one thread then stores the chunk's completion into the flag of the
// (prompt, block) chain as (generation << 32) | (chunk + 1).  The next chunk
// polls that flag with device-coherent loads (bounded: after about 0.2 s it
// records an error and goes on rather than hang), meets its workgroup at a
// barrier and reads the carry with device-coherent loads.  A generation that
// is new for every call makes stale flags from earlier calls harmless.
// Tickets are taken in increasing order, so the tile a workgroup waits for
// was taken earlier by a workgroup that is running: progress does not depend
// on how many workgroups are resident.
struct TileAt {
    int p, j, S, cb;
    long row0;
    bool last;
};

__device__ __forceinline__ TileAt tile_at(const Batch& bt, const ScanTiles& tl, int ticket) {
    TileAt x;
    x.cb = ticket % tl.ncb;
    const int t = ticket / tl.ncb;
    int lo = 0, hi = bt.P;  // the slot whose chunks include t: chunk_off[lo] <= t < chunk_off[lo + 1]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (tl.chunk_off[mid] <= t) lo = mid;
        else hi = mid;
    }
    x.p = batch_prompt(bt, lo);
    x.j = t - tl.chunk_off[lo];
    x.row0 = batch_row0(bt, x.p);
    const int L = batch_len(bt, x.p);
    x.S = min(kWave, L - kWave * x.j);
    x.last = kWave * (x.j + 1) >= L;
    return x;
}

__global__ void scan_ticket_reset(unsigned* ctl) { ctl[1] = 0; }

template <int COLS>
__global__ __launch_bounds__(COLS * 4) void scan_tile_kernel(const float* __restrict__ a, const float* __restrict__ b,
                                                            float* __restrict__ h, float* state, Batch bt,
                                                            ScanTiles tl, long E, unsigned long long* flags,
                                                            unsigned* ctl, unsigned gen, int ntickets) {
    constexpr int kLd = COLS + 1;
    constexpr int kLoadThreadsPerRow = COLS / 4;
    __shared__ float As[kWave * kLd];
    __shared__ float Bs[kWave * kLd];
    __shared__ int ticket_sh;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lr = tid / kLoadThreadsPerRow;  // load phase: rows lr + 16 r, 4 columns at lc
    const int lc = (tid % kLoadThreadsPerRow) * 4;
    const int cw = wave * kColsPerWave;       // column phase: this wave's 16 columns

    float ra[4][4], rb[4][4];
    auto issue_loads = [&](const TileAt& x) {
        const long tile0 = (long)x.cb * COLS;
        const bool ok = tile0 + lc < E;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = lr + 16 * r;
            f32x4 xa = {1.f, 1.f, 1.f, 1.f}, xb = {0.f, 0.f, 0.f, 0.f};
            if (row < x.S && ok) {
                const long off = (x.row0 + kWave * x.j + row) * E + tile0 + lc;
                xa = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a + off));
                xb = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(b + off));
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ra[r][i] = xa[i];
                rb[r][i] = xb[i];
            }
        }
    };
    auto take_ticket = [&]() {
        if (tid == 0) ticket_sh = (int)__hip_atomic_fetch_add(&ctl[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        const int t = ticket_sh;
        return t;
    };

    int cur = take_ticket();
    if (cur >= ntickets) return;
    TileAt x = tile_at(bt, tl, cur);
    issue_loads(x);
    while (true) {
        __syncthreads();  // the previous tile's h rows have left LDS, and every wave has read ticket_sh
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                As[(lr + 16 * r) * kLd + lc + i] = ra[r][i];
                Bs[(lr + 16 * r) * kLd + lc + i] = rb[r][i];
            }
        const int nxt = take_ticket();  // its barrier also publishes the tile in LDS
        TileAt y;
        if (nxt < ntickets) {
            y = tile_at(bt, tl, nxt);
            issue_loads(y);  // the next tile's rows are in flight during this tile
        }

        // Column phase from a zero carry: lane = row, 16 columns per wave.
        const long tile0 = (long)x.cb * COLS;
        float A[kColsPerWave], B[kColsPerWave];
#pragma unroll
        for (int g = 0; g < kColsPerWave; g += 4) {
            float a4[4], b4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a4[i] = As[lane * kLd + cw + g + i];
                b4[i] = Bs[lane * kLd + cw + g + i];
            }
            wave_scan4(a4, b4);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                A[g + i] = a4[i];
                B[g + i] = b4[i];
            }
        }

        // The carry: the incoming state for a prompt's first chunk, otherwise
        // the previous chunk's last h row once its workgroup has handed it over.
        const long ccol = tile0 + cw + (lane & 15);
        const bool ccol_ok = ccol < E;
        const long c0 = (long)kWave * x.j;
        float cv = 0.f;
        if (x.j == 0) {
            if (ccol_ok) cv = state[(long)x.p * E + ccol];
        } else {
            unsigned long long* flag = flags + (long)x.p * tl.ncb + x.cb;
            const unsigned long long want = ((unsigned long long)gen << 32) | (unsigned)x.j;
            if (tid == 0) {
                int n = 0;
                while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != want) {
                    if (++n > kScanWaitLimit) {
                        __hip_atomic_fetch_add(&ctl[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                }
            }
            __syncthreads();
            if (ccol_ok)
                cv = __hip_atomic_load(h + (x.row0 + c0 - 1) * E + ccol, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        float hlast[kColsPerWave];
#pragma unroll
        for (int i = 0; i < kColsPerWave; ++i) {
            const float hv = fmaf(A[i], readlane_f(cv, i), B[i]);
            hlast[i] = readlane_f(hv, x.S - 1);
            As[lane * kLd + cw + i] = hv;
        }
        __syncthreads();

        // Row phase.  The last row of a chunk that has a successor leaves
        // through device-coherent stores; the rest as nontemporal 16-byte stores.
        const bool lcol_ok = tile0 + lc < E;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = lr + 16 * r;
            if (row < x.S && lcol_ok) {
                const long off = (x.row0 + c0 + row) * E + tile0 + lc;
                const float* src = &As[row * kLd + lc];
                if (!x.last && row == kWave - 1) {
                    // one 16-byte store with the device-coherence bit (sc1, cache policy 16)
                    const auto rs = buffer_rsrc(h + (x.row0 + c0 + row) * E + tile0, COLS * 4);
                    const u32x4 v4 = {__float_as_uint(src[0]), __float_as_uint(src[1]), __float_as_uint(src[2]),
                                      __float_as_uint(src[3])};
                    __builtin_amdgcn_raw_buffer_store_b128(v4, rs, lc * 4, 0, kCoherent);
                } else {
                    __builtin_nontemporal_store(f32x4{src[0], src[1], src[2], src[3]},
                                                reinterpret_cast<f32x4*>(h + off));
                }
            }
        }
        if (x.last) {
            if (lane == 0) {
#pragma unroll
                for (int i = 0; i < kColsPerWave; ++i) {
                    const long col = tile0 + cw + i;
                    if (col < E) state[(long)x.p * E + col] = hlast[i];
                }
            }
        } else {
            if (lr + 48 == kWave - 1) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the wave with the last row
            __syncthreads();
            if (tid == 0)
                __hip_atomic_store(flags + (long)x.p * tl.ncb + x.cb,
                                   ((unsigned long long)gen << 32) | (unsigned)(x.j + 1), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
        if (nxt >= ntickets) break;
        x = y;
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

long scan_tiled_tiles_bound(long rows, int P, long E) {
    return (rows / kWave + P) * ((E + kScanTileCols - 1) / kScanTileCols);
}

size_t scan_workspace_bytes(int P, long E) {
    const long ncb = (E + kScanTileCols - 1) / kScanTileCols;
    return (size_t)P * ncb * sizeof(unsigned long long) + 256;
}

hipError_t launch_scan_tiled(const float* a, const float* b, float* h, float* state, const Batch& bt, long E,
                             void* workspace, hipStream_t st) {
    if (E % 4 != 0) return launch_cols<kScanCols>(a, b, h, state, state, bt, E, st);
    ScanTiles tl;
    tl.ncb = (int)((E + kScanTileCols - 1) / kScanTileCols);
    long tiles = 0;
    for (int s = 0; s < bt.P; ++s) {
        tl.chunk_off[s] = (int)tiles;
        tiles += (batch_len(bt, batch_prompt(bt, s)) + kWave - 1) / kWave;
    }
    tl.chunk_off[bt.P] = (int)tiles;
    if (tiles == 0) return hipSuccess;
    static std::atomic<unsigned> generation{0};
    unsigned gen;  // never 0 (also after wrapping): a zero-filled workspace holds no flag
    do {
        gen = generation.fetch_add(1) + 1;
    } while (gen == 0);
    auto* ctl = static_cast<unsigned*>(workspace);  // first 256 bytes: [0] timeouts, [1] next ticket
    auto* flags = reinterpret_cast<unsigned long long*>(static_cast<char*>(workspace) + 256);
    const int ntickets = (int)(tiles * tl.ncb);
    int cus = 0, dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                 hipSuccess)
        cus = 256;
    const int grid = std::min(ntickets, std::max(1, cus) * kScanTileBlocksPerCU);
    hipLaunchKernelGGL(scan_ticket_reset, dim3(1), dim3(1), 0, st, ctl);
    hipLaunchKernelGGL((scan_tile_kernel<kScanTileCols>), dim3((unsigned)grid), dim3(kScanTileCols * 4), 0, st, a, b, h,
                       state, bt, tl, E, flags, ctl, gen, ntickets);
    return hipGetLastError();
}


// ------------------------------------------------------- fixed device scratch
// The tiled driver's control block and completion flags in a file-scope
// device array instead of a caller's workspace, for callers that cannot
// allocate.  Each GPU holds its own copy until the process ends; its address
// comes from hipGetSymbolAddress, once per device, with that device current
// (the array's name in host code is not a device address).  The first call
// on a device zero-fills it with a kernel on the caller's stream.  Every call
// on one GPU shares it, so calls that may run at the same time on one GPU
// race; the ticket counter is reset by every launch and the flags carry the
// call's generation, so nothing else needs clearing between calls.
namespace {
static __device__ __align__(256) unsigned char scan_scratch[kScanStaticScratchBytes];

__global__ void scan_scratch_clear(uint4* p, long n16) {
    for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n16; i += (long)gridDim.x * blockDim.x)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}
}  // namespace

hipError_t launch_scan_tiled_static(const float* a, const float* b, float* h, float* state, const Batch& bt, long E,
                                    hipStream_t st) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* ptr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = nullptr;
    {
        std::lock_guard<std::mutex> lock(mu);
        p = ptr[dev];
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scan_scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            hipLaunchKernelGGL(scan_scratch_clear, dim3(64), dim3(256), 0, st, static_cast<uint4*>(p),
                               (long)(kScanStaticScratchBytes / 16));
            e = hipGetLastError();
            if (e != hipSuccess) return e;
            ptr[dev] = p;
        }
    }
    return launch_scan_tiled(a, b, h, state, bt, E, p, st);
}

}  // namespace lrc

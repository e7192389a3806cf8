// K0: depthwise causal short conv over rows, on gfx950.
//
// Source: "perf(mamba): prefill text prompts in multi-token chunks" and
// "perf(qwen3_5): prefill text prompts in multi-token chunks",
// Implementation -- each output row is a depthwise window over the K-1 rows
// kept as conv state followed by the chunk's rows; after the chunk, the state
// keeps the final K-1 rows of that window sequence.
//
// Row t's output depends only on rows t-K+1 .. t of the prompt (or of the
// incoming state before the prompt's first row), so splitting a prompt into
// 64-row chunks changes nothing: the driver and the chunk call both run this
// kernel over whole prompts.
//
// Mapping on CDNA4: a thread owns VEC adjacent channels (16 bytes: 4 fp32 or
// 8 bf16) of a tile of kTile rows; consecutive threads own consecutive
// channels, so every row of a tile is one contiguous 16-byte-per-lane access.
// The K-1 halo rows above a tile are re-read from L2.  Rows are loaded in
// groups of 8 before they are computed, so their loads are in flight
// together.  Taps and accumulation are FP32 in tap order 0 .. K-1; bf16
// outputs round to nearest even (the hardware conversion).  The
// tile-0 thread of each (prompt, channel group) is the only reader of the
// incoming state for those channels; it loads the new state's rows before it
// writes them, so the state may be updated in place.
#include "lrc_device.h"
#include "lrc_internal.h"

namespace lrc {
namespace {

// One wave per workgroup: four times as many workgroups as with 256 threads,
// which spreads the short prompts' tiles more evenly over the compute units
// (measured on the mixed prefill shapes: fp32 0.258 -> 0.250 ms, bf16
// 0.202 -> 0.183 ms; 128 threads sat in between, unrolls of 4 and 16 rows were
// no better).
constexpr int kThreads = 64;
constexpr int kUnroll = 8;

// Rows per tile: 32 for fp32, 64 for bf16 (measured best on the mixed prefill
// shapes; a taller bf16 tile re-reads fewer halo rows and gives each thread a
// longer run, while 16 or fewer rows were slower for both).
template <typename T>
constexpr int tile_rows() {
    return sizeof(T) == 2 ? 64 : 32;
}

template <typename T>
struct Io;

// The 16-byte row accesses of the streamed inputs and outputs are nontemporal:
// each row is read (or written) once, so it need not stay in the caches.
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <>
struct Io<float> {
    static constexpr int VEC = 4;
    __device__ static void load(const float* p, float* out) {
        const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
        out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
    }
    __device__ static void store(float* p, const float* in) {
        __builtin_nontemporal_store(f32x4{in[0], in[1], in[2], in[3]}, reinterpret_cast<f32x4*>(p));
    }
    __device__ static float one(const float* p) { return *p; }
    __device__ static void put(float* p, float x) { *p = x; }
};

template <>
struct Io<uint16_t> {
    static constexpr int VEC = 8;
    __device__ static void load(const uint16_t* p, float* out) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        const uint32_t wds[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = __uint_as_float(wds[i] << 16);
            out[2 * i + 1] = __uint_as_float(wds[i] & 0xffff0000u);
        }
    }
    // Round to nearest even with the hardware conversion (two values per instruction).
    __device__ static void store(uint16_t* p, const float* in) {
        typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
        bf16x8 v;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = static_cast<__bf16>(in[i]);
        __builtin_nontemporal_store(v, reinterpret_cast<bf16x8*>(p));
    }
    __device__ static float one(const uint16_t* p) { return bf16_to_f32(*p); }
    __device__ static void put(uint16_t* p, float x) { *reinterpret_cast<__bf16*>(p) = static_cast<__bf16>(x); }
};

// Loads VEC channels (or fewer at the ragged channel tail) of one row.
template <typename T, int VEC, bool FULL>
__device__ __forceinline__ void load_row(const T* p, int nc, float* out) {
    if (FULL) {
        Io<T>::load(p, out);
    } else {
#pragma unroll
        for (int i = 0; i < VEC; ++i) out[i] = i < nc ? Io<T>::one(p + i) : 0.f;
    }
}

template <typename T, int VEC, bool FULL>
__device__ __forceinline__ void store_row(T* p, int nc, const float* in) {
    if (FULL) {
        Io<T>::store(p, in);
    } else {
#pragma unroll
        for (int i = 0; i < VEC; ++i)
            if (i < nc) Io<T>::put(p + i, in[i]);
    }
}

// VEC channels per thread when the channel count keeps 16-byte alignment,
// otherwise one channel per thread (VEC = 1, FULL = false).
template <typename T, int K, int VEC>
__global__ __launch_bounds__(kThreads) void conv_rows_kernel(const T* __restrict__ x, T* __restrict__ y,
                                                            const T* state_in, T* state_out,
                                                            const float* __restrict__ w, const float* __restrict__ bias,
                                                            Batch bt, int C) {
    constexpr int H = K - 1;
    constexpr bool FULL = (VEC == Io<T>::VEC);
    constexpr int kTile = tile_rows<T>();
    const int c0 = (blockIdx.x * kThreads + threadIdx.x) * VEC;
    if (c0 >= C) return;
    const int nc = min(VEC, C - c0);
    const int p = batch_prompt(bt, blockIdx.y);
    const long row0 = batch_row0(bt, p);
    const int L = batch_len(bt, p);
    const int ntiles = max(1, (L + kTile - 1) / kTile);

    float wt[VEC][K > 0 ? K : 1];
    float bs[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
        const int c = min(c0 + i, C - 1);
#pragma unroll
        for (int j = 0; j < K; ++j) wt[i][j] = w[(long)c * K + j];
        bs[i] = bias ? bias[c] : 0.f;
    }
    const T* sp = state_in + (long)p * H * C + c0;

    for (int tile = blockIdx.z; tile < ntiles; tile += gridDim.z) {
        const int t0 = tile * kTile;
        // window[0..H-1] holds rows t-H .. t-1 of the state-extended sequence
        float win[H > 0 ? H : 1][VEC];
#pragma unroll
        for (int r = 0; r < H; ++r) {
            const int t = t0 - H + r;  // prompt-local row, negative = state row H + t
            if (t < 0)
                load_row<T, VEC, FULL>(sp + (long)(H + t) * C, nc, win[r]);
            else
                load_row<T, VEC, FULL>(x + (row0 + t) * C + c0, nc, win[r]);
        }
        const int n = min(kTile, L - t0);
        auto emit = [&](int i, const float* cur) {
            float out[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                float acc = bs[e];
#pragma unroll
                for (int j = 0; j < H; ++j) acc = fmaf(wt[e][j], win[j][e], acc);
                acc = fmaf(wt[e][H], cur[e], acc);
                out[e] = acc;
            }
            store_row<T, VEC, FULL>(y + (row0 + t0 + i) * C + c0, nc, out);
#pragma unroll
            for (int j = 0; j + 1 < H; ++j)
#pragma unroll
                for (int e = 0; e < VEC; ++e) win[j][e] = win[j + 1][e];
            if (H > 0) {
#pragma unroll
                for (int e = 0; e < VEC; ++e) win[H - 1][e] = cur[e];
            }
        };
        int i = 0;
        // groups of kUnroll rows: all loads first, so they are in flight together
        for (; i + kUnroll <= n; i += kUnroll) {
            float cur[kUnroll][VEC];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) load_row<T, VEC, FULL>(x + (row0 + t0 + i + u) * C + c0, nc, cur[u]);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) emit(i + u, cur[u]);
        }
        for (; i < n; ++i) {
            float cur[VEC];
            load_row<T, VEC, FULL>(x + (row0 + t0 + i) * C + c0, nc, cur);
            emit(i, cur);
        }
        if (tile == 0 && H > 0) {
            // New state: rows L .. L+H-1 of the state-extended sequence.
            float ns[H > 0 ? H : 1][VEC];
#pragma unroll
            for (int r = 0; r < H; ++r) {
                const int src = L + r - H;  // prompt-local row
                if (src < 0)
                    load_row<T, VEC, FULL>(sp + (long)(H + src) * C, nc, ns[r]);
                else
                    load_row<T, VEC, FULL>(x + (row0 + src) * C + c0, nc, ns[r]);
            }
            T* so = state_out + (long)p * H * C + c0;
#pragma unroll
            for (int r = 0; r < H; ++r) store_row<T, VEC, FULL>(so + (long)r * C, nc, ns[r]);
        }
    }
}

template <typename T, int K>
hipError_t launch_typed(const T* x, T* y, const T* s_in, T* s_out, const float* w, const float* bias, const Batch& bt,
                        int C, hipStream_t st) {
    constexpr int kTile = tile_rows<T>();
    int maxL = 0;
    for (int i = 0; i < bt.P; ++i) maxL = max(maxL, batch_len(bt, batch_prompt(bt, i)));
    const int tiles = max(1, min(65535, (maxL + kTile - 1) / kTile));
    constexpr int V = Io<T>::VEC;
    if (C % V == 0) {
        const dim3 grid((unsigned)((C / V + kThreads - 1) / kThreads), (unsigned)bt.P, (unsigned)tiles);
        hipLaunchKernelGGL((conv_rows_kernel<T, K, V>), grid, dim3(kThreads), 0, st, x, y, s_in, s_out, w, bias, bt,
                           C);
    } else {
        const dim3 grid((unsigned)((C + kThreads - 1) / kThreads), (unsigned)bt.P, (unsigned)tiles);
        hipLaunchKernelGGL((conv_rows_kernel<T, K, 1>), grid, dim3(kThreads), 0, st, x, y, s_in, s_out, w, bias, bt,
                           C);
    }
    return hipGetLastError();
}

template <typename T>
hipError_t launch_k(const void* x, void* y, const void* s_in, void* s_out, const float* w, const float* bias,
                    const Batch& bt, int C, int K, hipStream_t st) {
    const T* xi = static_cast<const T*>(x);
    T* yo = static_cast<T*>(y);
    const T* si = static_cast<const T*>(s_in);
    T* so = static_cast<T*>(s_out);
    switch (K) {
        case 1: return launch_typed<T, 1>(xi, yo, si, so, w, bias, bt, C, st);
        case 2: return launch_typed<T, 2>(xi, yo, si, so, w, bias, bt, C, st);
        case 3: return launch_typed<T, 3>(xi, yo, si, so, w, bias, bt, C, st);
        case 4: return launch_typed<T, 4>(xi, yo, si, so, w, bias, bt, C, st);
        case 5: return launch_typed<T, 5>(xi, yo, si, so, w, bias, bt, C, st);
        case 6: return launch_typed<T, 6>(xi, yo, si, so, w, bias, bt, C, st);
        case 7: return launch_typed<T, 7>(xi, yo, si, so, w, bias, bt, C, st);
        case 8: return launch_typed<T, 8>(xi, yo, si, so, w, bias, bt, C, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_conv(const void* x, void* y, const void* state_in, void* state_out, const float* w,
                       const float* bias, const Batch& bt, int C, int K, lrc_dtype dt, hipStream_t st) {
    if (dt == LRC_BF16) return launch_k<uint16_t>(x, y, state_in, state_out, w, bias, bt, C, K, st);
    return launch_k<float>(x, y, state_in, state_out, w, bias, bt, C, K, st);
}

}  // namespace lrc

// Device helpers shared by the gfx950 kernels of liblrc.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lrc {

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// DPP move of a float: lanes whose source lies outside their 16-lane row, or
// whose row is masked off by ROW_MASK, receive `old` instead.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_move(float old, float src) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src), CTRL, ROW_MASK, 0xf,
                                                      false));
}

// GFX9 DPP controls used by the wave scans.
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142;  // lane 15 of row r feeds every lane of row r + 1
constexpr int kRowBcast31 = 0x143;  // lane 31 feeds every lane of rows 2 and 3

// Inclusive prefix sum over the 64 lanes of a wave: sums within each 16-lane
// row by DPP shifts, then carries row totals forward by row broadcasts.
__device__ __forceinline__ float wave_prefix_sum(float x) {
    x += dpp_move<kRowShr1, 0xf>(0.f, x);
    x += dpp_move<kRowShr2, 0xf>(0.f, x);
    x += dpp_move<kRowShr4, 0xf>(0.f, x);
    x += dpp_move<kRowShr8, 0xf>(0.f, x);
    x += dpp_move<kRowBcast15, 0xa>(0.f, x);
    x += dpp_move<kRowBcast31, 0xc>(0.f, x);
    return x;
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// bf16 -> fp32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// Raw buffer resource over `bytes` bytes from p (stride 0, 32-bit data
// format, the gfx9 descriptor word).  Loads whose per-lane offset lies past
// the end return 0 and such stores are dropped; the scalar offset is not part
// of that check, so only uniform offsets that stay in range go there.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}
constexpr int kNontemporal = 2;  // cache-policy argument of the buffer builtins: streaming access

// e^x through the hardware base-2 exponential.
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

// Bounded wait until an LDS counter reaches v (acquire, workgroup scope).  For
// waits on another wave of the same workgroup that needs nothing from the
// waiting one, so the bound (about 2^20 polls) is never reached in practice;
// past it the wave goes on rather than hang, and its lane 0 adds one to
// *timeouts (a device counter the host reads back; its results are then
// not to be trusted).
constexpr int kLdsWaitLimit = 1 << 20;
__device__ __forceinline__ void lds_wait_at_least(int* x, int v, unsigned* timeouts) {
    int n = 0;
    while (__hip_atomic_load(x, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < v) {
        if (++n > kLdsWaitLimit) {
            if (lane_id() == 0) __hip_atomic_fetch_add(timeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
}

}  // namespace lrc

// Internal declarations shared by the HIP sources of liblrc.so.
// Not installed; the public surface is include/lrc.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lrc.h"

namespace lrc {

// Prompt layout of one launch, passed to kernels by value.  Either every
// prompt has `uniform` rows and prompt p starts at row p * uniform, or
// (uniform < 0) prompt p owns rows [row_off[p], row_off[p + 1]).  `order`
// lists prompt indices longest first; kernels map blockIdx.y to order[y] so
// that the longest sequential chains are dispatched first.
struct Batch {
    int P;
    int uniform;
    int row_off[LRC_MAX_PROMPTS + 1];
    int order[LRC_MAX_PROMPTS];
};

__host__ __device__ inline int batch_prompt(const Batch& b, int slot) {
    return b.uniform >= 0 ? slot : b.order[slot];
}
__host__ __device__ inline int batch_row0(const Batch& b, int p) {
    return b.uniform >= 0 ? p * b.uniform : b.row_off[p];
}
__host__ __device__ inline int batch_len(const Batch& b, int p) {
    return b.uniform >= 0 ? b.uniform : b.row_off[p + 1] - b.row_off[p];
}

// Compute units of the current device (0 if the query fails).
int compute_units();

// Device counter (one per GPU, in the library) of bounded LDS waits that gave
// up; the WKV kernels add to it.  nullptr if its address cannot be had.
unsigned* wait_timeouts_counter();

// Kernel launchers (one per op), defined next to their kernels.  They
// assume validated arguments and return the launch status.
hipError_t launch_conv(const void* x, void* y, const void* state_in, void* state_out, const float* w,
                       const float* bias, const Batch& bt, int C, int K, lrc_dtype dt, hipStream_t st);
hipError_t launch_scan(const float* a, const float* b, float* h, const float* h0, float* hS, const Batch& bt,
                       long E, hipStream_t st);
size_t scan_workspace_bytes(int P, long E);
long scan_tiled_tiles_bound(long rows, int P, long E);  // at least the tiled scan's tile count
hipError_t launch_scan_tiled(const float* a, const float* b, float* h, float* state, const Batch& bt, long E,
                             void* workspace, hipStream_t st);
// The tiled driver with its control block and flags in a fixed device array
// of kScanStaticScratchBytes (one per GPU) instead of a caller's workspace.
constexpr size_t kScanStaticScratchBytes = size_t(2) << 20;
hipError_t launch_scan_tiled_static(const float* a, const float* b, float* h, float* state, const Batch& bt, long E,
                                    hipStream_t st);
hipError_t launch_wkv4(const float* k, const float* v, const float* w, const float* u, float* wkv, float* num,
                       float* den, float* mx, const Batch& bt, int C, hipStream_t st);
hipError_t launch_wkv_tdecay(const float* k, const float* v, const float* w, const float* u, float* wkv, float* num,
                             float* den, float* mx, const Batch& bt, int C, hipStream_t st);
hipError_t launch_gdn(const void* q, const void* k, const void* v, const float* beta, const float* g, float* o,
                      const float* S_in, float* S_out, const Batch& bt, int Hk, int Hv, int dk, int dv,
                      lrc_dtype dt, hipStream_t st);
hipError_t launch_gdn_bf16_mfma(const void* q, const void* k, const void* v, const float* beta, const float* g,
                                float* o, const float* S_in, float* S_out, const Batch& bt, int Hk, int Hv, int dk,
                                int dv, bool split, hipStream_t st);
// The chunk-parallel bf16 form: one workspace block of gdn_cp_block_bytes per
// (chunk, value head); state [P, Hv, dk, dv] updated in place.
size_t gdn_cp_block_bytes(int dk, int dv);
hipError_t launch_gdn_chunk_parallel(const void* q, const void* k, const void* v, const float* beta, const float* g,
                                     float* o, float* state, const Batch& bt, int Hk, int Hv, int dk, int dv,
                                     void* ws, hipStream_t st);
hipError_t launch_unit_lower_inverse(const float* A, float* T, int batch, int n, hipStream_t st);
// `plane` is the element stride between mixed inputs in `out` (rows x C).
hipError_t launch_time_shift(const float* x, float* out, const float* state_in, float* state_out, const float* mix,
                             const Batch& bt, int C, int M, long plane, hipStream_t st);
hipError_t launch_mamba_mixer(const float* x, const float* dt, const float* A, const float* Bm, const float* Cm,
                              const float* Dp, float* y, const float* h_in, float* h_out, const Batch& bt, int Dm,
                              int N, hipStream_t st);

}  // namespace lrc

/*
 * lrc.h -- C ABI of liblrc.so: chunked prefill of recurrent sequence mixers
 * on AMD Instinct MI355X (gfx950).
 *
 * Each kernel takes an incoming recurrent state and a chunk of at most
 * LRC_MAX_ROWS rows, writes every row's output and the outgoing state, and
 * agrees with the token-by-token recurrence.  The prefill drivers run whole
 * prompts of any length, packed one after another along the row axis, as
 * consecutive chunks of LRC_MAX_ROWS rows with the state carried between
 * chunks on the device.
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers owned by the caller, except where an
 *    argument is marked "host".  Tensors are dense, row-major, innermost
 *    dimension last, and 16-byte aligned.  Outputs must not overlap inputs
 *    unless an argument says it may alias.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call is
 *    asynchronous on that stream, allocates no memory and keeps no state
 *    between calls (lrc_scan_prefill_static alone uses a fixed device array
 *    of the library, described there).  Calls on distinct buffers are
 *    thread-safe.
 *  - All arguments are validated on the host before anything is enqueued,
 *    without any HIP call.  On a validation error nothing is launched, no
 *    buffer is written, and lrc_last_error() (thread-local) explains it.
 *  - If a launch fails, the call returns LRC_ERR_LAUNCH after synchronizing
 *    the stream (so no queued work still reads the caller's buffers).  The
 *    recurrent states are then undefined and the caller must reset them;
 *    there is no rollback.
 *  - Rows = 0 (or an empty batch) is valid: outputs are untouched and the
 *    outgoing state equals the incoming one.
 *
 * Sources (page title, section):
 *  [mamba] "perf(mamba): prefill text prompts in multi-token chunks",
 *          Implementation.
 *  [rwkv]  "perf(rwkv): prefill text prompts in multi-token chunks",
 *          Implementation.
 *  [qwen]  "perf(qwen3_5): prefill text prompts in multi-token chunks",
 *          Implementation.
 */
#ifndef LRC_H
#define LRC_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Largest chunk.  All three pages cap a chunk at 64 rows: the triangular
   solve is padded to that size [qwen], the doubling scan stays cheap at it
   [mamba], and the [S+1, S] exponent tensor grows with its square [rwkv].
   A chunk call with more rows is rejected. */
#define LRC_MAX_ROWS 64
/* Largest number of prompts in one prefill-driver call (prompt offsets
   travel to the device by value, inside the kernel arguments). */
#define LRC_MAX_PROMPTS 256
/* Largest depthwise conv width. */
#define LRC_MAX_CONV_K 8
/* Largest number of mixed inputs one time-shift call produces. */
#define LRC_MAX_MIX 8

typedef enum {
    LRC_OK = 0,
    LRC_ERR_NULL = 1,   /* a required pointer is NULL */
    LRC_ERR_ROWS = 2,   /* chunk rows < 0 or > LRC_MAX_ROWS, or a prompt length < 0 */
    LRC_ERR_SHAPE = 3,  /* a size is outside the supported range */
    LRC_ERR_DTYPE = 4,  /* unsupported element type for this call */
    LRC_ERR_ALIGN = 5,  /* a tensor pointer is not 16-byte aligned */
    LRC_ERR_LAUNCH = 6, /* a HIP launch or runtime call failed */
    LRC_ERR_ALIAS = 7   /* an output overlaps an input it may not alias */
} lrc_status;

/* Element type of the inputs.  LRC_BF16_SPLIT (K3 only) takes bf16 inputs like
   LRC_BF16 and changes how FP32 intermediates reach the bf16 matrix cores. */
typedef enum { LRC_F32 = 0, LRC_BF16 = 1, LRC_BF16_SPLIT = 2 } lrc_dtype;

/* ------------------------------------------------------------------------
 * K0  Depthwise causal short conv over rows  [mamba], [qwen]
 *
 * The window of row t is the previous K-1 rows followed by the chunk rows:
 * xt = concat(state_in[K-1 rows], x[S rows]) along time, and
 *     y[t][c] = bias[c] + sum_{j<K} w[c][j] * xt[t+j][c]
 * (a causal cross-correlation: tap K-1 multiplies the current row).  No
 * activation.  The new conv state is the last K-1 rows of xt; for S < K-1
 * that keeps K-1-S of the old state rows.
 *
 *  x, y        [B, S, C]   dtype (F32, or BF16 with FP32 accumulation)
 *  state_in    [B, K-1, C] dtype
 *  state_out   [B, K-1, C] dtype; may alias state_in (in-place update)
 *  w           [C, K] float; bias [C] float or NULL
 *  1 <= K <= LRC_MAX_CONV_K, C >= 1, 0 <= S <= LRC_MAX_ROWS, B >= 0.
 * ---------------------------------------------------------------------- */
lrc_status lrc_conv_rows(const void* x, void* y, const void* state_in, void* state_out,
                         const float* w, const float* bias, int B, int S, int C, int K,
                         lrc_dtype dt, void* stream);

/* K0 driver.  x, y [R, C] hold P prompts packed along rows, prompt p owning
   lens_host[p] consecutive rows (R = sum of lens).  state [P, K-1, C] is
   read and updated in place.  Same result as lrc_conv_rows over consecutive
   64-row chunks of every prompt.  1 <= P <= LRC_MAX_PROMPTS. */
lrc_status lrc_conv_prefill(const void* x, void* y, void* state, const float* w, const float* bias,
                            const int* lens_host, int P, int C, int K, lrc_dtype dt, void* stream);

/* ------------------------------------------------------------------------
 * K1  Selective scan over rows  [mamba]
 *
 * For every state element e (E = D * N of them) independently:
 *     h_t = a_t h_{t-1} + b_t,  t = 0 .. S-1, starting from h0,
 * evaluated per chunk as a log-step parallel (doubling) scan of the pairs
 * (a, b) under (a2, b2) o (a1, b1) = (a2 a1, a2 b1 + b2) with the carried
 * state applied last: h_t = A_t h0 + B_t.  All FP32.  Output is every h_t;
 * the outgoing state is h at the last row.
 *
 *  a, b, h     [B, S, D, N] float
 *  h0          [B, D, N] float (incoming)
 *  hS          [B, D, N] float (outgoing); may alias h0
 *  D, N >= 1, 0 <= S <= LRC_MAX_ROWS, B >= 0.
 * ---------------------------------------------------------------------- */
lrc_status lrc_scan_rows(const float* a, const float* b, float* h, const float* h0, float* hS,
                         int B, int S, int D, int N, void* stream);

/* K1 driver: a, b, h [R, D, N] packed rows; state [P, D, N] in place. */
lrc_status lrc_scan_prefill(const float* a, const float* b, float* h, float* state,
                            const int* lens_host, int P, int D, int N, void* stream);

/* K1 driver, tiled form [mamba]: the same result as lrc_scan_prefill, bit for
 * bit (every chunk is the same doubling scan with the carried state applied
 * last).  The work is cut into tiles of (chunk, block of 128 state elements),
 * handed out in row order to persistent workgroups, instead of one workgroup
 * walking all chunks of a (prompt, block).  A tile takes its carry, the
 * previous chunk's last h row, from h once that chunk's tile has flagged it,
 * so the tiles in flight at any moment read whole rows together.
 *
 *  workspace        device memory of at least lrc_scan_workspace_size(P, D, N)
 *                   bytes, 16-byte aligned, owned by the caller.  It must be
 *                   zero-filled before its first use; the library never needs
 *                   it cleared again (every call tags its flags with a new
 *                   generation).  Calls that may run at the same time must not
 *                   share a workspace.
 *  The workspace begins with a 32-bit count of hand-overs that timed out
 *  (about 0.2 s each; the flags follow at byte 256); it stays 0 unless
 *  workgroups of one launch could not all make progress.  Returns LRC_ERR_SHAPE if the workspace
 *  is too small or the launch would need 2^31 workgroups or more.  With
 *  D * N not a multiple of 4 it runs the lrc_scan_prefill kernel. */
size_t lrc_scan_workspace_size(int P, int D, int N);
lrc_status lrc_scan_prefill_ws(const float* a, const float* b, float* h, float* state,
                               const int* lens_host, int P, int D, int N,
                               void* workspace, size_t workspace_bytes, void* stream);

/* K1 driver, tiled form, allocating nothing: for callers that cannot
 * allocate device memory or pass a workspace (code under stream capture,
 * tight serving loops, harnesses that forbid allocation).  Same arguments and
 * the same result, bit for bit, as lrc_scan_prefill_ws, whose workspace is
 * replaced here by a fixed device array inside the library: 2 MiB per GPU,
 * held from the first call on that GPU until the process ends, zero-filled
 * by that first call on `stream`.  It bounds P * ceil(D * N / 128) to
 * 262 112 (LRC_ERR_SHAPE beyond, before anything is launched).  Every call on
 * one GPU uses the same array: calls that may run at the same time on one GPU
 * (on streams with no ordering between them) race and must not be made.  The
 * call makes no hipMalloc or hipFree and no allocating library call. */
lrc_status lrc_scan_prefill_static(const float* a, const float* b, float* h, float* state,
                                   const int* lens_host, int P, int D, int N, void* stream);

/* ------------------------------------------------------------------------
 * K2  RWKV-4 WKV over rows  [rwkv]
 *
 * Per channel c the state keeps A = num e^max and B = den e^max of
 * A_t = e^w A_{t-1} + e^{k_t} v_t,  B_t = e^w B_{t-1} + e^{k_t}   (w < 0),
 * and row t of a chunk outputs
 *     wkv_t = (A_{t-1} + e^{u+k_t} v_t) / (B_{t-1} + e^{u+k_t}).
 * Relative to the incoming state, row t combines three kinds of exponents:
 * max_0 + t w (the state), k_i + (t-1-i) w for earlier rows i < t, and the
 * bonus u + k_t; every row shifts by its largest exponent before exp.  The
 * outgoing triple is the "row S" of that form: (num, den, max) with max the
 * largest exponent of the rows seen.  A fresh channel is (0, 0, -1e38).
 *
 *  k, v, wkv   [B, S, C] float
 *  w, u        [C] float (w < 0)
 *  num, den, mx [B, C] float, read and updated in place
 *  C >= 1, 0 <= S <= LRC_MAX_ROWS, B >= 0.
 * ---------------------------------------------------------------------- */
lrc_status lrc_wkv4_rows(const float* k, const float* v, const float* w, const float* u, float* wkv,
                         float* num, float* den, float* mx, int B, int S, int C, void* stream);

/* K2 driver: k, v, wkv [R, C] packed rows; num, den, mx [P, C] in place. */
lrc_status lrc_wkv4_prefill(const float* k, const float* v, const float* w, const float* u, float* wkv,
                            float* num, float* den, float* mx, const int* lens_host, int P, int C,
                            void* stream);

/* ------------------------------------------------------------------------
 * K3  Gated DeltaNet chunk  [qwen]
 *
 * For value head h (key head h / (Hv/Hk)) and a chunk of S rows with
 * gamma_t = sum_{i<=t} g_i (chunk-local, inclusive) and Gamma = e^gamma:
 *   A_ij = beta_i e^{gamma_i - gamma_j} k_i.k_j   (j < i), else 0
 *   (I + A) U = diag(beta) V - diag(beta Gamma) K S_0
 *   O   = diag(Gamma) Q S_0 + (e^{gamma_t - gamma_i} q_t.k_i)_{i <= t} U
 *   S_S = e^{gamma_S} S_0 + (K * e^{min(gamma_S - gamma, 0)})^T U
 * gamma_S is the last cumulative sum.  The inverse of I + A pads the chunk
 * to 64 rows with identity rows, inverts the eight 8x8 diagonal blocks as
 * (I+N)^-1 = (I-N)(I+N^2)(I+N^4), and then merges blocks pairwise at
 * 16, 32 and 64 rows with T21 = -T22 L21 T11.  Decay factors are formed element by element from
 * gamma differences, never as ratios of Gamma.  No scale is applied to q.
 *
 *  q, k        [B, S, Hk, dk]  dtype
 *  v           [B, S, Hv, dv]  dtype
 *  beta, g     [B, S, Hv]      float (g <= 0)
 *  o           [B, S, Hv, dv]  float
 *  S_in        [B, Hv, dk, dv] float
 *  S_out       [B, Hv, dk, dv] float; may alias S_in
 *  dk, dv in {32, 64, 128}; Hk >= 1; Hv a multiple of Hk.
 *  dtype F32: FP32 arithmetic throughout.  dtype BF16: bf16 q/k/v; the
 *  state, decays, inverse and every accumulation are FP32, and an FP32
 *  operand of a matrix product (S_0, T, the right-hand side, P, U) is
 *  rounded to bf16 once.  dtype BF16_SPLIT: the same inputs, with each such
 *  operand entered as a pair hi = bf16(x), lo = bf16(x - hi), about 16
 *  mantissa bits, for about 1.45x the time.  Other calls reject BF16_SPLIT
 *  with LRC_ERR_DTYPE.
 * ---------------------------------------------------------------------- */
lrc_status lrc_gdn_chunk(const void* q, const void* k, const void* v, const float* beta,
                         const float* g, float* o, const float* S_in, float* S_out, int B, int S,
                         int Hk, int Hv, int dk, int dv, lrc_dtype dt, void* stream);

/* K3 driver: q, k [R, Hk, dk], v [R, Hv, dv], beta, g [R, Hv], o [R, Hv, dv]
   packed rows; state [P, Hv, dk, dv] in place. */
lrc_status lrc_gdn_prefill(const void* q, const void* k, const void* v, const float* beta,
                           const float* g, float* o, float* state, const int* lens_host, int P,
                           int Hk, int Hv, int dk, int dv, lrc_dtype dt, void* stream);

/* K3 driver, chunk-parallel form [qwen], for launches with few prompts.
 * With T = (I + A)^-1 the chunk's U regroups as U = U' - W S_0, where
 * U' = T diag(beta) V and W = T diag(beta Gamma) K need no state.  A first
 * kernel forms A, T, W, U', the masked decayed Q K^T and the per-row decays of
 * every (chunk, value head) at once, into `workspace`; a second walks each
 * prompt's chunks and runs only the products with the state (W S_0, Q S_0,
 * the outputs and the state update).  Same arguments and results as
 * lrc_gdn_prefill (within the bf16 tolerance; the association differs), for
 * LRC_BF16 inputs only (LRC_ERR_DTYPE otherwise).  lrc_gdn_prefill is the
 * faster choice when prompts x value heads fill the GPU's compute units;
 * this form when they do not (one long prompt, say).
 *  workspace   device memory of at least lrc_gdn_workspace_bytes(P, R, Hk,
 *              Hv, dk, dv, dt) bytes for R = sum of lens, 16-byte aligned,
 *              owned by the caller, no initial contents needed; it must not
 *              overlap a tensor, and calls that may run at the same time must
 *              not share it.  (72.5 KiB per 64-row chunk and value head at
 *              dk = dv = 128.)
 * lrc_gdn_workspace_bytes returns 0 for arguments the call rejects. */
size_t lrc_gdn_workspace_bytes(int P, long total_rows, int Hk, int Hv, int dk, int dv, lrc_dtype dt);
lrc_status lrc_gdn_prefill_ws(const void* q, const void* k, const void* v, const float* beta,
                              const float* g, float* o, float* state, const int* lens_host, int P,
                              int Hk, int Hv, int dk, int dv, lrc_dtype dt, void* workspace,
                              size_t workspace_bytes, void* stream);

/* The triangular inverse of K3 on its own, at the precision K3 uses (FP32):
   T = (I + strictly_lower(A))^-1 for `batch` matrices of n x n, n <= 64,
   padded to 64 rows with identity: the diagonal 16x16 tiles as 8x8
   products on the vector ALUs, the level products on the FP32 matrix cores,
   as in the bf16 chunk kernel.  A, T [batch, n, n] float; T must not
   overlap A.  [qwen] */
lrc_status lrc_unit_lower_inverse(const float* A, float* T, int batch, int n, void* stream);

/* ------------------------------------------------------------------------
 * RWKV-4 time shift ([rwkv]: every mixed input combines each row with the
 * previous one, and the first row with the carried shift state; the chunk's
 * last row becomes the next shift state).  For each of M mixing vectors mu_j:
 *   out[j][t][c] = mu_j[c] x[t][c] + (1 - mu_j[c]) x[t-1][c],  x[-1] = state_in
 *   state_out    = x[S-1]  (state_in if S = 0)
 * One pass over x writes all M mixed inputs.
 *  x          [B, S, C]     float
 *  out        [M, B, S, C]  float (mixed input j is plane j)
 *  state_in   [B, C]        float
 *  state_out  [B, C]        float; may alias state_in
 *  mix        [M, C]        float
 *  1 <= M <= LRC_MAX_MIX.  Errors: as for the other chunk calls.
 * ---------------------------------------------------------------------- */
lrc_status lrc_time_shift_rows(const float* x, float* out, const float* state_in, float* state_out,
                               const float* mix, int B, int S, int C, int M, void* stream);

/* Time-shift driver: x [R, C] packed rows, out [M, R, C], state [P, C] in place. */
lrc_status lrc_time_shift_prefill(const float* x, float* out, float* state, const float* mix,
                                  const int* lens_host, int P, int C, int M, void* stream);

/* ------------------------------------------------------------------------
 * Mamba mixer rows with the scan's inputs formed and its output read out in
 * the same kernel ([mamba]: the mixer rows run h_t = a_t h_{t-1} + b_t
 * between forming a, b and reading h; here those are the selective
 * state-space step).  a, b and h stay on chip:
 *   a_t[d][n] = exp(dt[t][d] A[d][n]),   b_t[d][n] = dt[t][d] B[t][n] x[t][d]
 *   h_t = a_t h_{t-1} + b_t,             y[t][d] = sum_n C[t][n] h_t[d][n] + Dp[d] x[t][d]
 *  x, dt, y   [B, S, D]  float (dt as given, e.g. after softplus)
 *  Bm, Cm     [B, S, N]  float
 *  A          [D, N]     float
 *  Dp         [D]        float
 *  h_in       [B, D, N]  float
 *  h_out      [B, D, N]  float; may alias h_in
 *  N in {2, 4, 8, 16, 32, 64}.  Errors: as for the other chunk calls.
 * ---------------------------------------------------------------------- */
lrc_status lrc_mamba_mixer_rows(const float* x, const float* dt, const float* A, const float* Bm,
                                const float* Cm, const float* Dp, float* y, const float* h_in,
                                float* h_out, int B, int S, int D, int N, void* stream);

/* Mixer driver: x, dt, y [R, D], Bm, Cm [R, N] packed rows; state [P, D, N] in place. */
lrc_status lrc_mamba_mixer_prefill(const float* x, const float* dt, const float* A, const float* Bm,
                                   const float* Cm, const float* Dp, float* y, float* state,
                                   const int* lens_host, int P, int D, int N, void* stream);

/* ------------------------------------------------------------------------
 * WKV with a token-dependent decay.  [rwkv], Notes For Future Readers, says
 * that RWKV generations with a per-token decay call for a different chunk
 * form, and gives none; this is the reading that the RWKV-4 recurrence above
 * takes a decay w_t per row and channel in place of w:
 *   A_t = e^{w_t} A_{t-1} + e^{k_t} v_t,  B_t = e^{w_t} B_{t-1} + e^{k_t},
 *   wkv_t = (A_{t-1} + e^{u+k_t} v_t) / (B_{t-1} + e^{u+k_t}).
 * The state is the same (num, den, max) triple as for K2, and a decay that is
 * the same on every row gives the K2 result.
 *  k, v, w, wkv [B, S, C] float (w < 0)
 *  u            [C] float
 *  num, den, mx [B, C] float, read and updated in place
 *  C >= 1, 0 <= S <= LRC_MAX_ROWS, B >= 0.  Errors: as for the other chunk calls.
 * ---------------------------------------------------------------------- */
lrc_status lrc_wkv_tdecay_rows(const float* k, const float* v, const float* w, const float* u, float* wkv,
                               float* num, float* den, float* mx, int B, int S, int C, void* stream);

/* Driver: k, v, w, wkv [R, C] packed rows; num, den, mx [P, C] in place. */
lrc_status lrc_wkv_tdecay_prefill(const float* k, const float* v, const float* w, const float* u, float* wkv,
                                  float* num, float* den, float* mx, const int* lens_host, int P, int C,
                                  void* stream);

/* ------------------------------------------------------------------------
 * Diagnostics.  The WKV kernels (K2 and the token-dependent decay) pass each
 * chunk between the waves of a workgroup through counters in LDS, and a wave
 * waits for another with a bounded poll (about 2^20 polls).  A wait that runs
 * out goes on rather than hang and is counted on the device; the count stays
 * 0 unless a launch could not make progress, and outputs of a launch that
 * counted one are not to be trusted.  This call synchronizes `stream`, writes
 * the current GPU's count to *count_host (host memory), and with reset != 0
 * sets it back to 0. */
lrc_status lrc_wait_timeouts(unsigned* count_host, int reset, void* stream);

/* ------------------------------------------------------------------------ */
const char* lrc_status_string(lrc_status s);
/* Detail of the last error on the calling thread ("" if none). */
const char* lrc_last_error(void);
/* (major << 16) | (minor << 8) | patch */
int lrc_version(void);

#ifdef __cplusplus
}
#endif
#endif /* LRC_H */

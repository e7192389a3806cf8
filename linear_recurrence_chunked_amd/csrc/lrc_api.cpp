// C ABI of liblrc.so: argument validation, prompt layout, launch and error
// reporting.  Validation makes no HIP call, so a rejected call touches
// neither the device nor the stream.
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>
#include <numeric>

#include "lrc_internal.h"

namespace lrc {
namespace {
// Bounded LDS waits that gave up (see lds_wait_at_least), one counter per GPU.
__device__ unsigned g_wait_timeouts = 0;
}  // namespace

int compute_units() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return n;
}

unsigned* wait_timeouts_counter() {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static unsigned* ptr[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_wait_timeouts)) != hipSuccess) return nullptr;
        ptr[dev] = static_cast<unsigned*>(p);
    }
    return ptr[dev];
}
}  // namespace lrc

namespace {

thread_local char g_err[512] = "";

lrc_status fail(lrc_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

lrc_status ok() {
    g_err[0] = '\0';
    return LRC_OK;
}

constexpr uint64_t kMaxElems = 1ull << 46;  // sanity bound on any tensor's element count

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t esize(lrc_dtype dt) { return dt == LRC_BF16 || dt == LRC_BF16_SPLIT ? 2 : 4; }

bool overlap(const void* a, uint64_t abytes, const void* b, uint64_t bbytes) {
    if (!a || !b || abytes == 0 || bbytes == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + bbytes && b0 < a0 + abytes;
}

// A launch error leaves queued work behind: drain the stream before
// reporting, so nothing still reads the caller's buffers afterwards.
lrc_status check_launch(hipError_t e, hipStream_t st, const char* what) {
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) {
        (void)hipStreamSynchronize(st);
        return fail(LRC_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
    }
    return ok();
}

lrc_status uniform_batch(int B, int S, lrc::Batch& bt) {
    if (B < 0) return fail(LRC_ERR_SHAPE, "batch %d < 0", B);
    if (B > 65535) return fail(LRC_ERR_SHAPE, "batch %d > 65535 in one chunk call", B);
    if (S < 0 || S > LRC_MAX_ROWS) return fail(LRC_ERR_ROWS, "chunk rows %d outside [0, %d]", S, LRC_MAX_ROWS);
    bt.P = B;
    bt.uniform = S;
    return LRC_OK;
}

lrc_status packed_batch(const int* lens, int P, lrc::Batch& bt, long& rows) {
    if (!lens) return fail(LRC_ERR_NULL, "lens_host is NULL");
    if (P < 1 || P > LRC_MAX_PROMPTS) return fail(LRC_ERR_SHAPE, "prompts %d outside [1, %d]", P, LRC_MAX_PROMPTS);
    bt.P = P;
    bt.uniform = -1;
    long r = 0;
    for (int p = 0; p < P; ++p) {
        if (lens[p] < 0) return fail(LRC_ERR_ROWS, "prompt %d has length %d < 0", p, lens[p]);
        bt.row_off[p] = static_cast<int>(r);
        r += lens[p];
        if (r > 0x7fffffffL) return fail(LRC_ERR_SHAPE, "total rows exceed 2^31-1");
    }
    bt.row_off[P] = static_cast<int>(r);
    std::iota(bt.order, bt.order + P, 0);
    std::stable_sort(bt.order, bt.order + P, [&](int a, int b) { return lens[a] > lens[b]; });
    rows = r;
    return LRC_OK;
}

#define REQUIRE(cond, code, ...) \
    do {                         \
        if (!(cond)) return fail(code, __VA_ARGS__); \
    } while (0)

#define REQUIRE_PTR(p) REQUIRE((p) != nullptr, LRC_ERR_NULL, "%s is NULL", #p)
// Tensors with no elements (a chunk of zero rows) may be NULL.
#define REQUIRE_PTR_IF(p, nonempty) REQUIRE(!(nonempty) || (p) != nullptr, LRC_ERR_NULL, "%s is NULL", #p)
#define REQUIRE_ALIGN(p) REQUIRE(aligned16(p), LRC_ERR_ALIGN, "%s is not 16-byte aligned", #p)

// ---------------------------------------------------------------- K0 conv
lrc_status conv_common(const void* x, void* y, const void* s_in, void* s_out, const float* w, const float* bias,
                       long rows, int P, int C, int K, lrc_dtype dt) {
    REQUIRE_PTR_IF(x, rows > 0); REQUIRE_PTR_IF(y, rows > 0); REQUIRE_PTR(w);
    REQUIRE(K >= 1 && K <= LRC_MAX_CONV_K, LRC_ERR_SHAPE, "conv width %d outside [1, %d]", K, LRC_MAX_CONV_K);
    REQUIRE(C >= 1, LRC_ERR_SHAPE, "channels %d < 1", C);
    REQUIRE(dt == LRC_F32 || dt == LRC_BF16, LRC_ERR_DTYPE, "unsupported dtype %d", (int)dt);
    if (K > 1) { REQUIRE_PTR_IF(s_in, P > 0); REQUIRE_PTR_IF(s_out, P > 0); }
    REQUIRE_ALIGN(x); REQUIRE_ALIGN(y); REQUIRE_ALIGN(w);
    if (bias) REQUIRE_ALIGN(bias);
    if (K > 1) { REQUIRE_ALIGN(s_in); REQUIRE_ALIGN(s_out); }
    const uint64_t xb = (uint64_t)rows * C * esize(dt);
    const uint64_t sb = (uint64_t)P * (K - 1) * C * esize(dt);
    REQUIRE((uint64_t)rows * C < kMaxElems, LRC_ERR_SHAPE, "tensor too large");
    REQUIRE(!overlap(y, xb, x, xb), LRC_ERR_ALIAS, "y overlaps x");
    REQUIRE(!overlap(y, xb, s_in, sb) && !overlap(y, xb, s_out, sb), LRC_ERR_ALIAS, "y overlaps the conv state");
    REQUIRE(!overlap(s_out, sb, x, xb), LRC_ERR_ALIAS, "state_out overlaps x");
    REQUIRE(s_in == s_out || !overlap(s_out, sb, s_in, sb), LRC_ERR_ALIAS, "state_out partially overlaps state_in");
    REQUIRE(!overlap(y, xb, w, (uint64_t)C * K * 4), LRC_ERR_ALIAS, "y overlaps w");
    return LRC_OK;
}

// ---------------------------------------------------------------- K1 scan
lrc_status scan_common(const float* a, const float* b, float* h, const float* h0, float* hS, long rows, int P,
                       int D, int N) {
    REQUIRE_PTR_IF(a, rows > 0); REQUIRE_PTR_IF(b, rows > 0); REQUIRE_PTR_IF(h, rows > 0);
    REQUIRE_PTR_IF(h0, P > 0); REQUIRE_PTR_IF(hS, P > 0);
    REQUIRE(D >= 1 && N >= 1, LRC_ERR_SHAPE, "d_inner %d, d_state %d must be >= 1", D, N);
    const uint64_t E = (uint64_t)D * N;
    REQUIRE(E < (1ull << 31), LRC_ERR_SHAPE, "d_inner * d_state too large");
    REQUIRE((uint64_t)rows * E < kMaxElems, LRC_ERR_SHAPE, "tensor too large");
    REQUIRE_ALIGN(a); REQUIRE_ALIGN(b); REQUIRE_ALIGN(h); REQUIRE_ALIGN(h0); REQUIRE_ALIGN(hS);
    const uint64_t tb = (uint64_t)rows * E * 4, sb = (uint64_t)P * E * 4;
    REQUIRE(!overlap(h, tb, a, tb) && !overlap(h, tb, b, tb), LRC_ERR_ALIAS, "h overlaps a or b");
    REQUIRE(!overlap(h, tb, h0, sb) && !overlap(h, tb, hS, sb), LRC_ERR_ALIAS, "h overlaps the state");
    REQUIRE(!overlap(hS, sb, a, tb) && !overlap(hS, sb, b, tb), LRC_ERR_ALIAS, "state overlaps a or b");
    REQUIRE(h0 == hS || !overlap(hS, sb, h0, sb), LRC_ERR_ALIAS, "hS partially overlaps h0");
    return LRC_OK;
}

// ---------------------------------------------------------------- K2 wkv
lrc_status wkv_common(const float* k, const float* v, const float* w, const float* u, float* wkv, float* num,
                      float* den, float* mx, long rows, int P, int C) {
    REQUIRE_PTR_IF(k, rows > 0); REQUIRE_PTR_IF(v, rows > 0); REQUIRE_PTR(w); REQUIRE_PTR(u);
    REQUIRE_PTR_IF(wkv, rows > 0);
    REQUIRE_PTR_IF(num, P > 0); REQUIRE_PTR_IF(den, P > 0); REQUIRE_PTR_IF(mx, P > 0);
    REQUIRE(C >= 1, LRC_ERR_SHAPE, "channels %d < 1", C);
    REQUIRE((uint64_t)rows * C < kMaxElems, LRC_ERR_SHAPE, "tensor too large");
    REQUIRE_ALIGN(k); REQUIRE_ALIGN(v); REQUIRE_ALIGN(w); REQUIRE_ALIGN(u); REQUIRE_ALIGN(wkv);
    REQUIRE_ALIGN(num); REQUIRE_ALIGN(den); REQUIRE_ALIGN(mx);
    const uint64_t tb = (uint64_t)rows * C * 4, sb = (uint64_t)P * C * 4;
    REQUIRE(!overlap(wkv, tb, k, tb) && !overlap(wkv, tb, v, tb), LRC_ERR_ALIAS, "wkv overlaps k or v");
    const float* st[3] = {num, den, mx};
    for (int i = 0; i < 3; ++i) {
        REQUIRE(!overlap(wkv, tb, st[i], sb), LRC_ERR_ALIAS, "wkv overlaps the state");
        REQUIRE(!overlap(st[i], sb, k, tb) && !overlap(st[i], sb, v, tb), LRC_ERR_ALIAS, "state overlaps k or v");
        for (int j = i + 1; j < 3; ++j)
            REQUIRE(!overlap(st[i], sb, st[j], sb), LRC_ERR_ALIAS, "num, den and max overlap each other");
    }
    return LRC_OK;
}

// ---------------------------------------------------------------- WKV, token-dependent decay
lrc_status wkv_td_common(const float* k, const float* v, const float* w, const float* u, float* wkv, float* num,
                         float* den, float* mx, long rows, int P, int C) {
    REQUIRE_PTR_IF(k, rows > 0); REQUIRE_PTR_IF(v, rows > 0); REQUIRE_PTR_IF(w, rows > 0); REQUIRE_PTR(u);
    REQUIRE_PTR_IF(wkv, rows > 0);
    REQUIRE_PTR_IF(num, P > 0); REQUIRE_PTR_IF(den, P > 0); REQUIRE_PTR_IF(mx, P > 0);
    REQUIRE(C >= 1, LRC_ERR_SHAPE, "channels %d < 1", C);
    REQUIRE((uint64_t)rows * C < kMaxElems, LRC_ERR_SHAPE, "tensor too large");
    REQUIRE_ALIGN(k); REQUIRE_ALIGN(v); REQUIRE_ALIGN(w); REQUIRE_ALIGN(u); REQUIRE_ALIGN(wkv);
    REQUIRE_ALIGN(num); REQUIRE_ALIGN(den); REQUIRE_ALIGN(mx);
    const uint64_t tb = (uint64_t)rows * C * 4, sb = (uint64_t)P * C * 4;
    REQUIRE(!overlap(wkv, tb, k, tb) && !overlap(wkv, tb, v, tb) && !overlap(wkv, tb, w, tb), LRC_ERR_ALIAS,
            "wkv overlaps k, v or w");
    const float* st[3] = {num, den, mx};
    for (int i = 0; i < 3; ++i) {
        REQUIRE(!overlap(wkv, tb, st[i], sb), LRC_ERR_ALIAS, "wkv overlaps the state");
        REQUIRE(!overlap(st[i], sb, k, tb) && !overlap(st[i], sb, v, tb) && !overlap(st[i], sb, w, tb),
                LRC_ERR_ALIAS, "state overlaps k, v or w");
        for (int j = i + 1; j < 3; ++j)
            REQUIRE(!overlap(st[i], sb, st[j], sb), LRC_ERR_ALIAS, "num, den and max overlap each other");
    }
    return LRC_OK;
}

// ---------------------------------------------------------------- K3 gdn
lrc_status gdn_common(const void* q, const void* k, const void* v, const float* beta, const float* g, float* o,
                      const float* S_in, float* S_out, long rows, int P, int Hk, int Hv, int dk, int dv,
                      lrc_dtype dt) {
    REQUIRE_PTR_IF(q, rows > 0); REQUIRE_PTR_IF(k, rows > 0); REQUIRE_PTR_IF(v, rows > 0);
    REQUIRE_PTR_IF(beta, rows > 0); REQUIRE_PTR_IF(g, rows > 0); REQUIRE_PTR_IF(o, rows > 0);
    REQUIRE_PTR_IF(S_in, P > 0); REQUIRE_PTR_IF(S_out, P > 0);
    REQUIRE(dt == LRC_F32 || dt == LRC_BF16 || dt == LRC_BF16_SPLIT, LRC_ERR_DTYPE, "unsupported dtype %d", (int)dt);
    REQUIRE(Hk >= 1 && Hv >= 1 && Hv % Hk == 0, LRC_ERR_SHAPE, "value heads %d must be a positive multiple of key heads %d", Hv, Hk);
    REQUIRE(Hv <= 65535, LRC_ERR_SHAPE, "value heads %d > 65535", Hv);
    REQUIRE(dk == 32 || dk == 64 || dk == 128, LRC_ERR_SHAPE, "dk %d not in {32, 64, 128}", dk);
    REQUIRE(dv == 32 || dv == 64 || dv == 128, LRC_ERR_SHAPE, "dv %d not in {32, 64, 128}", dv);
    REQUIRE((uint64_t)rows * Hv * dv < kMaxElems, LRC_ERR_SHAPE, "tensor too large");
    REQUIRE_ALIGN(q); REQUIRE_ALIGN(k); REQUIRE_ALIGN(v); REQUIRE_ALIGN(beta); REQUIRE_ALIGN(g); REQUIRE_ALIGN(o);
    REQUIRE_ALIGN(S_in); REQUIRE_ALIGN(S_out);
    const uint64_t es = esize(dt);
    const uint64_t qb = (uint64_t)rows * Hk * dk * es, vb = (uint64_t)rows * Hv * dv * es;
    const uint64_t gb = (uint64_t)rows * Hv * 4, ob = (uint64_t)rows * Hv * dv * 4;
    const uint64_t sb = (uint64_t)P * Hv * dk * dv * 4;
    const void* ins[5] = {q, k, v, beta, g};
    const uint64_t inb[5] = {qb, qb, vb, gb, gb};
    for (int i = 0; i < 5; ++i) {
        REQUIRE(!overlap(o, ob, ins[i], inb[i]), LRC_ERR_ALIAS, "o overlaps an input");
        REQUIRE(!overlap(S_out, sb, ins[i], inb[i]), LRC_ERR_ALIAS, "S_out overlaps an input");
    }
    REQUIRE(!overlap(o, ob, S_in, sb) && !overlap(o, ob, S_out, sb), LRC_ERR_ALIAS, "o overlaps the state");
    REQUIRE(S_in == S_out || !overlap(S_out, sb, S_in, sb), LRC_ERR_ALIAS, "S_out partially overlaps S_in");
    return LRC_OK;
}

// ---------------------------------------------------------------- time shift
lrc_status shift_common(const float* x, float* out, const float* s_in, float* s_out, const float* mix, long rows,
                        int P, int C, int M) {
    REQUIRE_PTR_IF(x, rows > 0); REQUIRE_PTR_IF(out, rows > 0); REQUIRE_PTR(mix);
    REQUIRE_PTR_IF(s_in, P > 0); REQUIRE_PTR_IF(s_out, P > 0);
    REQUIRE(C >= 1, LRC_ERR_SHAPE, "channels %d < 1", C);
    REQUIRE(M >= 1 && M <= LRC_MAX_MIX, LRC_ERR_SHAPE, "mixed inputs %d outside [1, %d]", M, LRC_MAX_MIX);
    REQUIRE((uint64_t)rows * C * M < kMaxElems, LRC_ERR_SHAPE, "tensor too large");
    REQUIRE_ALIGN(x); REQUIRE_ALIGN(out); REQUIRE_ALIGN(s_in); REQUIRE_ALIGN(s_out); REQUIRE_ALIGN(mix);
    const uint64_t xb = (uint64_t)rows * C * 4, ob = xb * M, sb = (uint64_t)P * C * 4, mb = (uint64_t)M * C * 4;
    REQUIRE(!overlap(out, ob, x, xb) && !overlap(out, ob, mix, mb), LRC_ERR_ALIAS, "out overlaps x or mix");
    REQUIRE(!overlap(out, ob, s_in, sb) && !overlap(out, ob, s_out, sb), LRC_ERR_ALIAS, "out overlaps the state");
    REQUIRE(!overlap(s_out, sb, x, xb) && !overlap(s_out, sb, mix, mb), LRC_ERR_ALIAS, "state_out overlaps x or mix");
    REQUIRE(s_in == s_out || !overlap(s_out, sb, s_in, sb), LRC_ERR_ALIAS, "state_out partially overlaps state_in");
    return LRC_OK;
}

// ---------------------------------------------------------------- mamba mixer
lrc_status mixer_common(const float* x, const float* dt, const float* A, const float* Bm, const float* Cm,
                        const float* Dp, float* y, const float* h_in, float* h_out, long rows, int P, int D, int N) {
    REQUIRE_PTR_IF(x, rows > 0); REQUIRE_PTR_IF(dt, rows > 0); REQUIRE_PTR_IF(Bm, rows > 0);
    REQUIRE_PTR_IF(Cm, rows > 0); REQUIRE_PTR_IF(y, rows > 0);
    REQUIRE_PTR(A); REQUIRE_PTR(Dp); REQUIRE_PTR_IF(h_in, P > 0); REQUIRE_PTR_IF(h_out, P > 0);
    REQUIRE(D >= 1, LRC_ERR_SHAPE, "d_inner %d < 1", D);
    REQUIRE(N == 2 || N == 4 || N == 8 || N == 16 || N == 32 || N == 64, LRC_ERR_SHAPE,
            "d_state %d is not 2, 4, 8, 16, 32 or 64", N);
    REQUIRE((uint64_t)rows * D < kMaxElems && (uint64_t)P * D * N < kMaxElems, LRC_ERR_SHAPE, "tensor too large");
    REQUIRE_ALIGN(x); REQUIRE_ALIGN(dt); REQUIRE_ALIGN(A); REQUIRE_ALIGN(Bm); REQUIRE_ALIGN(Cm); REQUIRE_ALIGN(Dp);
    REQUIRE_ALIGN(y); REQUIRE_ALIGN(h_in); REQUIRE_ALIGN(h_out);
    const uint64_t xb = (uint64_t)rows * D * 4, bb = (uint64_t)rows * N * 4, sb = (uint64_t)P * D * N * 4;
    const uint64_t ab = (uint64_t)D * N * 4, db = (uint64_t)D * 4;
    const void* ins[] = {x, dt, Bm, Cm, A, Dp};
    const uint64_t inb[] = {xb, xb, bb, bb, ab, db};
    for (int i = 0; i < 6; ++i) {
        REQUIRE(!overlap(y, xb, ins[i], inb[i]), LRC_ERR_ALIAS, "y overlaps an input");
        REQUIRE(!overlap(h_out, sb, ins[i], inb[i]), LRC_ERR_ALIAS, "h_out overlaps an input");
    }
    REQUIRE(!overlap(y, xb, h_in, sb) && !overlap(y, xb, h_out, sb), LRC_ERR_ALIAS, "y overlaps the state");
    REQUIRE(h_in == h_out || !overlap(h_out, sb, h_in, sb), LRC_ERR_ALIAS, "h_out partially overlaps h_in");
    return LRC_OK;
}

}  // namespace


extern "C" {

lrc_status lrc_conv_rows(const void* x, void* y, const void* state_in, void* state_out, const float* w,
                         const float* bias, int B, int S, int C, int K, lrc_dtype dt, void* stream) {
    lrc::Batch bt;
    lrc_status s = uniform_batch(B, S, bt);
    if (s != LRC_OK) return s;
    if ((s = conv_common(x, y, state_in, state_out, w, bias, (long)B * S, B, C, K, dt)) != LRC_OK) return s;
    if (B == 0) return ok();
    auto st = static_cast<hipStream_t>(stream);
    return check_launch(lrc::launch_conv(x, y, state_in, state_out, w, bias, bt, C, K, dt, st), st, "conv");
}

lrc_status lrc_conv_prefill(const void* x, void* y, void* state, const float* w, const float* bias,
                            const int* lens_host, int P, int C, int K, lrc_dtype dt, void* stream) {
    thread_local lrc::Batch bt;
    long rows = 0;
    lrc_status s = packed_batch(lens_host, P, bt, rows);
    if (s != LRC_OK) return s;
    if ((s = conv_common(x, y, state, state, w, bias, rows, P, C, K, dt)) != LRC_OK) return s;
    auto st = static_cast<hipStream_t>(stream);
    return check_launch(lrc::launch_conv(x, y, state, state, w, bias, bt, C, K, dt, st), st, "conv prefill");
}

lrc_status lrc_scan_rows(const float* a, const float* b, float* h, const float* h0, float* hS, int B, int S, int D,
                         int N, void* stream) {
    lrc::Batch bt;
    lrc_status s = uniform_batch(B, S, bt);
    if (s != LRC_OK) return s;
    if ((s = scan_common(a, b, h, h0, hS, (long)B * S, B, D, N)) != LRC_OK) return s;
    if (B == 0) return ok();
    auto st = static_cast<hipStream_t>(stream);
    return check_launch(lrc::launch_scan(a, b, h, h0, hS, bt, (long)D * N, st), st, "scan");
}

lrc_status lrc_scan_prefill(const float* a, const float* b, float* h, float* state, const int* lens_host, int P,
                            int D, int N, void* stream) {
    thread_local lrc::Batch bt;
    long rows = 0;
    lrc_status s = packed_batch(lens_host, P, bt, rows);
    if (s != LRC_OK) return s;
    if ((s = scan_common(a, b, h, state, state, rows, P, D, N)) != LRC_OK) return s;
    auto st = static_cast<hipStream_t>(stream);
    return check_launch(lrc::launch_scan(a, b, h, state, state, bt, (long)D * N, st), st, "scan prefill");
}

size_t lrc_scan_workspace_size(int P, int D, int N) {
    if (P < 1 || D < 1 || N < 1) return 0;
    return lrc::scan_workspace_bytes(P, (long)D * N);
}

lrc_status lrc_scan_prefill_ws(const float* a, const float* b, float* h, float* state, const int* lens_host, int P,
                               int D, int N, void* workspace, size_t workspace_bytes, void* stream) {
    thread_local lrc::Batch bt;
    long rows = 0;
    lrc_status s = packed_batch(lens_host, P, bt, rows);
    if (s != LRC_OK) return s;
    if ((s = scan_common(a, b, h, state, state, rows, P, D, N)) != LRC_OK) return s;
    const long E = (long)D * N;
    const size_t need = lrc::scan_workspace_bytes(P, E);
    REQUIRE_PTR(workspace);
    REQUIRE(aligned16(workspace), LRC_ERR_ALIGN, "workspace is not 16-byte aligned");
    REQUIRE(workspace_bytes >= need, LRC_ERR_SHAPE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
    const uint64_t tb = (uint64_t)rows * E * 4, sb = (uint64_t)P * E * 4;
    REQUIRE(!overlap(workspace, need, a, tb) && !overlap(workspace, need, b, tb) && !overlap(workspace, need, h, tb) &&
                !overlap(workspace, need, state, sb),
            LRC_ERR_ALIAS, "workspace overlaps a tensor");
    REQUIRE(lrc::scan_tiled_tiles_bound(rows, P, E) < (1l << 31), LRC_ERR_SHAPE, "too many tiles for one launch");
    auto st = static_cast<hipStream_t>(stream);
    return check_launch(lrc::launch_scan_tiled(a, b, h, state, bt, E, workspace, st), st, "scan prefill (tiled)");
}

lrc_status lrc_scan_prefill_static(const float* a, const float* b, float* h, float* state, const int* lens_host,
                                   int P, int D, int N, void* stream) {
    thread_local lrc::Batch bt;
    long rows = 0;
    lrc_status s = packed_batch(lens_host, P, bt, rows);
    if (s != LRC_OK) return s;
    if ((s = scan_common(a, b, h, state, state, rows, P, D, N)) != LRC_OK) return s;
    const long E = (long)D * N;
    const size_t need = lrc::scan_workspace_bytes(P, E);
    REQUIRE(need <= lrc::kScanStaticScratchBytes, LRC_ERR_SHAPE,
            "%d prompts of %ld state elements need %zu bytes of scratch, more than the fixed %zu (at most %zu "
            "prompt x 128-element blocks)",
            P, E, need, lrc::kScanStaticScratchBytes, (lrc::kScanStaticScratchBytes - 256) / 8);
    REQUIRE(lrc::scan_tiled_tiles_bound(rows, P, E) < (1l << 31), LRC_ERR_SHAPE, "too many tiles for one launch");
    auto st = static_cast<hipStream_t>(stream);
    return check_launch(lrc::launch_scan_tiled_static(a, b, h, state, bt, E, st), st, "scan prefill (fixed scratch)");
}

lrc_status lrc_wait_timeouts(unsigned* count_host, int reset, void* stream) {
    REQUIRE_PTR(count_host);
    auto st = static_cast<hipStream_t>(stream);
    unsigned* c = lrc::wait_timeouts_counter();
    if (!c) return fail(LRC_ERR_LAUNCH, "wait-timeout counter: no device address");
    hipError_t e = hipMemcpyAsync(count_host, c, sizeof(unsigned), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e == hipSuccess && reset) {
        static const unsigned zero = 0;
        e = hipMemcpyAsync(c, &zero, sizeof(unsigned), hipMemcpyHostToDevice, st);
        if (e == hipSuccess) e = hipStreamSynchronize(st);
    }
    return check_launch(e, st, "wait-timeout counter");
}

lrc_status lrc_wkv4_rows(const float* k, const float* v, const float* w, const float* u, float* wkv, float* num,
                         float* den, float* mx, int B, int S, int C, void* stream) {
    lrc::Batch bt;
    lrc_status s = uniform_batch(B, S, bt);
    if (s != LRC_OK) return s;
    if ((s = wkv_common(k, v, w, u, wkv, num, den, mx, (long)B * S, B, C)) != LRC_OK) return s;
    if (B == 0) return ok();
    auto st = static_cast<hipStream_t>(stream);
    return check_launch(lrc::launch_wkv4(k, v, w, u, wkv, num, den, mx, bt, C, st), st, "wkv4");
}

lrc_status lrc_wkv4_prefill(const float* k, const float* v, const float* w, const float* u, float* wkv, float* num,
                            float* den, float* mx, const int* lens_host, int P, int C, void* stream) {
    thread_local lrc::Batch bt;
    long rows = 0;
    lrc_status s = packed_batch(lens_host, P, bt, rows);
    if (s != LRC_OK) return s;
    if ((s = wkv_common(k, v, w, u, wkv, num, den, mx, rows, P, C)) != LRC_OK) return s;
    auto st = static_cast<hipStream_t>(stream);
    return check_launch(lrc::launch_wkv4(k, v, w, u, wkv, num, den, mx, bt, C, st), st, "wkv4 prefill");
}

lrc_status lrc_wkv_tdecay_rows(const float* k, const float* v, const float* w, const float* u, float* wkv,
                               float* num, float* den, float* mx, int B, int S, int C, void* stream) {
    lrc::Batch bt;
    lrc_status s = uniform_batch(B, S, bt);
    if (s != LRC_OK) return s;
    if ((s = wkv_td_common(k, v, w, u, wkv, num, den, mx, (long)B * S, B, C)) != LRC_OK) return s;
    if (B == 0) return ok();
    auto st = static_cast<hipStream_t>(stream);
    return check_launch(lrc::launch_wkv_tdecay(k, v, w, u, wkv, num, den, mx, bt, C, st), st, "wkv tdecay");
}

lrc_status lrc_wkv_tdecay_prefill(const float* k, const float* v, const float* w, const float* u, float* wkv,
                                  float* num, float* den, float* mx, const int* lens_host, int P, int C,
                                  void* stream) {
    thread_local lrc::Batch bt;
    long rows = 0;
    lrc_status s = packed_batch(lens_host, P, bt, rows);
    if (s != LRC_OK) return s;
    if ((s = wkv_td_common(k, v, w, u, wkv, num, den, mx, rows, P, C)) != LRC_OK) return s;
    auto st = static_cast<hipStream_t>(stream);
    return check_launch(lrc::launch_wkv_tdecay(k, v, w, u, wkv, num, den, mx, bt, C, st), st,
                        "wkv tdecay prefill");
}

lrc_status lrc_gdn_chunk(const void* q, const void* k, const void* v, const float* beta, const float* g, float* o,
                         const float* S_in, float* S_out, int B, int S, int Hk, int Hv, int dk, int dv, lrc_dtype dt,
                         void* stream) {
    lrc::Batch bt;
    lrc_status s = uniform_batch(B, S, bt);
    if (s != LRC_OK) return s;
    if ((s = gdn_common(q, k, v, beta, g, o, S_in, S_out, (long)B * S, B, Hk, Hv, dk, dv, dt)) != LRC_OK) return s;
    if (B == 0) return ok();
    auto st = static_cast<hipStream_t>(stream);
    return check_launch(lrc::launch_gdn(q, k, v, beta, g, o, S_in, S_out, bt, Hk, Hv, dk, dv, dt, st), st, "gdn");
}

lrc_status lrc_gdn_prefill(const void* q, const void* k, const void* v, const float* beta, const float* g, float* o,
                           float* state, const int* lens_host, int P, int Hk, int Hv, int dk, int dv, lrc_dtype dt,
                           void* stream) {
    thread_local lrc::Batch bt;
    long rows = 0;
    lrc_status s = packed_batch(lens_host, P, bt, rows);
    if (s != LRC_OK) return s;
    if ((s = gdn_common(q, k, v, beta, g, o, state, state, rows, P, Hk, Hv, dk, dv, dt)) != LRC_OK) return s;
    auto st = static_cast<hipStream_t>(stream);
    return check_launch(lrc::launch_gdn(q, k, v, beta, g, o, state, state, bt, Hk, Hv, dk, dv, dt, st), st,
                        "gdn prefill");
}

size_t lrc_gdn_workspace_bytes(int P, long total_rows, int Hk, int Hv, int dk, int dv, lrc_dtype dt) {
    if (P < 1 || total_rows < 0 || Hk < 1 || Hv < 1 || Hv % Hk != 0 || dt != LRC_BF16) return 0;
    if ((dk != 32 && dk != 64 && dk != 128) || (dv != 32 && dv != 64 && dv != 128)) return 0;
    return (size_t)(total_rows / 64 + P) * Hv * lrc::gdn_cp_block_bytes(dk, dv);
}

lrc_status lrc_gdn_prefill_ws(const void* q, const void* k, const void* v, const float* beta, const float* g,
                              float* o, float* state, const int* lens_host, int P, int Hk, int Hv, int dk, int dv,
                              lrc_dtype dt, void* workspace, size_t workspace_bytes, void* stream) {
    thread_local lrc::Batch bt;
    long rows = 0;
    lrc_status s = packed_batch(lens_host, P, bt, rows);
    if (s != LRC_OK) return s;
    if ((s = gdn_common(q, k, v, beta, g, o, state, state, rows, P, Hk, Hv, dk, dv, dt)) != LRC_OK) return s;
    REQUIRE(dt == LRC_BF16, LRC_ERR_DTYPE, "the chunk-parallel form takes bf16 inputs (LRC_BF16) only");
    long chunks = 0;
    for (int p = 0; p < P; ++p) chunks += (lens_host[p] + 63) / 64;
    REQUIRE(chunks < (1l << 31), LRC_ERR_SHAPE, "too many chunks for one launch");
    const size_t need = (size_t)chunks * Hv * lrc::gdn_cp_block_bytes(dk, dv);
    REQUIRE_PTR_IF(workspace, need > 0);
    REQUIRE_ALIGN(workspace);
    REQUIRE(workspace_bytes >= need, LRC_ERR_SHAPE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
    const uint64_t es = esize(dt);
    const uint64_t qb = (uint64_t)rows * Hk * dk * es, vb = (uint64_t)rows * Hv * dv * es;
    const uint64_t gb = (uint64_t)rows * Hv * 4, ob = (uint64_t)rows * Hv * dv * 4;
    const uint64_t sb = (uint64_t)P * Hv * dk * dv * 4;
    const void* ts[7] = {q, k, v, beta, g, o, state};
    const uint64_t tb[7] = {qb, qb, vb, gb, gb, ob, sb};
    for (int i = 0; i < 7; ++i) REQUIRE(!overlap(workspace, need, ts[i], tb[i]), LRC_ERR_ALIAS, "workspace overlaps a tensor");
    if (need == 0) return ok();
    auto st = static_cast<hipStream_t>(stream);
    return check_launch(lrc::launch_gdn_chunk_parallel(q, k, v, beta, g, o, state, bt, Hk, Hv, dk, dv, workspace, st),
                        st, "gdn prefill (chunk-parallel)");
}

lrc_status lrc_unit_lower_inverse(const float* A, float* T, int batch, int n, void* stream) {
    REQUIRE_PTR(A); REQUIRE_PTR(T);
    REQUIRE(batch >= 0 && batch <= (1 << 30), LRC_ERR_SHAPE, "batch %d outside [0, 2^30]", batch);
    REQUIRE(n >= 0 && n <= LRC_MAX_ROWS, LRC_ERR_ROWS, "n %d outside [0, %d]", n, LRC_MAX_ROWS);
    REQUIRE_ALIGN(A); REQUIRE_ALIGN(T);
    const uint64_t bytes = (uint64_t)batch * n * n * 4;
    REQUIRE(!overlap(A, bytes, T, bytes), LRC_ERR_ALIAS, "T overlaps A");
    if (batch == 0 || n == 0) return ok();
    auto st = static_cast<hipStream_t>(stream);
    return check_launch(lrc::launch_unit_lower_inverse(A, T, batch, n, st), st, "unit_lower_inverse");
}

lrc_status lrc_time_shift_rows(const float* x, float* out, const float* state_in, float* state_out,
                               const float* mix, int B, int S, int C, int M, void* stream) {
    lrc::Batch bt;
    lrc_status s = uniform_batch(B, S, bt);
    if (s != LRC_OK) return s;
    if ((s = shift_common(x, out, state_in, state_out, mix, (long)B * S, B, C, M)) != LRC_OK) return s;
    if (B == 0) return ok();
    auto st = static_cast<hipStream_t>(stream);
    return check_launch(lrc::launch_time_shift(x, out, state_in, state_out, mix, bt, C, M, (long)B * S * C, st),
                        st, "time shift");
}

lrc_status lrc_time_shift_prefill(const float* x, float* out, float* state, const float* mix, const int* lens_host,
                                  int P, int C, int M, void* stream) {
    thread_local lrc::Batch bt;
    long rows = 0;
    lrc_status s = packed_batch(lens_host, P, bt, rows);
    if (s != LRC_OK) return s;
    if ((s = shift_common(x, out, state, state, mix, rows, P, C, M)) != LRC_OK) return s;
    auto st = static_cast<hipStream_t>(stream);
    return check_launch(lrc::launch_time_shift(x, out, state, state, mix, bt, C, M, rows * C, st), st,
                        "time shift prefill");
}

lrc_status lrc_mamba_mixer_rows(const float* x, const float* dt, const float* A, const float* Bm, const float* Cm,
                                const float* Dp, float* y, const float* h_in, float* h_out, int B, int S, int D,
                                int N, void* stream) {
    lrc::Batch bt;
    lrc_status s = uniform_batch(B, S, bt);
    if (s != LRC_OK) return s;
    if ((s = mixer_common(x, dt, A, Bm, Cm, Dp, y, h_in, h_out, (long)B * S, B, D, N)) != LRC_OK) return s;
    if (B == 0) return ok();
    auto st = static_cast<hipStream_t>(stream);
    return check_launch(lrc::launch_mamba_mixer(x, dt, A, Bm, Cm, Dp, y, h_in, h_out, bt, D, N, st), st,
                        "mamba mixer");
}

lrc_status lrc_mamba_mixer_prefill(const float* x, const float* dt, const float* A, const float* Bm, const float* Cm,
                                   const float* Dp, float* y, float* state, const int* lens_host, int P, int D, int N,
                                   void* stream) {
    thread_local lrc::Batch bt;
    long rows = 0;
    lrc_status s = packed_batch(lens_host, P, bt, rows);
    if (s != LRC_OK) return s;
    if ((s = mixer_common(x, dt, A, Bm, Cm, Dp, y, state, state, rows, P, D, N)) != LRC_OK) return s;
    auto st = static_cast<hipStream_t>(stream);
    return check_launch(lrc::launch_mamba_mixer(x, dt, A, Bm, Cm, Dp, y, state, state, bt, D, N, st), st,
                        "mamba mixer prefill");
}

const char* lrc_status_string(lrc_status s) {
    switch (s) {
        case LRC_OK: return "ok";
        case LRC_ERR_NULL: return "null pointer";
        case LRC_ERR_ROWS: return "row count out of range";
        case LRC_ERR_SHAPE: return "unsupported shape";
        case LRC_ERR_DTYPE: return "unsupported dtype";
        case LRC_ERR_ALIGN: return "misaligned pointer";
        case LRC_ERR_LAUNCH: return "kernel launch failed";
        case LRC_ERR_ALIAS: return "output overlaps an input";
    }
    return "unknown status";
}

const char* lrc_last_error(void) { return g_err; }

int lrc_version(void) { return (0 << 16) | (1 << 8) | 0; }

}  // extern "C"

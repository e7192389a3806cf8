// K3, bf16-input path: Gated DeltaNet chunked delta rule on CDNA4 matrix cores.
//
// Source: "perf(qwen3_5): prefill text prompts in multi-token chunks",
// Implementation.  For a chunk of S <= 64 rows of value head h (key head
// h / (Hv/Hk)), with gamma the chunk-local inclusive cumulative sum of g and
// Gamma = e^gamma:
//   A_ij = beta_i e^{gamma_i - gamma_j} k_i.k_j  (j < i)
//   U    = (I + A)^-1 (diag(beta) V - diag(beta Gamma) K S_0)
//   O    = diag(Gamma) Q S_0 + (e^{gamma_t - gamma_i} q_t.k_i)_{i <= t} U
//   S_S  = e^{gamma_S} S_0 + (K * e^{min(gamma_S - gamma, 0)})^T U
// gamma_S is the last entry of the same cumulative sum.
//
// Work split.  One workgroup owns a whole value head of one prompt, or of a
// lane of prompts run back to back (see the launcher), and walks their
// chunks.  It holds two kinds of waves, which run the same sequence of
// workgroup barriers, five per step in the split form (segments A .. E) and
// four in the default form, where C and D are one segment:
//  * dv/32 state waves, each owning 32 columns of the [dk x dv] state in MFMA
//    accumulators, swapped at each prompt boundary.  In step n they run the
//    chain that depends on the state for chunk n: K S_0, Q S_0 and the
//    right-hand side, then the loads of V of chunk n+1 (A), U (B), O (C), the
//    state update (D), and they build K^T of chunk n+1 and the diagonal tiles
//    of chunk n+2's A (E).  In the default form they also form the masked
//    decayed Q K^T (P) of chunk n+1 after U (B), into the P buffer that chunk
//    n does not use.  A lane's two 16-column groups are the even and the
//    odd columns of the wave's 32, so that V, O and the state move as column
//    pairs.  V, O and the state go through buffer resources; those of V and O
//    end after the chunk's rows, so rows past it need no test.
//  * 4 prep waves, which in step n prepare chunk n+1, the part that does not
//    depend on the state: the inverse (diagonal tiles in A, level 16 in B,
//    level 32 in C and D, each tile of T rounded to bf16 once final) and, in
//    the split form, P (D).  In the default form each prep wave forms the
//    tiles of level 32's Y that its tile of T needs itself, in registers, so
//    level 32 needs no barrier inside.  They stage chunk n+2 into LDS and keep the rows
//    of chunk n+3 in flight: in the default form prep waves 2 and 3, idle
//    during level 16, in B and waves 0 and 1, whose level-32 tiles are the
//    lighter ones, in D; in the split form all four in C.  They form the six
//    tiles of chunk n+2's masked K K^T below the diagonal (E).
// LDS holds K and Q of two chunks (by chunk parity), the per-row gamma,
// Gamma, beta and state-update decay of three, where the rows of four are
// and which prompt they belong to, one copy of A -> T (FP32), T (bf16) and
// K^T, and P (bf16) by chunk parity (one copy, with its lo parts, in the
// split form): each is written in a segment where no wave reads the copy it
// replaces.  About 148 KiB (156 KiB in the split form, which keeps Y in
// LDS), one workgroup per CU.
//
// Matrix cores: v_mfma_f32_16x16x32_bf16, FP32 accumulation.  The A operand
// of lane l is row l%16 with 8 k-values, the B operand column l%16 with the
// same 8 k-values, and the accumulator holds column l%16, rows 4(l/16) .. +3.
// A wave's own [rows x 16] accumulators serve directly as B operands when
// the k-values of lane group g are taken as rows {4g .. 4g+3} of one 16-row
// tile and {16+4g .. 16+4g+3} of the next; the A operands (K, Q, K^T, T, P)
// are stored in LDS with their contraction index permuted to match (kperm),
// so each A fragment is one 16-byte read.  K K^T and Q K^T take both operands
// from the same permuted rows, which leaves their sums unchanged.  The masked products are computed
// transposed (keys as rows), so each lane holds 4 consecutive keys of one
// query and writes them as one packed store.
// Accumulation is FP32 throughout.  An FP32 operand (S_0, the right-hand
// side, T, P, decayed U) is rounded to bf16 once on its way into the matrix
// cores.  With SPLIT it enters as a pair hi = bf16(x), lo = bf16(x - hi),
// about 16 mantissa bits, at the cost of more passes:
//                                                    passes    with SPLIT
//   K K^T, Q K^T        bf16 x bf16 (exact)            1          1
//   K S_0, Q S_0        bf16 x S_0                     1          2
//   K^T (d U)           bf16 x decayed U               1          2
//   T RHS, P U          FP32 x FP32                    1          3 (lo x lo dropped)
// Decay factors: on the diagonal 16x16 tiles e^{gamma_i - gamma_j} is formed
// per element; below them it is the product e^{gamma_i - gamma_c}
// e^{gamma_c - gamma_j} through the tile's first row c, both factors <= 1.
// The 64-row inverse (8x8 Neumann blocks, then 2x2 block levels) keeps T in
// FP32: the diagonal 16x16 tiles as 8x8 products on the vector ALUs, the
// level products as hi/lo bf16 pairs on the bf16 matrix cores or, with SPLIT,
// on the FP32 matrix cores.
#include <algorithm>
#include <cstddef>
#include <cstring>
#include <type_traits>

#include "lrc_device.h"
#include "lrc_internal.h"
#include "gdn_frag.h"
#include "tri_inverse.h"

namespace lrc {
namespace {

constexpr int kPrep = 4;     // waves that prepare the next chunk

// Row strides (bf16) of the operands read as fragments: a 16-byte read by 16
// rows is free of LDS bank conflicts when rows start 32 bytes apart modulo 128
// (row strides of 144 or 80 bf16; 136 and 72 cost about a quarter more per
// read).  The split form, whose lo copies need the room, keeps the narrower ones.
template <int DK, bool SPLIT>
struct PipeSmem {
    static constexpr int LDK = SPLIT ? DK + 8 : DK + 16;  // K, Q rows
    static constexpr int LT = SPLIT ? 72 : 80;            // T, P, K^T rows (64 columns)
    static constexpr int LO = SPLIT ? 64 * LT : 8;  // the lo copies are used with SPLIT only
    static constexpr int NPB = SPLIT ? 1 : 2;      // P buffers: by chunk parity in the default form
    __bf16 K[2][64 * LDK];  // chunk rows, by parity of the chunk index
    __bf16 Q[2][64 * LDK];
    __bf16 KT[DK * LT];     // K^T of the chunk whose state update comes next
    __bf16 T_hi[64 * LT];   // (I + A)^-1 in bf16 (with SPLIT: hi and lo parts)
    __bf16 T_lo[LO];
    __bf16 P_hi[NPB][64 * LT];  // masked decayed Q K^T
    __bf16 P_lo[LO];
    float M[64 * kTriLd];   // A, then T, in FP32
    float scratch[SPLIT ? kTriScratch : 4];  // Y of level 32 (the default form keeps it in registers)
    alignas(16) float dscratch[kPrep * tri::kDiagScratch];  // the diagonal tiles' 8x8 products
    float gam[3][64];       // per-row values, by chunk index mod 3
    float Gam[3][64];       // e^gamma
    float beta[3][64];
    float decS[3][64];      // e^{min(gamma_S - gamma_r, 0)}, 0 past the chunk
    alignas(16) int meta[4][4];  // by chunk index mod 4: its first row, its rows, its prompt
};
template <bool SPLIT>
constexpr bool meta_aligned() {
    using Big = PipeSmem<128, SPLIT>;
    using Small = PipeSmem<32, SPLIT>;
    return offsetof(Big, meta) % 16 == 0 && offsetof(Small, meta) % 16 == 0;
}
static_assert(meta_aligned<true>() && meta_aligned<false>(),
              "a chunk's record is written as one 16-byte store");

// Which prompts a workgroup row runs.  With n == 0, row y runs the prompt in
// slot y of the batch order alone; otherwise row y is a lane that runs slots
// off[y] .. off[y+1]-1 one after the other.
struct GdnLanes {
    int n;
    unsigned short off[LRC_MAX_PROMPTS + 1];
};

// A lane's chunks are those of its prompts in slot order (slots up to i1),
// prompts without rows skipped.  The cursor names one of them: slot i, prompt
// p, the chunk's first row, and the end of the prompt's rows.  All of it is
// uniform across the workgroup.  Past the lane's last chunk it names an empty
// chunk.
struct ChunkCursor {
    int i, p, row, end;
    __device__ void enter(const Batch& bt, int i1) {  // the first prompt with rows from slot i on
        for (; i < i1; ++i) {
            p = batch_prompt(bt, i);
            const int L = batch_len(bt, p);
            if (L > 0) {
                row = batch_row0(bt, p);
                end = row + L;
                return;
            }
        }
        row = end = 0;
    }
    __device__ void next(const Batch& bt, int i1) {
        row += 64;
        if (row >= end) {
            ++i;
            enter(bt, i1);
        }
    }
    __device__ int rows() const { return min(64, end - row); }
};

// One 16x16 tile of the FP32 matrix into its bf16 copy (with SPLIT: hi and lo copies).
template <bool SPLIT, int LT>
__device__ __forceinline__ void split_tile(const float* M, __bf16* hi, __bf16* lo, int ti, int tj, int lane) {
    const int r = 16 * ti + (lane >> 2), c = 16 * tj + 4 * (lane & 3);
    const floatx4 x = *reinterpret_cast<const floatx4*>(&M[r * kTriLd + c]);
    bf16x4 h, l;
    split4(x, h, l);
    *reinterpret_cast<bf16x4*>(&hi[r * LT + kperm(c)]) = h;
    if constexpr (SPLIT) *reinterpret_cast<bf16x4*>(&lo[r * LT + kperm(c)]) = l;
}

// Level 32 of the inverse, tile (TA, TB) of T21 = -T22 Y, Y = L21 T11, for
// one wave with no barrier: the wave forms the tiles of Y it needs itself and
// keeps them in registers (accumulator layout), then forms its tile of T21 as
// the transposed product Y^T T22^T, whose accumulator layout is T21's row
// layout, and writes it to T in bf16.  M is only read, so the four tiles need
// no ordering between waves; the FP32 T21 is never stored.
template <int TA, int TB, int LT>
__device__ __forceinline__ void lvl32_tile(const float* M, __bf16* T_hi) {
    using MM = tri::MmBf16Split;
    constexpr int ld = kTriLd;
    int lr, g;
    tri::lanes(lr, g);
    const tri_f4 zero = {0.f, 0.f, 0.f, 0.f};
    tri_f4 y[TA + 1];
#pragma unroll
    for (int c = 0; c <= TA; ++c) {  // Y(c, TB); T11 is block lower triangular
        y[c] = zero;
#pragma unroll
        for (int l = TB; l < 2; ++l)
            y[c] = MM::mm(y[c], tri::ld_row(M + (32 + 16 * c) * ld + 16 * l, ld, lr, g),
                          tri::ld_acc(M + 16 * l * ld + 16 * TB, ld, lr, g));
    }
    tri_f4 acc = zero;
#pragma unroll
    for (int c = 0; c <= TA; ++c)  // T22 is block lower triangular
        acc = MM::mm(acc, y[c], tri::ld_row(M + (32 + 16 * TA) * ld + 32 + 16 * c, ld, lr, g));
    bf16x4 h;
#pragma unroll
    for (int r = 0; r < 4; ++r) h[r] = static_cast<__bf16>(-acc[r]);
    *reinterpret_cast<bf16x4*>(&T_hi[(32 + 16 * TA + lr) * LT + kperm(16 * TB + 4 * g)]) = h;
}
template <int LT>
__device__ __forceinline__ void lvl32_direct(const float* M, __bf16* T_hi, int pw) {
    if (pw == 0) lvl32_tile<0, 0, LT>(M, T_hi);
    else if (pw == 1) lvl32_tile<0, 1, LT>(M, T_hi);
    else if (pw == 2) lvl32_tile<1, 0, LT>(M, T_hi);
    else lvl32_tile<1, 1, LT>(M, T_hi);
}

// K^T of the chunk in K buffer b into KT, by blocks of 4 rows x 8 stored
// columns, blocks t, t + stride, ...
template <int DK, class Sm>
__device__ __forceinline__ void build_kt(Sm& sm, int b, int t, int stride) {
    constexpr int LDK = Sm::LDK, LT = Sm::LT;
    for (int x = t; x < 2 * DK; x += stride) {
        // rows 4nn .. 4nn+3, stored columns 8m .. 8m+7 (dk indices kperm_inv of them)
        const int nn = x & 15, m = x >> 4;
        uint4 rw[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) rw[a] = *reinterpret_cast<const uint4*>(&sm.K[b][(4 * nn + a) * LDK + 8 * m]);
        const uint32_t d0[4] = {rw[0].x, rw[0].y, rw[0].z, rw[0].w};
        const uint32_t d1[4] = {rw[1].x, rw[1].y, rw[1].z, rw[1].w};
        const uint32_t d2[4] = {rw[2].x, rw[2].y, rw[2].z, rw[2].w};
        const uint32_t d3[4] = {rw[3].x, rw[3].y, rw[3].z, rw[3].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;  // high or low halves of two dwords
            uint2 out;
            out.x = __builtin_amdgcn_perm(d1[e >> 1], d0[e >> 1], sel);
            out.y = __builtin_amdgcn_perm(d3[e >> 1], d2[e >> 1], sel);
            *reinterpret_cast<uint2*>(&sm.KT[kperm_inv(8 * m + e) * LT + kperm(4 * nn)]) = out;
        }
    }
}

// Masked decayed K K^T of the chunk in buffers (b, rbuf) -> A in M: tile
// pairs first, first + stride, ... (NP of them; pairs past the last one are
// computed but not stored).
template <int DK, int NP, class Sm>
__device__ __forceinline__ void masked_kk(Sm& sm, int b, int rbuf, int first, int stride) {
    constexpr int LDK = Sm::LDK;
    constexpr int KS = DK / 32;
    int tid_c = threadIdx.x;
    asm volatile("" : "+v"(tid_c));
    const int lr = tid_c & 15, lg = (tid_c >> 4) & 3, lk = lg * 8, lq = lg * 4;
    floatx4 kk[NP];
#pragma unroll
    for (int x = 0; x < NP; ++x) kk[x] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int x = 0; x < NP; ++x) {
            int ti, tj;
            tile_pair(min(first + x * stride, 9), ti, tj);
            kk[x] = mfma(frag(&sm.K[b][(16 * tj + lr) * LDK + 32 * s + lk]),
                         frag(&sm.K[b][(16 * ti + lr) * LDK + 32 * s + lk]), kk[x]);
        }
    read_ahead<KS * NP, 2, 1, (NP < 3 ? NP : 3)>();
#pragma unroll
    for (int x = 0; x < NP; ++x)
        if (first + x * stride < 10) {
            int ti, tj;
            tile_pair(first + x * stride, ti, tj);
            const floatx4 dec = tile_decay(sm.gam[rbuf], ti, tj, lr, lq);
            const int i = 16 * ti + lr;
            const float bi = sm.beta[rbuf][i];
            floatx4 av;
#pragma unroll
            for (int r = 0; r < 4; ++r) av[r] = i > 16 * tj + lq + r ? bi * dec[r] * kk[x][r] : 0.f;
            *reinterpret_cast<floatx4*>(&sm.M[i * kTriLd + 16 * tj + lq]) = av;
        }
}

// Masked decayed K K^T tiles (TI0, TJ0) and, if TI1 >= 0, (TI1, TJ1) of the
// chunk in buffers (b, rbuf) -> A in M, with the tile indices known at compile
// time: a key fragment used by both tiles is read once per k-step, and a
// diagonal tile reads one fragment for both operands.
template <int DK, int TI0, int TJ0, int TI1, int TJ1, class Sm>
__device__ __forceinline__ void kk_tiles(Sm& sm, int b, int rbuf) {
    constexpr int LDK = Sm::LDK, KS = DK / 32, NP = TI1 >= 0 ? 2 : 1;
    constexpr int TI[2] = {TI0, TI1 >= 0 ? TI1 : TI0}, TJ[2] = {TJ0, TI1 >= 0 ? TJ1 : TJ0};
    int tid_c = threadIdx.x;
    asm volatile("" : "+v"(tid_c));
    const int lr = tid_c & 15, lg = (tid_c >> 4) & 3, lk = lg * 8, lq = lg * 4;
    floatx4 kk[NP];
#pragma unroll
    for (int x = 0; x < NP; ++x) kk[x] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int x = 0; x < NP; ++x)
            kk[x] = mfma(frag(&sm.K[b][(16 * TJ[x] + lr) * LDK + 32 * s + lk]),
                         frag(&sm.K[b][(16 * TI[x] + lr) * LDK + 32 * s + lk]), kk[x]);
#pragma unroll
    for (int x = 0; x < NP; ++x) {
        const floatx4 dec = tile_decay(sm.gam[rbuf], TI[x], TJ[x], lr, lq);
        const int i = 16 * TI[x] + lr;
        const float bi = sm.beta[rbuf][i];
        floatx4 av;
#pragma unroll
        for (int r = 0; r < 4; ++r) av[r] = i > 16 * TJ[x] + lq + r ? bi * dec[r] * kk[x][r] : 0.f;
        *reinterpret_cast<floatx4*>(&sm.M[i * kTriLd + 16 * TJ[x] + lq]) = av;
    }
}

// The ten tiles of A for the next chunk but one, in segment E: the six below
// the diagonal on the four prep waves (two, two, one, one; the pairs share a
// key fragment), the four diagonal ones on the state waves.
template <int DK, class Sm>
__device__ __forceinline__ void kk_prep(Sm& sm, int b, int rbuf, int pw) {
    if (pw == 0) kk_tiles<DK, 1, 0, 2, 0>(sm, b, rbuf);
    else if (pw == 1) kk_tiles<DK, 3, 0, 3, 1>(sm, b, rbuf);
    else if (pw == 2) kk_tiles<DK, 2, 1, -1, -1>(sm, b, rbuf);
    else kk_tiles<DK, 3, 2, -1, -1>(sm, b, rbuf);
}
template <int DK, int NS, class Sm>
__device__ __forceinline__ void kk_state(Sm& sm, int b, int rbuf, int w) {
    if constexpr (NS == 4) {
        if (w == 0) kk_tiles<DK, 0, 0, -1, -1>(sm, b, rbuf);
        else if (w == 1) kk_tiles<DK, 1, 1, -1, -1>(sm, b, rbuf);
        else if (w == 2) kk_tiles<DK, 2, 2, -1, -1>(sm, b, rbuf);
        else kk_tiles<DK, 3, 3, -1, -1>(sm, b, rbuf);
    } else if constexpr (NS == 2) {
        if (w == 0) kk_tiles<DK, 0, 0, 1, 1>(sm, b, rbuf);
        else kk_tiles<DK, 2, 2, 3, 3>(sm, b, rbuf);
    } else {
        static_assert(NS == 1, "one, two or four state waves");
        kk_tiles<DK, 0, 0, 1, 1>(sm, b, rbuf);
        kk_tiles<DK, 2, 2, 3, 3>(sm, b, rbuf);
    }
}

// Masked decayed Q K^T of the chunk in buffers (b, rbuf), key tile TJ with
// query tiles TI0 .. TI1, into P (bf16, queries as rows).  Computed transposed
// (keys as rows), so that one key fragment per k-step serves every query
// tile of the group.
template <int DK, int TJ, int TI0, int TI1, class Sm>
__device__ __forceinline__ void qk_group(Sm& sm, int b, int rbuf, __bf16* P) {
    constexpr int LDK = Sm::LDK, LT = Sm::LT, KS = DK / 32, NT = TI1 - TI0 + 1;
    int tid_c = threadIdx.x;
    asm volatile("" : "+v"(tid_c));
    const int lr = tid_c & 15, lg = (tid_c >> 4) & 3, lk = lg * 8, lq = lg * 4;
    floatx4 acc[NT];
#pragma unroll
    for (int x = 0; x < NT; ++x) acc[x] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const bf16x8 a = frag(&sm.K[b][(16 * TJ + lr) * LDK + 32 * s + lk]);
#pragma unroll
        for (int x = 0; x < NT; ++x) acc[x] = mfma(a, frag(&sm.Q[b][(16 * (TI0 + x) + lr) * LDK + 32 * s + lk]), acc[x]);
    }
    read_ahead<KS, NT + 1, NT, (KS < 3 ? KS : 3)>();
#pragma unroll
    for (int x = 0; x < NT; ++x) {
        const floatx4 pv4 = tile_decay(sm.gam[rbuf], TI0 + x, TJ, lr, lq) * acc[x];
        bf16x4 ph, pl;
        split4(pv4, ph, pl);
        *reinterpret_cast<bf16x4*>(&P[(16 * (TI0 + x) + lr) * LT + kperm(16 * TJ + lq)]) = ph;
    }
}

// All ten tiles of P, dealt to NS state waves by key tile: 3, 3, 2, 2 tiles
// for four waves (the last one takes the first and the last diagonal tile),
// 5 and 5 for two.
template <int DK, int NS, class Sm>
__device__ __forceinline__ void state_qk(Sm& sm, int b, int rbuf, __bf16* P, int w) {
    if constexpr (NS == 4) {
        if (w == 0) qk_group<DK, 0, 1, 3>(sm, b, rbuf, P);
        else if (w == 1) qk_group<DK, 1, 1, 3>(sm, b, rbuf, P);
        else if (w == 2) qk_group<DK, 2, 2, 3>(sm, b, rbuf, P);
        else {
            qk_group<DK, 0, 0, 0>(sm, b, rbuf, P);
            qk_group<DK, 3, 3, 3>(sm, b, rbuf, P);
        }
    } else if constexpr (NS == 2) {
        if (w == 0) {
            qk_group<DK, 0, 0, 3>(sm, b, rbuf, P);
            qk_group<DK, 3, 3, 3>(sm, b, rbuf, P);
        } else {
            qk_group<DK, 1, 1, 3>(sm, b, rbuf, P);
            qk_group<DK, 2, 2, 3>(sm, b, rbuf, P);
        }
    } else {
        static_assert(NS == 1, "one, two or four state waves");
        qk_group<DK, 0, 0, 3>(sm, b, rbuf, P);
        qk_group<DK, 1, 1, 3>(sm, b, rbuf, P);
        qk_group<DK, 2, 2, 3>(sm, b, rbuf, P);
        qk_group<DK, 3, 3, 3>(sm, b, rbuf, P);
    }
}

// Grid (value heads, prompts); NS = dv / 32 state waves, then kPrep prep waves.
template <int DK, int NS, bool SPLIT>
__global__ __launch_bounds__(64 * (NS + kPrep), 1) void gdn_pipe_kernel(const uint16_t* __restrict__ q,
                                                                        const uint16_t* __restrict__ k,
                                                                        const uint16_t* __restrict__ v,
                                                                        const float* __restrict__ beta,
                                                                        const float* __restrict__ g,
                                                                        float* __restrict__ o, const float* S_in,
                                                                        float* S_out, Batch bt, GdnLanes lanes,
                                                                        int Hk, int Hv, int dv) {
    static_assert(CG == 2, "a lane's column pair is one even and one odd column");
    using Sm = PipeSmem<DK, SPLIT>;
    constexpr int LDK = Sm::LDK;
    constexpr int LT = Sm::LT;
    constexpr int KS = DK / 32;             // k-steps over dk
    constexpr int RT = DK / 16;             // state row tiles
    constexpr int PS = SPLIT ? 2 : 1;       // passes of a product with one FP32 operand
    constexpr int PK = 64 * DK / 8;         // 16-byte pieces of a K (or Q) chunk
    extern __shared__ __align__(16) unsigned char smem_raw[];
    Sm& sm = *reinterpret_cast<Sm*>(smem_raw);

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool is_state = w < NS;
    const int pw = w - NS;  // prep wave index
    // The value heads of one key head read the same K and Q rows.  Workgroups
    // are dealt to the 8 XCDs in launch order, so heads that are 8 workgroups
    // apart share an XCD and its L2: the G = Hv/Hk siblings of a key head are
    // placed 8 apart, and the second read of each K, Q row is an L2 hit.
    const int G = Hv / Hk;
    int h = blockIdx.x;
    if (G > 1 && Hv % (8 * G) == 0) {
        const int r = h % (8 * G);
        h = h - r + (r % 8) * G + r / 8;
    }
    const int kh = h / G;
    const int i0 = lanes.n ? lanes.off[blockIdx.y] : blockIdx.y;
    const int i1 = lanes.n ? lanes.off[blockIdx.y + 1] : blockIdx.y + 1;
    int nc = 0;  // chunks of the lane
    for (int i = i0; i < i1; ++i) nc += (batch_len(bt, batch_prompt(bt, i)) + 63) >> 6;
    const uint32_t rowK = Hk * DK, rowV = Hv * dv;
    if (is_state) {
        // ================= state waves: chunk n, 32 state columns each
        // Lane l of a state wave holds columns col0 + 2 (l%16) + c, c = 0, 1: the
        // two column groups are the even and the odd columns, so that V, O and
        // the state move as pairs of adjacent columns.
        const int col0 = 32 * w;
        int s_lane = (lane >> 4) * 4 * dv + 2 * (lane & 15);
        asm volatile("" : "+v"(s_lane));
        floatx4 sacc[CG][RT];
        // The state block of prompt p through a buffer resource; the row
        // offsets are formed where they are used, not kept across the loop.
        auto state_rsrc = [&](const float* base, int p) {
            return buffer_rsrc(base + ((long)p * Hv + h) * DK * dv + col0, (uint32_t)(DK * dv * 4));
        };
        auto load_state = [&](int p) {
            const auto rs = state_rsrc(S_in, p);
            int sl = s_lane * 4, dv4 = dv * 4;
            asm volatile("" : "+v"(sl), "+s"(dv4));
#pragma unroll
            for (int tr = 0; tr < RT; ++tr)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(rs, sl, (16 * tr + r) * dv4, 0);
                    sacc[0][tr][r] = __uint_as_float(x[0]);
                    sacc[1][tr][r] = __uint_as_float(x[1]);
                }
        };
        auto store_state = [&](int p) {
            const auto rs = state_rsrc(S_out, p);
            int sl = s_lane * 4, dv4 = dv * 4;
            asm volatile("" : "+v"(sl), "+s"(dv4));
#pragma unroll
            for (int tr = 0; tr < RT; ++tr)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    __builtin_amdgcn_raw_buffer_store_b64(
                        u32x2{__float_as_uint(sacc[0][tr][r]), __float_as_uint(sacc[1][tr][r])}, rs, sl,
                        (16 * tr + r) * dv4, 0);
        };
        // Where a chunk's rows are and which prompt it belongs to, as the prep
        // waves recorded it when they fetched the chunk.
        auto meta = [&](int j, int f) { return __builtin_amdgcn_readfirstlane(sm.meta[j & 3][f]); };
        ChunkCursor first{i0};
        first.enter(bt, i1);
#pragma unroll
        for (int c = 0; c < CG; ++c)
#pragma unroll
            for (int tr = 0; tr < RT; ++tr) sacc[c][tr] = floatx4{0.f, 0.f, 0.f, 0.f};
        if (nc > 0) load_state(first.p);
        // V of the next chunk in accumulator layout: rows 16t + 4(l/16) + r, both columns of the lane
        uint32_t pv[16];
#pragma unroll
        for (int x = 0; x < 16; ++x) pv[x] = 0;
        __syncthreads();  // prologue: chunk 0 staged
        __syncthreads();  // prologue: A of chunk 0 in M

        for (int n = -1; n < nc; ++n) {
            const int cb = n & 1, nb = cb ^ 1;  // K/Q buffers of chunks n, n+1
            const int rb = (n + 3) % 3;         // row buffer of chunk n
            const bool do_state = n >= 0, do_next = n + 1 < nc;
            int Sn = 0;
            int tid_c = tid;
            asm volatile("" : "+v"(tid_c));
            const int lr = tid_c & 15, lg = (tid_c >> 4) & 3, lq = lg * 4;
            floatx4 ks0[CG][4], qs0[CG][4], u[CG][4];

            // ---- A: K S_0, Q S_0 and RHS = diag(beta) V - diag(beta Gamma) K S_0; V of chunk n+1
            if (do_state) {
#pragma unroll
                for (int c = 0; c < CG; ++c)
#pragma unroll
                    for (int t = 0; t < 4; ++t) ks0[c][t] = qs0[c][t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    bf16x8 bh[CG], bl[CG];
#pragma unroll
                    for (int c = 0; c < CG; ++c) acc_frag<SPLIT>(sacc[c][2 * s], sacc[c][2 * s + 1], bh[c], bl[c]);
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const bf16x8 ak = frag(&sm.K[cb][(16 * t + lr) * LDK + 32 * s + 8 * lg]);
                        const bf16x8 aq = frag(&sm.Q[cb][(16 * t + lr) * LDK + 32 * s + 8 * lg]);
#pragma unroll
                        for (int c = 0; c < CG; ++c) {
                            ks0[c][t] = mfma(ak, bh[c], ks0[c][t]);
                            if constexpr (SPLIT) ks0[c][t] = mfma(ak, bl[c], ks0[c][t]);
                            qs0[c][t] = mfma(aq, bh[c], qs0[c][t]);
                            if constexpr (SPLIT) qs0[c][t] = mfma(aq, bl[c], qs0[c][t]);
                        }
                    }
                }
                read_ahead<4 * KS, 2, 2 * PS * CG, SPLIT ? 2 : 3>();
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const floatx4 b4 = *reinterpret_cast<const floatx4*>(&sm.beta[rb][16 * t + lq]);
                    const floatx4 G4 = *reinterpret_cast<const floatx4*>(&sm.Gam[rb][16 * t + lq]);
#pragma unroll
                    for (int c = 0; c < CG; ++c)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            // rows past the chunk read V as zero; beta is 0 there as well
                            const float vv = c ? __uint_as_float(pv[4 * t + r] & 0xffff0000u)
                                               : __uint_as_float(pv[4 * t + r] << 16);
                            ks0[c][t][r] = b4[r] * (vv - G4[r] * ks0[c][t][r]);
                        }
                    // diag(Gamma) Q S_0 is where the accumulation of O starts (segment C)
                    if constexpr (!SPLIT)
#pragma unroll
                        for (int c = 0; c < CG; ++c) qs0[c][t] *= G4;
                }
            }
            if (do_next) {
                // V of chunk n+1, as soon as this chunk's RHS has used V of chunk n:
                // four segments ahead of its use.  Through a buffer resource that ends
                // after the chunk's S rows: rows past it read as zero (beta is zero
                // there too).  V is read once and O written once: both streaming.
                const int S = meta(n + 1, 1);
                const auto vrsrc = buffer_rsrc(v + meta(n + 1, 0) * (long)rowV + (long)h * dv + col0,
                                              (uint32_t)S * rowV * 2);
                uint32_t v_lane = (__umul24(lq, rowV) + 2 * lr) * 2;
                asm volatile("" : "+v"(v_lane));
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        pv[4 * t + r] = __builtin_amdgcn_raw_buffer_load_b32(vrsrc, v_lane + (16 * t + r) * rowV * 2, 0, kNontemporal);
            }
            __syncthreads();

            // ---- B: U = T RHS (T lower triangular: k-steps up to the row tile's diagonal)
            if (do_state) {
#pragma unroll
                for (int c = 0; c < CG; ++c)
#pragma unroll
                    for (int t = 0; t < 4; ++t) u[c][t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    bf16x8 bh[CG], bl[CG];
#pragma unroll
                    for (int c = 0; c < CG; ++c) acc_frag<SPLIT>(ks0[c][2 * s], ks0[c][2 * s + 1], bh[c], bl[c]);
#pragma unroll
                    for (int t = 2 * s; t < 4; ++t) {
                        const bf16x8 ah = frag(&sm.T_hi[(16 * t + lr) * LT + 32 * s + 8 * lg]);
                        bf16x8 al;
                        if constexpr (SPLIT) al = frag(&sm.T_lo[(16 * t + lr) * LT + 32 * s + 8 * lg]);
#pragma unroll
                        for (int c = 0; c < CG; ++c) {
                            u[c][t] = mfma(ah, bh[c], u[c][t]);
                            if constexpr (SPLIT) {
                                u[c][t] = mfma(ah, bl[c], u[c][t]);
                                u[c][t] = mfma(al, bh[c], u[c][t]);
                            }
                        }
                    }
                }
                read_ahead<6, SPLIT ? 2 : 1, (SPLIT ? 3 : 1) * CG, 2>();
            }
            // P of chunk n+1 into the other P buffer (the split form's prep waves
            // form it in D)
            if constexpr (!SPLIT)
                if (do_next) state_qk<DK, NS>(sm, nb, (n + 4) % 3, sm.P_hi[nb], w);
            __syncthreads();

            // ---- C: O = diag(Gamma) Q S_0 + P U
            if (do_state) {
                // the default form accumulates P U onto diag(Gamma) Q S_0 (scaled in A)
                floatx4 pu_split[SPLIT ? CG : 1][4];
                auto& pu = [&]() -> auto& {
                    if constexpr (SPLIT) return pu_split;
                    else return qs0;
                }();
                if constexpr (SPLIT)
#pragma unroll
                    for (int c = 0; c < CG; ++c)
#pragma unroll
                        for (int t = 0; t < 4; ++t) pu[c][t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    bf16x8 bh[CG], bl[CG];
#pragma unroll
                    for (int c = 0; c < CG; ++c) acc_frag<SPLIT>(u[c][2 * s], u[c][2 * s + 1], bh[c], bl[c]);
#pragma unroll
                    for (int t = 2 * s; t < 4; ++t) {
                        const bf16x8 ah = frag(&sm.P_hi[SPLIT ? 0 : cb][(16 * t + lr) * LT + 32 * s + 8 * lg]);
                        bf16x8 al;
                        if constexpr (SPLIT) al = frag(&sm.P_lo[(16 * t + lr) * LT + 32 * s + 8 * lg]);
#pragma unroll
                        for (int c = 0; c < CG; ++c) {
                            pu[c][t] = mfma(ah, bh[c], pu[c][t]);
                            if constexpr (SPLIT) {
                                pu[c][t] = mfma(ah, bl[c], pu[c][t]);
                                pu[c][t] = mfma(al, bh[c], pu[c][t]);
                            }
                        }
                    }
                }
                read_ahead<6, SPLIT ? 2 : 1, (SPLIT ? 3 : 1) * CG, SPLIT ? 2 : 3>();
                // Through a buffer resource that ends after the chunk's Sn rows: the
                // stores of rows past it are dropped, with no per-row test.
                Sn = meta(n, 1);
                const auto orsrc = buffer_rsrc(o + meta(n, 0) * (long)rowV + (long)h * dv + col0,
                                              (uint32_t)Sn * rowV * 4);
                uint32_t o_lane = (__umul24(lq, rowV) + 2 * lr) * 4;
                asm volatile("" : "+v"(o_lane));
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    floatx4 o4[CG];
                    if constexpr (SPLIT) {
                        const floatx4 G4 = *reinterpret_cast<const floatx4*>(&sm.Gam[rb][16 * t + lq]);
#pragma unroll
                        for (int c = 0; c < CG; ++c)
#pragma unroll
                            for (int r = 0; r < 4; ++r) o4[c][r] = fmaf(G4[r], qs0[c][t][r], pu[c][t][r]);
                    } else {
#pragma unroll
                        for (int c = 0; c < CG; ++c) o4[c] = pu[c][t];
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const u32x2 pair = {__float_as_uint(o4[0][r]), __float_as_uint(o4[1][r])};
                        __builtin_amdgcn_raw_buffer_store_b64(pair, orsrc, o_lane + (16 * t + r) * rowV * 4, 0, kNontemporal);
                    }
                }
            }
            // the default form runs C and D as one segment (the prep waves' level 32 needs no barrier there)
            if constexpr (SPLIT) __syncthreads();

            // ---- D: S_S = e^{gamma_S} S_0 + K^T (decS U)
            if (do_state) {
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const floatx4 d4 = *reinterpret_cast<const floatx4*>(&sm.decS[rb][16 * t + lq]);
#pragma unroll
                    for (int c = 0; c < CG; ++c) u[c][t] *= d4;
                }
                {
                    const float GS = sm.Gam[rb][Sn - 1];
#pragma unroll
                    for (int c = 0; c < CG; ++c)
#pragma unroll
                        for (int tr = 0; tr < RT; ++tr) sacc[c][tr] = sacc[c][tr] * GS;
                }
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    bf16x8 bh[CG], bl[CG];
#pragma unroll
                    for (int c = 0; c < CG; ++c) acc_frag<SPLIT>(u[c][2 * s], u[c][2 * s + 1], bh[c], bl[c]);
#pragma unroll
                    for (int tr = 0; tr < RT; ++tr) {
                        const bf16x8 a = frag(&sm.KT[(16 * tr + lr) * LT + 32 * s + 8 * lg]);
#pragma unroll
                        for (int c = 0; c < CG; ++c) {
                            sacc[c][tr] = mfma(a, bh[c], sacc[c][tr]);
                            if constexpr (SPLIT) sacc[c][tr] = mfma(a, bl[c], sacc[c][tr]);
                        }
                    }
                }
                read_ahead<2 * RT, SPLIT ? 2 : 1, PS * CG, SPLIT ? 2 : 4>();
            }
            __syncthreads();

            // ---- E: K^T of chunk n+1 by 4-row x 8-column blocks; the diagonal tiles of A of chunk n+2;
            //      after a prompt's last chunk, its state goes out and the next prompt's comes in
            if (do_state) {
                const int pn = meta(n, 2), pnext = do_next ? meta(n + 1, 2) : -1;
                if (pnext != pn) {
                    store_state(pn);
                    if (do_next) load_state(pnext);
                }
            }
            if (n + 2 < nc) kk_state<DK, NS>(sm, cb, (n + 5) % 3, w);
            if (do_next) build_kt<DK>(sm, nb, tid, 64 * NS);
            __syncthreads();
        }
        // Prompts without rows keep their state.
        if (S_in != S_out)
            for (int i = i0; i < i1; ++i) {
                const int p = batch_prompt(bt, i);
                if (batch_len(bt, p) == 0) {
                    load_state(p);
                    store_state(p);
                }
            }
    } else {
        // ================= prep waves: inverse of chunk n+1, staging of chunk n+2, A of chunk n+2
        constexpr int PT = 64 * kPrep;
        constexpr int NF = (2 * PK + PT - 1) / PT;
        const int pt = tid - 64 * NS;  // thread index among the prep waves
        uint4 pf[NF];                  // K and Q rows of a chunk, in flight to LDS
        float pg = 0.f, pb = 0.f;      // its g and beta (last prep wave)
        // Rows of a chunk through buffer resources that end after its S rows:
        // rows past it read as zero.  The piece offsets are a per-lane part and
        // a per-slot constant.  PT is a multiple of 2 PK / NF, so every slot is
        // all K or all Q.
        static_assert((2 * PK) % PT == 0, "every prep thread loads the same number of pieces");
        const uint32_t kq_lane = (__umul24(pt / (DK / 8), rowK) + (pt % (DK / 8)) * 8) * 2;
        ChunkCursor fc{i0};    // the next chunk to fetch
        fc.enter(bt, i1);
        int fetched_rows = 0;  // rows of the chunk in pf
        auto fetch = [&](int j) {  // chunk j of the lane
            const int S = fc.rows();
            const long r0 = fc.row;
            const auto krs = buffer_rsrc(k + (r0 * Hk + kh) * (long)DK, (uint32_t)S * rowK * 2);
            const auto qrs = buffer_rsrc(q + (r0 * Hk + kh) * (long)DK, (uint32_t)S * rowK * 2);
#pragma unroll
            for (int x = 0; x < NF; ++x) {
                const bool isq = x * PT >= PK;
                const uint32_t slot = (uint32_t)((x * PT - (isq ? PK : 0)) / (DK / 8)) * rowK * 2;
                const u32x4 d = __builtin_amdgcn_raw_buffer_load_b128(isq ? qrs : krs, kq_lane + slot, 0, 0);
                pf[x] = make_uint4(d[0], d[1], d[2], d[3]);
            }
            if (pw == kPrep - 1) {
                const auto grs = buffer_rsrc(g + r0 * Hv + h, (uint32_t)S * Hv * 4);
                const auto brs = buffer_rsrc(beta + r0 * Hv + h, (uint32_t)S * Hv * 4);
                pg = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(grs, __umul24(lane, Hv) * 4, 0, 0));
                pb = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(brs, __umul24(lane, Hv) * 4, 0, 0));
            }
            if (pw == kPrep - 1 && lane == 0)
                *reinterpret_cast<int4*>(sm.meta[j & 3]) = make_int4(fc.row, S, fc.p, 0);
            fetched_rows = S;
            fc.next(bt, i1);
        };
        // Rows past the chunk arrive as zeros; gamma stays flat there.
        auto stage = [&](int b, int rbuf) {
            const int S = fetched_rows;
#pragma unroll
            for (int x = 0; x < NF; ++x) {
                const int e = pt + x * PT;
                const bool isq = x * PT >= PK;
                const int ee = isq ? e - PK : e, r = ee / (DK / 8), c8 = (ee % (DK / 8)) * 8;
                __bf16* row = &(isq ? sm.Q[b] : sm.K[b])[r * LDK];
                *reinterpret_cast<uint2*>(&row[kperm(c8)]) = make_uint2(pf[x].x, pf[x].y);
                *reinterpret_cast<uint2*>(&row[kperm(c8 + 4)]) = make_uint2(pf[x].z, pf[x].w);
            }
            if (pw == kPrep - 1) {
                const float x = wave_prefix_sum(pg);  // gamma, inclusive over the chunk rows
                sm.gam[rbuf][lane] = x;
                sm.Gam[rbuf][lane] = fast_exp(x);
                sm.beta[rbuf][lane] = pb;
                const float gS = readlane_f(x, S - 1);  // the last cumulative sum
                sm.decS[rbuf][lane] = lane < S ? fast_exp(fminf(gS - x, 0.f)) : 0.f;
            }
        };
        // masked decayed Q K^T of the chunk in buffers (b, rbuf) -> P in bf16 (with SPLIT also its lo parts), transposed (keys as rows)
        auto masked_qk = [&](int b, int rbuf) {
            int tid_c = tid;
            asm volatile("" : "+v"(tid_c));
            const int lr = tid_c & 15, lg = (tid_c >> 4) & 3, lk = lg * 8, lq = lg * 4;
            constexpr int PPW = (10 + kPrep - 1) / kPrep;
            floatx4 qk[PPW];
#pragma unroll
            for (int x = 0; x < PPW; ++x) qk[x] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s)
#pragma unroll
                for (int x = 0; x < PPW; ++x) {
                    int ti, tj;
                    tile_pair(min(pw + x * kPrep, 9), ti, tj);  // past the last pair: computed, not stored
                    qk[x] = mfma(frag(&sm.K[b][(16 * tj + lr) * LDK + 32 * s + lk]),
                                 frag(&sm.Q[b][(16 * ti + lr) * LDK + 32 * s + lk]), qk[x]);
                }
            read_ahead<KS * PPW, 2, 1, 3>();
#pragma unroll
            for (int x = 0; x < PPW; ++x)
                if (pw + x * kPrep < 10) {
                    int ti, tj;
                    tile_pair(pw + x * kPrep, ti, tj);
                    const floatx4 pv4 = tile_decay(sm.gam[rbuf], ti, tj, lr, lq) * qk[x];
                    const int i = 16 * ti + lr;
                    bf16x4 ph, pl;
                    split4(pv4, ph, pl);
                    *reinterpret_cast<bf16x4*>(&sm.P_hi[0][i * LT + kperm(16 * tj + lq)]) = ph;
                    if constexpr (SPLIT) *reinterpret_cast<bf16x4*>(&sm.P_lo[i * LT + kperm(16 * tj + lq)]) = pl;
                }
        };

        // The inverse's tile products: FP32 matrix cores in the split form, whose
        // T enters the state products with about 16 bits; otherwise hi/lo bf16
        // pairs (about 2^-17 per product), since T is rounded to bf16 once anyway.
        using InvMM = typename std::conditional<SPLIT, tri::MmF32, tri::MmBf16Split>::type;
        // Tiles above the diagonal stay zero for the whole prompt.
        for (int e = pt; e < 64 * kTriLd; e += PT) sm.M[e] = 0.f;
        for (int e = pt; e < 64 * LT; e += PT) {
            sm.T_hi[e] = static_cast<__bf16>(0.f);
#pragma unroll
            for (int x = 0; x < Sm::NPB; ++x) sm.P_hi[x][e] = static_cast<__bf16>(0.f);
            if constexpr (SPLIT) sm.T_lo[e] = sm.P_lo[e] = static_cast<__bf16>(0.f);
        }
        if (nc > 0) {
            fetch(0);
            stage(0, 0);
        }
        if (nc > 1) fetch(1);
        __syncthreads();  // prologue: chunk 0 staged
        if (nc > 0) masked_kk<DK, 3>(sm, 0, 0, pw, kPrep);
        __syncthreads();  // prologue: A of chunk 0 in M

        for (int n = -1; n < nc; ++n) {
            const bool do_next = n + 1 < nc, do_stage = n + 2 < nc;
            const int nb = (n + 1) & 1, nrb = (n + 4) % 3;  // buffers of chunk n+1

            // ---- A: diagonal tiles of the inverse of chunk n+1
            if (do_next) tri::diag_valu<kPrep, true>(sm.M, sm.dscratch, pw);  // A is zero on and above its diagonal
            __syncthreads();

            // ---- B: level 16 (prep waves 0, 1); in the default form prep waves 2, 3
            //      stage their part of chunk n+2 into the buffers chunk n used, and
            //      put their part of chunk n+3 in flight
            if (do_next) tri::lvl16<kPrep, InvMM>(sm.M, pw);
            if constexpr (!SPLIT)
                if (do_stage && pw >= 2) {
                    stage(n & 1, (n + 5) % 3);
                    if (n + 3 < nc) fetch(n + 3);
                }
            __syncthreads();

            // ---- C: level 32 (in the split form its first half); the tiles of T that
            //      are final go to bf16; in the split form, chunk n+2 into the buffers
            //      chunk n used and chunk n+3 in flight
            if (do_next) {
                if constexpr (SPLIT) tri::lvl32a<kPrep, InvMM>(sm.M, sm.scratch, pw);
                else lvl32_direct<LT>(sm.M, sm.T_hi, pw);
                split_tile<SPLIT, LT>(sm.M, sm.T_hi, sm.T_lo, pw, pw, lane);
                if (pw == 0) split_tile<SPLIT, LT>(sm.M, sm.T_hi, sm.T_lo, 1, 0, lane);
                if (pw == 1) split_tile<SPLIT, LT>(sm.M, sm.T_hi, sm.T_lo, 3, 2, lane);
            }
            if constexpr (SPLIT) {
                if (do_stage) {
                    stage(n & 1, (n + 5) % 3);
                    if (n + 3 < nc) fetch(n + 3);
                }
                __syncthreads();

                // ---- D (split form): level 32 (second half) and its tile of T; P of chunk n+1
                if (do_next) {
                    tri::lvl32b<kPrep, InvMM>(sm.M, sm.scratch, pw);
                    tri::wave_sync();
                    split_tile<SPLIT, LT>(sm.M, sm.T_hi, sm.T_lo, 2 + (pw >> 1), pw & 1, lane);
                    masked_qk(nb, nrb);
                }
            } else {
                // the default form's D is this same segment: prep waves 0 and 1 stage their
                // half of chunk n+2 and put their part of chunk n+3 in flight
                if (do_stage && pw < 2) {
                    stage(n & 1, (n + 5) % 3);
                    if (n + 3 < nc) fetch(n + 3);
                }
            }
            __syncthreads();

            // ---- E: A of chunk n+2 into M (T of chunk n+1 is in bf16 now)
            if (do_stage) kk_prep<DK>(sm, n & 1, (n + 5) % 3, pw);
            __syncthreads();
        }
    }
}

// ---------------------------------------------------------------- lanes (host)
// A workgroup needs most of a CU's LDS, so a CU runs one at a time.  When the
// prompts' workgroups outnumber the CUs, the hardware starts each waiting
// workgroup on the first CU that frees up, and a short prompt can land behind
// a long one.  Instead the launch runs at most one row of Hv workgroups per
// group of Hv CUs, as lanes: each lane runs a set of prompts back to back, its
// chunks flowing through one pipeline.  The sets are chosen so that the
// largest lane (in chunks, plus a little per prompt for the state reload) is
// as small as the search below finds.

struct LanePlanner {
    int n = 0, k = 0, lb = 0, best_ms = 0;
    long nodes = 0, limit = 0;
    int cost[LRC_MAX_PROMPTS], item[LRC_MAX_PROMPTS], suffix[LRC_MAX_PROMPTS + 1];
    int load[LRC_MAX_PROMPTS], lane_of[LRC_MAX_PROMPTS], best[LRC_MAX_PROMPTS];

    // Longest first, each to the least loaded lane: the starting bound.
    void greedy() {
        for (int j = 0; j < k; ++j) load[j] = 0;
        for (int t = 0; t < n; ++t) {
            int j = 0;
            for (int x = 1; x < k; ++x)
                if (load[x] < load[j]) j = x;
            load[j] += cost[item[t]];
            best[item[t]] = j;
        }
        best_ms = 0;
        for (int j = 0; j < k; ++j) best_ms = std::max(best_ms, load[j]);
        for (int j = 0; j < k; ++j) load[j] = 0;
    }
    // Depth first over the items in decreasing cost, each tried in the lanes
    // of the few smallest distinct current loads that keep it below the best
    // found so far; a node budget bounds the search.
    void search(int t) {
        if (best_ms <= lb || nodes >= limit) return;
        ++nodes;
        if (t == n) {
            int ms = 0;
            for (int j = 0; j < k; ++j) ms = std::max(ms, load[j]);
            if (ms < best_ms) {
                best_ms = ms;
                for (int x = 0; x < n; ++x) best[item[x]] = lane_of[item[x]];
            }
            return;
        }
        long room = 0;
        for (int j = 0; j < k; ++j) room += std::max(0, best_ms - 1 - load[j]);
        if (room < suffix[t]) return;
        const int c = cost[item[t]];
        // the lanes of the kBranch smallest distinct loads, in increasing load
        constexpr int kBranch = 4;
        int by[kBranch], nb = 0;
        for (int j = 0; j < k; ++j) {
            bool dup = false;
            for (int x = 0; x < nb && !dup; ++x) dup = load[by[x]] == load[j];
            if (dup) continue;
            int x = nb < kBranch ? nb++ : kBranch;
            for (; x > 0 && load[by[x - 1]] > load[j]; --x)
                if (x < kBranch) by[x] = by[x - 1];
            if (x < kBranch) by[x] = j;
        }
        for (int x = 0; x < nb; ++x) {
            const int j = by[x];
            if (load[j] + c >= best_ms) break;
            load[j] += c;
            lane_of[item[t]] = j;
            search(t + 1);
            load[j] -= c;
            if (best_ms <= lb || nodes >= limit) return;
        }
    }
};

// Fills lanes.off and a copy of the batch whose order lists the lanes' slots
// back to back.  Prompts without rows go to lane 0 (they only copy state).
void plan_lanes(const Batch& bt, int k, Batch& out, GdnLanes& lanes) {
    LanePlanner pl;
    pl.k = k;
    long total = 0;
    int empty[LRC_MAX_PROMPTS], ne = 0;
    for (int s = 0; s < bt.P; ++s) {
        const int p = batch_prompt(bt, s), L = batch_len(bt, p);
        if (L == 0) {
            empty[ne++] = p;
            continue;
        }
        pl.cost[p] = 4 * ((L + 63) / 64) + 1;
        pl.item[pl.n++] = p;  // the batch order is by decreasing length already
        total += pl.cost[p];
    }
    pl.suffix[pl.n] = 0;
    for (int t = pl.n - 1; t >= 0; --t) pl.suffix[t] = pl.suffix[t + 1] + pl.cost[pl.item[t]];
    pl.lb = std::max(pl.n ? pl.cost[pl.item[0]] : 0, (int)((total + k - 1) / k));
    pl.greedy();
    pl.limit = std::min(2048, std::max(16, 8192 / k));  // a node costs a few k steps
    pl.search(0);
    out = bt;
    lanes.n = k;
    int s = 0;
    for (int j = 0; j < k; ++j) {
        lanes.off[j] = (unsigned short)s;
        for (int t = 0; t < pl.n; ++t)
            if (pl.best[pl.item[t]] == j) out.order[s++] = pl.item[t];
        if (j == 0)
            for (int x = 0; x < ne; ++x) out.order[s++] = empty[x];
    }
    lanes.off[k] = (unsigned short)s;
}

// The lanes of a packed batch (n == 0: one prompt per workgroup row).  The
// last plan is kept per host thread and reused for the same lengths.
void lanes_for(const Batch& bt, int Hv, Batch& run, GdnLanes& lanes) {
    lanes.n = 0;
    run = bt;
    if (bt.uniform >= 0 || bt.P < 2) return;
    const int k = compute_units() / Hv;
    if (k < 1 || k >= bt.P) return;
    thread_local struct {
        int P = -1, k = 0;
        int row_off[LRC_MAX_PROMPTS + 1];
        Batch run;
        GdnLanes lanes;
    } memo;
    if (memo.P == bt.P && memo.k == k &&
        std::memcmp(memo.row_off, bt.row_off, sizeof(int) * (bt.P + 1)) == 0) {
        run = memo.run;
        lanes = memo.lanes;
        return;
    }
    plan_lanes(bt, k, run, lanes);
    memo.P = bt.P;
    memo.k = k;
    std::memcpy(memo.row_off, bt.row_off, sizeof(int) * (bt.P + 1));
    memo.run = run;
    memo.lanes = lanes;
}

template <int DK, int NS, bool SPLIT>
hipError_t launch_pipe(const void* q, const void* k, const void* v, const float* beta, const float* g, float* o,
                       const float* S_in, float* S_out, const Batch& bt, int Hk, int Hv, int dv, hipStream_t st) {
    auto kern = gdn_pipe_kernel<DK, NS, SPLIT>;
    const size_t smem = sizeof(PipeSmem<DK, SPLIT>);
    // Opt in to more than 64 KiB of LDS once per process (a thread-safe static).
    static const hipError_t configured = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (configured != hipSuccess) return configured;
    Batch run;
    GdnLanes lanes;
    lanes_for(bt, Hv, run, lanes);
    const dim3 grid((unsigned)Hv, (unsigned)(lanes.n ? lanes.n : bt.P));
    hipLaunchKernelGGL(kern, grid, dim3(64 * (NS + kPrep)), smem, st, static_cast<const uint16_t*>(q),
                       static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), beta, g, o, S_in, S_out, run,
                       lanes, Hk, Hv, dv);
    return hipGetLastError();
}

template <int NS, bool SPLIT>
hipError_t launch_dk(const void* q, const void* k, const void* v, const float* beta, const float* g, float* o,
                     const float* S_in, float* S_out, const Batch& bt, int Hk, int Hv, int dk, int dv,
                     hipStream_t st) {
    switch (dk) {
        case 32: return launch_pipe<32, NS, SPLIT>(q, k, v, beta, g, o, S_in, S_out, bt, Hk, Hv, dv, st);
        case 64: return launch_pipe<64, NS, SPLIT>(q, k, v, beta, g, o, S_in, S_out, bt, Hk, Hv, dv, st);
        case 128: return launch_pipe<128, NS, SPLIT>(q, k, v, beta, g, o, S_in, S_out, bt, Hk, Hv, dv, st);
    }
    return hipErrorInvalidValue;
}

template <bool SPLIT>
hipError_t launch_dv(const void* q, const void* k, const void* v, const float* beta, const float* g, float* o,
                     const float* S_in, float* S_out, const Batch& bt, int Hk, int Hv, int dk, int dv,
                     hipStream_t st) {
    switch (dv) {
        case 32: return launch_dk<1, SPLIT>(q, k, v, beta, g, o, S_in, S_out, bt, Hk, Hv, dk, dv, st);
        case 64: return launch_dk<2, SPLIT>(q, k, v, beta, g, o, S_in, S_out, bt, Hk, Hv, dk, dv, st);
        case 128: return launch_dk<4, SPLIT>(q, k, v, beta, g, o, S_in, S_out, bt, Hk, Hv, dk, dv, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gdn_bf16_mfma(const void* q, const void* k, const void* v, const float* beta, const float* g,
                                float* o, const float* S_in, float* S_out, const Batch& bt, int Hk, int Hv, int dk,
                                int dv, bool split, hipStream_t st) {
    return split ? launch_dv<true>(q, k, v, beta, g, o, S_in, S_out, bt, Hk, Hv, dk, dv, st)
                 : launch_dv<false>(q, k, v, beta, g, o, S_in, S_out, bt, Hk, Hv, dk, dv, st);
}

}  // namespace lrc

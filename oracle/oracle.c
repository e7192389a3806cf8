/*
 * Float64 CPU oracle for chunked prefill of recurrent sequence mixers.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The product path
 * (the HIP library under linear_recurrence_chunked_amd/csrc) never calls it,
 * and the two share no source, header, table or helper.
 *
 * Every routine here walks a whole prompt one token at a time in float64,
 * in the order the recurrence is defined; none of them chunks, blocks or
 * reorders the work.  OpenMP parallelism is over independent channels or
 * heads only, so each channel's arithmetic is a plain sequential loop.
 * Compile without fast-math and with -ffp-contract=off.
 *
 * Sources (page title, section):
 *  - "perf(mamba): prefill text prompts in multi-token chunks", Implementation:
 *    the depthwise causal short conv whose window reaches back into a stored
 *    conv state, and the selective scan h_t = a_t h_{t-1} + b_t.
 *  - "perf(rwkv): prefill text prompts in multi-token chunks", Implementation:
 *    the RWKV-4 one-token WKV step, with A and B stored as (num, den, max).
 *  - "perf(qwen3_5): prefill text prompts in multi-token chunks",
 *    Implementation: the chunked Gated DeltaNet delta rule; its one-row case
 *    is the token step below.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Number of threads OpenMP will use for the parallel loops below. */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/*
 * Depthwise causal convolution over rows ("perf(mamba): ..." and
 * "perf(qwen3_5): ...", Implementation): the window of each row reaches back
 * into K-1 stored state rows before the chunk, and the state kept for the
 * next chunk is the final K-1 rows of state-then-chunk.
 *
 * Reading where the page is silent: the window is a causal cross-correlation,
 * tap K-1 multiplies the current row and tap 0 the oldest one; no activation;
 * bias optional (NULL = none).
 *
 *   xt(r) = state_in[r]        for r <  K-1
 *         = x[r-(K-1)]         for r >= K-1          (r = 0 .. S+K-2)
 *   y[t][c] = bias[c] + sum_{j<K} w[c][j] * xt(t+j)[c]
 *   state_out[r][c] = xt(S+r)[c],  r = 0 .. K-2
 *
 * x, y: [S][C]; state_in, state_out: [K-1][C]; w: [C][K]; bias: [C] or NULL.
 */
void oracle_conv_rows(const double* x, const double* state_in, const double* w,
                      const double* bias, int S, int C, int K, double* y,
                      double* state_out) {
    const int H = K - 1;
#pragma omp parallel for schedule(static)
    for (int c = 0; c < C; ++c) {
        for (int t = 0; t < S; ++t) {
            double acc = bias ? bias[c] : 0.0;
            for (int j = 0; j < K; ++j) {
                const int r = t + j;
                const double xv = (r < H) ? state_in[(size_t)r * C + c]
                                          : x[(size_t)(r - H) * C + c];
                acc += w[(size_t)c * K + j] * xv;
            }
            y[(size_t)t * C + c] = acc;
        }
        for (int r = 0; r < H; ++r) {
            const int src = S + r;
            state_out[(size_t)r * C + c] = (src < H) ? state_in[(size_t)src * C + c]
                                                     : x[(size_t)(src - H) * C + c];
        }
    }
}

/*
 * Selective scan ("perf(mamba): ...", Implementation): for every state
 * element e independently, h_t = a_t * h_{t-1} + b_t starting from h_0.
 * Output is every h_t (t = 0..S-1) and the final state.
 *
 * a, b, h: [S][E]; h0, hS: [E].
 */
void oracle_scan(const double* a, const double* b, const double* h0, int S, long E,
                 double* h, double* hS) {
#pragma omp parallel for schedule(static)
    for (long e = 0; e < E; ++e) {
        double s = h0[e];
        for (int t = 0; t < S; ++t) {
            const size_t i = (size_t)t * (size_t)E + (size_t)e;
            s = a[i] * s + b[i];
            h[i] = s;
        }
        hS[e] = s;
    }
}

/*
 * RWKV-4 WKV, one token at a time ("perf(rwkv): ...", Implementation).
 * The decoder keeps A_t = e^w A_{t-1} + e^{k_t} v_t and
 * B_t = e^w B_{t-1} + e^{k_t} as A = num * e^max, B = den * e^max, and emits
 * wkv_t = (A_{t-1} + e^{u+k_t} v_t) / (B_{t-1} + e^{u+k_t}).  Every exponential
 * is taken after a shift by the largest exponent among the terms it joins:
 *   output:  p = max(max, u+k_t)
 *   update:  q = max(max + w, k_t),  new max = q.
 * The empty state is (0, 0, -1e38): a finite stand-in for log 0.
 *
 * k, v, wkv: [S][C]; w, u: [C]; num, den, mx: [C], updated in place.
 */
void oracle_wkv4(const double* k, const double* v, const double* w, const double* u,
                 int S, int C, double* num, double* den, double* mx, double* wkv) {
#pragma omp parallel for schedule(static)
    for (int c = 0; c < C; ++c) {
        double aa = num[c], bb = den[c], pp = mx[c];
        const double wc = w[c], uc = u[c];
        for (int t = 0; t < S; ++t) {
            const size_t i = (size_t)t * C + c;
            const double kt = k[i], vt = v[i];
            /* output of row t: state before the row plus the bonus term */
            const double eb = uc + kt;
            const double p = pp > eb ? pp : eb;
            const double fs = exp(pp - p), fb = exp(eb - p);
            wkv[i] = (fs * aa + fb * vt) / (fs * bb + fb);
            /* state update with decay e^w and the new key */
            const double ed = pp + wc;
            const double q = ed > kt ? ed : kt;
            const double gs = exp(ed - q), gk = exp(kt - q);
            aa = gs * aa + gk * vt;
            bb = gs * bb + gk;
            pp = q;
        }
        num[c] = aa;
        den[c] = bb;
        mx[c] = pp;
    }
}

/*
 * WKV with a token-dependent decay ("perf(rwkv): ...", Notes For Future
 * Readers: RWKV generations with a per-token decay call for a different chunk
 * form).  The pages give no formula for those versions; the reading here is
 * the RWKV-4 step above with the channel decay w replaced by a decay w_t of
 * the row (w_t < 0), applied where the state moves past row t:
 *   A_t = e^{w_t} A_{t-1} + e^{k_t} v_t,  B_t = e^{w_t} B_{t-1} + e^{k_t},
 *   wkv_t = (A_{t-1} + e^{u+k_t} v_t) / (B_{t-1} + e^{u+k_t}),
 * with the same shifts by the largest exponent (update: q = max(max + w_t, k_t)).
 * A constant w_t = w is the RWKV-4 step.
 *
 * k, v, w, wkv: [S][C]; u: [C]; num, den, mx: [C], updated in place.
 */
void oracle_wkv_tdecay(const double* k, const double* v, const double* w, const double* u,
                       int S, int C, double* num, double* den, double* mx, double* wkv) {
#pragma omp parallel for schedule(static)
    for (int c = 0; c < C; ++c) {
        double aa = num[c], bb = den[c], pp = mx[c];
        const double uc = u[c];
        for (int t = 0; t < S; ++t) {
            const size_t i = (size_t)t * C + c;
            const double key = k[i], val = v[i], wt = w[i];
            /* output of row t: state before the row plus the bonus term */
            const double bonus = uc + key;
            const double top = pp > bonus ? pp : bonus;
            const double fs = exp(pp - top), fb = exp(bonus - top);
            wkv[i] = (fs * aa + fb * val) / (fs * bb + fb);
            /* state update with the row's decay e^{w_t} and the new key */
            const double decayed = pp + wt;
            const double q = decayed > key ? decayed : key;
            const double gs = exp(decayed - q), gk = exp(key - q);
            aa = gs * aa + gk * val;
            bb = gs * bb + gk;
            pp = q;
        }
        num[c] = aa;
        den[c] = bb;
        mx[c] = pp;
    }
}

/*
 * Gated DeltaNet, one token at a time ("perf(qwen3_5): ...", Implementation).
 * The page gives the chunk form; its one-row case (A = 0, Gamma = e^{g_t})
 * is this step, for value head h with key head kh = h / (Hv / Hk):
 *   u   = beta_t * (v_t - e^{g_t} S^T k_t)
 *   S  <- e^{g_t} S + k_t u^T              (dk x dv)
 *   o_t = S^T q_t                          (after the update)
 * No scale is applied to q.
 *
 * q, k: [S][Hk][dk]; v: [S][Hv][dv]; beta, g: [S][Hv];
 * S0, Sout: [Hv][dk][dv]; o: [S][Hv][dv].  dv <= 1024.
 * Each head evolves its state in place in Sout.
 */
void oracle_gdn(const double* q, const double* k, const double* v, const double* beta,
                const double* g, const double* S0, int S, int Hk, int Hv, int dk, int dv,
                double* o, double* Sout) {
    const int grp = Hv / Hk;
#pragma omp parallel for schedule(dynamic, 1)
    for (int h = 0; h < Hv; ++h) {
        const int kh = h / grp;
        double* St = Sout + (size_t)h * dk * dv;
        const double* Si = S0 + (size_t)h * dk * dv;
        for (size_t i = 0; i < (size_t)dk * dv; ++i) St[i] = Si[i];
        double uvec[1024];
        for (int t = 0; t < S; ++t) {
            const double* kt = k + ((size_t)t * Hk + kh) * dk;
            const double* qt = q + ((size_t)t * Hk + kh) * dk;
            const double* vt = v + ((size_t)t * Hv + h) * dv;
            const double bt = beta[(size_t)t * Hv + h];
            const double dec = exp(g[(size_t)t * Hv + h]);
            for (int j = 0; j < dv; ++j) {
                double sk = 0.0;
                for (int i = 0; i < dk; ++i) sk += St[(size_t)i * dv + j] * kt[i];
                uvec[j] = bt * (vt[j] - dec * sk);
            }
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j)
                    St[(size_t)i * dv + j] = dec * St[(size_t)i * dv + j] + kt[i] * uvec[j];
            double* ot = o + ((size_t)t * Hv + h) * dv;
            for (int j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int i = 0; i < dk; ++i) acc += St[(size_t)i * dv + j] * qt[i];
                ot[j] = acc;
            }
        }
    }
}

/*
 * Inverse of a unit lower-triangular matrix I + L ("perf(qwen3_5): ...",
 * Implementation, where the chunk form needs (I + A)^-1 for strictly lower A).  The
 * oracle uses textbook forward substitution, column by column:
 *   T[i][j] = [i == j] - sum_{j <= m < i} L[i][m] T[m][j].
 * Only the strictly lower part of L is read.
 *
 * L, T: batch x [n][n], row-major.
 */
void oracle_unit_lower_inverse(const double* L, int batch, int n, double* T) {
#pragma omp parallel for schedule(static)
    for (int bidx = 0; bidx < batch; ++bidx) {
        const double* Lb = L + (size_t)bidx * n * n;
        double* Tb = T + (size_t)bidx * n * n;
        for (int j = 0; j < n; ++j) {
            for (int i = 0; i < n; ++i) {
                if (i < j) {
                    Tb[(size_t)i * n + j] = 0.0;
                    continue;
                }
                double acc = (i == j) ? 1.0 : 0.0;
                for (int m = j; m < i; ++m) acc -= Lb[(size_t)i * n + m] * Tb[(size_t)m * n + j];
                Tb[(size_t)i * n + j] = acc;
            }
        }
    }
}

/*
 * RWKV-4 time shift ("perf(rwkv): prefill text prompts in multi-token
 * chunks", Implementation): each mixed input blends row t with row t-1, and
 * row 0 with the incoming shift state; the shift state kept for the next
 * chunk is the chunk's last row.
 *
 * Reading where the page is silent: the blend is RWKV-4's per-channel mix
 * mu x_t + (1 - mu) x_{t-1}, with M mixing vectors (one per mixed input:
 * key, value, receptance, ...) applied to the same rows.
 *
 *   xp(t) = state_in[c]  (t = 0),   x[t-1][c]  (t > 0)
 *   out[j][t][c] = mix[j][c] * x[t][c] + (1 - mix[j][c]) * xp(t)
 *   state_out[c] = x[S-1][c]  (S > 0),   state_in[c]  (S = 0)
 *
 * x: [S][C]; state_in, state_out: [C]; mix: [M][C]; out: [M][S][C].
 */
void oracle_time_shift(const double* x, const double* state_in, const double* mix, int S, int C, int M,
                       double* out, double* state_out) {
#pragma omp parallel for schedule(static)
    for (int c = 0; c < C; ++c) {
        double prev = state_in[c];
        for (int t = 0; t < S; ++t) {
            const double cur = x[(size_t)t * C + c];
            for (int j = 0; j < M; ++j) {
                const double mu = mix[(size_t)j * C + c];
                out[((size_t)j * S + t) * C + c] = mu * cur + (1.0 - mu) * prev;
            }
            prev = cur;
        }
        state_out[c] = prev;
    }
}

/*
 * Mamba selective-scan mixer rows with the discretisation and the readout
 * around the scan ("perf(mamba): prefill text prompts in multi-token
 * chunks", Implementation: the mixer rows run the scan h_t = a_t h_{t-1} + b_t
 * between the steps that form a, b and read h out).
 *
 * Reading where the page is silent: the selective state-space step of
 * Mamba -- a zero-order hold on A and an Euler step on B -- with the skip
 * term D and no output gate:
 *
 *   a_t[d][n] = exp(dt[t][d] * A[d][n])
 *   b_t[d][n] = dt[t][d] * Bm[t][n] * x[t][d]
 *   h_t[d][n] = a_t[d][n] h_{t-1}[d][n] + b_t[d][n]
 *   y[t][d]   = sum_n Cm[t][n] h_t[d][n] + Dp[d] x[t][d]
 *
 * x, dt: [S][Dm]; A: [Dm][N]; Bm, Cm: [S][N]; Dp: [Dm]; h0, hS: [Dm][N];
 * y: [S][Dm].  N <= 256.
 */
void oracle_mamba_mixer(const double* x, const double* dt, const double* A, const double* Bm,
                        const double* Cm, const double* Dp, const double* h0, int S, int Dm, int N,
                        double* y, double* hS) {
#pragma omp parallel for schedule(static)
    for (int d = 0; d < Dm; ++d) {
        double h[256];
        for (int n = 0; n < N; ++n) h[n] = h0[(size_t)d * N + n];
        for (int t = 0; t < S; ++t) {
            const double dtv = dt[(size_t)t * Dm + d];
            const double xv = x[(size_t)t * Dm + d];
            double acc = 0.0;
            for (int n = 0; n < N; ++n) {
                const double a = exp(dtv * A[(size_t)d * N + n]);
                const double b = dtv * Bm[(size_t)t * N + n] * xv;
                h[n] = a * h[n] + b;
                acc += Cm[(size_t)t * N + n] * h[n];
            }
            y[(size_t)t * Dm + d] = acc + Dp[d] * xv;
        }
        for (int n = 0; n < N; ++n) hS[(size_t)d * N + n] = h[n];
    }
}

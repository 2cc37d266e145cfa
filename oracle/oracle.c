/*
 * oracle.c -- plain fp64 CPU reference for the RDA gated delta rule.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file; only the tests, the smoke check and the bench's CPU
 * baseline leg use it.  It shares no code, header or table with the HIP
 * library.
 *
 * What it computes.  RDA ("Raon Delta Attention") is described on the page
 * "Raon-1 nano" (ai.satyajit.si), section "The other 1.5B: a hybrid built to
 * forget", as a gated delta-rule linear attention.  Its recurrent step, in
 * the order that section gives: scale the matrix state S by the decay a,
 * take the residual e = v - S'k of the scaled state S' at the key, and add
 * the rank-one update b e k^T (b the write strength, beta on the page).  The same page, section "The cache is small if the runtime
 * keeps it small", fixes the state as one 128 x 128 fp32 matrix per head.
 * With a scalar decay a_t in (0,1] and write strength b_t in [0,1] per token
 * and head, that step is the gated delta rule
 *
 *     S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T ,   o_t = S_t q_t
 *
 * written here in the page's order of operations:
 *
 *     S'  = a_t S_{t-1}            (decay)
 *     e   = v_t - S' k_t           (error against the decayed state)
 *     S_t = S' + b_t e k_t^T       (write with strength b_t)
 *     o_t = S_t q_t                (read-out after the update)
 *
 * which equals the product form exactly in real arithmetic.  The state is
 * stored row-major as S[i][j] with i the value channel (0..dv-1) and j the
 * key channel (0..dk-1).  Tokens are laid out [T, H, d]; gates [T, H].
 * No query scale and no normalisation happen here: q and k are used exactly
 * as given.  Tokens are processed strictly in order, one at a time; the only
 * parallelism is across independent (sequence, head) pairs.
 *
 * Every input is widened exactly to double before use; all arithmetic is
 * double.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_ARG 1
#define ORACLE_ERR_NOMEM 2

int oracle_version(void) { return 1; }

/* One token of the recurrence on one head's state S[dv][dk] (see header). */
static void oracle_token(double* S, double* e, int dk, int dv,
                         const float* q, const float* k, const float* v,
                         double a, double b, double* o) {
    /* decay */
    for (int i = 0; i < dv; ++i)
        for (int j = 0; j < dk; ++j)
            S[(size_t)i * dk + j] *= a;
    /* error against the decayed state: e = v - S k */
    for (int i = 0; i < dv; ++i) {
        double pred = 0.0;
        for (int j = 0; j < dk; ++j)
            pred += S[(size_t)i * dk + j] * (double)k[j];
        e[i] = (double)v[i] - pred;
    }
    /* write with strength b: S += b e k^T */
    for (int i = 0; i < dv; ++i)
        for (int j = 0; j < dk; ++j)
            S[(size_t)i * dk + j] += b * e[i] * (double)k[j];
    /* read-out with the updated state: o = S q */
    if (o) {
        for (int i = 0; i < dv; ++i) {
            double acc = 0.0;
            for (int j = 0; j < dk; ++j)
                acc += S[(size_t)i * dk + j] * (double)q[j];
            o[i] = acc;
        }
    }
}

/*
 * Prefill over packed variable-length sequences.
 *   q, k   : [total_tokens, H, dk] fp32 (bf16 inputs arrive widened exactly)
 *   v      : [total_tokens, H, dv] fp32
 *   a, b   : [total_tokens, H] fp32
 *   cu     : [num_seqs + 1] int32 token offsets, cu[0] = 0, non-decreasing,
 *            cu[num_seqs] = total_tokens; NULL means one sequence of all tokens
 *   S0     : [num_seqs, H, dv, dk] double, or NULL for zero initial states
 *   o      : [total_tokens, H, dv] double (output)
 *   S_final: [num_seqs, H, dv, dk] double (output, may be NULL)
 *   threads: OpenMP threads over (sequence, head) pairs; <= 0 means default
 * Returns 0, or a nonzero code for invalid arguments / allocation failure.
 */
int oracle_rda_prefill(const float* q, const float* k, const float* v,
                       const float* a, const float* b,
                       const int32_t* cu, int32_t num_seqs, int64_t total_tokens,
                       int32_t H, int32_t dk, int32_t dv,
                       const double* S0, double* o, double* S_final,
                       int32_t threads) {
    if (!q || !k || !v || !a || !b || !o) return ORACLE_ERR_ARG;
    if (H <= 0 || dk <= 0 || dv <= 0 || total_tokens < 0) return ORACLE_ERR_ARG;
    int32_t n_seq = cu ? num_seqs : 1;
    if (n_seq <= 0) return ORACLE_ERR_ARG;
    if (cu) {
        if (cu[0] != 0 || cu[n_seq] != total_tokens) return ORACLE_ERR_ARG;
        for (int32_t n = 0; n < n_seq; ++n)
            if (cu[n + 1] < cu[n]) return ORACLE_ERR_ARG;
    }
    const size_t dd = (size_t)dv * dk;
    const int64_t units = (int64_t)n_seq * H;
    int err = ORACLE_OK;
#ifdef _OPENMP
    int nt = threads > 0 ? threads : omp_get_max_threads();
#pragma omp parallel num_threads(nt)
#endif
    {
        double* S = (double*)malloc(dd * sizeof(double));
        double* e = (double*)malloc((size_t)dv * sizeof(double));
        if (!S || !e) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            err = ORACLE_ERR_NOMEM;
        } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
            for (int64_t u = 0; u < units; ++u) {
                const int32_t n = (int32_t)(u / H), h = (int32_t)(u % H);
                const int64_t t0 = cu ? cu[n] : 0;
                const int64_t t1 = cu ? cu[n + 1] : total_tokens;
                if (S0) memcpy(S, S0 + (size_t)u * dd, dd * sizeof(double));
                else memset(S, 0, dd * sizeof(double));
                for (int64_t t = t0; t < t1; ++t) {
                    const size_t th = (size_t)t * H + h;
                    oracle_token(S, e, dk, dv, q + th * dk, k + th * dk, v + th * dv,
                                 (double)a[th], (double)b[th], o + th * dv);
                }
                if (S_final) memcpy(S_final + (size_t)u * dd, S, dd * sizeof(double));
            }
        }
        free(S);
        free(e);
    }
    return err;
}

/*
 * One decode step: the same recurrence for a single token per (batch, head),
 * applied in place to the fp64 state.
 *   q, k : [B, H, dk] fp32;  v : [B, H, dv] fp32;  a, b : [B, H] fp32
 *   S    : [B, H, dv, dk] double, in/out
 *   o    : [B, H, dv] double, output
 */
int oracle_rda_decode_step(const float* q, const float* k, const float* v,
                           const float* a, const float* b,
                           int32_t B, int32_t H, int32_t dk, int32_t dv,
                           double* S, double* o, int32_t threads) {
    if (!q || !k || !v || !a || !b || !S || !o) return ORACLE_ERR_ARG;
    if (B < 0 || H <= 0 || dk <= 0 || dv <= 0) return ORACLE_ERR_ARG;
    const size_t dd = (size_t)dv * dk;
    const int64_t units = (int64_t)B * H;
    int err = ORACLE_OK;
#ifdef _OPENMP
    int nt = threads > 0 ? threads : omp_get_max_threads();
#pragma omp parallel num_threads(nt)
#endif
    {
        double* e = (double*)malloc((size_t)dv * sizeof(double));
        if (!e) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            err = ORACLE_ERR_NOMEM;
        } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 16)
#endif
            for (int64_t u = 0; u < units; ++u) {
                oracle_token(S + (size_t)u * dd, e, dk, dv, q + (size_t)u * dk,
                             k + (size_t)u * dk, v + (size_t)u * dv,
                             (double)a[u], (double)b[u], o + (size_t)u * dv);
            }
        }
        free(e);
    }
    return err;
}

/*
 * Per-channel (diagonal) decay: the variant where the decay is a vector over
 * the key channels instead of one scalar per token and head.  The vLLM
 * article on Raon-1 mini calls RDA a modification of Kimi Delta Attention,
 * whose decay is per channel, and the tiny-model card prints a low-rank
 * decay projection (f_a_proj, f_b_proj) whose output has the width of the
 * heads' key channels.  With alpha_t in (0,1]^dk the step, in the teardown's
 * order (decay, error against the decayed state, write, read-out), is
 *
 *     S'  = S_{t-1} diag(alpha_t)      (column j of S scaled by alpha_tj)
 *     e   = v_t - S' k_t
 *     S_t = S' + b_t e k_t^T
 *     o_t = S_t q_t
 *
 * alpha: [total_tokens, H, dk] fp32; everything else as in
 * oracle_rda_prefill / oracle_rda_decode_step.
 */
static void oracle_token_diag(double* Sd, double* err, int dk, int dv, const float* qv,
                              const float* kv, const float* vv, const float* alpha,
                              double beta, double* out) {
    for (int r = 0; r < dv; ++r) {
        double* row = Sd + (size_t)r * dk;
        double pr = 0.0;
        for (int c = 0; c < dk; ++c) {
            row[c] = row[c] * (double)alpha[c];
            pr += row[c] * (double)kv[c];
        }
        err[r] = (double)vv[r] - pr;
    }
    for (int r = 0; r < dv; ++r) {
        double* row = Sd + (size_t)r * dk;
        const double be = beta * err[r];
        for (int c = 0; c < dk; ++c) row[c] += be * (double)kv[c];
        if (out) {
            double acc = 0.0;
            for (int c = 0; c < dk; ++c) acc += row[c] * (double)qv[c];
            out[r] = acc;
        }
    }
}

int oracle_rda_prefill_diag(const float* q, const float* k, const float* v,
                            const float* alpha, const float* b, const int32_t* cu,
                            int32_t n_seq, int64_t total_tokens, int32_t H, int32_t dk,
                            int32_t dv, const double* S0, double* o, double* S_final,
                            int32_t threads) {
    if (!q || !k || !v || !alpha || !b || !o) return ORACLE_ERR_ARG;
    if (H <= 0 || dk <= 0 || dv <= 0 || total_tokens < 0 || n_seq <= 0) return ORACLE_ERR_ARG;
    if (!cu && n_seq != 1) return ORACLE_ERR_ARG;
    if (cu) {
        if (cu[0] != 0 || cu[n_seq] != total_tokens) return ORACLE_ERR_ARG;
        for (int32_t n = 0; n < n_seq; ++n)
            if (cu[n + 1] < cu[n]) return ORACLE_ERR_ARG;
    }
    const size_t dd = (size_t)dv * dk;
    const int64_t units = (int64_t)n_seq * H;
    int rc = ORACLE_OK;
#ifdef _OPENMP
    int nt = threads > 0 ? threads : omp_get_max_threads();
#pragma omp parallel num_threads(nt)
#endif
    {
        double* Sd = (double*)malloc(dd * sizeof(double));
        double* err = (double*)malloc((size_t)dv * sizeof(double));
        if (!Sd || !err) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            rc = ORACLE_ERR_NOMEM;
        } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
            for (int64_t u = 0; u < units; ++u) {
                const int32_t n = (int32_t)(u / H), h = (int32_t)(u % H);
                const int64_t first = cu ? cu[n] : 0, last = cu ? cu[n + 1] : total_tokens;
                if (S0) memcpy(Sd, S0 + (size_t)u * dd, dd * sizeof(double));
                else memset(Sd, 0, dd * sizeof(double));
                for (int64_t t = first; t < last; ++t) {
                    const size_t row = (size_t)t * H + h;
                    oracle_token_diag(Sd, err, dk, dv, q + row * dk, k + row * dk, v + row * dv,
                                      alpha + row * dk, (double)b[row], o + row * dv);
                }
                if (S_final) memcpy(S_final + (size_t)u * dd, Sd, dd * sizeof(double));
            }
        }
        free(Sd);
        free(err);
    }
    return rc;
}

int oracle_rda_decode_step_diag(const float* q, const float* k, const float* v,
                                const float* alpha, const float* b, int32_t B, int32_t H,
                                int32_t dk, int32_t dv, double* S, double* o) {
    if (!q || !k || !v || !alpha || !b || !S || !o) return ORACLE_ERR_ARG;
    if (B < 0 || H <= 0 || dk <= 0 || dv <= 0) return ORACLE_ERR_ARG;
    double* err = (double*)malloc((size_t)dv * sizeof(double));
    if (!err) return ORACLE_ERR_NOMEM;
    for (int64_t u = 0; u < (int64_t)B * H; ++u)
        oracle_token_diag(S + (size_t)u * dv * dk, err, dk, dv, q + (size_t)u * dk,
                          k + (size_t)u * dk, v + (size_t)u * dv, alpha + (size_t)u * dk,
                          (double)b[u], o + (size_t)u * dv);
    free(err);
    return 0;
}

/*
 * Output epilogue of the mixer: per output row of one head (dv channels),
 * an RMS normalisation with epsilon and a per-channel weight, times an
 * activation of the output gate.  The tiny-random/raon-1-mini model card,
 * section "Printing the model", lists the RDA block's o_norm as an RMS norm
 * over the head dimension with eps 1e-5 and a g_proj projection producing
 * the gate; the gate's activation is not printed, so `act` selects it:
 * 0 = sigmoid, 1 = SiLU (x sigmoid(x)), 2 = none.  w may be NULL (unit
 * weight); g may be NULL only with act = 2.
 *
 *     y_c = o_c / sqrt(mean_c'(o_c'^2) + eps) * w_c * act(g_c)
 */
int oracle_output_norm_gate(const float* o, const float* g, const float* w, double eps,
                            int32_t act, int64_t rows, int32_t dv, double* out) {
    if (rows < 0 || dv <= 0 || !out || (rows > 0 && !o)) return ORACLE_ERR_ARG;
    if (act < 0 || act > 2 || (act != 2 && rows > 0 && !g)) return ORACLE_ERR_ARG;
    for (int64_t r = 0; r < rows; ++r) {
        const float* orow = o + (size_t)r * dv;
        double ms = 0.0;
        for (int32_t c = 0; c < dv; ++c) ms += (double)orow[c] * (double)orow[c];
        ms /= dv;
        const double inv = 1.0 / sqrt(ms + eps);
        for (int32_t c = 0; c < dv; ++c) {
            double gate = 1.0;
            if (act != 2) {
                const double x = (double)g[(size_t)r * dv + c];
                const double sig = 1.0 / (1.0 + exp(-x));
                gate = act == 0 ? sig : x * sig;
            }
            out[(size_t)r * dv + c] = (double)orow[c] * inv * (w ? (double)w[c] : 1.0) * gate;
        }
    }
    return 0;
}

/*
 * Prologue of the mixer: the steps between the projections and the
 * recurrence, for packed sequences (cu: int32 [N+1], or NULL for one
 * sequence of T tokens).  The Raon-1 nano teardown (section "The cache is
 * small if the runtime keeps it small") keeps a short convolution window per
 * layer beside the recurrent state; its section "The other 1.5B" gives the
 * decoupled gates -- erase with beta = sigmoid(beta_raw), a separate write
 * gate sigmoid(beta_raw + delta) / sigmoid(beta_raw) scaling the value -- and
 * the decay bounded below by -5 in log space; the Raon-1 mini vLLM article
 * applies the write gate after the convolution, so the raw history is kept.
 * Per token t of sequence n and tensor x in (q, k, v), channel c of head h:
 *
 *   y = sum_{i<K} w[x][h][c][i] * raw_x(t - (K-1) + i)      (causal conv,
 *       raw_x of positions before the sequence from the history hist_in)
 *   y = silu(y) when act = 1 (act = 0: no activation)
 *   q, k: y / sqrt(sum_c y^2 + l2_eps)     v: y * sig(beta_raw + delta) / sig(beta_raw)
 *   b = sig(beta_raw),   a = exp(max(g_log, floor))
 *
 * Layouts: raw q, k, v [T, H, d] (values exact in fp32); w [3][H][d][K]
 * (q, k, v; tap K-1 multiplies the current token); hist [N][3][K-1][H][d]
 * with slot m holding the token m - (K-1) positions before the sequence's
 * first token (NULL: zeros); beta_raw, delta, g_log [T, H] (delta NULL: 0).
 * Outputs q, k, v as doubles [T, H, d], a, b [T, H] and hist_out (the raw
 * tokens at the last K-1 positions of each sequence, from hist_in where the
 * sequence is shorter), all double.
 */
int oracle_prologue(const float* xq, const float* xk, const float* xv, const float* w,
                    int32_t K, int32_t act, const float* hist_in, const float* beta_raw,
                    const float* delta, const float* g_log, double floor_log, double l2_eps,
                    const int32_t* cu, int32_t N, int64_t T, int32_t H, int32_t d,
                    double* q, double* k, double* v, double* a, double* b, double* hist_out) {
    if (K < 1 || K > 8 || (act != 0 && act != 1) || N < 1 || T < 0 || H <= 0 || d <= 0)
        return ORACLE_ERR_ARG;
    if (!cu && N != 1) return ORACLE_ERR_ARG;
    const float* raw[3] = {xq, xk, xv};
    double* out[3] = {q, k, v};
    const size_t hd = (size_t)H * d;
    double* y = (double*)malloc((size_t)d * sizeof(double));
    if (!y) return ORACLE_ERR_NOMEM;
    for (int32_t n = 0; n < N; ++n) {
        const int64_t t0 = cu ? cu[n] : 0, t1 = cu ? cu[n + 1] : T;
        if (t0 < 0 || t1 < t0 || t1 > T) { free(y); return ORACLE_ERR_ARG; }
        for (int64_t t = t0; t < t1; ++t) {
            for (int32_t h = 0; h < H; ++h) {
                const size_t tkh = (size_t)t * H + h;
                const double br = beta_raw[tkh];
                const double sig_b = 1.0 / (1.0 + exp(-br));
                const double dl = delta ? (double)delta[tkh] : 0.0;
                const double wgate = (1.0 / (1.0 + exp(-(br + dl)))) / sig_b;
                b[tkh] = sig_b;
                a[tkh] = exp(fmax((double)g_log[tkh], floor_log));
                for (int x = 0; x < 3; ++x) {
                    double ss = 0.0;
                    for (int32_t c = 0; c < d; ++c) {
                        double acc = 0.0;
                        for (int32_t i = 0; i < K; ++i) {
                            const int64_t pos = t - (K - 1) + i;   /* raw position */
                            double xr = 0.0;
                            if (pos >= t0) {
                                xr = raw[x][(size_t)pos * hd + (size_t)h * d + c];
                            } else if (hist_in) {
                                const int64_t m = pos - t0 + (K - 1);   /* history slot */
                                xr = hist_in[(((size_t)n * 3 + x) * (K - 1) + m) * hd +
                                             (size_t)h * d + c];
                            }
                            acc += (double)w[(((size_t)x * H + h) * d + c) * K + i] * xr;
                        }
                        if (act == 1) acc = acc / (1.0 + exp(-acc));
                        y[c] = acc;
                        ss += acc * acc;
                    }
                    const double scale = x < 2 ? 1.0 / sqrt(ss + l2_eps) : wgate;
                    for (int32_t c = 0; c < d; ++c) out[x][tkh * d + c] = y[c] * scale;
                }
            }
        }
        /* the history after the sequence: its last K-1 raw tokens */
        const int64_t len = t1 - t0;
        for (int x = 0; x < 3; ++x)
            for (int32_t m = 0; m < K - 1; ++m)
                for (size_t e = 0; e < hd; ++e) {
                    const int64_t pos = t1 - (K - 1) + m;
                    double val = 0.0;
                    if (pos >= t0)
                        val = raw[x][(size_t)pos * hd + e];
                    else if (hist_in)
                        val = hist_in[(((size_t)n * 3 + x) * (K - 1) + (m + len)) * hd + e];
                    hist_out[(((size_t)n * 3 + x) * (K - 1) + m) * hd + e] = val;
                }
    }
    free(y);
    return 0;
}

/* Number of OpenMP threads a call with `threads` would use. */
int oracle_threads(int32_t threads) {
#ifdef _OPENMP
    return threads > 0 ? threads : omp_get_max_threads();
#else
    (void)threads;
    return 1;
#endif
}

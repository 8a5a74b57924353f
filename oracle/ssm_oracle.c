/*
 * ssm_oracle.c -- plain, slow fp64 CPU oracle for the SSM scan + causal conv1d path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load this file's library.  The product path (the HIP library under
 * ssm_sequence_models_amd/) shares no code with it and never calls it.
 *
 * Sources (cited by page title and section; no line numbers):
 *   [LG]  "Understanding and Improving Length Generalization in Recurrent Models: reading
 *         notes" (arXiv:2507.02782v2).  Sec. 2.1 Eq. (1) (the recurrence and the initial
 *         state h_{-1}); Sec. 2.5 Eq. (4) (unrolling with a non-zero initial state);
 *         Sec. 2.6 (State Passing / TBTT: initial state in, final state out).
 *   [CC]  Causal-conv1d tutorial, chapter 7 "State, chunking and incremental inference".
 *         Sections: "defining the state through the extended sequence" (u, z_t, F);
 *         "single-token update maths"; "the physical cache may exceed the minimal history"
 *         (state_len, circular mode with cache_seqlens); "state indices for continuous
 *         batching" (conv_state_indices); "packed-sequence boundaries" (seq_idx).
 *
 * Everything is computed in double precision straight from the definitions: no chunking,
 * no blocking, no reordering.  Inputs arrive as doubles (the Python wrapper widens bf16 and
 * fp32 exactly); outputs are rounded once to the requested storage type.
 *
 * Readings taken where the pages leave a step open (all listed in the design notes):
 *   - a_t = exp(dt_t * A_h) and the input term dt_t * B_t * x_t (Mamba-2-style scalar decay;
 *     [LG] Sec. 2.5 says the transition enters in log space).  Parity unpinned beyond
 *     convention for the dt factor on B; with dt = 1 it is exactly Eq. (1).
 *   - each of a head's P channels is one copy of Eq. (1) sharing a_t, B_t, C_t; head h uses
 *     group g = h / (H / G).
 *   - seq_idx in the scan: the state is zeroed where seq_idx changes between t-1 and t;
 *     in the conv, the initial state S belongs to the segment of token 0.
 *   - phi is either the identity or SiLU, z * sigmoid(z).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Number of threads the parallel loops below use (1 without OpenMP). */
int orc_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Rounding modes for outputs. */
#define ORC_ROUND_NONE 0 /* keep fp64 */
#define ORC_ROUND_F32 1  /* round to nearest even fp32 */
#define ORC_ROUND_BF16 2 /* round to nearest even bfloat16 (8 significant bits) */

#define ORC_ACT_NONE 0
#define ORC_ACT_SILU 1

/* Round a double to bfloat16 precision, nearest-even, straight from the double (no
 * intermediate fp32 step, so no double rounding).  bfloat16 keeps 8 significant bits for
 * normal numbers (exponent down to 2^-126) and a fixed quantum of 2^-133 below that. */
static double round_bf16(double v) {
    if (v != v || v == 0.0 || isinf(v)) return v;
    int e;
    (void)frexp(fabs(v), &e); /* |v| = m * 2^e with m in [0.5, 1) */
    int q = e - 8;            /* quantum of an 8-significant-bit number of that size */
    if (q < -133) q = -133;
    double r = ldexp(nearbyint(ldexp(fabs(v), -q)), q);
    const double bf16_max = ldexp(255.0, 120); /* (2 - 2^-7) * 2^127 */
    if (r > bf16_max) r = INFINITY;
    return copysign(r, v);
}

double orc_round(double v, int mode) {
    if (mode == ORC_ROUND_F32) return (double)(float)v;
    if (mode == ORC_ROUND_BF16) return round_bf16(v);
    return v;
}

static double act_apply(double z, int act) {
    if (act == ORC_ACT_SILU) return z / (1.0 + exp(-z));
    return z;
}

static int64_t floor_mod(int64_t a, int64_t m) {
    int64_t r = a % m;
    return r < 0 ? r + m : r;
}

/* ---------------------------------------------------------------------------------------
 * Causal depthwise conv1d with state in / out ([CC] "defining the state through the
 * extended sequence", "packed-sequence boundaries").
 *
 *   u = [S_0 .. S_{K-2}, x_0 .. x_{L-1}]           (S oldest -> newest; S = 0 if absent)
 *   z_t = beta + sum_k w_k u_{t+k}                  (w_{K-1} multiplies the current x_t)
 *   out_t = round(phi(z_t)),   F = u[L : L+K-1]     (a raw copy; also right for L < K-1)
 *
 * With seq_idx, a tap contributes only when its token carries the same identity as the
 * output token (identity equality, as the page describes); S carries the identity of
 * token 0.  F stays the unmasked raw slice.
 *
 * Layouts: x, out [B][L][C]; w [C][K]; bias [C]; init_state, final_state [B][C][K-1];
 * seq_idx [B][L].
 * ------------------------------------------------------------------------------------- */
int orc_conv1d_fwd(const double* x, const double* w, const double* bias,
                   const double* init_state, double* final_state, const int32_t* seq_idx,
                   double* out, int64_t B, int64_t L, int64_t C, int64_t K, int act,
                   int out_round) {
    const int64_t U = K - 1 + L;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t c = 0; c < C; ++c) {
            double* u = (double*)malloc(sizeof(double) * (size_t)(U > 0 ? U : 1));
            int32_t* id = (int32_t*)malloc(sizeof(int32_t) * (size_t)(U > 0 ? U : 1));
            for (int64_t j = 0; j < U; ++j) {
                if (j < K - 1) {
                    u[j] = init_state ? init_state[(b * C + c) * (K - 1) + j] : 0.0;
                    id[j] = (seq_idx && L > 0) ? seq_idx[b * L + 0] : 0;
                } else {
                    u[j] = x[(b * L + (j - (K - 1))) * C + c];
                    id[j] = seq_idx ? seq_idx[b * L + (j - (K - 1))] : 0;
                }
            }
            for (int64_t t = 0; t < L; ++t) {
                double z = bias ? bias[c] : 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    if (seq_idx && id[t + k] != id[t + K - 1]) continue;
                    z += w[c * K + k] * u[t + k];
                }
                out[(b * L + t) * C + c] = orc_round(act_apply(z, act), out_round);
            }
            if (final_state) {
                for (int64_t r = 0; r < K - 1; ++r)
                    final_state[(b * C + c) * (K - 1) + r] = u[L + r];
            }
            free(u);
            free(id);
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------------------------
 * Decode update of the conv state ([CC] "single-token update maths", "the physical cache
 * may exceed the minimal history", "state indices for continuous batching").
 *
 * Row b uses pool slot s = indices[b] (or b).  A slot outside [0, n_slots) is skipped and
 * its output row is zero-filled.
 *
 * The K-1 history values are read from the pool BEFORE anything is written:
 *   circular (cache_seqlens given, p = cache_seqlens[b]):
 *       history j (j = 1 .. K-1 steps back) sits in slot floor_mod(p - j, state_len);
 *       new token i is written to slot floor_mod(p + i, state_len);
 *   linear (cache_seqlens NULL): the row holds the newest state_len inputs, oldest first;
 *       the history is its last K-1 entries; afterwards the row becomes the last state_len
 *       entries of (old row ++ new tokens).
 * Outputs follow the extended-sequence definition over [history, new tokens]; the pool
 * stores the raw inputs x (never the outputs).  cache_seqlens is read, never advanced.
 *
 * Layouts: x, out [B][C][L_new]; pool [n_slots][C][state_len]; w [C][K].
 * ------------------------------------------------------------------------------------- */
int orc_conv1d_update(const double* x, double* pool, const double* w, const double* bias,
                      const int32_t* indices, const int32_t* cache_seqlens, double* out,
                      int64_t B, int64_t C, int64_t L_new, int64_t K, int64_t state_len,
                      int64_t n_slots, int act, int out_round) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t c = 0; c < C; ++c) {
            const int64_t s = indices ? (int64_t)indices[b] : b;
            double* o = out + (b * C + c) * L_new;
            if (s < 0 || s >= n_slots) {
                for (int64_t i = 0; i < L_new; ++i) o[i] = 0.0;
                continue;
            }
            double* row = pool + (s * C + c) * state_len;
            const double* xr = x + (b * C + c) * L_new;
            const int64_t U = K - 1 + L_new;
            double* u = (double*)malloc(sizeof(double) * (size_t)U);
            /* u[0 .. K-2] = history oldest -> newest; u[K-1 ..] = new tokens */
            for (int64_t j = 1; j <= K - 1; ++j) {
                double h;
                if (cache_seqlens) {
                    const int64_t p = cache_seqlens[b];
                    h = row[floor_mod(p - j, state_len)];
                } else {
                    h = row[state_len - j];
                }
                u[K - 1 - j] = h;
            }
            for (int64_t i = 0; i < L_new; ++i) u[K - 1 + i] = xr[i];
            for (int64_t i = 0; i < L_new; ++i) {
                double z = bias ? bias[c] : 0.0;
                for (int64_t k = 0; k < K; ++k) z += w[c * K + k] * u[i + k];
                o[i] = orc_round(act_apply(z, act), out_round);
            }
            /* write the raw new inputs into the cache */
            if (cache_seqlens) {
                const int64_t p = cache_seqlens[b];
                for (int64_t i = 0; i < L_new; ++i) row[floor_mod(p + i, state_len)] = xr[i];
            } else {
                const int64_t total = state_len + L_new;
                double* ext = (double*)malloc(sizeof(double) * (size_t)total);
                for (int64_t i = 0; i < state_len; ++i) ext[i] = row[i];
                for (int64_t i = 0; i < L_new; ++i) ext[state_len + i] = xr[i];
                for (int64_t i = 0; i < state_len; ++i) row[i] = ext[total - state_len + i];
                free(ext);
            }
            free(u);
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------------------------
 * Selective scan with initial state in and final state out ([LG] Sec. 2.1 Eq. (1),
 * Sec. 2.5 Eq. (4), Sec. 2.6).  For every (b, h), with g = h / (H / G):
 *
 *   state[p][n] = h_{-1}[b][h][p][n]  (0 if absent)
 *   for t:  (state = 0 where seq_idx[b][t] != seq_idx[b][t-1], t > 0)
 *           a = exp(dt[b][t][h] * A[h])
 *           state[p][n] = a * state[p][n] + dt[b][t][h] * x[b][t][h][p] * Bm[b][t][g][n]
 *           y[b][t][h][p] = round(sum_n Cm[b][t][g][n] * state[p][n])
 *   final_state = round(state)
 *
 * Layouts: x, y [B][L][H][P]; dt [B][L][H]; A [H]; Bm, Cm [B][L][G][N];
 * init_state, final_state [B][H][P][N]; seq_idx [B][L].
 * ------------------------------------------------------------------------------------- */
int orc_scan_fwd(const double* x, const double* dt, const double* A, const double* Bm,
                 const double* Cm, const double* init_state, double* final_state,
                 const int32_t* seq_idx, double* y, int64_t B, int64_t L, int64_t H,
                 int64_t P, int64_t G, int64_t N, int y_round, int state_round) {
    const int64_t heads_per_group = H / G;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t h = 0; h < H; ++h) {
            const int64_t g = h / heads_per_group;
            double* st = (double*)malloc(sizeof(double) * (size_t)(P * N));
            for (int64_t e = 0; e < P * N; ++e)
                st[e] = init_state ? init_state[(b * H + h) * P * N + e] : 0.0;
            for (int64_t t = 0; t < L; ++t) {
                if (seq_idx && t > 0 && seq_idx[b * L + t] != seq_idx[b * L + t - 1])
                    for (int64_t e = 0; e < P * N; ++e) st[e] = 0.0;
                const double d = dt[(b * L + t) * H + h];
                const double a = exp(d * A[h]);
                const double* xt = x + ((b * L + t) * H + h) * P;
                const double* Bt = Bm + ((b * L + t) * G + g) * N;
                const double* Ct = Cm + ((b * L + t) * G + g) * N;
                for (int64_t p = 0; p < P; ++p) {
                    double acc = 0.0;
                    for (int64_t n = 0; n < N; ++n) {
                        st[p * N + n] = a * st[p * N + n] + d * xt[p] * Bt[n];
                        acc += Ct[n] * st[p * N + n];
                    }
                    y[((b * L + t) * H + h) * P + p] = orc_round(acc, y_round);
                }
            }
            if (final_state)
                for (int64_t e = 0; e < P * N; ++e)
                    final_state[(b * H + h) * P * N + e] = orc_round(st[e], state_round);
            free(st);
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------------------------
 * Decode step of the scan on a state pool: the same recurrence as orc_scan_fwd, token by
 * token over the L_new new tokens of request b, on pool slot s = indices[b] (or b).  The
 * state is carried in double precision across the L_new tokens of one call and stored back
 * rounded (state_round) at the end.  A slot outside [0, n_slots) is skipped and its y rows
 * are zero-filled; the pool is left untouched for it.
 *
 * Layouts: x, y [B][L_new][H][P]; dt [B][L_new][H]; Bm, Cm [B][L_new][G][N];
 * pool [n_slots][H][P][N].
 * ------------------------------------------------------------------------------------- */
int orc_step(const double* x, const double* dt, const double* A, const double* Bm,
             const double* Cm, double* pool, const int32_t* indices, double* y, int64_t B,
             int64_t L_new, int64_t H, int64_t P, int64_t G, int64_t N, int64_t n_slots,
             int y_round, int state_round) {
    const int64_t heads_per_group = H / G;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t h = 0; h < H; ++h) {
            const int64_t s = indices ? (int64_t)indices[b] : b;
            if (s < 0 || s >= n_slots) {
                for (int64_t t = 0; t < L_new; ++t)
                    for (int64_t p = 0; p < P; ++p) y[((b * L_new + t) * H + h) * P + p] = 0.0;
                continue;
            }
            const int64_t g = h / heads_per_group;
            double* st = pool + (s * H + h) * P * N;
            for (int64_t t = 0; t < L_new; ++t) {
                const double d = dt[(b * L_new + t) * H + h];
                const double a = exp(d * A[h]);
                const double* xt = x + ((b * L_new + t) * H + h) * P;
                const double* Bt = Bm + ((b * L_new + t) * G + g) * N;
                const double* Ct = Cm + ((b * L_new + t) * G + g) * N;
                for (int64_t p = 0; p < P; ++p) {
                    double acc = 0.0;
                    for (int64_t n = 0; n < N; ++n) {
                        st[p * N + n] = a * st[p * N + n] + d * xt[p] * Bt[n];
                        acc += Ct[n] * st[p * N + n];
                    }
                    y[((b * L_new + t) * H + h) * P + p] = orc_round(acc, y_round);
                }
            }
            for (int64_t e = 0; e < P * N; ++e) st[e] = orc_round(st[e], state_round);
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------------------------
 * Backward of the causal conv1d with state gradients ([CC] "backward with states, a unified
 * derivation"; "chunked training and truncated back-propagation").
 *
 * The loss depends on the outputs out_t = phi(z_t) (gradient dy_t) and on the final state F
 * (gradient q = dF).  With delta_t = dL/dz_t = dy_t * phi'(z_t) (the chain rule through phi;
 * phi' = 1 for the identity, sigma(z)(1 + z(1 - sigma(z))) for SiLU):
 *
 *   du_j = sum_t sum_k delta_t w_k [j = t + k] + [L <= j < L+K-1] q_{j-L}
 *   dS = du[0 : K-1],   dx = du[K-1 : K-1+L]
 *   dw_k = sum_{b,t} delta_t u_{t+k},   dbeta = sum_{b,t} delta_t
 *
 * With seq_idx, tap k of output t enters exactly where it entered the forward (same token
 * identity as output t); the direct path from F to the last K-1 inputs is unmasked, as F is.
 * z is recomputed from x, S, w, beta.  dw and dbeta sum over the batch (rows share weights).
 *
 * Layouts: x, dy, dx [B][L][C]; w, dw [C][K]; bias, dbias [C]; init_state, dfinal, dinit
 * [B][C][K-1]; seq_idx [B][L].  dfinal and init_state may be NULL (zero).
 * ------------------------------------------------------------------------------------- */
int orc_conv1d_bwd(const double* x, const double* w, const double* bias,
                   const double* init_state, const int32_t* seq_idx, const double* dy,
                   const double* dfinal, double* dx, double* dinit, double* dw, double* dbias,
                   int64_t B, int64_t L, int64_t C, int64_t K, int act, int dx_round,
                   int dstate_round, int dw_round) {
    const int64_t U = K - 1 + L;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < C; ++c) {
        const size_t nu = (size_t)(U > 0 ? U : 1);
        double* ext = (double*)malloc(sizeof(double) * nu);    /* u, the extended sequence */
        double* dext = (double*)malloc(sizeof(double) * nu);   /* dL/du */
        double* dz = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));  /* delta */
        int32_t* seg = (int32_t*)malloc(sizeof(int32_t) * nu); /* token identity of u_j */
        double* dwc = (double*)calloc((size_t)K, sizeof(double));
        double dbc = 0.0;
        for (int64_t b = 0; b < B; ++b) {
            const int32_t* sq = seq_idx ? seq_idx + b * L : NULL;
            for (int64_t j = 0; j < U; ++j) {
                const int64_t tx = j - (K - 1); /* token of u_j; < 0 for the state */
                ext[j] = tx < 0 ? (init_state ? init_state[(b * C + c) * (K - 1) + j] : 0.0)
                                : x[(b * L + tx) * C + c];
                seg[j] = sq ? sq[tx < 0 ? 0 : tx] : 0;
                dext[j] = 0.0;
            }
            /* delta_t = dy_t phi'(z_t), z_t recomputed with the forward's taps */
            for (int64_t t = 0; t < L; ++t) {
                double zt = bias ? bias[c] : 0.0;
                for (int64_t k = 0; k < K; ++k)
                    if (!sq || seg[t + k] == seg[t + K - 1]) zt += w[c * K + k] * ext[t + k];
                double dphi = 1.0;
                if (act == ORC_ACT_SILU) {
                    const double sg = 1.0 / (1.0 + exp(-zt));
                    dphi = sg * (1.0 + zt * (1.0 - sg));
                }
                dz[t] = dy[(b * L + t) * C + c] * dphi;
            }
            /* the convolution term of du, the weight and bias sums, then the direct path
             * from F to the last K-1 inputs */
            for (int64_t t = 0; t < L; ++t) {
                for (int64_t k = 0; k < K; ++k) {
                    if (sq && seg[t + k] != seg[t + K - 1]) continue;
                    dext[t + k] += dz[t] * w[c * K + k];
                    dwc[k] += dz[t] * ext[t + k];
                }
                dbc += dz[t];
            }
            if (dfinal)
                for (int64_t r = 0; r < K - 1; ++r) dext[L + r] += dfinal[(b * C + c) * (K - 1) + r];
            if (dinit)
                for (int64_t j = 0; j < K - 1; ++j)
                    dinit[(b * C + c) * (K - 1) + j] = orc_round(dext[j], dstate_round);
            for (int64_t t = 0; t < L; ++t)
                dx[(b * L + t) * C + c] = orc_round(dext[K - 1 + t], dx_round);
        }
        if (dw)
            for (int64_t k = 0; k < K; ++k) dw[c * K + k] = orc_round(dwc[k], dw_round);
        if (dbias) dbias[c] = orc_round(dbc, dw_round);
        free(ext);
        free(dext);
        free(dz);
        free(seg);
        free(dwc);
    }
    return 0;
}

/* ---------------------------------------------------------------------------------------
 * Gradient of the loss with respect to the scan's initial state ([LG] Sec. 2.5 Eq. (4), the
 * unrolled form with a non-zero initial state; Sec. 2.6, the state handed between chunks).
 *
 * h_{-1} enters y_t only through C_t^T (prod_{tau=0..t} a_tau) h_{-1}, and the final state
 * through (prod_{tau=0..L-1} a_tau) h_{-1}.  With dy (gradient of y) and dF (gradient of the
 * final state), per head h and channel p:
 *
 *   dh_{-1}[p][n] = sum_t dy_t[p] (prod_{tau<=t} a_tau) C_t[n]  +  (prod_{tau<L} a_tau) dF[p][n]
 *
 * a_tau = exp(dt_tau A_h).  With seq_idx the state is zeroed where the id changes, so only
 * tokens before the first change see h_{-1}, and dF reaches it only without any change.
 * The products are taken in time order, as the definition reads.
 *
 * Layouts: dt [B][L][H]; Cm [B][L][G][N]; dy [B][L][H][P]; dfinal, dh0 [B][H][P][N];
 * seq_idx [B][L].  dfinal may be NULL (zero).
 * ------------------------------------------------------------------------------------- */
int orc_scan_bwd_h0(const double* dt, const double* A, const double* Cm,
                    const int32_t* seq_idx, const double* dy, const double* dfinal, double* dh0,
                    int64_t B, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N,
                    int out_round) {
    const int64_t heads_per_group = H / G;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t h = 0; h < H; ++h) {
            const int64_t g = h / heads_per_group;
            double* acc = (double*)calloc((size_t)(P * N), sizeof(double));
            double prod = 1.0;
            int alive = 1;
            const int32_t* sq = seq_idx ? seq_idx + b * L : NULL;
            for (int64_t t = 0; t < L && alive; ++t) {
                if (sq && t > 0 && sq[t] != sq[t - 1]) {
                    alive = 0;
                    break;
                }
                prod *= exp(dt[(b * L + t) * H + h] * A[h]);
                const double* Ct = Cm + ((b * L + t) * G + g) * N;
                const double* dyt = dy + ((b * L + t) * H + h) * P;
                for (int64_t p = 0; p < P; ++p)
                    for (int64_t n = 0; n < N; ++n) acc[p * N + n] += dyt[p] * prod * Ct[n];
            }
            for (int64_t e = 0; e < P * N; ++e) {
                double v = acc[e];
                if (alive && dfinal) v += prod * dfinal[(b * H + h) * P * N + e];
                dh0[(b * H + h) * P * N + e] = orc_round(v, out_round);
            }
            free(acc);
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------------------------
 * Initial-state distributions for training ([LG] Sec. 2.6, the table of four interventions,
 * the Fitted Noise update Eqs. (5)-(6) and the State Passing procedure).
 *
 * Random numbers come from Philox4x64-10, the counter-based generator of Salmon, Moraes,
 * Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC 2011): a 256-bit counter
 * and a 128-bit key pass through ten rounds; each round multiplies counter words 0 and 2 by
 * fixed odd constants, keeps the 128-bit products' high and low halves, and mixes the high
 * halves with the other counter words and the round key; the key advances by fixed Weyl
 * increments between rounds.  Streams used here:
 *   key = (seed, purpose), counter = (block, offset, 0, 0); purpose 0 draws the Gaussian
 *   noise, purpose 1 the State Passing reset decisions.
 * ------------------------------------------------------------------------------------- */
#define ORC_PHILOX_M0 0xD2E7470EE14C6C93ULL
#define ORC_PHILOX_M1 0xCA5A826395121157ULL
#define ORC_PHILOX_W0 0x9E3779B97F4A7C15ULL
#define ORC_PHILOX_W1 0xBB67AE8584CAA73BULL

void orc_philox4x64_10(const uint64_t ctr_in[4], const uint64_t key_in[2], uint64_t out[4]) {
    uint64_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint64_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) { /* the key schedule: bumped before every round after the first */
            k0 += ORC_PHILOX_W0;
            k1 += ORC_PHILOX_W1;
        }
        const unsigned __int128 p0 = (unsigned __int128)ORC_PHILOX_M0 * c0;
        const unsigned __int128 p1 = (unsigned __int128)ORC_PHILOX_M1 * c2;
        const uint64_t hi0 = (uint64_t)(p0 >> 64), lo0 = (uint64_t)p0;
        const uint64_t hi1 = (uint64_t)(p1 >> 64), lo1 = (uint64_t)p1;
        c0 = hi1 ^ c1 ^ k0;
        c1 = lo1;
        c2 = hi0 ^ c3 ^ k1;
        c3 = lo0;
    }
    out[0] = c0;
    out[1] = c1;
    out[2] = c2;
    out[3] = c3;
}

/* Box-Muller: two uniforms u1 in (0, 1], u2 in [0, 1) give two independent standard normals
 * r cos(2 pi u2) and r sin(2 pi u2), r = sqrt(-2 ln u1). */
void orc_box_muller(double u1, double u2, double out[2]) {
    const double two_pi = 2.0 * acos(-1.0);
    const double r = sqrt(-2.0 * log(u1));
    out[0] = r * cos(two_pi * u2);
    out[1] = r * sin(two_pi * u2);
}

/* The standard normal of flat element e: block e / 8 of the purpose-0 stream gives four
 * pairs, pair j = (e % 8) / 2 from word j: u1 = (bits 40-63 + 1) 2^-24, u2 = (bits 8-31)
 * 2^-24 (24 bits from each 32-bit half; both exact in fp32); the cosine branch for even e
 * and the sine branch for odd e. */
static double standard_normal(uint64_t seed, uint64_t offset, int64_t e) {
    const uint64_t ctr[4] = {(uint64_t)(e / 8), offset, 0, 0};
    const uint64_t key[2] = {seed, 0};
    uint64_t w[4];
    orc_philox4x64_10(ctr, key, w);
    const uint64_t word = w[(e % 8) / 2];
    const double u1 = ((double)(word >> 40) + 1.0) * 0x1p-24;
    const double u2 = (double)((word >> 8) & 0xFFFFFFu) * 0x1p-24;
    double z[2];
    orc_box_muller(u1, u2, z);
    return z[e % 2];
}

/* Fitted Noise statistics ([LG] Sec. 2.6, Eqs. (5)-(6)): per head h,
 *   mean[h] <- (1 - beta) Mean(h_T) + beta mean[h],  var[h] <- (1 - beta) Variance(h_T) + beta var[h],
 * with Mean and Variance taken over the head's channels and state dimension (and, reading,
 * over the batch rows), Variance the population variance (mean squared deviation).  The new
 * batch's statistics carry weight 1 - beta.  final_state [B][H][P][N]; mean, var [H] in/out. */
int orc_state_stats_update(const double* fin, int64_t B, int64_t H, int64_t P, int64_t N,
                           double beta, double* mean, double* var, int out_round) {
    const int64_t per = P * N;
    const double count = (double)(B * per);
    for (int64_t h = 0; h < H; ++h) {
        double s = 0.0;
        for (int64_t b = 0; b < B; ++b)
            for (int64_t e = 0; e < per; ++e) s += fin[(b * H + h) * per + e];
        const double m = s / count;
        double ss = 0.0;
        for (int64_t b = 0; b < B; ++b)
            for (int64_t e = 0; e < per; ++e) {
                const double d = fin[(b * H + h) * per + e] - m;
                ss += d * d;
            }
        const double v = ss / count;
        mean[h] = orc_round((1.0 - beta) * m + beta * mean[h], out_round);
        var[h] = orc_round((1.0 - beta) * v + beta * var[h], out_round);
    }
    return 0;
}

/* Noise initial states ([LG] Sec. 2.6): Fitted Noise draws every element of head h
 * independently from N(mean[h], var[h]); Random Noise (mean == NULL) from N(0, sigma^2).
 * out [B][H][P][N]. */
int orc_initial_state_noise(double* out, int64_t B, int64_t H, int64_t P, int64_t N,
                            const double* mean, const double* var, double sigma, uint64_t seed,
                            uint64_t offset, int out_round) {
    const int64_t per = P * N;
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < B * H * per; ++e) {
        const int64_t h = (e / per) % H;
        const double z = standard_normal(seed, offset, e);
        const double v = mean ? mean[h] + sqrt(var[h]) * z : sigma * z;
        out[e] = orc_round(v, out_round);
    }
    return 0;
}

/* State Passing's occasional reset ([LG] Sec. 2.6): the carried state of row b is zeroed
 * with probability p, decided by word b % 4 of block b / 4 of the purpose-1 stream: zero iff
 * its top 32 bits are below floor(p 2^32).  Other rows are copied.  src, dst [B][per];
 * mask [B] receives 1 for a zeroed row. */
int orc_state_reset(const double* src, double* dst, uint8_t* mask, int64_t B, int64_t per,
                    double p, uint64_t seed, uint64_t offset) {
    double t = floor(p * 4294967296.0);
    if (t < 0.0) t = 0.0;
    if (t > 4294967296.0) t = 4294967296.0;
    const uint64_t threshold = (uint64_t)t;
    for (int64_t b = 0; b < B; ++b) {
        const uint64_t ctr[4] = {(uint64_t)(b / 4), offset, 0, 0};
        const uint64_t key[2] = {seed, 1};
        uint64_t w[4];
        orc_philox4x64_10(ctr, key, w);
        const int zero = (w[b % 4] >> 32) < threshold;
        mask[b] = (uint8_t)zero;
        for (int64_t e = 0; e < per; ++e) dst[b * per + e] = zero ? 0.0 : src[b * per + e];
    }
    return 0;
}

/* ---------------------------------------------------------------------------------------
 * Selective scan with a diagonal (per-state-dimension) transition ([LG] Sec. 2.1 Eq. (1)
 * with A_t = diag(a_t); Sec. 2.5: the diagonal case, its transition taken from log
 * coefficients).  For every (b, h), with g = h / (H / G), per state dimension n:
 *
 *   log a_t[n] = log_decay[b][t][h][n]       when log_decay is given (data-dependent gates),
 *              = dt[b][t][h] * A_vec[h][n]    otherwise (a fixed rate per state dimension);
 *   u_t = dt[b][t][h] (1 when dt is NULL)
 *   state[p][n] = a_t[n] state[p][n] + u_t x[b][t][h][p] Bm[b][t][g][n]
 *   y[b][t][h][p] = round(sum_n Cm[b][t][g][n] state[p][n])
 *
 * from h_{-1} (0 if absent), zeroed where seq_idx changes, final state returned.
 * Layouts as orc_scan_fwd; log_decay [B][L][H][N]; A_vec [H][N].
 * ------------------------------------------------------------------------------------- */
int orc_scan_fwd_vdecay(const double* x, const double* dt, const double* log_decay,
                        const double* A_vec, const double* Bm, const double* Cm,
                        const double* init_state, double* final_state, const int32_t* seq_idx,
                        double* y, int64_t B, int64_t L, int64_t H, int64_t P, int64_t G,
                        int64_t N, int y_round, int state_round) {
    const int64_t heads_per_group = H / G;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t h = 0; h < H; ++h) {
            const int64_t grp = h / heads_per_group;
            double* hs = (double*)malloc(sizeof(double) * (size_t)(P * N));
            double* an = (double*)malloc(sizeof(double) * (size_t)N);
            const int32_t* row_ids = seq_idx ? seq_idx + b * L : NULL;
            for (int64_t e = 0; e < P * N; ++e)
                hs[e] = init_state ? init_state[(b * H + h) * P * N + e] : 0.0;
            for (int64_t t = 0; t < L; ++t) {
                if (row_ids && t > 0 && row_ids[t] != row_ids[t - 1])
                    for (int64_t e = 0; e < P * N; ++e) hs[e] = 0.0;
                const double u = dt ? dt[(b * L + t) * H + h] : 1.0;
                for (int64_t n = 0; n < N; ++n)
                    an[n] = log_decay ? exp(log_decay[((b * L + t) * H + h) * N + n])
                                      : exp(u * A_vec[h * N + n]);
                const double* xt = x + ((b * L + t) * H + h) * P;
                const double* Bt = Bm + ((b * L + t) * G + grp) * N;
                const double* Ct = Cm + ((b * L + t) * G + grp) * N;
                for (int64_t p = 0; p < P; ++p) {
                    double out = 0.0;
                    for (int64_t n = 0; n < N; ++n) {
                        hs[p * N + n] = an[n] * hs[p * N + n] + u * xt[p] * Bt[n];
                        out += Ct[n] * hs[p * N + n];
                    }
                    y[((b * L + t) * H + h) * P + p] = orc_round(out, y_round);
                }
            }
            if (final_state)
                for (int64_t e = 0; e < P * N; ++e)
                    final_state[(b * H + h) * P * N + e] = orc_round(hs[e], state_round);
            free(an);
            free(hs);
        }
    }
    return 0;
}

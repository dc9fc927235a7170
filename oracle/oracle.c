/*
 * CPU oracle for the DFlash 2 path selector.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library.  The GPU
 * product path never calls it, and it shares no code with the GPU path.
 *
 * Everything here is the plain definition of each step, in float64, written
 * for a reader to check against the pages by eye:
 *
 *   "DFlash 2: Keep Drafting Parallel", section "A Lightweight Path Selector":
 *     - keep the top 16 candidates at each draft position;
 *     - score every adjacent pair (predecessor a, current candidate b) with
 *       the selector equation  S_t(a,b) = U_t(b) + < A(a) (.) H(h_t), B(b) >,
 *       where U_t is the drafter's own logit, A and B are 256-dimensional
 *       token embeddings and H(h_t) is a gate computed from the drafter's
 *       hidden state;
 *     - the only sequential work is one walk over the precomputed scores,
 *       starting from the last verified token.
 *
 * Readings taken where the pages are silent or truncated:
 *   - H(h_t) is a linear map d -> r without bias or activation:
 *       H[q] = sum_m W_H[q][m] * h_t[m]           (W_H stored [r][d]).
 *   - The walk is a max-sum (Viterbi) pass plus backtrack over the
 *     candidate lattice; the predecessor of the first draft position is the
 *     last verified token prev_tok.  The literal left-to-right greedy walk
 *     (orc_greedy) and the sampling walk (orc_sample: inverse-CDF draws from
 *     the softmax of each step's scores, uniforms supplied by the caller)
 *     are kept beside it as further walk modes.
 *   - Top-K order is value descending; equal values (IEEE equality, so
 *     -0 == +0) go to the lower vocabulary index.
 *   - Viterbi ties go to the smaller predecessor rank; the final pick goes
 *     to the smaller rank.
 *   - U_t(b) is the raw logit.
 *
 * The drafter's two-tap convolution (orc_conv2, section "A Lightweight Local
 * Convolution") and its LM head followed by top-K (orc_lmhead_topk, the
 * logits the selector starts from) are here too, and so is the counter-based
 * generator of the sampling walk's uniforms (orc_philox_uniforms,
 * Philox4x64-10); their readings are stated beside them.
 *
 * Parity pins (checked by the CPU test suite, not by this file): brute-force
 * enumeration of all K^P paths on tiny inputs, zeroed pair term reducing to
 * independent top-1 picks, K = 1 and P = 1 closed forms, exact integer
 * fixtures, logit-shift invariance, an independent lexicographic sort for
 * top-K, and numpy's Philox plus the published known answer for the
 * generator.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    double v;
    int32_t i;
} orc_item;

/* Order: larger value first; for equal values the lower index first. */
static int orc_item_cmp(const void* pa, const void* pb) {
    const orc_item* a = (const orc_item*)pa;
    const orc_item* b = (const orc_item*)pb;
    if (a->v > b->v) return -1;
    if (a->v < b->v) return 1;
    if (a->i < b->i) return -1;
    if (a->i > b->i) return 1;
    return 0;
}

/*
 * Top-K per row: sort the whole row and keep the first K entries
 * (section "A Lightweight Path Selector": top 16 candidates per position).
 *   x    [rows][V]   logits, already widened exactly to float64
 *   idx  [rows][K]   vocabulary index of the k-th best candidate
 *   val  [rows][K]   its logit U_t
 * Returns 0, or -1 on allocation failure / bad sizes.
 */
int orc_topk(const double* x, int64_t rows, int64_t V, int32_t K,
             int32_t* idx, double* val) {
    if (K < 1 || K > V) return -1;
    orc_item* items = (orc_item*)malloc(sizeof(orc_item) * (size_t)V);
    if (!items) return -1;
    for (int64_t row = 0; row < rows; ++row) {
        const double* xr = x + row * V;
        for (int64_t v = 0; v < V; ++v) {
            items[v].v = xr[v];
            items[v].i = (int32_t)v;
        }
        qsort(items, (size_t)V, sizeof(orc_item), orc_item_cmp);
        for (int32_t k = 0; k < K; ++k) {
            idx[row * K + k] = items[k].i;
            val[row * K + k] = items[k].v;
        }
    }
    free(items);
    return 0;
}

/*
 * Gate projection H = W_H h for every (sequence, position) row.
 *   h  [M][d], W [r][d], H [M][r]
 */
void orc_project(const double* h, const double* W, int64_t M, int64_t d,
                 int64_t r, double* H) {
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t q = 0; q < r; ++q) {
            double acc = 0.0;
            for (int64_t k = 0; k < d; ++k) acc += W[q * d + k] * h[m * d + k];
            H[m * r + q] = acc;
        }
    }
}

/*
 * The drafter's LM head followed by top-K, the upstream step the selector
 * consumes ("DFlash 2: Keep Drafting Parallel", section "A Lightweight Path
 * Selector": the selector works on the drafter's own logits and needs no
 * extra LM-head pass).  Read as a bias-free linear map of the drafter's
 * final hidden state onto the vocabulary:
 *     U_t(v) = sum_k W_lm[v][k] * h_t[k]
 * and then the same top-K order as orc_topk (value descending, equal values
 * to the lower index).
 *   X      [M][d]  hidden states (float storage of exact bf16/fp32 values)
 *   W      [V][d]  LM-head weight, one row per token
 *   idx    [M][K]  token id of the k-th best logit
 *   val    [M][K]  that logit, every product and sum in float64
 *   sigma  [M][K]  sum_k |W[v][k] h[k]| of that logit (scale for tolerances)
 * Returns 0, or -1 on bad sizes or allocation failure.
 */
int orc_lmhead_topk(const float* X, const float* W, int64_t M, int64_t d,
                    int64_t V, int32_t K, int32_t* idx, double* val,
                    double* sigma) {
    if (K < 1 || K > V || d < 1) return -1;
    double* logit = (double*)malloc(sizeof(double) * (size_t)V);
    double* row_val = (double*)malloc(sizeof(double) * (size_t)K);
    if (!logit || !row_val) {
        free(logit);
        free(row_val);
        return -1;
    }
    int rc = 0;
    for (int64_t m = 0; m < M && rc == 0; ++m) {
        const float* x = X + m * d;
        for (int64_t v = 0; v < V; ++v) {
            const float* w = W + v * d;
            double acc = 0.0;
            for (int64_t k = 0; k < d; ++k) acc += (double)w[k] * (double)x[k];
            logit[v] = acc;
        }
        rc = orc_topk(logit, 1, V, K, idx + m * K, row_val);
        for (int32_t j = 0; j < K && rc == 0; ++j) {
            const float* w = W + (int64_t)idx[m * K + j] * d;
            double s = 0.0;
            for (int64_t k = 0; k < d; ++k) s += fabs((double)w[k] * (double)x[k]);
            val[m * K + j] = row_val[j];
            sigma[m * K + j] = s;
        }
    }
    free(logit);
    free(row_val);
    return rc;
}

/*
 * Single LM-head logits for n given (row, token) pairs, with their scale:
 *   dot[i]   = sum_k W[v_i][k] * X[m_i][k]      (float64)
 *   absdot[i] = sum_k |W[v_i][k] * X[m_i][k]|
 */
void orc_lmhead_dot(const float* X, const float* W, int64_t d, const int64_t* m,
                    const int64_t* v, int64_t n, double* dot, double* absdot) {
    for (int64_t i = 0; i < n; ++i) {
        const float* x = X + m[i] * d;
        const float* w = W + v[i] * d;
        double acc = 0.0, s = 0.0;
        for (int64_t k = 0; k < d; ++k) {
            const double p = (double)w[k] * (double)x[k];
            acc += p;
            s += fabs(p);
        }
        dot[i] = acc;
        absdot[i] = s;
    }
}

/*
 * Pair scores, the selector equation of section "A Lightweight Path
 * Selector":  S_t(a, b) = U_t(b) + sum_q A[a][q] * H_t[q] * B[b][q].
 *
 *   cand  [Bn][P][K] candidate token ids (rank order)
 *   U     [Bn][P][K] their logits
 *   H     [Bn][P][r] gate vectors
 *   A, Bt [V][r]     token embeddings
 *   prev  [Bn]       last verified token per sequence
 *   S     [Bn][P][K][K]   S[b][t][i][j]: predecessor rank i, candidate rank j
 *   sigma [Bn][P][K][K]   |U| + sum_q |A H B|, the scale used for tolerances
 *
 * The predecessor of rank i at position t >= 1 is cand[b][t-1][i]; at t = 0
 * every row i uses prev[b] (only row 0 is meaningful; the rest repeat it).
 */
void orc_pair_scores(const int32_t* cand, const double* U, const double* H,
                     const double* A, const double* Bt, const int32_t* prev,
                     int64_t Bn, int64_t P, int64_t K, int64_t r,
                     double* S, double* sigma) {
    for (int64_t b = 0; b < Bn; ++b) {
        for (int64_t t = 0; t < P; ++t) {
            const double* Ht = H + (b * P + t) * r;
            for (int64_t i = 0; i < K; ++i) {
                int64_t a = (t == 0) ? prev[b] : cand[(b * P + (t - 1)) * K + i];
                for (int64_t j = 0; j < K; ++j) {
                    int64_t c = cand[(b * P + t) * K + j];
                    double u = U[(b * P + t) * K + j];
                    double dot = 0.0, mag = 0.0;
                    for (int64_t q = 0; q < r; ++q) {
                        double term = A[a * r + q] * Ht[q] * Bt[c * r + q];
                        dot += term;
                        mag += fabs(term);
                    }
                    int64_t o = ((b * P + t) * K + i) * K + j;
                    S[o] = u + dot;
                    if (sigma) sigma[o] = fabs(u) + mag;
                }
            }
        }
    }
}

/*
 * Max-sum walk over the candidate lattice with backtrack.
 *   delta_0[j] = S[b][0][0][j]
 *   delta_t[j] = max_i delta_{t-1}[i] + S[b][t][i][j]      (t = 1 .. P-1)
 *   psi_t[j]   = smallest i attaining that max
 *   j_{P-1}    = smallest j attaining max_j delta_{P-1}[j]
 *   j_{t-1}    = psi_t[j_t]
 * Outputs per sequence: rank path [P], token path [P] (cand[b][t][j_t]) and
 * the best score delta_{P-1}[j_{P-1}].
 * Returns 0, or -1 on allocation failure.
 */
int orc_viterbi(const double* S, const int32_t* cand, int64_t Bn, int64_t P,
                int64_t K, int32_t* path_rank, int32_t* path_tok, double* score) {
    double* delta = (double*)malloc(sizeof(double) * (size_t)(P * K));
    int32_t* psi = (int32_t*)malloc(sizeof(int32_t) * (size_t)(P * K));
    if (!delta || !psi) {
        free(delta);
        free(psi);
        return -1;
    }
    for (int64_t b = 0; b < Bn; ++b) {
        const double* Sb = S + b * P * K * K;
        for (int64_t j = 0; j < K; ++j) {
            delta[j] = Sb[j];           /* t = 0, row i = 0 */
            psi[j] = 0;
        }
        for (int64_t t = 1; t < P; ++t) {
            for (int64_t j = 0; j < K; ++j) {
                double best = delta[(t - 1) * K + 0] + Sb[(t * K + 0) * K + j];
                int32_t arg = 0;
                for (int64_t i = 1; i < K; ++i) {
                    double v = delta[(t - 1) * K + i] + Sb[(t * K + i) * K + j];
                    if (v > best) {
                        best = v;
                        arg = (int32_t)i;
                    }
                }
                delta[t * K + j] = best;
                psi[t * K + j] = arg;
            }
        }
        int32_t jb = 0;
        for (int64_t j = 1; j < K; ++j)
            if (delta[(P - 1) * K + j] > delta[(P - 1) * K + jb]) jb = (int32_t)j;
        score[b] = delta[(P - 1) * K + jb];
        int32_t j = jb;
        for (int64_t t = P - 1; t >= 0; --t) {
            path_rank[b * P + t] = j;
            path_tok[b * P + t] = cand[(b * P + t) * K + j];
            if (t > 0) j = psi[t * K + j];
        }
    }
    free(delta);
    free(psi);
    return 0;
}

/*
 * The greedy walk: the literal reading of "greedy follows the best successor
 * at each step" (same page and section).  Starting from the last verified
 * token, each position keeps the candidate whose pair score, given the token
 * just chosen, is largest:
 *   j_0 = argmax_j S[b][0][0][j]             (t = 0 predecessor is prev_tok)
 *   j_t = argmax_j S[b][t][j_{t-1}][j],      t >= 1
 *   score[b] = sum_t S[b][t][j_{t-1}][j_t]   (j_{-1} = row 0), summed from t = 0
 * Ties go to the smaller rank.  Outputs as for orc_viterbi.
 */
void orc_greedy(const double* S, const int32_t* cand, int64_t Bn, int64_t P,
                int64_t K, int32_t* path_rank, int32_t* path_tok, double* score) {
    for (int64_t b = 0; b < Bn; ++b) {
        const double* Sb = S + b * P * K * K;
        int64_t i = 0;                  /* rank of the predecessor */
        double total = 0.0;
        for (int64_t t = 0; t < P; ++t) {
            const double* row = Sb + (t * K + i) * K;
            int64_t jb = 0;
            for (int64_t j = 1; j < K; ++j)
                if (row[j] > row[jb]) jb = j;
            total += row[jb];
            path_rank[b * P + t] = (int32_t)jb;
            path_tok[b * P + t] = cand[(b * P + t) * K + jb];
            i = jb;
        }
        score[b] = total;
    }
}

/*
 * The sampling walk: "sampling draws from the same scores" (same page and
 * section), read as: from the last verified token, each position draws its
 * candidate from the softmax of the pair scores of the token just chosen,
 * at temperature tau, with the caller's uniform u[b][t] in [0, 1):
 *   q_t(j) = exp((S_t(i, j) - m) / tau) / sum_k exp((S_t(i, k) - m) / tau),
 *            m = max_k S_t(i, k), i = j_{t-1} (row 0 at t = 0)
 *   j_t    = the smallest j with u[b][t] < q_t(0) + ... + q_t(j)
 *            (if rounding leaves u above the last sum: the last j with
 *            q_t(j) > 0)
 * Outputs: ranks, tokens, prob[b][t] = q_t(j_t) (the draft probability that
 * rejection sampling needs), score[b] = sum_t S_t(j_{t-1}, j_t) from t = 0.
 * Returns 0, or -1 on allocation failure.
 */
int orc_sample(const double* S, const int32_t* cand, const double* u, int64_t Bn,
               int64_t P, int64_t K, double tau, int32_t* path_rank,
               int32_t* path_tok, double* prob, double* score) {
    double* q = (double*)malloc(sizeof(double) * (size_t)K);
    if (!q) return -1;
    for (int64_t b = 0; b < Bn; ++b) {
        const double* Sb = S + b * P * K * K;
        int64_t i = 0;
        double total = 0.0;
        for (int64_t t = 0; t < P; ++t) {
            const double* row = Sb + (t * K + i) * K;
            double m = row[0];
            for (int64_t j = 1; j < K; ++j)
                if (row[j] > m) m = row[j];
            double z = 0.0;
            for (int64_t j = 0; j < K; ++j) {
                q[j] = exp((row[j] - m) / tau);
                z += q[j];
            }
            for (int64_t j = 0; j < K; ++j) q[j] /= z;
            const double ub = u[b * P + t];
            int64_t pick = -1, last = 0;
            double cdf = 0.0;
            for (int64_t j = 0; j < K; ++j) {
                cdf += q[j];
                if (q[j] > 0.0) last = j;
                if (pick < 0 && ub < cdf) pick = j;
            }
            if (pick < 0) pick = last;
            total += row[pick];
            path_rank[b * P + t] = (int32_t)pick;
            path_tok[b * P + t] = cand[(b * P + t) * K + pick];
            prob[b * P + t] = q[pick];
            i = pick;
        }
        score[b] = total;
    }
    free(q);
    return 0;
}

/*
 * Best-versus-second path margin, from max-marginals.
 *   alpha_t = forward max-sum (delta above), beta_{P-1} = 0,
 *   beta_t[i] = max_j S[b][t+1][i][j] + beta_{t+1}[j],
 *   M_t[j] = alpha_t[j] + beta_t[j] = best score of a path through rank j at t.
 * Every path other than the best one leaves the best path's rank at some t,
 * so the second-best score is max over t and j != path_rank[t] of M_t[j].
 * second[b] = -inf when K == 1 (no other path).
 * Returns 0, or -1 on allocation failure.
 */
int orc_second_best(const double* S, const int32_t* path_rank, int64_t Bn,
                    int64_t P, int64_t K, double* second) {
    double* alpha = (double*)malloc(sizeof(double) * (size_t)(P * K));
    double* beta = (double*)malloc(sizeof(double) * (size_t)(P * K));
    if (!alpha || !beta) {
        free(alpha);
        free(beta);
        return -1;
    }
    for (int64_t b = 0; b < Bn; ++b) {
        const double* Sb = S + b * P * K * K;
        for (int64_t j = 0; j < K; ++j) alpha[j] = Sb[j];
        for (int64_t t = 1; t < P; ++t)
            for (int64_t j = 0; j < K; ++j) {
                double best = -INFINITY;
                for (int64_t i = 0; i < K; ++i) {
                    double v = alpha[(t - 1) * K + i] + Sb[(t * K + i) * K + j];
                    if (v > best) best = v;
                }
                alpha[t * K + j] = best;
            }
        for (int64_t j = 0; j < K; ++j) beta[(P - 1) * K + j] = 0.0;
        for (int64_t t = P - 2; t >= 0; --t)
            for (int64_t i = 0; i < K; ++i) {
                double best = -INFINITY;
                for (int64_t j = 0; j < K; ++j) {
                    double v = Sb[((t + 1) * K + i) * K + j] + beta[(t + 1) * K + j];
                    if (v > best) best = v;
                }
                beta[t * K + i] = best;
            }
        double sec = -INFINITY;
        for (int64_t t = 0; t < P; ++t)
            for (int64_t j = 0; j < K; ++j) {
                if (j == path_rank[b * P + t]) continue;
                double m = alpha[t * K + j] + beta[t * K + j];
                if (m > sec) sec = m;
            }
        second[b] = sec;
    }
    free(alpha);
    free(beta);
    return 0;
}

/*
 * Two-tap dynamic depthwise convolution ("DFlash 2: Keep Drafting Parallel",
 * section "A Lightweight Local Convolution", the equation for Conv_k):
 *   y_t[c] = k_{t,0}[c] * x_t[c] + k_{t,1}[c] * x_{t-1}[c]
 * with x_{-1} = x_prev (the last verified token's representation) and each
 * coefficient a learned base plus a correction from the current hidden state
 * shared by 16 consecutive channels.  Readings: the correction is a bias-free
 * linear map of x_t,
 *   corr_t[tap][g] = sum_m Wc[tap][g][m] * x_t[m],   g = 0 .. d/16 - 1,
 *   k_{t,tap}[c]   = base[tap][c] + corr_t[tap][c / 16].
 * x [Bn, P, d], x_prev [Bn, d], base [2, d], Wc [2, d/16, d], y [Bn, P, d];
 * sigma [Bn, P, d] gets the magnitude
 *   (|base0| + sum |Wc0 x|) |x_t| + (|base1| + sum |Wc1 x|) |x_{t-1}|
 * that scales the rounding error of any evaluation order.
 * d must be a multiple of 16.
 */
void orc_conv2(const double* x, const double* x_prev, const double* base, const double* Wc,
               int64_t Bn, int64_t P, int64_t d, double* y, double* sigma) {
    const int64_t G = d / 16;
    for (int64_t b = 0; b < Bn; ++b)
        for (int64_t t = 0; t < P; ++t) {
            const double* xt = x + (b * P + t) * d;
            const double* xp = (t == 0) ? x_prev + b * d : x + (b * P + t - 1) * d;
            double* yt = y + (b * P + t) * d;
            double* st = sigma + (b * P + t) * d;
            for (int64_t g = 0; g < G; ++g) {
                double corr[2], cmag[2];
                for (int tap = 0; tap < 2; ++tap) {
                    const double* w = Wc + ((int64_t)tap * G + g) * d;
                    double acc = 0.0, mag = 0.0;
                    for (int64_t m = 0; m < d; ++m) {
                        acc += w[m] * xt[m];
                        mag += fabs(w[m] * xt[m]);
                    }
                    corr[tap] = acc;
                    cmag[tap] = mag;
                }
                for (int64_t c = 16 * g; c < 16 * g + 16; ++c) {
                    const double k0 = base[c] + corr[0];
                    const double k1 = base[d + c] + corr[1];
                    yt[c] = k0 * xt[c] + k1 * xp[c];
                    st[c] = (fabs(base[c]) + cmag[0]) * fabs(xt[c]) +
                            (fabs(base[d + c]) + cmag[1]) * fabs(xp[c]);
                }
            }
        }
}

/*
 * Counter-based uniforms for the sampling walk (the selector's section:
 * sampling draws from the same scores, so each draft position needs one
 * uniform).  The generator is Philox4x64-10 as published by Salmon, Moraes,
 * Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC 2011):
 * a 4-word counter and a 2-word key; each of 10 rounds multiplies counter
 * words 0 and 2 by the two round multipliers, crosses the high and low
 * halves of the products with words 3 and 1 and the key, then bumps the key
 * by the two Weyl constants.
 *
 * Reading of how a draw maps onto the generator (the pages name none):
 * uniform i of a call with (seed, offset) is word (i mod 4) of the block at
 * counter (floor(i / 4), offset, 0, 0) under key (seed, 0), and the word x
 * becomes the float (x >> 40) * 2^-24, exact in fp32 and in [0, 1).
 */
static const uint64_t orc_philox_m0 = 0xD2E7470EE14C6C93ull;
static const uint64_t orc_philox_m1 = 0xCA5A826395121157ull;
static const uint64_t orc_philox_w0 = 0x9E3779B97F4A7C15ull;  /* golden ratio */
static const uint64_t orc_philox_w1 = 0xBB67AE8584CAA73Bull;  /* sqrt(3) - 1 */

void orc_philox4x64_10(const uint64_t ctr_in[4], const uint64_t key_in[2], uint64_t out[4]) {
    uint64_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint64_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        const unsigned __int128 p0 = (unsigned __int128)orc_philox_m0 * c0;
        const unsigned __int128 p1 = (unsigned __int128)orc_philox_m1 * c2;
        const uint64_t hi0 = (uint64_t)(p0 >> 64), lo0 = (uint64_t)p0;
        const uint64_t hi1 = (uint64_t)(p1 >> 64), lo1 = (uint64_t)p1;
        c0 = hi1 ^ c1 ^ k0;
        c1 = lo1;
        c2 = hi0 ^ c3 ^ k1;
        c3 = lo0;
        k0 += orc_philox_w0;
        k1 += orc_philox_w1;
    }
    out[0] = c0;
    out[1] = c1;
    out[2] = c2;
    out[3] = c3;
}

/* Uniforms first .. first + n - 1 of the call (seed, offset), as above. */
void orc_philox_uniforms(uint64_t seed, uint64_t offset, int64_t first, int64_t n, float* u) {
    const uint64_t key[2] = {seed, 0};
    for (int64_t k = 0; k < n; ++k) {
        const uint64_t i = (uint64_t)(first + k);
        const uint64_t ctr[4] = {i / 4, offset, 0, 0};
        uint64_t w[4];
        orc_philox4x64_10(ctr, key, w);
        u[k] = (float)((double)(w[i % 4] >> 40) * (1.0 / 16777216.0));
    }
}

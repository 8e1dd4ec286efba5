/*
 * Plain CPU oracle of the LongCat-Flash MoE layer forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the HIP library it checks.
 *
 * What it computes (LongCat-Flash Technical Report notes, "Key claims" and
 * "Method"; report §2.1, §2.2, §2.3.2, §2.4):
 *   - a router scores every expert of one pool that holds N SwiGLU FFN experts
 *     and Z zero-computation (identity) experts;
 *   - a per-expert bias, the quantity the PID controller adjusts from routing
 *     frequency (report §2.1.1), is added to the scores for selection only;
 *   - the K best keys are kept per token (K = 12 of 512 + 256 at full scale);
 *   - FFN experts' outputs are multiplied by the variance-compensation factor
 *     (report §2.3.2 Eq. 8, the "m*n" factor; one opaque scalar here);
 *   - zero-computation experts return their input;
 *   - the token's output is the gate-weighted sum of its K expert outputs
 *     (the "combine" half of dispatch/combine, report §2.2).
 * Readings taken where the pages are silent (softmax score, bias on the
 * logits, no gate renormalisation, SwiGLU form, ties to the lower expert id,
 * expert-major token-ascending row order) are listed with the build's design
 * notes.  They are "parity unpinned" against LongCat-Flash itself: the pages
 * print no router or expert formula.
 *
 * Precision: every accumulation runs in fp64 with sequential loops in index
 * order.  The one floating-point decision that yields integers (which K
 * experts a token keeps) is taken on fp32 keys = fp32 logit + fp32 bias, the
 * precision the GPU kernel decides in.
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math (no FTZ/DAZ, no reassociation).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>

/* ---- router scores -------------------------------------------------------
 * logits[t][e] = sum_h x[t][h] * wr[e][h]   (fp64, h ascending)
 * One score per expert of the whole pool, FFN and zero-computation experts
 * alike (K = 12 of 512 + 256 at full scale): Technical Report notes, Key
 * claims [§2.1, §2.4]. */
void oracle_router_logits(const float *x, const float *wr, int T, int H, int E,
                          double *logits)
{
    for (int t = 0; t < T; ++t) {
        const float *xr = x + (size_t)t * H;
        for (int e = 0; e < E; ++e) {
            const float *wrow = wr + (size_t)e * H;
            double acc = 0.0;
            for (int h = 0; h < H; ++h)
                acc += (double)xr[h] * (double)wrow[h];
            logits[(size_t)t * E + e] = acc;
        }
    }
}

/* ---- routing -------------------------------------------------------------
 * key[t][e] = logits32[t][e] + bias[e]       one fp32 addition
 * Top-K: K rounds, each taking the largest key not yet taken; a tie keeps the
 * smaller expert id (IEEE comparison, so -0.0 == +0.0; -inf is a valid key).
 * Slot order = the order of the rounds.
 * gate[t][k] = softmax over all E unbiased logits, read at the chosen expert;
 * no renormalisation over the K picks.  The bias only steers selection
 * (aux-loss-free lineage, Technical Report notes, Key claims [§2.1.1]).
 * counts[e] = number of tokens that chose e (the routing-frequency signal the
 * PID controller observes, same passage).
 * Returns 0, or -1 if any key is NaN (then outputs are unspecified). */
int oracle_route(const float *logits32, const float *bias, int T, int E, int K,
                 int32_t *idx, double *gate, int32_t *counts)
{
    float *key = (float *)malloc(sizeof(float) * (size_t)E);
    unsigned char *taken = (unsigned char *)malloc((size_t)E);
    int rc = 0;
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int t = 0; t < T; ++t) {
        const float *l = logits32 + (size_t)t * E;
        for (int e = 0; e < E; ++e) {
            key[e] = l[e] + bias[e];
            if (isnan(key[e])) rc = -1;
            taken[e] = 0;
        }
        /* softmax denominator over the unbiased logits, fp64 */
        double m = -INFINITY;
        for (int e = 0; e < E; ++e)
            if ((double)l[e] > m) m = (double)l[e];
        double den = 0.0;
        for (int e = 0; e < E; ++e) den += exp((double)l[e] - m);
        for (int k = 0; k < K; ++k) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || key[e] > key[best]) best = e;
            }
            taken[best] = 1;
            idx[(size_t)t * K + k] = best;
            gate[(size_t)t * K + k] = exp((double)l[best] - m) / den;
            counts[best] += 1;
        }
    }
    free(key);
    free(taken);
    return rc;
}

/* Softmax of the unbiased fp32 logits, fp64, read at given experts idx[t][k]
 * (the gate a token would get for any chosen set; same definition as above). */
void oracle_gates(const float *logits32, const int32_t *idx, int T, int E, int K,
                  double *gate)
{
    for (int t = 0; t < T; ++t) {
        const float *l = logits32 + (size_t)t * E;
        double m = -INFINITY;
        for (int e = 0; e < E; ++e)
            if ((double)l[e] > m) m = (double)l[e];
        double den = 0.0;
        for (int e = 0; e < E; ++e) den += exp((double)l[e] - m);
        for (int k = 0; k < K; ++k)
            gate[(size_t)t * K + k] =
                exp((double)l[idx[(size_t)t * K + k]] - m) / den;
    }
}

/* ---- dispatch as a local permutation --------------------------------------
 * The dispatch half of dispatch/combine (Technical Report notes, Key claims
 * [§2.2]) groups every FFN selection by expert.  Row order: expert-major and,
 * inside one expert, ascending token (a token picks an expert at most once,
 * so this order is unique).
 *   offsets[e] = first row of expert e, offsets[N] = S (number of FFN rows)
 *   row_src[r] = t*K + k of the selection held in row r
 *   slot_row[t*K + k] = its row, or -1 when it picked a zero expert (id >= N)
 * Returns S. */
int oracle_permute(const int32_t *idx, int T, int K, int N, int32_t *offsets,
                   int32_t *row_src, int32_t *slot_row)
{
    for (int s = 0; s < T * K; ++s) slot_row[s] = -1;
    int row = 0;
    for (int e = 0; e < N; ++e) {
        offsets[e] = row;
        for (int t = 0; t < T; ++t)
            for (int k = 0; k < K; ++k)
                if (idx[(size_t)t * K + k] == e) {
                    row_src[row] = t * K + k;
                    slot_row[(size_t)t * K + k] = row;
                    ++row;
                }
    }
    offsets[N] = row;
    return row;
}

/* ---- one FFN expert on one row ---------------------------------------------
 * SwiGLU expert with intermediate size I (per-expert FFN intermediate 2048 at
 * full scale, Technical Report notes, Key claims [§2.4]):
 *   a_j = sum_h x[h] * w13[j][h]          gate rows j = 0..I-1
 *   u_j = sum_h x[h] * w13[I + j][h]      up rows
 *   hh_j = a_j / (1 + exp(-a_j)) * u_j    silu(a) * u
 *   out[i] = sum_j hh_j * w2[i][j]        w2 is [H][I]
 * fp64 throughout. */
void oracle_ffn_row(const float *x, const float *w13, const float *w2, int H,
                    int I, double *out)
{
    double *hh = (double *)malloc(sizeof(double) * (size_t)I);
    for (int j = 0; j < I; ++j) {
        const float *g = w13 + (size_t)j * H;
        const float *u = w13 + (size_t)(I + j) * H;
        double a = 0.0, b = 0.0;
        for (int h = 0; h < H; ++h) {
            a += (double)x[h] * (double)g[h];
            b += (double)x[h] * (double)u[h];
        }
        hh[j] = a / (1.0 + exp(-a)) * b;
    }
    for (int i = 0; i < H; ++i) {
        const float *d = w2 + (size_t)i * I;
        double acc = 0.0;
        for (int j = 0; j < I; ++j) acc += hh[j] * (double)d[j];
        out[i] = acc;
    }
    free(hh);
}

/* Every row of the expert-grouped buffer through its expert.
 * x_perm [S][H]; w13 [N][2I][H]; w2 [N][H][I]; y_perm [S][H]. */
void oracle_expert_ffn(const float *x_perm, const int32_t *offsets, int N,
                       const float *w13, const float *w2, int H, int I,
                       double *y_perm)
{
    for (int e = 0; e < N; ++e)
        for (int r = offsets[e]; r < offsets[e + 1]; ++r)
            oracle_ffn_row(x_perm + (size_t)r * H,
                           w13 + (size_t)e * 2 * I * H,
                           w2 + (size_t)e * H * I, H, I,
                           y_perm + (size_t)r * H);
}

/* ---- zero-computation experts ----------------------------------------------
 * An identity expert returns its input ("identity mappers", Technical Report
 * notes, Key claims [§2.1]), so a token's share from them is
 *   y_acc[t] = (sum over its slots k with idx >= N of gate[t][k]) * x[t]. */
void oracle_zero_experts(const float *x, const int32_t *idx, const double *gate,
                         int T, int H, int K, int N, double *y_acc)
{
    for (int t = 0; t < T; ++t) {
        double gs = 0.0;
        for (int k = 0; k < K; ++k)
            if (idx[(size_t)t * K + k] >= N) gs += gate[(size_t)t * K + k];
        for (int h = 0; h < H; ++h)
            y_acc[(size_t)t * H + h] = gs * (double)x[(size_t)t * H + h];
    }
}

/* ---- combine -----------------------------------------------------------------
 * y[t] = y_acc[t] + sum over slots k with idx < N of s * gate[t][k] * y_perm[row]
 * s is the variance-compensation factor on fine-grained (FFN) expert outputs
 * (Technical Report notes, Key claims [§2.3.2 Eq. 8]); identity experts are
 * not scaled. */
void oracle_combine(const double *y_perm, const int32_t *slot_row,
                    const int32_t *idx, const double *gate, double s,
                    const double *y_acc, int T, int H, int K, int N, double *y)
{
    for (int t = 0; t < T; ++t) {
        double *yr = y + (size_t)t * H;
        for (int h = 0; h < H; ++h) yr[h] = y_acc[(size_t)t * H + h];
        for (int k = 0; k < K; ++k) {
            if (idx[(size_t)t * K + k] >= N) continue;
            double w = s * gate[(size_t)t * K + k];
            const double *src = y_perm + (size_t)slot_row[(size_t)t * K + k] * H;
            for (int h = 0; h < H; ++h) yr[h] += w * src[h];
        }
    }
}

/* ---- bias controller -----------------------------------------------------
 * Per FFN expert i (identity experts' biases are never touched: the notes
 * leave zero-computation experts out of the bias updates -- Technical Report
 * notes, Key claims [§2.1.1, §2.1.2]):
 *   err_i      = target / n_ffn - counts[i] / T
 *                (the expert's routing frequency below its share of the
 *                target number of activated FFN experts per token; summed
 *                over i it is target - FFN picks per token)
 *   integral_i = integral_i + err_i
 *   bias_i     = bias_i + kp * err_i + ki * integral_i + kd * (err_i - prev_i)
 *   prev_i     = err_i
 * The report's controller moves each FFN expert's bias by how often tokens
 * route to it, a refinement of the aux-loss-free update (bias += step *
 * sign(error)), so that the mean count of activated FFN experts holds a target
 * (Key claims [§2.1.1], Method).  The error, the increment form and the gains
 * are not on the pages: this is the plainest reading (the aux-loss-free
 * update with sign(err) replaced by a PID of err).  State in fp64. */
void oracle_bias_update(const int32_t *counts, int T, int n_ffn, double target, double kp,
                        double ki, double kd, double *bias, double *integral, double *prev) {
    for (int i = 0; i < n_ffn; ++i) {
        double err = target / (double)n_ffn - (double)counts[i] / (double)T;
        integral[i] = integral[i] + err;
        bias[i] = bias[i] + kp * err + ki * integral[i] + kd * (err - prev[i]);
        prev[i] = err;
    }
}

/* ---- router weight similarity --------------------------------------------
 * The report watches router stability through the pairwise cosine similarity
 * of the experts' router weight vectors (high similarity marks a router
 * collapsed by the load-balance term) -- Technical Report notes, Key claims
 * and Method [§3.1.3 Router Stability].  The vectors are the rows of w_router.
 *   dot[i][j] = sum_h w[i][h] * w[j][h]          (fp64, h ascending)
 *   sim[i][j] = dot[i][j] / (sqrt(dot[i][i]) * sqrt(dot[j][j]))
 * A row of zero norm has similarity 0 with every row, itself included.
 * Returns the mean of sim over the E*(E-1) ordered pairs i != j (0 if E = 1). */
double oracle_router_similarity(const float *w, int E, int H, double *sim)
{
    double *norm = (double *)malloc(sizeof(double) * (size_t)(E > 0 ? E : 1));
    for (int i = 0; i < E; ++i) {
        double acc = 0.0;
        for (int h = 0; h < H; ++h)
            acc += (double)w[(size_t)i * H + h] * (double)w[(size_t)i * H + h];
        norm[i] = sqrt(acc);
    }
    double total = 0.0;
    for (int i = 0; i < E; ++i) {
        for (int j = 0; j < E; ++j) {
            double acc = 0.0;
            for (int h = 0; h < H; ++h)
                acc += (double)w[(size_t)i * H + h] * (double)w[(size_t)j * H + h];
            double c = (norm[i] > 0.0 && norm[j] > 0.0) ? acc / (norm[i] * norm[j]) : 0.0;
            sim[(size_t)i * E + j] = c;
            if (i != j) total += c;
        }
    }
    free(norm);
    return E > 1 ? total / ((double)E * (double)(E - 1)) : 0.0;
}

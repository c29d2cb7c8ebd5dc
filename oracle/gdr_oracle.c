/*
 * gdr_oracle.c -- reference implementation of the gated delta-rule forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the parity oracle: a plain, slow,
 * sequential CPU recurrence in double precision.  Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg may load it.  It shares no
 * source, header, helper or constant with the GPU library, and the GPU library
 * never calls it.
 *
 * Every variant is written out as its own function, token by token, in the
 * notation of the pages:
 *
 *   S is the d_k x d_v fast-weight state of one head ("Kaczmarz Linear
 *   Attention", Implementation section: the state keeps the shape
 *   S in R^{d_k x d_v}).  Row index i runs over key channels, column index j
 *   over value channels.
 *
 *   The decay is applied first, giving the decayed previous state S~; the
 *   write then subtracts the read-out along the erase key and adds the value
 *   ("Kaczmarz Linear Attention", Theoretical derivation and KLA update rule
 *   sections: the target is the state closest to the decayed state S~_{t-1},
 *   the residual is e_t = v_t - S~_{t-1}^T k_t and the step is
 *   S_t = S~_{t-1} + beta_t k_t e_t^T).
 *
 *   The output reads the state after the update: o_t = S_t^T q_t.
 *
 * Variants ("Linear Attention Architectures: Mechanisms, Trade-offs, and
 * Cross-Layer Routing", the list of the four delta-rule mixers; "Gated
 * DeltaNet-2: Decoupling Erase and Write in Linear Attention", novelty and
 * technical-core sections; "Kaczmarz Linear Attention", KLA update rule):
 *
 *   DeltaNet      no decay, scalar write strength beta_t
 *   Gated DeltaNet  scalar decay alpha_t on the whole state, scalar beta_t
 *   KDA           channel-wise decay alpha_t[i] on the key rows, scalar beta_t
 *   GDN-2         channel-wise decay; separate channel-wise erase gate b_t
 *                 (key side) and write gate w_t (value side)
 *   KLA           scalar decay; beta_t = eta_t / (||k_t||^2 + eps)
 *
 * Array layouts (row-major, contiguous):
 *   q, k      [B, T, H, dk]      v        [B, T, H, dv]
 *   alpha     GDN, KLA: [B, T, H]; KDA, GDN-2: [B, T, H, dk]; DeltaNet: unused
 *   beta      DeltaNet, GDN, KDA: beta [B, T, H]; KLA: eta [B, T, H]
 *   erase_b   GDN-2: [B, T, H, dk]   write_w  GDN-2: [B, T, H, dv]
 *   state_in  [B, H, dk, dv] or NULL (zeros)
 *   state_out [B, H, dk, dv]         o        [B, T, H, dv]
 *   delta     [B, T, H, dv] or NULL: the residual each token writes,
 *             delta_t with S_t = S~_t + k_t delta_t^T (the error a layer passes
 *             on in cross-layer routing: "Linear Attention Architectures",
 *             the cross-layer routing section, where CLER passes the error and
 *             CLVR the value target)
 *
 * Each entry point processes one head (b, h); heads are independent, so the
 * caller may run different heads on different threads.
 */
#include <stdlib.h>
#include <string.h>

typedef struct {
    long B, T, H, dk, dv;
    const double *q, *k, *v;
    const double *alpha;
    const double *beta;
    const double *erase_b;
    const double *write_w;
    double eps;
    const double *state_in;
    double *state_out;
    double *o;
    double *delta;
} oracle_problem;

/* Offsets into the [B,T,H,d] token arrays and the [B,H,dk,dv] state. */
static long tok(const oracle_problem *p, long b, long t, long h, long d)
{
    return ((b * p->T + t) * p->H + h) * d;
}

static long gate(const oracle_problem *p, long b, long t, long h)
{
    return (b * p->T + t) * p->H + h;
}

static double *load_state(const oracle_problem *p, long b, long h)
{
    long n = p->dk * p->dv;
    double *S = (double *)malloc(sizeof(double) * (size_t)n);
    if (!S)
        return NULL;
    if (p->state_in)
        memcpy(S, p->state_in + (b * p->H + h) * n, sizeof(double) * (size_t)n);
    else
        memset(S, 0, sizeof(double) * (size_t)n);
    return S;
}

static void store_state(const oracle_problem *p, long b, long h, const double *S)
{
    long n = p->dk * p->dv;
    if (p->state_out)
        memcpy(p->state_out + (b * p->H + h) * n, S, sizeof(double) * (size_t)n);
}

/* o_t[j] = sum_i S[i][j] q_t[i], read after the update. */
static void read_out(const oracle_problem *p, long b, long t, long h, const double *S)
{
    const double *q = p->q + tok(p, b, t, h, p->dk);
    double *o = p->o + tok(p, b, t, h, p->dv);
    for (long j = 0; j < p->dv; ++j) {
        double acc = 0.0;
        for (long i = 0; i < p->dk; ++i)
            acc += S[i * p->dv + j] * q[i];
        o[j] = acc;
    }
}

/* delta_t[j] = scale * (x[j] - y[j]) (y may be NULL for zero), if requested. */
static void record_delta(const oracle_problem *p, long b, long t, long h, double scale,
                         const double *x, const double *xw, const double *y)
{
    if (!p->delta)
        return;
    double *d = p->delta + tok(p, b, t, h, p->dv);
    for (long j = 0; j < p->dv; ++j)
        d[j] = scale * ((xw ? xw[j] : 1.0) * x[j] - (y ? y[j] : 0.0));
}

/* DeltaNet: S <- S - beta k (k^T S) + beta k v^T. */
int oracle_deltanet_head(const oracle_problem *p, long b, long h)
{
    long dk = p->dk, dv = p->dv;
    double *S = load_state(p, b, h);
    double *kS = (double *)malloc(sizeof(double) * (size_t)dv);
    if (!S || !kS) {
        free(S);
        free(kS);
        return -1;
    }
    for (long t = 0; t < p->T; ++t) {
        const double *k = p->k + tok(p, b, t, h, dk);
        const double *v = p->v + tok(p, b, t, h, dv);
        double beta = p->beta[gate(p, b, t, h)];
        for (long j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (long i = 0; i < dk; ++i)
                acc += k[i] * S[i * dv + j];
            kS[j] = acc;
        }
        record_delta(p, b, t, h, beta, v, NULL, kS);
        for (long i = 0; i < dk; ++i)
            for (long j = 0; j < dv; ++j)
                S[i * dv + j] = S[i * dv + j] - beta * k[i] * kS[j] + beta * k[i] * v[j];
        read_out(p, b, t, h, S);
    }
    store_state(p, b, h, S);
    free(S);
    free(kS);
    return 0;
}

/* Gated DeltaNet: S <- alpha S (one scalar per head and token), then the
 * DeltaNet write against the decayed state. */
int oracle_gated_deltanet_head(const oracle_problem *p, long b, long h)
{
    long dk = p->dk, dv = p->dv;
    double *S = load_state(p, b, h);
    double *kS = (double *)malloc(sizeof(double) * (size_t)dv);
    if (!S || !kS) {
        free(S);
        free(kS);
        return -1;
    }
    for (long t = 0; t < p->T; ++t) {
        const double *k = p->k + tok(p, b, t, h, dk);
        const double *v = p->v + tok(p, b, t, h, dv);
        double alpha = p->alpha[gate(p, b, t, h)];
        double beta = p->beta[gate(p, b, t, h)];
        for (long i = 0; i < dk * dv; ++i)
            S[i] = alpha * S[i];
        for (long j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (long i = 0; i < dk; ++i)
                acc += k[i] * S[i * dv + j];
            kS[j] = acc;
        }
        record_delta(p, b, t, h, beta, v, NULL, kS);
        for (long i = 0; i < dk; ++i)
            for (long j = 0; j < dv; ++j)
                S[i * dv + j] = S[i * dv + j] - beta * k[i] * kS[j] + beta * k[i] * v[j];
        read_out(p, b, t, h, S);
    }
    store_state(p, b, h, S);
    free(S);
    free(kS);
    return 0;
}

/* Kimi Delta Attention: row i of S (key channel i) decays by alpha_t[i],
 * then the DeltaNet write against the decayed state. */
int oracle_kda_head(const oracle_problem *p, long b, long h)
{
    long dk = p->dk, dv = p->dv;
    double *S = load_state(p, b, h);
    double *kS = (double *)malloc(sizeof(double) * (size_t)dv);
    if (!S || !kS) {
        free(S);
        free(kS);
        return -1;
    }
    for (long t = 0; t < p->T; ++t) {
        const double *k = p->k + tok(p, b, t, h, dk);
        const double *v = p->v + tok(p, b, t, h, dv);
        const double *alpha = p->alpha + tok(p, b, t, h, dk);
        double beta = p->beta[gate(p, b, t, h)];
        for (long i = 0; i < dk; ++i)
            for (long j = 0; j < dv; ++j)
                S[i * dv + j] = alpha[i] * S[i * dv + j];
        for (long j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (long i = 0; i < dk; ++i)
                acc += k[i] * S[i * dv + j];
            kS[j] = acc;
        }
        record_delta(p, b, t, h, beta, v, NULL, kS);
        for (long i = 0; i < dk; ++i)
            for (long j = 0; j < dv; ++j)
                S[i * dv + j] = S[i * dv + j] - beta * k[i] * kS[j] + beta * k[i] * v[j];
        read_out(p, b, t, h, S);
    }
    store_state(p, b, h, S);
    free(S);
    free(kS);
    return 0;
}

/* Gated DeltaNet-2: channel-wise decay on the key rows; the read-out that is
 * erased goes through the erase gate on the key side,
 *   r_j = sum_i b_i k_i S~[i][j],
 * and the value written goes through the write gate on the value side:
 *   S[i][j] <- S~[i][j] - k_i r_j + k_i w_j v_j. */
int oracle_gdn2_head(const oracle_problem *p, long b, long h)
{
    long dk = p->dk, dv = p->dv;
    double *S = load_state(p, b, h);
    double *r = (double *)malloc(sizeof(double) * (size_t)dv);
    if (!S || !r) {
        free(S);
        free(r);
        return -1;
    }
    for (long t = 0; t < p->T; ++t) {
        const double *k = p->k + tok(p, b, t, h, dk);
        const double *v = p->v + tok(p, b, t, h, dv);
        const double *alpha = p->alpha + tok(p, b, t, h, dk);
        const double *eb = p->erase_b + tok(p, b, t, h, dk);
        const double *ww = p->write_w + tok(p, b, t, h, dv);
        for (long i = 0; i < dk; ++i)
            for (long j = 0; j < dv; ++j)
                S[i * dv + j] = alpha[i] * S[i * dv + j];
        for (long j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (long i = 0; i < dk; ++i)
                acc += eb[i] * k[i] * S[i * dv + j];
            r[j] = acc;
        }
        record_delta(p, b, t, h, 1.0, v, ww, r);
        for (long i = 0; i < dk; ++i)
            for (long j = 0; j < dv; ++j)
                S[i * dv + j] = S[i * dv + j] - k[i] * r[j] + k[i] * ww[j] * v[j];
        read_out(p, b, t, h, S);
    }
    store_state(p, b, h, S);
    free(S);
    free(r);
    return 0;
}

/* Kaczmarz Linear Attention: beta_t = eta_t / (||k_t||^2 + eps); decayed state
 * S~ = alpha_t S; residual e = v - S~^T k; S <- S~ + beta_t k e^T. */
int oracle_kla_head(const oracle_problem *p, long b, long h)
{
    long dk = p->dk, dv = p->dv;
    double *S = load_state(p, b, h);
    double *e = (double *)malloc(sizeof(double) * (size_t)dv);
    if (!S || !e) {
        free(S);
        free(e);
        return -1;
    }
    for (long t = 0; t < p->T; ++t) {
        const double *k = p->k + tok(p, b, t, h, dk);
        const double *v = p->v + tok(p, b, t, h, dv);
        double alpha = p->alpha[gate(p, b, t, h)];
        double eta = p->beta[gate(p, b, t, h)];
        double knorm2 = 0.0;
        for (long i = 0; i < dk; ++i)
            knorm2 += k[i] * k[i];
        double beta = eta / (knorm2 + p->eps);
        for (long i = 0; i < dk * dv; ++i)
            S[i] = alpha * S[i];
        for (long j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (long i = 0; i < dk; ++i)
                acc += S[i * dv + j] * k[i];
            e[j] = v[j] - acc;
        }
        record_delta(p, b, t, h, beta, e, NULL, NULL);
        for (long i = 0; i < dk; ++i)
            for (long j = 0; j < dv; ++j)
                S[i * dv + j] = S[i * dv + j] + beta * k[i] * e[j];
        read_out(p, b, t, h, S);
    }
    store_state(p, b, h, S);
    free(S);
    free(e);
    return 0;
}

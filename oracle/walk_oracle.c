/*
 * walk_oracle.c -- plain CPU oracle for the serial Markov draft walk of
 * DSpark's head.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  The GPU product path
 * never calls it, shares no code with it and must fail loudly without its own
 * HIP library.
 *
 * Source: "Keeping the Draft Walk on Chip: One Launch for DSpark's Markov
 * Head" (tie-pilot-qxw.github.io), sections "The serial part of a parallel
 * drafter" (the walk and its rounding points), "The idea: make the walk
 * resident" (ties go to the smallest token id; the token is chosen from the
 * very bf16 logits that are emitted) and "B200: the bf16 table fits on chip"
 * (fp32 accumulation, bias rounded to bf16, then the sum rounded to bf16).
 * Sampling follows vLLM PR #64442 "fused Markov sampling", section "Details"
 * (inverse CDF over softmax(cached logits / T) driven by one uniform per
 * request and step).
 *
 * Everything is computed in IEEE binary64 with plain loops:
 *   u_j      = W1[prev, j]                               (bf16 -> f64, exact)
 *   acc_v    = sum_j W2[v, j] * u_j   in ascending j     (products exact in f64)
 *   int8:      acc_v = scale_v * sum_j q[v, j] * u_j
 *   bias_v   = RNE_bf16(acc_v)        rounded straight from f64
 *   logit_v  = RNE_bf16(base_v + bias_v)  (the f64 sum of two bf16 is exact)
 *   single-rounding mode (ORACLE_SINGLE_ROUND): logit_v = RNE_bf16(base_v + acc_v),
 *            the sum rounded once, as the pages' H100 int8 kernel does ("Keeping
 *            the Draft Walk on Chip", section "Correctness", and the caption of
 *            Fig. 7) and as vLLM PR #64442 ("Details") writes its fp32 sum to
 *            the cache
 *   T == 0 : tok = smallest v with logit_v == max_w logit_w
 *   T  > 0 : M = max logit, w_v = exp((logit_v - M) / T), C_v = sum_{j<=v} w_j,
 *            Z = C_{V-1}, t = uniform * Z, tok = smallest v with C_v > t
 *            (if rounding leaves none, the largest v with w_v > 0).
 *   Gumbel-max mode (ORACLE_GUMBEL, T > 0): tok = smallest v maximising
 *            logit_v / T - ln(-ln U_v), one counter-based uniform U_v in (0, 1)
 *            per request, step and vocabulary row (the pages' in-kernel sampler
 *            for small batches: "Keeping the Draft Walk on Chip", section
 *            "The idea: make the walk resident"; argmax of the perturbed
 *            logits is an exact draw from softmax(logit / T)).
 *   prev     = tok for the next step.
 *
 * GRU head (oracle_gru_cell, oracle_walk_gru): a serial head whose state is
 * updated by a gated recurrent cell ("Keeping the Draft Walk on Chip",
 * section "Beyond DSpark: other serial heads": DeLS-Spec corrects its block
 * with a GRU, and every such head ends in the same vocabulary-wide matrix).
 * The cell is the standard GRU (Cho et al. 2014, "Learning Phrase
 * Representations using RNN Encoder-Decoder"), in the common form where the
 * reset gate scales the recurrent term after its matrix product; gates in the
 * order (r, z, n):
 *   r = sigmoid(Wir x + bir + Whr h + bhr)
 *   z = sigmoid(Wiz x + biz + Whz h + bhz)
 *   n = tanh(Win x + bin + r * (Whn h + bhn))
 *   h' = (1 - z) * n + z * h
 * with x = W1[prev] (the previous token's row of the rank-r table) and the
 * vocabulary matrix applied to u = bf16(h'):  logit = bf16(base + bf16(W2 u)).
 * RNN head (oracle_rnn_cell, oracle_walk_rnn; DSpark's own RNN head, read as
 * the standard tanh RNN cell): h' = tanh(Wih x + bih + Whh h + bhh), otherwise
 * the same walk.
 * Gated head (oracle_gated_cell, oracle_walk_gated; DSpark's own gated head).
 * The pages fix only its shape: one r x r matrix, small enough in int8 for
 * every CTA to apply it itself, so the update needs no state exchange.  They
 * give no equation; the reading taken here is the plainest single-matrix gated
 * update, a convex gate between the carried state and the new token's row:
 *   g  = sigmoid(s * (Gq h) + b)       Gq int8 codes [r][r], s, b per row
 *   h' = g * h + (1 - g) * x           x = W1[prev]
 * and the vocabulary matrix reads u = bf16(h') as for the other heads.  With
 * b -> -inf the gate closes (g = 0) and the walk is the Markov walk; with
 * b -> +inf the state never moves.
 * Domino's head (oracle_walk_domino): a GRU cell that also reads the drafter's
 * hidden states (same section).  Read here as the GRU above whose input at
 * step k is the concatenation x = [W1[prev]; H_k] of the previous token's row
 * and the drafter's hidden state H_k (d values) at block position k, so Wih
 * is [3r][r + d].
 *
 * Parallelism: OpenMP over vocabulary rows inside one GEMV.  Each row's sum
 * is formed by one thread in a fixed order, so results do not depend on the
 * thread count.
 */
#include <fenv.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* bf16 bit pattern -> its exact value as a double. */
static double bf16_value(uint16_t h) {
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Mode bits of oracle_step / oracle_walk. */
#define ORACLE_SINGLE_ROUND 1
#define ORACLE_GUMBEL 2

static int sample_gumbel(const double* logit, int V, double T, uint64_t seed, uint32_t round, int b, int k);

/* Round x to the nearest bf16 value (8 significant bits, exponent range of
 * binary32), ties to even, directly from binary64.  The result is returned as
 * a double that is exactly representable in bf16.  Overflow goes to +-inf. */
double oracle_rne_bf16(double x) {
    if (isnan(x) || isinf(x) || x == 0.0) return x;
    int e = ilogb(x);           /* x = m * 2^e with 1 <= |m| < 2 */
    if (e < -126) e = -126;     /* below the normal range the spacing is 2^-133 */
    /* scale so that one bf16 unit in the last place becomes 1.0, round to an
     * integer in the current (to-nearest-even) mode, scale back */
    double y = ldexp(nearbyint(ldexp(x, 7 - e)), e - 7);
    if (fabs(y) >= ldexp(1.0, 128)) y = copysign(INFINITY, x);
    return y;
}

/* bf16 bit pattern of a double that is exactly representable in bf16. */
uint16_t oracle_bf16_bits(double y) {
    float f = (float)y;         /* exact for bf16-representable values */
    uint32_t bits;
    memcpy(&bits, &f, sizeof bits);
    return (uint16_t)(bits >> 16);
}

/* Vectorised helpers for the Python side: RNE of n doubles (values and bits). */
void oracle_rne_bf16_array(const double* x, double* y, uint16_t* bits, long n) {
    for (long i = 0; i < n; ++i) {
        double v = oracle_rne_bf16(x[i]);
        if (y) y[i] = v;
        if (bits) bits[i] = oracle_bf16_bits(v);
    }
}

int oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* The smallest index holding the largest of V values (ties go to the smallest id). */
static int first_argmax(const double* x, int V) {
    int best = 0;
    for (int v = 1; v < V; ++v)
        if (x[v] > x[best]) best = v;   /* strict: the first maximum wins */
    return best;
}

/* Inverse-CDF draw over softmax(logit / T) from one uniform in [0, 1).
 * logit holds V finite values.  Returns the chosen token id. */
static int sample_inverse_cdf(const double* logit, int V, double T, double uniform) {
    double M = logit[0];
    for (int v = 1; v < V; ++v)
        if (logit[v] > M) M = logit[v];
    double* C = (double*)malloc(sizeof(double) * (size_t)V);
    if (!C) return -3;
    double run = 0.0;
    int last_positive = -1;
    for (int v = 0; v < V; ++v) {
        double w = exp((logit[v] - M) / T);
        if (w > 0.0) last_positive = v;
        run += w;
        C[v] = run;
    }
    double t = uniform * C[V - 1];
    int tok = -1;
    for (int v = 0; v < V; ++v) {
        if (C[v] > t) { tok = v; break; }
    }
    if (tok < 0) tok = last_positive;
    free(C);
    return tok;
}

/*
 * One step for one request.
 *   u        : W1 row of the previous token, r bf16 values (bits)
 *   W2       : [V][r] bf16 bits, or NULL when Q/scale are given
 *   Q, scale : [V][r] int8 and [V] f32 (int8 variant), else NULL
 *   base     : [V] bf16 bits of this step's base logits
 *   T        : temperature; exactly 0 selects greedy argmax
 *   uniform  : the step's uniform in [0,1) (ignored when T == 0)
 *   logits   : [V] bf16 bits out (may be NULL)
 *   scratch  : [V] doubles of caller-provided work space
 * Returns the token (>= 0) or a negative error (-2: a logit is not finite).
 */
static int oracle_step_impl(int V, int r, const uint16_t* u_bits,
                            const uint16_t* W2, const int8_t* Q, const float* scale,
                            const uint16_t* base, float T, float uniform,
                            uint16_t* logits, double* lg, int mode,
                            uint64_t seed, uint32_t round, int b, int k) {
    const int single = (mode & ORACLE_SINGLE_ROUND) != 0;
    double* u = (double*)malloc(sizeof(double) * (size_t)r);
    if (!u) return -3;
    for (int j = 0; j < r; ++j) u[j] = bf16_value(u_bits[j]);

    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int v = 0; v < V; ++v) {
        double acc = 0.0;
        if (W2) {
            const uint16_t* row = W2 + (size_t)v * (size_t)r;
            for (int j = 0; j < r; ++j) acc += bf16_value(row[j]) * u[j];
        } else {
            const int8_t* row = Q + (size_t)v * (size_t)r;
            double dot = 0.0;
            for (int j = 0; j < r; ++j) dot += (double)row[j] * u[j];
            acc = (double)scale[v] * dot;
        }
        /* double rounding: the bias is rounded to bf16 first; single: the sum once */
        double logit = single ? oracle_rne_bf16(bf16_value(base[v]) + acc)
                              : oracle_rne_bf16(bf16_value(base[v]) + oracle_rne_bf16(acc));
        if (!isfinite(logit)) bad = 1;
        lg[v] = logit;
        if (logits) logits[v] = oracle_bf16_bits(logit);
    }
    free(u);
    if (bad) return -2;

    if (T == 0.0f) return first_argmax(lg, V);
    if (mode & ORACLE_GUMBEL) return sample_gumbel(lg, V, (double)T, seed, round, b, k);
    return sample_inverse_cdf(lg, V, (double)T, (double)uniform);
}

/* Public single step (see oracle_step_impl; inverse-CDF sampling). */
int oracle_step(int V, int r, const uint16_t* u_bits, const uint16_t* W2,
                const int8_t* Q, const float* scale, const uint16_t* base,
                float T, float uniform, uint16_t* logits, int mode) {
    if (V <= 0 || r <= 0 || !u_bits || !base || (!W2 && (!Q || !scale))) return -1;
    double* lg = (double*)malloc(sizeof(double) * (size_t)V);
    if (!lg) return -3;
    int tok = oracle_step_impl(V, r, u_bits, W2, Q, scale, base, T, uniform, logits, lg,
                               mode & ORACLE_SINGLE_ROUND, 0, 0, 0, 0);
    free(lg);
    return tok;
}

/* Inverse-CDF draw on given bf16 logits (used to judge sampled GPU tokens
 * against the GPU's own emitted logits). */
int oracle_sample(int V, const uint16_t* logits, float T, float uniform) {
    if (V <= 0 || !logits || !(T > 0.0f)) return -1;
    double* lg = (double*)malloc(sizeof(double) * (size_t)V);
    if (!lg) return -3;
    for (int v = 0; v < V; ++v) lg[v] = bf16_value(logits[v]);
    int tok = sample_inverse_cdf(lg, V, (double)T, (double)uniform);
    free(lg);
    return tok;
}

/*
 * The whole walk for B independent requests.
 *   W1       : [V][r] bf16 bits
 *   W2       : [V][r] bf16 bits, or NULL with Q [V][r] int8 + scale [V] f32
 *   base     : [B][gamma][V] bf16 bits
 *   anchor   : [B] token ids in [0, V)
 *   T        : [B] temperatures (0 = greedy)
 *   uniforms : [B][gamma] in [0, 1), or NULL when every T is 0
 *   forced   : [B][gamma] or NULL.  When given, step k > 0 of request b uses
 *              prev = forced[b][k-1] instead of the oracle's own token
 *              (teacher forcing, so each step can be judged on its own).
 *   tokens   : [B][gamma] out
 *   logits   : [B][gamma][V] bf16 bits out, or NULL
 *   mode     : 0, or ORACLE_SINGLE_ROUND, ORACLE_GUMBEL (or both)
 *   seed, round : Gumbel-max mode only: the key and the device round counter
 *              of the uniforms (see oracle_gumbel_uniform)
 * Returns 0, or a negative error (-1 bad argument, -2 non-finite logit,
 * -3 out of memory).
 */
int oracle_walk_ex(int V, int r, int B, int gamma, const uint16_t* W1,
                   const uint16_t* W2, const int8_t* Q, const float* scale,
                   const uint16_t* base, const int32_t* anchor, const float* T,
                   const float* uniforms, const int32_t* forced, int32_t* tokens,
                   uint16_t* logits, int mode, uint64_t seed, uint32_t round) {
    if (V <= 0 || r <= 0 || B < 0 || gamma < 0 || !W1 || !base || !anchor || !T ||
        !tokens || (!W2 && (!Q || !scale)))
        return -1;
    if ((mode & ORACLE_GUMBEL) && B > 256) return -1;  /* request ids live in 8 counter bits */
    for (int b = 0; b < B; ++b) {
        if (T[b] != 0.0f && !uniforms && !(mode & ORACLE_GUMBEL)) return -1;
        if (anchor[b] < 0 || anchor[b] >= V) return -1;
    }
    double* lg = (double*)malloc(sizeof(double) * (size_t)V);
    if (!lg) return -3;
    for (int b = 0; b < B; ++b) {
        int prev = anchor[b];
        for (int k = 0; k < gamma; ++k) {
            if (forced && k > 0) prev = forced[(size_t)b * gamma + (k - 1)];
            if (prev < 0 || prev >= V) { free(lg); return -1; }
            const uint16_t* base_k = base + ((size_t)b * gamma + k) * (size_t)V;
            uint16_t* out = logits ? logits + ((size_t)b * gamma + k) * (size_t)V : NULL;
            float uni = uniforms ? uniforms[(size_t)b * gamma + k] : 0.0f;
            int tok = oracle_step_impl(V, r, W1 + (size_t)prev * (size_t)r, W2, Q, scale,
                                       base_k, T[b], uni, out, lg, mode, seed, round, b, k);
            if (tok < 0) { free(lg); return tok; }
            tokens[(size_t)b * gamma + k] = tok;
            prev = tok;
        }
    }
    free(lg);
    return 0;
}

/* The walk with inverse-CDF sampling (oracle_walk_ex without Gumbel-max). */
int oracle_walk(int V, int r, int B, int gamma, const uint16_t* W1,
                const uint16_t* W2, const int8_t* Q, const float* scale,
                const uint16_t* base, const int32_t* anchor, const float* T,
                const float* uniforms, const int32_t* forced, int32_t* tokens,
                uint16_t* logits, int mode) {
    return oracle_walk_ex(V, r, B, gamma, W1, W2, Q, scale, base, anchor, T, uniforms, forced,
                          tokens, logits, mode & ORACLE_SINGLE_ROUND, 0, 0);
}

/*
 * Counter-based uniforms, for walks that draw their uniforms on the device.
 * Philox-4x32 with 10 rounds, as defined in Salmon, Moraes, Dror and Shaw,
 * "Parallel Random Numbers: As Easy as 1, 2, 3" (SC 2011): each round
 * multiplies counter words 0 and 2 by the two round constants, keeps the high
 * and low halves of the 64-bit products, mixes the high halves with the
 * other two counter words and the key, and the key advances by the two Weyl
 * constants between rounds.
 */
static void mulhilo32(uint32_t a, uint32_t b, uint32_t* hi, uint32_t* lo) {
    const uint64_t p = (uint64_t)a * (uint64_t)b;
    *hi = (uint32_t)(p >> 32);
    *lo = (uint32_t)p;
}

void oracle_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
    uint32_t c[4] = {ctr_in[0], ctr_in[1], ctr_in[2], ctr_in[3]};
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        uint32_t hi0, lo0, hi1, lo1;
        mulhilo32(0xD2511F53u, c[0], &hi0, &lo0);
        mulhilo32(0xCD9E8D57u, c[2], &hi1, &lo1);
        const uint32_t n0 = hi1 ^ c[1] ^ k0;
        const uint32_t n2 = hi0 ^ c[3] ^ k1;
        c[0] = n0;
        c[1] = lo1;
        c[2] = n2;
        c[3] = lo0;
    }
    out[0] = c[0];
    out[1] = c[1];
    out[2] = c[2];
    out[3] = c[3];
}

/* The uniform of request b at step k of the walk whose device round counter
 * was `round`: counter (k, b, round, 0x44535721), key (seed low, seed high),
 * the first output word's top 24 bits as a multiple of 2^-24 in [0, 1). */
float oracle_device_uniform(uint64_t seed, uint32_t round, int b, int k) {
    const uint32_t ctr[4] = {(uint32_t)k, (uint32_t)b, round, 0x44535721u};
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    oracle_philox4x32_10(ctr, key, out);
    return (float)(out[0] >> 8) * (1.0f / 16777216.0f);
}

void oracle_device_uniforms(uint64_t seed, uint32_t round, int B, int gamma, float* out) {
    for (int b = 0; b < B; ++b)
        for (int k = 0; k < gamma; ++k) out[(size_t)b * gamma + k] = oracle_device_uniform(seed, round, b, k);
}

/*
 * Gumbel-max sampling.  The noise of vocabulary row v for request b at step k
 * of the walk whose device round counter was `round`: Philox-4x32-10 of the
 * counter (v / 4, 256 k + b, round, 0x47554D42) under the key (seed low, seed
 * high), output word v mod 4 (four consecutive rows share one call), mapped to
 * the odd multiple (2 (w >> 9) + 1) 2^-24 of 2^-24, which lies strictly inside
 * (0, 1) and is exact in binary32.  The Gumbel variate is -ln(-ln U).
 */
double oracle_gumbel_uniform(uint64_t seed, uint32_t round, int b, int k, int v) {
    const uint32_t ctr[4] = {(uint32_t)v >> 2, ((uint32_t)k << 8) | ((uint32_t)b & 0xFFu), round, 0x47554D42u};
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    oracle_philox4x32_10(ctr, key, out);
    return (double)(2u * (out[v & 3] >> 9) + 1u) * (1.0 / 16777216.0);
}

/* Perturbed scores logit_v / T - ln(-ln U_v) of one request and step. */
static void gumbel_scores(const double* logit, int V, double T, uint64_t seed, uint32_t round, int b, int k,
                          double* score) {
    for (int v = 0; v < V; ++v) {
        const double U = oracle_gumbel_uniform(seed, round, b, k, v);
        score[v] = logit[v] / T - log(-log(U));
    }
}

/* Gumbel-max draw: the smallest v with the largest perturbed score. */
static int sample_gumbel(const double* logit, int V, double T, uint64_t seed, uint32_t round, int b, int k) {
    double* sc = (double*)malloc(sizeof(double) * (size_t)V);
    if (!sc) return -3;
    gumbel_scores(logit, V, T, seed, round, b, k, sc);
    const int best = first_argmax(sc, V);
    free(sc);
    return best;
}

/* The perturbed scores for given bf16 logits (used to judge GPU tokens on the
 * GPU's own emitted logits); T > 0. */
int oracle_gumbel_scores(int V, const uint16_t* logits, float T, uint64_t seed, uint32_t round, int b, int k,
                         double* score) {
    if (V <= 0 || !logits || !score || !(T > 0.0f)) return -1;
    double* lg = (double*)malloc(sizeof(double) * (size_t)V);
    if (!lg) return -3;
    for (int v = 0; v < V; ++v) lg[v] = bf16_value(logits[v]);
    gumbel_scores(lg, V, (double)T, seed, round, b, k, score);
    free(lg);
    return 0;
}

/* Gumbel-max draw from given uniforms (no counter-based generator): the
 * definition of the sampler on its own, for worked examples. */
int oracle_gumbel_from_uniforms(int V, const double* logit, double T, const double* U) {
    if (V <= 0 || !logit || !U || !(T > 0.0)) return -1;
    for (int v = 0; v < V; ++v)
        if (!(U[v] > 0.0 && U[v] < 1.0)) return -1;
    double* sc = (double*)malloc(sizeof(double) * (size_t)V);
    if (!sc) return -3;
    for (int v = 0; v < V; ++v) sc[v] = logit[v] / T - log(-log(U[v]));
    const int best = first_argmax(sc, V);
    free(sc);
    return best;
}

/*
 * One GRU cell in binary64 (see the header).  x, h: r values; Wih, Whh:
 * [3r][r] bf16 bits, gate blocks (r, z, n); bih, bhh: [3r] f32; out: r values.
 */
void oracle_gru_cell_in(int r, int in, const double* x, const double* h, const uint16_t* Wih,
                        const uint16_t* Whh, const float* bih, const float* bhh, double* out) {
    for (int j = 0; j < r; ++j) {
        double gi[3], gh[3];
        for (int g = 0; g < 3; ++g) {
            const int row = g * r + j;
            double si = 0.0, sh = 0.0;
            for (int i = 0; i < in; ++i) si += bf16_value(Wih[(size_t)row * in + i]) * x[i];
            for (int i = 0; i < r; ++i) sh += bf16_value(Whh[(size_t)row * r + i]) * h[i];
            gi[g] = si + (double)bih[row];
            gh[g] = sh + (double)bhh[row];
        }
        const double rg = 1.0 / (1.0 + exp(-(gi[0] + gh[0])));
        const double zg = 1.0 / (1.0 + exp(-(gi[1] + gh[1])));
        const double ng = tanh(gi[2] + rg * gh[2]);
        out[j] = (1.0 - zg) * ng + zg * h[j];
    }
}

/* The GRU cell with an input as wide as the state (Wih [3r][r]). */
void oracle_gru_cell(int r, const double* x, const double* h, const uint16_t* Wih, const uint16_t* Whh,
                     const float* bih, const float* bhh, double* out) {
    oracle_gru_cell_in(r, r, x, h, Wih, Whh, bih, bhh, out);
}

/*
 * One tanh RNN cell in binary64: h' = tanh(Wih x + bih + Whh h + bhh).
 * Wih, Whh: [r][r] bf16 bits; bih, bhh: [r] f32.
 */
void oracle_rnn_cell(int r, const double* x, const double* h, const uint16_t* Wih, const uint16_t* Whh,
                     const float* bih, const float* bhh, double* out) {
    for (int j = 0; j < r; ++j) {
        double si = 0.0, sh = 0.0;
        for (int i = 0; i < r; ++i) {
            si += bf16_value(Wih[(size_t)j * r + i]) * x[i];
            sh += bf16_value(Whh[(size_t)j * r + i]) * h[i];
        }
        out[j] = tanh((si + (double)bih[j]) + (sh + (double)bhh[j]));
    }
}

/*
 * One step of the gated head in binary64 (see the header): per element j,
 * g_j = sigmoid(s_j * sum_i Gq[j][i] h_i + b_j), h'_j = g_j h_j + (1 - g_j) x_j.
 * Gq: [r][r] int8 codes; s, b: [r] f32.
 */
void oracle_gated_cell(int r, const double* x, const double* h, const int8_t* Gq, const float* s,
                       const float* b, double* out) {
    for (int j = 0; j < r; ++j) {
        double acc = 0.0;
        for (int i = 0; i < r; ++i) acc += (double)Gq[(size_t)j * r + i] * h[i];
        const double g = 1.0 / (1.0 + exp(-((double)s[j] * acc + (double)b[j])));
        out[j] = g * h[j] + (1.0 - g) * x[j];
    }
}

/*
 * A recurrent head's walk for B independent requests (free running, or teacher
 * forced); kind 1 = GRU, 2 = tanh RNN, 3 = gated head.  Arguments as
 * oracle_walk_ex, plus
 *   Wih, Whh, bih, bhh : the cell (see oracle_gru_cell, oracle_rnn_cell)
 *   Gq, gs, gb : the gated head's matrix, row scales and biases (kind 3)
 *   H, d     : kind 4 (Domino): the drafter's hidden states [B][gamma][d] bf16,
 *              the GRU's input is [W1[prev]; H[b][k]] and Wih is [3r][r + d]
 *   h0       : [B][r] initial states (f32)
 *   forced_h : [B][gamma][r] f32 or NULL.  When given, step k > 0 of request b
 *              starts from forced_h[b][k-1] instead of the oracle's own state.
 *   states   : [B][gamma][r] out, the states h_k in binary64 (may be NULL)
 * The GEMV operand of step k is bf16(h_k), rounded from binary64.
 */
static int walk_cell(int kind, int V, int r, int B, int gamma, const uint16_t* W1,
                     const uint16_t* W2, const int8_t* Q, const float* scale,
                     const uint16_t* Wih, const uint16_t* Whh, const float* bih, const float* bhh,
                     const int8_t* Gq, const float* gs, const float* gb, const uint16_t* H, int d,
                     const float* h0, const uint16_t* base, const int32_t* anchor, const float* T,
                     const float* uniforms, const int32_t* forced, const float* forced_h,
                     int32_t* tokens, uint16_t* logits, double* states, int mode, uint64_t seed,
                     uint32_t round) {
    if (V <= 0 || r <= 0 || B < 0 || gamma < 0 || !W1 || !h0 || !base || !anchor || !T || !tokens ||
        (!W2 && (!Q || !scale)))
        return -1;
    if (kind == 3 ? (!Gq || !gs || !gb) : (!Wih || !Whh || !bih || !bhh)) return -1;
    if (kind == 4 && (!H || d <= 0)) return -1;
    const int in = kind == 4 ? r + d : r;  /* the cell's input width */
    for (int b = 0; b < B; ++b) {
        if (T[b] != 0.0f && !uniforms && !(mode & ORACLE_GUMBEL)) return -1;
        if (anchor[b] < 0 || anchor[b] >= V) return -1;
    }
    double* lg = (double*)malloc(sizeof(double) * (size_t)V);
    double* x = (double*)malloc(sizeof(double) * (size_t)in);
    double* h = (double*)malloc(sizeof(double) * (size_t)r);
    double* hn = (double*)malloc(sizeof(double) * (size_t)r);
    uint16_t* ub = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)r);
    int rc = 0;
    if (!lg || !x || !h || !hn || !ub) rc = -3;
    for (int b = 0; b < B && rc == 0; ++b) {
        int prev = anchor[b];
        for (int i = 0; i < r; ++i) h[i] = (double)h0[(size_t)b * r + i];
        for (int k = 0; k < gamma && rc == 0; ++k) {
            if (forced && k > 0) prev = forced[(size_t)b * gamma + (k - 1)];
            if (forced_h && k > 0)
                for (int i = 0; i < r; ++i) h[i] = (double)forced_h[((size_t)b * gamma + (k - 1)) * r + i];
            if (prev < 0 || prev >= V) { rc = -1; break; }
            for (int i = 0; i < r; ++i) x[i] = bf16_value(W1[(size_t)prev * r + i]);
            for (int i = r; i < in; ++i) x[i] = bf16_value(H[((size_t)b * gamma + k) * (size_t)d + (i - r)]);
            if (kind == 1 || kind == 4) oracle_gru_cell_in(r, in, x, h, Wih, Whh, bih, bhh, hn);
            else if (kind == 2) oracle_rnn_cell(r, x, h, Wih, Whh, bih, bhh, hn);
            else oracle_gated_cell(r, x, h, Gq, gs, gb, hn);
            for (int i = 0; i < r; ++i) {
                h[i] = hn[i];
                ub[i] = oracle_bf16_bits(oracle_rne_bf16(hn[i]));
                if (states) states[((size_t)b * gamma + k) * r + i] = hn[i];
            }
            const uint16_t* base_k = base + ((size_t)b * gamma + k) * (size_t)V;
            uint16_t* out = logits ? logits + ((size_t)b * gamma + k) * (size_t)V : NULL;
            float uni = uniforms ? uniforms[(size_t)b * gamma + k] : 0.0f;
            int tok = oracle_step_impl(V, r, ub, W2, Q, scale, base_k, T[b], uni, out, lg, mode, seed, round,
                                       b, k);
            if (tok < 0) { rc = tok; break; }
            tokens[(size_t)b * gamma + k] = tok;
            prev = tok;
        }
    }
    free(lg); free(x); free(h); free(hn); free(ub);
    return rc;
}

/* The GRU head's walk (see walk_cell). */
int oracle_walk_gru(int V, int r, int B, int gamma, const uint16_t* W1,
                    const uint16_t* W2, const int8_t* Q, const float* scale,
                    const uint16_t* Wih, const uint16_t* Whh, const float* bih, const float* bhh,
                    const float* h0, const uint16_t* base, const int32_t* anchor, const float* T,
                    const float* uniforms, const int32_t* forced, const float* forced_h,
                    int32_t* tokens, uint16_t* logits, double* states, int mode, uint64_t seed,
                    uint32_t round) {
    return walk_cell(1, V, r, B, gamma, W1, W2, Q, scale, Wih, Whh, bih, bhh, NULL, NULL, NULL, NULL, 0, h0, base,
                     anchor, T, uniforms, forced, forced_h, tokens, logits, states, mode, seed, round);
}

/* The RNN head's walk: as oracle_walk_gru with the tanh RNN cell, Wih, Whh
 * [r][r], bih, bhh [r]. */
int oracle_walk_rnn(int V, int r, int B, int gamma, const uint16_t* W1,
                    const uint16_t* W2, const int8_t* Q, const float* scale,
                    const uint16_t* Wih, const uint16_t* Whh, const float* bih, const float* bhh,
                    const float* h0, const uint16_t* base, const int32_t* anchor, const float* T,
                    const float* uniforms, const int32_t* forced, const float* forced_h,
                    int32_t* tokens, uint16_t* logits, double* states, int mode, uint64_t seed,
                    uint32_t round) {
    return walk_cell(2, V, r, B, gamma, W1, W2, Q, scale, Wih, Whh, bih, bhh, NULL, NULL, NULL, NULL, 0, h0, base,
                     anchor, T, uniforms, forced, forced_h, tokens, logits, states, mode, seed, round);
}

/* The gated head's walk: as oracle_walk_gru with the gated update, Gq [r][r]
 * int8 codes, gs, gb [r] f32 (see oracle_gated_cell). */
int oracle_walk_gated(int V, int r, int B, int gamma, const uint16_t* W1,
                      const uint16_t* W2, const int8_t* Q, const float* scale,
                      const int8_t* Gq, const float* gs, const float* gb,
                      const float* h0, const uint16_t* base, const int32_t* anchor, const float* T,
                      const float* uniforms, const int32_t* forced, const float* forced_h,
                      int32_t* tokens, uint16_t* logits, double* states, int mode, uint64_t seed,
                      uint32_t round) {
    return walk_cell(3, V, r, B, gamma, W1, W2, Q, scale, NULL, NULL, NULL, NULL, Gq, gs, gb, NULL, 0, h0, base,
                     anchor, T, uniforms, forced, forced_h, tokens, logits, states, mode, seed, round);
}

/* Domino's head: as oracle_walk_gru with Wih [3r][r + d] and the drafter's
 * hidden states H [B][gamma][d] bf16 appended to every step's input. */
int oracle_walk_domino(int V, int r, int d, int B, int gamma, const uint16_t* W1,
                       const uint16_t* W2, const int8_t* Q, const float* scale,
                       const uint16_t* Wih, const uint16_t* Whh, const float* bih, const float* bhh,
                       const uint16_t* H, const float* h0, const uint16_t* base, const int32_t* anchor,
                       const float* T, const float* uniforms, const int32_t* forced, const float* forced_h,
                       int32_t* tokens, uint16_t* logits, double* states, int mode, uint64_t seed,
                       uint32_t round) {
    return walk_cell(4, V, r, B, gamma, W1, W2, Q, scale, Wih, Whh, bih, bhh, NULL, NULL, NULL, H, d, h0, base,
                     anchor, T, uniforms, forced, forced_h, tokens, logits, states, mode, seed, round);
}

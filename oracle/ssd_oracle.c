/*
 * ssd_oracle.c -- plain fp64 CPU oracle of one verify-and-pre-speculate round of
 * Speculative Speculative Decoding (SSD) with the Saguaro algorithm.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library.  The product path
 * (the HIP library and its Python binding) never calls it, and this file shares no
 * code, header, table or constant generator with that path.
 *
 * Sources.  The method is described by two summaries of the paper "Speculative
 * Speculative Decoding" (Kumar, Dao, May):
 *   [zh]  gist.science/zh/paper/2603.03251, technical part, section 2 (Methodology:
 *         basic flow; Challenge 1 geometric fan-out; Challenge 2 Saguaro sampling;
 *         Challenge 3 fallback), section 1 (the round is lossless);
 *   [nl]  gist.science/nl/paper/2603.03251, technical part, section 2 (Kernprincipes)
 *         and section 3 A (geometric fan-out), 3 B (Saguaro sampling), 3 C (fallback).
 * The pages assert losslessness and name the parts; they print no formula.  The
 * formulas below are the standard lossless speculative-sampling construction that
 * the lossless claim requires (accept with min(1, p/q'), resample from the
 * normalised residual max(p - q', 0), sample from p when every draft token is
 * accepted), with q' the Saguaro-reweighted draft law the draft actually samples
 * from.  Every reading of a step the pages leave open is marked READING below.
 *
 * Arithmetic: every probability is computed in IEEE double.  bf16 and fp32 inputs
 * are widened exactly.  The code follows the steps in the order of the round:
 *   fan-out -> softmax -> speculation cache -> Saguaro reweight -> verify ->
 *   bonus (residual) -> cache lookup,
 * with one plain loop per definition; the only library routines used are qsort
 * (sorting candidate ids) and exp/pow/floor from libm.
 *
 * The functions that draw uniforms take b_base, the global index of the first
 * sequence passed in, so that a sub-batch of a larger batch draws the same uniforms
 * as it would inside the whole batch.
 *
 * Pins: the Python tests check these functions against closed forms, numpy
 * library routines, exact enumeration on tiny vocabularies and numpy's own
 * Philox4x64 generator.  No function here is "parity unpinned".
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_F32 0
#define ORC_BF16 1

/* Purposes of the counter-based uniforms (key word 1). */
#define ORC_PURPOSE_ACCEPT 0
#define ORC_PURPOSE_BONUS 1
#define ORC_PURPOSE_DRAFT 2
#define ORC_PURPOSE_FALLBACK 3

/* Data-dependent error bits (per sequence). */
#define ORC_ERR_TOKEN_RANGE 1   /* a draft token outside [0, V) */
#define ORC_ERR_QPRIME_ZERO 2   /* q'(d) == 0 for a tested draft token */
#define ORC_ERR_LEN_RANGE 4     /* accept_len outside [0, K] given to a step */
#define ORC_ERR_SLOT_RANGE 8    /* a hit whose slot lies outside [0, Bf) */
#define ORC_ERR_HIST_RANGE 16   /* a history length outside [0, ld_hist] */

/* Near-tie / range exception bits (per sequence), decided from fp64 values. */
#define ORC_E1_ACCEPT_TIE 1
#define ORC_E2_CDF_TIE 2
#define ORC_E3_DEGENERATE_RESIDUAL 4
#define ORC_E4_FANOUT_TIE 8
#define ORC_E5_TINY_PROB 16

#define ORC_TIE_EPS 1e-5   /* accept near-tie |u - p/q'|, as the method's parity rule states */
#define ORC_RESID_EPS 1e-5
#define ORC_FANOUT_EPS 1e-9
#define ORC_TINY 1e-30

/* Threads the OpenMP loops below use (1 without OpenMP). */
int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the thread count of the OpenMP loops (no effect without OpenMP). */
void orc_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------------- */
/* Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as
 * 1, 2, 3", SC'11): ten rounds of two 64x64->128 multiplications per round with the
 * published multipliers, the key bumped by the published Weyl constants between
 * rounds. */
static void mulhilo64(uint64_t a, uint64_t b, uint64_t* hi, uint64_t* lo) {
    unsigned __int128 p = (unsigned __int128)a * (unsigned __int128)b;
    *hi = (uint64_t)(p >> 64);
    *lo = (uint64_t)p;
}

void orc_philox4x64_10(const uint64_t ctr_in[4], const uint64_t key_in[2], uint64_t out[4]) {
    const uint64_t M0 = 0xD2E7470EE14C6C93ULL, M1 = 0xCA5A826395121157ULL;
    const uint64_t W0 = 0x9E3779B97F4A7C15ULL, W1 = 0xBB67AE8584CAA73BULL;
    uint64_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint64_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        uint64_t hi0, lo0, hi1, lo1;
        mulhilo64(M0, c0, &hi0, &lo0);
        mulhilo64(M1, c2, &hi1, &lo1);
        uint64_t n0 = hi1 ^ c1 ^ k0;
        uint64_t n1 = lo1;
        uint64_t n2 = hi0 ^ c3 ^ k1;
        uint64_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += W0; k1 += W1;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* First output word for key (seed, purpose) and counter (round, b, i, w3). */
static uint64_t philox_word(uint64_t seed, uint64_t round, int purpose, int64_t b, int64_t i, uint64_t w3) {
    uint64_t ctr[4] = {round, (uint64_t)b, (uint64_t)i, w3};
    uint64_t key[2] = {seed, (uint64_t)purpose};
    uint64_t out[4];
    orc_philox4x64_10(ctr, key, out);
    return out[0];
}

/* READING: the uniforms of (sequence, position, purpose) are the top 24 bits of the
 * first output word of counter (round, b, i, w) scaled by 2^-24, a value in [0, 1)
 * that fp32 holds exactly; w = 0 gives the uniform of a test or of a draw's block,
 * w = 1 the second uniform of a draw (the id within the block). */
double orc_uniform(uint64_t seed, uint64_t round, int purpose, int64_t b, int64_t i) {
    return (double)(philox_word(seed, round, purpose, b, i, 0) >> 40) * (1.0 / 16777216.0);
}

double orc_uniform2(uint64_t seed, uint64_t round, int purpose, int64_t b, int64_t i) {
    return (double)(philox_word(seed, round, purpose, b, i, 1) >> 40) * (1.0 / 16777216.0);
}

uint32_t orc_uniform_u32(uint64_t seed, uint64_t round, int purpose, int64_t b, int64_t i) {
    return (uint32_t)(philox_word(seed, round, purpose, b, i, 0) >> 32);
}

/* ------------------------------------------------------------------------- */
static double load_logit(const void* base, int dtype, int64_t idx) {
    if (dtype == ORC_F32) return (double)((const float*)base)[idx];
    uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Row r = b*(K+1) + i of a [B, K+1, V] logit tensor with row stride ld, widened to
 * double into out[V]. */
static void load_row(const void* logits, int dtype, int64_t ld, int64_t r, int V, double* out) {
    for (int x = 0; x < V; ++x) out[x] = load_logit(logits, dtype, r * ld + x);
}

/* ------------------------------------------------------------------------- */
/* Geometric fan-out ([zh] section 2, Challenge 1; [nl] section 3 A): the budget B_f
 * of cached bonus candidates is split over acceptance lengths k = 0..K in
 * proportion to r^k.  READING: integer shares by the largest-remainder method,
 * remainders compared largest first with ties to the lower k.
 * Returns 0 on success, -1 on bad arguments.  *min_gap (nullable) receives the
 * smallest distance between two remainders, for the fan-out near-tie case. */
int orc_fanout(int K, int Bf, double r, int32_t* F, double* min_gap) {
    if (K < 1 || Bf < 0 || !(r > 0.0) || !(r <= 1.0)) return -1;
    double f[64], rem[64], wsum = 0.0;
    int given[64];
    if (K + 1 > 64) return -1;
    for (int k = 0; k <= K; ++k) wsum += pow(r, (double)k);
    int total = 0;
    for (int k = 0; k <= K; ++k) {
        f[k] = (double)Bf * pow(r, (double)k) / wsum;
        F[k] = (int32_t)floor(f[k]);
        rem[k] = f[k] - floor(f[k]);
        given[k] = 0;
        total += F[k];
    }
    int left = Bf - total;
    for (int n = 0; n < left; ++n) {
        int best = -1;
        for (int k = 0; k <= K; ++k) {
            if (given[k]) continue;
            if (best < 0 || rem[k] > rem[best]) best = k;
        }
        F[best] += 1;
        given[best] = 1;
    }
    if (min_gap) {
        double g = INFINITY;
        for (int a = 0; a <= K; ++a)
            for (int c = a + 1; c <= K; ++c) {
                double d = fabs(rem[a] - rem[c]);
                if (d < g) g = d;
            }
        *min_gap = g;
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Temperature softmax of one row ([zh] section 2 and section 4 name temperature as
 * an axis of the method; the round consumes p = softmax(z_p / T) and
 * q = softmax(z_q / T)).  READING: T = 0 is the greedy limit, a one-hot law on the
 * lowest id among the maxima. */
static void softmax_row(const double* z, int V, double T, double* m_out, double* s_out,
                        int32_t* arg_out, double* prob /* nullable */) {
    double m = z[0];
    int arg = 0;
    for (int x = 1; x < V; ++x)
        if (z[x] > m) { m = z[x]; arg = x; }
    double s;
    if (T > 0.0) {
        s = 0.0;
        for (int x = 0; x < V; ++x) s += exp((z[x] - m) / T);
        if (prob)
            for (int x = 0; x < V; ++x) prob[x] = exp((z[x] - m) / T) / s;
    } else {
        s = 1.0;
        if (prob)
            for (int x = 0; x < V; ++x) prob[x] = (x == arg) ? 1.0 : 0.0;
    }
    *m_out = m;
    *s_out = s;
    *arg_out = arg;
}

/* Probability of token x in a row whose statistics are (m, s, arg). */
static double row_prob(double zx, int x, double m, double s, int arg, double T) {
    if (T > 0.0) return exp((zx - m) / T) / s;
    return (x == arg) ? 1.0 : 0.0;
}

void orc_softmax(int B, int K, int V, int64_t ld, int dtype, const void* logits, double T,
                 double* row_max, double* row_sum, int32_t* row_argmax, double* probs) {
    const int64_t R = (int64_t)B * (K + 1);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < R; ++r) {
        double* z = (double*)malloc(sizeof(double) * V);
        load_row(logits, dtype, ld, r, V, z);
        softmax_row(z, V, T, &row_max[r], &row_sum[r], &row_argmax[r],
                    probs ? probs + r * (int64_t)V : NULL);
        free(z);
    }
}

/* ------------------------------------------------------------------------- */
/* Speculation cache ([zh] section 2, flow step 2-3 and Challenge 1; [nl] section 2
 * and 3 A): an outcome is (k accepted, bonus token); for each k the cache holds
 * F_k candidate bonus tokens.  READING: the candidates for length k are the F_k ids
 * of largest draft logit z_q[b, k, .] (ties to the lower id), i.e. the top-F of the
 * draft law at that position before reweighting, stored in that order at
 * cache_ids[b, O_k .. O_k + F_k - 1] with O_k = F_0 + ... + F_{k-1}.  The cached
 * draft mass is M_k = sum over the candidates of q_k(x). */
typedef struct { double v; int id; } orc_cand;

static int cand_cmp(const void* pa, const void* pb) {
    const orc_cand* a = (const orc_cand*)pa;
    const orc_cand* b = (const orc_cand*)pb;
    if (a->v > b->v) return -1;
    if (a->v < b->v) return 1;
    return (a->id < b->id) ? -1 : (a->id > b->id);
}

void orc_build_cache(int B, int K, int V, int64_t ld, int dtype, const void* q_logits, double T,
                     const int32_t* F, int Bf, int32_t* cache_ids, double* cache_mass) {
    (void)Bf;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bk = 0; bk < (int64_t)B * (K + 1); ++bk) {
        int b = (int)(bk / (K + 1)), k = (int)(bk % (K + 1));
        int Ok = 0;
        for (int j = 0; j < k; ++j) Ok += F[j];
        double* z = (double*)malloc(sizeof(double) * V);
        orc_cand* c = (orc_cand*)malloc(sizeof(orc_cand) * V);
        load_row(q_logits, dtype, ld, bk, V, z);
        double m, s;
        int32_t arg;
        softmax_row(z, V, T, &m, &s, &arg, NULL);
        for (int x = 0; x < V; ++x) { c[x].v = z[x]; c[x].id = x; }
        qsort(c, V, sizeof(orc_cand), cand_cmp);
        double M = 0.0;
        for (int j = 0; j < F[k]; ++j) {
            cache_ids[(int64_t)b * Bf + Ok + j] = c[j].id;
            M += row_prob(z[c[j].id], c[j].id, m, s, arg, T);
        }
        cache_mass[bk] = M;
        free(c);
        free(z);
    }
}

/* ------------------------------------------------------------------------- */
/* Saguaro sampling ([zh] section 2, Challenge 2; [nl] section 3 B): the draft law
 * is reweighted by a factor C on the cached top-F tokens and renormalised, which
 * moves residual mass onto the cached tokens.  READING: C in (0, 1],
 *   Z_k = 1 - (1 - C) M_k,   q'_k(x) = q_k(x) * (C if x in S_k else 1) / Z_k. */
static int in_cache(const int32_t* ids, int n, int x) {
    for (int j = 0; j < n; ++j)
        if (ids[j] == x) return 1;
    return 0;
}

void orc_saguaro(int B, int K, int V, int64_t ld, int dtype, const void* q_logits, double T,
                 const int32_t* F, int Bf, const int32_t* cache_ids, const double* cache_mass,
                 double C, double* Z, double* q_prime /* nullable [B, K+1, V] */) {
    const int64_t R = (int64_t)B * (K + 1);
    for (int64_t r = 0; r < R; ++r) Z[r] = 1.0 - (1.0 - C) * cache_mass[r];
    if (!q_prime) return;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < R; ++r) {
        int b = (int)(r / (K + 1)), k = (int)(r % (K + 1));
        int Ok = 0;
        for (int j = 0; j < k; ++j) Ok += F[j];
        const int32_t* S = cache_ids + (int64_t)b * Bf + Ok;
        double* z = (double*)malloc(sizeof(double) * V);
        load_row(q_logits, dtype, ld, r, V, z);
        double m, s;
        int32_t arg;
        softmax_row(z, V, T, &m, &s, &arg, NULL);
        for (int x = 0; x < V; ++x) {
            double w = in_cache(S, F[k], x) ? C : 1.0;
            q_prime[r * V + x] = row_prob(z[x], x, m, s, arg, T) * w / Z[r];
        }
        free(z);
    }
}

/* ------------------------------------------------------------------------- */
/* Draws.  READING (the pages fix no sampling mechanism; any exact one keeps the round
 * lossless): a draw from weights w over ids 0..V-1 takes two uniforms of its
 * (sequence, position, purpose), u1 (last counter word 0) and u2 (last counter word 1).  The ids are
 * split into blocks of ORC_BLOCK consecutive ids; u1 picks the block -- the smallest
 * block whose running sum of block masses exceeds u1 times their total -- and u2 the
 * id within it -- the smallest id whose running sum within the block exceeds u2 times
 * the block's mass.  Strict ">" over ascending order, so no zero weight is chosen; if
 * rounding leaves no crossing, the last block (id) of positive mass is taken.  The
 * law is w / sum(w) exactly as for one inverse CDF over all ids; two levels keep
 * each decision well conditioned: a block boundary is resolved against the whole
 * row's mass, an id boundary only against its block's. */
#define ORC_BLOCK 512

/* Inverse-CDF selection over n weights: the smallest j whose running sum exceeds
 * u * total (ascending j); if rounding leaves no such j, the largest j with w_j > 0.
 * *gap (nullable) receives min(|C(j*) - u|, |C(j*-1) - u|), C(j) = cumsum_j / total:
 * the distance of u to the two steps around j*. */
static int inverse_cdf(const double* w, int n, double total, double u, double* gap) {
    double target = u * total, run = 0.0, prev = 0.0;
    int pick = -1;
    for (int j = 0; j < n; ++j) {
        prev = run;
        run += w[j];
        if (run > target) { pick = j; break; }
    }
    if (pick < 0) {
        for (int j = n - 1; j >= 0; --j)
            if (w[j] > 0.0) { pick = j; break; }
        if (pick < 0) pick = n - 1;
        prev = total - w[pick];
        run = total;
    }
    if (gap) {
        double a = fabs(run / total - u), c = fabs(prev / total - u);
        *gap = a < c ? a : c;
    }
    return pick;
}

/* Block masses of w (ascending ids within a block), returning their sum. */
static double block_masses(const double* w, int V, double* W) {
    const int nb = (V + ORC_BLOCK - 1) / ORC_BLOCK;
    double tot = 0.0;
    for (int b = 0; b < nb; ++b) {
        const int e = (b + 1) * ORC_BLOCK < V ? (b + 1) * ORC_BLOCK : V;
        double m = 0.0;
        for (int x = b * ORC_BLOCK; x < e; ++x) m += w[x];
        W[b] = m;
        tot += m;
    }
    return tot;
}

/* The two-level draw: returns the id; *blk the block; gap[0], gap[1] (nullable) the
 * distances of u1 and u2 to the steps around the block and around the id. */
static int draw_two_level(const double* w, int V, double u1, double u2, int* blk, double* gap) {
    const int nb = (V + ORC_BLOCK - 1) / ORC_BLOCK;
    double* W = (double*)malloc(sizeof(double) * nb);
    const double tot = block_masses(w, V, W);
    const int b = inverse_cdf(W, nb, tot, u1, gap ? &gap[0] : NULL);
    const int x0 = b * ORC_BLOCK;
    const int n = (x0 + ORC_BLOCK < V ? x0 + ORC_BLOCK : V) - x0;
    const int j = inverse_cdf(w + x0, n, W[b], u2, gap ? &gap[1] : NULL);
    free(W);
    if (blk) *blk = b;
    return x0 + j;
}

/* Near-tie of a draw (E2).  A decision flips only when its uniform lies within the
 * arithmetic error of the GPU path's running sums from a step; the half-width of that
 * band is a quantity of the parity rule, not of the method (the oracle is exact up to
 * fp64 rounding).  draw_bands derives it per draw and per level. */
#define ORC_CDF_SIGMAS 6.0  /* random part of the E2 band, in standard deviations */

/* READING (parity rule): the GPU path applies the temperature as the fp32 scale
 * c = fp32(log2(e) / fp32(T)), so it samples at the temperature log2(e) / c. */
static double device_temperature(double T) {
    const float Tf = (float)T;
    const float c = (float)(1.4426950408889634 / (double)Tf);
    return 1.4426950408889634 / (double)c;
}

/* Standard deviation of the relative error of one GPU term 2^e (e the exponent
 * relative to the row maximum, in bits), for errors spread evenly within their
 * bounds (rms = bound / sqrt 3): exp2 within one fp32 ulp (2^-23), and the one
 * rounding of the fp32 exponent (half an ulp of e, times ln 2). */
static double term_err(double e) {
    const double a = 0x1p-23, b = 0x1p-24 * 0.6931471805599453 * (fabs(e) + 1.0);
    return sqrt((a * a + b * b) / 3.0);
}

/* The laws of one draw at temperature Tx, from the widened rows zp (target) and zq
 * (draft) and the nS cached ids S of the draft row:
 *   mode 0: w = p (the target row: bonus after all K accepted);
 *   mode 1: w = max(p - q', 0) (the residual after a rejection);
 *   mode 2: w = q' (the draft sampler);
 * with q' = q (C on S, else 1) / (1 - (1 - C) M).  Writes w, and the absolute term
 * error bounds a = p d(e_p), c = q' d(e_q) of each id (0 where the term is not part
 * of the law, and for the residual where p - q' cannot turn positive within them).
 * Returns sum w. */
static double draw_laws(int mode, const double* zp, const double* zq, int V, double Tx, const int32_t* S,
                        int nS, double C, double* w, double* a, double* c) {
    const double L2E = 1.4426950408889634;
    double mp = -INFINITY, mq = -INFINITY, sp = 0.0, sq = 0.0, Z = 1.0;
    if (mode != 2) {
        for (int x = 0; x < V; ++x) if (zp[x] > mp) mp = zp[x];
        for (int x = 0; x < V; ++x) sp += exp((zp[x] - mp) / Tx);
    }
    if (mode != 0) {
        for (int x = 0; x < V; ++x) if (zq[x] > mq) mq = zq[x];
        for (int x = 0; x < V; ++x) sq += exp((zq[x] - mq) / Tx);
        double M = 0.0;
        for (int j = 0; j < nS; ++j) M += exp((zq[S[j]] - mq) / Tx) / sq;
        Z = 1.0 - (1.0 - C) * M;
    }
    double total = 0.0;
    for (int x = 0; x < V; ++x) {
        double p = 0.0, qp = 0.0, ea = 0.0, ec = 0.0;
        if (mode != 2) {
            p = exp((zp[x] - mp) / Tx) / sp;
            ea = p > 0.0 ? p * term_err((zp[x] - mp) / Tx * L2E) : 0.0;
        }
        if (mode != 0) {
            qp = exp((zq[x] - mq) / Tx) / sq * (in_cache(S, nS, x) ? C : 1.0) / Z;
            ec = qp > 0.0 ? qp * term_err((zq[x] - mq) / Tx * L2E) : 0.0;
        }
        if (mode == 0) w[x] = p;
        else if (mode == 2) w[x] = qp;
        else {
            w[x] = p - qp > 0.0 ? p - qp : 0.0;
            if (!(p - qp > -(ea + ec))) ea = ec = 0.0;
        }
        a[x] = ea;
        c[x] = ec;
        total += w[x];
    }
    return total;
}

/* The CDF values of a draw just below and at its pick: block level (over block
 * masses, around block b) and id level (within block b, around id j). */
static void draw_cdf(const double* w, int V, int b, int j, double out[4]) {
    const int nb = (V + ORC_BLOCK - 1) / ORC_BLOCK;
    double* W = (double*)malloc(sizeof(double) * nb);
    const double tot = block_masses(w, V, W);
    double run = 0.0;
    for (int k = 0; k < b; ++k) run += W[k];
    out[0] = run / tot;
    out[1] = (run + W[b]) / tot;
    double r2 = 0.0;
    for (int x = b * ORC_BLOCK; x < j; ++x) r2 += w[x];
    out[2] = r2 / W[b];
    out[3] = (r2 + w[j]) / W[b];
    free(W);
}

/* Half-widths of the E2 bands of one draw (mode as for draw_laws) that picked id j in
 * block b at temperature T: band[0] for u1 (block level), band[1] for u2 (id level).
 * Each is
 *   cdf_eps
 *   + the shift of the level's normalised CDF at the two steps around the pick
 *     between the temperature the GPU path samples at and T (both exact, in fp64);
 *   + ORC_CDF_SIGMAS standard deviations of the GPU path's CDF error from
 *     independent per-term errors of standard deviation term_err: a random walk over the ids
 *     that can carry weight, sqrt(sum a^2 + c^2) over the row divided by its mass
 *     (block level), over the block divided by the block's mass (id level).
 * (The normalisers' own errors are means over many terms and far smaller.) */
static void draw_bands(int mode, const double* zp, const double* zq, int V, double T, const int32_t* S, int nS,
                       double C, int b, int j, double cdf_eps, double band[2]) {
    double* w = (double*)malloc(sizeof(double) * V);
    double* a = (double*)malloc(sizeof(double) * V);
    double* c = (double*)malloc(sizeof(double) * V);
    double cd[2][4];
    for (int pass = 0; pass < 2; ++pass) {
        const double Tx = pass == 0 ? T : device_temperature(T);
        double total = draw_laws(mode, zp, zq, V, Tx, S, nS, C, w, a, c);
        if (mode == 1 && !(total > 0.0))  /* degenerate residual: the draw falls back to p */
            total = draw_laws(0, zp, zq, V, Tx, S, nS, C, w, a, c);
        draw_cdf(w, V, b, j, cd[pass]);
        if (pass == 0) {
            double vr = 0.0, vb = 0.0, mb = 0.0;
            const int e = (b + 1) * ORC_BLOCK < V ? (b + 1) * ORC_BLOCK : V;
            for (int x = 0; x < V; ++x) vr += a[x] * a[x] + c[x] * c[x];
            for (int x = b * ORC_BLOCK; x < e; ++x) {
                vb += a[x] * a[x] + c[x] * c[x];
                mb += w[x];
            }
            band[0] = cdf_eps + ORC_CDF_SIGMAS * sqrt(vr) / total;
            band[1] = cdf_eps + ORC_CDF_SIGMAS * sqrt(vb) / mb;
        }
    }
    for (int l = 0; l < 2; ++l) {
        const double d0 = fabs(cd[1][2 * l] - cd[0][2 * l]), d1 = fabs(cd[1][2 * l + 1] - cd[0][2 * l + 1]);
        band[l] += d0 > d1 ? d0 : d1;
    }
    free(c);
    free(a);
    free(w);
}

/* Draft tokens for a synthetic round (harness step, not part of the timed round):
 * the draft samples d_i from its Saguaro-reweighted law q'_i ([zh] section 2,
 * Challenge 2: the reweighting is applied while the draft samples) by the two-level
 * draw with the uniforms of (b, i, DRAFT).  At T = 0 the draft is greedy. */
void orc_draft_sample(int B, int K, int V, int64_t ld, int dtype, const void* q_logits, double T,
                      const int32_t* F, int Bf, const int32_t* cache_ids, const double* Z, double C,
                      uint64_t seed, uint64_t round, int64_t b_base, double cdf_eps, int32_t* draft,
                      uint8_t* tie_flags /* [B,K] */, double* e2 /* nullable [B,K][4] */) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bi = 0; bi < (int64_t)B * K; ++bi) {
        int b = (int)(bi / K), i = (int)(bi % K);
        int64_t r = (int64_t)b * (K + 1) + i;
        int Oi = 0;
        for (int j = 0; j < i; ++j) Oi += F[j];
        const int32_t* S = cache_ids + (int64_t)b * Bf + Oi;
        double* z = (double*)malloc(sizeof(double) * V);
        double* w = (double*)malloc(sizeof(double) * V);
        load_row(q_logits, dtype, ld, r, V, z);
        double m, s;
        int32_t arg;
        softmax_row(z, V, T, &m, &s, &arg, NULL);
        uint8_t flag = 0;
        double info[4] = {INFINITY, 0.0, INFINITY, 0.0};
        if (T > 0.0) {
            for (int x = 0; x < V; ++x)
                w[x] = row_prob(z[x], x, m, s, arg, T) * (in_cache(S, F[i], x) ? C : 1.0) / Z[r];
            const double u1 = orc_uniform(seed, round, ORC_PURPOSE_DRAFT, b_base + b, i);
            const double u2 = orc_uniform2(seed, round, ORC_PURPOSE_DRAFT, b_base + b, i);
            double gap[2], band[2];
            int blk;
            draft[bi] = draw_two_level(w, V, u1, u2, &blk, gap);
            draw_bands(2, NULL, z, V, T, S, F[i], C, blk, draft[bi], cdf_eps, band);
            if (gap[0] < band[0] || gap[1] < band[1]) flag = ORC_E2_CDF_TIE;
            info[0] = gap[0]; info[1] = band[0]; info[2] = gap[1]; info[3] = band[1];
        } else {
            draft[bi] = arg;
        }
        if (e2)
            for (int l = 0; l < 4; ++l) e2[bi * 4 + l] = info[l];
        if (tie_flags) tie_flags[bi] = flag;
        free(w);
        free(z);
    }
}

/* ------------------------------------------------------------------------- */
/* Lossless verification ([zh] section 2, flow steps 2 and 4; [nl] section 2): the
 * target checks the K draft tokens of a sequence in order; the outcome is the
 * accepted length k.  READING (standard lossless speculative sampling):
 *   ratio_i = p_i(d_i) / q'_i(d_i), accept iff U(seed, round, b, i, ACCEPT) < ratio_i,
 *   k = first rejected position, or K when all are accepted;
 *   accept_prob_i = min(1, ratio_i).  At T = 0: accept iff d_i = argmax p_i.
 * Per sequence, e1 receives the accept near-tie and tiny-probability bits for the
 * positions tested (0 .. min(k, K-1)). */
void orc_verify(int B, int K, int V, int64_t ld, int dtype, const void* p_logits,
                const void* q_logits, double T, const int32_t* draft,
                const double* p_max, const double* p_sum, const int32_t* p_arg,
                const double* q_max, const double* q_sum, const int32_t* q_arg,
                const int32_t* F, int Bf, const int32_t* cache_ids, const double* Z, double C,
                uint64_t seed, uint64_t round, int64_t b_base, int32_t* accept_len,
                double* accept_prob, int32_t* err, uint8_t* exc) {
    for (int b = 0; b < B; ++b) {
        int k = K, e = 0, x_flags = 0;
        int Oi = 0;
        for (int i = 0; i < K; ++i) {
            int64_t r = (int64_t)b * (K + 1) + i;
            int d = draft[(int64_t)b * K + i];
            const int32_t* S = cache_ids + (int64_t)b * Bf + Oi;
            Oi += F[i];
            double ratio;
            int ok = 1;
            if (d < 0 || d >= V) {
                e |= ORC_ERR_TOKEN_RANGE;
                ok = 0;
                ratio = 0.0;
            } else if (T > 0.0) {
                const double zpd = load_logit(p_logits, dtype, r * ld + d);
                const double zqd = load_logit(q_logits, dtype, r * ld + d);
                double p = row_prob(zpd, d, p_max[r], p_sum[r], p_arg[r], T);
                double q = row_prob(zqd, d, q_max[r], q_sum[r], q_arg[r], T);
                double qp = q * (in_cache(S, F[i], d) ? C : 1.0) / Z[r];
                if (qp <= 0.0) {
                    e |= ORC_ERR_QPRIME_ZERO;
                    ok = 0;
                    ratio = 0.0;
                } else {
                    ratio = p / qp;
                }
                if (k == K) {
                    /* no earlier rejection: this position is tested */
                    double u = orc_uniform(seed, round, ORC_PURPOSE_ACCEPT, b_base + b, i);
                    if (fabs(u - ratio) < ORC_TIE_EPS) x_flags |= ORC_E1_ACCEPT_TIE;
                    /* a finite logit whose probability is this small is at the edge of
                     * the working range; a masked (-inf) logit has probability exactly 0
                     * in any precision, so its test is exact and not flagged */
                    if ((p < ORC_TINY && !isinf(zpd)) || (qp < ORC_TINY && !isinf(zqd)))
                        x_flags |= ORC_E5_TINY_PROB;
                }
            } else {
                ratio = (d == p_arg[r]) ? 1.0 : 0.0;
            }
            if (accept_prob) accept_prob[(int64_t)b * K + i] = ratio < 1.0 ? ratio : 1.0;
            if (k == K) {
                int acc;
                if (!ok) acc = 0;
                else if (T > 0.0) acc = orc_uniform(seed, round, ORC_PURPOSE_ACCEPT, b_base + b, i) < ratio;
                else acc = (d == p_arg[r]);
                if (!acc) k = i;
            }
        }
        accept_len[b] = k;
        if (err) err[b] |= e;
        if (exc) exc[b] |= (uint8_t)x_flags;
    }
}

/* ------------------------------------------------------------------------- */
/* Bonus token ([zh] section 2, flow step 2 and Challenge 2: the bonus comes from the
 * residual distribution; [nl] section 3 B).  READING (standard): with k the accepted
 * length,
 *   k < K:  w(x) = max(p_k(x) - q'_k(x), 0), Z_r = sum w; if Z_r == 0 (only through
 *           rounding) w = p_k;
 *   k = K:  w = p_K, Z_r = sum w;
 * bonus = the two-level draw from w with the uniforms of (b, k, BONUS).  At T = 0 the
 * bonus is argmax p_k.  resid (nullable [B, V]) receives w, resid_mass receives Z_r. */
void orc_residual_sample(int B, int K, int V, int64_t ld, int dtype, const void* p_logits,
                         const void* q_logits, double T,
                         const double* p_max, const double* p_sum, const int32_t* p_arg,
                         const double* q_max, const double* q_sum, const int32_t* q_arg,
                         const int32_t* F, int Bf, const int32_t* cache_ids, const double* Z, double C,
                         const int32_t* accept_len, uint64_t seed, uint64_t round, int64_t b_base,
                         double cdf_eps, int32_t* bonus, double* resid_mass, double* resid, int32_t* err,
                         uint8_t* exc, double* e2 /* nullable [B][4] */) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
        int k = accept_len[b];
        if (e2) {
            e2[b * 4 + 0] = e2[b * 4 + 2] = INFINITY;
            e2[b * 4 + 1] = e2[b * 4 + 3] = 0.0;
        }
        if (k < 0 || k > K) {
            bonus[b] = -1;
            if (resid_mass) resid_mass[b] = 0.0;
            if (err) err[b] |= ORC_ERR_LEN_RANGE;
            continue;
        }
        int64_t r = (int64_t)b * (K + 1) + k;
        if (!(T > 0.0)) {
            bonus[b] = p_arg[r];
            if (resid_mass) resid_mass[b] = 1.0;
            if (resid)
                for (int x = 0; x < V; ++x) resid[(int64_t)b * V + x] = (x == p_arg[r]) ? 1.0 : 0.0;
            continue;
        }
        int Ok = 0;
        for (int j = 0; j < k; ++j) Ok += F[j];
        const int32_t* S = cache_ids + (int64_t)b * Bf + Ok;
        double* w = (double*)malloc(sizeof(double) * V);
        double Zr = 0.0;
        for (int x = 0; x < V; ++x) {
            double p = row_prob(load_logit(p_logits, dtype, r * ld + x), x, p_max[r], p_sum[r], p_arg[r], T);
            if (k < K) {
                double q = row_prob(load_logit(q_logits, dtype, r * ld + x), x, q_max[r], q_sum[r], q_arg[r], T);
                double qp = q * (in_cache(S, F[k], x) ? C : 1.0) / Z[r];
                w[x] = p - qp > 0.0 ? p - qp : 0.0;
            } else {
                w[x] = p;
            }
            Zr += w[x];
        }
        uint8_t x_flags = 0;
        if (k < K && Zr < ORC_RESID_EPS) x_flags |= ORC_E3_DEGENERATE_RESIDUAL;
        if (Zr <= 0.0) {
            Zr = 0.0;
            for (int x = 0; x < V; ++x) {
                w[x] = row_prob(load_logit(p_logits, dtype, r * ld + x), x, p_max[r], p_sum[r], p_arg[r], T);
                Zr += w[x];
            }
        }
        const double u1 = orc_uniform(seed, round, ORC_PURPOSE_BONUS, b_base + b, k);
        const double u2 = orc_uniform2(seed, round, ORC_PURPOSE_BONUS, b_base + b, k);
        double gap[2], band[2];
        int blk;
        bonus[b] = draw_two_level(w, V, u1, u2, &blk, gap);
        double* zp = (double*)malloc(sizeof(double) * V);
        double* zq = (double*)malloc(sizeof(double) * V);
        load_row(p_logits, dtype, ld, r, V, zp);
        load_row(q_logits, dtype, ld, r, V, zq);
        draw_bands(k < K ? 1 : 0, zp, zq, V, T, S, F[k], C, blk, bonus[b], cdf_eps, band);
        free(zq);
        free(zp);
        if (gap[0] < band[0] || gap[1] < band[1]) x_flags |= ORC_E2_CDF_TIE;
        if (e2) {
            e2[b * 4 + 0] = gap[0];
            e2[b * 4 + 1] = band[0];
            e2[b * 4 + 2] = gap[1];
            e2[b * 4 + 3] = band[1];
        }
        if (resid_mass) resid_mass[b] = Zr;
        if (resid)
            for (int x = 0; x < V; ++x) resid[(int64_t)b * V + x] = w[x];
        if (exc) exc[b] |= x_flags;
        free(w);
    }
}

/* ------------------------------------------------------------------------- */
/* Cache lookup ([zh] section 2, flow step 4: hit returns the pre-speculated tokens,
 * miss falls back; Challenge 3: at large batch the fallback is a fast speculator,
 * e.g. random tokens; [nl] section 2 and 3 C).  hit = bonus in S_k, slot = O_k +
 * position in S_k or -1.  READING: on a miss with the uniform fallback the next
 * draft is K tokens floor(U32 * V / 2^32) with U32 = U32(seed, round, b, j,
 * FALLBACK); otherwise the fallback tokens are -1. */
void orc_cache_lookup(int B, int K, int V, const int32_t* F, int Bf, const int32_t* cache_ids,
                      const int32_t* accept_len, const int32_t* bonus, int fallback_uniform,
                      uint64_t seed, uint64_t round, int64_t b_base, uint8_t* hit, int32_t* slot,
                      int32_t* fallback_tokens, int32_t* err) {
    for (int b = 0; b < B; ++b) {
        int k = accept_len[b];
        int h = 0, sl = -1;
        if (k < 0 || k > K) {
            if (err) err[b] |= ORC_ERR_LEN_RANGE;
        } else {
            int Ok = 0;
            for (int j = 0; j < k; ++j) Ok += F[j];
            for (int j = 0; j < F[k]; ++j)
                if (cache_ids[(int64_t)b * Bf + Ok + j] == bonus[b]) { h = 1; sl = Ok + j; break; }
        }
        hit[b] = (uint8_t)h;
        slot[b] = sl;
        for (int j = 0; j < K; ++j) {
            int32_t t = -1;
            if (!h && fallback_uniform) {
                uint64_t x = orc_uniform_u32(seed, round, ORC_PURPOSE_FALLBACK, b_base + b, j);
                t = (int32_t)((x * (uint64_t)V) >> 32);
            }
            fallback_tokens[(int64_t)b * K + j] = t;
        }
    }
}

/* ------------------------------------------------------------------------- */
/* Next round's draft from the speculation cache ([zh] section 2 basic flow, step 4:
 * on a hit the pre-speculated tokens are returned at once; on a miss the fallback
 * speculator takes over; [nl] section 2 Kernprincipes).
 * READING: the cache holds, for every cached outcome (slot = O_k + rank), one
 * continuation of K tokens, values[b][slot][0..K-1].  On a hit the next draft is that
 * continuation; on a miss it is the fallback tokens of the lookup (the uniform random
 * speculator's K tokens, or -1 = left to the caller's primary speculator).  A hit
 * whose slot lies outside [0, Bf) is invalid input: error bit, next draft -1. */
void orc_cache_gather(int B, int K, int Bf, const int32_t* values, const uint8_t* hit,
                      const int32_t* slot, const int32_t* fallback_tokens, int32_t* next_draft,
                      int32_t* err) {
    for (int b = 0; b < B; ++b) {
        for (int j = 0; j < K; ++j) {
            int32_t t;
            if (!hit[b]) {
                t = fallback_tokens[(int64_t)b * K + j];
            } else if (slot[b] < 0 || slot[b] >= Bf) {
                t = -1;
                if (err && j == 0) err[b] |= ORC_ERR_SLOT_RANGE;
            } else {
                t = values[((int64_t)b * Bf + slot[b]) * K + j];
            }
            next_draft[(int64_t)b * K + j] = t;
        }
    }
}

/* ------------------------------------------------------------------------- */
/* Coverage statistics for choosing the fan-out ([zh] section 2 Challenge 1 and [nl]
 * section 3 A call the fan-out the solution of a constrained optimisation over
 * acceptance lengths).  READING: what the optimisation needs from each verified
 * round is, per sequence, the acceptance length k and the rank of the bonus token
 * within the draft row k in the cache order (larger logit first, ties to the lower
 * id): the bonus would have been a hit with any F_k > rank.
 *   rank = #{x : z_q[k](x) > z_q[k](t)} + #{x < t : z_q[k](x) = z_q[k](t)},
 * t the bonus.  hist[k][min(rank, R)] counts the sequences (bin R: rank >= R).
 * A sequence with k outside [0, K] or t outside [0, V) gets rank -1 and is not
 * counted.  hist (nullable) is accumulated, not cleared. */
void orc_bonus_rank(int B, int K, int V, int64_t ld, int dtype, const void* q_logits,
                    const int32_t* accept_len, const int32_t* bonus, int R, int32_t* rank_out,
                    uint32_t* hist) {
    for (int b = 0; b < B; ++b) {
        const int k = accept_len[b], t = bonus[b];
        if (k < 0 || k > K || t < 0 || t >= V) {
            if (rank_out) rank_out[b] = -1;
            continue;
        }
        const int64_t row = ((int64_t)b * (K + 1) + k) * ld;
        const double zt = load_logit(q_logits, dtype, row + t);
        int64_t rank = 0;
        for (int x = 0; x < V; ++x) {
            const double zx = load_logit(q_logits, dtype, row + x);
            if (zx > zt || (zx == zt && x < t)) ++rank;
        }
        if (rank_out) rank_out[b] = (int32_t)rank;
        if (hist) hist[(int64_t)k * (R + 1) + (rank < R ? rank : R)] += 1u;
    }
}

/* ------------------------------------------------------------------------- */
/* n-gram fallback speculator ([zh] section 2 Challenge 3 and [nl] section 3 C name an
 * n-gram model, next to random tokens, as the fast, low-quality speculator that a
 * large batch falls back to on a cache miss).  The pages describe it no further.
 * READING (prompt lookup over the sequence's own context):
 *   context   c = hist[b][0 .. len_b) ++ draft[b][0 .. k) ++ [bonus[b]], length L,
 *             k = accept_len[b] (the tokens the verified round appended);
 *   match     the largest n in [n_min, n_max] for which the last n tokens of c also
 *             occur earlier, ending at some e <= L - 2; among those occurrences the
 *             latest (largest e);
 *   proposal  the K tokens that followed that occurrence, t_j = x[e + 1 + j] over
 *             x = c ++ t (so when fewer than K tokens follow the occurrence the copy
 *             runs on over the tokens just proposed, with period L - 1 - e);
 *   no match  the uniform random tokens of the cache lookup's uniform fallback,
 *             (U32(seed, round, b, j, FALLBACK) * V) >> 32.
 * Only sequences that missed are served (all when hit is NULL); a hit gets tokens -1
 * and leaves next_draft alone, as the cache gather already wrote it.  A length k
 * outside [0, K] or len_b outside [0, ld_hist] is invalid input: error bit, tokens
 * -1.  match_n gets n (0 when there is no match), match_end gets e (-1). */
void orc_ngram_fallback(int B, int K, int V, const int32_t* hist, int64_t ld_hist,
                        const int32_t* hist_len, const int32_t* draft, const int32_t* accept_len,
                        const int32_t* bonus, const uint8_t* hit, int n_min, int n_max,
                        uint64_t seed, uint64_t round, int64_t b_base, int32_t* tokens,
                        int32_t* next_draft, int32_t* match_n, int32_t* match_end, int32_t* err) {
    for (int b = 0; b < B; ++b) {
        int32_t* out = tokens + (int64_t)b * K;
        int n_found = 0, e_found = -1;
        for (int j = 0; j < K; ++j) out[j] = -1;
        if (hit && hit[b]) {
            if (match_n) match_n[b] = 0;
            if (match_end) match_end[b] = -1;
            continue;
        }
        const int k = accept_len[b], len = hist_len[b];
        int bad = 0;
        if (k < 0 || k > K) { bad = 1; if (err) err[b] |= ORC_ERR_LEN_RANGE; }
        if (len < 0 || (int64_t)len > ld_hist) { bad = 1; if (err) err[b] |= ORC_ERR_HIST_RANGE; }
        if (!bad) {
            const int L = len + k + 1;
            int32_t* c = (int32_t*)malloc(sizeof(int32_t) * (size_t)(L + K));
            for (int x = 0; x < len; ++x) c[x] = hist[(int64_t)b * ld_hist + x];
            for (int x = 0; x < k; ++x) c[len + x] = draft[(int64_t)b * K + x];
            c[L - 1] = bonus[b];
            for (int n = n_max; n >= n_min && !n_found; --n) {
                if (n > L - 1) continue;  /* an earlier occurrence needs n <= e + 1 <= L - 1 */
                for (int e = L - 2; e >= n - 1; --e) {
                    int same = 1;
                    for (int j = 0; j < n && same; ++j) same = c[e - j] == c[L - 1 - j];
                    if (same) { n_found = n; e_found = e; break; }
                }
            }
            if (n_found) {
                for (int j = 0; j < K; ++j) c[L + j] = c[e_found + 1 + j];
                for (int j = 0; j < K; ++j) out[j] = c[L + j];
            } else {
                for (int j = 0; j < K; ++j) {
                    uint64_t x = orc_uniform_u32(seed, round, ORC_PURPOSE_FALLBACK, b_base + b, j);
                    out[j] = (int32_t)((x * (uint64_t)V) >> 32);
                }
            }
            free(c);
        }
        if (match_n) match_n[b] = n_found;
        if (match_end) match_end[b] = e_found;
        if (next_draft)
            for (int j = 0; j < K; ++j) next_draft[(int64_t)b * K + j] = out[j];
    }
}

/* ------------------------------------------------------------------------- */
/* The whole round in the order of the method: softmax (both models), cache build,
 * Saguaro reweight, verify, bonus, lookup.  All outputs in double / int. */
void orc_round(int B, int K, int V, int64_t ld, int dtype, const void* p_logits,
               const void* q_logits, double T, const int32_t* F, int Bf, double C,
               const int32_t* draft, uint64_t seed, uint64_t round, int64_t b_base, double cdf_eps,
               int fallback_uniform,
               double* p_max, double* p_sum, int32_t* p_arg, double* q_max, double* q_sum,
               int32_t* q_arg, int32_t* cache_ids, double* cache_mass, double* Z,
               int32_t* accept_len, double* accept_prob, int32_t* bonus, double* resid_mass,
               uint8_t* hit, int32_t* slot, int32_t* fallback_tokens, int32_t* err, uint8_t* exc,
               double* e2) {
    orc_softmax(B, K, V, ld, dtype, p_logits, T, p_max, p_sum, p_arg, NULL);
    orc_softmax(B, K, V, ld, dtype, q_logits, T, q_max, q_sum, q_arg, NULL);
    orc_build_cache(B, K, V, ld, dtype, q_logits, T, F, Bf, cache_ids, cache_mass);
    orc_saguaro(B, K, V, ld, dtype, q_logits, T, F, Bf, cache_ids, cache_mass, C, Z, NULL);
    for (int b = 0; b < B; ++b) { err[b] = 0; exc[b] = 0; }
    orc_verify(B, K, V, ld, dtype, p_logits, q_logits, T, draft, p_max, p_sum, p_arg, q_max, q_sum,
               q_arg, F, Bf, cache_ids, Z, C, seed, round, b_base, accept_len, accept_prob, err, exc);
    orc_residual_sample(B, K, V, ld, dtype, p_logits, q_logits, T, p_max, p_sum, p_arg, q_max, q_sum,
                        q_arg, F, Bf, cache_ids, Z, C, accept_len, seed, round, b_base, cdf_eps,
                        bonus, resid_mass, NULL, err, exc, e2);
    orc_cache_lookup(B, K, V, F, Bf, cache_ids, accept_len, bonus, fallback_uniform, seed, round,
                     b_base, hit, slot, fallback_tokens, err);
}

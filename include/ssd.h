/*
 * ssd.h -- C ABI of the MI355X (gfx950) verify-and-pre-speculate round of
 * Speculative Speculative Decoding (SSD) with the Saguaro algorithm.
 *
 * The round runs on logits the draft and target models have already produced.
 * Sources (two summaries of the paper "Speculative Speculative Decoding" by Kumar,
 * Dao and May):
 *   [zh] gist.science/zh/paper/2603.03251, technical part: section 1 (lossless SD),
 *        section 2 Methodology (basic flow; Challenge 1 geometric fan-out; Challenge 2
 *        Saguaro sampling; Challenge 3 fallback), section 4 (temperature, batch size);
 *   [nl] gist.science/nl/paper/2603.03251, technical part: section 2 (Kernprincipes),
 *        section 3 A (geometric fan-out), 3 B (Saguaro sampling), 3 C (fallback).
 * The pages name the parts and assert that the round is lossless; the formulas are
 * the standard lossless speculative-sampling construction, stated at each call.
 *
 * Conventions for every call
 *  - Logits are [B, K+1, V] row-major with row r = b*(K+1) + i and row stride `ld`
 *    elements (ld >= V).  Row i < K is draft position i; row K is the position after
 *    the last draft token.  fp32 or bf16 (bf16 is widened to fp32 in registers).
 *    Logits must be finite or -inf; a row needs at least one finite value.
 *    Rows are read as 16-byte vectors when the logits base is 16-byte aligned and
 *    ld * element size is a multiple of 16; other rows as aligned 16-byte blocks
 *    shifted into place (the allocation itself must be 16-byte aligned, as hipMalloc's
 *    are), which at B=64 K=8 V=128257 bf16 takes 1.2x as long per round.  With an odd
 *    vocabulary, pad the row stride (ld) to a multiple of 8 (bf16) or 4 (fp32)
 *    elements for the full rate.
 *  - Every pointer except those named *_host is device memory owned by the caller.
 *    The library allocates nothing, keeps no state between calls and never
 *    synchronises: every call enqueues its kernels on `stream` (a hipStream_t; NULL
 *    is the default stream) and returns.  Outputs must not alias inputs.
 *  - Argument errors are found on the host before any launch and return
 *    SSD_ERR_ARG with no side effect.  Shapes the kernels do not support return
 *    SSD_ERR_UNSUPPORTED; launch failures SSD_ERR_HIP (text in ssd_last_error()).
 *  - Data-dependent errors never trap: they OR bits into the optional per-sequence
 *    `dev_err[B]` (caller zeroes it): SSD_DEVERR_*.
 *  - `ws` is a workspace of at least ssd_workspace_bytes() bytes, 256-byte aligned,
 *    owned by the caller.  Its contents need no initialisation: every call writes
 *    the scratch it reads (per-tile partials, candidate keys, segment sums) before
 *    reading it, in a later kernel of the same call.  One workspace serves any
 *    number of calls on one stream; two calls that overlap in time must not share it.
 *  - Uniforms are counter-based: Philox4x64-10 (Salmon et al., SC'11) with key
 *    (seed, purpose) and counter (round, b, i, w); u = (word0 >> 40) * 2^-24 and
 *    u32 = word0 >> 32.  w = 0 for a test, a fallback token or a draw's first
 *    uniform u1, w = 1 for a draw's second uniform u2.  Purposes: SSD_PURPOSE_*.
 *    Results are reproducible from (seed, round).
 *  - A draw from weights w over ids 0..V-1 (the draft sampler and the bonus) takes
 *    two steps over blocks of 512 consecutive ids: u1 picks the block, the smallest
 *    one whose running sum of block weights exceeds u1 times the total; u2 picks the
 *    id inside it, the smallest one whose running sum from the block's first id
 *    exceeds u2 times the block's weight.  The law is w / sum(w), as for one inverse
 *    CDF over all ids; each decision is resolved against its own level's mass.  If
 *    rounding leaves no crossing, the last block (id) of positive weight is taken.
 */
#ifndef SSD_H
#define SSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SSD_OK = 0,
    SSD_ERR_ARG = 1,
    SSD_ERR_UNSUPPORTED = 2,
    SSD_ERR_HIP = 3,
    SSD_ERR_WORKSPACE = 4
} ssd_status;

typedef enum { SSD_F32 = 0, SSD_BF16 = 1 } ssd_dtype;

typedef enum { SSD_FALLBACK_NONE = 0, SSD_FALLBACK_UNIFORM = 1 } ssd_fallback;

enum { SSD_PURPOSE_ACCEPT = 0, SSD_PURPOSE_BONUS = 1, SSD_PURPOSE_DRAFT = 2, SSD_PURPOSE_FALLBACK = 3 };

enum {
    SSD_DEVERR_TOKEN_RANGE = 1,  /* a draft token outside [0, V): treated as rejected */
    SSD_DEVERR_QPRIME_ZERO = 2,  /* q'(d) == 0 (in fp64) for a tested draft token: rejected */
    SSD_DEVERR_LEN_RANGE = 4,    /* accept_len outside [0, K]: bonus -1, miss */
    SSD_DEVERR_SLOT_RANGE = 8,   /* a hit whose slot lies outside [0, Bf): next draft -1 */
    SSD_DEVERR_HIST_RANGE = 16   /* a history length outside [0, ld_hist]: n-gram tokens -1 */
};

/* Limits of this build. */
enum { SSD_MAX_K = 16, SSD_MAX_F = 64, SSD_MAX_NGRAM = 16 };

typedef struct {
    int32_t B;      /* sequences, >= 1 */
    int32_t K;      /* draft tokens per sequence, 1..SSD_MAX_K */
    int32_t V;      /* vocabulary, >= 2 */
    int64_t ld;     /* row stride in elements, >= V */
    int32_t dtype;  /* ssd_dtype */
    float T;        /* temperature >= 0; 0 selects the greedy (argmax) limit */
} ssd_shape;

typedef struct {
    uint64_t seed;
    uint64_t round;
} ssd_rng;

/* ssd_fanout -- geometric fan-out ([zh] section 2 Challenge 1; [nl] section 3 A):
 * splits the cache budget Bf over acceptance lengths k = 0..K in proportion to
 * r^k, integer shares by largest remainder (ties to the lower k), so that
 * sum F = Bf.  Host only; F_host has K+1 entries.  0 < r <= 1, Bf >= 0. */
ssd_status ssd_fanout(int32_t K, int32_t Bf, double r, int32_t* F_host);

/* Bytes of workspace the calls below need for this shape and budget. */
size_t ssd_workspace_bytes(const ssd_shape* shape, int32_t Bf);

/* ssd_softmax -- temperature softmax of every row ([zh] sections 2 and 4 use
 * temperature as an axis of the method):  m = max_x z(x),
 * s = sum_x exp((z(x) - m) / T), p(x) = exp((z(x) - m) / T) / s.  At T = 0:
 * s = 1 and p is one-hot on argmax (lowest id among the maxima).
 * Outputs [B*(K+1)]: row_max (fp32, an input value), row_sum (fp64); row_argmax
 * (int32, nullable) is the lowest id of the maximum; probs (nullable, [B, K+1, V]
 * fp32, dense) receives p. */
ssd_status ssd_softmax(const ssd_shape* shape, const void* logits, float* row_max, double* row_sum,
                       int32_t* row_argmax, float* probs, void* ws, size_t ws_bytes, void* stream);

/* ssd_build_cache -- the speculation cache keys ([zh] section 2 flow steps 2-3 and
 * Challenge 1; [nl] section 2 and 3 A).  For each sequence b and acceptance length
 * k = 0..K the cache holds F_k candidate bonus tokens: the F_k ids with the largest
 * draft logit z_q[b, k, .], ties to the lower id, stored in that order at
 * cache_ids[b, O_k + j] with O_k = F_0 + ... + F_{k-1} (cache_ids is [B, Bf]).
 * cache_mass[b*(K+1)+k] (fp64) = M_k = sum over those ids of q_k(x), with q from the
 * given draft row statistics (q_max, q_sum of ssd_softmax).  F_host [K+1] must
 * satisfy sum F = Bf and 0 <= F_k <= min(V, SSD_MAX_F). */
ssd_status ssd_build_cache(const ssd_shape* shape, const void* q_logits, const float* q_max,
                           const double* q_sum, const int32_t* F_host, int32_t Bf, int32_t* cache_ids,
                           double* cache_mass, void* ws, size_t ws_bytes, void* stream);

/* ssd_saguaro_reweight -- Saguaro sampling ([zh] section 2 Challenge 2; [nl] section
 * 3 B): the draft law is scaled by C in (0, 1] on the cached tokens S_k and
 * renormalised:  Z_k = 1 - (1 - C) M_k,  q'_k(x) = q_k(x) (C if x in S_k else 1) / Z_k.
 * Z [B*(K+1)] (fp64) is always written.  The rest is optional (pass NULL to skip):
 *  - q_prime [B, K+1, V] fp32 dense receives q';
 *  - draft [B, K] receives draft tokens drawn from q'_i (the two-step draw above,
 *    with the uniforms of (b, i, DRAFT)), or argmax z_q at T = 0.
 * Both optional outputs need q_logits, q_max, q_sum, q_argmax (T = 0), F_host, Bf,
 * cache_ids; draft also needs ws. */
ssd_status ssd_saguaro_reweight(const ssd_shape* shape, const double* cache_mass, float C, double* Z,
                                const void* q_logits, const float* q_max, const double* q_sum,
                                const int32_t* q_argmax, const int32_t* F_host, int32_t Bf,
                                const int32_t* cache_ids, float* q_prime, ssd_rng rng, int32_t* draft,
                                void* ws, size_t ws_bytes, void* stream);

/* ssd_verify -- lossless verification ([zh] section 1 and section 2 flow steps 2 and
 * 4; [nl] section 2): for i = 0..K-1 in order, ratio_i = p_i(d_i) / q'_i(d_i) and
 * draft token d_i is accepted iff U(seed, round, b, i, ACCEPT) < ratio_i; the
 * accepted length k is the first rejected position, or K.  At T = 0, d_i is
 * accepted iff d_i = argmax p_i (p_argmax required).  cache_ids is required whenever
 * Bf > 0, at every temperature (the membership of d_i in S_i is read from it).
 * accept_len [B] int32; accept_prob (nullable [B, K] fp32) = min(1, ratio_i) for
 * every i. */
ssd_status ssd_verify(const ssd_shape* shape, const void* p_logits, const void* q_logits,
                      const int32_t* draft, const float* p_max, const double* p_sum,
                      const int32_t* p_argmax, const float* q_max, const double* q_sum,
                      const int32_t* F_host, int32_t Bf, const int32_t* cache_ids, const double* Z,
                      float C, ssd_rng rng, int32_t* accept_len, float* accept_prob, int32_t* dev_err,
                      void* stream);

/* ssd_residual_sample -- the bonus token ([zh] section 2 flow step 2 and Challenge 2:
 * the bonus comes from the residual distribution; [nl] section 3 B).  With
 * k = accept_len[b]:  k < K: w(x) = max(p_k(x) - q'_k(x), 0) (w = p_k if the fp64 sum of
 * these weights is not above 0, which only rounding can cause);  k = K: w = p_K.
 * bonus[b] is drawn from w (the two-step draw above, with the uniforms of
 * (b, k, BONUS)).  At T = 0 the bonus is argmax p_k (p_argmax required).  resid_mass (nullable [B], fp64) receives sum(w).
 * The running sums that locate the bonus are kept in fp64. */
ssd_status ssd_residual_sample(const ssd_shape* shape, const void* p_logits, const void* q_logits,
                               const float* p_max, const double* p_sum, const int32_t* p_argmax,
                               const float* q_max, const double* q_sum, const int32_t* F_host,
                               int32_t Bf, const int32_t* cache_ids, const double* Z, float C,
                               const int32_t* accept_len, ssd_rng rng, int32_t* bonus,
                               double* resid_mass, int32_t* dev_err, void* ws, size_t ws_bytes,
                               void* stream);

/* ssd_cache_lookup -- cache hit on the verified outcome (k, bonus) ([zh] section 2
 * flow step 4 and Challenge 3; [nl] section 2 and 3 C).  hit[b] = 1 iff bonus is
 * one of the F_k cached ids of length k; slot[b] = O_k + its position, else -1.  On
 * a miss with SSD_FALLBACK_UNIFORM the next draft is K uniform random tokens
 * fallback_tokens[b, j] = (U32(seed, round, b, j, FALLBACK) * V) >> 32; every other
 * fallback entry is -1. */
ssd_status ssd_cache_lookup(int32_t B, int32_t K, int32_t V, const int32_t* F_host, int32_t Bf,
                            const int32_t* cache_ids, const int32_t* accept_len, const int32_t* bonus,
                            int32_t fallback, ssd_rng rng, uint8_t* hit, int32_t* slot,
                            int32_t* fallback_tokens, int32_t* dev_err, void* stream);

/* ssd_cache_gather -- the next round's draft from the speculation cache ([zh] section
 * 2 basic flow step 4: on a hit the pre-speculated tokens are available at once, on a
 * miss the fallback speculator takes over; [nl] section 2 Kernprincipes).  Reading of
 * the pages: the cache holds one continuation of K tokens per cached outcome, in a
 * value store values[B, Bf, K] (int32, slot-major as ssd_cache_lookup numbers the
 * slots).  next_draft[b, :] = values[b, slot[b], :] when hit[b], else
 * fallback_tokens[b, :] (uniform random tokens, or -1 = the caller's speculator).  A
 * hit whose slot lies outside [0, Bf) gives -1 and sets SSD_DEVERR_SLOT_RANGE.
 * hit [B] uint8, slot [B], fallback_tokens [B, K], next_draft [B, K] int32. */
ssd_status ssd_cache_gather(int32_t B, int32_t K, int32_t Bf, const int32_t* values, const uint8_t* hit,
                            const int32_t* slot, const int32_t* fallback_tokens, int32_t* next_draft,
                            int32_t* dev_err, void* stream);

/* ssd_ngram_fallback -- the n-gram fallback speculator ([zh] section 2 Challenge 3
 * and [nl] section 3 C name an n-gram model, next to random tokens, as the fast,
 * low-quality speculator a large batch falls back to on a miss; they give no rule).
 * Reading of the pages (prompt lookup over the sequence's own context):
 *   context   c = hist[b, 0 .. hist_len[b]) ++ draft[b, 0 .. k) ++ [bonus[b]], length
 *             L, with k = accept_len[b] (the tokens the verified round appended);
 *   match     the largest n in [n_min, n_max] whose last n tokens of c also occur
 *             ending at some e <= L - 2, and the latest such e;
 *   proposal  fallback_tokens[b, j] = c[e + 1 + (j mod (L - 1 - e))], j < K: the
 *             tokens that followed the occurrence, the copy running on over its own
 *             output when fewer than K follow;
 *   no match  the uniform random draft of ssd_cache_lookup's SSD_FALLBACK_UNIFORM,
 *             (U32(seed, round, b, j, FALLBACK) * V) >> 32.
 * Sequences with hit[b] != 0 get fallback_tokens -1 and keep their next_draft row (the
 * cache gather wrote it); hit NULL serves every sequence.  For every served sequence
 * next_draft[b, :] (nullable) is set to the proposal, match_n[b] (nullable) to n (0:
 * no match) and match_end[b] (nullable) to e (-1).  An accept_len outside [0, K]
 * sets SSD_DEVERR_LEN_RANGE, a hist_len outside [0, ld_hist] SSD_DEVERR_HIST_RANGE;
 * both give tokens -1.  Token values are opaque (no range check).
 * hist [B, ld_hist] int32 (may be NULL when ld_hist == 0), hist_len [B], draft [B, K],
 * accept_len [B], bonus [B] int32, hit [B] uint8.  1 <= n_min <= n_max <=
 * SSD_MAX_NGRAM, 1 <= K <= SSD_MAX_K, V >= 2; ld_hist above 2^31 - 18 returns
 * SSD_ERR_UNSUPPORTED. */
ssd_status ssd_ngram_fallback(int32_t B, int32_t K, int32_t V, const int32_t* hist, int64_t ld_hist,
                              const int32_t* hist_len, const int32_t* draft, const int32_t* accept_len,
                              const int32_t* bonus, const uint8_t* hit, int32_t n_min, int32_t n_max,
                              ssd_rng rng, int32_t* fallback_tokens, int32_t* next_draft, int32_t* match_n,
                              int32_t* match_end, int32_t* dev_err, void* stream);

/* Outputs of the fused round.  Required: cache_ids [B, Bf], accept_len [B], bonus
 * [B], hit [B], slot [B], fallback_tokens [B, K].  The rest are nullable. */
typedef struct {
    float* p_max;       /* [B*(K+1)] */
    double* p_sum;
    int32_t* p_argmax;
    float* q_max;
    double* q_sum;
    int32_t* q_argmax;
    int32_t* cache_ids;
    double* cache_mass; /* [B*(K+1)] */
    double* Z;          /* [B*(K+1)] */
    int32_t* accept_len;
    float* accept_prob; /* [B, K] */
    int32_t* bonus;
    double* resid_mass; /* [B] */
    uint8_t* hit;
    int32_t* slot;
    int32_t* fallback_tokens;
    int32_t* dev_err;   /* [B], OR-accumulated */
    const int32_t* cache_values;  /* input [B, Bf, K]: continuation per cache slot (needed when
                                     next_draft is given and Bf > 0) */
    int32_t* next_draft;          /* nullable [B, K]: the next draft, as ssd_cache_gather makes it */
} ssd_round_out;

/* Optional HIP events (hipEvent_t, may be NULL) recorded on `stream` around the
 * two streaming kernels of ssd_round: pass 1 over every row of both models (tile
 * partials of the softmax statistics and top-F candidates) and pass 2 over the rows
 * the bonus needs (residual tile sums).  The per-sequence finalisation (cache,
 * Saguaro, verification) runs between pass1_stop and pass2_start, the bonus
 * search and lookup after pass2_stop.  At T = 0 pass 2 does not run and its
 * events are not recorded. */
typedef struct {
    void* pass1_start;
    void* pass1_stop;
    void* pass2_start;
    void* pass2_stop;
} ssd_round_events;

/* ssd_round -- one whole verify-and-pre-speculate round in the method's order:
 * softmax of both models, cache build, Saguaro reweight, verification, bonus and
 * lookup, with the same arithmetic as the six separate calls (results are
 * bit-identical to chaining them).  Two streaming kernels: one over all
 * 2 B (K+1) rows, one over the <= 2 rows per sequence the bonus needs; each is
 * followed by a small per-sequence kernel. */
ssd_status ssd_round(const ssd_shape* shape, const void* p_logits, const void* q_logits,
                     const int32_t* draft, const int32_t* F_host, int32_t Bf, float C, ssd_rng rng,
                     int32_t fallback, const ssd_round_out* out, const ssd_round_events* events,
                     void* ws, size_t ws_bytes, void* stream);

/* ssd_round_devrng -- ssd_round with the round counter in device memory, for callers
 * that capture the round in a HIP graph and replay it: the kernels read *round_dev
 * (uint64, device memory, caller-owned) when they run, so the uniforms follow whatever
 * the caller wrote there before the replay (for instance a captured increment after
 * each round); the key is (seed, purpose) as for ssd_round.  Every other argument, the
 * outputs and the errors are those of ssd_round; with *round_dev == r the results are
 * bit-identical to ssd_round with rng = {seed, r}.  round_dev NULL returns SSD_ERR_ARG.
 * Writing *round_dev while a round that reads it runs is a race. */
ssd_status ssd_round_devrng(const ssd_shape* shape, const void* p_logits, const void* q_logits,
                            const int32_t* draft, const int32_t* F_host, int32_t Bf, float C, uint64_t seed,
                            const uint64_t* round_dev, int32_t fallback, const ssd_round_out* out,
                            const ssd_round_events* events, void* ws, size_t ws_bytes, void* stream);

/* ssd_round_noalloc -- ssd_round for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  It
 * takes no workspace: the round's scratch is a static device array of
 * SSD_NOALLOC_SCRATCH_BYTES inside the library, one copy per GPU, held until the
 * process ends.  The first call on a GPU looks up that GPU's copy
 * (hipGetSymbolAddress, with the stream's device current); no call allocates or frees
 * anything.  A shape whose ssd_workspace_bytes(shape, Bf) exceeds the array returns
 * SSD_ERR_WORKSPACE (text in ssd_last_error()) before any launch.  The array keeps
 * the last call's contents; the round writes every part of it it reads, so nothing
 * needs clearing.  Every call on one GPU uses the same array: calls that overlap in
 * time on one GPU (on different streams, or from different host threads) race and
 * must not be made.  Arguments, outputs, results and errors are otherwise those of
 * ssd_round (bit-identical for the same inputs). */
#define SSD_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20)
ssd_status ssd_round_noalloc(const ssd_shape* shape, const void* p_logits, const void* q_logits,
                             const int32_t* draft, const int32_t* F_host, int32_t Bf, float C, ssd_rng rng,
                             int32_t fallback, const ssd_round_out* out, const ssd_round_events* events,
                             void* stream);

/* ---------------------------------------------------------------------------
 * Choosing the fan-out from measured coverage.  [zh] section 2 Challenge 1 and [nl]
 * section 3 A say the fan-out solves a constrained optimisation over acceptance
 * lengths, favouring short, likely lengths; they print no objective.  Reading used
 * here: maximise the number of verified rounds whose bonus token the cache would
 * have held.  A bonus t verified at acceptance length k is held by the cache when
 * F_k exceeds its rank in the draft row k (cache order: larger logit first, ties to
 * the lower id), so the statistics are a histogram over (k, rank).
 *
 * ssd_bonus_rank -- per sequence, the rank of bonus[b] within draft row
 * k = accept_len[b]:  rank = #{x : z_q(x) > z_q(t)} + #{x < t : z_q(x) = z_q(t)}
 * (logits compared as fp32, -0 equal to +0).  rank_out [B] (nullable) receives it,
 * -1 when k lies outside [0, K] or t outside [0, V).  rank_hist (nullable,
 * [(K+1), R+1] uint32, accumulated: the caller zeroes it once and may add many
 * rounds) counts valid sequences per (k, min(rank, R)); bin R holds ranks >= R.
 * 1 <= R <= SSD_MAX_F; at least one output.  shape.T is not used (the order does
 * not depend on the temperature).  ws as for the other calls.  Calls that overlap
 * in time may share rank_hist (the merge is atomic). */
ssd_status ssd_bonus_rank(const ssd_shape* shape, const void* q_logits, const int32_t* accept_len,
                          const int32_t* bonus, int32_t R, int32_t* rank_out, uint32_t* rank_hist, void* ws,
                          size_t ws_bytes, void* stream);

/* ssd_fanout_optimize -- host only.  From rank_hist_host [(K+1), R+1] (as
 * ssd_bonus_rank accumulates it), the fan-out F_host [K+1] that maximises the
 * predicted hits  H(F) = sum_k sum_{j < F_k} hist[k][j]  over integers
 * 0 <= F_k <= min(Fmax, R) with sum F = Bf.  Among maximisers, the lexicographically
 * largest F (most candidates at the shortest lengths).  Exact (integer dynamic
 * programme).  hits_host / total_host (nullable) receive H(F) and the count of all
 * sequences in the histogram, so H / total is the predicted hit rate.
 * SSD_ERR_ARG when Bf > (K+1) min(Fmax, R) or an argument is out of range
 * (1 <= K <= SSD_MAX_K, 1 <= R <= SSD_MAX_F, 0 <= Fmax <= SSD_MAX_F, Bf >= 0). */
ssd_status ssd_fanout_optimize(int32_t K, int32_t Bf, int32_t Fmax, int32_t R, const uint32_t* rank_hist_host,
                               int32_t* F_host, uint64_t* hits_host, uint64_t* total_host);

/* ---------------------------------------------------------------------------
 * Fallback policy by batch size ([zh] section 2 Challenge 3; [nl] section 3 C):
 * on a miss the whole batch waits for the fallback speculator; small batches use
 * the slow, accurate primary speculator, large ones a fast, weak one (random
 * tokens, SSD_FALLBACK_UNIFORM), with a critical batch size b* between them.  The
 * pages print no formula.  Reading used here, with every input measured by the
 * caller:
 *   P(any miss) = 1 - prod_b h_b                 (h_b: hit probability of sequence b)
 *   time(f)     = t_verify + P(any miss) * t_f
 *   tokens(f)   = sum_b [ h_b n_hit + (1 - h_b) n_f ]
 *   f*          = argmax_f tokens(f) / time(f),   ties to the primary speculator. */
typedef struct {
    double t_verify;   /* time of one verification round (any unit, > 0) */
    double t_primary;  /* wait added when a miss falls back to the primary speculator (>= 0) */
    double t_random;   /* wait added when a miss falls back to random tokens (>= 0) */
    double n_hit;      /* expected tokens a sequence gains in a round after a hit (>= 0) */
    double n_primary;  /* ... after a miss served by the primary speculator (>= 0) */
    double n_random;   /* ... after a miss served by random tokens (>= 0) */
} ssd_fallback_model;

/* ssd_fallback_choose -- host only.  h_host [B] in [0, 1].  choice_host receives
 * SSD_FALLBACK_NONE (the caller's primary speculator) or SSD_FALLBACK_UNIFORM, the
 * value ssd_round and ssd_cache_lookup take; tput_primary / tput_random (nullable)
 * receive tokens / time of each. */
ssd_status ssd_fallback_choose(const ssd_fallback_model* model, int32_t B, const double* h_host,
                               int32_t* choice_host, double* tput_primary, double* tput_random);

/* ssd_fallback_critical_batch -- host only.  For a common hit probability h in
 * [0, 1], the smallest batch size b in [1, b_max] at which random tokens give a
 * strictly higher throughput than the primary speculator; 0 if there is none. */
ssd_status ssd_fallback_critical_batch(const ssd_fallback_model* model, double h, int32_t b_max,
                                       int32_t* b_star_host);

/* ---------------------------------------------------------------------------
 * Measurement.  ssd_stream_read -- reads `bytes` of device memory at `buf` once, in
 * the access shape of the vocabulary pass (each wave 8 KiB: eight non-temporal
 * 16-byte loads per lane), and computes nothing from them but an XOR; the time it
 * takes on the same buffers is the achievable read rate the round's streaming
 * kernels are measured against.  `sink` (device, one uint32) is written only in the
 * unlikely case that a wave's XOR equals a fixed constant (it exists so that the
 * loads cannot be removed).  buf 16-byte aligned, bytes a positive multiple of 16.
 * Not part of the round. */
ssd_status ssd_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

const char* ssd_status_string(ssd_status s);

/* Text of the last HIP error seen by this thread (empty if none). */
const char* ssd_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SSD_H */

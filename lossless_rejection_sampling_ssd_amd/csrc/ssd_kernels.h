// ssd_kernels.h -- launch interface between the C ABI layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

constexpr int kMaxKc = 16;

// Softmax partial of one wave tile of a row: its maximum m, the lowest id attaining
// it, s = sum of 2^{z c - o(m)} over the tile (o(m) = rint(m c)), and for draft rows
// of the cache the tile's candidate threshold (an order key; 0 admits every element)
// and how many candidate keys it stored.
struct WavePartial {
    float m;
    int arg;
    double s;
    uint32_t tau;
    int ncand;
    int pad0, pad1;
};

// Law parameters of one row (b, i) for pass 2 and the bonus: p(x) = tp inv_p, residual
// weights max(tp - tq rho_sel, 0), term offsets op (target) and oq (draft).
struct LawParams {
    double inv_p, rho, rhoC;
    float op, oq;
};

struct Pass1Args {
    const char* logits[2];
    int nmodel;       // 1, or 2 for the fused round (0 = target p, 1 = draft q)
    int topf_model;   // model whose rows collect top-F candidates, -1 for none
    int B, K1, V;
    int64_t ld_bytes;
    float c;          // log2(e) / T, 0 when greedy
    int greedy;
    int want_arg;
    int nt;           // wave tiles per row
    int cap;          // candidate slots per tile
    int F[kMaxKc + 1];
    int O[kMaxKc + 2];
    WavePartial* part;  // [B][nmodel][K1][nt]
    uint64_t* cand;     // [B][K1][nt][cap]
    const int32_t* draft;  // nullable [B, K]: the wave holding logit d_i of row i records it
    float* probe;          // [B][K][nmodel] logits at the draft tokens (when draft is set)
};

// Finalisation of the vocabulary pass per (sequence, position): row statistics,
// speculation cache, Saguaro normaliser and the test of the draft token.  The outcome
// of each test goes to vflag; the kernels after it take the accepted length from there
// (and, at T = 0, the bonus and lookup in a per-sequence kernel).
struct SeqFinal {
    const WavePartial* part;
    const uint64_t* cand;
    const char* p_logits;
    const char* q_logits;
    int B, K, V, nt, cap;
    int64_t ld_bytes;
    float c;
    int greedy;
    int F[kMaxKc + 1];
    int O[kMaxKc + 2];
    const int32_t* draft;  // [B, K]
    const float* probe;    // [B][K][2] logits at the draft tokens, recorded by pass 1
    float C;
    uint64_t seed, round;
    int fallback;
    int Bf;
    float* p_max;
    double* p_sum;
    int32_t* p_arg;
    float* q_max;
    double* q_sum;
    int32_t* q_arg;       // nullable
    int32_t* cache_ids;
    double* cache_mass;
    double* Z;
    int32_t* accept_len;
    float* accept_prob;   // nullable
    int32_t* bonus;       // written here only at T = 0
    double* resid_mass;   // nullable
    uint8_t* hit;
    int32_t* slot;
    int32_t* fallback_tokens;
    int32_t* dev_err;     // nullable
    const int32_t* cache_values;  // nullable [B, Bf, K]: continuation per cache slot
    int32_t* next_draft;          // [B, K] when cache_values is set
    int32_t* vflag;       // [B, K] workspace: bit 0 accepted, higher bits error bits
    const uint64_t* round_ptr;  // nullable: the round counter in device memory (replaces round)
    LawParams* law;             // nullable [B (K+1)]: receives each row's law parameters
};

struct Pass2Args {
    const char* p_logits;
    const char* q_logits;
    int B, K, V;
    int64_t ld_bytes;
    float c;
    float C;
    int mode;         // 0: bonus from the residual (per sequence); 1: draft tokens from q' (per (b, i))
    int nt;           // pass-2 tiles per row
    int F[kMaxKc + 1];
    int O[kMaxKc + 2];
    int Bf;
    const float* p_max;
    const double* p_sum;
    const float* q_max;
    const double* q_sum;
    const double* Z;
    const int32_t* cache_ids;
    const int32_t* accept_len;  // mode 0 without vflag: the accepted lengths
    const int32_t* vflag;       // mode 0: per-position test outcomes (accepted length = first rejection)
    int32_t* accept_len_out;    // with vflag: written by the bonus kernel
    uint64_t seed, round;
    double2* seg;       // [groups][nt] (weight sum, target-law sum) per wave tile
    int32_t* out_tok;   // bonus [B] or draft [B, K]
    double* resid_mass; // nullable
    int32_t* dev_err;   // nullable
    int do_lookup;
    const int32_t* cache_values;  // nullable [B, Bf, K] (with do_lookup)
    int32_t* next_draft;          // [B, K] when cache_values is set
    int fallback;
    uint8_t* hit;
    int32_t* slot;
    int32_t* fallback_tokens;
    const uint64_t* round_ptr;  // nullable: the round counter in device memory (replaces round)
    const LawParams* law;       // nullable [B (K+1)]: precomputed law of each row (else from the statistics)
};

int tile_elems(int dtype);
int tiles_per_row(int dtype, int V);   // pass-1 tiles
int tiles_per_row2(int dtype, int V);  // pass-2 tiles (half size)
int cand_cap(int Fmax);

hipError_t launch_pass1(int dtype, bool vec, const Pass1Args& a, hipStream_t st);
hipError_t launch_finalize_pos(int dtype, const SeqFinal& f, hipStream_t st);
hipError_t launch_finish_greedy(const SeqFinal& f, hipStream_t st);
hipError_t launch_pass2(int dtype, bool vec, const Pass2Args& a, int ngroups, hipStream_t st);
hipError_t launch_finalize_bonus(int dtype, bool vec, const Pass2Args& a, int ngroups, hipStream_t st);
hipError_t launch_combine_stats(const Pass1Args& a, float* m, double* s, int32_t* arg, hipStream_t st);
hipError_t launch_combine_topf(const Pass1Args& a, int Bf, const float* q_max, const double* q_sum,
                               int32_t* cache_ids, double* cache_mass, hipStream_t st);
hipError_t launch_probs(int dtype, const char* logits, int B, int K1, int V, int64_t ld_bytes, const float* m,
                        const double* s, const int32_t* arg, float c, int greedy, const int32_t* cache_ids,
                        const int* F, const int* O, int Bf, const double* Z, float C, float* out, hipStream_t st);
hipError_t launch_saguaro_z(const double* cache_mass, int R, float C, double* Z, hipStream_t st);
hipError_t launch_verify(int dtype, const char* p_logits, const char* q_logits, int B, int K, int V,
                         int64_t ld_bytes, const int32_t* draft, const float* p_max, const double* p_sum,
                         const int32_t* p_arg, const float* q_max, const double* q_sum, const int* F, const int* O,
                         int Bf, const int32_t* cache_ids, const double* Z, float C, float c, int greedy,
                         uint64_t seed, uint64_t round, int32_t* accept_len, float* accept_prob, int32_t* dev_err,
                         hipStream_t st);
// Greedy (T = 0) picks from per-row argmax: with accept_len == nullptr, out[b, i] =
// arg[b*(K+1) + i] for i < K (draft tokens); otherwise out[b] = arg[b*(K+1) + k_b]
// (bonus), mass[b] = 1.
hipError_t launch_greedy_pick(const int32_t* arg, int B, int K, const int32_t* accept_len, int32_t* out,
                              double* mass, int32_t* dev_err, hipStream_t st);
hipError_t launch_gather(int B, int K, int Bf, const int32_t* values, const uint8_t* hit, const int32_t* slot,
                         const int32_t* fallback_tokens, int32_t* next_draft, int32_t* dev_err, hipStream_t st);
// Rank of the bonus token within the draft row of its acceptance length, and the
// coverage histogram over (length, rank).
struct RankArgs {
    const char* q_logits;
    int B, K, V;
    int64_t ld_bytes;
    int nt;                     // pass-1 tiles per row
    const int32_t* accept_len;  // [B]
    const int32_t* bonus;       // [B]
    uint32_t* counts;           // workspace [B][nt]: per-tile count of ids ranked above the bonus
    int R;                      // histogram bins per length: ranks 0..R-1, bin R = rank >= R
    int32_t* rank_out;          // nullable [B]
    uint32_t* hist;             // nullable [(K+1)][R+1], accumulated
};
hipError_t launch_rank(int dtype, bool vec, const RankArgs& a, hipStream_t st);

// Read-only stream over nvec 16-byte vectors (the same-run read ceiling).
hipError_t launch_stream_read(const void* buf, int64_t nvec, uint32_t* sink, hipStream_t st);

hipError_t launch_lookup(int B, int K, int V, const int* F, const int* O, int Bf, const int32_t* cache_ids,
                         const int32_t* accept_len, const int32_t* bonus, int fallback, uint64_t seed,
                         uint64_t round, uint8_t* hit, int32_t* slot, int32_t* fallback_tokens, int32_t* dev_err,
                         hipStream_t st);

}  // namespace ssd

// ssd_kernels.h -- launch interface between the C ABI layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

constexpr int kMaxKc = 16;

// Softmax partial of one vocabulary chunk of a row: its maximum m, the lowest id
// attaining it, and s = sum of 2^{z c - o(m)} over the chunk (o(m) = rint(m c)).
struct RowPartial {
    float m;
    int arg;
    double s;
};

// Everything the sequence finaliser of the fused vocabulary pass needs.
struct SeqFinal {
    const int32_t* draft;  // [B, K]
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
};

struct Pass1Args {
    const char* logits[2];
    int nmodel;       // 1, or 2 for the fused round (0 = target p, 1 = draft q)
    int topf_model;   // model whose rows build top-F lists, -1 for none
    int B, K1, V;
    int64_t ld_bytes;
    float c;          // log2(e) / T, 0 when greedy
    int greedy;
    int want_arg;
    int nb;           // blocks per row
    int F[kMaxKc + 1];
    int O[kMaxKc + 2];
    int Fmax;         // slots per block list
    RowPartial* part;  // per sequence: [nmodel][K1][nb], sequence stride part_stride
    int64_t part_stride;
    uint64_t* topk;    // per sequence: [K1][nb][Fmax], sequence stride topk_stride
    int64_t topk_stride;
    unsigned* seq_counter;  // non-null: fused round with a per-sequence finaliser
    SeqFinal fin;
};

struct Pass2Args {
    const char* p_logits;
    const char* q_logits;
    int B, K, V;
    int64_t ld_bytes;
    float c;
    float C;
    int mode;         // 0: bonus from the residual (per sequence); 1: draft tokens from q' (per (b, i))
    int nb;
    int F[kMaxKc + 1];
    int O[kMaxKc + 2];
    int Bf;
    const float* p_max;
    const double* p_sum;
    const float* q_max;
    const double* q_sum;
    const double* Z;
    const int32_t* cache_ids;
    const int32_t* accept_len;
    uint64_t seed, round;
    double2* seg;       // per group: [nb * waves] (weight sum, target-law sum), group stride seg_stride
    int64_t seg_stride;
    unsigned* counter;  // [groups]
    int32_t* out_tok;   // bonus [B] or draft [B, K]
    double* resid_mass; // nullable
    int32_t* dev_err;   // nullable
    int do_lookup;
    int fallback;
    uint8_t* hit;
    int32_t* slot;
    int32_t* fallback_tokens;
};

int chunk_elems(int dtype);
int blocks_per_row(int dtype, int V);

hipError_t launch_pass1(int dtype, bool vec, const Pass1Args& a, hipStream_t st);
hipError_t launch_pass2(int dtype, bool vec, const Pass2Args& a, int nseq, hipStream_t st);
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
hipError_t launch_lookup(int B, int K, int V, const int* F, const int* O, int Bf, const int32_t* cache_ids,
                         const int32_t* accept_len, const int32_t* bonus, int fallback, uint64_t seed,
                         uint64_t round, uint8_t* hit, int32_t* slot, int32_t* fallback_tokens, int32_t* dev_err,
                         hipStream_t st);

}  // namespace ssd

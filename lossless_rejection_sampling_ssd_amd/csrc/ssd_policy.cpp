// ssd_policy.cpp -- host-only policies of the C ABI (include/ssd.h): the fan-out
// chosen from measured coverage, and the fallback speculator chosen by batch size.
// Plain C++ on the host; no device code, no allocation.
#include <cmath>
#include <cstdint>

#include "../../include/ssd.h"

namespace {

constexpr int kMaxBudget = (SSD_MAX_K + 1) * SSD_MAX_F;

struct Throughputs {
    double primary, random;
};

bool model_ok(const ssd_fallback_model* m) {
    if (!m) return false;
    const double v[6] = {m->t_verify, m->t_primary, m->t_random, m->n_hit, m->n_primary, m->n_random};
    for (double x : v)
        if (!std::isfinite(x) || x < 0.0) return false;
    return m->t_verify > 0.0;
}

// tokens / time of both fallbacks for B sequences with prod h_b = all_hit and
// sum h_b = hit_sum.
Throughputs throughputs(const ssd_fallback_model* m, int B, double all_hit, double hit_sum) {
    const double p_miss = 1.0 - all_hit, miss_sum = (double)B - hit_sum;
    Throughputs t;
    t.primary = (hit_sum * m->n_hit + miss_sum * m->n_primary) / (m->t_verify + p_miss * m->t_primary);
    t.random = (hit_sum * m->n_hit + miss_sum * m->n_random) / (m->t_verify + p_miss * m->t_random);
    return t;
}

}  // namespace

extern "C" {

ssd_status ssd_fanout_optimize(int32_t K, int32_t Bf, int32_t Fmax, int32_t R, const uint32_t* hist,
                               int32_t* F_host, uint64_t* hits_host, uint64_t* total_host) {
    if (!hist || !F_host || K < 1 || K > SSD_MAX_K || R < 1 || R > SSD_MAX_F || Fmax < 0 || Fmax > SSD_MAX_F ||
        Bf < 0)
        return SSD_ERR_ARG;
    const int K1 = K + 1, cap = Fmax < R ? Fmax : R;
    if (Bf > K1 * cap) return SSD_ERR_ARG;
    // gain[k][f]: sequences at length k whose bonus ranks below f
    static thread_local uint64_t gain[SSD_MAX_K + 1][SSD_MAX_F + 1];
    uint64_t total = 0;
    for (int k = 0; k < K1; ++k) {
        gain[k][0] = 0;
        for (int f = 1; f <= cap; ++f) gain[k][f] = gain[k][f - 1] + hist[(int64_t)k * (R + 1) + f - 1];
        for (int j = 0; j <= R; ++j) total += hist[(int64_t)k * (R + 1) + j];
    }
    // suffix optimum: opt[k][b] = most hits over lengths k..K spending exactly b
    // (every b in [0, (K1-k) cap] is reachable, the rest is never asked for)
    static thread_local uint64_t opt[SSD_MAX_K + 2][kMaxBudget + 1];
    for (int b = 0; b <= Bf; ++b) opt[K1][b] = 0;
    for (int k = K1 - 1; k >= 0; --k) {
        const int reach = (K1 - k) * cap;
        for (int b = 0; b <= Bf && b <= reach; ++b) {
            const int lo = b - (K1 - k - 1) * cap > 0 ? b - (K1 - k - 1) * cap : 0;
            const int hi = b < cap ? b : cap;
            uint64_t m = 0;
            for (int f = lo; f <= hi; ++f) {
                const uint64_t v = gain[k][f] + opt[k + 1][b - f];
                if (v > m) m = v;
            }
            opt[k][b] = m;
        }
    }
    // walk forward taking the largest share that keeps the optimum
    int left = Bf;
    for (int k = 0; k < K1; ++k) {
        const int lo = left - (K1 - k - 1) * cap > 0 ? left - (K1 - k - 1) * cap : 0;
        const int hi = left < cap ? left : cap;
        int pick = lo;
        for (int f = hi; f >= lo; --f)
            if (gain[k][f] + opt[k + 1][left - f] == opt[k][left]) {
                pick = f;
                break;
            }
        F_host[k] = pick;
        left -= pick;
    }
    if (hits_host) *hits_host = opt[0][Bf];
    if (total_host) *total_host = total;
    return SSD_OK;
}

ssd_status ssd_fallback_choose(const ssd_fallback_model* model, int32_t B, const double* h_host,
                               int32_t* choice_host, double* tput_primary, double* tput_random) {
    if (!model_ok(model) || B < 1 || !h_host || !choice_host) return SSD_ERR_ARG;
    for (int b = 0; b < B; ++b)
        if (!(h_host[b] >= 0.0 && h_host[b] <= 1.0)) return SSD_ERR_ARG;
    double all_hit = 1.0, hit_sum = 0.0;
    for (int b = 0; b < B; ++b) {
        all_hit *= h_host[b];
        hit_sum += h_host[b];
    }
    const Throughputs t = throughputs(model, B, all_hit, hit_sum);
    *choice_host = t.random > t.primary ? SSD_FALLBACK_UNIFORM : SSD_FALLBACK_NONE;
    if (tput_primary) *tput_primary = t.primary;
    if (tput_random) *tput_random = t.random;
    return SSD_OK;
}

ssd_status ssd_fallback_critical_batch(const ssd_fallback_model* model, double h, int32_t b_max,
                                       int32_t* b_star_host) {
    if (!model_ok(model) || !(h >= 0.0 && h <= 1.0) || b_max < 1 || !b_star_host) return SSD_ERR_ARG;
    *b_star_host = 0;
    double all_hit = 1.0, hit_sum = 0.0;  // the same products and sums as b copies of h
    for (int b = 1; b <= b_max; ++b) {
        all_hit *= h;
        hit_sum += h;
        const Throughputs t = throughputs(model, b, all_hit, hit_sum);
        if (t.random > t.primary) {
            *b_star_host = b;
            break;
        }
    }
    return SSD_OK;
}

}  // extern "C"

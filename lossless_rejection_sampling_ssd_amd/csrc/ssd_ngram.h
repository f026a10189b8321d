// ssd_ngram.h -- launch interface of the n-gram fallback speculator kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

constexpr int kMaxNgram = 16;  // longest n-gram matched

struct NgramArgs {
    int B, K, V;
    const int32_t* hist;  // [B, ld_hist]
    int64_t ld_hist;
    const int32_t* hist_len;  // [B]
    const int32_t* draft;     // [B, K]
    const int32_t* accept_len;
    const int32_t* bonus;
    const uint8_t* hit;  // nullable: every sequence is served
    int n_min, n_max;
    uint64_t seed, round;
    int32_t* tokens;      // [B, K]
    int32_t* next_draft;  // nullable [B, K]
    int32_t* match_n;     // nullable [B]
    int32_t* match_end;   // nullable [B]
    int32_t* dev_err;     // nullable [B]
};

hipError_t launch_ngram(const NgramArgs& a, hipStream_t st);

}  // namespace ssd

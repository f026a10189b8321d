// ssd_ngram.hip -- gfx950 kernel of the n-gram fallback speculator.
//
// The summaries of "Speculative Speculative Decoding" ([zh] gist.science/zh/paper/
// 2603.03251 section 2 Challenge 3; [nl] gist.science/nl/paper/2603.03251 section 3 C)
// name an n-gram model, next to random tokens, as the fast, low-quality speculator a
// large batch falls back to on a cache miss.  Here it is prompt lookup over the
// sequence's own context c = history ++ accepted draft tokens ++ bonus (length L):
// the longest n in [n_min, n_max] whose last n tokens also occur ending at some
// e <= L - 2, the latest such e, and the K tokens that followed it, the copy
// running on over its own output (token j is c[e + 1 + j mod (L - 1 - e)]).  With no
// match the proposal is the uniform random draft of the cache lookup.
//
// One block of sixteen waves per sequence.  Every candidate end e gets the length m(e)
// of the common suffix of c[..e] and c (at most min(n_max, L - 1, e + 1)); the
// answer is the largest key (m, e) with m >= n_min, so the longest n wins and, among
// equal n, the latest e.  The block scans the ends from the latest down in chunks of
// eight per thread (the first compares of a chunk are eight independent coalesced
// loads per thread; further compares only follow a first-token match) and stops
// after a chunk once some end reached the largest possible m: no earlier end can
// beat it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssd_device.h"
#include "ssd_ngram.h"

namespace ssd {
namespace {

constexpr int kNgBlock = 1024;
constexpr int kNgWaves = kNgBlock / kWave;
constexpr int kNgPer = 8;                       // candidate ends per thread per chunk
constexpr int kNgChunk = kNgBlock * kNgPer;     // ends per chunk
constexpr uint32_t kNgPurposeFallback = 3;  // the uniform fallback's generator purpose
constexpr int kNgErrLen = 4, kNgErrHist = 16;

// Token at position pos of the context of one sequence.
struct Context {
    const int32_t* hist;
    const int32_t* draft;
    int len, k, bonus;
    __device__ __forceinline__ int at(int pos) const {
        return pos < len ? hist[pos] : (pos < len + k ? draft[pos - len] : bonus);
    }
};

__global__ __launch_bounds__(kNgBlock) void ngram_kernel(const NgramArgs a) {
    __shared__ int suffix[kMaxNgram];
    __shared__ uint64_t wave_best[kNgWaves];
    const int b = blockIdx.x, tid = threadIdx.x;
    const int K = a.K;
    int32_t* out = a.tokens + (int64_t)b * K;
    int32_t* nd = a.next_draft ? a.next_draft + (int64_t)b * K : nullptr;
    // the per-sequence scalars are independent: request them together
    const int hit = a.hit ? a.hit[b] : 0;
    const int k = a.accept_len[b], len = a.hist_len[b], bonus = a.bonus[b];
    if (hit) {  // the cache gather has written this sequence's draft
        if (tid < K) out[tid] = -1;
        if (tid == 0) {
            if (a.match_n) a.match_n[b] = 0;
            if (a.match_end) a.match_end[b] = -1;
        }
        return;
    }
    const int bad = ((k < 0 || k > K) ? kNgErrLen : 0) | ((len < 0 || (int64_t)len > a.ld_hist) ? kNgErrHist : 0);
    if (bad) {
        if (tid < K) {
            out[tid] = -1;
            if (nd) nd[tid] = -1;
        }
        if (tid == 0) {
            if (a.match_n) a.match_n[b] = 0;
            if (a.match_end) a.match_end[b] = -1;
            if (a.dev_err) a.dev_err[b] |= bad;
        }
        return;
    }
    const Context c{a.hist + (int64_t)b * a.ld_hist, a.draft + (int64_t)b * K, len, k, bonus};
    const int L = len + k + 1;
    const int ncap = min(a.n_max, L - 1);  // an earlier occurrence ends at e <= L - 2
    if (tid < ncap) suffix[tid] = c.at(L - 1 - tid);
    __syncthreads();

    uint64_t best = 0ull;  // (m << 32) | e, 0 = none
    if (ncap >= a.n_min) {
        for (int top = L - 2; top >= 0; top -= kNgChunk) {  // trip count uniform over the block
            // the first compare of every end of the chunk: kNgPer independent loads
            int first[kNgPer];
#pragma unroll
            for (int j = 0; j < kNgPer; ++j) {
                const int e = top - j * kNgBlock - tid;
                first[j] = e >= 0 ? c.at(e) : 0;
            }
#pragma unroll
            for (int j = 0; j < kNgPer; ++j) {
                const int e = top - j * kNgBlock - tid;
                if (e >= 0 && first[j] == suffix[0]) {
                    const int lim = min(ncap, e + 1);
                    int m = 1;
                    while (m < lim && c.at(e - m) == suffix[m]) ++m;
                    if (m >= a.n_min) {
                        const uint64_t key = ((uint64_t)m << 32) | (uint32_t)e;
                        best = key > best ? key : best;
                    }
                }
            }
            if (__syncthreads_or((int)(best >> 32) == ncap)) break;
        }
    }
#pragma unroll
    for (int off = kWave / 2; off >= 1; off >>= 1) {
        const uint64_t o = __shfl_xor(best, off, kWave);
        best = o > best ? o : best;
    }
    if (tid % kWave == 0) wave_best[tid / kWave] = best;
    __syncthreads();
    best = wave_best[0];
#pragma unroll
    for (int w = 1; w < kNgWaves; ++w) best = wave_best[w] > best ? wave_best[w] : best;
    const int n = (int)(best >> 32);
    const int e = n ? (int)(uint32_t)best : -1;
    if (tid < K) {
        int t;
        if (n) {
            t = c.at(e + 1 + tid % (L - 1 - e));
        } else {
            const uint64_t x = philox_u32(a.seed, a.round, kNgPurposeFallback, (uint64_t)b, (uint64_t)tid);
            t = (int)((x * (uint64_t)a.V) >> 32);
        }
        out[tid] = t;
        if (nd) nd[tid] = t;
    }
    if (tid == 0) {
        if (a.match_n) a.match_n[b] = n;
        if (a.match_end) a.match_end[b] = e;
    }
}

}  // namespace

hipError_t launch_ngram(const NgramArgs& a, hipStream_t st) {
    if (a.B < 1 || a.K < 1 || a.K > kMaxK || a.n_min < 1 || a.n_max < a.n_min || a.n_max > kMaxNgram)
        return hipErrorInvalidValue;
    ngram_kernel<<<(unsigned)a.B, kNgBlock, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace ssd

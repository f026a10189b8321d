// ssd_kernels.hip -- gfx950 kernels of the verify-and-pre-speculate round of
// Speculative Speculative Decoding with the Saguaro algorithm.
//
// One round is four kernels; the two streaming ones carry all the bytes:
//  pass 1      every row of the target and draft logits [B, K+1, V] is read once.  The
//              unit of work is one wave64 and one tile of 8 x 16-byte vectors per
//              lane (4096 bf16 / 2048 fp32 elements); waves never wait for each
//              other.  Per tile: the softmax partial (max, sum of 2^{z c - o}), the
//              lowest-id argmax and, for draft rows of the cache, every element at
//              or above the F-th largest lane maximum of the tile (a lower bound of
//              the tile's F-th largest value) as a candidate key.
//  finalise    one block per sequence merges its rows: softmax statistics, cache ids
//              S_k (top F_k draft ids, ties to the lower id), M_k, the Saguaro
//              normaliser Z_k, and the lossless verification of the K draft tokens.
//  pass 2      only the rows the bonus needs (target row k, plus draft row k when
//              k < K) are read again; each wave sums the residual max(p - q', 0) of
//              its tile.
//  bonus       one wave per sequence locates the tile where the running sum crosses
//              u * sum, rescans that tile for the bonus id and does the cache lookup.
// Normalisers, cached masses, Z and every running sum that decides an integer are
// kept in fp64; per-element terms are fp32 exp2 of an exactly formed exponent.  The
// separate C-ABI calls reuse the same device code, so their results are
// bit-identical to the fused round.
#include "ssd_device.h"
#include "ssd_kernels.h"

#include <climits>
#include <type_traits>

namespace ssd {

enum { kPurposeAccept = 0, kPurposeBonus = 1, kPurposeDraft = 2, kPurposeFallback = 3 };
enum { kErrTokenRange = 1, kErrQprimeZero = 2, kErrLenRange = 4 };
constexpr int kSurvivorCap = 256;  // LDS slots per wave for the row's filtered candidates

int tile_elems(int dtype) { return dtype == 1 ? kTile<1> : kTile<0>; }
int tiles_per_row(int dtype, int V) {
    const int t = tile_elems(dtype);
    return (V + t - 1) / t;
}
int cand_cap(int Fmax) { return ((2 * Fmax + 16) + 7) / 8 * 8; }

// ============================================================================ shared pieces
// Row normalisation from the exchanged statistics (row max m, row sum
// s = sum_x 2^{(z_x - m) c}): p(x) = term(z_x, c, o) * inv with o = rint(m c).
// Sums relative to o(m) and the standard row sum differ by the factor
// f = 2^{o - m c} (|o - m c| <= 1/2); both directions use the same fp32 factor, so
// a sum converted to the standard form and back changes only by fp64 rounding.
__device__ __forceinline__ double offset_factor(float m, float c, float o) {
    return (double)__builtin_amdgcn_exp2f((float)((double)o - (double)m * (double)c));
}
struct RowNorm {
    float o;
    double inv;
};
__device__ __forceinline__ RowNorm row_norm(float m, double s_std, float c) {
    RowNorm r;
    r.o = offset_of(m, c);
    r.inv = offset_factor(m, c, r.o) / s_std;
    return r;
}
__device__ __forceinline__ double std_sum(float m, double s_rel, float c) {
    return s_rel * offset_factor(m, c, offset_of(m, c));
}

__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// (max, lowest-id argmax, sum relative to o(max)) merge; symmetric bit for bit.
__device__ __forceinline__ void merge_stats(float& m, double& s, int& arg, float m2, double s2, int a2, float c) {
    if (m2 > m || (m2 == m && a2 < arg)) arg = a2;
    merge_partial(m, s, m2, s2, c);
}

// Softmax statistics of one row from its nt tile partials, by one wave in a fixed
// order (lane-sequential, then a butterfly); every lane returns the same values.
__device__ inline void row_stats_wave(const WavePartial* P, int nt, float c, float& m, double& s, int& arg) {
    const int lane = lane_id();
    m = -INFINITY;
    s = 0.0;
    arg = INT_MAX;
    for (int t = lane; t < nt; t += kWave) {
        const WavePartial q = P[t];
        merge_stats(m, s, arg, q.m, q.s, q.arg, c);
    }
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const float m2 = __shfl_xor(m, off, kWave);
        const double s2 = __shfl_xor(s, off, kWave);
        const int a2 = __shfl_xor(arg, off, kWave);
        merge_stats(m, s, arg, m2, s2, a2, c);
    }
}

// Merge of the candidates of one draft row by one wave.  Candidate (tile t, slot s)
// is gathered by lane (s*nt + t) mod 64 into register u = (s*nt + t) / 64, so every
// load address is known up front and all loads of a row are in flight together.
constexpr int kCandRegs = 24;    // register slots per lane: up to 1536 candidates per row
constexpr int kMaxMergeTiles = 512;

struct TopfScratch {
    uint64_t surv[kSurvivorCap];  // keys at or above the value threshold
    uint64_t rank[kWave];         // the top F, placed by rank
    uint8_t nc[kMaxMergeTiles];   // candidates per tile
};

// The largest 32-bit value part T such that at least F of the nonzero keys have a
// value part >= T (the F-th largest value, ties counted), by the same radix select as
// wave_select_regs restricted to the value bits; 0 when there are at most F keys.
template <int KREG>
__device__ inline uint32_t wave_select_value(const uint64_t (&k)[KREG], int F) {
    int n = 0;
    uint32_t orv = 0u, andv = ~0u;
#pragma unroll
    for (int u = 0; u < KREG; ++u) {
        n += wave_popc(k[u] != 0ull);
        if (k[u] != 0ull) {
            orv |= (uint32_t)(k[u] >> 32);
            andv &= (uint32_t)(k[u] >> 32);
        }
    }
    if (n <= F) return 0u;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        orv |= (uint32_t)__shfl_xor((int)orv, m, kWave);
        andv &= (uint32_t)__shfl_xor((int)andv, m, kWave);
    }
    uint32_t diff = orv ^ andv;
    uint32_t T = andv & ~diff;
    while (diff) {
        const int bit = 31 - __clz(diff);
        diff &= ~(1u << bit);
        const uint64_t cand = (uint64_t)(T | (1u << bit)) << 32;
        int cnt = 0;
#pragma unroll
        for (int u = 0; u < KREG; ++u) cnt += wave_popc(k[u] >= cand);
        if (cnt >= F) T |= 1u << bit;
    }
    return T;
}

// Sorts the n <= kSurvivorCap distinct keys in sc.surv by rank and returns lane j =
// the j-th largest (0 past min(n, F)).
__device__ inline uint64_t rank_sort_lds(TopfScratch& sc, int n, int F) {
    const int lane = lane_id();
    uint64_t k[4];
    int rank[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int j = u * kWave + lane;
        k[u] = j < n ? sc.surv[j] : 0ull;
        rank[u] = 0;
    }
    if (n <= kWave) {
        for (int v = 0; v < n; ++v) rank[0] += sc.surv[v] > k[0];
    } else {
        for (int v = 0; v < n; ++v) {
            const uint64_t x = sc.surv[v];
#pragma unroll
            for (int u = 0; u < 4; ++u) rank[u] += x > k[u];
        }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
        if (k[u] != 0ull && rank[u] < F) sc.rank[rank[u]] = k[u];
    wave_sync_lds();
    const uint64_t key = lane < min(n, F) ? sc.rank[lane] : 0ull;
    wave_sync_lds();
    return key;
}

// Appends the keys of k[] that satisfy keep (in register, then lane order) to sc.surv;
// returns the count (keys past kSurvivorCap are counted, not stored).
template <int KREG>
__device__ inline int compact_keys(TopfScratch& sc, const uint64_t (&k)[KREG], uint64_t lo) {
    int n = 0;
#pragma unroll
    for (int u = 0; u < KREG; ++u) {
        const bool keep = k[u] != 0ull && k[u] >= lo;
        const int pos = n + lanes_below(keep);
        if (keep && pos < kSurvivorCap) sc.surv[pos] = k[u];
        n += wave_popc(keep);
    }
    wave_sync_lds();
    return n;
}

// Candidate key number j of a 64-tile chunk (flattened in tile order) of a row: the
// tile is the last one whose first slot is <= j.  start: the chunk's first slots, in
// sc.surv reinterpreted (slow path only).
__device__ __forceinline__ uint64_t chunk_key(const uint64_t* cand, int cap, int c0, const int* start, int j) {
    int lo = 0;
#pragma unroll
    for (int step = 32; step >= 1; step >>= 1)
        if (start[lo + step] <= j) lo += step;
    return cand[(int64_t)(c0 + lo) * cap + (j - start[lo])];
}

// Top F of one draft row from its tiles' candidate keys, by one wave.  The largest
// tile threshold bounds the row's F-th largest value from below (that tile alone has
// F elements at or above it), so only keys at or above it can be in the row's top F,
// and every such key is in its tile's list.  Keys are distinct (they carry the id).
// Returns lane j = the j-th largest key (0 past F).
__device__ __forceinline__ uint64_t row_topf_wave(const WavePartial* P, const uint64_t* cand, int nt, int cap, int F,
                                         TopfScratch& sc) {
    const int lane = lane_id();
    uint32_t tr = 0u;
    int max_nc = 0;
    for (int t = lane; t < nt; t += kWave) {
        const WavePartial q = P[t];
        tr = max(tr, q.tau);
        max_nc = max(max_nc, q.ncand);
        if (t < kMaxMergeTiles) sc.nc[t] = (uint8_t)q.ncand;
    }
    tr = wave_max_u32(tr);
    max_nc = (int)wave_max_u32((uint32_t)max_nc);
    const uint64_t floor_key = (uint64_t)tr << 32;
    wave_sync_lds();
    const int U = (int)(((int64_t)nt * max_nc + kWave - 1) / kWave);

    if (nt <= kMaxMergeTiles && U <= kCandRegs) {
        uint64_t k[kCandRegs];
        int t = lane % nt, sl = lane / nt;
        // opaque to the optimiser: keeps the 24 slot addresses from being hoisted out of
        // a caller's loop over rows (they would stay live in registers across it)
        __asm__ volatile("" : "+v"(t), "+v"(sl));
        const int dt = kWave % nt, ds = kWave / nt;
#pragma unroll
        for (int u = 0; u < kCandRegs; ++u) {
            uint64_t x = 0ull;
            if (u < U && sl < (int)sc.nc[t]) x = cand[(int64_t)t * cap + sl];
            k[u] = x >= floor_key ? x : 0ull;
            t += dt;
            sl += ds;
            if (t >= nt) {
                t -= nt;
                ++sl;
            }
        }
        const uint32_t T = wave_select_value<kCandRegs>(k, F);
        const uint64_t lo = (uint64_t)T << 32;
        int n = compact_keys<kCandRegs>(sc, k, lo);
        if (n > kSurvivorCap) {
            // many keys tie at the threshold value: select on the whole key
#pragma unroll
            for (int u = 0; u < kCandRegs; ++u) k[u] = k[u] >= lo ? k[u] : 0ull;
            const uint64_t T64 = wave_select_regs<kCandRegs>(k, F);
            n = compact_keys<kCandRegs>(sc, k, T64);
        }
        return rank_sort_lds(sc, n, F);
    }

    // Rows with more candidates than register slots: exact selection by F rounds of a
    // wave maximum below the previous key.
    int* start = reinterpret_cast<int*>(sc.surv);
    uint64_t key = 0ull, prev = ~0ull;
    for (int r = 0; r < F; ++r) {
        uint64_t best = 0ull;
        for (int c0 = 0; c0 < nt; c0 += kWave) {
            const int nc = c0 + lane < nt ? P[c0 + lane].ncand : 0;
            int incl = nc;
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) {
                const int y = __shfl_up(incl, off, kWave);
                if (lane >= off) incl += y;
            }
            const int tot = __shfl(incl, kWave - 1, kWave);
            start[lane] = incl - nc;
            wave_sync_lds();
            for (int j = lane; j < tot; j += kWave) {
                const uint64_t x = chunk_key(cand, cap, c0, start, j);
                if (x >= floor_key && x < prev && x > best) best = x;
            }
            wave_sync_lds();
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const uint64_t o = __shfl_xor(best, off, kWave);
            best = o > best ? o : best;
        }
        if (lane == r) key = best;
        prev = best;
    }
    return key;
}

// Cache ids (sorted) and cached mass M = sum of q(x) over them, of one draft row.
__device__ __forceinline__ double cache_row_wave(const WavePartial* P, const uint64_t* cand, int nt, int cap, int F, float mq,
                                        double sq, float c, int greedy, int32_t* ids_out, int* ids_lds,
                                        TopfScratch& sc) {
    const int lane = lane_id();
    if (F <= 0) return 0.0;
    const uint64_t key = row_topf_wave(P, cand, nt, cap, F, sc);
    const int id = key ? (int)key_id(key) : -1;
    if (lane < F) {
        ids_out[lane] = id;
        if (ids_lds) ids_lds[lane] = id;
    }
    double t = 0.0;
    if (lane < F && key) {
        if (greedy) {
            t = lane == 0 ? 1.0 : 0.0;
        } else {
            const RowNorm nq = row_norm(mq, sq, c);
            t = (double)term(key_val(key), c, nq.o) * nq.inv;
        }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) t += __shfl_xor(t, m, kWave);
    return t;
}

// Cache lookup of one verified outcome (k, tok) by one wave, plus the uniform
// fallback draft on a miss.  my_id: lane j < F_k holds the j-th cached id of outcome
// k (slot O_k + j); other lanes, and every lane when k is invalid (k < 0), hold -1.
__device__ inline void lookup_wave(int b, int K, int V, int k, int Ok, int my_id, int tok, int fallback,
                                   uint64_t seed, uint64_t round, uint8_t* hit, int32_t* slot, int32_t* fb) {
    const int lane = lane_id();
    const uint64_t mk = __ballot(k >= 0 && my_id >= 0 && my_id == tok);
    const bool h = mk != 0ull;
    if (lane == 0) {
        hit[b] = h ? 1 : 0;
        slot[b] = h ? Ok + (__ffsll((long long)mk) - 1) : -1;
    }
    for (int j = lane; j < K; j += kWave) {
        int32_t t = -1;
        if (!h && fallback) {
            const uint64_t u32 = philox_u32(seed, round, kPurposeFallback, (uint64_t)b, (uint64_t)j);
            t = (int32_t)((u32 * (uint64_t)V) >> 32);
        }
        fb[(int64_t)b * K + j] = t;
    }
}

// The cached id of lane j of outcome k of sequence b (-1 past F_k or for k invalid).
__device__ __forceinline__ int cached_id(const int32_t* cache_ids, int b, int Bf, int k, int K, const int* F,
                                         const int* O) {
    const int lane = lane_id();
    if (k < 0 || k > K || lane >= F[k]) return -1;
    return cache_ids[(int64_t)b * Bf + O[k] + lane];
}

// What lane i < K needs to test draft token d_i, loaded ahead of the row statistics:
// the token, both models' logits at it (when d_i is in range and T > 0) and the
// acceptance uniform.
struct DraftProbe {
    int d;
    float zp, zq;
    float u;
};

template <int DT>
__device__ inline DraftProbe probe_draft(const int32_t* draft, const char* p_logits, const char* q_logits,
                                         int64_t ld_bytes, int b, int K, int V, int greedy, uint64_t seed,
                                         uint64_t round) {
    const int i = lane_id();
    DraftProbe pr;
    pr.d = i < K ? draft[(int64_t)b * K + i] : 0;
    pr.zp = pr.zq = 0.f;
    if (i < K && !greedy && pr.d >= 0 && pr.d < V) {
        const int64_t r = (int64_t)b * (K + 1) + i;
        pr.zp = load_one<DT>(p_logits + r * ld_bytes, pr.d);
        pr.zq = load_one<DT>(q_logits + r * ld_bytes, pr.d);
    }
    pr.u = (i < K && !greedy) ? philox_uniform(seed, round, kPurposeAccept, (uint64_t)b, (uint64_t)i) : 0.f;
    return pr;
}

// Verification of the K draft tokens of sequence b by one wave: lane i < K tests
// position i with that position's row statistics.  Returns the accepted length k
// (same in every lane); writes accept_prob and the OR of the error bits to *errs.
__device__ inline int verify_wave(int b, int K, int V, const DraftProbe& pr, float mp, double sp, int argp, float mq,
                                  double sq, double Zi, bool in_cache, float C, float c, int greedy,
                                  float* accept_prob, int* errs) {
    const int i = lane_id();
    const bool act = i < K;
    const int d = pr.d;
    int err = 0;
    bool ok = act;
    double ratio = 0.0;
    if (act && (d < 0 || d >= V)) {
        err |= kErrTokenRange;
        ok = false;
    }
    if (ok) {
        if (greedy) {
            ratio = (d == argp) ? 1.0 : 0.0;
        } else {
            const RowNorm np = row_norm(mp, sp, c), nq = row_norm(mq, sq, c);
            const double p = (double)term(pr.zp, c, np.o) * np.inv;
            const double q = (double)term(pr.zq, c, nq.o) * nq.inv;
            const double qp = q * (in_cache ? (double)C : 1.0) / Zi;
            if (!(qp > 0.0)) {
                err |= kErrQprimeZero;
                ok = false;
            } else {
                ratio = p / qp;
            }
        }
    }
    bool acc = false;
    if (ok) acc = greedy ? ratio == 1.0 : (double)pr.u < ratio;
    const uint64_t rej = __ballot(act && !acc);
    const int k = rej ? (__ffsll((long long)rej) - 1) : K;
    if (act && accept_prob) accept_prob[(int64_t)b * K + i] = (float)(ratio < 1.0 ? ratio : 1.0);
    int e = err;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) e |= __shfl_xor(e, m, kWave);
    *errs = e;
    return k;
}

// ============================================================================ pass 1
template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void pass1_kernel(const Pass1Args a) {
    constexpr int N = ElemTraits<DT>::kPerVec;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int nblk = (a.nt + kWavesPerBlock - 1) / kWavesPerBlock;
    int bid = blockIdx.x;
    const int blk = bid % nblk;
    bid /= nblk;
    const int i = bid % a.K1;
    bid /= a.K1;
    const int model = bid % a.nmodel;
    const int b = bid / a.nmodel;
    const int t = blk * kWavesPerBlock + wave;
    if (t >= a.nt) return;
    const int64_t r = (int64_t)b * a.K1 + i;
    const char* row = a.logits[model] + r * a.ld_bytes;
    const int64_t tile0 = (int64_t)t * kTile<DT>;
    const int V = a.V;
    const float c = a.c;

    float x[kVecPerLane][N];
    {
        u32x4 raw[kVecPerLane];
        load_tile<DT, VEC>(row, tile0, V, lane, raw);
#pragma unroll
        for (int j = 0; j < kVecPerLane; ++j) unpack_vec<DT>(raw[j], x[j]);
    }

    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < kVecPerLane; ++j)
#pragma unroll
        for (int e = 0; e < N; ++e) m = fmaxf(m, x[j][e]);
    const float m_lane = m;

    int arg = INT_MAX;
    if (a.want_arg) {
#pragma unroll
        for (int j = 0; j < kVecPerLane; ++j)
#pragma unroll
            for (int e = 0; e < N; ++e) {
                const int64_t id = tile0 + (int64_t)(j * kWave + lane) * N + e;
                if (arg == INT_MAX && id < V && x[j][e] == m_lane) arg = (int)id;
            }
    }

    double s = 0.0;
    if (!a.greedy && m_lane != -INFINITY) {
        const float o = offset_of(m_lane, c);
        float vs[kVecPerLane];
#pragma unroll
        for (int j = 0; j < kVecPerLane; ++j) {
            float tt[N];
#pragma unroll
            for (int e = 0; e < N; ++e) tt[e] = term(x[j][e], c, o);
#pragma unroll
            for (int w = N / 2; w >= 1; w >>= 1)
#pragma unroll
                for (int e = 0; e < w; ++e) tt[e] += tt[e + w];
            vs[j] = tt[0];
        }
#pragma unroll
        for (int w = kVecPerLane / 2; w >= 1; w >>= 1)
#pragma unroll
            for (int j = 0; j < w; ++j) vs[j] += vs[j + w];
        s = (double)vs[0];
    }

    // ---- candidate keys of this tile (draft rows of the cache): every element at or
    // above the F-th largest lane maximum.
    const int F = a.F[i];
    uint32_t tau = 0u;
    int ncand = 0;
    if (model == a.topf_model && F > 0) {
        const bool lane_valid = tile0 + (int64_t)lane * N < V;
        tau = wave_select_u32(lane_valid ? ord32(m_lane) : 0u, F);
        const float tauf = tau ? unord32(tau) : -INFINITY;
        const int id0 = (int)tile0 + lane * N;
        const bool full = tile0 + kTile<DT> <= V;
        uint32_t mask[kVecPerLane];
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < kVecPerLane; ++j) {
            uint32_t mk = 0u;
#pragma unroll
            for (int e = 0; e < N; ++e)
                mk |= (x[j][e] >= tauf && (full || id0 + j * kWave * N + e < V)) ? (1u << e) : 0u;
            mask[j] = mk;
            cnt += __popc(mk);
        }
        int incl = cnt;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int y = __shfl_up(incl, off, kWave);
            if (lane >= off) incl += y;
        }
        const int tot = __shfl(incl, kWave - 1, kWave);
        uint64_t* out = a.cand + ((r * a.nt) + t) * a.cap;
        if (tot <= a.cap) {
            int pos = incl - cnt;
#pragma unroll
            for (int j = 0; j < kVecPerLane; ++j) {
                uint32_t mk = mask[j];
                while (mk) {
                    const int e = __ffs(mk) - 1;
                    mk &= mk - 1u;
                    float v = x[j][0];
#pragma unroll
                    for (int q = 1; q < N; ++q) v = (e == q) ? x[j][q] : v;
                    out[pos++] = cand_key(v, (uint32_t)(id0 + j * kWave * N + e));
                }
            }
            ncand = tot;
        } else {
            // More tied candidates than slots: store this tile's exact top F, found by
            // F rounds of a wave maximum below the previous key (re-reading the tile).
            uint64_t prev = ~0ull;
#pragma unroll 1
            for (int q = 0; q < F; ++q) {
                uint64_t best = 0ull;
#pragma unroll 1
                for (int j = 0; j < kVecPerLane; ++j) {
                    const int64_t e0 = tile0 + (int64_t)(j * kWave + lane) * N;
#pragma unroll 1
                    for (int e = 0; e < N; ++e) {
                        if (e0 + e < V) {
                            const uint64_t kk = cand_key(load_one<DT>(row, e0 + e), (uint32_t)(e0 + e));
                            if (kk < prev && kk > best) best = kk;
                        }
                    }
                }
#pragma unroll
                for (int off = 32; off >= 1; off >>= 1) {
                    const uint64_t o = __shfl_xor(best, off, kWave);
                    best = o > best ? o : best;
                }
                if (lane == 0) out[q] = best;
                prev = best;
            }
            ncand = F;
        }
    }

    // ---- tile partial
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float m2 = __shfl_xor(m, off, kWave);
        const double s2 = __shfl_xor(s, off, kWave);
        const int a2 = __shfl_xor(arg, off, kWave);
        merge_stats(m, s, arg, m2, s2, a2, c);
    }
    if (lane == 0) {
        WavePartial P;
        P.m = m;
        P.arg = arg;
        P.s = s;
        P.tau = tau;
        P.ncand = ncand;
        P.pad0 = P.pad1 = 0;
        a.part[(((int64_t)b * a.nmodel + model) * a.K1 + i) * a.nt + t] = P;
    }
}

// ============================================================================ finalise
constexpr int kFinWaves = 8;
constexpr int kFinBlock = kFinWaves * kWave;

struct FinShared {
    float m[2][kMaxK + 1];
    double s[2][kMaxK + 1];
    int arg[2][kMaxK + 1];
    double Z[kMaxK + 1];
    int ids[kMaxK + 1][kMaxF];
    TopfScratch tf[kFinWaves];
};

// One block of 8 waves per sequence.  Wave w < K+1 takes draft row w (statistics,
// cache ids, cached mass M, Saguaro Z = 1 - (1 - C) M), the next K+1 waves the target
// rows; the last wave loads what verification needs first and verifies once every
// row is done.
template <int DT>
__global__ __launch_bounds__(kFinBlock) void finalize_seq_kernel(const SeqFinal f) {
    __shared__ FinShared fs;
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int b = blockIdx.x;
    const int K = f.K, K1 = K + 1;
    const WavePartial* part = f.part + (int64_t)b * 2 * K1 * f.nt;
    const bool verifier = wave == kFinWaves - 1;
    DraftProbe pr{};
    if (verifier)
        pr = probe_draft<DT>(f.draft, f.p_logits, f.q_logits, f.ld_bytes, b, K, f.V, f.greedy, f.seed, f.round);

    for (int rr = wave; rr < 2 * K1; rr += kFinWaves) {
        const int model = rr < K1 ? 1 : 0, i = rr < K1 ? rr : rr - K1;
        const int64_t r = (int64_t)b * K1 + i;
        float m;
        double s;
        int arg;
        row_stats_wave(part + (int64_t)(model * K1 + i) * f.nt, f.nt, f.c, m, s, arg);
        s = f.greedy ? 1.0 : std_sum(m, s, f.c);
        if (lane == 0) {
            fs.m[model][i] = m;
            fs.s[model][i] = s;
            fs.arg[model][i] = arg;
            if (model) {
                f.q_max[r] = m;
                f.q_sum[r] = s;
                if (f.q_arg) f.q_arg[r] = arg;
            } else {
                f.p_max[r] = m;
                f.p_sum[r] = s;
                if (f.p_arg) f.p_arg[r] = arg;
            }
        }
        if (model) {
            const double M = cache_row_wave(part + (int64_t)(K1 + i) * f.nt, f.cand + r * f.nt * f.cap, f.nt, f.cap,
                                            f.F[i], m, s, f.c, f.greedy, f.cache_ids + (int64_t)b * f.Bf + f.O[i],
                                            fs.ids[i], fs.tf[wave]);
            const double Z = 1.0 - (1.0 - (double)f.C) * M;
            if (lane == 0) {
                f.cache_mass[r] = M;
                f.Z[r] = Z;
                fs.Z[i] = Z;
            }
        }
    }
    __syncthreads();

    if (!verifier) return;
    const int i = lane;
    const int ic = i < K ? i : 0;
    bool in_cache = false;
    for (int j = 0; j < f.F[ic]; ++j) in_cache |= fs.ids[ic][j] == pr.d;
    int errs;
    const int k = verify_wave(b, K, f.V, pr, fs.m[0][ic], fs.s[0][ic], fs.arg[0][ic], fs.m[1][ic], fs.s[1][ic],
                              fs.Z[ic], in_cache, f.C, f.c, f.greedy, f.accept_prob, &errs);
    if (lane == 0) {
        f.accept_len[b] = k;
        if (f.dev_err && errs) f.dev_err[b] |= errs;
    }
    if (f.greedy) {
        const int tok = fs.arg[0][k];
        if (lane == 0) {
            f.bonus[b] = tok;
            if (f.resid_mass) f.resid_mass[b] = 1.0;
        }
        const int my_id = lane < f.F[k] ? fs.ids[k][lane] : -1;
        lookup_wave(b, K, f.V, k, f.O[k], my_id, tok, f.fallback, f.seed, f.round, f.hit, f.slot, f.fallback_tokens);
    }
}

// ============================================================================ pass 2
enum { kWResid = 0, kWP = 1, kWQprime = 2 };

struct WParams {
    float c;
    float op, oq;       // offsets of the target / draft rows
    double inv_p;       // p(x) = term(z_p, c, op) * inv_p
    double sc_q, sc_qC; // q'(x) = term(z_q, c, oq) * (sc_qC if cached else sc_q)
};

// Row statistics of one (b, position), loaded together with no branch in between so
// that they travel with the tile loads.  Without a target law (draft sampling) the
// draft statistics stand in for it and are not used.
struct LawIn {
    float pm, qm;
    double ps, qs, Z;
};
__device__ __forceinline__ LawIn load_law(const Pass2Args& a, int64_t r) {
    const float* pmx = a.p_max ? a.p_max : a.q_max;
    const double* psx = a.p_sum ? a.p_sum : a.q_sum;
    LawIn L;
    L.pm = pmx[r];
    L.ps = psx[r];
    L.qm = a.q_max[r];
    L.qs = a.q_sum[r];
    L.Z = a.Z[r];
    return L;
}

__device__ __forceinline__ WParams make_wparams(float c, float C, bool with_p, const LawIn& L) {
    WParams w;
    w.c = c;
    w.op = 0.f;
    w.inv_p = 0.0;
    if (with_p) {
        const RowNorm np = row_norm(L.pm, L.ps, c);
        w.op = np.o;
        w.inv_p = np.inv;
    }
    const RowNorm nq = row_norm(L.qm, L.qs, c);
    w.oq = nq.o;
    w.sc_q = nq.inv / L.Z;
    w.sc_qC = w.sc_q * (double)C;
    return w;
}

// Weight of one element for the inverse-CDF scan (fp64); *pw receives p(x).
template <int MODE>
__device__ __forceinline__ double elem_weight_t(const WParams& w, float zp, float zq, bool in_cache, double* pw) {
    double p = 0.0;
    if (MODE != kWQprime) p = (double)term(zp, w.c, w.op) * w.inv_p;
    *pw = p;
    if (MODE == kWP) return p;
    const double q = (double)term(zq, w.c, w.oq) * (in_cache ? w.sc_qC : w.sc_q);
    if (MODE == kWQprime) return q;
    const double d = p - q;
    return d > 0.0 ? d : 0.0;
}

// Wave-private membership bitmap (kTile/32 words) of the cached ids of a row that
// fall in the tile [t0, t0 + kTile); lane j holds cached id j (or -1) in my_id.
template <int DT>
__device__ inline void tile_bitmap(uint32_t* bits, int64_t t0, int my_id) {
    const int lane = lane_id();
    for (int w = lane; w < kTile<DT> / 32; w += kWave) bits[w] = 0u;
    wave_sync_lds();
    if (my_id >= t0 && my_id < t0 + kTile<DT>)
        atomicOr(&bits[(my_id - t0) >> 5], 1u << ((my_id - t0) & 31));
    wave_sync_lds();
}

// Weights of one lane's vector j of a tile from the raw vectors of the target and
// draft rows; elements past V weigh 0.
template <int DT, int MODE>
__device__ __forceinline__ void vec_weights(const WParams& wp, u32x4 rp, u32x4 rq, int64_t e0, int V,
                                            const uint32_t* bits, int64_t t0, double* w, double* p) {
    constexpr int N = ElemTraits<DT>::kPerVec;
    float zp[N], zq[N];
    if (MODE != kWQprime) unpack_vec<DT>(rp, zp);
    if (MODE != kWP) unpack_vec<DT>(rq, zq);
    uint32_t cbits = 0u;
    if (MODE != kWP) cbits = bits[(e0 - t0) >> 5] >> ((e0 - t0) & 31);
#pragma unroll
    for (int e = 0; e < N; ++e) {
        w[e] = elem_weight_t<MODE>(wp, MODE != kWQprime ? zp[e] : 0.f, MODE != kWP ? zq[e] : 0.f, (cbits >> e) & 1u,
                                   &p[e]);
        if (e0 + e >= V) {
            w[e] = 0.0;
            p[e] = 0.0;
        }
    }
}

// Sums over one lane's part of a wave tile: sw of the weights, sp of p(x).  The tile
// and the row statistics are requested before any of them is used.
template <int DT, bool VEC, int MODE>
__device__ __forceinline__ void tile_sums(const Pass2Args& a, int64_t r, const char* prow, const char* qrow, int64_t t0,
                                          const int32_t* ids, int Fk, uint32_t* bits, double& sw, double& sp) {
    constexpr int N = ElemTraits<DT>::kPerVec;
    const int lane = lane_id();
    u32x4 rp[kVecPerLane], rq[kVecPerLane];
    if (MODE != kWQprime) load_tile<DT, VEC>(prow, t0, a.V, lane, rp);
    if (MODE != kWP) load_tile<DT, VEC>(qrow, t0, a.V, lane, rq);
    int my_id = -1;
    if (MODE != kWP && lane < Fk) my_id = ids[lane];
    const LawIn L = load_law(a, r);
    const WParams wp = make_wparams(a.c, a.C, MODE != kWQprime, L);
    if (MODE != kWP) tile_bitmap<DT>(bits, t0, my_id);
#pragma unroll
    for (int j = 0; j < kVecPerLane; ++j) {
        const int64_t e0 = t0 + (int64_t)(j * kWave + lane) * N;
        double w[N], p[N];
        vec_weights<DT, MODE>(wp, rp[j], rq[j], e0, a.V, bits, t0, w, p);
        double vw = 0.0, vp = 0.0;
#pragma unroll
        for (int e = 0; e < N; ++e) {
            vw += w[e];
            vp += p[e];
        }
        sw += vw;
        sp += vp;
    }
}

__device__ inline void pass2_group(const Pass2Args& a, int g, int& b, int& pos, bool& valid) {
    if (a.mode == 0) {
        b = g;
        pos = a.accept_len[b];
        valid = pos >= 0 && pos <= a.K;
    } else {
        b = g / a.K;
        pos = g % a.K;
        valid = true;
    }
    if (!valid) pos = 0;
}

__device__ __forceinline__ int pass2_mode(const Pass2Args& a, int pos) {
    return a.mode == 1 ? kWQprime : (pos < a.K ? kWResid : kWP);
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void pass2_kernel(const Pass2Args a) {
    __shared__ uint32_t bits[kWavesPerBlock][kTile<1> / 32];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int nblk = (a.nt + kWavesPerBlock - 1) / kWavesPerBlock;
    const int g = blockIdx.x / nblk;
    const int t = (blockIdx.x % nblk) * kWavesPerBlock + wave;
    if (t >= a.nt) return;
    int b, pos;
    bool valid;
    pass2_group(a, g, b, pos, valid);
    double sw = 0.0, sp = 0.0;
    if (valid) {
        const int64_t r = (int64_t)b * (a.K + 1) + pos;
        const int mode = pass2_mode(a, pos);
        const char* prow = a.p_logits ? a.p_logits + r * a.ld_bytes : nullptr;
        const char* qrow = a.q_logits + r * a.ld_bytes;
        const int64_t t0 = (int64_t)t * kTile<DT>;
        const int32_t* ids = a.cache_ids + (int64_t)b * a.Bf + a.O[pos];
        const int Fk = a.F[pos];
        if (mode == kWResid)
            tile_sums<DT, VEC, kWResid>(a, r, prow, qrow, t0, ids, Fk, bits[wave], sw, sp);
        else if (mode == kWP)
            tile_sums<DT, VEC, kWP>(a, r, prow, qrow, t0, ids, Fk, bits[wave], sw, sp);
        else
            tile_sums<DT, VEC, kWQprime>(a, r, prow, qrow, t0, ids, Fk, bits[wave], sw, sp);
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        sw += __shfl_xor(sw, m, kWave);
        sp += __shfl_xor(sp, m, kWave);
    }
    if (lane == 0) a.seg[(int64_t)g * a.nt + t] = make_double2(sw, sp);
}

// Rescan of one tile element by element in id order: the first id whose running sum
// (starting at base) exceeds thr, or with pick_last the last id of positive weight.
// The caller has issued the tile loads (rp, rq).
template <int DT, int MODE>
__device__ inline int rescan_tile(const WParams& wp, const u32x4 (&rp)[kVecPerLane], const u32x4 (&rq)[kVecPerLane],
                                  int64_t t0, int V, int my_id, uint32_t* bits, double base, double thr,
                                  bool pick_last) {
    constexpr int N = ElemTraits<DT>::kPerVec;
    const int lane = lane_id();
    if (MODE != kWP) tile_bitmap<DT>(bits, t0, my_id);
    double run = base;
    int found = -1, last_pos = -1;
#pragma unroll
    for (int j = 0; j < kVecPerLane; ++j) {
        const int64_t e0 = t0 + (int64_t)(j * kWave + lane) * N;
        double w[N], p[N];
        vec_weights<DT, MODE>(wp, rp[j], rq[j], e0, V, bits, t0, w, p);
        double ls = 0.0;
#pragma unroll
        for (int e = 0; e < N; ++e) ls += w[e];
        double incl = ls;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const double y = __shfl_up(incl, off, kWave);
            if (lane >= off) incl += y;
        }
        double cum = run + (incl - ls);
        int hitpos = -1, lastp = -1;
#pragma unroll
        for (int e = 0; e < N; ++e) {
            cum += w[e];
            if (hitpos < 0 && cum > thr) hitpos = (int)(e0 + e);
            if (w[e] > 0.0) lastp = (int)(e0 + e);
        }
        if (!pick_last && found < 0) {
            const uint64_t hm = __ballot(hitpos >= 0);
            if (hm) found = __shfl(hitpos, __ffsll((long long)hm) - 1, kWave);
        }
        const uint64_t lm = __ballot(lastp >= 0);
        if (lm) last_pos = __shfl(lastp, 63 - __clzll(lm), kWave);
        run += __shfl(incl, kWave - 1, kWave);
    }
    return found >= 0 ? found : (last_pos >= 0 ? last_pos : (int)min<int64_t>(t0, V - 1));
}

// Inclusive wave scan of x (fp64, lane order).
__device__ __forceinline__ double wave_scan_incl(double x) {
    const int lane = lane_id();
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const double y = __shfl_up(x, off, kWave);
        if (lane >= off) x += y;
    }
    return x;
}

// One wave per group: totals over the tiles in tile order, the tile where the running
// sum crosses u * total, the id inside it, and the cache lookup.  The tile sums of the
// first 64 tiles, the row statistics and the cached ids are requested together.
template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void finalize_bonus_kernel(const Pass2Args a, int ngroups) {
    __shared__ uint32_t bits[kWavesPerBlock][kTile<1> / 32];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int g = blockIdx.x * kWavesPerBlock + wave;
    if (g >= ngroups) return;
    int b, pos;
    bool valid;
    pass2_group(a, g, b, pos, valid);
    const int K = a.K;
    const int nt = a.nt;
    const double2* seg = a.seg + (int64_t)g * nt;
    int tok = -1;
    double Zused = 0.0;
    const int my_id = valid ? cached_id(a.cache_ids, b, a.Bf, pos, K, a.F, a.O) : -1;
    if (valid) {
        const int64_t r = (int64_t)b * (K + 1) + pos;
        const double2 v0 = lane < nt ? seg[lane] : make_double2(0.0, 0.0);
        const LawIn L = load_law(a, r);
        const uint32_t purpose = a.mode == 0 ? kPurposeBonus : kPurposeDraft;
        const double u = (double)philox_uniform(a.seed, a.round, purpose, (uint64_t)b, (uint64_t)pos);
        double tot_w = 0.0, tot_p = 0.0;
        for (int g0 = 0; g0 < nt; g0 += kWave) {
            const int j = g0 + lane;
            double2 v = v0;
            if (g0 > 0) v = j < nt ? seg[j] : make_double2(0.0, 0.0);
            tot_w += __shfl(wave_scan_incl(v.x), kWave - 1, kWave);
            tot_p += __shfl(wave_scan_incl(v.y), kWave - 1, kWave);
        }
        int mode = pass2_mode(a, pos);
        double Z = tot_w;
        const bool use_p = mode == kWResid && !(Z > 0.0);
        if (use_p) {
            mode = kWP;
            Z = tot_p;
        }
        Zused = Z;
        const double thr = u * Z;
        int gsel = -1, glast = -1;
        double gbase = 0.0, lastbase = 0.0, carry = 0.0;
        for (int g0 = 0; g0 < nt; g0 += kWave) {
            const int j = g0 + lane;
            double2 v = v0;
            if (g0 > 0) v = j < nt ? seg[j] : make_double2(0.0, 0.0);
            const double x = use_p ? v.y : v.x;
            const double incl = wave_scan_incl(x) + carry;
            const double excl = incl - x;
            const uint64_t cross = __ballot(j < nt && incl > thr);
            const uint64_t posm = __ballot(j < nt && x > 0.0);
            if (gsel < 0 && cross) {
                const int l = __ffsll((long long)cross) - 1;
                gsel = g0 + l;
                gbase = __shfl(excl, l, kWave);
            }
            if (posm) {
                const int l = 63 - __clzll(posm);
                glast = g0 + l;
                lastbase = __shfl(excl, l, kWave);
            }
            carry = __shfl(incl, kWave - 1, kWave);
        }
        bool pick_last = false;
        if (gsel < 0) {
            gsel = glast < 0 ? 0 : glast;
            gbase = lastbase;
            pick_last = true;
        }
        const int64_t t0 = (int64_t)gsel * kTile<DT>;
        const char* prow = a.p_logits ? a.p_logits + r * a.ld_bytes : nullptr;
        const char* qrow = a.q_logits + r * a.ld_bytes;
        u32x4 rp[kVecPerLane], rq[kVecPerLane];
        if (mode != kWQprime) load_tile<DT, VEC>(prow, t0, a.V, lane, rp);
        if (mode != kWP) load_tile<DT, VEC>(qrow, t0, a.V, lane, rq);
        const WParams wp = make_wparams(a.c, a.C, mode != kWQprime, L);
        if (mode == kWResid)
            tok = rescan_tile<DT, kWResid>(wp, rp, rq, t0, a.V, my_id, bits[wave], gbase, thr, pick_last);
        else if (mode == kWP)
            tok = rescan_tile<DT, kWP>(wp, rp, rq, t0, a.V, my_id, bits[wave], gbase, thr, pick_last);
        else
            tok = rescan_tile<DT, kWQprime>(wp, rp, rq, t0, a.V, my_id, bits[wave], gbase, thr, pick_last);
    }
    if (lane == 0) {
        if (a.mode == 0) {
            a.out_tok[b] = tok;
            if (a.resid_mass) a.resid_mass[b] = Zused;
            if (!valid && a.dev_err) a.dev_err[b] |= kErrLenRange;
        } else {
            a.out_tok[(int64_t)b * K + pos] = tok;
        }
    }
    if (a.mode == 0 && a.do_lookup)
        lookup_wave(b, K, a.V, valid ? pos : -1, valid ? a.O[pos] : 0, my_id, tok, a.fallback, a.seed, a.round, a.hit,
                    a.slot, a.fallback_tokens);
}

// ============================================================================ small kernels
// Per-row merges for the separate calls: one wave per row (same code as the round).
__global__ __launch_bounds__(kBlock) void combine_stats_kernel(const Pass1Args a, float* m_out, double* s_out,
                                                               int32_t* arg_out) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int64_t r = (int64_t)blockIdx.x * kWavesPerBlock + wave;
    if (r >= (int64_t)a.B * a.K1) return;
    float m;
    double s;
    int arg;
    row_stats_wave(a.part + r * a.nt, a.nt, a.c, m, s, arg);
    if (lane == 0) {
        m_out[r] = m;
        s_out[r] = a.greedy ? 1.0 : std_sum(m, s, a.c);
        if (arg_out) arg_out[r] = arg;
    }
}

__global__ __launch_bounds__(kBlock) void combine_topf_kernel(const Pass1Args a, int Bf, const float* q_max,
                                                              const double* q_sum, int32_t* cache_ids,
                                                              double* cache_mass) {
    __shared__ TopfScratch sc[kWavesPerBlock];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int64_t r = (int64_t)blockIdx.x * kWavesPerBlock + wave;
    if (r >= (int64_t)a.B * a.K1) return;
    const int b = (int)(r / a.K1), i = (int)(r % a.K1);
    const double M = cache_row_wave(a.part + r * a.nt, a.cand + r * a.nt * a.cap, a.nt, a.cap, a.F[i], q_max[r],
                                    q_sum[r], a.c, a.greedy, cache_ids + (int64_t)b * Bf + a.O[i], nullptr, sc[wave]);
    if (lane == 0) cache_mass[r] = M;
}

struct FO {
    int F[kMaxK + 1];
    int O[kMaxK + 2];
};

template <int DT>
__global__ void probs_kernel(const char* logits, int B, int K1, int V, int64_t ld_bytes, const float* m,
                             const double* s, const int32_t* arg, float c, int greedy, const int32_t* cache_ids, FO fo,
                             int Bf, const double* Z, float C, float* out) {
    const int64_t r = blockIdx.y;
    const int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (x >= V) return;
    const int b = (int)(r / K1), i = (int)(r % K1);
    double p;
    if (greedy) {
        p = (x == arg[r]) ? 1.0 : 0.0;
    } else {
        const RowNorm n = row_norm(m[r], s[r], c);
        p = (double)term(load_one<DT>(logits + r * ld_bytes, x), c, n.o) * n.inv;
    }
    if (Z) {
        bool in_cache = false;
        const int32_t* ids = cache_ids + (int64_t)b * Bf + fo.O[i];
        for (int j = 0; j < fo.F[i]; ++j) in_cache |= ids[j] == (int32_t)x;
        p = p * (in_cache ? (double)C : 1.0) / Z[r];
    }
    out[r * V + x] = (float)p;
}

__global__ void saguaro_z_kernel(const double* mass, int R, float C, double* Z) {
    const int r = blockIdx.x * blockDim.x + threadIdx.x;
    if (r < R) Z[r] = 1.0 - (1.0 - (double)C) * mass[r];
}

template <int DT>
__global__ void verify_kernel(const char* p_logits, const char* q_logits, int B, int K, int V, int64_t ld_bytes,
                              const int32_t* draft, const float* p_max, const double* p_sum, const int32_t* p_arg,
                              const float* q_max, const double* q_sum, FO fo, int Bf, const int32_t* cache_ids,
                              const double* Z, float C, float c, int greedy, uint64_t seed, uint64_t round,
                              int32_t* accept_len, float* accept_prob, int32_t* dev_err) {
    const int b = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (b >= B) return;
    const int lane = lane_id();
    const int K1 = K + 1;
    const int ic = lane < K ? lane : 0;
    const int64_t r = (int64_t)b * K1 + ic;
    const DraftProbe pr = probe_draft<DT>(draft, p_logits, q_logits, ld_bytes, b, K, V, greedy, seed, round);
    bool in_cache = false;
    const int32_t* ids = cache_ids + (int64_t)b * Bf + fo.O[ic];
    for (int j = 0; j < fo.F[ic]; ++j) in_cache |= ids[j] == pr.d;
    const float mp = greedy ? 0.f : p_max[r], mq = greedy ? 0.f : q_max[r];
    const double sp = greedy ? 1.0 : p_sum[r], sq = greedy ? 1.0 : q_sum[r];
    const int argp = greedy ? p_arg[r] : 0;
    const double Zi = greedy ? 1.0 : Z[r];
    int errs;
    const int k = verify_wave(b, K, V, pr, mp, sp, argp, mq, sq, Zi, in_cache, C, c, greedy, accept_prob, &errs);
    if (lane == 0) {
        accept_len[b] = k;
        if (dev_err && errs) dev_err[b] |= errs;
    }
}

__global__ void greedy_pick_kernel(const int32_t* arg, int B, int K, const int32_t* accept_len, int32_t* out,
                                   double* mass, int32_t* dev_err) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    const int K1 = K + 1;
    if (!accept_len) {
        if (t >= B * K) return;
        const int b = t / K, i = t % K;
        out[t] = arg[(int64_t)b * K1 + i];
    } else {
        if (t >= B) return;
        const int k = accept_len[t];
        const bool ok = k >= 0 && k <= K;
        out[t] = ok ? arg[(int64_t)t * K1 + k] : -1;
        if (mass) mass[t] = ok ? 1.0 : 0.0;
        if (!ok && dev_err) dev_err[t] |= kErrLenRange;
    }
}

__global__ void lookup_kernel(int B, int K, int V, FO fo, int Bf, const int32_t* cache_ids, const int32_t* accept_len,
                              const int32_t* bonus, int fallback, uint64_t seed, uint64_t round, uint8_t* hit,
                              int32_t* slot, int32_t* fb, int32_t* dev_err) {
    const int b = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (b >= B) return;
    const int k = accept_len[b];
    const bool ok = k >= 0 && k <= K;
    if (!ok && lane_id() == 0 && dev_err) dev_err[b] |= kErrLenRange;
    const int my_id = cached_id(cache_ids, b, Bf, ok ? k : -1, K, fo.F, fo.O);
    lookup_wave(b, K, V, ok ? k : -1, ok ? fo.O[k] : 0, my_id, bonus[b], fallback, seed, round, hit, slot, fb);
}

// ============================================================================ launchers
static FO make_fo(const int* F, const int* O, int K1) {
    FO fo;
    for (int i = 0; i <= kMaxK; ++i) fo.F[i] = i < K1 ? F[i] : 0;
    for (int i = 0; i <= kMaxK + 1; ++i) fo.O[i] = i <= K1 ? O[i] : 0;
    return fo;
}

template <typename Fn>
static hipError_t by_type(int dtype, bool vec, Fn&& fn) {
    if (dtype == 1) {
        if (vec)
            fn(std::integral_constant<int, 1>{}, std::true_type{});
        else
            fn(std::integral_constant<int, 1>{}, std::false_type{});
    } else {
        if (vec)
            fn(std::integral_constant<int, 0>{}, std::true_type{});
        else
            fn(std::integral_constant<int, 0>{}, std::false_type{});
    }
    return hipGetLastError();
}

hipError_t launch_pass1(int dtype, bool vec, const Pass1Args& a, hipStream_t st) {
    const int nblk = (a.nt + kWavesPerBlock - 1) / kWavesPerBlock;
    const int64_t grid = (int64_t)a.B * a.nmodel * a.K1 * nblk;
    if (grid <= 0 || grid > INT_MAX) return hipErrorInvalidValue;
    return by_type(dtype, vec, [&](auto DT, auto VEC) {
        pass1_kernel<decltype(DT)::value, decltype(VEC)::value><<<(unsigned)grid, kBlock, 0, st>>>(a);
    });
}

hipError_t launch_finalize_seq(int dtype, const SeqFinal& f, hipStream_t st) {
    if (dtype == 1)
        finalize_seq_kernel<1><<<f.B, kFinBlock, 0, st>>>(f);
    else
        finalize_seq_kernel<0><<<f.B, kFinBlock, 0, st>>>(f);
    return hipGetLastError();
}

hipError_t launch_pass2(int dtype, bool vec, const Pass2Args& a, int ngroups, hipStream_t st) {
    const int nblk = (a.nt + kWavesPerBlock - 1) / kWavesPerBlock;
    const int64_t grid = (int64_t)ngroups * nblk;
    if (grid <= 0 || grid > INT_MAX) return hipErrorInvalidValue;
    return by_type(dtype, vec, [&](auto DT, auto VEC) {
        pass2_kernel<decltype(DT)::value, decltype(VEC)::value><<<(unsigned)grid, kBlock, 0, st>>>(a);
    });
}

hipError_t launch_finalize_bonus(int dtype, bool vec, const Pass2Args& a, int ngroups, hipStream_t st) {
    const int grid = (ngroups + kWavesPerBlock - 1) / kWavesPerBlock;
    return by_type(dtype, vec, [&](auto DT, auto VEC) {
        finalize_bonus_kernel<decltype(DT)::value, decltype(VEC)::value><<<grid, kBlock, 0, st>>>(a, ngroups);
    });
}

hipError_t launch_combine_stats(const Pass1Args& a, float* m, double* s, int32_t* arg, hipStream_t st) {
    const int R = a.B * a.K1;
    combine_stats_kernel<<<(R + kWavesPerBlock - 1) / kWavesPerBlock, kBlock, 0, st>>>(a, m, s, arg);
    return hipGetLastError();
}

hipError_t launch_combine_topf(const Pass1Args& a, int Bf, const float* q_max, const double* q_sum,
                               int32_t* cache_ids, double* cache_mass, hipStream_t st) {
    const int R = a.B * a.K1;
    combine_topf_kernel<<<(R + kWavesPerBlock - 1) / kWavesPerBlock, kBlock, 0, st>>>(a, Bf, q_max, q_sum, cache_ids,
                                                                                      cache_mass);
    return hipGetLastError();
}

hipError_t launch_probs(int dtype, const char* logits, int B, int K1, int V, int64_t ld_bytes, const float* m,
                        const double* s, const int32_t* arg, float c, int greedy, const int32_t* cache_ids,
                        const int* F, const int* O, int Bf, const double* Z, float C, float* out, hipStream_t st) {
    dim3 grid((V + 255) / 256, B * K1);
    FO fo = F ? make_fo(F, O, K1) : FO{};
    if (dtype == 1)
        probs_kernel<1><<<grid, 256, 0, st>>>(logits, B, K1, V, ld_bytes, m, s, arg, c, greedy, cache_ids, fo, Bf, Z,
                                              C, out);
    else
        probs_kernel<0><<<grid, 256, 0, st>>>(logits, B, K1, V, ld_bytes, m, s, arg, c, greedy, cache_ids, fo, Bf, Z,
                                              C, out);
    return hipGetLastError();
}

hipError_t launch_saguaro_z(const double* cache_mass, int R, float C, double* Z, hipStream_t st) {
    saguaro_z_kernel<<<(R + 255) / 256, 256, 0, st>>>(cache_mass, R, C, Z);
    return hipGetLastError();
}

hipError_t launch_verify(int dtype, const char* p_logits, const char* q_logits, int B, int K, int V,
                         int64_t ld_bytes, const int32_t* draft, const float* p_max, const double* p_sum,
                         const int32_t* p_arg, const float* q_max, const double* q_sum, const int* F, const int* O,
                         int Bf, const int32_t* cache_ids, const double* Z, float C, float c, int greedy,
                         uint64_t seed, uint64_t round, int32_t* accept_len, float* accept_prob, int32_t* dev_err,
                         hipStream_t st) {
    const int per_block = kWavesPerBlock;
    const FO fo = make_fo(F, O, K + 1);
    if (dtype == 1)
        verify_kernel<1><<<(B + per_block - 1) / per_block, kBlock, 0, st>>>(
            p_logits, q_logits, B, K, V, ld_bytes, draft, p_max, p_sum, p_arg, q_max, q_sum, fo, Bf, cache_ids, Z, C,
            c, greedy, seed, round, accept_len, accept_prob, dev_err);
    else
        verify_kernel<0><<<(B + per_block - 1) / per_block, kBlock, 0, st>>>(
            p_logits, q_logits, B, K, V, ld_bytes, draft, p_max, p_sum, p_arg, q_max, q_sum, fo, Bf, cache_ids, Z, C,
            c, greedy, seed, round, accept_len, accept_prob, dev_err);
    return hipGetLastError();
}

hipError_t launch_greedy_pick(const int32_t* arg, int B, int K, const int32_t* accept_len, int32_t* out, double* mass,
                              int32_t* dev_err, hipStream_t st) {
    const int n = accept_len ? B : B * K;
    greedy_pick_kernel<<<(n + 255) / 256, 256, 0, st>>>(arg, B, K, accept_len, out, mass, dev_err);
    return hipGetLastError();
}

hipError_t launch_lookup(int B, int K, int V, const int* F, const int* O, int Bf, const int32_t* cache_ids,
                         const int32_t* accept_len, const int32_t* bonus, int fallback, uint64_t seed,
                         uint64_t round, uint8_t* hit, int32_t* slot, int32_t* fallback_tokens, int32_t* dev_err,
                         hipStream_t st) {
    const FO fo = make_fo(F, O, K + 1);
    lookup_kernel<<<(B + kWavesPerBlock - 1) / kWavesPerBlock, kBlock, 0, st>>>(
        B, K, V, fo, Bf, cache_ids, accept_len, bonus, fallback, seed, round, hit, slot, fallback_tokens, dev_err);
    return hipGetLastError();
}

}  // namespace ssd

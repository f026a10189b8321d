// ssd_kernels.hip -- gfx950 kernels of the verify-and-pre-speculate round of
// Speculative Speculative Decoding with the Saguaro algorithm.
//
// One round is four kernels (three at T = 0); the two streaming ones carry all
// the bytes:
//  pass 1      every row of the target and draft logits [B, K+1, V] is read once.  The
//              unit of work is one wave64 and one tile of 8 x 16-byte vectors per lane
//              (4096 bf16 / 2048 fp32 elements); waves never wait for each other.  Per
//              tile: the softmax partial (max, sum of 2^{z c - o}), the lowest-id argmax
//              and, for draft rows of the cache, every element at or above the F-th
//              largest lane maximum of its block of four tiles (a lower bound of the
//              row's F-th largest value) as a candidate key.
//  finalise    one wave per (sequence, position i): softmax statistics of both rows,
//              cache ids S_i (top F_i draft ids, ties to the lower id), M_i, the Saguaro
//              normaliser Z_i and the lossless test of draft token d_i, whose outcome
//              goes to a per-position flag.
//  pass 2      only the rows the bonus needs (target row k, plus draft row k when
//              k < K, k = the first rejected position) are read again; each wave sums
//              the residual max(p - q', 0) of its tile.
//  bonus       one block per sequence draws the bonus in two levels: the 512-id block
//              where the running sum of block weights crosses u1 * sum (tile sums
//              locate its tile, a rescan of that tile the block), then the id of
//              that block where the block's own running sum crosses u2 times its
//              weight; then the cache lookup.
//              At T = 0 pass 2 does not run and a per-sequence kernel takes the argmax.
// Normalisers, cached masses, Z and every running sum that decides an integer are
// kept in fp64; per-element terms are fp32 exp2 of an exactly formed exponent.  The
// separate C-ABI calls reuse the same device code, so their results are
// bit-identical to the fused round.
#include "ssd_device.h"
#include "ssd_kernels.h"

#include <algorithm>
#include <climits>
#include <type_traits>

namespace ssd {

enum { kPurposeAccept = 0, kPurposeBonus = 1, kPurposeDraft = 2, kPurposeFallback = 3 };
enum { kErrTokenRange = 1, kErrQprimeZero = 2, kErrLenRange = 4, kErrSlotRange = 8 };
constexpr int kXcds = 8;            // accelerator complex dies of MI355X
constexpr int kFinalizeTwoWaveMaxPairs = 1024;  // (b, i) pairs up to the chip's SIMD count
// Pass-2 grids of more than 8 tiles per SIMD take the lean weighing, for the bonus two
// tiles per wave where rows are 16-byte aligned; smaller ones (all waves resident at
// once) are bound by load latency, where the lean form's per-vector register pins cost
// more than its fewer instructions save and fewer waves would load less at once.
constexpr int64_t kPass2LeanMinTiles = 8192;

// Blocks are dealt to the XCDs round-robin (block x runs on XCD x mod 8), and each XCD
// has its own L2.  Every kernel of a round puts the work of sequence b on XCD b mod 8,
// so that what one kernel writes for a sequence (test outcomes, law parameters, cache
// ids, tile sums) is still in that XCD's L2 when the next kernel reads it.  Slot s of a
// per-(sequence, position) launch holds pair (b, i) with b mod 8 = s mod 8; the slots
// of an XCD take its sequences in order, positions innermost.
__host__ __device__ constexpr int xcd_slots(int B, int K1) { return (B + kXcds - 1) / kXcds * kXcds * K1; }
__device__ __forceinline__ void xcd_pair(int s, int K1, int& b, int& i) {
    const int y = s / kXcds;
    i = y % K1;
    b = (y / K1) * kXcds + s % kXcds;
}
constexpr int kSurvivorCap = 256;  // LDS slots per wave for the row's filtered candidates
constexpr int kStageCap = 160;     // LDS slots per wave for one tile's candidate keys (>= any cap)
constexpr int kHotCap = 128;       // LDS slots per wave for the vectors that hold candidates

int tile_elems(int dtype) { return dtype == 1 ? kTile<1> : kTile<0>; }
int tiles_per_row(int dtype, int V) {
    const int t = tile_elems(dtype);
    return (V + t - 1) / t;
}
int tiles_per_row2(int dtype, int V) {
    const int t = dtype == 1 ? kTile2<1> : kTile2<0>;
    return (V + t - 1) / t;
}
int cand_cap(int Fmax) { return ((2 * Fmax + 16) + 7) / 8 * 8; }  // <= 144 = cand_cap(64) <= kStageCap
// Candidate slots per tile that the finalisation reads before it knows the tile's count
// (pass 1 writes 0 past the keys up to there): with the block threshold a tile holds
// at most about F + 6 keys.  A row with more in some tile takes the general path.
__host__ __device__ __forceinline__ int spec_slots(int F, int cap) { return min(min(2 * F + 2, F + 8), cap); }
// Candidate keys are stored per unit: the four tiles of one pass-1 block (one row, one
// threshold), contiguously, in a region of kWavesPerBlock * cap slots.
__host__ __device__ __forceinline__ int units_per_row(int nt) { return (nt + kWavesPerBlock - 1) / kWavesPerBlock; }

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

// (max, sum relative to o(max), lowest-id argmax) of the whole wave from one partial
// per lane, each lane's sum relative to the offset of its own maximum; uniform result.
// Partial sums are moved to the common offset exactly (ldexp) and added in fp64.
__device__ __forceinline__ void wave_stats(float m_l, double s_l, int arg_l, float c, float& m, double& s, int& arg) {
    m = wave_max_f32(m_l);
    const float o = offset_of(m, c);
    const double sl = m_l == -INFINITY ? 0.0 : ldexp(s_l, (int)(offset_of(m_l, c) - o));
    s = wave_sum_f64(sl);
    arg = wave_min_i32(m_l == m ? arg_l : INT_MAX);
}

// (max, lowest-id argmax, sum relative to o(max)) merge; symmetric bit for bit.
__device__ __forceinline__ void merge_stats(float& m, double& s, int& arg, float m2, double s2, int a2, float c) {
    if (m2 > m || (m2 == m && a2 < arg)) arg = a2;
    merge_partial(m, s, m2, s2, c);
}

// What the candidate merge of a draft row needs from the row's tile partials: the
// largest tile threshold, the largest per-tile candidate count and (in LDS) every
// tile's count.
constexpr int kMaxMergeTiles = 512;
struct CandSummary {
    uint32_t tr;
    int max_nc;
};

// Softmax statistics of one row from its nt tile partials, by one wave in a fixed
// order (lane-sequential, then a butterfly); every lane returns the same values.
// With with_cands, the same single read of the partials also fills the candidate
// summary cs (per-unit counts to nc, which holds kMaxMergeTiles entries).
__device__ __forceinline__ void row_stats_wave(const WavePartial* P, int nt, float c, float& m, double& s, int& arg,
                                               bool with_cands, CandSummary& cs, uint16_t* nc) {
    const int lane = lane_id();
    m = -INFINITY;
    s = 0.0;
    arg = INT_MAX;
    uint32_t tr = 0u;
    int max_nc = 0;
    for (int t = lane; t < nt; t += kWave) {
        const WavePartial q = P[t];
        merge_stats(m, s, arg, q.m, q.s, q.arg, c);
        if (with_cands) {
            tr = max(tr, q.tau);
            max_nc = max(max_nc, q.ncand);
            if ((t & 3) == 0 && (t >> 2) < kMaxMergeTiles) nc[t >> 2] = (uint16_t)q.ncand;
        }
    }
    wave_stats(m, s, arg, c, m, s, arg);
    cs.tr = 0u;
    cs.max_nc = 0;
    if (with_cands) {
        cs.tr = wave_max_u32(tr);
        cs.max_nc = (int)wave_max_u32((uint32_t)max_nc);
        wave_sync_lds();
    }
}

// Merge of the candidates of one draft row by one wave.  Candidate (tile t, slot s)
// is gathered by lane (s*nt + t) mod 64 into register u = (s*nt + t) / 64, so every
// load address is known up front and all loads of a row are in flight together.
constexpr int kCandRegs = 24;    // register slots per lane: up to 1536 candidates per row

struct TopfScratch {
    uint64_t surv[kSurvivorCap + kWave];  // keys at or above the value threshold (+ one
                                          // discard slot per lane)
    uint64_t rank[kWave];                 // the top F, placed by rank
    uint32_t bins[256 + kWave];           // value histogram of the select (+ one discard
                                          // bin per lane)
    uint16_t nc[kMaxMergeTiles];          // candidates per unit (four tiles)
};

// The largest 32-bit value part T such that at least F of the nonzero keys among the
// first U slots have a value part >= T (the F-th largest value, ties counted); 0 when
// there are at most F keys.  Bits below the common prefix of the keys are resolved 8
// at a time, most significant first: each step counts the keys that match the value
// prefix found so far in a 256-bin LDS histogram of their next 8 bits and keeps the
// bin that holds the rank still sought.
template <int KREG>
__device__ inline uint32_t wave_select_value(const uint64_t (&k)[KREG], int U, int F, uint32_t* bins,
                                             bool first_step_only = false) {
    U = uniform(U);
    const int lane = lane_id();
    int n = 0;
    uint32_t orv = 0u, andv = ~0u;
#pragma unroll
    for (int u = 0; u < KREG; ++u) {
        if (u < U) {
            n += wave_popc(k[u] != 0ull);
            if (k[u] != 0ull) {
                orv |= (uint32_t)(k[u] >> 32);
                andv &= (uint32_t)(k[u] >> 32);
            }
        }
    }
    if (n <= F) return 0u;
    orv = wave_or_u32(orv);
    andv = wave_and_u32(andv);
    const uint32_t diff = orv ^ andv;
    if (diff == 0u) return andv;
    int hi = 32 - __clz(diff);                               // bits [hi, 32) are common
    const int lo = __ffs(diff) - 1;                          // so are bits [0, lo)
    uint32_t prefix = (hi >= 32 ? 0u : (andv >> hi) << hi) | (andv & ((1u << lo) - 1u));
    int need = F;
    while (hi > lo) {
        const int shift = hi - lo > 8 ? hi - 8 : lo;
        const uint32_t wmask = (1u << (hi - shift)) - 1u;
#pragma unroll
        for (int j = 0; j < 256 / kWave; ++j) bins[j * kWave + lane] = 0u;
        wave_sync_lds();
        // every lane adds in every slot (no per-lane branch): non-matching keys add to
        // the lane's own discard bin
#pragma unroll
        for (int u = 0; u < KREG; ++u) {
            if (u < U) {
                const uint32_t h = (uint32_t)(k[u] >> 32);
                const bool match = (k[u] != 0ull) & ((hi >= 32) | ((h >> (hi & 31)) == (prefix >> (hi & 31))));
                atomicAdd(&bins[match ? (h >> shift) & wmask : 256 + lane], 1u);
            }
        }
        wave_sync_lds();
        // lane l holds bins 4l .. 4l+3; counts of the bins above each one
        uint32_t c[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) c[j] = bins[4 * lane + j];
        const uint32_t lane_sum = c[0] + c[1] + c[2] + c[3];
        const uint32_t incl = wave_prefix_u32(lane_sum);
        int above = (int)(lane_u32(incl, kWave - 1) - incl);  // keys in the bins of higher lanes
        int hit_bin = -1, hit_above = 0;
#pragma unroll
        for (int j = 3; j >= 0; --j) {
            if (hit_bin < 0 && above < need && need <= above + (int)c[j]) {
                hit_bin = 4 * lane + j;
                hit_above = above;
            }
            above += (int)c[j];
        }
        const uint64_t hm = __ballot(hit_bin >= 0);
        const int src = uniform(__ffsll((long long)hm) - 1);
        const int bsel = (int)lane_u32((uint32_t)hit_bin, src);
        need -= (int)lane_u32((uint32_t)hit_above, src);
        prefix |= (uint32_t)bsel << shift;
        hi = shift;
        wave_sync_lds();
        if (first_step_only) {
            // lower bound of the bin holding the F-th largest value
            return (hi >= 32 ? 0u : (prefix >> hi) << hi) | (andv & ((1u << lo) - 1u) & ((1u << hi) - 1u));
        }
    }
    return prefix;
}

// Sorts the n <= kSurvivorCap distinct keys in sc.surv by rank and returns lane j =
// the j-th largest (0 past min(n, F)).
__device__ inline uint64_t rank_sort_lds(TopfScratch& sc, int n, int F) {
    const int lane = lane_id();
    n = uniform(n);
    uint64_t k[4];
    int rank[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        k[u] = 0ull;
        rank[u] = 0;
    }
    if (n <= kWave) {
        // one key per lane, compared with every key (LDS broadcast reads)
        k[0] = lane < n ? sc.surv[lane] : 0ull;
        for (int v = 0; v < n; ++v) rank[0] += sc.surv[v] > k[0];
    } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int j = u * kWave + lane;
            k[u] = j < n ? sc.surv[j] : 0ull;
        }
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

// Appends the nonzero keys >= lo among the first U slots of k[] (in slot, then lane
// order) to sc.surv; returns their count (keys past kSurvivorCap are counted, not
// stored).
template <int KREG>
__device__ inline int compact_keys(TopfScratch& sc, const uint64_t (&k)[KREG], int U, uint64_t lo) {
    U = uniform(U);
    int n = 0;
#pragma unroll
    for (int u = 0; u < KREG; ++u) {
        if (u < U) {
            const bool keep = (k[u] != 0ull) & (k[u] >= lo);
            const int pos = n + lanes_below(keep);
            sc.surv[keep && pos < kSurvivorCap ? pos : kSurvivorCap + lane_id()] = k[u];
            n += wave_popc(keep);
        }
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

// Loads slots s < R of every tile's candidate list (R <= cap, nt*R <= 64*KREG) in
// tile-major order: flat index f = t*R + s goes to lane f mod 64, register f / 64, so
// the lanes of one load cover consecutive slots of one or two tiles (few cache
// lines).  No load depends on the per-tile counts, so they can be requested with the
// tile partials.
template <int KREG>
__device__ __forceinline__ void gather_slots(const uint64_t* cand, int cap, int nt, int R, uint64_t (&k)[KREG]) {
    const int lane = lane_id();
    const int total = nt * R;
    int t = lane / R, sl = lane % R;
    // opaque to the optimiser: keeps the slot addresses from being hoisted out of a
    // caller's loop over rows (they would stay live in registers across it)
    __asm__ volatile("" : "+v"(t), "+v"(sl));
    const int dt = kWave / R, ds = kWave % R;
    // Every slot of a used register is loaded (no per-lane branch); slots past nt*R
    // read slot 0 of tile 0 and are dropped.
#pragma unroll
    for (int u = 0; u < KREG; ++u) {
        uint64_t x = 0ull;
        const bool in = u * kWave + lane < total;
        if (u * kWave < total) x = cand[in ? (int64_t)t * cap + sl : 0];  // uniform test
        k[u] = in ? x : 0ull;
        t += dt;
        sl += ds;
        if (sl >= R) {
            sl -= R;
            ++t;
        }
    }
}

// Keeps the gathered slots that hold a candidate (s < the tile's count, from nc) at
// or above floor_key; clears the rest.
template <int KREG>
__device__ __forceinline__ void mask_slots(uint64_t (&k)[KREG], int nt, int R, const uint16_t* nc,
                                           uint64_t floor_key) {
    const int lane = lane_id();
    int t = lane / R, sl = lane % R;
    const int dt = kWave / R, ds = kWave % R;
    int cnt[KREG], sls[KREG];
#pragma unroll
    for (int u = 0; u < KREG; ++u) {  // all count reads first, then the tests
        cnt[u] = nc[min(t, nt - 1)];
        sls[u] = sl;
        t += dt;
        sl += ds;
        if (sl >= R) {
            sl -= R;
            ++t;
        }
    }
#pragma unroll
    for (int u = 0; u < KREG; ++u) {
        const bool live = (sls[u] < cnt[u]) & (k[u] >= floor_key);
        k[u] = live ? k[u] : 0ull;
    }
}

// Top F (sorted, lane j = j-th largest, 0 past F) of the nonzero keys in the first U
// register slots: the F-th largest value by radix select, the keys at or above it by
// rank (a whole-key select first when more than kSurvivorCap keys tie there).
template <int KREG>
__device__ __forceinline__ uint64_t select_sorted(uint64_t (&k)[KREG], int U, int F, TopfScratch& sc,
                                                  uint64_t floor_key = 1ull) {
    // Keys below floor_key are dropped.  At most one key per lane: each lane places its
    // keys after those of the lanes below it (one prefix sum), and they are ranked.
    // Otherwise one histogram step usually leaves few enough keys (those in or above
    // the bin of the F-th largest value) to rank them all; failing that, resolve the
    // value exactly.
    // Every slot at or past U holds 0, so the counting and placing loops run over all
    // KREG slots with no test of U.
    U = uniform(U);
    uint32_t mine = 0u;
#pragma unroll
    for (int u = 0; u < KREG; ++u) mine += k[u] >= floor_key ? 1u : 0u;
    const uint32_t incl = wave_prefix_u32(mine);
    const int live = (int)lane_u32(incl, kWave - 1);
    if (live <= kWave) {
        // the comparisons are redone rather than kept (KREG masks would not fit in
        // scalar registers)
#pragma unroll
        for (int u = 0; u < KREG; ++u) __asm__ volatile("" : "+v"(k[u]));
        int pos = (int)(incl - mine);
#pragma unroll
        for (int u = 0; u < KREG; ++u) {
            const bool keep = k[u] >= floor_key;
            sc.surv[keep ? pos : kSurvivorCap + lane_id()] = k[u];
            pos += keep ? 1 : 0;
        }
        wave_sync_lds();
        return rank_sort_lds(sc, live, F);
    }
#pragma unroll
    for (int u = 0; u < KREG; ++u) k[u] = k[u] >= floor_key ? k[u] : 0ull;
    uint64_t lo = (uint64_t)wave_select_value<KREG>(k, U, F, sc.bins, true) << 32;
    int n = compact_keys<KREG>(sc, k, U, lo);
    if (n > kSurvivorCap) {
        lo = (uint64_t)wave_select_value<KREG>(k, U, F, sc.bins) << 32;
        n = compact_keys<KREG>(sc, k, U, lo);
    }
    if (n > kSurvivorCap) {
#pragma unroll
        for (int u = 0; u < KREG; ++u) k[u] = k[u] >= lo ? k[u] : 0ull;
        const uint64_t T64 = wave_select_regs<KREG>(k, F);
        n = compact_keys<KREG>(sc, k, U, T64);
    }
    return rank_sort_lds(sc, n, F);
}

// Top F of one draft row from its units' candidate keys (unit u: tiles 4u..4u+3, its
// count in the partial of tile 4u, stored at unit u of cand with stride capU), by one
// wave.  The largest threshold bounds the row's F-th largest value from below (that
// unit alone has F elements at or above it), so only keys at or above it can be in the
// row's top F, and every such key is in its unit's list.  Keys are distinct (they carry
// the id).  Returns lane j = the j-th largest key (0 past F).  cs and sc.nc (per unit)
// come from row_stats_wave.
__device__ __forceinline__ uint64_t row_topf_wave(const WavePartial* P, const uint64_t* cand, int nt, int capU,
                                                  int F, const CandSummary& cs, TopfScratch& sc) {
    const int lane = lane_id();
    const uint64_t floor_key = (uint64_t)cs.tr << 32;
    const int R = cs.max_nc;
    const int nu = units_per_row(nt);
    if (nu <= kMaxMergeTiles && (int64_t)nu * R <= (int64_t)kWave * kCandRegs) {
        uint64_t k[kCandRegs];
        gather_slots<kCandRegs>(cand, capU, nu, R, k);
        mask_slots<kCandRegs>(k, nu, R, sc.nc, floor_key);
        return select_sorted<kCandRegs>(k, (nu * R + kWave - 1) / kWave, F, sc);
    }

    // Rows with more candidates than register slots: exact selection by F rounds of a
    // wave maximum below the previous key.
    int* start = reinterpret_cast<int*>(sc.surv);
    uint64_t key = 0ull, prev = ~0ull;
    for (int r = 0; r < F; ++r) {
        uint64_t best = 0ull;
        for (int c0 = 0; c0 < nu; c0 += kWave) {
            const int nc = c0 + lane < nu ? P[(int64_t)(c0 + lane) * kWavesPerBlock].ncand : 0;
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
                const uint64_t x = chunk_key(cand, capU, c0, start, j);
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

// Cache ids and cached mass M = sum of q(x) over them, of one draft row, from its
// sorted top-F keys (lane j = j-th largest).
__device__ __forceinline__ double finish_cache_row(uint64_t key, int F, float mq, double sq, float c, int greedy,
                                                   int32_t* ids_out, int* ids_lds) {
    const int lane = lane_id();
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
    return wave_sum_f64(t);
}

// Value store of the speculation cache: one continuation of K tokens per cache slot
// (values [B, Bf, K]); when values is set the lookup also writes the next draft.
struct ValueStore {
    const int32_t* values = nullptr;
    int Bf = 0;
    int32_t* next_draft = nullptr;
};

// Cache lookup of one verified outcome (k, tok) by one wave, plus the uniform
// fallback draft on a miss.  my_id: lane j < F_k holds the j-th cached id of outcome
// k (slot O_k + j); other lanes, and every lane when k is invalid (k < 0), hold -1.
__device__ inline void lookup_wave(int b, int K, int V, int k, int Ok, int my_id, int tok, int fallback,
                                   uint64_t seed, uint64_t round, uint8_t* hit, int32_t* slot, int32_t* fb,
                                   const ValueStore& vs = ValueStore{}) {
    const int lane = lane_id();
    const uint64_t mk = __ballot(k >= 0 && my_id >= 0 && my_id == tok);
    const bool h = mk != 0ull;
    const int sl = h ? Ok + (__ffsll((long long)mk) - 1) : -1;
    if (lane == 0) {
        hit[b] = h ? 1 : 0;
        slot[b] = sl;
    }
    for (int j = lane; j < K; j += kWave) {
        int32_t t = -1;
        if (!h && fallback) {
            const uint64_t u32 = philox_u32(seed, round, kPurposeFallback, (uint64_t)b, (uint64_t)j);
            t = (int32_t)((u32 * (uint64_t)V) >> 32);
        }
        fb[(int64_t)b * K + j] = t;
        // next round's draft: the cached continuation on a hit, the fallback otherwise
        if (vs.next_draft) vs.next_draft[(int64_t)b * K + j] = h ? vs.values[((int64_t)b * vs.Bf + sl) * K + j] : t;
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

// What testing draft token d_i of sequence b needs, loaded ahead of the row statistics:
// the token, both models' logits at it (when d_i is in range and T > 0) and the
// acceptance uniform.
template <int DT>
__device__ __forceinline__ DraftProbe probe_draft(const int32_t* draft, const char* p_logits, const char* q_logits,
                                                  int64_t ld_bytes, int b, int i, int K, int V, int greedy,
                                                  uint64_t seed, uint64_t round) {
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

// Lossless test of one draft token d ~ q' against the target p: accepted when
// u < p(d) / q'(d) with q'(d) = q(d) (C if d is cached) / Z; at T = 0 accepted when d
// is the target argmax.  Two steps, so that the exponentials (which need only the row
// statistics) can run before the cache selection that gives Z and the membership.
struct DraftTerms {
    double p, q;  // p(d), q(d) in fp64 (T > 0)
    int err;
    bool ok;
};
__device__ __forceinline__ DraftTerms draft_terms(const DraftProbe& pr, int V, float mp, double sp, float mq,
                                                  double sq, float c, int greedy) {
    DraftTerms t{0.0, 0.0, 0, true};
    if (pr.d < 0 || pr.d >= V) {
        t.err |= kErrTokenRange;
        t.ok = false;
    } else if (!greedy) {
        // one element per test: both probabilities in fp64 from the exact exponents
        // (z c - o), so that a tiny p or q' does not underflow as an fp32 term would
        const RowNorm np = row_norm(mp, sp, c), nq = row_norm(mq, sq, c);
        t.p = exp2((double)pr.zp * (double)c - (double)np.o) * np.inv;
        t.q = exp2((double)pr.zq * (double)c - (double)nq.o) * nq.inv;
    }
    return t;
}
// *ratio gets p/q' (0 when not testable), *err the error bits.
__device__ __forceinline__ bool draft_decide(const DraftProbe& pr, const DraftTerms& t, int argp, double Zi,
                                             bool in_cache, float C, int greedy, double* ratio_out, int* err_out) {
    int err = t.err;
    bool ok = t.ok;
    double ratio = 0.0;
    if (ok) {
        if (greedy) {
            ratio = (pr.d == argp) ? 1.0 : 0.0;
        } else {
            const double qp = t.q * (in_cache ? (double)C : 1.0) / Zi;
            if (!(qp > 0.0)) {
                err |= kErrQprimeZero;
                ok = false;
            } else {
                ratio = t.p / qp;
            }
        }
    }
    *ratio_out = ratio;
    *err_out = err;
    return ok && (greedy ? ratio == 1.0 : (double)pr.u < ratio);
}
__device__ __forceinline__ bool test_draft(const DraftProbe& pr, int V, float mp, double sp, int argp, float mq,
                                           double sq, double Zi, bool in_cache, float C, float c, int greedy,
                                           double* ratio_out, int* err_out) {
    return draft_decide(pr, draft_terms(pr, V, mp, sp, mq, sq, c, greedy), argp, Zi, in_cache, C, greedy, ratio_out,
                        err_out);
}

// ============================================================================ pass 1
template <int DT, bool VEC, bool GREEDY>
__global__ __launch_bounds__(kBlock) void pass1_kernel(const Pass1Args a) {
    __shared__ uint64_t cand_stage[kWavesPerBlock][kStageCap + kWave];
    __shared__ u32x4 hot_vec[kWavesPerBlock][kHotCap];
    __shared__ int hot_id[kWavesPerBlock][kHotCap];
    __shared__ uint32_t lane_key[kWavesPerBlock][kWave];
    __shared__ int unit_cnt[kWavesPerBlock];
    constexpr int N = ElemTraits<DT>::kPerVec;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int nblk = (a.nt + kWavesPerBlock - 1) / kWavesPerBlock;
    // Block -> (row pair, model, tile group): the blocks of pair (b, i) go to XCD b mod 8,
    // where the finalisation of that pair later runs; each XCD streams its rows in order.
    const int bid = blockIdx.x;
    const int per = a.nmodel * nblk;
    const int y = bid / kXcds;
    int b, i;
    xcd_pair((y / per) * kXcds + bid % kXcds, a.K1, b, i);
    if (b >= a.B) return;
    const int model = (y % per) / nblk, blk = (y % per) % nblk;
    const int t = blk * kWavesPerBlock + wave;
    const int F = a.F[i];
    // draft rows of the cache: the block's waves meet at a barrier, so a wave past the
    // row's last tile stays (with no data) until then
    const bool topf = model == a.topf_model && F > 0;  // uniform over the block
    const bool tile_ok = t < a.nt;
    if (!tile_ok && !topf) return;
    const int64_t r = (int64_t)b * a.K1 + i;
    const char* row = a.logits[model] + r * a.ld_bytes;
    const int64_t tile0 = (int64_t)t * kTile<DT>;
    const int V = a.V;
    const float c = a.c;

    // The tile stays in its raw 16-byte vectors (32 registers for bf16, not 64) and is
    // widened element by element in each use.
    // the draft token of this row is requested with the tile, not after it
    const bool has_draft = a.draft && i < a.K1 - 1;
    const int d_tok = has_draft ? a.draft[(int64_t)b * (a.K1 - 1) + i] : -1;
    u32x4 raw[kVecPerLane];
    if (tile_ok) {
        load_tile<DT, VEC, kVecPerLane>(row, tile0, V, lane, raw);
    } else {
#pragma unroll
        for (int j = 0; j < kVecPerLane; ++j) raw[j] = neg_inf_vec<DT>();
    }

    // One pass over the lane's vectors: the maximum of each vector and, unless greedy,
    // the sum of 2^{z c - o} with o the offset of the running maximum; when the maximum
    // grows the partial sum moves to the new offset exactly (ldexp by o_old - o_new).
    // Maxima use the NaN-propagating maximum (v_maximum3_f32), which needs no operand
    // canonicalisation; logits are never NaN, and a zero maximum may come out as +0 where
    // fmax could give -0 (equal in every later comparison).  While the running maximum is
    // -inf the offset is -3e38 instead of 0: every term so far is exactly 0, and the
    // first finite maximum rescales that zero sum (ldexp by a saturated exponent).
    float vmax[kVecPerLane];  // maximum of each of the lane's vectors
    float m = -INFINITY;
    float s32 = 0.f, o = 0.f;
#pragma unroll
    for (int j = 0; j < kVecPerLane; ++j) {
        float x[N];
#pragma unroll
        for (int e = 0; e < N; ++e) x[e] = vec_elem<DT>(raw[j], e);
        float vm = x[0];
#pragma unroll
        for (int e = 1; e < N; e += 2)
            vm = e + 1 < N ? fmax3_nan(vm, x[e], x[e + 1]) : __builtin_elementwise_maximum(vm, x[e]);
        vmax[j] = vm;
        m = __builtin_elementwise_maximum(m, vm);
        if (!GREEDY) {
            const float on = rintf(__builtin_elementwise_maximum(m * c, -3e38f));
            s32 = ldexpf(s32, (int)(o - on));
            o = on;
            float tt[N];
#pragma unroll
            for (int e = 0; e < N; ++e) tt[e] = term(x[e], c, o);
#pragma unroll
            for (int w = N / 2; w >= 1; w >>= 1)
#pragma unroll
                for (int e = 0; e < w; ++e) tt[e] += tt[e + w];
            s32 += tt[0];
            // each vector's sum completes here: left free, the compiler sinks every
            // vector's terms below the loop and keeps all widened elements live at once
            // (137 VGPRs instead of 67)
            __asm__ volatile("" : "+v"(s32), "+v"(o));
        }
    }
    const float m_lane = m;
    const double s_lane = (double)s32;  // relative to offset_of(m_lane)
    // each later phase widens the elements afresh rather than keeping them live
    opaque_regs(raw);

    // Lowest id of the lane holding m_lane: the lane's ids ascend with (vector, element),
    // so it lies in the first vector whose maximum equals m_lane; only that vector's
    // elements are compared.  (Padding past V holds -inf; it can equal m_lane only when
    // every element of the lane is -inf, and then the id test excludes it.)
    int arg = INT_MAX;
    if (a.want_arg) {
        int jm = kVecPerLane;
#pragma unroll
        for (int j = kVecPerLane - 1; j >= 0; --j) jm = vmax[j] == m_lane ? j : jm;
        u32x4 v = raw[0];
#pragma unroll
        for (int j = 1; j < kVecPerLane; ++j) v = jm == j ? raw[j] : v;
        const int64_t id0 = tile0 + (int64_t)(jm * kWave + lane) * N;
        int em = N;
#pragma unroll
        for (int e = N - 1; e >= 0; --e) em = (vec_elem<DT>(v, e) == m_lane && id0 + e < V) ? e : em;
        if (jm < kVecPerLane && em < N) arg = (int)(id0 + em);
    }
    double s = s_lane;
    opaque_regs(raw);

    // ---- candidate keys of this tile (draft rows of the cache): every element at or
    // above tau, the F-th largest of the block's 256 lane maxima (its four tiles are
    // consecutive tiles of one row).  F lanes of the row hold an element at or above
    // tau, so the row's F-th largest value is at least tau and every element of the
    // row's top F is kept by its tile.  Only the (lane, vector) pairs whose vector
    // maximum reaches tau can hold one: they are few, so they are compacted through
    // LDS, one per lane, and examined there; the keys are staged in LDS and copied out
    // with one coalesced store per 64 keys.
    uint32_t tau = 0u;
    int ncand = 0;
    if (topf) {
        const bool lane_valid = tile_ok && tile0 + (int64_t)lane * N < V;
        lane_key[wave][lane] = lane_valid ? ord32(m_lane) : 0u;
        __syncthreads();
        uint32_t k4[kWavesPerBlock];
#pragma unroll
        for (int w = 0; w < kWavesPerBlock; ++w) k4[w] = lane_key[w][lane];
        // The 16 high bits of the order keys suffice (all of a bf16 value's): any tau
        // at or below the F-th largest lane maximum keeps the row's top F, one lower by
        // less than a bf16 step only admits a few more fp32 keys, and each further bit
        // costs a round of four ballots.  A bound below the key of -inf (a negative NaN
        // pattern as a float) means every element: it becomes the key of -inf.
        tau = wave_select_regs_u32<kWavesPerBlock>(k4, F, 0xFFFF0000u);
        if (tau != 0u && tau < ord32(-INFINITY)) tau = ord32(-INFINITY);
    }
    if (topf) {
        const float tauf = tau ? unord32(tau) : -INFINITY;
        const int id0 = (int)tile0 + lane * N;
        const bool full = tile0 + kTile<DT> <= V;
        // the unit (this block's four tiles) stores its keys contiguously: this tile's at
        // the sum of the counts of the tiles before it
        const int capU = kWavesPerBlock * a.cap;
        uint64_t* unit = a.cand + ((r * units_per_row(a.nt)) + blk) * (int64_t)capU;
        uint64_t* stage = cand_stage[wave];
        const int cap = a.cap;
        int n = 0;
        if (tile_ok) {
        // hot (lane, vector) pairs, counted per vector with a ballot (scalar masks)
        int H = 0;
#pragma unroll
        for (int j = 0; j < kVecPerLane; ++j) H += __popcll(__ballot(vmax[j] >= tauf));
        H = uniform(H);
        if (H <= kHotCap) {
            // compacted vector-major: the hot lanes of vector j follow those of vectors
            // below j, in lane order
            u32x4* hv = hot_vec[wave];
            int* hid = hot_id[wave];
            int q0 = 0;
#pragma unroll
            for (int j = 0; j < kVecPerLane; ++j) {
                const bool me = vmax[j] >= tauf;
                const uint64_t mj = __ballot(me);
                if (mj) {  // uniform
                    const int q = q0 + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mj >> 32),
                                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mj, 0u));
                    if (me) {
                        hv[q] = raw[j];
                        hid[q] = id0 + j * kWave * N;
                    }
                    q0 += __popcll(mj);
                }
            }
            wave_sync_lds();
            // one element per lane: element e of hot vector q is lane (q N + e) mod 64
            const uint32_t* hw = reinterpret_cast<const uint32_t*>(hv);
            for (int p0 = 0; p0 < H * N; p0 += kWave) {
                const int pp = p0 + lane;
                const bool live = pp < H * N;
                const int q = live ? pp / N : 0, e = pp % N;
                const uint32_t w = hw[q * 4 + (DT == 1 ? e >> 1 : e)];
                const float x = DT == 1 ? __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16)) : __uint_as_float(w);
                const int id = hid[q] + e;
                const bool hit = live && x >= tauf && (full || id < V);
                const uint64_t mk = __ballot(hit);
                const int pos = n + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mk >> 32),
                                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)mk, 0u));
                if (hit && pos < kStageCap) stage[pos] = cand_key(x, (uint32_t)id);
                n += __popcll(mk);
            }
        } else {
            // many hot vectors (a threshold at -inf, or heavy ties): element by element
            const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
            for (int j = 0; j < kVecPerLane; ++j) {
                if (__ballot(vmax[j] >= tauf) == 0ull) continue;
#pragma unroll
                for (int e = 0; e < N; ++e) {
                    const float v = vec_elem<DT>(raw[j], e);
                    const int id = id0 + j * kWave * N + e;
                    const bool hit = v >= tauf && (full || id < V);
                    const uint64_t mk = __ballot(hit);
                    if (mk) {  // uniform; the store itself is unconditional (misses go to
                               // the lane's discard slot)
                        const int pos = n + __popcll(mk & below);
                        stage[hit && pos < kStageCap ? pos : kStageCap + lane] = cand_key(v, (uint32_t)id);
                        n += __popcll(mk);
                    }
                }
            }
        }
        wave_sync_lds();
        }  // tile_ok
        // a tile with more tied keys than its stage stores its exact top F instead
        const bool exact = n > min(cap, kStageCap);
        unit_cnt[wave] = exact ? F : n;
        __syncthreads();
        int off = 0, total = 0;
#pragma unroll
        for (int w = 0; w < kWavesPerBlock; ++w) {
            const int cw = unit_cnt[w];
            off += w < wave ? cw : 0;
            total += cw;
        }
        if (tile_ok && !exact) {
            for (int q = lane; q < n; q += kWave) unit[off + q] = stage[q];
        } else if (tile_ok) {
            // F rounds of a wave maximum below the previous key (re-reading the tile)
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
                for (int o = 32; o >= 1; o >>= 1) {
                    const uint64_t x = __shfl_xor(best, o, kWave);
                    best = x > best ? x : best;
                }
                if (lane == 0) unit[off + q] = best;
                prev = best;
            }
        }
        // the slots a finalisation reads before it knows the count hold 0 past the keys
        if (wave == 0)
            for (int q = total + lane; q < spec_slots(F, capU); q += kWave) unit[q] = 0ull;
        ncand = wave == 0 ? total : 0;  // the unit's count, in its first tile's partial
    }

    if (!tile_ok) return;  // a wave past the row's last tile: nothing to record

    // ---- logit at the draft token of this row, if it falls in this tile
    if (has_draft) {
        const int d = d_tok;
        const int64_t off = (int64_t)d - tile0;
        if (d >= 0 && d < V && off >= 0 && off < kTile<DT>) {  // uniform
            const int owner = (int)((off / N) % kWave), jd = (int)(off / (N * kWave)), ed = (int)(off % N);
            if (lane == owner) {
                u32x4 v = raw[0];
#pragma unroll
                for (int j = 1; j < kVecPerLane; ++j) v = jd == j ? raw[j] : v;
                uint32_t w = v.x;
                const int q = DT == 1 ? ed >> 1 : ed;
                w = q == 1 ? v.y : w;
                w = q == 2 ? v.z : w;
                w = q == 3 ? v.w : w;
                if (DT == 1) w = (ed & 1) ? (w & 0xFFFF0000u) : (w << 16);
                a.probe[((int64_t)b * (a.K1 - 1) + i) * a.nmodel + model] = __uint_as_float(w);
            }
        }
    }

    // ---- tile partial
    wave_stats(m_lane, s, arg, c, m, s, arg);
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

// The weights are kept in the units of the target row's terms tp = term(z_p, c, op)
// (p(x) = tp * inv_p), so that no per-element scaling is needed: with tq = term(z_q,
// c, oq) and q'(x) = tq * sc_q * (C if cached else 1),
//   residual  max(p - q', 0) = inv_p * max(tp - tq * rho_sel, 0),  rho = sc_q / inv_p;
//   target    p              = inv_p * tp;
//   draft q'  (its own units)  tq * (C if cached else 1).
// The inverse CDF is invariant to the common factor; only the reported residual mass
// is scaled back by inv_p.
struct WParams {
    float c;
    float op, oq;        // offsets of the target / draft rows
    double inv_p;        // p(x) = tp * inv_p
    double rho, rhoC;    // draft-to-target unit ratio, off / on the cached ids
    double Cd;           // C as double (tq * C is exact in fp64)
};

// Row statistics of one (b, position), loaded together with no branch in between so
// that they travel with the tile loads.  Without a target law (draft sampling) the
// draft statistics stand in for it and are not used.
struct LawIn {
    float pm, qm;
    double ps, qs, Z;
};
// a / b for a positive normal b, to within about an ulp: the hardware reciprocal refined
// by two Newton steps, then one correction of the quotient.  Short latency, for the law
// parameters (their rounding moves each weight by a relative 1e-16 at most).
__device__ __forceinline__ double fdiv64(double a, double b) {
    double r = __builtin_amdgcn_rcp(b);
    double e = __builtin_fma(-b, r, 1.0);
    r = __builtin_fma(r, e, r);
    e = __builtin_fma(-b, r, 1.0);
    r = __builtin_fma(r, e, r);
    const double q = a * r;
    return __builtin_fma(__builtin_fma(-b, q, a), r, q);
}

// 1 / (row sum in units of 2^{z c - o}) for a row with maximum m and standard sum s.
__device__ __forceinline__ double law_inv(float m, double s, float c, float o) { return fdiv64(offset_factor(m, c, o), s); }
__device__ __forceinline__ double law_rho(double inv_q, double Z, double inv_p) { return fdiv64(fdiv64(inv_q, Z), inv_p); }

__device__ __forceinline__ WParams make_wparams(float c, float C, bool with_p, const LawIn& L) {
    WParams w;
    w.c = c;
    w.op = 0.f;
    w.inv_p = 0.0;
    w.rho = w.rhoC = 0.0;
    w.Cd = (double)C;
    w.oq = offset_of(L.qm, c);
    if (with_p) {
        w.op = offset_of(L.pm, c);
        w.inv_p = law_inv(L.pm, L.ps, c, w.op);
        w.rho = law_rho(law_inv(L.qm, L.qs, c, w.oq), L.Z, w.inv_p);
        w.rhoC = w.rho * w.Cd;
    }
    return w;
}

// The law parameters of row r as the finalisation computes them once per (b, i) for the
// fused round (the same expressions on the same values, so bit-identical to computing
// them per wave), in the LawParams record pass 2 and the bonus load.
__device__ __forceinline__ WParams wparams_from(const LawParams& P, float c, float C) {
    WParams w;
    w.c = c;
    w.op = P.op;
    w.oq = P.oq;
    w.inv_p = P.inv_p;
    w.rho = P.rho;
    w.rhoC = P.rhoC;
    w.Cd = (double)C;
    return w;
}

// ============================================================================ finalise
// Partial of tile `lane` of a row (the identity past nt), for rows of at most 64 tiles.
__device__ __forceinline__ WavePartial lane_partial(const WavePartial* P, int nt) {
    WavePartial q;
    if (lane_id() < nt) {
        q = P[lane_id()];
    } else {
        q.m = -INFINITY;
        q.arg = INT_MAX;
        q.s = 0.0;
        q.tau = 0u;
        q.ncand = 0;
        q.pad0 = q.pad1 = 0;
    }
    return q;
}

// Softmax statistics from one tile partial per lane; the same merges in the same order
// as row_stats_wave for a row of at most 64 tiles.
__device__ __forceinline__ void stats_from_lanes(const WavePartial& q, float c, float& m, double& s, int& arg) {
    m = -INFINITY;
    s = 0.0;
    arg = INT_MAX;
    merge_stats(m, s, arg, q.m, q.s, q.arg, c);
    wave_stats(m, s, arg, c, m, s, arg);
}

// Accepted length of sequence b from the per-position test outcomes (the first
// rejected position, K if none) and the OR of their error bits; every lane returns
// both.  Outcomes: bit 0 accepted, the bits above it the error bits.  v: lane j's
// outcome of position j (1 past K).
__device__ __forceinline__ int accepted_length_of(int v, int* errs) {
    const uint64_t rm = __ballot((v & 1) == 0);
    *errs = (int)wave_or_u32((uint32_t)(v >> 1));
    return rm ? (__ffsll((long long)rm) - 1) : kWave;
}
__device__ __forceinline__ int accepted_length(const int32_t* vflag, int b, int K, int* errs) {
    const int v = lane_id() < K ? vflag[(int64_t)b * K + lane_id()] : 1;
    return min(accepted_length_of(v, errs), K);
}

// One wave per (sequence b, position i): the statistics of target row i and draft
// row i, the cache ids of draft row i, its cached mass M, the Saguaro normaliser
// Z = 1 - (1 - C) M and the lossless test of draft token d_i.  For rows of at most 64
// tiles the tile partials, the first candidate slots of every unit and the logits at
// d_i are requested together.
// Three waves per SIMD (at most 168 VGPRs; unbounded it takes 170 and two), so that the
// 2,560 waves of a B=512 K=4 round are resident at once.
template <int DT, bool DEVRNG>
__global__ __launch_bounds__(kWave, 3) void finalize_pos_kernel(const SeqFinal f) {
    __shared__ TopfScratch sc;
    __shared__ LawParams law_lds;  // the target-row half of the law, kept across the select
    const int lane = threadIdx.x;
    const int K = f.K, K1 = K + 1, nt = f.nt;
    int b, i;  // one wave per block, pair (b, i) on XCD b mod 8
    xcd_pair(blockIdx.x, K1, b, i);
    if (b >= f.B) return;
    const WavePartial* part = f.part + (int64_t)b * 2 * K1 * nt;
    const bool fast = nt <= kWave;
    const int64_t r = (int64_t)b * K1 + i;
    const WavePartial* Pp = part + (int64_t)i * nt;
    const WavePartial* Pq = part + (int64_t)(K1 + i) * nt;
    const int nu = units_per_row(nt), capU = kWavesPerBlock * f.cap;
    const uint64_t* cr = f.cand + r * nu * (int64_t)capU;
    const int F = f.F[i];
    DraftProbe pr;
    pr.d = i < K ? f.draft[(int64_t)b * K + i] : 0;
    pr.zp = i < K ? f.probe[((int64_t)b * K + i) * 2 + 0] : 0.f;  // valid when d_i is in range
    pr.zq = i < K ? f.probe[((int64_t)b * K + i) * 2 + 1] : 0.f;
    const uint64_t round = DEVRNG ? *f.round_ptr : f.round;
    pr.u = (i < K && !f.greedy) ? philox_uniform(f.seed, round, kPurposeAccept, (uint64_t)b, (uint64_t)i) : 0.f;
    float mp, mq;
    double sp, sq;
    int ap, aq;
    CandSummary cs;
    uint64_t k[kCandRegs];
    int Rg = 0;
    int nc_lane = 0;
    if (fast) {
        const WavePartial qq = lane_partial(Pq, nt), pp = lane_partial(Pp, nt);
        if (F > 0) {
            Rg = min(spec_slots(F, capU), kWave * kCandRegs / nu);
            gather_slots<kCandRegs>(cr, capU, nu, Rg, k);
        }
        stats_from_lanes(qq, f.c, mq, sq, aq);
        stats_from_lanes(pp, f.c, mp, sp, ap);
        // Floor of the row's F-th largest value: the largest tile threshold, or a lower
        // bound of the F-th largest tile maximum (F tiles hold an element at or above
        // it; its 10 leading differing bits suffice) if higher.
        cs.tr = wave_max_u32(qq.tau);
        if (F > 0 && F < nt) cs.tr = max(cs.tr, wave_select_u32(lane < nt ? ord32(qq.m) : 0u, F, 10));
        cs.max_nc = (int)wave_max_u32((uint32_t)qq.ncand);
        nc_lane = __shfl(qq.ncand, min(kWavesPerBlock * lane, kWave - 1), kWave);  // unit `lane`
    } else {
        CandSummary unused;
        row_stats_wave(Pq, nt, f.c, mq, sq, aq, true, cs, sc.nc);
        row_stats_wave(Pp, nt, f.c, mp, sp, ap, false, unused, nullptr);
    }
    sq = f.greedy ? 1.0 : std_sum(mq, sq, f.c);
    sp = f.greedy ? 1.0 : std_sum(mp, sp, f.c);
    // the draft test's exponentials need only the statistics: before the cache select
    const DraftTerms dt = i < K ? draft_terms(pr, f.V, mp, sp, mq, sq, f.c, f.greedy) : DraftTerms{0.0, 0.0, 0, false};
    if (lane == 0) {
        f.q_max[r] = mq;
        f.q_sum[r] = sq;
        if (f.q_arg) f.q_arg[r] = aq;
        f.p_max[r] = mp;
        f.p_sum[r] = sp;
        if (f.p_arg) f.p_arg[r] = ap;
        if (f.law && !f.greedy) {
            law_lds.op = offset_of(mp, f.c);
            law_lds.inv_p = law_inv(mp, sp, f.c, law_lds.op);
        }
    }
    double M = 0.0;
    int my_id = -1;
    if (F > 0) {
        uint64_t key;
        if (fast && cs.max_nc <= Rg) {
            // every unit's keys lie in its first Rg slots, and the slots past them hold 0
            const uint64_t floor_key = cs.tr ? (uint64_t)cs.tr << 32 : 1ull;
            const int U = uniform((nu * Rg + kWave - 1) / kWave);  // unit-major slots in use
            if (U <= 4)
                key = select_sorted<4>(reinterpret_cast<uint64_t(&)[4]>(k), U, F, sc, floor_key);
            else if (U <= 8)
                key = select_sorted<8>(reinterpret_cast<uint64_t(&)[8]>(k), U, F, sc, floor_key);
            else if (U <= 12)
                key = select_sorted<12>(reinterpret_cast<uint64_t(&)[12]>(k), U, F, sc, floor_key);
            else
                key = select_sorted<kCandRegs>(k, U, F, sc, floor_key);
        } else {
            if (fast) {
                if (lane < nu) sc.nc[lane] = (uint16_t)nc_lane;
                wave_sync_lds();
            }
            key = row_topf_wave(Pq, cr, nt, capU, F, cs, sc);
        }
        M = finish_cache_row(key, F, mq, sq, f.c, f.greedy, f.cache_ids + (int64_t)b * f.Bf + f.O[i], nullptr);
        my_id = lane < F && key ? (int)key_id(key) : -1;
    }
    const double Z = 1.0 - (1.0 - (double)f.C) * M;
    if (lane == 0) {
        f.cache_mass[r] = M;
        f.Z[r] = Z;
        if (f.law && !f.greedy) {  // as make_wparams computes it from the same values
            LawParams P;
            P.op = law_lds.op;
            P.inv_p = law_lds.inv_p;
            P.oq = offset_of(mq, f.c);
            P.rho = law_rho(law_inv(mq, sq, f.c, P.oq), Z, P.inv_p);
            P.rhoC = P.rho * (double)f.C;
            f.law[r] = P;
        }
    }
    if (i < K) {
        const bool in_cache = __ballot(my_id >= 0 && my_id == pr.d) != 0ull;
        double ratio;
        int err;
        const bool acc = draft_decide(pr, dt, ap, Z, in_cache, f.C, f.greedy, &ratio, &err);
        if (lane == 0) {
            f.vflag[(int64_t)b * K + i] = (acc ? 1 : 0) | (err << 1);
            if (f.accept_prob) f.accept_prob[(int64_t)b * K + i] = (float)(ratio < 1.0 ? ratio : 1.0);
        }
    }
}

// The same finalisation by a block of two waves per (b, i), for rounds of at most one
// (b, i) per SIMD, where the one-wave kernel leaves SIMDs idle and each wave's chain of
// steps is the kernel's time.
template <int DT, bool DEVRNG>
__global__ __launch_bounds__(2 * kWave, 3) void finalize_pos2_kernel(const SeqFinal f) {
    // Two waves per (b, i).  Wave 0 takes the draft row: its statistics, the cache ids,
    // M, Z and whether d_i is cached.  Wave 1 takes the target row and the test of d_i:
    // it forms the draft row's statistics again from the same partials by the same merges
    // (the same values), so the test's exponentials run while wave 0 selects the cache;
    // the two meet once, for Z and the membership of d_i.
    __shared__ TopfScratch sc;  // wave 0
    __shared__ double hand_Z;
    __shared__ int hand_in;
    const int wave = uniform((int)(threadIdx.x / kWave)), lane = threadIdx.x % kWave;
    const int K = f.K, K1 = K + 1, nt = f.nt;
    int b, i;  // pair (b, i) on XCD b mod 8
    xcd_pair(blockIdx.x, K1, b, i);
    if (b >= f.B) return;  // uniform over the block
    const WavePartial* part = f.part + (int64_t)b * 2 * K1 * nt;
    const bool fast = nt <= kWave;
    const int64_t r = (int64_t)b * K1 + i;
    const WavePartial* Pp = part + (int64_t)i * nt;
    const WavePartial* Pq = part + (int64_t)(K1 + i) * nt;
    float mp = 0.f, mq = 0.f;
    double sp = 0.0, sq = 0.0;
    int ap = INT_MAX, aq = INT_MAX;
    DraftProbe pr;
    DraftTerms dt{0.0, 0.0, 0, false};
    if (wave == 0) {
        const int nu = units_per_row(nt), capU = kWavesPerBlock * f.cap;
        const uint64_t* cr = f.cand + r * nu * (int64_t)capU;
        const int F = f.F[i];
        const int d = i < K ? f.draft[(int64_t)b * K + i] : -1;
        CandSummary cs;
        uint64_t k[kCandRegs];
        int Rg = 0;
        int nc_lane = 0;
        if (fast) {
            const WavePartial qq = lane_partial(Pq, nt);
            if (F > 0) {
                Rg = min(spec_slots(F, capU), kWave * kCandRegs / nu);
                gather_slots<kCandRegs>(cr, capU, nu, Rg, k);
            }
            stats_from_lanes(qq, f.c, mq, sq, aq);
            // Floor of the row's F-th largest value: the largest tile threshold, or a lower
            // bound of the F-th largest tile maximum (F tiles hold an element at or above
            // it; its 10 leading differing bits suffice) if higher.
            cs.tr = wave_max_u32(qq.tau);
            if (F > 0 && F < nt) cs.tr = max(cs.tr, wave_select_u32(lane < nt ? ord32(qq.m) : 0u, F, 10));
            cs.max_nc = (int)wave_max_u32((uint32_t)qq.ncand);
            nc_lane = __shfl(qq.ncand, min(kWavesPerBlock * lane, kWave - 1), kWave);  // unit `lane`
        } else {
            row_stats_wave(Pq, nt, f.c, mq, sq, aq, true, cs, sc.nc);
        }
        sq = f.greedy ? 1.0 : std_sum(mq, sq, f.c);
        if (lane == 0) {
            f.q_max[r] = mq;
            f.q_sum[r] = sq;
            if (f.q_arg) f.q_arg[r] = aq;
        }
        double M = 0.0;
        int my_id = -1;
        if (F > 0) {
            uint64_t key;
            if (fast && cs.max_nc <= Rg) {
                // every unit's keys lie in its first Rg slots, and the slots past them hold 0
                const uint64_t floor_key = cs.tr ? (uint64_t)cs.tr << 32 : 1ull;
                const int U = uniform((nu * Rg + kWave - 1) / kWave);  // unit-major slots in use
                if (U <= 4)
                    key = select_sorted<4>(reinterpret_cast<uint64_t(&)[4]>(k), U, F, sc, floor_key);
                else if (U <= 8)
                    key = select_sorted<8>(reinterpret_cast<uint64_t(&)[8]>(k), U, F, sc, floor_key);
                else if (U <= 12)
                    key = select_sorted<12>(reinterpret_cast<uint64_t(&)[12]>(k), U, F, sc, floor_key);
                else
                    key = select_sorted<kCandRegs>(k, U, F, sc, floor_key);
            } else {
                if (fast) {
                    if (lane < nu) sc.nc[lane] = (uint16_t)nc_lane;
                    wave_sync_lds();
                }
                key = row_topf_wave(Pq, cr, nt, capU, F, cs, sc);
            }
            M = finish_cache_row(key, F, mq, sq, f.c, f.greedy, f.cache_ids + (int64_t)b * f.Bf + f.O[i], nullptr);
            my_id = lane < F && key ? (int)key_id(key) : -1;
        }
        const double Z = 1.0 - (1.0 - (double)f.C) * M;
        const bool in_cache = __ballot(my_id >= 0 && my_id == d) != 0ull;
        if (lane == 0) {
            f.cache_mass[r] = M;
            f.Z[r] = Z;
            hand_Z = Z;
            hand_in = in_cache ? 1 : 0;
        }
    } else {
        pr.d = i < K ? f.draft[(int64_t)b * K + i] : 0;
        pr.zp = i < K ? f.probe[((int64_t)b * K + i) * 2 + 0] : 0.f;  // valid when d_i is in range
        pr.zq = i < K ? f.probe[((int64_t)b * K + i) * 2 + 1] : 0.f;
        const uint64_t round = DEVRNG ? *f.round_ptr : f.round;
        pr.u = (i < K && !f.greedy) ? philox_uniform(f.seed, round, kPurposeAccept, (uint64_t)b, (uint64_t)i) : 0.f;
        if (fast) {
            const WavePartial qq = lane_partial(Pq, nt), pp = lane_partial(Pp, nt);
            stats_from_lanes(qq, f.c, mq, sq, aq);
            stats_from_lanes(pp, f.c, mp, sp, ap);
        } else {
            CandSummary unused;
            row_stats_wave(Pq, nt, f.c, mq, sq, aq, false, unused, nullptr);
            row_stats_wave(Pp, nt, f.c, mp, sp, ap, false, unused, nullptr);
        }
        sq = f.greedy ? 1.0 : std_sum(mq, sq, f.c);
        sp = f.greedy ? 1.0 : std_sum(mp, sp, f.c);
        if (i < K) dt = draft_terms(pr, f.V, mp, sp, mq, sq, f.c, f.greedy);
        if (lane == 0) {
            f.p_max[r] = mp;
            f.p_sum[r] = sp;
            if (f.p_arg) f.p_arg[r] = ap;
        }
    }
    __syncthreads();
    if (wave == 0) return;
    const double Z = hand_Z;
    if (lane == 0 && f.law && !f.greedy) {  // as make_wparams computes it from the same values
        LawParams P;
        P.op = offset_of(mp, f.c);
        P.inv_p = law_inv(mp, sp, f.c, P.op);
        P.oq = offset_of(mq, f.c);
        P.rho = law_rho(law_inv(mq, sq, f.c, P.oq), Z, P.inv_p);
        P.rhoC = P.rho * (double)f.C;
        f.law[r] = P;
    }
    if (i < K) {
        double ratio;
        int err;
        const bool acc = draft_decide(pr, dt, ap, Z, hand_in != 0, f.C, f.greedy, &ratio, &err);
        if (lane == 0) {
            f.vflag[(int64_t)b * K + i] = (acc ? 1 : 0) | (err << 1);
            if (f.accept_prob) f.accept_prob[(int64_t)b * K + i] = (float)(ratio < 1.0 ? ratio : 1.0);
        }
    }
}

// T = 0: one wave per sequence takes the accepted length from the test outcomes, the
// bonus (target argmax at that position) and the cache lookup.
template <bool DEVRNG>
__global__ __launch_bounds__(kBlock) void finish_greedy_kernel(const SeqFinal f) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    // sequence b on XCD b mod 8, four to a block
    const int b = ((int)(blockIdx.x / kXcds) * kWavesPerBlock + wave) * kXcds + (int)(blockIdx.x % kXcds);
    if (b >= f.B) return;
    const int K = f.K;
    int errs;
    const int k = accepted_length(f.vflag, b, K, &errs);
    const int tok = f.p_arg[(int64_t)b * (K + 1) + k];
    const int my_id = cached_id(f.cache_ids, b, f.Bf, k, K, f.F, f.O);
    if (lane == 0) {
        f.accept_len[b] = k;
        if (f.dev_err && errs) f.dev_err[b] |= errs;
        f.bonus[b] = tok;
        if (f.resid_mass) f.resid_mass[b] = 1.0;
    }
    const uint64_t round = DEVRNG ? *f.round_ptr : f.round;
    lookup_wave(b, K, f.V, k, f.O[k], my_id, tok, f.fallback, f.seed, round, f.hit, f.slot, f.fallback_tokens,
                ValueStore{f.cache_values, f.Bf, f.next_draft});
}

// ============================================================================ pass 2
enum { kWResid = 0, kWP = 1, kWQprime = 2 };

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

// Weight of one element for the inverse-CDF scan (fp64, in the units above); *pw
// receives tp.  A -inf logit (also the padding past V) has term 0 and weight 0.
template <int MODE>
__device__ __forceinline__ double elem_weight_t(const WParams& w, float zp, float zq, bool in_cache, double* pw) {
    double tp = 0.0;
    if (MODE != kWQprime) tp = (double)term(zp, w.c, w.op);
    *pw = tp;
    if (MODE == kWP) return tp;
    const double tq = (double)term(zq, w.c, w.oq);
    if (MODE == kWQprime) return in_cache ? tq * w.Cd : tq;
    const double d = __builtin_fma(-tq, in_cache ? w.rhoC : w.rho, tp);
    return d > 0.0 ? d : 0.0;
}

// Wave-private membership bitmap (kTile/32 words) of the cached ids of a row that
// fall in the tile [t0, t0 + kTile); lane j holds cached id j (or -1) in my_id.
template <int DT>
__device__ inline void tile_bitmap(uint32_t* bits, int64_t t0, int my_id) {
    const int lane = lane_id();
    for (int w = lane; w < kTile2<DT> / 32; w += kWave) bits[w] = 0u;
    wave_sync_lds();
    if (my_id >= t0 && my_id < t0 + kTile2<DT>)
        atomicOr(&bits[(my_id - t0) >> 5], 1u << ((my_id - t0) & 31));
    wave_sync_lds();
}

// Weights of one lane's vector j of a tile from the raw vectors of the target and
// draft rows.  The tile loads hold -inf past V, so those elements weigh 0.  LEAN weighs
// every element as uncached and weighs again, in a branch, the cached ones (F of V ids,
// so rarely any in a vector): the same values with fewer instructions per element, for
// grids whose time is their VALU work.
template <int DT, int MODE, bool LEAN = false>
__device__ __forceinline__ void vec_weights(const WParams& wp, u32x4 rp, u32x4 rq, int64_t e0, int V,
                                            const uint32_t* bits, int64_t t0, double* w, double* p) {
    constexpr int N = ElemTraits<DT>::kPerVec;
    float zp[N], zq[N];
    if (MODE != kWQprime) unpack_vec<DT>(rp, zp);
    if (MODE != kWP) unpack_vec<DT>(rq, zq);
    uint32_t cbits = 0u;
    if (MODE != kWP) cbits = bits[(e0 - t0) >> 5] >> ((e0 - t0) & 31);
    if (LEAN) {
        if (MODE != kWP) cbits &= (1u << N) - 1u;
#pragma unroll
        for (int e = 0; e < N; ++e)
            w[e] = elem_weight_t<MODE>(wp, MODE != kWQprime ? zp[e] : 0.f, MODE != kWP ? zq[e] : 0.f, false, &p[e]);
        if (MODE != kWP && cbits != 0u) {
#pragma unroll
            for (int e = 0; e < N; ++e) {
                double pw;
                if ((cbits >> e) & 1u)
                    w[e] = elem_weight_t<MODE>(wp, MODE != kWQprime ? zp[e] : 0.f, zq[e], true, &pw);
            }
        }
        return;
    }
#pragma unroll
    for (int e = 0; e < N; ++e) {
        w[e] = elem_weight_t<MODE>(wp, MODE != kWQprime ? zp[e] : 0.f, MODE != kWP ? zq[e] : 0.f, (cbits >> e) & 1u,
                                   &p[e]);
    }
}

// Sums over one lane's part of a wave tile: sw of the weights, sp of p(x).  The tile
// and the row statistics are requested before any of them is used.
template <int DT, bool VEC, int MODE, bool LEAN>
__device__ __forceinline__ void tile_sums(const Pass2Args& a, int64_t r, const char* prow, const char* qrow, int64_t t0,
                                          const int32_t* ids, int Fk, uint32_t* bits, double& sw, double& sp) {
    constexpr int N = ElemTraits<DT>::kPerVec;
    const int lane = lane_id();
    u32x4 rp[kVecPass2], rq[kVecPass2];
    if (MODE != kWQprime) load_tile<DT, VEC, kVecPass2>(prow, t0, a.V, lane, rp);
    if (MODE != kWP) load_tile<DT, VEC, kVecPass2>(qrow, t0, a.V, lane, rq);
    int my_id = -1;
    if (MODE != kWP && lane < Fk) my_id = ids[lane];
    const WParams wp = a.law ? wparams_from(a.law[r], a.c, a.C) : make_wparams(a.c, a.C, MODE != kWQprime, load_law(a, r));
    if (MODE != kWP) tile_bitmap<DT>(bits, t0, my_id);
#pragma unroll
    for (int j = 0; j < kVecPass2; ++j) {
        const int64_t e0 = t0 + (int64_t)(j * kWave + lane) * N;
        double w[N], p[N];
        vec_weights<DT, MODE, LEAN>(wp, rp[j], rq[j], e0, a.V, bits, t0, w, p);
        double vw = 0.0, vp = 0.0;
#pragma unroll
        for (int e = 0; e < N; ++e) {
            vw += w[e];
            vp += p[e];
        }
        sw += vw;
        sp += vp;
        // LEAN: each vector's sums complete here (left free, the compiler keeps every
        // vector's weights live at once, about twice the registers)
        if (LEAN) __asm__ volatile("" : "+v"(sw), "+v"(sp));
    }
}

__device__ inline void pass2_group(const Pass2Args& a, int g, int& b, int& pos, bool& valid, int* errs = nullptr) {
    if (a.mode == 0) {
        b = g;
        int e = 0;
        pos = a.vflag ? accepted_length(a.vflag, b, a.K, &e) : a.accept_len[b];
        if (errs) *errs = e;
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

// The crossing tile is rescanned by the four waves of a block, wave j taking vector j
// of the tile (ids t0 + (j*64 + lane)*N + e: vector, then lane, then element order).
struct BonusShare {
    double tot[kVecPass2];  // weight of each vector
    int lastp[kVecPass2];   // last id of positive weight in each vector (-1: none)
    int found;              // the id where the running sum crosses thr (-1: none)
};

// Phase 1, every wave: the weights of its vector, their total and last positive id,
// published in sh.  Returns the lane's weight sum (phase 2 needs it).
template <int DT, int MODE>
__device__ inline double rescan_vector_sums(const WParams& wp, u32x4 rp, u32x4 rq, int64_t t0, int V, int my_id,
                                            uint32_t* bits, int j, BonusShare& sh) {
    constexpr int N = ElemTraits<DT>::kPerVec;
    const int lane = lane_id();
    if (MODE != kWP) tile_bitmap<DT>(bits, t0, my_id);
    const int64_t e0 = t0 + (int64_t)(j * kWave + lane) * N;
    double w[N], p[N];
    vec_weights<DT, MODE>(wp, rp, rq, e0, V, bits, t0, w, p);
    double ls = 0.0;
    int lastp = -1;
#pragma unroll
    for (int e = 0; e < N; ++e) {
        ls += w[e];
        if (w[e] > 0.0) lastp = (int)(e0 + e);
    }
    const double tot = wave_sum_f64(ls);
    const int last = (int)wave_max_u32((uint32_t)(lastp + 1)) - 1;
    if (lane == 0) {
        sh.tot[j] = tot;
        sh.lastp[j] = last;
    }
    return ls;
}

// Phase 2, after a block barrier, block level: the draw block of the tile where the
// running sum of block weights (from base, in id order) first exceeds thr (-1: none).
template <int DT>
__device__ __forceinline__ int crossing_block(const BonusShare& sh, double base, double thr) {
    constexpr int VPB = kVecPerBlock<DT>;
    double run = base;
    int bx = -1;
#pragma unroll
    for (int k = 0; k < kBlocksPerTile2<DT>; ++k) {
        double wb = 0.0;
#pragma unroll
        for (int v = 0; v < VPB; ++v) wb += sh.tot[k * VPB + v];
        if (bx < 0) {
            if (run + wb > thr)
                bx = k;
            else
                run += wb;
        }
    }
    return bx;
}

// The last draw block of the tile holding a positive weight (-1: none).
template <int DT>
__device__ __forceinline__ int last_positive_block(const BonusShare& sh) {
    int bx = -1;
#pragma unroll
    for (int j = 0; j < kVecPass2; ++j)
        if (sh.lastp[j] >= 0) bx = j / kVecPerBlock<DT>;
    return bx;
}

// Id level inside block bx: thr = u2 times the block's weight, the vector of the block
// where the running sum from the block's first id first exceeds it (-1: none) and
// run = the sum before that vector.
template <int DT>
__device__ __forceinline__ int crossing_vector_in_block(const BonusShare& sh, int bx, double u2, double& run,
                                                        double& thr) {
    constexpr int VPB = kVecPerBlock<DT>;
    double wb = 0.0;
#pragma unroll
    for (int v = 0; v < VPB; ++v) wb += sh.tot[bx * VPB + v];
    thr = u2 * wb;
    run = 0.0;
    int jx = -1;
#pragma unroll
    for (int v = 0; v < VPB; ++v) {
        if (jx < 0) {
            if (run + sh.tot[bx * VPB + v] > thr)
                jx = bx * VPB + v;
            else
                run += sh.tot[bx * VPB + v];
        }
    }
    return jx;
}

// Phase 2, the wave of the crossing vector: the first id whose running sum (run before
// the vector, then the vector's ids in order) exceeds thr, recomputing its weights;
// published in sh.found.
template <int DT, int MODE>
__device__ inline void rescan_vector_find(const WParams& wp, u32x4 rp, u32x4 rq, int64_t t0, int V,
                                          const uint32_t* bits, int j, double ls, double run, double thr,
                                          BonusShare& sh) {
    constexpr int N = ElemTraits<DT>::kPerVec;
    const int lane = lane_id();
    const int64_t e0 = t0 + (int64_t)(j * kWave + lane) * N;
    double w[N], p[N];
    vec_weights<DT, MODE>(wp, rp, rq, e0, V, bits, t0, w, p);
    const double incl = wave_prefix_f64(ls);
    double cum = run + (incl - ls);
    int hitpos = -1;
#pragma unroll
    for (int e = 0; e < N; ++e) {
        cum += w[e];
        if (hitpos < 0 && cum > thr) hitpos = (int)(e0 + e);
    }
    const uint64_t hm = __ballot(hitpos >= 0);
    if (lane == 0) sh.found = hm ? (int)lane_u32((uint32_t)hitpos, uniform(__ffsll((long long)hm) - 1)) : -1;
}

// Inclusive wave scan of x (fp64, lane order).
__device__ __forceinline__ double wave_scan_incl(double x) { return wave_prefix_f64(x); }

// Bonus (or draft token) of one group by one block of four waves, a draw in two
// levels.  Block level, uniform u1: totals over the tiles in tile order and the tile
// where the running sum crosses u1 * total (every wave, alike), then inside it the
// draw block (512 ids) where the running sum of block weights crosses (wave j
// recomputes the weights of vector j of that tile).  Id level, uniform u2: the id of
// that block whose running sum from the block's first id crosses u2 times the block's
// weight.  Strict ">" in id order; with no crossing (rounding only) the last block,
// then the last id, of positive weight.  Wave 0 then does the cache lookup.  The tile
// sums of the first 64 tiles, the row statistics and the cached ids are requested
// together.
template <int DT, bool VEC, bool DEVRNG>
__device__ __forceinline__ void bonus_block(const Pass2Args& a, int g, int b, int pos, bool valid, int verrs,
                                            double2 v0, double2 v1, uint32_t* bits, BonusShare& sh, int wave,
                                            float upre) {
    const int lane = lane_id();
    const int K = a.K;
    const uint64_t round = DEVRNG ? *a.round_ptr : a.round;
    const int nt = a.nt;
    const double2* seg = a.seg + (int64_t)g * nt;
    double Zused = 0.0;
    int my_id = -1;
    int mode = pass2_mode(a, pos);
    bool pick_last = false;
    double gbase = 0.0, thr = 0.0, ls = 0.0, u2 = 0.0;
    int64_t t0 = 0;
    WParams wp{};
    u32x4 rp = neg_inf_vec<DT>(), rq = neg_inf_vec<DT>();
    if (valid) {
        const int64_t r = (int64_t)b * (K + 1) + pos;
        double u;
        if (a.mode == 0) {  // computed for every position before the accepted length was known
            u = (double)__shfl(upre, pos, kWave);
            u2 = (double)__shfl(upre, K + 1 + pos, kWave);
        } else {
            u = (double)philox_uniform(a.seed, round, kPurposeDraft, (uint64_t)b, (uint64_t)pos, 0);
            u2 = (double)philox_uniform(a.seed, round, kPurposeDraft, (uint64_t)b, (uint64_t)pos, 1);
        }
        // one chunk of at most 64 tiles (the usual case): the scan that gives the total
        // also locates the crossing
        const double incl_w = nt <= kWave ? wave_scan_incl(v0.x) : 0.0;
        double tot_w = 0.0, tot_p = 0.0;
        if (nt <= kWave) {
            tot_w = lane_f64(incl_w, kWave - 1);
        } else {
            for (int g0 = 0; g0 < nt; g0 += kWave) {
                const int j = g0 + lane;
                double2 v = v0;
                if (g0 > 0) v = g0 == kWave ? v1 : (j < nt ? seg[j] : make_double2(0.0, 0.0));
                tot_w += lane_f64(wave_scan_incl(v.x), kWave - 1);
            }
        }
        double Z = tot_w;
        const bool use_p = mode == kWResid && !(Z > 0.0);
        if (use_p) {
            for (int g0 = 0; g0 < nt; g0 += kWave) {
                const int j = g0 + lane;
                double2 v = v0;
                if (g0 > 0) v = g0 == kWave ? v1 : (j < nt ? seg[j] : make_double2(0.0, 0.0));
                tot_p += lane_f64(wave_scan_incl(v.y), kWave - 1);
            }
            mode = kWP;
            Z = tot_p;
        }
        thr = u * Z;
        int gsel = -1, glast = -1;
        double lastbase = 0.0, carry = 0.0;
        for (int g0 = 0; g0 < nt; g0 += kWave) {
            const int j = g0 + lane;
            double2 v = v0;
            if (g0 > 0) v = g0 == kWave ? v1 : (j < nt ? seg[j] : make_double2(0.0, 0.0));
            const double x = use_p ? v.y : v.x;
            const double incl = (nt <= kWave && !use_p ? incl_w : wave_scan_incl(x)) + carry;
            const double excl = incl - x;
            const uint64_t cross = __ballot(j < nt && incl > thr);
            const uint64_t posm = __ballot(j < nt && x > 0.0);
            if (gsel < 0 && cross) {
                const int l = uniform(__ffsll((long long)cross) - 1);
                gsel = g0 + l;
                gbase = lane_f64(excl, l);
            }
            if (posm) {
                const int l = uniform(63 - __clzll(posm));
                glast = g0 + l;
                lastbase = lane_f64(excl, l);
            }
            carry = lane_f64(incl, kWave - 1);
        }
        if (gsel < 0) {
            gsel = glast < 0 ? 0 : glast;
            gbase = lastbase;
            pick_last = true;
        }
        // this wave's vector of the crossing tile, the row statistics and the cached ids
        // travel together
        t0 = (int64_t)gsel * kTile2<DT>;
        const int64_t v0id = t0 + (int64_t)wave * kWave * ElemTraits<DT>::kPerVec;
        const char* prow = a.p_logits ? a.p_logits + r * a.ld_bytes : nullptr;
        const char* qrow = a.q_logits + r * a.ld_bytes;
        u32x4 tp[1], tq[1];
        tp[0] = rp;
        tq[0] = rq;
        if (mode != kWQprime) load_tile<DT, VEC, 1>(prow, v0id, a.V, lane, tp);
        if (mode != kWP) load_tile<DT, VEC, 1>(qrow, v0id, a.V, lane, tq);
        rp = tp[0];
        rq = tq[0];
        my_id = cached_id(a.cache_ids, b, a.Bf, pos, K, a.F, a.O);
        wp = a.law ? wparams_from(a.law[r], a.c, a.C) : make_wparams(a.c, a.C, mode != kWQprime, load_law(a, r));
        Zused = Z * wp.inv_p;  // the residual (or target) mass in probability units
        if (mode == kWResid)
            ls = rescan_vector_sums<DT, kWResid>(wp, rp, rq, t0, a.V, my_id, bits, wave, sh);
        else if (mode == kWP)
            ls = rescan_vector_sums<DT, kWP>(wp, rp, rq, t0, a.V, my_id, bits, wave, sh);
        else
            ls = rescan_vector_sums<DT, kWQprime>(wp, rp, rq, t0, a.V, my_id, bits, wave, sh);
    }
    if (threadIdx.x == 0) sh.found = -1;
    __syncthreads();
    double run = 0.0, thr2 = 0.0;
    int bx = -1, jx = -1;
    if (valid) {
        bx = pick_last ? -1 : crossing_block<DT>(sh, gbase, thr);
        if (bx < 0) bx = last_positive_block<DT>(sh);
        if (bx >= 0) jx = crossing_vector_in_block<DT>(sh, bx, u2, run, thr2);
    }
    if (jx == wave) {
        if (mode == kWResid)
            rescan_vector_find<DT, kWResid>(wp, rp, rq, t0, a.V, bits, wave, ls, run, thr2, sh);
        else if (mode == kWP)
            rescan_vector_find<DT, kWP>(wp, rp, rq, t0, a.V, bits, wave, ls, run, thr2, sh);
        else
            rescan_vector_find<DT, kWQprime>(wp, rp, rq, t0, a.V, bits, wave, ls, run, thr2, sh);
    }
    __syncthreads();
    if (wave != 0) return;
    int tok = -1;
    if (valid) {
        // fallbacks: the last positive id of the crossing vector, else of the block
        int last_pos = -1;
        if (jx >= 0) {
            last_pos = sh.lastp[jx];
        } else if (bx >= 0) {
#pragma unroll
            for (int v = 0; v < kVecPerBlock<DT>; ++v) last_pos = max(last_pos, sh.lastp[bx * kVecPerBlock<DT> + v]);
        }
        if (last_pos < 0) last_pos = (int)min<int64_t>(t0, a.V - 1);
        tok = sh.found >= 0 ? sh.found : last_pos;
    }
    if (lane == 0) {
        if (a.mode == 0) {
            a.out_tok[b] = tok;
            if (a.resid_mass) a.resid_mass[b] = Zused;
            if (a.vflag) {
                a.accept_len_out[b] = pos;
                if (a.dev_err && verrs) a.dev_err[b] |= verrs;
            }
            if (!valid && a.dev_err) a.dev_err[b] |= kErrLenRange;
        } else {
            a.out_tok[(int64_t)b * K + pos] = tok;
        }
    }
    if (a.mode == 0 && a.do_lookup)
        lookup_wave(b, K, a.V, valid ? pos : -1, valid ? a.O[pos] : 0, my_id, tok, a.fallback, a.seed, round, a.hit,
                    a.slot, a.fallback_tokens, ValueStore{a.cache_values, a.Bf, a.next_draft});
}

// One block of four waves per group when the bonus runs as a kernel of its own.
template <int DT, bool VEC, bool DEVRNG>
__global__ __launch_bounds__(kBlock) void finalize_bonus_kernel(const Pass2Args a, int ngroups) {
    static_assert(kVecPass2 == kWavesPerBlock, "one wave per vector of a pass-2 tile");
    __shared__ uint32_t bits[kWavesPerBlock][kTile2<1> / 32];
    __shared__ BonusShare sh;
    const int wave = threadIdx.x / kWave;
    const int g = blockIdx.x;
    if (g >= ngroups) return;  // uniform over the block
    const int lane = threadIdx.x % kWave;
    // the group's tile sums (their first two chunks of 64) do not depend on the accepted
    // length: request them first
    const double2 v0 = lane < a.nt ? a.seg[(int64_t)g * a.nt + lane] : make_double2(0.0, 0.0);
    const double2 v1 = kWave + lane < a.nt ? a.seg[(int64_t)g * a.nt + kWave + lane] : make_double2(0.0, 0.0);
    // the sequence's test outcomes (or its given accepted length), requested before the
    // uniforms below so that they load while those are computed
    int vf_or_len = 0;
    if (a.mode == 0) vf_or_len = a.vflag ? (lane < a.K ? a.vflag[(int64_t)g * a.K + lane] : 1) : a.accept_len[g];
    // the draw's two uniforms of each position k of sequence g, which lane j computes for
    // k = j mod (K+1), counter word j / (K+1), before the accepted length is known
    float upre = 0.f;
    if (a.mode == 0 && lane < 2 * (a.K + 1)) {
        const uint64_t round = DEVRNG ? *a.round_ptr : a.round;
        upre = philox_uniform(a.seed, round, kPurposeBonus, (uint64_t)g, (uint64_t)(lane % (a.K + 1)),
                              (uint64_t)(lane / (a.K + 1)));
    }
    int b, pos, verrs = 0;
    bool valid;
    if (a.mode == 0) {
        b = g;
        pos = vf_or_len;
        if (a.vflag) pos = min(accepted_length_of(vf_or_len, &verrs), a.K);
        valid = pos >= 0 && pos <= a.K;
        if (!valid) pos = 0;
    } else {
        pass2_group(a, g, b, pos, valid, &verrs);
    }
    bonus_block<DT, VEC, DEVRNG>(a, g, b, pos, valid, verrs, v0, v1, bits[wave], sh, wave, upre);
}

// One wave per (group, tile): the residual (or target-law) sums of the tile.
template <int DT, bool VEC, bool LEAN>
__global__ __launch_bounds__(kBlock) void pass2_kernel(const Pass2Args a, int ngroups) {
    __shared__ uint32_t bits[kWavesPerBlock][kTile2<1> / 32];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int nblk = (a.nt + kWavesPerBlock - 1) / kWavesPerBlock;
    // group g on XCD g mod 8 (the bonus block of group g is block g)
    const int y = blockIdx.x / kXcds;
    const int g = (y / nblk) * kXcds + blockIdx.x % kXcds;
    const int t = (y % nblk) * kWavesPerBlock + wave;
    if (g >= ngroups || t >= a.nt) return;
    int b, pos;
    bool valid;
    pass2_group(a, g, b, pos, valid);
    double sw = 0.0, sp = 0.0;
    if (valid) {
        const int64_t r = (int64_t)b * (a.K + 1) + pos;
        const int mode = pass2_mode(a, pos);
        const char* prow = a.p_logits ? a.p_logits + r * a.ld_bytes : nullptr;
        const char* qrow = a.q_logits + r * a.ld_bytes;
        const int64_t t0 = (int64_t)t * kTile2<DT>;
        const int32_t* ids = a.cache_ids + (int64_t)b * a.Bf + a.O[pos];
        const int Fk = a.F[pos];
        if (mode == kWResid)
            tile_sums<DT, VEC, kWResid, LEAN>(a, r, prow, qrow, t0, ids, Fk, bits[wave], sw, sp);
        else if (mode == kWP)
            tile_sums<DT, VEC, kWP, LEAN>(a, r, prow, qrow, t0, ids, Fk, bits[wave], sw, sp);
        else
            tile_sums<DT, VEC, kWQprime, LEAN>(a, r, prow, qrow, t0, ids, Fk, bits[wave], sw, sp);
    }
    sw = wave_sum_f64(sw);
    sp = wave_sum_f64(sp);
    if (lane == 0) a.seg[(int64_t)g * a.nt + t] = make_double2(sw, sp);
}

// Sums of one lane's vector (vw of the weights, vp of p(x)), every element weighed as
// uncached and summed as it is formed; a vector holding a cached id (F of V ids, so
// rarely) is summed again with each element's own weight.  Both are the select form's
// sums in its order, without the per-element arrays.
template <int DT, int MODE>
__device__ __forceinline__ void vec_sums(const WParams& wp, u32x4 rp, u32x4 rq, int64_t e0, const uint32_t* bits,
                                         int64_t t0, double& vw, double& vp) {
    constexpr int N = ElemTraits<DT>::kPerVec;
    uint32_t cbits = 0u;
    if (MODE != kWP) cbits = (bits[(e0 - t0) >> 5] >> ((e0 - t0) & 31)) & ((1u << N) - 1u);
    float zp[N], zq[N];
    if (MODE != kWQprime) unpack_vec<DT>(rp, zp);
    if (MODE != kWP) unpack_vec<DT>(rq, zq);
    vw = 0.0;
    vp = 0.0;
#pragma unroll
    for (int e = 0; e < N; ++e) {
        double pw;
        vw += elem_weight_t<MODE>(wp, MODE != kWQprime ? zp[e] : 0.f, MODE != kWP ? zq[e] : 0.f, false, &pw);
        vp += pw;
    }
    if (MODE != kWP && cbits != 0u) {
        // formed again from the raw vectors (kept from the compiler as new values, so the
        // fast path's terms are not held for this branch)
        __asm__ volatile("" : "+v"(rp), "+v"(rq));
        if (MODE != kWQprime) unpack_vec<DT>(rp, zp);
        unpack_vec<DT>(rq, zq);
        vw = 0.0;
        vp = 0.0;
#pragma unroll
        for (int e = 0; e < N; ++e) {
            double pw;
            vw += elem_weight_t<MODE>(wp, MODE != kWQprime ? zp[e] : 0.f, zq[e], (cbits >> e) & 1u, &pw);
            vp += pw;
        }
    }
}

// The law of a row (the same in every lane) in scalar registers.
__device__ __forceinline__ double uniform_f64(double v) {
    return __builtin_bit_cast(double, uniform(__builtin_bit_cast(uint64_t, v)));
}
__device__ __forceinline__ float uniform_f32(float v) {
    return __builtin_bit_cast(float, uniform(__builtin_bit_cast(uint32_t, v)));
}
__device__ __forceinline__ WParams uniform_wparams(WParams w) {
    w.c = uniform_f32(w.c);
    w.op = uniform_f32(w.op);
    w.oq = uniform_f32(w.oq);
    w.inv_p = uniform_f64(w.inv_p);
    w.rho = uniform_f64(w.rho);
    w.rhoC = uniform_f64(w.rhoC);
    w.Cd = uniform_f64(w.Cd);
    return w;
}

// Non-temporal loads of a pass-2 tile that lies inside the row (16-byte aligned rows).
template <int DT>
__device__ __forceinline__ void load_full_tile(const char* row, int t, int lane, u32x4 (&raw)[kVecPass2]) {
    const u32x4* base =
        reinterpret_cast<const u32x4*>(row + (int64_t)t * kTile2<DT> * ElemTraits<DT>::kBytes) + lane;
#pragma unroll
    for (int j = 0; j < kVecPass2; ++j) raw[j] = __builtin_nontemporal_load(base + j * kWave);
}

// Sums of one tile from its raw vectors, written to the tile's slot.
template <int DT, int MODE>
__device__ __forceinline__ void tile_sums_raw(const Pass2Args& a, int g, int t, const WParams& wp, int my_id,
                                              uint32_t* bits, const u32x4 (&rp)[kVecPass2],
                                              const u32x4 (&rq)[kVecPass2]) {
    constexpr int N = ElemTraits<DT>::kPerVec;
    const int lane = lane_id();
    const int64_t t0 = (int64_t)t * kTile2<DT>;
    if (MODE != kWP) tile_bitmap<DT>(bits, t0, my_id);
    double sw = 0.0, sp = 0.0;
#pragma unroll
    for (int j = 0; j < kVecPass2; ++j) {
        const int64_t e0 = t0 + (int64_t)(j * kWave + lane) * N;
        double vw, vp;
        vec_sums<DT, MODE>(wp, rp[j], rq[j], e0, bits, t0, vw, vp);
        sw += vw;
        sp += vp;
        __asm__ volatile("" : "+v"(sw), "+v"(sp));  // one vector's terms live at a time
    }
    sw = wave_sum_f64(sw);
    sp = wave_sum_f64(sp);
    if (lane == 0) a.seg[(int64_t)g * a.nt + t] = make_double2(sw, sp);
}

// Sums of tiles t and t + 1 (if t + 1 < te) of one row pair by one wave.  The second
// tile's loads are issued before the first tile is weighed (two register buffers), so
// its HBM reads overlap the first tile's arithmetic; they are issued on every path that
// weighs the first tile, so the wait before it covers that tile's loads alone.  A tile
// that reaches past V is loaded on its own.  Each tile's sums are those of tile_sums.
template <int DT, int MODE>
__device__ __forceinline__ void tile_pair(const Pass2Args& a, int g, int64_t r, const char* prow, const char* qrow,
                                          int t, int te, const int32_t* ids, int Fk, uint32_t* bits) {
    const int lane = lane_id();
    const int tf = min(te, a.V / kTile2<DT>);  // [t, tf): tiles inside the row
    u32x4 rp[2][kVecPass2], rq[2][kVecPass2];
    if (t < tf) {
        if (MODE != kWQprime) load_full_tile<DT>(prow, t, lane, rp[0]);
        if (MODE != kWP) load_full_tile<DT>(qrow, t, lane, rq[0]);
    }
    int my_id = -1;
    if (MODE != kWP && lane < Fk) my_id = ids[lane];
    WParams wp = a.law ? wparams_from(a.law[r], a.c, a.C) : make_wparams(a.c, a.C, MODE != kWQprime, load_law(a, r));
    wp = uniform_wparams(wp);
    if (t + 1 < tf) {
        if (MODE != kWQprime) load_full_tile<DT>(prow, t + 1, lane, rp[1]);
        if (MODE != kWP) load_full_tile<DT>(qrow, t + 1, lane, rq[1]);
        tile_sums_raw<DT, MODE>(a, g, t, wp, my_id, bits, rp[0], rq[0]);
        tile_sums_raw<DT, MODE>(a, g, t + 1, wp, my_id, bits, rp[1], rq[1]);
    } else if (t < tf) {
        tile_sums_raw<DT, MODE>(a, g, t, wp, my_id, bits, rp[0], rq[0]);
    }
    for (int tt = max(t, tf); tt < te; ++tt) {  // the row's ragged last tile
        if (MODE != kWQprime) load_tile<DT, true, kVecPass2>(prow, (int64_t)tt * kTile2<DT>, a.V, lane, rp[0]);
        if (MODE != kWP) load_tile<DT, true, kVecPass2>(qrow, (int64_t)tt * kTile2<DT>, a.V, lane, rq[0]);
        tile_sums_raw<DT, MODE>(a, g, tt, wp, my_id, bits, rp[0], rq[0]);
    }
}

// Large grids of 16-byte aligned rows: one wave per two adjacent tiles of a group, which
// halves the waves' chains of loads before their first tile (the group's test outcomes,
// then its law and tiles) and overlaps the second tile's reads with the first's weighing.
// Bounded to 4 waves per SIMD (two tile buffers).  One wave per block: a wave that ends
// frees a slot that the next wave can take at once (a block of four waits for four).
template <int DT>
__global__ __launch_bounds__(kWave, 4) void pass2_pair_kernel(const Pass2Args a, int ngroups) {
    __shared__ uint32_t bits[kTile2<1> / 32];
    const int wpg = (a.nt + 1) / 2;  // waves (blocks) per group
    // group g on XCD g mod 8 (the bonus block of group g is block g)
    const int y = blockIdx.x / kXcds;
    const int g = (y / wpg) * kXcds + blockIdx.x % kXcds;
    const int u = y % wpg;
    if (g >= ngroups) return;
    const int t = 2 * u, te = min(t + 2, a.nt);
    int b, pos;
    bool valid;
    pass2_group(a, g, b, pos, valid);
    if (!valid) {
        if (lane_id() == 0)
            for (int tt = t; tt < te; ++tt) a.seg[(int64_t)g * a.nt + tt] = make_double2(0.0, 0.0);
        return;
    }
    const int64_t r = (int64_t)b * (a.K + 1) + pos;
    const int mode = pass2_mode(a, pos);
    const char* prow = a.p_logits ? a.p_logits + r * a.ld_bytes : nullptr;
    const char* qrow = a.q_logits + r * a.ld_bytes;
    const int32_t* ids = a.cache_ids + (int64_t)b * a.Bf + a.O[pos];
    const int Fk = a.F[pos];
    if (mode == kWResid)
        tile_pair<DT, kWResid>(a, g, r, prow, qrow, t, te, ids, Fk, bits);
    else if (mode == kWP)
        tile_pair<DT, kWP>(a, g, r, prow, qrow, t, te, ids, Fk, bits);
    else
        tile_pair<DT, kWQprime>(a, g, r, prow, qrow, t, te, ids, Fk, bits);
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
    CandSummary cs;
    row_stats_wave(a.part + r * a.nt, a.nt, a.c, m, s, arg, false, cs, nullptr);
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
    float m;
    double s;
    int arg;
    CandSummary cs;
    row_stats_wave(a.part + r * a.nt, a.nt, a.c, m, s, arg, true, cs, sc[wave].nc);
    const int F = a.F[i];
    double M = 0.0;
    if (F > 0) {
        const int capU = kWavesPerBlock * a.cap;
        const uint64_t key = row_topf_wave(a.part + r * a.nt, a.cand + r * units_per_row(a.nt) * (int64_t)capU, a.nt,
                                           capU, F, cs, sc[wave]);
        M = finish_cache_row(key, F, q_max[r], q_sum[r], a.c, a.greedy, cache_ids + (int64_t)b * Bf + a.O[i], nullptr);
    }
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
    const bool act = lane < K;
    const int ic = act ? lane : 0;
    const int64_t r = (int64_t)b * K1 + ic;
    const DraftProbe pr = probe_draft<DT>(draft, p_logits, q_logits, ld_bytes, b, lane, K, V, greedy, seed, round);
    bool in_cache = false;
    const int32_t* ids = cache_ids + (int64_t)b * Bf + fo.O[ic];
    for (int j = 0; j < fo.F[ic]; ++j) in_cache |= ids[j] == pr.d;
    const float mp = greedy ? 0.f : p_max[r], mq = greedy ? 0.f : q_max[r];
    const double sp = greedy ? 1.0 : p_sum[r], sq = greedy ? 1.0 : q_sum[r];
    const int argp = greedy ? p_arg[r] : 0;
    const double Zi = greedy ? 1.0 : Z[r];
    double ratio = 0.0;
    int err = 0;
    bool acc = false;
    if (act) acc = test_draft(pr, V, mp, sp, argp, mq, sq, Zi, in_cache, C, c, greedy, &ratio, &err);
    const uint64_t rej = __ballot(act && !acc);
    const int k = rej ? (__ffsll((long long)rej) - 1) : K;
    if (act && accept_prob) accept_prob[(int64_t)b * K + lane] = (float)(ratio < 1.0 ? ratio : 1.0);
    err = (int)wave_or_u32((uint32_t)err);
    if (lane == 0) {
        accept_len[b] = k;
        if (dev_err && err) dev_err[b] |= err;
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

// Next draft from the value store for the separate call: one thread per (b, j).
__global__ void gather_kernel(int B, int K, int Bf, const int32_t* values, const uint8_t* hit, const int32_t* slot,
                              const int32_t* fb, int32_t* next_draft, int32_t* dev_err) {
    const int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (x >= (int64_t)B * K) return;
    const int b = (int)(x / K), j = (int)(x % K);
    int32_t t;
    if (!hit[b]) {
        t = fb[x];
    } else if (slot[b] < 0 || slot[b] >= Bf) {
        t = -1;
        if (j == 0 && dev_err) dev_err[b] |= kErrSlotRange;
    } else {
        t = values[((int64_t)b * Bf + slot[b]) * K + j];
    }
    next_draft[x] = t;
}

// ============================================================================ coverage statistics
// Rank of the bonus t within draft row k (k the acceptance length) in the cache
// order, larger logit first and ties to the lower id: the ids x with z(x) > z(t),
// plus those x < t with z(x) = z(t).  One wave per (sequence, tile) counts its tile;
// the comparison is on fp32 values (-0 equals +0, as in the order of the cache keys).
template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void rank_tile_kernel(const RankArgs a) {
    constexpr int N = ElemTraits<DT>::kPerVec;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int nblk = (a.nt + kWavesPerBlock - 1) / kWavesPerBlock;
    const int b = blockIdx.x / nblk;
    const int t = (blockIdx.x % nblk) * kWavesPerBlock + wave;
    if (t >= a.nt) return;
    const int k = uniform(a.accept_len[b]), tok = uniform(a.bonus[b]);
    uint32_t cnt = 0;
    if (k >= 0 && k <= a.K && tok >= 0 && tok < a.V) {
        const char* row = a.q_logits + ((int64_t)b * (a.K + 1) + k) * a.ld_bytes;
        const int64_t t0 = (int64_t)t * kTile<DT>;
        u32x4 raw[kVecPerLane];
        load_tile<DT, VEC, kVecPerLane>(row, t0, a.V, lane, raw);
        const float zt = load_one<DT>(row, tok);
        if (t0 + kTile<DT> <= tok || t0 > tok) {
            // the whole tile lies on one side of t: one comparison for all of it
            const bool below = t0 < tok;
#pragma unroll
            for (int j = 0; j < kVecPerLane; ++j) {
                float x[N];
                unpack_vec<DT>(raw[j], x);
#pragma unroll
                for (int e = 0; e < N; ++e) cnt += below ? (x[e] >= zt) : (x[e] > zt);
            }
        } else {
#pragma unroll
            for (int j = 0; j < kVecPerLane; ++j) {
                float x[N];
                unpack_vec<DT>(raw[j], x);
                const int64_t e0 = t0 + (int64_t)(j * kWave + lane) * N;
#pragma unroll
                for (int e = 0; e < N; ++e) cnt += (e0 + e < tok) ? (x[e] >= zt) : (x[e] > zt);
            }
        }
    }
    cnt = wave_sum_u32(cnt);
    if (lane == 0) a.counts[(int64_t)b * a.nt + t] = cnt;
}

// Sum of the tile counts per sequence (one wave per sequence, strided over the
// grid), histogram in LDS per block, merged into the global histogram with one
// vector atomic add per non-empty bin.
constexpr int kRankWaves = 16;
__global__ __launch_bounds__(kRankWaves * kWave) void rank_finish_kernel(const RankArgs a) {
    __shared__ uint32_t h[(kMaxK + 1) * (kMaxF + 1)];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int nbins = (a.K + 1) * (a.R + 1);
    for (int i = threadIdx.x; i < nbins; i += blockDim.x) h[i] = 0u;
    __syncthreads();
    for (int b = blockIdx.x * kRankWaves + wave; b < a.B; b += gridDim.x * kRankWaves) {
        uint32_t c = 0;
        for (int t = lane; t < a.nt; t += kWave) c += a.counts[(int64_t)b * a.nt + t];
        const uint32_t rank = wave_sum_u32(c);
        const int k = a.accept_len[b], tok = a.bonus[b];
        const bool valid = k >= 0 && k <= a.K && tok >= 0 && tok < a.V;
        if (lane == 0) {
            if (a.rank_out) a.rank_out[b] = valid ? (int32_t)rank : -1;
            if (valid && a.hist) atomicAdd(&h[k * (a.R + 1) + (rank < (uint32_t)a.R ? (int)rank : a.R)], 1u);
        }
    }
    __syncthreads();
    if (a.hist)
        for (int i = threadIdx.x; i < nbins; i += blockDim.x)
            if (h[i]) atomicAdd(&a.hist[i], h[i]);
}

// ============================================================================ read ceiling
// Read-only stream over a buffer in pass 1's access shape: one wave per 8 KiB (each
// lane eight non-temporal 16-byte loads, vector j of lane l at (j*64 + l)*16 bytes),
// nothing computed but an XOR that keeps the loads alive.  Its rate on the same
// buffers is the reference the vocabulary pass is measured against.
__global__ __launch_bounds__(kBlock) void stream_read_kernel(const u32x4* __restrict__ buf, int64_t nvec,
                                                             uint32_t* sink) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int64_t w = (int64_t)blockIdx.x * kWavesPerBlock + wave;
    const int64_t v0 = w * (kVecPerLane * kWave) + lane;
    u32x4 raw[kVecPerLane];
    if (v0 + (int64_t)(kVecPerLane - 1) * kWave < nvec) {
#pragma unroll
        for (int j = 0; j < kVecPerLane; ++j) raw[j] = __builtin_nontemporal_load(buf + v0 + j * kWave);
    } else {
#pragma unroll
        for (int j = 0; j < kVecPerLane; ++j) {
            const int64_t v = v0 + j * kWave;
            raw[j] = v < nvec ? buf[v] : u32x4{0u, 0u, 0u, 0u};
        }
    }
    uint32_t x = 0u;
#pragma unroll
    for (int j = 0; j < kVecPerLane; ++j) x ^= raw[j].x ^ raw[j].y ^ raw[j].z ^ raw[j].w;
    // a store that (almost) never happens, on a value that depends on every load
    if (x == 0x9E3779B9u) sink[0] = x;
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
    const int64_t grid = (int64_t)xcd_slots(a.B, a.K1) * a.nmodel * nblk;
    if (grid <= 0 || grid > INT_MAX) return hipErrorInvalidValue;
    return by_type(dtype, vec, [&](auto DT, auto VEC) {
        if (a.greedy)
            pass1_kernel<decltype(DT)::value, decltype(VEC)::value, true><<<(unsigned)grid, kBlock, 0, st>>>(a);
        else
            pass1_kernel<decltype(DT)::value, decltype(VEC)::value, false><<<(unsigned)grid, kBlock, 0, st>>>(a);
    });
}

hipError_t launch_finalize_pos(int dtype, const SeqFinal& f, hipStream_t st) {
    const int grid = xcd_slots(f.B, f.K + 1);
    const bool dev = f.round_ptr != nullptr;  // round counter in device memory
    if (f.B * (f.K + 1) <= kFinalizeTwoWaveMaxPairs) {
        if (dtype == 1 && dev)
            finalize_pos2_kernel<1, true><<<grid, 2 * kWave, 0, st>>>(f);
        else if (dtype == 1)
            finalize_pos2_kernel<1, false><<<grid, 2 * kWave, 0, st>>>(f);
        else if (dev)
            finalize_pos2_kernel<0, true><<<grid, 2 * kWave, 0, st>>>(f);
        else
            finalize_pos2_kernel<0, false><<<grid, 2 * kWave, 0, st>>>(f);
    } else {
        if (dtype == 1 && dev)
            finalize_pos_kernel<1, true><<<grid, kWave, 0, st>>>(f);
        else if (dtype == 1)
            finalize_pos_kernel<1, false><<<grid, kWave, 0, st>>>(f);
        else if (dev)
            finalize_pos_kernel<0, true><<<grid, kWave, 0, st>>>(f);
        else
            finalize_pos_kernel<0, false><<<grid, kWave, 0, st>>>(f);
    }
    return hipGetLastError();
}

hipError_t launch_finish_greedy(const SeqFinal& f, hipStream_t st) {
    const int grid = (f.B + kXcds * kWavesPerBlock - 1) / (kXcds * kWavesPerBlock) * kXcds;
    if (f.round_ptr)
        finish_greedy_kernel<true><<<grid, kBlock, 0, st>>>(f);
    else
        finish_greedy_kernel<false><<<grid, kBlock, 0, st>>>(f);
    return hipGetLastError();
}

hipError_t launch_pass2(int dtype, bool vec, const Pass2Args& a, int ngroups, hipStream_t st) {
    const int nblk = (a.nt + kWavesPerBlock - 1) / kWavesPerBlock;
    const int64_t grid = ((int64_t)ngroups + kXcds - 1) / kXcds * kXcds * nblk;
    if (grid <= 0 || grid > INT_MAX) return hipErrorInvalidValue;
    const bool lean = (int64_t)ngroups * a.nt > kPass2LeanMinTiles;
    if (lean && vec && a.mode == 0) {  // two tiles per wave (the draft law's one-row tiles keep one)
        const int64_t g2 = ((int64_t)ngroups + kXcds - 1) / kXcds * kXcds * ((a.nt + 1) / 2);
        if (g2 > INT_MAX) return hipErrorInvalidValue;
        if (dtype == 1)
            pass2_pair_kernel<1><<<(unsigned)g2, kWave, 0, st>>>(a, ngroups);
        else
            pass2_pair_kernel<0><<<(unsigned)g2, kWave, 0, st>>>(a, ngroups);
        return hipGetLastError();
    }
    return by_type(dtype, vec, [&](auto DT, auto VEC) {
        if (lean)
            pass2_kernel<decltype(DT)::value, decltype(VEC)::value, true><<<(unsigned)grid, kBlock, 0, st>>>(a, ngroups);
        else
            pass2_kernel<decltype(DT)::value, decltype(VEC)::value, false><<<(unsigned)grid, kBlock, 0, st>>>(a, ngroups);
    });
}

hipError_t launch_finalize_bonus(int dtype, bool vec, const Pass2Args& a, int ngroups, hipStream_t st) {
    const int grid = ngroups;
    return by_type(dtype, vec, [&](auto DT, auto VEC) {
        if (a.round_ptr)
            finalize_bonus_kernel<decltype(DT)::value, decltype(VEC)::value, true><<<grid, kBlock, 0, st>>>(a, ngroups);
        else
            finalize_bonus_kernel<decltype(DT)::value, decltype(VEC)::value, false><<<grid, kBlock, 0, st>>>(a, ngroups);
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

hipError_t launch_gather(int B, int K, int Bf, const int32_t* values, const uint8_t* hit, const int32_t* slot,
                         const int32_t* fallback_tokens, int32_t* next_draft, int32_t* dev_err, hipStream_t st) {
    const int64_t n = (int64_t)B * K;
    gather_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(B, K, Bf, values, hit, slot, fallback_tokens,
                                                               next_draft, dev_err);
    return hipGetLastError();
}

hipError_t launch_rank(int dtype, bool vec, const RankArgs& a, hipStream_t st) {
    const int nblk = (a.nt + kWavesPerBlock - 1) / kWavesPerBlock;
    const int64_t grid = (int64_t)a.B * nblk;
    if (grid <= 0 || grid > INT_MAX || a.R < 1 || a.R > kMaxF || a.K > kMaxK) return hipErrorInvalidValue;
    hipError_t e = by_type(dtype, vec, [&](auto DT, auto VEC) {
        rank_tile_kernel<decltype(DT)::value, decltype(VEC)::value><<<(unsigned)grid, kBlock, 0, st>>>(a);
    });
    if (e != hipSuccess) return e;
    const int g2 = (int)std::min<int64_t>(((int64_t)a.B + kRankWaves - 1) / kRankWaves, 256);
    rank_finish_kernel<<<g2, kRankWaves * kWave, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_stream_read(const void* buf, int64_t nvec, uint32_t* sink, hipStream_t st) {
    constexpr int64_t per_block = (int64_t)kVecPerLane * kWave * kWavesPerBlock;
    const int64_t grid = (nvec + per_block - 1) / per_block;
    if (grid <= 0 || grid > INT_MAX) return hipErrorInvalidValue;
    stream_read_kernel<<<(unsigned)grid, kBlock, 0, st>>>(static_cast<const u32x4*>(buf), nvec, sink);
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
